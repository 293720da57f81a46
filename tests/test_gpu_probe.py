"""The library's measurement probes (include/mala.h: mala_probe_mfma,
mala_probe_read) do the work whose rate bench.py reports: every wave of the
MFMA probe runs `iters` rounds of four 32x32x16 bf16 MFMAs on the operands it
builds from its lane index, and the read probe touches every word of the
buffer once.  Both are checked against values computed on the host."""
import numpy as np
import pytest
import torch

import adaptive_tile_skipping_amd as mala

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _bf16_round(x):
    """fp32 -> bf16 (round to nearest even) -> float64, on the host."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def test_mfma_probe_sums_match_the_host_product():
    dev = _dev()
    iters = 96
    sink = torch.zeros(mala.PROBE_SINK_WORDS, dtype=torch.float32, device=dev)
    flop = mala.probe_mfma(iters, sink)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    waves = 2 * cus * 4
    assert flop == waves * 4 * iters * 2.0 * 32 * 32 * 16
    # A[i][k] sits in lane i + 32 (k / 8), element k % 8, as 1e-3 (lane + e);
    # B[k][j] in lane j + 32 (k / 8), element k % 8, as 1e-3 (lane - e)
    A = np.zeros((32, 16))
    Bm = np.zeros((16, 32))
    for k in range(16):
        e, h = k % 8, k // 8
        for i in range(32):
            A[i, k] = _bf16_round(np.float32(1e-3) * np.float32(i + 32 * h + e))
            Bm[k, i] = _bf16_round(np.float32(1e-3) * np.float32(i + 32 * h - e))
    C = A @ Bm
    # lane 0 holds column 0, rows 8 (r / 4) + r % 4 of each accumulator
    rows = [8 * (r // 4) + r % 4 for r in range(16)]
    want = 4 * iters * C[rows, 0].sum()
    got = sink[:waves].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-4)
    assert np.all(sink[waves:].cpu().numpy() == 0.0)


def test_read_probe_touches_every_word_once():
    dev = _dev()
    g = torch.Generator(device="cpu").manual_seed(11)
    for n_words in (4, 1000, (1 << 22) + 12):           # tails of the unrolled loop included
        host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_words,), generator=g, dtype=torch.int64).to(torch.int32)
        src = host.to(dev)
        sink = torch.zeros(mala.PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
        nbytes = mala.probe_read(src, sink)
        torch.cuda.synchronize()
        assert nbytes == 4 * n_words
        want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, n_words


def test_probes_refuse_bad_arguments():
    dev = _dev()
    lib = mala.load_library()
    fsink = torch.zeros(mala.PROBE_SINK_WORDS, dtype=torch.float32, device=dev)
    isink = torch.zeros(mala.PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    src = torch.zeros(64, dtype=torch.int32, device=dev)
    assert lib.mala_probe_mfma(0, fsink.data_ptr(), None) == mala.MALA_ERR_INVALID_ARG
    assert lib.mala_probe_mfma(1, None, None) == mala.MALA_ERR_INVALID_ARG
    assert lib.mala_probe_read(src.data_ptr(), 20, isink.data_ptr(), None) == mala.MALA_ERR_INVALID_ARG
    assert lib.mala_probe_read(src.data_ptr() + 4, 64, isink.data_ptr(), None) == mala.MALA_ERR_INVALID_ARG
    assert lib.mala_probe_read(None, 64, isink.data_ptr(), None) == mala.MALA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        mala.probe_mfma(1, torch.zeros(16, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    assert float(fsink.abs().sum()) == 0.0 and int(isink.abs().sum()) == 0
