"""The Python binding refuses wrongly shaped, typed or placed tensors with
ValueError before calling the C ABI: a wrong-size buffer would otherwise be
read or written out of its bounds (or, at the same size, in the wrong order).
Nothing is enqueued: outputs passed in keep their contents."""
import pytest
import torch

import adaptive_tile_skipping_amd as mala

pytestmark = pytest.mark.gpu

B, L, HQ, HKV, D = 1, 300, 4, 2, 128


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _bf(*shape):
    return torch.randn(*shape, device=_dev()).to(torch.bfloat16)


@pytest.fixture(scope="module")
def qkv():
    return _bf(B, L, HQ, D), _bf(B, L, HKV, D), _bf(B, L, HKV, D)


def _sentinel_o():
    return torch.full((B, L, HQ, D), 7.0, dtype=torch.bfloat16, device=_dev())


@pytest.mark.parametrize("case", ["k_len", "v_heads", "o_shape", "lse_transposed", "lse_dtype", "stats_slots",
                                  "ws_dtype"])
def test_fwd_refuses(qkv, case):
    q, k, v = qkv
    dev = _dev()
    o = _sentinel_o()
    kw = {}
    if case == "k_len":
        k = _bf(B, L - 1, HKV, D)
    elif case == "v_heads":
        v = _bf(B, L, HKV + 1, D)
    elif case == "o_shape":
        o = torch.full((B, L, HQ - 1, D), 7.0, dtype=torch.bfloat16, device=dev)
    elif case == "lse_transposed":
        kw["lse"] = torch.empty((B, L, HQ), dtype=torch.float32, device=dev)   # same size, wrong order
    elif case == "lse_dtype":
        kw["lse"] = torch.empty((B, HQ, L), dtype=torch.float16, device=dev)
    elif case == "stats_slots":
        st = mala.make_stats(B, HQ, L, 128, 64, dev)
        st["kept_slots"] = torch.empty((B, HQ, L - 5), dtype=torch.int32, device=dev)
        kw["stats"] = st
    elif case == "ws_dtype":
        kw["ws"] = torch.empty(1 << 20, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        mala.mala_fwd(q, k, v, 1.0, o=o, **kw)
    torch.cuda.synchronize()
    if o.shape == (B, L, HQ, D):
        assert (o == 7.0).all()


@pytest.mark.parametrize("case", ["o_shape", "dout_shape", "lse_transposed", "dq_shape", "dk_shape", "dv_heads",
                                  "k_vs_v"])
def test_bwd_refuses(qkv, case):
    q, k, v = qkv
    dev = _dev()
    o, lse = mala.mala_fwd(q, k, v, 1.0)
    do = _bf(B, L, HQ, D)
    dq = torch.full((B, L, HQ, D), 7.0, dtype=torch.bfloat16, device=dev)
    kw = dict(dq=dq)
    if case == "o_shape":
        o = _bf(B, L, HQ, D - 8)
    elif case == "dout_shape":
        do = _bf(B, L - 1, HQ, D)
    elif case == "lse_transposed":
        lse = lse.permute(0, 2, 1).contiguous()
    elif case == "dq_shape":
        kw["dq"] = torch.empty((B, L, HKV, D), dtype=torch.bfloat16, device=dev)
    elif case == "dk_shape":
        kw["dk"] = torch.empty((B, L, HQ, D), dtype=torch.bfloat16, device=dev)
    elif case == "dv_heads":
        kw["dv"] = torch.empty((B, L, HKV + 1, D), dtype=torch.bfloat16, device=dev)
    elif case == "k_vs_v":
        v = _bf(B, L, HKV, D)[:, :L - 3]
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        mala.mala_bwd(q, k, v, o, do, lse, 1.0, **kw)
    torch.cuda.synchronize()
    assert (dq == 7.0).all()


@pytest.mark.parametrize("case", ["v_len", "k_heads", "q_strided", "o_shape", "lse_shape", "kept_shape",
                                  "bits_words", "seqlens_len"])
def test_decode_refuses(case):
    dev = _dev()
    Bd, N, Hq, Hkv = 2, 1000, 6, 2
    q = _bf(Bd, Hq, D)
    kc, vc = _bf(Bd, N, Hkv, D), _bf(Bd, N, Hkv, D)
    o = torch.full((Bd, Hq, D), 7.0, dtype=torch.bfloat16, device=dev)
    kw = dict(o=o)
    if case == "v_len":
        vc = _bf(Bd, N - 1, Hkv, D)
    elif case == "k_heads":
        kc = _bf(Bd, N, Hkv + 1, D)
    elif case == "q_strided":
        q = _bf(Bd, Hq, 2 * D)[:, :, :D]
    elif case == "o_shape":
        kw["o"] = torch.empty((Bd, Hq - 1, D), dtype=torch.bfloat16, device=dev)
    elif case == "lse_shape":
        kw["lse"] = torch.empty((Bd, Hkv), dtype=torch.float32, device=dev)
    elif case == "kept_shape":
        kw["kept_tiles"] = torch.empty((Bd, Hq), dtype=torch.int32, device=dev)
    elif case == "bits_words":
        kw["decision_bits"] = torch.empty((Bd, Hkv, 0), dtype=torch.int32, device=dev)
    elif case == "seqlens_len":
        kw["cache_seqlens"] = torch.full((Bd + 1,), N, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        mala.mala_decode(q, kc, vc, 1.0, **kw)
    with pytest.raises(ValueError):
        if case != "seqlens_len":
            mala.mala_decode_noalloc(q, kc, vc, 1.0, **{x: y for x, y in kw.items() if x != "cache_seqlens"})
        else:
            raise ValueError("mala_decode_noalloc takes no cache lengths")
    torch.cuda.synchronize()
    assert (o == 7.0).all()


def test_varlen_refuses_wrong_lse_and_outputs():
    dev = _dev()
    cu_q = torch.tensor([0, 100, 300], dtype=torch.int32, device=dev)
    cu_k = torch.tensor([0, 150, 450], dtype=torch.int32, device=dev)
    q, k, v = _bf(300, HQ, D), _bf(450, HKV, D), _bf(450, HKV, D)
    with pytest.raises(ValueError):
        mala.mala_fwd_varlen(q, k, v, cu_q, cu_k, 200, 300, 1.0,
                             lse=torch.empty((300, HQ), dtype=torch.float32, device=dev))
    o, lse = mala.mala_fwd_varlen(q, k, v, cu_q, cu_k, 200, 300, 1.0)
    with pytest.raises(ValueError):
        mala.mala_bwd_varlen(q, k, v, o, _bf(300, HQ, D), lse, cu_q, cu_k, 200, 300, 1.0,
                             dk=torch.empty((450, HQ, D), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        mala.mala_bwd_varlen(q, k, v[:449], o, _bf(300, HQ, D), lse, cu_q, cu_k, 200, 300, 1.0)
    torch.cuda.synchronize()
