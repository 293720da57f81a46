"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/mala.h, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import pytest

import adaptive_tile_skipping_amd as mala

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mala.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mala_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mala_fwd", "mala_fwd_workspace_size", "mala_fwd_varlen", "mala_fwd_varlen_workspace_size",
              "mala_bwd", "mala_bwd_workspace_size", "mala_bwd_varlen", "mala_bwd_varlen_workspace_size",
              "mala_decode", "mala_decode_workspace_size", "mala_decode_varlen", "mala_status_string",
              "mala_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = mala.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) <= set(mala.EXPORTS) | {"mala_version"}


def test_status_strings_and_version():
    lib = mala.load_library()
    for code, name in enumerate(["MALA_OK", "MALA_ERR_INVALID_ARG", "MALA_ERR_UNSUPPORTED",
                                 "MALA_ERR_WORKSPACE", "MALA_ERR_HIP"]):
        assert lib.mala_status_string(code).decode() == name
    assert b"gfx950" in lib.mala_version()


def _t4(ptr=16 * 1024, sb=8 * 1024, sl=8 * 16, sh=128):
    return mala.MalaT4(ptr, sb, sl, sh)


def _fwd(**kw):
    a = dict(q=_t4(), k=_t4(), v=_t4(), B=1, L=256, Hq=2, Hkv=1, d=128, tau=1.0, Bq=128, Bk=64,
             o=_t4(), lse=ctypes.c_void_p(4096), stats=None)
    a.update(kw)
    lib = mala.load_library()
    return lib.mala_fwd(a["q"], a["k"], a["v"], a["B"], a["L"], a["Hq"], a["Hkv"], a["d"], a["tau"],
                        a["Bq"], a["Bk"], a["o"], a["lse"], a["stats"], a.get("ws", ctypes.c_void_p(1 << 20)),
                        a.get("ws_bytes", 1 << 30), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=mala.MalaT4(None, 0, 0, 0)), mala.MALA_ERR_INVALID_ARG),
    (dict(lse=None), mala.MALA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), mala.MALA_ERR_INVALID_ARG),
    (dict(tau=-1.0), mala.MALA_ERR_INVALID_ARG),
    (dict(tau=float("nan")), mala.MALA_ERR_INVALID_ARG),
    (dict(tau=float("inf")), mala.MALA_ERR_INVALID_ARG),
    (dict(L=0), mala.MALA_ERR_INVALID_ARG),
    (dict(B=-1), mala.MALA_ERR_INVALID_ARG),
    (dict(q=_t4(ptr=16 * 1024 + 2)), mala.MALA_ERR_INVALID_ARG),    # misaligned pointer
    (dict(k=_t4(sl=130)), mala.MALA_ERR_INVALID_ARG),               # stride not a multiple of 8
    (dict(d=96), mala.MALA_ERR_UNSUPPORTED),
    (dict(Bq=64), mala.MALA_ERR_UNSUPPORTED),
    (dict(Bk=128), mala.MALA_ERR_UNSUPPORTED),
    (dict(ws=None), mala.MALA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), mala.MALA_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p((1 << 20) + 64)), mala.MALA_ERR_WORKSPACE),
])
def test_fwd_rejects_bad_arguments(kw, code):
    assert _fwd(**kw) == code


def test_fwd_workspace_holds_v_copy_and_work_queues():
    """The forward workspace is the fp16 V copy (B x Hkv x L rounded up to Bk
    keys of d values, as transposed tiles) followed by 256 bytes of work queues;
    one byte less is refused before any launch."""
    lib = mala.load_library()
    n = lib.mala_fwd_workspace_size(1, 1000, 4, 2, 128, 128, 64)
    assert n == 1 * 2 * 1024 * 128 * 2 + 256
    assert _fwd(L=1000, Hq=4, Hkv=2, ws_bytes=n - 1) == mala.MALA_ERR_WORKSPACE
    nv = lib.mala_fwd_varlen_workspace_size(3, 5000, 2, 128, 128, 64)
    assert nv == (5000 + 3 * 64) * 2 * 128 * 2 + 256


def test_bwd_workspace_and_errors():
    lib = mala.load_library()
    n = lib.mala_bwd_workspace_size(1, 1000, 4, 2, 128, 128, 64)
    assert n >= 2 * 4 * 1024 * 4          # D_i and LSE rows over the padded length (Hq = 4)
    assert lib.mala_bwd_workspace_size(1, 1000, 4, 2, 96, 128, 64) == 0
    t = _t4()
    args = [t, t, t, t, t, ctypes.c_void_p(4096), 1, 1000, 4, 2, 128, 1.0, 128, 64, t, t, t]
    # missing / small / misaligned workspace
    assert lib.mala_bwd(*args, None, 0, None, None) == mala.MALA_ERR_WORKSPACE
    assert lib.mala_bwd(*args, ctypes.c_void_p(1 << 20), n - 1, None, None) == mala.MALA_ERR_WORKSPACE
    assert lib.mala_bwd(*args, ctypes.c_void_p((1 << 20) + 16), n, None, None) == mala.MALA_ERR_WORKSPACE
    bad = list(args)
    bad[11] = -0.5
    assert lib.mala_bwd(*bad, ctypes.c_void_p(1 << 20), n, None, None) == mala.MALA_ERR_INVALID_ARG
    st = mala.MalaTileStats(None, None, 4096, None)   # omitted mass is forward-only
    assert lib.mala_bwd(*args, ctypes.c_void_p(1 << 20), n, ctypes.pointer(st), None) == mala.MALA_ERR_INVALID_ARG


def test_decode_workspace_and_errors():
    lib = mala.load_library()
    n = lib.mala_decode_workspace_size(8, 131072, 5, 1, 128, 64)
    assert n > 8 * 5 * 131072 * 2     # at least the fp16 probability spill
    assert lib.mala_decode_workspace_size(8, 131072, 5, 1, 128, 32) == 0
    t = _t4()
    q = ctypes.c_void_p(4096)
    base = [q, t, t, 2, 1000, 4, 2, 128, 1.0, 64, ctypes.c_void_p(8192), ctypes.c_void_p(12288), None, None]
    assert lib.mala_decode(*base, None, 0, None) == mala.MALA_ERR_WORKSPACE
    bad = list(base)
    bad[8] = float("nan")
    assert lib.mala_decode(*bad, ctypes.c_void_p(1 << 20), 1 << 30, None) == mala.MALA_ERR_INVALID_ARG
    bad = list(base)
    bad[9] = 32
    assert lib.mala_decode(*bad, ctypes.c_void_p(1 << 20), 1 << 30, None) == mala.MALA_ERR_UNSUPPORTED
    bad = list(base)
    bad[0] = ctypes.c_void_p(4098)
    assert lib.mala_decode(*bad, ctypes.c_void_p(1 << 20), 1 << 30, None) == mala.MALA_ERR_INVALID_ARG


def test_decode_noalloc_refuses_before_touching_the_gpu():
    """The allocation-free decode: argument errors as mala_decode, then
    MALA_ERR_WORKSPACE for shapes whose workspace exceeds the fixed scratch;
    neither reaches HIP (this runs without a GPU)."""
    lib = mala.load_library()
    cap = mala.DECODE_NOALLOC_MAX_BYTES
    hdr = open(os.path.join(ROOT, "include", "mala.h")).read()
    assert f"#define MALA_DECODE_NOALLOC_MAX_BYTES ({cap >> 20}u << 20)" in hdr
    # the benchmarked decode (8 sequences x 131072 keys, 5 q heads per KV head) fits; 64 sequences do not
    assert 0 < lib.mala_decode_workspace_size(8, 131072, 5, 1, 128, 64) <= cap
    assert lib.mala_decode_workspace_size(64, 131072, 5, 1, 128, 64) > cap
    t = _t4()
    q, o, lse = ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(12288)
    big = [q, t, t, 64, 131072, 5, 1, 128, 1.0, 64, o, lse, None, None, None]
    assert lib.mala_decode_noalloc(*big) == mala.MALA_ERR_WORKSPACE
    bad = list(big)
    bad[8] = float("nan")
    assert lib.mala_decode_noalloc(*bad) == mala.MALA_ERR_INVALID_ARG
    bad = [q, t, t, 2, 1000, 4, 2, 128, 1.0, 32, o, lse, None, None, None]
    assert lib.mala_decode_noalloc(*bad) == mala.MALA_ERR_UNSUPPORTED
    bad = [q, t, t, 2, 1000, 4, 3, 128, 1.0, 64, o, lse, None, None, None]     # Hq % Hkv != 0
    assert lib.mala_decode_noalloc(*bad) == mala.MALA_ERR_INVALID_ARG


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 128, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="GPU only"):
        mala.mala_fwd(x, x, x, 1.0)


def _t3(ptr=16 * 1024, sl=8 * 16, sh=128):
    return mala.MalaT3(ptr, sl, sh)


def _fwd_varlen(**kw):
    a = dict(q=_t3(), k=_t3(), v=_t3(), cu_q=ctypes.c_void_p(4096), cu_k=ctypes.c_void_p(8192), B=2,
             total_q=300, total_k=900, max_q=200, max_k=600, Hq=2, Hkv=1, d=128, tau=1.0, Bq=128, Bk=64,
             o=_t3(), lse=ctypes.c_void_p(12288), stats=None)
    a.update(kw)
    lib = mala.load_library()
    return lib.mala_fwd_varlen(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], a["B"], a["total_q"], a["total_k"],
                               a["max_q"], a["max_k"], a["Hq"], a["Hkv"], a["d"], a["tau"], a["Bq"], a["Bk"],
                               a["o"], a["lse"], a["stats"], a.get("ws", ctypes.c_void_p(1 << 20)),
                               a.get("ws_bytes", 1 << 30), None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu_q=None), mala.MALA_ERR_INVALID_ARG),
    (dict(cu_k=None), mala.MALA_ERR_INVALID_ARG),
    (dict(lse=None), mala.MALA_ERR_INVALID_ARG),
    (dict(q=mala.MalaT3(None, 0, 0)), mala.MALA_ERR_INVALID_ARG),
    (dict(o=_t3(ptr=16 * 1024 + 4)), mala.MALA_ERR_INVALID_ARG),
    (dict(k=_t3(sh=100)), mala.MALA_ERR_INVALID_ARG),
    (dict(B=0), mala.MALA_ERR_INVALID_ARG),
    (dict(max_q=700), mala.MALA_ERR_INVALID_ARG),          # longer than max_k
    (dict(max_q=400, max_k=950), mala.MALA_ERR_INVALID_ARG),  # beyond the totals
    (dict(total_q=-1), mala.MALA_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), mala.MALA_ERR_INVALID_ARG),
    (dict(tau=float("nan")), mala.MALA_ERR_INVALID_ARG),
    (dict(d=96), mala.MALA_ERR_UNSUPPORTED),
    (dict(Bq=64), mala.MALA_ERR_UNSUPPORTED),
    (dict(B=70000, total_q=70000, total_k=90000, max_q=100, max_k=600), mala.MALA_ERR_UNSUPPORTED),
    (dict(ws=None), mala.MALA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), mala.MALA_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16)), mala.MALA_ERR_WORKSPACE),
    # no query rows: nothing to do, nothing enqueued
    (dict(total_q=0, max_q=0), mala.MALA_OK),
])
def test_fwd_varlen_rejects_bad_arguments(kw, code):
    assert _fwd_varlen(**kw) == code


def test_fwd_varlen_workspace_size():
    lib = mala.load_library()
    # fp16 V copy with room for one more tile after each sequence
    assert lib.mala_fwd_varlen_workspace_size(3, 1000, 2, 128, 128, 64) >= (1000 + 3 * 64) * 2 * 128 * 2
    assert lib.mala_fwd_varlen_workspace_size(3, 1000, 2, 96, 128, 64) == 0


def test_decode_varlen_errors():
    lib = mala.load_library()
    t = _t4()
    q = ctypes.c_void_p(4096)
    tail = [2, 1000, 4, 2, 128, 1.0, 64, ctypes.c_void_p(8192), ctypes.c_void_p(12288), None, None]
    # the lengths array is required
    assert lib.mala_decode_varlen(q, t, t, None, *tail, ctypes.c_void_p(1 << 20), 1 << 30, None) == \
        mala.MALA_ERR_INVALID_ARG
    sl = ctypes.c_void_p(16384)
    assert lib.mala_decode_varlen(q, t, t, sl, *tail, None, 0, None) == mala.MALA_ERR_WORKSPACE
    bad = list(tail)
    bad[6] = 32
    assert lib.mala_decode_varlen(q, t, t, sl, *bad, ctypes.c_void_p(1 << 20), 1 << 30, None) == \
        mala.MALA_ERR_UNSUPPORTED


def test_bwd_varlen_workspace_and_errors():
    lib = mala.load_library()
    n = lib.mala_bwd_varlen_workspace_size(2, 300, 200, 600, 4, 2, 128, 128, 64)
    assert n >= 2 * 4 * (300 + 2 * 128) * 4       # D_i and LSE rows with Bq rows of padding per sequence
    assert lib.mala_bwd_varlen_workspace_size(2, 300, 200, 600, 4, 2, 96, 128, 64) == 0
    t = _t3()
    cq, ck, lse = ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(12288)
    head = [t, t, t, t, t, lse, cq, ck]
    mid = [2, 300, 900, 200, 600, 4, 2, 128, 1.0, 128, 64, t, t, t]
    ok_ws = [ctypes.c_void_p(1 << 20), 1 << 30]
    assert lib.mala_bwd_varlen(*head, *mid, None, 0, None, None) == mala.MALA_ERR_WORKSPACE
    bad = list(head)
    bad[6] = None
    assert lib.mala_bwd_varlen(*bad, *mid, *ok_ws, None, None) == mala.MALA_ERR_INVALID_ARG
    bad = list(mid)
    bad[3] = 700                                      # max_q > max_k
    assert lib.mala_bwd_varlen(*head, *bad, *ok_ws, None, None) == mala.MALA_ERR_INVALID_ARG
    bad = list(mid)
    bad[7] = 96
    assert lib.mala_bwd_varlen(*head, *bad, *ok_ws, None, None) == mala.MALA_ERR_UNSUPPORTED
    st = mala.MalaTileStats(None, None, 4096, None)    # omitted mass is forward-only
    assert lib.mala_bwd_varlen(*head, *mid, *ok_ws, ctypes.pointer(st), None) == mala.MALA_ERR_INVALID_ARG


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus above 1 exits with a message, before
    touching any device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one MI355X" in (r.stdout + r.stderr)
