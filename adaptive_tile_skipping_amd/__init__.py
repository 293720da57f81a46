"""Python binding of libmala (MALA fused causal attention for MI355X / gfx950).

Argument marshalling only: every step of the attention runs in the HIP
kernels of libmala.so, reached through its C ABI (include/mala.h) with ctypes.
PyTorch supplies device memory and the current HIP stream.  There is no CPU
fallback: if the library is missing or the tensors are not on a HIP device,
the calls raise.

Names follow the C ABI: mala_fwd, mala_fwd_varlen, mala_bwd, mala_bwd_varlen, mala_decode (with optional
per-sequence cache lengths: mala_decode_varlen), mala_decode_noalloc (decode
on the library's own fixed device scratch, for callers that cannot
allocate), plus the autograd wrapper `mala_attention` (saves only q, k, v, o
and lse for the backward).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmala.so")

MALA_OK, MALA_ERR_INVALID_ARG, MALA_ERR_UNSUPPORTED, MALA_ERR_WORKSPACE, MALA_ERR_HIP = range(5)


class MalaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({code})")
        self.code = code


class MalaT4(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sb", ctypes.c_int64), ("sl", ctypes.c_int64), ("sh", ctypes.c_int64)]


class MalaT3(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sl", ctypes.c_int64), ("sh", ctypes.c_int64)]


class MalaTileStats(ctypes.Structure):
    _fields_ = [("kept_tiles", ctypes.c_void_p), ("kept_slots", ctypes.c_void_p),
                ("omitted_mass", ctypes.c_void_p), ("decision_bits", ctypes.c_void_p)]


EXPORTS = ("mala_fwd", "mala_fwd_workspace_size", "mala_fwd_varlen", "mala_fwd_varlen_workspace_size",
           "mala_bwd", "mala_bwd_workspace_size", "mala_bwd_varlen", "mala_bwd_varlen_workspace_size",
           "mala_decode", "mala_decode_workspace_size", "mala_decode_varlen", "mala_decode_noalloc",
           "mala_probe_mfma", "mala_probe_mfma_flop", "mala_probe_read", "mala_status_string", "mala_version")

# include/mala.h: MALA_DECODE_NOALLOC_MAX_BYTES, MALA_PROBE_SINK_WORDS
DECODE_NOALLOC_MAX_BYTES = 64 << 20
PROBE_SINK_WORDS = 256 * 1024

_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libmala.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libmala.so not found at {p}: build it first "
                           "(python -m adaptive_tile_skipping_amd._build or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.mala_fwd_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.mala_fwd_workspace_size.restype = S
    lib.mala_fwd.argtypes = [MalaT4, MalaT4, MalaT4, I, I, I, I, I, F, I, I, MalaT4, P,
                             ctypes.POINTER(MalaTileStats), P, S, P]
    lib.mala_fwd.restype = I
    lib.mala_fwd_varlen_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.mala_fwd_varlen_workspace_size.restype = S
    lib.mala_fwd_varlen.argtypes = [MalaT3, MalaT3, MalaT3, P, P, I, I, I, I, I, I, I, I, F, I, I, MalaT3, P,
                                    ctypes.POINTER(MalaTileStats), P, S, P]
    lib.mala_fwd_varlen.restype = I
    lib.mala_bwd_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.mala_bwd_workspace_size.restype = S
    lib.mala_bwd.argtypes = [MalaT4, MalaT4, MalaT4, MalaT4, MalaT4, P, I, I, I, I, I, F, I, I,
                             MalaT4, MalaT4, MalaT4, P, S, ctypes.POINTER(MalaTileStats), P]
    lib.mala_bwd.restype = I
    lib.mala_bwd_varlen_workspace_size.argtypes = [I, I, I, I, I, I, I, I, I]
    lib.mala_bwd_varlen_workspace_size.restype = S
    lib.mala_bwd_varlen.argtypes = [MalaT3, MalaT3, MalaT3, MalaT3, MalaT3, P, P, P, I, I, I, I, I, I, I, I, F, I, I,
                                    MalaT3, MalaT3, MalaT3, P, S, ctypes.POINTER(MalaTileStats), P]
    lib.mala_bwd_varlen.restype = I
    lib.mala_decode_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.mala_decode_workspace_size.restype = S
    lib.mala_decode.argtypes = [P, MalaT4, MalaT4, I, I, I, I, I, F, I, P, P, P, P, P, S, P]
    lib.mala_decode.restype = I
    lib.mala_decode_varlen.argtypes = [P, MalaT4, MalaT4, P, I, I, I, I, I, F, I, P, P, P, P, P, S, P]
    lib.mala_decode_varlen.restype = I
    lib.mala_decode_noalloc.argtypes = [P, MalaT4, MalaT4, I, I, I, I, I, F, I, P, P, P, P, P]
    lib.mala_decode_noalloc.restype = I
    lib.mala_probe_mfma.argtypes = [I, P, P]
    lib.mala_probe_mfma.restype = I
    lib.mala_probe_mfma_flop.argtypes = [I]
    lib.mala_probe_mfma_flop.restype = ctypes.c_double
    lib.mala_probe_read.argtypes = [P, S, P, P]
    lib.mala_probe_read.restype = I
    lib.mala_status_string.argtypes = [I]
    lib.mala_status_string.restype = ctypes.c_char_p
    lib.mala_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, code: int):
    if code != MALA_OK:
        raise MalaError(fn, code, load_library().mala_status_string(code).decode())


def _t4(t: torch.Tensor) -> MalaT4:
    if t.dim() != 4:
        raise ValueError("expected a [B, L, H, d] tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError("libmala takes bfloat16 tensors")
    if t.stride(3) != 1:
        raise ValueError("the d dimension must be contiguous")
    return MalaT4(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _t3(t: torch.Tensor) -> MalaT3:
    if t.dim() != 3:
        raise ValueError("expected a packed [total, H, d] tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError("libmala takes bfloat16 tensors")
    if t.stride(2) != 1:
        raise ValueError("the d dimension must be contiguous")
    return MalaT3(t.data_ptr(), t.stride(0), t.stride(1))


def _dev_check(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise RuntimeError("libmala runs on the GPU only: tensors must live on a HIP device")


def _expect(t, shape, dtype, name: str, device, contiguous: bool = False):
    """Raise ValueError unless t has exactly this shape and dtype, lives on
    `device`, and (if asked) is contiguous.  Run before anything is enqueued:
    a wrongly shaped buffer would be read or written out of its bounds."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_stats(stats, B, Hq, rows, nQB, nKT, device, varlen: bool = False):
    """Shapes of the optional statistics outputs (make_stats /
    make_varlen_stats)."""
    if not stats:
        return
    row_shape = (Hq, rows) if varlen else (B, Hq, rows)
    _expect(stats.get("kept_tiles"), (B, Hq, nQB), torch.int32, "stats['kept_tiles']", device, True)
    _expect(stats.get("kept_slots"), row_shape, torch.int32, "stats['kept_slots']", device, True)
    _expect(stats.get("omitted_mass"), row_shape, torch.float32, "stats['omitted_mass']", device, True)
    _expect(stats.get("decision_bits"), (B, Hq, nQB, -(-nKT // 32)), torch.int32, "stats['decision_bits']", device,
            True)


def _check_ws(ws, device):
    if ws is not None and (ws.dtype != torch.uint8 or ws.device != device or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous uint8 tensor on the device of q")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stats_struct(stats: dict | None):
    if not stats:
        return None
    s = MalaTileStats(*(_ptr(stats.get(n)) for n in ("kept_tiles", "kept_slots", "omitted_mass", "decision_bits")))
    return ctypes.pointer(s)


def make_stats(B: int, Hq: int, L: int, Bq: int, Bk: int, device, omitted: bool = False) -> dict:
    """Allocate the optional statistics outputs of mala_fwd / mala_bwd."""
    nQB, nKT = -(-L // Bq), -(-L // Bk)
    st = {"kept_tiles": torch.empty((B, Hq, nQB), dtype=torch.int32, device=device),
          "kept_slots": torch.empty((B, Hq, L), dtype=torch.int32, device=device),
          "decision_bits": torch.empty((B, Hq, nQB, -(-nKT // 32)), dtype=torch.int32, device=device)}
    if omitted:
        st["omitted_mass"] = torch.empty((B, Hq, L), dtype=torch.float32, device=device)
    return st


def fwd_workspace(B, L, Hq, Hkv, d, Bq=128, Bk=64, device="cuda"):
    n = load_library().mala_fwd_workspace_size(B, L, Hq, Hkv, d, Bq, Bk)
    if n == 0:
        raise MalaError("mala_fwd_workspace_size", MALA_ERR_UNSUPPORTED, "unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mala_fwd(q, k, v, tau: float = 1.0, Bq: int = 128, Bk: int = 64, o=None, lse=None, stats: dict | None = None,
             ws=None):
    """Forward.  q [B,L,Hq,d], k/v [B,L,Hkv,d] bf16 on the GPU.
    Returns (o [B,L,Hq,d] bf16, lse [B,Hq,L] fp32)."""
    _dev_check(q, k, v)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, L, Hq, d] and k, v [B, L, Hkv, d]")
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    dev = q.device
    _expect(k, (B, L, Hkv, d), torch.bfloat16, "k", dev)
    _expect(v, (B, L, Hkv, d), torch.bfloat16, "v", dev)
    _expect(o, (B, L, Hq, d), torch.bfloat16, "o", dev)
    _expect(lse, (B, Hq, L), torch.float32, "lse", dev, True)
    _check_stats(stats, B, Hq, L, -(-L // Bq), -(-L // Bk), dev)
    _check_ws(ws, dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = fwd_workspace(B, L, Hq, Hkv, d, Bq, Bk, q.device)
    lib = load_library()
    rc = lib.mala_fwd(_t4(q), _t4(k), _t4(v), B, L, Hq, Hkv, d, float(tau), Bq, Bk, _t4(o),
                      _ptr(lse), _stats_struct(stats), _ptr(ws), ws.numel(), _stream(q))
    _check("mala_fwd", rc)
    return o, lse


def make_varlen_stats(B: int, Hq: int, total_q: int, max_q: int, max_k: int, Bq: int, Bk: int, device,
                      omitted: bool = False) -> dict:
    """Allocate the optional statistics outputs of mala_fwd_varlen."""
    nQB, nKT = max(1, -(-max_q // Bq)), max(1, -(-max_k // Bk))
    st = {"kept_tiles": torch.empty((B, Hq, nQB), dtype=torch.int32, device=device),
          "kept_slots": torch.empty((Hq, total_q), dtype=torch.int32, device=device),
          "decision_bits": torch.empty((B, Hq, nQB, -(-nKT // 32)), dtype=torch.int32, device=device)}
    if omitted:
        st["omitted_mass"] = torch.empty((Hq, total_q), dtype=torch.float32, device=device)
    return st


def fwd_varlen_workspace(B, total_k, Hkv, d, Bq=128, Bk=64, device="cuda"):
    n = load_library().mala_fwd_varlen_workspace_size(B, total_k, Hkv, d, Bq, Bk)
    if n == 0:
        raise MalaError("mala_fwd_varlen_workspace_size", MALA_ERR_UNSUPPORTED, "unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mala_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, tau: float = 1.0,
                    Bq: int = 128, Bk: int = 64, o=None, lse=None, stats: dict | None = None, ws=None):
    """Forward over packed variable-length sequences whose queries are the last
    Lq of their Lk keys (prefill, chunked prefill onto a cache, mixed batches).
    q [total_q,Hq,d], k/v [total_k,Hkv,d] bf16; cu_seqlens_* int32 [B+1] on the
    same device.  Returns (o [total_q,Hq,d] bf16, lse [Hq,total_q] fp32)."""
    _dev_check(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    dev = q.device
    _expect(k, (Tk, Hkv, d), torch.bfloat16, "k", dev)
    _expect(v, (Tk, Hkv, d), torch.bfloat16, "v", dev)
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or not c.is_contiguous() or c.dim() != 1 or c.device != dev:
            raise ValueError("cu_seqlens must be contiguous int32 [B + 1] tensors on the device of q")
    B = cu_seqlens_q.numel() - 1
    if B < 1 or cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 entries")
    _expect(o, (Tq, Hq, d), torch.bfloat16, "o", dev)
    _expect(lse, (Hq, Tq), torch.float32, "lse", dev, True)
    _check_stats(stats, B, Hq, Tq, max(1, -(-int(max_seqlen_q) // Bq)), max(1, -(-int(max_seqlen_k) // Bk)), dev,
                 varlen=True)
    _check_ws(ws, dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = fwd_varlen_workspace(B, Tk, Hkv, d, Bq, Bk, q.device)
    lib = load_library()
    rc = lib.mala_fwd_varlen(_t3(q), _t3(k), _t3(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Tq, Tk,
                             int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, d, float(tau), Bq, Bk, _t3(o),
                             _ptr(lse), _stats_struct(stats), _ptr(ws), ws.numel(), _stream(q))
    _check("mala_fwd_varlen", rc)
    return o, lse


def bwd_workspace(B, L, Hq, Hkv, d, Bq=128, Bk=64, device="cuda"):
    n = load_library().mala_bwd_workspace_size(B, L, Hq, Hkv, d, Bq, Bk)
    if n == 0:
        raise MalaError("mala_bwd_workspace_size", MALA_ERR_UNSUPPORTED, "unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mala_bwd(q, k, v, o, dout, lse, tau: float = 1.0, Bq: int = 128, Bk: int = 64,
             dq=None, dk=None, dv=None, ws=None, stats: dict | None = None):
    """Backward.  Returns (dq, dk, dv) bf16."""
    _dev_check(q, k, v, o, dout, lse)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, L, Hq, d] and k, v [B, L, Hkv, d]")
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    dev = q.device
    _expect(k, (B, L, Hkv, d), torch.bfloat16, "k", dev)
    _expect(v, (B, L, Hkv, d), torch.bfloat16, "v", dev)
    _expect(o, (B, L, Hq, d), torch.bfloat16, "o", dev)
    _expect(dout, (B, L, Hq, d), torch.bfloat16, "dout", dev)
    _expect(lse, (B, Hq, L), torch.float32, "lse", dev, True)
    _expect(dq, (B, L, Hq, d), torch.bfloat16, "dq", dev)
    _expect(dk, (B, L, Hkv, d), torch.bfloat16, "dk", dev)
    _expect(dv, (B, L, Hkv, d), torch.bfloat16, "dv", dev)
    _check_stats(stats, B, Hq, L, -(-L // Bq), -(-L // Bk), dev)
    _check_ws(ws, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if ws is None:
        ws = bwd_workspace(B, L, Hq, Hkv, d, Bq, Bk, q.device)
    lib = load_library()
    rc = lib.mala_bwd(_t4(q), _t4(k), _t4(v), _t4(o), _t4(dout), _ptr(lse), B, L, Hq, Hkv, d, float(tau), Bq, Bk,
                      _t4(dq), _t4(dk), _t4(dv), _ptr(ws), ws.numel(), _stats_struct(stats), _stream(q))
    _check("mala_bwd", rc)
    return dq, dk, dv


def bwd_varlen_workspace(B, total_q, max_q, max_k, Hq, Hkv, d, Bq=128, Bk=64, device="cuda"):
    n = load_library().mala_bwd_varlen_workspace_size(B, total_q, max_q, max_k, Hq, Hkv, d, Bq, Bk)
    if n == 0:
        raise MalaError("mala_bwd_varlen_workspace_size", MALA_ERR_UNSUPPORTED, "unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mala_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    tau: float = 1.0, Bq: int = 128, Bk: int = 64, dq=None, dk=None, dv=None, ws=None,
                    stats: dict | None = None):
    """Backward of mala_fwd_varlen.  Packed q/o/dout [total_q,Hq,d], k/v
    [total_k,Hkv,d] bf16, lse [Hq,total_q] fp32.  Returns (dq, dk, dv) bf16."""
    _dev_check(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    dev = q.device
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or not c.is_contiguous() or c.dim() != 1 or c.device != dev:
            raise ValueError("cu_seqlens must be contiguous int32 [B + 1] tensors on the device of q")
    B = cu_seqlens_q.numel() - 1
    if B < 1 or cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 entries")
    _expect(k, (Tk, Hkv, d), torch.bfloat16, "k", dev)
    _expect(v, (Tk, Hkv, d), torch.bfloat16, "v", dev)
    _expect(o, (Tq, Hq, d), torch.bfloat16, "o", dev)
    _expect(dout, (Tq, Hq, d), torch.bfloat16, "dout", dev)
    _expect(lse, (Hq, Tq), torch.float32, "lse", dev, True)
    _expect(dq, (Tq, Hq, d), torch.bfloat16, "dq", dev)
    _expect(dk, (Tk, Hkv, d), torch.bfloat16, "dk", dev)
    _expect(dv, (Tk, Hkv, d), torch.bfloat16, "dv", dev)
    _check_stats(stats, B, Hq, Tq, max(1, -(-int(max_seqlen_q) // Bq)), max(1, -(-int(max_seqlen_k) // Bk)), dev,
                 varlen=True)
    _check_ws(ws, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if ws is None:
        ws = bwd_varlen_workspace(B, Tq, max_seqlen_q, max_seqlen_k, Hq, Hkv, d, Bq, Bk, q.device)
    lib = load_library()
    rc = lib.mala_bwd_varlen(_t3(q), _t3(k), _t3(v), _t3(o), _t3(dout), _ptr(lse), _ptr(cu_seqlens_q),
                             _ptr(cu_seqlens_k), B, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, d,
                             float(tau), Bq, Bk, _t3(dq), _t3(dk), _t3(dv), _ptr(ws), ws.numel(),
                             _stats_struct(stats), _stream(q))
    _check("mala_bwd_varlen", rc)
    return dq, dk, dv


def _check_decode(q, kcache, vcache, Bk_dec, o, lse, kept_tiles, decision_bits):
    if q.dim() != 3 or kcache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and the caches [B, N, Hkv, d]")
    B, Hq, d = q.shape
    N, Hkv = kcache.shape[1], kcache.shape[2]
    dev = q.device
    _expect(q, (B, Hq, d), torch.bfloat16, "q", dev, True)
    _expect(kcache, (B, N, Hkv, d), torch.bfloat16, "kcache", dev)
    _expect(vcache, (B, N, Hkv, d), torch.bfloat16, "vcache", dev)
    _expect(o, (B, Hq, d), torch.bfloat16, "o", dev, True)
    _expect(lse, (B, Hq), torch.float32, "lse", dev, True)
    _expect(kept_tiles, (B, Hkv), torch.int32, "kept_tiles", dev, True)
    _expect(decision_bits, (B, Hkv, -(-(-(-N // Bk_dec)) // 32)), torch.int32, "decision_bits", dev, True)
    return B, Hq, d, N, Hkv


def decode_workspace(B, N, Hq, Hkv, d, Bk_dec=64, device="cuda"):
    n = load_library().mala_decode_workspace_size(B, N, Hq, Hkv, d, Bk_dec)
    if n == 0:
        raise MalaError("mala_decode_workspace_size", MALA_ERR_UNSUPPORTED, "unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def mala_decode(q, kcache, vcache, tau: float = 1.0, Bk_dec: int = 64, o=None, lse=None, kept_tiles=None, ws=None,
                decision_bits=None, cache_seqlens=None):
    """Decode one token.  q [B,Hq,d] bf16 contiguous; caches [B,N,Hkv,d] bf16.
    Returns (o [B,Hq,d] bf16, lse [B,Hq] fp32, kept_tiles [B,Hkv] int32).
    decision_bits: optional int32 tensor [B, Hkv, ceil(nT/32)] filled with the
    per-tile keep bits.  cache_seqlens: optional int32 [B] tensor on the same
    device; sequence b then uses only its first cache_seqlens[b] cache rows
    (mala_decode_varlen)."""
    _dev_check(q, kcache, vcache, cache_seqlens)
    B, Hq, d, N, Hkv = _check_decode(q, kcache, vcache, Bk_dec, o, lse, kept_tiles, decision_bits)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    kept_tiles = torch.empty((B, Hkv), dtype=torch.int32, device=q.device) if kept_tiles is None else kept_tiles
    if ws is None:
        ws = decode_workspace(B, N, Hq, Hkv, d, Bk_dec, q.device)
    lib = load_library()
    if cache_seqlens is None:
        rc = lib.mala_decode(_ptr(q), _t4(kcache), _t4(vcache), B, N, Hq, Hkv, d, float(tau), Bk_dec,
                             _ptr(o), _ptr(lse), _ptr(kept_tiles), _ptr(decision_bits), _ptr(ws), ws.numel(),
                             _stream(q))
        _check("mala_decode", rc)
    else:
        _expect(cache_seqlens, (B,), torch.int32, "cache_seqlens", q.device, True)
        rc = lib.mala_decode_varlen(_ptr(q), _t4(kcache), _t4(vcache), _ptr(cache_seqlens), B, N, Hq, Hkv, d,
                                    float(tau), Bk_dec, _ptr(o), _ptr(lse), _ptr(kept_tiles), _ptr(decision_bits),
                                    _ptr(ws), ws.numel(), _stream(q))
        _check("mala_decode_varlen", rc)
    return o, lse, kept_tiles


def mala_decode_noalloc(q, kcache, vcache, tau: float = 1.0, Bk_dec: int = 64, o=None, lse=None, kept_tiles=None,
                        decision_bits=None):
    """mala_decode on the library's fixed per-GPU scratch (no workspace; the
    C call allocates nothing).  Shapes as for mala_decode; the workspace the
    shape needs (decode_workspace_size) must not exceed
    DECODE_NOALLOC_MAX_BYTES.  Calls that overlap in time on one GPU share
    the scratch and race: serialise them."""
    _dev_check(q, kcache, vcache)
    B, Hq, d, N, Hkv = _check_decode(q, kcache, vcache, Bk_dec, o, lse, kept_tiles, decision_bits)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else lse
    kept_tiles = torch.empty((B, Hkv), dtype=torch.int32, device=q.device) if kept_tiles is None else kept_tiles
    rc = load_library().mala_decode_noalloc(_ptr(q), _t4(kcache), _t4(vcache), B, N, Hq, Hkv, d, float(tau), Bk_dec,
                                            _ptr(o), _ptr(lse), _ptr(kept_tiles), _ptr(decision_bits), _stream(q))
    _check("mala_decode_noalloc", rc)
    return o, lse, kept_tiles


def probe_mfma(iters: int, sink: torch.Tensor) -> float:
    """Enqueue the back-to-back bf16 MFMA probe (include/mala.h:
    mala_probe_mfma) on the current stream; returns the launch's FLOP count."""
    _dev_check(sink)
    _expect(sink, (PROBE_SINK_WORDS,), torch.float32, "sink", sink.device, contiguous=True)
    lib = load_library()
    _check("mala_probe_mfma", lib.mala_probe_mfma(int(iters), _ptr(sink), _stream(sink)))
    return float(lib.mala_probe_mfma_flop(int(iters)))


def probe_read(src: torch.Tensor, sink: torch.Tensor) -> int:
    """Enqueue the streaming-read probe (include/mala.h: mala_probe_read) over
    the bytes of a contiguous device tensor; returns the bytes read."""
    _dev_check(src, sink)
    if not src.is_contiguous():
        raise ValueError("probe_read: src must be contiguous")
    _expect(sink, (PROBE_SINK_WORDS,), torch.int32, "sink", src.device, contiguous=True)
    nbytes = src.numel() * src.element_size()
    lib = load_library()
    _check("mala_probe_read", lib.mala_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(src)))
    return nbytes


class MalaAttention(torch.autograd.Function):
    """Autograd wrapper: forward saves (q, k, v, o, lse) only -- no mask."""

    @staticmethod
    def forward(ctx, q, k, v, tau, Bq, Bk):
        o, lse = mala_fwd(q, k, v, tau, Bq, Bk)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (tau, Bq, Bk)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        tau, Bq, Bk = ctx.cfg
        dq, dk, dv = mala_bwd(q, k, v, o, do.contiguous(), lse, tau, Bq, Bk)
        return dq, dk, dv, None, None, None


def mala_attention(q, k, v, tau: float = 1.0, Bq: int = 128, Bk: int = 64):
    return MalaAttention.apply(q, k, v, tau, Bq, Bk)


class MalaAttentionVarlen(torch.autograd.Function):
    """Autograd wrapper of the packed variable-length path: forward saves
    (q, k, v, o, lse) only -- no mask."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, tau, Bq, Bk):
        o, lse = mala_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, tau, Bq, Bk)
        ctx.save_for_backward(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k)
        ctx.cfg = (max_seqlen_q, max_seqlen_k, tau, Bq, Bk)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, cq, ck = ctx.saved_tensors
        max_q, max_k, tau, Bq, Bk = ctx.cfg
        dq, dk, dv = mala_bwd_varlen(q, k, v, o, do.contiguous(), lse, cq, ck, max_q, max_k, tau, Bq, Bk)
        return dq, dk, dv, None, None, None, None, None, None, None


def mala_attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                          tau: float = 1.0, Bq: int = 128, Bk: int = 64):
    return MalaAttentionVarlen.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, tau, Bq, Bk)
