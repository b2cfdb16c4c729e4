"""Thin ctypes binding of libfa.so (include/fa.h).

Argument marshalling only: shapes, dtypes and devices of torch tensors are
checked, raw device pointers and the current HIP stream are passed to the C
entry points, and a non-zero status becomes :class:`FaError`.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.

The functions carry the C names and mirror their argument order; outputs are
caller-allocated tensors.  :func:`attention_fwd` / :func:`attention_bwd`
allocate the outputs for convenience.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_SCRATCH = 0, 1, 2, 3, 4
NOALLOC_MAX_ROWS = 1 << 22  # FA_NOALLOC_MAX_ROWS of include/fa.h
SYMBOLS = ("fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_bwd", "fa_fwd_gqa", "fa_bwd_gqa", "fa_bwd_gqa_bf16grad",
           "fa_fwd_dropout",
           "fa_bwd_dropout", "fa_decode_plan", "fa_decode", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dv",
           "fa_bwd_dk", "fa_bwd_dq", "fa_status_string", "fa_probe_mfma", "fa_probe_hbm_read", "fa_bwd_noalloc")


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


_lib = None


def load_library():
    """Load libfa.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m io_aware_tiled_fwd_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp] * 5 + [i, i, i, i, f, i, vp]
    lib.fa_fwd_f32.argtypes = [vp] * 5 + [i, i, i, i, f, i, vp]
    lib.fa_bwd.argtypes = [vp] * 10 + [i, i, i, i, f, i, vp]
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [i, i, i, i, f, i, vp]
    lib.fa_fwd_gqa.argtypes = [vp] * 5 + [i, i, i, i, i, f, i, vp]
    lib.fa_bwd_gqa.argtypes = [vp] * 10 + [i, i, i, i, i, f, i, vp]
    lib.fa_fwd_fp8.argtypes = [vp] * 5 + [i, i, i, i, i, f, f, f, f, i, vp]
    ull = ctypes.c_ulonglong
    lib.fa_bwd_gqa_bf16grad.argtypes = [vp] * 10 + [i, i, i, i, i, f, i, vp]
    lib.fa_fwd_dropout.argtypes = [vp] * 5 + [i, i, i, i, i, f, i, f, ull, ull, vp]
    lib.fa_bwd_dropout.argtypes = [vp] * 10 + [i, i, i, i, i, f, i, f, ull, ull, vp]
    lib.fa_decode_plan.argtypes = [i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_decode.argtypes = [vp] * 6 + [i, i, i, i, i, f, i, vp, ctypes.c_size_t, vp]
    lib.fa_bwd_preprocess.argtypes = [vp] * 3 + [i, i, i, i, vp]
    lib.fa_bwd_dv.argtypes = [vp] * 5 + [i, i, i, i, f, i, vp]
    lib.fa_bwd_dk.argtypes = [vp] * 7 + [i, i, i, i, f, i, vp]
    lib.fa_bwd_dkdv.argtypes = [vp] * 8 + [i, i, i, i, f, i, vp]
    lib.fa_bwd_dq.argtypes = [vp] * 7 + [i, i, i, i, f, i, vp]
    lib.fa_probe_mfma.argtypes = [i, i, vp, vp]
    lib.fa_probe_hbm_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    for fn in (lib.fa_fwd, lib.fa_fwd_f32, lib.fa_fwd_fp8, lib.fa_fwd_dropout, lib.fa_bwd_dropout,
               lib.fa_bwd_gqa_bf16grad, lib.fa_bwd, lib.fa_fwd_gqa, lib.fa_bwd_gqa, lib.fa_decode_plan,
               lib.fa_decode, lib.fa_bwd_preprocess, lib.fa_bwd_dkdv, lib.fa_bwd_dv, lib.fa_bwd_dk, lib.fa_bwd_dq,
               lib.fa_probe_mfma, lib.fa_probe_hbm_read, lib.fa_bwd_noalloc):
        fn.restype = ctypes.c_int
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def _stream_handle(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _check4(t, name, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")


def _shape(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _default_scale(d):
    return 1.0 / math.sqrt(d)


def fa_fwd(q, k, v, o, lse, causal=False, scale=None, stream=None) -> None:
    """bf16 forward into caller-allocated o (bf16 [B,H,N,d]) and lse (fp32 [B,H,N])."""
    B, H, N, d = _shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    _check4(lse, "lse", torch.float32)
    if tuple(lse.shape) != (B, H, N):
        raise ValueError(f"lse must have shape {(B, H, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, sc,
                               int(bool(causal)), ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")


def fa_fwd_f32(q, k, v, o, lse, causal=False, scale=None, stream=None) -> None:
    """fp32 forward into caller-allocated o (fp32 [B,H,N,d]) and lse (fp32 [B,H,N])."""
    B, H, N, d = _shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    _check4(lse, "lse", torch.float32)
    if tuple(lse.shape) != (B, H, N):
        raise ValueError(f"lse must have shape {(B, H, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, sc,
                                   int(bool(causal)), ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_f32")


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, causal=False, scale=None, stream=None) -> None:
    """bf16 backward into caller-allocated fp32 dq, dk, dv ([B,H,N,d]) and the
    fp32 workspace delta ([B,H,N])."""
    B, H, N, d = _shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    for t, n in ((lse, "lse"), (delta, "delta")):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != (B, H, N):
            raise ValueError(f"{n} must have shape {(B, H, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                               _ptr(dk), _ptr(dv), _ptr(delta), B, H, N, d, sc, int(bool(causal)),
                               ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=False, scale=None, stream=None) -> None:
    """fa_bwd without the delta workspace: the library keeps D in its static
    per-GPU array (B*H*N <= NOALLOC_MAX_ROWS) and allocates nothing."""
    B, H, N, d = _shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    _check4(lse, "lse", torch.float32)
    if tuple(lse.shape) != (B, H, N):
        raise ValueError(f"lse must have shape {(B, H, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                       _ptr(dk), _ptr(dv), B, H, N, d, sc, int(bool(causal)),
                                       ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_noalloc")


def _gqa_shapes(q, k):
    B, Hq, N, d = _shape(q)
    Hkv = int(k.shape[1]) if k.dim() == 4 else -1
    if k.dim() != 4 or tuple(k.shape) != (B, Hkv, N, d) or Hkv < 1 or Hq % Hkv:
        raise ValueError(f"k must be [B, Hkv, N, d] with Hkv dividing Hq={Hq}")
    return B, Hq, Hkv, N, d


def fa_fwd_gqa(q, k, v, o, lse, causal=False, scale=None, stream=None) -> None:
    """Grouped-head bf16 forward: q, o [B,Hq,N,d], k, v [B,Hkv,N,d], lse fp32
    [B,Hq,N]; query head h uses key/value head h // (Hq // Hkv)."""
    B, Hq, Hkv, N, d = _gqa_shapes(q, k)
    for t, n, shp in ((q, "q", (B, Hq, N, d)), (o, "o", (B, Hq, N, d)), (k, "k", (B, Hkv, N, d)),
                      (v, "v", (B, Hkv, N, d))):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    _check4(lse, "lse", torch.float32)
    if tuple(lse.shape) != (B, Hq, N):
        raise ValueError(f"lse must have shape {(B, Hq, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, sc,
                                   int(bool(causal)), ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_gqa")


def fa_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, delta, causal=False, scale=None, stream=None) -> None:
    """Grouped-head bf16 backward into caller-allocated fp32 dq [B,Hq,N,d],
    dk, dv [B,Hkv,N,d] (sums over each group's query heads) and the fp32
    workspace delta [B,Hq,N]."""
    B, Hq, Hkv, N, d = _gqa_shapes(q, k)
    for t, n, shp in ((q, "q", (B, Hq, N, d)), (o, "o", (B, Hq, N, d)), (dout, "dout", (B, Hq, N, d)),
                      (k, "k", (B, Hkv, N, d)), (v, "v", (B, Hkv, N, d))):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    for t, n, shp in ((dq, "dq", (B, Hq, N, d)), (dk, "dk", (B, Hkv, N, d)), (dv, "dv", (B, Hkv, N, d))):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    for t, n in ((lse, "lse"), (delta, "delta")):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != (B, Hq, N):
            raise ValueError(f"{n} must have shape {(B, Hq, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(delta), B, Hq, Hkv, N, d, sc, int(bool(causal)),
                                   ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_gqa")


def _check_bwd_args(q, k, v, dout, lse, delta, outs):
    B, H, N, d = _shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    for t, n in outs:
        _check4(t, n, torch.float32)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    for t, n in ((lse, "lse"), (delta, "delta")):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != (B, H, N):
            raise ValueError(f"{n} must have shape {(B, H, N)}")
    return B, H, N, d


def fa_bwd_preprocess(o, dout, delta, stream=None) -> None:
    """delta = rowsum(dout * o) (fp32 [B,H,N]) from bf16 o and dout."""
    B, H, N, d = _shape(o)
    for t, n in ((o, "o"), (dout, "dout")):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    _check4(delta, "delta", torch.float32)
    if tuple(delta.shape) != (B, H, N):
        raise ValueError(f"delta must have shape {(B, H, N)}")
    st = load_library().fa_bwd_preprocess(_ptr(o), _ptr(dout), _ptr(delta), B, H, N, d,
                                          ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_preprocess")


def fa_bwd_dv(q, k, lse, dout, dv, causal=False, scale=None, stream=None) -> None:
    """dV (fp32) given lse."""
    B, H, N, d = _shape(q)
    for t, n in ((q, "q"), (k, "k"), (dout, "dout")):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{n} must have shape {(B, H, N, d)}")
    _check4(dv, "dv", torch.float32)
    if tuple(dv.shape) != (B, H, N, d):
        raise ValueError(f"dv must have shape {(B, H, N, d)}")
    _check4(lse, "lse", torch.float32)
    if tuple(lse.shape) != (B, H, N):
        raise ValueError(f"lse must have shape {(B, H, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_dv(_ptr(q), _ptr(k), _ptr(lse), _ptr(dout), _ptr(dv), B, H, N, d, sc,
                                  int(bool(causal)), ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dv")


def fa_bwd_dk(q, k, v, lse, dout, delta, dk, causal=False, scale=None, stream=None) -> None:
    """dK (fp32) given lse and delta."""
    B, H, N, d = _check_bwd_args(q, k, v, dout, lse, delta, ((dk, "dk"),))
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_dk(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta),
                                  _ptr(dk), B, H, N, d, sc, int(bool(causal)),
                                  ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dk")


def fa_bwd_dkdv(q, k, v, lse, dout, delta, dk, dv, causal=False, scale=None, stream=None) -> None:
    """dK and dV (fp32) given lse and delta, in one stage."""
    B, H, N, d = _check_bwd_args(q, k, v, dout, lse, delta, ((dk, "dk"), (dv, "dv")))
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta),
                                    _ptr(dk), _ptr(dv), B, H, N, d, sc, int(bool(causal)),
                                    ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, lse, dout, delta, dq, causal=False, scale=None, stream=None) -> None:
    """dQ (fp32) given lse and delta."""
    B, H, N, d = _check_bwd_args(q, k, v, dout, lse, delta, ((dq, "dq"),))
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta),
                                  _ptr(dq), B, H, N, d, sc, int(bool(causal)),
                                  ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dq")


def attention_fwd(q, k, v, causal=False, scale=None, stream=None):
    """Allocating wrapper: returns (o, lse).  bf16 or fp32 inputs; bf16 k, v
    with fewer heads than q select the grouped-head entry point."""
    B, H, N, d = _shape(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if q.dtype == torch.float32:
        fa_fwd_f32(q, k, v, o, lse, causal, scale, stream)
    elif k.dim() == 4 and k.shape[1] != H:
        fa_fwd_gqa(q, k, v, o, lse, causal, scale, stream)
    else:
        fa_fwd(q, k, v, o, lse, causal, scale, stream)
    return o, lse


def attention_bwd(q, k, v, o, lse, dout, causal=False, scale=None, stream=None):
    """Allocating wrapper: returns (dq, dk, dv) in fp32 (dk, dv shaped like k)."""
    B, H, N, d = _shape(q)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty(tuple(k.shape), dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if k.dim() == 4 and k.shape[1] != H:
        fa_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, delta, causal, scale, stream)
    else:
        fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, causal, scale, stream)
    return dq, dk, dv


def fa_decode_plan(B, Hq, Hkv, Nk, d, num_splits=0):
    """(effective split count, workspace bytes) of a decode call."""
    sp, ws = ctypes.c_int(0), ctypes.c_size_t(0)
    st = load_library().fa_decode_plan(int(B), int(Hq), int(Hkv), int(Nk), int(d), int(num_splits),
                                       ctypes.byref(sp), ctypes.byref(ws))
    if st != FA_OK:
        raise FaError(st, "fa_decode_plan")
    return sp.value, ws.value


def _decode_shapes(q, k):
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("decode expects q [B, Hq, d] and k, v [B, Hkv, Nk, d]")
    B, Hq, d = (int(x) for x in q.shape)
    Hkv, Nk = int(k.shape[1]), int(k.shape[2])
    if tuple(k.shape) != (B, Hkv, Nk, d) or Hkv < 1 or Hq % Hkv:
        raise ValueError(f"k must be [B, Hkv, Nk, d] with Hkv dividing Hq={Hq}")
    return B, Hq, Hkv, Nk, d


def fa_decode(q, k, v, o, lse, kv_len=None, num_splits=0, workspace=None, scale=None, stream=None) -> None:
    """Split-KV decode into caller-allocated o (bf16 [B,Hq,d]) and lse (fp32
    [B,Hq]).  q bf16 [B,Hq,d]; k, v bf16 [B,Hkv,Nk,d]; kv_len int32 [B] on the
    device or None; workspace a device tensor of at least the bytes
    fa_decode_plan reports (None when that is 0)."""
    B, Hq, Hkv, Nk, d = _decode_shapes(q, k)
    for t, n, shp in ((q, "q", (B, Hq, d)), (o, "o", (B, Hq, d)), (k, "k", (B, Hkv, Nk, d)),
                      (v, "v", (B, Hkv, Nk, d))):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    _check4(lse, "lse", torch.float32)
    if tuple(lse.shape) != (B, Hq):
        raise ValueError(f"lse must have shape {(B, Hq)}")
    if kv_len is not None:
        _check4(kv_len, "kv_len", torch.int32)
        if tuple(kv_len.shape) != (B,):
            raise ValueError(f"kv_len must have shape {(B,)}")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_len) if kv_len is not None else None,
                                  _ptr(o), _ptr(lse), B, Hq, Hkv, Nk, d, sc, int(num_splits), ws_ptr, ws_bytes,
                                  ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_decode")


def attention_decode(q, k, v, kv_len=None, num_splits=0, scale=None, stream=None):
    """Allocating wrapper of fa_decode: returns (o, lse); the workspace is a
    torch allocation sized by fa_decode_plan."""
    B, Hq, Hkv, Nk, d = _decode_shapes(q, k)
    _, ws_bytes = fa_decode_plan(B, Hq, Hkv, Nk, d, num_splits)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=q.device) if ws_bytes else None
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    fa_decode(q, k, v, o, lse, kv_len=kv_len, num_splits=num_splits, workspace=ws, scale=scale, stream=stream)
    return o, lse


_FP8_DTYPES = tuple(t for t in (torch.uint8, getattr(torch, "float8_e4m3fn", None)) if t is not None)


def fa_fwd_fp8(q, k, v, o, lse, q_descale, k_descale, v_descale, causal=False, scale=None, stream=None) -> None:
    """fp8 forward: q [B,Hq,N,d], k, v [B,Hkv,N,d] holding OCP e4m3 bytes
    (torch.float8_e4m3fn or torch.uint8), real inputs = descale * stored value;
    into caller-allocated o (bf16 [B,Hq,N,d]) and lse (fp32 [B,Hq,N])."""
    B, Hq, Hkv, N, d = _gqa_shapes(q, k)
    for t, n, shp in ((q, "q", (B, Hq, N, d)), (k, "k", (B, Hkv, N, d)), (v, "v", (B, Hkv, N, d))):
        if not isinstance(t, torch.Tensor) or t.dtype not in _FP8_DTYPES:
            raise TypeError(f"{n} must be a float8_e4m3fn or uint8 tensor")
        _check4(t, n, t.dtype)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    _check4(o, "o", torch.bfloat16)
    if tuple(o.shape) != (B, Hq, N, d):
        raise ValueError(f"o must have shape {(B, Hq, N, d)}")
    _check4(lse, "lse", torch.float32)
    if tuple(lse.shape) != (B, Hq, N):
        raise ValueError(f"lse must have shape {(B, Hq, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, sc,
                                   float(q_descale), float(k_descale), float(v_descale), int(bool(causal)),
                                   ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")


def attention_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, causal=False, scale=None, stream=None):
    """Allocating wrapper of fa_fwd_fp8: returns (o bf16, lse fp32)."""
    B, Hq, N, d = _shape(q)
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q, k, v, o, lse, q_descale, k_descale, v_descale, causal=causal, scale=scale, stream=stream)
    return o, lse


def _check_gqa_fwd_args(q, k, v, o, lse):
    B, Hq, Hkv, N, d = _gqa_shapes(q, k)
    for t, n, shp in ((q, "q", (B, Hq, N, d)), (o, "o", (B, Hq, N, d)), (k, "k", (B, Hkv, N, d)),
                      (v, "v", (B, Hkv, N, d))):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    _check4(lse, "lse", torch.float32)
    if tuple(lse.shape) != (B, Hq, N):
        raise ValueError(f"lse must have shape {(B, Hq, N)}")
    return B, Hq, Hkv, N, d


def fa_fwd_dropout(q, k, v, o, lse, dropout_p, seed, offset=0, causal=False, scale=None, stream=None) -> None:
    """bf16 forward with attention dropout (shapes as fa_fwd_gqa): probabilities
    are dropped with the Philox mask of (seed, offset), kept ones rescaled;
    lse is that of the undropped scores."""
    B, Hq, Hkv, N, d = _check_gqa_fwd_args(q, k, v, o, lse)
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, sc,
                                       int(bool(causal)), float(dropout_p), int(seed), int(offset),
                                       ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_dropout")


def fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, delta, dropout_p, seed, offset=0, causal=False, scale=None,
                   stream=None) -> None:
    """Backward of fa_fwd_dropout (same seed and offset), shapes as fa_bwd_gqa."""
    B, Hq, Hkv, N, d = _gqa_shapes(q, k)
    for t, n, shp in ((q, "q", (B, Hq, N, d)), (o, "o", (B, Hq, N, d)), (dout, "dout", (B, Hq, N, d)),
                      (k, "k", (B, Hkv, N, d)), (v, "v", (B, Hkv, N, d))):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    for t, n, shp in ((dq, "dq", (B, Hq, N, d)), (dk, "dk", (B, Hkv, N, d)), (dv, "dv", (B, Hkv, N, d))):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    for t, n in ((lse, "lse"), (delta, "delta")):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != (B, Hq, N):
            raise ValueError(f"{n} must have shape {(B, Hq, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _ptr(delta), B, Hq, Hkv, N, d, sc, int(bool(causal)),
                                       float(dropout_p), int(seed), int(offset),
                                       ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dropout")


def attention_fwd_dropout(q, k, v, dropout_p, seed, offset=0, causal=False, scale=None, stream=None):
    """Allocating wrapper of fa_fwd_dropout: returns (o, lse)."""
    B, Hq, N, d = _shape(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    fa_fwd_dropout(q, k, v, o, lse, dropout_p, seed, offset, causal=causal, scale=scale, stream=stream)
    return o, lse


def attention_bwd_dropout(q, k, v, o, lse, dout, dropout_p, seed, offset=0, causal=False, scale=None, stream=None):
    """Allocating wrapper of fa_bwd_dropout: returns (dq, dk, dv) in fp32."""
    B, Hq, N, d = _shape(q)
    dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty(tuple(k.shape), dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    delta = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, delta, dropout_p, seed, offset, causal=causal, scale=scale,
                   stream=stream)
    return dq, dk, dv


def fa_bwd_gqa_bf16grad(q, k, v, o, lse, dout, dq, dk, dv, delta, causal=False, scale=None, stream=None) -> None:
    """fa_bwd_gqa with bf16 dq [B,Hq,N,d] and dk, dv [B,Hkv,N,d]."""
    B, Hq, Hkv, N, d = _gqa_shapes(q, k)
    for t, n, shp in ((q, "q", (B, Hq, N, d)), (o, "o", (B, Hq, N, d)), (dout, "dout", (B, Hq, N, d)),
                      (k, "k", (B, Hkv, N, d)), (v, "v", (B, Hkv, N, d)), (dq, "dq", (B, Hq, N, d)),
                      (dk, "dk", (B, Hkv, N, d)), (dv, "dv", (B, Hkv, N, d))):
        _check4(t, n, torch.bfloat16)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    for t, n in ((lse, "lse"), (delta, "delta")):
        _check4(t, n, torch.float32)
        if tuple(t.shape) != (B, Hq, N):
            raise ValueError(f"{n} must have shape {(B, Hq, N)}")
    sc = _default_scale(d) if scale is None else float(scale)
    st = load_library().fa_bwd_gqa_bf16grad(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                            _ptr(dk), _ptr(dv), _ptr(delta), B, Hq, Hkv, N, d, sc, int(bool(causal)),
                                            ctypes.c_void_p(_stream_handle(stream)))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_gqa_bf16grad")


# Measurement probes (include/fa_probe.h): not part of the attention method.
PROBE_READ_UNIT = 16 * 512 * 256 * 4  # fa_probe_hbm_read sizes are multiples of this (8 MiB)


def fa_probe_mfma(blocks, iters, sink, stream=None) -> None:
    """bf16 MFMA throughput loop: blocks * 8 * iters * 16 * 32768 FLOP; sink
    fp32 [blocks * 512] on the GPU (written, values meaningless)."""
    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() < blocks * 512:
        raise ValueError("sink must be a CUDA float32 tensor of at least blocks * 512 elements")
    st = load_library().fa_probe_mfma(blocks, iters, _ptr(sink), _stream_handle(stream))
    if st:
        raise FaError(st, "fa_probe_mfma")


def fa_probe_hbm_read(buf, sink, stream=None) -> None:
    """Non-temporal read sweep over the bytes of buf (a multiple of
    PROBE_READ_UNIT); sink int32 [256 * 512] on the GPU."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_cuda or not sink.is_cuda or sink.numel() < 256 * 512 or sink.element_size() != 4:
        raise ValueError("buf and sink must be CUDA tensors; sink of at least 256 * 512 4-byte elements")
    st = load_library().fa_probe_hbm_read(_ptr(buf), nbytes, _ptr(sink), _stream_handle(stream))
    if st:
        raise FaError(st, "fa_probe_hbm_read")
