"""fp64 CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and the
two share no code: the oracle is plain C (``oracle.c``) compiled with gcc.

Functions take and return numpy float64 arrays laid out ``[BH, N, d]``
(``[BH, N]`` for the logsumexp and D), C-contiguous.

* :func:`attn_fwd` -- the plain definition of softmax attention (per head,
  P = softmax(scale Q K^T), O = P V, L = natural-log logsumexp of the scaled
  scores), as on the "FlashAttention" deep-dive page, section "How it works".
* :func:`attn_bwd` -- its analytic gradients (same page and section: D =
  rowsum(dO * O), dS = P * (dP - D), then dQ, dK, dV).
* :func:`attn_fwd_gqa`, :func:`attn_bwd_gqa` -- the same with grouped heads
  (GQA/MQA: several query heads share one key/value head; same page,
  "Implementation notes"), gradients of shared K, V summed over the group.
* :func:`attn_decode` -- one query row per (batch, query head) against a
  key/value cache of which the first ``kv_len[b]`` keys are visible (the
  single-query decode of the deep-dive page, "Implementation notes"); the plain
  definition again.
* :func:`attn_fwd_dropout`, :func:`attn_bwd_dropout`,
  :func:`attn_fwd_rows_dropout` -- the same with dropout of the attention
  probabilities, the mask drawn from Philox4x32-10 by seed and offset (same
  page, "Implementation notes"); :func:`dropout_mask` and
  :func:`dropout_bytes` expose the mask and the generator's bytes, and
  :func:`philox4x32_10` the generator itself (pinned to the known-answer
  vectors published with the generator's reference implementation).
* :func:`attn_fwd_rows` -- the plain forward for listed query rows only.
* :func:`attn_fwd_tiled` -- a tiled forward: each key block reduced to a
  per-row summary, summaries folded with the online-softmax rescaling rule of
  that page, one division at the end; used only to show tiled == untiled.  It
  can trace the running (m, l, acc) of one row, which the worked example on
  the "Flash Attention and Memory-Efficient Attention Variants" page prints.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (plain C11, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
             "-o", tmp, _SRC, "-lm", "-lpthread"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_attn_fwd.argtypes = [_f64p] * 5 + [_i64, _i64, _i64, ctypes.c_double,
                                                      ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_bwd.argtypes = [_f64p] * 8 + [_i64, _i64, _i64, ctypes.c_double,
                                                      ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_fwd_tiled.argtypes = [_f64p] * 5 + [_i64, _i64, _i64, ctypes.c_double,
                                                            ctypes.c_int, _i64, _i64, _i64, _f64p]
        lib.oracle_attn_fwd_rows.argtypes = [_f64p] * 3 + [ctypes.POINTER(_i64), _i64, _f64p, _f64p,
                                                           _i64, _i64, _i64, ctypes.c_double,
                                                           ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_fwd_gqa.argtypes = [_f64p] * 5 + [_i64] * 5 + [ctypes.c_double, ctypes.c_int,
                                                                     ctypes.c_int]
        lib.oracle_attn_bwd_gqa.argtypes = [_f64p] * 8 + [_i64] * 5 + [ctypes.c_double, ctypes.c_int,
                                                                     ctypes.c_int]
        lib.oracle_attn_decode.argtypes = [_f64p] * 3 + [ctypes.POINTER(_i64), _f64p, _f64p] + [_i64] * 5 + [
            ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_decode.restype = ctypes.c_int
        u64, u8p = ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint8)
        lib.oracle_attn_fwd_dropout.argtypes = [_f64p] * 5 + [_i64] * 5 + [ctypes.c_double, ctypes.c_int,
                                                                         ctypes.c_double, u64, u64, ctypes.c_int]
        lib.oracle_attn_bwd_dropout.argtypes = [_f64p] * 8 + [_i64] * 5 + [ctypes.c_double, ctypes.c_int,
                                                                         ctypes.c_double, u64, u64, ctypes.c_int]
        lib.oracle_attn_fwd_rows_dropout.argtypes = [_f64p] * 3 + [ctypes.POINTER(_i64), _i64, _f64p, _f64p,
                                                                   _i64, _i64, _i64, ctypes.c_double, ctypes.c_int,
                                                                   ctypes.c_double, u64, u64, ctypes.c_int]
        lib.oracle_dropout_mask.argtypes = [u8p, _i64, _i64, ctypes.c_double, u64, u64]
        lib.oracle_dropout_bytes.argtypes = [u8p, _i64, _i64, u64, u64]
        u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
        lib.oracle_philox4x32_10.restype = ctypes.c_int
        for fn in (lib.oracle_attn_fwd_dropout, lib.oracle_attn_bwd_dropout, lib.oracle_attn_fwd_rows_dropout,
                   lib.oracle_dropout_mask, lib.oracle_dropout_bytes):
            fn.restype = ctypes.c_int
        lib.oracle_attn_fwd_gqa.restype = ctypes.c_int
        lib.oracle_attn_bwd_gqa.restype = ctypes.c_int
        lib.oracle_default_threads.argtypes = []
        for fn in (lib.oracle_attn_fwd, lib.oracle_attn_bwd, lib.oracle_attn_fwd_tiled,
                   lib.oracle_attn_fwd_rows, lib.oracle_default_threads):
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Threads the oracle uses by default: the CPUs this process may run on,
    capped by OMP_NUM_THREADS when that is set (a share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _threads(threads):
    return int(threads) if threads and threads > 0 else default_threads()


def _as3(x, name):
    a = np.ascontiguousarray(x, dtype=np.float64)
    if a.ndim == 2:
        a = a[None]
    if a.ndim != 3:
        raise ValueError(f"{name} must be [BH, N, d] or [N, d]")
    return a


def _ptr(a):
    return a.ctypes.data_as(_f64p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def attn_fwd(q, k, v, scale, causal=False, threads=0):
    """Returns (O [BH,N,d], L [BH,N]) in fp64."""
    q, k, v = _as3(q, "q"), _as3(k, "k"), _as3(v, "v")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have one shape")
    BH, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((BH, N), dtype=np.float64)
    _check(_load().oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), BH, N, d,
                                   float(scale), int(bool(causal)), _threads(threads)), "oracle_attn_fwd")
    return o, lse


def attn_bwd(q, k, v, dout, scale, causal=False, threads=0):
    """Returns (dQ, dK, dV, D) in fp64, where D = rowsum(dO * O) with the
    oracle's own O."""
    q, k, v, dout = (_as3(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")))
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout must have one shape")
    BH, N, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    delta = np.empty((BH, N), dtype=np.float64)
    _check(_load().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _ptr(delta), BH, N, d, float(scale),
                                   int(bool(causal)), _threads(threads)), "oracle_attn_bwd")
    return dq, dk, dv, delta


def _as4(x, name):
    a = np.ascontiguousarray(x, dtype=np.float64)
    if a.ndim != 4:
        raise ValueError(f"{name} must be [B, H, N, d]")
    return a


def attn_fwd_gqa(q, k, v, scale, causal=False, threads=0):
    """Grouped-head forward: q [B, Hq, N, d], k, v [B, Hkv, N, d] with Hq a
    multiple of Hkv; query head h uses key/value head h // (Hq // Hkv).
    Returns (O [B, Hq, N, d], L [B, Hq, N]) in fp64."""
    q, k, v = _as4(q, "q"), _as4(k, "k"), _as4(v, "v")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != (N, d) or Hq % Hkv:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing Hq")
    o = np.empty_like(q)
    lse = np.empty((B, Hq, N), dtype=np.float64)
    _check(_load().oracle_attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                                       float(scale), int(bool(causal)), _threads(threads)),
           "oracle_attn_fwd_gqa")
    return o, lse


def attn_bwd_gqa(q, k, v, dout, scale, causal=False, threads=0):
    """Grouped-head backward.  Returns (dQ [B, Hq, N, d], dK, dV [B, Hkv, N, d],
    D [B, Hq, N]); dK, dV sum over the query heads sharing each key/value head."""
    q, k, v, dout = _as4(q, "q"), _as4(k, "k"), _as4(v, "v"), _as4(dout, "dout")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if dout.shape != q.shape or k.shape != v.shape or k.shape[0] != B or k.shape[2:] != (N, d) or Hq % Hkv:
        raise ValueError("bad shapes for the grouped-head backward")
    dq = np.empty_like(q)
    dk, dv = np.empty_like(k), np.empty_like(k)
    delta = np.empty((B, Hq, N), dtype=np.float64)
    _check(_load().oracle_attn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                       _ptr(delta), B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
                                       _threads(threads)), "oracle_attn_bwd_gqa")
    return dq, dk, dv, delta


def attn_decode(q, k, v, scale, kv_len=None, threads=0):
    """Decode: q [B, Hq, d] (one query row per head), k, v [B, Hkv, Nk, d],
    Hkv dividing Hq; batch b sees keys j < kv_len[b] (all Nk when kv_len is
    None).  Returns (O [B, Hq, d], L [B, Hq]) in fp64."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k, v = _as4(k, "k"), _as4(v, "v")
    if q.ndim != 3:
        raise ValueError("q must be [B, Hq, d]")
    B, Hq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d or Hq % Hkv:
        raise ValueError("k, v must be [B, Hkv, Nk, d] with Hkv dividing Hq")
    lens = None
    if kv_len is not None:
        lens = np.ascontiguousarray(kv_len, dtype=np.int64)
        if lens.shape != (B,):
            raise ValueError("kv_len must have one entry per batch")
    o = np.empty_like(q)
    lse = np.empty((B, Hq), dtype=np.float64)
    _check(_load().oracle_attn_decode(_ptr(q), _ptr(k), _ptr(v),
                                      lens.ctypes.data_as(ctypes.POINTER(_i64)) if lens is not None else None,
                                      _ptr(o), _ptr(lse), B, Hq, Hkv, Nk, d, float(scale), _threads(threads)),
           "oracle_attn_decode")
    return o, lse


def dropout_threshold(p):
    """(thr, keep_scale): bytes below thr = floor(256 p + 1/2) (at most 255)
    are dropped; kept probabilities are scaled by 256 / (256 - thr)."""
    thr = min(255, int(np.floor(256.0 * float(p) + 0.5)))
    return thr, 256.0 / (256.0 - thr)


def _u8p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def dropout_mask(BH, N, p, seed, offset=0):
    """Keep mask [BH, N, N] (uint8: 1 kept) of flat query heads, rows, keys."""
    m = np.empty((BH, N, N), dtype=np.uint8)
    _check(_load().oracle_dropout_mask(_u8p(m), BH, N, float(p), int(seed), int(offset)), "oracle_dropout_mask")
    return m


def dropout_bytes(BH, N, seed, offset=0):
    """The Philox bytes [BH, N, N] the keep decisions compare with thr."""
    b = np.empty((BH, N, N), dtype=np.uint8)
    _check(_load().oracle_dropout_bytes(_u8p(b), BH, N, int(seed), int(offset)), "oracle_dropout_bytes")
    return b


def attn_fwd_dropout(q, k, v, scale, causal, p, seed, offset=0, threads=0):
    """Grouped-head forward (shapes as attn_fwd_gqa) with dropout p of the
    attention probabilities; L is that of the undropped scores."""
    q, k, v = _as4(q, "q"), _as4(k, "k"), _as4(v, "v")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != (N, d) or Hq % Hkv:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing Hq")
    o = np.empty_like(q)
    lse = np.empty((B, Hq, N), dtype=np.float64)
    _check(_load().oracle_attn_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                                           float(scale), int(bool(causal)), float(p), int(seed), int(offset),
                                           _threads(threads)), "oracle_attn_fwd_dropout")
    return o, lse


def attn_bwd_dropout(q, k, v, dout, scale, causal, p, seed, offset=0, threads=0):
    """Grouped-head backward with dropout p (the forward's mask).  Returns
    (dQ, dK, dV, D) like attn_bwd_gqa."""
    q, k, v, dout = _as4(q, "q"), _as4(k, "k"), _as4(v, "v"), _as4(dout, "dout")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if dout.shape != q.shape or k.shape != v.shape or k.shape[0] != B or k.shape[2:] != (N, d) or Hq % Hkv:
        raise ValueError("bad shapes for the grouped-head backward")
    dq = np.empty_like(q)
    dk, dv = np.empty_like(k), np.empty_like(k)
    delta = np.empty((B, Hq, N), dtype=np.float64)
    _check(_load().oracle_attn_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                           _ptr(delta), B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
                                           float(p), int(seed), int(offset), _threads(threads)),
           "oracle_attn_bwd_dropout")
    return dq, dk, dv, delta


def attn_fwd_rows_dropout(q, k, v, rows, scale, causal, p, seed, offset=0, threads=0):
    """attn_fwd_rows with dropout p ([BH, N, d] inputs, one key/value head per
    query head)."""
    q, k, v = _as3(q, "q"), _as3(k, "k"), _as3(v, "v")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have one shape")
    BH, N, d = q.shape
    idx = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((idx.size, d), dtype=np.float64)
    lse = np.empty(idx.size, dtype=np.float64)
    _check(_load().oracle_attn_fwd_rows_dropout(_ptr(q), _ptr(k), _ptr(v),
                                                idx.ctypes.data_as(ctypes.POINTER(_i64)), idx.size, _ptr(o),
                                                _ptr(lse), BH, N, d, float(scale), int(bool(causal)), float(p),
                                                int(seed), int(offset), _threads(threads)),
           "oracle_attn_fwd_rows_dropout")
    return o, lse


def attn_fwd_tiled(q, k, v, scale, causal=False, br=64, bc=64, trace_row=None):
    """Tiled online-softmax forward.  Returns (O, L) or, when ``trace_row`` is
    given, (O, L, trace) with trace[blk] = [m, l, acc_0 .. acc_{d-1}] of that
    row of head 0 after key block ``blk``."""
    q, k, v = _as3(q, "q"), _as3(k, "k"), _as3(v, "v")
    BH, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((BH, N), dtype=np.float64)
    nblk = -(-N // int(bc))
    trace = np.full((nblk, 2 + d), np.nan) if trace_row is not None else None
    _check(_load().oracle_attn_fwd_tiled(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), BH, N, d, float(scale),
        int(bool(causal)), int(br), int(bc), -1 if trace_row is None else int(trace_row),
        _ptr(trace) if trace is not None else None), "oracle_attn_fwd_tiled")
    return (o, lse) if trace is None else (o, lse, trace)


def attn_fwd_rows(q, k, v, rows, scale, causal=False, threads=0):
    """Forward for listed query rows only.  ``rows`` are flat indices
    bh * N + i into the [BH, N] row space.  Returns (O [len(rows), d],
    L [len(rows)])."""
    q, k, v = _as3(q, "q"), _as3(k, "k"), _as3(v, "v")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have one shape")
    BH, N, d = q.shape
    idx = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((idx.size, d), dtype=np.float64)
    lse = np.empty(idx.size, dtype=np.float64)
    _check(_load().oracle_attn_fwd_rows(_ptr(q), _ptr(k), _ptr(v),
                                        idx.ctypes.data_as(ctypes.POINTER(_i64)), idx.size,
                                        _ptr(o), _ptr(lse), BH, N, d, float(scale),
                                        int(bool(causal)), _threads(threads)),
           "oracle_attn_fwd_rows")
    return o, lse


def philox4x32_10(counter, key):
    """Philox4x32-10 of four 32-bit counter words and two key words (Salmon,
    Moraes, Dror and Shaw, SC 2011), the generator of the dropout mask.
    Returns the four output words as Python ints."""
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in counter])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (ctypes.c_uint32 * 4)()
    _check(_load().oracle_philox4x32_10(c, k, out), "oracle_philox4x32_10")
    return [int(x) for x in out]
