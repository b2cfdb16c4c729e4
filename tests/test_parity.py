"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Same seeded inputs on both sides; the oracle reads the exact fp64 widening of
the values the GPU receives.  Bars: fp32 O and L max-abs <= 1e-4; bf16 O and
fp32-out gradients max-abs <= 2e-2, L <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_fwd_amd import binding, inputs
from gpu_util import (TOL_BF16_GRAD, TOL_BF16_L, TOL_BF16_O, TOL_F32_L, TOL_F32_O, bf16_from_f64,
                      f64, maxabs, to_dev, upload)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _fwd(dev, causal, scale):
    return binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)


def _check_fwd(o, lse, ref_o, ref_l, tol_o, tol_l, what):
    eo, el = maxabs(o, ref_o), maxabs(lse, ref_l)
    _say(f"{what}: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= tol_o, f"{what}: O error {eo}"
    assert el <= tol_l, f"{what}: L error {el}"


def _check_invariants(dk, dv, dout, what):
    """On every head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, exact for the
    exact gradients.  The kernels round P and dS to bf16 (relative 2^-9) and
    take D from the bf16 O; the resulting per-key errors, of RMS about 1e-3 at
    these shapes, are independent across keys, so over N <= 8192 keys the sums
    stay near sqrt(N) * 1e-3 <= 0.09.  The bar is 0.1."""
    sdk = dk.double().sum(2).abs().max().item()
    sdv = (dv.double().sum(2) - dout.double().sum(2)).abs().max().item()
    _say(f"{what} invariants all heads: max|sum dK|={sdk:.3e} max|sum dV - sum dO|={sdv:.3e}")
    assert sdk <= 0.1 and sdv <= 0.1


# --- the five workloads ------------------------------------------------------

def test_c1_fp32_single_head():
    w = inputs.WORKLOADS["c1_f32_n256_d64"]
    ts = inputs.normal_qkv(w["B"], w["H"], w["N"], w["d"], w["seed"], dtype="f32")
    scale = inputs.default_scale(w["d"])
    _say("c1: fp32 B1 H1 N256 d64")
    o, lse = _fwd(upload(ts), False, scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attn_fwd(*(ts.f64[n].reshape(-1, w["N"], w["d"]) for n in "qkv"), scale)
    _check_fwd(f64(o).reshape(ref_o.shape), f64(lse).reshape(ref_l.shape), ref_o, ref_l, TOL_F32_O,
               TOL_F32_L, "c1")


def test_c2_bf16_all_heads():
    w = inputs.WORKLOADS["c2_bf16_n2048_d64"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    ts = inputs.normal_qkv(B, H, N, d, w["seed"])
    scale = inputs.default_scale(d)
    _say("c2: bf16 B4 H16 N2048 d64")
    o, lse = _fwd(upload(ts), False, scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attn_fwd(*(ts.f64[n].reshape(-1, N, d) for n in "qkv"), scale)
    _check_fwd(f64(o).reshape(ref_o.shape), f64(lse).reshape(ref_l.shape), ref_o, ref_l, TOL_BF16_O,
               TOL_BF16_L, "c2")


def test_c3_causal_sampled_heads():
    w = inputs.WORKLOADS["c3_bf16_causal_n8192_d128"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    ts = inputs.normal_qkv(B, H, N, d, w["seed"])
    scale = inputs.default_scale(d)
    _say("c3: bf16 causal B2 H32 N8192 d128")
    dev = upload(ts)
    o, lse = _fwd(dev, True, scale)
    torch.cuda.synchronize()
    heads = inputs.sample_heads(B * H, 4, w["seed"] + 1000)
    of, lf = f64(o).reshape(B * H, N, d), f64(lse).reshape(B * H, N)
    qkv = [ts.f64[n].reshape(B * H, N, d) for n in "qkv"]
    ref_o, ref_l = oracle.attn_fwd(*(x[heads] for x in qkv), scale, causal=True)
    _check_fwd(of[heads], lf[heads], ref_o, ref_l, TOL_BF16_O, TOL_BF16_L, f"c3 heads {heads}")
    # every head: causal row 0 is V row 0 bitwise, and L_0 = scale q_0 . k_0
    assert torch.equal(o[:, :, 0, :], dev["v"][:, :, 0, :])
    l0 = scale * np.sum(qkv[0][:, 0] * qkv[1][:, 0], -1)
    assert maxabs(lf[:, 0], l0) <= TOL_BF16_L


def test_c4_ragged_sampled_heads():
    """Workload 4 (N = 18000, not a multiple of any tile): four sampled heads,
    every row, against the oracle."""
    w = inputs.WORKLOADS["c4_bf16_n18000_d128"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    ts = inputs.normal_qkv(B, H, N, d, w["seed"])
    scale = inputs.default_scale(d)
    _say("c4: bf16 B1 H16 N18000 d128 (ragged)")
    o, lse = _fwd(upload(ts), False, scale)
    torch.cuda.synchronize()
    heads = inputs.sample_heads(B * H, 4, w["seed"] + 1000)
    qkv = [ts.f64[n].reshape(B * H, N, d) for n in "qkv"]
    ref_o, ref_l = oracle.attn_fwd(*(x[heads] for x in qkv), scale)
    _check_fwd(f64(o).reshape(B * H, N, d)[heads], f64(lse).reshape(B * H, N)[heads], ref_o, ref_l, TOL_BF16_O,
               TOL_BF16_L, f"c4 heads {heads}, all {N} rows")


def test_c3_causal_bwd_bench_shape_sampled_heads():
    """The benchmark's step at its full size (B2 H32 N8192 d128, causal, the same
    seeded inputs): the backward through fa_bwd (preprocess, the paired dK/dV
    kernel, dQ), every gradient of four sampled heads against the oracle; on
    every head the paired kernel's dK and dV agree with those of the two
    one-gradient kernels (fa_bwd_dk, fa_bwd_dv), which compute P themselves, to
    within rounding (_paired_close), so a P hand-over error on any head would
    show; and the column-sum invariants."""
    w = inputs.WORKLOADS["c3_bf16_causal_n8192_d128"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    ts = inputs.normal_qkv(B, H, N, d, w["seed"], with_dout=True)
    scale = inputs.default_scale(d)
    _say("c3 bwd: bf16 causal B2 H32 N8192 d128")
    dev = upload(ts)
    o, lse = _fwd(dev, True, scale)
    dq, dk, dv = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=True,
                                       scale=scale)
    torch.cuda.synchronize()
    delta = torch.empty_like(lse)
    sk, sv = torch.full_like(dk, float("nan")), torch.full_like(dv, float("nan"))
    binding.fa_bwd_preprocess(o, dev["do"], delta)
    binding.fa_bwd_dk(dev["q"], dev["k"], dev["v"], lse, dev["do"], delta, sk, True, scale)
    binding.fa_bwd_dv(dev["q"], dev["k"], lse, dev["do"], sv, True, scale)
    torch.cuda.synchronize()
    _paired_close(sk, dk, "c3 dk")
    _paired_close(sv, dv, "c3 dv")
    del sk, sv
    heads = inputs.sample_heads(B * H, 4, w["seed"] + 2000)
    arr = {n: ts.f64[n].reshape(B * H, N, d) for n in ("q", "k", "v", "do")}
    rq, rk, rv, _ = oracle.attn_bwd(*(arr[n][heads] for n in ("q", "k", "v", "do")), scale, causal=True)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = maxabs(f64(got).reshape(B * H, N, d)[heads], ref)
        _say(f"c3 bwd heads {heads}: max|d{name}|={e:.3e}")
        assert e <= TOL_BF16_GRAD, f"{name} error {e}"
    _check_invariants(dk, dv, dev["do"], "c3 bwd")


def test_c5_causal_fwd_bwd_sampled_heads():
    w = inputs.WORKLOADS["c5_bf16_causal_fwdbwd_n4096_d128"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    ts = inputs.normal_qkv(B, H, N, d, w["seed"], with_dout=True)
    scale = inputs.default_scale(d)
    _say("c5: bf16 causal fwd+bwd B4 H16 N4096 d128")
    dev = upload(ts)
    o, lse = _fwd(dev, True, scale)
    dq, dk, dv = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=True,
                                       scale=scale)
    torch.cuda.synchronize()
    heads = inputs.sample_heads(B * H, 4, w["seed"] + 1000)
    arr = {n: ts.f64[n].reshape(B * H, N, d) for n in ("q", "k", "v", "do")}
    ref_o, ref_l = oracle.attn_fwd(*(arr[n][heads] for n in "qkv"), scale, causal=True)
    _check_fwd(f64(o).reshape(B * H, N, d)[heads], f64(lse).reshape(B * H, N)[heads], ref_o, ref_l,
               TOL_BF16_O, TOL_BF16_L, f"c5 fwd heads {heads}")
    rq, rk, rv, _ = oracle.attn_bwd(*(arr[n][heads] for n in ("q", "k", "v", "do")), scale, causal=True)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = maxabs(f64(got).reshape(B * H, N, d)[heads], ref)
        _say(f"c5 bwd heads {heads}: max|d{name}|={e:.3e}")
        assert e <= TOL_BF16_GRAD, f"{name} error {e}"
    _check_invariants(dk, dv, dev["do"], "c5")


# --- small and ragged shapes ----------------------------------------------------

SMALL_N = [1, 2, 63, 65, 127, 129, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_f32_small_shapes(d, causal):
    for N in SMALL_N:
        ts = inputs.normal_qkv(1, 2, N, d, 100 + N, dtype="f32")
        scale = inputs.default_scale(d)
        o, lse = _fwd(upload(ts), causal, scale)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.attn_fwd(*(ts.f64[n].reshape(2, N, d) for n in "qkv"), scale, causal)
        _check_fwd(f64(o).reshape(2, N, d), f64(lse).reshape(2, N), ref_o, ref_l, TOL_F32_O, TOL_F32_L,
                   f"f32 N={N} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bwd_bf16_small_shapes(d, causal):
    for N in SMALL_N:
        ts = inputs.normal_qkv(1, 2, N, d, 200 + N, with_dout=True)
        scale = inputs.default_scale(d)
        dev = upload(ts)
        o, lse = _fwd(dev, causal, scale)
        dq, dk, dv = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=causal,
                                           scale=scale)
        torch.cuda.synchronize()
        arr = [ts.f64[n].reshape(2, N, d) for n in ("q", "k", "v", "do")]
        ref_o, ref_l = oracle.attn_fwd(*arr[:3], scale, causal)
        what = f"bf16 N={N} d={d} causal={causal}"
        _check_fwd(f64(o).reshape(2, N, d), f64(lse).reshape(2, N), ref_o, ref_l, TOL_BF16_O, TOL_BF16_L,
                   what)
        rq, rk, rv, _ = oracle.attn_bwd(*arr, scale, causal)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            e = maxabs(f64(got).reshape(2, N, d), ref)
            assert e <= TOL_BF16_GRAD, f"{what}: {name} error {e}"


def test_page_recipe_fp32():
    """The deep-dive page's self-test: n=300, d=64, its generator with seeds
    1/2/3, output within 1e-4 of naive attention."""
    n, d = 300, 64
    q, k, v = (inputs.page_generator(n, d, s) for s in (1, 2, 3))
    o, lse = binding.attention_fwd(*(torch.from_numpy(x).reshape(1, 1, n, d).cuda() for x in (q, k, v)),
                                   scale=1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attn_fwd(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                   float(np.float32(1.0 / math.sqrt(d))))
    _check_fwd(f64(o).reshape(1, n, d), f64(lse).reshape(1, n), ref_o, ref_l, TOL_F32_O, TOL_F32_L,
               "page recipe")


# --- closed forms ---------------------------------------------------------------

def _worked_inputs(d, dtype):
    q = np.zeros((1, 1, 4, d), np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    q[0, 0, 0, :2] = [1, 0]
    q[0, 0, 1:, :2] = [[0.5, -1.0], [2.0, 0.25], [-0.75, 1.5]]
    k[0, 0, :, :2] = [[1, 0], [0, 1], [3, 1], [-1, 1]]
    v[0, 0, :, :2] = [[1, 2], [3, 4], [5, 6], [7, 8]]
    if dtype == "bf16":
        return [to_dev(inputs.bf16_bits(x), "bf16") for x in (q, k, v)]
    return [to_dev(x, "f32") for x in (q, k, v)]


@pytest.mark.parametrize("d", [64, 128])
def test_worked_example(golden, d):
    g = golden("worked_example.txt")
    want_o, want_l = np.array(g["final_o_printed"][0]), 3.0 + math.log(g["tile2_l"][0][0])
    for dtype, tol in (("f32", TOL_F32_O), ("bf16", TOL_BF16_O)):
        o, lse = binding.attention_fwd(*_worked_inputs(d, dtype), scale=1.0)
        torch.cuda.synchronize()
        of = f64(o)[0, 0]
        assert maxabs(of[0, :2], want_o) <= tol, (dtype, of[0, :2])
        assert np.all(of[:, 2:] == 0)
        assert abs(f64(lse)[0, 0, 0] - want_l) <= 1e-4


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_and_zero_q(causal):
    B, H, N, d = 1, 4, 700, 128
    rng = np.random.default_rng(31)
    q = inputs.bf16_bits(rng.standard_normal((B, H, N, d), dtype=np.float32))
    k = inputs.bf16_bits(rng.standard_normal((B, H, N, d), dtype=np.float32))
    c = rng.standard_normal(d).astype(np.float32)
    vconst = inputs.bf16_bits(np.broadcast_to(c, (B, H, N, d)))
    o, _ = binding.attention_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(vconst, "bf16"), causal)
    torch.cuda.synchronize()
    cc = bf16_from_f64(c)
    # O_i = c: only P's bf16 rounding (relative 2^-9 of c) separates them
    assert maxabs(f64(o)[0, 0], np.broadcast_to(cc, (N, d))) <= 4 * 2 ** -9 * np.max(np.abs(cc)) + 1e-6
    # Q = 0: every p is exp2(0) = 1 exactly, so O is the (prefix) mean of V and L = ln(count)
    v = inputs.bf16_bits(rng.standard_normal((B, H, N, d), dtype=np.float32))
    z = np.zeros((B, H, N, d), np.uint16)
    o, lse = binding.attention_fwd(to_dev(z, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), causal)
    torch.cuda.synchronize()
    vf = inputs.bf16_to_f64(v)
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(vf, 2) / counts[:, None] if causal else vf.mean(2, keepdims=True).repeat(N, 2)
    # bf16 output rounding is relative (2^-9); allow twice that plus fp32 summation
    assert np.all(np.abs(f64(o) - mean) <= 2 ** -8 * np.abs(mean) + 1e-5)
    assert maxabs(f64(lse), np.log(counts)[None, None].repeat(H, 1)) <= 1e-5


def test_ragged_tail_is_not_dropped():
    """Tail keys (past the last full tile) aligned with every query and carrying
    a distinct constant value dominate the output: dropping them would be
    visible in O and in L."""
    B, H, N, d = 1, 2, 200, 128
    rng = np.random.default_rng(41)
    q = rng.standard_normal((B, H, N, d)).astype(np.float32) * 0.1
    q[..., 0] = 1.0
    k = rng.standard_normal((B, H, N, d)).astype(np.float32) * 0.1
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    k[:, :, 192:, 0] = 40.0  # keys 192..199 (8 keys in the ragged last tile)
    v[:, :, 192:, :] = 5.0
    qb, kb, vb = (inputs.bf16_bits(x) for x in (q, k, v))
    o, lse = binding.attention_fwd(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), False,
                                   scale=0.25)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attn_fwd(*(inputs.bf16_to_f64(x).reshape(2, N, d) for x in (qb, kb, vb)), 0.25)
    _check_fwd(f64(o).reshape(2, N, d), f64(lse).reshape(2, N), ref_o, ref_l, TOL_BF16_O, TOL_BF16_L,
               "ragged tail")
    assert np.all(np.abs(ref_o - 5.0) < 0.05)


def test_large_scores_stress():
    """Scores ~ N(0, 81): large rescaling steps between tiles."""
    B, H, N, d = 2, 2, 1000, 128
    rng = np.random.default_rng(51)
    q, k, v = (rng.standard_normal((B, H, N, d), dtype=np.float32) for _ in range(3))
    q *= 3
    k *= 3
    bits = [inputs.bf16_bits(x) for x in (q, k, v)]
    for causal in (False, True):
        o, lse = binding.attention_fwd(*(to_dev(b, "bf16") for b in bits), causal)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.attn_fwd(*(inputs.bf16_to_f64(b).reshape(4, N, d) for b in bits),
                                       inputs.default_scale(d), causal)
        _check_fwd(f64(o).reshape(4, N, d), f64(lse).reshape(4, N), ref_o, ref_l, TOL_BF16_O, TOL_BF16_L,
                   f"stress causal={causal}")


# --- determinism and the ABI on the device ----------------------------------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bitwise_reproducible(d, causal):
    """Two runs give bitwise equal outputs (no atomics, and no read of an LDS
    buffer while it is being refilled): per-head and grouped (Hq 4 / Hkv 2)
    forward and backward, and the fp8 forward."""
    ts = inputs.normal_qkv(2, 4, 1000, d, 61, with_dout=True)
    tg = inputs.normal_gqa(2, 4, 2, 1000, d, 62, with_dout=True)
    t8 = inputs.fp8_qkv(2, 4, 2, 1000, d, 63)
    dev, deg, de8 = upload(ts), upload(tg), upload(t8)
    runs = []
    for _ in range(2):
        out = []
        for x in (dev, deg):
            o, lse = _fwd(x, causal, None)
            grads = binding.attention_bwd(x["q"], x["k"], x["v"], o, lse, x["do"], causal=causal)
            out += [o, lse, *grads]
        out += list(binding.attention_fwd_fp8(de8["q"], de8["k"], de8["v"], t8.descale["q"], t8.descale["k"],
                                              t8.descale["v"], causal=causal))
        runs.append(out)
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_abi_errors_leave_outputs_untouched():
    import ctypes
    lib = binding.load_library()
    q = torch.randn(1, 2, 64, 128, device="cuda").to(torch.bfloat16)
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, 64), 7.0, device="cuda")
    p = [ctypes.c_void_p(t.data_ptr()) for t in (q, q, q, o, lse)]
    nul = ctypes.c_void_p(0)
    assert lib.fa_fwd(*p, 1, 2, 64, 96, ctypes.c_float(0.1), 0, nul) == 2
    assert lib.fa_fwd(*p, 1, 2, 64, 128, ctypes.c_float(float("nan")), 0, nul) == 1
    mis = list(p)
    mis[1] = ctypes.c_void_p(q.data_ptr() + 2)
    assert lib.fa_fwd(*mis, 1, 2, 64, 128, ctypes.c_float(0.1), 0, nul) == 1
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)
    with pytest.raises(binding.FaError):
        binding.fa_fwd(q[:, :, :, :96].contiguous(), q[:, :, :, :96].contiguous(),
                       q[:, :, :, :96].contiguous(), o[:, :, :, :96].contiguous(), lse)


def _paired_close(a, b, what):
    """The one-gradient kernels' dK or dV (a) against the paired kernel's (b) at
    d = 128.  Without dropout the paired kernel folds L and D into its score
    and dP products (an exact three-part bf16 split of -L/c and -D against a
    k-step of ones) where the one-gradient kernels subtract them after the
    product, so P and dP - D differ by a few fp32 roundings and a P element
    may round to the neighbouring bf16 value: the gradients agree to well
    under 1e-3 of their largest magnitude, while a P handed to the wrong lane
    or row would move them by O(1) of it."""
    e = (a - b).abs().max().item()
    m = b.abs().max().item()
    _say(f"{what}: one-gradient vs paired max|diff|={e:.3e} (max|x|={m:.3e})")
    assert e <= 1e-3 * m, f"{what}: paired kernel differs from the one-gradient kernels by {e} (max {m})"


@pytest.mark.parametrize("d", [64, 128])
def test_backward_stages_equal_fa_bwd(d):
    """fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq in stream order are fa_bwd; the
    one-gradient kernels (fa_bwd_dv, fa_bwd_dk) give the same dV and dK,
    bitwise at d = 64 (where fa_bwd runs them) and to within rounding at
    d = 128 (_paired_close), where fa_bwd_dkdv is the paired-wavefront kernel,
    so this also checks that P handed from one wavefront to its partner
    arrives intact, over several key blocks, causal diagonal blocks and a
    ragged tail."""
    for causal in (False, True):
        ts = inputs.normal_qkv(1, 3, 777, d, 71, with_dout=True)
        dev = upload(ts)
        o, lse = _fwd(dev, causal, None)
        dq, dk, dv = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=causal)
        delta = torch.empty_like(lse)
        sq, sk, sv, ok, ov = (torch.full_like(dq, float("nan")) for _ in range(5))
        binding.fa_bwd_preprocess(o, dev["do"], delta)
        binding.fa_bwd_dkdv(dev["q"], dev["k"], dev["v"], lse, dev["do"], delta, sk, sv, causal)
        binding.fa_bwd_dq(dev["q"], dev["k"], dev["v"], lse, dev["do"], delta, sq, causal)
        binding.fa_bwd_dv(dev["q"], dev["k"], lse, dev["do"], ov, causal)
        binding.fa_bwd_dk(dev["q"], dev["k"], dev["v"], lse, dev["do"], delta, ok, causal)
        torch.cuda.synchronize()
        for a, b in ((sq, dq), (sk, dk), (sv, dv)):
            assert torch.equal(a, b)
        if d == 64:
            assert torch.equal(ok, dk) and torch.equal(ov, dv)
        else:
            _paired_close(ok, dk, f"d128 causal={causal} dk")
            _paired_close(ov, dv, f"d128 causal={causal} dv")
