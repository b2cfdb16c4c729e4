"""Any finite softmax scale: negative, zero and large, on every GPU path,
against the fp64 oracle through the C ABI.

The deep-dive page ("FlashAttention", section "How it works") defines the
scores as S = Q K^T times the scale with no restriction on its sign.  The
kernels move the sign of the scale (or a zero) into the operand they keep in
registers, so besides the oracle bars these tests check the exact identities
that follow: with the scale negated, the forward equals the forward on -Q
bitwise, dK and dV are unchanged and dQ changes sign, bitwise; with scale 0
every visible key gets the same weight, so O is the mean of the visible V
rows, L = ln(count) and dQ = dK = 0.

Bars: the configs' bars (2e-2, 1e-3; fp32 1e-4) hold at the configs' scale
1/sqrt(d).  dQ and dK carry the factor `scale` and dS grows with the spread
of the scaled scores, so their rounding errors grow in proportion to |scale|;
above 1/sqrt(d) the gradient bar is 2e-2 * |scale| sqrt(d).
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_fwd_amd import binding, inputs
from gpu_util import TOL_BF16_GRAD, TOL_BF16_L, TOL_BF16_O, TOL_F32_L, TOL_F32_O, f64, maxabs, upload
from test_parity_fp8 import _check as fp8_check

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _scales(d):
    s = inputs.default_scale(d)
    return [-s, 0.0, -1.5 * s, 1.5 * s]


def _grad_bar(scale, d):
    return TOL_BF16_GRAD * max(1.0, abs(scale) * d ** 0.5)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_fwd_bwd_any_scale(d, causal):
    """bf16 forward and backward (every stage, both dK/dV kernels at d = 128
    through fa_bwd) at negative, zero and positive scales, ragged N = 300;
    also at 2^-90, where the paired dK/dV kernel still folds -L/c (about
    2^94) into its products, and at -1e-35, below 2^-100, where fa_bwd takes
    the separate dK and dV kernels instead."""
    N = 300
    ts = inputs.normal_qkv(1, 2, N, d, 1300 + d, with_dout=True)
    dev = upload(ts)
    arr = [ts.f64[n].reshape(2, N, d) for n in ("q", "k", "v", "do")]
    for scale in _scales(d) + [2.0 ** -90, -1e-35]:
        what = f"bf16 d={d} causal={causal} scale={scale}"
        _say(what)
        o, lse = binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
        dq, dk, dv = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=causal,
                                           scale=scale)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.attn_fwd(*arr[:3], scale, causal)
        rq, rk, rv, _ = oracle.attn_bwd(*arr, scale, causal)
        assert maxabs(f64(o).reshape(2, N, d), ref_o) <= TOL_BF16_O, what
        assert maxabs(f64(lse).reshape(2, N), ref_l) <= TOL_BF16_L, what
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            e = maxabs(f64(got).reshape(2, N, d), ref)
            assert e <= _grad_bar(scale, d), f"{what}: {name} error {e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_negated_scale_is_negated_q_bitwise(d, causal):
    """fa(q, k, v, -s) == fa(-q, k, v, s) bitwise for O and L; in the backward
    dV agrees bitwise and dQ changes sign bitwise.  Negating a bf16 value is
    exact, and every product of the scores changes sign exactly, so the scores,
    P, dP and dS are the same values in both calls and any deviation would be an
    error in how the kernels carry the sign.  dK = scale dS^T Q accumulates
    products with Q in one call and with -Q in the other; the matrix cores'
    fp32 accumulation does not round a negated sum to exactly the negated
    result (measured: up to 1.5 ulp apart), so dK is held to 2^-18 max|dK|
    (a few ulp) rather than bitwise."""
    N = 777
    ts = inputs.normal_qkv(1, 3, N, d, 1400 + d, with_dout=True)
    dev = upload(ts)
    s = inputs.default_scale(d)
    nq = -dev["q"]
    oa, la = binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=-s)
    ob, lb = binding.attention_fwd(nq, dev["k"], dev["v"], causal=causal, scale=s)
    ga = binding.attention_bwd(dev["q"], dev["k"], dev["v"], oa, la, dev["do"], causal=causal, scale=-s)
    gb = binding.attention_bwd(nq, dev["k"], dev["v"], ob, lb, dev["do"], causal=causal, scale=s)
    torch.cuda.synchronize()
    dk_dev, dk_max = (ga[1] - gb[1]).abs().max().item(), ga[1].abs().max().item()
    _say(f"d={d} causal={causal}: max |dK(q, -s) - dK(-q, s)| = {dk_dev:.3e}, max |dK| = {dk_max:.3e}")
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    assert torch.equal(ga[0], -gb[0])
    assert torch.equal(ga[2], gb[2])
    assert dk_dev <= 2.0 ** -18 * dk_max


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_closed_form(causal):
    """Scale 0: all visible scores are 0, so O_i is the mean of the visible V
    rows, L_i = ln(count_i), dQ = dK = 0 exactly and dV_j = sum over visible
    i of dO_i / count_i; ragged N = 300, d = 128."""
    B, H, N, d = 1, 2, 300, 128
    ts = inputs.normal_qkv(B, H, N, d, 1500, with_dout=True)
    dev = upload(ts)
    o, lse = binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=0.0)
    dq, dk, dv = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=causal, scale=0.0)
    torch.cuda.synchronize()
    vf, gf = ts.f64["v"], ts.f64["do"]
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(vf, 2) / counts[:, None] if causal else vf.mean(2, keepdims=True).repeat(N, 2)
    assert np.all(np.abs(f64(o) - mean) <= 2 ** -8 * np.abs(mean) + 1e-5)
    assert maxabs(f64(lse), np.log(counts)[None, None].repeat(H, 1)) <= 1e-5
    assert torch.all(dq == 0) and torch.all(dk == 0)
    w = gf / counts[:, None]
    want_dv = np.flip(np.cumsum(np.flip(w, 2), 2), 2) if causal else w.sum(2, keepdims=True).repeat(N, 2)
    assert maxabs(f64(dv), want_dv) <= TOL_BF16_GRAD
    ref_o, _ = oracle.attn_fwd(*(ts.f64[n].reshape(2, N, d) for n in "qkv"), 0.0, causal)
    assert maxabs(f64(o).reshape(2, N, d), ref_o) <= TOL_BF16_O


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_fwd_any_scale(causal):
    for d in (64, 128):
        N = 300
        ts = inputs.normal_qkv(1, 2, N, d, 1600 + d, dtype="f32")
        dev = upload(ts)
        for scale in _scales(d):
            o, lse = binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
            torch.cuda.synchronize()
            ref_o, ref_l = oracle.attn_fwd(*(ts.f64[n].reshape(2, N, d) for n in "qkv"), scale, causal)
            what = f"f32 d={d} causal={causal} scale={scale}"
            assert maxabs(f64(o).reshape(2, N, d), ref_o) <= TOL_F32_O, what
            assert maxabs(f64(lse).reshape(2, N), ref_l) <= TOL_F32_L, what


@pytest.mark.parametrize("d", [64, 128])
def test_grouped_and_dropout_any_scale(d):
    """Grouped heads (Hq 4, Hkv 2) and dropout (p = 0.25) at negative and zero
    scales, forward and backward, against the grouped and dropout oracles."""
    N, p, seed = 300, 0.25, 0xABCDEF
    ts = inputs.normal_gqa(2, 4, 2, N, d, 1700 + d, with_dout=True)
    dev = upload(ts)
    _, ks = oracle.dropout_threshold(p)
    for causal in (False, True):
        for scale in (-inputs.default_scale(d), 0.0):
            what = f"gqa d={d} causal={causal} scale={scale}"
            o, lse = binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
            g = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=causal, scale=scale)
            torch.cuda.synchronize()
            ref_o, ref_l = oracle.attn_fwd_gqa(ts.f64["q"], ts.f64["k"], ts.f64["v"], scale, causal)
            refs = oracle.attn_bwd_gqa(ts.f64["q"], ts.f64["k"], ts.f64["v"], ts.f64["do"], scale, causal)
            assert maxabs(f64(o), ref_o) <= TOL_BF16_O and maxabs(f64(lse), ref_l) <= TOL_BF16_L, what
            for got, ref in zip(g, refs[:3]):
                assert maxabs(f64(got), ref) <= TOL_BF16_GRAD, what
            what = f"dropout d={d} causal={causal} scale={scale}"
            o, lse = binding.attention_fwd_dropout(dev["q"], dev["k"], dev["v"], p, seed, 3, causal=causal,
                                                   scale=scale)
            g = binding.attention_bwd_dropout(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], p, seed, 3,
                                              causal=causal, scale=scale)
            torch.cuda.synchronize()
            ref_o, ref_l = oracle.attn_fwd_dropout(ts.f64["q"], ts.f64["k"], ts.f64["v"], scale, causal, p, seed, 3)
            refs = oracle.attn_bwd_dropout(ts.f64["q"], ts.f64["k"], ts.f64["v"], ts.f64["do"], scale, causal, p,
                                           seed, 3)
            assert maxabs(f64(o), ref_o) <= TOL_BF16_O * ks and maxabs(f64(lse), ref_l) <= TOL_BF16_L, what
            for got, ref in zip(g, refs[:3]):
                assert maxabs(f64(got), ref) <= TOL_BF16_GRAD * ks, what


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_any_scale(d):
    for causal in (False, True):
        ts = inputs.fp8_qkv(2, 4, 2, 300, d, 1800 + d)
        dev = upload(ts)
        for scale in (-inputs.default_scale(d), 0.0, -1.5 * inputs.default_scale(d)):
            o, lse = binding.attention_fwd_fp8(dev["q"], dev["k"], dev["v"], ts.descale["q"], ts.descale["k"],
                                               ts.descale["v"], causal=causal, scale=scale)
            torch.cuda.synchronize()
            fp8_check(f"fp8 d={d} causal={causal} scale={scale}", ts, o, lse, causal, scale)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_any_scale(d):
    B, Hq, Hkv, Nk = 3, 8, 2, 1000
    ts = inputs.decode_qkv(B, Hq, Hkv, Nk, d, 1900 + d)
    dev = upload(ts)
    lens = [Nk, 517, 1]
    dlen = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for scale in (-inputs.default_scale(d), 0.0, -1.5 * inputs.default_scale(d)):
        ref_o, ref_l = oracle.attn_decode(ts.f64["q"], ts.f64["k"], ts.f64["v"], scale, kv_len=lens)
        for splits in (0, 1, 3):
            o, lse = binding.attention_decode(dev["q"], dev["k"], dev["v"], kv_len=dlen, num_splits=splits,
                                              scale=scale)
            torch.cuda.synchronize()
            what = f"decode d={d} scale={scale} splits={splits}"
            assert maxabs(f64(o), ref_o) <= TOL_BF16_O and maxabs(f64(lse), ref_l) <= TOL_BF16_L, what
