"""Attention dropout on the GPU against the fp64 oracle, through the C ABI
(fa_fwd_dropout, fa_bwd_dropout).  Both sides draw the keep mask from their
own Philox4x32-10 with the same seed, offset and element-to-byte map, so the
masks agree exactly and the usual bf16 bars apply: O and fp32 gradients
max-abs <= 2e-2 (x the keep scale, which multiplies every kept term), L
<= 1e-3."""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_fwd_amd import binding, inputs
from gpu_util import TOL_BF16_GRAD, TOL_BF16_L, TOL_BF16_O, f64, maxabs, upload

pytestmark = pytest.mark.gpu

SEED = 0x5EED_0000_1234_ABCD


def _check(what, got, ref, tol):
    got = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got)
    e = maxabs(got.reshape(ref.shape), ref)
    print(f"{what}: max err {e:.3e}", flush=True)
    assert e <= tol, f"{what}: error {e}"


def _run(ts, p, causal, scale, offset=0, bwd=True):
    dev = upload(ts)
    o, lse = binding.attention_fwd_dropout(dev["q"], dev["k"], dev["v"], p, SEED, offset, causal=causal, scale=scale)
    grads = None
    if bwd:
        grads = binding.attention_bwd_dropout(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], p, SEED, offset,
                                              causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dev, o, lse, grads


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_dropout_small_shapes(d, causal, Hq, Hkv):
    for N, p in ((1, 0.1), (63, 0.5), (129, 0.1), (300, 0.25)):
        ts = inputs.normal_gqa(2, Hq, Hkv, N, d, 900 + N, with_dout=True)
        scale = inputs.default_scale(d)
        _, o, lse, (dq, dk, dv) = _run(ts, p, causal, scale, offset=N)
        _, ks = oracle.dropout_threshold(p)
        what = f"dropout p={p} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}"
        ref_o, ref_l = oracle.attn_fwd_dropout(ts.f64["q"], ts.f64["k"], ts.f64["v"], scale, causal, p, SEED, N)
        _check(what + " O", o, ref_o, TOL_BF16_O * ks)
        _check(what + " L", lse, ref_l, TOL_BF16_L)
        rq, rk, rv, _ = oracle.attn_bwd_dropout(ts.f64["q"], ts.f64["k"], ts.f64["v"], ts.f64["do"], scale, causal,
                                                p, SEED, N)
        _check(what + " dQ", dq, rq, TOL_BF16_GRAD * ks)
        _check(what + " dK", dk, rk, TOL_BF16_GRAD * ks)
        _check(what + " dV", dv, rv, TOL_BF16_GRAD * ks)


def test_dropout_n2048_causal_all_outputs():
    B, Hq, Hkv, N, d, p = 1, 4, 2, 2048, 128, 0.2
    ts = inputs.normal_gqa(B, Hq, Hkv, N, d, 20300, with_dout=True)
    scale = inputs.default_scale(d)
    _, o, lse, (dq, dk, dv) = _run(ts, p, True, scale, offset=5)
    _, ks = oracle.dropout_threshold(p)
    ref_o, ref_l = oracle.attn_fwd_dropout(ts.f64["q"], ts.f64["k"], ts.f64["v"], scale, True, p, SEED, 5)
    _check("dropout N2048 O", o, ref_o, TOL_BF16_O * ks)
    _check("dropout N2048 L", lse, ref_l, TOL_BF16_L)
    rq, rk, rv, _ = oracle.attn_bwd_dropout(ts.f64["q"], ts.f64["k"], ts.f64["v"], ts.f64["do"], scale, True, p,
                                            SEED, 5)
    _check("dropout N2048 dQ", dq, rq, TOL_BF16_GRAD * ks)
    _check("dropout N2048 dK", dk, rk, TOL_BF16_GRAD * ks)
    _check("dropout N2048 dV", dv, rv, TOL_BF16_GRAD * ks)


def test_dropout_causal_n8192_sampled_rows():
    """The benchmark's shape (B2 H32 N8192 d128, causal), p 0.1: forward rows
    of two heads, including the first and the last, against the oracle."""
    B, H, N, d, p = 2, 32, 8192, 128, 0.1
    ts = inputs.normal_qkv(B, H, N, d, 20301)
    scale = inputs.default_scale(d)
    _, o, lse, _ = _run(ts, p, True, scale, offset=9, bwd=False)
    _, ks = oracle.dropout_threshold(p)
    rng = np.random.default_rng(20302)
    got_o, got_l = f64(o).reshape(B * H, N, d), f64(lse).reshape(B * H, N)
    qf, kf, vf = (ts.f64[n].reshape(B * H, N, d) for n in ("q", "k", "v"))
    for bh in (0, 51):
        rows = np.unique(np.concatenate([[0, 1, N - 1], rng.choice(N, 197, replace=False)]))
        ref_o, ref_l = oracle.attn_fwd_rows_dropout(qf, kf, vf, bh * N + rows, scale, True, p, SEED, 9)
        _check(f"dropout N8192 head {bh} O", got_o[bh, rows], ref_o, TOL_BF16_O * ks)
        _check(f"dropout N8192 head {bh} L", got_l[bh, rows], ref_l, TOL_BF16_L)


def test_dropout_p0_equals_plain_path_and_seeds_matter():
    """p = 0 drops nothing: bitwise the plain forward and dQ; dK and dV to
    within rounding, since without dropout the paired dK/dV kernel folds L
    and D into its products while the dropout variant subtracts them after
    (the one-gradient comparison in test_parity.py states the bound).  The
    same seed and offset reproduce bitwise; another offset changes the
    output."""
    B, Hq, Hkv, N, d = 1, 4, 2, 500, 128
    ts = inputs.normal_gqa(B, Hq, Hkv, N, d, 20303, with_dout=True)
    scale = inputs.default_scale(d)
    dev, o0, l0, g0 = _run(ts, 0.0, True, scale)
    o, lse = binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale)
    g = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o0, o) and torch.equal(l0, lse)
    assert torch.equal(g0[0], g[0])  # dQ
    for a, b in zip(g0[1:], g[1:]):  # dK, dV
        assert (a - b).abs().max().item() <= 1e-3 * b.abs().max().item()
    _, o1, _, g1 = _run(ts, 0.3, True, scale, offset=1)
    _, o2, _, g2 = _run(ts, 0.3, True, scale, offset=1)
    _, o3, _, _ = _run(ts, 0.3, True, scale, offset=2)
    assert torch.equal(o1, o2) and all(torch.equal(a, b) for a, b in zip(g1, g2))
    assert not torch.equal(o1, o3)
