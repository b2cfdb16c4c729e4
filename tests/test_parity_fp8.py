"""fp8 (OCP e4m3) forward on the GPU against the fp64 oracle, through the C
ABI (fa_fwd_fp8).

The oracle is the plain definition of attention evaluated on the exact real
inputs (descale * e4m3 value).  The kernel's products of e4m3 values are
exact and accumulate in fp32, so the one rounding it adds beyond the bf16
path is P rounded to e4m3 as the operand of P V.  The bar for O is derived
from that rounding, per output element (O_it = sum_j w_ij v_jt, w = softmax
weights): the rounding moves each weight by at most
    dw_ij = max(2^-4 w_ij, 2^-10 max_j w_ij)
(relative half-ulp of a 3-bit mantissa; absolute half-spacing of e4m3
subnormals, 2^-10, in units where the largest P is >= 1), the errors are
independent and uniform, so the deviation has standard deviation
    sigma_it = sqrt(sum_j dw_ij^2 v_jt^2 / 3),
and the test allows 7 sigma_it + 2^-8 |O_it| (bf16 output rounding, twice
over) + 2e-4 (fp32 accumulation).  L carries no fp8 rounding: bar 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_fwd_amd import binding, inputs
from gpu_util import TOL_BF16_L, f64, maxabs, upload

pytestmark = pytest.mark.gpu


def fp8_bound(q, k, v, scale, causal, o_ref, rows=None):
    """Per-element bar for O (see the module docstring).  q [Hq, N, d],
    k, v [Hq, N, d] (already mapped to each query head), o_ref [Hq, R, d] for
    the query rows `rows` (all rows when None)."""
    H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    tau = np.empty((H, len(rows), d))
    for hh in range(H):
        S = scale * q[hh, rows] @ k[hh].T
        if causal:
            S[np.arange(N)[None, :] > rows[:, None]] = -np.inf
        W = np.exp(S - S.max(axis=1, keepdims=True))
        W /= W.sum(axis=1, keepdims=True)
        dW = np.where(W > 0, np.maximum(2.0 ** -4 * W, 2.0 ** -10 * W.max(axis=1, keepdims=True)), 0.0)
        sigma = np.sqrt((dW ** 2) @ (v[hh] ** 2) / 3.0)
        tau[hh] = 7.0 * sigma + 2.0 ** -8 * np.abs(o_ref[hh]) + 2e-4
    return tau


def _run(ts, causal, scale):
    dev = upload(ts)
    ds = ts.descale
    o, lse = binding.attention_fwd_fp8(dev["q"], dev["k"], dev["v"], ds["q"], ds["k"], ds["v"],
                                       causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _check(what, ts, o, lse, causal, scale):
    qf, kf, vf = ts.f64["q"], ts.f64["k"], ts.f64["v"]
    B, Hq, N, d = qf.shape
    G = Hq // kf.shape[1]
    ref_o, ref_l = oracle.attn_fwd_gqa(qf, kf, vf, scale, causal)
    got = f64(o)
    worst = 0.0
    for b in range(B):
        kk, vv = np.repeat(kf[b], G, axis=0), np.repeat(vf[b], G, axis=0)
        tau = fp8_bound(qf[b], kk, vv, scale, causal, ref_o[b])
        err = np.abs(got[b] - ref_o[b])
        assert np.all(np.isfinite(got[b]))
        worst = max(worst, float(np.max(err / tau)))
    el = maxabs(f64(lse), ref_l)
    print(f"{what}: max |err| / bar = {worst:.3f}, O max err {maxabs(got, ref_o):.3e}, L err {el:.3e}", flush=True)
    assert worst <= 1.0, what
    assert el <= TOL_BF16_L, what


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_fp8_small_shapes(d, causal, Hq, Hkv):
    for N in (1, 63, 129, 300):
        ts = inputs.fp8_qkv(2, Hq, Hkv, N, d, 700 + N)
        scale = inputs.default_scale(d)
        o, lse = _run(ts, causal, scale)
        _check(f"fp8 Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}", ts, o, lse, causal, scale)


def test_fp8_n2048_causal_all_rows():
    ts = inputs.fp8_qkv(1, 4, 4, 2048, 128, 20290)
    scale = inputs.default_scale(128)
    o, lse = _run(ts, True, scale)
    _check("fp8 B1 H4 N2048 d128 causal", ts, o, lse, True, scale)


def test_fp8_causal_n8192_sampled_rows():
    """The benchmark's shape (B2 H32 N8192 d128, causal): two heads, 300 rows
    each including the first and the last, against the oracle row by row."""
    B, H, N, d = 2, 32, 8192, 128
    ts = inputs.fp8_qkv(B, H, H, N, d, 20291)
    scale = inputs.default_scale(d)
    o, lse = _run(ts, True, scale)
    rng = np.random.default_rng(20292)
    got_o, got_l = f64(o).reshape(B * H, N, d), f64(lse).reshape(B * H, N)
    qf, kf, vf = (ts.f64[n].reshape(B * H, N, d) for n in ("q", "k", "v"))
    for bh in (0, 45):
        rows = np.unique(np.concatenate([[0, 1, N - 1], rng.choice(N, 297, replace=False)]))
        ref_o, ref_l = oracle.attn_fwd_rows(qf, kf, vf, bh * N + rows, scale, True)
        tau = fp8_bound(qf[bh:bh + 1], kf[bh:bh + 1], vf[bh:bh + 1], scale, True, ref_o[None], rows=rows)[0]
        ratio = float(np.max(np.abs(got_o[bh, rows] - ref_o) / tau))
        el = maxabs(got_l[bh, rows], ref_l)
        print(f"fp8 N8192 head {bh}: max |err| / bar = {ratio:.3f}, L err {el:.3e}", flush=True)
        assert ratio <= 1.0 and el <= TOL_BF16_L


def test_fp8_causal_row0_is_v0():
    """Causal row 0 has one visible key: P = 1 exactly (e4m3 holds 1), so
    O_0 = bf16(v_descale * v_0) bitwise."""
    ts = inputs.fp8_qkv(1, 3, 3, 200, 128, 20293)
    o, _ = _run(ts, True, inputs.default_scale(128))
    want = torch.from_numpy(ts.f64["v"][0, :, 0].astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(o[0, :, 0].cpu(), want)
