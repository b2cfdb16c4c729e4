"""Grouped heads (GQA / MQA) on the GPU against the fp64 oracle, through the
C ABI (fa_fwd_gqa, fa_bwd_gqa).  Same bars as the per-head parity tests:
bf16 O and fp32-out gradients max-abs <= 2e-2, L <= 1e-3."""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_fwd_amd import binding, inputs
from gpu_util import TOL_BF16_GRAD, TOL_BF16_L, TOL_BF16_O, f64, maxabs, upload

pytestmark = pytest.mark.gpu


def _run(ts, causal, scale):
    dev = upload(ts)
    o, lse = binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    grads = None
    if "do" in dev:
        grads = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dev, o, lse, grads


def _check(what, got, ref, tol):
    e = maxabs(f64(got).reshape(ref.shape), ref)
    print(f"{what}: max err {e:.3e}", flush=True)
    assert e <= tol, f"{what}: error {e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 1), (6, 3)])
def test_gqa_small_shapes(d, causal, Hq, Hkv):
    for N in (1, 63, 129, 300):
        ts = inputs.normal_gqa(2, Hq, Hkv, N, d, 300 + N, with_dout=True)
        scale = inputs.default_scale(d)
        _, o, lse, (dq, dk, dv) = _run(ts, causal, scale)
        what = f"gqa Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}"
        ref_o, ref_l = oracle.attn_fwd_gqa(ts.f64["q"], ts.f64["k"], ts.f64["v"], scale, causal)
        _check(what + " O", o, ref_o, TOL_BF16_O)
        _check(what + " L", lse, ref_l, TOL_BF16_L)
        rq, rk, rv, _ = oracle.attn_bwd_gqa(ts.f64["q"], ts.f64["k"], ts.f64["v"], ts.f64["do"], scale, causal)
        _check(what + " dQ", dq, rq, TOL_BF16_GRAD)
        _check(what + " dK", dk, rk, TOL_BF16_GRAD)
        _check(what + " dV", dv, rv, TOL_BF16_GRAD)


def test_gqa_group_of_four_n2048_causal():
    """A larger grouped workload, every output checked: B 2, Hq 8, Hkv 2,
    N 2048, d 128, causal (32 query blocks per head, four query heads per
    key/value head)."""
    B, Hq, Hkv, N, d = 2, 8, 2, 2048, 128
    ts = inputs.normal_gqa(B, Hq, Hkv, N, d, 20270, with_dout=True)
    scale = inputs.default_scale(d)
    _, o, lse, (dq, dk, dv) = _run(ts, True, scale)
    ref_o, ref_l = oracle.attn_fwd_gqa(ts.f64["q"], ts.f64["k"], ts.f64["v"], scale, True)
    _check("gqa n2048 O", o, ref_o, TOL_BF16_O)
    _check("gqa n2048 L", lse, ref_l, TOL_BF16_L)
    rq, rk, rv, _ = oracle.attn_bwd_gqa(ts.f64["q"], ts.f64["k"], ts.f64["v"], ts.f64["do"], scale, True)
    _check("gqa n2048 dQ", dq, rq, TOL_BF16_GRAD)
    _check("gqa n2048 dK", dk, rk, TOL_BF16_GRAD)
    _check("gqa n2048 dV", dv, rv, TOL_BF16_GRAD)


def test_gqa_matches_repeated_heads():
    """Grouped heads read the same K, V values as per-head attention with K, V
    repeated per query head: O, L and dQ are bitwise equal; dK, dV equal the
    per-head gradients summed over each group (to fp32 rounding)."""
    B, Hq, Hkv, N, d = 1, 6, 2, 500, 128
    ts = inputs.normal_gqa(B, Hq, Hkv, N, d, 20271, with_dout=True)
    scale = inputs.default_scale(d)
    dev, o, lse, (dq, dk, dv) = _run(ts, True, scale)
    G = Hq // Hkv
    kr, vr = (dev[n].repeat_interleave(G, dim=1).contiguous() for n in ("k", "v"))
    o1, lse1 = binding.attention_fwd(dev["q"], kr, vr, causal=True, scale=scale)
    dq1, dk1, dv1 = binding.attention_bwd(dev["q"], kr, vr, o1, lse1, dev["do"], causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, lse1) and torch.equal(dq, dq1)
    for got, per_head in ((dk, dk1), (dv, dv1)):
        summed = per_head.reshape(B, Hkv, G, N, d).sum(2)
        assert maxabs(f64(got), f64(summed)) <= 1e-4


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2)])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_gradients(Hq, Hkv, d):
    """fa_bwd_gqa_bf16grad stores the same fp32 accumulators rounded to bf16
    (nearest even): bitwise the fp32-gradient path's results rounded, and
    within the bf16 bar of the oracle."""
    for N, causal in ((129, True), (300, False), (1000, True)):
        ts = inputs.normal_gqa(2, Hq, Hkv, N, d, 1100 + N, with_dout=True)
        scale = inputs.default_scale(d)
        dev, o, lse, (dq, dk, dv) = _run(ts, causal, scale)
        dq16, dk16, dv16 = (torch.empty(t.shape, dtype=torch.bfloat16, device="cuda") for t in (dq, dk, dv))
        delta = torch.empty_like(lse)
        binding.fa_bwd_gqa_bf16grad(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], dq16, dk16, dv16, delta,
                                    causal=causal, scale=scale)
        torch.cuda.synchronize()
        for got, full in ((dq16, dq), (dk16, dk), (dv16, dv)):
            assert torch.equal(got, full.to(torch.bfloat16))
        rq, rk, rv, _ = oracle.attn_bwd_gqa(ts.f64["q"], ts.f64["k"], ts.f64["v"], ts.f64["do"], scale, causal)
        what = f"bf16 grads Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}"
        _check(what + " dQ", dq16, rq, TOL_BF16_GRAD)
        _check(what + " dK", dk16, rk, TOL_BF16_GRAD)
        _check(what + " dV", dv16, rv, TOL_BF16_GRAD)
