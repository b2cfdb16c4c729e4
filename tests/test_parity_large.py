"""Tensors of more than 2^31 elements: the "FlashAttention" deep-dive page
("Pitfalls") warns that 32-bit element offsets overflow there.

B1 H1040 N16384 d128 holds 2.18e9 > 2^31 elements per tensor (4.4 GB in
bf16, 8.7 GB per fp32 gradient).  Drawing 2e9 numbers on the host would take
minutes, so most heads are device-side copies of eight seeded base heads; head
0 and the last two heads (whose element offsets lie beyond 2^31, their byte
offsets beyond 2^32) get draws of their own that occur nowhere else, so a
kernel that wrapped an offset would read or write another head's data and
miss the oracle.  Outputs start as NaN so that an unwritten row shows too.
Checked: forward and backward of the three distinct heads against the
oracle; on every head causal row 0 equals V row 0 bitwise; the gradient
column-sum invariants on every head.
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_fwd_amd import binding, inputs
from gpu_util import TOL_BF16_GRAD, TOL_BF16_L, TOL_BF16_O, f64, maxabs

pytestmark = pytest.mark.gpu

B, H, N, D = 1, 1040, 16384, 128
NBASE = 8
UNIQUE = (0, H - 2, H - 1)


def _say(*a):
    print(*a, flush=True)


def _big_inputs(seed):
    """Per tensor: (device bf16 [B, H, N, D], {head: fp64 [N, D]} of the
    distinct heads).  Head h is base head h % NBASE except the UNIQUE heads."""
    assert B * H * N * D > 2 ** 31
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("q", "k", "v", "do"):
        base = inputs.bf16_bits(rng.standard_normal((NBASE, N, D), dtype=np.float32))
        own = inputs.bf16_bits(rng.standard_normal((len(UNIQUE), N, D), dtype=np.float32))
        base_dev = torch.from_numpy(base.view(np.int16)).view(torch.bfloat16).cuda()
        idx = torch.arange(H, device="cuda") % NBASE
        big = base_dev[idx].unsqueeze(0)  # [1, H, N, D], one gather
        del base_dev
        for i, hh in enumerate(UNIQUE):
            big[0, hh].copy_(torch.from_numpy(own[i].view(np.int16)).view(torch.bfloat16))
        out[name] = (big, {hh: inputs.bf16_to_f64(own[i]) for i, hh in enumerate(UNIQUE)})
    torch.cuda.synchronize()
    return out


def test_more_than_2_31_elements_fwd_bwd():
    scale = inputs.default_scale(D)
    _say(f"large: bf16 causal B{B} H{H} N{N} d{D}: {B * H * N * D:.3e} elements per tensor")
    t = _big_inputs(20310)
    q, k, v, do = (t[n][0] for n in ("q", "k", "v", "do"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    binding.fa_fwd(q, k, v, o, lse, causal=True, scale=scale)
    dq = torch.full((B, H, N, D), float("nan"), device="cuda")
    dk, dv = torch.full_like(dq, float("nan")), torch.full_like(dq, float("nan"))
    delta = torch.empty_like(lse)
    binding.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, causal=True, scale=scale)
    torch.cuda.synchronize()
    _say("large: GPU done")
    # every head: causal row 0 is V row 0 bitwise; invariants of the gradients
    assert torch.equal(o[:, :, 0, :], v[:, :, 0, :])
    sdk = dk.sum(2, dtype=torch.float64).abs().max().item()
    sdv = (dv.sum(2, dtype=torch.float64) - do.sum(2, dtype=torch.float64)).abs().max().item()
    _say(f"large invariants all heads: max|sum dK|={sdk:.3e} max|sum dV - sum dO|={sdv:.3e}")
    assert sdk <= 0.15 and sdv <= 0.15
    heads = list(UNIQUE)
    arr = {n: np.stack([t[n][1][hh] for hh in heads]) for n in ("q", "k", "v", "do")}
    ref_o, ref_l = oracle.attn_fwd(arr["q"], arr["k"], arr["v"], scale, causal=True)
    eo = maxabs(f64(o[0, heads]), ref_o)
    el = maxabs(f64(lse[0, heads]), ref_l)
    _say(f"large heads {heads}: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL_BF16_O and el <= TOL_BF16_L
    for hh in heads[1:]:  # the two heads past 2^31 elements: full backward against the oracle
        rq, rk, rv, _ = oracle.attn_bwd(*(arr[n][heads.index(hh)][None] for n in ("q", "k", "v", "do")), scale,
                                        causal=True)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            e = maxabs(f64(got[0, hh])[None], ref)
            _say(f"large bwd head {hh}: max|d{name}|={e:.3e}")
            assert e <= TOL_BF16_GRAD
