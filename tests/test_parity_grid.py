"""Every head of a grid: the workgroup-to-(head, block) mappings.

The forward and dQ kernels map a flat workgroup id to (head, query block)
through head_rank (fa_common.h).  When B*H is a multiple of the 8 XCDs, XCD
x takes the contiguous heads [x hp, (x + 1) hp), hp = B*H / 8, in groups of
g heads walked rank-major, g the largest divisor of hp with g * blocks <= 32;
otherwise the XCDs get contiguous task ranges (xcd_task).  The dK/dV kernels
keep xcd_task.  A slip in either mapping leaves a head unwritten or writes
one twice, which tests of sampled heads can miss, so here every head of each
shape is compared with the oracle, outputs prefilled with NaN.

Shapes (256-row query blocks, 128-key dK/dV blocks):
  B1 H16 N600 d128 causal     hp 2, 3 blocks: g = 2
  B2 H24 N1700 d64 causal     hp 6, 7 blocks: 32/7 = 4 does not divide 6, g = 3
  B1 H40 N1000 d64            hp 5, 4 blocks: g = 5
  B3 H2 N700 d128 causal      B*H = 6: xcd_task
  B1 H8 N9000 d64 causal      hp 1, 36 blocks: g = 1 (forward only: head-major)
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_fwd_amd import binding, inputs
from gpu_util import TOL_BF16_GRAD, TOL_BF16_L, TOL_BF16_O, f64, maxabs, upload

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


SHAPES = [
    (1, 16, 600, 128, True, True),
    (2, 24, 1700, 64, True, True),
    (1, 40, 1000, 64, False, True),
    (3, 2, 700, 128, True, True),
    (1, 8, 9000, 64, True, False),
]


@pytest.mark.parametrize("B,H,N,d,causal,bwd", SHAPES)
def test_every_head(B, H, N, d, causal, bwd):
    what = f"grid B{B} H{H} N{N} d{d} causal={causal}"
    _say(what)
    ts = inputs.normal_qkv(B, H, N, d, 40000 + B * 1000 + H + N, with_dout=True)
    scale = inputs.default_scale(d)
    dev = upload(ts)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    binding.fa_fwd(q, k, v, o, lse, causal=causal, scale=scale)
    BH = B * H
    arr = {n: ts.f64[n].reshape(BH, N, d) for n in ("q", "k", "v", "do")}
    ref_o, ref_l = oracle.attn_fwd(arr["q"], arr["k"], arr["v"], scale, causal=causal)
    if bwd:
        dq = torch.full((B, H, N, d), float("nan"), device="cuda")
        dk, dv = torch.full_like(dq, float("nan")), torch.full_like(dq, float("nan"))
        delta = torch.empty_like(lse)
        binding.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, causal=causal, scale=scale)
    torch.cuda.synchronize()
    eo = maxabs(f64(o).reshape(BH, N, d), ref_o)
    el = maxabs(f64(lse).reshape(BH, N), ref_l)
    _say(f"{what}: all {BH} heads max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL_BF16_O and el <= TOL_BF16_L
    if bwd:
        rq, rk, rv, _ = oracle.attn_bwd(arr["q"], arr["k"], arr["v"], arr["do"], scale, causal=causal)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            e = maxabs(f64(got).reshape(BH, N, d), ref)
            _say(f"{what}: all heads max|d{name}|={e:.3e}")
            assert e <= TOL_BF16_GRAD, f"{name} error {e}"
