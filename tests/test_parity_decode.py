"""Split-KV decode on the GPU against the fp64 oracle, through the C ABI
(fa_decode).  Bars as for the bf16 forward: O max-abs <= 2e-2, L <= 1e-3."""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_fwd_amd import binding, inputs
from gpu_util import TOL_BF16_L, TOL_BF16_O, f64, maxabs, upload

pytestmark = pytest.mark.gpu


def _decode(dev, kv_len=None, splits=0, scale=None):
    lens = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    o, lse = binding.attention_decode(dev["q"], dev["k"], dev["v"], kv_len=lens, num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _check(what, o, lse, ref_o, ref_l):
    eo = maxabs(f64(o), ref_o)
    got_l = f64(lse)
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty), f"{what}: -inf pattern of L"
    el = maxabs(got_l[~empty], ref_l[~empty])
    print(f"{what}: O err {eo:.3e}  L err {el:.3e}", flush=True)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_L, what


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 1), (64, 1)])
def test_decode_small_shapes(d, Hq, Hkv):
    for Nk in (1, 31, 255, 257, 1000):
        ts = inputs.decode_qkv(3, Hq, Hkv, Nk, d, 500 + Nk)
        dev = upload(ts)
        scale = inputs.default_scale(d)
        for kv_len in (None, [Nk, max(Nk // 2, 1), 0]):
            ref_o, ref_l = oracle.attn_decode(ts.f64["q"], ts.f64["k"], ts.f64["v"], scale, kv_len=kv_len)
            for splits in (0, 1, 3):
                o, lse = _decode(dev, kv_len, splits, scale)
                _check(f"Hq={Hq} Hkv={Hkv} Nk={Nk} d={d} lens={kv_len} splits={splits}", o, lse, ref_o, ref_l)


def test_decode_long_cache_grouped():
    """A Llama-3-70B-like decode step (8 key/value heads, 64 query heads,
    d 128), batch 2 with cache lengths 32768 and 20001: every output."""
    B, Hq, Hkv, Nk, d = 2, 64, 8, 32768, 128
    ts = inputs.decode_qkv(B, Hq, Hkv, Nk, d, 20280)
    dev = upload(ts)
    scale = inputs.default_scale(d)
    lens = [32768, 20001]
    ref_o, ref_l = oracle.attn_decode(ts.f64["q"], ts.f64["k"], ts.f64["v"], scale, kv_len=lens)
    results = {}
    for splits in (0, 1, 7):
        o, lse = _decode(dev, lens, splits, scale)
        _check(f"long cache splits={splits}", o, lse, ref_o, ref_l)
        results[splits] = (o, lse)
    o2, lse2 = _decode(dev, lens, 0, scale)  # same split count: bitwise reproducible
    assert torch.equal(o2, results[0][0]) and torch.equal(lse2, results[0][1])


def test_decode_closed_forms():
    """kv_len 1: O = v_0 exactly (P = 1) and L = scale q.k_0; kv_len 0: O = 0,
    L = -inf."""
    B, Hq, Hkv, Nk, d = 2, 8, 2, 300, 128
    ts = inputs.decode_qkv(B, Hq, Hkv, Nk, d, 20281)
    dev = upload(ts)
    scale = inputs.default_scale(d)
    for splits in (0, 1):
        o, lse = _decode(dev, [1, 0], splits, scale)
        G = Hq // Hkv
        v0 = dev["v"][0, :, 0].repeat_interleave(G, dim=0)
        assert torch.equal(o[0], v0)
        want_l = scale * np.einsum("hd,hd->h", ts.f64["q"][0], np.repeat(ts.f64["k"][0, :, 0], G, axis=0))
        assert maxabs(f64(lse[0]), want_l) <= 1e-5
        assert torch.all(o[1] == 0) and torch.all(torch.isneginf(lse[1]))


def test_decode_equals_last_row_of_causal_forward():
    """A decode step over n cached keys is the last row of the causal forward
    over that sequence (both on the GPU, different kernels)."""
    B, Hq, Hkv, n, d = 1, 8, 2, 1100, 128
    ts = inputs.normal_gqa(B, Hq, Hkv, n, d, 20282)
    dev = upload(ts)
    scale = inputs.default_scale(d)
    o_f, l_f = binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale)
    q_last = dev["q"][:, :, -1].contiguous()
    o, lse = binding.attention_decode(q_last, dev["k"], dev["v"], scale=scale)
    torch.cuda.synchronize()
    assert maxabs(f64(o), f64(o_f[:, :, -1])) <= 2 * TOL_BF16_O
    assert maxabs(f64(lse), f64(l_f[:, :, -1])) <= 2 * TOL_BF16_L
