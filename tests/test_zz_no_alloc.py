"""fa_bwd_noalloc (the backward without a caller workspace: D lives in the
library's static per-GPU array) against fa_bwd, through the C ABI.

Two calls in a row, the second smaller than the first (the array keeps the
previous call's contents, which the second call must not depend on), each
bitwise equal to fa_bwd on the same inputs; then a call beyond the array's
size is rejected with FA_ERR_SCRATCH and leaves the outputs untouched.
"""
import ctypes

import pytest
import torch

from io_aware_tiled_fwd_amd import binding, inputs
from gpu_util import upload

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def test_noalloc_backward_equals_fa_bwd():
    lib = binding.load_library()
    stream = torch.cuda.current_stream()
    for (B, H, N, d, causal, seed) in ((2, 4, 1000, 128, True, 2101), (1, 3, 300, 64, False, 2102)):
        print(f"noalloc: B{B} H{H} N{N} d{d} causal={causal}", flush=True)
        ts = inputs.normal_qkv(B, H, N, d, seed, with_dout=True)
        dev = upload(ts)
        scale = inputs.default_scale(d)
        o, lse = binding.attention_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
        ref = binding.attention_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=causal, scale=scale)
        got = [torch.full((B, H, N, d), float("nan"), device="cuda") for _ in range(3)]
        st = lib.fa_bwd_noalloc(_ptr(dev["q"]), _ptr(dev["k"]), _ptr(dev["v"]), _ptr(o), _ptr(lse),
                                _ptr(dev["do"]), *(_ptr(g) for g in got), B, H, N, d, ctypes.c_float(scale),
                                int(causal), ctypes.c_void_p(stream.cuda_stream))
        assert st == binding.FA_OK, binding.fa_status_string(st)
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            assert torch.equal(g, r)
    # beyond the static array: rejected before any launch, outputs untouched
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1, 64, device="cuda")
    out = torch.full((1, 1, 64, 64), 7.0, device="cuda")
    st = lib.fa_bwd_noalloc(*(_ptr(t) for t in (q, q, q, q, lse, q, out, out, out)), 1, 1,
                            binding.NOALLOC_MAX_ROWS + 64, 64, ctypes.c_float(0.125), 1,
                            ctypes.c_void_p(stream.cuda_stream))
    assert st == binding.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
