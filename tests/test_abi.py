"""The C ABI without a GPU: the library loads, exports what include/fa.h
declares, and rejects bad arguments before touching the device.

Only calls that the library's argument checks reject are made here; those
return before any HIP call, so no device is needed.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    """Function names declared in include/*.h (int/const char* returning)."""
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def lib():
    from io_aware_tiled_fwd_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libfa.so is not built (python -m io_aware_tiled_fwd_amd.build)")
    return binding.load_library()


def test_header_declares_the_entry_points():
    assert set(declared_functions()) >= {"fa_fwd", "fa_fwd_f32", "fa_bwd", "fa_status_string"}


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libfa.so does not export {name}"


def test_binding_names_match_header():
    from io_aware_tiled_fwd_amd import binding
    assert set(binding.SYMBOLS) == set(declared_functions())
    for name in binding.SYMBOLS:
        assert callable(getattr(binding, name))


def test_status_strings(lib):
    from io_aware_tiled_fwd_amd import binding
    assert binding.fa_status_string(0) == "FA_OK"
    for st in (1, 2, 3, 4):
        assert binding.fa_status_string(st).startswith("FA_ERR_")
    assert "unknown" in binding.fa_status_string(99)


# A non-null, 16-byte aligned fake address: every call below is rejected by the
# argument checks before any pointer is used or any kernel launched.
FAKE = ctypes.c_void_p(0x1000)
NUL = ctypes.c_void_p(0)


def _fwd(lib, ptrs, B=1, H=1, N=16, d=64, scale=0.125, causal=0, f32=False):
    fn = lib.fa_fwd_f32 if f32 else lib.fa_fwd
    return fn(*ptrs, B, H, N, d, ctypes.c_float(scale), causal, NUL)


@pytest.mark.parametrize("f32", [False, True])
def test_fwd_rejects_bad_arguments(lib, f32):
    ok = [FAKE] * 5
    for i in range(5):  # each null pointer
        ptrs = list(ok)
        ptrs[i] = NUL
        assert _fwd(lib, ptrs, f32=f32) == 1
    assert _fwd(lib, ok, B=0, f32=f32) == 1
    assert _fwd(lib, ok, H=-1, f32=f32) == 1
    assert _fwd(lib, ok, N=0, f32=f32) == 1
    assert _fwd(lib, ok, scale=float("nan"), f32=f32) == 1
    assert _fwd(lib, ok, scale=float("inf"), f32=f32) == 1
    # any finite scale is accepted unless |scale| log2(e) overflows fp32
    assert _fwd(lib, ok, scale=3.0e38, f32=f32) == 1
    assert _fwd(lib, ok, scale=-3.0e38, f32=f32) == 1
    assert _fwd(lib, ok, d=96, f32=f32) == 2
    assert _fwd(lib, ok, d=256, f32=f32) == 2
    assert _fwd(lib, ok, d=0, f32=f32) == 2
    # 2^62 elements or more
    assert _fwd(lib, ok, B=2 ** 20, H=2 ** 10, N=2 ** 25, d=128, f32=f32) == 1
    # misaligned pointer
    ptrs = list(ok)
    ptrs[2] = ctypes.c_void_p(0x1002)
    assert _fwd(lib, ptrs, f32=f32) == 1


def test_bwd_rejects_bad_arguments(lib):
    ok = [FAKE] * 10

    def call(ptrs, B=1, H=1, N=16, d=128, scale=0.1):
        return lib.fa_bwd(*ptrs, B, H, N, d, ctypes.c_float(scale), 1, NUL)

    for i in range(10):
        ptrs = list(ok)
        ptrs[i] = NUL
        assert call(ptrs) == 1
    assert call(ok, B=0) == 1
    assert call(ok, scale=float("-inf")) == 1
    assert call(ok, d=80) == 2
    ptrs = list(ok)
    ptrs[9] = ctypes.c_void_p(0x1004)
    assert call(ptrs) == 1


def test_bwd_stages_reject_bad_arguments(lib):
    """The backward stage entry points check pointers, shapes and alignment
    before any launch (fa_bwd_dkdv: q, k, v, lse, dO, delta, dk, dv)."""
    ok = [FAKE] * 8

    def dkdv(ptrs, B=1, H=1, N=16, d=128, scale=0.1):
        return lib.fa_bwd_dkdv(*ptrs, B, H, N, d, ctypes.c_float(scale), 1, NUL)

    for i in range(8):
        ptrs = list(ok)
        ptrs[i] = NUL
        assert dkdv(ptrs) == 1
    assert dkdv(ok, N=0) == 1
    assert dkdv(ok, scale=float("nan")) == 1
    assert dkdv(ok, d=96) == 2
    ptrs = list(ok)
    ptrs[7] = ctypes.c_void_p(0x1004)
    assert dkdv(ptrs) == 1
    assert lib.fa_bwd_dv(*([FAKE] * 4 + [NUL]), 1, 1, 16, 128, ctypes.c_float(0.1), 1, NUL) == 1
    assert lib.fa_bwd_dk(*([FAKE] * 7), 1, 1, 16, 80, ctypes.c_float(0.1), 1, NUL) == 2
    assert lib.fa_bwd_dq(*([FAKE] * 6 + [NUL]), 1, 1, 16, 128, ctypes.c_float(0.1), 1, NUL) == 1


def test_gqa_rejects_bad_arguments(lib):
    """Grouped heads: Hkv must be >= 1 and divide Hq; the shape checks of the
    per-head entry points apply to Hq."""
    def fwd(ptrs, B=1, Hq=4, Hkv=2, N=16, d=128, scale=0.1):
        return lib.fa_fwd_gqa(*ptrs, B, Hq, Hkv, N, d, ctypes.c_float(scale), 1, NUL)

    def bwd(ptrs, B=1, Hq=4, Hkv=2, N=16, d=128, scale=0.1):
        return lib.fa_bwd_gqa(*ptrs, B, Hq, Hkv, N, d, ctypes.c_float(scale), 1, NUL)

    def bwd16(ptrs, B=1, Hq=4, Hkv=2, N=16, d=128, scale=0.1):
        return lib.fa_bwd_gqa_bf16grad(*ptrs, B, Hq, Hkv, N, d, ctypes.c_float(scale), 1, NUL)

    for call, n in ((fwd, 5), (bwd, 10), (bwd16, 10)):
        ok = [FAKE] * n
        for i in range(n):
            ptrs = list(ok)
            ptrs[i] = NUL
            assert call(ptrs) == 1
        assert call(ok, Hkv=0) == 1
        assert call(ok, Hkv=-2) == 1
        assert call(ok, Hq=6, Hkv=4) == 1
        assert call(ok, Hq=2, Hkv=4) == 1
        assert call(ok, Hq=0, Hkv=1) == 1
        assert call(ok, d=96) == 2
        assert call(ok, scale=float("nan")) == 1


def test_fp8_rejects_bad_arguments(lib):
    def call(ptrs, B=1, Hq=4, Hkv=2, N=16, d=128, scale=0.1, qd=0.01, kd=0.01, vd=0.01):
        return lib.fa_fwd_fp8(*ptrs, B, Hq, Hkv, N, d, ctypes.c_float(scale), ctypes.c_float(qd), ctypes.c_float(kd),
                              ctypes.c_float(vd), 1, NUL)

    ok = [FAKE] * 5
    for i in range(5):
        ptrs = list(ok)
        ptrs[i] = NUL
        assert call(ptrs) == 1
    assert call(ok, Hkv=3) == 1
    assert call(ok, d=96) == 2
    assert call(ok, scale=float("nan")) == 1
    for bad in (0.0, -0.5, float("nan"), float("inf")):
        assert call(ok, qd=bad) == 1
        assert call(ok, kd=bad) == 1
        assert call(ok, vd=bad) == 1
    assert call(ok, scale=1e30, qd=1e30, kd=1e30) == 1  # folded exponent scale overflows
    assert call(ok, scale=-1e30, qd=1e30, kd=1e30) == 1
    ptrs = list(ok)
    ptrs[1] = ctypes.c_void_p(0x1001)
    assert call(ptrs) == 1


def test_dropout_rejects_bad_arguments(lib):
    def fwd(ptrs, p=0.1, offset=0, Hq=4, Hkv=2, d=128, scale=0.1):
        return lib.fa_fwd_dropout(*ptrs, 1, Hq, Hkv, 16, d, ctypes.c_float(scale), 1, ctypes.c_float(p), 7, offset,
                                  NUL)

    def bwd(ptrs, p=0.1, offset=0, Hq=4, Hkv=2, d=128, scale=0.1):
        return lib.fa_bwd_dropout(*ptrs, 1, Hq, Hkv, 16, d, ctypes.c_float(scale), 1, ctypes.c_float(p), 7, offset,
                                  NUL)

    for call, n in ((fwd, 5), (bwd, 10)):
        ok = [FAKE] * n
        for i in range(n):
            ptrs = list(ok)
            ptrs[i] = NUL
            assert call(ptrs) == 1
        for p in (-0.01, 1.0, 1.5, float("nan")):
            assert call(ok, p=p) == 1
        assert call(ok, offset=2 ** 32) == 1
        assert call(ok, Hkv=3) == 1
        assert call(ok, d=96) == 2
        assert call(ok, scale=float("nan")) == 1


def test_decode_plan(lib):
    """Split count and workspace size: host arithmetic only."""
    from io_aware_tiled_fwd_amd import binding
    # B1 Hq64 Hkv8 Nk131072 d128: automatic -> 256 workgroups / 8 groups = 32
    # splits of 4096 keys; workspace = splits * B * Hq * (d + 2) floats.
    assert binding.fa_decode_plan(1, 64, 8, 131072, 128) == (32, 32 * 64 * 130 * 4)
    # short caches: splits of at least 2048 keys (1024 below 64 workgroups)
    assert binding.fa_decode_plan(1, 64, 8, 32768, 128)[0] == 16
    assert binding.fa_decode_plan(1, 64, 8, 8192, 128)[0] == 8
    assert binding.fa_decode_plan(16, 32, 32, 8192, 128)[0] == 1
    assert binding.fa_decode_plan(1, 64, 8, 131072, 128, num_splits=1) == (1, 0)
    # at most ceil(Nk / 256) splits, chunks a multiple of 256 keys
    assert binding.fa_decode_plan(2, 4, 4, 1000, 64, num_splits=1000) == (4, 4 * 8 * 66 * 4)
    assert binding.fa_decode_plan(2, 4, 4, 1000, 64, num_splits=3) == (2, 2 * 8 * 66 * 4)
    assert binding.fa_decode_plan(2, 4, 4, 1, 64) == (1, 0)
    # G = 64 query heads per key/value head: two groups of 32 per split
    assert binding.fa_decode_plan(1, 64, 1, 65536, 128)[0] == 32
    for bad in ((0, 4, 4, 16, 64, 0), (1, 4, 3, 16, 64, 0), (1, 4, 4, 0, 64, 0), (1, 4, 4, 16, 64, -1)):
        assert lib.fa_decode_plan(*bad, None, None) == 1
    assert lib.fa_decode_plan(1, 4, 4, 16, 96, 0, None, None) == 2


def test_decode_rejects_bad_arguments(lib):
    """Every call here is rejected by the argument checks (no launch)."""
    def call(ptrs, kv_len=NUL, B=1, Hq=8, Hkv=2, Nk=4096, d=128, scale=0.1, splits=4, ws=FAKE, ws_bytes=1 << 30):
        return lib.fa_decode(*ptrs[:3], kv_len, *ptrs[3:], B, Hq, Hkv, Nk, d, ctypes.c_float(scale), splits, ws,
                             ws_bytes, NUL)

    ok = [FAKE] * 5  # q, k, v, o, lse
    for i in range(5):
        ptrs = list(ok)
        ptrs[i] = NUL
        assert call(ptrs) == 1
    assert call(ok, B=0) == 1
    assert call(ok, Hkv=3) == 1
    assert call(ok, Nk=0) == 1
    assert call(ok, d=96) == 2
    assert call(ok, scale=float("nan")) == 1
    assert call(ok, scale=-3.0e38) == 1
    assert call(ok, splits=-1) == 1
    assert call(ok, ws=NUL) == 1                  # 4 splits need a workspace
    assert call(ok, ws_bytes=4 * 8 * 130 * 4 - 4) == 1  # one float short
    assert call(ok, ws=ctypes.c_void_p(0x1008)) == 1   # misaligned workspace
    assert call(ok, kv_len=ctypes.c_void_p(0x1002), ws_bytes=0) == 1
    ptrs = list(ok)
    ptrs[4] = ctypes.c_void_p(0x1004)
    assert call(ptrs, ws_bytes=0) == 1
    assert call(ok, Nk=2 ** 24, d=128, ws_bytes=0) == 1  # one cache head over 2^31 bytes


def test_package_import_does_not_load_library():
    import importlib
    import io_aware_tiled_fwd_amd.inputs  # noqa: F401
    pkg = importlib.import_module("io_aware_tiled_fwd_amd")
    assert "fa_fwd" in pkg.__all__


def test_oracle_and_gpu_path_share_no_code():
    """Neither side imports or includes the other."""
    pkg = os.path.join(ROOT, "io_aware_tiled_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in re.sub(r"(#|//).*", "", text).lower() or f == "inputs.py", f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "io_aware_tiled_fwd_amd" not in text and "fa_common" not in text, f


def test_probe_rejections(lib):
    """The measurement probes check their arguments before any launch."""
    FA_ERR_INVALID_ARG = 1
    sink = FAKE
    assert lib.fa_probe_mfma(0, 10, sink, None) == FA_ERR_INVALID_ARG
    assert lib.fa_probe_mfma(4, 0, sink, None) == FA_ERR_INVALID_ARG
    assert lib.fa_probe_mfma(4, 10, None, None) == FA_ERR_INVALID_ARG
    unit = 16 * 512 * 256 * 4
    assert lib.fa_probe_hbm_read(sink, unit + 16, sink, None) == FA_ERR_INVALID_ARG
    assert lib.fa_probe_hbm_read(sink, 0, sink, None) == FA_ERR_INVALID_ARG
    assert lib.fa_probe_hbm_read(None, unit, sink, None) == FA_ERR_INVALID_ARG
    assert lib.fa_probe_hbm_read(ctypes.c_void_p(0x1008), unit, sink, None) == FA_ERR_INVALID_ARG


def test_bwd_noalloc_rejects_bad_arguments(lib):
    """fa_bwd_noalloc: the argument checks of fa_bwd, plus FA_ERR_SCRATCH when
    B*H*N exceeds its static workspace -- all before any HIP call."""
    from io_aware_tiled_fwd_amd import binding
    ok = [FAKE] * 9

    def call(ptrs, B=1, H=1, N=16, d=128, scale=0.1):
        return lib.fa_bwd_noalloc(*ptrs, B, H, N, d, ctypes.c_float(scale), 1, NUL)

    for i in range(9):
        ptrs = list(ok)
        ptrs[i] = NUL
        assert call(ptrs) == 1
    assert call(ok, N=0) == 1
    assert call(ok, d=96) == 2
    assert call(ok, scale=float("nan")) == 1
    ptrs = list(ok)
    ptrs[3] = ctypes.c_void_p(0x1004)
    assert call(ptrs) == 1
    assert call(ok, B=1, H=1, N=binding.NOALLOC_MAX_ROWS + 1, d=64) == 4
    assert call(ok, B=4, H=32, N=binding.NOALLOC_MAX_ROWS // 64, d=128) == 4
