"""Code-generation checks on the built library (CPU only: reads the gfx950 code
objects inside libfa.so with the ROCm LLVM tools, runs nothing on a GPU).

* No kernel makes a function call.  The kernels are built without packed-fp32
  instructions and with IEEE mode off, so ROCm device-library functions
  (threadIdx / blockIdx accessors, __umulhi, ...) are not inlined into them and
  each use becomes an s_swappc_b64 call; the kernels read hardware registers and
  use builtins instead, and this test keeps it that way.
* The kernels of the measured paths spill no registers.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "io_aware_tiled_fwd_amd", "libfa.so")
LLVM = "/opt/rocm/llvm/bin"
TOOLS = {t: os.path.join(LLVM, t) for t in ("llvm-objcopy", "llvm-objdump", "llvm-readelf", "clang-offload-bundler")}
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# Kernels (mangled-name fragments) that must not spill: the bf16 forward, the
# backward stages and the decode, as the benchmark and the GPU tests run them.
NO_SPILL = [
    "fwd_bf16_kernelILi128ELb1ELb0E", "fwd_bf16_kernelILi128ELb0ELb0E",
    "fwd_bf16_kernelILi64ELb1ELb0E", "fwd_bf16_kernelILi64ELb0ELb0E",
    "fwd_bf16_kernelILi128ELb1ELb1E",
    "bwd_dkdv_fused_kernelILi128ELb1ELb0ELb0EfE", "bwd_dkdv_fused_kernelILi128ELb0ELb0ELb0EfE",
    "bwd_dkdv_fused_kernelILi128ELb1ELb1ELb0EfE", "bwd_dkdv_fused_kernelILi128ELb1ELb0ELb1EfE",
    "bwd_dkdv_kernelILi128ELb1ELb1ELb0ELb0EfE", "bwd_dkdv_kernelILi128ELb1ELb0ELb0ELb0EfE",
    "bwd_dq_kernelILi128ELb1ELb0EfE", "bwd_preprocess_kernelILi128E",
    "fwd_fp8_kernelILi128ELb1E", "decode_split_kernelILi128ELb1E", "decode_merge_kernelILi128E",
]


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    if not os.path.exists(LIB):
        pytest.skip("libfa.so is not built")
    if not all(os.path.exists(p) for p in TOOLS.values()):
        pytest.skip("ROCm LLVM tools not found")
    tmp = tmp_path_factory.mktemp("co")
    fatbin = tmp / "fatbin.bin"
    subprocess.run([TOOLS["llvm-objcopy"], f"--dump-section=.hip_fatbin={fatbin}", LIB, os.devnull], check=True)
    data = fatbin.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in .hip_fatbin"
    objs = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        chunk = tmp / f"bundle{n}.bin"
        chunk.write_bytes(data[a:b])
        co = tmp / f"code{n}.co"
        r = subprocess.run([TOOLS["clang-offload-bundler"], "--unbundle", "--type=o", f"--targets={TARGET}",
                            f"--input={chunk}", f"--output={co}"], capture_output=True)
        if r.returncode == 0 and co.exists() and co.stat().st_size > 0:
            objs.append(co)
    assert objs, "no gfx950 code object found"
    return objs


def test_no_function_calls(code_objects):
    with_kernels = 0
    for co in code_objects:
        dis = subprocess.run([TOOLS["llvm-objdump"], "-d", str(co)], capture_output=True, text=True, check=True).stdout
        if "s_endpgm" not in dis:
            continue  # a code object with device data only (the static workspace of fa_api.hip)
        with_kernels += 1
        calls = dis.count("s_swappc_b64")
        assert calls == 0, f"{co.name}: {calls} function calls (s_swappc_b64) in the kernels"
    assert with_kernels >= 5, "fewer kernel code objects than sources with kernels"


# Kernels whose MFMAs must not wait on outstanding global loads: their
# register-resident operands are waited for once before the tile loop, so a
# vmcnt wait in front of an MFMA would mean a stall on a prefetch.  A wait for
# vmcnt(n) with n at least the number of loads a tile step keeps in flight
# (the forward's steps: 4) cannot stall and is allowed: the persistent
# forward's task loop leaves such no-op waits where the compiler cannot prove
# that the operand's load has completed.
NO_LOAD_WAIT = {
    "fwd_bf16_kernelILi128ELb1ELb0E": 4, "fwd_bf16_kernelILi128ELb0ELb0E": 4,
    "bwd_dkdv_fused_kernelILi128ELb1ELb0ELb0EfE": 0, "bwd_dkdv_fused_kernelILi128ELb0ELb0ELb0EfE": 0,
}


def test_mfmas_do_not_wait_on_loads(code_objects):
    seen = set()
    for co in code_objects:
        dis = subprocess.run([TOOLS["llvm-objdump"], "-d", str(co)], capture_output=True, text=True, check=True).stdout
        cur, prev = None, ""
        for line in dis.splitlines():
            m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
            if m:
                cur, prev = m.group(1), ""
                continue
            if cur is None or not any(f in cur for f in NO_LOAD_WAIT):
                continue
            seen.update(f for f in NO_LOAD_WAIT if f in cur)
            ins = line.strip()
            if ins.startswith("v_mfma") and prev.startswith("s_waitcnt") and "vmcnt" in prev:
                n = int(re.search(r"vmcnt\((\d+)\)", prev).group(1))
                limit = next(v for f, v in NO_LOAD_WAIT.items() if f in cur)
                assert limit and n >= limit, f"{cur}: {prev} before {ins[:40]}"
            if ins:
                prev = ins
    assert seen == set(NO_LOAD_WAIT), f"kernels not found: {set(NO_LOAD_WAIT) - seen}"


def test_hot_kernels_do_not_spill(code_objects):
    spills = {}
    for co in code_objects:
        notes = subprocess.run([TOOLS["llvm-readelf"], "--notes", str(co)], capture_output=True, text=True,
                               check=True).stdout
        name = None
        for line in notes.splitlines():
            m = re.match(r"\s+\.name:\s+(\S+)", line)
            if m:
                name = m.group(1)
            m = re.match(r"\s+\.vgpr_spill_count:\s+(\d+)", line)
            if m and name:
                spills[name] = int(m.group(1))
    for frag in NO_SPILL:
        hits = {n: c for n, c in spills.items() if frag in n}
        assert hits, f"kernel {frag} not found in the code objects"
        for n, c in hits.items():
            assert c == 0, f"{n} spills {c} VGPRs"


# Kernels whose MFMA chains must keep their LDS operand reads ahead of them
# (pin_read_ahead in fa_bwd.hip), and the largest fraction of their MFMAs
# that may sit right behind an s_waitcnt lgkmcnt(0).  Without the pinned
# order the compiler issued each read just before its MFMA and waited for it
# there: 44% of the paired kernel's MFMAs and 36% of the causal dQ kernel's,
# against under 7% with it.
READ_AHEAD = {
    "bwd_dkdv_fused_kernelILi128ELb1ELb0ELb0EfE": 0.10, "bwd_dkdv_fused_kernelILi128ELb0ELb0ELb0EfE": 0.10,
    "bwd_dq_kernelILi128ELb1ELb0EfE": 0.10,
}


def test_backward_chains_read_ahead(code_objects):
    counts = {}
    for co in code_objects:
        dis = subprocess.run([TOOLS["llvm-objdump"], "-d", str(co)], capture_output=True, text=True, check=True).stdout
        cur, prev = None, ""
        for line in dis.splitlines():
            m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
            if m:
                cur, prev = m.group(1), ""
                continue
            frag = next((f for f in READ_AHEAD if cur and f in cur), None)
            ins = line.strip()
            if frag is None or not ins:
                continue
            if ins.startswith("v_mfma"):
                total, waited = counts.get(frag, (0, 0))
                counts[frag] = (total + 1, waited + (prev.startswith("s_waitcnt") and "lgkmcnt(0)" in prev))
            prev = ins
    assert set(counts) == set(READ_AHEAD), f"kernels not found: {set(READ_AHEAD) - set(counts)}"
    for frag, (total, waited) in counts.items():
        assert waited <= READ_AHEAD[frag] * total, f"{frag}: {waited} of {total} MFMAs right after lgkmcnt(0)"
