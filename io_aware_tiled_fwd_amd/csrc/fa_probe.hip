// fa_probe.hip -- measurement probes (see fa_probe.h): a register-only bf16
// MFMA loop and a non-temporal HBM read sweep.  Neither is part of the
// attention method; bench.py times them to report measured ceilings beside
// the published MI355X peaks.
#include "fa.h"
#include "fa_common.h"
#include "fa_probe.h"

namespace fa {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kReadBlocks = 256;
constexpr int kReadUnroll = 4;

// Four independent accumulator chains per wavefront (a single dependent chain
// issues more slowly), 16 MFMAs per iteration.
__global__ __launch_bounds__(kProbeThreads, 1) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
    const int tid = thread_id();
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (bf16)(tid * 0.001f + j);
        b[j] = (bf16)(j * 0.5f);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c0 = mfma_bf16_32x32x16(a, b, c0);
            c1 = mfma_bf16_32x32x16(a, b, c1);
            c2 = mfma_bf16_32x32x16(a, b, c2);
            c3 = mfma_bf16_32x32x16(a, b, c3);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
    sink[(size_t)block_id() * kProbeThreads + tid] = s;
}

// Grid-stride sweep: thread t reads chunks t, t + T, ... (T threads in all),
// kReadUnroll of them in flight.  The caller's size is a multiple of
// T * kReadUnroll chunks, so every read is inside the buffer.
__global__ __launch_bounds__(kProbeThreads, 1) void hbm_read_probe_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                          unsigned* __restrict__ sink) {
    const size_t nth = (size_t)kReadBlocks * kProbeThreads;
    const size_t tid = (size_t)block_id() * kProbeThreads + thread_id();
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t i = tid; i < n16; i += kReadUnroll * nth) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * nth);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
    }
    sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace
}  // namespace fa

extern "C" int fa_probe_mfma(int blocks, int iters, float* sink, hipStream_t stream) {
    if (blocks < 1 || iters < 1 || !sink) return FA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(fa::mfma_probe_kernel, dim3(blocks), dim3(fa::kProbeThreads), 0, stream, iters, sink);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_probe_hbm_read(const void* buf, size_t bytes, unsigned* sink, hipStream_t stream) {
    const size_t unit = (size_t)16 * fa::kProbeThreads * fa::kReadBlocks * fa::kReadUnroll;
    if (!buf || !sink || bytes == 0 || bytes % unit != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
        return FA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(fa::hbm_read_probe_kernel, dim3(fa::kReadBlocks), dim3(fa::kProbeThreads), 0, stream,
                       static_cast<const fa::u32x4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
