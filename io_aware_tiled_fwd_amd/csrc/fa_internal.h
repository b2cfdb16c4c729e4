// fa_internal.h -- launchers behind the C ABI (argument checks happen in fa_api.hip).
#pragma once
#include <hip/hip_runtime.h>

namespace fa {

// Forward, bf16 in/out.  BH = batch * heads; d in {64, 128}.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                           int d, float scale, bool causal, hipStream_t stream);
// Forward, fp32 in/out.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH,
                          int N, int d, float scale, bool causal, hipStream_t stream);
// Backward: preprocess (delta), dK/dV kernel, dQ kernel, in stream order.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, float* delta, int BH, int N,
                           int d, float scale, bool causal, hipStream_t stream);

// The backward's stages, individually.
hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, int BH, int N, int d,
                                 hipStream_t stream);
hipError_t launch_bwd_dv(const void* q, const void* k, const float* lse, const void* dout, float* dv, int BH,
                         int N, int d, float scale, bool causal, hipStream_t stream);
hipError_t launch_bwd_dk(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, float* dk, int BH, int N, int d, float scale, bool causal,
                         hipStream_t stream);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, float* dq, int BH, int N, int d, float scale, bool causal,
                         hipStream_t stream);

}  // namespace fa
