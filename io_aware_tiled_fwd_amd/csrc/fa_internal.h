// fa_internal.h -- launchers behind the C ABI (argument checks happen in fa_api.hip).
//
// Head layout: q, o, dO, dq and the [*, N] statistics have B * Hq heads;
// k, v, dk, dv have B * Hkv heads, Hkv dividing Hq.  Query head h of batch b
// reads key/value head h / (Hq / Hkv) of batch b (Hkv = Hq: one to one).
#pragma once
#include <hip/hip_runtime.h>

#include "fa_common.h"

namespace fa {

// Workgroups per XCD for a persistent launch over `tasks` tasks: as many as
// fit on the XCD's CUs at once (blocks_per_cu per CU of the current device,
// whose compute units are split evenly over the 8 XCDs), fewer for small
// grids.  The grid is kNumXcd times this.
int persistent_per_xcd(int tasks, int blocks_per_cu);

// Workgroups of one kernel that fit on a CU at once, looked up once per
// kernel (keyed by its address: instantiations that share a signature differ
// in their register and LDS use).
int blocks_per_cu_of(const void* kernel, int threads);
template <typename Kern>
int blocks_per_cu(Kern kernel, int threads) {
    return blocks_per_cu_of(reinterpret_cast<const void*>(kernel), threads);
}

// Forward, bf16 in/out.  d in {64, 128}.  dropout: null for none.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                           int Hkv, int N, int d, float scale, bool causal, const DropoutParams* dropout,
                           hipStream_t stream);
// Forward, fp32 in/out (one key/value head per query head).
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH,
                          int N, int d, float scale, bool causal, hipStream_t stream);
// Backward: preprocess (delta), dK/dV and dQ kernels, in stream order.
// dropout: null for none, else the forward's mask is regenerated.
// grad_bf16: dq, dk, dv are bf16 (no dropout then), else fp32.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int Hq,
                           int Hkv, int N, int d, float scale, bool causal, const DropoutParams* dropout,
                           bool grad_bf16, hipStream_t stream);

// The backward's stages, individually.
hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, int BHq, int N, int d,
                                 hipStream_t stream);
hipError_t launch_bwd_dv(const void* q, const void* k, const float* lse, const void* dout, void* dv, int B,
                         int Hq, int Hkv, int N, int d, float scale, bool causal, const DropoutParams* dropout,
                         bool grad_bf16, hipStream_t stream);
hipError_t launch_bwd_dk(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, void* dk, int B, int Hq, int Hkv, int N, int d, float scale,
                         bool causal, const DropoutParams* dropout, bool grad_bf16, hipStream_t stream);
// dK and dV together (one kernel of paired wavefronts; bitwise equal to the two above).
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                           const float* delta, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, float scale,
                           bool causal, const DropoutParams* dropout, bool grad_bf16, hipStream_t stream);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, void* dq, int B, int Hq, int Hkv, int N, int d, float scale,
                         bool causal, const DropoutParams* dropout, bool grad_bf16, hipStream_t stream);

// Forward with fp8 (OCP e4m3) q, k, v and one dequantisation factor per
// tensor; bf16 o, fp32 lse.  Grouped heads as for launch_fwd_bf16.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                          int N, int d, float scale, float q_descale, float k_descale, float v_descale, bool causal,
                          hipStream_t stream);

// Split-KV decode.  q, o [B, Hq, d], lse [B, Hq]; k, v [B, Hkv, Nk, d];
// kv_len [B] (device, may be null).  The plan fixes the split of the cache:
// `splits` chunks of `chunk` keys (a multiple of 256), query heads of a group
// in `nqg` blocks of 32.  With splits > 1 the workspace holds the splits'
// partial triples: splits * B * Hq * (d + 2) floats.
struct DecodePlan {
    int splits, chunk, nqg;
};
DecodePlan decode_plan(int B, int Hq, int Hkv, int Nk, int num_splits);
hipError_t launch_decode(const void* q, const void* k, const void* v, const int* kv_len, void* o, float* lse, int B,
                         int Hq, int Hkv, int Nk, int d, float scale, const DecodePlan& plan, float* workspace,
                         hipStream_t stream);

}  // namespace fa
