// fa_api.hip -- the C ABI declared in include/fa.h: argument checks, dispatch.
//
// Every check runs before any launch, so an invalid call leaves all outputs
// untouched and launches nothing.  No C++ exception can cross the ABI (nothing
// here throws; the launchers only call the HIP C API).
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_internal.h"

// Static workspace of fa_bwd_noalloc: the backward's D = rowsum(dO * O) for up
// to FA_NOALLOC_MAX_ROWS rows (16 MiB), in the library's own device memory so
// that the entry point allocates nothing.  Each GPU the library runs on holds
// its own copy until the process ends.  Host code must never use this name as
// a device address (it is a host-side stand-in); it uses the address that
// hipGetSymbolAddress reports for the current device (noalloc_scratch below).
static __device__ __align__(256) float scratch[FA_NOALLOC_MAX_ROWS];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Any finite scale, of either sign or zero ("FlashAttention" deep-dive page,
// "How it works": S = Q K^T times the scale), as long as the kernels' exponent
// factor |scale| log2(e) is a finite fp32 value.
bool scale_ok(float scale) { return isfinite(scale) && isfinite(fabsf(scale) * 1.4426950408889634f); }

// Shared shape checks.  Returns FA_OK or the status to report.
int check_shape(int B, int H, int N, int d, float scale) {
    if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
    if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
    const int64_t bh = (int64_t)B * H;
    if (bh > INT32_MAX) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    // Element offsets are 64-bit; also keep the flat workgroup count < 2^31.
    if ((double)bh * (double)N * (double)d >= 4.611686018427388e18) return FA_ERR_INVALID_ARG;  // 2^62
    if ((double)bh * (double)((N + 63) / 64) >= 2147483647.0) return FA_ERR_INVALID_ARG;
    // One head of one fp32 [N, d] tensor is addressed through a 32-bit byte range.
    if ((double)N * (double)d * 4.0 > 2147483647.0) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

// Grouped heads: Hq query heads share Hkv key/value heads, Hkv dividing Hq.
int check_groups(int Hq, int Hkv) { return (Hkv < 1 || Hq % Hkv != 0) ? FA_ERR_INVALID_ARG : FA_OK; }

// Decode shapes: q [B, Hq, d], cache [B, Hkv, Nk, d].
int check_decode(int B, int Hq, int Hkv, int Nk, int d, int num_splits) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Nk < 1 || num_splits < 0) return FA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hq > INT32_MAX) return FA_ERR_INVALID_ARG;
    // One head of the cache is addressed through a 32-bit byte range.
    if ((double)Nk * (double)d * 2.0 > 2147483647.0) return FA_ERR_INVALID_ARG;
    if ((double)B * (double)Hkv * (double)Nk * (double)d >= 4.611686018427388e18) return FA_ERR_INVALID_ARG;
    // Workgroups: B * Hkv * ceil(G / 32) * splits, splits <= ceil(Nk / 256).
    const double groups = (double)B * Hkv * (double)((Hq / Hkv + 31) / 32);
    if (groups * (double)((Nk + 255) / 256) >= 2147483647.0) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

size_t decode_workspace_bytes(const fa::DecodePlan& p, int B, int Hq, int d) {
    return p.splits > 1 ? (size_t)p.splits * (size_t)B * (size_t)Hq * (size_t)(d + 2) * sizeof(float) : 0;
}

// Dropout probability in [0, 1); the offset is one 32-bit Philox counter word.
int check_dropout(float p, unsigned long long offset) {
    if (!(p >= 0.f && p < 1.f) || offset > 0xFFFFFFFFull) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

// thr = floor(256 p + 1/2) (at most 255): bytes below it are dropped.
fa::DropoutParams dropout_params(float p, unsigned long long seed, unsigned long long offset) {
    int thr = (int)floor(256.0 * (double)p + 0.5);
    if (thr > 255) thr = 255;
    return fa::DropoutParams{(uint32_t)thr, (float)(256.0 / (256.0 - thr)), (uint32_t)seed, (uint32_t)(seed >> 32),
                             (uint32_t)offset};
}

int from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(float** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
               int d, float scale, int causal, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    int st = check_shape(B, Hq, N, d, scale);
    if (st == FA_OK) st = check_groups(Hq, Hkv);
    if (st != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal != 0, nullptr, stream));
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, hipStream_t stream) {
    return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, scale, causal, stream);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
                   int d, float scale, int causal, float dropout_p, unsigned long long seed, unsigned long long offset,
                   hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    int st = check_shape(B, Hq, N, d, scale);
    if (st == FA_OK) st = check_groups(Hq, Hkv);
    if (st == FA_OK) st = check_dropout(dropout_p, offset);
    if (st != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    const fa::DropoutParams dp = dropout_params(dropout_p, seed, offset);
    return from_hip(fa::launch_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal != 0, &dp, stream));
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                   float* dq, float* dk, float* dv, float* delta, int B, int Hq, int Hkv, int N, int d, float scale,
                   int causal, float dropout_p, unsigned long long seed, unsigned long long offset,
                   hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !delta) return FA_ERR_INVALID_ARG;
    int st = check_shape(B, Hq, N, d, scale);
    if (st == FA_OK) st = check_groups(Hq, Hkv);
    if (st == FA_OK) st = check_dropout(dropout_p, offset);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv, delta};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    const fa::DropoutParams dp = dropout_params(dropout_p, seed, offset);
    return from_hip(fa::launch_bwd_bf16(q, k, v, o, lse, dO, dq, dk, dv, delta, B, Hq, Hkv, N, d, scale,
                                        causal != 0, &dp, false, stream));
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N, int d,
               float scale, float q_descale, float k_descale, float v_descale, int causal, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    int st = check_shape(B, Hq, N, d, scale);
    if (st == FA_OK) st = check_groups(Hq, Hkv);
    if (st != FA_OK) return st;
    const float ds[] = {q_descale, k_descale, v_descale};
    for (float x : ds)
        if (!isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID_ARG;
    if (!isfinite(fabsf(scale) * q_descale * k_descale * 1.4426950408889634f)) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, q_descale, k_descale, v_descale,
                                       causal != 0, stream));
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
               int d, float scale, int causal, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_fwd_f32(q, k, v, o, lse, B * H, N, d, scale, causal != 0, stream));
}

int fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
               float* dq, float* dk, float* dv, float* delta, int B, int Hq, int Hkv, int N, int d, float scale,
               int causal, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !delta) return FA_ERR_INVALID_ARG;
    int st = check_shape(B, Hq, N, d, scale);
    if (st == FA_OK) st = check_groups(Hq, Hkv);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv, delta};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_bwd_bf16(q, k, v, o, lse, dO, dq, dk, dv, delta, B, Hq, Hkv, N, d, scale,
                                        causal != 0, nullptr, false, stream));
}

int fa_bwd_gqa_bf16grad(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                        void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv, int N, int d, float scale,
                        int causal, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !delta) return FA_ERR_INVALID_ARG;
    int st = check_shape(B, Hq, N, d, scale);
    if (st == FA_OK) st = check_groups(Hq, Hkv);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv, delta};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_bwd_bf16(q, k, v, o, lse, dO, dq, dk, dv, delta, B, Hq, Hkv, N, d, scale,
                                        causal != 0, nullptr, true, stream));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
           float* dq, float* dk, float* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
           hipStream_t stream) {
    return fa_bwd_gqa(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, H, N, d, scale, causal, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                   float* dq, float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
                   hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    if ((int64_t)B * H * N > (int64_t)FA_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
    float* delta = nullptr;
    const int sst = noalloc_scratch(&delta);
    if (sst != FA_OK) return sst;
    // Every element of delta that the kernels read is written by the
    // preprocess kernel first, in stream order, so nothing needs clearing.
    return from_hip(fa::launch_bwd_bf16(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, H, N, d, scale, causal != 0,
                                        nullptr, false, stream));
}

int fa_bwd_preprocess(const void* o, const void* dO, float* delta, int B, int H, int N, int d,
                      hipStream_t stream) {
    if (!o || !dO || !delta) return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, 1.0f);
    if (st != FA_OK) return st;
    if (!aligned16(o) || !aligned16(dO) || !aligned16(delta)) return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_bwd_preprocess(o, dO, delta, B * H, N, d, stream));
}

int fa_bwd_dv(const void* q, const void* k, const float* lse, const void* dO, float* dv, int B, int H, int N, int d,
              float scale, int causal, hipStream_t stream) {
    if (!q || !k || !lse || !dO || !dv) return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, lse, dO, dv};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_bwd_dv(q, k, lse, dO, dv, B, H, H, N, d, scale, causal != 0, nullptr, false, stream));
}

int fa_bwd_dk(const void* q, const void* k, const void* v, const float* lse, const void* dO, const float* delta,
              float* dk, int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
    if (!q || !k || !v || !lse || !dO || !delta || !dk) return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, lse, dO, delta, dk};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    return from_hip(
        fa::launch_bwd_dk(q, k, v, lse, dO, delta, dk, B, H, H, N, d, scale, causal != 0, nullptr, false, stream));
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dO, const float* delta,
                float* dk, float* dv, int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
    if (!q || !k || !v || !lse || !dO || !delta || !dk || !dv) return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, lse, dO, delta, dk, dv};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_bwd_dkdv(q, k, v, lse, dO, delta, dk, dv, B, H, H, N, d, scale, causal != 0, nullptr,
                                        false, stream));
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO, const float* delta,
              float* dq, int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
    if (!q || !k || !v || !lse || !dO || !delta || !dq) return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, lse, dO, delta, dq};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    return from_hip(
        fa::launch_bwd_dq(q, k, v, lse, dO, delta, dq, B, H, H, N, d, scale, causal != 0, nullptr, false, stream));
}

int fa_decode_plan(int B, int Hq, int Hkv, int Nk, int d, int num_splits, int* splits, size_t* workspace_bytes) {
    const int st = check_decode(B, Hq, Hkv, Nk, d, num_splits);
    if (st != FA_OK) return st;
    const fa::DecodePlan p = fa::decode_plan(B, Hq, Hkv, Nk, num_splits);
    if (splits) *splits = p.splits;
    if (workspace_bytes) *workspace_bytes = decode_workspace_bytes(p, B, Hq, d);
    return FA_OK;
}

int fa_decode(const void* q, const void* k, const void* v, const int* kv_len, void* o, float* lse, int B, int Hq,
              int Hkv, int Nk, int d, float scale, int num_splits, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    const int st = check_decode(B, Hq, Hkv, Nk, d, num_splits);
    if (st != FA_OK) return st;
    if (!scale_ok(scale)) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_INVALID_ARG;
    if (kv_len && (reinterpret_cast<uintptr_t>(kv_len) & 3u) != 0) return FA_ERR_INVALID_ARG;
    const fa::DecodePlan p = fa::decode_plan(B, Hq, Hkv, Nk, num_splits);
    const size_t need = decode_workspace_bytes(p, B, Hq, d);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_decode(q, k, v, kv_len, o, lse, B, Hq, Hkv, Nk, d, scale, p,
                                      static_cast<float*>(workspace), stream));
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG:
            return "FA_ERR_INVALID_ARG: null pointer, misaligned pointer, bad size or head count, or a scale whose "
                   "magnitude times log2(e) is not a finite float";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension must be 64 or 128";
        case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error at launch";
        case FA_ERR_SCRATCH:
            return "FA_ERR_SCRATCH: B*H*N exceeds the static workspace of fa_bwd_noalloc (FA_NOALLOC_MAX_ROWS rows)";
        default: return "unknown fa_status";
    }
}

}  // extern "C"
