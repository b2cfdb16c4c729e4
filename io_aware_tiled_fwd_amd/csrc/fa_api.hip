// fa_api.hip -- the C ABI declared in include/fa.h: argument checks, dispatch.
//
// Every check runs before any launch, so an invalid call leaves all outputs
// untouched and launches nothing.  No C++ exception can cross the ABI (nothing
// here throws; the launchers only call the HIP C API).
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape checks.  Returns FA_OK or the status to report.
int check_shape(int B, int H, int N, int d, float scale) {
    if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
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

int from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

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
    return from_hip(fa::launch_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal != 0, stream));
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, hipStream_t stream) {
    return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, scale, causal, stream);
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
                                        causal != 0, stream));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
           float* dq, float* dk, float* dv, float* delta, int B, int H, int N, int d, float scale, int causal,
           hipStream_t stream) {
    return fa_bwd_gqa(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, H, N, d, scale, causal, stream);
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
    return from_hip(fa::launch_bwd_dv(q, k, lse, dO, dv, B, H, H, N, d, scale, causal != 0, stream));
}

int fa_bwd_dk(const void* q, const void* k, const void* v, const float* lse, const void* dO, const float* delta,
              float* dk, int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
    if (!q || !k || !v || !lse || !dO || !delta || !dk) return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, lse, dO, delta, dk};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_bwd_dk(q, k, v, lse, dO, delta, dk, B, H, H, N, d, scale, causal != 0, stream));
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO, const float* delta,
              float* dq, int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
    if (!q || !k || !v || !lse || !dO || !delta || !dq) return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, scale);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, lse, dO, delta, dq};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_bwd_dq(q, k, v, lse, dO, delta, dq, B, H, H, N, d, scale, causal != 0, stream));
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG:
            return "FA_ERR_INVALID_ARG: null pointer, misaligned pointer, bad size or head count, or non-finite scale";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension must be 64 or 128";
        case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error at launch";
        default: return "unknown fa_status";
    }
}

}  // extern "C"
