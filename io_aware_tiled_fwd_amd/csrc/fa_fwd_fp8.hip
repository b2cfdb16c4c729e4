// fa_fwd_fp8.hip -- FlashAttention forward with fp8 inputs for gfx950 (MI355X).
//
// The deep-dive pages name low-precision (fp8) attention as a later step of
// the method: the same tiled loop with both matrix products on the fp8 tensor
// units ("FlashAttention" deep-dive page, "Implementation notes"; "Why Flash
// Attention Is Fast", section on FlashAttention-3).  Here Q, K and V are OCP
// fp8 e4m3 values with one dequantisation factor per tensor (real value =
// factor * stored value).  Per tile of 64 keys:
//   S^T  = K Q^T         v_mfma_f32_32x32x64_f8f6f4, fp32 accumulation of exact
//                        fp8 x fp8 products; the factors of Q and K and the
//                        softmax scale are folded into one exponent scale
//   P    = 2^(S c - m)   fp32, lagging running max m as in the bf16 kernel,
//                        so 0 <= P < 2^8 (inside e4m3's range, max 448)
//   l   += rowsum(P)     from the fp32 P
//   O^T += V^T P~^T      P~ = P rounded to e4m3 (the only rounding the fp8
//                        path adds), fp8 MFMA, fp32 accumulation
// and finally O = acc * factor_V / l (bf16) and L = (m + log2 l) ln 2.
//
// The structure is that of the bf16 kernel (fa_fwd.hip): 8 wavefronts x 32
// query rows per workgroup, K and V^T staged once per tile in double-buffered
// LDS for all eight wavefronts, one barrier per tile, XCD-contiguous head-major
// task order, causal tiles skipped or masked.  What changes with fp8:
//  - an MFMA consumes 64 values of k per lane pair (32 bytes per lane), so S
//    of a 32-key block takes D/64 MFMAs and O^T one MFMA per 64 keys;
//  - only the consistency of the k index between the two operands matters
//    (the A and B operand layouts mirror each other), so every operand is
//    loaded as 32 contiguous bytes per lane: Q and K at dimensions
//    64 ks + 32 h .. +31, P^T and V^T at the key slots described below;
//  - V^T is produced with identity MFMAs in fp8 (exact: x * 1 and x * 0),
//    written back as e4m3 (exact, the values came from e4m3).
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));  // 32 fp8 values

constexpr int kF8Waves = 8;
constexpr int kF8Threads = 64 * kF8Waves;
constexpr int kF8Br = 32 * kF8Waves;  // query rows per workgroup
constexpr int kF8Bc = 64;             // keys per tile
constexpr int kFmtE4M3 = 0;           // operand format code of the f8f6f4 MFMA: fp8 e4m3

// C[32x32] += A[32x64] B[64x32], fp8 e4m3 operands, no block scaling.
__device__ __forceinline__ f32x16 mfma_f8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, kFmtE4M3, kFmtE4M3, 0, 0, 0, 0);
}

// Round two floats to e4m3 into the low (HI = false) or high half of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
    return cvt_e4m3x2<true>(c, d, cvt_e4m3x2<false>(a, b, 0u));
}

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
// 32 contiguous bytes of LDS (two 16-byte reads).
__device__ __forceinline__ i32x8 lds_read32(const uint8_t* p) {
    return join8(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 16));
}

// Key slots of the V^T rows.  In a 64-key tile, key 32 kb + 8 a + 4 h + e
// (a, e in 0..3) sits in score register i = 4 a + e of lane half h of block
// kb (the C layout); the P^T operand packs byte 16 kb + i of lane half h, and
// V^T row bytes 32 h + 16 kb + i hold that key, so lane half h reads the 32
// bytes [32 h, 32 h + 32) of a V^T row.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF8Threads, 1) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int BH, int nqb, ScoreScale ss, float v_descale, int Hq,
    int G) {
    const float scale_log2 = ss.c;
    constexpr int BC = kF8Bc;
    constexpr int KS = D + 16;   // K row stride (bytes): 16 consecutive rows hit distinct banks
    constexpr int VTS = BC + 16;  // V^T row stride (bytes), same property
    constexpr int NKS = D / 64;  // MFMAs per 32-key block of S
    constexpr int NDB = D / 32;  // 32-dimension blocks of O
    constexpr int KCH = BC * D / 16;  // 16-byte chunks of a K tile
    static_assert(KCH <= kF8Threads && kF8Threads % KCH == 0, "one K chunk per thread");
    constexpr int NVB = 2 * (D / 64);  // V blocks of 32 keys x 64 dimensions per tile
    constexpr int NVW = 2 * NVB;       // wavefronts that transpose V (two column halves per block)
    static_assert(NVW <= kF8Waves, "V transpose split");

    __shared__ __attribute__((aligned(16))) uint8_t sK[2][BC * KS];
    __shared__ __attribute__((aligned(16))) uint8_t sVt[2][D * VTS];

    const int tid = thread_id(), lane = tid & 63, w = wave_id();
    const int lq = lane & 31, h = lane >> 5;
    int bh, qb;
    if (!wg_coords(block_id(), BH, nqb, CAUSAL, bh, qb)) return;
    const int q0 = qb * kF8Br;
    const int qw0 = q0 + 32 * w;
    const int qrow = qw0 + lq;
    const int64_t base = (int64_t)bh * N * D;
    const int64_t kv_base = (int64_t)kv_head(bh, Hq, G) * N * D;

    const uint32_t head_bytes = (uint32_t)N * D;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, head_bytes);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_base, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_base, head_bytes);

    // Q^T operand of MFMA ks: Q[qrow][64 ks + 32 h .. +31].
    i32x8 qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int off = lq * D + 64 * ks + 32 * h;
        qf[ks] = join8(buffer_load16(qrs, off, qw0 * D), buffer_load16(qrs, off + 16, qw0 * D));
    }
    wait_vmem_loads();
    // The sign of the scale rides on Q (ScoreScale).
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (int)apply_sign((uint32_t)qf[ks][e], ss);

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m = -INFINITY, l = 0.f;
    float mneg = 0.f;  // -m, or 0 while m = -inf (a row with nothing visible yet)

    int ntiles = (N + BC - 1) / BC;
    if (CAUSAL) ntiles = min(ntiles, (min(q0 + kF8Br, N) - 1) / BC + 1);

    // Staging.  K: thread t < KCH loads row t / (D/16), 16-byte column t % (D/16).
    // V: wavefront w < NVW takes block vb = w / 2 (keys 32 (vb % 2) .., dims
    // 64 (vb / 2) ..) and column half nh = w % 2; a lane loads the 32 bytes
    // V[32 vk + lq][64 vd + 32 h .. +31], operand A of C = V I.
    const bool kload = tid < KCH;
    const int k_ld_off = (tid / (D / 16)) * D + 16 * (tid % (D / 16));
    const int k_st_off = (tid / (D / 16)) * KS + 16 * (tid % (D / 16));
    const bool vwave = w < NVW;
    const int vb = w >> 1, nh = w & 1, vk = vb & 1, vd = vb >> 1;
    const int va_off = (32 * vk + lq) * D + 64 * vd + 32 * h;
    // Identity operand: B[k][n] = (k == 32 nh + n) in the k order of the A load
    // above, i.e. lane (h, n) holds 1.0 (0x38) in byte n when h == nh.
    i32x8 ident = i32x8{};
    if (h == nh) ident[lq >> 2] = 0x38 << (8 * (lq & 3));
    u32x4 kreg = u32x4{};
    u32x4 va0 = u32x4{}, va1 = u32x4{};
    auto load_tile = [&](int j) {
        const int soff = j * BC * D;
        if (kload) kreg = buffer_load16(krs, k_ld_off, soff);
        if (vwave) {
            va0 = buffer_load16(vrs, va_off, soff);
            va1 = buffer_load16(vrs, va_off + 16, soff);
        }
    };
    auto store_tile = [&](int buf) {
        if (kload) *reinterpret_cast<u32x4*>(&sK[buf][k_st_off]) = kreg;
        if (vwave) {
            // C[key][n] = V[32 vk + key][64 vd + 32 nh + n]: lane (h, n)
            // register i holds key c_row(i, h), stored at slot 32 h + 16 vk + i.
            const f32x16 t = mfma_f8_32x32x64(join8(va0, va1), ident, f32x16{});
            *reinterpret_cast<u32x4*>(&sVt[buf][(64 * vd + 32 * nh + lq) * VTS + 32 * h + 16 * vk]) =
                u32x4{cvt_e4m3x4(t[0], t[1], t[2], t[3]), cvt_e4m3x4(t[4], t[5], t[6], t[7]),
                      cvt_e4m3x4(t[8], t[9], t[10], t[11]), cvt_e4m3x4(t[12], t[13], t[14], t[15])};
        }
    };

    const int k_off = lq * KS + 32 * h;
    const int v_off = lq * VTS + 32 * h;

    load_tile(0);
    store_tile(0);
    __syncthreads();
    // One key tile; MASKED tiles may cross a wave's diagonal or the ragged
    // end, the others carry no masking code (no branch splits their body).
    auto step = [&](int j, auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mask_tag)::value;
        const int buf = j & 1;
        load_tile(min(j + 1, ntiles - 1));  // in flight during this tile's math

        const int k0 = j * BC;
        if (!CAUSAL || !MASKED || __builtin_amdgcn_readfirstlane(k0 <= qw0 + 31)) {
            const uint8_t* kt = sK[buf];
            const uint8_t* vt = sVt[buf];
            f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    s[kb] = mfma_f8_32x32x64(lds_read32(kt + 32 * kb * KS + k_off + 64 * ks), qf[ks], s[kb]);

            i32x8 vf[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db) vf[db] = lds_read32(vt + 32 * db * VTS + v_off);

            if (MASKED && (k0 + BC > N || (CAUSAL && k0 + BC - 1 > qw0))) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = k0 + 32 * kb + c_row(i, h);
                        if (key >= N || (CAUSAL && key > qrow)) s[kb][i] = -INFINITY;
                    }
            }

            const float mx = pair_max(max32(s[0], s[1])) * scale_log2;
            if (__any(mx > m + kRescaleThreshold)) {  // wave-uniform branch
                const float m_new = fmaxf(m, mx);
                const float alpha = fast_exp2(m - m_new);
                l *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
                m = m_new;
                mneg = (m == -INFINITY) ? 0.f : -m;
            }
            float p[2][16];
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    p[kb][i] = fast_exp2(fmaf(s[kb][i], scale_log2, mneg));
                    // The two sums start from the first two values (p >= 0, so 0 + p = p).
                    if (kb == 0 && i < 2) (i ? rs1 : rs0) = p[kb][i];
                    else (i & 1 ? rs1 : rs0) += p[kb][i];
                }
            l += rs0 + rs1;
            // P~^T operand: byte 16 kb + i = e4m3(P of register i of block kb).
            i32x8 pf;
#pragma unroll
            for (int q4 = 0; q4 < 8; ++q4) {
                const int kb = q4 >> 2, i = 4 * (q4 & 3);
                pf[q4] = (int)cvt_e4m3x4(p[kb][i], p[kb][i + 1], p[kb][i + 2], p[kb][i + 3]);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] = mfma_f8_32x32x64(vf[db], pf, oacc[db]);
        }

        store_tile(buf ^ 1);
        __syncthreads();
    };
    // Tiles before j_split are wholly visible to every wave of the workgroup.
    const int j_split = CAUSAL ? min(ntiles, q0 / BC) : (N % BC ? ntiles - 1 : ntiles);
    for (int j = 0; j < j_split; ++j) step(j, std::false_type{});
    for (int j = j_split; j < ntiles; ++j) step(j, std::true_type{});

    const float lt = pair_sum(l);
    if (qrow < N) {
        const float inv = v_descale / lt;
        bf16* op = O + base + (int64_t)qrow * D + 4 * h;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bf16x4 o4;
#pragma unroll
                for (int e = 0; e < 4; ++e) o4[e] = (bf16)(oacc[db][4 * r + e] * inv);
                *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * r) = o4;
            }
        if (h == 0) LSE[(int64_t)bh * N + qrow] = (m + fast_log2(lt)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                          int N, int d, float scale, float q_descale, float k_descale, float v_descale, bool causal,
                          hipStream_t stream) {
    const int BH = B * Hq, G = Hq / Hkv;
    const int nqb = (N + kF8Br - 1) / kF8Br;
    const int grid = grid_for_tasks(nqb * BH);
    const ScoreScale ss = make_score_scale(scale, q_descale * k_descale, 0x80808080u);
    auto Qp = static_cast<const uint8_t*>(q);
    auto Kp = static_cast<const uint8_t*>(k);
    auto Vp = static_cast<const uint8_t*>(v);
    auto Op = static_cast<bf16*>(o);
#define FA_F8_LAUNCH(DD, CC)                                                                                 \
    do {                                                                                                     \
        hipLaunchKernelGGL((fwd_fp8_kernel<DD, CC>), dim3(grid), dim3(kF8Threads), 0, stream, Qp, Kp, Vp, Op, \
                           lse, N, BH, nqb, ss, v_descale, Hq, G);                                           \
        return hipGetLastError();                                                                            \
    } while (0)
    if (d == 64) {
        if (causal) FA_F8_LAUNCH(64, true);
        FA_F8_LAUNCH(64, false);
    }
    if (causal) FA_F8_LAUNCH(128, true);
    FA_F8_LAUNCH(128, false);
#undef FA_F8_LAUNCH
}

}  // namespace fa
