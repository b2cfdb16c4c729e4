// fa_fwd.hip -- FlashAttention forward for gfx950 (MI355X).
//
// Method: the per-query-block loop of the "FlashAttention" deep-dive page
// (tirogla.com), section "How it works": load a Q block once, walk the K/V
// blocks, keep a running row max m and row sum l, rescale the partial output
// by alpha = exp(m - m_new), accumulate P V, and finally store O = acc / l and
// L = m + log l.  Exponentials are taken in base 2 with log2(e) folded into the
// scale, S, l and acc are fp32 and P is rounded to bf16 only for the P V product
// (same page, "Implementation notes").  Causal masks skip key tiles entirely
// above the diagonal and mask only the tiles that cross it, which come last in
// the key loop (same page, "Implementation notes").  Keys past N are masked to
// -inf and query rows past N are computed on zeros and never stored (same
// page, the Triton kernel under "Code").
//
// Work split (FlashAttention-2's sequence-dimension parallelism, same page):
// one workgroup of 4 wavefronts per (batch*head, block of 128 query rows);
// each wavefront owns 32 query rows, so no softmax statistic is ever shared
// between wavefronts.  Each key tile of 64 keys is staged once in LDS and read
// by all four wavefronts:
//   K   row-major  [64 keys][d]   (+8 bf16 padding per row)
//   V^T transposed [d][64 slots]  (+8 bf16 padding per row), key -> key_slot()
// Global loads for tile j+1 are issued into registers before tile j is
// computed, so HBM/L2 latency overlaps the MFMA work.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kFwdBr = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBc = 64;              // keys per tile

// Map a flat workgroup id to (head, query block).  Consecutive ids walk the
// heads of one query block, so for causal masks every head's heaviest block
// (the last one) is dispatched first, and -- because the hardware deals ids
// round-robin to the 8 XCDs -- all blocks of a head land on the same XCD
// whenever the head count is a multiple of 8, keeping its K/V in one L2.
__device__ __forceinline__ void wg_coords(int id, int BH, int nqb, bool causal, int& bh, int& qb) {
    bh = id % BH;
    const int qi = id / BH;
    qb = causal ? (nqb - 1 - qi) : qi;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int BH, int nqb, float scale_log2) {
    constexpr int BC = kFwdBc;
    constexpr int KS = D + 8;   // LDS row stride of K (elements)
    constexpr int VS = BC + 8;  // LDS row stride of V^T (elements)
    constexpr int DCH = D / 8;  // 16-byte chunks per row
    constexpr int KCH = BC * DCH / kFwdThreads;  // K chunks loaded per thread
    constexpr int VKG = BC * DCH / kFwdThreads;  // keys per V group (4 at d=128, 2 at d=64)
    static_assert(KCH * kFwdThreads == BC * DCH, "K tile split");
    static_assert(VKG == 2 || VKG == 4, "V group");
    constexpr int VDCH_PER_WAVE = DCH / kFwdWaves;  // d chunks handled by one wave for V

    __shared__ __attribute__((aligned(16))) bf16 sK[BC * KS];
    __shared__ __attribute__((aligned(16))) bf16 sVt[D * VS];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lq = lane & 31, h = lane >> 5;
    int bh, qb;
    wg_coords(blockIdx.x, BH, nqb, CAUSAL, bh, qb);
    const int q0 = qb * kFwdBr;
    const int qw0 = q0 + 32 * w;  // first query row of this wave
    const int qrow = qw0 + lq;    // this lane's query row
    const int64_t base = (int64_t)bh * N * D;

    // Q^T operand: k-step ks holds Q[qrow][16 ks + 8 h .. +7].
    bf16x8 qf[D / 16];
    {
        const bf16* qp = Q + base + (int64_t)qrow * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            if (qrow < N) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
            else qf[ks] = bf16x8{};
        }
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m = -INFINITY;  // running max of the scaled (log2-domain) scores
    float l = 0.f;        // running partial sum of this lane's keys

    int ntiles = (N + BC - 1) / BC;
    if (CAUSAL) ntiles = min(ntiles, (min(q0 + kFwdBr, N) - 1) / BC + 1);

    // Register staging of the next tile.
    u32x4 kreg[KCH];
    u32x4 vreg[VKG];
    const int vdch = w * VDCH_PER_WAVE + (lane % VDCH_PER_WAVE);
    const int vkg = lane / VDCH_PER_WAVE;  // group of VKG keys
    auto load_tile = [&](int j) {
        const int k0 = j * BC;
#pragma unroll
        for (int r = 0; r < KCH; ++r) {
            const int c = tid + kFwdThreads * r;
            const int key = k0 + c / DCH, dch = c % DCH;
            kreg[r] = key < N ? *reinterpret_cast<const u32x4*>(K + base + (int64_t)key * D + 8 * dch)
                              : u32x4{};
        }
#pragma unroll
        for (int kk = 0; kk < VKG; ++kk) {
            const int key = k0 + vkg * VKG + kk;
            vreg[kk] = key < N ? *reinterpret_cast<const u32x4*>(V + base + (int64_t)key * D + 8 * vdch)
                               : u32x4{};
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int r = 0; r < KCH; ++r) {
            const int c = tid + kFwdThreads * r;
            *reinterpret_cast<u32x4*>(&sK[(c / DCH) * KS + 8 * (c % DCH)]) = kreg[r];
        }
        // Transpose VKG keys x 8 dims in registers: one store per dim.
        const int slot0 = key_slot(vkg * VKG);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            uint16_t e[VKG];
#pragma unroll
            for (int kk = 0; kk < VKG; ++kk) e[kk] = (uint16_t)(vreg[kk][t >> 1] >> (16 * (t & 1)));
            bf16* dst = &sVt[(8 * vdch + t) * VS + slot0];
            if constexpr (VKG == 4) {
                *reinterpret_cast<u32x2*>(dst) =
                    u32x2{(uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16)};
            } else {
                *reinterpret_cast<uint32_t*>(dst) = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
            }
        }
    };

    if (ntiles > 0) load_tile(0);
    for (int j = 0; j < ntiles; ++j) {
        __syncthreads();  // every wave is done reading the previous tile
        store_tile();
        __syncthreads();
        if (j + 1 < ntiles) load_tile(j + 1);

        const int k0 = j * BC;
        if (CAUSAL && k0 > qw0 + 31) continue;  // tile entirely above this wave's diagonal

        // S^T = K Q^T for two 32-key halves.
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
            const bf16* kp = &sK[(32 * kb + lq) * KS + 8 * h];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                s[kb] = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(kp + 16 * ks), qf[ks], s[kb]);
        }

        // Mask keys past N and, on tiles crossing the diagonal, keys after the query.
        const bool ragged = k0 + BC > N;
        const bool diag = CAUSAL && (k0 + BC - 1 > qw0);
        if (ragged || diag) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 32 * kb + c_row(i, h);
                    if (key >= N || (CAUSAL && key > qrow)) s[kb][i] = -INFINITY;
                }
        }

        // Online softmax in the log2 domain.
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m, mx * scale_log2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // fully masked so far
        const float alpha = fast_exp2(m - m_use);
        m = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(fmaf(s[kb][i], scale_log2, -m_use));
                s[kb][i] = p;
                rs += p;
            }
        l = fmaf(l, alpha, rs);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

        // P^T operands (bf16), k-step s2 covers keys 16 s2 .. 16 s2 + 15.
        bf16x8 pf[BC / 16];
#pragma unroll
        for (int s2 = 0; s2 < BC / 16; ++s2)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) pf[s2][jj] = (bf16)s[s2 >> 1][8 * (s2 & 1) + jj];

        // O^T += V^T P^T.
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const bf16* vp = &sVt[(32 * db + lq) * VS + 8 * h];
#pragma unroll
            for (int s2 = 0; s2 < BC / 16; ++s2)
                oacc[db] = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(vp + 16 * s2), pf[s2], oacc[db]);
        }
    }

    // Epilogue: O = acc / l, L = (m + log2 l) ln 2.
    const float lt = pair_sum(l);
    if (qrow < N) {
        const float inv = 1.f / lt;
        bf16* op = O + base + (int64_t)qrow * D + 4 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
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

// fp32 forward: the same loop with every product in fp32 on
// v_mfma_f32_32x32x2_f32 and P kept in fp32.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int BH, int nqb, float scale_log2) {
    constexpr int BC = kFwdBc;
    constexpr int KS = D + 2;  // odd-pair stride: 32 rows x 2 columns hit distinct banks
    constexpr int VS = D + 8;  // rows 4 apart land 32 banks apart
    constexpr int DCH = D / 4;  // 16-byte chunks per row
    constexpr int CH = BC * DCH / kFwdThreads;
    static_assert(CH * kFwdThreads == BC * DCH, "tile split");

    __shared__ __attribute__((aligned(16))) float sK[BC * KS];
    __shared__ __attribute__((aligned(16))) float sV[BC * VS];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lq = lane & 31, h = lane >> 5;
    int bh, qb;
    wg_coords(blockIdx.x, BH, nqb, CAUSAL, bh, qb);
    const int q0 = qb * kFwdBr;
    const int qw0 = q0 + 32 * w;
    const int qrow = qw0 + lq;
    const int64_t base = (int64_t)bh * N * D;

    float qf[D / 2];  // Q[qrow][2 ks + h]
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = qrow < N ? Q[base + (int64_t)qrow * D + 2 * ks + h] : 0.f;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m = -INFINITY, l = 0.f;

    int ntiles = (N + BC - 1) / BC;
    if (CAUSAL) ntiles = min(ntiles, (min(q0 + kFwdBr, N) - 1) / BC + 1);

    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BC;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            const int c = tid + kFwdThreads * r;
            const int key = c / DCH, dch = c % DCH;
            f32x4 kv = f32x4{}, vv = f32x4{};
            if (k0 + key < N) {
                kv = *reinterpret_cast<const f32x4*>(K + base + (int64_t)(k0 + key) * D + 4 * dch);
                vv = *reinterpret_cast<const f32x4*>(V + base + (int64_t)(k0 + key) * D + 4 * dch);
            }
            *reinterpret_cast<f32x2*>(&sK[key * KS + 4 * dch]) = f32x2{kv[0], kv[1]};
            *reinterpret_cast<f32x2*>(&sK[key * KS + 4 * dch + 2]) = f32x2{kv[2], kv[3]};
            *reinterpret_cast<f32x4*>(&sV[key * VS + 4 * dch]) = vv;
        }
        __syncthreads();
        if (CAUSAL && k0 > qw0 + 31) continue;

        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
            const float* kp = &sK[(32 * kb + lq) * KS + h];
#pragma unroll
            for (int ks = 0; ks < D / 2; ++ks) s[kb] = mfma_f32_32x32x2(kp[2 * ks], qf[ks], s[kb]);
        }
        const bool ragged = k0 + BC > N;
        const bool diag = CAUSAL && (k0 + BC - 1 > qw0);
        if (ragged || diag) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 32 * kb + c_row(i, h);
                    if (key >= N || (CAUSAL && key > qrow)) s[kb][i] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m, mx * scale_log2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        m = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(fmaf(s[kb][i], scale_log2, -m_use));
                s[kb][i] = p;
                rs += p;
            }
        l = fmaf(l, alpha, rs);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

        // O^T += V^T P^T, one k-step per score register: lane half h supplies key c_row(i, h).
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    oacc[db] = mfma_f32_32x32x2(sV[(32 * kb + c_row(i, h)) * VS + 32 * db + lq], s[kb][i],
                                                oacc[db]);
    }

    const float lt = pair_sum(l);
    if (qrow < N) {
        const float inv = 1.f / lt;
        float* op = O + base + (int64_t)qrow * D + 4 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<f32x4*>(op + 32 * db + 8 * r) =
                    f32x4{oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv, oacc[db][4 * r + 2] * inv,
                          oacc[db][4 * r + 3] * inv};
        if (h == 0) LSE[(int64_t)bh * N + qrow] = (m + fast_log2(lt)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                           int N, int d, float scale, bool causal, hipStream_t stream) {
    const int nqb = (N + kFwdBr - 1) / kFwdBr;
    const int grid = nqb * BH;
    const float sl2 = scale * kLog2e;
    auto Q = static_cast<const bf16*>(q);
    auto K = static_cast<const bf16*>(k);
    auto V = static_cast<const bf16*>(v);
    auto Op = static_cast<bf16*>(o);
#define FA_FWD_LAUNCH(DD, CC)                                                                          \
    do {                                                                                               \
        hipLaunchKernelGGL((fwd_bf16_kernel<DD, CC>), dim3(grid), dim3(kFwdThreads), 0, stream, Q, K, V, \
                           Op, lse, N, BH, nqb, sl2);                                                  \
        return hipGetLastError();                                                                      \
    } while (0)
    if (d == 64) {
        if (causal) FA_FWD_LAUNCH(64, true);
        FA_FWD_LAUNCH(64, false);
    }
    if (causal) FA_FWD_LAUNCH(128, true);
    FA_FWD_LAUNCH(128, false);
#undef FA_FWD_LAUNCH
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH,
                          int N, int d, float scale, bool causal, hipStream_t stream) {
    const int nqb = (N + kFwdBr - 1) / kFwdBr;
    const int grid = nqb * BH;
    const float sl2 = scale * kLog2e;
#define FA_FWD_LAUNCH(DD, CC)                                                                        \
    do {                                                                                             \
        hipLaunchKernelGGL((fwd_f32_kernel<DD, CC>), dim3(grid), dim3(kFwdThreads), 0, stream, q, k, v, \
                           o, lse, N, BH, nqb, sl2);                                                 \
        return hipGetLastError();                                                                    \
    } while (0)
    if (d == 64) {
        if (causal) FA_FWD_LAUNCH(64, true);
        FA_FWD_LAUNCH(64, false);
    }
    if (causal) FA_FWD_LAUNCH(128, true);
    FA_FWD_LAUNCH(128, false);
#undef FA_FWD_LAUNCH
}

}  // namespace fa
