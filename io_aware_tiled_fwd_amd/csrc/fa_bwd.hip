// fa_bwd.hip -- FlashAttention backward for gfx950 (MI355X).
//
// Method: the backward of the "FlashAttention" deep-dive page (tirogla.com),
// section "How it works": P is recomputed tile by tile from the saved
// logsumexp, P = exp(scale Q K^T - L); with D = rowsum(dO * O) and
// dS = P * (dP - D), dP = dO V^T, the gradients are dV = P^T dO,
// dK = scale dS^T Q and dQ = scale dS K.  Only the O(N) statistics L and D are
// read besides the O(N d) tensors; no N x N matrix reaches HBM.
//
// Three kernels run in stream order:
//   1. preprocess   D_i = sum_t dO_it O_it                    (bandwidth-bound)
//   2. dK/dV        one workgroup per 128 keys (32 per wavefront), walking the
//                   query blocks; the wavefront's K and V rows stay in
//                   registers as MFMA operands, dK and dV accumulate in
//                   registers and are written once.
//   3. dQ           one workgroup per 128 query rows (32 per wavefront),
//                   walking the key tiles; dQ accumulates in registers.
// dQ is produced without atomics, so the backward is bitwise reproducible (the
// deep-dive page's pitfalls section warns that atomic dQ accumulation is not).
//
// Causal masks skip (query block, key block) pairs entirely above the diagonal
// and mask only the pairs that cross it.  Rows past N are staged as zeros, with
// L = +inf (so P = 0) and D = 0, and are never stored.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBwdThreads = 256;

// Stages a [ROWS x D] bf16 tile from HBM through registers into LDS, row-major
// and/or transposed.  Each thread loads G consecutive rows x 8 dims (G 16-byte
// loads); the transposed copy puts those G values of each dim next to each
// other at key_slot(row), i.e. one 8- or 4-byte LDS store per dim.
template <int D, int ROWS>
struct TileStager {
    static constexpr int DCH = D / 8;
    static constexpr int G = ROWS * DCH / kBwdThreads;  // rows per thread
    static constexpr int DCH_PER_WAVE = DCH / 4;
    static_assert(G == 2 || G == 4, "rows per thread");
    static_assert(G * kBwdThreads == ROWS * DCH, "tile split");

    u32x4 reg[G];
    int dch, grp;

    __device__ explicit TileStager(int tid) {
        const int w = tid >> 6, lane = tid & 63;
        dch = w * DCH_PER_WAVE + lane % DCH_PER_WAVE;
        grp = lane / DCH_PER_WAVE;
    }
    // src points at row 0 of the head; rows >= N read as zero.
    __device__ void load(const bf16* src, int row0, int N) {
#pragma unroll
        for (int kk = 0; kk < G; ++kk) {
            const int row = row0 + grp * G + kk;
            reg[kk] = row < N ? *reinterpret_cast<const u32x4*>(src + (int64_t)row * D + 8 * dch) : u32x4{};
        }
    }
    __device__ void store_rows(bf16* lds, int stride) const {
#pragma unroll
        for (int kk = 0; kk < G; ++kk)
            *reinterpret_cast<u32x4*>(&lds[(grp * G + kk) * stride + 8 * dch]) = reg[kk];
    }
    __device__ void store_transposed(bf16* lds, int stride) const {
        const int slot0 = key_slot(grp * G);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            uint32_t e[G];
#pragma unroll
            for (int kk = 0; kk < G; ++kk) e[kk] = (reg[kk][t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
            bf16* dst = &lds[(8 * dch + t) * stride + slot0];
            if constexpr (G == 4) {
                *reinterpret_cast<u32x2*>(dst) = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
            } else {
                *reinterpret_cast<uint32_t*>(dst) = e[0] | (e[1] << 16);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O), fp32.  DCH lanes per row, one 16-byte chunk each.

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_preprocess_kernel(const bf16* __restrict__ O,
                                                                     const bf16* __restrict__ dO,
                                                                     float* __restrict__ Dl, int64_t rows) {
    constexpr int DCH = D / 8;
    constexpr int ROWS_PER_BLOCK = kBwdThreads / DCH;
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + tid / DCH;
    const int ch = tid % DCH;
    float acc = 0.f;
    if (row < rows) {
        const bf16x8 o = *reinterpret_cast<const bf16x8*>(O + row * D + 8 * ch);
        const bf16x8 g = *reinterpret_cast<const bf16x8*>(dO + row * D + 8 * ch);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
    // Reduce over the DCH consecutive lanes of the row (DCH is 8 or 16).
#pragma unroll
    for (int off = DCH / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, DCH);
    if (row < rows && ch == 0) Dl[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK, dV.  Per query block of 64 rows, staged in LDS:
//      Q   row-major [64][d]  and  Q^T  [d][64 slots]
//      dO  row-major [64][d]  and  dO^T [d][64 slots]
//      L (log2 domain, +inf past N) and D.
//    Per wavefront (32 keys) and 32-query half, with C tiles [query x key]:
//      S  = Q K^T            (A = Q rows from LDS, B = K^T from registers)
//      dP = dO V^T           (A = dO rows from LDS, B = V^T from registers)
//      P  = exp2(S c - L2), dS = P (dP - D)
//      dV^T += dO^T P        (A = dO^T from LDS, B = P from registers)
//      dK^T += Q^T dS        (A = Q^T from LDS, B = dS from registers)

constexpr int kDkvBq = 64;    // query rows per step
constexpr int kDkvBkv = 128;  // keys per workgroup

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    float* __restrict__ dK, float* __restrict__ dV, int N, int BH, int nkb, float scale_log2, float scale) {
    constexpr int BQ = kDkvBq;
    constexpr int RS = D + 8;   // row-major stride
    constexpr int TS = BQ + 8;  // transposed stride
    __shared__ __attribute__((aligned(16))) bf16 sQ[BQ * RS];
    __shared__ __attribute__((aligned(16))) bf16 sQt[D * TS];
    __shared__ __attribute__((aligned(16))) bf16 sdO[BQ * RS];
    __shared__ __attribute__((aligned(16))) bf16 sdOt[D * TS];
    __shared__ __attribute__((aligned(16))) float sL[BQ];
    __shared__ __attribute__((aligned(16))) float sD[BQ];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lq = lane & 31, h = lane >> 5;
    // Flat id -> (head, key block); key blocks ascend, so for causal masks the
    // heaviest blocks (the first ones, seen by the most queries) start first.
    const int bh = blockIdx.x % BH;
    const int kb = blockIdx.x / BH;
    const int k0 = kb * kDkvBkv;
    const int kw0 = k0 + 32 * w;
    const int key = kw0 + lq;
    const int64_t base = (int64_t)bh * N * D;

    // K^T and V^T operands of this lane's key.
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        if (key < N) {
            kf[ks] = *reinterpret_cast<const bf16x8*>(K + base + (int64_t)key * D + 16 * ks + 8 * h);
            vf[ks] = *reinterpret_cast<const bf16x8*>(V + base + (int64_t)key * D + 16 * ks + 8 * h);
        } else {
            kf[ks] = bf16x8{};
            vf[ks] = bf16x8{};
        }
    }
    f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dkacc[db] = f32x16{};
        dvacc[db] = f32x16{};
    }

    const int nqblk = (N + BQ - 1) / BQ;
    const int iq0 = CAUSAL ? k0 / BQ : 0;
    TileStager<D, BQ> stq(tid), stdo(tid);
    float lreg = 0.f, dreg = 0.f;
    auto load_block = [&](int iq) {
        const int i0 = iq * BQ;
        stq.load(Q + base, i0, N);
        stdo.load(dO + base, i0, N);
        if (tid < BQ) {
            const int r = i0 + tid;
            lreg = r < N ? LSE[(int64_t)bh * N + r] * kLog2e : INFINITY;
            dreg = r < N ? Dl[(int64_t)bh * N + r] : 0.f;
        }
    };
    if (iq0 < nqblk) load_block(iq0);
    for (int iq = iq0; iq < nqblk; ++iq) {
        __syncthreads();
        stq.store_rows(sQ, RS);
        stq.store_transposed(sQt, TS);
        stdo.store_rows(sdO, RS);
        stdo.store_transposed(sdOt, TS);
        if (tid < BQ) {
            sL[tid] = lreg;
            sD[tid] = dreg;
        }
        __syncthreads();
        if (iq + 1 < nqblk) load_block(iq + 1);

        const int i0 = iq * BQ;
        if (CAUSAL && i0 + BQ - 1 < kw0) continue;  // every query precedes every key of this wave
        const bool diag = CAUSAL && (i0 < kw0 + 31);

#pragma unroll
        for (int qh = 0; qh < BQ / 32; ++qh) {
            f32x16 s = f32x16{}, dp = f32x16{};
            const bf16* qp = &sQ[(32 * qh + lq) * RS + 8 * h];
            const bf16* gp = &sdO[(32 * qh + lq) * RS + 8 * h];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                s = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(qp + 16 * ks), kf[ks], s);
                dp = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(gp + 16 * ks), vf[ks], dp);
            }
            // Register i holds query 32 qh + c_row(i, h); four consecutive queries per float4.
            bf16x8 pf[2], dsf[2];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[32 * qh + 8 * r + 4 * h]);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[32 * qh + 8 * r + 4 * h]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * r + e;
                    float p = fast_exp2(fmaf(s[i], scale_log2, -l4[e]));
                    if (diag && key > i0 + 32 * qh + c_row(i, h)) p = 0.f;
                    const float ds = p * (dp[i] - d4[e]);
                    pf[i >> 3][i & 7] = (bf16)p;
                    dsf[i >> 3][i & 7] = (bf16)ds;
                }
            }
            // k-step s2 of this half covers queries 32 qh + 16 s2 .. +15 (slots 16 s2 + 8 h + j).
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const bf16* gtp = &sdOt[(32 * db + lq) * TS + 32 * qh + 8 * h];
                const bf16* qtp = &sQt[(32 * db + lq) * TS + 32 * qh + 8 * h];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    dvacc[db] = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(gtp + 16 * s2), pf[s2],
                                                   dvacc[db]);
                    dkacc[db] = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(qtp + 16 * s2), dsf[s2],
                                                   dkacc[db]);
                }
            }
        }
    }

    // Register i of block db holds dim 32 db + c_row(i, h) of this lane's key.
    if (key < N) {
        float* dkp = dK + base + (int64_t)key * D + 4 * h;
        float* dvp = dV + base + (int64_t)key * D + 4 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                *reinterpret_cast<f32x4*>(dkp + 32 * db + 8 * r) =
                    f32x4{dkacc[db][4 * r] * scale, dkacc[db][4 * r + 1] * scale, dkacc[db][4 * r + 2] * scale,
                          dkacc[db][4 * r + 3] * scale};
                *reinterpret_cast<f32x4*>(dvp + 32 * db + 8 * r) =
                    f32x4{dvacc[db][4 * r], dvacc[db][4 * r + 1], dvacc[db][4 * r + 2], dvacc[db][4 * r + 3]};
            }
    }
}

// ---------------------------------------------------------------------------
// 3. dQ.  Per key tile of 64 keys, staged in LDS:
//      K row-major [64][d],  K^T [d][64 slots],  V row-major [64][d].
//    Per wavefront (32 queries) and 32-key half, with C tiles [key x query]:
//      S^T  = K Q^T      (A = K rows from LDS, B = Q^T from registers)
//      dP^T = V dO^T     (A = V rows from LDS, B = dO^T from registers)
//      P^T = exp2(S^T c - L2), dS^T = P^T (dP^T - D)
//      dQ^T += K^T dS^T  (A = K^T from LDS, B = dS^T from registers)

constexpr int kDqBq = 128;  // query rows per workgroup
constexpr int kDqBkv = 64;  // keys per step

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    float* __restrict__ dQ, int N, int BH, int nqb, float scale_log2, float scale) {
    constexpr int BKV = kDqBkv;
    constexpr int RS = D + 8;
    constexpr int TS = BKV + 8;
    __shared__ __attribute__((aligned(16))) bf16 sK[BKV * RS];
    __shared__ __attribute__((aligned(16))) bf16 sKt[D * TS];
    __shared__ __attribute__((aligned(16))) bf16 sV[BKV * RS];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lq = lane & 31, h = lane >> 5;
    const int bh = blockIdx.x % BH;
    const int qi = blockIdx.x / BH;
    const int qb = CAUSAL ? (nqb - 1 - qi) : qi;  // heaviest query blocks first
    const int q0 = qb * kDqBq;
    const int qw0 = q0 + 32 * w;
    const int qrow = qw0 + lq;
    const int64_t base = (int64_t)bh * N * D;

    bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        if (qrow < N) {
            qf[ks] = *reinterpret_cast<const bf16x8*>(Q + base + (int64_t)qrow * D + 16 * ks + 8 * h);
            gf[ks] = *reinterpret_cast<const bf16x8*>(dO + base + (int64_t)qrow * D + 16 * ks + 8 * h);
        } else {
            qf[ks] = bf16x8{};
            gf[ks] = bf16x8{};
        }
    }
    const float l2 = qrow < N ? LSE[(int64_t)bh * N + qrow] * kLog2e : 0.f;
    const float dq_d = qrow < N ? Dl[(int64_t)bh * N + qrow] : 0.f;

    f32x16 dqacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqacc[db] = f32x16{};

    int ntiles = (N + BKV - 1) / BKV;
    if (CAUSAL) ntiles = min(ntiles, (min(q0 + kDqBq, N) - 1) / BKV + 1);
    TileStager<D, BKV> stk(tid), stv(tid);
    if (ntiles > 0) {
        stk.load(K + base, 0, N);
        stv.load(V + base, 0, N);
    }
    for (int j = 0; j < ntiles; ++j) {
        __syncthreads();
        stk.store_rows(sK, RS);
        stk.store_transposed(sKt, TS);
        stv.store_rows(sV, RS);
        __syncthreads();
        if (j + 1 < ntiles) {
            stk.load(K + base, (j + 1) * BKV, N);
            stv.load(V + base, (j + 1) * BKV, N);
        }
        const int k0 = j * BKV;
        if (CAUSAL && k0 > qw0 + 31) continue;
        const bool mask = (k0 + BKV > N) || (CAUSAL && k0 + BKV - 1 > qw0);

        bf16x8 dsf[BKV / 16];
#pragma unroll
        for (int kh = 0; kh < BKV / 32; ++kh) {
            f32x16 s = f32x16{}, dp = f32x16{};
            const bf16* kp = &sK[(32 * kh + lq) * RS + 8 * h];
            const bf16* vp = &sV[(32 * kh + lq) * RS + 8 * h];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                s = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(kp + 16 * ks), qf[ks], s);
                dp = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(vp + 16 * ks), gf[ks], dp);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = fast_exp2(fmaf(s[i], scale_log2, -l2));
                if (mask) {
                    const int kk = k0 + 32 * kh + c_row(i, h);
                    if (kk >= N || (CAUSAL && kk > qrow)) p = 0.f;
                }
                dsf[2 * kh + (i >> 3)][i & 7] = (bf16)(p * (dp[i] - dq_d));
            }
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const bf16* ktp = &sKt[(32 * db + lq) * TS + 8 * h];
#pragma unroll
            for (int s2 = 0; s2 < BKV / 16; ++s2)
                dqacc[db] = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(ktp + 16 * s2), dsf[s2], dqacc[db]);
        }
    }

    if (qrow < N) {
        float* dqp = dQ + base + (int64_t)qrow * D + 4 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<f32x4*>(dqp + 32 * db + 8 * r) =
                    f32x4{dqacc[db][4 * r] * scale, dqacc[db][4 * r + 1] * scale, dqacc[db][4 * r + 2] * scale,
                          dqacc[db][4 * r + 3] * scale};
    }
}

template <int D>
hipError_t launch_pre_t(const bf16* o, const bf16* dout, float* delta, int BH, int N, hipStream_t stream) {
    const int64_t rows = (int64_t)BH * N;
    constexpr int rows_per_block = kBwdThreads / (D / 8);
    const int grid = (int)((rows + rows_per_block - 1) / rows_per_block);
    hipLaunchKernelGGL((bwd_preprocess_kernel<D>), dim3(grid), dim3(kBwdThreads), 0, stream, o, dout, delta,
                       rows);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_t(const bf16* q, const bf16* k, const bf16* v, const float* lse, const bf16* dout,
                         const float* delta, float* dk, float* dv, int BH, int N, float scale,
                         hipStream_t stream) {
    const int nkb = (N + kDkvBkv - 1) / kDkvBkv;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(nkb * BH), dim3(kBwdThreads), 0, stream, q, k, v,
                       dout, lse, delta, dk, dv, N, BH, nkb, scale * kLog2e, scale);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const bf16* q, const bf16* k, const bf16* v, const float* lse, const bf16* dout,
                       const float* delta, float* dq, int BH, int N, float scale, hipStream_t stream) {
    const int nqb = (N + kDqBq - 1) / kDqBq;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(nqb * BH), dim3(kBwdThreads), 0, stream, q, k, v, dout,
                       lse, delta, dq, N, BH, nqb, scale * kLog2e, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, int BH, int N, int d,
                                 hipStream_t stream) {
    auto Op = static_cast<const bf16*>(o);
    auto G = static_cast<const bf16*>(dout);
    return d == 64 ? launch_pre_t<64>(Op, G, delta, BH, N, stream) : launch_pre_t<128>(Op, G, delta, BH, N, stream);
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                           const float* delta, float* dk, float* dv, int BH, int N, int d, float scale,
                           bool causal, hipStream_t stream) {
    auto Q = static_cast<const bf16*>(q);
    auto K = static_cast<const bf16*>(k);
    auto V = static_cast<const bf16*>(v);
    auto G = static_cast<const bf16*>(dout);
    if (d == 64)
        return causal ? launch_dkdv_t<64, true>(Q, K, V, lse, G, delta, dk, dv, BH, N, scale, stream)
                      : launch_dkdv_t<64, false>(Q, K, V, lse, G, delta, dk, dv, BH, N, scale, stream);
    return causal ? launch_dkdv_t<128, true>(Q, K, V, lse, G, delta, dk, dv, BH, N, scale, stream)
                  : launch_dkdv_t<128, false>(Q, K, V, lse, G, delta, dk, dv, BH, N, scale, stream);
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, float* dq, int BH, int N, int d, float scale, bool causal,
                         hipStream_t stream) {
    auto Q = static_cast<const bf16*>(q);
    auto K = static_cast<const bf16*>(k);
    auto V = static_cast<const bf16*>(v);
    auto G = static_cast<const bf16*>(dout);
    if (d == 64)
        return causal ? launch_dq_t<64, true>(Q, K, V, lse, G, delta, dq, BH, N, scale, stream)
                      : launch_dq_t<64, false>(Q, K, V, lse, G, delta, dq, BH, N, scale, stream);
    return causal ? launch_dq_t<128, true>(Q, K, V, lse, G, delta, dq, BH, N, scale, stream)
                  : launch_dq_t<128, false>(Q, K, V, lse, G, delta, dq, BH, N, scale, stream);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, float* delta, int BH, int N,
                           int d, float scale, bool causal, hipStream_t stream) {
    hipError_t e = launch_bwd_preprocess(o, dout, delta, BH, N, d, stream);
    if (e != hipSuccess) return e;
    e = launch_bwd_dkdv(q, k, v, lse, dout, delta, dk, dv, BH, N, d, scale, causal, stream);
    if (e != hipSuccess) return e;
    return launch_bwd_dq(q, k, v, lse, dout, delta, dq, BH, N, d, scale, causal, stream);
}

}  // namespace fa
