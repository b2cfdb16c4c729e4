// fa_bwd.hip -- FlashAttention backward for gfx950 (MI355X).
//
// Method: the backward of the "FlashAttention" deep-dive page (tirogla.com),
// section "How it works": P is recomputed tile by tile from the saved
// logsumexp, P = exp(scale Q K^T - L); with D = rowsum(dO * O) and
// dS = P * (dP - D), dP = dO V^T, the gradients are dV = P^T dO,
// dK = scale dS^T Q and dQ = scale dS K.  Only the O(N) statistics L and D are
// read besides the O(N d) tensors; no N x N matrix reaches HBM.
//
// Three stages run in stream order:
//   1. preprocess   D_i = sum_t dO_it O_it                    (bandwidth-bound)
//   2. dK, dV       at d = 128 one kernel of paired wavefronts (2'. below):
//                   a workgroup per 128 keys, walking the query blocks; one
//                   wavefront of a pair computes P and dV, hands P to its
//                   partner through LDS, and the partner computes dS and dK.
//                   At d = 64 two kernels (2. below), one workgroup per 256 keys
//                   (32 per wavefront), each recomputing S.  The wavefront's K
//                   (or V) rows stay in registers as MFMA operands, and its one
//                   gradient accumulates in registers and is written once, so
//                   two wavefronts share each SIMD.
//   3. dQ           one workgroup per 256 query rows (32 per wavefront),
//                   walking the key tiles; dQ accumulates in registers.
// Tiles are staged row-major in double-buffered LDS through buffer loads (rows
// past N read as zero); operands that must be transposed (dO^T, Q^T, K^T) are
// read with the gfx950 transposing LDS read, so no transposed copy is stored.
// dQ is produced without atomics, so the backward is bitwise reproducible (the
// deep-dive page's pitfalls section warns that atomic dQ accumulation is not).
//
// Causal masks skip (query block, key block) pairs entirely above the diagonal
// and mask only the pairs that cross it.  Rows past N are staged as zeros, with
// L = +inf (so P = 0) and D = 0, and are never stored.
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

#ifndef FA_BWD_WAVES
#define FA_BWD_WAVES 8
#endif
constexpr int kBwdWaves = FA_BWD_WAVES;
constexpr int kBwdThreads = 64 * kBwdWaves;

// Row stride (elements) of a bf16 [rows][D] LDS tile that is read both as
// 16-byte rows (MFMA operand M) and through ds_read_b64_tr_b16 (operand M^T),
// in the separate dK/dV kernels: 16 consecutive rows of one 16-byte column
// fall on distinct banks.  At d = 128 the transposing reads of this stride
// still meet 2-way conflicts; the paired dK/dV and the dQ kernels use the
// swizzled layout of pair_swz (below) instead.
template <int D>
constexpr int both_ways_stride() { return D == 128 ? D + 24 : D + 8; }

// The tiles that the paired dK/dV kernel (Q, dO) and the dQ kernel (K) read
// both as 16-byte rows (16 lanes: 16 consecutive rows, one column) and
// through ds_read_b64_tr_b16 (32 lanes: 4 consecutive rows x 64 bytes), at
// d = 128.  No padded stride serves both: the rows
// need a stride of 4 dwords (odd multiple) modulo 64 banks, the transposing
// reads 16 or 48.  Rows are therefore D + 32 elements apart (16 dwords
// modulo 64) and the 16-byte chunk c of row r sits at chunk c ^ pair_swz(r):
// 16 consecutive rows then cover 16 distinct 4-bank groups, and the 4 rows
// of a transposing read keep their 64 bytes on distinct banks.  The swizzle
// only permutes chunks within aligned groups of four, so column offsets of
// 64 bytes and row offsets of 16 rows remain plain additions.
__device__ __forceinline__ constexpr int pair_swz(int r) { return (r >> 2) & 3; }

// Pins the issue order of a chain of N MFMAs whose A operands come from LDS in
// R reads each: the reads of the first A MFMAs, then every MFMA followed by
// the reads of the MFMA A places on.  Without it the compiler issued each read
// right before its MFMA and waited for it there (one LDS round trip per MFMA),
// whatever order the source gave.  Applies to the basic block it sits in.
template <int N, int R, int A>
__device__ __forceinline__ void pin_read_ahead() {
    static_assert(A <= N, "read-ahead longer than the chain");
    __builtin_amdgcn_sched_group_barrier(0x100, R * A, 0);
#pragma unroll
    for (int i = 0; i < N - A; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
}

// Stages a [ROWS x D] bf16 tile: HBM -> registers (buffer loads, rows past the
// end read as zero) -> row-major LDS.  Thread t holds rows (t + 256 r) / DCH,
// 16-byte column t % DCH, r < CH.  The tile offset is a scalar, so the per-lane
// VGPR offset is fixed for the kernel's lifetime.
template <int D, int ROWS>
struct TileStager {
    static constexpr int DCH = D / 8;
    static constexpr int CH = ROWS * DCH / kBwdThreads;
    static constexpr int ROWS_PER_PASS = kBwdThreads / DCH;
    static_assert(CH * kBwdThreads == ROWS * DCH, "tile split");
    u32x4 reg[CH];
    int voff, lds_off;
    // SWIZZLED: chunk c of row r is stored at chunk c ^ pair_swz(r) (the
    // both-ways layout above; ROWS_PER_PASS is a multiple of 16, so the
    // thread's rows all share one swizzle).
    __device__ TileStager(int tid, int stride, bool swizzled = false) {
        const int row = tid / DCH, c = tid % DCH;
        voff = (row * D + 8 * c) * 2;
        lds_off = row * stride + 8 * (swizzled ? c ^ pair_swz(row) : c);
    }
    __device__ void load(__amdgpu_buffer_rsrc_t rs, int row0) {
#pragma unroll
        for (int r = 0; r < CH; ++r) reg[r] = buffer_load16(rs, voff + r * ROWS_PER_PASS * D * 2, row0 * D * 2);
    }
    __device__ void store(bf16* lds, int stride) const {
#pragma unroll
        for (int r = 0; r < CH; ++r)
            *reinterpret_cast<u32x4*>(&lds[lds_off + r * ROWS_PER_PASS * stride]) = reg[r];
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
    const int tid = thread_id();
    const int64_t row = (int64_t)block_id() * ROWS_PER_BLOCK + tid / DCH;
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
// 2. dK and dV, as two kernels of one template (each holds one fp32
//    accumulator, so two wavefronts fit per SIMD).  Per block of 64 query rows,
//    staged row-major in LDS (double buffered): Q, dO, and L (log2 domain, +inf
//    past N) and D.  Per wavefront (32 keys) and 32-query half, with C tiles
//    [query x key]:
//      S  = Q K^T            (A = Q rows from LDS, B = K^T from registers)
//      P  = exp2(S c - L2)
//      dV: dV^T += dO^T P    (A = dO^T: transposing LDS reads; B = P)
//      dK: dP = dO V^T       (A = dO rows from LDS, B = V^T from registers)
//          dS = P (dP - D);  dK^T += Q^T dS  (A = Q^T: transposing reads; B = dS)

// Gradient stores: fp32, or bf16 rounded to nearest even.
__device__ __forceinline__ void store_grad4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store_grad4(bf16* p, f32x4 v) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

constexpr int kDkvBq = 64;    // query rows per step
constexpr int kDkvBkv = 32 * kBwdWaves;  // keys per workgroup

// GROUPED: several query heads per key/value head (G = Hq / Hkv > 1).  Without
// it G is the constant 1 and the group loop disappears at compile time.
// DROPOUT: the forward's dropout mask (fa_common.h) is regenerated.  Its
// Philox words come per (query row, 16 keys), while a lane here holds one key
// and 16 queries: each lane draws the words of one query row of the 32 x 32
// tile, the keep bits of that row (one bit per key of the wavefront) go
// through a wavefront-private LDS word, and each lane reads back the bits of
// its key for its 16 queries.
// OutT: float or bf16 gradient output.
template <int D, bool CAUSAL, bool DK, bool GROUPED, bool DROPOUT, typename OutT>
__global__ __launch_bounds__(kBwdThreads, 8 / kBwdWaves) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    OutT* __restrict__ dOut, int N, int BKV, int nkb, ScoreScale ss, float out_scale, int Hq, int G_arg,
    DropoutParams drop) {
    const float scale_log2 = ss.c;
    const int G = GROUPED ? G_arg : 1;
    constexpr int BQ = kDkvBq;
    constexpr int RS = both_ways_stride<D>();
    __shared__ __attribute__((aligned(16))) bf16 sQ[2][BQ * RS];
    __shared__ __attribute__((aligned(16))) bf16 sdO[2][BQ * RS];
    __shared__ __attribute__((aligned(16))) float sL[2][BQ];
    __shared__ __attribute__((aligned(16))) float sD[2][BQ];
    __shared__ __attribute__((aligned(16))) uint32_t sKeep[DROPOUT ? kBwdWaves : 1][32];

    const int tid = thread_id(), lane = tid & 63, w = wave_id();
    const int lq = lane & 31, h = lane >> 5;
    // Flat id -> (key/value head, key block): XCD-contiguous, head-major; key
    // blocks ascend, so for causal masks the heaviest blocks (the first ones,
    // seen by the most queries) start first.  Head-major keeps the workgroups
    // that stream one head's Q and dO running together on one L2 (ordering
    // the blocks heaviest-first across all of an XCD's heads measured 4-10%
    // slower here).  The G query heads sharing the key/value
    // head (grouped heads) are walked one after the other, their
    // contributions summed in the same accumulators.
    const int task = xcd_task(block_id(), BKV * nkb);
    if (task >= BKV * nkb) return;
    const int kvh = task / nkb;
    const int kb = task % nkb;
    const int k0 = kb * kDkvBkv;
    const int kw0 = k0 + 32 * w;
    const int key = kw0 + lq;
    const int64_t base = (int64_t)kvh * N * D;
    const int qh0 = (kvh / (Hq / G)) * Hq + (kvh % (Hq / G)) * G;  // first query head of the group
    const uint32_t head_bytes = (uint32_t)N * D * 2;

    // K^T (and, for dK, V^T) operands of this lane's key (zero past N).
    bf16x8 kf[D / 16], vf[DK ? D / 16 : 1];
    {
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + base, head_bytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + base, head_bytes);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            kf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(krs, (lq * D + 16 * ks + 8 * h) * 2, kw0 * D * 2));
            if constexpr (DK)
                vf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(vrs, (lq * D + 16 * ks + 8 * h) * 2, kw0 * D * 2));
        }
        wait_vmem_loads();
        // The sign of the scale rides on K in S = Q K^T (ScoreScale); dK's own
        // factor, out_scale, is the signed scale.
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) kf[ks] = apply_sign(kf[ks], ss);
    }
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    const int nqblk = (N + BQ - 1) / BQ;
    const int iq0 = CAUSAL ? k0 / BQ : 0;
    // Steps whose query block starts before this workgroup's last key.
    const int iq_split = CAUSAL ? min(nqblk, (k0 + kDkvBkv - 1) / BQ + 1) : iq0;
    TileStager<D, BQ> stq(tid, RS), stg(tid, RS);
    float lreg = 0.f, dreg = 0.f;
    // Per-lane LDS offsets: 16-byte rows and transposing reads.
    const int row_off = lq * RS + 8 * h;
    const int tr_off = tr_row(lane) * RS + tr_col(lane);

    // All query blocks of query head qh (one of the group sharing this
    // key/value head), accumulated into acc.  The head's bases are set up
    // once, outside its step loop.
    auto run_head = [&](int qh_idx) {
        const int64_t qbase = (int64_t)qh_idx * N;
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + qbase * D, head_bytes);
        const __amdgpu_buffer_rsrc_t grs = make_rsrc(dO + qbase * D, head_bytes);
        const float* lse_h = LSE + qbase;
        const float* d_h = Dl + qbase;
        auto load_block = [&](int iq) {
            const int i0 = iq * BQ;
            stq.load(qrs, i0);
            stg.load(grs, i0);
            if (tid < BQ) {
                const int r = min(i0 + tid, N - 1);
                // Kept as loaded until the block is stored (scaling it here
                // would wait for the load at the start of the step).
                lreg = i0 + tid < N ? lse_h[r] : INFINITY;  // P = 0 past N
                if constexpr (DK) dreg = i0 + tid < N ? d_h[r] : 0.f;
            }
        };
        auto store_block = [&](int buf) {
            stq.store(sQ[buf], RS);
            stg.store(sdO[buf], RS);
            if (tid < BQ) {
                sL[buf][tid] = lreg * kLog2e;
                if constexpr (DK) sD[buf][tid] = dreg;
            }
        };

        // Loads and stores are unconditional (the last step re-stages the final
        // block into the idle buffer) so that no math waits on a pending load.
        if (iq0 < nqblk) {
            load_block(iq0);
            store_block(0);
        }
        __syncthreads();
        // One step of 64 query rows.  MASK applies the causal mask; only the
        // steps whose queries overlap this workgroup's keys (the first two)
        // need it, so the loop is split and the other steps carry no mask code.
        auto step = [&](int iq, auto mask_tag) {
            constexpr bool MASK = decltype(mask_tag)::value;
            const int buf = (iq - iq0) & 1;
            load_block(min(iq + 1, nqblk - 1));
            const int i0 = iq * BQ;
            // Skip blocks whose every query precedes every key of this wave
            // (never the case in the unmasked steps: no test there).
            if (!CAUSAL || !MASK || __builtin_amdgcn_readfirstlane(i0 + BQ - 1 >= kw0)) {
                const bf16* qt = sQ[buf];
                const bf16* gt = sdO[buf];
                // dV: the scores of every 32-query sub-block first, as
                // interleaved accumulation chains (one chain alone would wait
                // on each previous MFMA).  It has registers to spare: each Q
                // fragment is requested AHEAD MFMAs before its use (volatile
                // reads keep that order).
                constexpr int NQH = BQ / 32;
                f32x16 sv[DK ? 1 : NQH];
                if constexpr (!DK) {
                    constexpr int NR = NQH * (D / 16), AHEAD = 4;
                    auto qread = [&](int r) {
                        return lds_read16_early(qt + 32 * (r % NQH) * RS + row_off + 16 * (r / NQH));
                    };
                    bf16x8 qa[NR];
#pragma unroll
                    for (int r = 0; r < AHEAD; ++r) qa[r] = qread(r);
#pragma unroll
                    for (int qh = 0; qh < NQH; ++qh) sv[qh] = f32x16{};
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        if (r + AHEAD < NR) qa[r + AHEAD] = qread(r + AHEAD);
                        sv[r % NQH] = mfma_bf16_32x32x16(qa[r], kf[r / NQH], sv[r % NQH]);
                    }
                }
#pragma unroll
                for (int qh = 0; qh < NQH; ++qh) {
                    // (The keep bits are formed before the score MFMAs, while
                    // fewer accumulators are live.)
                    uint32_t keep_bits[4];  // bit lq of word e of group r: query 32 qh + 8 r + 4 h + e kept
                    if constexpr (DROPOUT) {
                        // Lane (h, lq) as query row i0 + 32 qh + lq: keep bits of keys 8 a + 4 h + e.
                        const u32x4 wd = dropout_words(drop, qh_idx, i0 + 32 * qh + lq, kw0 / 32, h);
                        uint32_t bits = 0;
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            bits |= (dropout_keep(wd, r, drop.thr) ? 1u : 0u) << (8 * (r >> 2) + 4 * h + (r & 3));
                        const auto sw = __builtin_amdgcn_permlane32_swap(bits, bits, false, false);
                        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                        if (h == 0) sKeep[w][lq] = sw[0] | sw[1];
                        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const u32x4 k4 = *reinterpret_cast<const u32x4*>(&sKeep[w][8 * r + 4 * h]);
                            keep_bits[r] = ((k4[0] >> lq) & 1u) | (((k4[1] >> lq) & 1u) << 1) |
                                           (((k4[2] >> lq) & 1u) << 2) | (((k4[3] >> lq) & 1u) << 3);
                        }
                    }
                    f32x16 s = f32x16{}, dp = f32x16{};
                    if constexpr (DK) {
#pragma unroll
                        for (int ks = 0; ks < D / 16; ++ks) {
                            const int off = 32 * qh * RS + row_off + 16 * ks;
                            s = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(qt + off), kf[ks], s);
                            dp = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(gt + off), vf[ks], dp);
                        }
                    } else {
                        s = sv[qh];
                    }
                    // Register i holds query 32 qh + c_row(i, h); four consecutive queries per float4.
                    float v[16];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[buf][32 * qh + 8 * r + 4 * h]);
                        f32x4 d4 = f32x4{};
                        if constexpr (DK) d4 = *reinterpret_cast<const f32x4*>(&sD[buf][32 * qh + 8 * r + 4 * h]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int i = 4 * r + e;
                            float p = fast_exp2(fmaf(s[i], scale_log2, -l4[e]));
                            if constexpr (MASK) {
                                if (key > i0 + 32 * qh + c_row(i, h)) p = 0.f;
                            }
                            if constexpr (DROPOUT) {
                                const bool kept = (keep_bits[r] >> e) & 1u;
                                if constexpr (DK) v[i] = p * ((kept ? drop.keep_scale * dp[i] : 0.f) - d4[e]);
                                else v[i] = kept ? p : 0.f;  // the keep scale rides in out_scale
                            } else {
                                v[i] = DK ? p * (dp[i] - d4[e]) : p;
                            }
                        }
                    }
                    // B operand (P for dV, dS for dK) of k-steps 0 and 1.
                    const bf16x8 bop0 = pack_bf16x8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
                    const bf16x8 bop1 = pack_bf16x8(v[8], v[9], v[10], v[11], v[12], v[13], v[14], v[15]);
                    // k-step s2 covers queries 32 qh + 16 s2 + {4h + e, 8 + 4h + e}.
                    const bf16* at = DK ? qt : gt;  // A = Q^T (dK) or dO^T (dV)
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
                        acc[db] = mfma_bf16_32x32x16(lds_read_tr_a(at + 32 * qh * RS + tr_off + 32 * db, RS), bop0,
                                                     acc[db]);
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
                        acc[db] = mfma_bf16_32x32x16(lds_read_tr_a(at + (32 * qh + 16) * RS + tr_off + 32 * db, RS),
                                                     bop1, acc[db]);
                }
            }
            store_block(buf ^ 1);
            __syncthreads();
        };
        for (int iq = iq0; iq < iq_split; ++iq) step(iq, std::true_type{});
        for (int iq = max(iq0, iq_split); iq < nqblk; ++iq) step(iq, std::false_type{});
    };
    // Grouped heads: the G query heads sharing this key/value head one after
    // the other, their contributions summed in the same accumulators.
    for (int g = 0; g < G; ++g) run_head(qh0 + g);

    // Register i of block db holds dim 32 db + c_row(i, h) of this lane's key.
    if (key < N) {
        OutT* op = dOut + base + (int64_t)key * D + 4 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_grad4(op + 32 * db + 8 * r,
                            f32x4{acc[db][4 * r] * out_scale, acc[db][4 * r + 1] * out_scale,
                                  acc[db][4 * r + 2] * out_scale, acc[db][4 * r + 3] * out_scale});
    }
}

// ---------------------------------------------------------------------------
// 2'. dK and dV in one kernel, by paired wavefronts (d = 128).  A workgroup
//    owns 128 keys; wavefront pair p (wavefronts p and p + 4) owns keys
//    32 p .. 32 p + 31.  The first of the pair computes S and P (as the dV
//    kernel does), hands P to its partner through LDS and accumulates dV; the
//    second computes dP and, with its partner's P, dS and dK.  S is thus
//    computed once for both gradients (8 products per tile instead of the
//    separate kernels' 10) while each wavefront still holds a single fp32
//    accumulator, so two wavefronts share each SIMD as before.  Per 64-query
//    step n:
//      phase 1  dV wavefront: S, P (masked), P -> LDS      dK wavefront: dP - D, then
//                                                          dK^T += Q^T dS of step n-1
//      barrier
//      phase 2  dV wavefront: dV^T += dO^T P              dK wavefront: dS of step n
//    so each wavefront's VALU work (softmax; dS) runs beside its partner's
//    MFMAs; the last step's dK products follow the loop.
//    Without dropout the row statistics ride in the products: the staged Q
//    and dO rows carry one more k-step, in their padding columns, holding
//    -L/c and -D split exactly into three bf16 parts (fold_parts), and the
//    wavefronts' register operands a matching k-step of ones, so the S chain
//    yields S - L/c (P = 2^(c (S - L/c))) and the dP chain dP - D.  That costs
//    one MFMA per eight and removes the per-row L and D values a lane would
//    otherwise read from LDS as four 16-byte broadcasts per 32 queries each.
//    With dropout (dS needs dP and D apart) L and D are read as in the
//    separate kernels, P crosses in fp32 and every value is formed by the
//    same operations in the same order as there, so the results are bitwise
//    theirs; the dV wavefront hands P with its sign bit set where the element
//    is dropped, and the dK wavefront needs no generator of its own.  (At
//    d = 64 the separate kernels are faster and are used instead.)
constexpr int kPairs = kBwdWaves / 2;
// MFMAs of read-ahead for the transposing-read operands of the dV and dK
// products.
#ifndef FA_TR_AHEAD
#define FA_TR_AHEAD 3
#endif
constexpr int kTrAhead = FA_TR_AHEAD;
constexpr int kFusedBkv = 32 * kPairs;  // keys per workgroup

// x as hi + mid + lo, three bf16 values whose sum is x exactly (x finite:
// each part takes the next 8 significant bits, and the residuals are exact
// in fp32), packed as the 8 elements {hi, mid, lo, 0, 0, 0, 0, 0}.  -inf
// (a row past N: P = 0) becomes {-inf, 0, 0, ...}.
__device__ __forceinline__ u32x4 fold_parts(float x) {
    bf16 hi = (bf16)x, mid = (bf16)0.f, lo = (bf16)0.f;
    if (x != -INFINITY) {
        const float r1 = x - (float)hi;
        mid = (bf16)r1;
        lo = (bf16)(r1 - (float)mid);
    }
    const bf16x8 v = {hi, mid, lo, (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    return __builtin_bit_cast(u32x4, v);
}

template <int D, bool CAUSAL, bool GROUPED, bool DROPOUT, typename OutT>
__global__ __launch_bounds__(kBwdThreads, 8 / kBwdWaves) void bwd_dkdv_fused_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    OutT* __restrict__ dKout, OutT* __restrict__ dVout, int N, int BKV, int nkb, ScoreScale ss, float dk_scale,
    float dv_scale, int Hq, int G_arg, DropoutParams drop, int nx) {
    const float scale_log2 = ss.c;
    static_assert(D == 128, "the paired kernel is built for d = 128");
    const int G = GROUPED ? G_arg : 1;
    constexpr int BQ = kDkvBq;
    constexpr int NQH = BQ / 32;
    constexpr int RS = D + 32;  // swizzled rows (pair_swz)
    constexpr bool FOLD = !DROPOUT;  // L and D ride in the products
    constexpr int NKS = D / 16 + (FOLD ? 1 : 0);  // k-steps of the S and dP chains
    static_assert(!FOLD || RS >= D + 16, "the folded k-step lives in the row padding");
    __shared__ __attribute__((aligned(16))) bf16 sQ[2][BQ * RS];
    __shared__ __attribute__((aligned(16))) bf16 sdO[2][BQ * RS];
    __shared__ __attribute__((aligned(16))) float sL[FOLD ? 1 : 2][BQ];
    __shared__ __attribute__((aligned(16))) float sD[FOLD ? 1 : 2][BQ];
    // P of pair p, sub-block qh, register group r, lane: one float4 per lane.
    __shared__ __attribute__((aligned(16))) f32x4 sP[kPairs][NQH][4][64];
    __shared__ __attribute__((aligned(16))) uint32_t sKeep[DROPOUT ? kPairs : 1][32];

    const int w = wave_id();
    // Wavefronts w and w + 4 share a SIMD (measured: pairing w with w + 1
    // instead is 7% slower), so each SIMD runs one wavefront of each role.
    const bool dvw = w < kPairs;  // wave-uniform role
    const int pr = dvw ? w : w - kPairs;
    // Persistent workgroups (nx per XCD) over the XCD's (key/value head, key
    // block) tasks in snake order, as in the forward.
    const int xi = block_id() % kNumXcd, ci = block_id() / kNumXcd;
    for (int round = 0;; ++round) {
    const int slot = round * nx + ((round & 1) ? nx - 1 - ci : ci);
    if (slot >= xcd_tasks(BKV * nkb)) break;  // past this XCD's share
    const int task = xcd_task(slot * kNumXcd + xi, BKV * nkb);
    if (task >= BKV * nkb) break;
    // (Lane offsets recomputed per task: hoisted out of the task loop they
    // would stay live across it.)
    int tid = thread_id();
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, lq = lane & 31, h = lane >> 5;
    const int kvh = task / nkb;
    const int kb = task % nkb;
    const int k0 = kb * kFusedBkv;
    const int kw0 = k0 + 32 * pr;
    const int key = kw0 + lq;
    const int64_t base = (int64_t)kvh * N * D;
    const int qh0 = (kvh / (Hq / G)) * Hq + (kvh % (Hq / G)) * G;
    const uint32_t head_bytes = (uint32_t)N * D * 2;

    // K^T (dV wavefront) or V^T (dK wavefront) operands of this lane's key;
    // with FOLD a last k-step of ones (lane half 0: elements 0..2) meets the
    // parts of -L/c or -D in the staged rows.
    bf16x8 kvf[NKS];
    if constexpr (FOLD) {
        const bf16 one = h == 0 ? (bf16)1.f : (bf16)0.f, z = (bf16)0.f;
        kvf[D / 16] = bf16x8{one, one, one, z, z, z, z, z};
    }
    {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((dvw ? K : V) + base, head_bytes);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            kvf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(rs, (lq * D + 16 * ks + 8 * h) * 2, kw0 * D * 2));
        wait_vmem_loads();
        // The dV wavefront's K carries the sign of the scale in S = Q K^T
        // (ScoreScale); dk_scale is the signed scale.
        if (dvw) {
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) kvf[ks] = apply_sign(kvf[ks], ss);
        }
    }
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    const int nqblk = (N + BQ - 1) / BQ;
    const int iq0 = CAUSAL ? k0 / BQ : 0;
    const int iq_split = CAUSAL ? min(nqblk, (k0 + kFusedBkv - 1) / BQ + 1) : iq0;
    TileStager<D, BQ> stq(tid, RS, true), stg(tid, RS, true);
    // L and D of the staged block's rows travel through the first wavefront's
    // lanes (thread t: row t).  L is kept as loaded until the block is stored:
    // scaling it at load time made that wavefront wait for the load, and with
    // it for the tile loads issued before it, at the start of every step
    // (carrying the rows on lanes of the dK wavefronts instead measured
    // slower).
    // -L/c is formed as -L2 times 1/c, the reciprocal taken once: a division
    // per step sat on the first wavefront's path to the step's end barrier.
    // Only the sum of the three parts matters, and c (S - L2 (1/c)) equals
    // c S - L2 to within rounding.  (The row index is kept in its own
    // variable: written as tid directly, the same code compiled to a register
    // allocation that ran 1-4% slower.)
    const bool stat_lane = tid < BQ;
    const int srow = tid;
    const float inv_c = 1.f / scale_log2;
    float lreg = 0.f, dreg = 0.f;
    // Row reads: k-step ks of row lq is logical chunk 2 ks + h, stored at
    // 4 (ks / 2) + ((2 (ks % 2) + h) ^ pair_swz(lq)); one base per parity of ks.
    const int row_off0 = lq * RS + 8 * (h ^ pair_swz(lq));
    const int row_off1 = lq * RS + 8 * ((2 + h) ^ pair_swz(lq));
    // Transposing reads: the lane's first row tr_row and second row tr_row + 8
    // have their own swizzles.
    const int trc = tr_col(lane);
    const int tr_off0 = tr_row(lane) * RS + 8 * ((trc >> 3) ^ pair_swz(tr_row(lane))) + (trc & 7);
    const int tr_off1 = (tr_row(lane) + 8) * RS + 8 * ((trc >> 3) ^ pair_swz(tr_row(lane) + 8)) + (trc & 7);
    auto read_tr = [&](const bf16* p) __attribute__((always_inline)) {
        const bf16x4 lo = lds_read_tr(p + tr_off0), hi = lds_read_tr(p + tr_off1);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    // Each role runs the loop as its own copy (DVW fixed at compile time), so
    // no role test branches inside a step and splits its scheduling regions;
    // both copies pass the same barriers.
    auto run_head = [&](int qh_idx, auto role_tag) __attribute__((always_inline)) {
        constexpr bool DVW = decltype(role_tag)::value;
        const int64_t qbase = (int64_t)qh_idx * N;
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + qbase * D, head_bytes);
        const __amdgpu_buffer_rsrc_t grs = make_rsrc(dO + qbase * D, head_bytes);
        const float* lse_h = LSE + qbase;
        const float* d_h = Dl + qbase;
        auto load_block = [&](int iq) {
            const int i0 = iq * BQ;
            stq.load(qrs, i0);
            stg.load(grs, i0);
            if (stat_lane) {
                const int r = min(i0 + srow, N - 1);
                lreg = i0 + srow < N ? lse_h[r] : INFINITY;
                dreg = i0 + srow < N ? d_h[r] : 0.f;
            }
        };
        auto store_block = [&](int buf) {
            stq.store(sQ[buf], RS);
            stg.store(sdO[buf], RS);
            if (stat_lane) {
                const float l2 = lreg * kLog2e;  // log2 domain; +inf past N
                if constexpr (FOLD) {
                    // Columns D .. D+7 of the row: the parts of -L/c and -D
                    // (l2 = +inf past N gives -inf: P = 0).
                    const int fc = srow * RS + 8 * ((D / 8) ^ pair_swz(srow));
                    *reinterpret_cast<u32x4*>(&sQ[buf][fc]) = fold_parts(-l2 * inv_c);
                    *reinterpret_cast<u32x4*>(&sdO[buf][fc]) = fold_parts(-dreg);
                } else {
                    sL[buf][srow] = l2;
                    sD[buf][srow] = dreg;
                }
            }
        };
        if constexpr (FOLD) {
            // Columns D+8 .. D+15 (the folded k-step of lane half 1) stay zero;
            // the tile stores never touch them.
            if (tid < 4 * BQ) {
                const int t = tid % BQ, b = (tid / BQ) & 1;
                bf16* dst = (tid / BQ) < 2 ? sQ[b] : sdO[b];
                *reinterpret_cast<u32x4*>(&dst[t * RS + 8 * ((D / 8 + 1) ^ pair_swz(t))]) = u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (iq0 < nqblk) {
            load_block(iq0);
            store_block(0);
        }
        __syncthreads();
        // The dK wavefront defers its dK MFMAs by one step: dS of step n is
        // formed in phase 2 of step n (beside its partner's dV MFMAs) and its
        // products are issued in phase 1 of step n + 1 (beside its partner's
        // softmax), against step n's Q tile, which stays in the other buffer
        // until step n + 1 stages over it at its end.
        bf16x8 dsk[2 * NQH];
        bool pend = false;      // wave-uniform: dsk holds an unissued step
        const bf16* q_prev = sQ[0];
        auto dk_products = [&](const bf16* qsrc) __attribute__((always_inline)) {
#pragma unroll
            for (int qh = 0; qh < NQH; ++qh) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc[db] = mfma_bf16_32x32x16(read_tr(qsrc + 32 * qh * RS + 32 * db), dsk[2 * qh], acc[db]);
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc[db] = mfma_bf16_32x32x16(read_tr(qsrc + (32 * qh + 16) * RS + 32 * db), dsk[2 * qh + 1],
                                                 acc[db]);
            }
            pin_read_ahead<2 * NQH * (D / 32), 2, kTrAhead>();
        };
        auto step = [&](int iq, auto mask_tag) __attribute__((always_inline)) {
            constexpr bool MASK = decltype(mask_tag)::value;
            const int buf = (iq - iq0) & 1;
            load_block(min(iq + 1, nqblk - 1));
            const int i0 = iq * BQ;
            const bool active = !CAUSAL || !MASK || __builtin_amdgcn_readfirstlane(i0 + BQ - 1 >= kw0);
            const bf16* qt = sQ[buf];
            const bf16* gt = sdO[buf];
            // Phase 1: S (dV wavefront, rows of Q) or dP (dK wavefront, rows of
            // dO) for every 32-query sub-block, as interleaved chains with each
            // row fragment requested AHEAD MFMAs before its use.
            f32x16 t[NQH];
            bf16x8 bop[2 * NQH];
            if (active) {
                const bf16* src = DVW ? qt : gt;
                constexpr int NR = NQH * NKS, AHEAD = 4;
                auto rread = [&](int r) {
                    const int ks = r / NQH;
                    return lds_read16_early(src + 32 * (r % NQH) * RS + ((ks & 1) ? row_off1 : row_off0) +
                                            32 * (ks >> 1));
                };
                bf16x8 ra[NR];
#pragma unroll
                for (int r = 0; r < AHEAD; ++r) ra[r] = rread(r);
#pragma unroll
                for (int qh = 0; qh < NQH; ++qh) t[qh] = f32x16{};
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    if (r + AHEAD < NR) ra[r + AHEAD] = rread(r + AHEAD);
                    t[r % NQH] = mfma_bf16_32x32x16(ra[r], kvf[r / NQH], t[r % NQH]);
                }
                pin_read_ahead<NR, 1, AHEAD>();
                // The dK wavefront forms dP - D while its partner computes P,
                // leaving one product per element for phase 2 (with FOLD the
                // chain has formed it).
                if constexpr (!DROPOUT && !FOLD && !DVW) {
                    {
#pragma unroll
                        for (int qh = 0; qh < NQH; ++qh)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[buf][32 * qh + 8 * r + 4 * h]);
#pragma unroll
                                for (int e = 0; e < 4; ++e) t[qh][4 * r + e] -= d4[e];
                            }
                    }
                }
                if constexpr (DVW) {
#pragma unroll
                    for (int qh = 0; qh < NQH; ++qh) {
                        uint32_t keep_bits[4];  // bit lq of word e of group r: query 32 qh + 8 r + 4 h + e kept
                        if constexpr (DROPOUT) {
                            const u32x4 wd = dropout_words(drop, qh_idx, i0 + 32 * qh + lq, kw0 / 32, h);
                            uint32_t bits = 0;
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                bits |= (dropout_keep(wd, r, drop.thr) ? 1u : 0u) << (8 * (r >> 2) + 4 * h + (r & 3));
                            const auto sw = __builtin_amdgcn_permlane32_swap(bits, bits, false, false);
                            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                            if (h == 0) sKeep[pr][lq] = sw[0] | sw[1];
                            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const u32x4 k4 = *reinterpret_cast<const u32x4*>(&sKeep[pr][8 * r + 4 * h]);
                                keep_bits[r] = ((k4[0] >> lq) & 1u) | (((k4[1] >> lq) & 1u) << 1) |
                                               (((k4[2] >> lq) & 1u) << 2) | (((k4[3] >> lq) & 1u) << 3);
                            }
                        }
                        float v[16];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            f32x4 l4 = f32x4{};
                            if constexpr (!FOLD) l4 = *reinterpret_cast<const f32x4*>(&sL[buf][32 * qh + 8 * r + 4 * h]);
                            f32x4 hand;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int i = 4 * r + e;
                                float p = FOLD ? fast_exp2(t[qh][i] * scale_log2)
                                               : fast_exp2(fmaf(t[qh][i], scale_log2, -l4[e]));
                                if constexpr (MASK) {
                                    if (key > i0 + 32 * qh + c_row(i, h)) p = 0.f;
                                }
                                if constexpr (DROPOUT) {
                                    const bool kept = (keep_bits[r] >> e) & 1u;
                                    v[i] = kept ? p : 0.f;  // the keep scale rides in dv_scale
                                    hand[e] = kept ? p : -p;
                                } else {
                                    v[i] = p;
                                    hand[e] = p;
                                }
                            }
                            sP[pr][qh][r][lane] = hand;
                        }
                        bop[2 * qh] = pack_bf16x8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
                        bop[2 * qh + 1] = pack_bf16x8(v[8], v[9], v[10], v[11], v[12], v[13], v[14], v[15]);
                    }
                }
            }
            if constexpr (!DVW) {
                if (pend) dk_products(q_prev);
            }
            __syncthreads();  // P of every pair is in LDS
            // Phase 2: dS (dK wavefront; its products follow in the next
            // step) and the dV products.
            if (active) {
                if constexpr (!DVW) {
#pragma unroll
                    for (int qh = 0; qh < NQH; ++qh) {
                        float v[16];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const f32x4 got = sP[pr][qh][r][lane];
                            if constexpr (DROPOUT) {
                                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[buf][32 * qh + 8 * r + 4 * h]);
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const float p = fabsf(got[e]);
                                    const bool kept = !__builtin_signbit(got[e]);
                                    v[4 * r + e] = p * ((kept ? drop.keep_scale * t[qh][4 * r + e] : 0.f) - d4[e]);
                                }
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e) v[4 * r + e] = got[e] * t[qh][4 * r + e];
                            }
                        }
                        dsk[2 * qh] = pack_bf16x8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
                        dsk[2 * qh + 1] = pack_bf16x8(v[8], v[9], v[10], v[11], v[12], v[13], v[14], v[15]);
                    }
                }
                // dV wavefront: A = dO^T by transposing reads; k-step s2 of
                // sub-block qh covers queries 32 qh + 16 s2 + {4h + e, 8 + 4h + e}.
                if constexpr (DVW) {
#pragma unroll
                    for (int qh = 0; qh < NQH; ++qh) {
#pragma unroll
                        for (int db = 0; db < D / 32; ++db)
                            acc[db] = mfma_bf16_32x32x16(read_tr(gt + 32 * qh * RS + 32 * db), bop[2 * qh], acc[db]);
#pragma unroll
                        for (int db = 0; db < D / 32; ++db)
                            acc[db] = mfma_bf16_32x32x16(read_tr(gt + (32 * qh + 16) * RS + 32 * db),
                                                         bop[2 * qh + 1], acc[db]);
                    }
                    pin_read_ahead<2 * NQH * (D / 32), 2, kTrAhead>();
                }
            }
            if constexpr (!DVW) {
                pend = active;
                q_prev = qt;
            }
            store_block(buf ^ 1);
            __syncthreads();
        };
        for (int iq = iq0; iq < iq_split; ++iq) step(iq, std::true_type{});
        for (int iq = max(iq0, iq_split); iq < nqblk; ++iq) step(iq, std::false_type{});
        // The last step's products: its Q tile is intact (the last staging
        // store went to the other buffer).
        if constexpr (!DVW) {
            if (pend) dk_products(q_prev);
        }
        // Grouped heads: the next head's prologue stages into buffer 0.
        if constexpr (GROUPED) __syncthreads();
    };
    if (dvw) {
        for (int g = 0; g < G; ++g) run_head(qh0 + g, std::true_type{});
    } else {
        for (int g = 0; g < G; ++g) run_head(qh0 + g, std::false_type{});
    }

    if (key < N) {
        OutT* op = (dvw ? dVout : dKout) + base + (int64_t)key * D + 4 * h;
        const float os = dvw ? dv_scale : dk_scale;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_grad4(op + 32 * db + 8 * r, f32x4{acc[db][4 * r] * os, acc[db][4 * r + 1] * os,
                                                        acc[db][4 * r + 2] * os, acc[db][4 * r + 3] * os});
    }
    // The dK wavefronts' last products read LDS after the last step's
    // barrier; the next task stages over it.
    __syncthreads();
    }  // task loop
}

// ---------------------------------------------------------------------------
// 3. dQ.  Per tile of keys (kDqBkv), staged row-major in LDS (double buffered): K
//    (read both as rows and transposed) and V (rows).
//    Per wavefront (32 queries) and 32-key part of the tile, with C tiles [key x query]:
//      S^T  = K Q^T      (A = K rows from LDS, B = Q^T from registers)
//      dP^T = V dO^T     (A = V rows from LDS, B = dO^T from registers)
//      P^T = exp2(S^T c - L2), dS^T = P^T (dP^T - D)
//      dQ^T += K^T dS^T  (A = K^T: transposing LDS reads; B = dS^T from registers)

constexpr int kDqBq = 32 * kBwdWaves;  // query rows per workgroup
// Keys per step: 128 at d = 64 (fewer barriers and staging rounds per key),
// 64 at d = 128, where the dS operands of 128 keys, live until the step's dQ
// products, no longer fit in the registers.
template <int D>
constexpr int kDqBkv = D == 64 ? 128 : 64;

// DROPOUT: dS = P (z dP - D) with z the forward's dropout factor (0 or the
// keep scale); a lane holds a query row and 16 keys per C tile, the layout
// one Philox call covers.
template <int D, bool CAUSAL, bool DROPOUT, typename OutT>
__global__ __launch_bounds__(kBwdThreads, 8 / kBwdWaves) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    OutT* __restrict__ dQ, int N, int BH, int nqb, ScoreScale ss, float scale, int Hq, int G,
    DropoutParams drop, int nx) {
    const float scale_log2 = ss.c;
    constexpr int BKV = kDqBkv<D>;
    // K is read both as rows and transposed: at d = 128 the swizzled layout of
    // pair_swz, at d = 64 a padded stride that serves both.
    constexpr bool SWZ = D == 128;
    constexpr int KS = SWZ ? D + 32 : both_ways_stride<D>();
    constexpr int VS = D + 8;  // rows only
    __shared__ __attribute__((aligned(16))) bf16 sK[2][BKV * KS];
    __shared__ __attribute__((aligned(16))) bf16 sV[2][BKV * VS];

    const int w = wave_id();
    // Persistent workgroups over the XCD's (head, query block) tasks in
    // snake order, as in the forward.
    const int xi = block_id() % kNumXcd, ci = block_id() / kNumXcd;
    for (int round = 0;; ++round) {
    const int slot = round * nx + ((round & 1) ? nx - 1 - ci : ci);
    if (slot >= xcd_tasks(BH * nqb)) break;  // past this XCD's share
    int bh, qb;
    if (!wg_coords(slot * kNumXcd + xi, BH, nqb, CAUSAL, bh, qb)) break;  // heaviest query blocks first
    int tid = thread_id();
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, lq = lane & 31, h = lane >> 5;
    const int q0 = qb * kDqBq;
    const int qw0 = q0 + 32 * w;
    const int qrow = qw0 + lq;
    const int64_t base = (int64_t)bh * N * D;
    const int64_t kv_base = (int64_t)kv_head(bh, Hq, G) * N * D;  // grouped heads share K, V
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_base, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_base, head_bytes);

    bf16x8 qf[D / 16], gf[D / 16];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, head_bytes);
        const __amdgpu_buffer_rsrc_t grs = make_rsrc(dO + base, head_bytes);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            qf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(qrs, (lq * D + 16 * ks + 8 * h) * 2, qw0 * D * 2));
            gf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(grs, (lq * D + 16 * ks + 8 * h) * 2, qw0 * D * 2));
        }
    }
    const int qr = min(qrow, N - 1);
    const float l2 = qrow < N ? LSE[(int64_t)bh * N + qr] * kLog2e : 0.f;
    const float dq_d = qrow < N ? Dl[(int64_t)bh * N + qr] : 0.f;

    f32x16 dqacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqacc[db] = f32x16{};

    int ntiles = (N + BKV - 1) / BKV;
    if (CAUSAL) ntiles = min(ntiles, (min(q0 + kDqBq, N) - 1) / BKV + 1);
    TileStager<D, BKV> stk(tid, KS, SWZ), stv(tid, VS);
    // K row reads: k-step ks of row lq is logical chunk 2 ks + h (swizzled:
    // one base per parity of ks); transposing reads of K^T: one base per row
    // of the lane (tr_row, tr_row + 8).
    const int k_off0 = lq * KS + 8 * (SWZ ? h ^ pair_swz(lq) : h);
    const int k_off1 = SWZ ? lq * KS + 8 * ((2 + h) ^ pair_swz(lq)) : k_off0 + 16;
    const int v_off = lq * VS + 8 * h;
    const int trc = tr_col(lane);
    const int tr_off0 = tr_row(lane) * KS + (SWZ ? 8 * ((trc >> 3) ^ pair_swz(tr_row(lane))) + (trc & 7) : trc);
    const int tr_off1 = (tr_row(lane) + 8) * KS +
                        (SWZ ? 8 * ((trc >> 3) ^ pair_swz(tr_row(lane) + 8)) + (trc & 7) : trc);

    stk.load(krs, 0);
    stv.load(vrs, 0);
    stk.store(sK[0], KS);
    stv.store(sV[0], VS);
    __syncthreads();
    // Q carries the sign of the scale in S^T = K Q^T (ScoreScale); the Q loads
    // were issued before the first tile's and have landed by now.  dQ's own
    // factor, `scale`, is the signed scale.
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = apply_sign(qf[ks], ss);
    // One key tile.  MASK masks keys past N and (causal) keys after the query;
    // only the tiles at the diagonal and the ragged end need it, and they come
    // last, so the loop is split and the other tiles carry no mask code.
    auto step = [&](int j, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int buf = j & 1;
        const int jn = min(j + 1, ntiles - 1);
        stk.load(krs, jn * BKV);
        stv.load(vrs, jn * BKV);
        const int k0 = j * BKV;
        // Skip tiles past this wave's last query.  The test stays on the
        // unmasked tiles too, although it always passes there: the branch
        // keeps the next tile's staging out of the math's scheduling region
        // (without it the compiler moved the LDS stores up, where they wait
        // for the global loads, and dQ ran 19% slower).
        if (!CAUSAL || __builtin_amdgcn_readfirstlane(k0 <= qw0 + 31)) {
            const bf16* kt = sK[buf];
            const bf16* vt = sV[buf];
            bf16x8 dsf[BKV / 16];
#pragma unroll
            for (int kh = 0; kh < BKV / 32; ++kh) {
                f32x16 s = f32x16{}, dp = f32x16{};
                // Row fragments requested AHEAD MFMAs before their use (even r:
                // K rows for S^T, odd r: V rows for dP^T); the compiler's own
                // order read them one or two MFMAs ahead and waited before most
                // MFMAs (non-causal N18000 4% slower, causal within 1%).
                constexpr int NR = 2 * (D / 16), AHEAD = 4;
                auto rread = [&](int r) {
                    const int ks = r >> 1;
                    return (r & 1) ? lds_read16_early(vt + 32 * kh * VS + v_off + 16 * ks)
                                   : lds_read16_early(kt + 32 * kh * KS + ((ks & 1) ? k_off1 : k_off0) +
                                                      32 * (ks >> 1));
                };
                bf16x8 ra[NR];
#pragma unroll
                for (int r = 0; r < AHEAD; ++r) ra[r] = rread(r);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    if (r + AHEAD < NR) ra[r + AHEAD] = rread(r + AHEAD);
                    if (r & 1) dp = mfma_bf16_32x32x16(ra[r], gf[r >> 1], dp);
                    else s = mfma_bf16_32x32x16(ra[r], qf[r >> 1], s);
                }
                pin_read_ahead<NR, 1, AHEAD>();
                float v[16];
                u32x4 dw;
                if constexpr (DROPOUT) dw = dropout_words(drop, bh, qrow, k0 / 32 + kh, h);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float p = fast_exp2(fmaf(s[i], scale_log2, -l2));
                    if constexpr (MASK) {
                        const int kk = k0 + 32 * kh + c_row(i, h);
                        if (kk >= N || (CAUSAL && kk > qrow)) p = 0.f;
                    }
                    if constexpr (DROPOUT)
                        v[i] = p * ((dropout_keep(dw, i, drop.thr) ? drop.keep_scale * dp[i] : 0.f) - dq_d);
                    else
                        v[i] = p * (dp[i] - dq_d);
                }
                dsf[2 * kh] = pack_bf16x8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
                dsf[2 * kh + 1] = pack_bf16x8(v[8], v[9], v[10], v[11], v[12], v[13], v[14], v[15]);
            }
            // dQ^T += K^T dS^T; k-step s2 covers keys 16 s2 + {4h + e, 8 + 4h + e}.
#pragma unroll
            for (int s2 = 0; s2 < BKV / 16; ++s2)
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                {
                    const bf16* p = kt + 16 * s2 * KS + 32 * db;
                    const bf16x4 lo = lds_read_tr(p + tr_off0), hi = lds_read_tr(p + tr_off1);
                    dqacc[db] = mfma_bf16_32x32x16(bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]},
                                                   dsf[s2], dqacc[db]);
                }
            pin_read_ahead<(BKV / 16) * (D / 32), 2, kTrAhead>();
        }
        stk.store(sK[buf ^ 1], KS);
        stv.store(sV[buf ^ 1], VS);
        __syncthreads();
    };
    // Tiles [j_split, ntiles) reach the diagonal of some wave or the ragged end.
    const int j_split = CAUSAL ? min(ntiles, q0 / BKV) : (N % BKV ? ntiles - 1 : ntiles);
    for (int j = 0; j < j_split; ++j) step(j, std::false_type{});
    for (int j = j_split; j < ntiles; ++j) step(j, std::true_type{});

    if (qrow < N) {
        OutT* dqp = dQ + base + (int64_t)qrow * D + 4 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_grad4(dqp + 32 * db + 8 * r,
                            f32x4{dqacc[db][4 * r] * scale, dqacc[db][4 * r + 1] * scale,
                                  dqacc[db][4 * r + 2] * scale, dqacc[db][4 * r + 3] * scale});
    }
    // (The last step ended on a barrier after its last LDS read, so the next
    // task may stage at once.)
    }  // task loop
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

constexpr DropoutParams kNoDropout{0u, 1.f, 0u, 0u, 0u};

template <int D, bool CAUSAL, bool DK, bool DROPOUT, typename OutT>
hipError_t launch_dkdv_d(const bf16* q, const bf16* k, const bf16* v, const float* lse, const bf16* dout,
                         const float* delta, OutT* out, int B, int Hq, int Hkv, int N, float scale,
                         const DropoutParams& dp, hipStream_t stream) {
    const int nkb = (N + kDkvBkv - 1) / kDkvBkv, BKV = B * Hkv;
    const dim3 grid(grid_for_tasks(nkb * BKV));
    // dV's elements carry no keep scale (kept: P, dropped: 0); it is applied on output.
    const float out_scale = DK ? scale : (DROPOUT ? dp.keep_scale : 1.0f);
    if (Hq == Hkv)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, DK, false, DROPOUT, OutT>), grid, dim3(kBwdThreads), 0, stream,
                           q, k, v, dout, lse, delta, out, N, BKV, nkb, make_score_scale(scale, 1.f, 0x80008000u), out_scale, Hq, 1, dp);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, DK, true, DROPOUT, OutT>), grid, dim3(kBwdThreads), 0, stream,
                           q, k, v, dout, lse, delta, out, N, BKV, nkb, make_score_scale(scale, 1.f, 0x80008000u), out_scale, Hq, Hq / Hkv, dp);
    return hipGetLastError();
}
template <int D, bool CAUSAL, bool DROPOUT, typename OutT>
hipError_t launch_dkdv_fused_d(const bf16* q, const bf16* k, const bf16* v, const float* lse, const bf16* dout,
                               const float* delta, OutT* dk, OutT* dv, int B, int Hq, int Hkv, int N, float scale,
                               const DropoutParams& dp, hipStream_t stream) {
    const int nkb = (N + kFusedBkv - 1) / kFusedBkv, BKV = B * Hkv;
    const float dv_scale = DROPOUT ? dp.keep_scale : 1.0f;
    const ScoreScale ss = make_score_scale(scale, 1.f, 0x80008000u);
    if (Hq == Hkv) {
        auto kern = bwd_dkdv_fused_kernel<D, CAUSAL, false, DROPOUT, OutT>;
        const int nx = persistent_per_xcd(nkb * BKV, blocks_per_cu(kern, kBwdThreads));
        hipLaunchKernelGGL(kern, dim3(kNumXcd * nx), dim3(kBwdThreads), 0, stream, q, k, v, dout, lse, delta, dk, dv,
                           N, BKV, nkb, ss, scale, dv_scale, Hq, 1, dp, nx);
    } else {
        auto kern = bwd_dkdv_fused_kernel<D, CAUSAL, true, DROPOUT, OutT>;
        const int nx = persistent_per_xcd(nkb * BKV, blocks_per_cu(kern, kBwdThreads));
        hipLaunchKernelGGL(kern, dim3(kNumXcd * nx), dim3(kBwdThreads), 0, stream, q, k, v, dout, lse, delta, dk, dv,
                           N, BKV, nkb, ss, scale, dv_scale, Hq, Hq / Hkv, dp, nx);
    }
    return hipGetLastError();
}
template <int D, bool CAUSAL>
hipError_t launch_dkdv_fused_t(const bf16* q, const bf16* k, const bf16* v, const float* lse, const bf16* dout,
                               const float* delta, void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale,
                               const DropoutParams* dropout, bool grad_bf16, hipStream_t stream) {
    if (grad_bf16)
        return launch_dkdv_fused_d<D, CAUSAL, false>(q, k, v, lse, dout, delta, static_cast<bf16*>(dk),
                                                     static_cast<bf16*>(dv), B, Hq, Hkv, N, scale, kNoDropout, stream);
    if (dropout)
        return launch_dkdv_fused_d<D, CAUSAL, true>(q, k, v, lse, dout, delta, static_cast<float*>(dk),
                                                    static_cast<float*>(dv), B, Hq, Hkv, N, scale, *dropout, stream);
    return launch_dkdv_fused_d<D, CAUSAL, false>(q, k, v, lse, dout, delta, static_cast<float*>(dk),
                                                 static_cast<float*>(dv), B, Hq, Hkv, N, scale, kNoDropout, stream);
}
// out: fp32, or bf16 when grad_bf16 (bf16 gradients have no dropout variant).
template <int D, bool CAUSAL, bool DK>
hipError_t launch_dkdv_t(const bf16* q, const bf16* k, const bf16* v, const float* lse, const bf16* dout,
                         const float* delta, void* out, int B, int Hq, int Hkv, int N, float scale,
                         const DropoutParams* dropout, bool grad_bf16, hipStream_t stream) {
    if (grad_bf16)
        return launch_dkdv_d<D, CAUSAL, DK, false>(q, k, v, lse, dout, delta, static_cast<bf16*>(out), B, Hq, Hkv, N,
                                                   scale, kNoDropout, stream);
    if (dropout)
        return launch_dkdv_d<D, CAUSAL, DK, true>(q, k, v, lse, dout, delta, static_cast<float*>(out), B, Hq, Hkv, N,
                                                  scale, *dropout, stream);
    return launch_dkdv_d<D, CAUSAL, DK, false>(q, k, v, lse, dout, delta, static_cast<float*>(out), B, Hq, Hkv, N,
                                               scale, kNoDropout, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_dq_t(const bf16* q, const bf16* k, const bf16* v, const float* lse, const bf16* dout,
                       const float* delta, void* dq, int B, int Hq, int Hkv, int N, float scale,
                       const DropoutParams* dropout, bool grad_bf16, hipStream_t stream) {
    const int nqb = (N + kDqBq - 1) / kDqBq, BH = B * Hq;
    const ScoreScale ss = make_score_scale(scale, 1.f, 0x80008000u);
    auto launch = [&](auto kern, auto* out, const DropoutParams& dp) {
        const int nx = persistent_per_xcd(nqb * BH, blocks_per_cu(kern, kBwdThreads));
        hipLaunchKernelGGL(kern, dim3(kNumXcd * nx), dim3(kBwdThreads), 0, stream, q, k, v, dout, lse, delta, out, N,
                           BH, nqb, ss, scale, Hq, Hq / Hkv, dp, nx);
        return hipGetLastError();
    };
    if (grad_bf16) return launch(bwd_dq_kernel<D, CAUSAL, false, bf16>, static_cast<bf16*>(dq), kNoDropout);
    if (dropout) return launch(bwd_dq_kernel<D, CAUSAL, true, float>, static_cast<float*>(dq), *dropout);
    return launch(bwd_dq_kernel<D, CAUSAL, false, float>, static_cast<float*>(dq), kNoDropout);
}

}  // namespace

hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, int BHq, int N, int d,
                                 hipStream_t stream) {
    auto Op = static_cast<const bf16*>(o);
    auto G = static_cast<const bf16*>(dout);
    return d == 64 ? launch_pre_t<64>(Op, G, delta, BHq, N, stream) : launch_pre_t<128>(Op, G, delta, BHq, N, stream);
}

hipError_t launch_bwd_dv(const void* q, const void* k, const float* lse, const void* dout, void* dv, int B, int Hq,
                         int Hkv, int N, int d, float scale, bool causal, const DropoutParams* dropout, bool grad_bf16,
                         hipStream_t stream) {
    auto Q = static_cast<const bf16*>(q);
    auto K = static_cast<const bf16*>(k);
    auto G = static_cast<const bf16*>(dout);
#define FA_DV(DD, CC) \
    launch_dkdv_t<DD, CC, false>(Q, K, K, lse, G, nullptr, dv, B, Hq, Hkv, N, scale, dropout, grad_bf16, stream)
    if (d == 64) return causal ? FA_DV(64, true) : FA_DV(64, false);
    return causal ? FA_DV(128, true) : FA_DV(128, false);
#undef FA_DV
}

hipError_t launch_bwd_dk(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, void* dk, int B, int Hq, int Hkv, int N, int d, float scale, bool causal,
                         const DropoutParams* dropout, bool grad_bf16, hipStream_t stream) {
    auto Q = static_cast<const bf16*>(q);
    auto K = static_cast<const bf16*>(k);
    auto V = static_cast<const bf16*>(v);
    auto G = static_cast<const bf16*>(dout);
#define FA_DK(DD, CC) \
    launch_dkdv_t<DD, CC, true>(Q, K, V, lse, G, delta, dk, B, Hq, Hkv, N, scale, dropout, grad_bf16, stream)
    if (d == 64) return causal ? FA_DK(64, true) : FA_DK(64, false);
    return causal ? FA_DK(128, true) : FA_DK(128, false);
#undef FA_DK
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                           const float* delta, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, float scale,
                           bool causal, const DropoutParams* dropout, bool grad_bf16, hipStream_t stream) {
    auto Q = static_cast<const bf16*>(q);
    auto K = static_cast<const bf16*>(k);
    auto V = static_cast<const bf16*>(v);
    auto G = static_cast<const bf16*>(dout);
    // At d = 64 the separate kernels are faster: their steps are too short
    // for the paired kernel's hand-over to pay.  Below |scale| = 2^-100 the
    // paired kernel's folded -L/c (L < 2^5 there) could leave the fp32 range,
    // so such calls take the separate kernels too (scale 0 folds exactly).
    const bool tiny = scale != 0.f && fabsf(scale) < 0x1p-100f;
    if (d == 64 || (tiny && !dropout)) {
        hipError_t e = launch_bwd_dv(q, k, lse, dout, dv, B, Hq, Hkv, N, d, scale, causal, dropout, grad_bf16, stream);
        if (e != hipSuccess) return e;
        return launch_bwd_dk(q, k, v, lse, dout, delta, dk, B, Hq, Hkv, N, d, scale, causal, dropout, grad_bf16,
                             stream);
    }
    return causal ? launch_dkdv_fused_t<128, true>(Q, K, V, lse, G, delta, dk, dv, B, Hq, Hkv, N, scale, dropout,
                                                   grad_bf16, stream)
                  : launch_dkdv_fused_t<128, false>(Q, K, V, lse, G, delta, dk, dv, B, Hq, Hkv, N, scale, dropout,
                                                    grad_bf16, stream);
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, void* dq, int B, int Hq, int Hkv, int N, int d, float scale, bool causal,
                         const DropoutParams* dropout, bool grad_bf16, hipStream_t stream) {
    auto Q = static_cast<const bf16*>(q);
    auto K = static_cast<const bf16*>(k);
    auto V = static_cast<const bf16*>(v);
    auto G = static_cast<const bf16*>(dout);
#define FA_DQ(DD, CC) launch_dq_t<DD, CC>(Q, K, V, lse, G, delta, dq, B, Hq, Hkv, N, scale, dropout, grad_bf16, stream)
    if (d == 64) return causal ? FA_DQ(64, true) : FA_DQ(64, false);
    return causal ? FA_DQ(128, true) : FA_DQ(128, false);
#undef FA_DQ
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv,
                           int N, int d, float scale, bool causal, const DropoutParams* dropout, bool grad_bf16,
                           hipStream_t stream) {
    hipError_t e = launch_bwd_preprocess(o, dout, delta, B * Hq, N, d, stream);
    if (e != hipSuccess) return e;
    e = launch_bwd_dkdv(q, k, v, lse, dout, delta, dk, dv, B, Hq, Hkv, N, d, scale, causal, dropout, grad_bf16,
                        stream);
    if (e != hipSuccess) return e;
    return launch_bwd_dq(q, k, v, lse, dout, delta, dq, B, Hq, Hkv, N, d, scale, causal, dropout, grad_bf16, stream);
}

}  // namespace fa
