// fa_decode.hip -- split-KV decode (Flash-Decoding) for gfx950 (MI355X).
//
// Method: the "FlashAttention" deep-dive page (tirogla.com), section
// "Implementation notes": with a single query row per head there is no
// query-block parallelism, so the key/value cache is cut into chunks processed
// in parallel, each producing a partial (m, l, acc) triple for its keys, and
// the triples are merged with the online-softmax rescaling rule:
//   m = max_s m_s,  l = sum_s 2^(m_s - m) l_s,  acc = sum_s 2^(m_s - m) acc_s,
//   O = acc / l,  L = (m + log2 l) ln 2                   (log2-domain m).
// Grouped heads (same section): the G query heads that share a key/value head
// are processed together as the 32 columns of one MFMA tile, so each K/V byte
// is read from HBM once for all of them.
//
// Kernel 1 (one workgroup of 8 wavefronts per (key/value head, group of up
// to 32 query heads, split)): each wavefront walks every 8th 32-key tile of
// the split, staging it through its own LDS region (HBM -> registers -> LDS;
// the next tile's loads are in flight while the current one is computed):
//   S^T  = K Q^T        (A = K rows from LDS, B = Q^T held in registers)
//   P^T  = 2^(S^T c - m) with a lagging running max m, as in the forward
//   O^T += V^T P^T      (A = V^T through transposing LDS reads, B = P^T)
// The eight wavefronts' triples are merged through LDS; with one split the
// workgroup writes O and L, otherwise its triple goes to the workspace.
// Kernel 2 merges the splits' triples of each (batch, query head) row.
//
// The kernel is bound by HBM bandwidth (K and V are read once, 4 d bytes per
// key per key/value head); the MFMA and LDS work per byte is an order of
// magnitude below their limits.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecTile = 32;                     // keys per wavefront step
constexpr int kDecChunk = kDecWaves * kDecTile;  // split granularity (keys)
constexpr int kDecSlots = 32;                    // query heads per workgroup (MFMA columns)
constexpr float kDecRescale = 8.0f;              // lagging-max threshold (log2 units)
constexpr int kDecAutoWorkgroups = 256;          // automatic split count: about one workgroup per CU

template <int D>
struct DecLayout {
    static constexpr int KS = D + 8;                   // K rows: 16-byte reads
    static constexpr int VS = D == 128 ? D + 24 : D + 8;  // V rows: transposing reads
    static constexpr int AS = D + 4;                   // fp32 partial rows of the merge
    static constexpr int WAVE_BYTES = kDecTile * (KS + VS) * 2;
    static constexpr int STAGE_BYTES = kDecWaves * WAVE_BYTES;
    static constexpr int MERGE_BYTES = kDecWaves * kDecSlots * AS * 4;
    static constexpr int BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
    static constexpr int DCH = D / 8;                  // 16-byte chunks per row
    static constexpr int CH = kDecTile * DCH / 64;     // chunks per lane per tile (K and V each)
};

// STREAM: every K/V byte of the split is read by this workgroup only (one
// query group), so the loads carry the non-temporal hint; with several query
// groups the neighbouring workgroups re-read the split from L2.
template <int D, bool STREAM>
__global__ __launch_bounds__(kDecThreads, 1) void decode_split_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const int* __restrict__ kv_len, float* __restrict__ part_acc, float* __restrict__ part_ml,
    bf16* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Nk, int nqg, int splits, int chunk,
    int tasks, int BHq, ScoreScale ss) {
    const float scale_log2 = ss.c;
    using L = DecLayout<D>;
    constexpr int NKS = D / 16;  // k-steps of S
    constexpr int NDB = D / 32;  // 32-dimension blocks of O
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
    __shared__ float sM[kDecWaves][kDecSlots], sL[kDecWaves][kDecSlots];

    const int tid = thread_id(), lane = tid & 63, w = wave_id();
    const int lq = lane & 31, h = lane >> 5;
    const int task = xcd_task(block_id(), tasks);
    if (task >= tasks) return;
    // Task order: (batch, key/value head), split, query group -- the query
    // groups of one split are neighbours and share its K/V in one XCD's L2.
    const int qg = task % nqg;
    const int s = (task / nqg) % splits;
    const int bkv = task / (nqg * splits);
    const int b = bkv / Hkv;
    const int G = Hq / Hkv;
    const int hq0 = b * Hq + (bkv % Hkv) * G + qg * kDecSlots;  // flat first query head
    const int nvalid = min(kDecSlots, G - qg * kDecSlots);

    int n = Nk;
    if (kv_len) n = min(max(kv_len[b], 0), Nk);
    const int k_begin = s * chunk;
    const int k_end = min(k_begin + chunk, n);
    const int ntile = k_end > k_begin ? (k_end - k_begin + kDecTile - 1) / kDecTile : 0;
    const int my_tiles = ntile > w ? (ntile - w + kDecWaves - 1) / kDecWaves : 0;

    // Q^T operand (query slots past the group read as zero).
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + (int64_t)hq0 * D, (uint32_t)(nvalid * D * 2));
    bf16x8 qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, buffer_load16(qrs, (lq * D + 16 * ks + 8 * h) * 2, 0));

    const int64_t kv_base = (int64_t)bkv * Nk * D;
    const uint32_t head_bytes = (uint32_t)Nk * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_base, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_base, head_bytes);

    bf16* sK = reinterpret_cast<bf16*>(smem + w * L::WAVE_BYTES);
    bf16* sV = sK + kDecTile * L::KS;
    // Lane chunk r of a tile: row lane / DCH + r * (64 / DCH), 16-byte column lane % DCH.
    const int ld_row = lane / L::DCH, ld_col = lane % L::DCH;
    constexpr int ROWS_PER_PASS = 64 / L::DCH;
    u32x4 kreg[L::CH], vreg[L::CH];
    auto load_tile = [&](int t) {
        const int soff = (k_begin + (w + kDecWaves * t) * kDecTile) * D * 2;
#pragma unroll
        for (int r = 0; r < L::CH; ++r) {
            const int voff = ((ld_row + r * ROWS_PER_PASS) * D + 8 * ld_col) * 2;
            if constexpr (STREAM) {
                kreg[r] = buffer_load16_nt(krs, voff, soff);
                vreg[r] = buffer_load16_nt(vrs, voff, soff);
            } else {
                kreg[r] = buffer_load16(krs, voff, soff);
                vreg[r] = buffer_load16(vrs, voff, soff);
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int r = 0; r < L::CH; ++r) {
            const int row = ld_row + r * ROWS_PER_PASS;
            *reinterpret_cast<u32x4*>(&sK[row * L::KS + 8 * ld_col]) = kreg[r];
            *reinterpret_cast<u32x4*>(&sV[row * L::VS + 8 * ld_col]) = vreg[r];
        }
    };
    const int k_off = lq * L::KS + 8 * h;
    const int tr_off = tr_row(lane) * L::VS + tr_col(lane);

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m = -INFINITY, l = 0.f;

    if (my_tiles > 0) {
        load_tile(0);
        store_tile();
    }
    // The sign of the scale rides on Q (ScoreScale); the Q loads were issued
    // before the first tile's and have landed by now.
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = apply_sign(qf[ks], ss);
    for (int t = 0; t < my_tiles; ++t) {
        // The region is this wavefront's own: LDS operations of one wavefront
        // execute in order, so a fence at wavefront scope (no instruction)
        // only keeps the compiler from moving reads across the writes.
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        load_tile(min(t + 1, my_tiles - 1));  // in flight during this tile's math
        const int key0 = k_begin + (w + kDecWaves * t) * kDecTile;

        f32x16 sc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            sc = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(sK + k_off + 16 * ks), qf[ks], sc);
        if (key0 + kDecTile > k_end) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (key0 + c_row(i, h) >= k_end) sc[i] = -INFINITY;
        }
        float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mx = fmaxf(fmaxf(mx, sc[i]), sc[i + 1]);
        mx = pair_max(mx) * scale_log2;
        if (__any(mx > m + kDecRescale)) {  // wave-uniform branch
            const float m_new = fmaxf(m, mx);
            const float alpha = fast_exp2(m - m_new);  // 0 on the first tile
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            m = m_new;
        }
        float rs = 0.f;
        bf16x8 pf[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(fmaf(sc[i], scale_log2, -m));
            rs += p;
            // k-step i/8 covers keys 16 (i/8) + 8 (j/4) + 4 h + j%4, j = i%8:
            // the k-order of the transposing V reads below.
            pf[i >> 3][i & 7] = (bf16)p;
        }
        l += rs;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                oacc[db] = mfma_bf16_32x32x16(lds_read_tr_a(sV + 16 * s2 * L::VS + 32 * db + tr_off, L::VS), pf[s2],
                                              oacc[db]);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        store_tile();  // the next tile (or this one again after the last)
    }

    // Merge the eight wavefronts' triples through LDS (the staging space is
    // free once every wavefront has passed the barrier).
    const float lt = pair_sum(l);
    __syncthreads();
    float* sAcc = reinterpret_cast<float*>(smem);
    {
        float* dst = sAcc + (w * kDecSlots + lq) * L::AS + 4 * h;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * r) =
                    f32x4{oacc[db][4 * r], oacc[db][4 * r + 1], oacc[db][4 * r + 2], oacc[db][4 * r + 3]};
        if (h == 0) {
            sM[w][lq] = m;
            sL[w][lq] = lt;
        }
    }
    __syncthreads();
    // 16 threads per query slot, D / 16 dimensions each.
    constexpr int PER = D / 16;
    const int slot = tid >> 4, d0 = (tid & 15) * PER;
    float mstar = -INFINITY;
#pragma unroll
    for (int v = 0; v < kDecWaves; ++v) mstar = fmaxf(mstar, sM[v][slot]);
    float acc[PER], lsum = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
    for (int v = 0; v < kDecWaves; ++v) {
        const float mv = sM[v][slot];
        const float wgt = mv == -INFINITY ? 0.f : fast_exp2(mv - mstar);  // a wavefront with no keys weighs 0
        lsum = fmaf(wgt, sL[v][slot], lsum);
        const float* src = sAcc + (v * kDecSlots + slot) * L::AS + d0;
#pragma unroll
        for (int e = 0; e < PER; e += 4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(src + e);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[e + c] = fmaf(wgt, a[c], acc[e + c]);
        }
    }
    if (slot >= nvalid) return;
    const int64_t row = hq0 + slot;
    if (splits == 1) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // no visible key: O = 0
        bf16* op = O + row * D + d0;
#pragma unroll
        for (int e = 0; e < PER; e += 4)
            *reinterpret_cast<bf16x4*>(op + e) =
                bf16x4{(bf16)(acc[e] * inv), (bf16)(acc[e + 1] * inv), (bf16)(acc[e + 2] * inv), (bf16)(acc[e + 3] * inv)};
        if (d0 == 0) LSE[row] = lsum > 0.f ? (mstar + fast_log2(lsum)) * kLn2 : -INFINITY;
    } else {
        const int64_t prow = (int64_t)s * BHq + row;
        float* pa = part_acc + prow * D + d0;
#pragma unroll
        for (int e = 0; e < PER; e += 4)
            *reinterpret_cast<f32x4*>(pa + e) = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
        if (d0 == 0) *reinterpret_cast<f32x2*>(part_ml + 2 * prow) = f32x2{mstar, lsum};
    }
}

// Merge of the splits' triples, one wavefront per (batch, query head) row.
// Lane s holds split s's (m, l) (64 splits per pass); the weights
// 2^(m_s - m) reach every lane by broadcast, and the accumulator rows of 16
// splits are requested before any is used.  A split with no visible key has
// m = -inf and weighs 0; a row with none at all gets O = 0 and L = -inf.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_acc,
                                                           const float* __restrict__ part_ml, bf16* __restrict__ O,
                                                           float* __restrict__ LSE, int BHq, int splits) {
    constexpr int PER = D / 64;
    constexpr int AHEAD = 16;
    const int row = block_id() * 4 + (thread_id() >> 6), lane = thread_id() & 63;
    if (row >= BHq) return;
    float mstar = -INFINITY;
    for (int s = lane; s < splits; s += 64) mstar = fmaxf(mstar, part_ml[2 * ((int64_t)s * BHq + row)]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mstar = fmaxf(mstar, __shfl_xor(mstar, off));
    float acc[PER], lsum = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int s0 = 0; s0 < splits; s0 += 64) {
        float wgt = 0.f;
        if (s0 + lane < splits) {
            const f32x2 ml = *reinterpret_cast<const f32x2*>(part_ml + 2 * ((int64_t)(s0 + lane) * BHq + row));
            wgt = ml[0] == -INFINITY ? 0.f : fast_exp2(ml[0] - mstar);
            lsum = fmaf(wgt, ml[1], lsum);
        }
        const int n = min(64, splits - s0);
        const float* src = part_acc + ((int64_t)s0 * BHq + row) * D + lane;
        for (int j0 = 0; j0 < n; j0 += AHEAD) {
            float a[AHEAD][PER];
#pragma unroll
            for (int j = 0; j < AHEAD; ++j)
#pragma unroll
                for (int e = 0; e < PER; ++e) a[j][e] = j0 + j < n ? src[(int64_t)(j0 + j) * BHq * D + 64 * e] : 0.f;
#pragma unroll
            for (int j = 0; j < AHEAD; ++j) {
                const float wj = __shfl(wgt, j0 + j);  // 0 past the last split
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj, a[j][e], acc[e]);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) O[(int64_t)row * D + lane + 64 * e] = (bf16)(acc[e] * inv);
    if (lane == 0) LSE[row] = lsum > 0.f ? (mstar + fast_log2(lsum)) * kLn2 : -INFINITY;
}

}  // namespace

DecodePlan decode_plan(int B, int Hq, int Hkv, int Nk, int num_splits) {
    DecodePlan p;
    const int nqg = (Hq / Hkv + kDecSlots - 1) / kDecSlots;
    const int max_splits = (Nk + kDecChunk - 1) / kDecChunk;
    int want = num_splits;
    if (want <= 0) {
        // About one workgroup per compute unit (one is resident per CU at a
        // time), but splits of at least 2048 keys -- 1024 when that would
        // leave fewer than 64 workgroups -- so that the fixed cost of a
        // workgroup (first tile's latency, the merge) stays small (measured
        // over batch 1..16, 8..32 key/value heads, 8K..128K keys).
        const long groups = (long)B * Hkv * nqg;
        want = (int)((kDecAutoWorkgroups + groups - 1) / groups);
        long cap = Nk / 2048;
        if (groups * cap < 64) cap = Nk / 1024;
        if (want > cap) want = (int)(cap > 1 ? cap : 1);
    }
    want = want < 1 ? 1 : (want > max_splits ? max_splits : want);
    const int per = (Nk + want - 1) / want;
    p.chunk = (per + kDecChunk - 1) / kDecChunk * kDecChunk;
    p.splits = (Nk + p.chunk - 1) / p.chunk;
    p.nqg = nqg;
    return p;
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const int* kv_len, void* o, float* lse, int B,
                         int Hq, int Hkv, int Nk, int d, float scale, const DecodePlan& plan, float* workspace,
                         hipStream_t stream) {
    const int BHq = B * Hq;
    const int tasks = B * Hkv * plan.nqg * plan.splits;
    float* pacc = workspace;
    float* pml = plan.splits > 1 ? workspace + (int64_t)plan.splits * BHq * d : nullptr;
    auto Qp = static_cast<const bf16*>(q);
    auto Kp = static_cast<const bf16*>(k);
    auto Vp = static_cast<const bf16*>(v);
    auto Op = static_cast<bf16*>(o);
    const ScoreScale ss = make_score_scale(scale, 1.f, 0x80008000u);
    const dim3 grid(grid_for_tasks(tasks)), mgrid((BHq + 3) / 4);
#define FA_DEC_LAUNCH(DD)                                                                                       \
    do {                                                                                                        \
        if (plan.nqg == 1)                                                                                      \
            hipLaunchKernelGGL((decode_split_kernel<DD, true>), grid, dim3(kDecThreads), 0, stream, Qp, Kp, Vp,  \
                               kv_len, pacc, pml, Op, lse, Hq, Hkv, Nk, plan.nqg, plan.splits, plan.chunk, tasks, \
                               BHq, ss);                                                                        \
        else                                                                                                    \
            hipLaunchKernelGGL((decode_split_kernel<DD, false>), grid, dim3(kDecThreads), 0, stream, Qp, Kp, Vp, \
                               kv_len, pacc, pml, Op, lse, Hq, Hkv, Nk, plan.nqg, plan.splits, plan.chunk, tasks, \
                               BHq, ss);                                                                        \
        hipError_t e = hipGetLastError();                                                                       \
        if (e != hipSuccess || plan.splits == 1) return e;                                                      \
        hipLaunchKernelGGL((decode_merge_kernel<DD>), mgrid, dim3(256), 0, stream, pacc, pml, Op, lse, BHq,     \
                           plan.splits);                                                                        \
        return hipGetLastError();                                                                               \
    } while (0)
    if (d == 64) FA_DEC_LAUNCH(64);
    FA_DEC_LAUNCH(128);
#undef FA_DEC_LAUNCH
}

}  // namespace fa
