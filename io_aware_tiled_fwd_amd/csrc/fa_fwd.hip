// fa_fwd.hip -- FlashAttention forward for gfx950 (MI355X).
//
// Method: the per-query-block loop of the "FlashAttention" deep-dive page
// (tirogla.com), section "How it works": load a Q block once, walk the K/V
// blocks, keep a running row max m and row sum l, rescale the partial output
// by alpha = exp(m - m_new), accumulate P V, and finally store O = acc / l and
// L = m + log l.  Exponentials are taken in base 2 with log2(e) folded into the
// scale, S, l and acc are fp32 and P is rounded to bf16 only for the P V product
// (same page, "Implementation notes").  Under a causal mask a key tile that
// lies wholly past a wavefront's last query is never computed, and the masking
// code runs only on the tiles the diagonal passes through, which the key loop
// reaches last (same page, "Implementation notes").  Keys past N are masked to
// -inf and query rows past N are computed on zeros and never stored (same
// page, the Triton kernel under "Code").
//
// Work split (FlashAttention-2's sequence-dimension parallelism, same page):
// one workgroup of 8 wavefronts per (batch*head, block of 256 query rows);
// each wavefront owns 32 query rows, so no softmax statistic is ever shared
// between wavefronts.  Each key tile of 64 keys is staged once in LDS, double
// buffered, and read by all eight wavefronts (two per SIMD), both tensors as
// plain row-major copies [64 keys][d]:
//   K  16-byte row reads                -> A operand of S^T = K Q^T
//   V  transposing reads (lds_read_tr_a) -> A operand V^T of O^T = V^T P^T
// The transposing read returns keys in the k order of the P^T registers
// (16 s + 8 (j/4) + 4 h + j%4), so P needs no shuffle.  Global loads for tile
// j+1 are issued into registers before tile j is computed and land in the
// other LDS buffers afterwards: one barrier per tile.
//
// Latency: the K fragments of S are read four MFMAs ahead, and the V^T
// fragments of the first two k-steps of O^T are read right after S, so that
// the exponentials of the softmax run while they arrive.  At d = 128 the
// unmasked tiles run instead as a hand-scheduled loop (fa_fwd_asm.inc) that
// issues the next tile's scores and this tile's P V between the softmax's
// VALU instructions.
//
// The grid is persistent: as many workgroups as fit on the GPU at once, each
// taking its XCD's (head, query block) tasks in snake order.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "fa_common.h"
#include "fa_fwd_asm.inc"
#include "fa_internal.h"

// FA_FWD_ASM = 0 builds the forward without the hand-scheduled key loop
// (every tile compiler-scheduled), for comparisons.
#ifndef FA_FWD_ASM
#define FA_FWD_ASM 1
#endif

namespace fa {

namespace {

constexpr int kFwdWaves = 8;
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kFwdBr = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBc = 64;              // keys per tile

typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// Byte address in LDS of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The four words of the buffer resource that make_rsrc builds, as SGPR
// operands of inline assembly.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return u32x4{lo, hi & 0xFFFFu, n, 0x00020000u};
}

// DROPOUT: P V uses P with the dropped elements zeroed (the dropout mask of
// fa_common.h); l and L stay those of the undropped P, and O carries the keep
// scale.
template <int D, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int BH, int nqb, ScoreScale ss, int Hq, int G,
    DropoutParams dp, int nx) {
    const float scale_log2 = ss.c;
    constexpr int BC = kFwdBc;
    constexpr int KS = D + 8;   // K row stride: 16 consecutive rows hit distinct banks (b128 reads)
    constexpr int VS = D + 32;   // V rows, read transposed: 4 rows x 64 B of a half wave on disjoint banks
    constexpr int DCH = D / 8;  // 16-byte chunks per row
    constexpr int CH = BC * DCH / kFwdThreads;  // K chunks per thread
    static_assert(CH * kFwdThreads == BC * DCH, "tile split");
    constexpr int NKS = D / 16;  // k-steps of S
    constexpr int NDB = D / 32;  // 32-dimension blocks of O
    constexpr int NPRE = 2;      // k-steps of O^T whose V^T fragments are read early

    __shared__ __attribute__((aligned(16))) bf16 sK[2][BC * KS];
    __shared__ __attribute__((aligned(16))) bf16 sV[2][BC * VS];

    const int w = wave_id();
    // Persistent workgroups: nx per XCD, as many as fit at once.  Workgroup ci of
    // XCD xi takes the XCD's tasks (wg_coords order: a head's query blocks
    // together, heaviest first) in snake order -- ci, then 2 nx - 1 - ci, then
    // 2 nx + ci, ... -- so that a heavy task and a light one alternate on every
    // CU.  Launching one workgroup per task instead left CUs idle between
    // tasks: workgroups are dealt to the XCDs in id order, so an XCD whose CUs
    // are all busy holds back the dispatch of the workgroups behind it.
    const int xi = block_id() % kNumXcd, ci = block_id() / kNumXcd;
    // (head, query block) of this workgroup's task in round r; false past the
    // XCD's share.
    auto task_of = [&](int r, int& bh_, int& qb_) -> bool {
        const int t = r * nx + ((r & 1) ? nx - 1 - ci : ci);
        if (t >= xcd_tasks(BH * nqb)) return false;
        return wg_coords(t * kNumXcd + xi, BH, nqb, CAUSAL, bh_, qb_);
    };
    constexpr int ROWS_PER_PASS = kFwdThreads / DCH;
    // The loads that open a task: this wave's Q fragments (the Q^T operand,
    // k-step ks = Q[row][16 ks + 8 h .. +7]) and the thread's chunks of K(0),
    // V(0) and K(1).  A task issues them for the next task right behind its
    // own output stores, so that their latency overlaps the stores' instead of
    // following it.
    bf16x8 qf[NKS];
    u32x4 k0p[CH], v0p[CH], k1p[CH];
    auto issue_task_loads = [&](int bh_, int qb_) __attribute__((always_inline)) {
        int t = thread_id();
        asm volatile("" : "+v"(t));
        const int ln = t & 63;
        const uint32_t hb = (uint32_t)N * D * 2;
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(Q + (int64_t)bh_ * N * D, hb);
        const int64_t kvb = (int64_t)kv_head(bh_, Hq, G) * N * D;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + kvb, hb);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(V + kvb, hb);
        const int qw = qb_ * kFwdBr + 32 * w;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qf[ks] = __builtin_bit_cast(
                bf16x8, buffer_load16(qr, ((ln & 31) * D + 16 * ks + 8 * (ln >> 5)) * 2, qw * D * 2));
        const int lo = ((t / DCH) * D + 8 * (t % DCH)) * 2;
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            k0p[r] = buffer_load16(kr, lo + r * ROWS_PER_PASS * D * 2, 0);
            v0p[r] = buffer_load16(vr, lo + r * ROWS_PER_PASS * D * 2, 0);
            k1p[r] = buffer_load16(kr, lo + r * ROWS_PER_PASS * D * 2, BC * D * 2);
        }
    };
    int bh, qb;
    if (!task_of(0, bh, qb)) return;
    issue_task_loads(bh, qb);
    for (int round = 0;; ++round) {
    // The lane's offsets are recomputed for every task (the empty asm hides
    // that they do not change): hoisted out of the task loop they would stay
    // live across it and push the kernel past its register budget.
    int tid = thread_id();
    asm volatile("" : "+v"(tid));
    int lane = tid & 63, lq = lane & 31, h = lane >> 5;
    const int q0 = qb * kFwdBr;
    const int qw0 = q0 + 32 * w;  // first query row of this wave
    int qrow = qw0 + lq;          // this lane's query row
    const int64_t base = (int64_t)bh * N * D;
    const int64_t kv_base = (int64_t)kv_head(bh, Hq, G) * N * D;  // grouped heads share K, V

    // Per-head buffer resources: rows past N read as zero.
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_base, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_base, head_bytes);

    // Accumulators and the running statistics: set by the assembly loop, or
    // to their initial values (O = 0, m = -inf, l = 0) before the first
    // compiler-scheduled tile.
    f32x16 oacc[NDB];
    float m;     // reference maximum of the scaled (log2-domain) scores
    float mneg;  // -m, or 0 while m = -inf (a row with nothing visible yet)
    float l;     // running partial sum over this lane's keys

    int ntiles = (N + BC - 1) / BC;
    if (CAUSAL) ntiles = min(ntiles, (min(q0 + kFwdBr, N) - 1) / BC + 1);

    // Staging of tile j+1 through registers, K and V alike as row-major
    // copies: thread chunk r covers row (tid + 512 r) / DCH, 16-byte column
    // tid % DCH.  Tile offsets ride in the scalar offset.
    int ld_off = ((tid / DCH) * D + 8 * (tid % DCH)) * 2;
    u32x4 kreg[CH], vreg[CH];
    auto load_tile = [&](int j) {
        const int soff = j * BC * D * 2;
#pragma unroll
        for (int r = 0; r < CH; ++r) kreg[r] = buffer_load16(krs, ld_off + r * ROWS_PER_PASS * D * 2, soff);
#pragma unroll
        for (int r = 0; r < CH; ++r) vreg[r] = buffer_load16(vrs, ld_off + r * ROWS_PER_PASS * D * 2, soff);
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            const int c = tid + kFwdThreads * r;
            *reinterpret_cast<u32x4*>(&sK[buf][(c / DCH) * KS + 8 * (c % DCH)]) = kreg[r];
            *reinterpret_cast<u32x4*>(&sV[buf][(c / DCH) * VS + 8 * (c % DCH)]) = vreg[r];
        }
    };

    // Per-lane offsets of the K rows and the V^T rows.
    int k_off = lq * KS + 8 * h;
    int v_off = tr_row(lane) * VS + tr_col(lane);

    // Tiles before j_split are wholly visible to every wave of the workgroup.
    const int j_split = CAUSAL ? min(ntiles, q0 / BC) : (N % BC ? ntiles - 1 : ntiles);

    // The unmasked tiles of the d = 128 forward run as one hand-scheduled
    // block of inline assembly (fa_fwd_asm.inc, written by gen_fwd_asm.py):
    // the next tile's score MFMAs and the current tile's P V MFMAs are issued
    // between the softmax's VALU instructions.  It stages K(0), V(0), K(1)
    // from the registers loaded here, computes every unmasked tile, and
    // leaves K(j_split), V(j_split) in LDS buffer j_split & 1 for the masked
    // tiles below, as the compiler-scheduled steps expect.
    constexpr bool kAsmLoop = FA_FWD_ASM && D == 128 && !DROPOUT;
    const bool use_asm = kAsmLoop && j_split >= 1;
    // Q's loads and the first tile's share one memory round trip; the one
    // wait for both keeps the compiler from guarding Q's uses in the loop.
    // Loads and stores of the compiler-scheduled steps are unconditional (the
    // last step re-reads the final tile into the idle buffer): every path
    // then drains the load counter at the store, so the compiler never makes
    // the math wait on a pending load.
    u32x8 kst, vst, k1st;  // the assembly loop's first tiles: K(0), V(0), K(1)
    // The task's opening loads (issued by the previous task, or before the
    // loop) and the previous task's output stores complete here.
    wait_vmem_loads();
    if (use_asm) {
#pragma unroll
        for (int r = 0; r < CH; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kst[4 * r + e] = k0p[r][e];
                vst[4 * r + e] = v0p[r][e];
                k1st[4 * r + e] = k1p[r][e];
            }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = apply_sign(qf[ks], ss);
    if (use_asm) {
        if constexpr (kAsmLoop) {
            u32x32 qall;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 w4 = __builtin_bit_cast(u32x4, qf[ks]);
#pragma unroll
                for (int e = 0; e < 4; ++e) qall[4 * ks + e] = w4[e];
            }
            const u32x4 krw = rsrc_words(K + kv_base, head_bytes);
            const u32x4 vrw = rsrc_words(V + kv_base, head_bytes);
            const uint32_t kaddr = lds_addr(sK[0] + k_off), vaddr = lds_addr(sV[0] + v_off);
            const uint32_t kw = lds_addr(sK[0] + (tid / DCH) * KS + 8 * (tid % DCH));
            const uint32_t vw = lds_addr(sV[0] + (tid / DCH) * VS + 8 * (tid % DCH));
            const uint32_t ld0 = ld_off, ld1 = ld_off + ROWS_PER_PASS * D * 2;
            f32x32 olo, ohi;
            float m_out, mneg_out, l_out;
            int cnt = j_split - 1, soffk, soffv;
            asm volatile(FA_FWD128_ASM
                         : [olo] "=" FA_FWD128_C_OLO(olo), [ohi] "=" FA_FWD128_C_OHI(ohi),
                           [kst] "+" FA_FWD128_C_KST(kst), [vst] "+" FA_FWD128_C_VST(vst),
                           [k1st] "+" FA_FWD128_C_K1ST(k1st), [m] "=" FA_FWD128_C_M(m_out),
                           [mneg] "=" FA_FWD128_C_MNEG(mneg_out), [l] "=" FA_FWD128_C_L(l_out), [cnt] "+s"(cnt),
                           [soffk] "=&s"(soffk), [soffv] "=&s"(soffv)
                         : [qf] FA_FWD128_C_QF(qall), [kaddr] FA_FWD128_C_KADDR(kaddr),
                           [vaddr] FA_FWD128_C_VADDR(vaddr), [kw] FA_FWD128_C_KW(kw), [vw] FA_FWD128_C_VW(vw),
                           [ld0] FA_FWD128_C_LD0(ld0), [ld1] FA_FWD128_C_LD1(ld1), [c] "s"(scale_log2),
                           [krs] "s"(krw), [vrs] "s"(vrw)
                         : FA_FWD128_CLOBBERS);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                oacc[0][i] = olo[i];
                oacc[1][i] = olo[16 + i];
                oacc[2][i] = ohi[i];
                oacc[3][i] = ohi[16 + i];
            }
            m = m_out;
            mneg = mneg_out;
            l = l_out;
            // Only the thread index stays in a register across the statement
            // (which leaves the compiler a few VGPRs); everything derived from
            // it is derived again here.
            asm volatile("" : "+v"(tid));
            lane = tid & 63;
            lq = lane & 31;
            h = lane >> 5;
            qrow = qw0 + lq;
            ld_off = ((tid / DCH) * D + 8 * (tid % DCH)) * 2;
            k_off = lq * KS + 8 * h;
            v_off = tr_row(lane) * VS + tr_col(lane);
        }
    } else {
        // (A zero the compiler cannot see through: a constant accumulator
        // initialisation is otherwise hoisted out of the task loop and held,
        // or spilled, across it.)
        float zero = 0.f;
        asm volatile("" : "+v"(zero));
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] = zero;
        m = -INFINITY;
        mneg = 0.f;
        l = 0.f;
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            kreg[r] = k0p[r];
            vreg[r] = v0p[r];
        }
        store_tile(0);
        __syncthreads();
    }
    // One key tile.  MASKED tiles may cross a wave's diagonal or the ragged
    // end; the others carry no masking code at all, so no branch splits their
    // loop body and the compiler schedules the scores, the softmax and P V
    // as one block (with the masking branch merely present, never taken, the
    // d = 64 forward ran 21% slower).
    auto step = [&](int j, auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mask_tag)::value;
        const int buf = j & 1;
        load_tile(min(j + 1, ntiles - 1));  // in flight during this tile's math

        const int k0 = j * BC;
        // Skip tiles entirely above this wave's diagonal (a scalar branch).
        if (!CAUSAL || !MASKED || __builtin_amdgcn_readfirstlane(k0 <= qw0 + 31)) {
            const bf16* kt = sK[buf];
            const bf16* vt = sV[buf];
            // S^T = K Q^T for two 32-key halves, the two accumulation chains interleaved.
            f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    s[kb] = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(kt + 32 * kb * KS + k_off + 16 * ks),
                                               qf[ks], s[kb]);
            // Issue order: four K reads, then one read per MFMA, so that each
            // MFMA's operand was requested four MFMAs earlier.
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * NKS - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

            bf16x8 vpre[NPRE][NDB];
#pragma unroll
            for (int s2 = 0; s2 < NPRE; ++s2)
#pragma unroll
                for (int db = 0; db < NDB; ++db) vpre[s2][db] = lds_read_tr_a(vt + 16 * s2 * VS + v_off + 32 * db, VS);

            // Mask keys past N and, on tiles crossing the diagonal, keys after the query.
            if (MASKED && (k0 + BC > N || (CAUSAL && k0 + BC - 1 > qw0))) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = k0 + 32 * kb + c_row(i, h);
                        if (key >= N || (CAUSAL && key > qrow)) s[kb][i] = -INFINITY;
                    }
            }

            // Online softmax in the log2 domain with a lagging reference max.
            const float mx = pair_max(max32(s[0], s[1])) * scale_log2;
            if (__any(mx > m + kRescaleThreshold)) {  // wave-uniform branch
                const float m_new = fmaxf(m, mx);
                const float alpha = fast_exp2(m - m_new);  // 0 on the first visible tile
                l *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
                m = m_new;
                mneg = (m == -INFINITY) ? 0.f : -m;
            }
            float rs0 = 0.f, rs1 = 0.f;
            bf16x8 pf[BC / 16];
            u32x4 dw[2];
            if constexpr (DROPOUT) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) dw[kb] = dropout_words(dp, bh, qrow, k0 / 32 + kb, h);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(fmaf(s[kb][i], scale_log2, mneg));
                    // The two sums start from the first two values (p >= 0, so 0 + p = p).
                    if (kb == 0 && i < 2) (i ? rs1 : rs0) = p;
                    else (i & 1 ? rs1 : rs0) += p;
                    float pv = p;
                    if constexpr (DROPOUT) pv = dropout_keep(dw[kb], i, dp.thr) ? p : 0.f;
                    // k-step s2 = 2 kb + i/8 covers keys 16 s2 + 8 (j/4) + 4 h + j%4, j = i%8
                    pf[2 * kb + (i >> 3)][i & 7] = (bf16)pv;
                }
            l += rs0 + rs1;

            // O^T += V^T P^T, k-step by k-step.
#pragma unroll
            for (int s2 = 0; s2 < BC / 16; ++s2)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 vf = s2 < NPRE ? vpre[s2 < NPRE ? s2 : 0][db]
                                                : lds_read_tr_a(vt + 16 * s2 * VS + v_off + 32 * db, VS);
                    oacc[db] = mfma_bf16_32x32x16(vf, pf[s2], oacc[db]);
                }
        }

        store_tile(buf ^ 1);  // buffers last read in the previous tile
        __syncthreads();
    };
    // (With the assembly loop every unmasked tile has run above.)
    if constexpr (!kAsmLoop)
        for (int j = 0; j < j_split; ++j) step(j, std::false_type{});
    for (int j = j_split; j < ntiles; ++j) step(j, std::true_type{});

    // Epilogue: O = acc / l, L = (m + log2 l) ln 2.
    const float lt = pair_sum(l);
    if (qrow < N) {
        const float inv = (DROPOUT ? dp.keep_scale : 1.f) / lt;
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
    // The next task's opening loads go out right behind this task's stores,
    // without waiting for the stores to complete: the wait at the next task's
    // start then covers both at once.
    int nbh, nqb_;
    const bool more = task_of(round + 1, nbh, nqb_);
    if (!more) break;
    issue_task_loads(nbh, nqb_);
    bh = nbh;
    qb = nqb_;
    }  // task loop
}

// fp32 forward: the same loop with every product in fp32 on
// v_mfma_f32_32x32x2_f32 and P kept in fp32.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int BH, int nqb, ScoreScale ss) {
    const float scale_log2 = ss.c;
    constexpr int BC = kFwdBc;
    constexpr int KS = D + 2;  // odd-pair stride: 32 rows x 2 columns hit distinct banks
    constexpr int VS = D + 8;  // rows 4 apart land 32 banks apart
    constexpr int DCH = D / 4;  // 16-byte chunks per row
    constexpr int CH = BC * DCH / kFwdThreads;
    static_assert(CH * kFwdThreads == BC * DCH, "tile split");

    __shared__ __attribute__((aligned(16))) float sK[BC * KS];
    __shared__ __attribute__((aligned(16))) float sV[BC * VS];

    const int tid = thread_id(), lane = tid & 63, w = tid >> 6;
    const int lq = lane & 31, h = lane >> 5;
    int bh, qb;
    if (!wg_coords(block_id(), BH, nqb, CAUSAL, bh, qb)) return;
    const int q0 = qb * kFwdBr;
    const int qw0 = q0 + 32 * w;
    const int qrow = qw0 + lq;
    const int64_t base = (int64_t)bh * N * D;

    float qf[D / 2];  // Q[qrow][2 ks + h]
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
        qf[ks] = apply_sign(qrow < N ? Q[base + (int64_t)qrow * D + 2 * ks + h] : 0.f, ss);

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

int blocks_per_cu_of(const void* kernel, int threads) {
    constexpr int kSlots = 256;
    static std::mutex mu;
    static const void* keys[kSlots];
    static int vals[kSlots];
    static int used = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (keys[i] == kernel) return vals[i];
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0) n = 1;
    if (used < kSlots) {
        keys[used] = kernel;
        vals[used] = n;
        ++used;
    }
    return n;
}

int persistent_per_xcd(int tasks, int blocks_per_cu) {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cu_count[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    int cus = (dev >= 0 && dev < kMaxDev) ? cu_count[dev].load(std::memory_order_relaxed) : 0;
    if (cus <= 0) {
        if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        if (dev >= 0 && dev < kMaxDev) cu_count[dev].store(cus, std::memory_order_relaxed);
    }
    const int per_xcd_tasks = (tasks + kNumXcd - 1) / kNumXcd;
    return std::max(1, std::min(per_xcd_tasks, std::max(1, blocks_per_cu) * std::max(1, cus / kNumXcd)));
}


hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                           int Hkv, int N, int d, float scale, bool causal, const DropoutParams* dropout,
                           hipStream_t stream) {
    const int BH = B * Hq, G = Hq / Hkv;
    const int nqb = (N + kFwdBr - 1) / kFwdBr;
    const ScoreScale ss = make_score_scale(scale, 1.f, 0x80008000u);
    auto Q = static_cast<const bf16*>(q);
    auto K = static_cast<const bf16*>(k);
    auto V = static_cast<const bf16*>(v);
    auto Op = static_cast<bf16*>(o);
    const DropoutParams dp = dropout ? *dropout : DropoutParams{0u, 1.f, 0u, 0u, 0u};
#define FA_FWD_LAUNCH(DD, CC, DR)                                                                          \
    do {                                                                                                   \
        const int nx = persistent_per_xcd(nqb * BH, blocks_per_cu(fwd_bf16_kernel<DD, CC, DR>, kFwdThreads)); \
        hipLaunchKernelGGL((fwd_bf16_kernel<DD, CC, DR>), dim3(kNumXcd * nx), dim3(kFwdThreads), 0, stream, Q, \
                           K, V, Op, lse, N, BH, nqb, ss, Hq, G, dp, nx);                                 \
        return hipGetLastError();                                                                          \
    } while (0)
#define FA_FWD_DROP(DD, CC)             \
    do {                                \
        if (dropout) FA_FWD_LAUNCH(DD, CC, true); \
        FA_FWD_LAUNCH(DD, CC, false);   \
    } while (0)
    if (d == 64) {
        if (causal) FA_FWD_DROP(64, true);
        FA_FWD_DROP(64, false);
    }
    if (causal) FA_FWD_DROP(128, true);
    FA_FWD_DROP(128, false);
#undef FA_FWD_DROP
#undef FA_FWD_LAUNCH
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH,
                          int N, int d, float scale, bool causal, hipStream_t stream) {
    const int nqb = (N + kFwdBr - 1) / kFwdBr;
    const int grid = grid_for_tasks(nqb * BH);
    const ScoreScale ss = make_score_scale(scale, 1.f, 0x80000000u);
#define FA_FWD_LAUNCH(DD, CC)                                                                        \
    do {                                                                                             \
        hipLaunchKernelGGL((fwd_f32_kernel<DD, CC>), dim3(grid), dim3(kFwdThreads), 0, stream, q, k, v, \
                           o, lse, N, BH, nqb, ss);                                                 \
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
