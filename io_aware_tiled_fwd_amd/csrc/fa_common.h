// fa_common.h -- types and wavefront helpers shared by the gfx950 attention kernels.
//
// MFMA operand layouts used throughout (gfx950, wave64; checked on hardware):
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l%32][(l/32)*8 + j], j = 0..7   (8 bf16)
//     B: lane l holds B[(l/32)*8 + j][l%32], j = 0..7   (8 bf16)
//     C: lane l, register i holds C[8*(i/4) + 4*(l/32) + i%4][l%32], i = 0..15
//   v_mfma_f32_32x32x2_f32    C[32x32] += A[32x2] * B[2x32]
//     A: lane l holds A[l%32][l/32];  B: lane l holds B[l/32][l%32];  C as above.
//
// Every kernel computes the TRANSPOSED score tile S^T = K Q^T so that one lane
// column is one query row: a row's statistics live in one lane and its partner
// lane l^32, and the output accumulator O^T = V^T P^T takes P^T straight from
// the score registers (the transposing reads below deliver V^T in their k order).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_exp_f32 computes 2^x (exp2(-inf) = 0); v_log_f32 computes log2(x).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine a value with the one held by lane l^32 (v_permlane32_swap).  Both
// lanes of a pair see the operands in the same order, so both get bitwise
// identical results.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane 16g + r receives element r%4 of the 8-byte chunks addressed by
// lanes 16g + 4e + r/4, e = 0..3 (checked on hardware).  Two such reads give
// the 8-element A operand of v_mfma_f32_32x32x16_bf16 for A = M^T, M stored
// row-major in LDS: see tr_row / tr_col.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}
// For A[m][k] = M[k][m] over a 32(m) x 16(k) block: lane l points its first
// read at M[tr_row(l)][tr_col(l)] and its second at M[tr_row(l) + 8][tr_col(l)].
// Lane half h = l/32 then holds k = 4h + e (first read) and 8 + 4h + e (second
// read): the k-order of a C tile's rows c_row(), so a score tile's registers
// can be the matching B operand without any shuffle.
__device__ __forceinline__ constexpr int tr_row(int lane) { return 4 * (lane >> 5) + ((lane & 15) >> 2); }
__device__ __forceinline__ constexpr int tr_col(int lane) { return 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }
__device__ __forceinline__ bf16x8 lds_read_tr_a(const bf16* p, int row_stride) {
    const bf16x4 lo = lds_read_tr(p), hi = lds_read_tr(p + 8 * row_stride);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// An LDS read that stays where it is written: a volatile access is neither
// sunk towards its use nor merged with others, so the data is in flight while
// the code in between runs.
__device__ __forceinline__ bf16x8 lds_read16_early(const bf16* p) {
    return *(const volatile __attribute__((address_space(3))) bf16x8*)(p);
}

// Workgroup ids are dealt round-robin to the 8 XCDs (each with its own L2).
// xcd_task() turns the flat id into a task index such that every XCD receives
// a contiguous range of tasks; launch grid_for_tasks(total) workgroups and let
// those with task >= total exit.  With tasks ordered head-major, the query
// blocks of one head run together on one XCD and share its K/V in that L2.
constexpr int kNumXcd = 8;
__host__ __device__ __forceinline__ constexpr int grid_for_tasks(int total) {
    return kNumXcd * ((total + kNumXcd - 1) / kNumXcd);
}
__device__ __forceinline__ int xcd_task(int id, int total) {
    const int per = (total + kNumXcd - 1) / kNumXcd;
    return (id % kNumXcd) * per + id / kNumXcd;
}
// Tasks per XCD under xcd_task and head_rank: an XCD's k-th workgroup has a
// task of its own only for k below this (beyond it xcd_task continues into
// the next XCD's range, which that XCD's workgroups cover).
__device__ __forceinline__ int xcd_tasks(int total) { return (total + kNumXcd - 1) / kNumXcd; }

// Map a flat workgroup id to (head, rank) for a grid of grid_for_tasks(nheads
// * nranks) workgroups, rank 0 being a head's heaviest block.  When nheads is
// a multiple of the XCD count, XCD x = id % 8 owns the contiguous heads
// [x hp, (x + 1) hp), hp = nheads / 8, so that a head's K/V (and grouped
// heads' shared K/V) stay in one L2.  The XCD's k-th workgroup (k = id / 8)
// takes its heads in groups of g, g the largest divisor of hp with g nranks <=
// 32 (the XCD's CUs), and walks a group rank-major: the heaviest blocks of its
// g heads, then the next rank.  A group is about one round of the XCD's CUs,
// so only g heads stream through the L2 at a time, and short causal grids no
// longer end on one head's heaviest blocks (head-major order left B4 H16
// N4096 17% above the ideal makespan).  Otherwise the XCDs receive contiguous
// task ranges (xcd_task), head-major, heaviest rank first within a head.
// Returns false for padding workgroups.
constexpr int kCusPerXcd = 32;
__device__ __forceinline__ bool head_rank(int id, int nheads, int nranks, int& head, int& rank) {
    if (nheads % kNumXcd == 0) {
        const int hp = nheads / kNumXcd, k = id / kNumXcd;
        if (k >= hp * nranks) return false;
        int g = max(1, min(hp, kCusPerXcd / nranks));
        while (hp % g) --g;
        const int gi = k / (g * nranks), r = k % (g * nranks);
        rank = r / g;
        head = (id % kNumXcd) * hp + gi * g + r % g;
        return true;
    }
    const int task = xcd_task(id, nheads * nranks);
    if (task >= nheads * nranks) return false;
    head = task / nranks;
    rank = task % nranks;
    return true;
}

// (head, query block) of a forward or dQ workgroup: under a causal mask the
// last query block is the heaviest.
__device__ __forceinline__ bool wg_coords(int id, int BH, int nqb, bool causal, int& bh, int& qb) {
    int qi;
    if (!head_rank(id, BH, nqb, bh, qi)) return false;
    qb = causal ? (nqb - 1 - qi) : qi;
    return true;
}

// Score scaling.  The method's scores are S = scale Q K^T for any finite
// scale ("FlashAttention" deep-dive page, "How it works").  The kernels need
// a positive factor c in P = 2^(s c - m): their row maxima are taken over the
// unscaled products s, masked scores are -inf before the factor is applied,
// and c = 0 would turn those into NaN.  The sign of the scale is therefore
// moved into the operand that each kernel keeps in registers (Q, or K in the
// dK/dV kernels): negating every element of one operand negates every product
// exactly, so |scale| (-s) is bitwise scale * s.  A zero scale zeroes that
// operand instead: every score is then exactly 0 = 0 * s, and c may be any
// positive number.  The gradients' own factor (dQ = scale dS K, dK = scale
// dS^T Q) keeps the signed scale.
struct ScoreScale {
    float c;        // positive factor of the log2-domain exponent: |scale| log2(e) (or log2(e) for scale 0)
    uint32_t keep;  // AND mask applied to the register-resident operand's words (0: zero it)
    uint32_t flip;  // then XOR mask: the sign bits of its elements when scale < 0, else 0
};
// sign_bits: the sign bits of one 32-bit word of the operand's element type
// (0x80008000 for bf16 pairs, 0x80000000 for fp32, 0x80808080 for fp8 bytes);
// extra: further positive factors of the exponent (fp8 dequantisation).
inline ScoreScale make_score_scale(float scale, float extra, uint32_t sign_bits) {
    const float c = __builtin_fabsf(scale) * extra * kLog2e;
    if (scale == 0.f || c == 0.f) return ScoreScale{kLog2e, 0u, 0u};  // all scores exactly 0
    return ScoreScale{c, 0xFFFFFFFFu, scale < 0.f ? sign_bits : 0u};
}
__device__ __forceinline__ uint32_t apply_sign(uint32_t w, const ScoreScale& ss) { return (w & ss.keep) ^ ss.flip; }
__device__ __forceinline__ bf16x8 apply_sign(bf16x8 x, const ScoreScale& ss) {
    u32x4 u = __builtin_bit_cast(u32x4, x);
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = apply_sign(u[e], ss);
    return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ float apply_sign(float x, const ScoreScale& ss) {
    return __uint_as_float(apply_sign(__float_as_uint(x), ss));
}

// Threshold (log2 units) by which a row's maximum must grow before the
// accumulator is rescaled.  Any reference value m gives the same exact result
// (O = acc / l and L = m + log2 l both carry it), so m may lag the true maximum:
// P = 2^(S c - m) then stays below 2^8, comfortably inside fp32 and bf16 range,
// and most key tiles skip the alpha rescale of the accumulator.
constexpr float kRescaleThreshold = 8.0f;

// Key/value head (flat over batches) read by flat query head bh, with Hq
// query heads per batch and G query heads per key/value head.
__device__ __forceinline__ int kv_head(int bh, int Hq, int G) { return (bh / Hq) * (Hq / G) + (bh % Hq) / G; }

// Attention dropout ("FlashAttention" deep-dive page, "Implementation notes":
// the backward regenerates the mask from a Philox seed and offset).  Element
// (bh, i, j) -- flat query head, query row, key -- takes byte 8 (j % 4) of word
// (j / 8) % 4 of Philox4x32-10(counter = (2 (j / 32) + (j / 4) % 2, i, bh,
// offset), key = seed) and is kept when that byte is >= thr; kept
// probabilities are multiplied by keep_scale = 256 / (256 - thr).  One Philox
// call thus covers the 16 keys 32 jb + 8 a + 4 hh + e (a, e < 4) of one row:
// exactly the keys that lane half hh holds in a 32-key C tile (c_row), with
// register r = 4 a + e taking byte e of word a.
struct DropoutParams {
    uint32_t thr;       // bytes below thr are dropped
    float keep_scale;   // 256 / (256 - thr)
    uint32_t seed_lo, seed_hi, offset;
};

// Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw ("Parallel
// Random Numbers: As Easy as 1, 2, 3", SC 2011): ten rounds of
// (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)),
// the key advanced by the Weyl constants before every round but the first.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // Full 64-bit products (one v_mad_u64_u32 each) give both halves.
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    return u32x4{c0, c1, c2, c3};
}

// The 16 dropout bytes of query row i, key block jb (32 keys), lane half hh.
__device__ __forceinline__ u32x4 dropout_words(const DropoutParams& dp, int bh, int i, int jb, int hh) {
    return philox4x32_10((uint32_t)(2 * jb + hh), (uint32_t)i, (uint32_t)bh, dp.offset, dp.seed_lo, dp.seed_hi);
}
// Whether register r's element (byte r % 4 of word r / 4) is kept.
__device__ __forceinline__ bool dropout_keep(const u32x4& w, int r, uint32_t thr) {
    return ((w[r >> 2] >> (8 * (r & 3))) & 0xFFu) >= thr;
}

// Buffer resource over [base, base + bytes): raw buffer loads whose byte offset
// (VGPR offset + SGPR offset) falls outside return zero (range checking of
// untyped buffer loads; the SGPR offset takes part, checked on hardware).  A
// ragged last tile therefore needs no branches: rows past N read as 0.
// The base and size are made wave-uniform explicitly so that the descriptor
// lives in SGPRs (a descriptor in VGPRs forces a loop around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// soff is made wave-uniform explicitly: an offset the compiler keeps in a VGPR
// would otherwise put a readfirstlane loop around the load.
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, __builtin_amdgcn_readfirstlane(soff), 0);
}
// The same load with the non-temporal hint (cache policy nt), for data read
// exactly once: a streaming read of 1 GiB measured 6.9-7.3 TB/s with it and
// 5.6-6.5 TB/s without it on gfx950.
__device__ __forceinline__ u32x4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, __builtin_amdgcn_readfirstlane(soff), 2);
}

// Round eight floats to bf16 (RNE) as four v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                              float a6, float a7) {
    const bf16x2 p0 = __builtin_convertvector(f32x2{a0, a1}, bf16x2);
    const bf16x2 p1 = __builtin_convertvector(f32x2{a2, a3}, bf16x2);
    const bf16x2 p2 = __builtin_convertvector(f32x2{a4, a5}, bf16x2);
    const bf16x2 p3 = __builtin_convertvector(f32x2{a6, a7}, bf16x2);
    return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                            __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)});
}

// Work-item and workgroup ids read straight from the hardware registers.  The
// threadIdx / blockIdx accessors go through device-library functions built with
// other target features than these kernels (packed fp32 is disabled here), so
// the compiler calls them instead of inlining them; so would __umulhi.
__device__ __forceinline__ int thread_id() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int block_id() { return (int)__builtin_amdgcn_workgroup_id_x(); }

// Waits until every global and buffer load this wavefront has issued has
// returned (s_waitcnt vmcnt(0)).  Called once after the loads of the
// register-resident operands, before the tile loop: without it the compiler's
// wait insertion, which does not know that those loads completed long before,
// guards their uses inside the loop with counts that include the loop's own
// prefetch loads, so a wavefront could stall on a prefetch it does not need yet.
__device__ __forceinline__ void wait_vmem_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Index of the calling wavefront in its workgroup, as a scalar (wave-uniform)
// value so that branches on it are scalar branches.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(thread_id() >> 6); }

// Maximum of the 32 score registers of two 32x32 C tiles (v_max3_f32 chains).
__device__ __forceinline__ float max32(const f32x16& a, const f32x16& b) {
    float x = fmaxf(a[0], a[1]), y = fmaxf(b[0], b[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
        x = fmaxf(fmaxf(x, a[i]), a[i + 1]);
        y = fmaxf(fmaxf(y, b[i]), b[i + 1]);
    }
    return fmaxf(x, y);
}

// Row (key or query) held by register i of lane half h in a 32x32 C tile.
__device__ __forceinline__ constexpr int c_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

}  // namespace fa
