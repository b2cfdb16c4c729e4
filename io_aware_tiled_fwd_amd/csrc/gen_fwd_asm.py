#!/usr/bin/env python3
"""Writes fa_fwd_asm.inc: the hand-scheduled key loop of the bf16 forward at d = 128.

Usage: python gen_fwd_asm.py [output]   (default: fa_fwd_asm.inc beside this file)

What the loop computes is the forward of the "FlashAttention" deep-dive page
(tirogla.com), section "How it works", for the key tiles that no mask touches;
fa_fwd.hip runs it and takes over for the masked tiles.  This script only fixes
the instruction order.  Per 64-key tile a wavefront (32 query rows) issues

    16 MFMAs  S^T(t+1) = K(t+1) Q^T      (two 32-key chains of 8 k-steps)
    16 MFMAs  O^T     += V(t)^T P(t)^T    (4 k-steps x 4 dimension blocks)
    ~130 VALU the softmax of tile t (scale, exp2, row sums, bf16 packing)
              and the row maximum of tile t+1

interleaved about four VALU instructions per MFMA, so that the matrix core and
the vector unit of a SIMD work at the same time.  A compiler-scheduled loop runs
the three parts one after another (scores, softmax, P V), and the two
wavefronts of a SIMD, which reach each tile barrier together, leave the matrix
core idle during the softmax.

K tiles are staged one tile ahead of V tiles: iteration t reads K(t+1) and V(t)
from LDS and stores K(t+2) and V(t+1), all in two LDS buffers per tensor, with
one barrier per tile.

The script also inserts every s_waitcnt and s_nop the code needs (the
compiler's hazard recognizer does not look inside inline assembly):
  * LDS and buffer-load results: lgkmcnt / vmcnt counts, in issue order;
  * an MFMA result read or overwritten by any other instruction: 12 wait
    states (v_mfma_f32_32x32x16_bf16 is an 8-pass instruction on gfx950);
  * a VALU result read by an MFMA or by v_permlane32_swap: 2 wait states;
  * a transcendental result read by a VALU instruction: 1 wait state;
  * a VALU write of a register that an MFMA read as its accumulator: 12.
These are the counts the compiler itself emits for the same instruction
pairs on gfx950.
"""
import os
import sys

BC = 64               # keys per tile


def configure(d):
    """Sets the module's layout and register map for head dimension d (64 or
    128); every function below reads them."""
    g = globals()
    g["D"] = d
    g["NKS"] = d // 16               # k-steps of the score chains
    g["NDB"] = d // 32               # 32-dimension blocks of O
    g["CH"] = BC * d // 8 // 512     # staged 16-byte chunks per thread and tensor
    g["KS"] = d + 8                  # K row stride in LDS (elements)
    g["VS"] = d + 32                 # V row stride in LDS (elements)
    g["KBUF"] = BC * g["KS"] * 2     # bytes of one K buffer
    g["VBUF"] = BC * g["VS"] * 2     # bytes of one V buffer
    g["K_KB"] = 32 * g["KS"] * 2     # the second 32-key half of a K tile
    g["V_S2"] = 16 * g["VS"] * 2     # a 16-key k-step of V
    g["V_HALF"] = 8 * g["VS"] * 2    # the second transposing read of a fragment
    g["K_CH"] = 32 * g["KS"] * 2     # the second staging chunk (32 rows on)
    g["V_CH"] = 32 * g["VS"] * 2
    g["TILE_BYTES"] = BC * d * 2
    # VGPR map (fa_fwd.hip binds the operands to these registers):
    #   O    O^T accumulators, block db in v[O + 16 db : +15]
    #   S    two score buffers of 32, key half kb in v[S + 16 kb : +15]
    #   QF   Q^T operand, k-step ks in v[QF + 4 ks : +3]
    #   KR, VR   K and V^T fragment rings (slots of 4)
    #   KST, VST staged K and V rows (CH chunks of 4)
    g["O"] = 0
    g["S"] = (d // 2, d // 2 + 32)
    g["QF"] = d // 2 + 64
    g["KR"] = g["QF"] + 4 * g["NKS"]
    g["VR"] = g["KR"] + 4 * NKR
    g["KST"] = g["VR"] + 4 * NVR
    g["VST"] = g["KST"] + 4 * g["CH"]
    base = g["VST"] + 4 * g["CH"]
    (g["M"], g["MNEG"], g["L"], g["RS0"], g["RS1"], g["T0"], g["T1"], g["T2"]) = range(base, base + 8)
    (g["KADDR"], g["VADDR"], g["KW"], g["VW"], g["LD0"], g["LD1"]) = range(base + 8, base + 14)
    g["K1ST"] = g["S"][1]            # K(1) staged in the prologue (score buffer 1 is free then)
    g["NVGPR"] = g["LD1"] + 1


NKR = 5               # K fragment ring slots
NVR = 5               # V^T fragment ring slots

MFMA_VALU_WS = 12     # MFMA result -> other instruction
VALU_MFMA_WS = 2      # VALU result -> MFMA operand
VALU_PERM_WS = 2      # VALU result -> v_permlane32_swap
TRANS_VALU_WS = 1     # v_exp_f32 result -> VALU
SRCC_WAR_WS = 12      # MFMA accumulator read -> VALU write


def vr(a, n=1):
    return f"v{a}" if n == 1 else f"v[{a}:{a + n - 1}]"


class Ins:
    """One instruction with the registers it reads and writes."""

    def __init__(self, text, kind, rd=(), wr=(), src_c=(), lds=False, vmem=False):
        self.text, self.kind = text, kind
        self.rd, self.wr, self.src_c = set(rd), set(wr), set(src_c)
        self.lds, self.vmem = lds, vmem


def rng(a, n):
    return range(a, a + n)


def mfma(dst, a, b, c):
    """v_mfma_f32_32x32x16_bf16 dst = a b + c (c None: zero)."""
    ctext = vr(c, 16) if c is not None else "0"
    rd = list(rng(a, 4)) + list(rng(b, 4)) + (list(rng(c, 16)) if c is not None else [])
    return Ins(f"v_mfma_f32_32x32x16_bf16 {vr(dst, 16)}, {vr(a, 4)}, {vr(b, 4)}, {ctext}", "mfma", rd,
               rng(dst, 16), src_c=rng(c, 16) if c is not None else ())


def valu(text, rd, wr, kind="valu"):
    return Ins(text, kind, rd, wr)


def ds_read_k(dst, off):
    return Ins(f"ds_read_b128 {vr(dst, 4)}, {vr(KADDR)} offset:{off}", "ds_read", [KADDR], rng(dst, 4), lds=True)


def ds_read_tr(dst, off):
    return Ins(f"ds_read_b64_tr_b16 {vr(dst, 2)}, {vr(VADDR)} offset:{off}", "ds_read", [VADDR], rng(dst, 2),
               lds=True)


def ds_write(addr, src, off):
    return Ins(f"ds_write_b128 {vr(addr)}, {vr(src, 4)} offset:{off}", "ds_write", [addr] + list(rng(src, 4)), (),
               lds=True)


def buf_load(dst, voff, rsrc, soff):
    return Ins(f"buffer_load_dwordx4 {vr(dst, 4)}, {vr(voff)}, %[{rsrc}], %[{soff}] offen", "vmem_load", [voff],
               rng(dst, 4), vmem=True)


def salu(text):
    return Ins(text, "salu")


def raw(text, kind="ctl"):
    return Ins(text, kind)


# ---------------------------------------------------------------- pieces

def k_read_off(kbuf, kb, ks):
    return kbuf * KBUF + kb * K_KB + 32 * ks


def v_read_off(vbuf, s2, db, half):
    return vbuf * VBUF + s2 * V_S2 + 64 * db + half * V_HALF


def softmax_part(sb, s2):
    """P for k-step s2 of the score buffer at sb, in place: x -> 2^(x c - m),
    added into the two partial row sums (even and odd registers, in the order
    of fa_fwd.hip's compiler-scheduled tiles), then packed to bf16 pairs in the
    first four registers of the k-step: those four are the B operand of the
    k-step's P V MFMAs."""
    base = sb + 16 * (s2 >> 1) + 8 * (s2 & 1)
    r = [base + i for i in range(8)]
    out = []
    for x in r:
        out.append(valu(f"v_fma_f32 {vr(x)}, %[c], {vr(x)}, {vr(MNEG)}", [x, MNEG], [x]))
    for x in r:
        out.append(valu(f"v_exp_f32 {vr(x)}, {vr(x)}", [x], [x], kind="trans"))
    def sums(q):
        a, b = r[2 * q], r[2 * q + 1]
        if s2 == 0 and q == 1:  # the sums start from the first two pairs
            return [valu(f"v_add_f32 {vr(RS0)}, {vr(r[0])}, {vr(a)}", [r[0], a], [RS0]),
                    valu(f"v_add_f32 {vr(RS1)}, {vr(r[1])}, {vr(b)}", [r[1], b], [RS1])]
        return [valu(f"v_add_f32 {vr(RS0)}, {vr(RS0)}, {vr(a)}", [RS0, a], [RS0]),
                valu(f"v_add_f32 {vr(RS1)}, {vr(RS1)}, {vr(b)}", [RS1, b], [RS1])]

    def pack(q):
        a, b = r[2 * q], r[2 * q + 1]
        return [valu(f"v_cvt_pk_bf16_f32 {vr(r[q])}, {vr(a)}, {vr(b)}", [a, b], [r[q]])]

    if s2 == 0:
        out += sums(1) + pack(0) + pack(1) + sums(2) + pack(2) + sums(3) + pack(3)
    else:
        for q in range(4):
            out += sums(q) + pack(q)
    return out


def row_sum_close():
    return [valu(f"v_add_f32 {vr(T0)}, {vr(RS0)}, {vr(RS1)}", [RS0, RS1], [T0]),
            valu(f"v_add_f32 {vr(L)}, {vr(L)}, {vr(T0)}", [L, T0], [L])]


def row_max(sb):
    """The maximum of the 32 registers of score buffer sb into T1 (v_max3 chains)."""
    out = []
    for kb, dst in ((0, T1), (1, T2)):
        b = sb + 16 * kb
        out.append(valu(f"v_max_f32 {vr(dst)}, {vr(b)}, {vr(b + 1)}", [b, b + 1], [dst]))
        for i in range(2, 16, 2):
            out.append(valu(f"v_max3_f32 {vr(dst)}, {vr(dst)}, {vr(b + i)}, {vr(b + i + 1)}", [dst, b + i, b + i + 1],
                            [dst]))
    out.append(valu(f"v_max_f32 {vr(T1)}, {vr(T1)}, {vr(T2)}", [T1, T2], [T1]))
    return out


def row_max_close():
    """Pair lanes l and l^32 (same query row), scale: T1 = max * c (the
    log2-domain maximum of the row over the tile)."""
    return [valu(f"v_mov_b32 {vr(T2)}, {vr(T1)}", [T1], [T2]),
            Ins(f"v_permlane32_swap_b32 {vr(T1)}, {vr(T2)}", "perm", [T1, T2], [T1, T2]),
            valu(f"v_max_f32 {vr(T1)}, {vr(T1)}, {vr(T2)}", [T1, T2], [T1]),
            valu(f"v_mul_f32 {vr(T1)}, %[c], {vr(T1)}", [T1], [T1])]


def rescale_test():
    """vcc = lanes whose maximum grew past m + 8 (the lagging reference)."""
    return [valu(f"v_add_f32 {vr(T2)}, 0x41000000, {vr(M)}", [M], [T2]),
            Ins(f"v_cmp_gt_f32 vcc, {vr(T1)}, {vr(T2)}", "valu", [T1, T2], [])]


def rescale_block():
    """m_new = max(m, T1); alpha = 2^(m - m_new); l and O scaled by alpha."""
    out = [raw("s_nop 7", "nop"), raw("s_nop 7", "nop")]  # the last P V MFMAs have written O
    out.append(valu(f"v_max_f32 {vr(T1)}, {vr(M)}, {vr(T1)}", [M, T1], [T1]))
    out.append(valu(f"v_sub_f32 {vr(T2)}, {vr(M)}, {vr(T1)}", [M, T1], [T2]))
    out.append(valu(f"v_exp_f32 {vr(T2)}, {vr(T2)}", [T2], [T2], kind="trans"))
    out.append(valu(f"v_mov_b32 {vr(M)}, {vr(T1)}", [T1], [M]))
    out.append(valu(f"v_xor_b32 {vr(MNEG)}, 0x80000000, {vr(T1)}", [T1], [MNEG]))
    out.append(valu(f"v_mul_f32 {vr(L)}, {vr(L)}, {vr(T2)}", [L, T2], [L]))
    for x in range(O, O + 16 * NDB):
        out.append(valu(f"v_mul_f32 {vr(x)}, {vr(T2)}, {vr(x)}", [T2, x], [x]))
    return out




# ---------------------------------------------------------------- schedules

def spread(items, slots, first, last):
    """Append items to slots[first..last] (inclusive), as evenly as possible,
    keeping their order."""
    n = last - first + 1
    for i, x in enumerate(items):
        slots[first + (i * n) // len(items)].append(x)


def mfma_stream(p, pattern, with_scores, kbuf, vbuf):
    """MFMAs of one tile in the order of pattern ('S': next score k-step,
    'P': next P V k-step / dimension block), each with the LDS reads of its
    operand issued as soon as the ring slot is free.  Returns (pre, slots):
    pre holds the reads issued before the first MFMA, slots[i] = [mfma i,
    reads issued right after it]."""
    sb, sn = S[p], S[p ^ 1]
    s_list = [(kb, ks) for ks in range(D // 16) for kb in range(2)] if with_scores else []
    pv = [(s2, db) for s2 in range(4) for db in range(NDB)]
    # operand reads, in the order their MFMAs come
    k_reads = []  # (reg, [Ins]) per score MFMA
    for f, (kb, ks) in enumerate(s_list):
        reg = KR + 4 * (f % NKR)
        k_reads.append((reg, [ds_read_k(reg, k_read_off(kbuf, kb, ks))]))
    v_reads = []
    for f, (s2, db) in enumerate(pv):
        reg = VR + 4 * (f % NVR)
        v_reads.append((reg, [ds_read_tr(reg, v_read_off(vbuf, s2, db, 0)),
                              ds_read_tr(reg + 2, v_read_off(vbuf, s2, db, 1))]))
    pre = []
    for f in range(min(NKR, len(k_reads))):
        pre += k_reads[f][1]
    # The first NVR V^T fragments have free ring slots from the start: with
    # score MFMAs in front, one is requested after each of those (the K reads
    # go first); otherwise all up front.
    early_v = {}
    n_first_s = len(pattern) - len(pattern.lstrip("S"))
    for f in range(min(NVR, len(v_reads))):
        if f < n_first_s:
            early_v.setdefault(f, []).extend(v_reads[f][1])
        else:
            pre += v_reads[f][1]
    slots = []
    si = pi = 0
    for ch in pattern:
        if ch == "S":
            kb, ks = s_list[si]
            dst = sn + 16 * kb
            ins = [mfma(dst, k_reads[si][0], QF + 4 * ks, dst if ks else None)]
            if si + NKR < len(k_reads):
                ins += k_reads[si + NKR][1]
            ins += early_v.get(si, [])
            si += 1
        else:
            s2, db = pv[pi]
            pf = sb + 16 * (s2 >> 1) + 8 * (s2 & 1)
            ins = [mfma(O + 16 * db, v_reads[pi][0], pf, O + 16 * db)]
            if pi + NVR < len(v_reads):
                ins += v_reads[pi + NVR][1]
            pi += 1
        slots.append(ins)
    assert si == len(s_list) and pi == len(pv)
    return pre, slots


# Per head dimension: the MFMA order of a steady-state tile ('S': the next
# score k-step of S(t+1), 'P': the next P V k-step and dimension block), the
# MFMA slots over which the four softmax parts and the row maximum are spread
# (first, last slot), and the slots after which the staged rows are stored.
# At d = 128 a tile has 32 MFMAs and ~4 VALU instructions per MFMA.  (A d = 64
# schedule -- 16 MFMAs for the same softmax, so the VALU work sets the pace --
# ran no faster than the compiler's schedule of the same step and is not
# emitted.)
SCHEDULE = {
    128: dict(pattern="S" * 7 + "P" * 4 + "S" * 3 + "P" * 4 + "S" * 6 + "P" * 8,
              parts=((0, 5), (6, 12), (13, 19), (20, 26)), rowmax=(27, 31), stores=(8, 14, 20, 26)),
}


def staged_stores(p):
    """The stores of one tile's staged rows (K(t+2) into K buffer p, V(t+1)
    into V buffer p^1), each followed by the load of the same rows one tile
    on, chunk by chunk: [K chunks..., V chunks...]."""
    groups = []
    for r in range(CH):
        g = [ds_write(KW, KST + 4 * r, p * KBUF + r * K_CH), buf_load(KST + 4 * r, LD0 + r, "krs", "soffk")]
        if r == CH - 1:
            g.append(salu(f"s_add_u32 %[soffk], %[soffk], {TILE_BYTES:#x}"))
        groups.append(g)
    for r in range(CH):
        g = [ds_write(VW, VST + 4 * r, (p ^ 1) * VBUF + r * V_CH), buf_load(VST + 4 * r, LD0 + r, "vrs", "soffv")]
        if r == CH - 1:
            g.append(salu(f"s_add_u32 %[soffv], %[soffv], {TILE_BYTES:#x}"))
        groups.append(g)
    return groups


def tile_iteration(p):
    """Steady-state tile t with S(t) in score buffer p: S(t+1), the softmax
    of S(t), O += V(t)^T P(t)^T, the maximum of S(t+1), the LDS stores of
    K(t+2) and V(t+1) (loaded during the previous tile) with the loads of
    K(t+3) and V(t+2), and the barrier.  K(t+1) is in K buffer p^1, V(t) in
    V buffer p; K(t+2) goes to K buffer p, V(t+1) to V buffer p^1."""
    sb, sn = S[p], S[p ^ 1]
    sch = SCHEDULE[D]
    out = []
    pre, slots = mfma_stream(p, sch["pattern"], True, p ^ 1, p)
    parts = [softmax_part(sb, s2) for s2 in range(4)]
    out += pre
    # the first part starts before the first MFMA (its K operand is in flight)
    out += parts[0][:8]
    parts[0] = parts[0][8:]
    parts[3] = parts[3] + row_sum_close()
    for part, (first, last) in zip(parts, sch["parts"]):
        spread(part, slots, first, last)
    spread(row_max(sn), slots, *sch["rowmax"])
    # LDS stores of the staged rows, spread over the tile: K(t+2) overwrites
    # K(t), read in the previous tile; V(t+1) overwrites V(t-1).  Each store
    # frees its registers for the global load of the same rows one tile on,
    # which then has a whole tile to arrive.
    for g, slot in zip(staged_stores(p), sch["stores"]):
        slots[slot] += g
    for s in slots:
        out += s
    out += row_max_close() + rescale_test()
    out += [raw("s_waitcnt lgkmcnt(0)", "wait"), raw("s_barrier", "barrier")]
    return out


def tile_last(p):
    """The last unmasked tile t, S(t) in score buffer p: softmax and P V only.
    Also stages V(t+1) into V buffer p^1 (K(t+1) is already in K buffer p^1)
    for the masked tiles that follow, and ends on a barrier."""
    sb = S[p]
    out = []
    pre, slots = mfma_stream(p, "P" * (4 * NDB), False, None, p)
    parts = [softmax_part(sb, s2) for s2 in range(4)]
    out += pre + parts[0]
    for s2 in range(1, 4):  # part s2 beside the P V MFMAs of k-step s2 - 1
        extra = row_sum_close() if s2 == 3 else []
        spread(parts[s2] + extra, slots, NDB * (s2 - 1), NDB * s2 - 1)
    for s in slots:
        out += s
    out += [ds_write(VW, VST + 4 * r, (p ^ 1) * VBUF + r * V_CH) for r in range(CH)]
    # (K(t+2) was loaded too, for nothing: the masked tiles stage their own.)
    out += [raw("s_waitcnt vmcnt(0) lgkmcnt(0)", "wait"), raw("s_barrier", "barrier")]
    return out


def prologue():
    """K(0), V(0) and K(1), already loaded into registers, go to LDS; then
    S(0) into score buffer 0, its maximum as the first reference m, O = 0."""
    out = [ds_write(KW, KST + 4 * r, r * K_CH) for r in range(CH)]
    out += [ds_write(VW, VST + 4 * r, r * V_CH) for r in range(CH)]
    out += [ds_write(KW, K1ST + 4 * r, KBUF + r * K_CH) for r in range(CH)]
    out += [salu(f"s_mov_b32 %[soffk], {2 * TILE_BYTES:#x}"), salu(f"s_mov_b32 %[soffv], {TILE_BYTES:#x}")]
    out += [buf_load(KST + 4 * r, LD0 + r, "krs", "soffk") for r in range(CH)]
    out += [buf_load(VST + 4 * r, LD0 + r, "vrs", "soffv") for r in range(CH)]
    out += [raw("s_waitcnt lgkmcnt(0)", "wait"), raw("s_barrier", "barrier")]
    # S(0): the score chains alone (buffer 1 of the scores is idle: use the
    # generic stream with a P V-free pattern)
    s_list = [(kb, ks) for ks in range(NKS) for kb in range(2)]
    reads = []
    for f, (kb, ks) in enumerate(s_list):
        reg = KR + 4 * (f % NKR)
        reads.append((reg, ds_read_k(reg, k_read_off(0, kb, ks))))
    for f in range(NKR):
        out.append(reads[f][1])
    slots = []
    for f, (kb, ks) in enumerate(s_list):
        dst = S[0] + 16 * kb
        s = [mfma(dst, reads[f][0], QF + 4 * ks, dst if ks else None)]
        if f + NKR < len(reads):
            s.append(reads[f + NKR][1])
        slots.append(s)
    zero = [valu(f"v_mov_b32 {vr(x)}, 0", [], [x]) for x in range(O, O + 16 * NDB)]
    zero += [valu(f"v_mov_b32 {vr(L)}, 0", [], [L])]
    spread(zero, slots, 0, len(slots) - 1)
    for s in slots:
        out += s
    out += row_max(S[0]) + row_max_close()
    out += [valu(f"v_mov_b32 {vr(M)}, {vr(T1)}", [T1], [M]),
            valu(f"v_xor_b32 {vr(MNEG)}, 0x80000000, {vr(T1)}", [T1], [MNEG]),
            salu(f"s_mov_b32 %[soffk], {3 * TILE_BYTES:#x}"), salu(f"s_mov_b32 %[soffv], {2 * TILE_BYTES:#x}")]
    # The first tile stores K(2) over K(0): every wavefront must have read
    # K(0) by then.
    out += [raw("s_barrier", "barrier")]
    return out


def program():
    """The whole asm statement: prologue, the loop over unmasked tiles (two
    tiles per trip: the score buffers alternate), the last tile, and the
    out-of-line rescale blocks.  %[cnt] = number of unmasked tiles - 1."""
    out = prologue()
    out += [raw(".Lfa_loop_%=:", "label"),
            salu("s_cmp_eq_u32 %[cnt], 0"), raw("s_cbranch_scc1 .Lfa_last0_%=", "branch")]
    out += tile_iteration(0)
    out += [raw("s_cbranch_vccnz .Lfa_rescale0_%=", "branch"), raw(".Lfa_back0_%=:", "label"),
            salu("s_sub_u32 %[cnt], %[cnt], 1"),
            salu("s_cmp_eq_u32 %[cnt], 0"), raw("s_cbranch_scc1 .Lfa_last1_%=", "branch")]
    out += tile_iteration(1)
    out += [raw("s_cbranch_vccnz .Lfa_rescale1_%=", "branch"), raw(".Lfa_back1_%=:", "label"),
            salu("s_sub_u32 %[cnt], %[cnt], 1"), raw("s_branch .Lfa_loop_%=", "branch")]
    out += [raw(".Lfa_last0_%=:", "label")] + tile_last(0) + [raw("s_branch .Lfa_end_%=", "branch")]
    out += [raw(".Lfa_last1_%=:", "label")] + tile_last(1) + [raw("s_branch .Lfa_end_%=", "branch")]
    out += [raw(".Lfa_rescale0_%=:", "label")] + rescale_block() + [raw("s_branch .Lfa_back0_%=", "branch")]
    out += [raw(".Lfa_rescale1_%=:", "label")] + rescale_block() + [raw("s_branch .Lfa_back1_%=", "branch")]
    # The code after the statement may read O at once: let the last P V
    # MFMAs finish writing it first.
    out += [raw(".Lfa_end_%=:", "label"), raw("s_nop 7", "nop"), raw("s_nop 7", "nop")]
    return out


# ---------------------------------------------------------------- waits and hazards

class Fixer:
    """Inserts s_waitcnt and s_nop into the instruction stream.

    It tracks, per VGPR, the last writer (MFMA, VALU, transcendental,
    permlane or memory) and when it issued, and the outstanding LDS and
    buffer-load operations in issue order; each instruction gets the waits
    and wait states its operands need.  Branches and labels carry this state
    (assemble() merges it at every label)."""

    def __init__(self):
        self.reset()

    def reset(self):
        self.ws = 0
        # register -> (wait-state count of the write, kind)
        self.last_write = {}
        self.last_srcc_read = {}
        self.lds = []   # outstanding LDS ops: set of registers each writes (reads: also registers it reads)
        self.vmem = []

    def _wait(self, out, which, n):
        out.append(f"s_waitcnt {which}({n})")

    def need_lds(self, regs, writes, out):
        """Wait for the LDS operations that write any of regs (RAW, WAW) or
        read any of writes (WAR: ds_write data and addresses)."""
        idx = -1
        for i, (wr, rd) in enumerate(self.lds):
            if wr & regs or rd & writes:
                idx = i
        if idx >= 0:
            n = len(self.lds) - idx - 1
            assert n <= 15
            self._wait(out, "lgkmcnt", n)
            self.lds = self.lds[idx + 1:]

    def need_vmem(self, regs, out):
        idx = -1
        for i, wr in enumerate(self.vmem):
            if wr & regs:
                idx = i
        if idx >= 0:
            n = len(self.vmem) - idx - 1
            self._wait(out, "vmcnt", n)
            self.vmem = self.vmem[idx + 1:]

    def nop(self, out, gap):
        while gap > 0:
            k = min(gap, 8)
            out.append(f"s_nop {k - 1}")
            self.ws += k
            gap -= k

    def emit(self, ins, out):
        k = ins.kind
        if k == "label":
            out.append(ins.text)
            return
        if k == "wait":
            out.append(ins.text)
            if "lgkmcnt(0)" in ins.text:
                self.lds = []
            if "vmcnt(0)" in ins.text:
                self.vmem = []
            return
        regs = ins.rd | ins.wr
        # data hazards through the memory counters
        self.need_lds(regs, ins.wr, out)
        if ins.lds and len(self.lds) == 15:  # the counter holds at most 15
            self._wait(out, "lgkmcnt", 14)
            self.lds = self.lds[1:]
        self.need_vmem(regs, out)
        if ins.lds and ins.kind == "ds_write":
            self.need_vmem(ins.rd, out)
        if k == "barrier":
            assert not self.lds, "barrier with LDS operations outstanding"
        # wait states: d = instructions issued since the writer (the writer
        # included); R wait states between them need d >= R + 1
        gap = 0
        for r in regs:
            if r in self.last_write:
                w, wk = self.last_write[r]
                d = self.ws - w
                if k == "mfma":
                    if wk == "mfma":
                        # accumulation chain: dst == srcC of the same MFMA
                        if r in ins.src_c and r in ins.wr:
                            continue
                        gap = max(gap, MFMA_VALU_WS + 1 - d)
                    elif wk in ("valu", "trans", "perm"):
                        gap = max(gap, VALU_MFMA_WS + 1 - d)
                else:
                    if wk == "mfma":
                        gap = max(gap, MFMA_VALU_WS + 1 - d)
                    elif wk == "trans" and k in ("valu", "trans", "perm"):
                        gap = max(gap, TRANS_VALU_WS + 1 - d)
                    if k == "perm" and wk in ("valu", "trans"):
                        gap = max(gap, VALU_PERM_WS + 1 - d)
        if k in ("valu", "trans", "perm"):
            for r in ins.wr:
                if r in self.last_srcc_read:
                    gap = max(gap, SRCC_WAR_WS + 1 - (self.ws - self.last_srcc_read[r]))
        self.nop(out, gap)
        out.append(ins.text)
        if k == "nop":
            self.ws += int(ins.text.split()[1]) + 1
            return
        for r in ins.wr:
            self.last_write[r] = (self.ws, k if k in ("mfma", "valu", "trans", "perm") else "mem")
        if k == "mfma":
            for r in ins.src_c:
                self.last_srcc_read[r] = self.ws
        if ins.lds:
            self.lds.append((set(ins.wr), set(ins.rd)))
            assert len(self.lds) <= 15
        if ins.vmem:
            self.vmem.append(set(ins.wr))
        self.ws += 1


def _snapshot(f):
    """Wait-state relevant history of a Fixer, relative to its current count."""
    lw = {r: (f.ws - w, k) for r, (w, k) in f.last_write.items() if f.ws - w <= MFMA_VALU_WS}
    sc = {r: f.ws - w for r, w in f.last_srcc_read.items() if f.ws - w <= SRCC_WAR_WS}
    return lw, sc, tuple(frozenset(x) for x in f.vmem)


def _merge(snaps):
    """Most recent write of each register over all paths; the outstanding
    buffer loads must be the same on every path."""
    lw, sc = {}, {}
    vm = {v for _, _, v in snaps if v is not None}
    if len(vm) > 1:  # only before the states have settled (checked at the end)
        vm = {max(vm, key=len)}
        _merge.conflicts += 1
    for slw, ssc, _ in snaps:
        for r, (d, k) in slw.items():
            if r not in lw or d < lw[r][0] or (d == lw[r][0] and k == "mfma"):
                lw[r] = (d, k)
        for r, d in ssc.items():
            sc[r] = min(d, sc.get(r, d))
    return lw, sc, (list(vm.pop()) if vm else [])


_merge.conflicts = 0


def _branch_target(text):
    parts = text.split()
    return parts[1] if parts[0].startswith("s_cbranch") or parts[0] == "s_branch" else None


def _all_fresh():
    """The state at a label no branch has reached yet: every register just
    written by an MFMA and read as an accumulator."""
    return ({r: (0, "mfma") for r in range(NVGPR)}, {r: 0 for r in range(NVGPR)}, None)


def assemble():
    """Runs the Fixer over the program until the states at the labels settle:
    a label's state merges its fall-through with every branch to it (the
    most recent write of each register over all paths)."""
    prog = program()
    at_branch = {}  # label -> list of snapshots from branches
    for _ in range(8):
        _merge.conflicts = 0
        f = Fixer()
        out = []
        seen = {}
        prev_fall = True
        for ins in prog:
            if ins.kind == "label":
                name = ins.text.rstrip(":")
                snaps = list(at_branch.get(name, [_all_fresh()]))
                if prev_fall:
                    snaps.append(_snapshot(f))
                assert not f.lds, f"LDS operations outstanding at {name}"
                lw, sc, vm = _merge(snaps)
                f.last_write = {r: (f.ws - d, k) for r, (d, k) in lw.items()}
                f.last_srcc_read = {r: f.ws - d for r, d in sc.items()}
                f.vmem = [set(x) for x in vm]
                out.append(ins.text)
                prev_fall = True
                continue
            if ins.kind == "branch":
                assert not f.lds, f"branch with LDS operations outstanding: {ins.text}"
                seen.setdefault(_branch_target(ins.text), []).append(_snapshot(f))
            f.emit(ins, out)
            prev_fall = not ins.text.startswith("s_branch")
        if seen == at_branch:
            assert _merge.conflicts == 0, "paths into a label disagree on outstanding loads"
            return out
        at_branch = seen
    raise RuntimeError("hazard states at labels did not settle")


def clobbers():
    pinned = set(range(O, O + 16 * NDB)) | set(range(QF, QF + 4 * NKS)) | set(range(KST, KST + 8 * CH))
    pinned |= set(range(K1ST, K1ST + 4 * CH))
    pinned |= {M, MNEG, L, KADDR, VADDR, KW, VW, LD0, LD1}
    return [f"v{r}" for r in range(NVGPR) if r not in pinned]


def emit(fh, d):
    configure(d)
    lines = assemble()
    pre = f"FA_FWD{d}"
    fh.write(f"// d = {d}: VGPRs v0..v{NVGPR - 1}.\n")
    fh.write(f"#define {pre}_NVGPR {NVGPR}\n")
    # register constraints of the operands bound to the asm statement
    cons = {"QF": vr(QF, 4 * NKS), "KST": vr(KST, 4 * CH), "VST": vr(VST, 4 * CH), "K1ST": vr(K1ST, 4 * CH),
            "M": vr(M), "MNEG": vr(MNEG), "L": vr(L), "KADDR": vr(KADDR), "VADDR": vr(VADDR), "KW": vr(KW),
            "VW": vr(VW), "LD0": vr(LD0), "LD1": vr(LD1)}
    if NDB == 4:
        cons.update(OLO=vr(O, 32), OHI=vr(O + 32, 32))
    else:
        cons.update(O=vr(O, 16 * NDB))
    for k, v in cons.items():
        fh.write(f'#define {pre}_C_{k} "{{{v}}}"\n')
    fh.write(f"#define {pre}_ASM \\\n")
    for ln in lines:
        fh.write(f'    "{ln}\\n" \\\n')
    fh.write('    ""\n')
    fh.write(f"#define {pre}_CLOBBERS " + ", ".join(f'"{c}"' for c in clobbers()) + ', "vcc", "scc", "memory"\n')
    return len(lines)


def main():
    dst = sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "fa_fwd_asm.inc")
    with open(dst, "w") as fh:
        fh.write("// Generated by gen_fwd_asm.py -- do not edit.\n")
        fh.write("// The hand-scheduled key loop of the bf16 forward (fa_fwd.hip) for the head\n")
        fh.write("// dimensions in SCHEDULE; register map and schedule in gen_fwd_asm.py.\n")
        n = [emit(fh, d) for d in sorted(SCHEDULE, reverse=True)]
    print(f"wrote {dst}: {n} lines")


if __name__ == "__main__":
    main()
