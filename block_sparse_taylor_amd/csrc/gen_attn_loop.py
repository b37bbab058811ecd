"""Generates attn_loop_d128.inc: the exact-item loop of the fused PISA forward
(D = 128, gfx950) as one inline-assembly block, software-pipelined by one item.

    python gen_attn_loop.py attn_loop_d128.inc

With one wave per SIMD the loop is bound by the wave's own instruction issue
(about one instruction per four cycles besides the MFMA pipe), so the
generator keeps the instruction count per item low: exact vmcnt/lgkmcnt waits
only where a value is consumed, one M0 write per four LDS DMAs (the
instruction's immediate offset moves the global and the LDS address alike),
buffer offsets held in SGPRs, and the softmax ordered so that no pad is needed
between an exp2 and its consumer.

Per step n (n = 0 .. ni - 2), one stream of 64 MFMAs:
  QK(n+1): S^T(n+1) = K(n+1) Q^T      32 MFMAs, K and Q^T from AGPRs
  PV(n):   O^T     += V(n)^T P(n)     32 MFMAs, V^T by transposed LDS reads
and between them: the softmax of item n (exp2 against the row reference, bf16
pack into P, bf16 dot2 row sums; the writes of P group g precede the PV MFMAs
that read it), the K loads of item n+2 (each after the last QK MFMA that reads
the AGPRs it overwrites), the V DMA of item n+1 into the other LDS tile, and
after the last QK MFMA the tail mask, row max and reference update of
S^T(n+1). The last item runs its softmax and PV alone. The softmax keeps a
fixed reference (a row's first finite tile max), tracks the running maximum
and flags a tile more than 64 (log2 units) above the reference; the caller
reruns with the exact maxima in that case.

Register plan (explicitly named, declared clobbered): a128-a191 K of the
next item (kreg[kt][ks]); a192-a255 the 16 Q^T operands of the query block
(loaded once at the start: operand 2 ks + qt holds, in lane l, query row
32 qt + l % 32, head dims 16 ks + 8 (l / 32) + (0..7)); v56-v119 / v120-v183 the S^T buffers of two
consecutive items; v184-v215 P; v216-v227 the bias operands of a
virtual-token item; with the second-order term v228-v229 the gate values
of a virtual-token item two ahead (per item parity, key l in lane l) and
v232-v243 three transposed-V operand buffers, without it v228-v243 four;
v244-v255
scratch (v244:v245 the pending item-list entry); s70-s90 loop state, buffer
descriptors, offsets and the bf16 pair (1, 1) for the row sums. The PV
accumulators (AGPRs), the softmax state and the per-lane addresses are
operands. At the end the Q^T operands are written to the wave's first V tile
in LDS (operand u at 1 KB u, lane l at 16 l) for the first-order term. VALU work is written in 4-byte encodings where one exists (an
8-byte instruction costs about a cycle more to issue). Hazard pads follow the
ones the compiler itself emits on gfx950:
12 wait states from an MFMA result to a VALU read, 2 from a VALU write to an
MFMA operand read, 1 from a transcendental result to a VALU read, 2 from a
VALU write to a permlane read and 3 from the permlane result, 1 from an M0
write to an LDS DMA.
"""
import os
import sys

D, KS, DT, CH, VL, RB = 128, 8, 4, 16, 16, 256
KA, QA, SREG, PREG, KBV, QBV, WV, VB, T = 128, 192, 56, 184, 216, 224, 228, 232, 244
NVB = 3                                   # transposed-V operand buffers (v232-v243; set per variant)
W_LAST = False                            # gate-value load after the K loads (else before)


def kreg(kt, ks): x = KA + 4 * (kt * KS + ks); return f"a[{x}:{x+3}]"
def sreg(b, kt, qt): x = SREG + 64 * b + 16 * (kt * 2 + qt); return f"v[{x}:{x+15}]"
def se(b, kt, qt, e): return f"v{SREG + 64 * b + 16 * (kt * 2 + qt) + e}"
def preg(kt, h, qt): x = PREG + 4 * ((kt * 2 + h) * 2 + qt); return f"v[{x}:{x+3}]"
def pw(kt, h, qt, w): return f"v{PREG + 4 * ((kt * 2 + h) * 2 + qt) + w}"
def qop(ks, qt): x = QA + 4 * (2 * ks + qt); return f"a[{x}:{x+3}]"   # Q^T operand
def vbuf(i): x = VB + 4 * i; return f"v[{x}:{x+3}]"
def vlo(i): x = VB + 4 * i; return f"v[{x}:{x+1}]"
def vhi(i): x = VB + 4 * i; return f"v[{x+2}:{x+3}]"
def t(i): return f"v{T + i}"


S_N, S_NI, S_OFFA, S_NVA, S_OFFB, S_NVB = 70, 71, 72, 73, 74, 75
S_KRS, S_VRS = 76, 80                     # 4-SGPR buffer descriptors
S_M0, S_C1, S_X, S_Y, S_C2, S_C3, S_ONES, S_NVC = 84, 85, 86, 87, 88, 89, 90, 91
S_WRS = 92                                # 4-SGPR descriptor of a gate-value DMA
SGPRS = list(range(70, 96))
SOFF = {0: "0", 4096: f"s{S_C1}", 8192: f"s{S_C2}", 12288: f"s{S_C3}"}
def SR(a, n=4): return f"s[{a}:{a+n-1}]"
ACC = [f"%[a{i}]" for i in range(8)]      # acc[dt][qt] -> a{2 dt + qt}
MINF = "0xff800000"
GROUPS = [(kt, h) for kt in range(2) for h in range(2)]
TR = {0: ["%[tr0_0]", "%[tr0_1]", "%[tr0_2]", "%[tr0_3]"],
      1: ["%[tr1_0]", "%[tr1_1]", "%[tr1_2]", "%[tr1_3]"]}
VLDS = {0: "%[vl0]", 1: "%[vl1]"}

L = []
def emit(s): L.append(s)

LBL = [0]
def label(name):
    LBL[0] += 1
    return f"PISA_{name}_{LBL[0]}_%="


class Op:
    """A scheduled unit: its lines; for an LDS read its id; for an MFMA the LDS
    reads and the previous step's VMEM ops it needs; the MFMA it must follow
    (after) and the MFMA it must precede (before); for a VMEM op its id."""
    def __init__(self, kind, lines, lds_id=None, needs=(), vneeds=(), after=-1, before=None, vm_id=None):
        self.kind, self.lines, self.lds_id, self.needs, self.vneeds = kind, lines, lds_id, tuple(needs), tuple(vneeds)
        self.after, self.before, self.vm_id = after, before, vm_id

    def cost(self):
        c = 0
        for ln in self.lines:
            if ln.startswith("v_exp_f32"):
                c += 4
            elif ln.startswith("s_nop"):
                c += int(ln.split()[1]) + 1
            else:
                c += 1
        return c


class Sched:
    """Merges an MFMA stream with LDS reads (issued a few MFMAs ahead), VMEM
    ops (in order, at most one per MFMA) and VALU ops (in order, about
    `budget` issue units per MFMA), with lgkmcnt/vmcnt waits only where an
    MFMA consumes data that may still be in flight. `prev_after[id]` is the
    number of VMEM ops issued after op `id` in the previous step."""
    def __init__(self, prev_after=None, n_lds=0):
        self.lds_seq, self.n_lds, self.lgkm_ok = {}, n_lds, n_lds - 1
        self.prev_after, self.vm_issued, self.prev_ok = prev_after or {}, 0, None

    def issue(self, op):
        lines = op.lines
        if op.kind == "valu" and op.vneeds:
            # a VALU op waiting for memory (the bias of a virtual-token item
            # for its gate values): the wait goes after the op's leading
            # branch (lines 0-1), so the exact items that skip it do not wait;
            # it is conditional, so later waits do not count on it
            need = min(self.prev_after[v] for v in op.vneeds)
            lines = lines[:2] + [f"s_waitcnt vmcnt({min(need + self.vm_issued, 63)})"] + lines[2:]
        for ln in lines:
            emit(ln)
        if op.lds_id is not None:
            self.lds_seq[op.lds_id] = self.n_lds
            self.n_lds += 1
        if op.kind == "vmem":
            self.vm_issued += 1

    def wait_lds(self, needs):
        if not needs:
            return
        last = max(self.lds_seq[n] for n in needs)
        if last <= self.lgkm_ok:
            return
        after = min(self.n_lds - 1 - last, 15)
        emit(f"s_waitcnt lgkmcnt({after})")
        self.lgkm_ok = self.n_lds - 1 - after

    def wait_vm(self, vneeds):
        if not vneeds:
            return
        need = min(self.prev_after[v] for v in vneeds)     # ops issued after the youngest needed one
        if self.prev_ok is not None and need >= self.prev_ok:
            return
        n = min(need + self.vm_issued, 63)
        emit(f"s_waitcnt vmcnt({n})")
        self.prev_ok = n - self.vm_issued

    def run(self, mfmas, lds, vmem, valu, lds_ahead=8, budget=8):
        li = mi = vi = 0
        for i, m in enumerate(mfmas):
            req = max((j for j in range(vi, len(valu)) if valu[j].before is not None and valu[j].before <= i), default=-1)
            forced = req >= vi
            while vi <= req:
                assert valu[vi].after < i, "dependence cycle in the schedule"
                self.issue(valu[vi])
                vi += 1
            horizon = set()
            for mm in mfmas[i:i + lds_ahead]:
                horizon.update(mm.needs)
            while li < len(lds) and lds[li].after < i and (lds[li].lds_id in horizon or lds[li].lds_id in m.needs):
                self.issue(lds[li])
                li += 1
            if forced:
                emit("s_nop 1")                    # VALU result -> MFMA operand read
            assert all(nd in self.lds_seq for nd in m.needs), "LDS read not issued before its MFMA"
            self.wait_lds(m.needs)
            self.wait_vm(m.vneeds)
            self.issue(m)
            # one VMEM op (an M0 write goes with the DMA after it)
            while mi < len(vmem) and vmem[mi].after <= i:
                op = vmem[mi]
                self.issue(op)
                mi += 1
                if op.kind == "vmem":
                    break
            spent = 0
            near = False
            while vi < len(valu) and valu[vi].after <= i and spent < budget:
                spent += valu[vi].cost()
                near |= valu[vi].before is not None and valu[vi].before <= i + 1
                self.issue(valu[vi])
                vi += 1
            if near:
                emit("s_nop 1")                    # VALU result -> the next MFMA's operand read
        for lst, k in ((lds, li), (vmem, mi), (valu, vi)):
            for op in lst[k:]:
                self.issue(op)


def rsrc_item(base, kind, off, nv):
    # descriptor of an item's K (kind "k") or V ("v") rows: the exact-block
    # base, or the virtual-token base when bit 16 of the item word is set;
    # num_records = the item's rows * RB for V, the whole 16 KB block for K
    lo_e, hi_e, lo_v, hi_v = {"k": ("%[kb_lo]", "%[kb_hi]", "%[kv_lo]", "%[kv_hi]"),
                              "v": ("%[vb_lo]", "%[vb_hi]", "%[vv_lo]", "%[vv_hi]")}[kind]
    emit(f"s_bitcmp1_b32 s{nv}, 16")
    emit(f"s_cselect_b32 s{S_X}, {lo_v}, {lo_e}")
    emit(f"s_cselect_b32 s{S_Y}, {hi_v}, {hi_e}")
    emit(f"s_add_u32 s{base}, s{S_X}, s{off}")
    emit(f"s_addc_u32 s{base+1}, s{S_Y}, 0")
    if kind == "k":
        emit(f"s_movk_i32 s{base+2}, {64 * RB}")
    else:
        emit(f"s_and_b32 s{S_X}, s{nv}, 0xffff")
        emit(f"s_lshl_b32 s{base+2}, s{S_X}, 8")
    emit(f"s_mov_b32 s{base+3}, 0x00020000")


def kbias_lines(off, nv, wpar):
    """for a virtual-token item: the A operand of the bias k-step. Key j = 64 g
    + 32 kt + lane % 32 of group g = off >> 14 gets b_j = log2(n_j) / c2
    (+ w_ij / scale with the second-order term: the item's gated values
    were loaded a step earlier into the gate register of parity wpar, key
    l in lane l; the lower lane half, which alone carries the operand, takes
    keys 32 .. 63 from the upper half by a lane swap), or -inf if block j is
    selected (exact) or past N, split into bf16 hi + lo in
    k-slots 0 and 1 of the lower lane half (zero elsewhere); with the constant
    B operand (1, 1 in slots 0, 1) one MFMA k-step adds b_j to S^T."""
    skip = label("nokb")
    out = [f"s_bitcmp1_b32 s{nv}, 16", f"s_cbranch_scc0 {skip}",
           f"s_lshr_b32 s{S_X}, s{off}, 11",                  # 8 g: byte offset of its two selection words
           f"s_add_u32 s{S_X}, s{S_X}, %[sbase]",
           f"v_mov_b32 {t(6)}, s{S_X}",
           f"ds_read_b64 v[{T+6}:{T+7}], {t(6)}",
           "s_waitcnt lgkmcnt(0)",
           f"v_readfirstlane_b32 s{S_X}, {t(6)}",
           f"v_readfirstlane_b32 s{S_Y}, {t(7)}",
           "s_nop 1"]
    j, tmp, sel, pk = t(2), t(3), t(6), t(7)
    for kt in range(2):
        word = f"s{S_X}" if kt == 0 else f"s{S_Y}"
        if kt and WITH_SO[0]:
            # keys 32 .. 63 (upper lanes of the gate register) to the lower
            # lanes of pk: the swap exchanges tmp's upper and pk's lower half
            out += [f"v_mov_b32 {tmp}, v{WV + wpar}", f"v_mov_b32 {pk}, v{WV + wpar}", "s_nop 1",
                    f"v_permlane32_swap_b32 {tmp}, {pk}", "s_nop 2"]
        out += [f"v_bfe_u32 {j}, %[koff], 4, 5",                 # lane % 32 (koff = 16 lane)
                f"v_lshrrev_b32_e64 {tmp}, 8, s{off}",           # 64 g
                f"v_add_u32 {j}, {j}, {tmp}"]
        if kt:
            out.append(f"v_add_u32 {j}, 32, {j}")
        out += [f"v_bfe_u32 {sel}, {word}, {j}, 1",              # block j selected
                f"v_cmp_le_u32 vcc, %[nblk], {j}",
                f"v_cndmask_b32_e64 {sel}, {sel}, 1, vcc",       # or j >= N
                f"v_cmp_eq_u32 vcc, %[nm1], {j}",
                f"v_cndmask_b32 {tmp}, %[bfull], %[blast], vcc"] # b_j
        if WITH_SO[0]:
            # second-order term: + w_ij / scale (the gated table row of this
            # query block; keys past N are -inf anyway)
            out.append(f"v_fma_f32 {tmp}, {f'v{WV + wpar}' if kt == 0 else pk}, %[winv], {tmp}")
        out += [f"v_mov_b32 {j}, {tmp}",
                f"v_cvt_pk_bf16_f32 {pk}, {j}, {j}",
                f"v_and_b32 {pk}, 0xffff0000, {pk}",             # hi as fp32
                f"v_sub_f32 {j}, {j}, {pk}",                      # lo = b - hi (exact)
                f"v_cvt_pk_bf16_f32 {pk}, {pk}, {j}",            # (hi, lo)
                f"v_mov_b32 {tmp}, 0xff80",
                f"v_cmp_eq_u32 vcc, 0, {sel}",
                f"v_cndmask_b32 {pk}, {tmp}, {pk}, vcc",         # selected: (-inf, 0)
                f"v_bfe_u32 {tmp}, %[koff], 9, 1",               # lane half
                f"v_subrev_u32 {tmp}, 1, {tmp}",                 # lower half: all ones
                f"v_and_b32 {pk}, {pk}, {tmp}",
                f"v_mov_b32 v{KBV + 4 * kt}, {pk}"]
    out.append(f"{skip}:")
    return out


def bias_mfma_op(sb, nv):
    """the bias k-step of a virtual-token item (skipped for exact blocks)."""
    skip = label("nobias")
    lines = [f"s_bitcmp1_b32 s{nv}, 16", f"s_cbranch_scc0 {skip}"]
    for kt in range(2):
        for qt in range(2):
            lines.append(f"v_mfma_f32_32x32x16_bf16 {sreg(sb, kt, qt)}, v[{KBV + 4 * kt}:{KBV + 4 * kt + 3}], "
                         f"v[{QBV}:{QBV + 3}], {sreg(sb, kt, qt)}")
    lines.append(f"{skip}:")
    return Op("mfma", lines)


def kload_op(kt, ks, after):
    # packed K: k-step ks of key tile kt is the contiguous 1 KB run at 8192 kt + 1024 ks
    off = 1024 * (KS * kt + ks)
    return Op("vmem", [f"buffer_load_dwordx4 {kreg(kt, ks)}, %[koff], {SR(S_KRS)}, {SOFF[off & ~4095]} offen offset:{off & 4095}"],
              after=after, vm_id=("k", kt, ks))


def wload_ops(off, nv, wpar):
    """the gated second-order values of an item two ahead (group g = off >> 14:
    entry 64 g + l of the query block's row in lane l) -> the gate register of
    parity wpar. The descriptor covers exactly the group's part of the row:
    size 0 for an exact block or without the second-order term, so no byte
    outside the row is addressed."""
    return [Op("vmem", [
        f"s_lshr_b32 s{S_Y}, s{off}, 6",                   # 256 g
        f"s_add_u32 s{S_WRS}, %[wrow_lo], s{S_Y}",
        f"s_addc_u32 s{S_WRS + 1}, %[wrow_hi], 0",
        f"s_sub_u32 s{S_WRS + 2}, %[wbytes], s{S_Y}",        # 4 N - 256 g (> 0 for a virtual group)
        f"s_bitcmp1_b32 s{nv}, 16",
        f"s_cselect_b32 s{S_WRS + 2}, s{S_WRS + 2}, 0",
        f"buffer_load_dword v{WV + wpar}, %[wlane], {SR(S_WRS)}, 0 offen"], vm_id=("w", 0))]


def vm_list(vl, qk_last_reader, woff, wnv, wpar):
    """the step's VMEM ops in issue order: the V DMA of the next item (rows
    4 i .. 4 i + 3 -> LDS tile + 1024 i; M0 set once per four; its tile was
    last read in the previous step), the K loads (ks-major, each after the
    last QK MFMA reading its registers, + 1) and the gate-value loads of the
    item after next (their register parity was last read in the previous
    step)."""
    ops = []
    for a in range(4):
        ops.append(Op("m0", [f"s_add_u32 m0, {vl}, {4096 * a}" if a else f"s_mov_b32 m0, {vl}", "s_nop 0"]))
        for b in range(4):
            i = 4 * a + b
            ops.append(Op("vmem", [f"buffer_load_dwordx4 %[voff], {SR(S_VRS)}, {SOFF[4096 * a]} offen offset:{1024 * b} lds"],
                          vm_id=("d", i)))
    if WITH_SO[0] and not W_LAST:
        ops += wload_ops(woff, wnv, wpar)
    for ks in range(KS):
        for kt in range(2):
            ops.append(kload_op(kt, ks, qk_last_reader[(kt, ks)] + 1))
    if WITH_SO[0] and W_LAST:
        ops += wload_ops(woff, wnv, wpar)
    return ops


def prev_after_of(vm):
    ids = [o.vm_id for o in vm if o.kind == "vmem"]
    return {v: len(ids) - 1 - k for k, v in enumerate(ids)}


def qk_ops(sb, vneed):
    """S^T(sb) = K Q^T: 32 MFMAs (k-step-major; both operands in AGPRs) and
    the index of the last MFMA reading each K operand."""
    mf, idx = [], {}
    for ks in range(KS):
        for kt in range(2):
            for qt in range(2):
                src_c = "0" if ks == 0 else sreg(sb, kt, qt)
                idx[(kt, qt, ks)] = len(mf)
                mf.append(Op("mfma", [f"v_mfma_f32_32x32x16_bf16 {sreg(sb, kt, qt)}, {kreg(kt, ks)}, {qop(ks, qt)}, {src_c}"],
                             vneeds=[("k", kt, ks)] if vneed else []))
    last = {(kt, ks): max(idx[(kt, qt, ks)] for qt in range(2)) for kt in range(2) for ks in range(KS)}
    return mf, [], last


def pv_ops(par, base, vneed):
    """O^T += V^T P: 32 MFMAs (group-major) and their 32 transposed V reads from tile par.
    base(k) is the position of PV MFMA k in the step's MFMA stream."""
    if isinstance(base, int):
        b0 = base
        base = lambda k: b0 + k
    mf, lds = [], []
    pairs = [(kt, h, dt) for (kt, h) in GROUPS for dt in range(DT)]
    for r, (kt, h, dt) in enumerate(pairs):
        for qt in range(2):
            mf.append(Op("mfma", [f"v_mfma_f32_32x32x16_bf16 {ACC[dt * 2 + qt]}, {vbuf(r % NVB)}, {preg(kt, h, qt)}, {ACC[dt * 2 + qt]}"],
                         needs=[("v", r, 0), ("v", r, 1)], vneeds=[("d", i) for i in range(VL)] if vneed else []))
    for r, (kt, h, dt) in enumerate(pairs):
        r0 = 32 * kt + 16 * h
        after = base(2 * (r - NVB) + 1) if r >= NVB else -1   # buffer r % NVB last read by pair r - NVB
        lds.append(Op("lds", [f"ds_read_b64_tr_b16 {vlo(r % NVB)}, {TR[par][dt]} offset:{r0 * RB}"], lds_id=("v", r, 0), after=after))
        lds.append(Op("lds", [f"ds_read_b64_tr_b16 {vhi(r % NVB)}, {TR[par][dt]} offset:{(r0 + 8) * RB}"], lds_id=("v", r, 1), after=after))
    return mf, lds


def mask_lines(sb, nv):
    """keys >= nv of S^T(sb) -> -inf (only the ragged last block of a sequence)."""
    skip = label("nomask")
    out = [f"s_cmp_lt_u32 s{nv}, 64", f"s_cbranch_scc0 {skip}", "s_nop 7", "s_nop 4", f"v_mov_b32 {t(7)}, {MINF}"]
    for kt in range(2):
        for e in range(16):
            key = 32 * kt + 8 * (e // 4) + (e % 4)
            out.append(f"v_add_u32 {t(6)}, {key}, %[kb4]")
            out.append(f"v_cmp_gt_u32 vcc, s{nv}, {t(6)}")
            for qt in range(2):
                out.append(f"v_cndmask_b32 {se(sb, kt, qt, e)}, {t(7)}, {se(sb, kt, qt, e)}, vcc")
    out.append(f"{skip}:")
    return out


def max_lines(sb):
    """row max of S^T(sb) (scaled by c2) for both query tiles, reference
    update, running maximum, restart flag, and -reference in t4 / t5."""
    a = [t(2), t(3)]
    v = [[se(sb, kt, qt, e) for kt in range(2) for e in range(16)] for qt in range(2)]
    out = ["s_nop 7", "s_nop 4"]                  # MFMA results -> VALU
    for qt in range(2):
        out.append(f"v_max3_f32 {a[qt]}, {v[qt][0]}, {v[qt][1]}, {v[qt][2]}")
    for i in range(3, 31, 2):
        for qt in range(2):
            out.append(f"v_max3_f32 {a[qt]}, {a[qt]}, {v[qt][i]}, {v[qt][i+1]}")
    for qt in range(2):
        out.append(f"v_max_f32 {a[qt]}, {a[qt]}, {v[qt][31]}")
    out += [f"v_mov_b32 {t(6)}, {a[0]}", f"v_mov_b32 {t(7)}, {a[1]}", "s_nop 1",
            f"v_permlane32_swap_b32 {a[0]}, {t(6)}", f"v_permlane32_swap_b32 {a[1]}, {t(7)}", "s_nop 2"]
    for qt in range(2):
        out.append(f"v_max_f32 {a[qt]}, {a[qt]}, {t(6 + qt)}")
    for qt in range(2):
        out.append(f"v_mul_f32 {a[qt]}, {a[qt]}, %[c2]")
    for qt in range(2):
        m2 = f"%[m2{qt}]"
        out += [f"v_max_f32 %[mx{qt}], %[mx{qt}], {a[qt]}",
                f"v_cmp_eq_f32 vcc, {MINF}, {m2}",
                f"v_cndmask_b32 {m2}, {m2}, {a[qt]}, vcc",
                f"v_add_f32 {t(6 + qt)}, 0x42800000, {m2}",
                f"v_cmp_gt_f32 vcc, {a[qt]}, {t(6 + qt)}",
                f"v_cndmask_b32_e64 %[need], %[need], 1, vcc",
                f"v_cmp_eq_f32 vcc, {MINF}, {m2}",
                f"v_cndmask_b32_e64 {t(4 + qt)}, {m2}, 0, vcc",
                f"v_xor_b32 {t(4 + qt)}, 0x80000000, {t(4 + qt)}"]
    return out


def softmax_ops(sb, pv_first):
    """exp2(S^T c2 - m) of S^T(sb) packed into P in pairs; the exp2 of pair p
    is separated from its consumers by the FMAs of pair p + 1. The writes of P
    group g precede the first PV MFMA of that group (pv_base + 8 g)."""
    pairs = []
    for gi, (kt, h) in enumerate(GROUPS):
        for qt in range(2):
            for w in range(4):
                pairs.append((gi, kt, h, qt, w))

    def tmp(p): return t(8 + 2 * (p % 2)), t(9 + 2 * (p % 2))

    def F(p):
        gi, kt, h, qt, w = pairs[p]
        x0, x1 = tmp(p)
        e = 8 * h + 2 * w
        return [Op("valu", [f"v_fma_f32 {x0}, {se(sb, kt, qt, e)}, %[c2], {t(4 + qt)}"]),
                Op("valu", [f"v_fma_f32 {x1}, {se(sb, kt, qt, e + 1)}, %[c2], {t(4 + qt)}"])]

    def E(p):
        x0, x1 = tmp(p)
        return [Op("valu", [f"v_exp_f32 {x0}, {x0}"]), Op("valu", [f"v_exp_f32 {x1}, {x1}"])]

    def C(p, pad=False):
        gi, kt, h, qt, w = pairs[p]
        x0, x1 = tmp(p)
        return [Op("valu", (["s_nop 0"] if pad else []) + [f"v_cvt_pk_bf16_f32 {pw(kt, h, qt, w)}, {x0}, {x1}"],
                   before=pv_first[gi]),
                Op("valu", [f"v_dot2c_f32_bf16 %[l{qt}], s{S_ONES}, {pw(kt, h, qt, w)}"])]

    ops = F(0) + E(0)
    for p in range(1, len(pairs)):
        ops += F(p) + C(p - 1) + E(p)
    ops += C(len(pairs) - 1, pad=True)
    return ops


def read_entry(dst_off, dst_nv):
    emit(f"v_readfirstlane_b32 s{dst_off}, {t(0)}")
    emit(f"v_readfirstlane_b32 s{dst_nv}, {t(1)}")
    emit("s_nop 1")


def read_list(index_lines):
    # list entry s{S_X} (computed by index_lines) -> v244:v245
    for ln in index_lines:
        emit(ln)
    emit(f"s_lshl_b32 s{S_X}, s{S_X}, 3")
    emit(f"v_add_u32 {t(0)}, s{S_X}, %[il]")
    emit(f"ds_read_b64 v[{T}:{T+1}], {t(0)}")


def full_step(par, vm_order):
    """item n = S_N: S^T(n) in buffer par (masked, reference updated), K(n+1)
    loading into the AGPRs, V(n) in tile par; offA/nvA = item n+1; the
    pending list read holds entry n+2."""
    emit(f"; ---- pipelined step, parity {par}")
    emit("s_waitcnt lgkmcnt(0)")
    read_entry(S_OFFB, S_NVB)
    rsrc_item(S_VRS, "v", S_OFFA, S_NVA)                  # V of item n+1
    rsrc_item(S_KRS, "k", S_OFFB, S_NVB)                  # K of item n+2
    read_list([f"s_add_u32 s{S_X}, s{S_N}, 3", f"s_sub_u32 s{S_Y}, s{S_NI}, 1", f"s_min_u32 s{S_X}, s{S_X}, s{S_Y}"])
    s = Sched(prev_after=prev_after_of(vm_order), n_lds=1)
    mq, lq, last = qk_ops(1 - par, vneed=True)
    mq.append(bias_mfma_op(1 - par, S_NVA))
    # MFMA stream: the PV groups of item n interleaved with the QK k-steps of
    # item n+1, so that the softmax of item n (which feeds PV group by group)
    # spreads over the whole step
    nq = len(mq)
    order = ([("q", k) for k in range(16)] + [("p", k) for k in range(8)] + [("q", k) for k in range(16, 24)] +
             [("p", k) for k in range(8, 16)] + [("q", k) for k in range(24, nq)] + [("p", k) for k in range(16, 32)])
    posq = {k: n for n, (w, k) in enumerate(order) if w == "q"}
    posp = {k: n for n, (w, k) in enumerate(order) if w == "p"}
    last = {key: posq[v] for key, v in last.items()}
    mp, lp = pv_ops(par, lambda k: posp[k], vneed=True)
    vm = vm_list(VLDS[1 - par], last, S_OFFB, S_NVB, par)      # gate values of item n+2
    assert [o.vm_id for o in vm] == [o.vm_id for o in vm_order]
    # the bias of a virtual item n+1 first (its gate values arrived a step
    # ago), then the softmax of item n
    valu = [Op("valu", kbias_lines(S_OFFA, S_NVA, 1 - par), before=posq[nq - 1],
               vneeds=[("w", 0)] if WITH_SO[0] else [])]
    valu += softmax_ops(par, [posp[8 * gi] for gi in range(4)])
    valu.append(Op("valu", mask_lines(1 - par, S_NVA), after=posq[nq - 1]))
    if TRACK_MAX[0]:
        valu += [Op("valu", [ln], after=posq[nq - 1]) for ln in max_lines(1 - par)]
    mf = [mq[k] if w == "q" else mp[k] for (w, k) in order]
    s.run(mf, lq + lp, vm, valu)
    snapshot()
    emit(f"s_mov_b32 s{S_OFFA}, s{S_OFFB}")
    emit(f"s_mov_b32 s{S_NVC}, s{S_NVA}")
    emit(f"s_mov_b32 s{S_NVA}, s{S_NVB}")
    emit(f"s_add_u32 s{S_N}, s{S_N}, 1")


def snapshot():
    # after the softmax of an exact item: the row sums so far (the virtual
    # tokens, which come last, add l_tail = l - ls)
    skip = label("virt")
    emit(f"s_bitcmp1_b32 s{S_NVC}, 16")
    emit(f"s_cbranch_scc1 {skip}")
    emit("v_mov_b32 %[ls0], %[l0]")
    emit("v_mov_b32 %[ls1], %[l1]")
    emit(f"{skip}:")


def tail(par):
    """the last item: softmax of S^T(par), PV from tile par."""
    emit(f"; ---- last item, parity {par}")
    emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
    for o in softmax_ops(par, [8 * gi for gi in range(4)]):
        for ln in o.lines:
            emit(ln)
    snapshot()
    emit("s_nop 1")
    mp, lp = pv_ops(par, 0, vneed=False)
    Sched().run(mp, lp, [], [])


def program():
    done, tail0, tail1, loop, empty = (label("done"), label("tail0"), label("tail1"), label("loop"),
                                       label("empty"))
    emit(f"s_mov_b32 s{S_M0}, m0")
    emit("s_nop 4")                                # the accumulator was just written by VALU
    emit(f"s_mov_b32 s{S_NI}, %[ni]")
    emit(f"s_mov_b32 s{S_N}, 0")
    emit(f"s_movk_i32 s{S_C1}, 4096")
    emit(f"s_movk_i32 s{S_C2}, 8192")
    emit(f"s_movk_i32 s{S_C3}, 12288")
    emit(f"s_mov_b32 s{S_WRS + 3}, 0x00020000")    # gate-value descriptor, word 3 (words 0-2 per DMA)
    # the Q^T operands (rows past T read zero: the descriptor's range)
    emit(f"s_mov_b32 s{S_VRS}, %[q_lo]")
    emit(f"s_mov_b32 s{S_VRS + 1}, %[q_hi]")
    emit(f"s_mov_b32 s{S_VRS + 2}, %[q_bytes]")
    emit(f"s_mov_b32 s{S_VRS + 3}, 0x00020000")
    for ks in range(KS):
        for qt in range(2):
            emit(f"buffer_load_dwordx4 {qop(ks, qt)}, %[qoff], {SR(S_VRS)}, {SOFF[8192 * qt]} offen offset:{32 * ks}")
    emit(f"s_cmp_eq_u32 s{S_NI}, 0")
    emit(f"s_cbranch_scc1 {empty}")
    emit(f"s_mov_b32 s{S_ONES}, 0x3f803f80")       # bf16 (1, 1)
    # constant parts of the bias operands: B = (1, 1, 0, ...) in the lower lane half
    emit(f"v_bfe_u32 {t(6)}, %[koff], 9, 1")        # lane half
    emit(f"v_subrev_u32 {t(6)}, 1, {t(6)}")
    emit(f"v_and_b32 {t(6)}, s{S_ONES}, {t(6)}")
    emit(f"v_mov_b32 v{QBV}, {t(6)}")
    for r in list(range(QBV + 1, QBV + 4)) + [KBV + 1, KBV + 2, KBV + 3, KBV + 5, KBV + 6, KBV + 7]:
        emit(f"v_mov_b32 v{r}, 0")
    # item 0: its K, then (pipelined with QK(0)) K of item 1 and V of item 0
    emit(f"ds_read_b64 v[{T}:{T+1}], %[il]")
    emit("s_waitcnt lgkmcnt(0)")
    read_entry(S_OFFB, S_NVB)
    emit(f"s_mov_b32 s{S_NVC}, s{S_NVB}")
    rsrc_item(S_KRS, "k", S_OFFB, S_NVB)
    rsrc_item(S_VRS, "v", S_OFFB, S_NVB)
    if WITH_SO[0]:
        for op in wload_ops(S_OFFB, S_NVB, 0):        # gate values of item 0 (waited with K(0))
            for ln in op.lines:
                emit(ln)
    for ks in range(KS):
        for kt in range(2):
            for ln in kload_op(kt, ks, -1).lines:
                emit(ln)
    read_list([f"s_sub_u32 s{S_Y}, s{S_NI}, 1", f"s_min_u32 s{S_X}, s{S_Y}, 1"])   # entry 1 (clamped)
    emit("s_waitcnt lgkmcnt(0)")
    read_entry(S_OFFA, S_NVA)
    rsrc_item(S_KRS, "k", S_OFFA, S_NVA)
    read_list([f"s_sub_u32 s{S_Y}, s{S_NI}, 1", f"s_min_u32 s{S_X}, s{S_Y}, 2"])   # entry 2 (clamped), pending
    emit("s_waitcnt vmcnt(0)")                     # K(0)
    mq, lq, last = qk_ops(0, vneed=False)
    vm0 = vm_list(VLDS[0], last, S_OFFA, S_NVA, 1)             # gate values of item 1
    Sched(n_lds=1).run(mq + [bias_mfma_op(0, S_NVB)], lq, vm0, [Op("valu", kbias_lines(S_OFFB, S_NVB, 0), before=len(mq))])
    for ln in mask_lines(0, S_NVB):
        emit(ln)
    for ln in max_lines(0):
        emit(ln)
    emit(f"{loop}:")
    emit(f"s_add_u32 s{S_Y}, s{S_N}, 1")
    emit(f"s_cmp_ge_u32 s{S_Y}, s{S_NI}")
    emit(f"s_cbranch_scc1 {tail0}")
    full_step(0, vm0)
    emit(f"s_add_u32 s{S_Y}, s{S_N}, 1")
    emit(f"s_cmp_ge_u32 s{S_Y}, s{S_NI}")
    emit(f"s_cbranch_scc1 {tail1}")
    full_step(1, vm0)
    emit(f"s_branch {loop}")
    for lab, par in ((tail0, 0), (tail1, 1)):
        emit(f"{lab}:")
        tail(par)
        emit(f"s_branch {done}")
    emit(f"{empty}:")                              # no items
    emit(f"{done}:")
    emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
    # the Q^T operands to the wave's first V tile (free now) for the caller:
    # operand u at bytes [1024 u, 1024 u + 1024), lane l at 16 l
    for u in range(2 * KS):
        for r in range(4):
            emit(f"v_accvgpr_read_b32 v{SREG + 4 * u + r}, a{QA + 4 * u + r}")
    for u in range(2 * KS):
        emit(f"ds_write_b128 %[qdump], v[{SREG + 4 * u}:{SREG + 4 * u + 3}] offset:{1024 * u}")
    emit("s_waitcnt lgkmcnt(0)")
    emit("s_nop 15")
    emit("s_nop 15")                               # last accumulator MFMAs before later reads
    emit(f"s_mov_b32 m0, s{S_M0}")


TRACK_MAX = [True]
WITH_SO = [True]
bodies = {}
for name, track, so in (("PISA_ATTN_LOOP_D128_ASM", False, False), ("PISA_ATTN_LOOP_D128_SAFE_ASM", True, False),
                        ("PISA_ATTN_LOOP_D128_SO_ASM", False, True), ("PISA_ATTN_LOOP_D128_SO_SAFE_ASM", True, True)):
    L.clear()
    TRACK_MAX[0], WITH_SO[0] = track, so
    VB, NVB = (232, 3) if so else (228, 4)
    program()
    bodies[name] = list(L)
clob = ([f'"v{i}"' for i in range(SREG, 256)] + [f'"a{i}"' for i in range(KA, 256)] +
        [f'"s{i}"' for i in SGPRS])
out = ["// Generated by gen_attn_loop.py (do not edit): the D = 128 item loop of the fused PISA forward for gfx950.",
       "// PISA_ATTN_LOOP_D128_ASM: the row maximum of the first item only (sets the reference);",
       "// PISA_ATTN_LOOP_D128_SAFE_ASM: the row maximum of every item, the restart flag and the running maximum;",
       "// the _SO_ variants add the gated second-order term to the virtual tokens' logits (a kernel",
       "// instantiation holds one pair: two pairs in one kernel measured ~15% slower)."]
for name, body in bodies.items():
    out.append(f"#define {name} \\")
    out.append(" \\\n".join('    "' + l + '\\n"' for l in body))
    out.append("")
out.append("#define PISA_ATTN_LOOP_D128_CLOBBERS " + ", ".join(clob) + ', "vcc", "scc", "memory"')
dst = sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.path.dirname(os.path.abspath(__file__)), "attn_loop_d128.inc")
open(dst, "w").write("\n".join(out) + "\n")
print(sum(len(b) for b in bodies.values()), "instructions/labels ->", dst)
