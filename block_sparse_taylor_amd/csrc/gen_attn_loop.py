"""Generates attn_loop_d128.inc: the exact-item loop of the fused PISA forward
(D = 128, gfx950) as one inline-assembly block.

    python gen_attn_loop.py attn_loop_d128.inc

Register plan inside the block (all explicitly named and declared clobbered,
so they live across the whole loop): v56-v119 K operands of the current item
(kreg[kt][ks], loaded one item ahead from the packed copy of K, one
contiguous 1 KB run per load), v120-v183 the S^T accumulators
(s[kt][qt]), v184-v215 the bf16 P operands, v216-v231 Q^T operand buffers,
v232-v243 transposed-V operand buffers, v244-v255 scratch; s70-s89 loop
state and buffer descriptors. The PV accumulators, the softmax state and the
per-lane addresses are operands. Every wait (vmcnt, lgkmcnt) and every
hazard pad (s_nop) is explicit: the compiler's hazard recognizer does not see
inside inline assembly. The pads follow the ones the compiler itself emits for
the same dependences on gfx950: 12 wait states from an MFMA result to a VALU
read, 1 from a transcendental result to a VALU read, 2 from a VALU write to a
permlane read and 3 from the permlane result, 1 from an M0 write to an LDS DMA.

Per item (step), with the V tiles of parity p = item % 2:
  phase A: S^T = K Q^T (32 MFMAs, k-step-major) interleaved with the Q^T
           reads, the 16 V DMA instructions of this item (into parity p) and
           the 16 K loads of the next item (each after the MFMAs that read the
           registers it overwrites);
  phase B: O^T += V^T P of the previous item (32 MFMAs, transposed reads of
           parity 1 - p) interleaved with the softmax of this item (row max,
           reference update, exp2, bf16 pack into P once that group of P is no
           longer read, bf16 dot2 row sums).
The softmax keeps a fixed reference (first finite tile max of a row), tracks
the running tile maximum and flags a tile that exceeds the reference by more
than 64 (log2 units); the caller reruns with the exact maxima in that case.
"""
import os
import sys

D, KS, DT, CH, RPI, VL, RB, QP = 128, 8, 4, 16, 4, 16, 256, 136
KREG, SREG, PREG, QB, VB, T = 56, 120, 184, 216, 232, 244


def kreg(kt, ks): b = KREG + 4 * (kt * KS + ks); return f"v[{b}:{b+3}]"
def sreg(kt, qt): b = SREG + 16 * (kt * 2 + qt); return f"v[{b}:{b+15}]"
def se(kt, qt, e): return f"v{SREG + 16 * (kt * 2 + qt) + e}"
def preg(kt, h, qt): b = PREG + 4 * ((kt * 2 + h) * 2 + qt); return f"v[{b}:{b+3}]"
def pw(kt, h, qt, w): return f"v{PREG + 4 * ((kt * 2 + h) * 2 + qt) + w}"
def qbuf(i): b = QB + 4 * i; return f"v[{b}:{b+3}]"
def vbuf(i): b = VB + 4 * i; return f"v[{b}:{b+3}]"
def vlo(i): b = VB + 4 * i; return f"v[{b}:{b+1}]"
def vhi(i): b = VB + 4 * i; return f"v[{b+2}:{b+3}]"
def t(i): return f"v{T + i}"


S_N, S_NI, S_OFF, S_NV, S_NVC, S_X = 70, 71, 72, 73, 74, 75
S_KRS, S_VRS = 76, 80          # 4-SGPR buffer descriptors
S_M0, S_SOFF, S_NOFF, S_NNV, S_Y = 84, 85, 86, 87, 89
SGPRS = list(range(70, 90))
def SR(a, n=4): return f"s[{a}:{a+n-1}]"
ACC = [f"%[a{i}]" for i in range(8)]   # acc[dt][qt] -> a{2 dt + qt}
MINF = "0xff800000"

L = []
def emit(s): L.append(s)

LBL = [0]
def label(name):
    LBL[0] += 1
    return f"PISA_{name}_{LBL[0]}_%="


def rsrc(base, lo, hi, off, nv):
    # {address = (hi:lo) + off, stride 0, num_records = nv * RB (nv = None:
    # the whole 64-row block), word 3}
    emit(f"s_add_u32 s{base}, {lo}, s{off}")
    emit(f"s_addc_u32 s{base+1}, {hi}, 0")
    if nv is None:
        emit(f"s_movk_i32 s{base+2}, {64 * RB}")
    else:
        emit(f"s_lshl_b32 s{base+2}, s{nv}, 8")
    emit(f"s_mov_b32 s{base+3}, 0x00020000")


def dma(i, vl):
    # V rows 4 i .. 4 i + 3 of the current item -> LDS tile vl + 1024 i (lane l: +16 l)
    emit(f"s_add_u32 m0, {vl}, {1024 * i}")
    emit(f"s_movk_i32 s{S_SOFF}, {1024 * i}")
    emit("s_nop 0")
    emit(f"buffer_load_dwordx4 %[voff], {SR(S_VRS)}, s{S_SOFF} offen lds")


def kload_lines(kt, ks):
    # packed K: k-step ks of key tile kt (chunks 2 ks, 2 ks + 1 of its 32 rows)
    # is the contiguous 1 KB run at 8192 kt + 1024 ks; lane l reads its 16
    # bytes at 16 l (%[koff])
    off = 1024 * (KS * kt + ks)
    return [f"s_movk_i32 s{S_Y}, {off & ~4095}",
            f"buffer_load_dwordx4 {kreg(kt, ks)}, %[koff], {SR(S_KRS)}, s{S_Y} offen offset:{off & 4095}"]


def kload(kt, ks):
    for ln in kload_lines(kt, ks):
        emit(ln)


def qread(qt, ks, buf):
    emit(f"ds_read_b128 {qbuf(buf)}, %[qa] offset:{(qt * 32 * QP) * 2 + 16 * ks}")


GROUPS = [(kt, h) for kt in range(2) for h in range(2)]


class Op:
    """One scheduled unit: its lines, its kind, the LDS reads it needs, and the
    MFMA (index in the phase) it must follow."""
    def __init__(self, kind, lines, lds_id=None, needs=(), after=-1):
        self.kind, self.lines, self.lds_id, self.needs, self.after = kind, lines, lds_id, tuple(needs), after


class Sched:
    """Merges an MFMA stream with LDS reads (issued a few MFMAs ahead, waits
    computed from the issue order) and other ops (spread evenly, each after the
    MFMA it depends on)."""
    def __init__(self):
        self.lds_seq = {}      # lds id -> issue number
        self.n_lds = 0

    def issue(self, op):
        for ln in op.lines:
            emit(ln)
        if op.lds_id is not None:
            self.lds_seq[op.lds_id] = self.n_lds
            self.n_lds += 1

    def wait_for(self, needs):
        if not needs:
            return
        last = max(self.lds_seq[n] for n in needs)
        after = self.n_lds - 1 - last
        emit(f"s_waitcnt lgkmcnt({min(after, 15)})")

    def run(self, mfmas, lds, others, lds_ahead=8):
        """mfmas: list of Op (needs = LDS ids); lds: Op list in the order their
        consumers appear, each with .after = the MFMA index it must follow
        (register reuse); others: Op list in program order."""
        li = 0
        oi = 0
        n = len(mfmas)
        quota = (len(others) + n - 1) // n if n else 0
        for i, m in enumerate(mfmas):
            # LDS reads needed by the next lds_ahead MFMAs (and allowed now)
            horizon = set()
            for mm in mfmas[i:i + lds_ahead]:
                horizon.update(mm.needs)
            while li < len(lds) and lds[li].after < i and (lds[li].lds_id in horizon or lds[li].lds_id in m.needs):
                self.issue(lds[li])
                li += 1
            assert all(nd in self.lds_seq for nd in m.needs), "LDS read not issued before its MFMA"
            self.wait_for(m.needs)
            self.issue(m)
            k = 0
            while oi < len(others) and k < quota and others[oi].after <= i:
                self.issue(others[oi])
                oi += 1
                k += 1
        while li < len(lds):
            self.issue(lds[li])
            li += 1
        while oi < len(others):
            self.issue(others[oi])
            oi += 1


def phase_a_ops(vl):
    """S^T = K Q^T MFMAs (ks-major), their Q reads, the V DMA of the current item and
    the K loads of the next."""
    mf, lds, oth = [], [], []
    idx = {}
    for ks in range(KS):
        for kt in range(2):
            for qt in range(2):
                src_c = "0" if ks == 0 else sreg(kt, qt)
                b = (ks % 2) * 2 + qt
                idx[(kt, qt, ks)] = len(mf)
                mf.append(Op("mfma", [f"v_mfma_f32_32x32x16_bf16 {sreg(kt, qt)}, {kreg(kt, ks)}, {qbuf(b)}, {src_c}"],
                             needs=[("q", qt, ks)]))
    for ks in range(KS):
        for qt in range(2):
            # buffer (ks % 2) * 2 + qt last read by the MFMAs of k-step ks - 2
            after = max(idx[(kt, qt, ks - 2)] for kt in range(2)) if ks >= 2 else -1
            lds.append(Op("lds", [f"ds_read_b128 {qbuf((ks % 2) * 2 + qt)}, %[qa] offset:{(qt * 32 * QP) * 2 + 32 * ks}"],
                          lds_id=("q", qt, ks), after=after))
    dmas = []
    for i in range(VL):
        dmas.append(Op("vmem", [f"s_add_u32 m0, {vl}, {1024 * i}", f"s_movk_i32 s{S_SOFF}, {1024 * i}", "s_nop 0",
                                f"buffer_load_dwordx4 %[voff], {SR(S_VRS)}, s{S_SOFF} offen lds"]))
    kls = []
    for ks in range(KS):
        for kt in range(2):
            last_reader = max(idx[(kt, qt, ks)] for qt in range(2))
            kls.append(Op("vmem", kload_lines(kt, ks), after=last_reader + 1))
    # DMA first (no constraint), the K loads as their registers free up
    oth = dmas + kls
    return mf, lds, oth


def softmax_max_lines(qt):
    out = []
    a = t(2 + qt)
    v = [se(kt, qt, e) for kt in range(2) for e in range(16)]
    out.append(f"v_max3_f32 {a}, {v[0]}, {v[1]}, {v[2]}")
    for i in range(3, 31, 2):
        out.append(f"v_max3_f32 {a}, {a}, {v[i]}, {v[i+1]}")
    out.append(f"v_max_f32 {a}, {a}, {v[31]}")
    out.append(f"v_mov_b32 {t(6 + qt)}, {a}")
    out.append("s_nop 1")
    out.append(f"v_permlane32_swap_b32 {a}, {t(6 + qt)}")
    out.append("s_nop 2")
    out.append(f"v_max_f32 {a}, {a}, {t(6 + qt)}")
    out.append(f"v_mul_f32 {a}, {a}, %[c2]")
    m2 = f"%[m2{qt}]"
    out.append(f"v_max_f32 %[mx{qt}], %[mx{qt}], {a}")
    out.append(f"v_cmp_eq_f32 vcc, {MINF}, {m2}")
    out.append(f"v_cndmask_b32 {m2}, {m2}, {a}, vcc")
    out.append(f"v_add_f32 {t(6 + qt)}, 0x42800000, {m2}")
    out.append(f"v_cmp_gt_f32 vcc, {a}, {t(6 + qt)}")
    out.append(f"v_cndmask_b32_e64 %[need], %[need], 1, vcc")
    out.append(f"v_cmp_eq_f32 vcc, {MINF}, {m2}")
    out.append(f"v_cndmask_b32_e64 {t(4 + qt)}, {m2}, 0, vcc")
    out.append(f"v_xor_b32 {t(4 + qt)}, 0x80000000, {t(4 + qt)}")
    return out


def softmax_ops():
    """the softmax of the current item as VALU ops; ops writing P of PV group g
    carry after = the index of that group's last MFMA (set by the caller)."""
    ops = [Op("valu", ["s_nop 7", "s_nop 4"])]          # S^T MFMA results -> VALU
    for qt in range(2):
        for ln in softmax_max_lines(qt):
            ops.append(Op("valu", [ln]))
    for gi, (kt, h) in enumerate(GROUPS):
        for qt in range(2):
            nm = t(4 + qt)
            for w in range(4):
                e = 8 * h + 2 * w
                x0, x1 = t(8 + 2 * (w % 2)), t(9 + 2 * (w % 2))
                ops.append(Op("valu", [f"v_fma_f32 {x0}, {se(kt, qt, e)}, %[c2], {nm}"]))
                ops.append(Op("valu", [f"v_fma_f32 {x1}, {se(kt, qt, e + 1)}, %[c2], {nm}"]))
                ops.append(Op("valu", [f"v_exp_f32 {x0}, {x0}"]))
                ops.append(Op("valu", [f"v_exp_f32 {x1}, {x1}", "s_nop 0"]))
                ops.append(Op("valu", [f"v_cvt_pk_bf16_f32 {pw(kt, h, qt, w)}, {x0}, {x1}"], after=("group", gi)))
                ops.append(Op("valu", [f"v_dot2c_f32_bf16 %[l{qt}], 0x3f803f80, {pw(kt, h, qt, w)}"], after=("group", gi)))
    return ops


def pv_ops(trs):
    """PV MFMAs of the previous item (group-major) and their transposed V reads."""
    mf, lds = [], []
    pairs = [(kt, h, dt) for (kt, h) in GROUPS for dt in range(DT)]
    for r, (kt, h, dt) in enumerate(pairs):
        for qt in range(2):
            mf.append(Op("mfma", [f"v_mfma_f32_32x32x16_bf16 {ACC[dt * 2 + qt]}, {vbuf(r % 3)}, {preg(kt, h, qt)}, {ACC[dt * 2 + qt]}"],
                         needs=[("v", r, 0), ("v", r, 1)]))
    for r, (kt, h, dt) in enumerate(pairs):
        r0 = 32 * kt + 16 * h
        after = 2 * (r - 3) + 1 if r >= 3 else -1       # buffer r % 3 last read by pair r - 3
        lds.append(Op("lds", [f"ds_read_b64_tr_b16 {vlo(r % 3)}, {trs[dt]} offset:{r0 * RB}"], lds_id=("v", r, 0), after=after))
        lds.append(Op("lds", [f"ds_read_b64_tr_b16 {vhi(r % 3)}, {trs[dt]} offset:{(r0 + 8) * RB}"], lds_id=("v", r, 1), after=after))
    return mf, lds


def resolve_after(ops, mfma_count_per_group=8):
    for o in ops:
        if isinstance(o.after, tuple):
            o.after = mfma_count_per_group * (o.after[1] + 1) - 1


TR = {0: ["%[tr0_0]", "%[tr0_1]", "%[tr0_2]", "%[tr0_3]"],
      1: ["%[tr1_0]", "%[tr1_1]", "%[tr1_2]", "%[tr1_3]"]}


def mask_block():
    skip = label("nomask")
    emit(f"s_cmp_lt_u32 s{S_NVC}, 64")
    emit(f"s_cbranch_scc0 {skip}")
    emit("s_nop 7")
    emit("s_nop 4")
    emit(f"v_mov_b32 {t(7)}, {MINF}")
    for kt in range(2):
        for e in range(16):
            key = 32 * kt + 8 * (e // 4) + (e % 4)
            emit(f"v_add_u32 {t(6)}, {key}, %[kb4]")
            emit(f"v_cmp_gt_u32 vcc, s{S_NVC}, {t(6)}")
            for qt in range(2):
                emit(f"v_cndmask_b32 {se(kt, qt, e)}, {t(7)}, {se(kt, qt, e)}, vcc")
    emit(f"{skip}:")


def step(par, first):
    vl = "%[vl0]" if par == 0 else "%[vl1]"
    emit(f"; ---- item step, V tile parity {par}{' (first item)' if first else ''}")
    emit("s_waitcnt vmcnt(0) lgkmcnt(0)")      # this item's K, the previous item's V, the next entry
    emit(f"v_readfirstlane_b32 s{S_NOFF}, {t(0)}")
    emit(f"v_readfirstlane_b32 s{S_NNV}, {t(1)}")
    emit("s_nop 1")
    rsrc(S_VRS, "%[vb_lo]", "%[vb_hi]", S_OFF, S_NV)
    rsrc(S_KRS, "%[kb_lo]", "%[kb_hi]", S_NOFF, None)
    emit(f"s_mov_b32 s{S_NVC}, s{S_NV}")
    # prefetch the list entry after next (used by the next step)
    emit(f"s_add_u32 s{S_X}, s{S_N}, 2")
    emit(f"s_sub_u32 s{S_Y}, s{S_NI}, 1")
    emit(f"s_min_u32 s{S_X}, s{S_X}, s{S_Y}")
    emit(f"s_lshl_b32 s{S_X}, s{S_X}, 3")
    emit(f"v_add_u32 {t(0)}, s{S_X}, %[il]")
    sa = Sched()
    sa.issue(Op("lds", [f"ds_read_b64 v[{T}:{T+1}], {t(0)}"], lds_id=("list",)))
    mf, lds, oth = phase_a_ops(vl)
    sa.run(mf, lds, oth)
    mask_block()
    sm = softmax_ops()
    if first:
        for o in sm:
            for ln in o.lines:
                emit(ln)
    else:
        mfb, ldsb = pv_ops(TR[1 - par])
        resolve_after(sm)
        sb = Sched()
        sb.run(mfb, ldsb, sm)
    emit(f"s_mov_b32 s{S_OFF}, s{S_NOFF}")
    emit(f"s_mov_b32 s{S_NV}, s{S_NNV}")
    emit(f"s_add_u32 s{S_N}, s{S_N}, 1")


def final_pv(par):
    mfb, ldsb = pv_ops(TR[par])
    sb = Sched()
    sb.run(mfb, ldsb, [])


def program():
    done, end0, end1, loop = label("done"), label("end0"), label("end1"), label("loop")
    emit(f"s_mov_b32 s{S_M0}, m0")
    emit("s_nop 4")                                # the accumulator was just written by VALU
    emit(f"s_mov_b32 s{S_NI}, %[ni]")
    emit(f"s_mov_b32 s{S_N}, 0")
    emit(f"s_cmp_eq_u32 s{S_NI}, 0")
    emit(f"s_cbranch_scc1 {done}")
    emit(f"ds_read_b64 v[{T}:{T+1}], %[il]")     # item 0: list entry, K loads
    emit("s_waitcnt lgkmcnt(0)")
    emit(f"v_readfirstlane_b32 s{S_OFF}, {t(0)}")
    emit(f"v_readfirstlane_b32 s{S_NV}, {t(1)}")
    emit("s_nop 1")
    rsrc(S_KRS, "%[kb_lo]", "%[kb_hi]", S_OFF, None)
    for kt in range(2):
        for ks in range(KS):
            kload(kt, ks)
    # item 1's entry (clamped) for the first step
    emit(f"s_sub_u32 s{S_Y}, s{S_NI}, 1")
    emit(f"s_min_u32 s{S_X}, s{S_Y}, 1")
    emit(f"s_lshl_b32 s{S_X}, s{S_X}, 3")
    emit(f"v_add_u32 {t(0)}, s{S_X}, %[il]")
    emit(f"ds_read_b64 v[{T}:{T+1}], {t(0)}")
    step(0, True)
    emit(f"{loop}:")
    emit(f"s_cmp_ge_u32 s{S_N}, s{S_NI}")
    emit(f"s_cbranch_scc1 {end1}")                 # the last item's V is in parity 0
    step(1, False)
    emit(f"s_cmp_ge_u32 s{S_N}, s{S_NI}")
    emit(f"s_cbranch_scc1 {end0}")                 # the last item's V is in parity 1
    step(0, False)
    emit(f"s_branch {loop}")
    for lab, par in ((end1, 0), (end0, 1)):
        emit(f"{lab}:")
        emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
        final_pv(par)
        emit(f"s_branch {done}")
    emit(f"{done}:")
    emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
    emit("s_nop 15")
    emit("s_nop 15")                               # last accumulator MFMAs before later reads
    emit(f"s_mov_b32 m0, s{S_M0}")


program()
clob = [f'"v{i}"' for i in range(KREG, 256)] + [f'"s{i}"' for i in SGPRS]
out = ["// Generated by gen_attn_loop.py (do not edit): the D = 128 exact-item loop of the fused PISA forward for gfx950.",
       "#define PISA_ATTN_LOOP_D128_ASM \\"]
out.append(" \\\n".join('    "' + l + '\\n"' for l in L))
out.append("")
out.append("#define PISA_ATTN_LOOP_D128_CLOBBERS " + ", ".join(clob) + ', "vcc", "scc", "memory"')
dst = sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.path.dirname(os.path.abspath(__file__)), "attn_loop_d128.inc")
open(dst, "w").write("\n".join(out) + "\n")
print(len(L), "instructions/labels ->", dst)
