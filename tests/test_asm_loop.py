"""The inline-assembly item loop of the fused forward is generated: the
committed include must be exactly what the generator produces."""

import os
import re
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_taylor_amd", "csrc")


def test_generated_loop_is_current():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "loop.inc")
        subprocess.run([sys.executable, os.path.join(CSRC, "gen_attn_loop.py"), out], check=True,
                       capture_output=True)
        with open(out) as f:
            fresh = f.read()
    with open(os.path.join(CSRC, "attn_loop_d128.inc")) as f:
        committed = f.read()
    assert fresh == committed, "attn_loop_d128.inc is stale: rerun gen_attn_loop.py"


def _expand(kind, text):
    regs = {int(x) for x in re.findall(rf"\b{kind}(\d+)\b", text)}
    for lo, hi in re.findall(rf"\b{kind}\[(\d+):(\d+)\]", text):
        regs.update(range(int(lo), int(hi) + 1))
    return regs


def test_loop_register_plan():
    with open(os.path.join(CSRC, "attn_loop_d128.inc")) as f:
        text = f.read()
    body, clob = text.split("#define PISA_ATTN_LOOP_D128_CLOBBERS")
    body = re.sub(r"%\[\w+\]", "", body)       # operands the compiler allocates
    declared = {k: {int(x) for x in re.findall(rf'"{k}(\d+)"', clob)} for k in "vas"}
    # every register the loop names explicitly is declared clobbered
    for k in "vas":
        named = _expand(k, body)
        assert named <= declared[k], (k, sorted(named - declared[k]))
    # the compiler keeps v0-v55 and a0-a127 (the PV accumulators) for itself
    assert min(declared["v"]) >= 56 and min(declared["a"]) >= 128
    # the loop's instruction set: global memory is read with vector loads
    # (buffer, global) only, never written; LDS is read, and written only with
    # vector LDS writes (the Q^T copy at the end); scalar instructions are ALU
    # and control flow
    ops = set(re.findall(r'^\s*"\s*([a-z_0-9]+)', body, re.M))
    allowed = {
        "buffer_load_dword", "buffer_load_dwordx4", "ds_read_b32", "ds_read_b128", "ds_read_b64", "ds_read_b64_tr_b16",
        "ds_write_b128",
        "global_load_dword", "s_add_u32", "s_addc_u32", "s_and_b32", "s_bitcmp1_b32", "s_branch",
        "s_cbranch_scc0", "s_cbranch_scc1", "s_cmp_eq_u32", "s_cmp_ge_u32", "s_cmp_lt_u32",
        "s_cselect_b32", "s_lshl_b32", "s_lshr_b32", "s_min_u32", "s_mov_b32", "s_movk_i32",
        "s_nop", "s_sub_u32", "s_waitcnt", "v_accvgpr_read_b32", "v_accvgpr_write_b32", "v_add_f32", "v_add_u32",
        "v_and_b32", "v_bfe_u32", "v_cmp_eq_f32", "v_cmp_eq_u32", "v_cmp_gt_f32", "v_cmp_gt_u32",
        "v_cmp_le_u32", "v_cndmask_b32", "v_cndmask_b32_e64", "v_cvt_pk_bf16_f32",
        "v_dot2c_f32_bf16", "v_exp_f32", "v_fma_f32", "v_lshlrev_b32", "v_lshrrev_b32_e64",
        "v_max3_f32", "v_max_f32", "v_mfma_f32_32x32x16_bf16", "v_min_u32", "v_mov_b32",
        "v_mul_f32", "v_permlane32_swap_b32", "v_readfirstlane_b32", "v_sub_f32", "v_subrev_u32",
        "v_xor_b32",
    }
    assert ops and ops <= allowed, sorted(ops - allowed)
