"""The build rejects kernels that spill to scratch (its parser must match the
kernel-resource remarks hipcc prints, file:line:col: remark: ...), and device
assembly in which a register loaded by inline assembly is written by anything
else or stored from another register after its explicit wait."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("q8k_build", os.path.join(ROOT, "quantized_q8kpack_fp32_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


LOG = """\
csrc/moe.hip:159:1: remark: Function Name: _ZN3q8k10moe_kernelILb0EEEvPKh [-Rpass-analysis=kernel-resource-usage]
csrc/moe.hip:159:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
csrc/moe.hip:159:1: remark:     ScratchSize [bytes/lane]: 376 [-Rpass-analysis=kernel-resource-usage]
csrc/moe.hip:201:1: remark: Function Name: _ZN3q8k10moe_kernelILb1EEEvPKh [-Rpass-analysis=kernel-resource-usage]
csrc/moe.hip:201:1: remark:     VGPRs: 111 [-Rpass-analysis=kernel-resource-usage]
csrc/moe.hip:201:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_spilling_kernel_is_named():
    b = _build_module()
    bad = b._check_scratch(LOG, "moe.hip")
    assert bad == ["moe.hip: void q8k::moe_kernel<false>(unsigned char const*): 376 bytes/lane of scratch"]


def test_only_named_test_kernels_may_spill():
    """The exemption names test-support instantiations only: the product
    kernel of the same template still fails the gate."""
    b = _build_module()
    log = LOG.replace("_ZN3q8k10moe_kernelILb0EEEvPKh",
                      "_ZN3q8k12_GLOBAL__N_123prefill_regw_q4k_kernelILb0ELb1ELb0EEEvPKhliPKaPKfPKsllPfPKiPK15HIP_vector_"
                      "typeIiLj4EESC_iPi")
    assert b._check_scratch(log, "prefill_regw.hip") == []
    log = LOG.replace("_ZN3q8k10moe_kernelILb0EEEvPKh",
                      "_ZN3q8k12_GLOBAL__N_123prefill_regw_q4k_kernelILb0ELb0ELb0EEEvPKhliPKaPKfPKsllPfPKiPK15HIP_vector_"
                      "typeIiLj4EESC_iPi")
    assert len(b._check_scratch(log, "prefill_regw.hip")) == 1


def test_clean_log_passes():
    b = _build_module()
    clean = "\n".join(l for l in LOG.splitlines() if "Lb0" not in l and "376" not in l and "256" not in l)
    assert b._check_scratch(clean, "moe.hip") == []


# Device assembly shaped like the mixture-of-experts walk: two inline-assembly
# loads, an explicit wait naming them, and the LDS stores of the loaded data.
ASM_GOOD = """\
_ZN3q8k4walkEv:                         ; @_ZN3q8k4walkEv
; %bb.0:
	;;#ASMSTART
	buffer_load_dwordx4 v[110:113], v154, s[44:47], 0 offen
	;;#ASMEND
	;;#ASMSTART
	buffer_load_dwordx4 v[114:117], v156, s[44:47], 0 offen
	;;#ASMEND
	;;#ASMSTART
	buffer_load_dwordx4 v146, s[12:15], 0 offen lds
	;;#ASMEND
	v_add_u32_e32 v2, 16, v3
	;;#ASMSTART
	s_waitcnt vmcnt(5)
	;;#ASMEND
	;;#ASMSTART
	s_waitcnt lgkmcnt(0)
	;;#ASMEND
	ds_write_b128 v166, v[110:113] offset:384
	ds_write_b128 v189, v[114:117] offset:384
	v_mfma_i32_32x32x32_i8 v[54:69], v[6:9], v[10:13], 0
	s_endpgm
"""


def test_inline_loads_kept_in_place_pass():
    b = _build_module()
    assert b._check_asm_loads(ASM_GOOD, "moe_mfma.hip") == []


def test_copy_of_an_inflight_register_is_refused():
    """The register allocator moved a loaded value before the wait: the stores
    then read registers no load wrote, and the load's registers are rewritten."""
    b = _build_module()
    bad = ASM_GOOD.replace("	v_add_u32_e32 v2, 16, v3\n",
                           "	v_mov_b64_e32 v[130:131], v[110:111]\n	v_mov_b64_e32 v[110:111], v[20:21]\n")
    bad = bad.replace("ds_write_b128 v166, v[110:113]", "ds_write_b128 v166, v[130:133]")
    problems = b._check_asm_loads(bad, "moe_mfma.hip")
    assert len(problems) == 2
    assert "v110 is written by 'v_mov_b64_e32 v[110:111], v[20:21]'" in problems[0]
    assert "ds_write_b128 v166, v[130:133]" in problems[1]


def test_lds_copies_and_other_functions_are_not_loads():
    """A buffer-unit copy into LDS writes no register, and a function without
    inline-assembly loads is not checked."""
    b = _build_module()
    asm = ASM_GOOD.replace("v_add_u32_e32 v2, 16, v3", "v_add_u32_e32 v146, 16, v3")
    assert b._check_asm_loads(asm, "moe_mfma.hip") == []
    other = "_ZN3q8k5otherEv:\n\tv_mov_b32_e32 v110, 0\n\ts_endpgm\n"
    assert b._check_asm_loads(ASM_GOOD + other, "moe_mfma.hip") == []


def test_compiler_use_of_m0_is_refused():
    """M0 set inside inline assembly (the LDS copies) is fine; an M0 use the
    compiler emitted itself is named."""
    b = _build_module()
    ok = "_ZN3q8k4copyEv:\n\t;;#ASMSTART\n\ts_mov_b32 m0, s4\n\ts_nop 0\n\tbuffer_load_dword v1, s[0:3], 0 offen lds\n\t;;#ASMEND\n\ts_endpgm\n"
    assert b._check_m0(ok, "prefill_regw.hip") == []
    bad = ok.replace("\ts_endpgm\n", "\ts_mov_b32 m0, -1\n\tds_read_b32 v2, v3\n\ts_endpgm\n")
    problems = b._check_m0(bad, "prefill_regw.hip")
    assert len(problems) == 1 and "s_mov_b32 m0, -1" in problems[0]
