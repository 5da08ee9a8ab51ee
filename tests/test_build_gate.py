"""The build rejects kernels that spill to scratch: its parser must match the
kernel-resource remarks hipcc prints (file:line:col: remark: ...)."""
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
