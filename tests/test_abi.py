"""The C ABI library on the CPU: it loads, exports every symbol declared in
include/q8k.h, sizes buffers as documented, and refuses bad arguments by name
before touching the GPU (no kernel is launched here).

Named refusals and the 256-multiple width rule: "One kernel, any device"
(cajeta.dev/xpu/, section 1, checked launches) and "Language models on the
device: the cajeta-llm kernels" (section 3.2); SKaiNET's "Kernel SPI and the
selection algorithm" (decline reasons, block alignment).
"""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def q():
    import quantized_q8kpack_fp32_amd as q

    return q


def header_functions():
    src = open(os.path.join(ROOT, "include", "q8k.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M))


def test_exports_every_declared_symbol(q):
    declared = header_functions()
    assert declared == set(q.EXPORTED), declared ^ set(q.EXPORTED)
    for name in declared:
        assert hasattr(q.lib, name), name


def test_act_layout(q):
    total, od, ob = q.q8k_act_layout(1, 4096)
    assert (od, ob, total) == (4096, 4352, 4608)
    total, od, ob = q.q8k_act_layout(512, 14336)
    assert od == 512 * 14336 and od % 256 == 0
    assert ob == od + 4 * 512 * 56 and ob % 256 == 0
    assert total == ob + 2 * 8 * 512 * 56
    assert q.q8k_act_bytes(3, 1000) == 0 and q.q8k_act_bytes(-1, 256) == 0


def test_weight_bytes(q):
    assert q.q8k_weight_bytes(q.Q8K_Q4_K, 4096, 4096) == 9437184
    assert q.q8k_weight_bytes(q.Q8K_Q6_K_GGUF, 32000, 4096) == 107520000
    assert q.q8k_weight_bytes(q.Q8K_Q5_K, 4096, 4096) == 4096 * 16 * 176
    nblk = 32000 * 16
    assert q.q8k_weight_bytes(q.Q8K_Q6_K_RELAID, 32000, 4096) == ((2 * nblk + 255) // 256) * 256 + 208 * nblk
    assert q.q8k_weight_bytes(9, 1, 256) == 0


A16 = 1 << 20  # an aligned fake device address: never dereferenced (refused first)


def refused(q, status_name, fn, *args):
    with pytest.raises(q.Q8KError) as ei:
        fn(*args)
    assert ei.value.name == status_name, str(ei.value)
    return str(ei.value)


def test_k_must_be_multiple_of_256(q):
    msg = refused(q, "Q8K_ERR_SHAPE", q.qmatvec, q.Q8K_Q4_K, A16, 4, 1000, A16, A16, 0)
    assert "K=1000" in msg and "256" in msg
    refused(q, "Q8K_ERR_SHAPE", q.q8k_pack, A16, 1, 0, A16, 0)
    refused(q, "Q8K_ERR_SHAPE", q.q8k_pack, A16, 1, -256, A16, 0)
    refused(q, "Q8K_ERR_SHAPE", q.qmatmul_prefill, q.Q8K_Q4_K, A16, 8, 300, A16, 4, A16, None, 0, 0)
    refused(q, "Q8K_ERR_SHAPE", q.qmatvec, q.Q8K_Q4_K, A16, 4, (1 << 24) + 256, A16, A16, 0)


def test_negative_sizes(q):
    refused(q, "Q8K_ERR_SHAPE", q.qmatvec, q.Q8K_Q4_K, A16, -1, 256, A16, A16, 0)
    refused(q, "Q8K_ERR_SHAPE", q.q8k_pack, A16, -3, 256, A16, 0)
    refused(q, "Q8K_ERR_SHAPE", q.qmatmul_prefill, q.Q8K_Q4_K, A16, 8, 256, A16, -1, A16, None, 0, 0)


def test_null_and_alignment(q):
    refused(q, "Q8K_ERR_NULL", q.qmatvec, q.Q8K_Q4_K, None, 4, 256, A16, A16, 0)
    refused(q, "Q8K_ERR_NULL", q.q8k_pack, None, 1, 256, A16, 0)
    msg = refused(q, "Q8K_ERR_ALIGN", q.qmatvec, q.Q8K_Q4_K, A16 + 4, 4, 256, A16, A16, 0)
    assert "16-byte" in msg
    refused(q, "Q8K_ERR_ALIGN", q.qmatvec, q.Q8K_Q4_K, A16, 4, 256, A16 + 8, A16, 0)
    refused(q, "Q8K_ERR_ALIGN", q.qmatvec, q.Q8K_Q4_K, A16, 4, 256, A16, A16 + 2, 0)
    refused(q, "Q8K_ERR_ALIGN", q.q8k_bind_q6k, A16 + 1, 4, 256, A16, 0)


def test_qtype_refusals(q):
    msg = refused(q, "Q8K_ERR_QTYPE", q.qmatvec, q.Q8K_Q6_K_GGUF, A16, 4, 256, A16, A16, 0)
    assert "q8k_bind_q6k" in msg
    refused(q, "Q8K_ERR_QTYPE", q.qmatvec, 42, A16, 4, 256, A16, A16, 0)
    msg = refused(q, "Q8K_ERR_QTYPE", q.qmatmul_prefill, q.Q8K_Q6_K_GGUF, A16, 8, 256, A16, 4, A16, None, 0, 0)
    assert "q8k_bind_q6k" in msg
    refused(q, "Q8K_ERR_QTYPE", q.qmatmul_prefill, 42, A16, 8, 256, A16, 4, A16, None, 0, 0)
    # every served format has a prefill tile: empty calls are accepted and enqueue nothing
    for qt in (q.Q8K_Q4_K, q.Q8K_Q5_K, q.Q8K_Q6_K_RELAID):
        q.qmatmul_prefill(qt, A16, 8, 256, A16, 0, A16, None, 0, 0)


def test_fused_decode_arguments(q):
    f = q.qmatvec_f32
    refused(q, "Q8K_ERR_ARG", f, q.Q8K_Q4_K, A16, 4, 256, A16, 0, A16, None, 0)
    refused(q, "Q8K_ERR_ARG", f, q.Q8K_Q4_K, A16, 4, 256, A16, q.Q8K_COLS_MAX + 1, A16, None, 0)
    refused(q, "Q8K_ERR_SHAPE", f, q.Q8K_Q4_K, A16, 4, 1000, A16, 1, A16, None, 0)
    # the packed columns must fit 64 KiB of LDS: ncols * (K + K/256*20) bytes
    msg = refused(q, "Q8K_ERR_SHAPE", f, q.Q8K_Q4_K, A16, 4, 14336, A16, 5, A16, None, 0)
    assert "LDS" in msg and "q8k_pack" in msg
    f(q.Q8K_Q4_K, A16, 0, 14336, A16, 4, A16, None, 0)  # 4 * 15456 bytes fit; rows == 0 enqueues nothing
    refused(q, "Q8K_ERR_ALIGN", f, q.Q8K_Q4_K, A16, 4, 256, A16 + 4, 1, A16, None, 0)
    refused(q, "Q8K_ERR_ALIGN", f, q.Q8K_Q4_K, A16, 4, 256, A16, 1, A16, A16 + 8, 0)
    refused(q, "Q8K_ERR_NULL", f, q.Q8K_Q4_K, A16, 4, 256, None, 1, A16, None, 0)
    refused(q, "Q8K_ERR_QTYPE", f, q.Q8K_Q6_K_GGUF, A16, 4, 256, A16, 1, A16, None, 0)


def test_batched_and_moe_arguments(q):
    refused(q, "Q8K_ERR_ARG", q.qmatvec_batched, q.Q8K_Q4_K, A16, 4, 256, A16, 0, A16, 0)
    refused(q, "Q8K_ERR_ARG", q.qmatvec_batched, q.Q8K_Q4_K, A16, 4, 256, A16, q.Q8K_COLS_MAX + 1, A16, 0)
    refused(q, "Q8K_ERR_ARG", q.qmatvec_moe, q.Q8K_Q4_K, A16, 8, 4, 256, A16, 16, A16, A16, 0, A16, 0)
    refused(q, "Q8K_ERR_ARG", q.qmatvec_moe, q.Q8K_Q4_K, A16, 8, 4, 256, A16, 16, A16, A16, 9, A16, 0)
    refused(q, "Q8K_ERR_ARG", q.qmatvec_moe, q.Q8K_Q4_K, A16, 0, 4, 256, A16, 16, A16, A16, 1, A16, 0)
    refused(q, "Q8K_ERR_ARG", q.qmatvec_moe, q.Q8K_Q4_K, A16, 8, 4, 256, A16, q.Q8K_MOE_MAX_TOKENS + 1,
            A16, A16, 2, A16, 0)
    refused(q, "Q8K_ERR_ARG", q.qmatvec_moe, q.Q8K_Q4_K, A16, 128, 4, 256, A16, 2, A16, A16,
            q.Q8K_MOE_MAX_TOPK + 1, A16, 0)
    refused(q, "Q8K_ERR_NULL", q.qmatvec_moe, q.Q8K_Q4_K, A16, 8, 4, 256, A16, 16, None, A16, 2, A16, 0)


def moe_prefill_ws_bytes(E, rows, T, topk):
    """The documented MoE prefill workspace: fp32 per-pair results [P][rows],
    then (256-aligned) a 16-byte chunk count, a 16-byte entry per possible
    chunk and P int32 pair indices; P pairs over E experts make at most
    P // 128 + min(E, P) chunks of at most 128 pairs."""
    up = lambda b: -(-b // 256) * 256
    P = T * topk
    if P == 0 or rows == 0:
        return 0
    chunks = P // 128 + min(E, P)
    return up(4 * P * rows) + up(16 + 16 * chunks + 4 * P)


def test_moe_prefill_chunk_bound():
    """The chunk bound P // 128 + min(E, P) holds for every split of P pairs
    over E experts (ceil(n / 128) summed over the experts), and is reached;
    brute force over small cases."""
    import itertools

    reached = False
    for E in range(1, 4):
        for P in range(0, 400, 43):
            worst = 0
            for cuts in itertools.combinations_with_replacement(range(P + 1), E - 1):
                b = (0, *cuts, P)
                worst = max(worst, sum(-(-(b[i + 1] - b[i]) // 128) for i in range(E)))
            bound = P // 128 + min(E, P)
            assert worst <= bound, (E, P, worst)
            reached |= worst == bound
    assert reached


def test_prefill_moe_arguments(q):
    f = q.qmatmul_prefill_moe
    # E, topk, qtype, T*K, workspace
    refused(q, "Q8K_ERR_ARG", f, q.Q8K_Q4_K, A16, 0, 4, 256, A16, 16, A16, A16, 1, A16, A16, 1 << 20, 0)
    refused(q, "Q8K_ERR_ARG", f, q.Q8K_Q4_K, A16, 8, 4, 256, A16, 16, A16, A16, 9, A16, A16, 1 << 20, 0)
    refused(q, "Q8K_ERR_ARG", f, q.Q8K_Q4_K, A16, 128, 4, 256, A16, 2, A16, A16, q.Q8K_MOE_MAX_TOPK + 1, A16,
            A16, 1 << 20, 0)
    msg = refused(q, "Q8K_ERR_QTYPE", f, q.Q8K_Q6_K_GGUF, A16, 8, 4, 256, A16, 16, A16, A16, 2, A16, A16, 1 << 20, 0)
    assert "q8k_bind_q6k" in msg
    msg = refused(q, "Q8K_ERR_SHAPE", f, q.Q8K_Q4_K, A16, 8, 4, 16384, A16, 1 << 16, A16, A16, 2, A16, A16,
                  1 << 40, 0)
    assert "2^30" in msg
    need = q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q4_K, 8, 4, 256, 16, 2)
    assert need == moe_prefill_ws_bytes(8, 4, 16, 2) == 1024
    assert q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q5_K, 8, 4, 256, 16, 2) == need
    assert q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q6_K_RELAID, 8, 4, 256, 16, 2) == need
    # 512 tokens, top-2 of 8 experts of 14336 rows: the per-pair results dominate
    assert q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q4_K, 8, 14336, 4096, 512, 2) == \
        moe_prefill_ws_bytes(8, 14336, 512, 2)
    assert q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q4_K, 4096, 8, 256, 3, 64) == moe_prefill_ws_bytes(4096, 8, 3, 64)
    assert q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q4_K, 8, 4, 256, 0, 2) == 0
    assert q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q4_K, 8, 0, 256, 16, 2) == 0
    refused(q, "Q8K_ERR_WORKSPACE", f, q.Q8K_Q4_K, A16, 8, 4, 256, A16, 16, A16, A16, 2, A16, A16, need - 1, 0)
    refused(q, "Q8K_ERR_NULL", f, q.Q8K_Q4_K, A16, 8, 4, 256, A16, 16, None, A16, 2, A16, A16, need, 0)
    assert q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q6_K_GGUF, 8, 4, 256, 16, 2) == 0


def test_prefill_f32_arguments(q):
    """The prefill from fp32 tokens: its workspace is the sync words (one
    256-byte-padded run: an error word, three pad words, two words per token
    tile and K split) followed by qmatmul_prefill's split-K partials."""
    f = q.qmatmul_prefill_f32
    for qt in (q.Q8K_Q4_K, q.Q8K_Q5_K, q.Q8K_Q6_K_RELAID):
        assert q.qmatmul_prefill_f32_workspace_bytes(qt, 4096, 14336, 512) == 256  # 4 tiles, no split
        assert q.qmatmul_prefill_f32_workspace_bytes(qt, 4096, 14336, 32) == \
            256 + q.qmatmul_prefill_workspace_bytes(qt, 4096, 14336, 32) == 256 + 4 * 32 * 4096 * 4
        assert q.qmatmul_prefill_f32_workspace_bytes(qt, 64, 256, 128 * 60) == 512  # 60 tiles: 4 * (4 + 120) bytes
        assert q.qmatmul_prefill_f32_workspace_bytes(qt, 0, 256, 4) == 0
    need = q.qmatmul_prefill_f32_workspace_bytes(q.Q8K_Q4_K, 64, 256, 4)
    refused(q, "Q8K_ERR_WORKSPACE", f, q.Q8K_Q4_K, A16, 64, 256, A16, 4, A16, A16, A16, need - 1, 0)
    refused(q, "Q8K_ERR_NULL", f, q.Q8K_Q4_K, A16, 64, 256, A16, 4, A16, A16, None, need, 0)
    refused(q, "Q8K_ERR_NULL", f, q.Q8K_Q4_K, A16, 64, 256, None, 4, A16, A16, A16, need, 0)
    refused(q, "Q8K_ERR_ALIGN", f, q.Q8K_Q4_K, A16, 64, 256, A16 + 4, 4, A16, A16, A16, need, 0)
    refused(q, "Q8K_ERR_ALIGN", f, q.Q8K_Q4_K, A16, 64, 256, A16, 4, A16 + 8, A16, A16, need, 0)
    refused(q, "Q8K_ERR_SHAPE", f, q.Q8K_Q4_K, A16, 64, 300, A16, 4, A16, A16, A16, need, 0)
    refused(q, "Q8K_ERR_QTYPE", f, q.Q8K_Q6_K_GGUF, A16, 64, 256, A16, 4, A16, A16, A16, need, 0)
    # more row tiles than compute units (no device here: the library assumes 256)
    msg = refused(q, "Q8K_ERR_SHAPE", f, q.Q8K_Q4_K, A16, 64 * 256 + 1, 256, A16, 4, A16, A16, A16, 1 << 20, 0)
    assert "q8k_pack + qmatmul_prefill" in msg
    assert q.q8k_debug_last_launches() == []
    f(q.Q8K_Q4_K, A16, 0, 256, A16, 4, A16, A16, None, 0, 0)  # nothing to do
    f(q.Q8K_Q4_K, A16, 64, 256, A16, 0, A16, A16, None, 0, 0)


def test_empty_inputs_enqueue_nothing(q):
    # zero rows / tokens are valid and return before any launch
    q.qmatvec(q.Q8K_Q4_K, A16, 0, 256, A16, A16, 0)
    q.qmatvec_f32(q.Q8K_Q5_K, A16, 0, 256, A16, 2, A16, A16, 0)
    q.q8k_pack(A16, 0, 256, A16, 0)
    q.qmatvec_moe(q.Q8K_Q4_K, A16, 8, 4, 256, A16, 0, A16, A16, 2, A16, 0)
    q.qmatmul_prefill(q.Q8K_Q4_K, A16, 8, 256, A16, 0, A16, None, 0, 0)
    q.qmatmul_prefill_moe(q.Q8K_Q4_K, A16, 8, 4, 256, A16, 0, A16, A16, 2, A16, None, 0, 0)
    q.q8k_bind_q6k(A16, 0, 256, A16, 0)


def test_status_strings(q):
    assert q.q8k_status_str(0) == "Q8K_OK"
    assert q.q8k_status_str(7) == "Q8K_ERR_LAUNCH"
    assert q.q8k_status_str(99) == "Q8K_ERR_UNKNOWN"


def test_refused_call_records_no_launch(q):
    """A refusal enqueues nothing: the launch record of the call is empty."""
    refused(q, "Q8K_ERR_SHAPE", q.qmatvec, q.Q8K_Q4_K, A16, 4, 1000, A16, A16, 0)
    assert q.q8k_debug_last_launches() == []
    refused(q, "Q8K_ERR_QTYPE", q.q8k_debug_moe_subblock_sums, q.Q8K_Q6_K_GGUF, A16, 2, 4, 256, A16, 1, A16, A16, 1,
            A16, A16, 0)
    assert q.q8k_debug_last_launches() == []


def test_census_reads_the_kernel_table(q):
    """The census maps launch records to kernels through the library's symbol
    table: it must find the kernels of every family."""
    import census

    names = {census.short(n) for n in census.kernel_names(q).values()}
    for k in ("pack_kernel", "bind_q6k_kernel", "matvec_q4k_kernel<1, 2, false, false>",
              "matvec_q6k_kernel<1, false, false>", "matvec_f32_q4k_kernel<1, 2, false>",
              "moe_mfma_q4k_kernel<false, false>", "prefill_regw_q4k_kernel<false, false, false>",
              "prefill_q4k_kernel<2, false, false>", "prefill_regw_q4k_kernel<false, false, true>",
              "prefill_q4k_kernel<1, false, true>", "moe_group_kernel", "moe_combine_kernel<4>"):
        assert k in names, k
    assert not any(n.startswith("prefill_q4k_kernel<0") for n in names), "the Q4_K prefill runs the register tile"
