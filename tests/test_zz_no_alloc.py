"""The allocation-free MoE prefill (qmatmul_prefill_moe_noalloc) against the
entry point it mirrors (qmatmul_prefill_moe with a caller workspace): two
calls in a row on the library's scratch, the second smaller, each bit-equal to
the workspace form and within the tolerance of the oracle; the largest
workload the scratch holds; and the refusal beyond it.
"""
import numpy as np
import pytest

import oracle
import synth
from census import tracked
from gpu_helpers import assert_close, host, pack_on_device, poisoned, poisoned_f32, to_dev

pytestmark = pytest.mark.gpu

_FMT = {"q4k": ("Q8K_Q4_K", oracle.Q4_K, synth.q4k_weights), "q5k": ("Q8K_Q5_K", oracle.Q5_K, synth.q5k_weights),
        "q6k": ("Q8K_Q6_K_RELAID", oracle.Q6_K, synth.q6k_weights)}


@pytest.fixture(scope="module")
def q():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_q8kpack_fp32_amd as q

    oracle.build()
    return tracked(q)


def _case(q, fmt, E, rows, K, T, topk, seed, check_oracle=True):
    qname, ot, gen = _FMT[fmt]
    qt = getattr(q, qname)
    g = np.random.default_rng(seed)
    w = gen(g, E * rows, K)
    if fmt == "q6k":
        wd = poisoned(q.q8k_weight_bytes(q.Q8K_Q6_K_RELAID, E * rows, K))
        q.q8k_bind_q6k(to_dev(w), E * rows, K, wd)
    else:
        wd = to_dev(w)
    x = synth.activations(g, T, K)
    ids, rw = synth.moe_routing(g, T, E, topk)
    xq = pack_on_device(q, x)
    idd, rwd = to_dev(ids.astype(np.int32)), to_dev(rw)
    y = poisoned_f32(T, rows)
    q.qmatmul_prefill_moe_noalloc(qt, wd, E, rows, K, xq, T, idd, rwd, topk, y)
    got = host(y)
    if check_oracle:
        oqs, od, obs = oracle.q8k_pack(x)
        want, A = oracle.moe(ot, w, E, rows, K, oqs, od, obs, ids, rw, nthreads=16)
        assert_close(got, want, A, f"noalloc moe prefill {fmt} E={E} rows={rows} T={T}")
    wsb = q.qmatmul_prefill_moe_workspace_bytes(qt, E, rows, K, T, topk)
    y2 = poisoned_f32(T, rows)
    q.qmatmul_prefill_moe(qt, wd, E, rows, K, xq, T, idd, rwd, topk, y2, poisoned(wsb), wsb)
    assert np.array_equal(got.view(np.uint32), host(y2).view(np.uint32)), "differs from the workspace form"


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_noalloc_two_calls_second_smaller(q, fmt):
    _case(q, fmt, 8, 512, 1024, 200, 2, 301)
    _case(q, fmt, 4, 130, 512, 37, 3, 302)


def test_noalloc_largest_workload(q):
    """8 experts of 14336 x 4096, 512 tokens, top-2: 58.7 MB of workspace."""
    assert q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q4_K, 8, 14336, 4096, 512, 2) <= q.Q8K_NOALLOC_SCRATCH_BYTES
    _case(q, "q4k", 8, 14336, 4096, 512, 2, 303, check_oracle=False)


def test_noalloc_refuses_beyond_scratch(q):
    E, rows, K, T, topk = 8, 14336, 256, 600, 2
    assert q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q4_K, E, rows, K, T, topk) > q.Q8K_NOALLOC_SCRATCH_BYTES
    with pytest.raises(q.Q8KError) as ei:
        q.qmatmul_prefill_moe_noalloc(q.Q8K_Q4_K, 1 << 20, E, rows, K, 1 << 20, T, 1 << 20, 1 << 20, topk, 1 << 20)
    assert ei.value.name == "Q8K_ERR_WORKSPACE" and "scratch" in str(ei.value)
    assert q.q8k_debug_last_launches() == []
