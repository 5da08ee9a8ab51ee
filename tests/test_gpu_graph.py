"""HIP graph replay of the whole path gives the eager results, replay after
replay.  The bench times decode steps as graph replays, so this guards that
the captured launches (no memset nodes: every output is fully overwritten by a
kernel) reproduce eager execution exactly.
"""
import os

import numpy as np
import pytest

import synth
from census import tracked
from gpu_helpers import pack_on_device, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_q8kpack_fp32_amd as q

    return tracked(q)


def test_graph_replays_match_eager(q):
    import torch

    dev = torch.device("cuda")
    g = np.random.default_rng(5)
    rows, K, T, E, topk, M = 512, 1024, 4, 4, 2, 70
    w4 = to_dev(synth.q4k_weights(g, E * rows, K))
    w5 = to_dev(synth.q5k_weights(g, rows, K))
    w6g = to_dev(synth.q6k_weights(g, rows, K))
    w6 = torch.empty(q.q8k_weight_bytes(q.Q8K_Q6_K_RELAID, rows, K), dtype=torch.uint8, device=dev)
    q.q8k_bind_q6k(w6g, rows, K, w6)
    x = to_dev(synth.activations(g, M, K))
    ids_h, rw_h = synth.moe_routing(g, T, E, topk)
    ids, rw = to_dev(ids_h), to_dev(rw_h)
    xq = torch.empty(q.q8k_act_bytes(M, K), dtype=torch.uint8, device=dev)
    xq1 = torch.empty(q.q8k_act_bytes(1, K), dtype=torch.uint8, device=dev)
    xqT = torch.empty(q.q8k_act_bytes(T, K), dtype=torch.uint8, device=dev)
    y4 = torch.empty(rows, dtype=torch.float32, device=dev)
    y6 = torch.empty(rows, dtype=torch.float32, device=dev)
    yb = torch.empty(T * rows, dtype=torch.float32, device=dev)
    ym = torch.empty(T * rows, dtype=torch.float32, device=dev)
    yp = torch.empty(M * rows, dtype=torch.float32, device=dev)
    yp5 = torch.empty(M * rows, dtype=torch.float32, device=dev)
    yp6 = torch.empty(M * rows, dtype=torch.float32, device=dev)
    yf4 = torch.empty(rows, dtype=torch.float32, device=dev)
    yf6 = torch.empty(rows, dtype=torch.float32, device=dev)
    xqf = torch.empty(q.q8k_act_bytes(1, K), dtype=torch.uint8, device=dev)
    yb5 = torch.empty(T * rows, dtype=torch.float32, device=dev)
    ypm = torch.empty(T * rows, dtype=torch.float32, device=dev)
    ws_bytes = q.qmatmul_prefill_workspace_bytes(q.Q8K_Q4_K, rows, K, M)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    wsm_bytes = q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q4_K, E, rows, K, T, topk)
    wsm = torch.empty(wsm_bytes, dtype=torch.uint8, device=dev)
    # the prefill from fp32 tokens: its sync words start at zero and every
    # call (each replay) leaves them so
    xqp = torch.empty(q.q8k_act_bytes(M, K), dtype=torch.uint8, device=dev)
    ypf = torch.empty(M * rows, dtype=torch.float32, device=dev)
    ypf6 = torch.empty(M * rows, dtype=torch.float32, device=dev)
    wsf_bytes = q.qmatmul_prefill_f32_workspace_bytes(q.Q8K_Q4_K, rows, K, M)
    wsf = torch.zeros(wsf_bytes, dtype=torch.uint8, device=dev)
    outs = [xq, xq1, xqT, y4, y6, yb, ym, yp, yp5, yp6, yf4, yf6, xqf, yb5, ypm, xqp, ypf, ypf6]

    def path():
        q.q8k_pack(x, M, K, xq)
        q.q8k_pack(x[:1], 1, K, xq1)
        q.q8k_pack(x[:T], T, K, xqT)
        q.qmatvec(q.Q8K_Q4_K, w4, rows, K, xq1, y4)
        q.qmatvec(q.Q8K_Q6_K_RELAID, w6, rows, K, xq1, y6)
        q.qmatvec_batched(q.Q8K_Q4_K, w4, rows, K, xqT, T, yb)
        q.qmatvec_moe(q.Q8K_Q4_K, w4, E, rows, K, xqT, T, ids, rw, topk, ym)
        q.qmatmul_prefill(q.Q8K_Q4_K, w4, rows, K, xq, M, yp, ws, ws_bytes)
        q.qmatmul_prefill(q.Q8K_Q5_K, w5, rows, K, xq, M, yp5, ws, ws_bytes)
        q.qmatmul_prefill(q.Q8K_Q6_K_RELAID, w6, rows, K, xq, M, yp6, ws, ws_bytes)
        q.qmatvec_f32(q.Q8K_Q4_K, w4, rows, K, x[:1], 1, yf4, None)
        q.qmatvec_f32(q.Q8K_Q6_K_RELAID, w6, rows, K, x[:1], 1, yf6, xqf)
        q.qmatvec_batched(q.Q8K_Q5_K, w5, rows, K, xqT, T, yb5)
        q.qmatmul_prefill_moe(q.Q8K_Q4_K, w4, E, rows, K, xqT, T, ids, rw, topk, ypm, wsm, wsm_bytes)
        q.qmatmul_prefill_f32(q.Q8K_Q4_K, w4, rows, K, x, M, xqp, ypf, wsf, wsf_bytes)
        q.qmatmul_prefill_f32(q.Q8K_Q6_K_RELAID, w6, rows, K, x, M, xqp, ypf6, wsf, wsf_bytes)

    path()
    torch.cuda.synchronize()

    def defined(name, o):
        """The bytes a call defines: the three q8_K sections (padding between
        them is not written by any kernel), or the whole fp32 output."""
        if o.dtype != torch.uint8:
            return o.view(torch.uint8)
        tok = {"xq": M, "xq1": 1, "xqT": T, "xqf": 1, "xqp": M}[name]
        total, od, ob = q.q8k_act_layout(tok, K)
        nb = K // 256
        return torch.cat([o[: tok * K], o[od: od + 4 * tok * nb], o[ob: ob + 16 * tok * nb]])

    names = ["xq", "xq1", "xqT", "y4", "y6", "yb", "ym", "yp", "yp5", "yp6", "yf4", "yf6", "xqf", "yb5", "ypm", "xqp",
             "ypf", "ypf6"]
    eager = [defined(n, o).clone() for n, o in zip(names, outs)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    side = pack_on_device(q, synth.activations(g, 2, K))  # eager work between replays
    for rep in range(3):
        for o in outs:
            o.fill_(0x7F if o.dtype == torch.uint8 else float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(names, outs, eager):
            assert torch.equal(defined(name, o), e), f"replay {rep}: {name} differs from eager"
        assert not wsf[:256].any(), f"replay {rep}: sync words not back at zero"
        y_side = torch.empty(rows, dtype=torch.float32, device=dev)
        q.qmatvec(q.Q8K_Q4_K, w4, rows, K, side, y_side)
        torch.cuda.synchronize()


def test_package_imported_before_torch_launches(q):
    """A fresh process that imports the package before torch still launches
    on the device torch's tensors live on (one HIP runtime in the process)."""
    import subprocess
    import sys

    code = ("import quantized_q8kpack_fp32_amd as q, torch, numpy as np\n"
            "x = torch.ones(1, 256, device='cuda')\n"
            "xq = torch.empty(q.q8k_act_bytes(1, 256), dtype=torch.uint8, device='cuda')\n"
            "q.q8k_pack(x, 1, 256, xq)\n"
            "torch.cuda.synchronize()\n"
            "assert int(xq[0].item()) == 127, xq[:4]\n"
            "print('ok')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]
