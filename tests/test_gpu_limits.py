"""GPU parity at the largest sizes the C ABI accepts.

K reaches 2^24 (the mat-vec and prefill limit); a prefill tile then spans
128 tokens x 2^24 code bytes, the largest 32-bit buffer offsets the producers
form.  The one-launch decode takes the largest K whose packed token fits one
workgroup's 64 KB of LDS, and the MoE prefill the largest T*K below 2^30.
Only the token rows drawn from synth/ are compared with the oracle; the other
rows are zero, and their outputs must be exactly zero.
"""
import numpy as np
import pytest

import oracle
import synth
from census import tracked
from gpu_helpers import assert_close, assert_exact, host, pack_on_device, poisoned, poisoned_f32, to_dev

pytestmark = pytest.mark.gpu

K_MAX = 1 << 24


@pytest.fixture(scope="module")
def q():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_q8kpack_fp32_amd as q

    oracle.build()
    return tracked(q)


def _weights(q, fmt, g, rows, K):
    if fmt == "q4k":
        w = synth.q4k_weights(g, rows, K)
        return w, to_dev(w), q.Q8K_Q4_K, oracle.Q4_K
    if fmt == "q5k":
        w = synth.q5k_weights(g, rows, K)
        return w, to_dev(w), q.Q8K_Q5_K, oracle.Q5_K
    w = synth.q6k_weights(g, rows, K)
    wd = poisoned(q.q8k_weight_bytes(q.Q8K_Q6_K_RELAID, rows, K))
    q.q8k_bind_q6k(to_dev(w), rows, K, wd)
    return w, wd, q.Q8K_Q6_K_RELAID, oracle.Q6_K


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_matvec_largest_k(q, fmt):
    rows, K = 3, K_MAX
    g = np.random.default_rng(200)
    w, wd, qt, ot = _weights(q, fmt, g, rows, K)
    x = synth.activations(g, 1, K)
    y = poisoned_f32(rows)
    q.qmatvec(qt, wd, rows, K, pack_on_device(q, x), y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(ot, w, rows, K, oqs, od, obs)
    assert_close(host(y), want[0], A[0], f"qmatvec {fmt} K=2^24")


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_one_launch_decode_largest_k(q, fmt):
    """60672 = the largest multiple of 256 whose packed token (codes, scales
    and sums: K * 276/256 bytes) fits 64 KB; one more block is refused."""
    rows, K = 70, 60672
    g = np.random.default_rng(201)
    w, wd, qt, ot = _weights(q, fmt, g, rows, K)
    x = synth.activations(g, 1, K)
    y = poisoned_f32(rows)
    q.qmatvec_f32(qt, wd, rows, K, to_dev(x), 1, y, None)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(ot, w, rows, K, oqs, od, obs)
    assert_close(host(y), want[0], A[0], f"qmatvec_f32 {fmt} K={K}")
    with pytest.raises(q.Q8KError) as ei:
        q.qmatvec_f32(qt, wd, rows, K + 256, to_dev(np.zeros((1, K + 256), np.float32)), 1, y, None)
    assert ei.value.name == "Q8K_ERR_SHAPE"


def _sparse_tokens(T, K, rows_from_synth, g):
    """fp32 [T][K] on the device: zero except the listed rows, which come
    from synth/ (returned on the host too)."""
    import torch

    x = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    host_rows = {}
    for t in rows_from_synth:
        xr = synth.activations(g, 1, K)
        host_rows[t] = xr
        x[t] = to_dev(xr[0])
    return x, host_rows


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_prefill_largest_k_full_tile(q, fmt):
    """128 tokens x K = 2^24: token 127's codes sit 127 * 2^24 bytes into the
    tile, the largest offset a producer forms."""
    rows, K, M = 3, K_MAX, 128
    g = np.random.default_rng(202)
    w, wd, qt, ot = _weights(q, fmt, g, rows, K)
    x, xr = _sparse_tokens(M, K, (0, 127), g)
    xq = poisoned(q.q8k_act_bytes(M, K))
    q.q8k_pack(x, M, K, xq)
    del x
    y = poisoned_f32(M, rows)
    wsb = q.qmatmul_prefill_workspace_bytes(qt, rows, K, M)
    q.qmatmul_prefill(qt, wd, rows, K, xq, M, y, poisoned(wsb) if wsb else None, wsb)
    got = host(y)
    for t, xt in xr.items():
        oqs, od, obs = oracle.q8k_pack(xt)
        want, A = oracle.matvec(ot, w, rows, K, oqs, od, obs)
        assert_close(got[t], want[0], A[0], f"prefill {fmt} K=2^24 token {t}")
    zero = np.ones(M, bool)
    zero[list(xr)] = False
    assert_exact(got[zero], np.zeros((zero.sum(), rows), np.float32), "zero tokens")


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_prefill_largest_k_last_code_bytes(q, fmt):
    """A full 128-token tile at K = 2^24 spans exactly 2^31 code bytes.  Token
    127 is zero except the last 16 values of its last block, so its output
    depends only on the tile's last 16 code bytes: a buffer range one byte
    short would drop the last dword of codes."""
    import torch

    rows, K, M = 3, K_MAX, 128
    g = np.random.default_rng(204)
    w, wd, qt, ot = _weights(q, fmt, g, rows, K)
    tail = np.zeros((1, K), np.float32)
    tail[0, K - 16:] = g.standard_normal(16).astype(np.float32)
    x = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    x[M - 1, K - 16:] = to_dev(tail[0, K - 16:])
    xq = poisoned(q.q8k_act_bytes(M, K))
    q.q8k_pack(x, M, K, xq)
    del x
    y = poisoned_f32(M, rows)
    wsb = q.qmatmul_prefill_workspace_bytes(qt, rows, K, M)
    q.qmatmul_prefill(qt, wd, rows, K, xq, M, y, poisoned(wsb) if wsb else None, wsb)
    got = host(y)
    oqs, od, obs = oracle.q8k_pack(tail)
    want, A = oracle.matvec(ot, w, rows, K, oqs, od, obs)
    assert_close(got[M - 1], want[0], A[0], f"prefill {fmt} K=2^24, token 127's last 16 values")
    assert_exact(got[:M - 1], np.zeros((M - 1, rows), np.float32), "zero tokens")


def test_prefill_moe_largest_tk(q):
    """T * K just below 2^30 (64 tokens, K = 2^24 - 256): the gathered token
    offsets reach 63 * K."""
    E, rows, T, topk = 2, 3, 64, 1
    K = K_MAX - 256
    g = np.random.default_rng(203)
    w = synth.q4k_weights(g, E * rows, K)
    x, xr = _sparse_tokens(T, K, (0, 63), g)
    xq = poisoned(q.q8k_act_bytes(T, K))
    q.q8k_pack(x, T, K, xq)
    del x
    ids = np.zeros((T, topk), np.int32)
    ids[63, 0] = 1
    ids[1::2, 0] = 1
    rw = np.full((T, topk), 0.75, np.float32)
    y = poisoned_f32(T, rows)
    wsb = q.qmatmul_prefill_moe_workspace_bytes(q.Q8K_Q4_K, E, rows, K, T, topk)
    q.qmatmul_prefill_moe(q.Q8K_Q4_K, to_dev(w), E, rows, K, xq, T, to_dev(ids), to_dev(rw), topk, y, poisoned(wsb),
                          wsb)
    got = host(y)
    for t, xt in xr.items():
        oqs, od, obs = oracle.q8k_pack(xt)
        want, A = oracle.moe(oracle.Q4_K, w, E, rows, K, oqs, od, obs, ids[t:t + 1], rw[t:t + 1])
        assert_close(got[t:t + 1], want, A, f"moe prefill K={K} token {t}")
    zero = np.ones(T, bool)
    zero[list(xr)] = False
    assert_exact(got[zero], np.zeros((zero.sum(), rows), np.float32), "zero tokens")
