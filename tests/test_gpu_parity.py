"""GPU parity: every entry point of the C ABI against the CPU oracle.

Inputs are seeded and synthetic (synth/), outputs are poisoned with 0xFF before
every call, integer results (q8_K bytes, int32 sub-block sums, relaid weight
bytes) must match bit-exactly and fp32 outputs must satisfy
|err| <= 1e-5 * sum|terms| + 1e-6 against the oracle's fp64 result.

Method: "Language models on the device: the cajeta-llm kernels"
(cajeta.dev/xpu/kernels-llm/), sections 1 (q8_K, K-quants, Q6_K split), 2.1
(decode mat-vec), 2.2 (batched), 2.3 (prefill tiles), 2.4 (MoE decode).
"""
import os

import numpy as np
import pytest

import oracle
import synth
from census import tracked
from gpu_helpers import (assert_close, assert_exact, host, pack_on_device, poisoned, poisoned_f32, poisoned_i32,
                         split_act, to_dev)

pytestmark = pytest.mark.gpu

NTH = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def q():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_q8kpack_fp32_amd as q

    oracle.build()
    return tracked(q)


def q4k(seed, rows, K):
    return synth.q4k_weights(np.random.default_rng(seed), rows, K)


def acts(seed, T, K):
    return synth.activations(np.random.default_rng(seed + 7919), T, K)


# ================================================================== a1 pack
def special_blocks(K):
    """Blocks that exercise the quantiser's corners (one per 256 values)."""
    nb = K // 256
    g = np.random.default_rng(99)
    x = g.standard_normal((nb, 256)).astype(np.float32)
    kinds = [
        lambda v: v,                                   # N(0,1)
        lambda v: np.zeros_like(v),                    # all zero -> d = 0
        lambda v: np.round(v * 40) / 2 + 0.0 * v,     # many exact halves
        lambda v: v * np.float32(1e-39),               # subnormal inputs
        lambda v: v * np.float32(1e30),                # huge inputs
        lambda v: np.where(np.arange(256) == 17, np.float32(-3.0), 0).astype(np.float32),  # one value
        lambda v: np.full_like(v, 0.5),                # constant block
        lambda v: v * np.float32(1e-38) / np.abs(v).max(),  # 127/amax overflows
    ]
    for b in range(nb):
        x[b] = kinds[b % len(kinds)](x[b])
    # exact ties: amax = 127 makes the inverse scale 1
    if nb > 2:
        x[2, 0] = 127.0
    return x.reshape(1, K)


@pytest.mark.parametrize("T,K", [(1, 256), (1, 1024), (3, 4096), (17, 512), (16, 4096), (512, 14336)])
def test_pack_bit_exact(q, T, K):
    x = acts(T * 31 + K, T, K)
    xq = pack_on_device(q, x)
    qs, d, bs = split_act(q, host(xq), T, K)
    oqs, od, obs = oracle.q8k_pack(x)
    assert_exact(qs, oqs, "codes")
    assert_exact(d, od, "scales")
    assert_exact(bs, obs, "sums")


@pytest.mark.parametrize("K", [2048, 4096])
def test_pack_special_blocks_bit_exact(q, K):
    x = special_blocks(K)
    xq = pack_on_device(q, x)
    qs, d, bs = split_act(q, host(xq), 1, K)
    oqs, od, obs = oracle.q8k_pack(x)
    assert_exact(qs, oqs, "codes")
    assert_exact(d, od, "scales")
    assert_exact(bs, obs, "sums")


# ================================================================== a9 wave reduction
def test_wave_reduction_closed_form(q):
    """The wave reduction every mat-vec ends with, on the closed form the pages
    print for their reduce helpers: thread t of 256 holds t, each wave's sum is
    4096 w + 2016 and the four add to 32640 (exact in fp32).  A dropped or
    doubled lane, or a wrong DPP row step, changes a sum."""
    out = poisoned_f32(5)
    q.q8k_debug_wave_sums(out)
    assert_exact(host(out), np.array([2016, 6112, 10208, 14304, 32640], np.float32), "wave sums")


# ================================================================== a3 Q4_K decode
@pytest.mark.parametrize("rows,K,seed", [(256, 1024, 0), (4096, 4096, 1), (37, 256, 5), (13, 768, 6),
                                         (70, 1280, 7), (9, 14336, 8)])
def test_q4k_subblock_sums_bit_exact(q, rows, K, seed):
    """qmatvec's own kernel, with its sums flag: int32 sub-block sums equal the
    oracle's bit for bit, and its y equals qmatvec's bit for bit."""
    w = q4k(seed, rows, K)
    x = acts(seed, 1, K)
    xq = pack_on_device(q, x)
    S = poisoned_i32(rows, K // 32)
    y = poisoned_f32(rows)
    q.q8k_debug_subblock_sums(q.Q8K_Q4_K, to_dev(w), rows, K, xq, y, S)
    oqs, od, obs = oracle.q8k_pack(x)
    assert_exact(host(S), oracle.subblock_sums(oracle.Q4_K, w, rows, K, oqs[0]), "S")
    want, A = oracle.matvec(oracle.Q4_K, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want[0], A[0], "y of the sums kernel")
    y1 = poisoned_f32(rows)
    q.qmatvec(q.Q8K_Q4_K, to_dev(w), rows, K, xq, y1)
    assert np.array_equal(host(y1).view(np.uint32), host(y).view(np.uint32))


@pytest.mark.parametrize("rows,K,seed", [(256, 1024, 0), (4096, 4096, 1), (37, 256, 5), (13, 768, 6),
                                         (70, 1280, 7), (9, 14336, 8), (1, 256, 9)])
def test_q4k_matvec(q, rows, K, seed):
    w = q4k(seed, rows, K)
    x = acts(seed, 1, K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(rows)
    q.qmatvec(q.Q8K_Q4_K, to_dev(w), rows, K, xq, y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(oracle.Q4_K, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want[0], A[0], f"q4k {rows}x{K}")


def test_q4k_matvec_extreme_scales(q):
    """Subnormal fp16 dmin, zero d, the largest fp16 scales and zero blocks."""
    rows, K = 64, 1024
    w = q4k(21, rows, K).reshape(-1, 144).copy()
    f16 = lambda v: np.array([v], np.float16).view(np.uint8)
    w[0::4, 0:2] = f16(0.0)
    w[1::4, 2:4] = f16(3e-7)          # subnormal fp16
    w[2::4, 0:2] = f16(60000.0)
    w[3::4, 2:4] = f16(60000.0)
    w = w.reshape(-1)
    x = special_blocks(K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(rows)
    q.qmatvec(q.Q8K_Q4_K, to_dev(w), rows, K, xq, y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(oracle.Q4_K, w, rows, K, oqs, od, obs)
    assert_close(host(y), want[0], A[0], "q4k extreme")


# ================================================================== Q5_K decode (NEXT row)
def q5k(seed, rows, K):
    return synth.q5k_weights(np.random.default_rng(seed), rows, K)


@pytest.mark.parametrize("rows,K,seed", [(256, 1024, 50), (4096, 4096, 51), (37, 256, 52), (13, 768, 53),
                                         (9, 14336, 54)])
def test_q5k_subblock_sums_bit_exact(q, rows, K, seed):
    w = q5k(seed, rows, K)
    x = acts(seed, 1, K)
    xq = pack_on_device(q, x)
    S = poisoned_i32(rows, K // 32)
    y = poisoned_f32(rows)
    q.q8k_debug_subblock_sums(q.Q8K_Q5_K, to_dev(w), rows, K, xq, y, S)
    oqs, od, obs = oracle.q8k_pack(x)
    assert_exact(host(S), oracle.subblock_sums(oracle.Q5_K, w, rows, K, oqs[0]), "S")
    want, A = oracle.matvec(oracle.Q5_K, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want[0], A[0], "y of the sums kernel")
    y1 = poisoned_f32(rows)
    q.qmatvec(q.Q8K_Q5_K, to_dev(w), rows, K, xq, y1)
    assert np.array_equal(host(y1).view(np.uint32), host(y).view(np.uint32))


@pytest.mark.parametrize("rows,K,seed", [(256, 1024, 50), (4096, 4096, 51), (37, 256, 52), (13, 768, 53),
                                         (70, 1280, 55), (9, 14336, 54), (1, 256, 56)])
def test_q5k_matvec(q, rows, K, seed):
    w = q5k(seed, rows, K)
    x = acts(seed, 1, K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(rows)
    q.qmatvec(q.Q8K_Q5_K, to_dev(w), rows, K, xq, y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(oracle.Q5_K, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want[0], A[0], f"q5k {rows}x{K}")


def test_q5k_matvec_extreme_scales(q):
    """Subnormal fp16 dmin, zero d, the largest fp16 scales and zero blocks."""
    rows, K = 64, 1024
    w = q5k(57, rows, K).reshape(-1, 176).copy()
    f16 = lambda v: np.array([v], np.float16).view(np.uint8)
    w[0::4, 0:2] = f16(0.0)
    w[1::4, 2:4] = f16(3e-7)          # subnormal fp16
    w[2::4, 0:2] = f16(60000.0)
    w[3::4, 2:4] = f16(60000.0)
    w = w.reshape(-1)
    x = special_blocks(K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(rows)
    q.qmatvec(q.Q8K_Q5_K, to_dev(w), rows, K, xq, y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(oracle.Q5_K, w, rows, K, oqs, od, obs)
    assert_close(host(y), want[0], A[0], "q5k extreme")


def test_q5k_without_fifth_bits_matches_q4k_kernel(q):
    """A Q5_K weight with every qh byte zero runs the same integer sums and
    epilogue as the Q4_K kernel on the same fields: bit-identical outputs."""
    rows, K = 512, 2048
    nb = K // 256
    w4 = q4k(58, rows, K).reshape(rows * nb, 144)
    w5 = np.zeros((rows * nb, 176), np.uint8)
    w5[:, 0:16] = w4[:, 0:16]
    w5[:, 48:176] = w4[:, 16:144]
    xq = pack_on_device(q, acts(58, 1, K))
    y4 = poisoned_f32(rows)
    y5 = poisoned_f32(rows)
    q.qmatvec(q.Q8K_Q4_K, to_dev(w4.reshape(-1)), rows, K, xq, y4)
    q.qmatvec(q.Q8K_Q5_K, to_dev(w5.reshape(-1)), rows, K, xq, y5)
    assert np.array_equal(host(y4).view(np.uint32), host(y5).view(np.uint32))


# ================================================================== a2 bind + a4 Q6_K decode
def q6k_bound(q, seed, rows, K):
    w = synth.q6k_weights(np.random.default_rng(seed), rows, K)
    wr = poisoned(q.q8k_weight_bytes(q.Q8K_Q6_K_RELAID, rows, K))
    q.q8k_bind_q6k(to_dev(w), rows, K, wr)
    return w, wr


@pytest.mark.parametrize("rows,K", [(3, 256), (32000, 4096), (5, 768)])
def test_q6k_bind_bit_exact(q, rows, K):
    w, wr = q6k_bound(q, 2, rows, K)
    nblk = rows * K // 256
    got = host(wr)
    prefix, bodies = oracle.q6k_relayout(w, nblk)
    pad = ((2 * nblk + 255) // 256) * 256
    assert_exact(got[: 2 * nblk].view(np.uint16), prefix, "prefix")
    assert_exact(got[pad: pad + 208 * nblk], bodies, "bodies")


@pytest.mark.parametrize("rows,K,seed", [(32000, 4096, 2), (37, 256, 11), (100, 1280, 12), (7, 14336, 13)])
def test_q6k_subblock_sums_bit_exact(q, rows, K, seed):
    """qmatvec's Q6_K kernel as it ships (4 lanes per block, the (h, lh) lane
    map, the row walk), with its sums flag."""
    w, wr = q6k_bound(q, seed, rows, K)
    x = acts(seed, 1, K)
    xq = pack_on_device(q, x)
    S = poisoned_i32(rows, K // 16)
    y = poisoned_f32(rows)
    q.q8k_debug_subblock_sums(q.Q8K_Q6_K_RELAID, wr, rows, K, xq, y, S)
    oqs, od, obs = oracle.q8k_pack(x)
    assert_exact(host(S), oracle.subblock_sums(oracle.Q6_K, w, rows, K, oqs[0]), "S")
    want, A = oracle.matvec(oracle.Q6_K, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want[0], A[0], "y of the sums kernel")
    y1 = poisoned_f32(rows)
    q.qmatvec(q.Q8K_Q6_K_RELAID, wr, rows, K, xq, y1)
    assert np.array_equal(host(y1).view(np.uint32), host(y).view(np.uint32))


@pytest.mark.parametrize("rows,K,seed", [(32000, 4096, 2), (37, 256, 11), (100, 1280, 12), (7, 14336, 13)])
def test_q6k_matvec(q, rows, K, seed):
    w, wr = q6k_bound(q, seed, rows, K)
    x = acts(seed, 1, K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(rows)
    q.qmatvec(q.Q8K_Q6_K_RELAID, wr, rows, K, xq, y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(oracle.Q6_K, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want[0], A[0], f"q6k {rows}x{K}")


# ================================================================== a5 batched
@pytest.mark.parametrize("ncols", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_batched(q, ncols, fmt):
    rows, K = (4096, 4096) if fmt != "q6k" else (1000, 4096)
    if fmt == "q4k":
        w = q4k(1, rows, K)
        wd, qt, ot = to_dev(w), q.Q8K_Q4_K, oracle.Q4_K
    elif fmt == "q5k":
        w = q5k(59, rows, K)
        wd, qt, ot = to_dev(w), q.Q8K_Q5_K, oracle.Q5_K
    else:
        w, wd = q6k_bound(q, 2, rows, K)
        qt, ot = q.Q8K_Q6_K_RELAID, oracle.Q6_K
    x = acts(40 + ncols, ncols, K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(ncols, rows)
    q.qmatvec_batched(qt, wd, rows, K, xq, ncols, y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(ot, w, rows, K, oqs, od, obs, nthreads=NTH)
    got = host(y)
    assert_close(got, want, A, f"batched {fmt} ncols={ncols}")
    # each column is the single-column mat-vec of that token, bit for bit
    for c in range(ncols):
        xq1 = pack_on_device(q, x[c:c + 1])
        y1 = poisoned_f32(rows)
        q.qmatvec(qt, wd, rows, K, xq1, y1)
        assert np.array_equal(host(y1).view(np.uint32), got[c].view(np.uint32)), f"column {c}"


@pytest.mark.parametrize("fmt,ncols", [("q4k", 4), ("q4k", 5), ("q5k", 2), ("q5k", 8)])
def test_batched_long_rows(q, fmt, ncols):
    """K = 14336: up to four columns are staged in LDS, five or more read the
    packed token from global memory (they exceed one workgroup's LDS); both
    match the oracle and the single-column mat-vec bit for bit."""
    rows, K = 300, 14336
    w = (q4k if fmt == "q4k" else q5k)(60 + ncols, rows, K)
    qt, ot = (q.Q8K_Q4_K, oracle.Q4_K) if fmt == "q4k" else (q.Q8K_Q5_K, oracle.Q5_K)
    wd = to_dev(w)
    x = acts(61 + ncols, ncols, K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(ncols, rows)
    q.qmatvec_batched(qt, wd, rows, K, xq, ncols, y)
    got = host(y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(ot, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(got, want, A, f"batched {fmt} K={K} ncols={ncols}")
    for c in (0, ncols - 1):
        y1 = poisoned_f32(rows)
        q.qmatvec(qt, wd, rows, K, pack_on_device(q, x[c:c + 1]), y1)
        assert np.array_equal(host(y1).view(np.uint32), got[c].view(np.uint32)), f"column {c}"


# ================================================================== fused pack + decode (NEXT row)
def fused_weights(q, fmt, seed, rows, K):
    """-> (host GGUF bytes, device weight, C qtype, oracle qtype)."""
    qname, ot, gen = _PF_FMT[fmt]
    w = gen(np.random.default_rng(seed), rows, K)
    return w, pf_weights(q, fmt, w, rows, K), getattr(q, qname), ot


@pytest.mark.parametrize("fmt,rows,K,ncols,seed", [
    ("q4k", 4096, 4096, 1, 80), ("q4k", 37, 256, 1, 81), ("q4k", 130, 14336, 1, 82), ("q4k", 1000, 4096, 4, 83),
    ("q4k", 70, 1280, 8, 84), ("q4k", 9, 14336, 4, 85),
    ("q5k", 4096, 4096, 1, 86), ("q5k", 13, 768, 3, 87), ("q5k", 70, 1280, 8, 88),
    ("q6k", 1000, 4096, 1, 89), ("q6k", 37, 256, 2, 90), ("q6k", 130, 14336, 1, 91), ("q6k", 70, 4608, 8, 92),
])
def test_fused_decode_equals_pack_then_matvec(q, fmt, rows, K, ncols, seed):
    """One fused launch from fp32 activations gives q8k_pack + qmatvec_batched
    bit for bit, its packed copy equals q8k_pack's bytes, and both match the
    oracle within the tolerance."""
    w, wd, qt, ot = fused_weights(q, fmt, seed, rows, K)
    x = acts(seed, ncols, K)
    if ncols > 1:
        x[1] = special_blocks(K)[0]
    y = poisoned_f32(ncols, rows)
    xq_f = poisoned(q.q8k_act_bytes(ncols, K))
    q.qmatvec_f32(qt, wd, rows, K, to_dev(x), ncols, y, xq_f)
    xq = pack_on_device(q, x)
    y2 = poisoned_f32(ncols, rows)
    q.qmatvec_batched(qt, wd, rows, K, xq, ncols, y2)
    got = host(y)
    assert np.array_equal(got.view(np.uint32), host(y2).view(np.uint32))
    assert np.array_equal(host(xq_f), host(xq))
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(ot, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(got, want, A, f"fused {fmt} {rows}x{K} ncols={ncols}")


def test_fused_decode_without_packed_copy(q):
    """xq_out = NULL: the same outputs, nothing else written."""
    rows, K = 300, 2048
    w, wd, qt, _ = fused_weights(q, "q4k", 93, rows, K)
    x = to_dev(acts(93, 2, K))
    y1 = poisoned_f32(2, rows)
    y2 = poisoned_f32(2, rows)
    xq = poisoned(q.q8k_act_bytes(2, K))
    q.qmatvec_f32(qt, wd, rows, K, x, 2, y1, xq)
    q.qmatvec_f32(qt, wd, rows, K, x, 2, y2, None)
    assert np.array_equal(host(y1).view(np.uint32), host(y2).view(np.uint32))


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_fused_qkv_one_launch_equals_three(q, fmt):
    """q, k and v weights concatenated row-wise are one weight: one fused
    launch gives each part's outputs bit for bit as three separate launches."""
    K = 4096
    parts = [(4096, 94), (1024, 95), (1024, 96)]
    ws = [_PF_FMT[fmt][2](np.random.default_rng(sd), r, K) for r, sd in parts]
    rows = sum(r for r, _ in parts)
    wd = pf_weights(q, fmt, np.concatenate(ws), rows, K)
    qt = getattr(q, _PF_FMT[fmt][0])
    x = to_dev(acts(94, 1, K))
    y = poisoned_f32(rows)
    q.qmatvec_f32(qt, wd, rows, K, x, 1, y, None)
    got = host(y)
    r0 = 0
    for (r, _), wp in zip(parts, ws):
        yp = poisoned_f32(r)
        q.qmatvec_f32(qt, pf_weights(q, fmt, wp, r, K), r, K, x, 1, yp, None)
        assert np.array_equal(got[r0:r0 + r].view(np.uint32), host(yp).view(np.uint32))
        r0 += r


# ================================================================== a6 MoE decode
def moe_case(q, fmt, E, rows, K, T, topk, seed, ids=None):
    g = np.random.default_rng(seed)
    if fmt == "q4k":
        w = synth.q4k_weights(g, E * rows, K)
        wd, qt, ot = to_dev(w), q.Q8K_Q4_K, oracle.Q4_K
    elif fmt == "q5k":
        w = synth.q5k_weights(g, E * rows, K)
        wd, qt, ot = to_dev(w), q.Q8K_Q5_K, oracle.Q5_K
    else:
        w = synth.q6k_weights(g, E * rows, K)
        wd = poisoned(q.q8k_weight_bytes(q.Q8K_Q6_K_RELAID, E * rows, K))
        q.q8k_bind_q6k(to_dev(w), E * rows, K, wd)
        qt, ot = q.Q8K_Q6_K_RELAID, oracle.Q6_K
    x = synth.activations(g, T, K)
    r_ids, rw = synth.moe_routing(g, T, E, topk)
    if ids is None:
        ids = r_ids
    xq = pack_on_device(q, x)
    y = poisoned_f32(T, rows)
    q.qmatvec_moe(qt, wd, E, rows, K, xq, T, to_dev(ids.astype(np.int32)), to_dev(rw), topk, y)
    oqs, od, obs = oracle.q8k_pack(x)
    return host(y), w, ot, oqs, od, obs, ids, rw


@pytest.mark.parametrize("fmt,E,rows,K,T,topk,seed", [
    ("q4k", 8, 14336, 4096, 16, 2, 3),     # the MoE decode layer shape
    ("q4k", 4, 100, 512, 5, 3, 31),
    ("q4k", 8, 37, 1280, 1, 2, 32),
    ("q4k", 16, 64, 256, 200, 4, 33),      # many tokens: several token slots per lane
    ("q4k", 2, 40, 88064, 3, 2, 38),       # one packed token per LDS stage: a slab per token
    ("q4k", 2, 40, 131072, 3, 2, 39),      # a packed token beyond the LDS stage: one lane per row
    ("q6k", 8, 300, 1024, 16, 2, 34),
    ("q6k", 8, 14336, 4096, 16, 2, 46),    # the MoE decode layer shape in relaid Q6_K
    ("q6k", 2, 40, 83968, 3, 2, 47),       # Q6_K: one packed token per LDS stage, a slab per token
    ("q6k", 2, 40, 88064, 3, 2, 48),       # Q6_K: a packed token beyond the stage: the per-chunk kernel
    ("q6k", 1, 29, 256, 3, 1, 49),         # Q6_K: one expert, one slot, fewer rows than a tile
    ("q6k", 64, 40, 512, 5, 64, 50),       # Q6_K: topk at its limit, two tokens per slab
    ("q6k", 4, 8200, 256, 40, 4, 51),      # Q6_K: two row tiles per workgroup, two token slabs
    ("q5k", 8, 14336, 4096, 16, 2, 35),    # the MoE decode layer shape in Q5_K
    ("q5k", 4, 100, 512, 5, 3, 36),
    ("q5k", 16, 64, 256, 200, 4, 37),
    ("q4k", 64, 40, 512, 5, 64, 42),       # topk at its limit: two tokens per slab, every expert hit
    ("q5k", 1, 29, 256, 3, 1, 43),         # one expert, one slot, fewer rows than a tile
    ("q5k", 2, 40, 88064, 3, 2, 40),       # one packed token per LDS stage: a slab per token
    ("q5k", 2, 40, 131072, 3, 2, 41),      # a packed token beyond the LDS stage: one lane per row
    # more row tiles than compute units (two per workgroup) and two slabs of tokens (32, then 8)
    ("q4k", 4, 8200, 256, 40, 4, 44),
    ("q5k", 4, 8200, 256, 40, 4, 45),
])
def test_moe(q, fmt, E, rows, K, T, topk, seed):
    got, w, ot, oqs, od, obs, ids, rw = moe_case(q, fmt, E, rows, K, T, topk, seed)
    want, A = oracle.moe(ot, w, E, rows, K, oqs, od, obs, ids, rw, nthreads=NTH)
    assert_close(got, want, A, f"moe {fmt} E={E} rows={rows} T={T}")


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
def test_moe_crowded_expert_and_bad_ids(q, fmt):
    """20 tokens all choose experts 0 and 1 (more pairs than one group holds);
    an id outside [0, E) selects nothing."""
    E, rows, K, T, topk = 4, 50, 512, 20, 2
    ids = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    ids[3, 1] = 7      # out of range: dropped
    ids[5, 0] = -1     # out of range: dropped
    got, w, ot, oqs, od, obs, ids, rw = moe_case(q, fmt, E, rows, K, T, topk, 77, ids=ids)
    ok = (ids >= 0) & (ids < E)
    want, A = oracle.moe(ot, w, E, rows, K, oqs, od, obs, np.where(ok, ids, 0), np.where(ok, rw, 0).astype(np.float32))
    assert_close(got, want, A, f"moe crowded {fmt}")


# ================================================================== MoE prefill (NEXT row)
_PF_FMT = {"q4k": ("Q8K_Q4_K", oracle.Q4_K, synth.q4k_weights),
           "q5k": ("Q8K_Q5_K", oracle.Q5_K, synth.q5k_weights),
           "q6k": ("Q8K_Q6_K_RELAID", oracle.Q6_K, synth.q6k_weights)}


def pf_weights(q, fmt, w, nrows, K):
    """Host GGUF blocks -> the device weight the prefill takes (Q6_K: bound by q8k_bind_q6k)."""
    if fmt != "q6k":
        return to_dev(w)
    wd = poisoned(q.q8k_weight_bytes(q.Q8K_Q6_K_RELAID, nrows, K))
    q.q8k_bind_q6k(to_dev(w), nrows, K, wd)
    return wd


def moe_prefill_case(q, E, rows, K, T, topk, seed, ids=None, fmt="q4k"):
    qname, _, gen = _PF_FMT[fmt]
    qt = getattr(q, qname)
    g = np.random.default_rng(seed)
    w = gen(g, E * rows, K)
    x = synth.activations(g, T, K)
    r_ids, rw = synth.moe_routing(g, T, E, topk)
    if ids is None:
        ids = r_ids
    xq = pack_on_device(q, x)
    y = poisoned_f32(T, rows)
    wsb = q.qmatmul_prefill_moe_workspace_bytes(qt, E, rows, K, T, topk)
    ws = poisoned(wsb)
    q.qmatmul_prefill_moe(qt, pf_weights(q, fmt, w, E * rows, K), E, rows, K, xq, T, to_dev(ids.astype(np.int32)),
                          to_dev(rw), topk, y, ws, wsb)
    oqs, od, obs = oracle.q8k_pack(x)
    return host(y), w, oqs, od, obs, ids, rw


@pytest.mark.parametrize("fmt,E,rows,K,T,topk,seed", [
    ("q4k", 8, 512, 4096, 512, 2, 60),     # ~128 pairs per expert: one or two chunks each
    ("q4k", 4, 130, 768, 37, 3, 61),       # ragged row tile, a few pairs per expert
    ("q4k", 16, 64, 256, 200, 4, 62),      # many experts
    ("q4k", 2, 96, 512, 1, 1, 63),         # one token
    ("q4k", 300, 64, 256, 40, 8, 66),      # more experts than pairs: one-pair chunks
    ("q4k", 2500, 8, 256, 64, 4, 73),      # more experts than grouping threads: several per thread
    ("q5k", 8, 512, 4096, 512, 2, 67),
    ("q5k", 4, 130, 768, 37, 3, 68),
    ("q5k", 2, 96, 512, 1, 1, 69),
    ("q6k", 8, 512, 4096, 512, 2, 74),
    ("q6k", 4, 130, 768, 37, 3, 75),
    ("q6k", 2, 96, 512, 1, 1, 76),
])
def test_prefill_moe(q, fmt, E, rows, K, T, topk, seed):
    got, w, oqs, od, obs, ids, rw = moe_prefill_case(q, E, rows, K, T, topk, seed, fmt=fmt)
    want, A = oracle.moe(_PF_FMT[fmt][1], w, E, rows, K, oqs, od, obs, ids, rw, nthreads=NTH)
    assert_close(got, want, A, f"moe prefill {fmt} E={E} rows={rows} T={T}")


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_prefill_moe_crowded_expert_and_bad_ids(q, fmt):
    """300 tokens all choose expert 0 first (three chunks, the last ragged);
    ids outside [0, E) select nothing."""
    E, rows, K, T, topk = 4, 100, 512, 300, 2
    g = np.random.default_rng(64)
    ids = np.stack([np.zeros(T, np.int32), g.integers(1, E, T).astype(np.int32)], axis=1)
    ids[7, 1] = 9
    ids[11, 0] = -2
    got, w, oqs, od, obs, ids, rw = moe_prefill_case(q, E, rows, K, T, topk, 64, ids=ids, fmt=fmt)
    ok = (ids >= 0) & (ids < E)
    want, A = oracle.moe(_PF_FMT[fmt][1], w, E, rows, K, oqs, od, obs, np.where(ok, ids, 0),
                         np.where(ok, rw, 0).astype(np.float32), nthreads=NTH)
    assert_close(got, want, A, f"moe prefill crowded {fmt}")


def test_prefill_moe_all_ids_out_of_range(q):
    """No pair selects an expert: no chunk is made and y is all zeros."""
    E, rows, K, T, topk = 4, 70, 256, 9, 2
    ids = np.full((T, topk), 5, np.int32)
    ids[0, 0] = -1
    got, *_ = moe_prefill_case(q, E, rows, K, T, topk, 70, ids=ids)
    assert_exact(got, np.zeros((T, rows), np.float32), "no pair selects an expert")


def test_prefill_moe_rows_equal_decode_moe(q):
    """The prefill form and the decode form compute the same y (within the
    tolerance: their fp32 sums run in different orders)."""
    E, rows, K, T, topk = 8, 256, 1024, 16, 2
    got, w, oqs, od, obs, ids, rw = moe_prefill_case(q, E, rows, K, T, topk, 65)
    g = np.random.default_rng(65)  # the same draws as moe_prefill_case
    _ = synth.q4k_weights(g, E * rows, K)
    x = synth.activations(g, T, K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(T, rows)
    q.qmatvec_moe(q.Q8K_Q4_K, to_dev(w), E, rows, K, xq, T, to_dev(ids.astype(np.int32)), to_dev(rw), topk, y)
    want, A = oracle.moe(oracle.Q4_K, w, E, rows, K, oqs, od, obs, ids, rw)
    assert_close(host(y), want, A, "decode moe")
    assert_close(got, want, A, "prefill moe")


# ================================================================== a7 prefill (+ Q5_K)
def run_prefill(q, fmt, w, rows, K, x):
    M = x.shape[0]
    qt = getattr(q, _PF_FMT[fmt][0])
    xq = pack_on_device(q, x)
    y = poisoned_f32(M, rows)
    ws_bytes = q.qmatmul_prefill_workspace_bytes(qt, rows, K, M)
    ws = poisoned(ws_bytes) if ws_bytes else None
    q.qmatmul_prefill(qt, pf_weights(q, fmt, w, rows, K), rows, K, xq, M, y, ws, ws_bytes)
    return host(y)


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_prefill_output_four_byte_aligned(q, fmt):
    """y one float past a 16-byte boundary, with enough tiles that K is not
    split (the tiles store y themselves): their 16-byte result stores fall
    back to 4-byte stores.  Every output against the oracle (the last token
    tile ragged, 44 tokens), and the floats on either side of y keep their
    poison."""
    M, rows, K = 300, 5508, 256  # 3 x 87 = 261 tiles: no split
    w = _PF_FMT[fmt][2](np.random.default_rng(96), rows, K)
    x = acts(96, M, K)
    qt = getattr(q, _PF_FMT[fmt][0])
    assert q.qmatmul_prefill_workspace_bytes(qt, rows, K, M) == 0
    buf = poisoned_f32(M * rows + 2)
    y = buf[1:1 + M * rows]
    assert y.data_ptr() % 16 == 4
    q.qmatmul_prefill(qt, pf_weights(q, fmt, w, rows, K), rows, K, pack_on_device(q, x), M, y, None, 0)
    b = host(buf)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(_PF_FMT[fmt][1], w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(b[1:1 + M * rows].reshape(M, rows), want, A, f"prefill {fmt} into a 4-byte aligned y")
    assert b[:1].view(np.uint32)[0] == 0xFFFFFFFF and b[-1:].view(np.uint32)[0] == 0xFFFFFFFF


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,rows,K,seed", [(1, 64, 256, 41), (17, 100, 512, 42), (64, 64, 256, 43),
                                           (127, 256, 1024, 44), (200, 130, 768, 45), (65, 4096, 256, 46)])
def test_prefill_full(q, fmt, M, rows, K, seed):
    w = _PF_FMT[fmt][2](np.random.default_rng(seed), rows, K)
    x = acts(seed, M, K)
    got = run_prefill(q, fmt, w, rows, K, x)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(_PF_FMT[fmt][1], w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(got, want, A, f"prefill {fmt} M={M} N={rows} K={K}")


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_prefill_down_projection_full(q, fmt):
    """The 512-token x 4096-row x 14336 prefill: all 2,097,152 outputs against
    the oracle."""
    M, rows, K = 512, 4096, 14336
    w = _PF_FMT[fmt][2](np.random.default_rng(4), rows, K)
    x = acts(4, M, K)
    got = run_prefill(q, fmt, w, rows, K, x)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(_PF_FMT[fmt][1], w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(got, want, A, f"prefill {fmt} 512x4096x14336")


# ================================================================== integer sums of the shipped tiles
@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,rows,K,seed", [(130, 130, 768, 140), (200, 70, 1024, 141), (129, 65, 256, 142),
                                           (1, 64, 512, 143)])
def test_prefill_block_sums_bit_exact(q, fmt, M, rows, K, seed):
    """qmatmul_prefill's own tile with its sums flag: every block's integer
    sum I_b = sum_j sc_j S_j (the value the tile folds into y) equals the
    oracle's bit for bit, and y equals qmatmul_prefill's bit for bit."""
    w = _PF_FMT[fmt][2](np.random.default_rng(seed), rows, K)
    x = acts(seed, M, K)
    qt = getattr(q, _PF_FMT[fmt][0])
    wd = pf_weights(q, fmt, w, rows, K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(M, rows)
    I = poisoned_i32(M, rows, K // 256)
    q.q8k_debug_prefill_block_sums(qt, wd, rows, K, xq, M, y, I)
    oqs, od, obs = oracle.q8k_pack(x)
    assert_exact(host(I), oracle.block_sums(_PF_FMT[fmt][1], w, rows, K, oqs), f"I {fmt}")
    want, A = oracle.matvec(_PF_FMT[fmt][1], w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want, A, f"y of the sums tile {fmt}")
    y1 = poisoned_f32(M, rows)
    q.qmatmul_prefill(qt, wd, rows, K, xq, M, y1, None, 0)
    assert np.array_equal(host(y1).view(np.uint32), host(y).view(np.uint32))


@pytest.mark.parametrize("fmt,E,rows,K,T,topk,seed", [
    ("q4k", 4, 100, 512, 5, 3, 150), ("q4k", 8, 300, 1024, 16, 2, 151), ("q4k", 2, 40, 256, 20, 2, 152),
    ("q5k", 4, 100, 512, 5, 3, 153), ("q5k", 8, 300, 1024, 16, 2, 154),
    ("q6k", 4, 100, 512, 5, 3, 155), ("q6k", 8, 300, 1024, 16, 2, 156), ("q6k", 2, 40, 256, 20, 2, 157),
])
def test_moe_subblock_sums_bit_exact(q, fmt, E, rows, K, T, topk, seed):
    """qmatvec_moe's matrix-core kernel with its sums flag: each (token, slot)
    pair's sub-block sums S_j against its expert equal the oracle's bit for
    bit (more than 8 pairs per expert in the 20-token case: several groups);
    an out-of-range id's entries stay unwritten; its y equals qmatvec_moe's
    bit for bit."""
    g = np.random.default_rng(seed)
    gen, qt, ot = {"q4k": (synth.q4k_weights, q.Q8K_Q4_K, oracle.Q4_K),
                   "q5k": (synth.q5k_weights, q.Q8K_Q5_K, oracle.Q5_K),
                   "q6k": (synth.q6k_weights, q.Q8K_Q6_K_RELAID, oracle.Q6_K)}[fmt]
    w = gen(g, E * rows, K)
    x = synth.activations(g, T, K)
    ids, rw = synth.moe_routing(g, T, E, topk)
    ids = ids.astype(np.int32)
    ids[1, topk - 1] = E + 3  # selects nothing
    xq = pack_on_device(q, x)
    y = poisoned_f32(T, rows)
    S = poisoned_i32(T * topk, rows, K // (16 if fmt == "q6k" else 32))  # Q6_K: 16-value sub-blocks
    wd = pf_weights(q, fmt, w, E * rows, K)
    q.q8k_debug_moe_subblock_sums(qt, wd, E, rows, K, xq, T, to_dev(ids), to_dev(rw), topk, y, S)
    got = host(S)
    oqs, od, obs = oracle.q8k_pack(x)
    per = w.size // E
    want = np.full_like(got, -1)  # poisoned entries read as -1
    for t in range(T):
        for k in range(topk):
            e = int(ids[t, k])
            if 0 <= e < E:
                want[t * topk + k] = oracle.subblock_sums(ot, w[e * per:(e + 1) * per], rows, K, oqs[t])
    assert_exact(got, want, f"moe S {fmt}")
    ok = ids < E
    wy, A = oracle.moe(ot, w, E, rows, K, oqs, od, obs, np.where(ok, ids, 0), np.where(ok, rw, 0).astype(np.float32),
                       nthreads=NTH)
    assert_close(host(y), wy, A, f"moe y of the sums kernel {fmt}")
    y1 = poisoned_f32(T, rows)
    q.qmatvec_moe(qt, wd, E, rows, K, xq, T, to_dev(ids), to_dev(rw), topk, y1)
    assert np.array_equal(host(y1).view(np.uint32), host(y).view(np.uint32)), f"moe y {fmt}: sums flag changed y"


# ================================================================== every column count of every route
_STAGE_K = 1280    # every batched width 2..8 fits one workgroup's LDS: the staged kernel
_GLOBAL_K = 65536  # no batched width 2..8 fits: the kernel reading packed columns from global memory


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("ncols", range(1, 9))
@pytest.mark.parametrize("K", [_STAGE_K, _GLOBAL_K])
def test_batched_every_width(q, fmt, ncols, K):
    rows = 33
    w, wd, qt, ot = fused_weights(q, fmt, 160 + ncols, rows, K)
    x = acts(161 + ncols, ncols, K)
    xq = pack_on_device(q, x)
    y = poisoned_f32(ncols, rows)
    q.qmatvec_batched(qt, wd, rows, K, xq, ncols, y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(ot, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want, A, f"batched {fmt} ncols={ncols} K={K}")


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("ncols", range(1, 9))
def test_fused_every_width(q, fmt, ncols):
    rows, K = 70, 1024
    w, wd, qt, ot = fused_weights(q, fmt, 170 + ncols, rows, K)
    x = acts(171 + ncols, ncols, K)
    y = poisoned_f32(ncols, rows)
    q.qmatvec_f32(qt, wd, rows, K, to_dev(x), ncols, y, None)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(ot, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want, A, f"fused {fmt} ncols={ncols}")


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,rows,K,splits", [(32, 4096, 14336, 4), (128, 4096, 14336, 4), (77, 130, 4096, 2),
                                             (5, 64, 14336, 7), (1, 70, 4096, 2)])
def test_prefill_split_k(q, fmt, M, rows, K, splits):
    """Problems whose tiles do not fill the device split K across workgroups;
    the fixup adds the partials in split order.  All outputs against the
    oracle (ragged M and rows; 2, 4 and 7 splits)."""
    w = _PF_FMT[fmt][2](np.random.default_rng(180 + M), rows, K)
    x = acts(181 + M, M, K)
    qt = getattr(q, _PF_FMT[fmt][0])
    wsb = q.qmatmul_prefill_workspace_bytes(qt, rows, K, M)
    assert wsb == splits * M * rows * 4, (wsb, splits)
    got = run_prefill(q, fmt, w, rows, K, x)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(_PF_FMT[fmt][1], w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(got, want, A, f"split-K prefill {fmt} M={M} N={rows} K={K}")


def test_prefill_split_k_refuses_short_workspace(q):
    rows, K, M = 4096, 14336, 32
    wsb = q.qmatmul_prefill_workspace_bytes(q.Q8K_Q4_K, rows, K, M)
    assert wsb > 0
    with pytest.raises(q.Q8KError) as ei:
        q.qmatmul_prefill(q.Q8K_Q4_K, 1 << 20, rows, K, 1 << 20, M, 1 << 20, 1 << 20, wsb - 4)
    assert ei.value.name == "Q8K_ERR_WORKSPACE"


def test_prefill_q5k_largest_fields(q):
    """Q5_K blocks at the top of every field (scales and mins 63, quants 31)
    against tokens at +-127: the per-block integer sums reach their largest
    magnitude, and every plane of the split scale is at its maximum."""
    from gguf_pack import pack_q5k_block

    rows, K, M = 64, 2048, 130
    nb = K // 256
    g = np.random.default_rng(71)
    blocks = []
    for r in range(rows * nb):
        kind = r % 4
        sc = np.full(8, 63) if kind < 2 else g.integers(0, 64, 8)
        mn = np.full(8, 63) if kind in (0, 2) else g.integers(0, 64, 8)
        qv = np.full(256, 31) if kind == 0 else g.integers(0, 32, 256)
        blocks.append(pack_q5k_block(float(g.uniform(1e-3, 4e-3)), float(g.uniform(0, 8e-3)), sc, mn, qv))
    w = np.concatenate(blocks)
    x = np.where(g.random((M, K)) < 0.5, -1.0, 1.0).astype(np.float32) * 3.0
    x[: M // 2] = np.abs(x[: M // 2])  # the first half: every value +3, so codes at +127
    got = run_prefill(q, "q5k", w, rows, K, x)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(oracle.Q5_K, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(got, want, A, "prefill q5k largest fields")


def test_prefill_q6k_extreme_scales_and_quants(q):
    """Q6_K blocks at the corners of the value weight sc * (q - 32): scales
    -128 and 127 against quants 0 and 63 (w = 4096, -4064, -4032, 3937),
    zero scales, and tokens at +-127, so both digit planes reach their ends."""
    from gguf_pack import pack_q6k_block

    rows, K, M = 96, 1024, 130
    nb = K // 256
    g = np.random.default_rng(77)
    corners = [(-128, 0), (-128, 63), (127, 0), (127, 63)]
    blocks = []
    for r in range(rows * nb):
        kind = r % 5
        if kind < 4:
            sc, qq = corners[kind]
            scv = np.full(16, sc)
            qv = np.full(256, qq)
            qv[::7] = g.integers(0, 64, qv[::7].shape)
        else:
            scv = np.where(g.random(16) < 0.3, 0, g.integers(-128, 128, 16))
            qv = g.integers(0, 64, 256)
        blocks.append(pack_q6k_block(float(g.uniform(1e-4, 1e-3)), scv, qv))
    w = np.concatenate(blocks)
    x = np.where(g.random((M, K)) < 0.5, -3.0, 3.0).astype(np.float32)
    x[: M // 2] = 3.0
    got = run_prefill(q, "q6k", w, rows, K, x)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(oracle.Q6_K, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(got, want, A, "prefill q6k extremes")


def test_prefill_q6k_matches_batched_decode(q):
    """The Q6_K prefill and eight-column batched decode of the same relaid
    weight and tokens agree within the tolerance (integer sums are exact in
    both; only the fp32 block sums run in different orders)."""
    rows, K, M = 200, 2048, 8
    w = synth.q6k_weights(np.random.default_rng(78), rows, K)
    x = acts(78, M, K)
    got = run_prefill(q, "q6k", w, rows, K, x)
    wd = pf_weights(q, "q6k", w, rows, K)
    xq = pack_on_device(q, x)
    yb = poisoned_f32(M, rows)
    q.qmatvec_batched(q.Q8K_Q6_K_RELAID, wd, rows, K, xq, M, yb)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(oracle.Q6_K, w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(yb), want, A, "batched q6k")
    assert_close(got, want, A, "prefill q6k")


def test_prefill_q5k_without_fifth_bits_matches_q4k(q):
    """A Q5_K weight with every qh byte zero is the Q4_K matrix on the same
    fields: the Q5_K prefill (whose fifth-bit plane then adds exact zeros)
    and the Q4_K prefill (a different tile) both match the Q4_K oracle."""
    rows, K, M = 130, 1024, 140
    nb = K // 256
    w4 = q4k(72, rows, K).reshape(rows * nb, 144)
    w5 = np.zeros((rows * nb, 176), np.uint8)
    w5[:, 0:16] = w4[:, 0:16]
    w5[:, 48:176] = w4[:, 16:144]
    x = acts(72, M, K)
    y4 = run_prefill(q, "q4k", w4.reshape(-1), rows, K, x)
    y5 = run_prefill(q, "q5k", w5.reshape(-1), rows, K, x)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(oracle.Q4_K, w4.reshape(-1), rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(y4, want, A, "q4k prefill")
    assert_close(y5, want, A, "q5k prefill without fifth bits")


# ================================================================== fused pack + prefill (NEXT row)
def run_prefill_f32(q, fmt, wd, rows, K, x, ws=None):
    """qmatmul_prefill_f32 on host fp32 tokens -> (y, q8_K bytes, workspace).
    A fresh workspace is zeroed (its sync words must start at zero)."""
    import torch

    M = x.shape[0]
    qt = getattr(q, _PF_FMT[fmt][0])
    xq = poisoned(q.q8k_act_bytes(M, K))
    y = poisoned_f32(M, rows)
    wsb = q.qmatmul_prefill_f32_workspace_bytes(qt, rows, K, M)
    if ws is None:
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    q.qmatmul_prefill_f32(qt, wd, rows, K, to_dev(x), M, xq, y, ws, wsb)
    return y, xq, ws


def sync_words(q, fmt, rows, K, M, ws):
    """The workspace's sync words (error word first) as int32."""
    qt = getattr(q, _PF_FMT[fmt][0])
    n = q.qmatmul_prefill_f32_workspace_bytes(qt, rows, K, M) - q.qmatmul_prefill_workspace_bytes(qt, rows, K, M)
    return host(ws[:n]).view(np.int32)


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,rows,K,seed", [(1, 64, 256, 300), (77, 130, 2048, 301), (200, 130, 768, 302),
                                           (129, 65, 512, 303), (32, 4096, 14336, 304), (5, 64, 14336, 305)])
def test_prefill_f32(q, fmt, M, rows, K, seed):
    """The prefill from fp32 tokens, packed inside the launch: every output
    against the oracle, the q8_K bytes it writes against the oracle's pack,
    and the sync words back at zero (ragged tiles; split-K at 32 x 4096 x
    14336 and 5 x 64 x 14336)."""
    w = _PF_FMT[fmt][2](np.random.default_rng(seed), rows, K)
    x = acts(seed, M, K)
    y, xq, ws = run_prefill_f32(q, fmt, pf_weights(q, fmt, w, rows, K), rows, K, x)
    oqs, od, obs = oracle.q8k_pack(x)
    qs, d, bs = split_act(q, host(xq), M, K)
    assert_exact(qs, oqs, "codes")
    assert_exact(d, od, "scales")
    assert_exact(bs, obs, "sums")
    want, A = oracle.matvec(_PF_FMT[fmt][1], w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want, A, f"fused prefill {fmt} M={M} N={rows} K={K}")
    assert not sync_words(q, fmt, rows, K, M, ws).any()


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_prefill_f32_down_projection_full(q, fmt):
    """The 512-token x 4096-row x 14336 prefill from fp32 tokens: all
    2,097,152 outputs against the oracle, and bit for bit the result of
    q8k_pack followed by qmatmul_prefill (xq byte for byte q8k_pack's)."""
    M, rows, K = 512, 4096, 14336
    w = _PF_FMT[fmt][2](np.random.default_rng(4), rows, K)
    x = acts(4, M, K)
    wd = pf_weights(q, fmt, w, rows, K)
    y, xq, ws = run_prefill_f32(q, fmt, wd, rows, K, x)
    got = host(y)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(_PF_FMT[fmt][1], w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(got, want, A, f"fused prefill {fmt} 512x4096x14336")
    assert not sync_words(q, fmt, rows, K, M, ws).any()
    xq2 = pack_on_device(q, x)
    y2 = poisoned_f32(M, rows)
    q.qmatmul_prefill(getattr(q, _PF_FMT[fmt][0]), wd, rows, K, xq2, M, y2, None, 0)
    assert np.array_equal(got.view(np.uint32), host(y2).view(np.uint32)), "differs from pack + prefill"
    total, od_, ob_ = q.q8k_act_layout(M, K)
    a, b = host(xq), host(xq2)
    for lo, hi in ((0, M * K), (od_, od_ + 4 * M * (K // 256)), (ob_, ob_ + 16 * M * (K // 256))):
        assert np.array_equal(a[lo:hi], b[lo:hi]), "q8_K bytes differ from q8k_pack's"


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("M,rows,K,seed", [(1000, 4096, 1024, 320), (256, 16384, 256, 321)])
def test_prefill_f32_more_workgroups_than_compute_units(q, fmt, M, rows, K, seed):
    """Grids beyond one workgroup per compute unit: 8 token tiles x 64 row
    tiles (512 workgroups, groups start as earlier ones finish), and row tiles
    as many as the device's compute units (each group fills the device)."""
    w = _PF_FMT[fmt][2](np.random.default_rng(seed), rows, K)
    x = acts(seed, M, K)
    y, xq, ws = run_prefill_f32(q, fmt, pf_weights(q, fmt, w, rows, K), rows, K, x)
    oqs, od, obs = oracle.q8k_pack(x)
    want, A = oracle.matvec(_PF_FMT[fmt][1], w, rows, K, oqs, od, obs, nthreads=NTH)
    assert_close(host(y), want, A, f"fused prefill {fmt} M={M} N={rows} K={K}")
    assert not sync_words(q, fmt, rows, K, M, ws).any()


def test_prefill_f32_calls_share_a_workspace(q):
    """Stream-ordered calls of different shapes on one workspace: each leaves
    the sync words at zero for the next, and each result matches the oracle."""
    import torch

    cases = [(200, 130, 768, 310), (32, 4096, 14336, 311), (1, 64, 256, 312), (200, 130, 768, 313)]
    wsb = max(q.qmatmul_prefill_f32_workspace_bytes(q.Q8K_Q4_K, r, K, M) for M, r, K, _ in cases)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    runs = []
    for M, rows, K, seed in cases:  # enqueued back to back, no synchronisation
        w = q4k(seed, rows, K)
        x = acts(seed, M, K)
        y, _, _ = run_prefill_f32(q, "q4k", to_dev(w), rows, K, x, ws)
        runs.append((w, x, rows, K, y))
    for w, x, rows, K, y in runs:
        oqs, od, obs = oracle.q8k_pack(x)
        want, A = oracle.matvec(oracle.Q4_K, w, rows, K, oqs, od, obs, nthreads=NTH)
        assert_close(host(y), want, A, f"shared workspace M={x.shape[0]} N={rows} K={K}")
    assert not host(ws[:256]).view(np.int32).any()


def test_prefill_f32_refuses_rows_beyond_the_device(q):
    """The row tiles of a token tile wait for each other, so more of them than
    the device has compute units is refused before anything is enqueued."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows, K, M = 64 * cus + 1, 256, 4
    with pytest.raises(q.Q8KError) as ei:
        q.qmatmul_prefill_f32(q.Q8K_Q4_K, 1 << 20, rows, K, 1 << 20, M, 1 << 20, 1 << 20, 1 << 20, 1 << 30)
    assert ei.value.name == "Q8K_ERR_SHAPE"
    assert q.q8k_debug_last_launches() == []


# ================================================================== empty inputs
def test_empty_calls_leave_outputs_untouched(q):
    y = poisoned_f32(8)
    w = to_dev(q4k(0, 8, 256))
    xq = pack_on_device(q, acts(0, 1, 256))
    q.qmatvec(q.Q8K_Q4_K, w, 0, 256, xq, y)
    q.qmatmul_prefill(q.Q8K_Q4_K, w, 8, 256, xq, 0, y, None, 0)
    assert np.isnan(host(y)).all()
