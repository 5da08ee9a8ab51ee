"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a library routine (numpy's
float16 widening, numpy integer/fp64 products), a closed form worked out by
hand (tests/golden/), an invariant of the quantiser, or brute force on small
inputs.  The method is the one of "Language models on the device: the
cajeta-llm kernels" (cajeta.dev/xpu/kernels-llm/), section 1.
"""
import json
import os

import numpy as np
import pytest

import synth
from gguf_pack import pack_q4k_block, pack_q5k_block, pack_q6k_block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- fp16
def test_f16_decode_exhaustive(orc):
    """O1 against numpy's IEEE half->single widening over all 65,536 patterns."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = orc.f16_to_f32_array(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# --------------------------------------------------------------------------- block decode
@pytest.mark.parametrize("seed", range(20))
def test_q4k_roundtrip_random_fields(orc, seed):
    g = np.random.default_rng(1000 + seed)
    sc = g.integers(0, 64, 8)
    mn = g.integers(0, 64, 8)
    q = g.integers(0, 16, 256)
    d = float(np.float16(g.uniform(1e-3, 1e-2)))
    dmin = float(np.float16(g.uniform(0, 1e-2)))
    blk = pack_q4k_block(d, dmin, sc, mn, q)
    d2, dmin2, sc2, mn2, q2 = orc.q4k_fields(blk)
    assert d2 == np.float32(d) and dmin2 == np.float32(dmin)
    assert np.array_equal(sc2, sc) and np.array_equal(mn2, mn) and np.array_equal(q2, q)


@pytest.mark.parametrize("seed", range(20))
def test_q6k_roundtrip_random_fields(orc, seed):
    g = np.random.default_rng(2000 + seed)
    sc = g.integers(-128, 128, 16)
    q = g.integers(0, 64, 256)
    d = float(np.float16(g.uniform(1e-4, 1e-3)))
    blk = pack_q6k_block(d, sc, q)
    d2, sc2, q2 = orc.q6k_fields(blk)
    assert d2 == np.float32(d)
    assert np.array_equal(sc2.astype(np.int64), sc) and np.array_equal(q2, q)


@pytest.mark.parametrize("seed", range(20))
def test_q5k_roundtrip_random_fields(orc, seed):
    g = np.random.default_rng(3000 + seed)
    sc = g.integers(0, 64, 8)
    mn = g.integers(0, 64, 8)
    q = g.integers(0, 32, 256)
    d = float(np.float16(g.uniform(5e-4, 5e-3)))
    dmin = float(np.float16(g.uniform(0, 1e-2)))
    blk = pack_q5k_block(d, dmin, sc, mn, q)
    d2, dmin2, sc2, mn2, q2 = orc.q5k_fields(blk)
    assert d2 == np.float32(d) and dmin2 == np.float32(dmin)
    assert np.array_equal(sc2, sc) and np.array_equal(mn2, mn) and np.array_equal(q2, q)


def test_q5k_fifth_bit_positions(orc):
    """Bit j of qh[l] (byte 16 + l) is bit 4 of value l of sub-block j, i.e. of value 32j + l."""
    for j in range(8):
        for l in (0, 13, 31):
            blk = np.zeros(176, np.uint8)
            blk[16 + l] = 1 << j
            _, _, _, _, q = orc.q5k_fields(blk)
            want = np.zeros(256, np.uint8)
            want[32 * j + l] = 16
            assert np.array_equal(q, want)


def test_q5k_without_fifth_bits_equals_q4k(orc):
    """qh = 0 leaves the Q4_K block with the same d, dmin, scales and nibbles:
    the oracle's Q4_K result (pinned above) must come out bit for bit."""
    g = np.random.default_rng(21)
    rows, K, T = 6, 768, 3
    nb = K // 256
    w4 = synth.q4k_weights(g, rows, K).reshape(rows * nb, 144)
    w5 = np.zeros((rows * nb, 176), np.uint8)
    w5[:, 0:16] = w4[:, 0:16]
    w5[:, 48:176] = w4[:, 16:144]
    qs, d8, bs = orc.q8k_pack(synth.activations(g, T, K))
    y4, a4 = orc.matvec(orc.Q4_K, w4.reshape(-1), rows, K, qs, d8, bs)
    y5, a5 = orc.matvec(orc.Q5_K, w5.reshape(-1), rows, K, qs, d8, bs)
    assert np.array_equal(y4, y5) and np.array_equal(a4, a5)


def test_q5k_all_fifth_bits_closed_form(orc):
    """Setting every fifth bit adds 16 to every quant, so the result grows by
    sum_b d8_b * d_b * sum_j sc_j * 16 * bsum_bj (fields read back by the packer's
    inverse, not by the oracle)."""
    g = np.random.default_rng(22)
    K = 512
    nb = K // 256
    flds = []
    blocks0, blocks1 = [], []
    for b in range(nb):
        sc = g.integers(0, 64, 8)
        mn = g.integers(0, 64, 8)
        q = g.integers(0, 16, 256)
        d = float(np.float16(g.uniform(5e-4, 5e-3)))
        dmin = float(np.float16(g.uniform(0, 1e-2)))
        flds.append((d, sc))
        blocks0.append(pack_q5k_block(d, dmin, sc, mn, q))
        blocks1.append(pack_q5k_block(d, dmin, sc, mn, q + 16))
    w0 = np.concatenate(blocks0)
    w1 = np.concatenate(blocks1)
    qs, d8, bs = orc.q8k_pack(synth.activations(g, 1, K))
    y0, A0 = orc.matvec(orc.Q5_K, w0, 1, K, qs, d8, bs)
    y1, A1 = orc.matvec(orc.Q5_K, w1, 1, K, qs, d8, bs)
    want = 0.0
    for b in range(nb):
        d, sc = flds[b]
        want += float(d8[0, b]) * d * float(np.dot(sc.astype(np.int64) * 16, bs[0, 8 * b:8 * b + 8].astype(np.int64)))
    assert abs((y1[0, 0] - y0[0, 0]) - want) <= 1e-12 * (A0[0, 0] + A1[0, 0])


def test_q4k_single_byte_positions(orc):
    """Byte 32c+l of the quants carries value 64c+l (low nibble) and 64c+32+l (high)."""
    for c in range(4):
        for l in (0, 7, 31):
            blk = np.zeros(144, np.uint8)
            blk[16 + 32 * c + l] = 0x52  # low nibble 2, high nibble 5
            _, _, _, _, q = orc.q4k_fields(blk)
            want = np.zeros(256, np.uint8)
            want[64 * c + l] = 2
            want[64 * c + 32 + l] = 5
            assert np.array_equal(q, want)


def test_hand_blocks_golden(orc):
    with open(os.path.join(GOLDEN, "kquant_hand_blocks.json")) as f:
        cases = json.load(f)["cases"]
    for cs in cases:
        if cs["fmt"] == "q4k":
            blk = pack_q4k_block(cs["d"], cs["dmin"], cs["sc"], cs["m"], [cs["q_all"]] * 256)
            w = orc.dequant(orc.Q4_K, blk, 1, 256)
        elif cs["fmt"] == "q5k":
            blk = pack_q5k_block(cs["d"], cs["dmin"], cs["sc"], cs["m"], [cs["q_all"]] * 256)
            w = orc.dequant(orc.Q5_K, blk, 1, 256)
        else:
            blk = pack_q6k_block(cs["d"], cs["sc"], [cs["q_all"]] * 256)
            w = orc.dequant(orc.Q6_K, blk, 1, 256)
        assert w.sum() == cs["sum_w"], cs["name"]


# --------------------------------------------------------------------------- q8_K pack
def test_q8k_golden_rounding(orc):
    with open(os.path.join(GOLDEN, "q8k_rounding.json")) as f:
        cases = json.load(f)["cases"]
    for cs in cases:
        x = np.zeros((1, 256), np.float32)
        n = len(cs["x_head"])
        x[0, :n] = cs["x_head"]
        qs, d, bs = orc.q8k_pack(x)
        assert list(qs[0, :n]) == cs["qs_head"], cs["name"]
        assert not qs[0, n:].any()
        if "d" in cs:
            assert d[0, 0] == np.float32(cs["d"])
        else:
            num, den = cs["d_is_fp32_quotient"]
            assert d[0, 0] == np.float32(num) / np.float32(den)
        assert list(bs[0]) == cs["bsums"]


@pytest.mark.parametrize("scale", [1.0, 1e-3, 37.5, 1e4])
def test_q8k_invariants(orc, scale):
    g = np.random.default_rng(7)
    x = (g.standard_normal((6, 1024)) * scale).astype(np.float32)
    x[1, 256:512] = 0.0  # an all-zero block
    x[2, :256] = -np.abs(x[2, :256])  # negative extreme
    qs, d, bs = orc.q8k_pack(x)
    xb = x.reshape(6, 4, 256)
    qb = qs.reshape(6, 4, 256).astype(np.int64)
    assert np.abs(qb).max() <= 127
    for t in range(6):
        for b in range(4):
            amax = np.abs(xb[t, b]).max()
            if amax == 0:
                assert d[t, b] == 0 and not qb[t, b].any() and not bs[t, 8 * b:8 * b + 8].any()
                continue
            i = int(np.argmax(np.abs(xb[t, b])))
            assert qb[t, b, i] == (127 if xb[t, b, i] > 0 else -127)
            assert d[t, b] == np.float32(amax) / np.float32(127.0)
            # reconstruction error within half a step (plus fp32 slack)
            err = np.abs(xb[t, b].astype(np.float64) - float(d[t, b]) * qb[t, b])
            assert err.max() <= float(d[t, b]) * (0.5 + 1e-5)
            # sums are the 32-value group sums of the codes
            assert np.array_equal(bs[t, 8 * b:8 * b + 8], qb[t, b].reshape(8, 32).sum(1))


# --------------------------------------------------------------------------- integer sums
def test_q4k_subblock_sums_closed_form(orc):
    """All quants 1 and qs_i = (i mod 255) - 127: S_j is the plain sum of that slice."""
    K = 512
    blk = pack_q4k_block(1.0, 0.0, [1] * 8, [0] * 8, [1] * 256)
    w = np.tile(blk, (3, K // 256)).reshape(-1)
    qs = ((np.arange(K) % 255) - 127).astype(np.int8)
    S = orc.subblock_sums(orc.Q4_K, w, 3, K, qs)
    want = np.array([sum((i % 255) - 127 for i in range(32 * j, 32 * j + 32)) for j in range(K // 32)])
    for r in range(3):
        assert np.array_equal(S[r], want)


def test_q6k_subblock_sums_closed_form(orc):
    """All quants 33 (value +1): S_s is the plain sum of the 16-value slice."""
    K = 512
    blk = pack_q6k_block(1.0, [1] * 16, [33] * 256)
    w = np.tile(blk, (2, K // 256)).reshape(-1)
    qs = ((np.arange(K) * 7 % 255) - 127).astype(np.int8)
    S = orc.subblock_sums(orc.Q6_K, w, 2, K, qs)
    want = qs.astype(np.int64).reshape(-1, 16).sum(1)
    assert np.array_equal(S[0], want) and np.array_equal(S[1], want)


_GEN = {1: synth.q4k_weights, 2: synth.q6k_weights, 3: synth.q5k_weights}
_BB = {1: 144, 2: 210, 3: 176}


@pytest.mark.parametrize("qtype", [1, 2, 3])
def test_subblock_sums_brute_force(orc, qtype):
    """Integer sums against numpy products of the decoded quants."""
    g = np.random.default_rng(11 + qtype)
    rows, K = 5, 768
    w = _GEN[qtype](g, rows, K)
    qs = g.integers(-127, 128, K).astype(np.int8)
    S = orc.subblock_sums(qtype, w, rows, K, qs)
    bb = _BB[qtype]
    fields = {1: orc.q4k_fields, 2: orc.q6k_fields, 3: orc.q5k_fields}[qtype]
    for r in range(rows):
        qv = []
        for b in range(K // 256):
            blk = w[(r * (K // 256) + b) * bb:(r * (K // 256) + b + 1) * bb]
            qv.append(fields(blk)[-1].astype(np.int64) - (32 if qtype == 2 else 0))
        qv = np.concatenate(qv)
        gs = 16 if qtype == 2 else 32
        assert np.array_equal(S[r], (qv * qs).reshape(-1, gs).sum(1))


# --------------------------------------------------------------------------- epilogue
@pytest.mark.parametrize("qtype", [1, 2, 3])
@pytest.mark.parametrize("seed", range(8))
def test_matvec_equals_dequant_then_dot(orc, qtype, seed):
    """Integer-structured result = fp64 dequantise-then-dot (brute force)."""
    g = np.random.default_rng(100 * qtype + seed)
    rows, K, T = 7, 256 * (1 + seed % 4), 2
    w = _GEN[qtype](g, rows, K)
    x = synth.activations(g, T, K)
    qs, d8, bs = orc.q8k_pack(x)
    y, A = orc.matvec(qtype, w, rows, K, qs, d8, bs)
    W = orc.dequant(qtype, w, rows, K)
    xhat = np.repeat(d8.astype(np.float64), 256, axis=1) * qs
    ybf = xhat @ W.T
    assert np.allclose(y, ybf, rtol=0, atol=1e-12 * np.abs(A).max() + 1e-300)
    assert np.all(A >= np.abs(y) - 1e-12 * A)
    # against the unquantised activations: error bounded by half a step per value
    yx = x.astype(np.float64) @ W.T
    bound = 0.5 * (np.abs(W)[None, :, :] * np.repeat(d8.astype(np.float64), 256, axis=1)[:, None, :]).sum(-1)
    assert np.all(np.abs(y - yx) <= bound * (1 + 1e-6))


def test_matvec_textbook_dot(orc):
    """d = 1, sc = 1, dmin = 0 and d8 = 1 (amax = 127): y is the plain integer dot."""
    g = np.random.default_rng(5)
    K, rows = 1024, 4
    q = g.integers(0, 16, (rows, K // 256, 256))
    w = np.concatenate([pack_q4k_block(1.0, 0.0, [1] * 8, [5] * 8, q[r, b])
                        for r in range(rows) for b in range(K // 256)])
    x = g.integers(-126, 127, (1, K)).astype(np.float32)
    x[0, ::256] = 127.0  # amax = 127 in every block -> d8 = 1, qs = x
    qs, d8, bs = orc.q8k_pack(x)
    assert np.all(d8 == 1.0) and np.array_equal(qs[0].astype(np.int64), x[0].astype(np.int64))
    y, _ = orc.matvec(orc.Q4_K, w, rows, K, qs, d8, bs)
    want = q.reshape(rows, K) @ x[0].astype(np.int64)
    assert np.array_equal(y[0], want.astype(np.float64))


def test_matvec_min_term_sign(orc):
    """A block with q = 0 leaves only the min term: y = -dmin * sum_j m_j * bsum_j."""
    K = 256
    mn = [3, 0, 1, 4, 1, 5, 9, 2]
    w = pack_q4k_block(0.5, 0.25, [7] * 8, mn, [0] * 256)
    x = np.zeros((1, K), np.float32)
    x[0, :] = 1.0
    x[0, 0] = 127.0  # d8 = 1, qs = [127, 1, 1, ...]
    qs, d8, bs = orc.q8k_pack(x)
    y, _ = orc.matvec(orc.Q4_K, w, 1, K, qs, d8, bs)
    bsum = [127 + 31] + [32] * 7
    assert y[0, 0] == -0.25 * sum(m * s for m, s in zip(mn, bsum))


# --------------------------------------------------------------------------- variants
def test_batched_and_prefill_rows_equal_single(orc):
    g = np.random.default_rng(9)
    rows, K, T = 6, 512, 5
    w = synth.q4k_weights(g, rows, K)
    qs, d8, bs = orc.q8k_pack(synth.activations(g, T, K))
    y, _ = orc.matvec(orc.Q4_K, w, rows, K, qs, d8, bs)
    for t in range(T):
        y1, _ = orc.matvec(orc.Q4_K, w, rows, K, qs[t:t + 1], d8[t:t + 1], bs[t:t + 1])
        assert np.array_equal(y[t], y1[0])


def test_threads_do_not_change_results(orc):
    g = np.random.default_rng(10)
    rows, K, T = 33, 512, 3
    w = synth.q6k_weights(g, rows, K)
    qs, d8, bs = orc.q8k_pack(synth.activations(g, T, K))
    y1, a1 = orc.matvec(orc.Q6_K, w, rows, K, qs, d8, bs, nthreads=1)
    y4, a4 = orc.matvec(orc.Q6_K, w, rows, K, qs, d8, bs, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(a1, a4)


@pytest.mark.parametrize("qtype", [1, 3])
def test_moe_equals_weighted_single_calls(orc, qtype):
    g = np.random.default_rng(12)
    E, rows, K, T, topk = 4, 9, 512, 6, 2
    w = _GEN[qtype](g, E * rows, K)
    qs, d8, bs = orc.q8k_pack(synth.activations(g, T, K))
    ids, rw = synth.moe_routing(g, T, E, topk)
    y, A = orc.moe(qtype, w, E, rows, K, qs, d8, bs, ids, rw)
    per = rows * (K // 256) * _BB[qtype]
    for t in range(T):
        acc = np.zeros(rows)
        for k in range(topk):
            e = ids[t, k]
            ye, _ = orc.matvec(qtype, w[e * per:(e + 1) * per], rows, K, qs[t:t + 1], d8[t:t + 1], bs[t:t + 1])
            acc = acc + float(rw[t, k]) * ye[0]
        assert np.array_equal(y[t], acc)


def test_q6k_relayout_bytes(orc):
    g = np.random.default_rng(13)
    w = synth.q6k_weights(g, 3, 512)
    prefix, bodies = orc.q6k_relayout(w, 6)
    blocks = w.reshape(6, 210)
    assert np.array_equal(bodies.reshape(6, 208), blocks[:, :208])
    assert np.array_equal(prefix, blocks[:, 208:210].copy().view(np.uint16).ravel())


def test_moe_routing_generator_shape():
    g = np.random.default_rng(0)
    ids, rw = synth.moe_routing(g, 16, 8, 2)
    assert ids.shape == (16, 2) and all(len(set(r)) == 2 for r in ids.tolist())
    assert np.allclose(rw.sum(1), 1.0, atol=1e-6) and (rw > 0).all()


# --------------------------------------------------------------------------- tolerance terms and block sums
def _golden_terms():
    with open(os.path.join(GOLDEN, "tolerance_terms.json")) as f:
        return json.load(f)


def _golden_token(gt):
    """The two hand-worked token blocks (fp32 values chosen so the codes are exact)."""
    blk = np.zeros(256, np.float32)
    blk[0] = 127.0
    blk[1:32] = -1.0
    for j, c in enumerate(gt["group_values"]):
        blk[32 * (j + 1):32 * (j + 2)] = c
    return np.concatenate([blk, 0.5 * blk])[None, :]


def _golden_block(fmt, b):
    if fmt == "q6k":
        return pack_q6k_block(b["d"], b["sc"], [b["q_all"]] * 256)
    pk = pack_q5k_block if fmt == "q5k" else pack_q4k_block
    return pk(b["d"], b["dmin"], b["sc"], b["m"], [b["q_all"]] * 256)


_FMT_Q = {"q4k": 1, "q6k": 2, "q5k": 3}


def test_golden_token_codes(orc):
    gt = _golden_terms()["token"]
    qs, d8, bs = orc.q8k_pack(_golden_token(gt))
    assert list(d8[0]) == gt["d8"]
    assert list(bs[0, :8]) == gt["bsums"] and list(bs[0, 8:]) == gt["bsums"]
    assert np.array_equal(qs[0, :256], qs[0, 256:])


@pytest.mark.parametrize("name", ["q4k_two_blocks", "q5k_two_blocks", "q6k_two_blocks"])
def test_golden_sum_of_terms(orc, name):
    """y, the tolerance scale A = sum|terms|, the sub-block sums S and the block
    sums I of hand-worked blocks, exactly (a scaled, dropped or signed term
    changes A)."""
    g = _golden_terms()
    cs = next(c for c in g["cases"] if c["name"] == name)
    qt = _FMT_Q[cs["fmt"]]
    blk = _golden_block(cs["fmt"], cs["block"])
    w = np.concatenate([blk, blk])
    qs, d8, bs = orc.q8k_pack(_golden_token(g["token"]))
    y, A = orc.matvec(qt, w, 1, 512, qs, d8, bs)
    assert y[0, 0] == cs["y"] and A[0, 0] == cs["A"]
    S = orc.subblock_sums(qt, w, 1, 512, qs[0])
    assert list(S[0, :len(cs["S"])]) == cs["S"] and list(S[0, len(cs["S"]):]) == cs["S"]
    assert list(orc.block_sums(qt, w, 1, 512, qs)[0, 0]) == cs["I"]


def test_golden_moe_sum_of_terms(orc):
    """Two experts with a negative router weight: A sums |rw| times each expert's terms."""
    g = _golden_terms()
    cs = next(c for c in g["cases"] if c["name"] == "moe_q4k_signed_router")
    w = np.concatenate([np.concatenate([_golden_block("q4k", e)] * 2) for e in cs["experts"]])
    qs, d8, bs = orc.q8k_pack(_golden_token(g["token"]))
    ids = np.array([cs["ids"]], np.int32)
    rw = np.array([cs["rw"]], np.float32)
    y, A = orc.moe(orc.Q4_K, w, 2, 1, 512, qs, d8, bs, ids, rw)
    assert y[0, 0] == cs["y"] and A[0, 0] == cs["A"]


@pytest.mark.parametrize("qtype", [1, 2, 3])
def test_block_sums_equal_integer_dot_of_dequantised_block(orc, qtype):
    """With d = 1 (and dmin = 0) the dequantised block is sc_j * q (Q6_K:
    sc_s * (q - 32)), integer valued: I_b is then its plain integer dot with the
    codes (brute force over the pinned dequantisation)."""
    g = np.random.default_rng(40 + qtype)
    rows, K, T = 4, 768, 3
    w = _GEN[qtype](g, rows, K).reshape(rows * (K // 256), _BB[qtype]).copy()
    one = np.array([1.0], np.float16).view(np.uint8)
    if qtype == 2:
        w[:, 208:210] = one
    else:
        w[:, 0:2] = one
        w[:, 2:4] = 0
    w = w.reshape(-1)
    qs = g.integers(-127, 128, (T, K)).astype(np.int8)
    I = orc.block_sums(qtype, w, rows, K, qs)
    W = orc.dequant(qtype, w, rows, K)
    assert np.array_equal(W, np.round(W))
    want = (qs.astype(np.int64)[:, None, :] * W.astype(np.int64)[None, :, :]).reshape(T, rows, K // 256, 256).sum(-1)
    assert np.array_equal(I, want)
