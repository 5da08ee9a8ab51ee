"""Test-side GGUF block writers: fields -> bytes.

The oracle only reads blocks (bytes -> fields); these writers go the other way
and are written separately from it, so a round trip through both catches a
wrong shift, mask or index on either side.  Layouts are the public GGUF Q4_K
(144 bytes), Q5_K (176 bytes) and Q6_K (210 bytes) definitions.
"""
from __future__ import annotations

import numpy as np


def _f16_bytes(v: float) -> np.ndarray:
    return np.array([v], np.float16).view(np.uint8)


def pack_q4k_block(d: float, dmin: float, sc, mn, q) -> np.ndarray:
    sc = np.asarray(sc, np.int64)
    mn = np.asarray(mn, np.int64)
    q = np.asarray(q, np.int64)
    assert sc.shape == (8,) and mn.shape == (8,) and q.shape == (256,)
    assert sc.min() >= 0 and sc.max() < 64 and mn.min() >= 0 and mn.max() < 64
    assert q.min() >= 0 and q.max() < 16
    out = np.zeros(144, np.uint8)
    out[0:2] = _f16_bytes(d)
    out[2:4] = _f16_bytes(dmin)
    s = np.zeros(12, np.int64)
    for j in range(4):
        # bytes 0..3: scale j (6 bits) + top two bits of scale j+4
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        # bytes 4..7: min j (6 bits) + top two bits of min j+4
        s[j + 4] = (mn[j] & 63) | ((mn[j + 4] >> 4) << 6)
        # bytes 8..11: low nibbles of scale j+4 (low half) and min j+4 (high half)
        s[j + 8] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
    out[4:16] = s.astype(np.uint8)
    qs = np.zeros(128, np.int64)
    for c in range(4):
        for l in range(32):
            qs[32 * c + l] = q[64 * c + l] | (q[64 * c + 32 + l] << 4)
    out[16:144] = qs.astype(np.uint8)
    return out


def pack_q5k_block(d: float, dmin: float, sc, mn, q) -> np.ndarray:
    """Q5_K: d, dmin and the 12 scale/min bytes as in Q4_K, then qh[32] (bit j
    of qh[l] is bit 4 of value l of sub-block j), then the low nibbles packed
    as Q4_K packs its quants."""
    q = np.asarray(q, np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() < 32
    q4 = pack_q4k_block(d, dmin, sc, mn, q & 15)
    qh = np.zeros(32, np.int64)
    for j in range(8):
        for l in range(32):
            qh[l] |= ((q[32 * j + l] >> 4) & 1) << j
    out = np.zeros(176, np.uint8)
    out[0:16] = q4[0:16]
    out[16:48] = qh.astype(np.uint8)
    out[48:176] = q4[16:144]
    return out


def pack_q6k_block(d: float, sc, q) -> np.ndarray:
    sc = np.asarray(sc, np.int64)
    q = np.asarray(q, np.int64)
    assert sc.shape == (16,) and q.shape == (256,)
    assert sc.min() >= -128 and sc.max() < 128 and q.min() >= 0 and q.max() < 64
    ql = np.zeros(128, np.int64)
    qh = np.zeros(64, np.int64)
    for h in range(2):
        for t in range(4):
            for l in range(32):
                v = q[128 * h + 32 * t + l]
                ql[64 * h + 32 * (t & 1) + l] |= (v & 15) << (4 * (t >> 1))
                qh[32 * h + l] |= (v >> 4) << (2 * t)
    out = np.zeros(210, np.uint8)
    out[0:128] = ql.astype(np.uint8)
    out[128:192] = qh.astype(np.uint8)
    out[192:208] = (sc & 255).astype(np.uint8)
    out[208:210] = _f16_bytes(d)
    return out
