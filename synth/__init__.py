"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the method's arithmetic: it only draws random numbers
and writes them into buffers of the documented byte layouts.  Both the oracle
and the HIP path consume what it returns; neither is imported here.

Why raw random bytes give the documented field distributions:

* Q4_K (144-byte GGUF block): the 12 scale bytes hold eight 6-bit scales and
  eight 6-bit mins, 96 bits in all, one-to-one.  Uniform random bytes therefore
  give every scale and min uniform on 0..63, independently; the 128 quant bytes
  hold 256 nibbles, one-to-one, so uniform bytes give quants uniform on 0..15.
  Only the two fp16 fields (d at byte 0, dmin at byte 2) are drawn as reals and
  rounded to fp16 (numpy's float16 cast rounds to nearest even).
* Q5_K (176-byte GGUF block): the same d, dmin and 12 scale/min bytes as
  Q4_K, then 32 bytes whose 256 bits are the fifth bits of the 256 values
  one-to-one, then 128 bytes of low nibbles: uniform bytes give quants uniform
  on 0..31.
* Q6_K (210-byte GGUF block): ql (128 bytes) and qh (64 bytes) hold 256 4-bit
  and 256 2-bit fields one-to-one, so uniform bytes give 6-bit quants uniform on
  0..63; the 16 int8 scales are uniform bytes, i.e. uniform on -128..127; d
  (fp16 at byte 208) is drawn as a real.

Workloads (the sizes of the decode / MoE / prefill shapes the pages discuss:
a 7B/8B-class attention projection, an output head, a Mixtral-like MoE layer
and a 512-row prefill of a down-projection) are listed in ``WORKLOADS``.
"""
from __future__ import annotations

import numpy as np

QK = 256
Q4K_BLOCK_BYTES = 144
Q5K_BLOCK_BYTES = 176
Q6K_BLOCK_BYTES = 210


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def _f16_bits(vals: np.ndarray) -> np.ndarray:
    return vals.astype(np.float16).view(np.uint16)


def q4k_weights(g: np.random.Generator, rows: int, K: int,
                d_range=(1e-3, 1e-2), dmin_range=(0.0, 1e-2)) -> np.ndarray:
    """rows x K weight as GGUF Q4_K blocks, flat uint8 [rows * K/256 * 144]."""
    assert K % QK == 0
    nblk = rows * (K // QK)
    blk = g.integers(0, 256, size=(nblk, Q4K_BLOCK_BYTES), dtype=np.uint8)
    d = _f16_bits(g.uniform(*d_range, size=nblk))
    dmin = _f16_bits(g.uniform(*dmin_range, size=nblk))
    blk[:, 0:2] = d.view(np.uint8).reshape(nblk, 2)
    blk[:, 2:4] = dmin.view(np.uint8).reshape(nblk, 2)
    return blk.reshape(-1)


def q5k_weights(g: np.random.Generator, rows: int, K: int,
                d_range=(5e-4, 5e-3), dmin_range=(0.0, 1e-2)) -> np.ndarray:
    """rows x K weight as GGUF Q5_K blocks, flat uint8 [rows * K/256 * 176]."""
    assert K % QK == 0
    nblk = rows * (K // QK)
    blk = g.integers(0, 256, size=(nblk, Q5K_BLOCK_BYTES), dtype=np.uint8)
    d = _f16_bits(g.uniform(*d_range, size=nblk))
    dmin = _f16_bits(g.uniform(*dmin_range, size=nblk))
    blk[:, 0:2] = d.view(np.uint8).reshape(nblk, 2)
    blk[:, 2:4] = dmin.view(np.uint8).reshape(nblk, 2)
    return blk.reshape(-1)


def q6k_weights(g: np.random.Generator, rows: int, K: int, d_range=(1e-4, 1e-3)) -> np.ndarray:
    """rows x K weight as GGUF Q6_K blocks, flat uint8 [rows * K/256 * 210]."""
    assert K % QK == 0
    nblk = rows * (K // QK)
    blk = g.integers(0, 256, size=(nblk, Q6K_BLOCK_BYTES), dtype=np.uint8)
    d = _f16_bits(g.uniform(*d_range, size=nblk))
    blk[:, 208:210] = d.view(np.uint8).reshape(nblk, 2)
    return blk.reshape(-1)


def activations(g: np.random.Generator, T: int, K: int) -> np.ndarray:
    """fp32 activations ~ N(0, 1), shape [T, K]."""
    return g.standard_normal(size=(T, K)).astype(np.float32)


def moe_routing(g: np.random.Generator, T: int, E: int, topk: int):
    """Per token: topk distinct experts drawn uniformly without replacement, and
    router weights = softmax over the topk chosen logits ~ N(0, 1)."""
    ids = np.stack([g.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    logits = g.standard_normal(size=(T, topk))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    rw = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, rw


# name -> (kind, parameters); seeds are the workload's index.
WORKLOADS = {
    "tiny_q4k_256x1024": dict(kind="matvec", qtype="q4k", rows=256, K=1024, T=1, seed=0),
    "decode_q4k_4096x4096": dict(kind="matvec", qtype="q4k", rows=4096, K=4096, T=1, seed=1),
    "decode_q6k_32000x4096": dict(kind="matvec", qtype="q6k", rows=32000, K=4096, T=1, seed=2),
    "moe_q4k_8x14336x4096_t16_top2": dict(kind="moe", qtype="q4k", E=8, rows=14336, K=4096, T=16, topk=2, seed=3),
    "prefill_q4k_4096x14336_m512": dict(kind="prefill", qtype="q4k", rows=4096, K=14336, T=512, seed=4),
}
