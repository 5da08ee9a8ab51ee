"""CPU oracle for the q8_K-packed K-quant path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports it, and this package never imports the product.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc, no HIP headers);
this module only builds it and marshals numpy arrays.  See ``oracle.c`` for the
passages of "Language models on the device: the cajeta-llm kernels"
(cajeta.dev/xpu/kernels-llm/, section 1) each function follows and for the
readings taken where the page is silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

QK = 256
Q4_K = 1
Q6_K = 2
Q5_K = 3
Q4K_BLOCK_BYTES = 144
Q6K_BLOCK_BYTES = 210
Q5K_BLOCK_BYTES = 176


def build(force: bool = False) -> str:
    """Compile liboracle.so with plain gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.or_f16_to_f32.restype = ctypes.c_float
    lib.or_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.or_q4k_fields.argtypes = [P, P, P, P, P, P]
    lib.or_q6k_fields.argtypes = [P, P, P, P]
    lib.or_q5k_fields.argtypes = [P, P, P, P, P, P]
    lib.or_dequant_q5k.argtypes = [P, I64, I64, P]
    lib.or_subblock_sums_q5k.argtypes = [P, I64, I64, P, P]
    lib.or_dequant_q4k.argtypes = [P, I64, I64, P]
    lib.or_dequant_q6k.argtypes = [P, I64, I64, P]
    lib.or_q8k_pack.argtypes = [P, I64, I64, P, P, P]
    lib.or_subblock_sums_q4k.argtypes = [P, I64, I64, P, P]
    lib.or_subblock_sums_q6k.argtypes = [P, I64, I64, P, P]
    lib.or_matvec.restype = ctypes.c_int
    lib.or_matvec.argtypes = [ctypes.c_int, P, I64, I64, P, P, P, I64, P, P, ctypes.c_int]
    lib.or_moe.restype = ctypes.c_int
    lib.or_moe.argtypes = [ctypes.c_int, P, I64, I64, I64, P, P, P, I64, P, P, I64, P, P, ctypes.c_int]
    lib.or_q6k_relayout.argtypes = [P, I64, P, P]
    lib.or_block_sums.restype = ctypes.c_int
    lib.or_block_sums.argtypes = [ctypes.c_int, P, I64, I64, P, I64, P]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
def f16_to_f32(h: int) -> float:
    return float(_load().or_f16_to_f32(int(h)))


def f16_to_f32_array(bits: np.ndarray) -> np.ndarray:
    lib = _load()
    bits = _c(bits, np.uint16).ravel()
    out = np.empty(bits.shape, np.float32)
    f = lib.or_f16_to_f32
    for i in range(bits.size):
        out[i] = f(int(bits[i]))
    return out


def q4k_fields(block: np.ndarray):
    """Decode one 144-byte Q4_K block -> (d, dmin, sc[8], m[8], q[256])."""
    block = _c(block, np.uint8)
    assert block.size == Q4K_BLOCK_BYTES
    d = np.zeros(1, np.float32)
    dmin = np.zeros(1, np.float32)
    sc = np.zeros(8, np.uint8)
    mn = np.zeros(8, np.uint8)
    q = np.zeros(QK, np.uint8)
    _load().or_q4k_fields(_p(block), _p(d), _p(dmin), _p(sc), _p(mn), _p(q))
    return float(d[0]), float(dmin[0]), sc, mn, q


def q5k_fields(block: np.ndarray):
    """Decode one 176-byte Q5_K block -> (d, dmin, sc[8], m[8], q[256] in 0..31)."""
    block = _c(block, np.uint8)
    assert block.size == Q5K_BLOCK_BYTES
    d = np.zeros(1, np.float32)
    dmin = np.zeros(1, np.float32)
    sc = np.zeros(8, np.uint8)
    mn = np.zeros(8, np.uint8)
    q = np.zeros(QK, np.uint8)
    _load().or_q5k_fields(_p(block), _p(d), _p(dmin), _p(sc), _p(mn), _p(q))
    return float(d[0]), float(dmin[0]), sc, mn, q


def q6k_fields(block: np.ndarray):
    """Decode one 210-byte Q6_K block -> (d, sc[16] int8, q[256] in 0..63)."""
    block = _c(block, np.uint8)
    assert block.size == Q6K_BLOCK_BYTES
    d = np.zeros(1, np.float32)
    sc = np.zeros(16, np.int8)
    q = np.zeros(QK, np.uint8)
    _load().or_q6k_fields(_p(block), _p(d), _p(sc), _p(q))
    return float(d[0]), sc, q


def dequant(qtype: int, w: np.ndarray, rows: int, K: int) -> np.ndarray:
    w = _c(w, np.uint8)
    out = np.empty((rows, K), np.float64)
    if qtype == Q4_K:
        _load().or_dequant_q4k(_p(w), rows, K, _p(out))
    elif qtype == Q5_K:
        _load().or_dequant_q5k(_p(w), rows, K, _p(out))
    else:
        _load().or_dequant_q6k(_p(w), rows, K, _p(out))
    return out


def q8k_pack(x: np.ndarray):
    """fp32 [T, K] -> (qs int8 [T, K], d fp32 [T, K/256], bsums int16 [T, K/32])."""
    x = _c(x, np.float32)
    T, K = x.shape
    assert K % QK == 0
    qs = np.empty((T, K), np.int8)
    d = np.empty((T, K // QK), np.float32)
    bs = np.empty((T, K // 32), np.int16)
    _load().or_q8k_pack(_p(x), T, K, _p(qs), _p(d), _p(bs))
    return qs, d, bs


def subblock_sums(qtype: int, w: np.ndarray, rows: int, K: int, qs_row: np.ndarray) -> np.ndarray:
    """Exact int32 sub-block sums of every weight row against one token's codes."""
    w = _c(w, np.uint8)
    qs_row = _c(qs_row, np.int8).ravel()
    assert qs_row.size == K
    if qtype == Q4_K:
        S = np.empty((rows, K // 32), np.int32)
        _load().or_subblock_sums_q4k(_p(w), rows, K, _p(qs_row), _p(S))
    elif qtype == Q5_K:
        S = np.empty((rows, K // 32), np.int32)
        _load().or_subblock_sums_q5k(_p(w), rows, K, _p(qs_row), _p(S))
    else:
        S = np.empty((rows, K // 16), np.int32)
        _load().or_subblock_sums_q6k(_p(w), rows, K, _p(qs_row), _p(S))
    return S


def block_sums(qtype: int, w: np.ndarray, rows: int, K: int, qs) -> np.ndarray:
    """Exact integer block sums I[T, rows, K/256] = sum_j sc_j * S_j (Q6_K:
    sum_s sc_s * S_s): each block's scale-weighted integer dot, before the
    floating-point epilogue.  qs: int8 [T, K] (or [K])."""
    w = _c(w, np.uint8)
    qs = _c(qs, np.int8)
    T = qs.shape[0] if qs.ndim == 2 else 1
    I = np.empty((T, rows, K // QK), np.int64)
    rc = _load().or_block_sums(qtype, _p(w), rows, K, _p(qs), T, _p(I))
    if rc != 0:
        raise ValueError(f"or_block_sums refused ({rc})")
    return I


def matvec(qtype: int, w: np.ndarray, rows: int, K: int, qs, d8, bsums, nthreads: int = 1):
    """y[T, rows] (fp64) and A[T, rows] = sum |terms|, for T packed tokens."""
    w = _c(w, np.uint8)
    qs = _c(qs, np.int8)
    d8 = _c(d8, np.float32)
    bsums = _c(bsums, np.int16)
    T = qs.shape[0] if qs.ndim == 2 else 1
    y = np.empty((T, rows), np.float64)
    A = np.empty((T, rows), np.float64)
    rc = _load().or_matvec(qtype, _p(w), rows, K, _p(qs), _p(d8), _p(bsums), T, _p(y), _p(A), int(nthreads))
    if rc != 0:
        raise ValueError(f"or_matvec refused ({rc})")
    return y, A


def moe(qtype: int, w, E: int, rows: int, K: int, qs, d8, bsums, ids, rw, nthreads: int = 1):
    w = _c(w, np.uint8)
    qs = _c(qs, np.int8)
    d8 = _c(d8, np.float32)
    bsums = _c(bsums, np.int16)
    ids = _c(ids, np.int32)
    rw = _c(rw, np.float32)
    T, topk = ids.shape
    y = np.empty((T, rows), np.float64)
    A = np.empty((T, rows), np.float64)
    rc = _load().or_moe(qtype, _p(w), E, rows, K, _p(qs), _p(d8), _p(bsums), T, _p(ids), _p(rw), topk,
                        _p(y), _p(A), int(nthreads))
    if rc != 0:
        raise ValueError(f"or_moe refused ({rc})")
    return y, A


def q6k_relayout(w: np.ndarray, nblocks: int):
    """210-byte Q6_K blocks -> (prefix uint16 [nblocks], bodies uint8 [nblocks*208])."""
    w = _c(w, np.uint8)
    prefix = np.empty(nblocks, np.uint16)
    bodies = np.empty(nblocks * 208, np.uint8)
    _load().or_q6k_relayout(_p(w), nblocks, _p(prefix), _p(bodies))
    return prefix, bodies
