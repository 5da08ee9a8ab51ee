"""Python binding of libq8k (the C ABI in include/q8k.h).

Argument marshalling only: every step of the path runs in the gfx950 kernels
behind the C ABI.  PyTorch provides device memory and streams.  There is no
CPU fallback: if libq8k.so is missing the import raises.

Functions keep the C names and argument order; tensors are passed for device
buffers (their ``data_ptr()`` is used) and the stream defaults to torch's
current stream.  A refusal raises :class:`Q8KError` carrying the status name
and the library's message.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "Q8K_Q4_K", "Q8K_Q5_K", "Q8K_Q6_K_RELAID", "Q8K_Q6_K_GGUF", "Q8K_COLS_MAX", "Q8K_MOE_MAX_TOKENS", "Q8K_MOE_MAX_TOPK", "Q8KError",
    "lib", "LIB_PATH", "q8k_act_bytes", "q8k_act_layout", "q8k_weight_bytes", "q8k_pack", "q8k_bind_q6k",
    "qmatvec", "qmatvec_batched", "qmatvec_f32", "qmatvec_moe", "qmatmul_prefill_workspace_bytes", "qmatmul_prefill",
    "qmatmul_prefill_f32_workspace_bytes", "qmatmul_prefill_f32",
    "qmatmul_prefill_moe_workspace_bytes", "qmatmul_prefill_moe", "qmatmul_prefill_moe_noalloc",
    "Q8K_NOALLOC_SCRATCH_BYTES", "q8k_debug_subblock_sums", "q8k_debug_prefill_block_sums", "q8k_debug_moe_subblock_sums",
    "q8k_debug_wave_sums", "q8k_debug_last_launches", "q8k_status_str", "q8k_last_error", "EXPORTED",
]

Q8K_Q4_K = 1
Q8K_Q6_K_RELAID = 2
Q8K_Q6_K_GGUF = 3
Q8K_Q5_K = 4
Q8K_COLS_MAX = 8
Q8K_MOE_MAX_TOKENS = 256
Q8K_MOE_MAX_TOPK = 64
Q8K_NOALLOC_SCRATCH_BYTES = 64 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq8k.so")

# every symbol declared in include/q8k.h
EXPORTED = (
    "q8k_act_bytes", "q8k_act_layout", "q8k_weight_bytes", "q8k_pack", "q8k_bind_q6k", "qmatvec",
    "qmatvec_batched", "qmatvec_f32", "qmatvec_moe", "qmatmul_prefill_workspace_bytes", "qmatmul_prefill",
    "qmatmul_prefill_f32_workspace_bytes", "qmatmul_prefill_f32",
    "qmatmul_prefill_moe_workspace_bytes", "qmatmul_prefill_moe", "qmatmul_prefill_moe_noalloc",
    "q8k_debug_subblock_sums", "q8k_debug_prefill_block_sums", "q8k_debug_moe_subblock_sums",
    "q8k_debug_wave_sums", "q8k_debug_last_launches", "q8k_status_str", "q8k_last_error",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libq8k.so not found at {LIB_PATH}: build it first "
        "(python -m quantized_q8kpack_fp32_amd.build or __graft_entry__.build())"
    )

# torch first: its HIP runtime carries the same soname (libamdhip64.so.7) as
# the ROCm copy libq8k.so was linked against, so once torch has loaded it the
# library binds to that same runtime.  Loaded the other way round, torch
# would bring a second HIP runtime into the process, and the library's
# launches would not see the device that torch's tensors live on.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_INT = ctypes.c_int

lib.q8k_act_bytes.restype = _SZ
lib.q8k_act_bytes.argtypes = [_I64, _I64]
lib.q8k_act_layout.restype = _SZ
lib.q8k_act_layout.argtypes = [_I64, _I64, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]
lib.q8k_weight_bytes.restype = _SZ
lib.q8k_weight_bytes.argtypes = [_INT, _I64, _I64]
lib.q8k_pack.restype = _INT
lib.q8k_pack.argtypes = [_P, _I64, _I64, _P, _P]
lib.q8k_bind_q6k.restype = _INT
lib.q8k_bind_q6k.argtypes = [_P, _I64, _I64, _P, _P]
lib.qmatvec.restype = _INT
lib.qmatvec.argtypes = [_INT, _P, _I64, _I64, _P, _P, _P]
lib.qmatvec_batched.restype = _INT
lib.qmatvec_batched.argtypes = [_INT, _P, _I64, _I64, _P, _I64, _P, _P]
lib.qmatvec_f32.restype = _INT
lib.qmatvec_f32.argtypes = [_INT, _P, _I64, _I64, _P, _I64, _P, _P, _P]
lib.qmatvec_moe.restype = _INT
lib.qmatvec_moe.argtypes = [_INT, _P, _I64, _I64, _I64, _P, _I64, _P, _P, ctypes.c_int32, _P, _P]
lib.qmatmul_prefill_workspace_bytes.restype = _SZ
lib.qmatmul_prefill_workspace_bytes.argtypes = [_INT, _I64, _I64, _I64]
lib.qmatmul_prefill.restype = _INT
lib.qmatmul_prefill.argtypes = [_INT, _P, _I64, _I64, _P, _I64, _P, _P, _SZ, _P]
lib.qmatmul_prefill_f32_workspace_bytes.restype = _SZ
lib.qmatmul_prefill_f32_workspace_bytes.argtypes = [_INT, _I64, _I64, _I64]
lib.qmatmul_prefill_f32.restype = _INT
lib.qmatmul_prefill_f32.argtypes = [_INT, _P, _I64, _I64, _P, _I64, _P, _P, _P, _SZ, _P]
lib.qmatmul_prefill_moe_workspace_bytes.restype = _SZ
lib.qmatmul_prefill_moe_workspace_bytes.argtypes = [_INT, _I64, _I64, _I64, _I64, ctypes.c_int32]
lib.qmatmul_prefill_moe.restype = _INT
lib.qmatmul_prefill_moe.argtypes = [_INT, _P, _I64, _I64, _I64, _P, _I64, _P, _P, ctypes.c_int32, _P, _P, _SZ, _P]
lib.qmatmul_prefill_moe_noalloc.restype = _INT
lib.qmatmul_prefill_moe_noalloc.argtypes = [_INT, _P, _I64, _I64, _I64, _P, _I64, _P, _P, ctypes.c_int32, _P, _P]
lib.q8k_debug_subblock_sums.restype = _INT
lib.q8k_debug_subblock_sums.argtypes = [_INT, _P, _I64, _I64, _P, _P, _P, _P]
lib.q8k_debug_prefill_block_sums.restype = _INT
lib.q8k_debug_prefill_block_sums.argtypes = [_INT, _P, _I64, _I64, _P, _I64, _P, _P, _P]
lib.q8k_debug_moe_subblock_sums.restype = _INT
lib.q8k_debug_moe_subblock_sums.argtypes = [_INT, _P, _I64, _I64, _I64, _P, _I64, _P, _P, ctypes.c_int32, _P, _P, _P]
lib.q8k_debug_wave_sums.restype = _INT
lib.q8k_debug_wave_sums.argtypes = [_P, _P]
lib.q8k_debug_last_launches.restype = _INT
lib.q8k_debug_last_launches.argtypes = [ctypes.POINTER(_P), _INT]
lib.q8k_status_str.restype = ctypes.c_char_p
lib.q8k_status_str.argtypes = [_INT]
lib.q8k_last_error.restype = ctypes.c_char_p
lib.q8k_last_error.argtypes = []


class Q8KError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = q8k_status_str(status)
        super().__init__(f"{self.name}: {message}")


def q8k_status_str(status: int) -> str:
    return lib.q8k_status_str(int(status)).decode()


def q8k_last_error() -> str:
    return lib.q8k_last_error().decode()


def _ptr(t) -> int | None:
    """Device pointer of a tensor, or an int passed through (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int) -> None:
    if st != 0:
        raise Q8KError(st, q8k_last_error())


# ------------------------------------------------------------------ sizing
def q8k_act_bytes(T: int, K: int) -> int:
    return int(lib.q8k_act_bytes(T, K))


def q8k_act_layout(T: int, K: int):
    """-> (total_bytes, off_d, off_bsums) of a q8_K buffer of T tokens."""
    od, ob = _SZ(0), _SZ(0)
    total = lib.q8k_act_layout(T, K, ctypes.byref(od), ctypes.byref(ob))
    return int(total), int(od.value), int(ob.value)


def q8k_weight_bytes(qtype: int, rows: int, K: int) -> int:
    return int(lib.q8k_weight_bytes(qtype, rows, K))


def qmatmul_prefill_workspace_bytes(qtype: int, rows: int, K: int, M: int) -> int:
    return int(lib.qmatmul_prefill_workspace_bytes(qtype, rows, K, M))


# -------------------------------------------------------------- operations
def q8k_pack(x, T: int, K: int, xq, stream=None) -> None:
    _check(lib.q8k_pack(_ptr(x), T, K, _ptr(xq), _stream(stream)))


def q8k_bind_q6k(w_gguf, rows: int, K: int, w_relaid, stream=None) -> None:
    _check(lib.q8k_bind_q6k(_ptr(w_gguf), rows, K, _ptr(w_relaid), _stream(stream)))


def qmatvec(qtype: int, w, rows: int, K: int, xq, y, stream=None) -> None:
    _check(lib.qmatvec(qtype, _ptr(w), rows, K, _ptr(xq), _ptr(y), _stream(stream)))


def qmatvec_batched(qtype: int, w, rows: int, K: int, xq, ncols: int, y, stream=None) -> None:
    _check(lib.qmatvec_batched(qtype, _ptr(w), rows, K, _ptr(xq), ncols, _ptr(y), _stream(stream)))


def qmatvec_f32(qtype: int, w, rows: int, K: int, x, ncols: int, y, xq_out=None, stream=None) -> None:
    _check(lib.qmatvec_f32(qtype, _ptr(w), rows, K, _ptr(x), ncols, _ptr(y), _ptr(xq_out), _stream(stream)))


def qmatvec_moe(qtype: int, w, E: int, rows: int, K: int, xq, T: int, ids, rw, topk: int, y, stream=None) -> None:
    _check(lib.qmatvec_moe(qtype, _ptr(w), E, rows, K, _ptr(xq), T, _ptr(ids), _ptr(rw), topk, _ptr(y),
                           _stream(stream)))


def qmatmul_prefill(qtype: int, w, rows: int, K: int, xq, M: int, y, ws=None, ws_bytes: int = 0,
                    stream=None) -> None:
    _check(lib.qmatmul_prefill(qtype, _ptr(w), rows, K, _ptr(xq), M, _ptr(y), _ptr(ws), ws_bytes,
                               _stream(stream)))


def qmatmul_prefill_f32_workspace_bytes(qtype: int, rows: int, K: int, M: int) -> int:
    return int(lib.qmatmul_prefill_f32_workspace_bytes(qtype, rows, K, M))


def qmatmul_prefill_f32(qtype: int, w, rows: int, K: int, x, M: int, xq, y, ws=None, ws_bytes: int = 0,
                        stream=None) -> None:
    _check(lib.qmatmul_prefill_f32(qtype, _ptr(w), rows, K, _ptr(x), M, _ptr(xq), _ptr(y), _ptr(ws), ws_bytes,
                                   _stream(stream)))


def qmatmul_prefill_moe_workspace_bytes(qtype: int, E: int, rows: int, K: int, T: int, topk: int) -> int:
    return int(lib.qmatmul_prefill_moe_workspace_bytes(qtype, E, rows, K, T, topk))


def qmatmul_prefill_moe(qtype: int, w, E: int, rows: int, K: int, xq, T: int, ids, rw, topk: int, y, ws=None,
                        ws_bytes: int = 0, stream=None) -> None:
    _check(lib.qmatmul_prefill_moe(qtype, _ptr(w), E, rows, K, _ptr(xq), T, _ptr(ids), _ptr(rw), topk, _ptr(y),
                                   _ptr(ws), ws_bytes, _stream(stream)))


def qmatmul_prefill_moe_noalloc(qtype: int, w, E: int, rows: int, K: int, xq, T: int, ids, rw, topk: int, y,
                                stream=None) -> None:
    _check(lib.qmatmul_prefill_moe_noalloc(qtype, _ptr(w), E, rows, K, _ptr(xq), T, _ptr(ids), _ptr(rw), topk,
                                           _ptr(y), _stream(stream)))


def q8k_debug_subblock_sums(qtype: int, w, rows: int, K: int, xq, y, S, stream=None) -> None:
    _check(lib.q8k_debug_subblock_sums(qtype, _ptr(w), rows, K, _ptr(xq), _ptr(y), _ptr(S), _stream(stream)))


def q8k_debug_prefill_block_sums(qtype: int, w, rows: int, K: int, xq, M: int, y, I, stream=None) -> None:
    _check(lib.q8k_debug_prefill_block_sums(qtype, _ptr(w), rows, K, _ptr(xq), M, _ptr(y), _ptr(I),
                                            _stream(stream)))


def q8k_debug_moe_subblock_sums(qtype: int, w, E: int, rows: int, K: int, xq, T: int, ids, rw, topk: int, y, S,
                                stream=None) -> None:
    _check(lib.q8k_debug_moe_subblock_sums(qtype, _ptr(w), E, rows, K, _ptr(xq), T, _ptr(ids), _ptr(rw), topk,
                                           _ptr(y), _ptr(S), _stream(stream)))


def q8k_debug_wave_sums(out, stream=None) -> None:
    _check(lib.q8k_debug_wave_sums(_ptr(out), _stream(stream)))


def q8k_debug_last_launches() -> list:
    """Host kernel handles the calling thread's last operation enqueued, in order."""
    buf = (_P * 16)()
    n = int(lib.q8k_debug_last_launches(buf, 16))
    return [int(buf[i] or 0) for i in range(min(n, 16))] + [0] * max(0, n - 16)
