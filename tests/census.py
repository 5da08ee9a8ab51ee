"""The kernel census: every kernel compiled into libq8k.so must be value-checked
by some test against an oracle value ("One kernel, any device", section 5,
and "Language models on the device", section 6: after a test run every
registered kernel is credited by a value check or excused by name; running is
not coverage).

How a kernel is credited:
  * the library records, per calling thread, the host handles of the kernels
    its last operation enqueued (q8k_debug_last_launches);
  * the GPU tests call the library through ``tracked(q)``, which appends that
    record to ``CENSUS.pending`` after every operation;
  * the value-check helpers (gpu_helpers.assert_close / assert_exact, which
    compare with the oracle) move the pending kernels to ``CENSUS.checked``;
    comparisons of one kernel against another do not credit anything;
  * each GPU test starts with an empty pending list.

Kernel names come from the library's symbol table (``nm``): a kernel's host
handle is a data symbol whose demangled name is the kernel's signature, and
its run-time address is the symbol's value plus the library's load base
(known from an exported function's address).
"""
from __future__ import annotations

import ctypes
import functools
import subprocess


class Census:
    def __init__(self):
        self.pending: list[int] = []
        self.checked: set[int] = set()
        self.ran: set[int] = set()

    def note(self, handles):
        self.pending.extend(handles)
        self.ran.update(handles)

    def credit(self):
        self.checked.update(self.pending)
        self.pending.clear()


CENSUS = Census()

# Set by tests/conftest.py: the session selects every GPU test (a census over a
# partial run would be meaningless).
WHOLE_GPU_RUN = False


@functools.lru_cache(maxsize=1)
def kernel_table(lib_path: str):
    """-> (symbol value of q8k_act_bytes, {symbol value: demangled kernel name})."""
    out = subprocess.run(["nm", "-C", "--defined-only", lib_path], capture_output=True, text=True,
                         check=True).stdout
    kernels, anchor = {}, None
    for line in out.splitlines():
        parts = line.split(" ", 2)
        if len(parts) != 3:
            continue
        value, kind, name = parts
        if name == "q8k_act_bytes":
            anchor = int(value, 16)
        # kernel handles: data symbols named by a kernel signature in q8k
        elif kind in "dDvV" and name.endswith(")") and "q8k::" in name and "_kernel" in name:
            kernels[int(value, 16)] = name
    assert anchor is not None, "q8k_act_bytes not found in the symbol table"
    return anchor, kernels


def kernel_names(q) -> dict[int, str]:
    """{run-time handle address: kernel name} for every kernel in the library."""
    anchor, kernels = kernel_table(q.LIB_PATH)
    base = ctypes.cast(q.lib.q8k_act_bytes, ctypes.c_void_p).value - anchor
    return {base + v: n for v, n in kernels.items()}


def short(name: str) -> str:
    """'void q8k::ns::kern<1, true>(args)' -> 'kern<1, true>'."""
    head = name[: name.rfind("(")] if name.endswith(")") else name
    depth = 0
    for i in range(len(head) - 1, -1, -1):
        c = head[i]
        if c == ">":
            depth += 1
        elif c == "<":
            depth -= 1
        elif c == ":" and depth == 0:
            return head[i + 1:]
    return head


# Operations of the binding that launch kernels (everything else is sizing or
# error text).
_OPS = ("q8k_pack", "q8k_bind_q6k", "qmatvec", "qmatvec_batched", "qmatvec_f32", "qmatvec_moe", "qmatmul_prefill",
        "qmatmul_prefill_f32", "qmatmul_prefill_moe", "qmatmul_prefill_moe_noalloc", "q8k_debug_subblock_sums",
        "q8k_debug_prefill_block_sums", "q8k_debug_moe_subblock_sums", "q8k_debug_wave_sums")


class _Tracked:
    """The binding module with every operation followed by a census note."""

    def __init__(self, q):
        self._q = q

    def __getattr__(self, name):
        v = getattr(self._q, name)
        if name not in _OPS:
            return v

        def call(*a, **k):
            try:
                return v(*a, **k)
            finally:
                CENSUS.note(self._q.q8k_debug_last_launches())

        return call


def tracked(q):
    return _Tracked(q)
