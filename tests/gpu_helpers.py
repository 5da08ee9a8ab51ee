"""Device-side helpers for the GPU parity tests (torch for memory only).

The value checks here (assert_close, assert_exact) compare a GPU result with
the oracle; a passing check credits the kernels that the test's calls have
launched since the last check (census.CENSUS).
"""
from __future__ import annotations

import numpy as np

from census import CENSUS

TOL_REL = 1e-5  # |err| <= 1e-5 * sum|terms| + 1e-6  (fp32 outputs)
TOL_ABS = 1e-6


def dev():
    import torch

    return torch.device("cuda")


def to_dev(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def poisoned(nbytes: int):
    """A fresh device byte buffer filled with 0xFF (reads as NaN if unwritten)."""
    import torch

    return torch.full((max(nbytes, 16),), 0xFF, dtype=torch.uint8, device=dev())


def poisoned_f32(*shape):
    import torch

    return poisoned(4 * int(np.prod(shape))).view(torch.float32)[: int(np.prod(shape))].view(*shape)


def poisoned_i32(*shape):
    import torch

    return poisoned(4 * int(np.prod(shape))).view(torch.int32)[: int(np.prod(shape))].view(*shape)


def host(t) -> np.ndarray:
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()


def pack_on_device(q, x: np.ndarray):
    """fp32 [T, K] -> device q8_K buffer (packed by the HIP kernel)."""
    T, K = x.shape
    xd = to_dev(x.astype(np.float32))
    xq = poisoned(q.q8k_act_bytes(T, K))
    q.q8k_pack(xd, T, K, xq)
    return xq


def split_act(q, xq_host: np.ndarray, T: int, K: int):
    total, od, ob = q.q8k_act_layout(T, K)
    nb = K // 256
    qs = xq_host[: T * K].view(np.int8).reshape(T, K)
    d = xq_host[od: od + 4 * T * nb].view(np.float32).reshape(T, nb)
    bs = xq_host[ob: ob + 2 * 8 * T * nb].view(np.int16).reshape(T, nb * 8)
    return qs, d, bs


def assert_exact(got: np.ndarray, want: np.ndarray, what: str = ""):
    """Bit-exact equality with an oracle value (integers, bytes); credits the
    pending kernels."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype.kind == "f":
        same = np.array_equal(got.view(np.uint32 if got.itemsize == 4 else np.uint64),
                              want.astype(got.dtype).view(np.uint32 if got.itemsize == 4 else np.uint64))
    else:
        same = np.array_equal(got.astype(np.int64), want.astype(np.int64))
    if not same:
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} entries differ from the oracle; first at {tuple(bad[0])}: "
                             f"got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")
    CENSUS.credit()


def assert_close(got: np.ndarray, want: np.ndarray, A: np.ndarray, what: str = ""):
    """|err| <= 1e-5 * A + 1e-6 against the oracle (fp32 outputs); credits the
    pending kernels."""
    got = np.asarray(got, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output (an unwritten element?)"
    err = np.abs(got - want)
    bound = TOL_REL * A + TOL_ABS
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} outputs out of tolerance; worst at {i}: got {got[i]!r} "
                             f"want {want[i]!r} err {err[i]:.3g} bound {bound[i]:.3g}")
    CENSUS.credit()
