#!/usr/bin/env python3
"""Benchmark of the q8_K-packed K-quant path on one MI355X.

Headline (one JSON line on stdout): the 4096x4096 Q4_K decode step -- pack one
fp32 token into q8_K on the device, then the Q4_K mat-vec -- as algorithmic
HBM GB/s.  The other workloads of the path (Q6_K output-head decode, MoE
decode, 512-token prefill GEMM, batched decode, the q8_K pack of a prefill
batch) are measured in the same run and reported under "workloads".

Protocol (measurement discipline of "One kernel, any device", section 5, and
the five interleaved rounds / medians of its section 4.2):
  * inputs are resident in HBM before timing starts;
  * weights are rotated through R distinct copies whose total is at least 2x
    the 256 MB Infinity Cache, so every weight read comes from HBM;
  * W untimed eager warmup steps; then the K steps are captured once into a
    HIP graph (launch-bound decode loops are replayed as graphs, so host
    launch overhead does not pace the GPU), the graph is replayed once
    untimed, and exactly K steps are timed as one replay between two device
    synchronisations;
  * the dominant kernel's per-launch duration comes from HIP events on the
    stream it runs on, bracketing a replayed graph of back-to-back launches
    of that kernel alone (rotating weight copies);
  * a workload's numbers are reported together with its parity result
    against the CPU oracle, computed in the same run.

The CPU baseline is the oracle as it stands (plain C, not tuned), timed on
this host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_K decode mat-vec HBM GB/s (% of peak); prefill int8 TOPS (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POP/s
HEADLINE_KERNEL = "matvec_f32_q4k_kernel<1, 2, false>"  # the one launch of the headline decode step
MALL_BYTES = 256 << 20         # Infinity Cache
TOL_REL, TOL_ABS = 1e-5, 1e-6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


_CS = "quantized_q8kpack_fp32_amd/csrc/"
KERNEL_SOURCES = {
    "matvec_q4k": [_CS + "matvec.hip", _CS + "kquant.h", _CS + "q8k_device.h"],
    "matvec_q6k": [_CS + "matvec.hip", _CS + "kquant.h", _CS + "q8k_device.h"],
    "moe": [_CS + "moe_mfma.hip", _CS + "q4k_planes.h", _CS + "q8k_device.h"],
    "matvec_q5k": [_CS + "matvec.hip", _CS + "kquant.h", _CS + "q8k_device.h"],
    "moe_q5k": [_CS + "moe_mfma.hip", _CS + "q4k_planes.h", _CS + "q8k_device.h"],
    "moe_q6k": [_CS + "moe_mfma.hip", _CS + "q4k_planes.h", _CS + "q8k_device.h"],
    "prefill_q4k": [_CS + "prefill_regw.hip", _CS + "q4k_planes.h", _CS + "q8k_device.h"],
    "moe_prefill_q4k": [_CS + "prefill_regw.hip", _CS + "q4k_planes.h", _CS + "prefill.hip", _CS + "q8k_device.h"],
    "prefill_q5k": [_CS + "prefill.hip", _CS + "q8k_device.h"],
    "prefill_q4k_m32": [_CS + "prefill_regw.hip", _CS + "prefill.hip", _CS + "q4k_planes.h", _CS + "q8k_device.h"],
    "prefill_q4k_m128": [_CS + "prefill_regw.hip", _CS + "prefill.hip", _CS + "q4k_planes.h", _CS + "q8k_device.h"],
    "prefill_q6k": [_CS + "prefill.hip", _CS + "q8k_device.h"],
    "moe_prefill_q6k": [_CS + "prefill.hip", _CS + "q8k_device.h"],
    "moe_prefill_q5k": [_CS + "prefill.hip", _CS + "q8k_device.h"],
    "pack": [_CS + "pack.hip", _CS + "q8k_device.h", _CS + "q8k_quant.h"],
    "fused_q4k": [_CS + "matvec.hip", _CS + "kquant.h", _CS + "q8k_device.h", _CS + "q8k_quant.h"],
    "batched_q4k_c4": [_CS + "matvec.hip", _CS + "kquant.h", _CS + "q8k_device.h", _CS + "q8k_quant.h"],
    "batched_q4k_c8": [_CS + "matvec.hip", _CS + "kquant.h", _CS + "q8k_device.h", _CS + "q8k_quant.h"],
    "fused_q5k": [_CS + "matvec.hip", _CS + "kquant.h", _CS + "q8k_device.h", _CS + "q8k_quant.h"],
    "fused_q6k": [_CS + "matvec.hip", _CS + "kquant.h", _CS + "q8k_device.h", _CS + "q8k_quant.h"],
    "prefill_f32_q4k": [_CS + "prefill_regw.hip", _CS + "prefill_pack.h", _CS + "q4k_planes.h", _CS + "q8k_device.h",
                        _CS + "q8k_quant.h"],
    "prefill_f32_q6k": [_CS + "prefill.hip", _CS + "prefill_pack.h", _CS + "q8k_device.h", _CS + "q8k_quant.h"],
}


def traffic_record(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    the kernel's source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_sha") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- helpers
def graph_of(torch, fn, n):
    """Capture fn(0..n-1) into one HIP graph on a side stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    return g


def replay_us(torch, g, n, reps=1):
    """Mean per-call time of a graph of n calls, from HIP events on the
    replay stream (torch's current stream)."""
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / (n * reps)


class StreamCalib:
    """The plain streaming read of quantized_q8kpack_fp32_amd/csrc/calib.hip
    (libq8k_calib.so, a library of its own): the time one read of N bytes
    takes, over rotated buffers like the workloads' weights, as the
    practical ceiling each bandwidth-bound workload is read against."""

    def __init__(self, torch):
        import ctypes

        path = os.path.join(ROOT, "quantized_q8kpack_fp32_amd", "libq8k_calib.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} missing: build first (__graft_entry__.build())")
        self.torch = torch
        self.lib = ctypes.CDLL(path)
        self.lib.q8k_calib_stream_read.restype = ctypes.c_int
        self.lib.q8k_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                                   ctypes.c_void_p]
        self.lib.q8k_calib_stream_variants.restype = ctypes.c_int
        self.nvar = int(self.lib.q8k_calib_stream_variants())
        self.lib.q8k_calib_stream_workgroups.restype = ctypes.c_int64
        self.lib.q8k_calib_stream_workgroups.argtypes = [ctypes.c_int64]
        self.cache = {}

    def sweep(self, nbytes: int) -> dict:
        """Per-variant times (us per launch) of a streaming read of nbytes."""
        self.cache.pop(-(-nbytes // 16) * 16, None)
        self.per_variant = {}
        self.us(nbytes)
        return dict(self.per_variant)

    def us(self, nbytes: int) -> float:
        """Mean per-launch time of a streaming read of nbytes (graph of >= 64
        back-to-back launches over R rotated copies totalling >= 2x the MALL),
        the fastest of the kernel's variants."""
        torch = self.torch
        n = -(-nbytes // 16) * 16
        if n in self.cache:
            return self.cache[n]
        R = rotations(n)
        bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(R)]
        sink = torch.empty(int(self.lib.q8k_calib_stream_workgroups(n)), dtype=torch.int32, device="cuda")

        best = None
        for v in range(self.nvar):
            def launch(i, v=v):
                st = self.lib.q8k_calib_stream_read(bufs[i % R].data_ptr(), n, sink.data_ptr(), v,
                                                    torch.cuda.current_stream().cuda_stream)
                assert st == 0, f"stream read launch failed ({st})"

            for i in range(R):
                launch(i)
            torch.cuda.synchronize()
            k = R * max(1, -(-64 // R))
            g = graph_of(torch, launch, k)
            t = replay_us(torch, g, k, reps=2)
            del g
            if hasattr(self, "per_variant"):
                self.per_variant[v] = round(t, 3)
            best = t if best is None else min(best, t)
        t = best
        del bufs, sink
        torch.cuda.empty_cache()
        self.cache[n] = t
        return t


def close(got, want, A):
    got = np.asarray(got, np.float64)
    return bool(np.isfinite(got).all() and (np.abs(got - want) <= TOL_REL * A + TOL_ABS).all())


def otime(wl, fn, *a, **k):
    """Call an oracle function, adding its wall time to wl.oracle_s (the
    oracle's time for the workload's step, on ncores() threads)."""
    t0 = time.perf_counter()
    r = fn(*a, **k)
    wl.oracle_s = getattr(wl, "oracle_s", 0.0) + time.perf_counter() - t0
    return r


def rotations(nbytes: int, minimum: int = 2) -> int:
    return max(minimum, -(-2 * MALL_BYTES // max(nbytes, 1)))


# ---------------------------------------------------------------- workloads
_BLOCK_BYTES = {"q4k": 144, "q5k": 176, "q6k": 210}


def _oracle_qtype(oracle, fmt):
    return {"q4k": oracle.Q4_K, "q5k": oracle.Q5_K, "q6k": oracle.Q6_K}[fmt]


class Decode:
    """One token through q8k_pack + qmatvec (Q4_K, Q5_K or relaid Q6_K); with
    fused=True through the one-launch qmatvec_f32 instead."""

    def __init__(self, q, torch, fmt, rows, K, seed, R=None, fused=False):
        import synth

        self.q, self.torch, self.fmt, self.rows, self.K, self.fused = q, torch, fmt, rows, K, fused
        g = np.random.default_rng(seed)
        dev = torch.device("cuda")
        if fmt in ("q4k", "q5k"):
            self.w_host = (synth.q4k_weights if fmt == "q4k" else synth.q5k_weights)(g, rows, K)
            w0 = torch.from_numpy(self.w_host).to(dev)
            self.qt = q.Q8K_Q4_K if fmt == "q4k" else q.Q8K_Q5_K
        else:
            self.w_host = synth.q6k_weights(g, rows, K)
            wg = torch.from_numpy(self.w_host).to(dev)
            w0 = torch.empty(q.q8k_weight_bytes(q.Q8K_Q6_K_RELAID, rows, K), dtype=torch.uint8, device=dev)
            q.q8k_bind_q6k(wg, rows, K, w0)
            del wg
            self.qt = q.Q8K_Q6_K_RELAID
        self.wbytes_alg = rows * (K // 256) * _BLOCK_BYTES[fmt]
        self.R = R or rotations(w0.numel())
        self.ws = [w0] + [w0.clone() for _ in range(self.R - 1)]
        self.x_host = synth.activations(g, 1, K)
        self.x = torch.from_numpy(self.x_host).to(dev)
        self.xq = torch.empty(q.q8k_act_bytes(1, K), dtype=torch.uint8, device=dev)
        self.y = torch.empty(rows, dtype=torch.float32, device=dev)
        nb = K // 256
        # algorithmic bytes: weight once, q8_K codes+scales (+ sums for Q4_K/Q5_K) once, output once
        self.mv_bytes = self.wbytes_alg + K + 4 * nb + (16 * nb if fmt != "q6k" else 0) + 4 * rows
        self.pack_bytes = 4 * K + K + 4 * nb + 16 * nb
        self.step_bytes = self.mv_bytes + self.pack_bytes
        if fused:
            # one launch: weight once, fp32 activations in, output out
            self.mv_bytes = self.step_bytes = self.wbytes_alg + 4 * K + 4 * rows

    def step(self, i):
        if not self.fused:
            self.q.q8k_pack(self.x, 1, self.K, self.xq)
        self.main(i)

    def main(self, i):
        if self.fused:
            self.q.qmatvec_f32(self.qt, self.ws[i % self.R], self.rows, self.K, self.x, 1, self.y, None)
        else:
            self.q.qmatvec(self.qt, self.ws[i % self.R], self.rows, self.K, self.xq, self.y)

    def parity(self):
        import oracle

        self.step(0)
        got = self.y.cpu().numpy()
        qs, d, bs = otime(self, oracle.q8k_pack, self.x_host)
        want, A = otime(self, oracle.matvec, _oracle_qtype(oracle, self.fmt), self.w_host, self.rows, self.K, qs, d, bs,
                                nthreads=ncores())
        return close(got, want[0], A[0])


class Batched(Decode):
    def __init__(self, q, torch, fmt, rows, K, seed, ncols):
        super().__init__(q, torch, fmt, rows, K, seed)
        import synth

        self.ncols = ncols
        g = np.random.default_rng(seed + 1)
        self.x_host = synth.activations(g, ncols, K)
        dev = torch.device("cuda")
        self.x = torch.from_numpy(self.x_host).to(dev)
        self.xq = torch.empty(q.q8k_act_bytes(ncols, K), dtype=torch.uint8, device=dev)
        self.y = torch.empty(ncols * rows, dtype=torch.float32, device=dev)
        nb = K // 256
        self.mv_bytes = self.wbytes_alg + ncols * (K + 4 * nb + 16 * nb + 4 * rows)

    def step(self, i):
        self.q.q8k_pack(self.x, self.ncols, self.K, self.xq)
        self.main(i)

    def main(self, i):
        self.q.qmatvec_batched(self.qt, self.ws[i % self.R], self.rows, self.K, self.xq, self.ncols, self.y)

    def parity(self):
        import oracle

        self.step(0)
        got = self.y.cpu().numpy().reshape(self.ncols, self.rows)
        qs, d, bs = otime(self, oracle.q8k_pack, self.x_host)
        want, A = otime(self, oracle.matvec, _oracle_qtype(oracle, self.fmt), self.w_host, self.rows, self.K, qs, d, bs,
                                nthreads=ncores())
        return close(got, want, A)


class MoE:
    """16 tokens, top-2 of 8 Q4_K (or Q5_K) experts of 14336 x 4096: pack + qmatvec_moe."""

    def __init__(self, q, torch, E=8, rows=14336, K=4096, T=16, topk=2, seed=3, fmt="q4k"):
        import synth

        self.q, self.torch, self.E, self.rows, self.K, self.T, self.topk = q, torch, E, rows, K, T, topk
        self.fmt = fmt
        self.qt, gen = _prefill_format(q, synth, fmt)  # Q4_K, Q5_K or relaid Q6_K
        g = np.random.default_rng(seed)
        dev = torch.device("cuda")
        self.w_host = gen(g, E * rows, K)
        w0 = _device_weight(q, torch, fmt, self.w_host, E * rows, K)
        self.R = rotations(w0.numel())
        self.ws = [w0] + [w0.clone() for _ in range(self.R - 1)]
        self.x_host = synth.activations(g, T, K)
        self.ids_host, self.rw_host = synth.moe_routing(g, T, E, topk)
        self.x = torch.from_numpy(self.x_host).to(dev)
        self.ids = torch.from_numpy(self.ids_host).to(dev)
        self.rw = torch.from_numpy(self.rw_host).to(dev)
        self.xq = torch.empty(q.q8k_act_bytes(T, K), dtype=torch.uint8, device=dev)
        self.y = torch.empty(T * rows, dtype=torch.float32, device=dev)
        nb = K // 256
        hit = len(set(self.ids_host.ravel().tolist()))
        self.experts_hit = hit
        self.mv_bytes = hit * rows * nb * _BLOCK_BYTES[fmt] + T * (K + 20 * nb) + 8 * T * topk + 4 * T * rows
        self.pack_bytes = T * (4 * K + K + 20 * nb)
        self.step_bytes = self.mv_bytes + self.pack_bytes

    def step(self, i):
        self.q.q8k_pack(self.x, self.T, self.K, self.xq)
        self.main(i)

    def main(self, i):
        self.q.qmatvec_moe(self.qt, self.ws[i % self.R], self.E, self.rows, self.K, self.xq, self.T,
                           self.ids, self.rw, self.topk, self.y)

    def parity(self):
        import oracle

        self.step(0)
        got = self.y.cpu().numpy().reshape(self.T, self.rows)
        qs, d, bs = otime(self, oracle.q8k_pack, self.x_host)
        want, A = otime(self, oracle.moe, _oracle_qtype(oracle, self.fmt), self.w_host, self.E, self.rows, self.K, qs, d, bs,
                             self.ids_host, self.rw_host, nthreads=ncores())
        return close(got, want, A)


def _prefill_format(q, synth, fmt):
    return {"q4k": (q.Q8K_Q4_K, synth.q4k_weights), "q5k": (q.Q8K_Q5_K, synth.q5k_weights),
            "q6k": (q.Q8K_Q6_K_RELAID, synth.q6k_weights)}[fmt]


def _device_weight(q, torch, fmt, w_host, nrows, K):
    """GGUF blocks on the device in the form the kernels read (Q6_K: relaid at bind)."""
    wg = torch.from_numpy(w_host).to(torch.device("cuda"))
    if fmt != "q6k":
        return wg
    w0 = torch.empty(q.q8k_weight_bytes(q.Q8K_Q6_K_RELAID, nrows, K), dtype=torch.uint8, device=wg.device)
    q.q8k_bind_q6k(wg, nrows, K, w0)
    return w0


class Prefill:
    """512 tokens through q8k_pack + qmatmul_prefill against a 4096 x 14336 Q4_K (Q5_K, relaid Q6_K) weight."""

    def __init__(self, q, torch, rows=4096, K=14336, M=512, seed=4, fmt="q4k"):
        import synth

        self.q, self.torch, self.rows, self.K, self.M, self.fmt = q, torch, rows, K, M, fmt
        self.qt, gen = _prefill_format(q, synth, fmt)
        g = np.random.default_rng(seed)
        dev = torch.device("cuda")
        self.w_host = gen(g, rows, K)
        w0 = _device_weight(q, torch, fmt, self.w_host, rows, K)
        self.R = rotations(w0.numel())
        self.ws = [w0] + [w0.clone() for _ in range(self.R - 1)]
        self.x_host = synth.activations(g, M, K)
        self.x = torch.from_numpy(self.x_host).to(dev)
        self.xq = torch.empty(q.q8k_act_bytes(M, K), dtype=torch.uint8, device=dev)
        self.y = torch.empty(M * rows, dtype=torch.float32, device=dev)
        self.ws_bytes = q.qmatmul_prefill_workspace_bytes(self.qt, rows, K, M)
        self.wsp = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev) if self.ws_bytes else None
        self.ops = 2 * M * rows * K
        nb = K // 256
        self.pack_bytes = M * (4 * K + K + 20 * nb)

    def step(self, i):
        self.q.q8k_pack(self.x, self.M, self.K, self.xq)
        self.main(i)

    def main(self, i):
        self.q.qmatmul_prefill(self.qt, self.ws[i % self.R], self.rows, self.K, self.xq, self.M, self.y, self.wsp,
                               self.ws_bytes)

    def parity(self):
        import oracle

        self.step(0)
        got = self.y.cpu().numpy().reshape(self.M, self.rows)
        qs, d, bs = otime(self, oracle.q8k_pack, self.x_host)
        want, A = otime(self, oracle.matvec, _oracle_qtype(oracle, self.fmt), self.w_host, self.rows, self.K, qs, d, bs,
                                nthreads=ncores())
        return close(got, want, A)  # every output


def pack_parity(q, torch, p) -> bool:
    """The packed buffer the replays left in p.xq against the oracle's q8k_pack of
    the same tokens: codes, scales and sub-block sums, byte for byte."""
    import oracle

    torch.cuda.synchronize()
    buf = p.xq.cpu().numpy()
    _, od, ob = q.q8k_act_layout(p.M, p.K)
    nb = p.K // 256
    qs, d, bs = oracle.q8k_pack(p.x_host)
    return (buf[: p.M * p.K].view(np.int8).tobytes() == qs.tobytes()
            and buf[od: od + 4 * p.M * nb].tobytes() == d.tobytes()
            and buf[ob: ob + 16 * p.M * nb].tobytes() == bs.tobytes())


class PrefillF32(Prefill):
    """The same step from fp32 tokens as one call: qmatmul_prefill_f32 packs
    the tokens inside the GEMM launch (xq receives q8k_pack's bytes)."""

    def __init__(self, q, torch, **kw):
        super().__init__(q, torch, **kw)
        self.ws_bytes = q.qmatmul_prefill_f32_workspace_bytes(self.qt, self.rows, self.K, self.M)
        # sync words zero before the first call; every call leaves them so
        self.wsp = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=torch.device("cuda"))

    def step(self, i):
        self.main(i)

    def main(self, i):
        self.q.qmatmul_prefill_f32(self.qt, self.ws[i % self.R], self.rows, self.K, self.x, self.M, self.xq, self.y,
                                   self.wsp, self.ws_bytes)

    def parity(self):
        ok = super().parity()  # one call, every output against the oracle
        sync = self.wsp[:256].cpu().numpy().view(np.int32)
        return ok and not sync.any()


class MoEPrefill:
    """512 tokens, top-2 of 8 Q4_K (Q5_K, relaid Q6_K) experts of 14336 x 4096: pack + qmatmul_prefill_moe."""

    def __init__(self, q, torch, E=8, rows=14336, K=4096, T=512, topk=2, seed=7, fmt="q4k"):
        import synth

        self.q, self.torch, self.E, self.rows, self.K, self.T, self.topk = q, torch, E, rows, K, T, topk
        self.fmt = fmt
        self.qt, gen = _prefill_format(q, synth, fmt)
        g = np.random.default_rng(seed)
        dev = torch.device("cuda")
        self.w_host = gen(g, E * rows, K)
        w0 = _device_weight(q, torch, fmt, self.w_host, E * rows, K)
        self.R = rotations(w0.numel())
        self.ws = [w0] + [w0.clone() for _ in range(self.R - 1)]
        self.x_host = synth.activations(g, T, K)
        self.ids_host, self.rw_host = synth.moe_routing(g, T, E, topk)
        self.x = torch.from_numpy(self.x_host).to(dev)
        self.ids = torch.from_numpy(self.ids_host).to(dev)
        self.rw = torch.from_numpy(self.rw_host).to(dev)
        self.xq = torch.empty(q.q8k_act_bytes(T, K), dtype=torch.uint8, device=dev)
        self.y = torch.empty(T * rows, dtype=torch.float32, device=dev)
        self.ws_bytes = q.qmatmul_prefill_moe_workspace_bytes(self.qt, E, rows, K, T, topk)
        self.wsp = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        # useful int8 operations: every (token, slot) pair against its expert's rows
        self.ops = 2 * T * topk * rows * K
        nb = K // 256
        self.pack_bytes = T * (4 * K + K + 20 * nb)

    def step(self, i):
        self.q.q8k_pack(self.x, self.T, self.K, self.xq)
        self.main(i)

    def main(self, i):
        self.q.qmatmul_prefill_moe(self.qt, self.ws[i % self.R], self.E, self.rows, self.K, self.xq, self.T,
                                   self.ids, self.rw, self.topk, self.y, self.wsp, self.ws_bytes)

    def parity(self):
        """Every token against the oracle's MoE (the same per-token formula)."""
        import oracle

        self.step(0)
        got = self.y.cpu().numpy().reshape(self.T, self.rows)
        qs, d, bs = otime(self, oracle.q8k_pack, self.x_host)
        want, A = otime(self, oracle.moe, _oracle_qtype(oracle, self.fmt), self.w_host, self.E, self.rows, self.K, qs, d, bs,
                             self.ids_host, self.rw_host, nthreads=ncores())
        return close(got, want, A)


def ncores() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


TIMING_ROUNDS = 5


def rounds_summary(r):
    """Median, min and spread ((max - min) / median) of per-round times."""
    m = float(np.median(r))
    return {"rounds": len(r), "median": round(m, 3), "min": round(min(r), 3),
            "spread": round((max(r) - min(r)) / m, 4)}


def run_timed(torch, wl, steps, warmup):
    """-> (seconds per step over exactly `steps` timed steps, dominant-kernel us
    per launch (the median of TIMING_ROUNDS replays), the per-round times)."""
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    g = graph_of(torch, wl.step, steps)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del g
    n = wl.R * max(1, -(-64 // wl.R))  # whole rotations, at least 64 launches
    gk = graph_of(torch, wl.main, n)
    rounds = [replay_us(torch, gk, n) for _ in range(TIMING_ROUNDS)]
    del gk
    return (t1 - t0) / steps, float(np.median(rounds)), rounds


# ---------------------------------------------------------------- CPU baseline
def gpu_env(torch) -> dict:
    """The device and software the figures were measured on."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": rocm, "hip_runtime": torch.version.hip,
            "torch": torch.__version__}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s: float):
    """The oracle's pack + Q4_K mat-vec of the 4096x4096 decode step, timed on
    this host: three runs of about budget_s / 6 seconds each with one thread
    and with all usable cores (rows split over threads); medians of the three."""
    import oracle
    import synth

    oracle.build()
    g = np.random.default_rng(1)
    rows, K = 4096, 4096
    w = synth.q4k_weights(g, rows, K)
    x = synth.activations(g, 1, K)
    nb = K // 256
    step_bytes = rows * nb * 144 + K + 20 * nb + 4 * rows + 4 * K + K + 20 * nb

    def run(nth, seconds):
        n, t0 = 0, time.perf_counter()
        while True:
            qs, d, bs = oracle.q8k_pack(x)
            oracle.matvec(oracle.Q4_K, w, rows, K, qs, d, bs, nthreads=nth)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                return (time.perf_counter() - t0) / n, n

    out = {}
    for label, nth in (("one_thread", 1), ("all_cores", ncores())):
        runs = sorted(run(nth, budget_s / 6) for _ in range(3))
        dt, n = runs[1]
        out[label] = {"threads": nth, "ms_per_step": round(dt * 1e3, 3), "GB/s": round(step_bytes / dt / 1e9, 4),
                      "runs_ms": [round(r[0] * 1e3, 3) for r in runs], "steps_in_median_run": n}
    allc = out["all_cores"]
    return {"value": allc["GB/s"], "unit": "GB/s", "cores": allc["threads"], "kind": "oracle",
            "sample": f"the 4096x4096 Q4_K decode step (q8_K pack + mat-vec, fp64 epilogue), repeated for about "
                      f"{budget_s / 6:.1f} s per run; median of 3 runs; value = all {allc['threads']} threads, "
                      f"{allc['ms_per_step']} ms per step; one thread {out['one_thread']['ms_per_step']} ms per step",
            "cpu_model": cpu_model(), "one_thread": out["one_thread"], "all_cores": allc}


def cpu_configs():
    """The oracle on the other configurations, on this host, with one thread
    and with all usable cores: the 32000x4096 Q6_K and the 8-expert MoE decode
    steps (pack + product, medians of 3 runs each), and the 512-token prefill
    (one all-core run over the full output; one thread on 16 of its 512 token
    rows, scaled by 32).  Same shapes, seeds and input recipes as the
    workloads; the oracle's time does not depend on the values."""
    import oracle
    import synth

    oracle.build()
    nth = ncores()

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)

    out = {}
    g = np.random.default_rng(2)
    rows, K = 32000, 4096
    w = synth.q6k_weights(g, rows, K)
    x = synth.activations(g, 1, K)

    def q6(n):
        qs, d, bs = oracle.q8k_pack(x)
        oracle.matvec(oracle.Q6_K, w, rows, K, qs, d, bs, nthreads=n)

    t1, ta = timed(lambda: q6(1), 3), timed(lambda: q6(nth), 3)
    out["decode_q6k_32000x4096"] = {"one_thread_ms": round(t1[1] * 1e3, 3), "all_cores_ms": round(ta[1] * 1e3, 3),
                                     "threads": nth, "runs": "median of 3"}
    del w
    g = np.random.default_rng(3)
    E, rows, K, T, topk = 8, 14336, 4096, 16, 2
    w = synth.q4k_weights(g, E * rows, K)
    x = synth.activations(g, T, K)
    ids, rw = synth.moe_routing(g, T, E, topk)

    def moe(n):
        qs, d, bs = oracle.q8k_pack(x)
        oracle.moe(oracle.Q4_K, w, E, rows, K, qs, d, bs, ids, rw, nthreads=n)

    t1, ta = timed(lambda: moe(1), 3), timed(lambda: moe(nth), 3)
    out["moe_q4k_8x14336x4096_t16_top2"] = {"one_thread_ms": round(t1[1] * 1e3, 3),
                                             "all_cores_ms": round(ta[1] * 1e3, 3), "threads": nth,
                                             "runs": "median of 3"}
    del w
    g = np.random.default_rng(4)
    rows, K, M = 4096, 14336, 512
    w = synth.q4k_weights(g, rows, K)
    x = synth.activations(g, M, K)

    def pf(xx, n):
        qs, d, bs = oracle.q8k_pack(xx)
        oracle.matvec(oracle.Q4_K, w, rows, K, qs, d, bs, nthreads=n)

    ta = timed(lambda: pf(x, nth), 1)
    t1 = timed(lambda: pf(x[:16], 1), 1)
    out["prefill_q4k_4096x14336_m512"] = {"one_thread_ms": round(t1[0] * 32 * 1e3, 1),
                                           "all_cores_ms": round(ta[0] * 1e3, 1), "threads": nth,
                                           "runs": "one run each; one thread on 16 of the 512 token rows, x 32"}
    return out


# ---------------------------------------------------------------- profiling
PROFILE_TARGETS = {
    "decode_q4k": "qmatvec on the 4096x4096 Q4_K decode workload",
    "decode_q6k": "qmatvec on the 32000x4096 relaid Q6_K workload",
    "moe": "qmatvec_moe on the 8 x 14336x4096 Q4_K, 16-token top-2 workload",
    "decode_q5k": "qmatvec on the 4096x4096 Q5_K decode workload",
    "fused_q4k": "qmatvec_f32 (pack inside the launch) on the 4096x4096 Q4_K decode workload",
    "batched4": "qmatvec_batched, 4 packed columns, on the 4096x4096 Q4_K workload",
    "batched8": "qmatvec_batched, 8 packed columns, on the 4096x4096 Q4_K workload",
    "fused_q5k": "qmatvec_f32 (pack inside the launch) on the 4096x4096 Q5_K decode workload",
    "fused_q6k": "qmatvec_f32 (pack inside the launch) on the 32000x4096 relaid Q6_K workload",
    "moe_q5k": "qmatvec_moe on the 8 x 14336x4096 Q5_K, 16-token top-2 workload",
    "moe_q6k": "qmatvec_moe on the 8 x 14336x4096 relaid Q6_K, 16-token top-2 workload",
    "prefill": "qmatmul_prefill on the 4096x14336 Q4_K, 512-token workload",
    "moe_prefill": "qmatmul_prefill_moe on the 8 x 14336x4096 Q4_K, 512-token top-2 workload",
    "prefill_q5k": "qmatmul_prefill on the 4096x14336 Q5_K, 512-token workload",
    "moe_prefill_q5k": "qmatmul_prefill_moe on the 8 x 14336x4096 Q5_K, 512-token top-2 workload",
    "prefill_q6k": "qmatmul_prefill on the 4096x14336 relaid Q6_K, 512-token workload",
    "moe_prefill_q6k": "qmatmul_prefill_moe on the 8 x 14336x4096 relaid Q6_K, 512-token top-2 workload",
    "pack": "q8k_pack of 512 x 14336 fp32 activations",
    "prefill_m32": "qmatmul_prefill (split-K and fixup) on the 4096x14336 Q4_K, 32-token workload",
    "prefill_m128": "qmatmul_prefill (split-K and fixup) on the 4096x14336 Q4_K, 128-token workload",
    "prefill_f32": "qmatmul_prefill_f32 (q8_K pack inside the launch) on the 4096x14336 Q4_K, 512-token workload",
    "prefill_f32_q6k": "qmatmul_prefill_f32 (q8_K pack inside the launch) on the 4096x14336 relaid Q6_K, 512-token "
                       "workload",
    "copy": "a plain 256 MiB device-to-device copy (torch), the counter calibration reference",
}


def profile_run(q, torch, target, launches):
    """A few eager launches of one kernel with its inputs already resident, so
    that one rocprofv3 counter pass sees only that kernel's dispatches."""
    if target == "copy":
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(launches):
            dst.copy_(src)
    else:
        wl = {"decode_q4k": lambda: Decode(q, torch, "q4k", 4096, 4096, seed=1),
              "decode_q6k": lambda: Decode(q, torch, "q6k", 32000, 4096, seed=2),
              "moe": lambda: MoE(q, torch),
              "decode_q5k": lambda: Decode(q, torch, "q5k", 4096, 4096, seed=5),
              "fused_q4k": lambda: Decode(q, torch, "q4k", 4096, 4096, seed=1, fused=True),
              "batched4": lambda: Batched(q, torch, "q4k", 4096, 4096, seed=1, ncols=4),
              "batched8": lambda: Batched(q, torch, "q4k", 4096, 4096, seed=1, ncols=8),
              "fused_q5k": lambda: Decode(q, torch, "q5k", 4096, 4096, seed=5, fused=True),
              "fused_q6k": lambda: Decode(q, torch, "q6k", 32000, 4096, seed=2, fused=True),
              "moe_q5k": lambda: MoE(q, torch, seed=6, fmt="q5k"),
              "moe_q6k": lambda: MoE(q, torch, seed=14, fmt="q6k"),
              "prefill": lambda: Prefill(q, torch),
              "moe_prefill": lambda: MoEPrefill(q, torch),
              "prefill_q5k": lambda: Prefill(q, torch, seed=8, fmt="q5k"),
              "moe_prefill_q5k": lambda: MoEPrefill(q, torch, seed=9, fmt="q5k"),
              "prefill_q6k": lambda: Prefill(q, torch, seed=10, fmt="q6k"),
              "moe_prefill_q6k": lambda: MoEPrefill(q, torch, seed=11, fmt="q6k"),
              "pack": lambda: Prefill(q, torch),
              "prefill_m32": lambda: Prefill(q, torch, M=32, seed=12),
              "prefill_m128": lambda: Prefill(q, torch, M=128, seed=13),
              "prefill_f32": lambda: PrefillF32(q, torch),
              "prefill_f32_q6k": lambda: PrefillF32(q, torch, seed=10, fmt="q6k")}[target]()
        wl.step(0)
        torch.cuda.synchronize()
        for i in range(launches):
            if target == "pack":
                q.q8k_pack(wl.x, wl.M, wl.K, wl.xq)
            else:
                wl.main(i)
    torch.cuda.synchronize()
    print(json.dumps({"profiled": target, "launches": launches, "what": PROFILE_TARGETS[target]}), flush=True)


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only-headline", action="store_true", help="skip the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", choices=sorted(PROFILE_TARGETS), default=None,
                    help="run only a few launches of one workload's kernel (for rocprofv3 counter passes)")
    ap.add_argument("--launches", type=int, default=8)
    ap.add_argument("--stream-sweep", action="store_true",
                    help="print the streaming-read calibration's per-variant times for the decode workloads' sizes")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (--gpus {args.gpus} requested); "
              "sharding across GPUs is described in the design notes but not implemented", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import quantized_q8kpack_fp32_amd as q

    if args.profile:
        profile_run(q, torch, args.profile, args.launches)
        return
    if args.stream_sweep:
        calib = StreamCalib(torch)
        for n in (9469952, 11567104, 37273600, 107652160, 265229568, 1 << 30):
            t = calib.sweep(n)
            print(json.dumps({"bytes": n, "R": rotations(-(-n // 16) * 16), "us": t,
                              "best_TBs": round(n / min(t.values()) / 1e6, 3)}), flush=True)
        return

    # ---- headline: 4096x4096 Q4_K decode step, one launch (q8_K pack inside)
    log("headline: decode_q4k_4096x4096")
    hd = Decode(q, torch, "q4k", 4096, 4096, seed=1, fused=True)
    parity = hd.parity()
    sec, mv_us, mv_rounds = run_timed(torch, hd, args.steps, args.warmup)
    value = hd.step_bytes / sec / 1e9
    achieved = hd.mv_bytes / (mv_us * 1e-6) / 1e9
    tr = traffic_record("fused_q4k")
    calib = StreamCalib(torch)
    st_us = calib.us(hd.mv_bytes)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode_q4k_4096x4096", "rows": 4096, "K": 4096, "tokens": 1,
                   "weight": "GGUF Q4_K, 144 B per 256 values", "weight_copies_rotated": hd.R,
                   "step": "qmatvec_f32 (q8_K pack inside the launch)", "step_bytes": hd.step_bytes,
                   "timing": "hip graph replay",
                   "parity": "pass" if parity else "FAIL"},
        "env": gpu_env(torch),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": tr,
                     "kernel": HEADLINE_KERNEL, "launch_us": round(mv_us, 3),
                     "launch_us_rounds": rounds_summary(mv_rounds),
                     "algorithmic_bytes_per_launch": hd.mv_bytes,
                     "stream_read": {"us": round(st_us, 3), "GB/s": round(hd.mv_bytes / (st_us * 1e-6) / 1e9, 2),
                                     "frac": round(st_us / mv_us, 4),
                                     "what": "a plain 16-byte streaming read of the same bytes (csrc/calib.hip), "
                                             "same rotation and timing; frac = its time / the kernel's time"}},
    }
    del hd
    torch.cuda.empty_cache()

    # ---- the other workloads of the path
    if not args.only_headline:
        wl = {}
        steps = max(20, min(args.steps, 100))

        def oracle_fields(w, s):
            """The oracle's time for the same step (all ncores() threads, from the
            parity check) and the GPU step's speed-up over it."""
            o = getattr(w, "oracle_s", None)
            if o is None:
                return {}
            return {"oracle_ms": round(o * 1e3, 3), "oracle_threads": ncores(),
                    "gpu_speedup_vs_oracle": round(o / s, 1)}

        def decode_entry(name, d, kernel=None):
            p = d.parity()
            s, us, r = run_timed(torch, d, steps, 5)
            gbs = d.mv_bytes / (us * 1e-6) / 1e9
            sus = calib.us(d.mv_bytes)
            wl[name] = {"parity": "pass" if p else "FAIL", "kernel_us": round(us, 3),
                        "kernel_us_rounds": rounds_summary(r), "GB/s": round(gbs, 1),
                        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "stream_read_us": round(sus, 3),
                        "frac_stream_read": round(sus / us, 4), "step_ms": round(s * 1e3, 4),
                        "bytes_per_launch": d.mv_bytes, "weight_copies_rotated": d.R, **oracle_fields(d, s)}
            if kernel:
                wl[name]["traffic"] = traffic_record(kernel)

        # the same step as two launches: q8k_pack, then qmatvec on the packed token
        log("workload: decode_q4k_4096x4096_pack_then_matvec")
        decode_entry("decode_q4k_4096x4096_pack_then_matvec", Decode(q, torch, "q4k", 4096, 4096, seed=1),
                     "matvec_q4k")
        torch.cuda.empty_cache()
        for name, fmt, rows, seed in (("decode_fused_q5k_4096x4096", "q5k", 4096, 5),
                                      ("decode_fused_q6k_32000x4096", "q6k", 32000, 2)):
            log(f"workload: {name}")
            decode_entry(name, Decode(q, torch, fmt, rows, 4096, seed=seed, fused=True), "fused_" + fmt)
            torch.cuda.empty_cache()
        log("workload: decode_q6k_32000x4096")
        decode_entry("decode_q6k_32000x4096", Decode(q, torch, "q6k", 32000, 4096, seed=2), "matvec_q6k")
        torch.cuda.empty_cache()
        for nc in (4, 8):
            log(f"workload: batched_q4k_4096x4096_cols{nc}")
            decode_entry(f"batched_q4k_4096x4096_cols{nc}", Batched(q, torch, "q4k", 4096, 4096, seed=1, ncols=nc),
                         f"batched_q4k_c{nc}")
            torch.cuda.empty_cache()
        log("workload: moe_q4k_8x14336x4096_t16_top2")
        m = MoE(q, torch)
        decode_entry("moe_q4k_8x14336x4096_t16_top2", m, "moe")
        wl["moe_q4k_8x14336x4096_t16_top2"]["experts_hit"] = m.experts_hit
        del m
        torch.cuda.empty_cache()
        # Q5_K: the Q4_K decode shape and the MoE layer shape with 176-byte blocks
        log("workload: decode_q5k_4096x4096")
        decode_entry("decode_q5k_4096x4096", Decode(q, torch, "q5k", 4096, 4096, seed=5), "matvec_q5k")
        torch.cuda.empty_cache()
        log("workload: moe_q5k_8x14336x4096_t16_top2")
        m = MoE(q, torch, seed=6, fmt="q5k")
        decode_entry("moe_q5k_8x14336x4096_t16_top2", m, "moe_q5k")
        wl["moe_q5k_8x14336x4096_t16_top2"]["experts_hit"] = m.experts_hit
        del m
        torch.cuda.empty_cache()
        # relaid Q6_K experts at the same layer shape
        log("workload: moe_q6k_8x14336x4096_t16_top2")
        m = MoE(q, torch, seed=14, fmt="q6k")
        decode_entry("moe_q6k_8x14336x4096_t16_top2", m, "moe_q6k")
        wl["moe_q6k_8x14336x4096_t16_top2"]["experts_hit"] = m.experts_hit
        del m
        torch.cuda.empty_cache()
        for name, key, make in (
                ("prefill_q4k_4096x14336_m512", "prefill_q4k", lambda: Prefill(q, torch)),
                ("prefill_q5k_4096x14336_m512", "prefill_q5k", lambda: Prefill(q, torch, seed=8, fmt="q5k")),
                ("prefill_q6k_4096x14336_m512", "prefill_q6k", lambda: Prefill(q, torch, seed=10, fmt="q6k")),
                # small token counts: split-K fills the device (the fixup launch is timed with the tile)
                ("prefill_q4k_4096x14336_m32", "prefill_q4k_m32", lambda: Prefill(q, torch, M=32, seed=12)),
                ("prefill_q4k_4096x14336_m128", "prefill_q4k_m128", lambda: Prefill(q, torch, M=128, seed=13)),
                # the step from fp32 tokens in one launch (pack inside); compare its kernel_us with the
                # two-launch step_ms of the same workload above
                ("prefill_f32_q4k_4096x14336_m512", "prefill_f32_q4k", lambda: PrefillF32(q, torch)),
                ("prefill_f32_q6k_4096x14336_m512", "prefill_f32_q6k",
                 lambda: PrefillF32(q, torch, seed=10, fmt="q6k")),
                ("moe_prefill_q4k_8x14336x4096_t512_top2", "moe_prefill_q4k", lambda: MoEPrefill(q, torch)),
                ("moe_prefill_q5k_8x14336x4096_t512_top2", "moe_prefill_q5k",
                 lambda: MoEPrefill(q, torch, seed=9, fmt="q5k")),
                ("moe_prefill_q6k_8x14336x4096_t512_top2", "moe_prefill_q6k",
                 lambda: MoEPrefill(q, torch, seed=11, fmt="q6k"))):
            log(f"workload: {name}")
            p = make()
            ok = p.parity()
            s, us, r = run_timed(torch, p, max(10, steps // 4), 3)
            tops = p.ops / (us * 1e-6) / 1e12
            wl[name] = {
                "parity": "pass" if ok else "FAIL", "kernel_us": round(us, 2), "kernel_us_rounds": rounds_summary(r),
                "TOPS": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                "step_ms": round(s * 1e3, 4), "ops_per_launch": p.ops, "weight_copies_rotated": p.R,
                "traffic": traffic_record(key), **oracle_fields(p, s)}
            del p
            torch.cuda.empty_cache()
        p = Prefill(q, torch)
        # q8_K pack of the 512 x 14336 batch, timed on its own
        gp = graph_of(torch, lambda i: q.q8k_pack(p.x, p.M, p.K, p.xq), 32)
        pus = replay_us(torch, gp, 32, reps=2)
        del gp
        sus = calib.us(p.pack_bytes)
        wl["pack_512x14336"] = {"parity": "pass" if pack_parity(q, torch, p) else "FAIL",
                                "kernel_us": round(pus, 2), "GB/s": round(p.pack_bytes / (pus * 1e-6) / 1e9, 1),
                                "frac_hbm": round(p.pack_bytes / (pus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "stream_read_us": round(sus, 3), "frac_stream_read": round(sus / pus, 4),
                                "bytes_per_launch": p.pack_bytes, "traffic": traffic_record("pack")}
        del p
        out["workloads"] = wl

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        if not args.only_headline:
            log("cpu baseline, other configurations")
            out["cpu_baseline"]["configs"] = cpu_configs()

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
