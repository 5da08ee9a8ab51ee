"""Build libq8k.so in-tree for gfx950 with hipcc.

Every source is compiled for gfx950 only, with packed FP32 instructions
disabled, and the kernel resource report of each translation unit is checked:
a kernel that uses scratch (spills) fails the build, since a spilling kernel is
not a tuned kernel (the build gate idea of "One kernel, any device", section
2.2).  Sources that load registers with inline assembly also have their device
assembly checked (ASM_LOAD_CHECKED): registers loaded by inline assembly stay
in place, and M0, which the LDS copies set, is used by nothing else.  Usage: ``python quantized_q8kpack_fp32_amd/build.py`` (or via
``__graft_entry__.build()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libq8k.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "pack.hip", "matvec.hip", "moe.hip", "moe_mfma.hip", "prefill.hip", "prefill_regw.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-Rpass-analysis=kernel-resource-usage",
    "-I", os.path.join(ROOT, "include"),
]

_SCRATCH = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH_SIZE = re.compile(r"ScratchSize \[bytes/lane\]: (\d+)")


# Per-source flags.  The tiles with register-resident weight planes (prefill,
# mixture-of-experts decode) fold the matrix-core results with vector
# instructions, so their MFMAs must write ordinary VGPRs (the accumulation-register form would add a copy per
# result).
SOURCE_FLAGS = {"prefill_regw.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "moe_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, build_dir: str = BUILD_DIR, defines=()) -> tuple[str, str]:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *[f"-D{d}" for d in defines], "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


# Test-support instantiations that may spill: they store the integer sums of
# the product kernel beside its full register file (a spill moves data and
# changes no result; these kernels are never timed).  Demangled names.
MAY_SPILL = (
    "void q8k::(anonymous namespace)::prefill_regw_q4k_kernel<false, true, false>(",
    "void q8k::prefill_q4k_kernel<1, true, false>(",
)


def _demangle(names: list[str]) -> dict[str, str]:
    if not names:
        return {}
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    out = r.stdout.splitlines() if r.returncode == 0 else names
    return dict(zip(names, out))


def _check_scratch(log: str, src: str) -> list[str]:
    """Return 'kernel: N bytes' for every kernel in the report that uses scratch."""
    found = []
    name = None
    for line in log.splitlines():
        m = _SCRATCH.search(line)
        if m:
            name = m.group(1)
            continue
        m = _SCRATCH_SIZE.search(line)
        if m and name is not None and int(m.group(1)) > 0:
            found.append((name, int(m.group(1))))
    dem = _demangle([n for n, _ in found])
    return [f"{src}: {dem.get(n, n)}: {b} bytes/lane of scratch" for n, b in found
            if not dem.get(n, n).startswith(MAY_SPILL)]


# Sources whose inline assembly the compiler cannot see into, checked in their
# device assembly:
# - register loads by inline-assembly buffer loads, waited for with an explicit
#   count (the mixture-of-experts decode's weight walk): the compiler takes such
#   a register as written when the load is issued, so nothing keeps it from
#   copying or reusing the register while the load is still in flight.  The
#   build refuses the source unless (1) no other instruction writes a register
#   that such a load writes, and (2) the LDS stores that follow each explicit
#   wait store exactly such registers;
# - buffer-unit copies into LDS, which set M0 inside the assembly: M0 is a
#   reserved register, so the compiler does not restore it after the copies,
#   and the build refuses the source if the compiler itself uses M0 anywhere.
ASM_LOAD_CHECKED = ("moe_mfma.hip", "prefill_regw.hip")
_FUNC = re.compile(r"^(_Z\S+):")
_VRANGE = re.compile(r"^v\[(\d+):(\d+)\]$|^v(\d+)$")


def _vregs(tok: str) -> set[int]:
    m = _VRANGE.match(tok.rstrip(","))
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def _check_asm_loads(asm: str, src: str) -> list[str]:
    """Problems with inline-assembly register loads in device assembly (see ASM_LOAD_CHECKED)."""
    problems = []
    func, lines = None, []
    funcs = []
    for line in asm.splitlines():
        m = _FUNC.match(line)
        if m:
            func, lines = m.group(1), []
            funcs.append((func, lines))
        elif func is not None:
            lines.append(line.strip())
    for name, body in funcs:
        loaded, stored, other = set(), [], {}
        in_asm = after_wait = False
        for t in body:
            if t.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if t.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not t or t.startswith((";", ".")):
                continue
            op = t.split()[0]
            if in_asm:
                if op.startswith("buffer_load") and not t.endswith(" lds"):
                    loaded |= _vregs(t.split()[1])
                elif op == "s_waitcnt" and "vmcnt" in t:
                    after_wait = True
                continue
            if op.startswith("ds_write") and after_wait:
                stored.append((t, _vregs(t.split()[2])))
                continue
            if op.startswith("s_waitcnt"):
                continue
            after_wait = False
            if op.startswith(("s_", "ds_write", "buffer_store", "global_store", "buffer_load")) or " " not in t:
                continue
            for r in _vregs(t.split()[1]):
                other.setdefault(r, t)
        if not loaded:
            continue
        dem = _demangle([name]).get(name, name)
        clobbered = sorted(r for r in other if r in loaded)
        if clobbered:
            problems.append(f"{src}: {dem}: v{clobbered[0]} is written by '{other[clobbered[0]]}' "
                            f"besides an inline-assembly load")
        for t, regs in stored:
            if regs and not regs <= loaded:
                problems.append(f"{src}: {dem}: '{t}' after an explicit wait stores registers no "
                                f"inline-assembly load wrote")
                break
    return problems


def _check_m0(asm: str, src: str) -> list[str]:
    """Compiler instructions (outside inline assembly) that use M0."""
    in_asm, found = False, []
    for line in asm.splitlines():
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
        elif t.startswith(";;#ASMEND"):
            in_asm = False
        elif not in_asm and t and not t.startswith((";", ".")) and re.search(r"\bm0\b", t):
            found.append(f"{src}: the compiler uses M0 ('{t}'), which the inline-assembly LDS copies overwrite")
    return found[:3]


def _device_asm(src: str, build_dir: str, defines=()) -> str:
    out = os.path.join(build_dir, os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC, *[f for f in FLAGS if f != "-Rpass-analysis=kernel-resource-usage"], *SOURCE_FLAGS.get(src, []),
           *[f"-D{d}" for d in defines], "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    with open(out) as f:
        return f.read()


def build(verbose: bool = False, out: str = OUT, build_dir: str = BUILD_DIR, defines=()) -> str:
    """Compile and link; `defines` override compile-time tile parameters."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(ASM_LOAD_CHECKED))) as ex:
        asms = [ex.submit(_device_asm, s, build_dir, defines) for s in ASM_LOAD_CHECKED]
        results = list(ex.map(lambda s: _compile(s, build_dir, defines), SOURCES))
        asm_texts = [a.result() for a in asms]
    problems = []
    for src, (_, log) in zip(SOURCES, results):
        problems += _check_scratch(log, src)
        if verbose:
            sys.stderr.write(log)
    if problems:
        raise RuntimeError("kernels using scratch (spills):\n  " + "\n  ".join(problems))
    for src, asm in zip(ASM_LOAD_CHECKED, asm_texts):
        problems += _check_asm_loads(asm, src) + _check_m0(asm, src)
    if problems:
        raise RuntimeError("inline assembly not safe in the compiled code:\n  " + "\n  ".join(problems))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


CALIB_SRC = "calib.hip"
CALIB_OUT = os.path.join(HERE, "libq8k_calib.so")


def build_calib(out: str = CALIB_OUT, build_dir: str = BUILD_DIR) -> str:
    """The benchmark's streaming-read calibration kernel, a library of its own
    (csrc/calib.hip; not part of libq8k)."""
    os.makedirs(build_dir, exist_ok=True)
    obj, _ = _compile(CALIB_SRC, build_dir)
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, obj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_calib())
