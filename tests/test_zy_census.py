"""The kernel census over a whole GPU run ("One kernel, any device", section
5; "Language models on the device", section 6): every kernel compiled into
libq8k.so must have been value-checked against the oracle by some test in
this run, or be excused by name here with its reason.  Running is not
coverage: a kernel launched only by comparisons of one kernel with another is
uncovered.  An excuse for a kernel that was checked anyway is stale and fails
too.  The file name sorts after every GPU test module, so the whole run has
finished when this test runs; over a partial run (-k, node ids, deselected GPU
tests) it is skipped.
"""
import pytest

import census

pytestmark = pytest.mark.gpu

# kernel (short name) -> why it is not value-checked
EXCUSED: dict[str, str] = {}


def test_every_kernel_value_checked():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not census.WHOLE_GPU_RUN:
        pytest.skip("partial GPU run: the census needs every GPU test")
    import quantized_q8kpack_fp32_amd as q

    names = census.kernel_names(q)
    checked = {census.short(names[h]) for h in census.CENSUS.checked if h in names}
    ran = {census.short(names[h]) for h in census.CENSUS.ran if h in names}
    unknown = [h for h in census.CENSUS.ran if h not in names]
    assert not unknown, f"launch records name handles that are not kernels of the library: {unknown[:4]}"
    every = {census.short(n) for n in names.values()}
    uncovered = sorted(every - checked - set(EXCUSED))
    stale = sorted(set(EXCUSED) & checked)
    lines = [f"UNCOVERED {k}" + (" (ran, never value-checked)" if k in ran else " (never ran)") for k in uncovered]
    lines += [f"STALE EXCUSE {k}" for k in stale]
    print(f"census: {len(checked)} of {len(every)} kernels value-checked")
    assert not lines, "\n".join(lines)
