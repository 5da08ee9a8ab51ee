import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# ---- the kernel census (tests/census.py): a GPU test starts with nothing
# pending, so only its own launches can be credited by its value checks; the
# census test asserts coverage only after a whole GPU run.
@pytest.fixture(autouse=True)
def _census_reset(request):
    if request.node.get_closest_marker("gpu") is not None:
        from census import CENSUS

        CENSUS.pending.clear()
    yield


def pytest_collection_modifyitems(session, config, items):
    """A run is whole when it selects by the gpu marker alone over the test
    directory: no -k, no node ids, nothing deselected among GPU tests."""
    import census

    keyword = config.getoption("keyword", "") or ""
    args = [a for a in config.args if not a.startswith("-")]
    by_node = any("::" in a or a.endswith(".py") for a in args)
    census.WHOLE_GPU_RUN = (not keyword) and (not by_node) and (config.getoption("markexpr", "") == "gpu")


def pytest_deselected(items):
    import census

    if any(i.get_closest_marker("gpu") is not None for i in items if "census" not in i.nodeid):
        census.WHOLE_GPU_RUN = False


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build()
    return oracle
