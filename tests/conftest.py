import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_order(item):
    """GPU tests of the forward, BlockMask-builder and decode kernels run first, then the
    dense backward, the backward with score changes, the BlockMask backward, the address-
    limit cases (multi-GB strided tensors and page pools), and the allocation-free decode
    test last.  A GPU fault ends the whole test process, so kernels
    with a longer GPU record are checked before newer ones."""
    base = os.path.basename(str(item.fspath))
    if base.startswith("test_zz_"):
        return 4
    if base == "test_gpu_large_addresses.py":
        return 3.5
    name = base + "::" + item.name
    if "backward_blockmask" in name:
        return 3
    if "backward_score_mod" in name:
        return 2
    if "backward" in name or "readme" in name:
        return 1
    return 0


def pytest_collection_modifyitems(session, config, items):
    items.sort(key=_gpu_order)  # stable: file and parameter order kept within each rank
