import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases (minutes of CPU or GPU time)")


def _gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if any("gpu" in item.keywords for item in items) and not _gpu_available():
        skip = pytest.mark.skip(reason="no GPU visible to torch")
        for item in items:
            if "gpu" in item.keywords:
                item.add_marker(skip)


# With SPLITKV_CHECK_VIOLATIONS=1 (and SPLITKV_LIBRARY naming the
# bounds-checked build, libsplitkv_checked.so), every GPU test ends by
# reading the library's bounds-check record: any global index a forward
# kernel derived outside its buffer during the test fails it.
@pytest.fixture(autouse=True)
def _bounds_check_record(request):
    yield
    if os.environ.get("SPLITKV_CHECK_VIOLATIONS") != "1" or "gpu" not in request.keywords:
        return
    from split_kv_attention_amd import _lib

    n, site, index, limit = _lib.sk_check_violations()
    assert n == 0, f"{n} out-of-bounds indices, the first at site {site}: {index} >= {limit}"
