import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


@pytest.fixture(scope="session")
def gpu_lib():
    """The C-ABI library on a GPU; fails (not skips) when the HIP path is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    from paged_kv_cache_attn_amd import binding

    return binding


@pytest.fixture(autouse=True)
def _announce(request):
    """Name each test on the real stderr before it runs (survives a hard GPU fault)."""
    sys.__stderr__.write(f"\n[start] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
