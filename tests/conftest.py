import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case, minutes of host work")


POISON_BYTE = 0xA5


def _poisoned_empty(*shape, dtype, device):
    """torch.empty, then every element set to a poison value: NaN for floating dtypes, 0xA5 bytes otherwise.
    An output element that a kernel never writes then fails the comparison with the oracle (a NaN fails every
    tolerance; a poison byte matches an expected code byte by chance only)."""
    import torch
    t = torch.empty(*shape, dtype=dtype, device=device)
    if t.is_floating_point():
        t.fill_(float("nan"))
    else:
        t.view(torch.uint8).fill_(POISON_BYTE)
    return t


@pytest.fixture(autouse=True)
def poison_library_buffers(request):
    """GPU tests: every buffer the binding allocates for the library (outputs, weight state, workspace) starts
    out poisoned instead of holding whatever the caching allocator last left there."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    from bit_nf4_quantized_15_amd import qlora
    saved = qlora.empty_hook
    qlora.empty_hook = _poisoned_empty
    try:
        yield
    finally:
        qlora.empty_hook = saved
