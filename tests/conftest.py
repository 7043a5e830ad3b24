import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU oracle run")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) on a machine without a GPU when they are
    # selected anyway; on a machine with a GPU they run.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(params=["nw4", "nw8", "split"])
def fwd_form(request):
    """Forces one form of the plain causal bf16 forward for one test: 4- or
    8-wave workgroups over the whole key range, or the key-range split."""
    import alibi_linear_position_amd as alibi
    lib = alibi.load_library()
    nw, split = {"nw4": (4, 1), "nw8": (8, 1), "split": (0, 2)}[request.param]
    assert lib.alibi_debug_fwd_waves(nw) == 0
    assert lib.alibi_debug_fwd_split(split) == 0
    yield request.param
    assert lib.alibi_debug_fwd_waves(0) == 0
    assert lib.alibi_debug_fwd_split(0) == 0


@pytest.fixture(params=[4, 8], ids=["nw4", "nw8"])
def fwd_waves(request):
    """Forces 4- or 8-wave workgroups in the bf16 forward kernel for one test."""
    import alibi_linear_position_amd as alibi
    lib = alibi.load_library()
    assert lib.alibi_debug_fwd_waves(request.param) == 0
    yield request.param
    assert lib.alibi_debug_fwd_waves(0) == 0


@pytest.fixture(params=[1, 2], ids=["qb1", "qb2"])
def bwd_form(request):
    """Forces the backward's dK/dV kernel to 32-row (fp32 P hand-off) or 64-row
    (fp16 P hand-off) query tiles for one test."""
    import alibi_linear_position_amd as alibi
    lib = alibi.load_library()
    assert lib.alibi_debug_bwd_query_blocks(request.param) == 0
    yield request.param
    assert lib.alibi_debug_bwd_query_blocks(0) == 0
