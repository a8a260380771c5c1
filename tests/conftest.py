import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests must never fall back to anything: skip them loudly when no GPU
    # is visible, so `-m "not gpu"` and CPU-only runs stay green.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def plan():
    """Force GEMM launch plans for one test: plan(gemm_cfg=..., gemm_slots=...,
    gemm_split=..., decode_wide=...); the automatic plans are restored after."""
    import fp8_block_scaled_token_amd as fq
    yield fq.fp8q_set_plan_override
    fq.fp8q_set_plan_override()
