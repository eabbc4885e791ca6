import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def to_np(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor: bf16 as raw uint16 bits, everything else as is."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) or float32 -> float64 values."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


@pytest.fixture(scope="session")
def oracle():
    from oracle import Oracle
    return Oracle()


def gpu_available() -> bool:
    try:
        return torch.cuda.is_available()
    except Exception:
        return False
