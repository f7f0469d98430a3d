"""Shared test plumbing: device copies of synthetic inputs and error measures."""

import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Tolerances stated for this method: loss relative error 1e-5 for fp32 inputs
# and 2e-3 for bf16; gradient max-abs error 1e-2 * max|grad| for bf16.  For
# fp32 gradients (not stated) 1e-4 * max|grad|: fp32 accumulation over
# K <= 4096 products keeps well inside it.
LOSS_RTOL = {"f32": 1e-5, "bf16": 2e-3}
GRAD_RTOL = {"f32": 1e-4, "bf16": 1e-2}


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_dev(t, dev):
    import torch
    if t.bits is not None:
        return torch.from_numpy(t.bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(t.values)).to(dev)


def host(x) -> np.ndarray:
    return x.float().cpu().numpy().astype(np.float64)


def grad_err(got, want) -> float:
    """max |got - want| / max |want|."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.abs(want).max()
    return float(np.abs(got - want).max() / (den if den > 0 else 1.0))


def say(msg: str) -> None:
    print(msg, flush=True)
