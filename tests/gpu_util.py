"""Shared helpers of the GPU parity tests (no test functions here)."""
import numpy as np
import torch

DEV = torch.device("cuda:0")
RTOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2}


def bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def rel_err_rows(got: np.ndarray, want: np.ndarray) -> float:
    """max over rows of ||got - want||_inf / ||want||_inf (rows = last axis)."""
    g = got.reshape(-1, got.shape[-1]).astype(np.float64)
    w = want.reshape(-1, want.shape[-1]).astype(np.float64)
    den = np.maximum(np.abs(w).max(axis=1), 1e-30)
    return float((np.abs(g - w).max(axis=1) / den).max())


def say(msg: str) -> None:
    print(msg, flush=True)
