"""Shared helpers of the GPU parity tests (no test functions here)."""
import numpy as np
import torch

DEV = torch.device("cuda:0")
RTOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2}
# The tolerances above are the stated outer bounds for each row type.  Both sides read the same
# bf16 or f16 rows and widen them to fp32 exactly; the kernels then compute in fp32 and the oracle
# in fp64, so only the fp32 path's rounding separates them, as it does for fp32 rows.  Checking
# that bound as well makes a loss of precision far inside the 2e-2 storage bound fail.
ARITH_RTOL = 1e-5


def check_attn(err: float, dtype: str, what: str) -> None:
    """Assert an attention relative error against the stated and the arithmetic bound."""
    assert err <= RTOL[dtype], f"{what}: rel err {err} above the stated {RTOL[dtype]} for {dtype} rows"
    assert err <= ARITH_RTOL, f"{what}: rel err {err} above the fp32-arithmetic bound {ARITH_RTOL} ({dtype} rows)"


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
