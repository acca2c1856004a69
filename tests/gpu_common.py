"""Helpers for the GPU parity tests: tolerances, error metrics, and moving
device tensors to the host for the oracle."""
import sys

import numpy as np
import torch

# Tolerances of the method's acceptance bar: fp32 max-abs 1e-5; bf16 max-abs
# 2e-2 and relative L2 5e-3, both against the fp64 oracle on the same rounded
# inputs.
TOL = {torch.float32: dict(max_abs=1e-5, rel_l2=None), torch.bfloat16: dict(max_abs=2e-2, rel_l2=5e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a device tensor (bf16 and fp32 upcast exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def errors(got: np.ndarray, ref: np.ndarray):
    diff = got.astype(np.float64) - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm(diff.ravel()) / denom) if denom > 0 else float(np.linalg.norm(diff.ravel()))
    return max_abs, rel


def assert_close(got: np.ndarray, ref: np.ndarray, dtype, what: str):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    max_abs, rel = errors(got, ref)
    tol = TOL[dtype]
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    if got.size:
        i = np.unravel_index(int(np.abs(got - ref).argmax()), got.shape)
        say(f"    worst element at {tuple(int(j) for j in i)}: got {got[i]!r} oracle {ref[i]!r}; "
            f"max |oracle| {float(np.abs(ref).max()):.3f}")
    assert max_abs <= tol["max_abs"], f"{what}: max_abs {max_abs:.3e} > {tol['max_abs']}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{what}: rel_l2 {rel:.3e} > {tol['rel_l2']}"
    return max_abs, rel


def assert_close_scaled(got: np.ndarray, ref: np.ndarray, dtype, what: str):
    """Per-element bound for outputs of size O(1) and above.

    The fixed max-abs bar suits the standard workloads, whose outputs are
    averages of many values (|o| of order 0.1).  With sharp weights or a
    context of a few keys an output is close to single value entries (|o| up
    to ~6), and the probe terms B/l and (c/l) o^SA, which nearly cancel, are
    of that size too.  In bf16 the output rounding and the roundings of P and
    P*R to bf16 each cost up to half an ulp of such values, so the bound is
    2^-7 |oracle| (at most two bf16 ulps) + 1.5e-2.  In fp32, scores of up to
    ~130 in log2 units round their exponent argument by ~2^-24 * 130 ~ 8e-6,
    a relative error of the weights of that size, so the bound is
    1e-5 + 4e-6 |oracle|.  rel-L2 stays at 5e-3.
    """
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bf16 = dtype == torch.bfloat16
    bound = (2.0 ** -7 * np.abs(ref) + 1.5e-2) if bf16 else (4e-6 * np.abs(ref) + 1e-5)
    max_abs, rel = errors(got, ref)
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} worst/bound={float((err / bound).max()):.3f}")
    assert (err <= bound).all(), f"{what}: {int((err > bound).sum())} elements beyond the bound"
    assert rel <= 5e-3, f"{what}: rel_l2 {rel:.3e}"


def gpu_available() -> bool:
    return torch.cuda.is_available()
