"""Shared helpers for the GPU parity tests: move seeded inputs to the device
(exact bytes), run the library through its binding, and compare with the
oracle under the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

# parity gates: normwise error against the largest oracle value
TOL_BF16 = 2e-2          # max|y - y_or| <= 2e-2 * max|y_or|
TOL_F32 = 1e-4           # max|y - y_or| <= 1e-4 * max|y_or|


def to_dev(t: W.Tensor, device="cuda") -> torch.Tensor:
    if t.dtype == W.BF16:
        return torch.from_numpy(t.storage.astype(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(t.storage).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def torch_dtype(dt: str):
    return torch.bfloat16 if dt == W.BF16 else torch.float32


def table_for(case: W.LinearCase, device="cuda"):
    import adapter_lora_amd as ml
    A = [to_dev(a, device) for a in case.A]
    B = [to_dev(b, device) for b in case.B]
    return ml.LoraTable(A, B, case.ranks, case.slice_sizes, case.K, torch_dtype(case.dtype),
                        device)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, base: np.ndarray = None,
                 what: str = "", roundings: int = 1):
    """The normwise gate above, plus a tighter element-wise gate derived from the
    arithmetic: each output rounding costs at most half an ulp (<= 2^-8 |y|
    for bf16, counted `roundings` times for repeated in-place updates, whose
    intermediate values lie between y_base and y) plus fp32 accumulation
    error (<= 1e-3 of the largest delta)."""
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    tol = TOL_BF16 if dtype == W.BF16 else TOL_F32
    assert err <= tol * scale + 1e-30, f"{what}: max err {err:.3e} > {tol} * {scale:.3e}"
    if base is not None and ref.size:
        dmax = float(np.max(np.abs(ref - base)))
        mag = np.maximum(np.abs(ref), np.abs(base))
        if dtype == W.BF16:
            bound = roundings * 2.0 ** -8 * mag + 1e-3 * dmax + 1e-30
        else:
            bound = roundings * 2.0 ** -22 * mag + 1e-5 * dmax + 1e-30
        bad = np.abs(got - ref) > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the element-wise "
                               f"bound; worst {float(np.max(np.abs(got - ref) - bound)):.3e}")
    return err, scale
