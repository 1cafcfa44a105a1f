"""Shared test plumbing: layout moves between the oracle's [C][T][H][W] float64
arrays and the library's [T][H][W][C] device tensors, and the parity metrics.

Tolerances (from the workload statement): fp32 max|d| / max|ref| <= 1e-4;
bf16 max|d| / max|ref| <= 1.5e-2 and mean|d| / mean|ref| <= 2e-3, over every
compared value.  A bf16 store alone has relative error <= 2^-9 (mean about
2^-10 ~ 1e-3 of |ref| on average), which is what the mean bound leaves room for.
These bounds gate every layer and fused block, with the oracle fed the layer's
own GPU input.

A whole multi-layer bf16 stack compared with the storage-rounded oracle run end
to end gets a wider bound (STACK_*): every stored tensor is rounded to bf16, and
a one-ulp difference in a fp32 sum before a store (summation order) flips a
rounding that later layers carry forward.  Measured on the CPU with the oracle
alone (test_oracle.py::test_stack_rounding_divergence), such perturbations move a
17-conv stack's output by ~1e-2 max / ~5e-3 mean relative; the stack bound is 3x
that.
"""
from __future__ import annotations

import numpy as np
import torch

FP32_MAX_REL = 1e-4
BF16_MAX_REL = 1.5e-2
BF16_MEAN_REL = 2e-3
STACK_MAX_REL = 3e-2
STACK_MEAN_REL = 1.5e-2


def to_oracle(x_cthw: torch.Tensor) -> np.ndarray:
    """A [C][T][H][W] CPU tensor (fp32 or bf16) as float64 numpy."""
    return x_cthw.detach().to("cpu").to(torch.float64).numpy()


def to_device_cl(x_cthw: torch.Tensor, device="cuda") -> torch.Tensor:
    """[C][T][H][W] -> contiguous [T][H][W][C] on the device (same dtype)."""
    return x_cthw.permute(1, 2, 3, 0).contiguous().to(device)


def from_device_cl(y_thwc: torch.Tensor) -> np.ndarray:
    """[T][H][W][C] device tensor -> [C][T][H][W] float64 numpy."""
    return y_thwc.detach().to("cpu").to(torch.float64).permute(3, 0, 1, 2).contiguous().numpy()


def rel_errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    return float(d.max() / max(np.abs(ref).max(), 1e-30)), float(d.mean() / max(np.abs(ref).mean(), 1e-30))


def assert_bf16_close(got, ref, what=""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    mx, mn = rel_errors(got, ref)
    assert mx <= BF16_MAX_REL and mn <= BF16_MEAN_REL, "%s: max-rel %.3g (<= %g), mean-rel %.3g (<= %g)" % (
        what, mx, BF16_MAX_REL, mn, BF16_MEAN_REL)
    return mx, mn


def assert_stack_close(got, ref, what=""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    mx, mn = rel_errors(got, ref)
    assert mx <= STACK_MAX_REL and mn <= STACK_MEAN_REL, "%s: max-rel %.3g (<= %g), mean-rel %.3g (<= %g)" % (
        what, mx, STACK_MAX_REL, mn, STACK_MEAN_REL)
    return mx, mn


def assert_fp32_close(got, ref, what=""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    mx, _ = rel_errors(got, ref)
    assert mx <= FP32_MAX_REL, "%s: max-abs-rel %.3g > %g" % (what, mx, FP32_MAX_REL)
    return mx


def say(msg: str):
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print(msg, flush=True)
