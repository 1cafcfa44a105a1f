"""Shared test plumbing: layout moves between the oracle's [C][T][H][W] float64
arrays and the library's [T][H][W][C] device tensors, and the parity metrics.

Tolerances (from the workload statement): fp32 max|d| / max|ref| <= 1e-4;
bf16 max|d| / max|ref| <= 1.5e-2 and mean|d| / mean|ref| <= 2e-3, over every
compared value.  A bf16 store alone has relative error <= 2^-9 (mean about
2^-10 ~ 1e-3 of |ref| on average), which is what the mean bound leaves room for.
These bounds gate every layer and fused block, with the oracle fed the layer's
own GPU input.

A whole multi-layer bf16 stack compared with the storage-rounded oracle run end
to end gets a wider bound, one per configuration: every stored tensor is rounded
to bf16, and a difference of a few fp32 ulps in a sum before a store (summation
order) flips a rounding that later layers carry forward.  golden/stack_bounds.txt
holds, per configuration of stack_cases.py, 1.5x the largest drift of the
oracle from itself under such perturbations (3 seeds), written by
golden/make_stack_bounds.py from the oracle alone.
"""
from __future__ import annotations

import numpy as np
import torch

FP32_MAX_REL = 1e-4
BF16_MAX_REL = 1.5e-2
BF16_MEAN_REL = 2e-3
_STACK_BOUNDS = None


def stack_bound(case: str):
    """(max-rel, mean-rel) end-to-end bound of a stack_cases configuration."""
    global _STACK_BOUNDS
    if _STACK_BOUNDS is None:
        import os
        import sys
        gold = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
        if gold not in sys.path:
            sys.path.insert(0, gold)
        import make_stack_bounds
        _STACK_BOUNDS = make_stack_bounds.read()
    if case not in _STACK_BOUNDS:
        raise KeyError("no end-to-end bound recorded for stack case %r" % case)
    return _STACK_BOUNDS[case]


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


def assert_stack_close(got, ref, case, what=""):
    """The end-to-end check of a whole stack at the bound recorded for ``case``."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    bmax, bmean = stack_bound(case)
    mx, mn = rel_errors(got, ref)
    assert mx <= bmax and mn <= bmean, "%s [%s]: max-rel %.3g (<= %.3g), mean-rel %.3g (<= %.3g)" % (
        what, case, mx, bmax, mn, bmean)
    return mx, mn


def assert_fp32_close(got, ref, what=""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    mx, _ = rel_errors(got, ref)
    assert mx <= FP32_MAX_REL, "%s: max-abs-rel %.3g > %g" % (what, mx, FP32_MAX_REL)
    return mx


def say(msg: str):
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print(msg, flush=True)
