"""Helpers for the GPU tests: moving bf16 bit arrays to the device and back,
and the parity bar (max-abs 2e-2, mean-abs 2e-3 on bf16 outputs against the
fp64 oracle; for gradients, which are not bounded by the values as outputs are,
2e-2 + 2^-7 |ref| per element: a bf16 gradient near 8 rounds by up to 1.6e-2 on
its own, and 2^-7 |ref| allows that storage rounding and as much again from the
bf16 operands)."""
import sys

import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t if dtype is None else t.to(dtype)).to("cuda")


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def assert_parity(got: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    d = np.abs(got - ref)
    mx, mn = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mn:.3e} over {d.size} values")
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}"


def assert_grad_parity(got: np.ndarray, ref: np.ndarray, what: str):
    """Gradient bar: |got - ref| <= 2e-2 + 2^-7 |ref| per element and mean-abs <= 2e-3 +
    2^-8 mean |ref|.  The relative terms are two bf16 roundings of up to 2^-8 |value| each
    (P and dS as MFMA operands, the stored gradient); the mean bar takes half of the
    per-element one, which only matters where gradients are sums of a few O(1) terms
    (a sequence of one token)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    d = np.abs(got - ref)
    allowed = MAX_ABS + 2.0 ** -7 * np.abs(ref)
    worst = float(np.max(d / allowed)) if d.size else 0.0
    mn = float(d.mean()) if d.size else 0.0
    mean_bar = MEAN_ABS + 2.0 ** -8 * (float(np.abs(ref).mean()) if d.size else 0.0)
    say(f"  {what}: max-abs {float(d.max()) if d.size else 0.0:.3e} (max |ref| {float(np.abs(ref).max()):.2f}), "
        f"worst err / (2e-2 + 2^-7 |ref|) {worst:.3f}, mean-abs {mn:.3e} (bar {mean_bar:.3e})")
    assert worst <= 1.0 and mn <= mean_bar, f"{what}: worst {worst:.3f} of the bar, mean-abs {mn:.3e} > {mean_bar:.3e}"
