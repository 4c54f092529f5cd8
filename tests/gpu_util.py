"""Helpers for the GPU tests: moving bf16 bit arrays to the device and back,
and the parity bar (max-abs 2e-2, mean-abs 2e-3 on bf16 outputs against the
fp64 oracle)."""
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
