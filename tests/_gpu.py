"""Helpers shared by the GPU parity tests: device tensors from the seeded
workloads, tolerance checks, and a loud skip/fail policy for the device."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from learned_token_pruning_gatescore_amd import workloads as wl


def device():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    import learned_token_pruning_gatescore_amd as tg

    tg.load()  # raises if the HIP library is missing: GPU tests never fall back
    return torch.device("cuda:0")


def say(*a):
    """Name the case before GPU work, flushed, so a lost run still says what ran."""
    print("[case]", *a, file=sys.stderr, flush=True)


def dev_tensor(x: np.ndarray, dtype: str, dev):
    return wl.to_torch(x, dtype, dev)


def to_np(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def assert_scores_close(got, ref, rtol, what="scores"):
    """|got - ref| <= rtol * max(|ref|, rms(ref)) element-wise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = rtol * np.maximum(np.abs(ref), rms)
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} outside tolerance; worst at {i}: "
                             f"got {got.flat[i]!r} ref {ref.flat[i]!r} (rtol {rtol}, rms {rms:.3g})")


def assert_maxabs(got, ref, atol, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    err = np.where(both_inf, 0.0, np.abs(got - ref))
    m = float(np.nanmax(err)) if err.size else 0.0
    assert not np.isnan(err).any(), f"{what}: NaN"
    assert m <= atol, f"{what}: max-abs error {m:.3e} > {atol:.1e}"
    return m
