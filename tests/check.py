"""Acceptance check of a BF16 GPU result against the FP64 oracle.

Bound, per computed element:  |D - D_ref| <= 2^-7 |D_ref| + 1e-3 * rms(D_ref),
with rms taken over the computed elements of the call.  BF16 round-to-nearest
costs at most 2^-8 relative; the other 2^-8 and the absolute term cover FP32
promotion order and the matrix core's internal summation order.  Rows that are
not computed must keep their prefilled bits exactly.
"""
from __future__ import annotations

import numpy as np
import torch

REL_TOL = 2.0 ** -7
ABS_TOL_RMS = 1e-3


def bf16_to_f64(d: torch.Tensor) -> np.ndarray:
    # widened by torch, not numpy: a sentinel that happens to be a signalling NaN
    # makes numpy's float32 -> float64 cast warn
    return d.detach().to("cpu").to(torch.float64).numpy()


def bf16_bits(d: torch.Tensor) -> np.ndarray:
    return d.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)


CHUNK = 1 << 24   # elements compared at a time (keeps whole-output checks of large shapes small in memory)


def within_tolerance(got: np.ndarray, ref: np.ndarray):
    """(ok, worst ratio err/bound, rms) for arrays of computed elements."""
    got = np.asarray(got, dtype=np.float64).reshape(-1)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return True, 0.0, 0.0
    # rms over every computed element of the call, then the bound chunk by chunk
    ss = 0.0
    for i in range(0, ref.size, CHUNK):
        r = ref[i:i + CHUNK]
        ss += float(np.dot(r, r))
    rms = float(np.sqrt(ss / ref.size))
    ok, ratio = True, 0.0
    for i in range(0, ref.size, CHUNK):
        g, r = got[i:i + CHUNK], ref[i:i + CHUNK]
        if not np.isfinite(g).all():
            return False, float("inf"), rms
        bound = REL_TOL * np.abs(r) + ABS_TOL_RMS * rms
        err = np.abs(g - r)
        ok = ok and bool(np.all(err <= bound))
        ratio = max(ratio, float(np.max(err / np.maximum(bound, 1e-300))))
    return ok, ratio, rms


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    ok, ratio, rms = within_tolerance(got, ref)
    assert ok, f"{what}: error exceeds bound (worst err/bound = {ratio:.3g}, rms(ref) = {rms:.3g})"
    return ratio
