"""Cross-step reuse measurements, in exact arithmetic (oracle; test infrastructure only).

The Sol Engine "H3 on device" page (cross-step cache paragraph) gates recomputation
across denoising steps with a cheap change detector. Here the detector is the
relative change of the pooled block means between two steps, and the cost of
reusing a mask is measured by its overlap with the fresh one.
"""
from __future__ import annotations

import math

import numpy as np


def mask_overlap(mask_a, mask_b) -> np.ndarray:
    """int64 [B, H, 2]: (#(i, j) kept in both, #(i, j) kept in mask_a); non-zero bytes count as kept."""
    a = np.asarray(mask_a) != 0
    b = np.asarray(mask_b) != 0
    both = np.logical_and(a, b).sum(axis=(2, 3))
    na = a.sum(axis=(2, 3))
    return np.stack([both, na], axis=-1).astype(np.int64)


def pooled_change(prev, cur):
    """(sum (cur - prev)^2, sum prev^2) over all pooled values, summed exactly (math.fsum of the rounded terms)."""
    p = np.asarray(prev, dtype=np.float64).ravel()
    c = np.asarray(cur, dtype=np.float64).ravel()
    d = c - p
    return math.fsum((d * d).tolist()), math.fsum((p * p).tolist())


def relative_change(prev, cur) -> float:
    d2, p2 = pooled_change(prev, cur)
    return math.sqrt(d2 / p2) if p2 > 0 else (0.0 if d2 == 0 else math.inf)


def keeps_mask(ref, cur, threshold: float, force: bool) -> bool:
    """The gate: keep the mask selected from `ref` iff not forced and
    sum (cur - ref)^2 <= (threshold * threshold) * sum ref^2, in fp64 in that order
    (a relative L2 change of the pooled block means of at most `threshold`)."""
    if force:
        return False
    d2, p2 = pooled_change(ref, cur)
    return d2 <= (threshold * threshold) * p2


def reuse_schedule(pooled_steps, threshold: float):
    """Run the gate over a sequence of per-step pooled means (step 0 is always
    selected fresh). Returns, per step, (recomputed, index of the step whose
    pooled means the mask in use was selected from)."""
    out = []
    ref = None
    for s, cur in enumerate(pooled_steps):
        if s == 0 or not keeps_mask(pooled_steps[ref], cur, threshold, False):
            ref = s
            out.append((True, s))
        else:
            out.append((False, ref))
    return out
