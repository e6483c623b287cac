"""Shared test helpers: device transfer and the parity rules.

Parity rules (floating point decides the top-k integers, so they come with a
margin rule):
* a top-k list whose oracle margin (smallest gap among its first k + 1
  sorted logits) exceeds TAU must equal the oracle's list index for index;
* a list with a smaller margin may only reorder or swap entries whose oracle
  logits lie within TAU of the oracle's value at that position; such lists are
  counted and reported;
* floating outputs: max|x - ref| <= tol * max|ref| per tensor, tol = 2e-2
  for bf16 storage and 1e-5 for float32 storage.
Integers downstream of the top-k (tree tokens, accepted lengths, paths,
compaction) are compared bit for bit, fed the oracle's own upstream values.
"""
from __future__ import annotations

import numpy as np

TAU = {"bf16": 1e-4, "f32": 1e-5}
TOL = {"bf16": 2e-2, "f32": 1e-5}


def to_dev(a: np.ndarray, device="cuda"):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_dev(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_or_f32_to_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def check_topk(gpu_idx: np.ndarray, gpu_val: np.ndarray, ref_idx: np.ndarray, ref_val: np.ndarray,
               margin: np.ndarray, k: int, tau: float, tol: float, logits_of=None):
    """Compare one set of lists [R, k]; returns the number of near-tie lists.

    logits_of(r, indices) -> oracle logits of those indices for row r (needed
    only when a near-tie list differs from the oracle's).
    """
    ties = 0
    R = ref_idx.shape[0]
    for r in range(R):
        gi, ri = gpu_idx[r, :k], ref_idx[r, :k]
        if margin[r] > tau:
            assert np.array_equal(gi, ri), "row %d: top-k %s != oracle %s (margin %.3g)" % (r, gi, ri, margin[r])
        else:
            ties += 1
            if not np.array_equal(gi, ri):
                assert logits_of is not None, "row %d differs inside a near tie and no logits to check" % r
                lg = logits_of(r, gi)
                assert np.all(np.abs(lg - ref_val[r, :k]) <= tau), "row %d: near-tie swap beyond tau" % r
    err = rel_err(gpu_val[:, :k], ref_val[:, :k])
    assert err <= tol, "top-k values: relative error %.3g > %.3g" % (err, tol)
    return ties
