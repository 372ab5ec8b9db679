"""Test infrastructure: decode storage-format arrays into the oracle's float64 inputs, run the oracle
on (samples of) a workload, and compare with the GPU path by the acceptance rules:

* index sets: bit-exact where the relative gap at the k-th boundary exceeds 1e-4, otherwise a valid
  top-k within 1e-4 of the k-th score;
* attention outputs: per query, max |gpu - ref| / max |ref| over that query's heads and dims,
  and the largest of these over the queries checked <= 2e-3 for fp32/bf16 caches, 2e-2 for fp8
  caches (the call-wide ratio is kept as a statistic);
* top-k on identical scores: bit-exact (integer work).
"""
from __future__ import annotations

import numpy as np

from oracle import csa_oracle as orc
from oracle.numerics import bf16_decode, e4m3_decode

ATT_TOL = {"f32": 2e-3, "bf16": 2e-3, "e4m3": 2e-2}
GAP_EXACT = 1e-4


def dec(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_decode(a.view(np.uint16))
    if dtype == "e4m3":
        return e4m3_decode(a.view(np.uint8))
    return np.asarray(a, np.float64)


def to_np(t) -> np.ndarray:
    """torch tensor (GPU or CPU) -> numpy, bf16 codes as uint16."""
    import torch
    t = t.detach().cpu()
    if t.dtype in (torch.int16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(gpu - ref)) if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def rel_err_per_query(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per query (leading axis): max |gpu - ref| / max |ref| over the query's other axes. A query
    whose reference is all zero (no keys) reports its absolute error."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    n = ref.shape[0]
    num = np.abs(gpu - ref).reshape(n, -1).max(axis=1) if ref.size else np.zeros(n)
    den = np.abs(ref).reshape(n, -1).max(axis=1) if ref.size else np.zeros(n)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def store_f64(c, r, scale, pos0=0):
    """(c, r, scale, pos0) tuple of float64 arrays for one sequence (the oracle's store form)."""
    return (c, r, scale, pos0)


def check_topk_valid(idx_gpu: np.ndarray, scores64: np.ndarray, n_vis: int, k: int):
    """A valid top-k when the boundary is a near-tie: right size, distinct, visible, ascending,
    -1 padded, every selected score within 1e-4 (relative) of the k-th largest, and every visible
    entry scoring more than 1e-4 (relative) above the k-th largest selected."""
    take = min(k, n_vis)
    sel = idx_gpu[:take]
    assert (idx_gpu[take:] == -1).all()
    assert len(set(sel.tolist())) == take
    assert (sel >= 0).all() and (sel < n_vis).all()
    assert (np.diff(sel) > 0).all()
    if n_vis > k:
        kth = np.sort(scores64[:n_vis])[::-1][k - 1]
        tol = GAP_EXACT * max(abs(kth), 1e-30)
        assert (scores64[sel] >= kth - tol).all()
        must = np.nonzero(scores64[:n_vis] > kth + tol)[0]
        assert np.isin(must, sel).all(), "an entry clearly above the k-th score was dropped"
