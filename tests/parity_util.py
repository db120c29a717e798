"""Comparison helpers for the parity tests (no arithmetic of the layer)."""
from __future__ import annotations

import numpy as np

# relative max-abs bounds: max|gpu - oracle| / max|oracle|
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_max_abs(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    diff = np.max(np.abs(gpu - ref)) if ref.size else 0.0
    if scale == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return float(diff / scale)


def assert_close(name: str, gpu, ref, dtype: str) -> float:
    e = rel_max_abs(gpu, ref)
    assert e <= TOL[dtype], f"{name}: relative max-abs error {e:.3e} > {TOL[dtype]:.0e}"
    return e


def check_selection(gpu_idx: np.ndarray, oracle_idx: np.ndarray, scores: np.ndarray, k: int,
                    rel: float = 1e-5) -> int:
    """Selected ids must equal the oracle's, except at tokens whose k-th and
    (k+1)-th oracle scores are within `rel`: there any choice among the
    near-tied groups is correct.  Returns the number of exempted tokens."""
    gpu_idx = np.asarray(gpu_idx)
    oracle_idx = np.asarray(oracle_idx)
    T, G = scores.shape
    assert gpu_idx.shape == oracle_idx.shape == (T, k)
    assert np.all(np.diff(gpu_idx, axis=1) > 0), "ids must be ascending and distinct"
    assert gpu_idx.min() >= 0 and gpu_idx.max() < G
    srt = -np.sort(-scores, axis=1)
    sk = srt[:, k - 1]
    nxt = srt[:, k] if k < G else np.full(T, -np.inf)
    tie = np.abs(sk - nxt) <= rel * np.maximum(np.abs(sk), np.abs(nxt))
    mism = np.any(gpu_idx != oracle_idx, axis=1)
    bad = mism & ~tie
    assert not np.any(bad), f"{int(bad.sum())} tokens select different groups, first {np.flatnonzero(bad)[:5]}"
    # near ties: groups clearly above the band are kept; every chosen group is in or above the band
    for t in np.flatnonzero(mism & tie):
        band = rel * max(abs(sk[t]), abs(nxt[t]))
        must = set(np.flatnonzero(scores[t] > sk[t] + band).tolist())
        chosen = set(gpu_idx[t].tolist())
        assert must <= chosen, f"token {t}: dropped a group above the tie band"
        assert all(scores[t, g] >= sk[t] - band for g in chosen), f"token {t}: chose a group below the band"
    return int((mism & tie).sum())
