"""Decision margins of top-K routing, for the parity tests: where the GPU
ranks float32 keys and the oracle float64 ones, a selection can only
differ at a token whose smallest gap between a kept and a dropped
candidate (group or expert) is below the two sides' key difference."""
from __future__ import annotations

import numpy as np


def selection_keys(logits, bias, score: str, bias_mode: str) -> np.ndarray:
    """float64 selection keys: the float32 biased logits, or for a
    selection-only bias the score of the logits plus the bias."""
    z = np.asarray(logits, dtype=np.float32)
    if bias_mode == "logit":
        if bias is not None:
            z = (z + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
        return z.astype(np.float64)
    z = z.astype(np.float64)
    if score == "softmax":
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
    else:
        p = 1.0 / (1.0 + np.exp(-z))
    return p + (0.0 if bias is None else np.asarray(bias, dtype=np.float64)[None, :])


def _gap(sorted_desc, k):
    """sorted_desc[:, k-1] - sorted_desc[:, k] with non-finite gaps as inf."""
    if k >= sorted_desc.shape[1]:
        return np.full(sorted_desc.shape[0], np.inf)
    gap = sorted_desc[:, k - 1] - sorted_desc[:, k]
    return np.where(np.isfinite(gap), gap, np.inf)


def decision_margins(key, K: int, n_groups: int = 0, topk_groups: int = 0) -> np.ndarray:
    """Per-token smallest gap over the decisions of a (grouped) top-K:
    the topk_groups-th against the next group score (group score = sum of
    the group's two largest keys), then the K-th against the next key among
    the kept groups' experts."""
    key = np.array(key, dtype=np.float64)
    T, E = key.shape
    m = np.full(T, np.inf)
    if n_groups > 1:
        eg = E // n_groups
        kg = key.reshape(T, n_groups, eg)
        gs = -np.sort(-kg, axis=2)[:, :, :min(2, eg)].sum(axis=2)
        m = np.minimum(m, _gap(-np.sort(-gs, axis=1), topk_groups))
        keep = np.zeros_like(gs, dtype=bool)
        np.put_along_axis(keep, np.argsort(-gs, axis=1, kind="stable")[:, :topk_groups], True, 1)
        key = np.where(np.repeat(keep, eg, axis=1), key, -np.inf)
    return np.minimum(m, _gap(-np.sort(-key, axis=1), K))
