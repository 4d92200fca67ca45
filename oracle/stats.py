"""Oracle GroupNorm statistics for patch-split tensors. Float64.

Test infrastructure: only tests, the smoke check and the benchmark's CPU-baseline leg use it.

When a tensor is split into spatial patches, GroupNorm still has to use the statistics of the whole
tensor. That means the global mean, and the variance about that global mean divided by the total
count. Per-patch means and Bessel's correction are both wrong ("Add tiled VAE parallelism & extended
model support", PatchGroupNorm commit message). Each patch therefore reports (count, mean, M2) over
the positions it owns, and the parts are merged with the pairwise update of Chan, Golub and LeVeque
(1979, "Updating formulae and a pairwise algorithm for computing sample variances"):
- n = sum n_i;
- mean = sum n_i * mean_i / n;
- M2 = sum (M2_i + n_i * (mean_i - mean)^2).
These are algebraic identities, so the merge over any split equals the two-pass result on the whole.
"""
from __future__ import annotations

import numpy as np


def group_moments(x: np.ndarray, groups: int):
    """(count, mean, M2) per (sample, group) over the positions of ``x``, two-pass.

    Returns three arrays of shape [N, groups]; count is an exact integer (int64).
    """
    x = np.asarray(x, dtype=np.float64)
    n, c = x.shape[0], x.shape[-1]
    xg = x.reshape(n, -1, groups, c // groups)
    count = np.full((n, groups), xg.shape[1] * xg.shape[3], dtype=np.int64)
    mean = np.empty((n, groups))
    m2 = np.empty((n, groups))
    for g in range(groups):
        part = xg[:, :, g, :]
        mu = part.mean(axis=(1, 2))
        dev = part - mu[:, None, None]
        mean[:, g] = mu
        m2[:, g] = (dev * dev).sum(axis=(1, 2))
    return count, mean, m2


def chan_combine(parts):
    """Merge a sequence of (count, mean, M2) triples (arrays of equal shape) into one triple."""
    parts = list(parts)
    counts = [np.asarray(p[0], dtype=np.int64) for p in parts]
    n = sum(counts)
    mean = sum(c.astype(np.float64) * np.asarray(p[1], dtype=np.float64)
               for c, p in zip(counts, parts)) / n
    m2 = sum(np.asarray(p[2], dtype=np.float64)
             + c.astype(np.float64) * (np.asarray(p[1], dtype=np.float64) - mean) ** 2
             for c, p in zip(counts, parts))
    return n, mean, m2


def normalize_with(x: np.ndarray, groups: int, mean, var, eps: float, gamma=None, beta=None):
    """(x - mean) / sqrt(var + eps) * gamma + beta with given per-(sample, group) mean and var."""
    x = np.asarray(x, dtype=np.float64)
    n, c = x.shape[0], x.shape[-1]
    xg = x.reshape(n, -1, groups, c // groups)
    mean = np.asarray(mean, dtype=np.float64)[:, None, :, None]
    var = np.asarray(var, dtype=np.float64)[:, None, :, None]
    y = ((xg - mean) / np.sqrt(var + eps)).reshape(x.shape)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)
    return y
