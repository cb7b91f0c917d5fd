"""Token and key-column selectors (oracle; test infrastructure only).

Basis: FlashLoop abstract -- loop updates concentrate on a small subset of
tokens (token-sparse update) and attention differences on a sparse, stable
subset of key columns.  The pages fix no rule; the readings used are:

* kept-token count per sequence n = clamp(ceil(rho * T - 1e-9), 1, T);
* a selector keeps the ``n`` largest keys, ties going to the lower index, and
  returns the kept indices in ascending order.
"""
from __future__ import annotations

import math

import numpy as np


def n_selected(rho: float, tokens: int) -> int:
    """Kept-token count for keep fraction ``rho`` over ``tokens`` rows."""
    if tokens <= 0:
        return 0
    n = math.ceil(rho * tokens - 1e-9)
    return max(1, min(tokens, n))


def top_n_ascending(keys: np.ndarray, n: int) -> np.ndarray:
    """Indices of the ``n`` largest entries of a 1-D key vector.

    Order is by (key descending, index ascending); the kept set is returned
    sorted ascending.  Keys must be finite.
    """
    keys = np.asarray(keys)
    if keys.ndim != 1:
        raise ValueError("keys must be 1-D")
    if not np.all(np.isfinite(keys)):
        raise ValueError("keys must be finite")
    n = max(0, min(int(n), keys.shape[0]))
    idx = np.arange(keys.shape[0])
    order = np.lexsort((idx, -keys.astype(np.float64)))
    return np.sort(order[:n]).astype(np.int32)
