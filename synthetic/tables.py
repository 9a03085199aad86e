"""Seeded probability tables and embeddings for cache-update tests.

Plain draws only: uniform, bf16-quantised (many exact ties) or constant
probabilities, and normal embeddings. No step of the method lives here.
"""
from __future__ import annotations

import numpy as np


def random_probs(rows: int, n_spk: int, seed: int, kind: str = "uniform") -> np.ndarray:
    """float32 (rows, n_spk) in [0, 1].

    kind: "uniform" U(0,1); "q256" multiples of 1/256 (ties between rows are
    common, as with bf16-quantised outputs); "coarse" multiples of 1/8 (heavy
    ties, exact 0.5 included); "equal" every entry 0.75 (all keys tie).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.random((rows, n_spk)).astype(np.float32)
    if kind == "uniform":
        return p
    if kind == "q256":
        return (np.floor(p * 256.0) / 256.0).astype(np.float32)
    if kind == "coarse":
        return (np.floor(p * 8.0) / 8.0).astype(np.float32)
    if kind == "equal":
        return np.full((rows, n_spk), 0.75, dtype=np.float32)
    raise ValueError(kind)


def random_embeddings(rows: int, dim: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.normal(0.0, 1.0, size=(rows, dim)).astype(np.float32)
