"""Seeded synthetic inputs for the sparse COO layer -- shared by the tests, the
benchmark and the smoke check.

This module holds no arithmetic of the method: it only draws random supports,
values and activations with the shapes, sparsities and distributions of the
workloads that the SNACK paper ("Beyond Masked Sparsity", Tables 2, 3, 11, 12
and Figures 2-3) and its GPT-2 experiment (Table 4) measure.  Both the HIP path
and the oracle consume what it returns; neither is imported here.

Recipe (every generator is numpy's PCG64, seeded from a SHA-256 of a text key
such as "c4/support/s95", so streams are reproducible across machines):

* support: ``nnz = M*K*(100 - s)//100`` distinct positions drawn uniformly
  without replacement from the M*K grid, returned in a random (unsorted)
  order so that canonicalisation is always exercised;
* weight values: normal with std ``1/sqrt((1 - s) * K)`` (the expected fan-in;
  for the 500x500 95 % layer this is 0.2);
* X, dY and regression targets: standard normal, fp32.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np


def rng_for(key: str) -> np.random.Generator:
    digest = hashlib.sha256(key.encode("utf-8")).digest()
    return np.random.Generator(np.random.PCG64(int.from_bytes(digest[:16], "little")))


def nnz_for(M: int, K: int, sparsity_pct: int) -> int:
    """Number of stored positions for an integer sparsity percentage (floor)."""
    return (M * K * (100 - int(sparsity_pct))) // 100


def weight_std(K: int, sparsity_pct: int) -> float:
    return 1.0 / float(np.sqrt((100 - sparsity_pct) / 100.0 * K))


def sample_positions(N: int, nnz: int, rng: np.random.Generator) -> np.ndarray:
    """nnz distinct integers from [0, N), uniformly, in random order (int64)."""
    if nnz < 0 or nnz > N:
        raise ValueError("nnz out of range")
    if nnz == 0:
        return np.empty(0, np.int64)
    if 3 * nnz >= N:
        return rng.permutation(N)[:nnz].astype(np.int64)
    got = np.empty(0, np.int64)
    while got.shape[0] < nnz:
        need = nnz - got.shape[0]
        extra = rng.integers(0, N, size=int(need * 1.08) + 64, dtype=np.int64)
        got = np.unique(np.concatenate([got, extra]))
    pick = rng.choice(got.shape[0], size=nnz, replace=False)
    return got[pick]


def random_layer(M: int, K: int, nnz: int, key: str, std: float | None = None):
    """(rows int32, cols int32, vals float32) with distinct positions, unsorted."""
    rng = rng_for(key + "/support")
    pos = sample_positions(M * K, nnz, rng)
    rows = (pos // K).astype(np.int32)
    cols = (pos % K).astype(np.int32)
    if std is None:
        std = 1.0 / np.sqrt(max(nnz, 1) / max(M, 1))
    vals = (rng_for(key + "/values").standard_normal(nnz) * std).astype(np.float32)
    return rows, cols, vals


def normal(shape, key: str, std: float = 1.0) -> np.ndarray:
    return (rng_for(key).standard_normal(shape) * std).astype(np.float32)


@dataclass
class LayerShape:
    M: int          # out_features
    K: int          # in_features
    sparsity: int   # percent

    @property
    def nnz(self) -> int:
        return nnz_for(self.M, self.K, self.sparsity)

    @property
    def std(self) -> float:
        return weight_std(self.K, self.sparsity)


@dataclass
class Workload:
    name: str
    description: str
    layers: list = field(default_factory=list)  # list of LayerShape
    batches: tuple = (1,)
    iters: int = 1
    prune_every: int = 0
    lr: float = 0.01


def workloads() -> dict:
    """The five synthetic workloads (stand-ins for the pages' measurements)."""
    w = {}
    w["c1"] = Workload("c1", "500x500, 95% sparse, batch 1, fwd + dX + dW",
                       [LayerShape(500, 500, 95)], batches=(1,))
    w["c2"] = Workload("c2", "5000x5000 sparsity sweep 50/70/90/95/99%, batch 1-2, forward only",
                       [LayerShape(5000, 5000, s) for s in (50, 70, 90, 95, 99)], batches=(1, 2))
    w["c3"] = Workload("c3", "10000x10000 at 90/95/99%, batch 4, 100 SGD iterations lr 0.01, MSE",
                       [LayerShape(10000, 10000, s) for s in (90, 95, 99)], batches=(4,), iters=100)
    w["c4"] = Workload("c4", "10000x10000, 95% sparse, batch 1..64, fwd+bwd, drop/regrow 30% every 10 iters",
                       [LayerShape(10000, 10000, 95)], batches=(1, 2, 4, 8, 16, 32, 64), iters=10,
                       prune_every=10)
    w["c5"] = Workload("c5", "GPT-2-small MLP stack: 12 x (768->3072, GELU, 3072->768) at 90/99%, 1024 tokens",
                       [LayerShape(3072, 768, s) for s in (90, 99)] + [LayerShape(768, 3072, s) for s in (90, 99)],
                       batches=(1024,), iters=50, prune_every=50)
    return w
