"""Seeded synthetic inputs for the MLP shard workloads.

This module draws random numbers and rounds them to the storage type; it
holds none of the method's arithmetic.  Both the HIP path and the oracle are
fed from it.

Recipe (the pages fix only shapes and distributions; the rest is a choice):

* Each tensor has its own CPU ``torch.Generator`` seeded with
  ``seed * 1_000_003 + tag * 1024 + rank`` (tags: X=1, W1=2, b1=3, W2=4,
  dZ=5), so a shard's values do not depend on how many other shards are drawn.
* Values are ``torch.randn(float32) * std``: std 1 for X and dZ, ``std_w``
  (0.02) for W1, W2 and b1.  bf16 workloads round once to bf16
  (round-to-nearest-even, torch's conversion); fp32 workloads keep fp32.
* Shard r of W1 is the ``[h, n]`` block of columns ``[r*n, (r+1)*n)``; shard r
  of W2 is the ``[n, h]`` block of rows ``[r*n, (r+1)*n)`` (rank-ordered, the
  concatenation order of the page "张量并行实战", section "PyTorch 实现示例").
"""
from __future__ import annotations

import torch

from .configs import Workload

TAG_X, TAG_W1, TAG_B1, TAG_W2, TAG_DZ = 1, 2, 3, 4, 5


def _gen(seed: int, tag: int, rank: int = 0) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1_000_003 + tag * 1024 + rank)
    return g


def storage_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def draw(shape, std: float, seed: int, tag: int, rank: int, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, dtype=torch.float32, generator=_gen(seed, tag, rank))
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make_inputs(w: Workload, seed: int = 0, ranks=None, with_dz: bool | None = None) -> dict:
    """Host tensors for workload ``w``.

    Returns ``{"X": [T,h], "W1": {r: [h,n]}, "b1": {r: [n] or None},
    "W2": {r: [n,h]}, "dZ": [T,h] or None}`` in the storage dtype.
    """
    dt = storage_dtype(w)
    ranks = tuple(w.ranks if ranks is None else ranks)
    with_dz = w.backward if with_dz is None else with_dz
    out = {"X": draw((w.T, w.h), 1.0, seed, TAG_X, 0, dt), "W1": {}, "b1": {}, "W2": {}}
    for r in ranks:
        out["W1"][r] = draw((w.h, w.n), w.std_w, seed, TAG_W1, r, dt)
        if not w.bias:
            out["b1"][r] = None
        elif w.bias_zero:
            out["b1"][r] = torch.zeros(w.n, dtype=dt)
        else:
            out["b1"][r] = draw((w.n,), w.std_w, seed, TAG_B1, r, dt)
        if w.row_layer:
            out["W2"][r] = draw((w.n, w.h), w.std_w, seed, TAG_W2, r, dt)
    out["dZ"] = draw((w.T, w.h), 1.0, seed, TAG_DZ, 0, dt) if with_dz else None
    return out
