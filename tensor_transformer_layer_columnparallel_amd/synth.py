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

from .configs import AttnWorkload, Workload

TAG_X, TAG_W1, TAG_B1, TAG_W2, TAG_DZ = 1, 2, 3, 4, 5
TAG_WQKV, TAG_BQKV, TAG_O, TAG_WO = 6, 7, 8, 9
TAG_DQKV, TAG_DZO = 10, 11


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


def make_attn_inputs(aw: AttnWorkload, seed: int = 0) -> dict:
    """Host tensors for an attention-projection workload, unsharded:
    ``{"X": [T,h], "Wqkv": [h,3h] = [Wq | Wk | Wv], "bqkv": [3h],
    "O": [T,h] (the attention core's output, drawn), "Wo": [h,h]}``.
    Same recipe as :func:`make_inputs` (std 1 for activations, std_w for
    weights and biases, one bf16 rounding)."""
    dt = torch.float32 if aw.dtype == "f32" else torch.bfloat16
    h = aw.h
    return {"X": draw((aw.T, h), 1.0, seed, TAG_X, 0, dt),
            "Wqkv": draw((h, 3 * h), aw.std_w, seed, TAG_WQKV, 0, dt),
            "bqkv": draw((3 * h,), aw.std_w, seed, TAG_BQKV, 0, dt),
            "O": draw((aw.T, h), 1.0, seed, TAG_O, 0, dt),
            "Wo": draw((h, h), aw.std_w, seed, TAG_WO, 0, dt)}


def make_attn_grads(aw: AttnWorkload, seed: int = 0) -> dict:
    """Output gradients for the attention projections' backward, unsharded:
    ``{"dQKV": [T,3h] (of [Q | K | V]), "dZ": [T,h] (of the output
    projection)}``, drawn N(0, 1) and rounded once like the activations."""
    dt = torch.float32 if aw.dtype == "f32" else torch.bfloat16
    return {"dQKV": draw((aw.T, 3 * aw.h), 1.0, seed, TAG_DQKV, 0, dt),
            "dZ": draw((aw.T, aw.h), 1.0, seed, TAG_DZO, 0, dt)}


def qkv_columns(aw: AttnWorkload, r: int) -> torch.Tensor:
    """Column indices of [Wq | Wk | Wv] that rank r owns: its heads' columns
    of Q, then of K, then of V (a head-boundary split, not a contiguous
    block of the fused weight)."""
    w = aw.w
    return torch.cat([torch.arange(part * aw.h + r * w, part * aw.h + (r + 1) * w)
                      for part in range(3)])


def attn_shard(aw: AttnWorkload, full: dict, r: int) -> dict:
    """Rank r's operands: W_qkv_r [h, 3h/t], b_qkv_r [3h/t], O_r [T, h/t]
    (the columns of its heads) and W_o_r [h/t, h] (the matching rows)."""
    cols = qkv_columns(aw, r)
    w = aw.w
    return {"Wqkv": full["Wqkv"][:, cols].contiguous(), "bqkv": full["bqkv"][cols].contiguous(),
            "O": full["O"][:, r * w:(r + 1) * w].contiguous(),
            "Wo": full["Wo"][r * w:(r + 1) * w, :].contiguous()}
