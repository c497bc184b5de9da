"""Helpers for GPU-vs-oracle parity tests: the tolerance metrics, running
one shard through the C ABI, and comparisons on sampled outputs."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances: fp32 workloads within 1e-5 relative Frobenius error; bf16
# workloads within 4e-3 relative Frobenius error and a max abs error of at
# most 1e-2 of the reference's max abs value.
F32_REL_FRO = 1e-5
BF16_REL_FRO = 4e-3
BF16_MAX_RATIO = 1e-2


def to_np64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rel_fro(got, ref) -> float:
    got, ref = to_np64(got), to_np64(ref)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def max_ratio(got, ref) -> float:
    got, ref = to_np64(got), to_np64(ref)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0)) if ref.size else 0.0


def assert_close(got, ref, dtype: str, what: str = ""):
    got, ref = to_np64(got), to_np64(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rf = rel_fro(got, ref)
    if dtype == "f32":
        assert rf <= F32_REL_FRO, f"{what}: rel_fro {rf:.3e} > {F32_REL_FRO}"
    else:
        mr = max_ratio(got, ref)
        assert rf <= BF16_REL_FRO, f"{what}: rel_fro {rf:.3e} > {BF16_REL_FRO}"
        assert mr <= BF16_MAX_RATIO, f"{what}: max ratio {mr:.3e} > {BF16_MAX_RATIO}"
    return rf


def dev(x, device="cuda"):
    return None if x is None else x.to(device).contiguous()


def gpu_shard_fwd(B, w, d, r, stream=None):
    """Runs tp_mlp_shard_fwd for rank r of workload w on device inputs d."""
    T, h, n = w.T, w.h, w.n
    dt = d["X"].dtype
    H = torch.empty(T, n, dtype=dt, device="cuda")
    Y = torch.empty(T, n, dtype=dt, device="cuda")
    Z = torch.empty(T, h, dtype=torch.float32, device="cuda")
    B.tp_mlp_shard_fwd(d["X"], d["W1"][r], d["b1"][r], d["W2"][r], H, Y, Z, T, h, w.ffn, w.t, r,
                       dt, stream=stream)
    return Y, H, Z


def gpu_shard_bwd(B, w, d, r, Y, H, with_db1=True, stream=None):
    T, h, n = w.T, w.h, w.n
    dt = d["X"].dtype
    dY = torch.empty(T, n, dtype=dt, device="cuda")
    dW2 = torch.empty(n, h, dtype=torch.float32, device="cuda")
    dW1 = torch.empty(h, n, dtype=torch.float32, device="cuda")
    dX = torch.empty(T, h, dtype=torch.float32, device="cuda")
    db1 = torch.empty(n, dtype=torch.float32, device="cuda") if with_db1 else None
    B.tp_mlp_shard_bwd(d["X"], d["W1"][r], d["W2"][r], Y, H, d["dZ"], dY, dW2, dW1, dX, db1,
                       T, h, w.ffn, w.t, r, dt, stream=stream)
    return {"dY": dY, "dW2": dW2, "dW1": dW1, "dX": dX, "db1": db1}


def to_device(inputs: dict) -> dict:
    out = {"X": dev(inputs["X"]), "dZ": dev(inputs["dZ"])}
    for k in ("W1", "b1", "W2"):
        out[k] = {r: dev(v) for r, v in inputs[k].items()}
    return out


def sample_indices(extent: int, count: int, seed: int) -> np.ndarray:
    """First, last and a few seeded interior indices (sorted, unique)."""
    rng = np.random.default_rng(seed)
    idx = {0, extent - 1, extent // 2}
    idx.update(rng.integers(0, extent, size=max(0, count - 3)).tolist())
    return np.array(sorted(i for i in idx if 0 <= i < extent))
