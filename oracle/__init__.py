"""fp64 CPU oracle for one tensor-parallel rank's share of a transformer MLP.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or runs it, and
it imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (plain double-precision loops, OpenMP
over output rows).  This module loads it with ctypes and adds:

* thin numpy wrappers (argument marshalling only), and
* *sampled* evaluations for full-size checks.  A sample is always the same
  method applied to a smaller instance of itself, never a rewritten formula:
  - a subset R of token rows: every output row of the forward, and the rows
    of dY_i and dX_i, depend only on the same rows of X and dZ, so the oracle
    run on X[R], dZ[R] yields exactly those rows;
  - a subset J of a shard's columns: by the column split of the page
    "Tensor Parallelism原理与实践" §2.1 a set of columns of W1_i (with the same
    rows of W2_i) is itself a narrower column shard, so the oracle run on
    W1_i[:, J], b1_i[J], W2_i[J, :] yields exactly Y_i[:, J], H_i[:, J],
    dY_i[:, J], dW1_i[:, J] and dW2_i[J, :].

Parity pins for every function here live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile oracle.c (or another source, e.g. a test's deliberately broken
    copy) into a shared library with gcc (portable x86-64 code, no
    -march=native, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               "-D_DEFAULT_SOURCE", src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = load_library(_LIB_PATH)
    return _lib


def load_library(path: str):
    """Loads a build of oracle.c and declares its functions' signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    sig = {
        "oracle_gelu_tanh": [dp, dp, i64],
        "oracle_gelu_tanh_grad": [dp, dp, i64],
        "oracle_matmul": [dp, dp, dp, i64, i64, i64],
        "oracle_column_linear": [dp, dp, dp, dp, i64, i64, i64, ctypes.c_int],
        "oracle_row_linear": [dp, dp, dp, i64, i64, i64],
        "oracle_mlp_shard_fwd": [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64],
        "oracle_mlp_shard_bwd": [dp] * 11 + [i64, i64, i64],
        "oracle_linear_bwd": [dp] * 6 + [i64, i64, i64],
        "oracle_shard_sum": [dp, dp, ctypes.c_int, i64],
        "oracle_shard_concat": [dp, dp, ctypes.c_int, i64, i64],
        "oracle_reduce_scatter": [dp, dp, ctypes.c_int, i64, i64, ctypes.c_int],
        "oracle_layernorm": [dp, dp, dp, dp, i64, i64, ctypes.c_double],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    return lib


def _f64(a) -> np.ndarray:
    """Widen to a C-contiguous float64 array (exact for bf16 / fp32 values)."""
    if hasattr(a, "detach"):  # torch tensor: widen on the host
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def gelu_tanh(y) -> np.ndarray:
    y = _f64(y)
    out = np.empty_like(y)
    _load().oracle_gelu_tanh(_p(y), _p(out), y.size)
    return out


def gelu_tanh_grad(y) -> np.ndarray:
    y = _f64(y)
    out = np.empty_like(y)
    _load().oracle_gelu_tanh_grad(_p(y), _p(out), y.size)
    return out


def matmul(A, B) -> np.ndarray:
    A, B = _f64(A), _f64(B)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    C = np.empty((M, N), dtype=np.float64)
    _load().oracle_matmul(_p(A), _p(B), _p(C), M, K, N)
    return C


def column_linear(X, W_i, b_i=None, gelu: bool = False) -> np.ndarray:
    """Y_i = X W_i + b_i (optionally g(Y_i)) for one column shard."""
    X, W_i = _f64(X), _f64(W_i)
    b_i = None if b_i is None else _f64(b_i)
    T, h = X.shape
    h2, n = W_i.shape
    assert h == h2 and (b_i is None or b_i.shape == (n,))
    Y = np.empty((T, n), dtype=np.float64)
    _load().oracle_column_linear(_p(X), _p(W_i), _p(b_i), _p(Y), T, h, n, int(gelu))
    return Y


def row_linear(X_i, W_i) -> np.ndarray:
    """Z_i = X_i W_i, the row-parallel partial (no bias)."""
    X_i, W_i = _f64(X_i), _f64(W_i)
    T, n = X_i.shape
    n2, h = W_i.shape
    assert n == n2
    Z = np.empty((T, h), dtype=np.float64)
    _load().oracle_row_linear(_p(X_i), _p(W_i), _p(Z), T, n, h)
    return Z


def mlp_shard_fwd(X, W1_i, b1_i, W2_i):
    """Returns (Y_i, H_i, Z_i) for one shard; b1_i may be None."""
    X, W1_i, W2_i = _f64(X), _f64(W1_i), _f64(W2_i)
    b1_i = None if b1_i is None else _f64(b1_i)
    T, h = X.shape
    h2, n = W1_i.shape
    assert h == h2 and W2_i.shape == (n, h)
    Y = np.empty((T, n)); H = np.empty((T, n)); Z = np.empty((T, h))
    _load().oracle_mlp_shard_fwd(_p(X), _p(W1_i), _p(b1_i), _p(W2_i), _p(Y), _p(H), _p(Z),
                                 T, h, n)
    return Y, H, Z


def mlp_shard_bwd(X, W1_i, b1_i, W2_i, dZ):
    """Returns dict(dY, dW2, dW1, dX, db1) for one shard.  The shard's forward
    values Y_i, H_i are recomputed here by the oracle's own forward."""
    X, W1_i, W2_i, dZ = _f64(X), _f64(W1_i), _f64(W2_i), _f64(dZ)
    T, h = X.shape
    n = W1_i.shape[1]
    Y, H, _ = mlp_shard_fwd(X, W1_i, b1_i, W2_i)
    dY = np.empty((T, n)); dW2 = np.empty((n, h)); dW1 = np.empty((h, n))
    dX = np.empty((T, h)); db1 = np.empty(n)
    _load().oracle_mlp_shard_bwd(_p(X), _p(W1_i), _p(W2_i), _p(Y), _p(H), _p(dZ),
                                 _p(dY), _p(dW2), _p(dW1), _p(dX), _p(db1), T, h, n)
    return {"dY": dY, "dW2": dW2, "dW1": dW1, "dX": dX, "db1": db1}


def shard_sum(parts) -> np.ndarray:
    """Σ_r parts[r] in rank order; parts is [t, ...]."""
    parts = _f64(parts)
    t = parts.shape[0]
    out = np.empty(parts.shape[1:], dtype=np.float64)
    _load().oracle_shard_sum(_p(parts), _p(out), t, out.size)
    return out


def shard_concat(parts) -> np.ndarray:
    """Concatenate [t, rows, cols] shards along the last dim in rank order."""
    parts = _f64(parts)
    t, rows, cols = parts.shape
    out = np.empty((rows, t * cols), dtype=np.float64)
    _load().oracle_shard_concat(_p(parts), _p(out), t, rows, cols)
    return out


def reduce_scatter(parts, rank: int) -> np.ndarray:
    """Rank ``rank``'s block of rows of Σ_r parts[r]; parts is [t, rows, cols]
    with rows divisible by t."""
    parts = _f64(parts)
    t, rows, cols = parts.shape
    assert rows % t == 0 and 0 <= rank < t
    out = np.empty((rows // t, cols), dtype=np.float64)
    _load().oracle_reduce_scatter(_p(parts), _p(out), t, rows, cols, rank)
    return out


def layernorm(x, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """Row-wise layer normalisation of x [rows, cols] (biased variance)."""
    x = _f64(x)
    rows, cols = x.shape
    g = None if gamma is None else _f64(gamma)
    b = None if beta is None else _f64(beta)
    y = np.empty_like(x)
    _load().oracle_layernorm(_p(x), _p(g), _p(b), _p(y), rows, cols, float(eps))
    return y


def linear_bwd(X, W, dY, with_db: bool = True) -> dict:
    """dict(dX, dW, db) of one linear shard Y = X W + b (db None unless
    with_db): dX = dY W^T, dW = X^T dY, db = column sums of dY."""
    X, W, dY = _f64(X), _f64(W), _f64(dY)
    T, k = X.shape
    k2, n = W.shape
    assert k == k2 and dY.shape == (T, n)
    dX = np.empty((T, k)); dW = np.empty((k, n))
    db = np.empty(n) if with_db else None
    _load().oracle_linear_bwd(_p(X), _p(W), _p(dY), _p(dX), _p(dW), _p(db), T, k, n)
    return {"dX": dX, "dW": dW, "db": db}


# ---------------------------------------------------------------- sampling

def mlp_shard_fwd_rows(X, W1_i, b1_i, W2_i, rows):
    """(Y_i, H_i, Z_i) restricted to token rows ``rows``."""
    rows = np.asarray(rows)
    return mlp_shard_fwd(_f64(X[rows]), W1_i, b1_i, W2_i)


def mlp_shard_bwd_rows(X, W1_i, b1_i, W2_i, dZ, rows):
    """dY_i[rows, :] and dX_i[rows, :]: the backward on the token subset
    (the dW entries such a run returns are partial sums and are dropped)."""
    rows = np.asarray(rows)
    g = mlp_shard_bwd(_f64(X[rows]), W1_i, b1_i, W2_i, _f64(dZ[rows]))
    return {"dY": g["dY"], "dX": g["dX"]}


def mlp_shard_bwd_cols(X, W1_i, b1_i, W2_i, dZ, cols):
    """dY_i[:, cols], dW1_i[:, cols], dW2_i[cols, :] and db1_i[cols]: the
    backward of the narrower column shard made of ``cols`` (its dX is a
    partial and is dropped)."""
    cols = np.asarray(cols)
    W1_i, W2_i = _f64(W1_i), _f64(W2_i)
    b = None if b1_i is None else _f64(b1_i)[cols]
    g = mlp_shard_bwd(X, W1_i[:, cols], b, W2_i[cols, :], dZ)
    return {"dY": g["dY"], "dW1": g["dW1"], "dW2": g["dW2"], "db1": g["db1"]}
