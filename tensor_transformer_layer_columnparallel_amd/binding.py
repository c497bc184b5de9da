"""ctypes binding of libtpmlp (declared in include/tp_mlp.h).

Argument marshalling only: tensors become device pointers, torch dtypes
become the ABI's enum values, a missing stream becomes torch's current
stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind.  If the library is missing, importing this
module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so the library binds to it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpmlp.so")

TP_OK = 0
TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_INDIVISIBLE, TP_ERR_RANK = -1, -2, -3, -4
TP_ERR_DTYPE, TP_ERR_ALIGN, TP_ERR_HIP, TP_ERR_ARG = -5, -6, -7, -8
TP_F32, TP_BF16 = 0, 1
TP_ACT_NONE, TP_ACT_GELU_TANH = 0, 1
TP_REDUCE_SUM, TP_REDUCE_CONCAT, TP_REDUCE_CONCAT_TOKENS = 0, 1, 2

ABI_FUNCTIONS = ("tp_column_linear", "tp_row_linear", "tp_mlp_shard_fwd",
                 "tp_mlp_shard_bwd", "tp_shard_reduce", "tp_shard_reduce_scatter",
                 "tp_layernorm", "tp_status_string")


class TPError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_text(status)})")


def load_library() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.tp_column_linear.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, ci, ci, ci, vp]
    lib.tp_row_linear.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ci, ci, vp]
    lib.tp_mlp_shard_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, ci, vp]
    lib.tp_mlp_shard_bwd.argtypes = [vp] * 11 + [i64, i64, i64, ci, ci, ci, vp]
    lib.tp_shard_reduce.argtypes = [vp, vp, i64, i64, ci, ci, ci, ci, vp]
    lib.tp_shard_reduce_scatter.argtypes = [vp, vp, i64, i64, ci, ci, ci, ci, vp]
    lib.tp_layernorm.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_float, ci, ci, vp]
    for name in ABI_FUNCTIONS[:-1]:
        getattr(lib, name).restype = ci
    lib.tp_status_string.argtypes = [ci]
    lib.tp_status_string.restype = ctypes.c_char_p
    return lib


_lib = load_library()


def status_text(status: int) -> str:
    return _lib.tp_status_string(int(status)).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr() or None
    return int(x) or None


def _dt(d) -> int:
    if d in (torch.float32, "f32", TP_F32):
        return TP_F32
    if d in (torch.bfloat16, "bf16", TP_BF16):
        return TP_BF16
    return int(d)  # passed through; the library rejects unknown values


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def _ret(fn: str, status: int, check: bool) -> int:
    if check and status != TP_OK:
        raise TPError(fn, status)
    return status


def tp_column_linear(X, W_i, b_i, Y_i, pre_save, tokens, in_features, out_features, t, rank,
                     dtype, out_dtype, act, stream=None, check=True) -> int:
    st = _lib.tp_column_linear(_ptr(X), _ptr(W_i), _ptr(b_i), _ptr(Y_i), _ptr(pre_save),
                               tokens, in_features,
                               out_features, t, rank, _dt(dtype), _dt(out_dtype), int(act),
                               _stream(stream))
    return _ret("tp_column_linear", st, check)


def tp_row_linear(X_i, W_i, Z_i, tokens, in_features, out_features, t, rank, dtype,
                  out_dtype, stream=None, check=True) -> int:
    st = _lib.tp_row_linear(_ptr(X_i), _ptr(W_i), _ptr(Z_i), tokens, in_features, out_features,
                            t, rank, _dt(dtype), _dt(out_dtype), _stream(stream))
    return _ret("tp_row_linear", st, check)


def tp_mlp_shard_fwd(X, W1_i, b1_i, W2_i, H_i, Y_i_save, Z_i, tokens, h, ffn, t, rank, dtype,
                     stream=None, check=True) -> int:
    st = _lib.tp_mlp_shard_fwd(_ptr(X), _ptr(W1_i), _ptr(b1_i), _ptr(W2_i), _ptr(H_i),
                               _ptr(Y_i_save), _ptr(Z_i), tokens, h, ffn, t, rank, _dt(dtype),
                               _stream(stream))
    return _ret("tp_mlp_shard_fwd", st, check)


def tp_mlp_shard_bwd(X, W1_i, W2_i, Y_i, H_i, dZ, dY_i, dW2_i, dW1_i, dX_i, db1_i, tokens, h,
                     ffn, t, rank, dtype, stream=None, check=True) -> int:
    st = _lib.tp_mlp_shard_bwd(_ptr(X), _ptr(W1_i), _ptr(W2_i), _ptr(Y_i), _ptr(H_i), _ptr(dZ),
                               _ptr(dY_i), _ptr(dW2_i), _ptr(dW1_i), _ptr(dX_i), _ptr(db1_i),
                               tokens, h, ffn, t, rank, _dt(dtype), _stream(stream))
    return _ret("tp_mlp_shard_bwd", st, check)


def tp_shard_reduce(parts, out, tokens, cols, t, op, in_dtype, out_dtype, stream=None,
                    check=True) -> int:
    st = _lib.tp_shard_reduce(_ptr(parts), _ptr(out), tokens, cols, t, int(op), _dt(in_dtype),
                              _dt(out_dtype), _stream(stream))
    return _ret("tp_shard_reduce", st, check)


def tp_shard_reduce_scatter(parts, out, tokens, cols, t, rank, in_dtype, out_dtype, stream=None,
                            check=True) -> int:
    st = _lib.tp_shard_reduce_scatter(_ptr(parts), _ptr(out), tokens, cols, t, rank,
                                      _dt(in_dtype), _dt(out_dtype), _stream(stream))
    return _ret("tp_shard_reduce_scatter", st, check)


def tp_layernorm(x, gamma, beta, y, tokens, cols, eps, in_dtype, out_dtype, stream=None,
                 check=True) -> int:
    st = _lib.tp_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), tokens, cols, float(eps),
                           _dt(in_dtype), _dt(out_dtype), _stream(stream))
    return _ret("tp_layernorm", st, check)


def tp_status_string(status: int) -> str:
    return status_text(status)
