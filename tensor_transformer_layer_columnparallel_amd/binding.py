"""ctypes binding of libtpmlp (declared in include/tp_mlp.h).

Argument marshalling only: tensors become device pointers, torch dtypes
become the ABI's enum values, a missing stream becomes torch's current
stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind.  If the library is missing, importing this
module raises.

Tensor arguments are checked before the call, because the library sees only
addresses: a tensor must be a contiguous device tensor whose element size
matches the element type it is declared with and which holds at least the
elements the call reads or writes (ValueError otherwise).  Plain integer
addresses are passed through unchecked.  Shape arguments the library itself
rejects (negative, indivisible, unknown types) skip the size check and get
the library's status.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loads torch's HIP runtime first, so the library binds to it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpmlp.so")

TP_OK = 0
TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_INDIVISIBLE, TP_ERR_RANK = -1, -2, -3, -4
TP_ERR_DTYPE, TP_ERR_ALIGN, TP_ERR_HIP, TP_ERR_ARG, TP_ERR_OVERLAP = -5, -6, -7, -8, -9
TP_F32, TP_BF16 = 0, 1
TP_ACT_NONE, TP_ACT_GELU_TANH = 0, 1
TP_REDUCE_SUM, TP_REDUCE_CONCAT, TP_REDUCE_CONCAT_TOKENS = 0, 1, 2

ABI_FUNCTIONS = ("tp_column_linear", "tp_row_linear", "tp_mlp_shard_fwd",
                 "tp_mlp_layer_fwd", "tp_mlp_shard_bwd", "tp_linear_bwd", "tp_shard_reduce",
                 "tp_shard_reduce_scatter", "tp_layernorm", "tp_shard_reduce_scatter_layernorm",
                 "tp_status_string")


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
    lib.tp_mlp_layer_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, vp]
    lib.tp_mlp_shard_bwd.argtypes = [vp] * 11 + [i64, i64, i64, ci, ci, ci, vp]
    lib.tp_linear_bwd.argtypes = [vp] * 6 + [i64, i64, i64, ci, vp]
    lib.tp_shard_reduce.argtypes = [vp, vp, i64, i64, ci, ci, ci, ci, vp]
    lib.tp_shard_reduce_scatter.argtypes = [vp, vp, i64, i64, ci, ci, ci, ci, vp]
    lib.tp_layernorm.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_float, ci, ci, vp]
    lib.tp_shard_reduce_scatter_layernorm.argtypes = [vp, vp, vp, vp, i64, i64, ci, ci,
                                                      ctypes.c_float, ci, ci, vp]
    for name in ABI_FUNCTIONS[:-1]:
        getattr(lib, name).restype = ci
    lib.tp_status_string.argtypes = [ci]
    lib.tp_status_string.restype = ctypes.c_char_p
    return lib


_lib = load_library()


def status_text(status: int) -> str:
    return _lib.tp_status_string(int(status)).decode()


_ELT_BYTES = {TP_F32: 4, TP_BF16: 2}


def _ptr(x, name: str = "tensor", dtype=None, count: int | None = None):
    """Device address of x.  For a tensor: checks the element size against
    ``dtype`` (an ABI element type) and that it holds ``count`` elements."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        es = _ELT_BYTES.get(dtype)
        if es is not None and x.element_size() != es:
            raise ValueError(f"{name}: element size {x.element_size()} does not match the "
                             f"declared element type ({es} bytes)")
        if count is not None and count >= 0 and x.numel() < count:
            raise ValueError(f"{name}: holds {x.numel()} elements, the call uses {count}")
        if not x.is_contiguous():
            raise ValueError(f"{name}: must be contiguous (the library reads dense row-major "
                             "memory)")
        if x.device.type != "cuda":
            raise ValueError(f"{name}: must be a device tensor, not on {x.device}")
        return x.data_ptr() or None
    return int(x) or None


def _split(total: int, t: int) -> int:
    """total / t where the library accepts it, else -1 (no size check)."""
    return total // t if t > 0 and total >= 0 and total % t == 0 else -1


def _prod(*dims) -> int:
    return -1 if any(d < 0 for d in dims) else math.prod(dims)


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
    dt, odt, n = _dt(dtype), _dt(out_dtype), _split(out_features, t)
    st = _lib.tp_column_linear(_ptr(X, "X", dt, _prod(tokens, in_features)),
                               _ptr(W_i, "W_i", dt, _prod(in_features, n)),
                               _ptr(b_i, "b_i", dt, n),
                               _ptr(Y_i, "Y_i", odt, _prod(tokens, n)),
                               _ptr(pre_save, "pre_save", dt, _prod(tokens, n)),
                               tokens, in_features, out_features, t, rank, dt, odt, int(act),
                               _stream(stream))
    return _ret("tp_column_linear", st, check)


def tp_row_linear(X_i, W_i, Z_i, tokens, in_features, out_features, t, rank, dtype,
                  out_dtype, stream=None, check=True) -> int:
    dt, odt, k = _dt(dtype), _dt(out_dtype), _split(in_features, t)
    st = _lib.tp_row_linear(_ptr(X_i, "X_i", dt, _prod(tokens, k)),
                            _ptr(W_i, "W_i", dt, _prod(k, out_features)),
                            _ptr(Z_i, "Z_i", odt, _prod(tokens, out_features)),
                            tokens, in_features, out_features, t, rank, dt, odt, _stream(stream))
    return _ret("tp_row_linear", st, check)


def tp_mlp_shard_fwd(X, W1_i, b1_i, W2_i, H_i, Y_i_save, Z_i, tokens, h, ffn, t, rank, dtype,
                     stream=None, check=True) -> int:
    dt, n = _dt(dtype), _split(ffn, t)
    st = _lib.tp_mlp_shard_fwd(_ptr(X, "X", dt, _prod(tokens, h)),
                               _ptr(W1_i, "W1_i", dt, _prod(h, n)),
                               _ptr(b1_i, "b1_i", dt, n),
                               _ptr(W2_i, "W2_i", dt, _prod(n, h)),
                               _ptr(H_i, "H_i", dt, _prod(tokens, n)),
                               _ptr(Y_i_save, "Y_i_save", dt, _prod(tokens, n)),
                               _ptr(Z_i, "Z_i", TP_F32, _prod(tokens, h)),
                               tokens, h, ffn, t, rank, dt, _stream(stream))
    return _ret("tp_mlp_shard_fwd", st, check)


def tp_mlp_layer_fwd(X, W1, b1, W2, H, Y_save, Z, tokens, h, ffn, t, dtype, stream=None,
                     check=True) -> int:
    """Every rank's shard forward at once; W1 [t][h][n], b1 [t][n], W2 [t][n][h],
    H and Y_save [t][tokens][n], Z [t][tokens][h] (fp32)."""
    dt, n = _dt(dtype), _split(ffn, t)
    tt = t if t > 0 else -1
    st = _lib.tp_mlp_layer_fwd(_ptr(X, "X", dt, _prod(tokens, h)),
                               _ptr(W1, "W1", dt, _prod(tt, h, n)),
                               _ptr(b1, "b1", dt, _prod(tt, n)),
                               _ptr(W2, "W2", dt, _prod(tt, n, h)),
                               _ptr(H, "H", dt, _prod(tt, tokens, n)),
                               _ptr(Y_save, "Y_save", dt, _prod(tt, tokens, n)),
                               _ptr(Z, "Z", TP_F32, _prod(tt, tokens, h)),
                               tokens, h, ffn, t, dt, _stream(stream))
    return _ret("tp_mlp_layer_fwd", st, check)


def tp_mlp_shard_bwd(X, W1_i, W2_i, Y_i, H_i, dZ, dY_i, dW2_i, dW1_i, dX_i, db1_i, tokens, h,
                     ffn, t, rank, dtype, stream=None, check=True) -> int:
    dt, n = _dt(dtype), _split(ffn, t)
    Th, Tn, hn = _prod(tokens, h), _prod(tokens, n), _prod(h, n)
    st = _lib.tp_mlp_shard_bwd(_ptr(X, "X", dt, Th), _ptr(W1_i, "W1_i", dt, hn),
                               _ptr(W2_i, "W2_i", dt, hn), _ptr(Y_i, "Y_i", dt, Tn),
                               _ptr(H_i, "H_i", dt, Tn), _ptr(dZ, "dZ", dt, Th),
                               _ptr(dY_i, "dY_i", dt, Tn), _ptr(dW2_i, "dW2_i", TP_F32, hn),
                               _ptr(dW1_i, "dW1_i", TP_F32, hn), _ptr(dX_i, "dX_i", TP_F32, Th),
                               _ptr(db1_i, "db1_i", TP_F32, n),
                               tokens, h, ffn, t, rank, dt, _stream(stream))
    return _ret("tp_mlp_shard_bwd", st, check)


def tp_linear_bwd(X, W, dY, dX, dW, db, tokens, in_features, out_features, dtype, stream=None,
                  check=True) -> int:
    dt = _dt(dtype)
    Tk, Tn, kn = (_prod(tokens, in_features), _prod(tokens, out_features),
                  _prod(in_features, out_features))
    st = _lib.tp_linear_bwd(_ptr(X, "X", dt, Tk), _ptr(W, "W", dt, kn), _ptr(dY, "dY", dt, Tn),
                            _ptr(dX, "dX", TP_F32, Tk), _ptr(dW, "dW", TP_F32, kn),
                            _ptr(db, "db", TP_F32, out_features), tokens, in_features,
                            out_features, dt, _stream(stream))
    return _ret("tp_linear_bwd", st, check)


def tp_shard_reduce(parts, out, tokens, cols, t, op, in_dtype, out_dtype, stream=None,
                    check=True) -> int:
    idt, odt = _dt(in_dtype), _dt(out_dtype)
    n_out = _prod(tokens, cols) if int(op) == TP_REDUCE_SUM else _prod(t, tokens, cols)
    st = _lib.tp_shard_reduce(_ptr(parts, "parts", idt, _prod(t, tokens, cols)),
                              _ptr(out, "out", odt, n_out), tokens, cols, t, int(op), idt, odt,
                              _stream(stream))
    return _ret("tp_shard_reduce", st, check)


def tp_shard_reduce_scatter(parts, out, tokens, cols, t, rank, in_dtype, out_dtype, stream=None,
                            check=True) -> int:
    idt, odt = _dt(in_dtype), _dt(out_dtype)
    st = _lib.tp_shard_reduce_scatter(_ptr(parts, "parts", idt, _prod(t, tokens, cols)),
                                      _ptr(out, "out", odt, _prod(_split(tokens, t), cols)),
                                      tokens, cols, t, rank, idt, odt, _stream(stream))
    return _ret("tp_shard_reduce_scatter", st, check)


def tp_layernorm(x, gamma, beta, y, tokens, cols, eps, in_dtype, out_dtype, stream=None,
                 check=True) -> int:
    idt, odt = _dt(in_dtype), _dt(out_dtype)
    st = _lib.tp_layernorm(_ptr(x, "x", idt, _prod(tokens, cols)),
                           _ptr(gamma, "gamma", odt, cols), _ptr(beta, "beta", odt, cols),
                           _ptr(y, "y", odt, _prod(tokens, cols)), tokens, cols, float(eps),
                           idt, odt, _stream(stream))
    return _ret("tp_layernorm", st, check)


def tp_shard_reduce_scatter_layernorm(parts, gamma, beta, y, tokens, cols, t, rank, eps,
                                      in_dtype, out_dtype, stream=None, check=True) -> int:
    idt, odt = _dt(in_dtype), _dt(out_dtype)
    st = _lib.tp_shard_reduce_scatter_layernorm(
        _ptr(parts, "parts", idt, _prod(t, tokens, cols)), _ptr(gamma, "gamma", odt, cols),
        _ptr(beta, "beta", odt, cols), _ptr(y, "y", odt, _prod(_split(tokens, t), cols)), tokens,
        cols, t, rank, float(eps), idt, odt, _stream(stream))
    return _ret("tp_shard_reduce_scatter_layernorm", st, check)


def tp_status_string(status: int) -> str:
    return status_text(status)
