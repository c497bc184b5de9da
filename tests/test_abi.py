"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU (every
call here fails validation, so no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_mlp.h")


def _declared_functions():
    text = open(HEADER).read()
    return re.findall(r"TP_API\s+(?:const\s+)?\w+\s*\*?\s*(tp_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def B():
    from tensor_transformer_layer_columnparallel_amd import binding
    return binding


@pytest.fixture(scope="module")
def Bfake(B):
    """The binding, for calls with fake addresses.  Those calls must fail
    validation; should one of them not, it would launch on a bogus address,
    so they run only where no GPU is visible."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("fake-address validation tests run only without a visible GPU")
    return B


def test_header_declares_the_entry_points_and_status_string():
    assert set(_declared_functions()) == {
        "tp_column_linear", "tp_row_linear", "tp_mlp_shard_fwd", "tp_mlp_layer_fwd",
        "tp_mlp_shard_bwd",
        "tp_linear_bwd", "tp_shard_reduce", "tp_shard_reduce_scatter", "tp_layernorm",
        "tp_shard_reduce_scatter_layernorm", "tp_status_string"}


def test_library_exports_every_declared_symbol(B):
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_package_exposes_every_entry_point(B):
    import tensor_transformer_layer_columnparallel_amd as pkg
    for name in _declared_functions():
        assert name in B.ABI_FUNCTIONS, name
        assert callable(getattr(pkg, name)), name
    assert pkg.TP_REDUCE_CONCAT_TOKENS == 2 and pkg.TP_BF16 == 1


def test_status_strings(B):
    for st in range(0, -10, -1):
        assert B.tp_status_string(st) and B.tp_status_string(st) != "unknown status"
    assert B.tp_status_string(12345) == "unknown status"


# Fake, 16-byte-aligned device addresses: validation must reject each call
# before any HIP call is made, so they are never dereferenced.
P = 0x10000
P2 = 0x20000
MIS = 0x10008


def test_column_linear_rejects(Bfake):
    B = Bfake
    f = lambda **kw: B.tp_column_linear(**{**dict(
        X=P, W_i=P, b_i=None, Y_i=P, pre_save=None, tokens=32, in_features=768, out_features=3072, t=4,
        rank=0, dtype=B.TP_BF16, out_dtype=B.TP_BF16, act=B.TP_ACT_NONE, stream=0,
        check=False), **kw})
    assert f(X=None) == B.TP_ERR_NULL
    assert f(Y_i=None) == B.TP_ERR_NULL
    assert f(W_i=MIS) == B.TP_ERR_ALIGN
    assert f(b_i=MIS) == B.TP_ERR_ALIGN
    assert f(out_features=3080, t=3) == B.TP_ERR_INDIVISIBLE  # 3080 = 8 * 385
    assert f(out_features=3072 + 4) == B.TP_ERR_SHAPE        # not a multiple of 8
    assert f(t=4, out_features=4 * 12) == B.TP_ERR_SHAPE     # shard width 12
    assert f(rank=4) == B.TP_ERR_RANK
    assert f(rank=-1) == B.TP_ERR_RANK
    assert f(t=0) == B.TP_ERR_RANK
    assert f(tokens=-1) == B.TP_ERR_SHAPE
    assert f(in_features=0) == B.TP_ERR_SHAPE
    assert f(in_features=770) == B.TP_ERR_SHAPE
    assert f(dtype=B.TP_F32, out_dtype=B.TP_BF16) == B.TP_ERR_DTYPE
    assert f(dtype=7) == B.TP_ERR_DTYPE
    assert f(act=5) == B.TP_ERR_ARG
    assert f(pre_save=P2) == B.TP_ERR_ARG                   # save without activation
    assert f(pre_save=MIS, act=B.TP_ACT_GELU_TANH) == B.TP_ERR_ALIGN
    # an operand of 2^31 bytes or more
    assert f(tokens=1 << 20, in_features=1 << 10) == B.TP_ERR_SHAPE


def test_row_linear_rejects(Bfake):
    B = Bfake
    f = lambda **kw: B.tp_row_linear(**{**dict(
        X_i=P, W_i=P, Z_i=P, tokens=8, in_features=64, out_features=32, t=2, rank=1,
        dtype=B.TP_BF16, out_dtype=B.TP_F32, stream=0, check=False), **kw})
    assert f(Z_i=None) == B.TP_ERR_NULL
    assert f(in_features=72, t=2) == B.TP_ERR_SHAPE          # 36-wide shard
    assert f(in_features=64, t=3) == B.TP_ERR_INDIVISIBLE
    assert f(rank=2) == B.TP_ERR_RANK
    assert f(out_features=36) == B.TP_ERR_SHAPE


def test_mlp_fwd_bwd_reject(Bfake):
    B = Bfake
    fwd = lambda **kw: B.tp_mlp_shard_fwd(**{**dict(
        X=P, W1_i=P, b1_i=None, W2_i=P, H_i=P, Y_i_save=None, Z_i=P, tokens=16, h=64,
        ffn=256, t=8, rank=0, dtype=B.TP_BF16, stream=0, check=False), **kw})
    assert fwd(H_i=None) == B.TP_ERR_NULL
    assert fwd(Y_i_save=MIS) == B.TP_ERR_ALIGN
    assert fwd(ffn=260) == B.TP_ERR_SHAPE
    assert fwd(ffn=264, t=5) == B.TP_ERR_INDIVISIBLE
    assert fwd(ffn=264, t=8) == B.TP_ERR_SHAPE               # shard width 33
    assert fwd(dtype=3) == B.TP_ERR_DTYPE
    bwd = lambda **kw: B.tp_mlp_shard_bwd(**{**dict(
        X=P, W1_i=P, W2_i=P, Y_i=P, H_i=P, dZ=P, dY_i=P, dW2_i=P, dW1_i=P, dX_i=P, db1_i=None,
        tokens=16, h=64, ffn=256, t=8, rank=7, dtype=B.TP_BF16, stream=0, check=False), **kw})
    assert bwd(dZ=None) == B.TP_ERR_NULL
    assert bwd(db1_i=MIS) == B.TP_ERR_ALIGN
    assert bwd(rank=8) == B.TP_ERR_RANK
    assert bwd(h=60) == B.TP_ERR_SHAPE


def test_mlp_layer_fwd_rejects(Bfake):
    B = Bfake
    f = lambda **kw: B.tp_mlp_layer_fwd(**{**dict(
        X=P, W1=P, b1=None, W2=P, H=P2, Y_save=None, Z=P2, tokens=16, h=64, ffn=256, t=8,
        dtype=B.TP_BF16, stream=0, check=False), **kw})
    assert f(X=None) == B.TP_ERR_NULL
    assert f(W2=None) == B.TP_ERR_NULL
    assert f(H=None) == B.TP_ERR_NULL
    assert f(Z=None) == B.TP_ERR_NULL
    assert f(b1=MIS) == B.TP_ERR_ALIGN
    assert f(Y_save=MIS) == B.TP_ERR_ALIGN
    assert f(W1=MIS) == B.TP_ERR_ALIGN
    assert f(t=0) == B.TP_ERR_RANK
    assert f(t=-2) == B.TP_ERR_RANK
    assert f(ffn=264, t=5) == B.TP_ERR_INDIVISIBLE
    assert f(ffn=264, t=8) == B.TP_ERR_SHAPE               # shard width 33
    assert f(ffn=260) == B.TP_ERR_SHAPE
    assert f(h=60) == B.TP_ERR_SHAPE
    assert f(tokens=-1) == B.TP_ERR_SHAPE
    assert f(dtype=3) == B.TP_ERR_DTYPE
    # one rank's block of 2^31 bytes or more
    assert f(tokens=1 << 20, h=1 << 10, ffn=8 * 64) == B.TP_ERR_SHAPE


def test_linear_bwd_rejects(Bfake):
    B = Bfake
    f = lambda **kw: B.tp_linear_bwd(**{**dict(
        X=P, W=P, dY=P, dX=P2, dW=P2, db=None, tokens=32, in_features=768, out_features=256,
        dtype=B.TP_BF16, stream=0, check=False), **kw})
    assert f(X=None) == B.TP_ERR_NULL
    assert f(dW=None) == B.TP_ERR_NULL
    assert f(db=MIS) == B.TP_ERR_ALIGN
    assert f(dY=MIS) == B.TP_ERR_ALIGN
    assert f(in_features=770) == B.TP_ERR_SHAPE
    assert f(out_features=0) == B.TP_ERR_SHAPE
    assert f(tokens=-1) == B.TP_ERR_SHAPE
    assert f(tokens=1 << 20, in_features=1 << 10) == B.TP_ERR_SHAPE   # dX over 2^31 bytes
    assert f(dtype=7) == B.TP_ERR_DTYPE


def test_shard_reduce_rejects(Bfake):
    B = Bfake
    f = lambda **kw: B.tp_shard_reduce(**{**dict(
        parts=P, out=P2, tokens=4, cols=16, t=8, op=B.TP_REDUCE_SUM, in_dtype=B.TP_F32,
        out_dtype=B.TP_F32, stream=0, check=False), **kw})
    assert f(op=3) == B.TP_ERR_ARG
    assert f(op=B.TP_REDUCE_CONCAT, out_dtype=B.TP_BF16) == B.TP_ERR_DTYPE
    assert f(op=B.TP_REDUCE_CONCAT_TOKENS, out_dtype=B.TP_BF16) == B.TP_ERR_DTYPE
    assert f(parts=None) == B.TP_ERR_NULL
    assert f(out=MIS) == B.TP_ERR_ALIGN
    assert f(t=0) == B.TP_ERR_RANK
    assert f(cols=12) == B.TP_ERR_SHAPE
    assert f(tokens=-3) == B.TP_ERR_SHAPE


def test_reduce_scatter_rejects(Bfake):
    B = Bfake
    f = lambda **kw: B.tp_shard_reduce_scatter(**{**dict(
        parts=P, out=P2, tokens=16, cols=16, t=8, rank=3, in_dtype=B.TP_F32,
        out_dtype=B.TP_BF16, stream=0, check=False), **kw})
    assert f(parts=None) == B.TP_ERR_NULL
    assert f(out=MIS) == B.TP_ERR_ALIGN
    assert f(rank=8) == B.TP_ERR_RANK
    assert f(rank=-1) == B.TP_ERR_RANK
    assert f(t=0) == B.TP_ERR_RANK
    assert f(tokens=12) == B.TP_ERR_INDIVISIBLE
    assert f(cols=12) == B.TP_ERR_SHAPE
    assert f(in_dtype=7) == B.TP_ERR_DTYPE


def test_layernorm_rejects(Bfake):
    B = Bfake
    f = lambda **kw: B.tp_layernorm(**{**dict(
        x=P, gamma=None, beta=None, y=P2, tokens=4, cols=16, eps=1e-5, in_dtype=B.TP_F32,
        out_dtype=B.TP_BF16, stream=0, check=False), **kw})
    assert f(x=None) == B.TP_ERR_NULL
    assert f(gamma=MIS) == B.TP_ERR_ALIGN
    assert f(cols=20) == B.TP_ERR_SHAPE
    assert f(tokens=-1) == B.TP_ERR_SHAPE
    assert f(eps=-1.0) == B.TP_ERR_ARG
    assert f(eps=float("nan")) == B.TP_ERR_ARG
    assert f(eps=float("inf")) == B.TP_ERR_ARG
    assert f(y=P) == B.TP_ERR_ARG          # in place needs equal types
    assert f(out_dtype=5) == B.TP_ERR_DTYPE


def test_reduce_scatter_layernorm_rejects(Bfake):
    B = Bfake
    f = lambda **kw: B.tp_shard_reduce_scatter_layernorm(**{**dict(
        parts=P, gamma=None, beta=None, y=P2, tokens=16, cols=16, t=8, rank=3, eps=1e-5,
        in_dtype=B.TP_F32, out_dtype=B.TP_BF16, stream=0, check=False), **kw})
    assert f(parts=None) == B.TP_ERR_NULL
    assert f(y=None) == B.TP_ERR_NULL
    assert f(beta=MIS) == B.TP_ERR_ALIGN
    assert f(rank=8) == B.TP_ERR_RANK
    assert f(t=0) == B.TP_ERR_RANK
    assert f(tokens=12) == B.TP_ERR_INDIVISIBLE
    assert f(cols=12) == B.TP_ERR_SHAPE
    assert f(tokens=-8) == B.TP_ERR_SHAPE
    assert f(eps=float("nan")) == B.TP_ERR_ARG
    assert f(eps=-1.0) == B.TP_ERR_ARG
    assert f(out_dtype=5) == B.TP_ERR_DTYPE


def test_binding_checks_tensor_arguments(Bfake):
    B = Bfake
    # The binding refuses tensors the library would misread, before the call:
    # wrong element size, too few elements, non-contiguous, not on the device.
    # The other arguments are plain (unchecked) addresses.
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    T, h, ffn, t = 32, 64, 256, 2
    n = ffn // t
    call = lambda **kw: B.tp_column_linear(**{**dict(
        X=P, W_i=P, b_i=None, Y_i=P, pre_save=None, tokens=T, in_features=h, out_features=ffn,
        t=t, rank=0, dtype=bf, out_dtype=bf, act=B.TP_ACT_NONE, stream=0), **kw})
    with pytest.raises(ValueError, match="X: element size"):
        call(X=torch.zeros(T, h, dtype=f32))
    with pytest.raises(ValueError, match="X: holds"):
        call(X=torch.zeros(T, h, dtype=bf), tokens=T + 1)
    with pytest.raises(ValueError, match="Y_i: holds"):
        call(Y_i=torch.zeros(T, n - 8, dtype=bf))
    with pytest.raises(ValueError, match="Y_i: element size"):
        call(Y_i=torch.zeros(T, n, dtype=bf), out_dtype=f32)
    with pytest.raises(ValueError, match="X: must be contiguous"):
        call(X=torch.zeros(h, T, dtype=bf).t())
    with pytest.raises(ValueError, match="X: must be a device tensor"):
        call(X=torch.zeros(T, h, dtype=bf))
    with pytest.raises(ValueError, match="Z_i: element size"):
        B.tp_mlp_shard_fwd(P, P, None, P, P, None, torch.zeros(T, h, dtype=bf), T, h, ffn, t, 0,
                           bf, stream=0)
    with pytest.raises(ValueError, match="out: holds"):
        B.tp_shard_reduce(P, torch.zeros(T, h), T, h, 2, B.TP_REDUCE_CONCAT, f32, f32, stream=0)
    # shapes the library rejects itself skip the size check and return its status
    assert (ffn + 8) % 5 != 0
    assert B.tp_column_linear(P, P, None, P, None, T, h, ffn + 8, 5, 0, bf, bf,
                              B.TP_ACT_NONE, stream=0, check=False) == B.TP_ERR_INDIVISIBLE


# Byte ranges for the overlap checks: Q + k is k bytes past Q (16-aligned).
Q = 0x1000000


def test_outputs_may_not_overlap_inputs_or_each_other(Bfake):
    B = Bfake
    OV = B.TP_ERR_OVERLAP
    T, h, ffn, t = 32, 64, 256, 2
    n = ffn // t
    bf = B.TP_BF16
    # disjoint regions: each argument 1 MiB apart
    r = [Q + i * (1 << 20) for i in range(16)]
    # column: Y_i over X; pre_save over Y_i; Y_i in the bias
    col = lambda **kw: B.tp_column_linear(**{**dict(
        X=r[0], W_i=r[1], b_i=r[2], Y_i=r[3], pre_save=r[4], tokens=T, in_features=h,
        out_features=ffn, t=t, rank=0, dtype=bf, out_dtype=bf, act=B.TP_ACT_GELU_TANH, stream=0,
        check=False), **kw})
    assert col(Y_i=r[0] + T * h * 2 - 16) == OV          # last 16 bytes of X
    assert col(pre_save=r[3] + 16) == OV
    assert col(b_i=r[3] + 32) == OV
    # row: Z_i over W_i
    row = lambda **kw: B.tp_row_linear(**{**dict(
        X_i=r[0], W_i=r[1], Z_i=r[2], tokens=T, in_features=ffn, out_features=h, t=t, rank=1,
        dtype=bf, out_dtype=B.TP_F32, stream=0, check=False), **kw})
    assert row(Z_i=r[1]) == OV
    # shard forward: Z_i over H_i; H_i over W2_i
    fwd = lambda **kw: B.tp_mlp_shard_fwd(**{**dict(
        X=r[0], W1_i=r[1], b1_i=r[2], W2_i=r[3], H_i=r[4], Y_i_save=r[5], Z_i=r[6], tokens=T,
        h=h, ffn=ffn, t=t, rank=0, dtype=bf, stream=0, check=False), **kw})
    assert fwd(Z_i=r[4] + 16) == OV
    assert fwd(H_i=r[3]) == OV
    assert fwd(Y_i_save=r[0]) == OV
    # layer forward: the stacked partials reach into the second rank's H
    lay = lambda **kw: B.tp_mlp_layer_fwd(**{**dict(
        X=r[0], W1=r[1], b1=r[2], W2=r[3], H=r[4], Y_save=r[5], Z=r[6], tokens=T, h=h, ffn=ffn,
        t=t, dtype=bf, stream=0, check=False), **kw})
    assert lay(Z=r[4] + T * n * 2) == OV                 # rank 1's block of H
    assert lay(H=r[3] + n * h * 2) == OV                 # rank 1's block of W2
    # shard backward: dX over dZ; dW1 over dW2; db1 over Y_i
    bwd = lambda **kw: B.tp_mlp_shard_bwd(**{**dict(
        X=r[0], W1_i=r[1], W2_i=r[2], Y_i=r[3], H_i=r[4], dZ=r[5], dY_i=r[6], dW2_i=r[7],
        dW1_i=r[8], dX_i=r[9], db1_i=r[10], tokens=T, h=h, ffn=ffn, t=t, rank=0, dtype=bf,
        stream=0, check=False), **kw})
    assert bwd(dX_i=r[5]) == OV
    assert bwd(dW1_i=r[7] + 64) == OV
    assert bwd(db1_i=r[3]) == OV
    assert bwd(dY_i=r[4]) == OV                          # dY_i in place of H_i
    # linear backward: dW over X
    lin = lambda **kw: B.tp_linear_bwd(**{**dict(
        X=r[0], W=r[1], dY=r[2], dX=r[3], dW=r[4], db=r[5], tokens=T, in_features=h,
        out_features=n, dtype=bf, stream=0, check=False), **kw})
    assert lin(dW=r[0]) == OV
    assert lin(db=r[3] + 16) == OV
    # shard reduce: CONCAT's output is t blocks long
    red = lambda **kw: B.tp_shard_reduce(**{**dict(
        parts=r[0], out=r[1], tokens=T, cols=h, t=t, op=B.TP_REDUCE_SUM, in_dtype=B.TP_F32,
        out_dtype=B.TP_F32, stream=0, check=False), **kw})
    assert red(out=r[0] + t * T * h * 4 - 16) == OV
    assert red(out=r[0] - T * h * 4 + 16) == OV          # SUM output ends inside parts
    assert red(op=B.TP_REDUCE_CONCAT, out=r[0] - t * T * h * 4 + 16) == OV
    rs = lambda **kw: B.tp_shard_reduce_scatter(**{**dict(
        parts=r[0], out=r[1], tokens=T, cols=h, t=t, rank=1, in_dtype=B.TP_F32,
        out_dtype=B.TP_F32, stream=0, check=False), **kw})
    assert rs(out=r[0] + 256) == OV
    # layer norm: a shifted output overlaps its input (exactly in place is allowed)
    ln = lambda **kw: B.tp_layernorm(**{**dict(
        x=r[0], gamma=r[1], beta=r[2], y=r[3], tokens=T, cols=h, eps=1e-5, in_dtype=B.TP_F32,
        out_dtype=B.TP_F32, stream=0, check=False), **kw})
    assert ln(y=r[0] + 16) == OV
    assert ln(y=r[1]) == OV
    # fused reduce-scatter + layer norm: the output over the partials or gamma
    rl = lambda **kw: B.tp_shard_reduce_scatter_layernorm(**{**dict(
        parts=r[0], gamma=r[1], beta=r[2], y=r[3], tokens=T, cols=h, t=t, rank=1, eps=1e-5,
        in_dtype=B.TP_F32, out_dtype=B.TP_F32, stream=0, check=False), **kw})
    assert rl(y=r[0] + t * T * h * 4 - 16) == OV
    assert rl(y=r[1]) == OV
