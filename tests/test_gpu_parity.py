"""GPU parity: every entry point of libtpmlp against the fp64 oracle on the
same seeded inputs, element by element: reduced sizes (several tiles plus
ragged tails) and the full workload sizes (the GPT-3 shard's forward and
backward, the full-layer emulation's summed output, the GPT-3 attention
shard).  Only the cases at the boundary's largest accepted operands, and two
large ragged-token backward shapes, are compared on sampled rows and columns
the oracle computes directly."""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity_utils import (assert_close, dev, gpu_shard_bwd, gpu_shard_fwd, max_ratio,
                          sample_indices, to_device, to_np64)
from tensor_transformer_layer_columnparallel_amd import configs, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from tensor_transformer_layer_columnparallel_amd import binding
    return binding


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _whole(got, ref, dtype, what):
    """Compares a whole output tensor with the oracle's and logs the two
    error measures the tolerance is stated in."""
    rf = assert_close(got, ref, dtype, what)
    _log(f"parity {what}: rel_fro {rf:.3e} max_ratio {max_ratio(got, ref):.3e} "
         f"({to_np64(ref).size} elements)")


def _unsharded(inputs, ranks):
    W1 = np.concatenate([to_np64(inputs["W1"][r]) for r in ranks], axis=1)
    W2 = np.concatenate([to_np64(inputs["W2"][r]) for r in ranks], axis=0)
    b = [inputs["b1"][r] for r in ranks]
    b1 = None if b[0] is None else np.concatenate([to_np64(x) for x in b])
    return W1, b1, W2


def _full_check(B, w, seed=0, backward=True):
    """Element-by-element fwd (+bwd) of every shard of w vs the oracle."""
    d_h = synth.make_inputs(w, seed=seed, with_dz=backward)
    d = to_device(d_h)
    for r in w.ranks:
        Y, H, Z = gpu_shard_fwd(B, w, d, r)
        if backward:
            g = gpu_shard_bwd(B, w, d, r, Y, H)
        torch.cuda.synchronize()
        rY, rH, rZ = oracle.mlp_shard_fwd(d_h["X"], d_h["W1"][r], d_h["b1"][r], d_h["W2"][r])
        assert_close(Y, rY, w.dtype, f"{w.name} r{r} Y")
        assert_close(H, rH, w.dtype, f"{w.name} r{r} H")
        assert_close(Z, rZ, w.dtype, f"{w.name} r{r} Z")
        if backward:
            rg = oracle.mlp_shard_bwd(d_h["X"], d_h["W1"][r], d_h["b1"][r], d_h["W2"][r],
                                      d_h["dZ"])
            for k in ("dY", "dW2", "dW1", "dX", "db1"):
                assert_close(g[k], rg[k], w.dtype, f"{w.name} r{r} {k}")


# ----------------------------------------------------------------- tiny fp32

def test_tiny_mlp_f32_both_shards_sum_to_unsharded(B):
    w = configs.TINY_F32
    _log(f"case {w.name}")
    d_h = synth.make_inputs(w)
    d = to_device(d_h)
    parts = torch.empty(w.t, w.T, w.h, dtype=torch.float32, device="cuda")
    dxp = torch.empty(w.t, w.T, w.h, dtype=torch.float32, device="cuda")
    for r in w.ranks:
        Y, H, Z = gpu_shard_fwd(B, w, d, r)
        parts[r].copy_(Z)
        dxp[r].copy_(gpu_shard_bwd(B, w, d, r, Y, H)["dX"])
    Zsum = torch.empty(w.T, w.h, dtype=torch.float32, device="cuda")
    dX = torch.empty_like(Zsum)
    B.tp_shard_reduce(parts, Zsum, w.T, w.h, w.t, B.TP_REDUCE_SUM, B.TP_F32, B.TP_F32)
    B.tp_shard_reduce(dxp, dX, w.T, w.h, w.t, B.TP_REDUCE_SUM, B.TP_F32, B.TP_F32)
    torch.cuda.synchronize()
    W1, b1, W2 = _unsharded(d_h, w.ranks)
    _, _, rZ = oracle.mlp_shard_fwd(d_h["X"], W1, b1, W2)
    rg = oracle.mlp_shard_bwd(d_h["X"], W1, b1, W2, d_h["dZ"])
    assert_close(Zsum, rZ, "f32", "tiny Z = Z_0 + Z_1")
    assert_close(dX, rg["dX"], "f32", "tiny dX = dX_0 + dX_1")


def test_tiny_mlp_f32_each_shard_fwd_bwd(B):
    _full_check(B, configs.TINY_F32)


# ------------------------------------------------ column-parallel linear only

def test_column_linear_768_rank0(B):
    w = configs.COLUMN_768
    _log(f"case {w.name}")
    d_h = synth.make_inputs(w)
    X, W, b = dev(d_h["X"]), dev(d_h["W1"][0]), dev(d_h["b1"][0])
    Y = torch.empty(w.T, w.n, dtype=torch.bfloat16, device="cuda")
    B.tp_column_linear(X, W, b, Y, None, w.T, w.h, w.ffn, w.t, 0, B.TP_BF16, B.TP_BF16, B.TP_ACT_NONE)
    torch.cuda.synchronize()
    ref = oracle.column_linear(d_h["X"], d_h["W1"][0], d_h["b1"][0])
    assert_close(Y, ref, "bf16", "column 768 Y_0")


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_column_linear_ragged(B, act, out_dt):
    # T = 300 (2 full 128-row tiles + 44), n = 200 (one full tile + 72)
    w = configs.scaled(configs.GPT3_SHARD, "col_ragged", T=300, h=264, ffn=800, t=4)
    _log(f"case column ragged act={act} out={out_dt}")
    d_h = synth.make_inputs(w, with_dz=False)
    X, W, b = dev(d_h["X"]), dev(d_h["W1"][0]), dev(d_h["b1"][0])
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    Y = torch.empty(w.T, w.n, dtype=odt, device="cuda")
    B.tp_column_linear(X, W, b, Y, None, w.T, w.h, w.ffn, w.t, 0, B.TP_BF16, odt, act)
    torch.cuda.synchronize()
    ref = oracle.column_linear(d_h["X"], d_h["W1"][0], d_h["b1"][0], gelu=bool(act))
    assert_close(Y, ref, "bf16", f"column ragged act={act}")


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_column_linear_tile_kernel_epilogues(B, act, out_dt):
    # Shapes the tile kernel takes (M >= 256, N >= 192, K % 32 == 0) with a
    # ragged M and N tail: the bias and bias + GeLU epilogues into bf16 and
    # into fp32 (the fp32 plain/bias results are staged through LDS).
    w = configs.scaled(configs.GPT3_SHARD, "col_tile", T=300, h=512, ffn=1600, t=4)
    _log(f"case column tile act={act} out={out_dt}")
    d_h = synth.make_inputs(w, with_dz=False)
    X, W, b = dev(d_h["X"]), dev(d_h["W1"][0]), dev(d_h["b1"][0])
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    Y = torch.empty(w.T, w.n, dtype=odt, device="cuda")
    B.tp_column_linear(X, W, b, Y, None, w.T, w.h, w.ffn, w.t, 0, B.TP_BF16, odt, act)
    torch.cuda.synchronize()
    ref = oracle.column_linear(d_h["X"], d_h["W1"][0], d_h["b1"][0], gelu=bool(act))
    assert_close(Y, ref, "bf16", f"column tile act={act} out={out_dt}")


def test_small_tile_instance_every_epilogue(B):
    # Products with fewer than 128 tiles of 256 x 192 run on 128 x 96 tiles.
    # 770 x 544 -> 416 (12 large tiles, 7 x 5 small ones, ragged in M and N)
    # through every epilogue those instances serve: bias + GeLU with the
    # pre-activation saved, bias with bf16 output and plain bf16 row products
    # (at most one small tile per CU and K >= 256: the K-split workgroups,
    # K = 320 + 224), bias with fp32 (LDS-staged) output and plain fp32 row
    # products (four-wave workgroups), and the NT product of a linear
    # backward's dX (770 x 416 -> 544, K a multiple of 32 and not of 64);
    # element-wise vs the oracle.
    T, k, n = 770, 544, 416
    bf, f32 = torch.bfloat16, torch.float32
    g = torch.Generator().manual_seed(71)
    X = (torch.randn(T, k, generator=g)).to(bf)
    W = (0.02 * torch.randn(k, n, generator=g)).to(bf)
    b = (0.02 * torch.randn(n, generator=g)).to(bf)
    Xd, Wd, bd = dev(X), dev(W), dev(b)
    H = torch.empty(T, n, dtype=bf, device="cuda")
    Y = torch.empty(T, n, dtype=bf, device="cuda")
    B.tp_column_linear(Xd, Wd, bd, H, Y, T, k, n, 1, 0, bf, bf, B.TP_ACT_GELU_TANH)
    Yb = torch.empty(T, n, dtype=bf, device="cuda")
    B.tp_column_linear(Xd, Wd, bd, Yb, None, T, k, n, 1, 0, bf, bf, B.TP_ACT_NONE)
    Yf = torch.empty(T, n, dtype=f32, device="cuda")
    B.tp_column_linear(Xd, Wd, bd, Yf, None, T, k, n, 1, 0, bf, f32, B.TP_ACT_NONE)
    Zf = torch.empty(T, n, dtype=f32, device="cuda")
    B.tp_row_linear(Xd, Wd, Zf, T, k, n, 1, 0, bf, f32)
    Zb = torch.empty(T, n, dtype=bf, device="cuda")
    B.tp_row_linear(Xd, Wd, Zb, T, k, n, 1, 0, bf, bf)
    dY = (torch.randn(T, n, generator=g)).to(bf)
    dX = torch.empty(T, k, dtype=f32, device="cuda")
    dW = torch.empty(k, n, dtype=f32, device="cuda")
    B.tp_linear_bwd(Xd, Wd, dev(dY), dX, dW, None, T, k, n, bf)
    torch.cuda.synchronize()
    rY = oracle.column_linear(X, W, b)
    _whole(Y, rY, "bf16", "small tiles: saved pre-activation")
    _whole(H, oracle.column_linear(X, W, b, gelu=True), "bf16", "small tiles: GeLU")
    _whole(Yb, rY, "bf16", "small tiles: bias, bf16 out")
    _whole(Yf, rY, "bf16", "small tiles: bias, fp32 out")
    rZ = oracle.row_linear(X, W)
    _whole(Zf, rZ, "bf16", "small tiles: plain fp32")
    _whole(Zb, rZ, "bf16", "small tiles: plain bf16")
    ref = oracle.linear_bwd(X, W, dY, with_db=False)
    _whole(dX, ref["dX"], "bf16", "small tiles: NT dX")
    _whole(dW, ref["dW"], "bf16", "linear bwd dW (TN)")


@pytest.mark.parametrize("T,k,n", [(4000, 288, 1000), (1000, 288, 488), (520, 2080, 200)],
                         ids=["four-wave", "split-288", "split-2080"])
def test_small_tile_register_epilogues(B, T, k, n):
    # The register-path epilogues (bias + GeLU with the pre-activation saved,
    # bias, plain; bf16 out) on both 128 x 96 instances: 4000 x 288 -> 1000
    # has 32 x 11 small tiles, more than the CUs, so it takes the four-wave
    # workgroups; the other two have at most one small tile per CU and take
    # the two K-split pipelines, with halves of 192 + 96 and 1088 + 992 k
    # (the second pipeline's last loads past K read zeros).  Ragged in M and
    # N; element-wise vs the oracle.
    _log(f"case small tiles register epilogues {T}x{k}x{n}")
    bf = torch.bfloat16
    g = torch.Generator().manual_seed(73)
    X = torch.randn(T, k, generator=g).to(bf)
    W = (0.02 * torch.randn(k, n, generator=g)).to(bf)
    b = (0.02 * torch.randn(n, generator=g)).to(bf)
    Xd, Wd, bd = dev(X), dev(W), dev(b)
    H = torch.empty(T, n, dtype=bf, device="cuda")
    Y = torch.empty(T, n, dtype=bf, device="cuda")
    B.tp_column_linear(Xd, Wd, bd, H, Y, T, k, n, 1, 0, bf, bf, B.TP_ACT_GELU_TANH)
    Yb = torch.empty(T, n, dtype=bf, device="cuda")
    B.tp_column_linear(Xd, Wd, bd, Yb, None, T, k, n, 1, 0, bf, bf, B.TP_ACT_NONE)
    Zb = torch.empty(T, n, dtype=bf, device="cuda")
    B.tp_row_linear(Xd, Wd, Zb, T, k, n, 1, 0, bf, bf)
    torch.cuda.synchronize()
    rY = oracle.column_linear(X, W, b)
    _whole(Y, rY, "bf16", "small tiles: saved pre-activation")
    _whole(H, oracle.column_linear(X, W, b, gelu=True), "bf16", "small tiles: GeLU")
    _whole(Yb, rY, "bf16", "small tiles: bias, bf16 out")
    _whole(Zb, oracle.row_linear(X, W), "bf16", "small tiles: plain bf16")


@pytest.mark.parametrize("n", [200, 208, 216, 224, 232, 240],
                         ids=lambda n: f"n{n}-tail{n % 48}")
def test_bf16_epilogue_every_column_tail(B, n):
    # The bf16 epilogues pair neighbouring 16-column fragments through a lane
    # exchange and store (load, for the saved pre-activation) eight columns
    # per lane.  A wave covers 48 columns, so N can end 8, 16, 24, 32, 40 or
    # 48 columns into a wave's range: n % 48 runs through all six.  Each n on
    # the K-split workgroups (300 rows), the four-wave 128 x 96 instance
    # (12000 rows) and the 256 x 192 tiles (16400 rows): bias + GeLU with the
    # pre-activation saved; and the shard forward + backward at 300 tokens,
    # whose GeLU' product (dY with the bias gradient) reads the saved
    # pre-activation that way; element-wise vs the oracle.
    bf = torch.bfloat16
    k = 256
    g = torch.Generator().manual_seed(79)
    W = (0.02 * torch.randn(k, n, generator=g)).to(bf)
    b = (0.02 * torch.randn(n, generator=g)).to(bf)
    Wd, bd = dev(W), dev(b)
    for T in (300, 12000, 16400):
        _log(f"case bf16 epilogue tail n={n} T={T}")
        X = torch.randn(T, k, generator=g).to(bf)
        H = torch.empty(T, n, dtype=bf, device="cuda")
        Y = torch.empty(T, n, dtype=bf, device="cuda")
        B.tp_column_linear(dev(X), Wd, bd, H, Y, T, k, n, 1, 0, bf, bf, B.TP_ACT_GELU_TANH)
        torch.cuda.synchronize()
        assert_close(Y, oracle.column_linear(X, W, b), "bf16", f"tail n={n} T={T} Y")
        assert_close(H, oracle.column_linear(X, W, b, gelu=True), "bf16", f"tail n={n} T={T} H")
    w = configs.Workload(f"tail{n}", T=300, h=k, ffn=n, t=1, dtype="bf16", ranks=(0,), bias=True)
    _full_check(B, w, seed=83)


def test_row_linear_ragged_partials_sum(B):
    # row-parallel partials of t = 4 ranks, summed on the device
    T, n_full, hout, t = 77, 512, 136, 4
    _log("case row ragged")
    g = torch.Generator().manual_seed(11)
    Xf = torch.randn(T, n_full, generator=g).bfloat16()
    Wf = (0.02 * torch.randn(n_full, hout, generator=g)).bfloat16()
    k = n_full // t
    parts = torch.empty(t, T, hout, dtype=torch.float32, device="cuda")
    for r in range(t):
        B.tp_row_linear(dev(Xf[:, r * k:(r + 1) * k]), dev(Wf[r * k:(r + 1) * k]), parts[r], T,
                        n_full, hout, t, r, B.TP_BF16, B.TP_F32)
    Z = torch.empty(T, hout, dtype=torch.float32, device="cuda")
    B.tp_shard_reduce(parts, Z, T, hout, t, B.TP_REDUCE_SUM, B.TP_F32, B.TP_F32)
    torch.cuda.synchronize()
    assert_close(Z, oracle.row_linear(Xf, Wf), "bf16", "row partial sum")


# ------------------------------------- attention block: QKV and output proj

def _attn_qkv_gpu(B, aw, d, s, r):
    T, h = aw.T, aw.h
    Y = torch.empty(T, aw.qkv_width, dtype=torch.bfloat16, device="cuda")
    st = B.tp_column_linear(dev(d["X"]), dev(s["Wqkv"]), dev(s["bqkv"]), Y, None, T, h, 3 * h,
                            aw.t, r, B.TP_BF16, B.TP_BF16, B.TP_ACT_NONE)
    assert st == 0
    return Y


def test_attention_qkv_head_shards_small(B):
    """Every rank's QKV projection (heads split on boundaries) vs the oracle."""
    aw = configs.ATTN_SMALL
    d = synth.make_attn_inputs(aw)
    for r in aw.ranks:
        _log(f"case {aw.name} qkv rank {r}")
        s = synth.attn_shard(aw, d, r)
        Y = _attn_qkv_gpu(B, aw, d, s, r)
        torch.cuda.synchronize()
        assert_close(Y, oracle.column_linear(d["X"], s["Wqkv"], s["bqkv"]), "bf16",
                     f"{aw.name} QKV r{r}")


def test_attention_output_projection_small(B):
    """Row-parallel output projection of every rank, summed on the device,
    vs the oracle's unsharded O W_o."""
    aw = configs.ATTN_SMALL
    d = synth.make_attn_inputs(aw)
    T, h = aw.T, aw.h
    parts = torch.empty(aw.t, T, h, dtype=torch.float32, device="cuda")
    for r in range(aw.t):
        _log(f"case {aw.name} out-proj rank {r}")
        s = synth.attn_shard(aw, d, r)
        assert B.tp_row_linear(dev(s["O"]), dev(s["Wo"]), parts[r], T, h, h, aw.t, r, B.TP_BF16,
                               B.TP_F32) == 0
    Z = torch.empty(T, h, dtype=torch.float32, device="cuda")
    B.tp_shard_reduce(parts, Z, T, h, aw.t, B.TP_REDUCE_SUM, B.TP_F32, B.TP_F32)
    torch.cuda.synchronize()
    assert_close(Z, oracle.row_linear(d["O"], d["Wo"]), "bf16", f"{aw.name} O W_o")


def test_attention_gpt3_shard_whole_tensors(B):
    """GPT-3-shaped attention shard (96 heads, t = 8, rank 3) at full size,
    in the bench's launch configuration, on every element of the QKV output
    and of the output projection's fp32 partial."""
    aw = configs.ATTN_GPT3
    r = aw.ranks[0]
    _log(f"case {aw.name} rank {r}")
    d = synth.make_attn_inputs(aw)
    s = synth.attn_shard(aw, d, r)
    Y = _attn_qkv_gpu(B, aw, d, s, r)
    Z = torch.empty(aw.T, aw.h, dtype=torch.float32, device="cuda")
    assert B.tp_row_linear(dev(s["O"]), dev(s["Wo"]), Z, aw.T, aw.h, aw.h, aw.t, r, B.TP_BF16,
                           B.TP_F32) == 0
    torch.cuda.synchronize()
    _whole(Y, oracle.column_linear(d["X"], s["Wqkv"], s["bqkv"]), "bf16", f"{aw.name} QKV")
    _whole(Z, oracle.row_linear(s["O"], s["Wo"]), "bf16", f"{aw.name} out-proj")


LINEAR_BWD = [
    # (T, in, out): the weight gradient's path on the device
    (300, 264, 200),   # T % 32 != 0: the tile kernel's TN layout (both operands transposed in LDS)
    (288, 512, 384),   # out <= in: dY^T, product stored transposed
    (288, 384, 768),   # out > in, dX in two products over K (partials in dW), dW via TN
    (512, 192, 4096),  # dX too few tiles: eight products over K, summed in order
    (300, 200, 2048),  # four products over K, ragged M and N tails
    (256, 192, 192),   # below a tile in M: the general kernel
    (64, 136, 520),
    (33, 96, 64),
]


@pytest.mark.parametrize("shape", LINEAR_BWD, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_linear_bwd_matches_oracle(B, shape, dt):
    T, k, n = shape
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    _log(f"case linear bwd {shape} {dt}")
    X = synth.draw((T, k), 1.0, 3, synth.TAG_X, 0, tdt)
    W = synth.draw((k, n), 0.02, 3, synth.TAG_W1, 0, tdt)
    dY = synth.draw((T, n), 1.0, 3, synth.TAG_DZ, 0, tdt)
    dX = torch.full((T, k), float("nan"), device="cuda")
    dW = torch.full((k, n), float("nan"), device="cuda")
    db = torch.full((n,), float("nan"), device="cuda")
    B.tp_linear_bwd(dev(X), dev(W), dev(dY), dX, dW, db, T, k, n, tdt)
    torch.cuda.synchronize()
    g = oracle.linear_bwd(X, W, dY)
    for name, got in (("dX", dX), ("dW", dW), ("db", db)):
        assert_close(got, g[name], dt, f"linear bwd {shape} {dt} {name}")


def test_linear_bwd_split_over_k_is_deterministic(B):
    # the dX products over K ranges and their ordered sum give the same bytes
    # on every run
    T, k, n = 512, 192, 4096
    X = dev(synth.draw((T, k), 1.0, 4, synth.TAG_X, 0, torch.bfloat16))
    W = dev(synth.draw((k, n), 0.02, 4, synth.TAG_W1, 0, torch.bfloat16))
    dY = dev(synth.draw((T, n), 1.0, 4, synth.TAG_DZ, 0, torch.bfloat16))
    outs = []
    for _ in range(3):
        dX, dW, db = (torch.empty(T, k, device="cuda"), torch.empty(k, n, device="cuda"),
                      torch.empty(n, device="cuda"))
        B.tp_linear_bwd(X, W, dY, dX, dW, db, T, k, n, torch.bfloat16)
        outs.append((dX, dW, db))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert all(torch.equal(a, b) for a, b in zip(o, outs[0]))


@pytest.mark.parametrize("shape", [(2047, 4096, 3072), (1000, 1536, 12288)],
                         ids=lambda s: "x".join(map(str, s)))
def test_linear_bwd_ragged_tokens_large_sampled(B, shape):
    """Token counts that are not whole 32-deep slabs put the weight gradient
    on the TN products (both operands read transposed, slab pairs with a
    ragged last pair): 2047 tokens over 16 x 16 tiles, and 1000 tokens after
    dX split into eight products over K.  Sampled rows of dX and columns of
    dW and db against the oracle."""
    T, k, n = shape
    _log(f"case linear bwd ragged tokens {shape}")
    X = synth.draw((T, k), 1.0, 6, synth.TAG_X, 0, torch.bfloat16)
    W = synth.draw((k, n), 0.02, 6, synth.TAG_W1, 0, torch.bfloat16)
    dY = synth.draw((T, n), 1.0, 6, synth.TAG_DZ, 0, torch.bfloat16)
    dX = torch.full((T, k), float("nan"), device="cuda")
    dW = torch.full((k, n), float("nan"), device="cuda")
    db = torch.full((n,), float("nan"), device="cuda")
    B.tp_linear_bwd(dev(X), dev(W), dev(dY), dX, dW, db, T, k, n, B.TP_BF16)
    torch.cuda.synchronize()
    assert not torch.isnan(dW).any() and not torch.isnan(dX).any()
    rows = sample_indices(T, 4, seed=21)
    cols = sample_indices(n, 6, seed=22)
    _log(f"case linear bwd ragged tokens {shape} rows {rows.tolist()} cols {cols.tolist()}")
    g = oracle.linear_bwd(X[rows], W, dY[rows], with_db=False)
    assert_close(dX[rows], g["dX"], "bf16", f"{shape} dX rows")
    g = oracle.linear_bwd(X, W[:, cols], dY[:, cols])
    assert_close(dW[:, cols], g["dW"], "bf16", f"{shape} dW cols")
    assert_close(db[cols], g["db"], "bf16", f"{shape} db cols")


def test_linear_bwd_empty_tokens(B):
    k, n = 64, 128
    ph = torch.empty(8, dtype=torch.bfloat16, device="cuda")   # [0, *] arrays have no storage
    phf = torch.empty(8, dtype=torch.float32, device="cuda")
    W = torch.randn(k, n, device="cuda").bfloat16()
    dW = torch.full((k, n), 7.0, device="cuda")
    db = torch.full((n,), 7.0, device="cuda")
    B.tp_linear_bwd(ph, W, ph, phf, dW, db, 0, k, n, B.TP_BF16)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW) == 0 and torch.count_nonzero(db) == 0


def test_attention_gpt3_backward_whole_tensors(B):
    """Backward of rank 3's GPT-3-shaped attention projections (QKV on head
    boundaries: out <= in, dY^T path; output projection: out > in, dX over
    four K ranges and dW on the TN product) on every element of dX, dW and
    db."""
    aw = configs.ATTN_GPT3
    r = aw.ranks[0]
    T, h, w = aw.T, aw.h, aw.w
    _log(f"case {aw.name} backward rank {r}")
    d = synth.make_attn_inputs(aw)
    s = synth.attn_shard(aw, d, r)
    gr = synth.make_attn_grads(aw)
    dQ = gr["dQKV"][:, synth.qkv_columns(aw, r)].contiguous()
    n = 3 * w
    dX = torch.empty(T, h, device="cuda"); dW = torch.empty(h, n, device="cuda")
    db = torch.empty(n, device="cuda")
    B.tp_linear_bwd(dev(d["X"]), dev(s["Wqkv"]), dev(dQ), dX, dW, db, T, h, n, B.TP_BF16)
    dO = torch.empty(T, w, device="cuda"); dWo = torch.empty(w, h, device="cuda")
    B.tp_linear_bwd(dev(s["O"]), dev(s["Wo"]), dev(gr["dZ"]), dO, dWo, None, T, w, h, B.TP_BF16)
    torch.cuda.synchronize()
    g = oracle.linear_bwd(d["X"], s["Wqkv"], dQ)
    _whole(dX, g["dX"], "bf16", "QKV dX")
    _whole(dW, g["dW"], "bf16", "QKV dW")
    _whole(db, g["db"], "bf16", "QKV db")
    g = oracle.linear_bwd(s["O"], s["Wo"], gr["dZ"], with_db=False)
    _whole(dO, g["dX"], "bf16", "out-proj dO")
    _whole(dWo, g["dW"], "bf16", "out-proj dW")


def test_row_partials_in_bf16_then_summed_in_fp32(B):
    # Low-precision exchange (page "Tensor Parallelism原理与实践" §4.1 keeps fp32
    # for the reduction itself): each rank's row-parallel partial stored as
    # bf16, the t partials summed in fp32 in rank order.
    T, n_full, hout, t = 300, 1024, 392, 4
    _log("case row partials bf16 -> fp32 sum")
    g = torch.Generator().manual_seed(12)
    Xf = torch.randn(T, n_full, generator=g).bfloat16()
    Wf = (0.02 * torch.randn(n_full, hout, generator=g)).bfloat16()
    k = n_full // t
    parts = torch.empty(t, T, hout, dtype=torch.bfloat16, device="cuda")
    for r in range(t):
        B.tp_row_linear(dev(Xf[:, r * k:(r + 1) * k]), dev(Wf[r * k:(r + 1) * k]), parts[r], T,
                        n_full, hout, t, r, B.TP_BF16, B.TP_BF16)
    Z = torch.empty(T, hout, dtype=torch.float32, device="cuda")
    B.tp_shard_reduce(parts, Z, T, hout, t, B.TP_REDUCE_SUM, B.TP_BF16, B.TP_F32)
    torch.cuda.synchronize()
    assert_close(Z, oracle.row_linear(Xf, Wf), "bf16", "bf16 partials summed")


# ------------------------------------------------- reduced MLP, full compare

REDUCED = [
    # (T, h, ffn, t): several tiles in every dimension plus ragged tails
    (300, 384, 1024, 4),     # T ragged
    (33, 200, 800, 4),       # T < tile, n = h = 200 ragged
    (1, 64, 256, 2),         # a single token
    (130, 136, 1088, 8),     # n = 136, h = 136
    (256, 512, 2048, 8),     # exact tiles
    (270, 328, 2624, 8),     # K = 328 not a multiple of 64; ragged K = 270 in x^T dy
    (520, 768, 4096, 8),     # two 256-row tiles + 8 rows, 512-wide shard
    (64, 4096, 8192, 2),     # 4096 x 4096 weight gradients: 256-wide tiles
    (288, 256, 1024, 1),     # n = 4h: dW1 from X^T (dY^T would not fit in dX's memory)
    (288, 544, 2304, 8),     # K = 544 and K = T = 288: an odd number of 32-deep slabs
                             # in the tile kernel (half of the last 64-deep unit past K),
                             # in the forward and in the transposed weight gradients
    (8448, 32, 192, 1),      # more than 256 h tokens: the dY product's 33 row-block
                             # partials would not fit in dW2's 32 rows, so db1 sums the
                             # stored dY instead
]


@pytest.mark.parametrize("shape", REDUCED, ids=lambda s: "x".join(map(str, s)))
def test_reduced_mlp_fwd_bwd_bf16(B, shape):
    T, h, ffn, t = shape
    w = configs.scaled(configs.GPT3_SHARD, "reduced_bf16", T=T, h=h, ffn=ffn, t=t,
                       ranks=(0, t - 1))
    _log(f"case reduced bf16 {shape}")
    _full_check(B, w)


def _random_shapes(count, seed):
    """Seeded (T, h, ffn, t) with feature widths that are multiples of 8:
    mixes tile-kernel and general-kernel products, ragged tails in every
    dimension, K % 32 != 0, token counts that take the transposed weight
    gradients (T % 32 == 0) and shard widths on both sides of 2h."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        t = int(rng.choice([1, 2, 3, 4, 8]))
        # mostly K % 32 == 0 (the tile kernel's K-contiguous operands)
        h = int(32 * rng.integers(2, 26) if rng.random() < 0.75 else 8 * rng.integers(4, 100))
        u = rng.random()
        n = int(32 * rng.integers(6, 28) if u < 0.5 else
                8 * rng.integers(24, 110) if u < 0.85 else 8 * rng.integers(4, 24))
        u = rng.random()
        T = int(rng.integers(1, 256) if u < 0.25 else
                rng.integers(256, 760) if u < 0.6 else 32 * rng.integers(8, 24))
        out.append((T, h, n * t, t))
    return out


@pytest.mark.parametrize("shape", _random_shapes(32, seed=11), ids=lambda s: "x".join(map(str, s)))
def test_random_shapes_fwd_bwd_bf16(B, shape):
    T, h, ffn, t = shape
    w = configs.scaled(configs.GPT3_SHARD, "random_bf16", T=T, h=h, ffn=ffn, t=t, ranks=(t - 1,))
    _log(f"case random bf16 {shape}")
    _full_check(B, w, seed=T + h)


@pytest.mark.parametrize("shape", _random_shapes(6, seed=12), ids=lambda s: "x".join(map(str, s)))
def test_random_shapes_fwd_bwd_f32(B, shape):
    T, h, ffn, t = shape
    w = configs.scaled(configs.TINY_F32, "random_f32", T=T, h=h, ffn=ffn, t=t, ranks=(0,),
                       bias_zero=False)
    _log(f"case random f32 {shape}")
    _full_check(B, w, seed=T + h)


def test_reduced_mlp_fwd_bwd_f32(B):
    w = configs.scaled(configs.TINY_F32, "reduced_f32", T=150, h=136, ffn=544, t=2)
    _log("case reduced f32")
    _full_check(B, w)


def test_empty_tokens(B):
    _log("case empty tokens")
    h, ffn, t = 64, 256, 2
    n = ffn // t
    # Empty tensors have no storage; pass an aligned placeholder wherever the
    # ABI requires a pointer to a [0, *] array.
    ph = torch.empty(8, dtype=torch.bfloat16, device="cuda")
    phf = torch.empty(8, dtype=torch.float32, device="cuda")
    W1 = torch.randn(h, n, device="cuda").bfloat16()
    W2 = torch.randn(n, h, device="cuda").bfloat16()
    B.tp_mlp_shard_fwd(ph, W1, None, W2, ph, None, phf, 0, h, ffn, t, 0, B.TP_BF16)
    dW2 = torch.full((n, h), 7.0, device="cuda")
    dW1 = torch.full((h, n), 7.0, device="cuda")
    db1 = torch.full((n,), 7.0, device="cuda")
    B.tp_mlp_shard_bwd(ph, W1, W2, ph, ph, ph, ph, dW2, dW1, phf, db1, 0, h, ffn, t, 0,
                       B.TP_BF16)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW2) == 0 and torch.count_nonzero(dW1) == 0
    assert torch.count_nonzero(db1) == 0


def test_overlapping_outputs_are_rejected_before_any_launch(B):
    """Real device buffers whose byte ranges overlap: the entry points return
    TP_ERR_OVERLAP and leave the memory as it was."""
    _log("case overlapping outputs")
    T, h, ffn, t = 64, 128, 512, 4
    n = ffn // t
    bf, f32 = torch.bfloat16, torch.float32
    g = torch.Generator(device="cuda").manual_seed(5)
    X = torch.randn(T, h, device="cuda", generator=g).to(bf)
    W1 = torch.randn(h, n, device="cuda", generator=g).to(bf)
    W2 = torch.randn(n, h, device="cuda", generator=g).to(bf)
    buf = torch.randn(T * n + T * h + 64, device="cuda", generator=g)   # fp32 words
    snap = buf.clone()
    H = buf.view(bf)[: T * n].view(T, n)          # bytes [0, 2 T n)
    Z_in_H = buf[T * n // 4:][: T * h]            # starts at byte T n, inside H
    Z_after_H = buf[T * n // 2:][: T * h]         # starts at byte 2 T n, just past H
    # Z_i starting inside H_i
    assert B.tp_mlp_shard_fwd(X, W1, None, W2, H, None, Z_in_H, T, h, ffn, t, 0, bf,
                              check=False) == B.TP_ERR_OVERLAP
    # the row layer writing its partial over its own input
    assert B.tp_row_linear(H, W2, Z_in_H, T, ffn, h, t, 0, bf, f32,
                           check=False) == B.TP_ERR_OVERLAP
    # the shard sum writing into its own partials
    parts = buf[: 2 * T * h].view(2, T, h)
    assert B.tp_shard_reduce(parts, parts[1], T, h, 2, B.TP_REDUCE_SUM, f32, f32,
                             check=False) == B.TP_ERR_OVERLAP
    # the backward's dX_i starting inside dZ
    bb = torch.randn(2 * T * h, device="cuda", generator=g)
    bb_snap = bb.clone()
    dZ = bb.view(bf)[: T * h].view(T, h)          # bytes [0, 2 T h)
    dX_in_dZ = bb[T * h // 4:][: T * h].view(T, h)  # starts at byte T h
    dY = torch.empty(T, n, dtype=bf, device="cuda")
    dW2, dW1 = torch.empty(n, h, device="cuda"), torch.empty(h, n, device="cuda")
    assert B.tp_mlp_shard_bwd(X, W1, W2, H, H, dZ, dY, dW2, dW1, dX_in_dZ, None, T, h, ffn, t,
                              0, bf, check=False) == B.TP_ERR_OVERLAP
    torch.cuda.synchronize()
    assert torch.equal(buf, snap) and torch.equal(bb, bb_snap), "a rejected call wrote"
    # adjacent but disjoint ranges are accepted (and computed correctly)
    assert B.tp_mlp_shard_fwd(X, W1, None, W2, H, None, Z_after_H, T, h, ffn, t, 0, bf,
                              check=False) == 0
    torch.cuda.synchronize()
    _, rH, rZ = oracle.mlp_shard_fwd(X.cpu(), W1.cpu(), None, W2.cpu())
    assert_close(H, rH, "bf16", "adjacent H")
    assert_close(Z_after_H.view(T, h), rZ, "bf16", "adjacent Z")


# ----------------------------------------------------- invariants on device

def test_column_shards_concat_bitexact_to_unsharded(B):
    # Rank-ordered concatenation of the column shards equals the unsharded
    # product bit for bit: each output element sums over K in the same order.
    T, h, ffn, t = 200, 256, 1024, 4
    _log("case concat invariant")
    g = torch.Generator().manual_seed(5)
    X = dev(torch.randn(T, h, generator=g).bfloat16())
    W = (0.02 * torch.randn(h, ffn, generator=g)).bfloat16()
    b = (0.02 * torch.randn(ffn, generator=g)).bfloat16()
    full = torch.empty(T, ffn, dtype=torch.bfloat16, device="cuda")
    B.tp_column_linear(X, dev(W), dev(b), full, None, T, h, ffn, 1, 0, B.TP_BF16, B.TP_BF16,
                       B.TP_ACT_GELU_TANH)
    n = ffn // t
    parts = torch.empty(t, T, n, dtype=torch.bfloat16, device="cuda")
    for r in range(t):
        B.tp_column_linear(X, dev(W[:, r * n:(r + 1) * n]), dev(b[r * n:(r + 1) * n]), parts[r],
                           None, T, h, ffn, t, r, B.TP_BF16, B.TP_BF16, B.TP_ACT_GELU_TANH)
    cat = torch.empty(T, ffn, dtype=torch.bfloat16, device="cuda")
    B.tp_shard_reduce(parts, cat, T, n, t, B.TP_REDUCE_CONCAT, B.TP_BF16, B.TP_BF16)
    torch.cuda.synchronize()
    assert torch.equal(cat, full)


def test_deterministic_rerun(B):
    w = configs.scaled(configs.GPT3_SHARD, "det", T=260, h=512, ffn=2048, t=4)
    _log("case determinism")
    d = to_device(synth.make_inputs(w))
    outs = []
    for _ in range(2):
        Y, H, Z = gpu_shard_fwd(B, w, d, 0)
        g = gpu_shard_bwd(B, w, d, 0, Y, H)
        torch.cuda.synchronize()
        outs.append([Y, H, Z] + [g[k] for k in ("dY", "dW2", "dW1", "dX", "db1")])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_gpt3_shard_step_is_bitwise_reproducible(B):
    """The GPT-3-shaped shard's forward and backward (every product layout,
    384-slab pipelines) three times back to back: every output identical to
    the bit."""
    w = configs.GPT3_SHARD
    T, h, n = w.T, w.h, w.n
    _log("case full-size step reproducibility")
    bf = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(23)
    X = torch.randn(T, h, device="cuda", generator=g).to(bf)
    W1 = (torch.randn(h, n, device="cuda", generator=g) * 0.02).to(bf)
    b1 = (torch.randn(n, device="cuda", generator=g) * 0.02).to(bf)
    W2 = (torch.randn(n, h, device="cuda", generator=g) * 0.02).to(bf)
    dZ = torch.randn(T, h, device="cuda", generator=g).to(bf)
    runs = []
    for _ in range(3):
        o = {"H": torch.empty(T, n, dtype=bf, device="cuda"),
             "Y": torch.empty(T, n, dtype=bf, device="cuda"),
             "Z": torch.empty(T, h, device="cuda"), "dY": torch.empty(T, n, dtype=bf, device="cuda"),
             "dW2": torch.empty(n, h, device="cuda"), "dW1": torch.empty(h, n, device="cuda"),
             "dX": torch.empty(T, h, device="cuda"), "db1": torch.empty(n, device="cuda")}
        B.tp_mlp_shard_fwd(X, W1, b1, W2, o["H"], o["Y"], o["Z"], T, h, w.ffn, w.t, 0, bf)
        B.tp_mlp_shard_bwd(X, W1, W2, o["Y"], o["H"], dZ, o["dY"], o["dW2"], o["dW1"], o["dX"],
                           o["db1"], T, h, w.ffn, w.t, 0, bf)
        runs.append(o)
    torch.cuda.synchronize()
    for o in runs[1:]:
        for k in o:
            assert torch.equal(o[k], runs[0][k]), f"{k} differs between runs"
    assert torch.isfinite(runs[0]["dW1"]).all() and torch.count_nonzero(runs[0]["dX"]) > 0


def test_side_stream_matches_default_stream(B):
    # Calls only enqueue on the stream they are given: a forward + backward on
    # a separate stream gives the same bytes as on the default stream.
    w = configs.scaled(configs.GPT3_SHARD, "stream", T=260, h=512, ffn=2048, t=4)
    _log("case side stream")
    d = to_device(synth.make_inputs(w))
    Y0, H0, Z0 = gpu_shard_fwd(B, w, d, 0)
    g0 = gpu_shard_bwd(B, w, d, 0, Y0, H0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        Y1, H1, Z1 = gpu_shard_fwd(B, w, d, 0, stream=side.cuda_stream)
        g1 = gpu_shard_bwd(B, w, d, 0, Y1, H1, stream=side.cuda_stream)
    side.synchronize()
    for a, b in zip([Y0, H0, Z0] + [g0[k] for k in ("dY", "dW2", "dW1", "dX", "db1")],
                    [Y1, H1, Z1] + [g1[k] for k in ("dY", "dW2", "dW1", "dX", "db1")]):
        assert torch.equal(a, b)


def test_step_captured_in_a_hip_graph_replays_bit_identical(B):
    # The library enqueues only kernels (no allocation, memset or copy), so a
    # whole forward + backward can be captured in a HIP graph.  Each replay
    # (outputs cleared by eager work in between) must give the eager bytes.
    w = configs.scaled(configs.GPT3_SHARD, "graph", T=288, h=544, ffn=2304, t=8)
    _log(f"case {w.name}: eager run, capture, three replays")
    d = to_device(synth.make_inputs(w))
    T, h, n = w.T, w.h, w.n
    bf = torch.bfloat16
    H = torch.empty(T, n, dtype=bf, device="cuda")
    Y = torch.empty(T, n, dtype=bf, device="cuda")
    Z = torch.empty(T, h, device="cuda")
    dY = torch.empty(T, n, dtype=bf, device="cuda")
    dW2 = torch.empty(n, h, device="cuda")
    dW1 = torch.empty(h, n, device="cuda")
    dX = torch.empty(T, h, device="cuda")
    db1 = torch.empty(n, device="cuda")
    outs = (H, Y, Z, dY, dW2, dW1, dX, db1)

    def step():
        B.tp_mlp_shard_fwd(d["X"], d["W1"][0], d["b1"][0], d["W2"][0], H, Y, Z, T, h, w.ffn,
                           w.t, 0, bf)
        B.tp_mlp_shard_bwd(d["X"], d["W1"][0], d["W2"][0], Y, H, d["dZ"], dY, dW2, dW1, dX,
                           db1, T, h, w.ffn, w.t, 0, bf)

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(("H", "Y", "Z", "dY", "dW2", "dW1", "dX", "db1"), outs, eager):
            assert torch.equal(o, e), f"replay {rep}: {name} differs from the eager run"


def test_two_ranks_concurrently_on_two_streams_match_serial(B):
    # The library keeps no state between or during calls (its scratch is the
    # caller's outputs), so two shards' forward + backward in flight at once
    # on two streams must give the bytes of the serial runs.
    w = configs.scaled(configs.GPT3_SHARD, "two_streams", T=288, h=544, ffn=2304, t=8,
                       ranks=(0, 5))
    _log(f"case {w.name}: serial, then concurrent on two streams")
    d = to_device(synth.make_inputs(w))
    serial = {}
    for r in w.ranks:
        Y, H, Z = gpu_shard_fwd(B, w, d, r)
        serial[r] = (Y, H, Z, gpu_shard_bwd(B, w, d, r, Y, H))
    torch.cuda.synchronize()
    streams = {r: torch.cuda.Stream() for r in w.ranks}
    conc = {}
    for _ in range(2):
        for r in w.ranks:
            with torch.cuda.stream(streams[r]):
                Y, H, Z = gpu_shard_fwd(B, w, d, r, stream=streams[r])
                conc[r] = (Y, H, Z, gpu_shard_bwd(B, w, d, r, Y, H, stream=streams[r]))
        torch.cuda.synchronize()
        for r in w.ranks:
            (Ys, Hs, Zs, gs), (Yc, Hc, Zc, gc) = serial[r], conc[r]
            for name, a, b in (("Y", Ys, Yc), ("H", Hs, Hc), ("Z", Zs, Zc)):
                assert torch.equal(a, b), f"rank {r}: {name} differs"
            for k in ("dY", "dW2", "dW1", "dX", "db1"):
                assert torch.equal(gs[k], gc[k]), f"rank {r}: {k} differs"


def test_all_ones_and_identity(B):
    _log("case all-ones / identity")
    T, h, n = 64, 768, 256
    ones_x = torch.ones(T, h, dtype=torch.bfloat16, device="cuda")
    ones_w = torch.ones(h, n, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(T, n, dtype=torch.float32, device="cuda")
    B.tp_row_linear(ones_x, ones_w, Z, T, h, n, 1, 0, B.TP_BF16, B.TP_F32)
    X = torch.randn(T, 256, device="cuda").bfloat16()
    Y = torch.empty(T, 256, dtype=torch.bfloat16, device="cuda")
    eye = torch.eye(256, device="cuda").bfloat16()
    B.tp_column_linear(X, eye, None, Y, None, T, 256, 256, 1, 0, B.TP_BF16, B.TP_BF16, B.TP_ACT_NONE)
    torch.cuda.synchronize()
    assert torch.all(Z == h)
    assert torch.equal(Y, X)


@pytest.mark.parametrize("t", [1, 2, 3, 8])
def test_shard_reduce_sum_and_concat(B, t):
    _log(f"case shard reduce t={t}")
    T, cols = 129, 264
    g = torch.Generator().manual_seed(20 + t)
    parts = torch.randn(t, T, cols, generator=g)
    p_dev = dev(parts)
    S = torch.empty(T, cols, device="cuda")
    B.tp_shard_reduce(p_dev, S, T, cols, t, B.TP_REDUCE_SUM, B.TP_F32, B.TP_F32)
    C = torch.empty(T, t * cols, device="cuda")
    B.tp_shard_reduce(p_dev, C, T, cols, t, B.TP_REDUCE_CONCAT, B.TP_F32, B.TP_F32)
    pb = dev(parts.bfloat16())
    Sb = torch.empty(T, cols, device="cuda")
    B.tp_shard_reduce(pb, Sb, T, cols, t, B.TP_REDUCE_SUM, B.TP_BF16, B.TP_F32)
    Cb = torch.empty(T, t * cols, dtype=torch.bfloat16, device="cuda")
    B.tp_shard_reduce(pb, Cb, T, cols, t, B.TP_REDUCE_CONCAT, B.TP_BF16, B.TP_BF16)
    torch.cuda.synchronize()
    ref = oracle.shard_sum(parts)
    # t fp32 additions in rank order: at most (t-1) roundings of 2^-24 each
    err = np.abs(to_np64(S) - ref)
    bound = (t - 1) * 2.0 ** -24 * oracle.shard_sum(np.abs(to_np64(parts))) + 1e-30
    assert np.all(err <= bound)
    assert np.array_equal(to_np64(C), oracle.shard_concat(parts))
    assert np.array_equal(to_np64(Cb), oracle.shard_concat(parts.bfloat16()))
    refb = oracle.shard_sum(parts.bfloat16())
    boundb = (t - 1) * 2.0 ** -24 * oracle.shard_sum(np.abs(to_np64(parts.bfloat16()))) + 1e-30
    assert np.all(np.abs(to_np64(Sb) - refb) <= boundb)


# ------------------------------------------------------ full workload sizes

@pytest.fixture(scope="module")
def gpt3_run(B):
    w = configs.GPT3_SHARD
    _log(f"case {w.name}: generating inputs")
    d_h = synth.make_inputs(w)
    d = to_device(d_h)
    _log(f"case {w.name}: GPU forward + backward")
    Y, H, Z = gpu_shard_fwd(B, w, d, 0)
    g = gpu_shard_bwd(B, w, d, 0, Y, H)
    torch.cuda.synchronize()
    out = {"Y": Y.cpu(), "H": H.cpu(), "Z": Z.cpu()}
    out.update({k: v.cpu() for k, v in g.items()})
    del d
    torch.cuda.empty_cache()
    return w, d_h, out


def test_gpt3_shard_forward_whole_tensors(gpt3_run):
    # The GPT-3 shard's forward (configuration 3) against the oracle on every
    # element of Y_i, H_i and Z_i.
    w, d_h, out = gpt3_run
    _log(f"case {w.name}: oracle forward (whole tensors)")
    rY, rH, rZ = oracle.mlp_shard_fwd(d_h["X"], d_h["W1"][0], d_h["b1"][0], d_h["W2"][0])
    _whole(out["Y"], rY, "bf16", "gpt3 Y")
    _whole(out["H"], rH, "bf16", "gpt3 H")
    _whole(out["Z"], rZ, "bf16", "gpt3 Z")


def test_gpt3_shard_backward_whole_tensors(gpt3_run):
    # The GPT-3 shard's backward (configuration 4) against the oracle on every
    # element of dY_i, dW2_i, dW1_i, dX_i and db1_i.  The weight gradients
    # (1536 tiles each) take the grouped tile walk.
    w, d_h, out = gpt3_run
    _log(f"case {w.name}: oracle backward (whole tensors)")
    g = oracle.mlp_shard_bwd(d_h["X"], d_h["W1"][0], d_h["b1"][0], d_h["W2"][0], d_h["dZ"])
    for k in ("dY", "dW2", "dW1", "dX", "db1"):
        _whole(out[k], g[k], "bf16", f"gpt3 {k}")


@pytest.mark.parametrize("T,k,n", [(1000, 96, 24920), (1024, 24920, 992)],
                         ids=["column_row_1000x96x24920", "linear_bwd_1024x24920x992"])
def test_grouped_tile_walk_elementwise(B, T, k, n):
    # Products of more than two waves of 256 x 192 tiles walk each XCD's
    # tiles in groups of four tile rows.  Here 4 x 130 = 520 tiles (a multiple
    # of the 8 XCDs, so the XCD remap applies as well), with ragged M and N
    # tails, compared element by element:
    #   (1000, 96, 24920): the column layer (bias + GeLU, Y saved) and the row
    #     layer's plain fp32 product, both NN;
    #   (1024, 24920, 992): a linear shard's backward, whose dX is an NT
    #     product and whose dW is dY^T X stored transposed (NN, M = 992).
    bf = torch.bfloat16
    g = torch.Generator().manual_seed(T + k + n)
    r = lambda *sh, std=1.0: (torch.randn(*sh, generator=g) * std).to(bf)
    if k == 96:
        X, W, b = r(T, k), r(k, n, std=0.02), r(n, std=0.02)
        H = torch.empty(T, n, dtype=bf, device="cuda")
        Y = torch.empty(T, n, dtype=bf, device="cuda")
        Z = torch.empty(T, n, dtype=torch.float32, device="cuda")
        Xd, Wd, bd = dev(X), dev(W), dev(b)
        B.tp_column_linear(Xd, Wd, bd, H, Y, T, k, n, 1, 0, bf, bf, B.TP_ACT_GELU_TANH)
        B.tp_row_linear(Xd, Wd, Z, T, k, n, 1, 0, bf, torch.float32)
        torch.cuda.synchronize()
        _whole(Y, oracle.column_linear(X, W, b), "bf16", "grouped walk: column Y")
        _whole(H, oracle.column_linear(X, W, b, gelu=True), "bf16", "grouped walk: column H")
        _whole(Z, oracle.row_linear(X, W), "bf16", "grouped walk: row Z")
    else:
        X, W, dY = r(T, k), r(k, n, std=0.02), r(T, n)
        dX = torch.empty(T, k, dtype=torch.float32, device="cuda")
        dW = torch.empty(k, n, dtype=torch.float32, device="cuda")
        db = torch.empty(n, dtype=torch.float32, device="cuda")
        B.tp_linear_bwd(dev(X), dev(W), dev(dY), dX, dW, db, T, k, n, bf)
        torch.cuda.synchronize()
        ref = oracle.linear_bwd(X, W, dY)
        _whole(dX, ref["dX"], "bf16", "grouped walk: dX")
        _whole(dW, ref["dW"], "bf16", "grouped walk: dW")
        _whole(db, ref["db"], "bf16", "grouped walk: db")


MAX_OPERAND_BYTES = 2**31 - 1   # the boundary rejects any larger operand


def test_largest_accepted_activation_column_sampled(B):
    # X [65535, 16384] bf16 is 32 KiB under 2^31 bytes: the tile kernel's
    # 32-bit buffer offsets reach their largest values; 65535 rows leave a
    # 255-row last tile.  One more token is rejected.
    w = configs.scaled(configs.GPT3_SHARD, "largest_x", T=65535, h=16384, ffn=256, t=1,
                       backward=False)
    assert w.T * w.h * 2 <= MAX_OPERAND_BYTES < (w.T + 1) * w.h * 2
    _log(f"case {w.name}: generating inputs")
    d_h = synth.make_inputs(w, with_dz=False)
    X, W, b = dev(d_h["X"]), dev(d_h["W1"][0]), dev(d_h["b1"][0])
    H = torch.empty(w.T, w.n, dtype=torch.bfloat16, device="cuda")
    Y = torch.empty(w.T, w.n, dtype=torch.bfloat16, device="cuda")
    _log(f"case {w.name}: column layer")
    B.tp_column_linear(X, W, b, H, Y, w.T, w.h, w.ffn, w.t, 0, B.TP_BF16, B.TP_BF16,
                       B.TP_ACT_GELU_TANH)
    torch.cuda.synchronize()
    # raw addresses: the library's own size check, not the binding's
    ptrs = [x.data_ptr() for x in (X, W, b, H, Y)]
    assert B.tp_column_linear(*ptrs, w.T + 1, w.h, w.ffn, w.t, 0, B.TP_BF16, B.TP_BF16,
                              B.TP_ACT_GELU_TANH, check=False) == B.TP_ERR_SHAPE
    rows = sample_indices(w.T, 8, seed=5)
    rows = np.union1d(rows, np.arange(w.T - 255, w.T, 37))   # the ragged last tile
    _log(f"case {w.name} rows {rows.tolist()}")
    Xr = d_h["X"][torch.from_numpy(rows)]
    rY = oracle.column_linear(Xr, d_h["W1"][0], d_h["b1"][0], gelu=False)
    rH = oracle.column_linear(Xr, d_h["W1"][0], d_h["b1"][0], gelu=True)
    idx = torch.from_numpy(rows).cuda()
    assert_close(Y[idx], rY, "bf16", "largest X: Y rows")
    assert_close(H[idx], rH, "bf16", "largest X: H rows")


def test_largest_accepted_fp32_outputs_fwd_bwd_sampled(B):
    # Z and dX [32736, 16384] fp32 are just under 2^31 bytes; T % 32 == 0, so
    # the weight gradients take the transposed-operand products (X^T of 1 GiB
    # staged in dX).  T = 32768 is rejected.
    w = configs.scaled(configs.GPT3_SHARD, "largest_fp32_out", T=32736, h=16384, ffn=256, t=1)
    assert w.T * w.h * 4 <= MAX_OPERAND_BYTES < 32768 * w.h * 4
    _log(f"case {w.name}: generating inputs")
    d_h = synth.make_inputs(w)
    d = to_device(d_h)
    _log(f"case {w.name}: forward + backward")
    Y, H, Z = gpu_shard_fwd(B, w, d, 0)
    g = gpu_shard_bwd(B, w, d, 0, Y, H)
    torch.cuda.synchronize()
    ptrs = [x.data_ptr() for x in (d["X"], d["W1"][0], d["b1"][0], d["W2"][0], H, Y, Z)]
    assert B.tp_mlp_shard_fwd(*ptrs, 32768, w.h, w.ffn, w.t, 0, B.TP_BF16,
                              check=False) == B.TP_ERR_SHAPE
    out = {"Y": Y.cpu(), "H": H.cpu(), "Z": Z.cpu()}
    out.update({k: v.cpu() for k, v in g.items()})
    del d, Y, H, Z, g
    torch.cuda.empty_cache()
    rows = sample_indices(w.T, 4, seed=6)
    cols = np.array([0, w.n - 1])
    _log(f"case {w.name} rows {rows.tolist()} cols {cols.tolist()}")
    rY, rH, rZ = oracle.mlp_shard_fwd_rows(d_h["X"], d_h["W1"][0], d_h["b1"][0], d_h["W2"][0],
                                           rows)
    assert_close(out["Y"][rows], rY, "bf16", "largest fp32: Y rows")
    assert_close(out["H"][rows], rH, "bf16", "largest fp32: H rows")
    assert_close(out["Z"][rows], rZ, "bf16", "largest fp32: Z rows")
    gr = oracle.mlp_shard_bwd_rows(d_h["X"], d_h["W1"][0], d_h["b1"][0], d_h["W2"][0],
                                   d_h["dZ"], rows)
    assert_close(out["dY"][rows], gr["dY"], "bf16", "largest fp32: dY rows")
    assert_close(out["dX"][rows], gr["dX"], "bf16", "largest fp32: dX rows")
    _log(f"case {w.name}: oracle column subset")
    gc = oracle.mlp_shard_bwd_cols(d_h["X"], d_h["W1"][0], d_h["b1"][0], d_h["W2"][0],
                                   d_h["dZ"], cols)
    assert_close(out["dW1"][:, cols], gc["dW1"], "bf16", "largest fp32: dW1 cols")
    assert_close(out["dW2"][cols, :], gc["dW2"], "bf16", "largest fp32: dW2 rows")
    assert_close(out["db1"][cols], gc["db1"], "bf16", "largest fp32: db1")


def test_full_layer_emulation_8_shards_whole_output(B):
    w = configs.FULL_LAYER_8
    _log(f"case {w.name}: generating inputs")
    d_h = synth.make_inputs(w)
    d = to_device(d_h)
    parts = torch.empty(w.t, w.T, w.h, dtype=torch.float32, device="cuda")
    H = torch.empty(w.T, w.n, dtype=torch.bfloat16, device="cuda")
    _log(f"case {w.name}: 8 shards + shard-sum on the GPU")
    for r in w.ranks:
        B.tp_mlp_shard_fwd(d["X"], d["W1"][r], None, d["W2"][r], H, None, parts[r], w.T, w.h,
                           w.ffn, w.t, r, B.TP_BF16)
    Z = torch.empty(w.T, w.h, dtype=torch.float32, device="cuda")
    B.tp_shard_reduce(parts, Z, w.T, w.h, w.t, B.TP_REDUCE_SUM, B.TP_F32, B.TP_F32)
    # The same layer with the 8 shards' products batched into two launches:
    # every tile computes what the per-shard call computes, so the partials
    # and their sum agree bit for bit.
    _log(f"case {w.name}: all shards batched (tp_mlp_layer_fwd) + shard-sum")
    W1s = torch.stack([d["W1"][r] for r in w.ranks])
    W2s = torch.stack([d["W2"][r] for r in w.ranks])
    Hs = torch.empty(w.t, w.T, w.n, dtype=torch.bfloat16, device="cuda")
    parts_b = torch.empty_like(parts)
    B.tp_mlp_layer_fwd(d["X"], W1s, None, W2s, Hs, None, parts_b, w.T, w.h, w.ffn, w.t,
                       B.TP_BF16)
    Zb = torch.empty_like(Z)
    B.tp_shard_reduce(parts_b, Zb, w.T, w.h, w.t, B.TP_REDUCE_SUM, B.TP_F32, B.TP_F32)
    torch.cuda.synchronize()
    assert torch.equal(parts_b, parts), "batched partials differ from the per-shard ones"
    assert torch.equal(Zb, Z), "batched layer output differs from the per-shard one"
    assert torch.equal(Hs[w.t - 1], H), "batched H of the last shard differs"
    Zc = Z.cpu()
    del d, parts, parts_b, W1s, W2s, Hs
    torch.cuda.empty_cache()
    # The summed layer output (configuration 5) against the unsharded oracle,
    # X [4096, 8192] through W1 [8192, 28672] and W2 [28672, 8192], on every
    # element.
    _log(f"case {w.name}: unsharded oracle (whole output)")
    W1, b1, W2 = _unsharded(d_h, w.ranks)
    _, _, rZ = oracle.mlp_shard_fwd(d_h["X"], W1, b1, W2)
    _whole(Zc, rZ, "bf16", "full layer Z")


LAYER_FWD = [  # (tokens, h, ffn, t, dtype, bias, save)
    (300, 512, 8 * 224, 8, "bf16", True, True),    # tile kernel, ragged M and N tails
    (512, 384, 4 * 384, 4, "bf16", False, True),   # tile kernel, whole tiles, no bias
    (96, 256, 2 * 128, 2, "bf16", True, False),    # shard narrower than a tile: general kernel
    (64, 128, 512, 4, "f32", True, True),          # fp32: general kernel, one launch per shard
    (272, 256, 1 * 448, 1, "bf16", True, True),    # t = 1: the unsharded layer
    # 40 small tiles per shard (K-split pipelines), 320 for the batch
    (1000, 256, 8 * 480, 8, "bf16", True, True),
    (0, 256, 8 * 192, 8, "bf16", True, True),      # no tokens: nothing to do
    # three shards of 66 large tiles each (198 in the batch, not a multiple of the
    # 8 XCDs: no remap), ragged M and N; each shard alone runs on 128 x 96 tiles
    (1500, 256, 3 * 2104, 3, "bf16", True, True),
]


@pytest.mark.parametrize("shape", LAYER_FWD, ids=lambda s: "x".join(map(str, s)))
def test_layer_fwd_matches_each_shard_and_the_oracle(B, shape):
    T, h, ffn, t, dt, bias, save = shape
    _log(f"case layer fwd {shape}")
    w = configs.Workload("layer_fwd", T=T, h=h, ffn=ffn, t=t, dtype=dt, ranks=tuple(range(t)),
                         bias=bias)
    n = w.n
    d_h = synth.make_inputs(w, seed=21)
    d = to_device(d_h)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    W1s = torch.stack([d["W1"][r] for r in range(t)])
    W2s = torch.stack([d["W2"][r] for r in range(t)])
    b1s = torch.stack([d["b1"][r] for r in range(t)]) if bias else None
    # stacked outputs followed by NaN sentinels inside the same allocation
    Hf, Hs = _nan_padded(torch.zeros(t, T, n, dtype=tdt, device="cuda"))
    Yf, Ys = _nan_padded(torch.zeros(t, T, n, dtype=tdt, device="cuda"))
    Zf, Zs = _nan_padded(torch.zeros(t, T, h, dtype=torch.float32, device="cuda"))
    if not T:
        # Empty arrays have no storage; NaN-filled placeholders stand for the
        # [0, *] arrays and must come back untouched.
        ph = torch.full((64,), float("nan"), dtype=tdt, device="cuda")
        phf = torch.full((64,), float("nan"), device="cuda")
        assert B.tp_mlp_layer_fwd(ph, W1s, b1s, W2s, ph, ph, phf, T, h, ffn, t, tdt) == 0
        torch.cuda.synchronize()
        assert torch.isnan(ph).all() and torch.isnan(phf).all()
        return
    B.tp_mlp_layer_fwd(d["X"], W1s, b1s, W2s, Hs, Ys if save else None, Zs, T, h, ffn, t, tdt)
    torch.cuda.synchronize()
    assert torch.isnan(Hf[Hs.numel():]).all() and torch.isnan(Zf[Zs.numel():]).all()
    assert torch.isnan(Yf[Ys.numel():]).all()
    if not save:
        assert torch.count_nonzero(Ys) == 0
    for r in range(t):
        Y, H, Z = gpu_shard_fwd(B, w, d, r)
        torch.cuda.synchronize()
        assert torch.equal(Hs[r], H), f"H[{r}] differs from the per-shard call"
        assert torch.equal(Zs[r], Z), f"Z[{r}] differs from the per-shard call"
        if save:
            assert torch.equal(Ys[r], Y), f"Y[{r}] differs from the per-shard call"
        rY, rH, rZ = oracle.mlp_shard_fwd(d_h["X"], d_h["W1"][r], d_h["b1"][r], d_h["W2"][r])
        assert_close(Hs[r], rH, dt, f"layer fwd H[{r}]")
        assert_close(Zs[r], rZ, dt, f"layer fwd Z[{r}]")
    Zsum = torch.empty(T, h, dtype=torch.float32, device="cuda")
    B.tp_shard_reduce(Zs, Zsum, T, h, t, B.TP_REDUCE_SUM, B.TP_F32, B.TP_F32)
    torch.cuda.synchronize()
    W1, b1, W2 = _unsharded(d_h, range(t))
    _, _, rZ = oracle.mlp_shard_fwd(d_h["X"], W1, b1, W2)
    assert_close(Zsum, rZ, dt, "layer fwd: sum of the partials vs the unsharded layer")


def test_layer_fwd_stacked_weights_beyond_2gib_sampled(B):
    """Eight shards of 302 MB weights each: the stacked W1 and W2 are 2.4 GB, so
    the later shards sit more than 2^31 bytes past the base pointer (64-bit
    shard offsets); every shard's partial and their sum, on sampled rows,
    against the oracle shard by shard."""
    T, h, t = 256, 12288, 8
    n = 12288
    ffn = n * t
    _log(f"case layer fwd, stacked weights of {2 * t * h * n / 2**30:.1f} GiB: drawing on the device")
    g = torch.Generator(device="cuda").manual_seed(17)
    bf = torch.bfloat16
    X = torch.randn(T, h, device="cuda", generator=g).to(bf)
    W1 = (torch.randn(t, h, n, device="cuda", generator=g) * 0.02).to(bf)
    W2 = (torch.randn(t, n, h, device="cuda", generator=g) * 0.02).to(bf)
    b1 = (torch.randn(t, n, device="cuda", generator=g) * 0.02).to(bf)
    H = torch.empty(t, T, n, dtype=bf, device="cuda")
    Z = torch.empty(t, T, h, dtype=torch.float32, device="cuda")
    assert W1.numel() * 2 > 2**31 and W2.numel() * 2 > 2**31
    B.tp_mlp_layer_fwd(X, W1, b1, W2, H, None, Z, T, h, ffn, t, bf)
    Zs = torch.empty(T, h, dtype=torch.float32, device="cuda")
    B.tp_shard_reduce(Z, Zs, T, h, t, B.TP_REDUCE_SUM, torch.float32, torch.float32)
    torch.cuda.synchronize()
    rows = sample_indices(T, 3, seed=17)
    Xr = X[rows].cpu()
    ref_sum = np.zeros((len(rows), h))
    for r in range(t):
        _log(f"case layer fwd beyond 2 GiB: oracle rows {rows.tolist()} of shard {r}")
        _, rH, rZ = oracle.mlp_shard_fwd(Xr, W1[r].cpu(), b1[r].cpu(), W2[r].cpu())
        assert_close(H[r][rows], rH, "bf16", f"stacked H[{r}] rows")
        assert_close(Z[r][rows], rZ, "bf16", f"stacked Z[{r}] rows")
        ref_sum += rZ
    assert_close(Zs[rows], ref_sum, "bf16", "stacked layer sum rows")
    del W1, W2, H, Z
    torch.cuda.empty_cache()


def _nan_padded(x, pad=1 << 16):
    """x on the device, followed inside the same allocation by `pad` NaNs."""
    flat = torch.full((x.numel() + pad,), float("nan"), dtype=x.dtype, device="cuda")
    flat[:x.numel()].copy_(x.reshape(-1))
    return flat, flat[:x.numel()].view(x.shape)


@pytest.mark.parametrize("shape", [(270, 512, 2048, 8), (300, 384, 1024, 4), (520, 768, 4096, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ragged_tails_touch_nothing_past_the_operands(B, shape):
    # Ragged token counts (the K of the x^T dy products) and shard widths that
    # are not multiples of the tile (ragged N of the forward products): every
    # operand and output sits at the start of an allocation whose remaining
    # bytes are NaN.  A read past an operand would put NaN into the results;
    # a write past an output would overwrite the NaN tail.
    T, h, ffn, t = shape
    w = configs.scaled(configs.GPT3_SHARD, "ragged_pad", T=T, h=h, ffn=ffn, t=t)
    n = w.n
    _log(f"case padded ragged {shape}")
    d_h = synth.make_inputs(w)
    bufs, dev_in = {}, {}
    for k, x in (("X", d_h["X"]), ("W1", d_h["W1"][0]), ("b1", d_h["b1"][0]),
                 ("W2", d_h["W2"][0]), ("dZ", d_h["dZ"])):
        bufs[k], dev_in[k] = _nan_padded(x.to("cuda"))
    outs = {}
    for k, shp, dt in (("H", (T, n), torch.bfloat16), ("Y", (T, n), torch.bfloat16),
                       ("Z", (T, h), torch.float32), ("dY", (T, n), torch.bfloat16),
                       ("dW2", (n, h), torch.float32), ("dW1", (h, n), torch.float32),
                       ("dX", (T, h), torch.float32), ("db1", (n,), torch.float32)):
        bufs[k], outs[k] = _nan_padded(torch.zeros(shp, dtype=dt, device="cuda"))
    bf = torch.bfloat16
    B.tp_mlp_shard_fwd(dev_in["X"], dev_in["W1"], dev_in["b1"], dev_in["W2"], outs["H"], outs["Y"],
                       outs["Z"], T, h, ffn, t, 0, bf)
    B.tp_mlp_shard_bwd(dev_in["X"], dev_in["W1"], dev_in["W2"], outs["Y"], outs["H"], dev_in["dZ"],
                       outs["dY"], outs["dW2"], outs["dW1"], outs["dX"], outs["db1"], T, h, ffn, t,
                       0, bf)
    torch.cuda.synchronize()
    for k, buf in bufs.items():
        size = (dev_in[k] if k in dev_in else outs[k]).numel()
        assert torch.isnan(buf[size:]).all(), f"{k}: bytes past the tensor were written"
    _, _, rZ = oracle.mlp_shard_fwd(d_h["X"], d_h["W1"][0], d_h["b1"][0], d_h["W2"][0])
    rg = oracle.mlp_shard_bwd(d_h["X"], d_h["W1"][0], d_h["b1"][0], d_h["W2"][0], d_h["dZ"])
    assert_close(outs["Z"], rZ, "bf16", "padded Z")
    for k in ("dY", "dW2", "dW1", "dX", "db1"):
        assert_close(outs[k], rg[k], "bf16", f"padded {k}")


# ------------------------------------------- sequence parallelism: RS, LN, AG

@pytest.mark.parametrize("t", [1, 2, 4, 8])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_reduce_scatter_each_rank(B, t, out_dt):
    T, cols = 24 * t, 136
    _log(f"case reduce-scatter t={t} out={out_dt}")
    g = torch.Generator().manual_seed(20 + t)
    parts_h = torch.randn(t, T, cols, generator=g)
    parts = dev(parts_h)
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    for r in range(t):
        out = torch.empty(T // t, cols, dtype=odt, device="cuda")
        B.tp_shard_reduce_scatter(parts, out, T, cols, t, r, B.TP_F32, odt)
        torch.cuda.synchronize()
        ref = oracle.reduce_scatter(parts_h, r)
        if out_dt == "f32":
            # fp32 adds in rank order: within t roundings of the exact sum
            bound = t * 2.0**-24 * np.abs(to_np64(parts_h[:, r * (T // t):(r + 1) * (T // t)])).sum(0)
            assert np.all(np.abs(to_np64(out) - ref) <= bound + 1e-30)
        else:
            assert_close(out, ref, "bf16", f"reduce-scatter t={t} r={r}")


def test_concat_tokens_is_the_stacked_layout_bitexact(B):
    t, Tr, cols = 8, 33, 200
    _log("case concat tokens")
    g = torch.Generator().manual_seed(31)
    parts = dev(torch.randn(t, Tr, cols, generator=g).bfloat16())
    out = torch.empty(t * Tr, cols, dtype=torch.bfloat16, device="cuda")
    B.tp_shard_reduce(parts, out, Tr, cols, t, B.TP_REDUCE_CONCAT_TOKENS, B.TP_BF16, B.TP_BF16)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.cat([parts[r].cpu() for r in range(t)], dim=0))


@pytest.mark.parametrize("in_dt,out_dt", [("f32", "f32"), ("f32", "bf16"), ("bf16", "bf16"),
                                          ("bf16", "f32")])
@pytest.mark.parametrize("T,cols", [(77, 520), (9, 12296), (9, 17008), (5, 33008)])
def test_layernorm_matches_oracle(B, in_dt, out_dt, T, cols):
    # rows held in registers, one, two and four 8-column octets per thread
    # of 1024 (520, 12296, 17008 columns), and rows read three times (33008)
    _log(f"case layernorm {in_dt}->{out_dt} {T}x{cols}")
    g = torch.Generator().manual_seed(41)
    idt = torch.float32 if in_dt == "f32" else torch.bfloat16
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    x_h = (3.0 * torch.randn(T, cols, generator=g) + 1.5).to(idt)
    gam_h = (1.0 + 0.1 * torch.randn(cols, generator=g)).to(odt)
    bet_h = (0.1 * torch.randn(cols, generator=g)).to(odt)
    x_h[5 % T] = 2.0                   # a constant row: y = beta exactly
    y = torch.empty(T, cols, dtype=odt, device="cuda")
    B.tp_layernorm(dev(x_h), dev(gam_h), dev(bet_h), y, T, cols, 1e-5, idt, odt)
    y2 = torch.empty_like(y)
    B.tp_layernorm(dev(x_h), dev(gam_h), dev(bet_h), y2, T, cols, 1e-5, idt, odt)
    torch.cuda.synchronize()
    ref = oracle.layernorm(x_h, gam_h, bet_h, 1e-5)
    if out_dt == "f32":
        rf = np.linalg.norm(to_np64(y) - ref) / np.linalg.norm(ref)
        assert rf <= 1e-5, rf
    else:
        assert_close(y, ref, "bf16", f"layernorm {in_dt}->{out_dt}")
    assert torch.equal(y[5 % T].cpu(), bet_h)
    assert torch.equal(y.cpu(), y2.cpu())          # fixed reduction order


@pytest.mark.parametrize("affine", [True, False])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T,cols", [(77, 520), (9, 17008), (5, 33008)])
def test_layernorm_in_place(B, dt, T, cols, affine):
    # y == x is allowed for equal types: the registers-held rows and the
    # three-pass rows (33008 columns) give the out-of-place bits in place;
    # without gamma and beta (NULL) the scale is 1 and the shift 0
    _log(f"case layernorm in place {dt} {T}x{cols} affine={affine}")
    g = torch.Generator().manual_seed(43)
    t_dt = torch.float32 if dt == "f32" else torch.bfloat16
    x_h = (2.0 * torch.randn(T, cols, generator=g) - 0.5).to(t_dt)
    gam_h = (1.0 + 0.1 * torch.randn(cols, generator=g)).to(t_dt) if affine else None
    bet_h = (0.1 * torch.randn(cols, generator=g)).to(t_dt) if affine else None
    gam = dev(gam_h) if affine else None
    bet = dev(bet_h) if affine else None
    y = torch.empty(T, cols, dtype=t_dt, device="cuda")
    B.tp_layernorm(dev(x_h), gam, bet, y, T, cols, 1e-5, t_dt, t_dt)
    x = dev(x_h)
    B.tp_layernorm(x, gam, bet, x, T, cols, 1e-5, t_dt, t_dt)
    torch.cuda.synchronize()
    assert torch.equal(x.cpu(), y.cpu())
    ref = oracle.layernorm(x_h, gam_h, bet_h, 1e-5)
    if dt == "f32":
        rf = np.linalg.norm(to_np64(x) - ref) / np.linalg.norm(ref)
        assert rf <= 1e-5, rf
    else:
        assert_close(x, ref, "bf16", "layernorm in place")


@pytest.mark.parametrize("in_dt,out_dt", [("f32", "bf16"), ("f32", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("T,cols,t", [(24, 136, 8), (18, 12296, 3), (4, 33008, 2), (64, 520, 1)])
def test_reduce_scatter_layernorm_fused(B, in_dt, out_dt, T, cols, t):
    # The fused call gives the bits of the two calls it replaces (the
    # ReduceScatter with an fp32 output, then the layer norm of that output)
    # for every rank, and matches the oracle's sum-then-normalise.  Widths
    # cover one, two and four octets per thread of the register-resident
    # rows and the three-pass rows; t = 3 takes the kernel's runtime rank loop.
    _log(f"case reduce-scatter + layer norm {in_dt}->{out_dt} T={T} cols={cols} t={t}")
    g = torch.Generator().manual_seed(61)
    idt = torch.float32 if in_dt == "f32" else torch.bfloat16
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    parts_h = (2.0 * torch.randn(t, T, cols, generator=g) + 0.5).to(idt)
    gam_h = (1.0 + 0.1 * torch.randn(cols, generator=g)).to(odt)
    bet_h = (0.1 * torch.randn(cols, generator=g)).to(odt)
    parts, gam, bet = dev(parts_h), dev(gam_h), dev(bet_h)
    for r in range(t):
        y = torch.empty(T // t, cols, dtype=odt, device="cuda")
        B.tp_shard_reduce_scatter_layernorm(parts, gam, bet, y, T, cols, t, r, 1e-5, idt, odt)
        s32 = torch.empty(T // t, cols, dtype=torch.float32, device="cuda")
        B.tp_shard_reduce_scatter(parts, s32, T, cols, t, r, idt, torch.float32)
        y2 = torch.empty_like(y)
        B.tp_layernorm(s32, gam, bet, y2, T // t, cols, 1e-5, torch.float32, odt)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), f"rank {r}: fused result differs from the two calls"
        ref = oracle.layernorm(oracle.reduce_scatter(parts_h, r), gam_h, bet_h, 1e-5)
        if out_dt == "f32":
            assert rel_fro_ok(y, ref)
        else:
            assert_close(y, ref, "bf16", f"rs+ln rank {r}")


def rel_fro_ok(got, ref):
    rf = np.linalg.norm(to_np64(got) - ref) / np.linalg.norm(ref)
    return rf <= 1e-5


def test_sequence_parallel_chain_gpt3_whole(B):
    """Row-layer partials of t = 8 ranks at the GPT-3 shape -> ReduceScatter
    to rank 3's 256 tokens (fp32) -> layer norm -> bf16 -> token AllGather
    stand-in, against the oracle on every element of the shard."""
    T, h, t, r = 2048, 12288, 8, 3
    _log("case sequence-parallel chain gpt3")
    g = torch.Generator().manual_seed(51)
    parts_h = torch.randn(t, T, h, generator=g)
    gam_h = (1.0 + 0.1 * torch.randn(h, generator=g)).bfloat16()
    bet_h = (0.1 * torch.randn(h, generator=g)).bfloat16()
    parts = dev(parts_h)
    rs = torch.empty(T // t, h, dtype=torch.float32, device="cuda")
    B.tp_shard_reduce_scatter(parts, rs, T, h, t, r, B.TP_F32, B.TP_F32)
    y = torch.empty(T // t, h, dtype=torch.bfloat16, device="cuda")
    B.tp_layernorm(rs, dev(gam_h), dev(bet_h), y, T // t, h, 1e-5, B.TP_F32, B.TP_BF16)
    shards = torch.empty(t, T // t, h, dtype=torch.bfloat16, device="cuda")
    shards[r] = y
    full = torch.empty(T, h, dtype=torch.bfloat16, device="cuda")
    B.tp_shard_reduce(shards, full, T // t, h, t, B.TP_REDUCE_CONCAT_TOKENS, B.TP_BF16, B.TP_BF16)
    torch.cuda.synchronize()
    ref_rs = oracle.reduce_scatter(parts_h, r)
    # the fp32 sum: within the summation bound of t - 1 additions
    bound = (t - 1) * 2.0 ** -24 * oracle.reduce_scatter(parts_h.abs(), r) + 1e-30
    assert np.all(np.abs(to_np64(rs) - ref_rs) <= bound)
    _whole(y, oracle.layernorm(ref_rs, gam_h, bet_h, 1e-5), "bf16", "sp chain layer norm")
    assert torch.equal(full[r * (T // t):(r + 1) * (T // t)].cpu(), y.cpu())
    # the same shard from the fused reduce-scatter + layer norm, bit for bit
    yf = torch.empty_like(y)
    B.tp_shard_reduce_scatter_layernorm(parts, dev(gam_h), dev(bet_h), yf, T, h, t, r, 1e-5,
                                        B.TP_F32, B.TP_BF16)
    torch.cuda.synchronize()
    assert torch.equal(yf, y)
