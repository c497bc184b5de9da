"""The GPU parity bars catch a single wrong tile (CPU only).

The bf16 bar is a relative Frobenius error of 4e-3 over the whole tensor and
a max |error| of 1e-2 of max |reference|.  A kernel mistake confined to one
256 x 192 output tile (one missing 32-deep k slab, the bias left out or the
activation applied twice, two rows or a 16 x 16 fragment swapped) barely
moves the Frobenius error of a large tensor, so the max-ratio bar is what
must catch it.  Here the reference is the oracle's forward of a seeded
shard, the "correct" result is that reference rounded to bf16 (which must
pass), and each planted mistake changes one tile of it (which must fail).
"""
import numpy as np
import pytest
import torch

import oracle
from parity_utils import assert_close

T, H, N = 768, 2048, 576          # three tile rows, three tile columns of 256 x 192
TM, TN, BK = 256, 192, 32


@pytest.fixture(scope="module")
def shard():
    g = torch.Generator().manual_seed(11)
    bf = torch.bfloat16
    X = torch.randn(T, H, generator=g).to(bf).double().numpy()
    W = (0.02 * torch.randn(H, N, generator=g)).to(bf).double().numpy()
    b = (0.02 * torch.randn(N, generator=g)).to(bf).double().numpy()
    pre = oracle.column_linear(X, W, b)
    act = oracle.column_linear(X, W, b, gelu=True)
    return X, W, b, pre, act


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).double().numpy()


def tile(tm, tn):
    return slice(tm * TM, (tm + 1) * TM), slice(tn * TN, (tn + 1) * TN)


def test_the_rounded_reference_passes(shard):
    *_, pre, act = shard
    assert_close(bf16(pre), pre, "bf16", "pre-activation")
    assert_close(bf16(act), act, "bf16", "activation")


def mistakes(X, W, b, pre, act):
    r, c = tile(1, 2)
    out = {}
    # one 32-deep k slab missing from one tile's sum (a wait or ring-index slip)
    k = slice(5 * BK, 6 * BK)
    m = act.copy()
    m[r, c] = oracle.gelu_tanh(pre[r, c] - X[r, k] @ W[k, c])
    out["one k slab missing in one tile"] = m
    # the bias left out of one tile
    m = act.copy()
    m[r, c] = oracle.gelu_tanh(pre[r, c] - b[c])
    out["bias missing in one tile"] = m
    # the activation applied twice in one tile
    m = act.copy()
    m[r, c] = oracle.gelu_tanh(act[r, c])
    out["GeLU applied twice in one tile"] = m
    # two rows of one tile exchanged (a lane-to-row slip in the epilogue)
    m = act.copy()
    rows = np.arange(TM, 2 * TM)
    rows[[3, 17]] = rows[[17, 3]]
    m[TM:2 * TM, c] = act[rows, c]
    out["two rows of one tile swapped"] = m
    # one 16 x 16 fragment stored transposed
    m = act.copy()
    f = act[TM + 32:TM + 48, 2 * TN + 16:2 * TN + 32]
    m[TM + 32:TM + 48, 2 * TN + 16:2 * TN + 32] = f.T
    out["one fragment transposed"] = m
    # one tile from the neighbouring column block (a tile-index slip)
    m = act.copy()
    m[r, c] = act[r, tile(1, 1)[1]]
    out["one tile's columns from the neighbour"] = m
    return out


@pytest.mark.parametrize("name", ["one k slab missing in one tile", "bias missing in one tile",
                                  "GeLU applied twice in one tile", "two rows of one tile swapped",
                                  "one fragment transposed", "one tile's columns from the neighbour"])
def test_a_wrong_tile_fails_the_bar(shard, name):
    X, W, b, pre, act = shard
    bad = bf16(mistakes(X, W, b, pre, act)[name])
    with pytest.raises(AssertionError):
        assert_close(bad, act, "bf16", name)
