"""Workload shapes for one tensor-parallel rank's MLP shard.

Names follow the pages' notation: ``T`` tokens, ``h`` hidden size, ``ffn`` the
inner width (4h for the GPT-3 shape), ``t`` the tensor-parallel degree and
``n = ffn / t`` the shard width.  Weight shards are stored ``[in, out]`` and
used as ``x @ W`` (page "张量并行实战", section "PyTorch 实现示例").
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    h: int                 # hidden size (input width of the column layer)
    ffn: int               # full inner width before the split
    t: int                 # tensor-parallel degree
    dtype: str             # "f32" or "bf16"
    ranks: tuple = (0,)    # shards computed on the one GPU
    bias: bool = True      # whether b1 is drawn (N(0, std_w)) or absent
    bias_zero: bool = False  # bias present but all zeros
    gelu: bool = True      # column layer followed by the activation
    row_layer: bool = True  # whether the row-parallel layer follows
    backward: bool = False
    std_w: float = 0.02
    note: str = field(default="", compare=False)

    @property
    def n(self) -> int:
        assert self.ffn % self.t == 0
        return self.ffn // self.t

    def fwd_flops(self) -> float:
        """GEMM multiply-add FLOPs of one shard's forward (2*M*N*K per GEMM)."""
        f = 2.0 * self.T * self.h * self.n
        return f * (2 if self.row_layer else 1) * len(self.ranks)

    def bwd_flops(self) -> float:
        """Four GEMMs of the same size as one forward GEMM."""
        return 4 * 2.0 * self.T * self.h * self.n * len(self.ranks)


# Tiny MLP in fp32, both shards of t=2, zero biases; compared as Z_0 + Z_1
# against the unsharded layer.
TINY_F32 = Workload("tiny_mlp_f32_t2", T=32, h=128, ffn=512, t=2, dtype="f32",
                    ranks=(0, 1), bias=True, bias_zero=True, backward=True,
                    note="X[32,128], W1[128,512], W2[512,128], both shards")

# Column-parallel linear only (page 3's layer, 768 -> 3072, t=4, rank 0),
# no activation, bf16 output.
COLUMN_768 = Workload("column_linear_768x3072_t4", T=4096, h=768, ffn=3072, t=4,
                      dtype="bf16", ranks=(0,), bias=True, bias_zero=True, gelu=False,
                      row_layer=False,
                      note="X[4096,768] (32x128 tokens), W_0[768,768], Y_0 bf16")

# GPT-3-shaped MLP shard, h=12288, ffn=49152, t=8, rank 0: forward and backward.
GPT3_SHARD = Workload("gpt3_mlp_shard_t8", T=2048, h=12288, ffn=49152, t=8,
                      dtype="bf16", ranks=(0,), bias=True, backward=True,
                      note="X[2048,12288], W1_0[12288,6144], W2_0[6144,12288]")

# Full-layer emulation: all 8 shards of h=8192, ffn=28672 in sequence, no bias,
# then the fp32 shard-sum of the 8 partial outputs.
FULL_LAYER_8 = Workload("full_layer_emulation_t8", T=4096, h=8192, ffn=28672, t=8,
                        dtype="bf16", ranks=tuple(range(8)), bias=False,
                        note="X[4096,8192], W1_r[8192,3584], W2_r[3584,8192], r=0..7")

ALL = {w.name: w for w in (TINY_F32, COLUMN_768, GPT3_SHARD, FULL_LAYER_8)}


@dataclass(frozen=True)
class AttnWorkload:
    """One rank's share of an attention block's two projections: the QKV
    projection split column-wise on head boundaries (rank r owns heads
    [r*H/t, (r+1)*H/t) of Q, K and V) and the output projection split
    row-wise (pages "PaddlePaddle张量并行", introduction; "张量并行实战",
    section "扩展思考：适配Transformer模块"; "Tensor Parallelism原理与实践",
    section 4.2).  The attention core between the two is not part of it."""
    name: str
    T: int           # tokens
    h: int           # hidden size
    heads: int       # attention heads
    t: int           # tensor-parallel degree
    dtype: str = "bf16"
    ranks: tuple = (0,)
    std_w: float = 0.02
    note: str = field(default="", compare=False)

    @property
    def w(self) -> int:
        """Columns of Q (or K, or V) a rank owns: heads/t heads of h/heads."""
        assert self.h % self.heads == 0 and self.heads % self.t == 0
        return self.h // self.t

    @property
    def qkv_width(self) -> int:
        return 3 * self.w

    def qkv_flops(self) -> float:
        return 2.0 * self.T * self.h * self.qkv_width

    def out_flops(self) -> float:
        return 2.0 * self.T * self.w * self.h


# Small attention shard for element-wise parity: 8 heads of 64, t=4.
ATTN_SMALL = AttnWorkload("attn_shard_small_t4", T=300, h=512, heads=8, t=4, ranks=(0, 1, 2, 3),
                          note="X[300,512], W_qkv_r[512,384], W_o_r[128,512]")

# GPT-3-shaped attention shard: 96 heads of 128, t=8 (12 heads per rank).
ATTN_GPT3 = AttnWorkload("gpt3_attn_shard_t8", T=2048, h=12288, heads=96, t=8, ranks=(3,),
                         note="X[2048,12288], W_qkv_r[12288,4608], W_o_r[1536,12288]")


def scaled(w: Workload, name: str, **kw) -> Workload:
    """A copy of ``w`` with some shape fields replaced (reduced parity cases)."""
    d = dict(w.__dict__)
    d.update(kw)
    d["name"] = name
    return Workload(**d)


def scaled_attn(aw: AttnWorkload, name: str, **kw) -> AttnWorkload:
    """A copy of ``aw`` with some shape fields replaced."""
    d = dict(aw.__dict__)
    d.update(kw)
    d["name"] = name
    if "ranks" not in kw:
        d["ranks"] = tuple(range(d["t"]))
    return AttnWorkload(**d)
