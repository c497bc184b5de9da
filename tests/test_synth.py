"""The seeded input generator: reproducible bytes, right shapes and spread."""
import hashlib

import torch

from tensor_transformer_layer_columnparallel_amd import configs, synth


def _digest(d):
    h = hashlib.sha256()
    for k in sorted(d):
        v = d[k]
        vs = [v[r] for r in sorted(v)] if isinstance(v, dict) else [v]
        for x in vs:
            if x is not None:
                h.update(x.view(torch.uint8).numpy().tobytes() if x.dtype == torch.bfloat16
                         else x.numpy().tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes_other_seed_other_bytes():
    w = configs.TINY_F32
    a, b = synth.make_inputs(w, seed=0), synth.make_inputs(w, seed=0)
    c = synth.make_inputs(w, seed=1)
    assert _digest(a) == _digest(b) != _digest(c)


def test_shapes_dtypes_and_spread():
    w = configs.scaled(configs.GPT3_SHARD, "small", T=256, h=512, ffn=2048)
    d = synth.make_inputs(w)
    assert d["X"].shape == (256, 512) and d["X"].dtype == torch.bfloat16
    assert d["W1"][0].shape == (512, 256) and d["W2"][0].shape == (256, 512)
    assert d["b1"][0].shape == (256,) and d["dZ"].shape == (256, 512)
    assert abs(d["X"].float().std().item() - 1.0) < 0.02
    assert abs(d["W1"][0].float().std().item() - 0.02) < 0.001


def test_shard_values_do_not_depend_on_other_ranks():
    w = configs.FULL_LAYER_8
    small = configs.scaled(w, "s", T=16, h=64, ffn=256)
    all_r = synth.make_inputs(small)
    only3 = synth.make_inputs(small, ranks=(3,))
    assert torch.equal(all_r["W1"][3], only3["W1"][3])
    assert torch.equal(all_r["W2"][3], only3["W2"][3])
    assert all_r["b1"][3] is None


def test_tiny_f32_zero_bias_and_fp32():
    d = synth.make_inputs(configs.TINY_F32)
    assert d["X"].dtype == torch.float32 and set(d["W1"]) == {0, 1}
    assert torch.count_nonzero(d["b1"][0]) == 0
