"""The seeded input generator: SplitMix64 stream and Box-Muller normals."""
import math

import numpy as np
import torch

import moe_synth as ms


def test_splitmix64_reference_sequence():
    # SplitMix64 seeded with 0: the first three outputs of the published generator
    z = ms.raw_draws(0, 0, 3, "cpu")
    got = [int(v) & ms.MASK64 for v in z]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_tensor_hash_matches_python_ints():
    key = ms.stream_key(0, ms.TAGS["w1"])
    idx = [0, 1, 17, 12345, 2 ** 31 + 7]
    for i in idx:
        t = int(ms.raw_draws(key, i, 1, "cpu")[0]) & ms.MASK64
        assert t == ms.mix64_int((key + (i + 1) * ms.GAMMA) & ms.MASK64)


def test_normals_moments_and_determinism():
    v = ms.normals(0, 1, 400_000, "cpu")
    assert abs(v.mean().item()) < 0.01 and abs(v.std().item() - 1.0) < 0.01
    assert torch.equal(v[:1001], ms.normals(0, 1, 1001, "cpu"))   # prefix-stable
    assert not torch.equal(v[:1000], ms.normals(0, 2, 1000, "cpu"))  # per-tag streams differ


def test_layer_shapes_and_scales():
    cfg = ms.CONFIGS["skew"]
    L = ms.make_layer(cfg, "cpu", T=256, want=("x", "w_router", "bias", "x_prev"))
    assert L["x"].shape == (256, cfg.d) and L["x"].dtype == torch.bfloat16
    assert L["w_router"].shape == (cfg.E, cfg.d)
    assert L["bias"][0].item() == 3.0 and (L["bias"][1:] == 0).all()
    assert abs(L["w_router"].float().std().item() - 1 / math.sqrt(cfg.d)) < 0.01 / math.sqrt(cfg.d) * 10
    t = ms.CONFIGS["tiny"]
    Lt = ms.make_layer(t, "cpu")
    assert Lt["w2"].shape == (t.E, t.d, t.d_ff) and Lt["w1"].shape == (t.E, t.d_ff, t.d)
    assert Lt["x"].dtype == torch.float32 and Lt["bias"] is None
