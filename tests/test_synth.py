"""The seeded input recipe: determinism, shapes, masking statistics, bf16
rounding.  CPU only."""

import numpy as np
import pytest

from lm_head_linear_bf16_amd import synth


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0],
                                 dtype=np.float32)])
    bits = synth.f32_to_bf16_bits(x)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, tb)
    back = synth.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_targets_recipe_tiny():
    w = synth.WORKLOADS["tiny"]
    t, p = synth.targets(w)
    t2, p2 = synth.targets(w)
    np.testing.assert_array_equal(t, t2)
    np.testing.assert_array_equal(p, p2)
    assert t.shape == (128,) and t.dtype == np.int64 and p.dtype == np.float32
    ok = t != -100
    assert np.all((t[ok] >= 0) & (t[ok] < w.V))
    # p_mask is constant per sequence and within [0.05, 1)
    for b in range(w.B):
        seg = p[b * w.L:(b + 1) * w.L]
        assert np.all(seg == seg[0]) and 0.05 <= seg[0] < 1.0


def test_masked_fraction_and_block_padding():
    w = synth.WORKLOADS["block"]
    t, p = synth.targets(w)
    assert t.shape == (w.N,)
    pos = np.arange(w.N) % w.L
    pad = pos >= w.L - 154
    assert np.all(t[pad] == -100) and np.all(p[pad] == 1.0)
    # p_mask constant within each 4-token block (outside padding)
    pb = p.reshape(-1, 4)
    full = ~pad.reshape(-1, 4).any(axis=1)
    assert np.all(pb[full] == pb[full][:, :1])
    # masked fraction among non-padding rows ~ E[t] = 0.525
    frac = np.mean(t[~pad] != -100)
    assert 0.49 < frac < 0.56
    assert w.total == 0 and synth.WORKLOADS["headline"].total == 8192


def test_headline_and_shard_shapes():
    w = synth.WORKLOADS["headline"]
    assert (w.N, w.H, w.V, w.label_smoothing, w.logit_scale) == (8192, 2560, 151936, 0.1, 0.5)
    s = synth.WORKLOADS["shard"]
    assert (s.N, s.H, s.V_local, s.vocab_start) == (32768, 5120, 18992, 56976)
    t, _ = synth.targets(s)
    ok = t != -100
    inshard = (t >= s.vocab_start) & (t < s.vocab_start + s.V_local) & ok
    assert 0.10 < inshard.sum() / ok.sum() < 0.15


def test_weight_shards_concatenate():
    w = synth.custom("small_shard", 1, 16, 8, 40, shards=4, shard_k=1)
    full = synth.weight(w)
    assert full.values.shape == (40, 8) and full.bits.dtype == np.uint16
    for k in range(4):
        np.testing.assert_array_equal(synth.weight(w, shard=k).bits, full.bits[10 * k:10 * (k + 1)])


def test_fp32_workload_has_no_bits():
    w = synth.WORKLOADS["tiny"]
    h = synth.hidden(w)
    assert h.bits is None and h.values.dtype == np.float32 and h.values.shape == (128, 64)
    W = synth.weight(w)
    assert abs(W.values.std() - 0.125) < 0.01
