"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39, 0.0, -0.0], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_slices_are_deterministic_and_independent():
    w = synth.WORKLOADS["llama32k"]
    a = synth.keys(w, 0, 3, 256)
    b = synth.keys(w, 0, 3, 256)
    c = synth.keys(w, 0, 4, 256)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    full = synth.all_keys(w.replace(T=512), threads=4)
    assert np.array_equal(full[0, 3, :256], synth.keys(w.replace(T=512), 0, 3, 256))


def test_grid_and_dtype():
    w = synth.WORKLOADS["glm32k"]
    K = synth.keys(w, 0, 1, 1000)
    assert np.array_equal(np.rint(K.astype(np.float64) * 16) / 16, K.astype(np.float64))
    assert np.array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(K)), K)
    V = synth.values(w, 0, 1, 1000)
    assert np.array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(V)), V)
    t = synth.WORKLOADS["tiny"]
    assert synth.keys(t, 0, 0).dtype == np.float32


def test_planted_positions():
    for name in ["tiny", "llama32k", "qwen128k"]:
        w = synth.WORKLOADS[name]
        p = synth.planted_positions(w, 0)
        assert p[0] == 0 and np.all(np.diff(p) > 0) and p[-1] < w.T - w.W
        assert len(p) == w.planted_count()
    assert synth.WORKLOADS["tiny"].planted_count() == 4
    assert synth.WORKLOADS["llama32k"].planted_count() == 655


def test_budgets():
    assert synth.WORKLOADS["llama32k"].k == 1638
    assert synth.WORKLOADS["qwen128k"].k == 6553
    assert synth.WORKLOADS["tiny"].k == 8
