"""The seeded generators: bf16 rounding agrees with torch's, shapes and seeds are stable."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    v = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * np.float32(3.0)
    v[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact ties
    ours = workloads.f32_to_bf16_bits(v)
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(workloads.bf16_bits_to_f32(ours),
                          torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_weights_are_seeded_and_scaled():
    a = workloads.weight(8, 16, 5)
    b = workloads.weight(8, 16, 5)
    assert a.dtype == np.float32 and np.array_equal(a, b)
    big = workloads.weight(512, 512, 7)
    assert abs(float(big.std()) - 0.02) < 1e-3


def test_outliers_fraction():
    base = workloads.weight(1024, 512, 9)
    out = workloads.weight(1024, 512, 9, outlier_seed=10)
    frac = float(np.mean(base != out))
    assert 0.008 < frac < 0.012
