"""Oracle pins: the widely-linear split and its inverse (Theorem 1, "Step 1")."""
import numpy as np

import oracle
import pins
import workloads


def test_split_identity_random():
    pins.check_split_identity(oracle.split)


def test_split_identity_tiny_workload():
    """The tiny 256x256 workload: U x + W conj(x) equals R x~ to 1e-12."""
    R = workloads.TINY.weight()
    U, W = oracle.split(R)
    x = workloads.activations(1, 256, workloads.TINY_X_SEED, "f32").values.astype(np.float64)
    xc = x[:, :128] + 1j * x[:, 128:]
    y = xc @ U.T + np.conj(xc) @ W.T
    assert pins.rel_l2(np.concatenate([y.real, y.imag], axis=1), x @ R.astype(np.float64).T) <= 1e-12


def test_split_hand_worked():
    pins.check_split_hand(oracle.split)


def test_split_unique():
    pins.check_split_unique(oracle.split)


def test_unsplit_reconstructs_exactly():
    """R is rebuilt bit for bit from (U, W) whenever the fp64 sums are exact, which holds for
    fp32 entries of similar magnitude (the pages call the map lossless)."""
    for seed in (0, 1, 2):
        R = workloads.weight(64, 96, seed)
        U, W = oracle.split(R)
        assert np.array_equal(oracle.unsplit(U, W), R.astype(np.float64))
    # dyadic integers: always exact
    rng = np.random.default_rng(3)
    R = rng.integers(-1000, 1000, size=(10, 30)).astype(np.float32)
    assert np.array_equal(oracle.unsplit(*oracle.split(R)), R.astype(np.float64))


def test_split_rejects_odd_shape():
    import pytest
    with pytest.raises(AssertionError):
        oracle.split(np.zeros((3, 4), dtype=np.float32))
