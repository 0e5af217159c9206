"""Pins of R = U . Hadamard . bit-reversal and of the clip thresholds."""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128])
def test_hadamard_matches_scipy_and_sylvester(d):
    H = oracle.hadamard_unnormalized(d)
    assert np.array_equal(H, scipy.linalg.hadamard(d))
    if d > 1:
        h = oracle.hadamard_unnormalized(d // 2)
        assert np.array_equal(H, np.block([[h, h], [h, -h]]))
    assert np.array_equal(H @ H.T, d * np.eye(d))


def test_bitrev_closed_form():
    assert [oracle.bitrev(i, 3) for i in range(8)] == [0, 4, 2, 6, 1, 5, 3, 7]
    for bits in (6, 7):
        n = 1 << bits
        assert all(oracle.bitrev(oracle.bitrev(i, bits), bits) == i for i in range(n))
        P = oracle.bitrev_permutation(n)
        assert np.array_equal(P, P.T) and np.array_equal(P @ P, np.eye(n))


def test_identity_u_gives_permuted_hadamard_exactly():
    for d in (64, 128):
        R = oracle.rotation(np.eye(d, dtype=np.float32))
        H = scipy.linalg.hadamard(d) / math.sqrt(d)
        bits = d.bit_length() - 1
        perm = [oracle.bitrev(j, bits) for j in range(d)]
        assert np.array_equal(R, H[:, perm].astype(np.float32))
    R = oracle.rotation(np.eye(64, dtype=np.float32))
    assert set(np.unique(R)) == {np.float32(-0.125), np.float32(0.125)}


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b_32k"])
def test_rotation_orthogonal(name):
    w = synth.WORKLOADS[name]
    for kind in (0, 1):
        U = synth.random_orthogonal_u(w, kind)
        R = oracle.rotation(U).astype(np.float64)
        for h in range(R.shape[0]):
            assert np.abs(R[h] @ R[h].T - np.eye(w.head_dim)).max() <= 2e-6
    # fp64 (no fp32 rounding of U or R): orthogonal to rounding level
    d = 128
    q = np.linalg.qr(np.random.default_rng(0).standard_normal((d, d)))[0]
    R64 = q @ oracle.hadamard_unnormalized(d) @ oracle.bitrev_permutation(d) / math.sqrt(d)
    assert np.abs(R64 @ R64.T - np.eye(d)).max() <= 1e-12


def test_rotation_matches_its_definition():
    # R = U . H . Pi / sqrt(d) evaluated without the oracle's own H and Pi:
    # scipy's Hadamard matrix, and Pi as the column permutation j -> bitrev(j)
    # by reversing j's binary digits.  U lies on the 2^-40 grid, so U . H is
    # exact in fp64 and both sides round the same two times.
    for name in ("tiny", "qwen3_8b_32k"):
        w = synth.WORKLOADS[name]
        d = w.head_dim
        bits = d.bit_length() - 1
        perm = [int(format(j, f"0{bits}b")[::-1], 2) for j in range(d)]
        U = synth.random_orthogonal_u(w, 0)
        R = oracle.rotation(U)
        for h in range(U.shape[0]):
            ref = ((U[h].astype(np.float64) @ scipy.linalg.hadamard(d))[:, perm] / math.sqrt(d)).astype(np.float32)
            assert np.array_equal(R[h], ref), (name, h)


def test_rotation_is_exact_on_the_grid():
    # with U on the 2^-40 grid, U.H.Pi has no rounding: a dense fp64 product in
    # a different association order gives the same bits
    w = synth.WORKLOADS["tiny"]
    U = synth.random_orthogonal_u(w, 0)[0].astype(np.float64)
    d = w.head_dim
    H, P = oracle.hadamard_unnormalized(d), oracle.bitrev_permutation(d)
    a = (U @ H) @ P
    b = U @ (H @ P)
    c = np.array([[math.fsum(U[i, k] * (H @ P)[k, j] for k in range(d)) for j in range(d)]
                  for i in range(4)])
    assert np.array_equal(a, b) and np.array_equal(a[:4], c)


def test_percentile_matches_numpy_linear():
    rng = np.random.default_rng(2)
    for n in (10, 101, 4096):
        v = np.sort(np.abs(rng.standard_normal(n) * 3).astype(np.float32))
        for pct in (0.0, 50.0, 99.0, 100.0):
            got = oracle.percentile_linear(v, pct)
            ref = np.percentile(v.astype(np.float64), pct, method="linear")
            assert abs(got - ref) <= 4e-16 * max(1.0, abs(ref))


def test_clip_thresholds_cover_99_percent():
    w = synth.WORKLOADS["tiny"]
    U = synth.random_orthogonal_u(w, 0)
    R = oracle.rotation(U)
    cal = synth.bf16_bits(synth.calibration_tokens(w, 0, 4096))
    c = oracle.clip_thresholds(cal[0], R[0])
    y = oracle.bf16_bits_to_f64(cal[0]) @ R[0].astype(np.float64)
    frac_inside = (np.abs(y) <= c[None, :]).mean(axis=0)
    assert np.all(np.abs(frac_inside - 0.99) <= 0.0015)
    assert np.all(2 * c / 3 < 65504)
