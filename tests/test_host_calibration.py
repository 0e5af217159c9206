"""The library's host eigensolver (oscar_calib_rotation) against the
oracle's eigenbasis: eigenvalues, the signed and rounded U, and R = U H Pi;
argument checks of the calibration calls that fail before any device work."""
import ctypes
import math

import numpy as np
import pytest

import bit_kv_cache_segment_amd as ok
import oracle
import synth


def _oracle_rotation(C):
    U, w = oracle.eigenbasis(C)
    Ug = oracle.rotation_grid(U)
    return oracle.rotation(Ug), Ug, w


@pytest.mark.parametrize("name,n", [("g4_d64", 512), ("g4_d128", 2048)])
def test_eigensolver_matches_oracle(name, n):
    d = 64 if name.endswith("64") else 128
    w = synth.Workload("calib_" + name, 60 + d, 1, 8, 2, d, d, 0, 0)
    q, k, v = synth.calibration_activations(w, n)
    qb, kb, vb = (synth.bf16_bits(x) for x in (q, k, v))
    covs = [oracle.query_covariance(qb, 2), oracle.value_covariance(qb, kb, vb, 1 / math.sqrt(d))]
    for C in covs:
        for h in range(2):
            C32 = C[h].astype(np.float32)       # both sides take the same fp32 matrix
            R, U, ev = ok.oscar_calib_rotation(C32)
            R_or, U_or, ev_or = _oracle_rotation(C32.astype(np.float64))
            assert np.allclose(ev, ev_or, rtol=0, atol=1e-9 * ev_or[0])
            # the Jacobi and LAPACK eigenvectors agree to ~1e-12; after the
            # rounding to fp32 nearly every entry is equal, the rest 1 ulp apart
            diff = np.abs(U.astype(np.float64) - U_or)
            assert np.all(diff <= np.abs(U_or) * 2.0**-23 + 2.0**-40), diff.max()
            assert (diff == 0).mean() > 0.99
            assert np.all(np.abs(R.astype(np.float64) - R_or) <= 2e-7)


def test_eigensolver_hand_worked():
    r = 1 / math.sqrt(2)
    R, U, ev = ok.oscar_calib_rotation(np.array([[2, 1], [1, 2]], dtype=np.float32))
    assert np.allclose(ev, [3, 1], atol=1e-15)
    assert np.array_equal(U, oracle.rotation_grid(np.array([[r, r], [r, -r]])))
    # a diagonal matrix: U is the permutation sorting the diagonal down, and
    # R that permutation times H Pi
    D = np.diag(np.array([1.0, 5.0, 3.0, 4.0], dtype=np.float32))
    R, U, ev = ok.oscar_calib_rotation(D)
    assert list(ev) == [5.0, 4.0, 3.0, 1.0]
    P = np.zeros((4, 4), dtype=np.float32)
    for c, i in enumerate([1, 3, 2, 0]):
        P[i, c] = 1
    assert np.array_equal(U, P)
    assert np.array_equal(R, ok.oscar_build_rotation(P))


def test_calibration_argument_errors():
    L = ok.lib()
    bad = [np.zeros((3, 3), np.float32), np.array([[np.nan, 0], [0, 1]], np.float32)]
    for C in bad:
        R = np.empty_like(C)
        rc = L.oscar_calib_rotation(C.shape[0], ok._np_ptr(C), None, ok._np_ptr(R), None)
        assert rc == ok.EINVAL
    C = np.eye(4, dtype=np.float32)
    assert L.oscar_calib_rotation(4, ok._np_ptr(C), None, None, None) == ok.EINVAL
    P = ctypes.c_void_p
    # n = 0 does nothing; shape and alignment checks come before any device work
    assert L.oscar_calib_covariance(0, 8, 2, 128, None, None, None, 1.0, None, None, None, 0, None) == ok.OK
    assert L.oscar_calib_covariance(4, 8, 2, 96, P(16), P(16), P(16), 1.0, P(16), P(16), P(16), 1 << 20,
                                    None) == ok.EINVAL
    assert L.oscar_calib_covariance(4, 8, 3, 128, P(16), P(16), P(16), 1.0, P(16), P(16), P(16), 1 << 20,
                                    None) == ok.EINVAL
    assert L.oscar_calib_attention(4, 8, 2, 128, P(16), P(24), P(16), 1.0, P(16), None) == ok.EINVAL  # k misaligned
    assert L.oscar_calib_attention(4, 8, 2, 128, P(16), P(16), P(16), float("nan"), P(16), None) == ok.EINVAL
    assert L.oscar_calib_covariance(4, 8, 2, 128, P(16), P(16), P(16), 1.0, P(16), P(16), P(16), 100,
                                    None) == ok.EINVAL                                          # workspace
    assert ok.oscar_calib_workspace_bytes(10, 8, 128) == 10 * 8 * 128 * 4


def test_lloyd_max_fit_matches_oracle():
    # the library's offline fit and the oracle's, each from the same tokens,
    # rotation and thresholds: identical codebooks
    import harness
    for name in ("tiny", "qwen3_8b_32k"):
        w = synth.WORKLOADS[name]
        RK, RV, cK, cV = harness.tables(w, n_cal=1024)
        for kind, (R, clip) in enumerate(((RK, cK), (RV, cV))):
            cal = synth.bf16_bits(synth.calibration_tokens(w, kind, 1024))
            for h in range(min(2, w.num_kv_heads)):
                lib_L = ok.oscar_lloyd_max_codebook(cal[h], R[h], clip[h], w.group_size)
                or_L = oracle.lloyd_max_codebook(oracle.normalized_values(cal[h], R[h], clip[h], w.group_size))
                assert list(lib_L) == list(or_L), (name, kind, h, lib_L, or_L)
                assert lib_L[0] < lib_L[1] < lib_L[2] < lib_L[3]


def test_lloyd_max_pool_calls_on_host_only_pools():
    cfg = ok.make_config(4, 8, 2, 64, 64, 50, 10, 1, ok.POOL_HOST_ONLY | ok.POOL_LLOYD_MAX)
    p = ok.Pool(cfg, None, None, None, None)
    with pytest.raises(ok.OscarError) as ei:
        p.prefill_len(0, 400)                 # no codebook yet
    assert ei.value.code == ok.EINVAL and "codebook" in str(ei.value)
    bad = np.array([[10, 5, 20, 30]] * 2, np.uint8)
    good = np.array([[40, 79, 114, 154]] * 2, np.uint8)
    with pytest.raises(ok.OscarError):
        p.set_codebook(bad, good)             # not non-decreasing
    p.set_codebook(good, good)
    p.prefill_len(0, 400)
    p.append([0], None, None)
    with pytest.raises(ok.OscarError):
        p.set_codebook(good, good)            # a sequence is not empty
    p.release(0)
    p.set_codebook(good, good)
    with pytest.raises(ok.OscarError):        # excludes the BF16 history
        ok.Pool(ok.make_config(4, 8, 2, 64, 64, 50, 10, 1, ok.POOL_HOST_ONLY | ok.POOL_LLOYD_MAX | 4),
                None, None, None, None)
    q = ok.Pool(ok.make_config(4, 8, 2, 64, 64, 50, 10, 1, ok.POOL_HOST_ONLY), None, None, None, None)
    with pytest.raises(ok.OscarError):        # not a Lloyd-Max pool
        q.set_codebook(good, good)
