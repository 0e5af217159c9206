"""Pins of the oracle's calibration: the covariances against hand-worked
cases and closed forms, the eigenbasis against hand-worked cases and its
defining invariants, and the whole offline step against a planted
covariance."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _num(t):
    return math.log(3.0) if t == "ln3" else float(Fraction(t))


def _bf16(x):
    """uint16 bf16 bits of values that bf16 holds exactly."""
    a = np.asarray(x, dtype=np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), x
    return (bits >> 16).astype(np.uint16)


def _to_bf16(x):
    """uint16 bf16 bits of x, rounded to nearest even."""
    return synth.bf16_bits(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16))


def _cases():
    out, cur = [], None
    for ln in open(os.path.join(HERE, "golden", "calibration_cases.txt")):
        ln = ln.strip()
        if not ln or ln.startswith("#"):
            continue
        if ln.startswith("case "):
            _, kind, *kv = ln.split()
            cur = {"kind": kind, **{a: int(b) for a, b in (x.split("=") for x in kv)}, "rows": [], "C": {}}
            continue
        if ln == "end":
            out.append(cur)
            continue
        lhs, rhs = (x.strip() for x in ln.split("="))
        if lhs == "scale":
            cur["scale"] = _num(rhs)
        elif lhs.startswith("C"):
            cur["C"][int(lhs.split()[1])] = np.array([[_num(t) for t in r.split()] for r in rhs.split(";")])
        else:
            name, t, h = lhs.split()
            cur["rows"].append((name, int(t), int(h), [_num(x) for x in rhs.split()]))
    return out


CASES = _cases()


@pytest.mark.parametrize("i", range(len(CASES)))
def test_covariance_hand_worked(i):
    c = CASES[i]
    d = len(c["rows"][0][3])
    arr = {"q": np.zeros((c["n"], c["hq"], d), np.float32), "k": np.zeros((c["n"], c["hkv"], d), np.float32),
           "v": np.zeros((c["n"], c["hkv"], d), np.float32)}
    for name, t, h, vals in c["rows"]:
        arr[name][t, h] = vals
    if c["kind"] == "query_covariance":
        got = oracle.query_covariance(_bf16(arr["q"]), c["hkv"])
    else:
        got = oracle.value_covariance(_bf16(arr["q"]), _bf16(arr["k"]), _bf16(arr["v"]), c["scale"])
    assert got.shape == (c["hkv"], d, d)
    for kv, want in c["C"].items():
        assert np.allclose(got[kv], want, rtol=1e-12, atol=1e-12), (kv, got[kv], want)


def test_value_covariance_uniform_scores_is_prefix_means():
    # equal logits in every row (zero queries): S V is the running mean of V
    rng = np.random.default_rng(0)
    n, d = 40, 8
    v = rng.standard_normal((n, 1, d)).astype(np.float32)
    k = rng.standard_normal((n, 1, d)).astype(np.float32)
    vb, kb = _to_bf16(v), _to_bf16(k)
    V = oracle.bf16_bits_to_f64(vb)[:, 0]
    means = np.cumsum(V, axis=0) / np.arange(1, n + 1)[:, None]
    got = oracle.value_covariance(np.zeros((n, 2, d), np.uint16), kb, vb, 0.7)
    assert np.allclose(got[0], 2 * means.T @ means, rtol=1e-12, atol=1e-10)


def test_value_covariance_sharp_scores_pick_the_best_key():
    # a very large scale turns each row of S into the indicator of the
    # best visible key: S V selects rows of V
    rng = np.random.default_rng(1)
    n, d = 24, 4
    q = rng.standard_normal((n, 1, d)).astype(np.float32)
    k = rng.standard_normal((n, 1, d)).astype(np.float32)
    v = rng.standard_normal((n, 1, d)).astype(np.float32)
    qb, kb, vb = (_to_bf16(x) for x in (q, k, v))
    Q, K, V = (oracle.bf16_bits_to_f64(x)[:, 0] for x in (qb, kb, vb))
    best = [int(np.argmax(K[: t + 1] @ Q[t])) for t in range(n)]
    gap = min(np.diff(np.sort(K[: t + 1] @ Q[t]))[-1] for t in range(1, n))
    sel = V[best]
    got = oracle.value_covariance(qb, kb, vb, 80.0 / gap)   # others weigh < e^-80
    assert np.allclose(got[0], sel.T @ sel, rtol=1e-9, atol=1e-9)


def test_eigenbasis_hand_worked():
    U, w = oracle.eigenbasis(np.diag([1.0, 5.0, 3.0]))
    assert np.allclose(w, [5, 3, 1])
    assert np.array_equal(U, np.array([[0, 0, 1], [1, 0, 0], [0, 1, 0]], dtype=float))
    # [[2,1],[1,2]]: eigenvalues 3, 1 with (1,1)/sqrt2 and (1,-1)/sqrt2 (the
    # first of two equal magnitudes is made positive)
    U, w = oracle.eigenbasis(np.array([[2.0, 1.0], [1.0, 2.0]]))
    r = 1 / math.sqrt(2)
    assert np.allclose(w, [3, 1], atol=1e-14)
    assert np.allclose(U, [[r, r], [r, -r]], atol=1e-14)
    # a negative largest entry is flipped
    U, w = oracle.eigenbasis(np.array([[4.0, 0.0], [0.0, 1.0]]) - 0)
    assert np.array_equal(U, np.eye(2))


def test_eigenbasis_invariants():
    rng = np.random.default_rng(2)
    A = rng.standard_normal((64, 200))
    C = A @ A.T
    U, w = oracle.eigenbasis(C)
    assert np.all(np.diff(w) <= 0)
    assert np.allclose(U.T @ U, np.eye(64), atol=1e-12)
    assert np.allclose(U.T @ C @ U, np.diag(w), atol=1e-9 * w[0])
    for c in range(64):
        j = np.argmax(np.abs(U[:, c]))
        assert U[j, c] > 0


def test_rotation_grid():
    rng = np.random.default_rng(3)
    U = rng.standard_normal((16, 16)) * 0.3
    U[0, :3] = [3 * 2.0**-42, 2.0**-42, -5 * 2.0**-41]   # below 2^-17: off the grid in fp32
    G = oracle.rotation_grid(U).astype(np.float64)
    assert np.array_equal(G * 2.0**40, np.round(G * 2.0**40))
    assert np.all(np.abs(G - U) <= np.abs(U) * 2.0**-24 + 2.0**-41)
    assert list(G[0, :3]) == [2.0**-40, 0.0, -2 * 2.0**-40]   # nearest, ties to even


def test_planted_query_covariance_recovers_its_axes():
    # queries z diag(sigma) B^T: the eigenbasis of Q^T Q is B (up to the
    # column signs the convention fixes) with eigenvalues ~ n sigma^2
    rng = np.random.default_rng(4)
    n, d = 20000, 16
    B, _ = np.linalg.qr(rng.standard_normal((d, d)))
    sigma = 2.0 ** (-np.arange(d) / 3.0)
    q = (rng.standard_normal((n, d)) * sigma) @ B.T
    qb = _to_bf16(q.astype(np.float32)[:, None, :])
    U, w = oracle.eigenbasis(oracle.query_covariance(qb, 1)[0])
    for c in range(6):
        assert abs(U[:, c] @ B[:, c]) > 0.995, c
    assert np.allclose(w[:6] / n, sigma[:6] ** 2, rtol=0.1)


def test_calibrate_layer_gives_orthogonal_rotations():
    rng = np.random.default_rng(5)
    n, Hq, Hkv, d = 256, 4, 2, 64
    q, k, v = (_to_bf16(rng.standard_normal((n, H, d)).astype(np.float32))
               for H in (Hq, Hkv, Hkv))
    RK, RV, cK, cV = oracle.calibrate_layer(q, k, v, 1 / 8)
    for R in (*RK, *RV):
        assert np.allclose(R.astype(np.float64).T @ R, np.eye(d), atol=1e-6)
    assert cK.shape == (Hkv, d) and np.all(cK > 0) and np.all(cV > 0)
    # R_K of kv head 0 is U . H . Pi with U the query eigenbasis of heads 0, 1
    U, _ = oracle.eigenbasis(oracle.query_covariance(q, Hkv)[0])
    assert np.array_equal(RK[0], oracle.rotation(oracle.rotation_grid(U)))
