"""GPU parity of the calibration statistics: S V (oscar_calib_attention)
and the covariances Q^T Q and V^T S^T S V (oscar_calib_covariance) against
the oracle's fp64 definitions, over several shapes and ragged lengths; and
the whole offline step (device covariances, host eigenbasis, rotation, clip
thresholds) feeding a pool whose decode matches the oracle's pool built
from the oracle's own calibration.

Tolerances: S V is computed in fp32 (logits, exponentials, sums), so each
output row carries a relative error of a few fp32 ulps times the
accumulation depth: 1e-5 row-relative.  The Gram matrices sum n fp32
products (exact for the bf16 query, rounded for S V) in four interleaved
fp32 accumulators: error <= about (n/4) 2^-24 sum|x_i x_j| in the worst
case, far less in practice; 2e-5 of the largest entry (a diagonal one)."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_segment_amd as ok
import harness
import oracle
import synth
from gpu_common import TOL

pytestmark = pytest.mark.gpu

SHAPES = {"g4_d128": (8, 2, 128), "g1_d64": (4, 4, 64), "g8_d128": (16, 2, 128)}
LENGTHS = [1, 7, 64, 333, 1000]


def _workload(name):
    Hq, Hkv, d = SHAPES[name]
    return synth.Workload("calib_" + name, 70 + list(SHAPES).index(name), 1, Hq, Hkv, d, d, 0, 0)


def _inputs(w, n):
    q, k, v = synth.calibration_activations(w, n)
    return (q, k, v), tuple(synth.bf16_bits(x) for x in (q, k, v))


@pytest.mark.parametrize("shape", list(SHAPES))
def test_scores_times_values(shape):
    w = _workload(shape)
    scale = 1 / math.sqrt(w.head_dim)
    for n in LENGTHS:
        (q, k, v), (qb, kb, vb) = _inputs(w, n)
        out = ok.oscar_calib_attention(q.cuda().view(torch.uint16), k.cuda().view(torch.uint16),
                                       v.cuda().view(torch.uint16), scale)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()
        Q, K, V = (oracle.bf16_bits_to_f64(x) for x in (qb, kb, vb))
        g = w.num_q_heads // w.num_kv_heads
        worst = 0.0
        for h in range(w.num_q_heads):
            ref = oracle.causal_scores(Q[:, h], K[:, h // g], scale) @ V[:, h // g]
            worst = max(worst, oracle.row_rel_err(got[:, h], ref))
        assert worst <= 1e-5, (n, worst)


@pytest.mark.parametrize("shape", list(SHAPES))
def test_covariances(shape):
    w = _workload(shape)
    scale = 1 / math.sqrt(w.head_dim)
    Hkv, d = w.num_kv_heads, w.head_dim
    for n in LENGTHS:
        (q, k, v), (qb, kb, vb) = _inputs(w, n)
        ck = torch.zeros((Hkv, d, d), dtype=torch.float32, device="cuda")
        cv = torch.zeros_like(ck)
        ok.oscar_calib_covariance(*(x.cuda().view(torch.uint16) for x in (q, k, v)), scale, ck, cv)
        torch.cuda.synchronize()
        for got, ref in ((ck, oracle.query_covariance(qb, Hkv)), (cv, oracle.value_covariance(qb, kb, vb, scale))):
            got = got.double().cpu().numpy()
            for h in range(Hkv):
                err = np.abs(got[h] - ref[h]).max() / np.abs(ref[h]).max()
                assert err <= 2e-5, (n, h, err)


def test_covariances_accumulate_over_sequences():
    w = _workload("g4_d128")
    scale = 1 / math.sqrt(w.head_dim)
    Hkv, d = w.num_kv_heads, w.head_dim
    ck = torch.zeros((Hkv, d, d), dtype=torch.float32, device="cuda")
    cv = torch.zeros_like(ck)
    refk = np.zeros((Hkv, d, d))
    refv = np.zeros((Hkv, d, d))
    for n in (200, 57):        # two sequences: the first 200 and the first 57 tokens
        (q, k, v), (qb, kb, vb) = _inputs(w, n)
        ok.oscar_calib_covariance(*(x.cuda().view(torch.uint16) for x in (q, k, v)), scale, ck, cv)
        refk += oracle.query_covariance(qb, Hkv)
        refv += oracle.value_covariance(qb, kb, vb, scale)
    torch.cuda.synchronize()
    for got, ref in ((ck, refk), (cv, refv)):
        got = got.double().cpu().numpy()
        assert np.abs(got - ref).max() / np.abs(ref).max() <= 2e-5


def test_calibration_end_to_end():
    # the offline step on a Qwen3-8B-shaped layer from one calibration
    # sequence of 2048 tokens: device covariances, host eigenbasis.  What is
    # unique is compared: the eigenvalues, and the eigenvectors of eigenvalues
    # well apart from their neighbours; near-equal eigenvalues leave their
    # eigenvectors free to mix within the pair, so for all of U the test
    # checks that it diagonalizes the oracle's fp64 covariance.  Expected
    # size of the differences: the fp32 covariance is ~1e-6 (relative to the
    # largest eigenvalue) from the fp64 one; an eigenvector moves by that over
    # its eigenvalue gap.
    w0 = synth.WORKLOADS["qwen3_8b_32k"]
    w = synth.Workload("calib_layer", 80, 2, w0.num_q_heads, w0.num_kv_heads, w0.head_dim, w0.group_size, 0, 0)
    Hkv, d, n = w.num_kv_heads, w.head_dim, 2048
    scale = 1 / math.sqrt(d)
    (q, k, v), (qb, kb, vb) = _inputs(w, n)
    ck = torch.zeros((Hkv, d, d), dtype=torch.float32, device="cuda")
    cv = torch.zeros_like(ck)
    ok.oscar_calib_covariance(*(x.cuda().view(torch.uint16) for x in (q, k, v)), scale, ck, cv)
    torch.cuda.synchronize()
    refs = (oracle.query_covariance(qb, Hkv), oracle.value_covariance(qb, kb, vb, scale))
    separated = 0
    for C_gpu, C_or in zip((ck.cpu().numpy(), cv.cpu().numpy()), refs):
        for h in range(Hkv):
            R, U, ev = ok.oscar_calib_rotation(C_gpu[h])
            U_or, ev_or = oracle.eigenbasis(C_or[h])
            top = ev_or[0]
            assert np.abs(ev - ev_or).max() <= 1e-5 * top
            U64 = U.astype(np.float64)
            assert np.abs(C_or[h] @ U64 - U64 * ev[None, :]).max() <= 2e-5 * top
            assert np.allclose(U64.T @ U64, np.eye(d), atol=1e-6)
            gap = np.minimum(np.r_[np.inf, -np.diff(ev_or)], np.r_[-np.diff(ev_or), np.inf])
            for c in np.nonzero(gap > 1e-2 * top)[0]:
                assert U64[:, c] @ U_or[:, c] >= 1 - 1e-6, (h, c)
                separated += 1
            assert np.array_equal(R, ok.oscar_build_rotation(U))
    assert separated >= 2 * Hkv
