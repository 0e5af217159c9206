"""Pins of the oracle's attention: brute force on tiny inputs, the textbook
routine, the online-softmax merge, and the rotation conventions."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth


def _brute(q, K, V, scale):
    T, d = K.shape
    logits = [scale * sum(q[c] * K[t][c] for c in range(d)) for t in range(T)]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    tot = math.fsum(w)
    return np.array([math.fsum(w[t] * V[t][c] for t in range(T)) / tot for c in range(d)])


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(1)
    for T in (1, 2, 7):
        q, K, V = rng.standard_normal(4), rng.standard_normal((T, 4)), rng.standard_normal((T, 4))
        got = oracle.attention(q, K, V, 0.5)
        assert np.abs(got - _brute(q, K, V, 0.5)).max() <= 1e-13


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(2)
    q, K, V = rng.standard_normal(64), rng.standard_normal((300, 64)), rng.standard_normal((300, 64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
        torch.from_numpy(V)[None, None], scale=0.125)[0, 0, 0].numpy()
    assert np.abs(oracle.attention(q, K, V, 0.125) - ref).max() <= 1e-12


def test_one_token_gives_v():
    v = np.array([[1.5, -2.0, 3.25, 0.0]])
    assert np.array_equal(oracle.attention(np.ones(4), np.ones((1, 4)), v, 1.0), v[0])


@pytest.mark.parametrize("cuts", [(3,), (0, 5), (1, 2, 9), (10,)])
def test_merge_of_partials_equals_single_softmax(cuts):
    rng = np.random.default_rng(3)
    T = 10
    q, K, V = rng.standard_normal(8), rng.standard_normal((T, 8)) * 3, rng.standard_normal((T, 8))
    edges = [0, *cuts, T]
    parts = [oracle.partial_attention(q, K[a:b], V[a:b], 0.7) for a, b in zip(edges[:-1], edges[1:])]
    m, l, acc = oracle.merge_partials(parts)
    assert np.abs(acc / l - oracle.attention(q, K, V, 0.7)).max() <= 1e-12


def test_derotation_convention():
    # history stored as y = x R (row vectors) decodes with y R^T; with an
    # exactly orthogonal fp64 R and no quantization that is the identity, and
    # attention over such a pool equals attention over the raw tokens.
    rng = np.random.default_rng(4)
    d = 64
    R = np.linalg.qr(rng.standard_normal((d, d)))[0]
    K = rng.standard_normal((50, d))
    V = rng.standard_normal((50, d))
    q = rng.standard_normal(d)
    Kd = (K @ R) @ R.T
    Vd = (V @ R) @ R.T
    assert np.abs(oracle.attention(q, Kd, Vd, 0.125) - oracle.attention(q, K, V, 0.125)).max() <= 1e-12
    # the attention that the decode path computes in the rotated basis (q R,
    # then acc R^T) is the same quantity
    Kr, Vr = K @ R, V @ R
    w = np.exp(0.125 * (Kr @ (q @ R)) - (0.125 * (Kr @ (q @ R))).max())
    rot = ((w @ Vr) / w.sum()) @ R.T
    assert np.abs(rot - oracle.attention(q, K, V, 0.125)).max() <= 1e-12


def test_history_decodes_back_in_the_original_basis():
    # A history token x is stored as codes of y = clip(x R); it decodes to
    # deq . R^T.  R is orthogonal to ~2e-6, so the decoded token lies within
    # |deq - y| (2-norm) of clip(x R) . R^T, computed here directly.
    w = synth.WORKLOADS["tiny"]
    L = w.len_lo
    k = synth.bf16_bits(synth.kv_tokens(w, 0, 0, 0, L))
    v = synth.bf16_bits(synth.kv_tokens(w, 1, 0, 0, L))
    RK, RV = oracle.rotation(synth.random_orthogonal_u(w, 0)), oracle.rotation(synth.random_orthogonal_u(w, 1))
    cK = np.full((w.num_kv_heads, w.head_dim), 2.5, dtype=np.float32)
    cV = np.full((w.num_kv_heads, w.head_dim), 2.5, dtype=np.float32)
    st = oracle.build_sequence(k, v, RK, RV, cK, cV, w.group_size, heads=[0])
    _, hist, _ = oracle.segments(L)
    x = oracle.bf16_bits_to_f64(k[hist.start:hist.stop, 0])
    y = np.clip(x @ RK[0].astype(np.float64), -2.5, 2.5)
    ref = y @ RK[0].astype(np.float64).T
    pk, s16, z16 = st.hist[("K", 0)]
    deq = oracle.dequantize(pk, s16, z16, w.group_size)
    err = np.linalg.norm(st.K[hist.start:hist.stop, 0] - ref, axis=1)
    bound = np.linalg.norm(deq - y, axis=1) * (1 + 1e-4) + 1e-4
    assert np.all(err <= bound)


def test_tiny_workload_sequence_end_to_end():
    w = synth.WORKLOADS["tiny"]
    L = w.len_lo
    k = synth.bf16_bits(synth.kv_tokens(w, 0, 0, 0, L))
    v = synth.bf16_bits(synth.kv_tokens(w, 1, 0, 0, L))
    RK, RV = oracle.rotation(synth.random_orthogonal_u(w, 0)), oracle.rotation(synth.random_orthogonal_u(w, 1))
    cK = np.stack([oracle.clip_thresholds(c, RK[h]) for h, c in enumerate(synth.bf16_bits(synth.calibration_tokens(w, 0, 4096)))])
    cV = np.stack([oracle.clip_thresholds(c, RV[h]) for h, c in enumerate(synth.bf16_bits(synth.calibration_tokens(w, 1, 4096)))])
    st = oracle.build_sequence(k, v, RK, RV, cK, cV, w.group_size)
    # sink and recent are the raw bf16 tokens; history differs from raw
    sink, hist, recent = oracle.segments(L)
    raw = oracle.bf16_bits_to_f64(k)
    assert np.array_equal(st.K[:64], raw[:64]) and np.array_equal(st.K[hist.stop:], raw[hist.stop:])
    assert len(hist) == 704 and not np.array_equal(st.K[hist.start:hist.stop], raw[hist.start:hist.stop])
    # history error in the rotated basis obeys the codec bound elementwise
    pk, s16, z16 = st.hist[("K", 0)]
    y = np.empty((704, w.head_dim), dtype=np.float32)
    oracle.lib().oracle_rotate_many(oracle._ptr(np.ascontiguousarray(k[hist.start:hist.stop, 0])), 704,
                                    w.head_dim, oracle._ptr(np.ascontiguousarray(RK[0])), oracle._ptr(y))
    y = np.clip(y, -cK[0], cK[0]).astype(np.float64)
    deq = oracle.dequantize(pk, s16, z16, w.group_size)
    assert np.all(np.abs(deq - y) <= np.repeat(oracle.f16_table()[s16], w.group_size, -1) * 0.5001 + 1e-3)
    q = synth.bf16_bits(synth.queries(w, 0))[0]
    out = oracle.attend_sequence(st, q, 1 / math.sqrt(w.head_dim))
    assert np.all(np.isfinite(out))
    # identical queries in a GQA group give identical rows
    q2 = q.copy()
    q2[1] = q2[0]
    out2 = oracle.attend_sequence(st, q2, 1 / math.sqrt(w.head_dim))
    assert np.array_equal(out2[0], out2[1])


def _golden_cases(name):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    cases, cur = [], {}
    with open(path) as f:
        for ln in f:
            ln = ln.strip()
            if not ln or ln.startswith("#"):
                continue
            key, val = ln.split(":", 1)
            cur[key] = val.strip()
            if key == "expect":
                cases.append(cur)
                cur = {}
    return cases


def _rows(text):
    return np.array([[float(x) for x in r.split()] for r in text.split("|")])


def test_row_relative_error_hand_worked():
    # the parity metric of every attention check, against hand-worked cases
    cases = _golden_cases("row_rel_err.txt")
    assert len(cases) == 4
    for c in cases:
        num, den = (int(x) for x in c["expect"].split("/"))
        got = oracle.row_rel_err(_rows(c["got"]), _rows(c["ref"]))
        assert got == pytest.approx(num / den, rel=1e-15, abs=0.0), c


def _random_sequence_tokens(L, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L, Hkv, d))
    V = rng.standard_normal((L, Hkv, d))
    return oracle.SeqTokens(L, K, V, {})


def _bf16(x):
    return synth.bf16_bits(torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def test_prefill_attention_brute_force_tiny():
    # every query attends to its own position and all earlier ones only
    L, Hkv, g, d, n_q = 7, 2, 2, 4, 4
    st = _random_sequence_tokens(L, Hkv, d, 11)
    qb = _bf16(np.random.default_rng(12).standard_normal((n_q, Hkv * g, d)))
    q = oracle.bf16_bits_to_f64(qb)
    got = oracle.prefill_attention(st, qb, 0.6)
    for i in range(n_q):
        p = L - n_q + i
        for h in range(Hkv * g):
            ref = _brute(q[i, h], st.K[:p + 1, h // g], st.V[:p + 1, h // g], 0.6)
            assert np.abs(got[i, h] - ref).max() <= 1e-13


def test_prefill_attention_matches_torch_causal_sdpa_fp64():
    # a prompt's full prefill (n_q = L) is textbook causal attention
    L, Hkv, g, d = 40, 2, 4, 16
    st = _random_sequence_tokens(L, Hkv, d, 13)
    qb = _bf16(np.random.default_rng(14).standard_normal((L, Hkv * g, d)))
    q = torch.from_numpy(oracle.bf16_bits_to_f64(qb)).permute(1, 0, 2)            # [Hq][L][d]
    K = torch.from_numpy(st.K).permute(1, 0, 2).repeat_interleave(g, dim=0)       # [Hq][L][d]
    V = torch.from_numpy(st.V).permute(1, 0, 2).repeat_interleave(g, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], K[None], V[None], is_causal=True,
                                                           scale=0.25)[0].permute(1, 0, 2).numpy()
    assert np.abs(oracle.prefill_attention(st, qb, 0.25) - ref).max() <= 1e-12
    # a chunk (the last 9 positions) with the mask offset: torch's boolean mask
    n_q = 9
    mask = torch.arange(L)[None, :] <= (L - n_q + torch.arange(n_q))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q[None, :, L - n_q:], K[None], V[None], attn_mask=mask,
                                                           scale=0.25)[0].permute(1, 0, 2).numpy()
    assert np.abs(oracle.prefill_attention(st, qb[L - n_q:], 0.25) - ref).max() <= 1e-12


def test_prefill_attention_last_query_is_decode_and_ignores_later_tokens():
    w = synth.WORKLOADS["tiny"]
    L, n_q = w.len_lo, 5
    k = synth.bf16_bits(synth.kv_tokens(w, 0, 0, 0, L))
    v = synth.bf16_bits(synth.kv_tokens(w, 1, 0, 0, L))
    RK, RV = oracle.rotation(synth.random_orthogonal_u(w, 0)), oracle.rotation(synth.random_orthogonal_u(w, 1))
    c = np.full((w.num_kv_heads, w.head_dim), 2.5, dtype=np.float32)
    st = oracle.build_sequence(k, v, RK, RV, c, c, w.group_size)
    qb = synth.bf16_bits(synth.queries(w, 0, batch=n_q))
    got = oracle.prefill_attention(st, qb, 0.125)
    # the last query sees the whole pool: decode attention
    assert np.abs(got[-1] - oracle.attend_sequence(st, qb[-1], 0.125)).max() <= 1e-12
    # each query equals decode attention over the prefix ending at its position
    for i in range(n_q):
        p = L - n_q + i
        pre = oracle.SeqTokens(p + 1, st.K[:p + 1], st.V[:p + 1], {})
        assert np.abs(got[i] - oracle.attend_sequence(pre, qb[i], 0.125)).max() <= 1e-12
    # changing tokens after a query's position leaves it unchanged
    st2 = oracle.SeqTokens(L, st.K.copy(), st.V.copy(), {})
    st2.K[L - 2:] += 5.0
    st2.V[L - 2:] -= 3.0
    got2 = oracle.prefill_attention(st2, qb, 0.125)
    assert np.array_equal(got2[: n_q - 2], got[: n_q - 2]) and not np.allclose(got2[-1], got[-1])
