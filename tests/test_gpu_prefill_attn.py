"""GPU parity of prefill / chunked-prefill attention over the three-segment
pool (oscar_prefill_attn) against the oracle's causal attention over the
decoded pool: every query row within 2e-3 (row-relative).  Cases: a whole
prompt (queries in the sink, the history and the recent window), a chunk
longer than the recent window appended to a prefilled sequence (its first
queries' own positions are already in the INT2 history), small chunks,
n_q = 1 against decode attention, a long context whose tiles are cut
into several splits, and the benchmark's full-size chunk (two query heads
checked, every query)."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_segment_amd as ok
import harness
import oracle
import synth
from gpu_common import TOL, oracle_sequence

pytestmark = pytest.mark.gpu

SHAPES = {  # (Hq, Hkv, d, G)
    "g4_d128_G128": (8, 2, 128, 128),
    "g8_d128_G64": (16, 2, 128, 64),
    "g1_d64_G64": (4, 4, 64, 64),
    "g2_d64_G64": (4, 2, 64, 64),
    "g16_d128_G128": (32, 2, 128, 128),
}


def _workload(name, batch):
    Hq, Hkv, d, G = SHAPES[name]
    return synth.Workload("pf_" + name, 80 + list(SHAPES).index(name), batch, Hq, Hkv, d, G, 0, 0)


def _queries(w, seq, n_q, step):
    # rows of one sequence's queries: a fresh seeded draw per (sequence, step)
    return synth.queries(w, step * 64 + seq, batch=n_q)


def _check(pool, w, seq, L, n_q, step, out=None):
    q = _queries(w, seq, n_q, step)
    qd = q.to("cuda").view(torch.uint16).contiguous()
    got = pool.prefill_attn(seq, qd)
    torch.cuda.synchronize()
    st, _, _ = oracle_sequence(w, seq, L)
    ref = oracle.prefill_attention(st, synth.bf16_bits(q), 1 / math.sqrt(w.head_dim))
    g = got.double().cpu().numpy()
    err = oracle.row_rel_err(g.reshape(-1, w.head_dim), ref.reshape(-1, w.head_dim))
    assert err <= TOL, (seq, L, n_q, err)
    return got, err


@pytest.mark.parametrize("shape", list(SHAPES))
def test_prompt_prefill_and_chunks(shape):
    w = _workload(shape, 3)
    lengths = [700, 1000, 90]
    steps = 300
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths, extra_tokens=steps, slack_pages=2)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=3)
    harness.prefill_all(pool, w, lengths)
    # a whole prompt: every position's query
    _check(pool, w, 0, 700, 700, 0)
    _check(pool, w, 2, 90, 90, 0)
    # a chunk of 300 tokens appended to sequence 1 (1000 -> 1300): the
    # chunk's first 44 positions have left the recent window
    for t in range(steps):
        k_new, v_new = harness.step_tokens(w, [700, 1000 + t, 90], [1])
        pool.append([1], k_new, v_new)
    _check(pool, w, 1, 1300, 300, 1)
    # small chunks and a single query
    for n_q in (1, 2, 3, 17):
        _check(pool, w, 1, 1300, n_q, 2 + n_q)


def test_single_query_equals_decode():
    w = _workload("g4_d128_G128", 1)
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, [1500], extra_tokens=0)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=1)
    harness.prefill_all(pool, w, [1500])
    q = _queries(w, 0, 1, 9).to("cuda").view(torch.uint16).contiguous()
    a = pool.prefill_attn(0, q)
    b = pool.decode([0], q)
    torch.cuda.synchronize()
    ra = oracle.row_rel_err(a.double().cpu().numpy().reshape(-1, w.head_dim),
                            b.double().cpu().numpy().reshape(-1, w.head_dim))
    assert ra <= TOL


@pytest.mark.parametrize("shape", ["g4_d128_G128", "g16_d128_G128", "g8_d128_G64", "g2_d64_G64"])
def test_long_context_chunk_with_split_plans(shape):
    # 64 queries over 20,000 tokens: 1 to 8 tiles of 128 rows x 2 kv heads,
    # far fewer blocks than block slots, so each tile's pages are cut into
    # several splits and merged
    w = _workload(shape, 1)
    L, n_q = 20000, 64
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, [L], extra_tokens=0)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=1)
    harness.prefill_all(pool, w, [L])
    _check(pool, w, 0, L, n_q, 5)


def test_bench_chunk_full_size_sampled_heads():
    # the prefill benchmark's launch: the last 2048 queries of a 32,768-token
    # prompt, 32 query / 8 kv heads (d 128, G 128); query heads 0 and 31 (kv
    # heads 0 and 7) of every query against the oracle
    w = synth.WORKLOADS["qwen3_8b_32k"]
    L, n_q = 32768, 2048
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, [L])
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=1)
    harness.prefill_all(pool, w, [L])
    q = synth.queries(w, 0, batch=n_q)
    got = pool.prefill_attn(0, q.to("cuda").view(torch.uint16).contiguous())
    torch.cuda.synchronize()
    g = w.num_q_heads // w.num_kv_heads
    heads = [0, w.num_q_heads - 1]
    st, _, _ = oracle_sequence(w, 0, L, heads=sorted({h // g for h in heads}))
    ref = oracle.prefill_attention(st, synth.bf16_bits(q), 1 / math.sqrt(w.head_dim), heads=heads)
    out = got.double().cpu().numpy()
    for h in heads:
        err = oracle.row_rel_err(out[:, h], ref[:, h])
        assert err <= TOL, (h, err)


def test_query_elements_beyond_fp16_range():
    # queries times 2^17 (elements up to ~10^6, past fp16's 65504): the
    # matrix-core path scales such rows by an exact power of two before its
    # fp16 rotation and back after it
    w = _workload("g4_d128_G128", 1)
    L, n_q = 700, 40
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, [L], extra_tokens=0)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=1)
    harness.prefill_all(pool, w, [L])
    q = _queries(w, 0, n_q, 11) * 2.0 ** 17
    got = pool.prefill_attn(0, q.to("cuda").view(torch.uint16).contiguous())
    torch.cuda.synchronize()
    st, _, _ = oracle_sequence(w, 0, L)
    ref = oracle.prefill_attention(st, synth.bf16_bits(q), 1 / math.sqrt(w.head_dim))
    g = got.double().cpu().numpy()
    assert np.isfinite(g).all()
    err = oracle.row_rel_err(g.reshape(-1, w.head_dim), ref.reshape(-1, w.head_dim))
    assert err <= TOL, err


def test_prefill_attn_rejects_bad_arguments():
    w = _workload("g4_d128_G128", 2)
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, [400, 0], extra_tokens=0)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=2)
    harness.prefill_all(pool, w, [400])
    q = _queries(w, 0, 401, 0).to("cuda").view(torch.uint16).contiguous()
    with pytest.raises(ok.OscarError) as ei:
        pool.prefill_attn(0, q)  # more queries than tokens
    assert ei.value.code == ok.EINVAL
    with pytest.raises(ok.OscarError) as ei:
        pool.prefill_attn(1, q[:1])  # empty sequence
    assert ei.value.code == ok.EINVAL
    small = torch.empty(4, dtype=torch.float32, device="cuda")
    with pytest.raises(ok.OscarError) as ei:
        pool.prefill_attn(0, q[:10], workspace=small)
    assert ei.value.code == ok.EINVAL
