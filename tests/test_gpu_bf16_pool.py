"""GPU parity of the BF16-history pool (OSCAR_POOL_BF16_HISTORY), the
baseline the INT2 history is compared with: the same three-segment pool
with history tokens kept as they are.  Attention must equal the plain
softmax attention over the raw bf16 tokens (the oracle's definition,
within 2e-3 row-relative); history tokens, windows and page tables must be
bit-exact, over prefill, appends (evictions) and steps."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_segment_amd as ok
import harness
import oracle
import synth
from gpu_common import TOL, check_windows

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 63, 64, 65, 300, 319, 320, 321, 383, 384, 385, 1000]
SHAPES = {"g4_d128": (8, 2, 128, 128), "g8_d128": (16, 2, 128, 64), "g1_d64": (4, 4, 64, 64),
          "g16_d128": (32, 2, 128, 128)}


def _raw(w, b, L):
    k = synth.bf16_bits(synth.kv_tokens(w, 0, b, 0, L))
    v = synth.bf16_bits(synth.kv_tokens(w, 1, b, 0, L))
    return oracle.SeqTokens(L, oracle.bf16_bits_to_f64(k), oracle.bf16_bits_to_f64(v), {}), k, v


def _pool(w, lengths, extra, flags=0):
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths, extra_tokens=extra, slack_pages=3, flags=ok.POOL_BF16_HISTORY | flags)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=len(lengths))
    harness.prefill_all(pool, w, lengths)
    m = oracle.PoolModel(cfg.num_pages, cfg.page_shuffle_seed, cfg.max_pages_per_seq)
    for b, L in enumerate(lengths):
        m.prefill(b, int(L))
    return pool, m


def _check_all(pool, w, lengths, out, q_bits, rows_of=None):
    worst = 0.0
    for b, L in enumerate(lengths):
        st, k, v = _raw(w, b, L)
        ref = oracle.attend_sequence(st, q_bits[b], 1 / math.sqrt(w.head_dim))
        worst = max(worst, oracle.row_rel_err(out[b].double().cpu().numpy(), ref))
    assert worst <= TOL, worst
    return worst


def _check_state(pool, w, m, lengths):
    for b, L in enumerate(lengths):
        assert list(pool.page_table(b)) == m.table[b]
        st, k, v = _raw(w, b, L)
        n_hist = max(0, L - 320)
        if n_hist:
            hk, hv = ok.oscar_export_history_bf16(pool.handle, b, 0, n_hist, w.num_kv_heads, w.head_dim)
            assert np.array_equal(hk, k[64:64 + n_hist]) and np.array_equal(hv, v[64:64 + n_hist])
        check_windows(pool, w, b, L, k, v, range(w.num_kv_heads))


@pytest.mark.parametrize("shape", list(SHAPES))
def test_bf16_history_pool_matches_plain_attention(shape):
    Hq, Hkv, d, G = SHAPES[shape]
    w = synth.Workload("bf16_" + shape, 90 + list(SHAPES).index(shape), len(EDGE_LENS), Hq, Hkv, d, G, 0, 0)
    lengths = list(EDGE_LENS)
    steps = 40
    pool, m = _pool(w, lengths, steps)
    q = synth.queries(w, 0, device="cuda", batch=len(lengths))
    out = pool.decode(list(range(len(lengths))), q.view(torch.uint16))
    torch.cuda.synchronize()
    _check_all(pool, w, lengths, out, synth.bf16_bits(q.cpu()))
    rng = np.random.default_rng(7)
    for step in range(1, steps + 1):
        order = [int(x) for x in rng.permutation(len(lengths))]
        k_new, v_new = harness.step_tokens(w, lengths, order)
        q = synth.queries(w, step, device="cuda", batch=len(lengths))
        qo = q[torch.as_tensor(order, device="cuda")].contiguous().view(torch.uint16)
        out = pool.step(order, k_new, v_new, qo)
        m.append(order)
        for b in order:
            lengths[b] += 1
        if step % 10 == 0 or step == 1:
            torch.cuda.synchronize()
            inv = torch.as_tensor(np.argsort(order), device="cuda")
            _check_all(pool, w, lengths, out[inv], synth.bf16_bits(q.cpu()))
    _check_state(pool, w, m, lengths)


def test_bf16_history_pool_deterministic_and_wide():
    # 300 sequences (two launches), deterministic page order: two calls agree
    # bitwise and match the oracle
    n = 300
    w = synth.Workload("bf16_wide", 95, n, 4, 2, 64, 64, 0, 0)
    rng = np.random.default_rng(9)
    lengths = [int(rng.integers(1, 1500)) for _ in range(n)]
    pool, m = _pool(w, lengths, 2, flags=ok.POOL_DETERMINISTIC)
    ids = list(range(n))
    k_new, v_new = harness.step_tokens(w, lengths, ids)
    q = synth.queries(w, 1, device="cuda", batch=n).view(torch.uint16)
    out = pool.step(ids, k_new, v_new, q)
    m.append(ids)
    lengths = [L + 1 for L in lengths]
    a = pool.decode(ids, q)
    b = pool.decode(ids, q)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, out)
    qb = synth.bf16_bits(q.cpu())
    for s in (0, 1, 255, 256, 299):
        st, _, _ = _raw(w, s, lengths[s])
        ref = oracle.attend_sequence(st, qb[s], 1 / math.sqrt(w.head_dim))
        assert oracle.row_rel_err(out[s].double().cpu().numpy(), ref) <= TOL
    for s in ids:
        assert list(pool.page_table(s)) == m.table[s]


def test_bf16_history_pool_refuses_int2_only_calls():
    w = synth.Workload("bf16_refuse", 96, 1, 8, 2, 128, 128, 0, 0)
    pool, m = _pool(w, [700], 0)
    with pytest.raises(ok.OscarError) as ei:
        pool.export_history(0, 0, 10)
    assert ei.value.code == ok.EINVAL
    q = synth.queries(w, 0, device="cuda", batch=4).view(torch.uint16)
    with pytest.raises(ok.OscarError) as ei:
        pool.prefill_attn(0, q)
    assert ei.value.code == ok.EINVAL
