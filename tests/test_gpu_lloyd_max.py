"""GPU parity of the Lloyd-Max codebook variant (OSCAR_POOL_LLOYD_MAX):
codes, fp16 scale/zero, windows and page tables bit-exact against the
oracle's nearest-level encoding with the oracle's own codebooks (the
library's offline fit gives the same codebooks, a CPU test), and decode
attention within 2e-3 row-relative of the oracle's attention over the pool
decoded with those levels; over the segment-edge lengths, shuffled appends
and steps, on four shapes; prefill attention over such a pool."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_segment_amd as ok
import harness
import oracle
import synth
from gpu_common import TOL, check_rows, check_windows, oracle_codebooks, oracle_sequence

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 63, 64, 65, 300, 319, 320, 321, 383, 384, 385, 1000]
SHAPES = {  # (Hq, Hkv, d, G)
    "g4_d128_G128": (8, 2, 128, 128),
    "g8_d128_G64": (16, 2, 128, 64),
    "g1_d64_G64": (4, 4, 64, 64),
    "g16_d128_G128": (32, 2, 128, 128),
}


def _workload(name):
    Hq, Hkv, d, G = SHAPES[name]
    return synth.Workload("lm_" + name, 90 + list(SHAPES).index(name), len(EDGE_LENS), Hq, Hkv, d, G, 0, 0)


def _pool(w, lengths, extra, flags=0):
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths, extra_tokens=extra, slack_pages=3, flags=ok.POOL_LLOYD_MAX | flags)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=len(lengths))
    Lk, Lv = harness.codebooks(w, RK, RV, cK, cV)
    pool.set_codebook(Lk, Lv)
    return pool, cfg, (Lk, Lv)


def _check_codes(pool, w, b, st):
    n_hist = max(0, st.L - oracle.WINDOW)
    if n_hist == 0:
        return
    codes, params = pool.export_history(b, 0, n_hist)
    for h in range(w.num_kv_heads):
        for kvi, name in enumerate(("K", "V")):
            pk, s16, z16 = st.hist[(name, h)]
            assert np.array_equal(codes[:, h, kvi], pk), (b, h, name)
            assert np.array_equal(params[:, h, kvi, :, 0], s16) and np.array_equal(params[:, h, kvi, :, 1], z16)


def _check_all(w, out, lengths, step, ids):
    q = synth.bf16_bits(synth.queries(w, step, batch=len(lengths)))
    worst = 0.0
    for i, b in enumerate(ids):
        st, _, _ = oracle_sequence(w, b, lengths[b], lloyd_max=True)
        worst = max(worst, check_rows(out[i], st, q[b], w, list(range(w.num_q_heads))))
    return worst


@pytest.mark.parametrize("shape", list(SHAPES))
def test_edge_lengths_appends_and_steps(shape):
    w = _workload(shape)
    lengths = list(EDGE_LENS)
    steps = 70
    pool, cfg, cb = _pool(w, lengths, steps)
    Lk_or, Lv_or = oracle_codebooks(w)
    assert np.array_equal(cb[0], Lk_or) and np.array_equal(cb[1], Lv_or)
    m = oracle.PoolModel(cfg.num_pages, cfg.page_shuffle_seed, cfg.max_pages_per_seq)
    harness.prefill_all(pool, w, lengths)
    for b, L in enumerate(lengths):
        m.prefill(b, L)
    ids = list(range(len(lengths)))
    q = synth.queries(w, 0, device="cuda", batch=len(lengths))
    out = pool.decode(ids, q.view(torch.uint16))
    torch.cuda.synchronize()
    worst = _check_all(w, out, lengths, 0, ids)
    rng = np.random.default_rng(5)
    for step in range(1, steps + 1):
        order = [int(x) for x in rng.permutation(len(lengths))]
        k_new, v_new = harness.step_tokens(w, lengths, order)
        q = synth.queries(w, step, device="cuda", batch=len(lengths))
        qo = q[torch.as_tensor(order, device="cuda")].contiguous().view(torch.uint16)
        if step % 2:
            out = pool.step(order, k_new, v_new, qo)
        else:
            pool.append(order, k_new, v_new)
            out = pool.decode(order, qo)
        m.append(order)
        for b in order:
            lengths[b] += 1
        if step % 10 == 0 or step <= 2:
            torch.cuda.synchronize()
            worst = max(worst, _check_all(w, out, lengths, step, order))
    torch.cuda.synchronize()
    for b, L in enumerate(lengths):
        assert pool.length(b) == L
        assert list(pool.page_table(b)) == m.table[b]
        st, k, v = oracle_sequence(w, b, L, lloyd_max=True)
        _check_codes(pool, w, b, st)
        check_windows(pool, w, b, L, k, v, range(w.num_kv_heads))
    print(f"{shape}: worst row error {worst:.2e}")


def test_deterministic_pool_is_bitwise_reproducible():
    w = _workload("g4_d128_G128")
    lengths = [5000, 777, 2100]
    pool, cfg, _ = _pool(w, lengths, 0, flags=ok.POOL_DETERMINISTIC)
    harness.prefill_all(pool, w, lengths)
    q = synth.queries(w, 3, device="cuda", batch=3).view(torch.uint16)
    a = pool.decode([0, 1, 2], q).clone()
    b = pool.decode([0, 1, 2], q).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    _check_all(w, a, lengths, 3, [0, 1, 2])


@pytest.mark.parametrize("shape", ["g4_d128_G128", "g8_d128_G64", "g1_d64_G64"])
def test_prefill_attention_over_a_lloyd_max_pool(shape):
    # the last n_q positions of a prompt attend causally over the pool with
    # the codebook's levels: within 2e-3 of the oracle's prefill attention
    w = _workload(shape)
    lengths = [1400, 700]
    pool, cfg, _ = _pool(w, lengths, 0)
    harness.prefill_all(pool, w, lengths)
    for seq, L, n_q in ((0, 1400, 1400), (0, 1400, 300), (1, 700, 5)):
        q = synth.queries(w, 500 + n_q, batch=n_q)
        out = pool.prefill_attn(seq, q.to("cuda").view(torch.uint16).contiguous())
        torch.cuda.synchronize()
        st, _, _ = oracle_sequence(w, seq, L, lloyd_max=True)
        ref = oracle.prefill_attention(st, synth.bf16_bits(q), 1 / math.sqrt(w.head_dim))
        err = oracle.row_rel_err(out.double().cpu().numpy().reshape(-1, w.head_dim), ref.reshape(-1, w.head_dim))
        print(f"{shape}: seq {seq}, n_q {n_q}: worst row error {err:.2e}")
        assert err <= TOL, (seq, n_q, err)
