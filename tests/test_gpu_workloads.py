"""GPU parity at the full workload sizes: whole page tables, sampled
(sequence, kv head) pairs compared bit-exactly on their codes and within
2e-3 on attention, and the 256-step serving run through oscar_decode_step
(the call the benchmark times) with every evicted token of every pair
compared bit-exactly at the end."""
import numpy as np
import pytest
import torch

import bit_kv_cache_segment_amd as ok
import harness
import oracle
import synth
from gpu_common import check_evicted, check_history_codes, check_rows, check_windows, oracle_sequence

pytestmark = pytest.mark.gpu


def _setup(w, extra=0):
    lengths = [int(x) for x in synth.lengths(w)]
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths, extra_tokens=extra)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=w.batch)
    harness.prefill_all(pool, w, lengths)
    m = oracle.PoolModel(cfg.num_pages, cfg.page_shuffle_seed, cfg.max_pages_per_seq)
    for b, L in enumerate(lengths):
        m.prefill(b, L)
    return pool, cfg, m, lengths


def _sampled_check(pool, w, lengths, out, step, pairs):
    q = synth.bf16_bits(synth.queries(w, step))
    g = w.gqa
    errs = []
    for b, kv in pairs:
        st, k, v = oracle_sequence(w, b, lengths[b], heads=[kv])
        rows = list(range(kv * g, (kv + 1) * g))
        errs.append(check_rows(out[b], st, q[b], w, rows))
        check_history_codes(pool, w, b, st, [kv])
        check_windows(pool, w, b, lengths[b], k, v, [kv])
    return max(errs)


@pytest.mark.parametrize("name", ["qwen3_8b_32k", "large_batch_8k", "qwen3_32b_64k"])
def test_decode_workload(name):
    w = synth.WORKLOADS[name]
    pool, cfg, m, lengths = _setup(w)
    for b in range(w.batch):
        assert list(pool.page_table(b)) == m.table[b]
    q = synth.queries(w, 0, device="cuda").view(torch.uint16)
    out = pool.decode(list(range(w.batch)), q)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(w.config_id)
    pairs = [(int(rng.integers(0, w.batch)), int(rng.integers(0, w.num_kv_heads))) for _ in range(2)]
    pairs.append((w.batch - 1, w.num_kv_heads - 1))
    err = _sampled_check(pool, w, lengths, out, 0, pairs)
    print(f"{name}: sampled pairs {pairs} max row-relative error {err:.2e}")


def test_fused_serving_steps():
    w = synth.WORKLOADS["fused_64x_4k_64k"]
    pool, cfg, m, lengths = _setup(w, extra=w.steps)
    rng = np.random.default_rng(55)
    ids = list(range(w.batch))
    checks = {1, 64, 128, 256}
    for step in range(1, w.steps + 1):
        k_new, v_new = harness.step_tokens(w, lengths)
        q = synth.queries(w, step, device="cuda").view(torch.uint16)
        out = pool.step(ids, k_new, v_new, q)
        m.append(ids)
        for b in ids:
            lengths[b] += 1
        if step in checks:
            torch.cuda.synchronize()
            for b in ids:
                assert list(pool.page_table(b)) == m.table[b]
            pair = (int(rng.integers(0, w.batch)), int(rng.integers(0, w.num_kv_heads)))
            err = _sampled_check(pool, w, lengths, out, step, [pair])
            print(f"step {step}: pair {pair} error {err:.2e}", flush=True)
    # every token the 256 steps evicted, of every (sequence, kv head) pair
    n = check_evicted(pool, w, ids, lengths, w.steps)
    assert n == w.batch * w.num_kv_heads * 2 * w.steps
