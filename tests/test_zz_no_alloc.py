"""oscar_decode_step_static, the decode step for callers that cannot
allocate device memory (its partials live in the library's static
workspace), against oscar_decode_step with a caller workspace: two
deterministic pools driven identically must stay bit for bit equal (outputs,
page tables, codes), call after call, with the batch shrinking from one call
to the next; outputs also within 2e-3 of the oracle.  A step whose plan
needs more than the static workspace is refused before anything changes."""
import numpy as np
import pytest
import torch

import bit_kv_cache_segment_amd as ok
import harness
import oracle
import synth
from gpu_common import check_rows, oracle_sequence

pytestmark = pytest.mark.gpu


def _pair_of_pools(w, lengths, extra):
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths, extra_tokens=extra, slack_pages=2, flags=ok.POOL_DETERMINISTIC)
    pools = []
    for _ in range(2):
        p = ok.Pool(cfg, RK, RV, cK, cV, max_batch=len(lengths))
        harness.prefill_all(p, w, lengths)
        pools.append(p)
    return pools


def _run(w, lengths, batches, oracle_rows):
    ref, sta = _pair_of_pools(w, lengths, extra=len(batches))
    lengths = list(lengths)
    for step, ids in enumerate(batches, start=1):
        print(f"{w.name}: call {step}, {len(ids)} sequences", flush=True)
        k_new, v_new = harness.step_tokens(w, lengths, ids)
        q = synth.queries(w, step, device="cuda", batch=len(lengths))
        qo = q[torch.as_tensor(ids, device="cuda")].contiguous().view(torch.uint16)
        a = ref.step(ids, k_new, v_new, qo)
        b = sta.step_static(ids, k_new, v_new, qo)
        for s in ids:
            lengths[s] += 1
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        qb = synth.bf16_bits(q.cpu())
        for i, s in enumerate(ids[:oracle_rows]):
            st, _, _ = oracle_sequence(w, s, lengths[s])
            check_rows(b[i], st, qb[s], w, list(range(w.num_q_heads)))
    for s in range(len(lengths)):
        assert ref.length(s) == sta.length(s) == lengths[s]
        assert list(ref.page_table(s)) == list(sta.page_table(s))
        n_hist = max(0, lengths[s] - 320)
        if n_hist:
            ha = ref.export_history(s, 0, n_hist)
            hb = sta.export_history(s, 0, n_hist)
            assert all(np.array_equal(x, y) for x, y in zip(ha, hb))


def test_static_step_matches_the_workspace_step_fused():
    # one launch pair per call (every block resident at once)
    w = synth.Workload("static_fused", 60, 6, 8, 2, 128, 128, 0, 0)
    lengths = [1000, 385, 320, 64, 1, 2000]
    _run(w, lengths, [[0, 1, 2, 3, 4, 5], [5, 0, 2]], oracle_rows=6)


def test_static_step_matches_the_workspace_step_wide():
    # 300 sequences x 4 kv heads: several rounds of blocks, so the step runs
    # as the append launch and then the decode launches, 256 sequences each
    n = 300
    w = synth.Workload("static_wide", 61, n, 8, 4, 64, 64, 0, 0)
    rng = np.random.default_rng(3)
    lengths = [int(rng.integers(1, 1400)) for _ in range(n)]
    _run(w, lengths, [list(range(n)), [int(x) for x in rng.permutation(n)[:100]]], oracle_rows=4)


def test_static_step_refuses_a_plan_larger_than_its_workspace():
    # 256 sequences x 128 query heads need 2 x 256 x 128 x 130 x 4 bytes of
    # partials (34 MB) at least: more than the static 32 MiB
    n = 256
    w = synth.Workload("static_big", 62, n, 128, 8, 128, 128, 0, 0)
    lengths = [1] * n
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths, extra_tokens=1)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=n)
    harness.prefill_all(pool, w, lengths)
    ids = list(range(n))
    k_new, v_new = harness.step_tokens(w, lengths, ids)
    q = synth.queries(w, 1, device="cuda").view(torch.uint16)
    with pytest.raises(ok.OscarError) as ei:
        pool.step_static(ids, k_new, v_new, q)
    assert ei.value.code == ok.EINVAL and "static workspace" in str(ei.value)
    assert all(pool.length(s) == 1 for s in ids)
    out = pool.step(ids, k_new, v_new, q)  # the caller-workspace step takes it
    torch.cuda.synchronize()
    assert all(pool.length(s) == 2 for s in ids)
    qb = synth.bf16_bits(synth.queries(w, 1))
    for s in (0, n - 1):
        st, _, _ = oracle_sequence(w, s, 2)
        check_rows(out[s], st, qb[s], w, list(range(w.num_q_heads)))
