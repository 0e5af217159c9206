"""Every decode kernel instance the library builds, run on the GPU at least
once: head dim d in {64, 128}, group size G in {64, 128} (G <= d) and
1, 2, 4, 8 or 16 query heads per kv head, each for affine pools and for
Lloyd-Max pools.  Five sequences over the segment edges (window only, an
exact window, a ragged last page, several pages) are decoded, stepped once
(append, eviction, decode in one call) and decoded again; attention within
2e-3 row-relative of the oracle at both points, and the evicted entries of
every kv head bit-exact."""
import numpy as np
import pytest
import torch

import bit_kv_cache_segment_amd as ok
import harness
import oracle
import synth
from gpu_common import check_evicted, check_rows, oracle_sequence

pytestmark = pytest.mark.gpu

LENGTHS = [1, 320, 385, 1000, 2100]
INSTANCES = [(d, G, g) for d, G in ((64, 64), (128, 64), (128, 128)) for g in (1, 2, 4, 8, 16)]


def _id(x):
    d, G, g = x
    return f"d{d}_G{G}_g{g}"


@pytest.mark.parametrize("lloyd", [False, True], ids=["affine", "lloyd_max"])
@pytest.mark.parametrize("inst", INSTANCES, ids=[_id(x) for x in INSTANCES])
def test_instance(inst, lloyd):
    d, G, g = inst
    Hkv = 2
    w = synth.Workload(f"inst_{_id(inst)}", 150 + INSTANCES.index(inst), len(LENGTHS), g * Hkv, Hkv, d, G, 0, 0)
    lengths = list(LENGTHS)
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths, extra_tokens=1, slack_pages=2, flags=ok.POOL_LLOYD_MAX if lloyd else 0)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=len(lengths))
    if lloyd:
        pool.set_codebook(*harness.codebooks(w, RK, RV, cK, cV))
    harness.prefill_all(pool, w, lengths)
    ids = list(range(len(lengths)))
    worst = 0.0

    def check(out, step):
        nonlocal worst
        q = synth.bf16_bits(synth.queries(w, step, batch=len(lengths)))
        for b, L in enumerate(lengths):
            st, _, _ = oracle_sequence(w, b, L, lloyd_max=lloyd)
            worst = max(worst, check_rows(out[b], st, q[b], w, list(range(w.num_q_heads))))

    out = pool.decode(ids, synth.queries(w, 0, device="cuda", batch=len(lengths)).view(torch.uint16))
    torch.cuda.synchronize()
    check(out, 0)
    k_new, v_new = harness.step_tokens(w, lengths)
    out = pool.step(ids, k_new, v_new, synth.queries(w, 1, device="cuda", batch=len(lengths)).view(torch.uint16))
    for b in ids:
        lengths[b] += 1
    torch.cuda.synchronize()
    check(out, 1)
    check_evicted(pool, w, [b for b in ids if lengths[b] > oracle.WINDOW], lengths, 1, lloyd_max=lloyd)
    print(f"{_id(inst)} {'lloyd_max' if lloyd else 'affine'}: worst row error {worst:.2e}")
