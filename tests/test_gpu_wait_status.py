"""A bounded wait inside a decode block that gives up is reported, not
silent.  The give-up is forced from the host: a pool created while
OSCAR_WAIT_SPIN_LIMIT=0 gives up every such wait at once (its waves then
read data that may be stale, always inside the pool; nothing faults or
hangs).  oscar_pool_check and the exports must then fail with EHIP, while a
pool created normally in the same process still passes."""
import pytest
import torch

import bit_kv_cache_segment_amd as ok
import harness
import synth

pytestmark = pytest.mark.gpu


def _pool(w, lengths, extra):
    RK, RV, cK, cV = harness.tables(w)
    cfg = harness.config_for(w, lengths, extra_tokens=extra, slack_pages=2)
    p = ok.Pool(cfg, RK, RV, cK, cV, max_batch=len(lengths))
    harness.prefill_all(p, w, lengths)
    return p


def test_a_wait_that_gives_up_is_reported(monkeypatch):
    w = synth.Workload("wait_status", 70, 3, 8, 2, 128, 128, 0, 0)
    lengths = [1000, 385, 64]
    normal = _pool(w, lengths, 2)
    monkeypatch.setenv("OSCAR_WAIT_SPIN_LIMIT", "0")
    forced = _pool(w, lengths, 2)
    monkeypatch.delenv("OSCAR_WAIT_SPIN_LIMIT")
    ids = [0, 1, 2]
    for step in (1, 2):
        k_new, v_new = harness.step_tokens(w, [L + step - 1 for L in lengths], ids)
        q = synth.queries(w, step, device="cuda", batch=3).view(torch.uint16).contiguous()
        normal.step(ids, k_new, v_new, q)
        forced.step(ids, k_new, v_new, q)
    torch.cuda.synchronize()
    normal.check()
    normal.export_history(0, 0, 10)
    with pytest.raises(ok.OscarError) as ei:
        forced.check()
    assert ei.value.code == ok.EHIP and "gave up" in str(ei.value)
    with pytest.raises(ok.OscarError) as ei:
        forced.export_history(0, 0, 10)
    assert ei.value.code == ok.EHIP
    with pytest.raises(ok.OscarError) as ei:
        forced.export_window(1)
    assert ei.value.code == ok.EHIP
    normal.check()
