"""CPU tests of the library's host side: exported symbols, host bookkeeping
(lengths, page tables, free list) against the oracle's pool model, error
paths, and the offline helpers (R construction, clip calibration)."""
import os
import re
import subprocess

import numpy as np
import pytest

import bit_kv_cache_segment_amd as ok
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "oscar.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^(?:int|const char \*)\s*(oscar_\w+)\(", header, re.M))
    assert declared == set(ok.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", ok.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (oscar_\w+)$", nm, re.M))
    assert declared <= exported
    lib = ok.lib()
    for name in declared:
        getattr(lib, name)


def _host_pool(num_pages=300, maxp=40, seed=1234, max_seqs=6):
    cfg = ok.make_config(max_seqs, 8, 2, 64, 64, num_pages, maxp, seed, ok.POOL_HOST_ONLY)
    return ok.Pool(cfg, None, None, None, None)


def _state(p, n):
    return ([p.length(s) for s in range(n)], [list(p.page_table(s)) for s in range(n)], p.free_pages())


def test_host_bookkeeping_matches_oracle_pool_model():
    rng = np.random.default_rng(0)
    p = _host_pool()
    m = oracle.PoolModel(num_pages=300, seed=1234, max_pages_per_seq=40)
    for step in range(400):
        op = rng.integers(0, 10)
        if op == 0:
            s = int(rng.integers(0, 6))
            if p.length(s) == 0:
                L = int(rng.integers(0, 1200))
                need = max(0, -(-(L - 320) // 64))
                if need <= min(p.free_pages(), 40):
                    p.prefill_len(s, L)
                    m.prefill(s, L)
        elif op == 1:
            s = int(rng.integers(0, 6))
            p.release(s)
            m.release(s)
        else:
            ids = [int(x) for x in rng.permutation(6)[: rng.integers(1, 7)]]
            try:
                p.append(ids, None, None)
            except ok.OscarError:
                continue
            m.append(ids)
        for s in range(6):
            assert p.length(s) == m.length.get(s, 0)
            assert list(p.page_table(s)) == m.table.get(s, [])
        assert p.free_pages() == len(m.free)
    assert sum(p.length(s) for s in range(6)) > 0


def test_host_bookkeeping_with_forks_matches_oracle_pool_model():
    # prefix sharing: forks, copies on write and releases of shared pages
    rng = np.random.default_rng(1)
    p = _host_pool(num_pages=120, maxp=30, seed=77, max_seqs=8)
    m = oracle.PoolModel(num_pages=120, seed=77, max_pages_per_seq=30)
    forks = cows = 0
    for step in range(1500):
        op = rng.integers(0, 12)
        s = int(rng.integers(0, 8))
        if op == 0:
            if p.length(s) == 0:
                L = int(rng.integers(0, 1500))
                if max(0, -(-(L - 320) // 64)) <= min(p.free_pages(), 30):
                    p.prefill_len(s, L)
                    m.prefill(s, L)
        elif op == 1:
            p.release(s)
            m.release(s)
        elif op <= 3:
            d = int(rng.integers(0, 8))
            try:
                p.fork(s, d)
            except ok.OscarError as e:
                assert d == s or p.length(d) != 0, e
                continue
            m.fork(s, d)
            forks += p.length(s) > 320
        else:
            live = [q for q in range(8) if p.length(q) > 0]
            ids = [int(x) for x in rng.permutation(live)[: rng.integers(0, len(live) + 1)]]
            before = {i: list(p.page_table(i)) for i in ids}
            try:
                p.append(ids, None, None)
            except ok.OscarError:
                continue
            m.append(ids)
            after = {i: list(p.page_table(i)) for i in ids}
            cows += sum(len(after[i]) == len(before[i]) and after[i] != before[i] for i in ids)
        for q in range(8):
            assert p.length(q) == m.length.get(q, 0)
            assert list(p.page_table(q)) == m.table.get(q, [])
        assert p.free_pages() == len(m.free)
    assert forks > 20 and cows > 20, (forks, cows)


def test_fork_errors():
    p = _host_pool()
    p.prefill_len(0, 400)
    p.prefill_len(1, 10)
    before = _state(p, 6)
    for args, code in [((0, 0), ok.EINVAL), ((0, 1), ok.EINVAL), ((0, 6), ok.EINVAL), ((-1, 2), ok.EINVAL)]:
        with pytest.raises(ok.OscarError) as ei:
            p.fork(*args)
        assert ei.value.code == code and _state(p, 6) == before
    p.fork(2, 3)                       # an empty source leaves the target empty
    assert _state(p, 6) == before
    # ENOMEM: a copy on write needs a free page like a new page does
    q = _host_pool(num_pages=2, maxp=4)
    q.prefill_len(0, 330)              # history 10 tokens: one page
    q.fork(0, 1)
    q.prefill_len(2, 384)              # the last free page
    with pytest.raises(ok.OscarError) as ei:
        q.append([1], None, None)
    assert ei.value.code == ok.ENOMEM
    q.release(2)
    q.append([1, 0], None, None)       # seq 1 copies; seq 0 then writes in place
    assert q.page_table(0) != q.page_table(1) and q.free_pages() == 0


def test_errors_leave_state_unchanged():
    p = _host_pool(num_pages=10, maxp=4)
    p.prefill_len(0, 320 + 3 * 64)          # 3 pages
    p.prefill_len(1, 320 + 64 * 4)          # 4 pages -> 7 used, 3 free
    before = _state(p, 6)
    cases = [
        (lambda: p.append([0, 0], None, None), ok.EINVAL),      # repeated id
        (lambda: p.append([7], None, None), ok.EINVAL),         # id out of range
        (lambda: p.append([1], None, None), ok.ERANGE),         # would need a 5th page
        (lambda: p.prefill_len(0, 10), ok.EINVAL),              # not empty
        (lambda: p.prefill_len(2, 320 + 64 * 5), ok.ERANGE),    # > max_pages_per_seq
        (lambda: p.prefill_len(2, 320 + 64 * 3 + 1), ok.ENOMEM),  # 4 pages, 3 free
        (lambda: p.prefill_len(-1, 10), ok.EINVAL),
    ]
    for fn, code in cases:
        with pytest.raises(ok.OscarError) as ei:
            fn()
        assert ei.value.code == code, ei.value
        assert _state(p, 6) == before
    # ENOMEM in an append: three sequences each needing a page, two free
    p.prefill_len(2, 320 + 64)      # 1 page -> 2 free
    p.prefill_len(3, 320 + 64)      # 1 page -> 1 free
    p.prefill_len(4, 320)           # no history yet
    before = _state(p, 6)
    with pytest.raises(ok.OscarError) as ei:
        p.append([2, 3, 4], None, None)
    assert ei.value.code == ok.ENOMEM and _state(p, 6) == before
    ids = np.zeros(1, dtype=np.int32)
    rc = ok.lib().oscar_decode_attn(p.handle, ok._np_ptr(ids), 1, None, None, 1.0, None, 0, None)
    assert rc == ok.EINVAL and "host-only" in ok.lib().oscar_last_error().decode()
    rc = ok.lib().oscar_decode_step(p.handle, ok._np_ptr(ids), 1, None, None, None, None, 1.0, None, 0, None)
    assert rc == ok.EINVAL and "host-only" in ok.lib().oscar_last_error().decode()
    assert _state(p, 6) == before
    # profiling: argument checks come before the host-only check
    for args, msg in [((4, 0, 1), "mask"), ((4, 8, 1), "mask"), ((4, 1, 0), "every"), ((0, 1, 1), "max_calls"),
                      ((4, 1, 2), "host-only")]:
        rc = ok.lib().oscar_profile_begin(p.handle, *args)
        assert rc == ok.EINVAL and msg in ok.lib().oscar_last_error().decode(), (args, msg)


@pytest.mark.parametrize("kw", [dict(head_dim=96), dict(group_size=32), dict(num_q_heads=6),
                                dict(num_q_heads=12, num_kv_heads=4), dict(max_seqs=0),
                                dict(group_size=128, head_dim=64), dict(num_pages=-1), dict(flags=16), dict(flags=12)])
def test_bad_configs_rejected(kw):
    base = dict(max_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=64, group_size=64, num_pages=4,
                max_pages_per_seq=2)
    base.update(kw)
    cfg = ok.make_config(**base)
    with pytest.raises(ok.OscarError) as ei:
        ok.oscar_pool_bytes(cfg)
    assert ei.value.code == ok.EINVAL


def test_known_flags_accepted():
    for flags in (ok.POOL_HOST_ONLY, ok.POOL_DETERMINISTIC, ok.POOL_HOST_ONLY | ok.POOL_DETERMINISTIC):
        cfg = ok.make_config(2, 8, 2, 64, 64, 4, 2, flags=flags)
        assert ok.oscar_pool_bytes(cfg) > 0


def test_bad_clip_thresholds_rejected_before_device_access():
    cfg = ok.make_config(2, 8, 2, 64, 64, 4, 2)
    R = np.tile(np.eye(64, dtype=np.float32), (2, 1, 1))
    good = np.ones((2, 64), dtype=np.float32)
    fake = ok.lib()
    import ctypes
    n = ok.oscar_pool_bytes(cfg)
    for bad in (np.zeros((2, 64), np.float32), np.full((2, 64), 70000, np.float32),
                np.full((2, 64), np.nan, np.float32)):
        h = ctypes.c_void_p()
        rc = fake.oscar_pool_create(ctypes.byref(cfg), ctypes.c_void_p(256), n, ok._np_ptr(R), ok._np_ptr(R),
                                    ok._np_ptr(np.ascontiguousarray(bad)), ok._np_ptr(good), None, ctypes.byref(h))
        assert rc == ok.EINVAL
    h = ctypes.c_void_p()
    rc = fake.oscar_pool_create(ctypes.byref(cfg), ctypes.c_void_p(256), n - 1, ok._np_ptr(R), ok._np_ptr(R),
                                ok._np_ptr(good), ok._np_ptr(good), None, ctypes.byref(h))
    assert rc == ok.EINVAL and "required" in ok.lib().oscar_last_error().decode()


def test_sizes():
    w = synth.WORKLOADS["qwen3_8b_32k"]
    cfg = ok.make_config(16, 32, 8, 128, 128, 8112, 507)
    n = ok.oscar_pool_bytes(cfg)
    assert n % 256 == 0
    assert n >= 8112 * 8 * 4608 + 16 * 8 * 320 * 128 * 2 * 2
    assert ok.oscar_decode_workspace_bytes(cfg, 16) > 16 * 32 * 130 * 4


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b_32k", "large_batch_8k"])
def test_offline_tables_bit_exact_with_oracle(name):
    w = synth.WORKLOADS[name]
    for kind in (0, 1):
        U = synth.random_orthogonal_u(w, kind)
        R_lib = np.stack([ok.oscar_build_rotation(u) for u in U])
        R_orc = oracle.rotation(U)
        assert np.array_equal(R_lib.view(np.uint32), R_orc.view(np.uint32))
        cal = synth.bf16_bits(synth.calibration_tokens(w, kind, 1024))
        for h in (0, w.num_kv_heads - 1):
            c_lib = ok.oscar_calibrate_clip(cal[h], R_lib[h], 99.0)
            c_orc = oracle.clip_thresholds(cal[h], R_orc[h], 99.0)
            assert np.array_equal(c_lib.view(np.uint32), c_orc.view(np.uint32))


def test_pool_check_on_host_only_pools_and_null():
    p = _host_pool()
    ok.oscar_pool_check(p.handle, host_only=True)  # nothing ran on a device
    rc = ok.lib().oscar_pool_check(None, None)
    assert rc == ok.EINVAL


def test_pool_required_bytes_is_pool_plus_full_launch_workspace():
    for max_seqs in (1, 6, 300):
        cfg = ok.make_config(max_seqs, 32, 8, 128, 128, 100, 40, 5)
        dev, ws = ok.oscar_pool_required_bytes(cfg)
        assert dev == ok.oscar_pool_bytes(cfg)
        assert ws == ok.oscar_decode_workspace_bytes(cfg, min(max_seqs, 256))
    bad = ok.make_config(0, 32, 8, 128, 128, 100, 40, 5)
    with pytest.raises(ok.OscarError) as ei:
        ok.oscar_pool_required_bytes(bad)
    assert ei.value.code == ok.EINVAL


def test_export_state_refuses_host_only_pools():
    p = _host_pool()
    p.prefill_len(0, 500)
    table = np.zeros(40, dtype=np.int32)
    rc = ok.lib().oscar_export_state(p.handle, 0, table.ctypes.data_as(ok._P), None, None, None)
    assert rc == ok.EINVAL
