"""Pins of the pool semantics: segment boundaries, the recent ring, page
allocation, and the bit accounting printed on the pages."""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_segments_hand_worked():
    for L, sl, hs, hl, rs, rl in (map(int, r) for r in _rows("segments.txt")):
        sink, hist, recent = oracle.segments(L)
        assert (len(sink), hist.start, len(hist), recent.start, len(recent)) == (sl, hs, hl, rs, rl), L
        assert len(sink) + len(hist) + len(recent) == L


def test_ring_eviction_takes_oldest_and_reuses_its_slot():
    # simulate the recent window slot by slot from an empty sequence
    slots = {}
    for L in range(0, 2000):
        sink, hist, recent = oracle.segments(L)
        # the window holds exactly the positions of the recent segment
        assert sorted(slots.values()) == list(recent)
        if L >= oracle.WINDOW:
            evicted = oracle.SINK + (L - oracle.WINDOW)
            assert evicted == recent.start                    # the oldest recent token
            assert oracle.ring_slot(evicted) == oracle.ring_slot(L)
        if L >= oracle.SINK:
            slots[oracle.ring_slot(L)] = L
    assert len(slots) == 256


def test_free_list_is_a_seeded_permutation():
    a = oracle.free_list(1000, 42)
    assert sorted(a) == list(range(1000))
    assert a == oracle.free_list(1000, 42) and a != oracle.free_list(1000, 43)
    assert a != list(range(1000))


def test_free_list_generator_and_shuffle_match_published_outputs():
    # SplitMix64 against its published reference outputs, Fisher-Yates
    # against a case worked by hand (tests/golden/free_list.txt)
    for row in _rows("free_list.txt"):
        if row[0] == "S":
            g = oracle.splitmix64_stream(int(row[1]))
            assert [next(g) for _ in row[2:]] == [int(v) for v in row[2:]]
        else:
            assert oracle.free_list(int(row[1]), int(row[2])) == [int(v) for v in row[3:]]


def test_pool_model_pages():
    pm = oracle.PoolModel(num_pages=200, seed=9, max_pages_per_seq=64)
    fl = list(pm.free)
    pm.prefill(0, 320 + 130)            # 130 history tokens -> 3 pages
    pm.prefill(1, 100)                  # no history
    assert pm.table[0] == fl[:3] and pm.table.get(1) == []
    # appends: seq 0 at n_hist 130..191 needs no page until n_hist = 192
    for _ in range(62):
        pm.append([1, 0])
    assert pm.table[0] == fl[:3]
    pm.append([1, 0])                   # seq 0 evicts history index 192 -> new page
    assert pm.table[0] == fl[:4]
    assert pm.length[0] == 450 + 63 and pm.length[1] == 163
    pm.release(0)
    assert pm.free[-4:] == fl[:4]
    used = [p for t in pm.table.values() for p in t]
    assert len(used) == len(set(used))


def test_bits_per_element_matches_the_article():
    for L, G, want in _rows("bits_per_element.txt"):
        assert round(oracle.bits_per_element(int(L), int(G)), 2) == float(want)


def test_synthetic_generator_properties():
    w = synth.WORKLOADS["qwen3_8b_32k"]
    assert synth.mix32_int(0) == int(synth._mix32(__import__("torch").tensor([0]))[0])
    t = synth._normal_table_np()
    assert np.array_equal(t, -t[::-1]) and abs(t.mean()) < 1e-6 and abs(t.std() - 1) < 2e-3
    k = synth.kv_tokens(w, 0, 3, 1000, 64).float().numpy()
    out = synth.outlier_channels(w, 0)
    for h in range(w.num_kv_heads):
        assert len(set(out[h])) == 4
        plain = np.delete(k[:, h, :], out[h], axis=1)
        assert abs(plain.std() - 1) < 0.1 and abs(k[:, h, out[h]].std() - 20) < 3
    # a token's value depends only on its position: two overlapping draws agree
    a = synth.kv_tokens(w, 1, 5, 100, 50)
    b = synth.kv_tokens(w, 1, 5, 120, 50)
    assert (a[20:] == b[:30]).all()


def test_prefix_sharing_hand_worked():
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "prefix_sharing.txt")
    F = oracle.free_list(10, 77)
    m = oracle.PoolModel(10, 77, 8)
    for ln in open(path):
        ln = ln.strip()
        if not ln or ln.startswith("#"):
            continue
        if ln.startswith("free "):
            assert m.free == [F[int(k)] for k in ln.split()[1].split(",")]
            continue
        op, want = (x.strip() for x in ln.split("|"))
        name, *args = op.split()
        args = [int(a) for a in args]
        if name == "prefill":
            m.prefill(args[0], args[1])
        elif name == "fork":
            m.fork(args[0], args[1])
        elif name == "append":
            m.append(args)
        elif name == "release":
            m.release(args[0])
        for item in want.split():
            seq, pages = item.split(":")
            assert m.table[int(seq)] == [F[int(k)] for k in pages.split(",") if k != ""], (op, item)
    # every page is back exactly once
    assert sorted(m.free) == list(range(10)) and all(v == 0 for v in m.refs.values())


def test_prefix_sharing_invariants_random():
    # random operations: a page is held by exactly as many tables as its
    # count says; held pages are never on the free list; nothing is lost
    rng = np.random.default_rng(3)
    m = oracle.PoolModel(400, 5, 60)
    for _ in range(3000):
        op = rng.integers(0, 10)
        s = int(rng.integers(0, 8))
        if op == 0 and m.length.get(s, 0) == 0:
            L = int(rng.integers(0, 1500))
            if -(-max(0, L - 320) // 64) <= min(len(m.free), 20):
                m.prefill(s, L)
        elif op == 1:
            d = int(rng.integers(0, 8))
            if d != s and m.length.get(d, 0) == 0:
                m.fork(s, d)
        elif op == 2:
            m.release(s)
        else:
            ids = [int(x) for x in rng.permutation(8)[: rng.integers(1, 9)]]
            if len(m.free) >= len(ids) and all(len(m.table.get(i, [])) < 59 for i in ids):
                m.append(ids)
        held = {}
        for t in m.table.values():
            for pg in t:
                held[pg] = held.get(pg, 0) + 1
        assert all(m.refs[pg] == c for pg, c in held.items())
        assert not set(held) & set(m.free)
        assert len(held) + len(m.free) == 400
