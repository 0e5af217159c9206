"""GPU parity of prefix sharing (oscar_fork_seq): forked sequences share
their history pages, and a sequence about to write into a shared last page
copies it first.  Each sequence's tokens are a composite stream (the
source's tokens before the fork, its own after); attention must match the
oracle's pool built from that stream within 2e-3 row-relative error, and
codes, scale/zero, windows and page tables (against the oracle's pool model
with forks) must be bit-exact, through fused steps and separate
append + decode calls, chained forks, and releases of sources whose pages
forks still hold; and prefill attention over forked sequences."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_segment_amd as ok
import harness
import oracle
import synth
from gpu_common import TOL, check_history_codes, check_windows, oracle_codebooks, oracle_tables

pytestmark = pytest.mark.gpu

SHAPES = {  # (Hq, Hkv, d, G)
    "g4_d128_G128": (8, 2, 128, 128),
    "g8_d128_G64": (16, 2, 128, 64),
    "g1_d64_G64": (4, 4, 64, 64),
}
INF = 1 << 30
# sources: history 74 (COW at slot 10), 680 (COW at slot 40), 64 (a full
# last page: the next append starts a page, no copy), none yet (window only)
SOURCES = [394, 1000, 384, 300]


def _workload(name, flags=0):
    Hq, Hkv, d, G = SHAPES[name]
    return synth.Workload("fork_" + name, 40 + list(SHAPES).index(name) + 5 * bool(flags) + 3 * bool(flags & 8), 10,
                          Hq, Hkv, d, G, 0, 0)


def _tokens(w, segs, L):
    k = np.zeros((L, w.num_kv_heads, w.head_dim), dtype=np.uint16)
    v = np.zeros_like(k)
    for b, a, e in segs:
        e = min(e, L)
        if a < e:
            k[a:e] = synth.bf16_bits(synth.kv_tokens(w, 0, b, a, e - a))
            v[a:e] = synth.bf16_bits(synth.kv_tokens(w, 1, b, a, e - a))
    return k, v


class Run:
    """Pool, oracle pool model and per-sequence token streams."""

    def __init__(self, w, flags):
        self.w, self.flags = w, flags
        RK, RV, cK, cV = harness.tables(w)
        n_seqs = 10
        cfg = harness.config_for(w, [1000] * n_seqs, extra_tokens=100, slack_pages=4, flags=flags)
        self.pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=n_seqs)
        if flags & ok.POOL_LLOYD_MAX:
            self.pool.set_codebook(*harness.codebooks(w, RK, RV, cK, cV))
        self.model = oracle.PoolModel(cfg.num_pages, cfg.page_shuffle_seed, cfg.max_pages_per_seq)
        self.segs, self.stream, self.length = {}, {}, {}
        self.n_seqs = n_seqs

    def prefill(self, seq, stream, L):
        w = self.w
        k = synth.kv_tokens(w, 0, stream, 0, L, device="cuda").view(torch.uint16)
        v = synth.kv_tokens(w, 1, stream, 0, L, device="cuda").view(torch.uint16)
        self.pool.prefill(seq, k, v)
        self.model.prefill(seq, L)
        self.segs[seq] = [(stream, 0, INF)]
        self.stream[seq], self.length[seq] = stream, L

    def fork(self, src, dst, stream):
        self.pool.fork(src, dst)
        self.model.fork(src, dst)
        Lf = self.length[src]
        self.segs[dst] = [(b, a, min(e, Lf)) for b, a, e in self.segs[src] if a < Lf] + [(stream, Lf, INF)]
        self.stream[dst], self.length[dst] = stream, Lf

    def release(self, seq):
        self.pool.release(seq)
        self.model.release(seq)
        del self.segs[seq], self.stream[seq], self.length[seq]

    def new_tokens(self, ids):
        w = self.w
        st = [self.stream[s] for s in ids]
        pos = [self.length[s] for s in ids]
        k = synth.kv_tokens_at(w, 0, st, pos, device="cuda").view(torch.uint16).contiguous()
        v = synth.kv_tokens_at(w, 1, st, pos, device="cuda").view(torch.uint16).contiguous()
        return k, v

    def oracle_seq(self, seq):
        w, L = self.w, self.length[seq]
        k, v = _tokens(w, self.segs[seq], L)
        if self.flags & ok.POOL_BF16_HISTORY:
            return oracle.SeqTokens(L, oracle.bf16_bits_to_f64(k), oracle.bf16_bits_to_f64(v), {}), k, v
        RK, RV, cK, cV = oracle_tables(w)
        cb = oracle_codebooks(w) if self.flags & ok.POOL_LLOYD_MAX else None
        return oracle.build_sequence(k, v, RK, RV, cK, cV, w.group_size, codebook=cb), k, v

    def check_out(self, ids, out, q_bits):
        worst = 0.0
        for i, s in enumerate(ids):
            st, _, _ = self.oracle_seq(s)
            ref = oracle.attend_sequence(st, q_bits[i], 1 / math.sqrt(self.w.head_dim))
            worst = max(worst, oracle.row_rel_err(out[i].double().cpu().numpy(), ref))
        assert worst <= TOL, worst
        return worst

    def check_state(self):
        w, heads = self.w, range(self.w.num_kv_heads)
        for s in range(self.n_seqs):
            assert self.pool.length(s) == self.length.get(s, 0)
            assert list(self.pool.page_table(s)) == self.model.table.get(s, []), s
        assert self.pool.free_pages() == len(self.model.free)
        for s, L in self.length.items():
            st, k, v = self.oracle_seq(s)
            check_windows(self.pool, w, s, L, k, v, heads)
            n_hist = max(0, L - oracle.WINDOW)
            if self.flags & ok.POOL_BF16_HISTORY:
                if n_hist:
                    hk, hv = ok.oscar_export_history_bf16(self.pool.handle, s, 0, n_hist, w.num_kv_heads,
                                                          w.head_dim)
                    assert np.array_equal(hk, k[64:64 + n_hist]) and np.array_equal(hv, v[64:64 + n_hist])
            else:
                check_history_codes(self.pool, w, s, st, heads)


def _drive(run, steps, seed):
    """Forks at the start, steps over random subsets in random order (fused
    and separate calls alternating), a chained fork, a release of a source
    whose pages forks hold, and a new prompt into the freed slot."""
    w = run.w
    for s, L in enumerate(SOURCES):
        run.prefill(s, s, L)
    for s in range(4):
        run.fork(s, 4 + s, 4 + s)
    shared = sum(run.model.refs[pg] > 1 for pg in run.model.refs)
    assert shared > 0
    rng = np.random.default_rng(seed)
    worst = 0.0
    cows = 0
    for step in range(1, steps + 1):
        if step == 20:
            run.fork(4, 8, 8)          # a fork of a fork
        if step == 35:
            run.release(0)             # its pages stay with seqs 4 and 8
        if step == 45:
            run.prefill(0, 9, 700)     # reuses freed pages
        live = sorted(run.length)
        ids = [int(x) for x in rng.permutation(live)[: rng.integers(max(1, len(live) // 2), len(live) + 1)]]
        before = {s: list(run.pool.page_table(s)) for s in ids}
        k_new, v_new = run.new_tokens(ids)
        q = synth.queries(w, step, device="cuda", batch=len(ids))
        if step % 2:
            out = run.pool.step(ids, k_new, v_new, q.view(torch.uint16))
        else:
            run.pool.append(ids, k_new, v_new)
            out = run.pool.decode(ids, q.view(torch.uint16))
        run.model.append(ids)
        for s in ids:
            run.length[s] += 1
        for s in ids:
            after = list(run.pool.page_table(s))
            cows += len(after) == len(before[s]) and after != before[s]
        if step % 10 == 0 or step in (1, 2, 21, 46):
            torch.cuda.synchronize()
            worst = max(worst, run.check_out(ids, out, synth.bf16_bits(q.cpu())))
    torch.cuda.synchronize()
    run.check_state()
    assert cows >= 3, cows
    return worst


def _check_prefill(run, seqs, n_q):
    """Prefill attention of the last n_q positions of forked sequences (their
    history partly in pages they share, partly in copied pages) against the
    oracle's causal attention over the composite token stream."""
    w = run.w
    for s in seqs:
        q = synth.queries(w, 500 + s, batch=n_q)
        got = run.pool.prefill_attn(s, q.to("cuda").view(torch.uint16).contiguous())
        torch.cuda.synchronize()
        st, _, _ = run.oracle_seq(s)
        ref = oracle.prefill_attention(st, synth.bf16_bits(q), 1 / math.sqrt(w.head_dim))
        err = oracle.row_rel_err(got.double().cpu().numpy().reshape(-1, w.head_dim), ref.reshape(-1, w.head_dim))
        assert err <= TOL, (s, err)


@pytest.mark.parametrize("shape", list(SHAPES))
def test_forks_match_oracle(shape):
    w = _workload(shape)
    run = Run(w, 0)
    worst = _drive(run, 60, 7)
    _check_prefill(run, [5, 8], 300)
    print(f"{shape}: worst row error {worst:.2e}")


def test_forks_bf16_history_pool():
    w = _workload("g4_d128_G128", ok.POOL_BF16_HISTORY)
    run = Run(w, ok.POOL_BF16_HISTORY)
    _drive(run, 40, 8)


def test_forks_lloyd_max_pool():
    w = _workload("g8_d128_G64", ok.POOL_LLOYD_MAX)
    run = Run(w, ok.POOL_LLOYD_MAX)
    _drive(run, 40, 9)
    _check_prefill(run, [5, 8], 300)


def test_fork_then_release_everything_returns_every_page():
    w = _workload("g1_d64_G64")
    run = Run(w, 0)
    total = run.pool.free_pages()
    run.prefill(0, 0, 1000)
    run.fork(0, 1, 1)
    run.fork(1, 2, 2)
    k_new, v_new = run.new_tokens([2, 0, 1])
    run.pool.append([2, 0, 1], k_new, v_new)
    run.model.append([2, 0, 1])
    for s in (2, 0, 1):
        run.length[s] += 1
    torch.cuda.synchronize()
    run.check_state()
    for s in (0, 2, 1):
        run.release(s)
    assert run.pool.free_pages() == total == len(run.model.free)
