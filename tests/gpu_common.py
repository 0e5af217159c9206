"""Helpers shared by the GPU tests: oracle-side tables and per-sequence
references.  The oracle builds everything from the seeded generators on its
own; nothing here reads a value computed by the HIP path."""
import functools
import math

import numpy as np
import torch

import oracle
import synth

TOL = 2e-3   # max over rows of ||out - ref||_inf / ||ref||_inf


@functools.lru_cache(maxsize=None)
def oracle_tables(name_or_w, n_cal=4096):
    w = synth.WORKLOADS[name_or_w] if isinstance(name_or_w, str) else name_or_w
    R = [oracle.rotation(synth.random_orthogonal_u(w, kind)) for kind in (0, 1)]
    clips = []
    for kind in (0, 1):
        cal = synth.bf16_bits(synth.calibration_tokens(w, kind, n_cal))
        clips.append(np.stack([oracle.clip_thresholds(cal[h], R[kind][h]) for h in range(w.num_kv_heads)]))
    return R[0], R[1], clips[0], clips[1]


@functools.lru_cache(maxsize=None)
def oracle_codebooks(name_or_w, n_cal=4096):
    """(L_K, L_V) uint8 [Hkv][4]: the oracle's Lloyd-Max fit on the
    calibration tokens with the oracle's own tables."""
    w = synth.WORKLOADS[name_or_w] if isinstance(name_or_w, str) else name_or_w
    RK, RV, cK, cV = oracle_tables(w, n_cal)
    out = []
    for kind, (R, c) in enumerate(((RK, cK), (RV, cV))):
        cal = synth.bf16_bits(synth.calibration_tokens(w, kind, n_cal))
        out.append(np.stack([oracle.lloyd_max_codebook(oracle.normalized_values(cal[h], R[h], c[h], w.group_size))
                             for h in range(w.num_kv_heads)]))
    return out[0], out[1]


def oracle_sequence(w, b, L, heads=None, lloyd_max=False):
    """Oracle pool contents of synthetic sequence b at length L (optionally only
    some kv heads: the others stay raw and must not be used); lloyd_max: with
    the oracle's Lloyd-Max codebooks."""
    RK, RV, cK, cV = oracle_tables(w)
    hs = list(range(w.num_kv_heads)) if heads is None else list(heads)
    k = np.zeros((L, w.num_kv_heads, w.head_dim), dtype=np.uint16)
    v = np.zeros_like(k)
    k[:, hs] = synth.bf16_bits(synth.kv_tokens(w, 0, b, 0, L, heads=hs))
    v[:, hs] = synth.bf16_bits(synth.kv_tokens(w, 1, b, 0, L, heads=hs))
    cb = oracle_codebooks(w) if lloyd_max else None
    return oracle.build_sequence(k, v, RK, RV, cK, cV, w.group_size, heads=hs, codebook=cb), k, v


def check_history_codes(pool, w, seq, st, heads, first=0, count=None):
    """Bit-exact comparison of exported history codes/params with the oracle's."""
    n_hist = max(0, st.L - oracle.WINDOW)
    count = n_hist - first if count is None else count
    if count <= 0:
        return
    codes, params = pool.export_history(seq, first, count)
    for h in heads:
        for kvi, name in enumerate(("K", "V")):
            pk, s16, z16 = st.hist[(name, h)]
            assert np.array_equal(codes[:, h, kvi], pk[first:first + count]), (seq, h, name)
            assert np.array_equal(params[:, h, kvi, :, 0], s16[first:first + count]), (seq, h, name)
            assert np.array_equal(params[:, h, kvi, :, 1], z16[first:first + count]), (seq, h, name)


def check_windows(pool, w, seq, L, k, v, heads):
    sk, sv, rk, rv = pool.export_window(seq)
    sink, hist, recent = oracle.segments(L)
    for h in heads:
        for p in sink:
            assert np.array_equal(sk[p, h], k[p, h]) and np.array_equal(sv[p, h], v[p, h])
        for p in recent:
            s = oracle.ring_slot(p)
            assert np.array_equal(rk[s, h], k[p, h]) and np.array_equal(rv[s, h], v[p, h])


def check_rows(out_gpu, st, q_bits, w, rows):
    """Attention parity for query heads `rows` of one sequence."""
    ref = oracle.attend_sequence(st, q_bits, 1 / math.sqrt(w.head_dim), heads=rows)
    got = out_gpu.detach().cpu().numpy().astype(np.float64)
    err = oracle.row_rel_err(got[rows], ref[rows])
    assert err <= TOL, f"row-relative error {err:.3e} > {TOL}"
    return err


def check_evicted(pool, w, seqs, lengths, count, lloyd_max=False):
    """Every kv head of each sequence in `seqs`: the last `count` history
    entries (the tokens the latest appends evicted) bit-exact against the
    oracle's encoding of those tokens alone (with the oracle's Lloyd-Max
    codebooks if lloyd_max).  lengths[b]: length now.  Returns the number of
    (token, kv head, K|V) encodings compared."""
    RK, RV, cK, cV = oracle_tables(w)
    cb = oracle_codebooks(w) if lloyd_max else None
    checked = 0
    for b in seqs:
        n_hist = max(0, int(lengths[b]) - oracle.WINDOW)
        c = min(count, n_hist)
        if c <= 0:
            continue
        first = n_hist - c
        codes, params = pool.export_history(b, first, c)
        pos0 = oracle.SINK + first
        toks = [synth.bf16_bits(synth.kv_tokens(w, kind, b, pos0, c)) for kind in (0, 1)]
        for h in range(w.num_kv_heads):
            for kvi, (R, clip) in enumerate(((RK, cK), (RV, cV))):
                if cb is None:
                    pk, s16, z16 = oracle.encode(toks[kvi][:, h], R[h], clip[h], w.group_size)
                else:
                    pk, s16, z16 = oracle.encode_lut(toks[kvi][:, h], R[h], clip[h], w.group_size, cb[kvi][h])
                assert np.array_equal(codes[:, h, kvi], pk), (b, h, kvi)
                assert np.array_equal(params[:, h, kvi, :, 0], s16), (b, h, kvi)
                assert np.array_equal(params[:, h, kvi, :, 1], z16), (b, h, kvi)
                checked += c
    return checked
