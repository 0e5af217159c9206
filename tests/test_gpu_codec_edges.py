"""GPU parity of the codec's degenerate cases through all three encoders
(bulk prefill, the append kernel, the append inside the fused step):

* zero tokens (+0 and -0): every group range is 0, so the fp16 scale is 0,
  every code 0 and the zero point +0;
* tokens scaled by 2^-20 and 2^-24: the group scale is a sub-normal fp16
  number, and where it rounds below (max - min)/3 the codes are clamped to 3;
* a pool whose clip thresholds are 2^-20 on every channel: every rotated
  channel of an ordinary token clips, so groups hold +-c only (codes 0 and 3)
  or a single value (scale 0);
* a pool at the largest thresholds the fp16 scale allows (65504), with
  tokens of magnitude ~2^12, so scales sit near the top of the fp16 range.

Codes, scale/zero and windows are compared bit for bit with the oracle;
attention rows within 2e-3 (with a softmax scale that keeps the logits of the
large tokens of order one)."""
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

SHAPES = {"d128_G64": (8, 2, 128, 64), "d128_G128": (8, 2, 128, 128), "d64_G64": (4, 1, 64, 64)}
LENGTHS = [330, 700, 1000, 385]
STEPS = 40


def _tokens(w, kind, case, b, L):
    """uint16 bf16 bits [L][Hkv][d] of sequence b for one edge case.  The
    values come from the seeded generator; this only zeroes or rescales them
    by powers of two (exact in bf16)."""
    x = synth.kv_tokens(w, kind, b, 0, L).float()
    if case == "mixed":
        pos = torch.arange(L)
        sel = pos % 5
        x[sel == 0] = 0.0
        x[sel == 1] = -0.0
        x[sel == 2] *= 2.0 ** -20
        x[sel == 3] *= 2.0 ** -24
    elif case == "large":
        x *= 2.0 ** 12
    return synth.bf16_bits(x.to(torch.bfloat16))


def _tables(w, case):
    RK, RV, cK, cV = harness.tables(w)
    if case == "tiny_clip":
        cK = np.full_like(cK, 2.0 ** -20)
        cV = np.full_like(cV, 2.0 ** -20)
    elif case == "large":
        cK = np.full_like(cK, 65504.0)
        cV = np.full_like(cV, 65504.0)
    return RK, RV, cK, cV


def _oracle_tables(w, case):
    from gpu_common import oracle_tables
    RK, RV, cK, cV = oracle_tables(w)
    if case == "tiny_clip":
        cK = np.full_like(cK, 2.0 ** -20)
        cV = np.full_like(cV, 2.0 ** -20)
    elif case == "large":
        cK = np.full_like(cK, 65504.0)
        cV = np.full_like(cV, 65504.0)
    return RK, RV, cK, cV


def _check_seq(pool, w, case, b, L, tk, tv, q_bits, out_row, scale, rows=True):
    RK, RV, cK, cV = _oracle_tables(w, case)
    k, v = tk[b][:L], tv[b][:L]
    st = oracle.build_sequence(k, v, RK, RV, cK, cV, w.group_size)
    n_hist = max(0, L - oracle.WINDOW)
    if n_hist:
        codes, params = pool.export_history(b, 0, n_hist)
        for h in range(w.num_kv_heads):
            for i, name in enumerate("KV"):
                pk, s16, z16 = st.hist[(name, h)]
                assert np.array_equal(codes[:, h, i], pk), (case, b, h, name)
                assert np.array_equal(params[:, h, i, :, 0], s16), (case, b, h, name)
                assert np.array_equal(params[:, h, i, :, 1], z16), (case, b, h, name)
    check_windows(pool, w, b, L, k, v, range(w.num_kv_heads))
    if rows:
        ref = oracle.attend_sequence(st, q_bits, scale)
        err = oracle.row_rel_err(out_row.detach().cpu().numpy().astype(np.float64), ref)
        assert err <= TOL, (case, b, err)
    return st


def _params_seen(pool, w, b, L):
    n_hist = max(0, L - oracle.WINDOW)
    _, params = pool.export_history(b, 0, n_hist)
    return params


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("case", ["mixed", "tiny_clip", "large"])
def test_codec_edge_cases_through_every_encoder(case, shape):
    Hq, Hkv, d, G = SHAPES[shape]
    w = synth.Workload(f"edge_codec_{case}_{shape}", 50 + list(SHAPES).index(shape), len(LENGTHS), Hq, Hkv, d, G, 0, 0)
    lengths = list(LENGTHS)
    final = [L + STEPS for L in lengths]
    tk = [_tokens(w, 0, case, b, final[b]) for b in range(len(lengths))]
    tv = [_tokens(w, 1, case, b, final[b]) for b in range(len(lengths))]
    RK, RV, cK, cV = _tables(w, case)
    cfg = harness.config_for(w, lengths, extra_tokens=STEPS, slack_pages=2)
    pool = ok.Pool(cfg, RK, RV, cK, cV, max_batch=len(lengths))
    for b, L in enumerate(lengths):
        k = torch.from_numpy(tk[b][:L].view(np.int16)).cuda().view(torch.uint16)
        v = torch.from_numpy(tv[b][:L].view(np.int16)).cuda().view(torch.uint16)
        pool.prefill(b, k, v)
    # logits of order one for every case
    scale = (2.0 ** -12 if case == "large" else 1.0) / math.sqrt(d)
    ids = list(range(len(lengths)))
    for step in range(1, STEPS + 1):
        order = ids[step % len(ids):] + ids[: step % len(ids)]
        kn = np.stack([tk[b][lengths[b]] for b in order])
        vn = np.stack([tv[b][lengths[b]] for b in order])
        kn = torch.from_numpy(kn.view(np.int16)).cuda().view(torch.uint16)
        vn = torch.from_numpy(vn.view(np.int16)).cuda().view(torch.uint16)
        q = synth.queries(w, step, device="cuda", batch=len(ids))
        qo = q[torch.as_tensor(order, device="cuda")].contiguous().view(torch.uint16)
        # odd steps: the append kernel, then decode; even steps: the fused step
        if step % 2:
            pool.append(order, kn, vn)
            out = pool.decode(order, qo, softmax_scale=scale)
        else:
            out = pool.step(order, kn, vn, qo, softmax_scale=scale)
        for b in order:
            lengths[b] += 1
        if step in (1, 2, STEPS - 1, STEPS):
            torch.cuda.synchronize()
            qb = synth.bf16_bits(q.cpu())
            for i, b in enumerate(order):
                _check_seq(pool, w, case, b, lengths[b], tk, tv, qb[b], out[i], scale)
    # the degenerate parameters really occurred
    params = np.concatenate([_params_seen(pool, w, b, lengths[b]).reshape(-1, 2) for b in ids])
    s = params[:, 0]
    if case == "mixed":
        assert (s == 0).any()                           # zero range
        assert ((s > 0) & (s < 0x0400)).any()           # sub-normal fp16 scale
        assert (params[s == 0][:, 1] == 0).any()        # +0 zero point
    elif case == "tiny_clip":
        assert (s < 0x0400).all()                       # every scale sub-normal
    else:
        assert (s >= 0x7000).any()                      # scales >= 2^13
