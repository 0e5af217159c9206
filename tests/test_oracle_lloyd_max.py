"""Pins of the oracle's Lloyd-Max codebook variant: the fit against closed
forms (a uniform distribution, two point masses, symmetric data), Lloyd's
own properties (the error never grows, the levels end at their cells'
means), hand-worked quantization cases, and agreement with the affine codec
for the codebook of uniform levels."""
import os

import numpy as np
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16(a):
    return synth.bf16_bits(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16))


def _cases():
    out = []
    cur = None
    for ln in open(os.path.join(HERE, "golden", "lloyd_max_cases.txt")):
        ln = ln.strip()
        if not ln or ln.startswith("#"):
            continue
        key, rest = ln.split(" ", 1)
        if key == "case":
            cur = {"L": np.array([int(x) for x in rest.split()], dtype=np.uint8)}
            out.append(cur)
        elif key == "y":
            runs = [r.strip().split(" x") for r in rest.split(",")]
            cur["runs"] = [(np.float32(float(v)), int(n)) for v, n in runs]
        elif key == "codes":
            cur["codes"] = [int(c) for c in rest.split(",")]
    return out


def test_quantize_hand_worked():
    for c in _cases():
        y = np.concatenate([np.full(n, v, dtype=np.float32) for v, n in c["runs"]])
        assert len(y) == 64
        codes = np.empty(64, np.uint8)
        s16 = np.empty(1, np.uint16)
        z16 = np.empty(1, np.uint16)
        oracle.lib().oracle_quantize_lut(oracle._ptr(y), 64, 64, oracle._ptr(c["L"]), oracle._ptr(codes),
                                         oracle._ptr(s16), oracle._ptr(z16))
        want = np.concatenate([np.full(n, code) for (v, n), code in
                               zip(c["runs"], c["codes"] * (len(c["runs"]) if len(c["codes"]) == 1 else 1))])
        assert np.array_equal(codes, want), (c["L"], codes)


def test_fit_uniform_distribution():
    # uniform on [0, 3]: the optimal cells are the four quarters, levels at
    # their midpoints 0.375, 1.125, 1.875, 2.625 -> 24, 72, 120, 168
    u = ((np.arange(300000) + 0.5) / 100000).astype(np.float32)
    assert np.allclose(oracle.lloyd_max_levels(u), [0.375, 1.125, 1.875, 2.625], atol=2e-5)
    assert list(oracle.lloyd_max_codebook(u)) == [24, 72, 120, 168]


def test_fit_two_point_masses_keeps_empty_cells():
    u = np.r_[np.zeros(100), np.full(100, 3.0)].astype(np.float32)
    assert list(oracle.lloyd_max_codebook(u)) == [0, 64, 128, 192]


def test_fit_symmetric_data_gives_a_symmetric_codebook():
    # values v and 3 - v on the fit's own grid (multiples of 2^-20, exact in
    # fp32), odd multiples so none lies on the first thresholds 0.5, 1.5, 2.5
    rng = np.random.default_rng(0)
    k = 2 * rng.integers(0, 3 * 2 ** 19, 5000) + 1
    u = (np.r_[k, 3 * 2 ** 20 - k] / 2.0 ** 20).astype(np.float32)
    lv = oracle.lloyd_max_levels(u)
    assert np.allclose(lv + lv[::-1], 3.0, atol=1e-12)
    L = oracle.lloyd_max_codebook(u).astype(int)
    assert all(L[k] + L[3 - k] == 192 for k in range(4))


def test_fit_error_never_grows_and_ends_at_the_cell_means():
    rng = np.random.default_rng(1)
    u = np.clip(rng.normal(1.5, 0.6, 20000), 0, 3).astype(np.float32)
    U = np.rint(u.astype(np.float64) * oracle.LLOYD_GRID) / oracle.LLOYD_GRID

    def mse(lv):
        thr = (lv[:-1] + lv[1:]) / 2
        return ((U - lv[(U[:, None] > thr[None, :]).sum(1)]) ** 2).mean()

    errs = [mse(oracle.lloyd_max_levels(u, it)) for it in range(12)]
    assert all(b <= a + 1e-15 for a, b in zip(errs, errs[1:]))
    assert errs[-1] < 0.8 * errs[0]
    lv = oracle.lloyd_max_levels(u)
    thr = (lv[:-1] + lv[1:]) / 2
    cell = (U[:, None] > thr[None, :]).sum(1)
    assert np.allclose([U[cell == k].mean() for k in range(4)], lv, atol=1e-6)


def test_fit_hand_worked_tie():
    # u = 0, 0.5, 3: the first thresholds are 0.5, 1.5, 2.5, so 0.5 lies on
    # one and joins the lower cell: levels 0.25, 1 (empty), 2 (empty), 3;
    # the next thresholds 0.625, 1.5, 2.5 keep the cells -> 16, 64, 128, 192
    u = np.array([0.0, 0.5, 3.0], np.float32)
    assert list(oracle.lloyd_max_levels(u, 1)) == [0.25, 1.0, 2.0, 3.0]
    assert list(oracle.lloyd_max_codebook(u)) == [16, 64, 128, 192]


def test_fit_ignores_groups_without_scale():
    u = ((np.arange(300000) + 0.5) / 100000).astype(np.float32)
    assert list(oracle.lloyd_max_codebook(np.r_[u, np.full(5000, np.nan, np.float32)])) == [24, 72, 120, 168]


def test_uniform_codebook_matches_the_affine_codec_off_ties():
    # L = 0, 64, 128, 192 puts the levels at z + k s: the codes are the
    # affine ones except at u = 1.5 exactly (rint rounds that to 2, the
    # codebook to the lower level); decoding gives the same values
    rng = np.random.default_rng(2)
    d, G = 128, 64
    x = _bf16(rng.standard_normal((200, d)) * np.exp(rng.normal(0, 2, (200, 1))))
    R = np.eye(d, dtype=np.float32)
    clip = np.full(d, 1e4, dtype=np.float32)
    L = np.array([0, 64, 128, 192], np.uint8)
    pa, sa, za = oracle.encode(x, R, clip, G)
    pl, sl, zl = oracle.encode_lut(x, R, clip, G, L)
    assert np.array_equal(sa, sl) and np.array_equal(za, zl)
    u = oracle.normalized_values(x, R, clip, G)
    ca, cl = oracle.unpack(pa), oracle.unpack(pl)
    assert np.array_equal(ca[u != 1.5], cl[u != 1.5])
    assert np.all(cl[u == 1.5] == 1)
    same = ca == cl
    assert np.array_equal(oracle.dequantize(pa, sa, za, G)[same], oracle.dequantize_lut(pl, sl, zl, G, L)[same])
    # and back in the original basis, with a real rotation: the same tokens
    U = np.linalg.qr(rng.standard_normal((d, d)))[0]
    Rr = oracle.rotation(oracle.rotation_grid(U))
    pa, sa, za = oracle.encode(x, Rr, clip, G)
    pl, sl, zl = oracle.encode_lut(x, Rr, clip, G, L)
    rows = np.all(oracle.unpack(pa) == oracle.unpack(pl), axis=1)
    assert rows.sum() > 100
    assert np.allclose(oracle.decode_history(pa, sa, za, G, Rr)[rows],
                       oracle.decode_history_lut(pl, sl, zl, G, L, Rr)[rows], rtol=0, atol=1e-12)


def test_nearest_level_and_error_bound():
    # every channel's level is the nearest of the four (the midpoint rule),
    # so |y - level| <= s * max(L_0, (L_{k+1} - L_k) / 2, 192 - L_3) / 64 up
    # to the fp16 rounding of s and z
    rng = np.random.default_rng(3)
    d, G = 128, 128
    x = _bf16(rng.standard_normal((300, d)) * np.exp(rng.normal(0, 2, (300, 1))))
    R = np.eye(d, dtype=np.float32)
    clip = np.full(d, 1e30, dtype=np.float32)
    L = np.array([40, 79, 114, 154], np.uint8)
    pk, s16, z16 = oracle.encode_lut(x, R, clip, G, L)
    u = oracle.normalized_values(x, R, clip, G).astype(np.float64)
    lv = L.astype(np.float64) / 64
    best = np.abs(u[..., None] - lv).min(-1)
    got = np.abs(u - lv[oracle.unpack(pk)])
    assert np.all(got <= best + 1e-12)
