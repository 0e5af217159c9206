"""Pins of the oracle's per-token codec against facts fixed outside the oracle:
IEEE binary16 rounding (numpy), exhaustive byte round trips, hand-worked
cases in tests/golden, and closed-form error bounds."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ---- binary16 ----------------------------------------------------------------

def test_f16_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_table()
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_f16_encode_ties_and_subnormals_match_numpy():
    rng = np.random.default_rng(7)
    # every finite fp16 value, every midpoint between neighbours (exact in fp32),
    # and points just beside the midpoints
    vals = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    beside = np.concatenate([np.nextafter(mids32, np.float32(np.inf)),
                             np.nextafter(mids32, np.float32(0))])
    rand = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 12, 20000))).astype(np.float32)
    edges = np.array([65504, 65519.99, 65520, 65536, 1e9, 2**-24, 2**-25, 2**-25 * 1.0000001,
                      2**-26, 2**-14, 2**-14 * 0.99999, 0.0], dtype=np.float32)
    x = np.concatenate([vals.astype(np.float32), mids32, beside, rand, edges])
    x = np.concatenate([x, -x])
    got = oracle.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


# ---- pack / unpack -----------------------------------------------------------

def test_pack_unpack_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    codes = oracle.unpack(b[None, :])[0]
    assert codes.max() <= 3
    # low bits first: byte 0b11100100 holds codes 0,1,2,3
    assert list(oracle.unpack(np.array([[0xE4]], dtype=np.uint8))[0]) == [0, 1, 2, 3]
    assert np.array_equal(oracle.pack(codes[None, :])[0], b)
    # the C unpack agrees with the numpy one
    out = np.empty(1024, dtype=np.uint8)
    oracle.lib().oracle_unpack(oracle._ptr(b), 1024, oracle._ptr(out))
    assert np.array_equal(out, codes)


# ---- rotation ----------------------------------------------------------------

def test_fma_chain_hand_worked_case():
    rows = [ln.split()[1:] for ln in _lines("fma_chain.txt") if ln.startswith("R ")]
    R = np.array([[int(h, 16) for h in r] for r in rows], dtype=np.uint32).view(np.float32)
    x = np.array([int(h, 16) for h in _lines("fma_chain.txt")[4].split()[1:]], dtype=np.uint16)
    want = np.array([int(h, 16) for h in _lines("fma_chain.txt")[5].split()[1:]], dtype=np.uint32)
    y = np.empty(4, dtype=np.float32)
    oracle.lib().oracle_rotate(oracle._ptr(x), oracle._ptr(np.ascontiguousarray(R)), 4, oracle._ptr(y))
    assert np.array_equal(y.view(np.uint32), want)


def test_rotation_is_row_vector_times_R():
    # a non-symmetric R: the C chain must agree with x @ R (not R @ x) up to
    # the fp32 accumulation bound d * 2^-24 * sum |x_i R_ij|
    rng = np.random.default_rng(3)
    d = 64
    R = rng.standard_normal((d, d)).astype(np.float32)
    x32 = rng.standard_normal((16, d)).astype(np.float32)
    xb = (x32.view(np.uint32) >> 16).astype(np.uint16)          # truncate to bf16
    xf = oracle.bf16_bits_to_f64(xb)
    y = np.empty((16, d), dtype=np.float32)
    oracle.lib().oracle_rotate_many(oracle._ptr(xb), 16, d, oracle._ptr(R), oracle._ptr(y))
    exact = xf @ R.astype(np.float64)
    bound = d * 2.0**-24 * (np.abs(xf) @ np.abs(R.astype(np.float64)))
    assert np.all(np.abs(y - exact) <= bound)
    wrong = xf @ R.astype(np.float64).T
    assert np.abs(y - wrong).max() > 1.0


# ---- quantization ------------------------------------------------------------

def test_quantize_hand_worked_cases():
    for ln in _lines("quantize_cases.txt"):
        ys, ps, cs, bs = [p.split() for p in ln.split("|")]
        y = np.array([float(v) for v in ys], dtype=np.float32)[None, :]
        codes, s16, z16 = oracle.quantize(y, 4)
        assert s16[0, 0] == int(ps[0], 16) and z16[0, 0] == int(ps[1], 16), ln
        assert list(codes[0]) == [int(c) for c in cs], ln
        assert oracle.pack(codes)[0, 0] == int(bs[0], 16), ln


def test_quantize_grid_round_trip_and_bounds():
    rng = np.random.default_rng(11)
    G, d = 32, 128
    # groups that already sit on a 4-level fp16 grid reproduce exactly
    z = oracle.f16_table()[oracle.f32_to_f16_bits(rng.uniform(-8, 8, 40).astype(np.float32))]
    s = np.array([0.25, 0.5, 0.75, 1.5, 3.0, 0.125, 2.0, 0.375] * 5)
    codes = rng.integers(0, 4, (40, G))
    codes[:, 0], codes[:, 1] = 0, 3                      # hit min and max
    y = (codes * s[:, None] + z[:, None]).astype(np.float32)
    assert np.array_equal(y.astype(np.float64), codes * s[:, None] + z[:, None])
    c2, s16, z16 = oracle.quantize(y, G)
    assert np.array_equal(c2, codes)
    assert np.array_equal(oracle.f16_table()[s16[:, 0]], s)
    # random groups: |dequant - y| <= s/2 + |z - min| + 3 |s - range/3| (closed form)
    y = (rng.standard_normal((200, d)) * rng.uniform(0.01, 50, (200, 1))).astype(np.float32)
    codes, s16, z16 = oracle.quantize(y, G)
    deq = oracle.dequantize(oracle.pack(codes), s16, z16, G)
    yg = y.astype(np.float64).reshape(200, d // G, G)
    mn, mx = yg.min(-1), yg.max(-1)
    sv, zv = oracle.f16_table()[s16], oracle.f16_table()[z16]
    bound = sv / 2 + np.abs(zv - mn) + 3 * np.abs(sv - (mx - mn) / 3)
    err = np.abs(deq.reshape(200, d // G, G) - yg).max(-1)
    assert np.all(err <= bound * (1 + 1e-6))
    # the group minimum maps to code 0 and the maximum to code 3
    cg = codes.reshape(200, d // G, G)
    assert np.all(np.take_along_axis(cg, yg.argmin(-1)[..., None], -1) == 0)
    assert np.all(np.take_along_axis(cg, yg.argmax(-1)[..., None], -1) == 3)


def test_constant_group_gives_zero_scale():
    y = np.full((1, 64), 3.3, dtype=np.float32)
    codes, s16, z16 = oracle.quantize(y, 64)
    assert s16[0, 0] == 0 and np.all(codes == 0)
    assert oracle.f16_table()[z16[0, 0]] == np.float16(3.3)


def test_encode_matches_steps():
    # encode = rotate -> clip -> quantize -> pack, composed from the pinned steps
    rng = np.random.default_rng(5)
    d, G = 128, 64
    R = np.linalg.qr(rng.standard_normal((d, d)))[0].astype(np.float32)
    c = np.full(d, 1.5, dtype=np.float32)
    x = (rng.standard_normal((8, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    pk, s16, z16 = oracle.encode(x, R, c, G)
    y = np.empty((8, d), dtype=np.float32)
    oracle.lib().oracle_rotate_many(oracle._ptr(x), 8, d, oracle._ptr(R), oracle._ptr(y))
    y = np.clip(y, -c, c)
    codes, s2, z2 = oracle.quantize(y, G)
    assert np.array_equal(pk, oracle.pack(codes))
    assert np.array_equal(s16, s2) and np.array_equal(z16, z2)
    assert np.abs(y).max() <= 1.5


def test_signed_zero_groups_store_plus_zero():
    # a group of zeros of both signs: range and minimum are stored as +0
    y = np.array([[0.0, -0.0, 0.0, -0.0], [-0.0, -0.0, -0.0, -0.0]], dtype=np.float32)
    codes, s16, z16 = oracle.quantize(y, 4)
    assert np.all(s16 == 0) and np.all(z16 == 0) and np.all(codes == 0)
