"""The oracle's pins catch plausible mistakes.

C codec: each case copies oracle/oscar_oracle.c, plants one mistake by a
textual edit, builds the copy with the same flags and runs the codec pins
(tests/test_oracle_codec.py) against it.  Python parts: each case replaces
one oracle function, for the test's duration only, by a copy with one
mistake and runs the rotation, attention and pool pins.  Either way at least
one pin must fail.  The oracle's own files are never modified."""
import ctypes
import math
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_attention
import test_oracle_calibration
import test_oracle_codec as pins
import test_oracle_lloyd_max
import test_oracle_pool
import test_oracle_rotation

# name: (text in oscar_oracle.c, replacement)
MISTAKES = {
    "rotation unfused (mul, then add)": (
        "acc = fmaf(bf16_to_f32(x[i]), R[(size_t)i * d + j], acc);",
        "acc = bf16_to_f32(x[i]) * R[(size_t)i * d + j] + acc;"),
    "rotation summed in reverse order": (
        "for (int i = 0; i < d; ++i)\n            acc = fmaf(",
        "for (int i = d - 1; i >= 0; --i)\n            acc = fmaf("),
    "rotation R x instead of x R": (
        "R[(size_t)i * d + j], acc)",
        "R[(size_t)j * d + i], acc)"),
    "clip on one side only": (
        "y[j] = fminf(fmaxf(y[j], -c[j]), c[j]);",
        "y[j] = fminf(y[j], c[j]);"),
    "codes rounded half away from zero": (
        "q = rintf((v[k] - z) / s);",
        "q = roundf((v[k] - z) / s);"),
    "codes from the unrounded scale": (
        "float s = oracle_f16_to_f32(s16);",
        "float s = range / 3.0f;"),
    "codes from the unrounded zero point": (
        "float z = oracle_f16_to_f32(z16);",
        "float z = mn;"),
    "negative zero kept as the zero point": (
        "oracle_f32_to_f16(mn + 0.0f)",
        "oracle_f32_to_f16(mn)"),
    "codes not clamped to 0..3": (
        "q = fminf(fmaxf(q, 0.0f), 3.0f);",
        "(void)0;"),
    "codes by the reciprocal of the scale": (
        "q = rintf((v[k] - z) / s);",
        "q = rintf((v[k] - z) * (1.0f / s));"),
    "scale from the range times fp32(1/3)": (
        "oracle_f32_to_f16(range / 3.0f)",
        "oracle_f32_to_f16(range * (1.0f / 3.0f))"),
    "group minimum and maximum skip an element": (
        "for (int k = 1; k < G; ++k) {",
        "for (int k = 2; k < G; ++k) {"),
    "pack with the first code in the high bits": (
        "codes[4 * b] | (codes[4 * b + 1] << 2) |\n                             (codes[4 * b + 2] << 4) | (codes[4 * b + 3] << 6)",
        "(codes[4 * b] << 6) | (codes[4 * b + 1] << 4) |\n                             (codes[4 * b + 2] << 2) | codes[4 * b + 3]"),
    "codebook ties to the upper level": (
        "c = (u > t[0]) + (u > t[1]) + (u > t[2]);",
        "c = (u >= t[0]) + (u >= t[1]) + (u >= t[2]);"),
    "codebook thresholds at the upper levels": (
        "t[k] = (float)(L[k] + L[k + 1]) / 128.0f;",
        "t[k] = (float)L[k + 1] / 64.0f;"),
    "normalised value without the zero point": (
        "u[g * G + k] = s != 0.0f ? (y[g * G + k] - z) / s : NAN;",
        "u[g * G + k] = s != 0.0f ? y[g * G + k] / s : NAN;"),
    "unpack from the high bits": (
        "codes[i] = (bytes[i / 4] >> (2 * (i % 4))) & 3;",
        "codes[i] = (bytes[i / 4] >> (2 * (3 - i % 4))) & 3;"),
}

PINS = ([getattr(pins, n) for n in dir(pins) if n.startswith("test_")]
        + [getattr(test_oracle_lloyd_max, n) for n in dir(test_oracle_lloyd_max) if n.startswith("test_")])


def _planted(tmp_path, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, old
    c = tmp_path / "planted.c"
    c.write_text(src.replace(old, new))
    so = tmp_path / "libplanted.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", str(so), str(c), "-lm"])
    return oracle.configure(ctypes.CDLL(str(so)))


@pytest.mark.parametrize("name", list(MISTAKES))
def test_planted_mistake_fails_a_pin(name, tmp_path, monkeypatch):
    monkeypatch.setattr(oracle, "_lib", _planted(tmp_path, *MISTAKES[name]))
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no codec pin catches: {name}"


def test_unplanted_copy_passes_every_pin(tmp_path, monkeypatch):
    # the same machinery with no edit: every pin passes, so a failure above
    # is the planted mistake's
    monkeypatch.setattr(oracle, "_lib", _planted(tmp_path, "void oracle_rotate(", "void oracle_rotate("))
    for pin in PINS:
        pin()


def _calls(module):
    """The module's pins as zero-argument calls (parametrized ones expanded)."""
    out = []
    for name in dir(module):
        fn = getattr(module, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            out.append((name, fn))
            continue
        argname, values = marks[0].args[0], marks[0].args[1]
        out += [(f"{name}[{v}]", (lambda f, v: lambda: f(v))(fn, v)) for v in values]
    return out


PY_PINS = (_calls(test_oracle_rotation) + _calls(test_oracle_attention) + _calls(test_oracle_pool)
           + _calls(test_oracle_calibration) + _calls(test_oracle_lloyd_max))


def _bad_hadamard(d):
    i, j = np.arange(d)[:, None], np.arange(d)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i | j)
    return np.where(pc % 2 == 0, 1.0, -1.0)


def _bad_rotation(U):
    U = np.asarray(U, dtype=np.float32)
    d = U.shape[-1]
    S = oracle.hadamard_unnormalized(d) @ oracle.bitrev_permutation(d) @ U.astype(np.float64)
    return (S / math.sqrt(float(d))).astype(np.float32)


def _bad_percentile(a, pct):
    n = len(a)
    h = n * (pct / 100.0)
    k = min(int(math.floor(h)), n - 1)
    return float(a[k]) + (h - k) * (float(a[min(k + 1, n - 1)]) - float(a[k]))


def _bad_free_list(num_pages, seed):
    a = list(range(num_pages))
    g = oracle.splitmix64_stream(seed)
    for i in range(num_pages - 1, 0, -1):
        j = next(g) % i
        a[i], a[j] = a[j], a[i]
    return a


def _bad_attention(q, K, V, scale):
    logits = scale * (K @ q)
    w = np.exp(logits - logits.max())
    return w @ V


def _bad_merge(parts):
    m = max(p[0] for p in parts)
    l, acc = 0.0, 0.0
    for mi, li, ai in parts:
        w = 0.0 if mi == -math.inf else math.exp(m - mi)
        l, acc = l + w * li, acc + w * ai
    return m, l, acc


def _bad_segments(L):
    n_hist = max(0, L - oracle.WINDOW + 1)
    return (range(0, min(L, oracle.SINK)), range(oracle.SINK, oracle.SINK + n_hist),
            range(oracle.SINK + n_hist, max(L, oracle.SINK + n_hist)))


def _bad_append(self, seq_ids):
    for s_ in seq_ids:
        L = self.length.get(s_, 0)
        if L >= oracle.WINDOW and (L - oracle.WINDOW) % oracle.PAGE == 1:
            self.table.setdefault(s_, []).append(self._take())
        self.length[s_] = L + 1


def _rel_err_variant(kind):
    def f(got, ref):
        got = np.asarray(got, dtype=np.float64).reshape(-1, ref.shape[-1])
        ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
        diff = np.abs(got - ref)
        if kind == "global":
            return float(diff.max() / np.abs(ref).max())
        if kind == "got":
            return float((diff.max(axis=1) / np.abs(got).max(axis=1)).max())
        if kind == "mean":
            return float((diff.max(axis=1) / np.abs(ref).max(axis=1)).mean())
        if kind == "l2":
            return float((np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)).max())
        return float((diff.max(axis=1) / ref.max(axis=1)).max())  # signed maximum
    return f


def _prefill_variant(kind):
    def f(st, q_bf16, scale, heads=None):
        n_q, Hq, d = q_bf16.shape
        L = st.L
        g = Hq // st.K.shape[1]
        q = oracle.bf16_bits_to_f64(q_bf16)
        pos = (np.arange(n_q) if kind == "first" else L - n_q + np.arange(n_q))
        if kind == "self":
            visible = np.arange(L)[None, :] < pos[:, None]
        elif kind == "late":
            visible = np.arange(L)[None, :] <= pos[:, None] + 1
        elif kind == "none":
            visible = np.ones((n_q, L), dtype=bool)
        else:
            visible = np.arange(L)[None, :] <= pos[:, None]
        out = np.full((n_q, Hq, d), np.nan)
        for h in (range(Hq) if heads is None else heads):
            logits = np.where(visible, scale * (q[:, h, :] @ st.K[:, h // g, :].T), -np.inf)
            w = np.exp(logits - logits.max(axis=1, keepdims=True))
            out[:, h, :] = (w @ st.V[:, h // g, :]) / w.sum(axis=1, keepdims=True)
        return out
    return f


def _scores_no_mask(q, k, scale):
    logits = scale * (q @ k.T)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def _value_cov_variant(kind):
    def f(q_bf16, k_bf16, v_bf16, scale):
        q, k, v = (oracle.bf16_bits_to_f64(x) for x in (q_bf16, k_bf16, v_bf16))
        n, Hq, d = q.shape
        Hkv = k.shape[1]
        g = Hq // Hkv
        C = np.zeros((Hkv, d, d))
        for h in range(Hq):
            S = oracle.causal_scores(q[:, h, :], k[:, h // g, :], scale)
            V = v[:, h // g, :]
            if kind == "S":
                C[h // g] += V.T @ S @ V
            elif kind == "mean":
                C[h // g] += V.T @ S.T @ S @ V / g
            else:  # keys in place of the values
                K = k[:, h // g, :]
                C[h // g] += K.T @ S.T @ S @ K
        return C
    return f


def _query_cov_mod(q_bf16, num_kv_heads):
    q = oracle.bf16_bits_to_f64(q_bf16)
    n, Hq, d = q.shape
    C = np.zeros((num_kv_heads, d, d))
    for h in range(Hq):
        C[h % num_kv_heads] += q[:, h, :].T @ q[:, h, :]
    return C


def _eigen_variant(kind):
    def f(C):
        w, V = np.linalg.eigh(np.asarray(C, dtype=np.float64))
        if kind == "ascending":
            return V, w
        order = np.argsort(-w, kind="stable")
        return V[:, order], w[order]   # no sign convention
    return f


def _lloyd_variant(kind):
    def f(u, iters=oracle.LLOYD_ITERS):
        u = np.asarray(u, dtype=np.float32).ravel()
        U = np.rint(u[~np.isnan(u)].astype(np.float64) * oracle.LLOYD_GRID).astype(np.int64)
        lev = np.array([0.5, 1.5, 2.5, 3.5]) if kind == "init" else np.array([0.0, 1.0, 2.0, 3.0])
        for _ in range(iters):
            thr = (lev[:-1] + lev[1:]) * (oracle.LLOYD_GRID / 2)
            cell = ((U[:, None] >= thr[None, :]) if kind == "ge" else (U[:, None] > thr[None, :])).sum(axis=1)
            new = np.zeros(4) if kind == "empty0" else lev.copy()
            for k in range(4):
                sel = U[cell == k]
                if len(sel):
                    new[k] = float(int(sel.sum())) / float(len(sel)) / oracle.LLOYD_GRID
            lev = new
        return lev
    return f


def _dequant_lut_32(packed, s16, z16, G, L):
    codes = oracle.unpack(packed)
    lv = np.asarray(L, dtype=np.float64)[codes] / 32.0
    s = np.repeat(oracle.f16_table()[s16], G, axis=-1)
    z = np.repeat(oracle.f16_table()[z16], G, axis=-1)
    return lv * s + z


PY_MISTAKES = {
    "bit reversal left out": ("bitrev", lambda i, bits: i),
    "Hadamard sign from popcount(i | j)": ("hadamard_unnormalized", _bad_hadamard),
    "R = Hadamard . bit-reversal . U": ("rotation", _bad_rotation),
    "percentile position N p instead of (N - 1) p": ("percentile_linear", _bad_percentile),
    "Fisher-Yates j = next() mod i": ("free_list", _bad_free_list),
    "history decoded by R instead of R^T": ("decode_history",
                                             lambda pk, s16, z16, G, R: oracle.dequantize(pk, s16, z16, G) @ np.asarray(R, dtype=np.float64)),
    "softmax weights not normalised": ("attention", _bad_attention),
    "merge weights exp(m - m_i)": ("merge_partials", _bad_merge),
    "history starts one token early": ("segments", _bad_segments),
    "recent ring of 255 slots": ("ring_slot", lambda pos: (pos - oracle.SINK) % 255),
    "bits per element with one fp16 parameter": ("bits_per_element",
                                                 lambda L, G: (max(0, L - oracle.WINDOW) * (2 + 16 / G) + min(L, oracle.WINDOW) * 16) / L),
    "row error as one ratio over all rows": ("row_rel_err", _rel_err_variant("global")),
    "row error relative to the result, not the reference": ("row_rel_err", _rel_err_variant("got")),
    "row errors averaged instead of the largest": ("row_rel_err", _rel_err_variant("mean")),
    "row error in Euclidean norms": ("row_rel_err", _rel_err_variant("l2")),
    "row error over the signed maximum of the reference": ("row_rel_err", _rel_err_variant("signed")),
    "prefill query does not see its own position": ("prefill_attention", _prefill_variant("self")),
    "prefill query sees one position too many": ("prefill_attention", _prefill_variant("late")),
    "prefill queries taken at the first positions": ("prefill_attention", _prefill_variant("first")),
    "prefill without the causal mask": ("prefill_attention", _prefill_variant("none")),
    "calibration scores without the causal mask": ("causal_scores", _scores_no_mask),
    "value covariance V^T S V": ("value_covariance", _value_cov_variant("S")),
    "value covariance averaged over the query heads": ("value_covariance", _value_cov_variant("mean")),
    "value covariance of the keys": ("value_covariance", _value_cov_variant("K")),
    "query head h to kv head h mod Hkv": ("query_covariance", _query_cov_mod),
    "eigenvalues ascending": ("eigenbasis", _eigen_variant("ascending")),
    "eigenvector signs left as computed": ("eigenbasis", _eigen_variant("nosign")),
    "U not rounded to the grid": ("rotation_grid", lambda U: np.asarray(U, dtype=np.float32)),
    "Lloyd cells take values on a threshold upward": ("lloyd_max_levels", _lloyd_variant("ge")),
    "Lloyd empty cell set to 0": ("lloyd_max_levels", _lloyd_variant("empty0")),
    "Lloyd started from levels 0.5, 1.5, 2.5, 3.5": ("lloyd_max_levels", _lloyd_variant("init")),
    "codebook levels rounded down": ("lloyd_max_codebook",
                                     lambda u, iters=oracle.LLOYD_ITERS: np.clip(np.floor(oracle.lloyd_max_levels(u, iters) * 64), 0, 255).astype(np.uint8)),
    "codebook levels read as L / 32": ("dequantize_lut", _dequant_lut_32),
    "Lloyd-Max history decoded by R instead of R^T": (
        "decode_history_lut",
        lambda pk, s16, z16, G, L, R: oracle.dequantize_lut(pk, s16, z16, G, L) @ np.asarray(R, dtype=np.float64)),
}


@pytest.mark.parametrize("name", list(PY_MISTAKES))
def test_planted_python_mistake_fails_a_pin(name, monkeypatch):
    attr, bad = PY_MISTAKES[name]
    monkeypatch.setattr(oracle, attr, bad)
    failed = []
    for pin_name, pin in PY_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin_name)
    assert failed, f"no pin catches: {name}"


def test_planted_page_allocation_mistake_fails_a_pin(monkeypatch):
    monkeypatch.setattr(oracle.PoolModel, "append", _bad_append)
    failed = []
    for pin_name, pin in PY_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin_name)
    assert failed, "no pin catches a page taken one slot late"


def _append_no_cow(self, seq_ids):
    for s_ in seq_ids:
        L = self.length.get(s_, 0)
        if L >= oracle.WINDOW and (L - oracle.WINDOW) % oracle.PAGE == 0:
            self.table.setdefault(s_, []).append(self._take())
        self.length[s_] = L + 1


def _append_cow_before_peers(self, seq_ids):
    # copy on write taken after every new page of the call, not in call order
    later = []
    for s_ in seq_ids:
        L = self.length.get(s_, 0)
        if L >= oracle.WINDOW:
            n_hist = L - oracle.WINDOW
            if n_hist % oracle.PAGE == 0:
                self.table.setdefault(s_, []).append(self._take())
            elif self.refs[self.table[s_][n_hist // oracle.PAGE]] > 1:
                later.append((s_, n_hist // oracle.PAGE))
        self.length[s_] = L + 1
    for s_, i in later:
        self.refs[self.table[s_][i]] -= 1
        self.table[s_][i] = self._take()


def _release_ignoring_refs(self, seq):
    self.free.extend(self.table.get(seq, []))
    self.table[seq] = []
    self.length[seq] = 0


def _fork_without_refs(self, src, dst):
    self.table[dst] = list(self.table.get(src, []))
    self.length[dst] = self.length.get(src, 0)


POOL_MISTAKES = {
    "shared page written in place (no copy on write)": ("append", _append_no_cow),
    "copies on write taken after the call's new pages": ("append", _append_cow_before_peers),
    "release frees pages other sequences hold": ("release", _release_ignoring_refs),
    "fork does not count the shared pages": ("fork", _fork_without_refs),
}


@pytest.mark.parametrize("name", list(POOL_MISTAKES))
def test_planted_prefix_sharing_mistake_fails_a_pin(name, monkeypatch):
    attr, bad = POOL_MISTAKES[name]
    monkeypatch.setattr(oracle.PoolModel, attr, bad)
    failed = []
    for pin_name, pin in PY_PINS:
        try:
            pin()
        except (AssertionError, KeyError):
            failed.append(pin_name)
    assert failed, f"no pin catches: {name}"


def test_python_pins_pass_unplanted():
    for pin_name, pin in PY_PINS:
        pin()
