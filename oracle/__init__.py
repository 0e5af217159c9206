"""CPU oracle for OSCAR's three-segment INT2 KV pool and its decode attention.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library ``bit_kv_cache_segment_amd`` and never imports it;
the seeded generators in ``synth`` are the only thing both sides use.

What is computed, and where it is described (the news article on OSCAR,
"Beyond TurboQuant: Together AI brings 2-bit KV Cache to real serving",
sanyangsrq.com, cited below as "the article"):

* R = U . Hadamard . bit-reversal (article, section "OSCAR aims the rotation
  at attention": U aligns attention-relevant directions, the Hadamard matrix
  spreads outlier energy, the bit-reversal permutation balances the INT2
  groups).  ``rotation``.
* clip thresholds fixed offline per layer and head from a few calibration
  samples (same section).  ``clip_thresholds``; the percentile is our
  reading.
* the per-token codec rotate -> clip -> quantize -> pack, four 2-bit values
  per byte (section "From offline calibration to online inference").
  ``encode`` (plain C in ``oscar_oracle.c``).
* the three-segment token pool: BF16 sink of 64 tokens | INT2 history |
  BF16 recent window of 256 tokens; new tokens enter the recent window and
  the oldest recent token moves to the history (same section).
  ``segments``, ``ring_slot``, ``PoolModel``.
* decode attention: the INT2 part is unpacked and dequantized with scale and
  zero point, the BF16 part covers sink and recent, and the two are merged
  by an online softmax (same section).  The oracle computes the *plain
  definition* this decomposition reaches: softmax attention over every token
  of the decoded pool, in fp64 (``attention``), where a history token decodes
  to dequant(codes) . R^T.  ``partial_attention``/``merge_partials`` write
  out the online-softmax merge itself so that its equality with one softmax
  can be pinned.
* prefill attention over the pool: each of the last n_q positions attends
  causally (to itself and every earlier position) over the same decoded
  pool.  ``prefill_attention``.
* calibration: the query covariance Q^T Q sets U for K, the score-weighted
  value covariance V^T S^T S V sets U for V (section "OSCAR aims the
  rotation at attention"); U is their eigenbasis.  ``query_covariance``,
  ``value_covariance``, ``eigenbasis``, ``calibrate_layer``.

Parity pins live in ``tests/test_oracle_*.py``.  Parity unpinned: the
relation of the synthetic quantization error to the article's accuracy
figures (no model weights or datasets exist here).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

SINK = 64
RECENT = 256
PAGE = 64
WINDOW = SINK + RECENT

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oscar_oracle.c")
_LIB = os.path.join(_HERE, "liboscar_oracle.so")


# gcc flags of the C codec: no fast-math, no FP contraction; -mfma lets fmaf,
# which is exact either way, compile to the hardware instruction.
CFLAGS = ["-O2", "-mfma", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile the C codec with gcc (CFLAGS)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = configure(ctypes.CDLL(build()))
    return _lib


def configure(L):
    """Declare the C codec's signatures on a loaded library (also used by the
    tests that load a copy of the codec with a planted mistake)."""
    P = ctypes.c_void_p
    L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    L.oracle_f32_to_f16.restype = ctypes.c_uint16
    L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_f16_to_f32.restype = ctypes.c_float
    L.oracle_rotate.argtypes = [P, P, ctypes.c_int, P]
    L.oracle_clip.argtypes = [P, P, ctypes.c_int]
    L.oracle_quantize.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P]
    L.oracle_pack.argtypes = [P, ctypes.c_int, P]
    L.oracle_unpack.argtypes = [P, ctypes.c_int, P]
    L.oracle_encode.argtypes = [P, ctypes.c_long, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
    L.oracle_normalized.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    L.oracle_quantize_lut.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P, P]
    L.oracle_encode_lut.argtypes = [P, ctypes.c_long, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P]
    L.oracle_normalized_many.argtypes = [P, ctypes.c_long, ctypes.c_int, ctypes.c_int, P, P, P]
    L.oracle_rotate_many.argtypes = [P, ctypes.c_long, ctypes.c_int, P, P]
    return L


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    L = lib()
    return np.array([L.oracle_f32_to_f16(float(v)) for v in x.ravel()],
                    dtype=np.uint16).reshape(x.shape)


def f16_bits_to_f64(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    L = lib()
    return np.array([L.oracle_f16_to_f32(int(v)) for v in h.ravel()],
                    dtype=np.float64).reshape(h.shape)


def bf16_bits_to_f64(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# R = U . H . Pi  (article, "OSCAR aims the rotation at attention")
# ---------------------------------------------------------------------------

def bitrev(i: int, bits: int) -> int:
    r = 0
    for _ in range(bits):
        r = (r << 1) | (i & 1)
        i >>= 1
    return r


def hadamard_unnormalized(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix in natural order: H[i][j] = (-1)^popcount(i & j)."""
    i = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(pc % 2 == 0, 1.0, -1.0)


def bitrev_permutation(d: int) -> np.ndarray:
    """Pi[i][j] = 1 iff j = bitrev(i) (symmetric, an involution)."""
    bits = d.bit_length() - 1
    P = np.zeros((d, d))
    for i in range(d):
        P[i, bitrev(i, bits)] = 1.0
    return P


def rotation(U: np.ndarray) -> np.ndarray:
    """fp32 R = U . (H_unnormalized / sqrt(d)) . Pi for each head, U fp32 [..][d][d].

    U . H_unnormalized . Pi is exact in fp64 because U lies on a 2**-40 grid
    (see ``synth.random_orthogonal_u``); the single division by sqrt(d) is
    then rounded to fp64 and that result to fp32.
    """
    U = np.asarray(U, dtype=np.float32)
    d = U.shape[-1]
    H = hadamard_unnormalized(d)
    P = bitrev_permutation(d)
    S = U.astype(np.float64) @ H @ P
    return (S / math.sqrt(float(d))).astype(np.float32)


# ---------------------------------------------------------------------------
# clip thresholds (offline, per head and rotated channel)
# ---------------------------------------------------------------------------

CLIP_PERCENTILE = 99.0


def percentile_linear(sorted_vals: np.ndarray, pct: float) -> float:
    """Linear-interpolation percentile of an ascending fp32 array, in fp64:
    h = (N-1) pct/100, k = floor(h), lo + (h - k)(hi - lo)."""
    n = len(sorted_vals)
    h = (n - 1) * (pct / 100.0)
    k = int(math.floor(h))
    lo = float(sorted_vals[k])
    hi = float(sorted_vals[min(k + 1, n - 1)])
    return lo + (h - k) * (hi - lo)


def clip_thresholds(calib_bf16: np.ndarray, R: np.ndarray, pct: float = CLIP_PERCENTILE) -> np.ndarray:
    """c[j] = percentile of |(x R)[j]| over calibration tokens, rounded to fp32.

    calib_bf16: uint16 [N][d]; R fp32 [d][d].  The rotation is the same fp32
    FMA chain the codec uses.
    """
    x = np.ascontiguousarray(calib_bf16, dtype=np.uint16)
    R = np.ascontiguousarray(R, dtype=np.float32)
    N, d = x.shape
    y = np.empty((N, d), dtype=np.float32)
    lib().oracle_rotate_many(_ptr(x), N, d, _ptr(R), _ptr(y))
    a = np.sort(np.abs(y), axis=0)
    return np.array([percentile_linear(a[:, j], pct) for j in range(d)], dtype=np.float32)


# ---------------------------------------------------------------------------
# calibration statistics and the eigenbasis U (offline, per layer and head)
# ---------------------------------------------------------------------------

def query_covariance(q_bf16: np.ndarray, num_kv_heads: int) -> np.ndarray:
    """fp64 [Hkv][d][d]: Q^T Q per kv head, summed over the query heads that
    share it (query head h belongs to kv head h // g).

    The article (section "OSCAR aims the rotation at attention") has the K
    rotation follow the query covariance, because K's error reaches the
    logits through Q K^T.  q_bf16: uint16 [n][Hq][d] calibration queries."""
    q = bf16_bits_to_f64(q_bf16)
    n, Hq, d = q.shape
    g = Hq // num_kv_heads
    C = np.zeros((num_kv_heads, d, d))
    for h in range(Hq):
        C[h // g] += q[:, h, :].T @ q[:, h, :]
    return C


def causal_scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S [n][n] fp64: row t is the softmax of scale q_t . k_j over j <= t
    (zero for j > t): the attention scores of a calibration sequence."""
    n = q.shape[0]
    logits = scale * (q @ k.T)
    logits[np.triu_indices(n, 1)] = -np.inf
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def value_covariance(q_bf16: np.ndarray, k_bf16: np.ndarray, v_bf16: np.ndarray, scale: float) -> np.ndarray:
    """fp64 [Hkv][d][d]: V^T S^T S V per kv head, summed over its query
    heads, S the causal attention scores of that query head (same section:
    V's error is weighted by the scores before it reaches the output).
    q_bf16 uint16 [n][Hq][d]; k_bf16, v_bf16 uint16 [n][Hkv][d]."""
    q = bf16_bits_to_f64(q_bf16)
    k = bf16_bits_to_f64(k_bf16)
    v = bf16_bits_to_f64(v_bf16)
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    C = np.zeros((Hkv, d, d))
    for h in range(Hq):
        S = causal_scores(q[:, h, :], k[:, h // g, :], scale)
        V = v[:, h // g, :]
        C[h // g] += V.T @ S.T @ S @ V
    return C


def eigenbasis(C: np.ndarray):
    """(U [d][d], eigenvalues [d]) of a symmetric matrix, fp64: the columns
    of U are orthonormal eigenvectors, eigenvalues in descending order, and
    each column's entry of largest magnitude (the first such) is positive.
    The order and the sign are our reading (the article fixes neither)."""
    w, V = np.linalg.eigh(np.asarray(C, dtype=np.float64))
    order = np.argsort(-w, kind="stable")
    w, V = w[order], V[:, order]
    for c in range(V.shape[1]):
        if V[np.argmax(np.abs(V[:, c])), c] < 0:
            V[:, c] = -V[:, c]
    return V, w


def rotation_grid(U: np.ndarray) -> np.ndarray:
    """U as ``rotation`` takes it: rounded to fp32, then to the nearest
    multiple of 2**-40 (so that U . H . Pi is exact in fp64)."""
    u = np.asarray(U, dtype=np.float32).astype(np.float64)
    return (np.round(u * 2.0**40) / 2.0**40).astype(np.float32)


def calibrate_layer(q_bf16, k_bf16, v_bf16, scale: float, pct: float = CLIP_PERCENTILE):
    """The offline step of one layer from one calibration sequence: per kv
    head, U_K from the query covariance and U_V from the score-weighted
    value covariance, R = U . H . Pi, and clip thresholds of the calibration
    K and V tokens rotated by R.  Returns (R_K, R_V, clip_K, clip_V), fp32."""
    Hkv = k_bf16.shape[1]
    CK = query_covariance(q_bf16, Hkv)
    CV = value_covariance(q_bf16, k_bf16, v_bf16, scale)
    out = []
    for C in (CK, CV):
        out.append(np.stack([rotation(rotation_grid(eigenbasis(C[h])[0])) for h in range(Hkv)]))
    clips = [np.stack([clip_thresholds(np.ascontiguousarray(x[:, h, :]), out[i][h], pct) for h in range(Hkv)])
             for i, x in enumerate((k_bf16, v_bf16))]
    return out[0], out[1], clips[0], clips[1]


# ---------------------------------------------------------------------------
# per-token codec (C)
# ---------------------------------------------------------------------------

def encode(x_bf16: np.ndarray, R: np.ndarray, clip: np.ndarray, G: int):
    """Rotate, clip, quantize, pack N vectors.  Returns (packed u8 [N][d/4],
    scale16 u16 [N][d/G], zero16 u16 [N][d/G])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    N, d = x.shape
    R = np.ascontiguousarray(R, dtype=np.float32)
    clip = np.ascontiguousarray(clip, dtype=np.float32)
    packed = np.empty((N, d // 4), dtype=np.uint8)
    s16 = np.empty((N, d // G), dtype=np.uint16)
    z16 = np.empty((N, d // G), dtype=np.uint16)
    lib().oracle_encode(_ptr(x), N, d, G, _ptr(R), _ptr(clip), _ptr(packed), _ptr(s16), _ptr(z16))
    return packed, s16, z16


# ---------------------------------------------------------------------------
# Lloyd-Max codebook variant (article, section "Why this matters for
# long-context agents": the OSCAR code pairs the rotation with a Lloyd-Max
# codebook).  Reading: the group's fp16 scale s and zero point z stay; the
# four levels become z + (L_k / 64) s for a codebook L (integers 0..255,
# non-decreasing, per kv head and K|V) fitted offline by Lloyd's algorithm
# on the normalised values u = (y - z) / s of calibration tokens; a channel
# takes the nearest level (ties to the lower).
# ---------------------------------------------------------------------------

LLOYD_ITERS = 32
LLOYD_GRID = 2 ** 20   # u is fitted on multiples of 2^-20 (exact integer sums)


def normalized_values(x_bf16: np.ndarray, R: np.ndarray, clip: np.ndarray, G: int) -> np.ndarray:
    """fp32 u [N][d] = (y - z) / s of N bf16 vectors after rotation and clip
    (the codec's own arithmetic, in C); NaN for groups with s == 0."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    N, d = x.shape
    u = np.empty((N, d), dtype=np.float32)
    lib().oracle_normalized_many(_ptr(x), N, d, G, _ptr(np.ascontiguousarray(R, dtype=np.float32)),
                                 _ptr(np.ascontiguousarray(clip, dtype=np.float32)), _ptr(u))
    return u


def lloyd_max_levels(u: np.ndarray, iters: int = LLOYD_ITERS) -> np.ndarray:
    """Lloyd's algorithm for a 4-level scalar quantizer of the values u
    (NaN entries, the s == 0 groups, are left out), fp64 levels.

    The values are taken on the grid of 2^-20 (U = rint(u 2^20), integers,
    so every cell sum is exact).  Start from the uniform levels 0, 1, 2, 3;
    each iteration sets the thresholds midway between neighbouring levels,
    puts a value in cell k when it lies above exactly k thresholds, and moves
    each level to the mean of its cell (a level whose cell is empty stays)."""
    u = np.asarray(u, dtype=np.float32).ravel()
    U = np.rint(u[~np.isnan(u)].astype(np.float64) * LLOYD_GRID).astype(np.int64)
    lev = np.array([0.0, 1.0, 2.0, 3.0])
    for _ in range(iters):
        thr = (lev[:-1] + lev[1:]) * (LLOYD_GRID / 2)      # in grid units
        cell = (U[:, None] > thr[None, :]).sum(axis=1)
        new = lev.copy()
        for k in range(4):
            sel = U[cell == k]
            if len(sel):
                new[k] = float(int(sel.sum())) / float(len(sel)) / LLOYD_GRID
        lev = new
    return lev


def lloyd_max_codebook(u: np.ndarray, iters: int = LLOYD_ITERS) -> np.ndarray:
    """uint8 [4]: the fitted levels on the stored grid, L_k = rint(64 level_k)
    (ties to even), clamped to 0..255."""
    return np.clip(np.rint(lloyd_max_levels(u, iters) * 64.0), 0, 255).astype(np.uint8)


def encode_lut(x_bf16: np.ndarray, R: np.ndarray, clip: np.ndarray, G: int, L: np.ndarray):
    """``encode`` with codebook L (uint8 [4]): nearest-level codes."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    N, d = x.shape
    packed = np.empty((N, d // 4), dtype=np.uint8)
    s16 = np.empty((N, d // G), dtype=np.uint16)
    z16 = np.empty((N, d // G), dtype=np.uint16)
    lib().oracle_encode_lut(_ptr(x), N, d, G, _ptr(np.ascontiguousarray(R, dtype=np.float32)),
                            _ptr(np.ascontiguousarray(clip, dtype=np.float32)),
                            _ptr(np.ascontiguousarray(L, dtype=np.uint8)), _ptr(packed), _ptr(s16), _ptr(z16))
    return packed, s16, z16


def dequantize_lut(packed, s16, z16, G: int, L) -> np.ndarray:
    """z + s L[code] / 64 in fp64 (exact)."""
    codes = unpack(packed)
    lv = np.asarray(L, dtype=np.float64)[codes] / 64.0
    s = np.repeat(f16_table()[s16], G, axis=-1)
    z = np.repeat(f16_table()[z16], G, axis=-1)
    return lv * s + z


def quantize(y: np.ndarray, G: int):
    """Quantize already rotated+clipped fp32 vectors y [N][d]: (codes, s16, z16)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    N, d = y.shape
    codes = np.empty((N, d), dtype=np.uint8)
    s16 = np.empty((N, d // G), dtype=np.uint16)
    z16 = np.empty((N, d // G), dtype=np.uint16)
    L = lib()
    for t in range(N):
        L.oracle_quantize(_ptr(y[t]), d, G, _ptr(codes[t]), _ptr(s16[t]), _ptr(z16[t]))
    return codes, s16, z16


def pack(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] // 4,), dtype=np.uint8)
    flat_in = codes.reshape(-1, codes.shape[-1])
    flat_out = out.reshape(-1, out.shape[-1])
    for r in range(flat_in.shape[0]):
        lib().oracle_pack(_ptr(flat_in[r]), flat_in.shape[1], _ptr(flat_out[r]))
    return out


def unpack(packed: np.ndarray) -> np.ndarray:
    """Four codes per byte, low bits first (plain numpy)."""
    p = np.asarray(packed, dtype=np.uint8)
    shifts = np.array([0, 2, 4, 6], dtype=np.uint8)
    return ((p[..., :, None] >> shifts) & 3).reshape(p.shape[:-1] + (p.shape[-1] * 4,))


def dequantize(packed: np.ndarray, s16: np.ndarray, z16: np.ndarray, G: int) -> np.ndarray:
    """code * s + z in fp64 (exact: every fp16 value is a multiple of 2**-24 below 2**17)."""
    codes = unpack(packed).astype(np.float64)
    s = f16_table()[s16]
    z = f16_table()[z16]
    s = np.repeat(s, G, axis=-1)
    z = np.repeat(z, G, axis=-1)
    return codes * s + z


_f16_table = None


def f16_table() -> np.ndarray:
    """fp64 value of every binary16 bit pattern (from the C decoder)."""
    global _f16_table
    if _f16_table is None:
        _f16_table = f16_bits_to_f64(np.arange(65536, dtype=np.uint16))
    return _f16_table


# ---------------------------------------------------------------------------
# pool semantics
# ---------------------------------------------------------------------------

def segments(L: int):
    """(sink, history, recent) position ranges of a sequence of length L."""
    n_hist = max(0, L - WINDOW)
    sink = range(0, min(L, SINK))
    hist = range(SINK, SINK + n_hist)
    recent = range(SINK + n_hist, max(L, SINK + n_hist))
    return sink, hist, recent


def ring_slot(pos: int) -> int:
    """Recent-window slot of a position (>= SINK) in the 256-slot ring."""
    return (pos - SINK) % RECENT


def bits_per_element(L: int, G: int) -> float:
    """Stored bits per K (or V) element: 2-bit codes + 2 fp16 params per group
    for the history, 16 bits for sink and recent."""
    n_hist = max(0, L - WINDOW)
    return (n_hist * (2 + 32 / G) + min(L, WINDOW) * 16) / L


M64 = (1 << 64) - 1


def splitmix64_stream(seed: int):
    """Vigna's SplitMix64 generator."""
    state = seed & M64
    while True:
        state = (state + 0x9E3779B97F4A7C15) & M64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
        yield z ^ (z >> 31)


def free_list(num_pages: int, seed: int) -> list:
    """Fisher-Yates shuffle of [0, num_pages) driven by SplitMix64(seed):
    for i = n-1 down to 1, j = next() mod (i+1), swap entries i and j."""
    a = list(range(num_pages))
    g = splitmix64_stream(seed)
    for i in range(num_pages - 1, 0, -1):
        j = next(g) % (i + 1)
        a[i], a[j] = a[j], a[i]
    return a


@dataclass
class PoolModel:
    """Host bookkeeping of the pool: lengths, page tables, page references.

    Pages are popped from the front of the shuffled free list; a page is
    taken when a history token lands on slot 0 of a new page.  Within one
    append call sequences are served in the order given; a prefill takes its
    pages in history order.

    Prefix sharing (the article's compatibility with a radix prefix cache):
    ``fork`` gives an empty sequence the whole state of another, its history
    pages shared (each page counts the page tables that hold it).  Only the
    history's last page is ever written again, when the next evicted token
    lands in it; a sequence about to write into a page that another sequence
    also holds first takes a page of its own from the free list (at that
    point of the call's order) and copies the page into it (copy on write).
    Releasing a sequence drops its references; pages that nobody holds any
    more go, in page table order, to the back of the free list.
    """
    num_pages: int
    seed: int
    max_pages_per_seq: int
    free: list = field(default_factory=list)
    length: dict = field(default_factory=dict)
    table: dict = field(default_factory=dict)
    refs: dict = field(default_factory=dict)

    def __post_init__(self):
        self.free = free_list(self.num_pages, self.seed)

    def _take(self):
        if not self.free:
            raise MemoryError("pool out of pages")
        pg = self.free.pop(0)
        self.refs[pg] = 1
        return pg

    def prefill(self, seq: int, L: int):
        assert self.length.get(seq, 0) == 0
        n_hist = max(0, L - WINDOW)
        n_pages = -(-n_hist // PAGE)
        assert n_pages <= self.max_pages_per_seq and n_pages <= len(self.free)
        self.table[seq] = [self._take() for _ in range(n_pages)]
        self.length[seq] = L

    def append(self, seq_ids):
        for s in seq_ids:
            L = self.length.get(s, 0)
            if L >= WINDOW:                   # recent full: evict the oldest
                n_hist = L - WINDOW
                if n_hist % PAGE == 0:
                    self.table.setdefault(s, []).append(self._take())
                else:                          # writes into its last page
                    i = n_hist // PAGE
                    pg = self.table[s][i]
                    if self.refs[pg] > 1:      # shared: copy on write
                        self.refs[pg] -= 1
                        self.table[s][i] = self._take()
            self.length[s] = L + 1

    def fork(self, src: int, dst: int):
        assert self.length.get(dst, 0) == 0 and not self.table.get(dst)
        self.table[dst] = list(self.table.get(src, []))
        for pg in self.table[dst]:
            self.refs[pg] += 1
        self.length[dst] = self.length.get(src, 0)

    def release(self, seq: int):
        for pg in self.table.get(seq, []):
            self.refs[pg] -= 1
            if self.refs[pg] == 0:
                self.free.append(pg)
        self.table[seq] = []
        self.length[seq] = 0


# ---------------------------------------------------------------------------
# attention: the plain definition over the decoded pool (fp64)
# ---------------------------------------------------------------------------

def decode_history(packed, s16, z16, G: int, R: np.ndarray) -> np.ndarray:
    """History tokens back in the original basis: dequant(codes) . R^T (fp64)."""
    rot = dequantize(packed, s16, z16, G)
    return rot @ np.asarray(R, dtype=np.float64).T


def decode_history_lut(packed, s16, z16, G: int, L, R: np.ndarray) -> np.ndarray:
    """History tokens of the Lloyd-Max variant back in the original basis:
    dequant_lut(codes) . R^T (fp64)."""
    return dequantize_lut(packed, s16, z16, G, L) @ np.asarray(R, dtype=np.float64).T


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query head over T tokens, fp64.
    q [d], K [T][d], V [T][d] -> out [d]."""
    logits = scale * (K @ q)
    m = logits.max()
    w = np.exp(logits - m)
    return (w @ V) / w.sum()


def partial_attention(q, K, V, scale):
    """(m, l, acc) of one query over a token subset: m = max logit,
    l = sum exp(logit - m), acc = sum exp(logit - m) V.  Empty set:
    (-inf, 0, 0)."""
    if len(K) == 0:
        return -math.inf, 0.0, np.zeros(V.shape[-1])
    logits = scale * (K @ q)
    m = logits.max()
    w = np.exp(logits - m)
    return m, w.sum(), w @ V


def merge_partials(parts):
    """Online-softmax merge: m = max m_i, w_i = exp(m_i - m),
    l = sum w_i l_i, acc = sum w_i acc_i; result acc / l."""
    m = max(p[0] for p in parts)
    l = 0.0
    acc = 0.0
    for mi, li, ai in parts:
        w = 0.0 if mi == -math.inf else math.exp(mi - m)
        l = l + w * li
        acc = acc + w * ai
    return m, l, acc


@dataclass
class SeqTokens:
    """Decoded pool contents of one sequence, per kv head: K, V [L][Hkv][d] fp64,
    plus the history encodings (packed, s16, z16 per K/V) for bit-exact checks."""
    L: int
    K: np.ndarray
    V: np.ndarray
    hist: dict


def build_sequence(k_bf16: np.ndarray, v_bf16: np.ndarray, R_K, R_V, clip_K, clip_V, G: int,
                   heads=None, codebook=None) -> SeqTokens:
    """Pool contents of a sequence whose tokens (positions 0..L-1) are
    k_bf16/v_bf16 uint16 [L][Hkv][d]: sink and recent kept as bf16, history
    positions encoded by the codec and decoded again.  codebook: None for the
    affine levels, else (L_K, L_V) uint8 [Hkv][4] (the Lloyd-Max variant)."""
    L, Hkv, d = k_bf16.shape
    heads = range(Hkv) if heads is None else heads
    _, hist, _ = segments(L)
    K = bf16_bits_to_f64(k_bf16)
    V = bf16_bits_to_f64(v_bf16)
    enc = {}
    if len(hist):
        h0, h1 = hist.start, hist.stop
        for kv in heads:
            for i, (name, src, R, c, dst) in enumerate((("K", k_bf16, R_K, clip_K, K), ("V", v_bf16, R_V, clip_V, V))):
                if codebook is None:
                    pk, s16, z16 = encode(src[h0:h1, kv, :], R[kv], c[kv], G)
                    dst[h0:h1, kv, :] = decode_history(pk, s16, z16, G, R[kv])
                else:
                    pk, s16, z16 = encode_lut(src[h0:h1, kv, :], R[kv], c[kv], G, codebook[i][kv])
                    dst[h0:h1, kv, :] = decode_history_lut(pk, s16, z16, G, codebook[i][kv], R[kv])
                enc[(name, kv)] = (pk, s16, z16)
    return SeqTokens(L, K, V, enc)


def attend_sequence(st: SeqTokens, q_bf16: np.ndarray, scale: float, heads=None) -> np.ndarray:
    """out [Hq][d] fp64 for one sequence; q uint16 [Hq][d]; kv head = h // g."""
    Hq, d = q_bf16.shape
    Hkv = st.K.shape[1]
    g = Hq // Hkv
    q = bf16_bits_to_f64(q_bf16)
    out = np.full((Hq, d), np.nan)
    for h in (range(Hq) if heads is None else heads):
        kv = h // g
        out[h] = attention(q[h], st.K[:, kv, :], st.V[:, kv, :], scale)
    return out


def prefill_attention(st: SeqTokens, q_bf16: np.ndarray, scale: float, heads=None) -> np.ndarray:
    """Causal attention of the last n_q positions of a sequence over its pool
    (prefill, or one chunk of a chunked prefill, over the three-segment pool:
    article, section "From offline calibration to online inference").
    Query i sits at position p = L - n_q + i and attends, with softmax, to
    positions 0..p of the pool as it stands: sink and recent tokens as stored
    (bf16), history tokens decoded (dequant . R^T).  q_bf16 uint16
    [n_q][Hq][d]; returns fp64 [n_q][Hq][d]; kv head = h // (Hq/Hkv).

    Written per head as one masked softmax: logits = scale q K^T over all L
    tokens, positions after a query's own set to -inf, then softmax rows and
    a product with V."""
    n_q, Hq, d = q_bf16.shape
    L = st.L
    assert 1 <= n_q <= L
    Hkv = st.K.shape[1]
    g = Hq // Hkv
    q = bf16_bits_to_f64(q_bf16)
    pos = L - n_q + np.arange(n_q)
    visible = np.arange(L)[None, :] <= pos[:, None]          # [n_q][L]
    out = np.full((n_q, Hq, d), np.nan)
    for h in (range(Hq) if heads is None else heads):
        kv = h // g
        logits = scale * (q[:, h, :] @ st.K[:, kv, :].T)      # [n_q][L]
        logits = np.where(visible, logits, -np.inf)
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        out[:, h, :] = (w @ st.V[:, kv, :]) / w.sum(axis=1, keepdims=True)
    return out


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got - ref||_inf / ||ref||_inf."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return float((num / den).max())
