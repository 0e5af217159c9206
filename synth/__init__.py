"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module only *draws numbers*: token values, query values, sequence
lengths, the random orthogonal matrices that stand in for the calibrated
eigenbasis U, and the outlier-channel choice.  It contains none of the OSCAR
method's arithmetic (no rotation, clipping, quantization, packing, paging or
attention); both the oracle and the HIP path compute those on their own.

Generator (counter based, identical on CPU and GPU because it is integer
arithmetic plus one table lookup and one fp32 multiply):

* ``mix32(x)``: a two-multiply xorshift 32-bit integer mixer,
  ``x ^= x>>16; x *= 0x21f0aaad; x ^= x>>15; x *= 0x735a2d97; x ^= x>>15``
  (all mod 2**32), in the style of Wellons' hash-prospector mixers.
* ``key(seed, stream) = mix32(mix32(seed) ^ stream)``.
* ``u(key, i) = mix32(mix32(key ^ (i >> 32)) ^ (i & 0xffffffff))`` for a
  64-bit element counter ``i``.
* a normal value is ``T[u >> 16]`` with ``T[k] = fp32(Phi^-1((k + 1/2) / 65536))``
  (a 65,536-entry table of standard-normal quantiles, built once in fp64);
* K/V tokens multiply 4 seeded "outlier" channels per (kv head, K|V) by 20 in
  fp32 and round to bf16 (round to nearest even).

Streams: 0 lengths, 1 page shuffle seed, 2 U for K, 3 U for V,
4 calibration tokens, 5 K tokens, 6 V tokens, 7 queries, 8 calibration
queries, 9 the orthogonal axes of the calibration queries' covariance.
A token's value depends only on (seed, K|V, sequence, position, head,
channel), so a prompt and the tokens appended to it later come from one
stream and any sampled token can be regenerated without storing the pool.
"""
from __future__ import annotations

import dataclasses
import functools

import numpy as np
import torch

M32 = 0xFFFFFFFF
STREAM_LENGTHS, STREAM_SHUFFLE, STREAM_UK, STREAM_UV = 0, 1, 2, 3
STREAM_CALIB, STREAM_K, STREAM_V, STREAM_Q = 4, 5, 6, 7
STREAM_CALIB_Q, STREAM_CALIB_B = 8, 9
OUTLIER_CHANNELS = 4
OUTLIER_FACTOR = 20.0
POS_BITS = 20          # positions < 2**20 (1M tokens per sequence)
MAX_SEQ_ID = 1 << 16


def mix32_int(x: int) -> int:
    """Scalar reference of the 32-bit mixer (Python ints)."""
    x &= M32
    x ^= x >> 16
    x = (x * 0x21F0AAAD) & M32
    x ^= x >> 15
    x = (x * 0x735A2D97) & M32
    x ^= x >> 15
    return x


def _mix32(x: torch.Tensor) -> torch.Tensor:
    # x: int64 tensor holding values in [0, 2**32). Every product below is
    # < 2**63, so int64 arithmetic is exact on every device.
    x = x ^ (x >> 16)
    x = (x * 0x21F0AAAD) & M32
    x = x ^ (x >> 15)
    x = (x * 0x735A2D97) & M32
    x = x ^ (x >> 15)
    return x


def stream_key(seed: int, stream: int) -> int:
    return mix32_int(mix32_int(seed) ^ (stream & M32))


def uniform_u32(key: int, index: torch.Tensor) -> torch.Tensor:
    """u(key, i) for an int64 tensor of non-negative counters i < 2**62."""
    hi = index >> 32
    lo = index & M32
    return _mix32(_mix32(hi ^ key) ^ lo)


@functools.lru_cache(maxsize=None)
def _normal_table_np() -> np.ndarray:
    from scipy.special import ndtri
    k = np.arange(65536, dtype=np.float64)
    return ndtri((k + 0.5) / 65536.0).astype(np.float32)


_table_cache: dict = {}


def normal_table(device) -> torch.Tensor:
    dev = torch.device(device)
    key = (dev.type, dev.index)
    t = _table_cache.get(key)
    if t is None:
        t = torch.from_numpy(_normal_table_np()).to(dev)
        _table_cache[key] = t
    return t


def normals_f32(key: int, index: torch.Tensor) -> torch.Tensor:
    u = uniform_u32(key, index)
    return normal_table(index.device)[u >> 16]


# ---------------------------------------------------------------------------
# Workload shapes
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and seed of one synthetic decode workload."""
    name: str
    config_id: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    group_size: int
    len_lo: int            # prompt lengths are uniform integers in [len_lo, len_hi]
    len_hi: int
    steps: int = 0         # fused append+evict+decode steps (0 = decode only)

    @property
    def seed_base(self) -> int:
        return 1000 * self.config_id

    def seed(self, stream: int) -> int:
        return self.seed_base + stream

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    # batch 1, GQA 2, d 64, L 1024 = sink 64 + history 704 + recent 256, G 64
    "tiny": Workload("tiny", 1, 1, 4, 2, 64, 64, 1024, 1024),
    # Qwen3-8B-shaped layer: batch 16, 32/8 heads, d 128, L 32768, G 128
    "qwen3_8b_32k": Workload("qwen3_8b_32k", 2, 16, 32, 8, 128, 128, 32768, 32768),
    # large batch: 128 sequences, L uniform in [4096, 8192], G 64
    "large_batch_8k": Workload("large_batch_8k", 3, 128, 32, 8, 128, 64, 4096, 8192),
    # Qwen3-32B-shaped layer: batch 32, 64/8 heads (GQA 8), L 65536, G 128
    "qwen3_32b_64k": Workload("qwen3_32b_64k", 4, 32, 64, 8, 128, 128, 65536, 65536),
    # fused serving step: batch 64, L uniform in [4096, 65536], 256 steps
    # (the group size is not fixed by the workload description; 128 is used)
    "fused_64x_4k_64k": Workload("fused_64x_4k_64k", 5, 64, 32, 8, 128, 128, 4096, 65536, steps=256),
    # one sequence of 100,000 tokens, Qwen3-8B-shaped layer (the latency
    # case: decode at 100K context, batch 1)
    "qwen3_8b_100k_b1": Workload("qwen3_8b_100k_b1", 6, 1, 32, 8, 128, 128, 100000, 100000),
}


def lengths(w: Workload) -> np.ndarray:
    rng = np.random.default_rng([w.seed(STREAM_LENGTHS)])
    if w.len_lo == w.len_hi:
        return np.full(w.batch, w.len_lo, dtype=np.int64)
    return rng.integers(w.len_lo, w.len_hi + 1, size=w.batch).astype(np.int64)


def page_shuffle_seed(w: Workload) -> int:
    return int(np.random.default_rng([w.seed(STREAM_SHUFFLE)]).integers(0, 2**63 - 1))


def outlier_channels(w: Workload, kind: int) -> np.ndarray:
    """[Hkv][4] distinct channel indices scaled by 20 (kind 0 = K, 1 = V)."""
    rng = np.random.default_rng([w.seed_base, 100 + kind])
    return np.stack([np.sort(rng.choice(w.head_dim, OUTLIER_CHANNELS, replace=False))
                     for _ in range(w.num_kv_heads)]).astype(np.int64)


def _outlier_mask(outliers: np.ndarray, d: int, device) -> torch.Tensor:
    m = np.ones((outliers.shape[0], d), dtype=np.float32)
    for h in range(outliers.shape[0]):
        m[h, outliers[h]] = OUTLIER_FACTOR
    return torch.from_numpy(m).to(device)


def kv_tokens(w: Workload, kind: int, seq: int, pos0: int, count: int,
              device="cpu", heads=None) -> torch.Tensor:
    """bf16 [count][H][d] tokens at positions pos0 .. pos0+count-1 of ``seq``
    for kv heads ``heads`` (default: all Hkv heads)."""
    assert 0 <= seq < MAX_SEQ_ID and 0 <= pos0 and pos0 + count <= (1 << POS_BITS)
    Hkv, d = w.num_kv_heads, w.head_dim
    heads = list(range(Hkv)) if heads is None else list(heads)
    key = stream_key(w.seed(STREAM_K if kind == 0 else STREAM_V), 0)
    pos = torch.arange(pos0, pos0 + count, dtype=torch.int64, device=device)
    head = torch.tensor(heads, dtype=torch.int64, device=device)
    ch = torch.arange(d, dtype=torch.int64, device=device)
    idx = (((seq << POS_BITS) + pos)[:, None, None] * Hkv + head[None, :, None]) * d + ch[None, None, :]
    vals = normals_f32(key, idx)
    vals = vals * _outlier_mask(outlier_channels(w, kind), d, device)[heads][None]
    return vals.to(torch.bfloat16)


def calibration_tokens(w: Workload, kind: int, n: int, device="cpu") -> torch.Tensor:
    """bf16 [Hkv][n][d] calibration tokens drawn from the K (kind 0) or V
    (kind 1) distribution (same outlier channels as the data)."""
    Hkv, d = w.num_kv_heads, w.head_dim
    key = stream_key(w.seed(STREAM_CALIB), kind)
    head = torch.arange(Hkv, dtype=torch.int64, device=device)
    tok = torch.arange(n, dtype=torch.int64, device=device)
    ch = torch.arange(d, dtype=torch.int64, device=device)
    idx = (head[:, None, None] * n + tok[None, :, None]) * d + ch[None, None, :]
    vals = normals_f32(key, idx)
    vals = vals * _outlier_mask(outlier_channels(w, kind), d, device)[:, None, :]
    return vals.to(torch.bfloat16)


CALIB_Q_DECAY = 16.0   # calibration query axis c has standard deviation 2^(-c / 16)


def calibration_activations(w: Workload, n: int):
    """(q bf16 [n][Hq][d], k, v bf16 [n][Hkv][d]) of one calibration sequence,
    on the CPU.  K and V are the calibration tokens (the data's distribution,
    outlier channels included).  Queries have a planted anisotropic
    covariance: per query head, z diag(sigma) B^T with z standard normal
    (counter generator, stream 8), sigma_c = 2^(-c/16), and B an orthogonal
    matrix per kv head (QR of a seeded Gaussian, stream 9), shared by the
    kv head's query heads; the product is taken in fp64 and rounded to bf16."""
    Hq, Hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    g = Hq // Hkv
    k = calibration_tokens(w, 0, n).permute(1, 0, 2).contiguous()
    v = calibration_tokens(w, 1, n).permute(1, 0, 2).contiguous()
    key = stream_key(w.seed(STREAM_CALIB_Q), 0)
    idx = ((torch.arange(n, dtype=torch.int64)[:, None, None] * Hq + torch.arange(Hq)[None, :, None]) * d
           + torch.arange(d)[None, None, :])
    z = normals_f32(key, idx).double()
    sigma = torch.pow(2.0, -torch.arange(d, dtype=torch.float64) / CALIB_Q_DECAY)
    rng = np.random.default_rng([w.seed(STREAM_CALIB_B)])
    q = torch.empty((n, Hq, d), dtype=torch.float64)
    for kv in range(Hkv):
        B, r = np.linalg.qr(rng.standard_normal((d, d)))
        B = torch.from_numpy(B * np.sign(np.diag(r))[None, :])
        for h in range(kv * g, kv * g + g):
            q[:, h, :] = (z[:, h, :] * sigma) @ B.T
    return q.to(torch.bfloat16), k, v


def queries(w: Workload, step: int, device="cpu", batch: int | None = None) -> torch.Tensor:
    """bf16 [B][Hq][d] standard-normal queries for decode step ``step``."""
    B = w.batch if batch is None else batch
    Hq, d = w.num_q_heads, w.head_dim
    key = stream_key(w.seed(STREAM_Q), 0)
    b = torch.arange(B, dtype=torch.int64, device=device)
    h = torch.arange(Hq, dtype=torch.int64, device=device)
    c = torch.arange(d, dtype=torch.int64, device=device)
    idx = (((step << 16) + b)[:, None, None] * Hq + h[None, :, None]) * d + c[None, None, :]
    return normals_f32(key, idx).to(torch.bfloat16)


def random_orthogonal_u(w: Workload, kind: int) -> np.ndarray:
    """fp32 [Hkv][d][d] stand-in for the calibrated eigenbasis U.

    Q factor of a seeded Gaussian matrix with column signs chosen so that the
    triangular factor has a positive diagonal (this makes the factorisation
    unique), rounded to fp32 and then to the grid of multiples of 2**-40 (a
    no-op except for entries below 2**-17).  On that grid every partial sum
    of +-U entries over at most 2**7 terms is an integer multiple of 2**-40
    below 2**47, hence exact in fp64 in any order.
    """
    d = w.head_dim
    rng = np.random.default_rng([w.seed(STREAM_UK if kind == 0 else STREAM_UV)])
    out = np.empty((w.num_kv_heads, d, d), dtype=np.float32)
    for h in range(w.num_kv_heads):
        g = rng.standard_normal((d, d))
        q, r = np.linalg.qr(g)
        q = q * np.sign(np.diag(r))[None, :]
        q32 = q.astype(np.float32).astype(np.float64)
        out[h] = (np.round(q32 * 2.0**40) / 2.0**40).astype(np.float32)
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 view (numpy) of a bf16 tensor's bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def kv_tokens_at(w: Workload, kind: int, seqs, positions, device="cpu") -> torch.Tensor:
    """bf16 [n][Hkv][d]: the token at positions[i] of sequence seqs[i], for each i."""
    Hkv, d = w.num_kv_heads, w.head_dim
    key = stream_key(w.seed(STREAM_K if kind == 0 else STREAM_V), 0)
    s = torch.as_tensor(np.asarray(seqs, dtype=np.int64), device=device)
    p = torch.as_tensor(np.asarray(positions, dtype=np.int64), device=device)
    head = torch.arange(Hkv, dtype=torch.int64, device=device)
    ch = torch.arange(d, dtype=torch.int64, device=device)
    idx = (((s << POS_BITS) + p)[:, None, None] * Hkv + head[None, :, None]) * d + ch[None, None, :]
    vals = normals_f32(key, idx)
    vals = vals * _outlier_mask(outlier_channels(w, kind), d, device)[None]
    return vals.to(torch.bfloat16)
