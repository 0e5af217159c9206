"""GPU-side setup shared by the GPU tests, the smoke check and the benchmark:
offline tables through the library's own helpers, pool sizing, and prefill
of synthetic sequences.  It never imports the CPU oracle."""
from __future__ import annotations

import math

import numpy as np
import torch

import bit_kv_cache_segment_amd as oscar
import synth

N_CALIB = 4096


def tables(w: synth.Workload, n_cal: int = N_CALIB):
    """(R_K, R_V [Hkv][d][d], clip_K, clip_V [Hkv][d]) from the library's
    offline helpers: R = U.H.Pi and 99th-percentile clip thresholds."""
    R = []
    for kind in (0, 1):
        U = synth.random_orthogonal_u(w, kind)
        R.append(np.stack([oscar.oscar_build_rotation(u) for u in U]))
    clips = []
    for kind in (0, 1):
        cal = synth.bf16_bits(synth.calibration_tokens(w, kind, n_cal))
        clips.append(np.stack([oscar.oscar_calibrate_clip(cal[h], R[kind][h], 99.0)
                               for h in range(w.num_kv_heads)]))
    return R[0], R[1], clips[0], clips[1]


def codebooks(w: synth.Workload, R_K, R_V, clip_K, clip_V, n_cal: int = N_CALIB):
    """(L_K, L_V) uint8 [Hkv][4]: Lloyd-Max codebooks from the library's
    offline fit on the calibration tokens."""
    out = []
    for kind, (R, clip) in enumerate(((R_K, clip_K), (R_V, clip_V))):
        cal = synth.bf16_bits(synth.calibration_tokens(w, kind, n_cal))
        out.append(np.stack([oscar.oscar_lloyd_max_codebook(cal[h], R[h], clip[h], w.group_size)
                             for h in range(w.num_kv_heads)]))
    return out[0], out[1]


def pages_needed(L: int) -> int:
    return max(0, -(-(L - 320) // 64))


def config_for(w: synth.Workload, lengths, extra_tokens: int = 0, slack_pages: int = 0,
               max_seqs: int | None = None, seed: int | None = None, flags: int = 0):
    lengths = [int(x) for x in lengths]
    need = sum(pages_needed(L + extra_tokens) for L in lengths)
    maxp = max([pages_needed(L + extra_tokens) for L in lengths] + [1])
    return oscar.make_config(max_seqs or len(lengths), w.num_q_heads, w.num_kv_heads, w.head_dim,
                             w.group_size, need + slack_pages, maxp,
                             synth.page_shuffle_seed(w) if seed is None else seed, flags)


def prefill_all(pool: oscar.Pool, w: synth.Workload, lengths, seq_ids=None, stream=None):
    """Prefill sequence seq_ids[b] with positions 0..L_b-1 of synthetic sequence b."""
    seq_ids = list(range(len(lengths))) if seq_ids is None else list(seq_ids)
    for b, L in enumerate(lengths):
        L = int(L)
        k = synth.kv_tokens(w, 0, b, 0, L, device="cuda").view(torch.uint16)
        v = synth.kv_tokens(w, 1, b, 0, L, device="cuda").view(torch.uint16)
        pool.prefill(seq_ids[b], k, v, stream)
        del k, v


def step_tokens(w: synth.Workload, lengths, seqs=None):
    """bf16 bits [B][Hkv][d] of the next token (position L_b) of each sequence."""
    seqs = list(range(len(lengths))) if seqs is None else list(seqs)
    pos = [int(lengths[b]) for b in seqs]
    k = synth.kv_tokens_at(w, 0, seqs, pos, device="cuda")
    v = synth.kv_tokens_at(w, 1, seqs, pos, device="cuda")
    return k.view(torch.uint16).contiguous(), v.view(torch.uint16).contiguous()


def softmax_scale(w: synth.Workload) -> float:
    return 1.0 / math.sqrt(w.head_dim)
