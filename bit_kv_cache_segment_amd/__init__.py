"""Python binding of liboscar.so, the MI355X (gfx950) HIP implementation of
OSCAR's three-segment 2-bit KV pool (eviction + decode attention).

Every function here only marshals arguments to the C ABI declared in
``include/oscar.h``; all the work runs in the HIP kernels of the library.
PyTorch supplies device memory and streams.  Importing this package does
not need a GPU; loading the library fails loudly if it has not been built
(``python -m bit_kv_cache_segment_amd.build`` or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboscar.so")

SINK_TOKENS = 64
RECENT_TOKENS = 256
PAGE_TOKENS = 64
MAX_BATCH_PER_LAUNCH = 256
POOL_HOST_ONLY = 1
POOL_DETERMINISTIC = 2
POOL_BF16_HISTORY = 4
POOL_LLOYD_MAX = 8

OK, EHIP, ENOMEM, EINVAL, ERANGE = 0, -5, -12, -22, -34
_NAMES = {EHIP: "EHIP", ENOMEM: "ENOMEM", EINVAL: "EINVAL", ERANGE: "ERANGE"}

# every symbol include/oscar.h declares
EXPORTS = (
    "oscar_pool_bytes", "oscar_pool_required_bytes", "oscar_decode_workspace_bytes", "oscar_pool_create", "oscar_pool_destroy",
    "oscar_prefill", "oscar_append_evict", "oscar_decode_attn", "oscar_decode_step",
    "oscar_decode_step_static", "oscar_prefill_workspace_bytes", "oscar_prefill_attn", "oscar_pool_check",
    "oscar_release_seq", "oscar_fork_seq", "oscar_pool_set_codebook", "oscar_lloyd_max_codebook",
    "oscar_seq_length", "oscar_page_table", "oscar_free_pages", "oscar_export_history",
    "oscar_export_state", "oscar_export_history_bf16", "oscar_export_window", "oscar_build_rotation", "oscar_calibrate_clip",
    "oscar_calib_workspace_bytes", "oscar_calib_attention", "oscar_calib_covariance", "oscar_calib_rotation", "oscar_profile_begin",
    "oscar_profile_end", "oscar_last_error",
)


class OscarError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class PoolConfig(ctypes.Structure):
    _fields_ = [
        ("max_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("page_shuffle_seed", ctypes.c_uint64),
    ]


class Profile(ctypes.Structure):
    _fields_ = [
        ("n_decode_main", ctypes.c_int32), ("ms_decode_main", ctypes.c_float),
        ("n_decode_merge", ctypes.c_int32), ("ms_decode_merge", ctypes.c_float),
        ("n_append", ctypes.c_int32), ("ms_append", ctypes.c_float),
    ]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load liboscar.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "oscar_pool_bytes": [_P, _P],
            "oscar_pool_required_bytes": [_P, _P, _P],
            "oscar_decode_workspace_bytes": [_P, _I32, _P],
            "oscar_pool_create": [_P, _P, _SZ, _P, _P, _P, _P, _P, _P],
            "oscar_pool_destroy": [_P],
            "oscar_prefill": [_P, _I32, _P, _P, _I32, _P],
            "oscar_append_evict": [_P, _P, _I32, _P, _P, _P],
            "oscar_decode_attn": [_P, _P, _I32, _P, _P, ctypes.c_float, _P, _SZ, _P],
            "oscar_decode_step": [_P, _P, _I32, _P, _P, _P, _P, ctypes.c_float, _P, _SZ, _P],
            "oscar_decode_step_static": [_P, _P, _I32, _P, _P, _P, _P, ctypes.c_float, _P],
            "oscar_prefill_workspace_bytes": [_P, _I32, _P],
            "oscar_prefill_attn": [_P, _I32, _I32, _P, _P, ctypes.c_float, _P, _SZ, _P],
            "oscar_pool_check": [_P, _P],
            "oscar_release_seq": [_P, _I32],
            "oscar_fork_seq": [_P, _I32, _I32, _P],
            "oscar_pool_set_codebook": [_P, _P, _P, _P],
            "oscar_lloyd_max_codebook": [_I32, _I32, ctypes.c_int64, _P, _P, _P, _I32, _P],
            "oscar_seq_length": [_P, _I32, _P],
            "oscar_page_table": [_P, _I32, _P, _I32, _P],
            "oscar_free_pages": [_P, _P],
            "oscar_export_history": [_P, _I32, _I32, _I32, _P, _P, _P],
            "oscar_export_state": [_P, _I32, _P, _P, _P, _P],
            "oscar_export_history_bf16": [_P, _I32, _I32, _I32, _P, _P, _P],
            "oscar_export_window": [_P, _I32, _P, _P, _P, _P, _P],
            "oscar_build_rotation": [_I32, _P, _P],
            "oscar_calibrate_clip": [_I32, ctypes.c_int64, _P, _P, ctypes.c_double, _P],
            "oscar_calib_workspace_bytes": [_I32, _I32, _I32, _P],
            "oscar_calib_attention": [_I32, _I32, _I32, _I32, _P, _P, _P, ctypes.c_float, _P, _P],
            "oscar_calib_covariance": [_I32, _I32, _I32, _I32, _P, _P, _P, ctypes.c_float, _P, _P, _P, _SZ, _P],
            "oscar_calib_rotation": [_I32, _P, _P, _P, _P],
            "oscar_profile_begin": [_P, _I32, ctypes.c_uint32, _I32],
            "oscar_profile_end": [_P, _P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.oscar_last_error.argtypes = []
        L.oscar_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != OK:
        raise OscarError(rc, lib().oscar_last_error().decode())


def _np_ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _dev_ptr(t):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "expected a contiguous device tensor"
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ids(seq_ids) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int32))


# ---------------------------------------------------------------------------
# one wrapper per C entry point (same names)
# ---------------------------------------------------------------------------

def oscar_pool_bytes(cfg: PoolConfig) -> int:
    n = ctypes.c_size_t()
    _check(lib().oscar_pool_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def oscar_pool_required_bytes(cfg: PoolConfig):
    """(device bytes of the pool, decode workspace bytes for a full launch)."""
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().oscar_pool_required_bytes(ctypes.byref(cfg), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def oscar_decode_workspace_bytes(cfg: PoolConfig, max_batch: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().oscar_decode_workspace_bytes(ctypes.byref(cfg), max_batch, ctypes.byref(n)))
    return n.value


def oscar_pool_create(cfg: PoolConfig, device_buf, nbytes: int, R_K, R_V, clip_K, clip_V, stream=None):
    """R_*: host fp32 [Hkv][d][d]; clip_*: host fp32 [Hkv][d] (numpy).  device_buf: a
    device tensor (or None for a host-only pool).  Returns an opaque handle."""
    arrs = [None if a is None else np.ascontiguousarray(a, dtype=np.float32) for a in (R_K, R_V, clip_K, clip_V)]
    ptrs = [None if a is None else _np_ptr(a) for a in arrs]
    h = ctypes.c_void_p()
    host_only = bool(cfg.flags & POOL_HOST_ONLY)
    dptr = None if device_buf is None else _dev_ptr(device_buf)
    st = None if host_only else _stream(stream)
    _check(lib().oscar_pool_create(ctypes.byref(cfg), dptr, nbytes, *ptrs, st, ctypes.byref(h)))
    return h


def oscar_pool_destroy(h):
    _check(lib().oscar_pool_destroy(h))


def oscar_prefill(h, seq: int, k, v, L: int, stream=None, host_only=False):
    _check(lib().oscar_prefill(h, seq, _dev_ptr(k), _dev_ptr(v), L, None if host_only else _stream(stream)))


def oscar_append_evict(h, seq_ids, k_new, v_new, stream=None, host_only=False):
    ids = _ids(seq_ids)
    _check(lib().oscar_append_evict(h, _np_ptr(ids), len(ids), _dev_ptr(k_new), _dev_ptr(v_new),
                                    None if host_only else _stream(stream)))


def oscar_decode_attn(h, seq_ids, q, out, softmax_scale: float, workspace, stream=None):
    ids = _ids(seq_ids)
    _check(lib().oscar_decode_attn(h, _np_ptr(ids), len(ids), _dev_ptr(q), _dev_ptr(out),
                                   float(softmax_scale), _dev_ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def oscar_decode_step(h, seq_ids, k_new, v_new, q, out, softmax_scale: float, workspace, stream=None):
    ids = _ids(seq_ids)
    _check(lib().oscar_decode_step(h, _np_ptr(ids), len(ids), _dev_ptr(k_new), _dev_ptr(v_new), _dev_ptr(q),
                                   _dev_ptr(out), float(softmax_scale), _dev_ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def oscar_decode_step_static(h, seq_ids, k_new, v_new, q, out, softmax_scale: float, stream=None):
    ids = _ids(seq_ids)
    _check(lib().oscar_decode_step_static(h, _np_ptr(ids), len(ids), _dev_ptr(k_new), _dev_ptr(v_new),
                                          _dev_ptr(q), _dev_ptr(out), float(softmax_scale), _stream(stream)))


def oscar_prefill_workspace_bytes(cfg: PoolConfig, n_q: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().oscar_prefill_workspace_bytes(ctypes.byref(cfg), n_q, ctypes.byref(n)))
    return n.value


def oscar_prefill_attn(h, seq: int, q, out, softmax_scale: float, workspace, stream=None):
    """q: device bf16 [n_q][Hq][d] (the last n_q positions' queries); out fp32, same shape."""
    _check(lib().oscar_prefill_attn(h, seq, q.shape[0], _dev_ptr(q), _dev_ptr(out), float(softmax_scale),
                                    _dev_ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))


def oscar_pool_check(h, stream=None, host_only=False):
    _check(lib().oscar_pool_check(h, None if host_only else _stream(stream)))


def oscar_release_seq(h, seq: int):
    _check(lib().oscar_release_seq(h, seq))


def oscar_fork_seq(h, src: int, dst: int, stream=None, host_only=False):
    _check(lib().oscar_fork_seq(h, src, dst, None if host_only else _stream(stream)))


def oscar_seq_length(h, seq: int) -> int:
    L = ctypes.c_int32()
    _check(lib().oscar_seq_length(h, seq, ctypes.byref(L)))
    return L.value


def oscar_page_table(h, seq: int, capacity: int) -> np.ndarray:
    out = np.zeros(max(capacity, 1), dtype=np.int32)
    n = ctypes.c_int32()
    _check(lib().oscar_page_table(h, seq, _np_ptr(out), capacity, ctypes.byref(n)))
    return out[: n.value].copy()


def oscar_free_pages(h) -> int:
    n = ctypes.c_int32()
    _check(lib().oscar_free_pages(h, ctypes.byref(n)))
    return n.value


def oscar_export_history(h, seq: int, first: int, count: int, Hkv: int, d: int, G: int, stream=None):
    """Returns (codes u8 [count][Hkv][2][d/4], params u16 [count][Hkv][2][d/G][2])."""
    codes = np.zeros((count, Hkv, 2, d // 4), dtype=np.uint8)
    params = np.zeros((count, Hkv, 2, d // G, 2), dtype=np.uint16)
    _check(lib().oscar_export_history(h, seq, first, count, _np_ptr(codes), _np_ptr(params), _stream(stream)))
    return codes, params


def oscar_export_state(h, seq: int, max_pages: int, codes_dev, params_dev, stream=None) -> np.ndarray:
    """Enqueue the device export of a sequence's history (canonical layout) into
    codes_dev (uint8) / params_dev (uint16) device tensors; returns the page-table
    row (int32 [max_pages], -1 past its end)."""
    table = np.zeros(max(max_pages, 1), dtype=np.int32)
    _check(lib().oscar_export_state(h, seq, _np_ptr(table), _dev_ptr(codes_dev), _dev_ptr(params_dev),
                                    _stream(stream)))
    return table[:max_pages]


def oscar_export_history_bf16(h, seq: int, first: int, count: int, Hkv: int, d: int, stream=None):
    """BF16-history pools: (k, v) bf16 bits [count][Hkv][d] of history entries [first, first+count)."""
    k = np.zeros((count, Hkv, d), dtype=np.uint16)
    v = np.zeros((count, Hkv, d), dtype=np.uint16)
    _check(lib().oscar_export_history_bf16(h, seq, first, count, _np_ptr(k), _np_ptr(v), _stream(stream)))
    return k, v


def oscar_export_window(h, seq: int, Hkv: int, d: int, stream=None):
    """Returns bf16 bit patterns (sink_k, sink_v [64][Hkv][d], recent_k, recent_v [256][Hkv][d])."""
    outs = [np.zeros((n, Hkv, d), dtype=np.uint16) for n in (SINK_TOKENS, SINK_TOKENS, RECENT_TOKENS, RECENT_TOKENS)]
    _check(lib().oscar_export_window(h, seq, *[_np_ptr(o) for o in outs], _stream(stream)))
    return tuple(outs)


def oscar_build_rotation(U: np.ndarray) -> np.ndarray:
    """R = U . H . Pi for one head (host fp32 [d][d])."""
    U = np.ascontiguousarray(U, dtype=np.float32)
    d = U.shape[-1]
    R = np.empty((d, d), dtype=np.float32)
    _check(lib().oscar_build_rotation(d, _np_ptr(U), _np_ptr(R)))
    return R


def oscar_calibrate_clip(x_bf16: np.ndarray, R: np.ndarray, pct: float = 99.0) -> np.ndarray:
    """Per-channel clip thresholds from host bf16 tokens x [n][d] (uint16 bits)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    R = np.ascontiguousarray(R, dtype=np.float32)
    n, d = x.shape
    out = np.empty(d, dtype=np.float32)
    _check(lib().oscar_calibrate_clip(d, n, _np_ptr(x), _np_ptr(R), float(pct), _np_ptr(out)))
    return out


LLOYD_ITERS = 32


def oscar_lloyd_max_codebook(x_bf16: np.ndarray, R: np.ndarray, clip: np.ndarray, G: int,
                             iters: int = LLOYD_ITERS) -> np.ndarray:
    """uint8 [4] Lloyd-Max codebook of one head from host bf16 tokens x [n][d] (uint16 bits)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    n, d = x.shape
    R = np.ascontiguousarray(R, dtype=np.float32)
    clip = np.ascontiguousarray(clip, dtype=np.float32)
    out = np.empty(4, dtype=np.uint8)
    _check(lib().oscar_lloyd_max_codebook(d, G, n, _np_ptr(x), _np_ptr(R), _np_ptr(clip), iters, _np_ptr(out)))
    return out


def oscar_calib_workspace_bytes(n: int, num_q_heads: int, head_dim: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().oscar_calib_workspace_bytes(n, num_q_heads, head_dim, ctypes.byref(b)))
    return b.value


def oscar_calib_attention(q, k, v, softmax_scale: float, out=None, stream=None):
    """S V per query head (device fp32 [n][Hq][d]) of one calibration sequence:
    q bf16 [n][Hq][d], k, v bf16 [n][Hkv][d] (device tensors)."""
    import torch
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    if out is None:
        out = torch.empty((n, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().oscar_calib_attention(n, Hq, Hkv, d, _dev_ptr(q), _dev_ptr(k), _dev_ptr(v),
                                       float(softmax_scale), _dev_ptr(out), _stream(stream)))
    return out


def oscar_calib_covariance(q, k, v, softmax_scale: float, cov_k, cov_v, workspace=None, stream=None):
    """Adds Q^T Q and (S V)^T (S V) per kv head to cov_k, cov_v (device fp32 [Hkv][d][d])."""
    import torch
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    if workspace is None:
        workspace = torch.empty(max(1, oscar_calib_workspace_bytes(n, Hq, d)), dtype=torch.uint8, device=q.device)
    _check(lib().oscar_calib_covariance(n, Hq, Hkv, d, _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), float(softmax_scale),
                                        _dev_ptr(cov_k), _dev_ptr(cov_v), _dev_ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))


def oscar_calib_rotation(cov: np.ndarray):
    """(R, U [d][d] fp32, eigenvalues [d] fp64, descending) of one head's host covariance."""
    cov = np.ascontiguousarray(cov, dtype=np.float32)
    d = cov.shape[-1]
    R = np.empty((d, d), dtype=np.float32)
    U = np.empty((d, d), dtype=np.float32)
    w = np.empty(d, dtype=np.float64)
    _check(lib().oscar_calib_rotation(d, _np_ptr(cov), _np_ptr(U), _np_ptr(R), _np_ptr(w)))
    return R, U, w


PROFILE_DECODE_MAIN, PROFILE_DECODE_MERGE, PROFILE_APPEND = 1, 2, 4


def oscar_profile_begin(h, max_calls: int, kernels: int = PROFILE_DECODE_MAIN, every: int = 1):
    _check(lib().oscar_profile_begin(h, max_calls, kernels, every))


def oscar_profile_end(h) -> Profile:
    out = Profile()
    _check(lib().oscar_profile_end(h, ctypes.byref(out)))
    return out


# ---------------------------------------------------------------------------
# convenience: a pool that owns its torch device buffers
# ---------------------------------------------------------------------------

def make_config(max_seqs, num_q_heads, num_kv_heads, head_dim, group_size, num_pages,
                max_pages_per_seq, page_shuffle_seed=0, flags=0) -> PoolConfig:
    return PoolConfig(max_seqs, num_q_heads, num_kv_heads, head_dim, group_size, num_pages,
                      max_pages_per_seq, flags, page_shuffle_seed & (2**64 - 1))


class Pool:
    """A pool whose device buffer and decode workspace are torch tensors."""

    def __init__(self, cfg: PoolConfig, R_K, R_V, clip_K, clip_V, max_batch: int = 256,
                 device="cuda", stream=None):
        import torch
        self.cfg = cfg
        self.host_only = bool(cfg.flags & POOL_HOST_ONLY)
        if self.host_only:
            self.buf = None
            self.workspace = None
            self.handle = oscar_pool_create(cfg, None, 0, None, None, None, None)
        else:
            nbytes = oscar_pool_bytes(cfg)
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self.workspace = torch.empty(max(oscar_decode_workspace_bytes(cfg, max_batch), 4) // 4,
                                         dtype=torch.float32, device=device)
            self.handle = oscar_pool_create(cfg, self.buf, nbytes, R_K, R_V, clip_K, clip_V, stream)

    def close(self):
        if self.handle is not None:
            oscar_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill(self, seq, k, v, stream=None):
        L = 0 if k is None else k.shape[0]
        oscar_prefill(self.handle, seq, k, v, L, stream, host_only=self.host_only)

    def prefill_len(self, seq, L):
        """Host-only pools: prefill bookkeeping for a prompt of length L."""
        _check(lib().oscar_prefill(self.handle, seq, None, None, L, None))

    def append(self, seq_ids, k_new, v_new, stream=None):
        oscar_append_evict(self.handle, seq_ids, k_new, v_new, stream, host_only=self.host_only)

    def decode(self, seq_ids, q, out=None, softmax_scale=None, stream=None):
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if softmax_scale is None:
            softmax_scale = 1.0 / float(np.sqrt(self.cfg.head_dim))
        oscar_decode_attn(self.handle, seq_ids, q, out, softmax_scale, self.workspace, stream)
        return out

    def step(self, seq_ids, k_new, v_new, q, out=None, softmax_scale=None, stream=None):
        """append(seq_ids, k_new, v_new) then decode(seq_ids, q) in one call."""
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if softmax_scale is None:
            softmax_scale = 1.0 / float(np.sqrt(self.cfg.head_dim))
        oscar_decode_step(self.handle, seq_ids, k_new, v_new, q, out, softmax_scale, self.workspace, stream)
        return out

    def step_static(self, seq_ids, k_new, v_new, q, out=None, softmax_scale=None, stream=None):
        """step() with the library's static workspace (oscar_decode_step_static)."""
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if softmax_scale is None:
            softmax_scale = 1.0 / float(np.sqrt(self.cfg.head_dim))
        oscar_decode_step_static(self.handle, seq_ids, k_new, v_new, q, out, softmax_scale, stream)
        return out

    def prefill_attn(self, seq, q, out=None, softmax_scale=None, workspace=None, stream=None):
        """Causal attention of the last q.shape[0] positions of `seq` (oscar_prefill_attn)."""
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if softmax_scale is None:
            softmax_scale = 1.0 / float(np.sqrt(self.cfg.head_dim))
        if workspace is None:
            n = oscar_prefill_workspace_bytes(self.cfg, q.shape[0])
            workspace = torch.empty(max(n, 4) // 4, dtype=torch.float32, device=q.device)
        oscar_prefill_attn(self.handle, seq, q, out, softmax_scale, workspace, stream)
        return out

    def check(self, stream=None):
        """oscar_pool_check: raises OscarError(EHIP) if a decode wait gave up."""
        oscar_pool_check(self.handle, stream, host_only=self.host_only)

    def length(self, seq):
        return oscar_seq_length(self.handle, seq)

    def page_table(self, seq):
        return oscar_page_table(self.handle, seq, self.cfg.max_pages_per_seq)

    def free_pages(self):
        return oscar_free_pages(self.handle)

    def release(self, seq):
        oscar_release_seq(self.handle, seq)

    def set_codebook(self, levels_k, levels_v, stream=None):
        """Lloyd-Max pools: uint8 [Hkv][4] codebooks for K and V."""
        lk = np.ascontiguousarray(levels_k, dtype=np.uint8)
        lv = np.ascontiguousarray(levels_v, dtype=np.uint8)
        _check(lib().oscar_pool_set_codebook(self.handle, _np_ptr(lk), _np_ptr(lv),
                                             None if self.host_only else _stream(stream)))

    def fork(self, src, dst, stream=None):
        """Prefix sharing: empty sequence dst takes src's state, history pages shared."""
        oscar_fork_seq(self.handle, src, dst, stream, host_only=self.host_only)

    def export_history(self, seq, first, count, stream=None):
        c = self.cfg
        return oscar_export_history(self.handle, seq, first, count, c.num_kv_heads, c.head_dim,
                                    c.group_size, stream)

    def profile_begin(self, max_calls, kernels=PROFILE_DECODE_MAIN, every=1):
        oscar_profile_begin(self.handle, max_calls, kernels, every)

    def profile_end(self) -> Profile:
        return oscar_profile_end(self.handle)

    def export_window(self, seq, stream=None):
        return oscar_export_window(self.handle, seq, self.cfg.num_kv_heads, self.cfg.head_dim, stream)
