// Eviction / prefill encoder for gfx950: rotate by R, clip, quantize to four
// levels with a group-wise fp16 scale and zero point, pack 2-bit codes into
// the paged history, and maintain the BF16 sink and recent windows.
//
// Method: news article on OSCAR (sanyangsrq.com), section "From offline
// calibration to online inference" — the oldest recent-window token is
// rotated, clipped, quantized and packed (four 2-bit values per byte) by one
// fused kernel and moved into the INT2 history; section "OSCAR aims the
// rotation at attention" — R = U . Hadamard . bit-reversal and the clip
// thresholds are fixed offline.
//
// Arithmetic (kept identical to the definition so codes are reproducible):
//   y_j = fma chain over i = 0..d-1 of x_i * R[i][j] in fp32 from +0,
//   y_j = min(max(y_j, -c_j), c_j),
//   per group of G channels: s = fp16_rne((max - min) / 3), z = fp16_rne(min),
//   code = s == 0 ? 0 : clamp(rint((y - z) / s), 0, 3), with the fp16 s, z.
// One thread owns one output channel j and keeps column j of R in registers,
// so every token costs d fused multiply-adds per thread in a fixed order.
// The rotation is d x d per token (~33 MFLOP per step for 64 sequences x 8
// heads x K,V): it is far too small to pay for MFMA tiles, and MFMA would not
// reproduce the fixed accumulation order the codes are defined with.
#include <algorithm>

#include "oscar_internal.h"

namespace oscar {
namespace {

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f16_bits(float f) {
  _Float16 h = (_Float16)f; // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_val(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Lane permutations inside each 16-lane row (DPP): swap neighbours, swap
// pairs, mirror each half row, mirror the row.  Four of them reach every
// lane of the row.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <class Op>
__device__ __forceinline__ uint32_t row16_reduce(uint32_t v, Op op) {
  v = op(v, dpp_u<0xB1>(v));  // quad_perm [1,0,3,2]
  v = op(v, dpp_u<0x4E>(v));  // quad_perm [2,3,0,1]
  v = op(v, dpp_u<0x141>(v)); // row_half_mirror
  return op(v, dpp_u<0x140>(v)); // row_mirror
}
__device__ __forceinline__ float lane_f(float v, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}
__device__ __forceinline__ float fmin_u(uint32_t a, uint32_t b) { return fminf(__uint_as_float(a), __uint_as_float(b)); }
__device__ __forceinline__ float fmax_u(uint32_t a, uint32_t b) { return fmaxf(__uint_as_float(a), __uint_as_float(b)); }
// Minimum / maximum over the 64 lanes of the wave: rows by DPP, then the
// four row results by readlane.  Exact in any order.
__device__ __forceinline__ float wave_min(float v) {
  v = __uint_as_float(row16_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) { return __float_as_uint(fmin_u(a, b)); }));
  return fminf(fminf(lane_f(v, 0), lane_f(v, 16)), fminf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_max(float v) {
  v = __uint_as_float(row16_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) { return __float_as_uint(fmax_u(a, b)); }));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
// OR of a value over the 16 lanes of an aligned lane group.
__device__ __forceinline__ uint32_t or16(uint32_t v) {
  return row16_reduce(v, [](uint32_t a, uint32_t b) { return a | b; });
}

// Quantize this thread's clipped value y (channel j) of one token.  `red`
// is LDS scratch of 2 * (D/64) floats.  Returns the code and sets the
// group's fp16 scale/zero bits (uniform over the group).
template <int D, int G>
__device__ __forceinline__ uint32_t quantize_channel(float y, float *red, uint16_t &s16, uint16_t &z16,
                                                     bool lut = false, uint32_t lw = 0) {
  const int j = threadIdx.x, w = j / 64;
  float mn = wave_min(y), mx = wave_max(y);
  if (G > 64) {
    // a group spans G/64 waves: combine through LDS
    if ((j & 63) == 0) {
      red[2 * w] = mn;
      red[2 * w + 1] = mx;
    }
    __syncthreads();
    const int w0 = (j / G) * (G / 64);
    mn = red[2 * w0];
    mx = red[2 * w0 + 1];
#pragma unroll
    for (int k = 1; k < G / 64; ++k) {
      mn = fminf(mn, red[2 * (w0 + k)]);
      mx = fmaxf(mx, red[2 * (w0 + k) + 1]);
    }
    __syncthreads();
  }
  // "+ 0.0f" stores an exactly zero range or minimum as +0 whatever the
  // sign of the zeros min/max returned
  s16 = f16_bits(((mx - mn) + 0.0f) / 3.0f);
  z16 = f16_bits(mn + 0.0f);
  const float s = f16_val(s16), z = f16_val(z16);
  if (lut) return lut_code(y, z, s, lw);
  float q = 0.0f;
  if (s != 0.0f) q = fminf(fmaxf(rintf((y - z) / s), 0.0f), 3.0f);
  return (uint32_t)q;
}

// Write token slot t's K code of channel j: 16 lanes assemble one dword.
template <int D>
__device__ __forceinline__ void store_k_code(uint8_t *blk, int t, uint32_t code) {
  const int j = threadIdx.x;
  uint32_t dw = or16(code << (2 * (j & 15)));
  if ((j & 15) == 0) {
    const int r = (j & 63) / 16, m = j / 64;
    *(uint32_t *)(blk + kcode_dword_off(D, t, r, m)) = dw;
  }
}

template <int D, int G>
__device__ __forceinline__ void store_params(uint8_t *blk, int off, uint16_t s16, uint16_t z16) {
  if ((threadIdx.x % G) == 0) *(uint32_t *)(blk + off) = (uint32_t)s16 | ((uint32_t)z16 << 16);
}

// ---------------------------------------------------------------------------
// Prefill: one block per (history page of the prompt, kv head, K|V).
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(D) void prefill_encode_kernel(PoolDev p, int seq, const uint16_t *__restrict__ k,
                                                           const uint16_t *__restrict__ v, int n_hist) {
  const int pg_idx = blockIdx.x, kv = blockIdx.y, kind = blockIdx.z, j = threadIdx.x;
  const int Hkv = p.Hkv;
  const float *R = (kind ? p.RV : p.RK) + (size_t)kv * D * D;
  const float c = (kind ? p.clipV : p.clipK)[kv * D + j];
  const uint16_t *src = kind ? v : k;
  __shared__ float xs[kPage][D];
  __shared__ float red[2 * (D / 64)];

  float rc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) rc[i] = R[i * D + j];

  const int t0 = pg_idx * kPage;
  const int nt = min(kPage, n_hist - t0);
  for (int t = 0; t < nt; ++t)
    xs[t][j] = bf16f(src[((size_t)(kSink + t0 + t) * Hkv + kv) * D + j]);
  __syncthreads();

  const int page = p.page_table[(size_t)seq * p.maxp + pg_idx];
  uint8_t *blk = p.pages + ((size_t)page * Hkv + kv) * p.block_bytes;
  const uint32_t lw = p.lut ? p.codebook[kind * Hkv + kv] : 0u;
  uint32_t vdw[kPage / 16] = {0, 0, 0, 0};
  for (int t = 0; t < nt; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) acc = fmaf(xs[t][i], rc[i], acc);
    const float y = fminf(fmaxf(acc, -c), c);
    uint16_t s16, z16;
    const uint32_t code = quantize_channel<D, G>(y, red, s16, z16, p.lut != 0, lw);
    if (kind == 0) {
      store_k_code<D>(blk, t, code);
      store_params<D, G>(blk, kparam_off(D, G, t, j / G), s16, z16);
    } else {
      vdw[t / 16] |= code << vbit(t % 16);
      store_params<D, G>(blk, vparam_off(D, G, t, j / G), s16, z16);
    }
  }
  if (kind == 1) {
#pragma unroll
    for (int tb = 0; tb < kPage / 16; ++tb)
      if (tb * 16 < nt) *(uint32_t *)(blk + vcode_dword_off(D, tb, j)) = vdw[tb];
  }
}

// Prefill of a BF16-history pool: the history tokens are copied into their
// pages.  grid (history pages, Hkv, K|V), block D.
template <int D>
__global__ __launch_bounds__(D) void prefill_copy_kernel(PoolDev p, int seq, const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v, int n_hist) {
  const int pg_idx = blockIdx.x, kv = blockIdx.y, kind = blockIdx.z, j = threadIdx.x, Hkv = p.Hkv;
  const uint16_t *src = kind ? v : k;
  const int page = p.page_table[(size_t)seq * p.maxp + pg_idx];
  uint16_t *dst = (uint16_t *)(p.pages + ((size_t)page * Hkv + kv) * p.block_bytes) + (kind ? kPage * D : 0);
  const int t0 = pg_idx * kPage, nt = min(kPage, n_hist - t0);
  for (int t = 0; t < nt; ++t) dst[t * D + j] = src[((size_t)(kSink + t0 + t) * Hkv + kv) * D + j];
}

// Prefill: copy sink and recent positions into the BF16 windows.
// grid (window positions, Hkv), block D: position index u < n_sink is sink
// position u; otherwise recent position n_hist + 64 + (u - n_sink).
template <int D>
__global__ void prefill_window_kernel(PoolDev p, int seq, const uint16_t *__restrict__ k,
                                      const uint16_t *__restrict__ v, int n_sink, int n_hist) {
  const int u = blockIdx.x, kv = blockIdx.y, j = threadIdx.x, Hkv = p.Hkv;
  int pos;
  size_t dst;
  if (u < n_sink) {
    pos = u;
    dst = (((size_t)seq * Hkv + kv) * kSink + pos) * D + j;
    p.sinkK[dst] = k[((size_t)pos * Hkv + kv) * D + j];
    p.sinkV[dst] = v[((size_t)pos * Hkv + kv) * D + j];
  } else {
    pos = kSink + n_hist + (u - n_sink);
    dst = (((size_t)seq * Hkv + kv) * kRecent + (pos - kSink) % kRecent) * D + j;
    p.recentK[dst] = k[((size_t)pos * Hkv + kv) * D + j];
    p.recentV[dst] = v[((size_t)pos * Hkv + kv) * D + j];
  }
}

// ---------------------------------------------------------------------------
// Append: grid (ceil(n / spb), Hkv, K|V), block D: spb consecutive
// sequences per block, one after the other, so that column j of R (the
// loads of a thread) is read once per block rather than once per sequence.
// Per sequence, the loads a token needs (its page id, the evicted element)
// are issued together before they are used.
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(D) void append_kernel(PoolDev p, AppendBatch b, const uint16_t *__restrict__ k_new,
                                                   const uint16_t *__restrict__ v_new, int spb) {
  const int kv = blockIdx.y, kind = blockIdx.z, j = threadIdx.x, Hkv = p.Hkv;
  const int e0 = blockIdx.x * spb, e1 = min(b.n, e0 + spb);
  __shared__ float xs[D];
  __shared__ float red[2 * (D / 64)];
  // column j of R, loaded once for the block's sequences (a block whose
  // sequences do not evict, or a BF16-history pool, leaves it unused)
  float rc[D];
  {
    const float *R = (kind ? p.RV : p.RK) + (size_t)kv * D * D;
#pragma unroll
    for (int i = 0; i < D; ++i) rc[i] = R[i * D + j];
  }
  for (int e = e0; e < e1; ++e) {
    const int seq = b.seq[e], L = b.len[e]; // length before the append
    const uint16_t xnew = (kind ? v_new : k_new)[((size_t)e * Hkv + kv) * D + j];
    if (L < kSink) {
      (kind ? p.sinkV : p.sinkK)[(((size_t)seq * Hkv + kv) * kSink + L) * D + j] = xnew;
      continue;
    }
    const int slot = (L - kSink) % kRecent;
    uint16_t *rs = (kind ? p.recentV : p.recentK) + (((size_t)seq * Hkv + kv) * kRecent + slot) * D;
    if (L < kWindow) {
      rs[j] = xnew;
      continue;
    }
    // evict the oldest recent token (held in this slot) into history n_hist
    const int n_hist = L - kWindow, pg_idx = n_hist / kPage, t = n_hist % kPage;
    const int page = b.new_page[e] >= 0 ? b.new_page[e] : p.page_table[(size_t)seq * p.maxp + pg_idx];
    if (p.bf16_hist) {
      // BF16-history pool: the token is copied as it is
      uint16_t *dst = (uint16_t *)(p.pages + ((size_t)page * Hkv + kv) * p.block_bytes) + (kind ? kPage * D : 0);
      dst[t * D + j] = rs[j];
      rs[j] = xnew; // this thread read element j above; no other thread touches it
      if (b.new_page[e] >= 0 && kv == 0 && kind == 0 && j == 0) p.page_table[(size_t)seq * p.maxp + pg_idx] = page;
      continue;
    }
    const float xj = bf16f(rs[j]);
    const float c = (kind ? p.clipV : p.clipK)[kv * D + j];
    // (the branches above are block-uniform; the previous sequence's reads
    // of xs and red ended before the barriers of its quantization)
    xs[j] = xj;
    rs[j] = xnew; // this thread read element j above; no other thread touches it
    __syncthreads();
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) acc = fmaf(xs[i], rc[i], acc);
    const float y = fminf(fmaxf(acc, -c), c);
    uint16_t s16, z16;
    const uint32_t code =
        quantize_channel<D, G>(y, red, s16, z16, p.lut != 0, p.lut ? p.codebook[kind * Hkv + kv] : 0u);
    if (b.new_page[e] >= 0 && kv == 0 && kind == 0 && j == 0) p.page_table[(size_t)seq * p.maxp + pg_idx] = page;
    uint8_t *blk = p.pages + ((size_t)page * Hkv + kv) * p.block_bytes;
    if (kind == 0) {
      store_k_code<D>(blk, t, code);
      store_params<D, G>(blk, kparam_off(D, G, t, j / G), s16, z16);
    } else {
      // a byte holds four tokens of channel j (those with equal k & 1 and
      // k >> 3, k = t % 16); the first of them, k & 6 == 0, starts the byte
      const int k = t % 16;
      uint8_t *byte = blk + vcode_dword_off(D, t / 16, j) + vbit(k) / 8;
      const int sh = vbit(k) % 8;
      const uint32_t old = (k & 6) == 0 ? 0u : *byte;
      *byte = (uint8_t)((old & ~(3u << sh)) | (code << sh));
      store_params<D, G>(blk, vparam_off(D, G, t, j / G), s16, z16);
    }
  }
}

// ---------------------------------------------------------------------------
// Export of a sequence's history in the canonical layout (device to device):
// one thread per output word.  Threads [0, nc) write code dwords: word
// (i, h, kind, w) holds canonical bytes 4w .. 4w + 3 of history entry i,
// i.e. channels 16w .. 16w + 15, four per byte, the first in the low bits.
// Threads [nc, nc + np) write the fp16 (scale, zero) pair of (i, h, kind,
// group).  Every read stays inside the entry's (page, head) block.
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ void export_state_kernel(PoolDev p, int seq, int n_hist, uint32_t *__restrict__ codes,
                                    uint32_t *__restrict__ params) {
  constexpr int CW = D / 16, NG = D / G; // code dwords and groups per (entry, head, kind)
  const long Hkv = p.Hkv;
  const long nc = (long)n_hist * Hkv * 2 * CW, np = (long)n_hist * Hkv * 2 * NG;
  const long x = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= nc + np) return;
  const bool is_code = x < nc;
  const long y = is_code ? x : x - nc;
  const int per = is_code ? CW : NG;
  const int w = (int)(y % per);
  const long ihk = y / per;
  const int kind = (int)(ihk % 2);
  const int h = (int)((ihk / 2) % Hkv);
  const int i = (int)(ihk / (2 * Hkv));
  const int t = i % kPage;
  const int page = p.page_table[(size_t)seq * p.maxp + i / kPage];
  const uint8_t *blk = p.pages + ((size_t)page * Hkv + h) * p.block_bytes;
  if (!is_code) {
    params[y] = *(const uint32_t *)(blk + (kind ? vparam_off(D, G, t, w) : kparam_off(D, G, t, w)));
    return;
  }
  uint32_t out = 0;
  if (kind == 0) {
    // channels 16 w + k, k < 16: one K code dword (quad r, 64-channel block m)
    const uint32_t kw = *(const uint32_t *)(blk + kcode_dword_off(D, t, w % 4, w / 4));
    out = kw; // channel 16 w + k at bits 2k, as the canonical bytes hold it
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t vw = *(const uint32_t *)(blk + vcode_dword_off(D, t / 16, 16 * w + k));
      out |= ((vw >> vbit(t % 16)) & 3u) << (2 * k);
    }
  }
  codes[y] = out;
}

// ---------------------------------------------------------------------------
// Prefix sharing.  Copy on write: grid (n, chunks), 256 threads; the blocks
// of page c.src[i] for every kv head, one contiguous run of Hkv x block_bytes
// bytes (a multiple of 16), go to page c.dst[i], 16 bytes per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_pages_kernel(PoolDev p, PageCopies c) {
  const size_t bytes = (size_t)p.Hkv * p.block_bytes, words = bytes / 16;
  const uint4 *src = (const uint4 *)(p.pages + (size_t)c.src[blockIdx.x] * bytes);
  uint4 *dst = (uint4 *)(p.pages + (size_t)c.dst[blockIdx.x] * bytes);
  for (size_t i = (size_t)blockIdx.y * 256 + threadIdx.x; i < words; i += (size_t)gridDim.y * 256) dst[i] = src[i];
}

// Fork: grid (chunks, 5), 256 threads.  Regions 0..3 are sequence src's
// sinkK, sinkV, recentK, recentV (Hkv x slots x d bf16 each, a multiple of 16
// bytes), copied to sequence dst 16 bytes per thread; region 4 is the first
// np entries of its page-table row.
__global__ __launch_bounds__(256) void fork_kernel(PoolDev p, int src, int dst, int np) {
  const int r = blockIdx.y;
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x, stride = (size_t)gridDim.x * 256;
  if (r == 4) {
    for (size_t i = tid; i < (size_t)np; i += stride)
      p.page_table[(size_t)dst * p.maxp + i] = p.page_table[(size_t)src * p.maxp + i];
    return;
  }
  const size_t words = (size_t)p.Hkv * (r < 2 ? kSink : kRecent) * p.d * 2 / 16;
  const uint16_t *base = r == 0 ? p.sinkK : r == 1 ? p.sinkV : r == 2 ? p.recentK : p.recentV;
  const uint4 *from = (const uint4 *)base + (size_t)src * words;
  uint4 *to = (uint4 *)base + (size_t)dst * words;
  for (size_t i = tid; i < words; i += stride) to[i] = from[i];
}

template <int D, int G>
hipError_t export_impl(const PoolDev &p, int seq, int n_hist, uint8_t *codes, uint16_t *params, hipStream_t s) {
  const long total = (long)n_hist * p.Hkv * 2 * (D / 16 + D / G);
  const int threads = 256;
  const long blocks = (total + threads - 1) / threads;
  if (blocks > 0)
    hipLaunchKernelGGL((export_state_kernel<D, G>), dim3((unsigned)blocks), dim3(threads), 0, s, p, seq, n_hist,
                       (uint32_t *)codes, (uint32_t *)params);
  return hipGetLastError();
}

template <int D, int G>
hipError_t prefill_impl(const PoolDev &p, int seq, const uint16_t *k, const uint16_t *v, int L, hipStream_t s) {
  const int n_hist = max(0, L - kWindow);
  const int n_sink = min(L, kSink);
  const int n_rec = L - n_sink - n_hist;
  if (n_sink + n_rec > 0)
    hipLaunchKernelGGL(prefill_window_kernel<D>, dim3(n_sink + n_rec, p.Hkv), dim3(D), 0, s, p, seq, k, v,
                       n_sink, n_hist);
  if (n_hist > 0) {
    const int np = (n_hist + kPage - 1) / kPage;
    if (p.bf16_hist)
      hipLaunchKernelGGL((prefill_copy_kernel<D>), dim3(np, p.Hkv, 2), dim3(D), 0, s, p, seq, k, v, n_hist);
    else
      hipLaunchKernelGGL((prefill_encode_kernel<D, G>), dim3(np, p.Hkv, 2), dim3(D), 0, s, p, seq, k, v, n_hist);
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t append_impl(const PoolDev &p, const AppendBatch &b, const uint16_t *kn, const uint16_t *vn,
                       hipStream_t s, const KernelTimer &t) {
  // sequences per block: about 512 blocks (two per compute unit), at most 8
  const int spb = std::max(1, std::min(8, b.n * p.Hkv * 2 / 512));
  if (t.on) (void)hipEventRecord(t.ev[0], s);
  hipLaunchKernelGGL((append_kernel<D, G>), dim3((b.n + spb - 1) / spb, p.Hkv, 2), dim3(D), 0, s, p, b, kn, vn, spb);
  if (t.on) (void)hipEventRecord(t.ev[1], s);
  return hipGetLastError();
}

} // namespace

hipError_t launch_prefill(const PoolDev &p, int seq, const uint16_t *k, const uint16_t *v, int L, hipStream_t s) {
  if (p.d == 128 && p.G == 128) return prefill_impl<128, 128>(p, seq, k, v, L, s);
  if (p.d == 128 && p.G == 64) return prefill_impl<128, 64>(p, seq, k, v, L, s);
  if (p.d == 64 && p.G == 64) return prefill_impl<64, 64>(p, seq, k, v, L, s);
  return hipErrorInvalidValue;
}

hipError_t launch_export(const PoolDev &p, int seq, int n_hist, uint8_t *codes, uint16_t *params, hipStream_t s) {
  if (p.d == 128 && p.G == 128) return export_impl<128, 128>(p, seq, n_hist, codes, params, s);
  if (p.d == 128 && p.G == 64) return export_impl<128, 64>(p, seq, n_hist, codes, params, s);
  if (p.d == 64 && p.G == 64) return export_impl<64, 64>(p, seq, n_hist, codes, params, s);
  return hipErrorInvalidValue;
}

hipError_t launch_copy_pages(const PoolDev &p, const PageCopies &c, hipStream_t s) {
  if (c.n <= 0) return hipSuccess;
  const size_t words = (size_t)p.Hkv * p.block_bytes / 16;
  const unsigned chunks = (unsigned)std::min<size_t>((words + 255) / 256, 16);
  hipLaunchKernelGGL(copy_pages_kernel, dim3(c.n, chunks), dim3(256), 0, s, p, c);
  return hipGetLastError();
}

hipError_t launch_fork(const PoolDev &p, int src, int dst, int np, hipStream_t s) {
  const size_t words = (size_t)p.Hkv * kRecent * p.d * 2 / 16; // the largest region
  const unsigned chunks = (unsigned)std::min<size_t>((words + 255) / 256, 64);
  hipLaunchKernelGGL(fork_kernel, dim3(chunks, 5), dim3(256), 0, s, p, src, dst, np);
  return hipGetLastError();
}

hipError_t launch_append(const PoolDev &p, const AppendBatch &b, const uint16_t *kn, const uint16_t *vn,
                         hipStream_t s, const KernelTimer &t) {
  if (p.d == 128 && p.G == 128) return append_impl<128, 128>(p, b, kn, vn, s, t);
  if (p.d == 128 && p.G == 64) return append_impl<128, 64>(p, b, kn, vn, s, t);
  if (p.d == 64 && p.G == 64) return append_impl<64, 64>(p, b, kn, vn, s, t);
  return hipErrorInvalidValue;
}

} // namespace oscar
