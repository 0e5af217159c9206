// Decode attention over the three-segment pool on gfx950.
//
// Method: news article on OSCAR (sanyangsrq.com), section "From offline
// calibration to online inference": decode handles the two precisions
// separately — an INT2 kernel unpacks the history, dequantizes with scale
// and zero point and accumulates in floating point; a BF16 kernel covers the
// sink and recent tokens; an online softmax merges the two results.
//
// Launches (one stream):
//   decode_main_kernel: two block roles in one grid.
//     * split blocks, one per (sequence, kv head, run of pages): rotate the
//       g = Hq/Hkv queries by R_K, attend to the INT2 history in the rotated
//       basis, write a partial (m, l, acc) per query head;
//     * window blocks, one per (sequence, kv head): attend to the BF16 sink
//       and recent tokens with the raw queries, write one partial.
//   decode_merge_kernel: one block per (sequence, kv head): merge the split
//     partials, de-rotate the history accumulator by R_V^T, merge with the
//     window partial, normalise, write fp32.
// Softmax runs in base 2: logits are pre-multiplied by scale * log2(e).
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_val(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int D, int G, int GQ>
struct Smem {
  float qs[GQ][D];             // scaled (and, for history, rotated) queries
  float qsum[GQ][D / G];       // per-group sums of the rotated queries
  float P[kWaves][GQ][64];     // softmax numerators of the current tile
  float vsz[kWaves][64][2 * (D / G)]; // V scale/zero of the current page
  float M[kWaves][GQ], L[kWaves][GQ];
  float A[kWaves][GQ][D];      // per-wave accumulators for the block merge
};

// Online-softmax update of one 64-token tile for one wave.  lg: this lane's
// logits (-inf for an empty lane).  Writes the tile's numerators to P and
// returns the rescale factor of each head through alpha.
template <int GQ>
__device__ __forceinline__ void softmax_tile(const float (&lg)[GQ], float (&m_run)[GQ], float (&l_run)[GQ],
                                             float (&alpha)[GQ], float (*P)[64], int lane) {
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const float mt = wave_max(lg[h]);
    const float mnew = fmaxf(m_run[h], mt);
    alpha[h] = exp2f(m_run[h] - mnew); // m_run = -inf at the start gives 0
    const float pr = exp2f(lg[h] - mnew);
    l_run[h] = l_run[h] * alpha[h] + wave_sum(pr);
    m_run[h] = mnew;
    P[h][lane] = pr;
  }
}

// Merge the per-wave (m, l, acc) of a block and store one partial per head.
template <int D, int G, int GQ>
__device__ void block_merge_store(Smem<D, G, GQ> &sm, const float (&m_run)[GQ], const float (&l_run)[GQ],
                                  const float (&acc)[GQ][D / 64], float *dst /*[GQ][D+2]*/) {
  const int tid = threadIdx.x, w = tid / 64, lane = tid % 64;
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    if (lane == 0) {
      sm.M[w][h] = m_run[h];
      sm.L[w][h] = l_run[h];
    }
#pragma unroll
    for (int k = 0; k < D / 64; ++k) sm.A[w][h][lane + 64 * k] = acc[h][k];
  }
  __syncthreads();
  for (int idx = tid; idx < GQ * D; idx += kThreads) {
    const int h = idx / D, c = idx % D;
    float m = -INFINITY;
    for (int ww = 0; ww < kWaves; ++ww) m = fmaxf(m, sm.M[ww][h]);
    float a = 0.f, l = 0.f;
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = sm.M[ww][h] == -INFINITY ? 0.f : exp2f(sm.M[ww][h] - m);
      a += f * sm.A[ww][h][c];
      l += f * sm.L[ww][h];
    }
    float *o = dst + (size_t)h * (D + 2);
    o[c] = a;
    if (c == 0) {
      o[D] = m;
      o[D + 1] = l;
    }
  }
}

template <int D, int G, int GQ>
__global__ __launch_bounds__(kThreads) void decode_main_kernel(PoolDev p, DecodeBatch b, const uint16_t *__restrict__ q,
                                                               float qscale, float *__restrict__ ws) {
  __shared__ Smem<D, G, GQ> sm;
  const int tid = threadIdx.x, w = tid / 64, lane = tid % 64;
  const int Hkv = p.Hkv, Hq = p.Hq;
  float *ws_win = ws;
  float *ws_hist = ws + (size_t)b.n * Hq * (D + 2);

  float m_run[GQ], l_run[GQ], alpha[GQ], acc[GQ][D / 64];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) acc[h][k] = 0.f;
  }

  if ((int)blockIdx.x < b.hist_blocks) {
    // ---------------- INT2 history split ----------------
    const int blk = blockIdx.x, kv = blk % Hkv, sidx = blk / Hkv;
    int lo = 0, hi = b.n;
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (b.split_prefix[mid] <= sidx) lo = mid;
      else hi = mid;
    }
    const int e = lo, s = sidx - b.split_prefix[e];
    const int seq = b.seq[e], n_hist = b.len[e] - kWindow;
    const int np = (n_hist + kPage - 1) / kPage;
    const int p0 = s * b.pages_per_split, p1 = min(np, p0 + b.pages_per_split);

    // q_rot = q . R_K, scaled by softmax_scale * log2(e)
    float(*qraw)[D] = (float(*)[D]) & sm.A[0][0][0];
    for (int idx = tid; idx < GQ * D; idx += kThreads)
      qraw[idx / D][idx % D] = bf16f(q[((size_t)e * Hq + kv * GQ + idx / D) * D + idx % D]);
    __syncthreads();
    const float *RK = p.RK + (size_t)kv * D * D;
    for (int idx = tid; idx < GQ * D; idx += kThreads) {
      const int h = idx / D, j = idx % D;
      float a = 0.f;
      for (int i = 0; i < D; ++i) a = fmaf(qraw[h][i], RK[i * D + j], a);
      sm.qs[h][j] = a * qscale;
    }
    __syncthreads();
    for (int idx = tid; idx < GQ * (D / G); idx += kThreads) {
      const int h = idx / (D / G), gi = idx % (D / G);
      float a = 0.f;
      for (int c = gi * G; c < (gi + 1) * G; ++c) a += sm.qs[h][c];
      sm.qsum[h][gi] = a;
    }
    __syncthreads();

    const int iters = (p1 - p0 + kWaves - 1) / kWaves;
    for (int it = 0; it < iters; ++it) {
      const int pi = p0 + it * kWaves + w;
      const bool active = pi < p1;
      const uint8_t *blkp = nullptr;
      int ntok = 0;
      if (active) {
        const int page = p.page_table[(size_t)seq * p.maxp + pi];
        blkp = p.pages + ((size_t)page * Hkv + kv) * p.block_bytes;
        ntok = min(kPage, n_hist - pi * kPage);
      }
      const int t = lane;
      const bool valid = active && t < ntok;
      if (active) {
        float lg[GQ];
#pragma unroll
        for (int h = 0; h < GQ; ++h) lg[h] = -INFINITY;
        if (valid) {
          float dot[GQ][D / G];
#pragma unroll
          for (int h = 0; h < GQ; ++h)
#pragma unroll
            for (int gi = 0; gi < D / G; ++gi) dot[h][gi] = 0.f;
#pragma unroll
          for (int m = 0; m < D / 64; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t dw = *(const uint32_t *)(blkp + kcode_dword_off(D, t, r, m));
#pragma unroll
              for (int k = 0; k < 16; ++k) {
                const int c = 64 * m + 16 * r + k;
                const float fc = (float)((dw >> (2 * k)) & 3u);
#pragma unroll
                for (int h = 0; h < GQ; ++h) dot[h][c / G] = fmaf(sm.qs[h][c], fc, dot[h][c / G]);
              }
            }
#pragma unroll
          for (int h = 0; h < GQ; ++h) lg[h] = 0.f;
#pragma unroll
          for (int gi = 0; gi < D / G; ++gi) {
            const uint32_t sz = *(const uint32_t *)(blkp + kparam_off(D, G, t, gi));
            const float sc = f16_val(sz & 0xffffu), zp = f16_val(sz >> 16);
#pragma unroll
            for (int h = 0; h < GQ; ++h) lg[h] += sc * dot[h][gi] + zp * sm.qsum[h][gi];
          }
#pragma unroll
          for (int gi = 0; gi < D / G; ++gi) {
            const uint32_t sz = *(const uint32_t *)(blkp + vparam_off(D, G, t, gi));
            sm.vsz[w][t][2 * gi] = f16_val(sz & 0xffffu);
            sm.vsz[w][t][2 * gi + 1] = f16_val(sz >> 16);
          }
        }
        softmax_tile<GQ>(lg, m_run, l_run, alpha, sm.P[w], lane);
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
          for (int k = 0; k < D / 64; ++k) acc[h][k] *= alpha[h];
      }
      __syncthreads();
      if (active) {
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
          const int c = lane + 64 * k;
          uint32_t vdw[4];
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) vdw[tb] = *(const uint32_t *)(blkp + vcode_dword_off(D, tb, c));
          for (int tt = 0; tt < ntok; ++tt) {
            const float code = (float)((vdw[tt / 16] >> (2 * (tt % 16))) & 3u);
            const float v = fmaf(code, sm.vsz[w][tt][2 * (c / G)], sm.vsz[w][tt][2 * (c / G) + 1]);
#pragma unroll
            for (int h = 0; h < GQ; ++h) acc[h][k] = fmaf(sm.P[w][h][tt], v, acc[h][k]);
          }
        }
      }
      __syncthreads();
    }
    block_merge_store<D, G, GQ>(sm, m_run, l_run, acc, ws_hist + (size_t)blk * GQ * (D + 2));
  } else {
    // ---------------- BF16 sink + recent window ----------------
    const int idx0 = blockIdx.x - b.hist_blocks, e = idx0 / Hkv, kv = idx0 % Hkv;
    const int seq = b.seq[e], L = b.len[e];
    const int n_sink = min(L, kSink), n_rec = min(max(L - kSink, 0), kRecent), n_win = n_sink + n_rec;
    for (int idx = tid; idx < GQ * D; idx += kThreads)
      sm.qs[idx / D][idx % D] = bf16f(q[((size_t)e * Hq + kv * GQ + idx / D) * D + idx % D]) * qscale;
    __syncthreads();
    const uint16_t *sinkK = p.sinkK + ((size_t)seq * Hkv + kv) * kSink * D;
    const uint16_t *sinkV = p.sinkV + ((size_t)seq * Hkv + kv) * kSink * D;
    const uint16_t *recK = p.recentK + ((size_t)seq * Hkv + kv) * kRecent * D;
    const uint16_t *recV = p.recentV + ((size_t)seq * Hkv + kv) * kRecent * D;
    const int nch = (n_win + 63) / 64;
    const int iters = (nch + kWaves - 1) / kWaves;
    for (int it = 0; it < iters; ++it) {
      const int ch = it * kWaves + w;
      const bool active = ch < nch;
      const int ntok = active ? min(64, n_win - ch * 64) : 0;
      if (active) {
        const int u = ch * 64 + lane;
        float lg[GQ];
#pragma unroll
        for (int h = 0; h < GQ; ++h) lg[h] = -INFINITY;
        if (lane < ntok) {
          const uint16_t *row = u < n_sink ? sinkK + (size_t)u * D : recK + (size_t)(u - n_sink) * D;
#pragma unroll
          for (int h = 0; h < GQ; ++h) lg[h] = 0.f;
          for (int c = 0; c < D; ++c) {
            const float kc = bf16f(row[c]);
#pragma unroll
            for (int h = 0; h < GQ; ++h) lg[h] = fmaf(sm.qs[h][c], kc, lg[h]);
          }
        }
        softmax_tile<GQ>(lg, m_run, l_run, alpha, sm.P[w], lane);
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
          for (int k = 0; k < D / 64; ++k) acc[h][k] *= alpha[h];
      }
      __syncthreads();
      if (active) {
        for (int tt = 0; tt < ntok; ++tt) {
          const int u = ch * 64 + tt;
          const uint16_t *row = u < n_sink ? sinkV + (size_t)u * D : recV + (size_t)(u - n_sink) * D;
#pragma unroll
          for (int k = 0; k < D / 64; ++k) {
            const float v = bf16f(row[lane + 64 * k]);
#pragma unroll
            for (int h = 0; h < GQ; ++h) acc[h][k] = fmaf(sm.P[w][h][tt], v, acc[h][k]);
          }
        }
      }
      __syncthreads();
    }
    block_merge_store<D, G, GQ>(sm, m_run, l_run, acc, ws_win + ((size_t)e * Hq + kv * GQ) * (D + 2));
  }
}

template <int D, int GQ>
__global__ __launch_bounds__(D) void decode_merge_kernel(PoolDev p, DecodeBatch b, float *__restrict__ out,
                                                         const float *__restrict__ ws) {
  const int e = blockIdx.x, kv = blockIdx.y, c = threadIdx.x;
  const int Hkv = p.Hkv, Hq = p.Hq;
  const float *ws_win = ws;
  const float *ws_hist = ws + (size_t)b.n * Hq * (D + 2);
  const int s0 = b.split_prefix[e], S = b.split_prefix[e + 1] - s0;
  const float *RVt = p.RVt + (size_t)kv * D * D;
  __shared__ float AH[D];
  for (int h = 0; h < GQ; ++h) {
    const float *win = ws_win + ((size_t)e * Hq + kv * GQ + h) * (D + 2);
    const float mw = win[D], lw = win[D + 1], aw = win[c];
    float o;
    if (S > 0) {
      float mH = -INFINITY;
      for (int s = 0; s < S; ++s)
        mH = fmaxf(mH, ws_hist[(((size_t)(s0 + s) * Hkv + kv) * GQ + h) * (D + 2) + D]);
      float lH = 0.f, aH = 0.f;
      for (int s = 0; s < S; ++s) {
        const float *part = ws_hist + (((size_t)(s0 + s) * Hkv + kv) * GQ + h) * (D + 2);
        const float f = exp2f(part[D] - mH);
        lH = fmaf(f, part[D + 1], lH);
        aH = fmaf(f, part[c], aH);
      }
      AH[c] = aH;
      __syncthreads();
      float der = 0.f;
      for (int j = 0; j < D; ++j) der = fmaf(AH[j], RVt[(size_t)j * D + c], der);
      __syncthreads();
      const float m = fmaxf(mw, mH), fw = exp2f(mw - m), fh = exp2f(mH - m);
      o = (fw * aw + fh * der) / (fw * lw + fh * lH);
    } else {
      o = aw / lw;
    }
    out[((size_t)e * Hq + kv * GQ + h) * D + c] = o;
  }
}

template <int D, int G, int GQ>
hipError_t decode_impl(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float *out, float scale,
                       float *ws, hipStream_t s, const KernelTimer &tm, const KernelTimer &tg) {
  const int blocks = b.hist_blocks + b.n * p.Hkv;
  if (tm.on) (void)hipEventRecord(tm.ev[0], s);
  hipLaunchKernelGGL((decode_main_kernel<D, G, GQ>), dim3(blocks), dim3(kThreads), 0, s, p, b, q, scale * kLog2e, ws);
  if (tm.on) (void)hipEventRecord(tm.ev[1], s);
  if (tg.on) (void)hipEventRecord(tg.ev[0], s);
  hipLaunchKernelGGL((decode_merge_kernel<D, GQ>), dim3(b.n, p.Hkv), dim3(D), 0, s, p, b, out, (const float *)ws);
  if (tg.on) (void)hipEventRecord(tg.ev[1], s);
  return hipGetLastError();
}

template <int D, int G>
hipError_t decode_g(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float *out, float scale, float *ws,
                    hipStream_t s, const KernelTimer &tm, const KernelTimer &tg) {
  switch (p.Hq / p.Hkv) {
  case 1: return decode_impl<D, G, 1>(p, b, q, out, scale, ws, s, tm, tg);
  case 2: return decode_impl<D, G, 2>(p, b, q, out, scale, ws, s, tm, tg);
  case 4: return decode_impl<D, G, 4>(p, b, q, out, scale, ws, s, tm, tg);
  case 8: return decode_impl<D, G, 8>(p, b, q, out, scale, ws, s, tm, tg);
  case 16: return decode_impl<D, G, 16>(p, b, q, out, scale, ws, s, tm, tg);
  }
  return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_decode(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float *out, float scale,
                         float *ws, hipStream_t s, const KernelTimer &tm, const KernelTimer &tg) {
  if (p.d == 128 && p.G == 128) return decode_g<128, 128>(p, b, q, out, scale, ws, s, tm, tg);
  if (p.d == 128 && p.G == 64) return decode_g<128, 64>(p, b, q, out, scale, ws, s, tm, tg);
  if (p.d == 64 && p.G == 64) return decode_g<64, 64>(p, b, q, out, scale, ws, s, tm, tg);
  return hipErrorInvalidValue;
}

} // namespace oscar
