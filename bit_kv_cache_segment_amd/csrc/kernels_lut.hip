// Decode attention over a pool whose history uses the Lloyd-Max codebook
// variant (pool flag OSCAR_POOL_LLOYD_MAX; news article on OSCAR,
// sanyangsrq.com, section "Why this matters for long-context agents": the
// OSCAR code pairs the attention-aware rotation with a Lloyd-Max codebook).
// Pages, codes, scale/zero layout, allocator and merge are the INT2 pool's;
// a history value decodes to z + (L[code] / 64) s with the pair's codebook L
// (four bytes, one per level, held as one dword per kv head and K|V).
//
// One block per (sequence, kv head, split of its pages), 8 waves, all on the
// VALU.  The codebook lookup is a byte permute of the codebook dword with
// the code as selector, then an unsigned-byte-to-float conversion: three
// instructions per value with the bit-field extract, the same for K and V.
// Lane (ts, cc) takes channels 8 cc .. 8 cc + 7 of token ts of a pass
// (D/8 lanes per token).  Logits are taken in the rotated basis: the block
// first forms q . R_K for its heads in fp32 (shared memory); the history
// accumulator is de-rotated by R_V^T once, in the epilogue.  The pair's
// window (sink and recent, bf16 as stored) is attended by the block of the
// last split with the raw query, in its own state, and written to the
// window slot of the workspace; the pages' partial goes to the split slot,
// so the INT2 path's merge completes the attention.
#include "bf_common.h"

#include <hip/hip_ext.h>

namespace oscar {
namespace {

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// L[c] / 64 of a codebook dword: byte c selected, converted, scaled (exact).
__device__ __forceinline__ float level(uint32_t lut, uint32_t c) {
  return (float)(__builtin_amdgcn_perm(lut, lut, c) & 0xffu) * 0.015625f;
}

template <int D, int GQ>
struct LutSmem {
  BfSmem<D, GQ> bf;          // raw query rows (window), wave states
  alignas(16) float qr[GQ][D]; // q . R_K, fp32
};

// The history pages [pg, ...) one at a time: for each pass of TPI tokens a
// lane dequantizes its 8 K and 8 V values, forms its part of the GQ logits
// (summed over the D/8 lanes of the token), and updates its state.
template <int D, int G, int GQ>
__device__ __forceinline__ void lut_page(BfState<GQ> &st, const uint8_t *__restrict__ blk, int ntok,
                                         const float (*qr)[D], float qscale, uint32_t lk, uint32_t lv, int lane) {
  constexpr int LPT = D / 8, TPI = 64 / LPT;
  const int ts = lane / LPT, cc = lane % LPT;
  const int ch0 = 8 * cc, w16 = ch0 / 16, k0 = ch0 % 16, g = ch0 / G;
  // rotated query rows: in registers for up to 4 heads, else read from
  // shared memory per token (register room goes to the accumulators)
  constexpr int QR = GQ <= 4 ? GQ : 1;
  float q8[QR][8];
#pragma unroll
  for (int h = 0; h < QR; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) q8[h][i] = qr[h][ch0 + i];
  for (int t0 = 0; t0 < kPage; t0 += TPI) {
    const int t = t0 + ts;
    const bool ok = t < ntok;
    const int tl = ok ? t : 0; // loads stay inside the page
    const uint32_t kw = *(const uint32_t *)(blk + kcode_dword_off(D, tl, w16 % 4, w16 / 4));
    const uint32_t kp = *(const uint32_t *)(blk + kparam_off(D, G, tl, g));
    const uint32_t vp = *(const uint32_t *)(blk + vparam_off(D, G, tl, g));
    uint32_t vw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vw[i] = *(const uint32_t *)(blk + vcode_dword_off(D, tl / 16, ch0 + i));
    const float ks = f16_to_f32(kp & 0xffffu), kz = f16_to_f32(kp >> 16);
    const float vs = f16_to_f32(vp & 0xffffu), vz = f16_to_f32(vp >> 16);
    const int vb = vbit(tl % 16);
    float kf[8], vf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kf[i] = fmaf(ks, level(lk, (kw >> (2 * (k0 + i))) & 3u), kz);
      vf[i] = fmaf(vs, level(lv, (vw[i] >> vb) & 3u), vz);
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float d = 0.f;
      if constexpr (GQ <= 4) {
#pragma unroll
        for (int i = 0; i < 8; ++i) d = fmaf(q8[h][i], kf[i], d);
      } else {
        const float4 qa = *(const float4 *)&qr[h][ch0], qb = *(const float4 *)&qr[h][ch0 + 4];
        const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) d = fmaf(qv[i], kf[i], d);
      }
      d = lanes_sum<LPT>(d);
      const float sc = ok ? d * qscale : -INFINITY;
      const bool jump = sc > st.m[h] + kLazy;
      if (__any(jump)) {
        const float mn = jump ? sc : st.m[h];
        const float al = jump ? fast_exp2(st.m[h] - mn) : 1.f;
        st.l[h] *= al;
#pragma unroll
        for (int j = 0; j < 8; ++j) st.acc[h][j] *= al;
        st.m[h] = mn;
      }
      const float pr = ok ? fast_exp2(sc - st.m[h]) : 0.f;
      st.l[h] += pr;
#pragma unroll
      for (int j = 0; j < 8; ++j) st.acc[h][j] = fmaf(pr, vf[j], st.acc[h][j]);
    }
  }
}

template <int GQ>
__device__ __forceinline__ void reset(BfState<GQ> &st) {
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[h][j] = 0.f;
  }
}

template <int D, int G, int GQ>
__global__ __launch_bounds__(64 * kBfWaves) void decode_lut_kernel(PoolDev p, DecodeBatch b, const uint16_t *__restrict__ q,
                                                                    float qscale, float *__restrict__ ws) {
  constexpr int W = kBfWaves, WG = GQ <= 4 ? 8 : (GQ <= 8 ? 4 : 2);
  __shared__ LutSmem<D, GQ> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int blk = blockIdx.x, Hkv = p.Hkv, Hq = p.Hq;
  int s, e, kv;
  block_split(b, Hkv, blk, s, e, kv);
  const int S = karg_u8(b.nsplit, e);
  const int seq = b.seq[e], L = b.len[e];
  const int n_hist = max(L - kWindow, 0), np = (n_hist + kPage - 1) / kPage;
  int p0, p1;
  split_range(np, S, s, b.win_units, p0, p1);
  const bool with_window = s == S - 1;

  {
    const uint32_t *src = (const uint32_t *)(q + ((size_t)karg_u16(b.row, e) * Hq + kv * GQ) * D);
    for (int idx = tid; idx < GQ * D / 2; idx += 64 * W) sm.bf.q2[idx / (D / 2)][idx % (D / 2)] = src[idx];
  }
  if (tid == 0) sm.bf.claim = (uint32_t)p0;
  __syncthreads();
  // q . R_K per head: thread (h, j) runs the chain over i (R_K rows read
  // across threads j, coalesced)
  {
    const float *RK = p.RK + (size_t)kv * D * D;
    for (int idx = tid; idx < GQ * D; idx += 64 * W) {
      const int h = idx / D, j = idx % D;
      float a = 0.f;
      for (int i = 0; i < D; i += 2) {
        const uint32_t qw = sm.bf.q2[h][i / 2];
        a = fmaf(__uint_as_float(qw << 16), RK[(size_t)i * D + j], a);
        a = fmaf(__uint_as_float(qw & 0xffff0000u), RK[(size_t)(i + 1) * D + j], a);
      }
      sm.qr[h][j] = a;
    }
  }
  __syncthreads();

  float *ws_win = ws, *ws_hist = ws + (size_t)b.n * Hq * (D + 2);
  const int slot = (e * Hkv + kv) * karg_u8(b.nsplit, 0) + s;
  BfState<GQ> st;
  reset(st);
  if (with_window) {
    const int n_sink = min(L, kSink), n_rec = min(max(L - kSink, 0), kRecent);
    const size_t wb = ((size_t)seq * Hkv + kv);
    bf_tokens<D, GQ, WG>(st, p.sinkK + wb * kSink * D, p.sinkV + wb * kSink * D, n_sink, w, W, sm.bf.q2, qscale, lane);
    bf_tokens<D, GQ, WG>(st, p.recentK + wb * kRecent * D, p.recentV + wb * kRecent * D, n_rec, w, W, sm.bf.q2,
                         qscale, lane);
    wave_state_to_smem<D, GQ>(sm.bf, st, w, lane);
    __syncthreads();
    float *dst = ws_win + ((size_t)e * Hq + kv * GQ) * (D + 2);
    for (int idx = tid; idx < GQ * D; idx += 64 * W) {
      const int h = idx / D, c = idx % D;
      float a, m, l;
      block_combine<D, GQ>(sm.bf, h, c, a, m, l);
      dst[(size_t)h * (D + 2) + c] = a;
      if (c == 0) {
        dst[(size_t)h * (D + 2) + D] = m;
        dst[(size_t)h * (D + 2) + D + 1] = l;
      }
    }
    __syncthreads(); // the wave states are rewritten below
    reset(st);
  }

  // history pages of the split, one page per wave at a time
  const int32_t *ptab = p.page_table + (size_t)seq * p.maxp;
  const uint32_t lk = p.codebook[kv], lv = p.codebook[Hkv + kv];
  int next_static = p0 + w;
  for (;;) {
    int pg;
    if (p.deterministic) {
      pg = next_static;
      next_static += W;
    } else {
      uint32_t c = 0;
      if (lane == 0) c = atomicAdd(&sm.bf.claim, 1u);
      pg = __builtin_amdgcn_readfirstlane((int)c);
    }
    if (pg >= p1) break;
    const int ntok = min(kPage, n_hist - pg * kPage);
    lut_page<D, G, GQ>(st, p.pages + ((size_t)ptab[pg] * Hkv + kv) * p.block_bytes, ntok, sm.qr, qscale, lk, lv,
                       lane);
  }
  wave_state_to_smem<D, GQ>(sm.bf, st, w, lane);
  __syncthreads();
  // the waves' sum, still in the rotated basis, into qr (free now), then
  // de-rotated: out[c] = sum_i acc[i] R_V[c][i]
  float *dst = ws_hist + (size_t)slot * GQ * (D + 2);
  for (int idx = tid; idx < GQ * D; idx += 64 * W) {
    const int h = idx / D, c = idx % D;
    float a, m, l;
    block_combine<D, GQ>(sm.bf, h, c, a, m, l);
    sm.qr[h][c] = a;
    if (c == 0) {
      dst[(size_t)h * (D + 2) + D] = m;
      dst[(size_t)h * (D + 2) + D + 1] = l;
    }
  }
  __syncthreads();
  const float *RV = p.RV + (size_t)kv * D * D;
  for (int idx = tid; idx < GQ * D; idx += 64 * W) {
    const int h = idx / D, c = idx % D;
    const float4 *row = (const float4 *)(RV + (size_t)c * D);
    float a = 0.f;
    for (int i4 = 0; i4 < D / 4; ++i4) {
      const float4 r4 = row[i4];
      a = fmaf(sm.qr[h][4 * i4 + 0], r4.x, a);
      a = fmaf(sm.qr[h][4 * i4 + 1], r4.y, a);
      a = fmaf(sm.qr[h][4 * i4 + 2], r4.z, a);
      a = fmaf(sm.qr[h][4 * i4 + 3], r4.w, a);
    }
    dst[(size_t)h * (D + 2) + c] = a;
  }
}

template <int D, int G, int GQ>
hipError_t lut_impl(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float scale, float *ws, hipStream_t s,
                    const KernelTimer &tm) {
  hipExtLaunchKernelGGL((decode_lut_kernel<D, G, GQ>), dim3(b.hist_blocks), dim3(64 * kBfWaves), 0, s,
                        tm.on ? tm.ev[0] : nullptr, tm.on ? tm.ev[1] : nullptr, 0, p, b, q, scale * kLog2e, ws);
  return hipGetLastError();
}

template <int D, int G>
hipError_t lut_dg(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float scale, float *ws, hipStream_t s,
                  const KernelTimer &tm) {
  switch (p.Hq / p.Hkv) {
  case 1: return lut_impl<D, G, 1>(p, b, q, scale, ws, s, tm);
  case 2: return lut_impl<D, G, 2>(p, b, q, scale, ws, s, tm);
  case 4: return lut_impl<D, G, 4>(p, b, q, scale, ws, s, tm);
  case 8: return lut_impl<D, G, 8>(p, b, q, scale, ws, s, tm);
  case 16: return lut_impl<D, G, 16>(p, b, q, scale, ws, s, tm);
  }
  return hipErrorInvalidValue;
}

template <int D, int G>
int lut_blocks_dg(const PoolDev &p) {
  int nb = 0;
  hipError_t e = hipErrorInvalidValue;
  const int t = 64 * kBfWaves;
  switch (p.Hq / p.Hkv) {
  case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_lut_kernel<D, G, 1>, t, 0); break;
  case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_lut_kernel<D, G, 2>, t, 0); break;
  case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_lut_kernel<D, G, 4>, t, 0); break;
  case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_lut_kernel<D, G, 8>, t, 0); break;
  case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_lut_kernel<D, G, 16>, t, 0); break;
  }
  return e == hipSuccess ? nb : 0;
}

} // namespace

int lut_decode_blocks_per_cu(const PoolDev &p) {
  if (p.d == 128 && p.G == 128) return lut_blocks_dg<128, 128>(p);
  if (p.d == 128 && p.G == 64) return lut_blocks_dg<128, 64>(p);
  if (p.d == 64 && p.G == 64) return lut_blocks_dg<64, 64>(p);
  return 0;
}

// The history part of a decode launch on a Lloyd-Max pool; the merge is the
// INT2 path's (launch_decode_merge).
hipError_t launch_decode_lut(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float scale, float *ws,
                             hipStream_t s, const KernelTimer &tm) {
  if (p.d == 128 && p.G == 128) return lut_dg<128, 128>(p, b, q, scale, ws, s, tm);
  if (p.d == 128 && p.G == 64) return lut_dg<128, 64>(p, b, q, scale, ws, s, tm);
  if (p.d == 64 && p.G == 64) return lut_dg<64, 64>(p, b, q, scale, ws, s, tm);
  return hipErrorInvalidValue;
}

} // namespace oscar
