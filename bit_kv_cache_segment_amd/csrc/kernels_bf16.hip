// Decode attention over a pool whose history is kept in BF16 (pool flag
// OSCAR_POOL_BF16_HISTORY): the same three-segment pool, pages, allocator
// and merge as the INT2 pool, with history tokens copied rather than
// rotated, clipped, quantized and packed.  It is the baseline the 2-bit
// history is measured against (news article on OSCAR, sanyangsrq.com,
// section "Small models keep hard reasoning": decode up to ~3x faster than
// BF16 at 100K context, batch 1).
//
// A (page, kv head) block holds the page's 64 tokens: K bf16 [64][d], then
// V bf16 [64][d].  One block per (sequence, kv head, split of its pages),
// all arithmetic on the VALU in fp32: bf16 dot2 for q.k, a lazy online
// softmax per lane (the reference moves only when a logit exceeds it by
// 2^8), fp32 products for p.v.  A wave load covers 512/d consecutive token
// rows (1 KB); lane (ts, cc) holds channels 8 cc .. 8 cc + 7 of token ts.
// The waves take pages from a shared-memory counter (or in a fixed order in
// deterministic pools); the block holding a pair's last split also takes
// the window.  Its partial (window and pages together) goes to the window
// slot of the workspace, every other split's to its split slot, so the
// merge kernel of the INT2 path completes the attention unchanged.
#include "bf_common.h"

#include <hip/hip_ext.h>

namespace oscar {
namespace {

template <int D, int GQ>
__global__ __launch_bounds__(64 * kBfWaves) void decode_bf16_kernel(PoolDev p, DecodeBatch b, const uint16_t *__restrict__ q,
                                                                     float qscale, float *__restrict__ ws) {
  constexpr int W = kBfWaves, LPT = D / 8, WG = GQ <= 4 ? 8 : (GQ <= 8 ? 4 : 2);
  __shared__ BfSmem<D, GQ> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int ts = lane / LPT, cc = lane % LPT;
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
    for (int idx = tid; idx < GQ * D / 2; idx += 64 * W) sm.q2[idx / (D / 2)][idx % (D / 2)] = src[idx];
  }
  if (tid == 0) sm.claim = (uint32_t)p0;
  __syncthreads();

  BfState<GQ> st;
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[h][j] = 0.f;
  }
  if (with_window) {
    const int n_sink = min(L, kSink), n_rec = min(max(L - kSink, 0), kRecent);
    const size_t wb = ((size_t)seq * Hkv + kv);
    // token groups round robin over the waves, sink then recent
    bf_tokens<D, GQ, WG>(st, p.sinkK + wb * kSink * D, p.sinkV + wb * kSink * D, n_sink, w, W, sm.q2, qscale, lane);
    bf_tokens<D, GQ, WG>(st, p.recentK + wb * kRecent * D, p.recentV + wb * kRecent * D, n_rec, w, W, sm.q2, qscale,
                         lane);
  }
  // history pages of the split, one page per wave at a time
  const int32_t *ptab = p.page_table + (size_t)seq * p.maxp;
  int next_static = p0 + w;
  for (;;) {
    int pg;
    if (p.deterministic) {
      pg = next_static;
      next_static += W;
    } else {
      uint32_t c = 0;
      if (lane == 0) c = atomicAdd(&sm.claim, 1u);
      pg = __builtin_amdgcn_readfirstlane((int)c);
    }
    if (pg >= p1) break;
    const int ntok = min(kPage, n_hist - pg * kPage);
    const uint16_t *kb = (const uint16_t *)(p.pages + ((size_t)ptab[pg] * Hkv + kv) * p.block_bytes);
    bf_tokens<D, GQ, WG>(st, kb, kb + kPage * D, ntok, 0, 1, sm.q2, qscale, lane);
  }
  wave_state_to_smem<D, GQ>(sm, st, w, lane);
  __syncthreads();
  // the block's partial: window slot for the last split (window and its
  // pages), split slot otherwise; the last split's own slot stays empty
  float *ws_win = ws, *ws_hist = ws + (size_t)b.n * Hq * (D + 2);
  const int slot = (e * Hkv + kv) * karg_u8(b.nsplit, 0) + s;
  float *dst = with_window ? ws_win + ((size_t)e * Hq + kv * GQ) * (D + 2) : ws_hist + (size_t)slot * GQ * (D + 2);
  for (int idx = tid; idx < GQ * D; idx += 64 * W) {
    const int h = idx / D, c = idx % D;
    float a, m, l;
    block_combine<D, GQ>(sm, h, c, a, m, l);
    dst[(size_t)h * (D + 2) + c] = a;
    if (c == 0) {
      dst[(size_t)h * (D + 2) + D] = m;
      dst[(size_t)h * (D + 2) + D + 1] = l;
    }
  }
  if (with_window) {
    float *e0 = ws_hist + (size_t)slot * GQ * (D + 2);
    for (int idx = tid; idx < GQ * (D + 2); idx += 64 * W) e0[idx] = idx % (D + 2) == D ? -INFINITY : 0.f;
  }
}

template <int D, int GQ>
hipError_t bf16_impl(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float scale, float *ws, hipStream_t s,
                     const KernelTimer &tm) {
  hipExtLaunchKernelGGL((decode_bf16_kernel<D, GQ>), dim3(b.hist_blocks), dim3(64 * kBfWaves), 0, s,
                        tm.on ? tm.ev[0] : nullptr, tm.on ? tm.ev[1] : nullptr, 0, p, b, q, scale * kLog2e, ws);
  return hipGetLastError();
}

template <int D>
hipError_t bf16_d(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float scale, float *ws, hipStream_t s,
                  const KernelTimer &tm) {
  switch (p.Hq / p.Hkv) {
  case 1: return bf16_impl<D, 1>(p, b, q, scale, ws, s, tm);
  case 2: return bf16_impl<D, 2>(p, b, q, scale, ws, s, tm);
  case 4: return bf16_impl<D, 4>(p, b, q, scale, ws, s, tm);
  case 8: return bf16_impl<D, 8>(p, b, q, scale, ws, s, tm);
  case 16: return bf16_impl<D, 16>(p, b, q, scale, ws, s, tm);
  }
  return hipErrorInvalidValue;
}

template <int D>
int bf16_blocks_d(const PoolDev &p) {
  int nb = 0;
  hipError_t e = hipErrorInvalidValue;
  const int t = 64 * kBfWaves;
  switch (p.Hq / p.Hkv) {
  case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_bf16_kernel<D, 1>, t, 0); break;
  case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_bf16_kernel<D, 2>, t, 0); break;
  case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_bf16_kernel<D, 4>, t, 0); break;
  case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_bf16_kernel<D, 8>, t, 0); break;
  case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_bf16_kernel<D, 16>, t, 0); break;
  }
  return e == hipSuccess ? nb : 0;
}

} // namespace

int bf16_decode_blocks_per_cu(const PoolDev &p) {
  if (p.d == 128) return bf16_blocks_d<128>(p);
  if (p.d == 64) return bf16_blocks_d<64>(p);
  return 0;
}

// The history part of a decode launch on a BF16-history pool; the merge is
// the INT2 path's (launch_decode_merge).
hipError_t launch_decode_bf16(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float scale, float *ws,
                              hipStream_t s, const KernelTimer &tm) {
  if (p.d == 128) return bf16_d<128>(p, b, q, scale, ws, s, tm);
  if (p.d == 64) return bf16_d<64>(p, b, q, scale, ws, s, tm);
  return hipErrorInvalidValue;
}

} // namespace oscar
