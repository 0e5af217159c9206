// Decode attention over the three-segment pool on gfx950.
//
// Method: news article on OSCAR (sanyangsrq.com), section "From offline
// calibration to online inference": decode handles the two precisions
// separately — an INT2 kernel unpacks the history, dequantizes with scale
// and zero point and accumulates in floating point; a BF16 kernel covers the
// sink and recent tokens; an online softmax merges the two results.
//
// Launches (one stream):
//   decode_main_kernel, one block per (sequence, kv head, split of its
//     history pages), one block per compute unit (4 x occupancy waves):
//     * the block rotates the g = Hq/Hkv queries by R_K, scales them and
//       lays them out as int8-limb MFMA operands (in shared memory);
//     * its waves stream the split's INT2 pages in the rotated basis,
//       taking pages from a shared counter;
//     * the block that holds the pair's last split also attends to the
//       BF16 sink and recent tokens with the raw queries (four waves, two
//       for 16 query heads, while the others stream pages); in a decode
//       step (oscar_decode_step) two of those waves first append the new
//       token: its slot before the window is read, the evicted token's
//       rotation, clip, quantization and packing after it;
//     * the block merges its waves and de-rotates the history accumulator
//       by R_V^T; it writes one partial (m, l, acc) per query head for the
//       history and, if it holds it, one for the window; when no pair of the
//       launch is split it combines the two itself and writes the rows.
//   decode_merge_kernel, one block per (sequence, kv head), when some pair
//     is split: merge the partials, normalise, write fp32.
// Softmax runs in base 2: logits are pre-multiplied by scale * log2(e).
//
// History pages (per wave):
//   QK^T on v_mfma_i32_16x16x64_i8.  The rotated query of each head is put
//   on a fixed-point grid q_int = rint(q 2^E) with |q_int| <= 2^18 and split
//   into three signed byte limbs; an MFMA row is one (head, limb).  2-bit
//   codes become int8 operands with AND masks (5 VALU ops per 16 codes).
//   The integer products are exact; recombining the limbs in fp32 leaves a
//   relative error near 2^-18 of the query's largest element.
//     logit = s_t * (q_int . code_t) 2^-E + z_t * sum(q)   per group.
//   PV on v_mfma_f32_16x16x32_f16.  V codes are stored so that one AND with
//   0x00030003 << 2i yields tokens (2i, 2i+1) of a 16-token block as two fp16
//   sub-normals code * 4^e * 2^-24; the factor 4^-e, the token's V scale and
//   a pool constant 2^pv_shift go into the fp16 softmax weight P' of the A
//   operand, the 2^24 / 2^pv_shift is undone once at the end.  The zero-point
//   term sum_t p_t z_t is accumulated on the VALU.
// Lloyd-Max codebook pools (LUT = true; news article on OSCAR, section "Why
//   this matters for long-context agents": the rotation paired with a
//   Lloyd-Max codebook): a level is z + (L[code] / 64) s.  The same MFMAs
//   run on level bytes instead of codes: one byte permute per dword of codes
//   turns four codes into their levels (the codebook dword is the permute
//   table).  K bytes carry L - 128 as signed int8 (the zero point absorbs
//   the + 2 s); the query grid is 2^17 (2^16 for groups of 128 channels
//   when a level is 0) so a group's sum stays below 2^31.
//   V bytes carry L unsigned into the low byte of each fp16 half (two
//   sub-normals L * 2^-24 per dword, no 4^e factors).
#include "oscar_internal.h"

#include <hip/hip_ext.h>

namespace oscar {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// P' rows hold 64 fp16 weights plus 8 of padding: the PV operand reads of 8
// lanes (rows n .. n+7 at one column) then fall on distinct LDS banks.
constexpr int kPRow = 72;
constexpr float kLazy = 8.f; // log2 headroom of the lazy softmax reference (host keeps 2^kLazy in pv_shift)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Waves per SIMD the register budget is sized for (3 where it fits without
// spilling: more waves in flight hide more HBM latency).
constexpr int main_occupancy(int D, int G, int GQ) { return (GQ <= 4 || (GQ == 8 && D == G)) ? 3 : (GQ <= 8 ? 2 : 1); }
// Waves of a decode_main block: one block fills a compute unit, so no unit
// holds blocks of different ages (the issue arbiter favours older waves);
// inside a block the waves share pages dynamically.
constexpr int main_waves(int D, int G, int GQ) { return 4 * main_occupancy(D, G, GQ); }


__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16lo(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xffffu)); }
__device__ __forceinline__ float f16hi(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(b >> 16)); }

// Sum over aligned groups of N lanes (N = 8 or 16) by DPP butterflies; every
// lane of a group ends with the same bits (each step adds a commuted pair).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float lanes_sum(float v) {
  v += dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v); // row_half_mirror: quad 0 <-> quad 1 of each 8 lanes
  if constexpr (N == 16) v += dpp_f<0x140>(v); // row_mirror: halves of each 16 lanes
  return v;
}

// Maximum over aligned groups of 16 lanes (one DPP row), in every lane, of
// values that are not NaN.  It runs on order-preserving integer keys (the
// bits of a non-negative float; the magnitude bits flipped for a negative
// one), so each step is one integer max with a DPP operand: a float max
// would canonicalise the DPP result first (two more instructions per step).
__device__ __forceinline__ int fkey(float f) {
  const int i = __float_as_int(f);
  return i ^ ((i >> 31) & 0x7fffffff);
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float row16_max_dpp(float f) {
  int v = fkey(f);
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x141>(v));
  v = max(v, dpp_i<0x140>(v));
  return __int_as_float(fkey(__int_as_float(v)));  // the key map is its own inverse
}
// Value of lane k (wave-uniform result).
__device__ __forceinline__ float lane_f(float v, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}
// Maximum / sum over all 64 lanes: DPP inside each 16-lane row, then the
// four row results by readlane.  Every lane gets the result.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = row16_max_dpp(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = lanes_sum<16>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float wave_min_dpp(float v) {
  v = fminf(v, dpp_f<0xB1>(v));
  v = fminf(v, dpp_f<0x4E>(v));
  v = fminf(v, dpp_f<0x141>(v));
  v = fminf(v, dpp_f<0x140>(v));
  return fminf(fminf(lane_f(v, 0), lane_f(v, 16)), fminf(lane_f(v, 32), lane_f(v, 48)));
}
// OR over the 16 lanes of each DPP row.
__device__ __forceinline__ uint32_t row16_or(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false);
  return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false);
}

// 2^x by the hardware instruction (x = -inf gives 0; results below the
// normal range flush to 0, which a softmax weight can afford).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Byte / half-word entries of a kernel-argument array, read through their
// dword: scalar loads (a sub-dword load would be a vector load).  The
// arrays start at 4-byte offsets.
__device__ __forceinline__ int karg_u8(const uint8_t *a, int i) {
  return (int)((((const uint32_t *)a)[i >> 2] >> (8 * (i & 3))) & 0xffu);
}
__device__ __forceinline__ int karg_u16(const uint16_t *a, int i) {
  return (int)((((const uint32_t *)a)[i >> 1] >> (16 * (i & 1))) & 0xffffu);
}

// A D x D fp32 rotation table in shared memory: 1 KB chunks of 256 / D
// rows, each followed by 16 pad floats, so that rows of chunks whose index
// differs mod 4 start 16 banks apart.
constexpr int kChunkPad = 16;
template <int D>
struct RTable {
  static constexpr int RPC = 256 / D; // rows per chunk
  alignas(16) float c[D * D / 256][256 + kChunkPad];
};

// Copy a D x D fp32 table into shared memory with direct global-to-LDS
// loads: each wave instruction moves one 1 KB chunk (lane i -> bytes
// 16 i .. 16 i + 15) and takes no registers.  Wave w copies chunks w, w + nw,
// ...  The caller waits for the loads (vmcnt) before a barrier and reads.
template <int D>
__device__ __forceinline__ void stage_table(RTable<D> &dst, const float *src, int w, int nw, int lane) {
  constexpr int NC = D * D / 256;
  for (int c = w; c < NC; c += nw)
    __builtin_amdgcn_global_load_lds((const void *)(src + c * 256 + lane * 4),
                                     (__attribute__((address_space(3))) void *)(&dst.c[c][0]), 16, 0, 0);
}

// Row stride (floats) of a head-interleaved table xT[D][.]: row j holds
// channel j of every head; padded so that rows 1 KB-chunk apart fall in
// distinct banks for 16-byte reads.
constexpr int qpad(int GQ) { return GQ >= 4 ? GQ + 4 : GQ; }

template <int GQ>
__device__ __forceinline__ void load_heads(float (&x)[GQ], const float *row) {
  if constexpr (GQ >= 4) {
#pragma unroll
    for (int h = 0; h < GQ; h += 4) {
      const float4 t = *(const float4 *)(row + h);
      x[h] = t.x;
      x[h + 1] = t.y;
      x[h + 2] = t.z;
      x[h + 3] = t.w;
    }
  } else if constexpr (GQ == 2) {
    const float2 t = *(const float2 *)row;
    x[0] = t.x;
    x[1] = t.y;
  } else {
    x[0] = row[0];
  }
}

// y[h][c] = sum_j xT[j][h] R[j][c] for the GQ heads: wave w computes the
// blocks of 16 columns cb = w, w + W, ...; lane (c16, quarter qq) sums the
// rows of the chunks with index = qq mod 4 (the four quarters read distinct
// banks of R and each quarter reads one xT row, broadcast), then the
// quarters are added across the wave.  emit(h, c, y) sees each result once,
// in a lane of quarter h mod 4.
template <int D, int GQ, int W, class Emit>
__device__ __forceinline__ void contract_columns(const float *xT, const RTable<D> &R, int w, int lane, Emit emit) {
  constexpr int RPC = RTable<D>::RPC, NCB = D / 16, QP = qpad(GQ);
  const int c16 = lane & 15, qq = lane >> 4;
  for (int cb = w; cb < NCB; cb += W) {
    const int c = 16 * cb + c16;
    float a[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) a[h] = 0.f;
#pragma unroll 4
    for (int t = 0; t < D / (4 * RPC); ++t)
#pragma unroll
      for (int b = 0; b < RPC; ++b) {
        const int ch = 4 * t + qq;
        const float rv = R.c[ch][b * D + c];
        float x[GQ];
        load_heads<GQ>(x, xT + (ch * RPC + b) * QP);
#pragma unroll
        for (int h = 0; h < GQ; ++h) a[h] = fmaf(x[h], rv, a[h]);
      }
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      a[h] += __shfl_xor(a[h], 16, 64);
      a[h] += __shfl_xor(a[h], 32, 64);
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h)
      if ((h & 3) == qq) emit(h, c, a[h]);
  }
}

// Order LDS traffic of the lanes of one wave (no cross-wave barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// shared memory
// ---------------------------------------------------------------------------
template <int D, int GQ, int NW>
struct WinSmem {
  alignas(16) uint32_t q2[NW][GQ][D / 2]; // query rows as bf16 pairs, one copy per wave
  float M[NW][GQ], L[NW][GQ];
  float A[NW][GQ][D];
  // fused step: the evicted K and V rows, and how many of the K / V appends
  // have published their slot writes and their page writes
  float app_x[2][D];
  int app_slot_done, app_page_done;
};

// Waves of a history block that process the pair's window while the others
// start on the pages; they join the page stream afterwards.
// (Two for 16 query heads per kv head, whose per-wave window state would not
// fit in shared memory next to the rotation table.)
constexpr int win_waves(int W, int GQ) { return GQ >= 16 ? 2 : (W < 4 ? W : 4); }

// Query record built by a history block: the int8-limb MFMA A operands
// [row tiles][d/64][64 lanes][4 words], then per-head group sums of the
// rotated query (at 0) and the fixed-point factors 2^-(E+4) (at 32).
template <int D, int GQ>
struct QueryPrep {
  alignas(16) float qT[D][qpad(GQ)]; // query rows, head-interleaved
  float qs[GQ][D];                   // rotated, scaled query rows
};
template <int D, int GQ>
constexpr int query_record_words() { return (GQ >= 4 ? GQ / 4 : 1) * (D / 64) * 256 + 64; }

template <int D, int G, int GQ, int W>
struct HistSmem {
  static constexpr int NG = D / G;
  RTable<D> R;                          // R_K (query prep), then R_V^T (de-rotation)
  float alpha[W][16];  // per-wave rescale factors of the PV rows
  float zsum[W][16][NG];
  alignas(16) float M[W][GQ];
  float L[W][GQ];
  alignas(16) float Mb[16];             // block maximum per head: max of the waves' M
  alignas(16) float mT[D][qpad(GQ)];    // block-merged accumulators (rotated basis), head-interleaved
  uint32_t rec[query_record_words<D, GQ>()]; // the pair's query record
  int32_t ids[kIdCache];                // page ids of a segment of the split
  uint32_t claim;                       // next page of the segment to hand out
  uint32_t exited;                      // waves out of the page loop
  WinSmem<D, GQ, win_waves(W, GQ)> win;     // window results of the window waves
  union alignas(16) {
    QueryPrep<D, GQ> pre;               // prologue: query preparation
    _Float16 P[W][NG][16][kPRow];       // page loop: P' rows per wave (padded)
    float A[W][GQ][D + 4];              // epilogue: per-wave accumulators (rows padded so
                                        // that a wave's four head rows write distinct banks)
  } u;
};


template <int D, int G, int GQ, int W>
union MainSmem {
  HistSmem<D, G, GQ, W> h;
  WinSmem<D, GQ, W> w;
};

// Merge per-wave (M, L, A) of the W waves in shared memory and store one
// partial per head.
// (out != nullptr: the pair has no other partial, so the normalised rows
// acc / l go to out[GQ][D] instead.)
template <int D, int GQ, int W>
__device__ void block_merge_store(const float (*M)[GQ], const float (*L)[GQ], const float (*A)[GQ][D],
                                  float *dst /*[GQ][D+2]*/, float *out = nullptr) {
  const int tid = threadIdx.x;
  for (int idx = tid; idx < GQ * D; idx += W * 64) {
    const int h = idx / D, c = idx % D;
    float m = -INFINITY;
    for (int ww = 0; ww < W; ++ww) m = fmaxf(m, M[ww][h]);
    float a = 0.f, l = 0.f;
    for (int ww = 0; ww < W; ++ww) {
      const float f = M[ww][h] == -INFINITY ? 0.f : exp2f(M[ww][h] - m);
      a += f * A[ww][h][c];
      l += f * L[ww][h];
    }
    if (out) {
      out[(size_t)h * D + c] = a / l;
      continue;
    }
    float *o = dst + (size_t)h * (D + 2);
    o[c] = a;
    if (c == 0) {
      o[D] = m;
      o[D + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// BF16 sink + recent window of one (sequence, kv head), up to 320 tokens.
// A wave load covers TPI consecutive token rows (1 KB): lane (ts, cc) holds
// channels 8 cc .. 8 cc + 7 of token TPI gi + ts.  Token groups gi go round
// robin over the waves; each wave issues the K and V loads of WG groups at
// once, then computes them: QK^T by bf16 dot2 and a DPP sum over the D/8
// lanes of a token, a lazy online softmax per lane (reference moved only
// when a logit exceeds it by kLazy), PV into fp32 accumulators of the lane's
// 8 channels.  Token slots and waves are merged at the end.
// ---------------------------------------------------------------------------
template <int D, int G, int GQ, int NW>
constexpr int win_groups() {
  constexpr int TPI = 512 / D, nk = (kWindow / TPI + NW - 1) / NW; // groups per wave
  // unified VGPR file share of a wave, at most 256 addressable VGPRs
  constexpr int budget = 512 / main_occupancy(D, G, GQ) / 8 * 8 < 256 ? 512 / main_occupancy(D, G, GQ) / 8 * 8 : 256;
  constexpr int fit = (budget - 10 * GQ - 48) / 8;           // 8 registers per group in flight
  constexpr int hk = fit < 1 ? 1 : (fit < nk ? fit : nk);
  constexpr int passes = (nk + hk - 1) / hk;
  return (nk + passes - 1) / passes;
}

// Window tokens of one (sequence, kv head) processed by NW waves: wave wi
// takes the token groups wi, wi + NW, ... and leaves its (m, l, acc) in
// sm.M[wi], sm.L[wi], sm.A[wi] (a block merge combines the NW waves).
template <int D, int G, int GQ, int NW>
__device__ void window_waves(WinSmem<D, GQ, NW> &sm, const PoolDev &p, const DecodeBatch &b, const uint16_t *q,
                             float qscale, int e, int kv, int wi) {
  constexpr int LPT = D / 8, TPI = 64 / LPT, WG = win_groups<D, G, GQ, NW>();
  const int lane = threadIdx.x % 64;
  const int ts = lane / LPT, cc = lane % LPT;
  const int Hkv = p.Hkv, Hq = p.Hq;
  const int seq = b.seq[e], L = b.len[e];
  const int n_sink = min(L, kSink), n_rec = min(max(L - kSink, 0), kRecent), n_win = n_sink + n_rec;
  const int n_hist = max(L - kWindow, 0);
  {
    // this wave's copy of the query rows: no block barrier needed
    const uint32_t *src = (const uint32_t *)(q + ((size_t)karg_u16(b.row, e) * Hq + kv * GQ) * D);
    for (int idx = lane; idx < GQ * D / 2; idx += 64) sm.q2[wi][idx / (D / 2)][idx % (D / 2)] = src[idx];
  }
  wave_sync();
  const uint16_t *sinkK = p.sinkK + ((size_t)seq * Hkv + kv) * kSink * D;
  const uint16_t *sinkV = p.sinkV + ((size_t)seq * Hkv + kv) * kSink * D;
  const uint16_t *recK = p.recentK + ((size_t)seq * Hkv + kv) * kRecent * D;
  const uint16_t *recV = p.recentV + ((size_t)seq * Hkv + kv) * kRecent * D;

  float m_ref[GQ], l_run[GQ], acc[GQ][8];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m_ref[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
  }
  const int ngroups = (n_win + TPI - 1) / TPI;
  const int nk = (ngroups - wi + NW - 1) / NW; // groups of this wave
  for (int k0 = 0; k0 < nk; k0 += WG) {
    u32x4 kr[WG], vr[WG];
#pragma unroll
    for (int i = 0; i < WG; ++i) {
      const int u = (wi + NW * (k0 + i)) * TPI + ts;
      kr[i] = vr[i] = u32x4{0u, 0u, 0u, 0u};
      if (k0 + i < nk && u < n_win) {
        const size_t off = (size_t)(u < n_sink ? u : u - n_sink) * D + 8 * cc;
        kr[i] = __builtin_nontemporal_load((const u32x4 *)((u < n_sink ? sinkK : recK) + off));
        vr[i] = __builtin_nontemporal_load((const u32x4 *)((u < n_sink ? sinkV : recV) + off));
      }
    }
#pragma unroll
    for (int i = 0; i < WG; ++i) {
      if (k0 + i >= nk) break;
      const int u = (wi + NW * (k0 + i)) * TPI + ts;
      const bool ok = u < n_win;
      float vf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[2 * j] = __uint_as_float(vr[i][j] << 16);
        vf[2 * j + 1] = __uint_as_float(vr[i][j] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const u32x4 qv = *(const u32x4 *)&sm.q2[wi][h][4 * cc];
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // element copies first: a bit cast of a vector element itself
          // would read element 0
          const uint32_t kw = kr[i][j], qw = qv[j];
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw), __builtin_bit_cast(bf16x2, qw), d, false);
        }
        d = lanes_sum<LPT>(d);
        const float sc = ok ? d * qscale : -INFINITY;
        const bool jump = sc > m_ref[h] + kLazy;
        if (__any(jump)) {
          const float mn = jump ? sc : m_ref[h];
          const float al = jump ? fast_exp2(m_ref[h] - mn) : 1.f;
          l_run[h] *= al;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[h][j] *= al;
          m_ref[h] = mn;
        }
        const float pr = ok ? fast_exp2(sc - m_ref[h]) : 0.f;
        l_run[h] += pr;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(pr, vf[j], acc[h][j]);
      }
    }
  }
  // merge the TPI token slots of the wave (lanes cc, cc + LPT, ...)
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float m = m_ref[h];
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float f = m_ref[h] == -INFINITY ? 0.f : exp2f(m_ref[h] - m);
    float l = l_run[h] * f;
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) l += __shfl_xor(l, o, 64);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = acc[h][j] * f;
#pragma unroll
      for (int o = LPT; o < 64; o <<= 1) a += __shfl_xor(a, o, 64);
      acc[h][j] = a;
    }
    if (lane == 0) {
      sm.M[wi][h] = m;
      sm.L[wi][h] = l;
    }
    if (ts == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.A[wi][h][8 * cc + j] = acc[h][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Append of a fused step, by waves 0 (K, kind 0) and 1 (V, kind 1) of the
// block that holds the pair's window: the same eviction as the append
// kernel.  The new token goes to its sink or recent slot; when the window is
// full, the slot's old token is rotated (fixed-order fp32 FMA chain over
// i = 0..d-1 from +0), clipped, quantized per group (fp16 scale and zero)
// and packed into history index n_hist0 = L0 - 320 (L0: length before the
// append).  The slot write is published (app_slot_done) before the
// rotation, the page writes (app_page_done) after it, each with a
// workgroup-scope release after the wave's stores have completed; readers
// acquire the counter.  The old token is read, and the V code dwords
// updated, at device scope (no L1 line of them is ever cached in the
// block), so every later read of the slot or the page misses in L1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float f16_val(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Bounded wait for a shared-memory counter (every wave reaches its end):
// at most p.wait_limit polls.  A wait that gives up is not silent: lane 0
// of the wave ORs kStatusWaitGaveUp into the pool's status word (a vector
// atomic), which the host turns into an error at its next synchronising
// call; the wave then goes on, so the block still ends.
__device__ __forceinline__ void wait_count(int *c, int target, const PoolDev &p) {
  for (int it = 0; it < p.wait_limit; ++it) {
    if (__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(2);
  }
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(p.status, kStatusWaitGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish(int *c, int lane) {
  __builtin_amdgcn_s_waitcnt(0); // this wave's stores and atomics have completed
  if (lane == 0) __hip_atomic_fetch_add(c, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

struct AppendIn {
  const uint16_t *k, *v; // [n][Hkv][d] bf16 in batch row order
};

// First part: the slot (the old token kept in shared memory when it is
// evicted), published; the window reads the slot after this.
template <int D, int GQ, int NW>
__device__ void fused_append_slot(WinSmem<D, GQ, NW> &sm, const PoolDev &p, const DecodeBatch &b, const AppendIn &in,
                                  int e, int kv, int kind, int lane) {
  const int Hkv = p.Hkv, seq = b.seq[e], L0 = b.len[e] - 1;
  const uint16_t *xn = (kind ? in.v : in.k) + ((size_t)karg_u16(b.row, e) * Hkv + kv) * D;
  const bool evict = L0 >= kWindow;
  {
    // the slot: dword u of the row (channels 2u, 2u + 1) by lane u
    uint32_t *row;
    if (L0 < kSink) row = (uint32_t *)((kind ? p.sinkV : p.sinkK) + (((size_t)seq * Hkv + kv) * kSink + L0) * D);
    else row = (uint32_t *)((kind ? p.recentV : p.recentK) + (((size_t)seq * Hkv + kv) * kRecent + (L0 - kSink) % kRecent) * D);
    if (lane < D / 2) {
      const uint32_t nw = ((const uint32_t *)xn)[lane];
      if (evict) {
        const uint32_t old = __hip_atomic_load(row + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.app_x[kind][2 * lane] = __uint_as_float(old << 16);
        sm.app_x[kind][2 * lane + 1] = __uint_as_float(old & 0xffff0000u);
      }
      row[lane] = nw;
    }
  }
  publish(&sm.app_slot_done, lane);
}

// Second part: the evicted token into the history, published; only the
// pass over the pair's last page, after the page loop, reads it, so this
// runs after the wave's share of the window.  The K rotation reads R_K from
// the block's shared-memory table (it holds R_K until the epilogue); the V
// rotation reads the columns of R_V as rows of R_V^T, 16 bytes per load.
template <int D, int G, int GQ, int NW>
__device__ void fused_append_page(WinSmem<D, GQ, NW> &sm, const RTable<D> &RK_lds, const PoolDev &p,
                                  const DecodeBatch &b, int e, int kv, int kind, int lane) {
  constexpr int CPL = D / 64; // channels lane + 64 c of this lane
  const int Hkv = p.Hkv, seq = b.seq[e], L0 = b.len[e] - 1;
  if (L0 >= kWindow) {
    wave_sync(); // this wave's writes of the old token to shared memory
    const int n_hist0 = L0 - kWindow, t = n_hist0 % kPage;
    const int page = b.new_page[e] >= 0 ? b.new_page[e] : p.page_table[(size_t)seq * p.maxp + n_hist0 / kPage];
    const float *clip = (kind ? p.clipV : p.clipK) + (size_t)kv * D;
    float y[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) y[c] = 0.f;
    if (kind == 0) {
      constexpr int RPC = RTable<D>::RPC;
#pragma unroll 16
      for (int i = 0; i < D; ++i) {
        const float xi = sm.app_x[0][i];
#pragma unroll
        for (int c = 0; c < CPL; ++c) y[c] = fmaf(xi, RK_lds.c[i / RPC][(i % RPC) * D + lane + 64 * c], y[c]);
      }
    } else {
      // column j of R_V is row j of R_V^T: 16-byte loads, four rows of the
      // chain each
      const float4 *col[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) col[c] = (const float4 *)(p.RVt + ((size_t)kv * D + lane + 64 * c) * D);
#pragma unroll 8
      for (int i4 = 0; i4 < D / 4; ++i4) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float4 r4 = col[c][i4];
          y[c] = fmaf(sm.app_x[1][4 * i4 + 0], r4.x, y[c]);
          y[c] = fmaf(sm.app_x[1][4 * i4 + 1], r4.y, y[c]);
          y[c] = fmaf(sm.app_x[1][4 * i4 + 2], r4.z, y[c]);
          y[c] = fmaf(sm.app_x[1][4 * i4 + 3], r4.w, y[c]);
        }
      }
    }
    uint32_t code[CPL];
    uint16_t s16[CPL], z16[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float cl = clip[lane + 64 * c];
      y[c] = fminf(fmaxf(y[c], -cl), cl);
    }
    // group minima / maxima: G = 64 -> group c; G = 128 -> every channel
    float mn[CPL], mx[CPL];
    if constexpr (G == 64) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        mn[c] = wave_min_dpp(y[c]);
        mx[c] = wave_max_dpp(y[c]);
      }
    } else {
      float a = y[0], bmax = y[0];
#pragma unroll
      for (int c = 1; c < CPL; ++c) {
        a = fminf(a, y[c]);
        bmax = fmaxf(bmax, y[c]);
      }
      a = wave_min_dpp(a);
      bmax = wave_max_dpp(bmax);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        mn[c] = a;
        mx[c] = bmax;
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      // "+ 0.0f" stores an exactly zero range or minimum as +0
      s16[c] = f16_bits(((mx[c] - mn[c]) + 0.0f) / 3.0f);
      z16[c] = f16_bits(mn[c] + 0.0f);
      const float sc = f16_val(s16[c]), ze = f16_val(z16[c]);
      if (p.lut) {
        // codebook pools: the nearest level
        code[c] = lut_code(y[c], ze, sc, p.codebook[kind * Hkv + kv]);
      } else {
        float qv = 0.0f;
        if (sc != 0.0f) qv = fminf(fmaxf(rintf((y[c] - ze) / sc), 0.0f), 3.0f);
        code[c] = (uint32_t)qv;
      }
    }
    uint8_t *blk = p.pages + ((size_t)page * Hkv + kv) * p.block_bytes;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = lane + 64 * c, g = j / G;
      if (kind == 0) {
        // 16 lanes assemble the dword of channels 64 c + 16 r + k
        const uint32_t dw = row16_or(code[c] << (2 * (lane & 15)));
        if ((lane & 15) == 0) *(uint32_t *)(blk + kcode_dword_off(D, t, lane >> 4, c)) = dw;
        if (j % G == 0) *(uint32_t *)(blk + kparam_off(D, G, t, g)) = (uint32_t)s16[c] | ((uint32_t)z16[c] << 16);
      } else {
        // token t's two bits in channel j's dword; the first token of a
        // byte clears the byte, later ones their own two bits
        const int k = t % 16, bit = vbit(k);
        uint32_t *dw = (uint32_t *)(blk + vcode_dword_off(D, t / 16, j));
        atomicAnd(dw, (k & 6) == 0 ? ~(0xffu << (8 * (bit / 8))) : ~(3u << bit));
        atomicOr(dw, code[c] << bit);
        if (j % G == 0) *(uint32_t *)(blk + vparam_off(D, G, t, g)) = (uint32_t)s16[c] | ((uint32_t)z16[c] << 16);
      }
    }
    if (b.new_page[e] >= 0 && kind == 0 && kv == 0 && lane == 0)
      p.page_table[(size_t)seq * p.maxp + n_hist0 / kPage] = page;
  }
  publish(&sm.app_page_done, lane);
}

// A block that holds only a pair's window: all its waves take part.
template <int D, int G, int GQ>
__device__ void window_block(WinSmem<D, GQ, main_waves(D, G, GQ)> &sm, const PoolDev &p, const DecodeBatch &b,
                             const uint16_t *q, float qscale, float *ws_win, float *out, const AppendIn &in, int e,
                             int kv) {
  constexpr int W = main_waves(D, G, GQ);
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (b.fused) {
    // (a pair that evicts always holds its last page in this split, so
    // here the append only writes the new token)
    if (threadIdx.x == 0) sm.app_slot_done = sm.app_page_done = 0;
    __syncthreads();
    if (w < 2) fused_append_slot<D, GQ, W>(sm, p, b, in, e, kv, w, threadIdx.x & 63);
    wait_count(&sm.app_slot_done, 2, p);
  }
  window_waves<D, G, GQ, W>(sm, p, b, q, qscale, e, kv, w);
  __syncthreads();
  block_merge_store<D, GQ, W>(sm.M, sm.L, sm.A, ws_win + ((size_t)e * p.Hq + kv * GQ) * (D + 2),
                              b.direct ? out + ((size_t)karg_u16(b.row, e) * p.Hq + kv * GQ) * D : nullptr);
}

// ---------------------------------------------------------------------------
// Query preparation, by the whole history block, in shared memory:
//   qs = (q . R_K) * scale * log2(e)          (fp32)
//   E  = 18 - e  with max|qs| = f 2^e, f in [0.5, 1)   ->  |qs 2^E| < 2^18
//   A operand word [rt][mi][lane][v]: lane = (row m, k-quad r); row
//     m = 4 hh + limb of head 4 rt + hh; byte j of register v holds limb
//     `limb` of rint(qs[h][c] 2^E) * {16, 4, 1, 16}[v], c = 64 mi + 16 r + 4 j + v.
//   Limbs are balanced signed bytes: X = a0 + 2^8 a1 + 2^16 a2.
// Record tail: qsum[h][g] (group sums of qs) at 0, kfac[h] = 2^-(E+4) at 32.
// Codebook pools (LUT): E = 17 - e (16 - e for groups of 128 channels when
// a level is 0), no {16, 4, 1, 16} factors, and kfac = 2^-(E+6) (the code
// bytes carry 64 x the level, less 128).
// On entry R holds R_K and qT the query rows (after a barrier).  The product
// is taken by column blocks; then one wave per head finds E and the group
// sums and writes the head's words.  On exit (after a barrier) rec holds the
// record.
// ---------------------------------------------------------------------------
template <int D, int G, int GQ, int W, bool LUT = false>
__device__ void query_prep(QueryPrep<D, GQ> &pr, uint32_t *rec, const RTable<D> &R, float qscale, int tid,
                           int ebits = 18) {
  constexpr int NG = D / G, MI = D / 64, RT = GQ >= 4 ? GQ / 4 : 1;
  static_assert(G == 64 || G == D, "channel groups of 64, or one group per token");
  const int w = tid >> 6, lane = tid & 63;
  contract_columns<D, GQ, W>(&pr.qT[0][0], R, w, lane, [&](int h, int c, float y) { pr.qs[h][c] = y * qscale; });
  __syncthreads();
  float *tail = (float *)(rec + RT * MI * 256);
  // lane -> (k-quad r, limb row lam, register v) of the head's words
  const int r = lane >> 4, lam = (lane >> 2) & 3, v = lane & 3;
  // codebook pools: the code bytes carry L - 128 (|.| <= 128), no 4^e factor
  const int mult = LUT ? 1 : (v == 1 ? 4 : (v == 2 ? 1 : 16));
  for (int h = w; h < 4 * RT; h += W) { // heads >= GQ (when GQ < 4) get zero words
    const bool live = h < GQ;
    float x[MI], mx = 0.f; // lane holds channels lane + 64 k
#pragma unroll
    for (int k = 0; k < MI; ++k) {
      x[k] = live ? pr.qs[h][lane + 64 * k] : 0.f;
      mx = fmaxf(mx, fabsf(x[k]));
    }
    mx = wave_max_dpp(mx);
    if (G == 64) {
#pragma unroll
      for (int k = 0; k < MI; ++k) {
        const float sum = wave_sum_dpp(x[k]);
        if (live && lane == 0) tail[h * NG + k] = sum;
      }
    } else {
      float a = 0.f;
#pragma unroll
      for (int k = 0; k < MI; ++k) a += x[k];
      a = wave_sum_dpp(a);
      if (live && lane == 0) tail[h * NG] = a;
    }
    int ex = 0;
    frexpf(mx, &ex);
    // |q_int| <= 2^ebits: 2^18 (affine codes: products <= 2^18 * 48), or for
    // codebook bytes (products <= |q_int| |L - 128|) 2^17, or 2^16 for groups
    // of 128 channels with a level of 0 (|L - 128| = 128): a group's sum
    // stays below 2^31
    const int E = mx > 0.f ? ebits - ex : 0;
    if (live && lane == 0) tail[32 + h] = ldexpf(1.f, LUT ? -(E + 6) : -(E + 4));
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      uint32_t word = 0;
      if (live && lam < 3) {
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int X = (int)rintf(ldexpf(pr.qs[h][64 * mi + 16 * r + 4 * j4 + v], E)) * mult;
          const int a0 = (int)(int8_t)(X & 0xff);
          const int X1 = (X - a0) >> 8;
          const int a1 = (int)(int8_t)(X1 & 0xff);
          const int a2 = (X1 - a1) >> 8;
          const int limb = lam == 0 ? a0 : (lam == 1 ? a1 : a2);
          word |= ((uint32_t)limb & 0xffu) << (8 * j4);
        }
      }
      rec[(((h >> 2) * MI + mi) * 64 + 16 * r + 4 * (h & 3) + lam) * 4 + v] = word;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// INT2 history split block.
// ---------------------------------------------------------------------------
template <int D, int G>
struct PageRegs {
  u32x4 kc[D / 64]; // K codes of tokens 4n..4n+3, quad r (D/4 bytes)
  u32x4 vc[D / 64]; // V codes of channels {16j+n}, token block r (D/4 bytes)
  u32x4 kp[D / G];  // K (scale, zero) of tokens 4n..4n+3
  u32x4 vp[D / G];  // V (scale, zero)
};

// Loads of one (page, kv head) block through a buffer resource over it.  A
// page past the end (valid false) gets a resource of zero bytes: its loads
// return zeros without a memory access, yet count like the others, so the
// loop's waits stay exact and no load is left in flight behind the loop.
template <int D, int G>
__device__ __forceinline__ void load_page(PageRegs<D, G> &pr, const uint8_t *blk, bool valid, int bytes, int n,
                                          int r) {
  constexpr int NG = D / G;
  constexpr int kWord3 = 0x00020000; // raw buffer, 32-bit data format
  constexpr int kNT = 2;             // non-temporal: every byte is read once per call
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)blk, 0, valid ? bytes : 0, kWord3);
  // codes: 1 KB contiguous per instruction; params: 16 lanes share 256 B.
  const int lane = 16 * r + n;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    pr.kc[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane + 1024 * i, 0, kNT);
    pr.vc[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * D + 16 * lane + 1024 * i, 0, kNT);
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    pr.kp[g] = __builtin_amdgcn_raw_buffer_load_b128(rs, 32 * D + 16 * NG * n + 16 * g, 0, kNT);
    pr.vp[g] = __builtin_amdgcn_raw_buffer_load_b128(rs, 32 * D + 256 * NG + 16 * NG * n + 16 * g, 0, kNT);
  }
}

// Pages a wave keeps in flight beyond the one it computes (register budget).
template <int D, int G, int GQ>
constexpr int kPrefetch = (D == 64 || (G == D && GQ <= 4)) ? 2 : 1;

template <int D, int G, int GQ, bool LUT = false>
__device__ void history_block(HistSmem<D, G, GQ, main_waves(D, G, GQ)> &sm, const PoolDev &p, const DecodeBatch &b,
                              float *ws_hist, float *ws_win, float *out, const uint16_t *q, float qscale,
                              const AppendIn &in, int slot, int e, int kv, int p0, int p1, bool with_window) {
  constexpr int W = main_waves(D, G, GQ), NT = 64 * W, WW = win_waves(W, GQ);
  constexpr int NG = D / G;                // scale/zero groups per token
  constexpr int MI = D / 64;               // i8 MFMAs per 16-token tile (64 channels each)
  constexpr int RT = GQ >= 4 ? GQ / 4 : 1; // MFMA row tiles of 4 heads x 4 limb rows
  constexpr int NJ = D / 16;               // PV column tiles of 16 channels
  // With at most 8 heads, rows GQ .. 2 GQ - 1 of the PV tile are free: they
  // carry the fp16 remainder of each head's weights (P' = hi + lo, ~22
  // bits), and the epilogue adds their output rows to the heads' rows.
  constexpr bool LO = 2 * GQ <= 16;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 15, r = lane >> 4;
  const int Hkv = p.Hkv;
  const int seq = b.seq[e], n_hist = b.len[e] - kWindow;
  const int np = (n_hist + kPage - 1) / kPage;

  // bits of the query's fixed-point grid (see query_prep)
  int qbits = 18;
  if constexpr (LUT) {
    const uint32_t cb = p.codebook[kv];
    const bool zero_level = ((cb - 0x01010101u) & ~cb & 0x80808080u) != 0u; // some L_k == 0
    qbits = (G == 64 || !zero_level) ? 17 : 16;
  }
  const int32_t *ptab = p.page_table + (size_t)seq * p.maxp;
  const size_t hstride = (size_t)Hkv * p.block_bytes;
  const size_t hoff = (size_t)kv * p.block_bytes;
  // In a fused step the block holding the window appends; when that
  // evicts, the pair's last page (the plan keeps it in this split) is taken
  // after the loop, once the append has written it.
  const bool fused_evict = b.fused && with_window && b.len[e] - 1 >= kWindow;
  const int pf = fused_evict ? np - 1 : full_pages_end(n_hist, p0, p1); // p0 <= pf <= p1

  // ---- prologue: R_K (direct to shared memory; no such load may be
  // outstanding in the page loop, where the compiler would order every
  // shared-memory access after it), the query rows and the first segment's
  // page ids are staged; the block builds the query record.
  stage_table<D>(sm.R, p.RK + (size_t)kv * D * D, w, W, lane);
  {
    const uint16_t *qrow = q + ((size_t)karg_u16(b.row, e) * p.Hq + kv * GQ) * D;
    for (int idx = tid; idx < GQ * D; idx += NT) sm.u.pre.qT[idx % D][idx / D] = bf16f(qrow[idx]);
  }
  for (int i = p0 + tid; i < min(pf, p0 + kIdCache); i += NT) sm.ids[i - p0] = ptab[i];
  if (tid == 0) {
    sm.claim = (uint32_t)p0;
    sm.exited = 0u;
    sm.win.app_slot_done = sm.win.app_page_done = 0;
  }
  for (int idx = tid; idx < W * 16; idx += NT) sm.alpha[idx / 16][idx % 16] = 1.f;
  if (tid < 16) sm.Mb[tid] = -INFINITY;
  __builtin_amdgcn_s_waitcnt(0); // the direct loads of R_K have landed
  __syncthreads();

  // Page stream state.  Segment [seg0, segf) of the split's full pages has
  // its ids in shared memory; deterministic pools take pages w, w + W, ...
  // of the segment, others take them from the shared counter.
  constexpr int PF = kPrefetch<D, G, GQ>, NB = PF + 1;
  const bool det = p.deterministic != 0;
  int seg0 = p0, segf = min(pf, p0 + kIdCache), next_static = p0 + w;
  auto take = [&]() __attribute__((always_inline)) {
    uint32_t c = 0;
    if (!det && lane == 0) c = atomicAdd(&sm.claim, 1u);
    const int pg = det ? next_static : (int)__builtin_amdgcn_readlane(c, 0);
    next_static += W;
    return pg;
  };
  auto load = [&](PageRegs<D, G> &buf, int page) __attribute__((always_inline)) {
    const int id = __builtin_amdgcn_readfirstlane(sm.ids[min(page, segf - 1) - seg0]);
    load_page<D, G>(buf, p.pages + (size_t)id * hstride + hoff, page < segf, p.block_bytes, n, r);
  };
  PageRegs<D, G> buf[NB];
  int pg[NB];
  // The first WW waves take the pair's window (if this block holds it)
  // before joining the page stream; the other waves issue the loads of
  // their first pages before the query preparation, which then overlaps
  // them.  The two kinds of wave run the same barriers (query_prep's) on
  // separate code paths, so the registers of the primed pages are not held
  // across the window.  Each wave then zeroes its own P' rows (only this
  // wave touches them; rows no head owns stay zero for the whole loop).
  auto finish_prologue = [&]() __attribute__((always_inline)) {
    query_prep<D, G, GQ, W, LUT>(sm.u.pre, sm.rec, sm.R, qscale, tid, qbits);
    u32x4 *P = (u32x4 *)&sm.u.P[w][0][0][0];
    for (int idx = lane; idx < NG * 16 * kPRow / 8; idx += 64) P[idx] = u32x4{0u, 0u, 0u, 0u};
  };
  bool primed = false;
  if (!(with_window && w < WW)) {
    if (p0 < pf) {
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        pg[i] = take();
        load(buf[i], pg[i]);
      }
      primed = true;
    }
    finish_prologue();
  } else {
    finish_prologue();
    if (b.fused) {
      if (w < 2) fused_append_slot<D, GQ, WW>(sm.win, p, b, in, e, kv, w, lane);
      wait_count(&sm.win.app_slot_done, 2, p);
    }
    window_waves<D, G, GQ, WW>(sm.win, p, b, q, qscale, e, kv, w);
    if (b.fused && w < 2) fused_append_page<D, G, GQ, WW>(sm.win, sm.R, p, b, e, kv, w, lane);
  }
  auto stage = [&](int s0, int sf) __attribute__((always_inline)) {
    for (int i = s0 + tid; i < sf; i += NT) sm.ids[i - s0] = ptab[i];
    if (tid == 0) sm.claim = (uint32_t)s0;
    __syncthreads();
  };

  // this pair's query record
  const uint32_t *rec = sm.rec;
  const float *tail = (const float *)(rec + RT * MI * 256);
  v4i Aq[RT][MI];
  float kfac[RT], ikfac[RT], qsum[RT][NG];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) Aq[rt][mi] = *(const v4i *)(rec + ((rt * MI + mi) * 64 + lane) * 4);
    const int hs = min(rt * 4 + r, GQ - 1); // head of this lane in the logit layout
    kfac[rt] = tail[32 + hs];
    ikfac[rt] = 1.f / kfac[rt];
#pragma unroll
    for (int g = 0; g < NG; ++g) qsum[rt][g] = tail[hs * NG + g] / kfac[rt]; // exact: kfac = 2^-k
  }

  // per-token factor of P': 2^pv_shift * 4^-e(k), k = token within its
  // 16-token block, e = pair index (k >> 1), or (k >> 1) - 5 past the shift
  // (codebook pools: the V bytes are unshifted, so 2^pv_shift alone)
  float pfac[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const int k = (4 * n + T) & 15, i = k >> 1;
    const int ee = i <= 4 ? i : i - 5;
    pfac[T] = ldexpf(1.f, LUT ? p.pv_shift : p.pv_shift - 2 * ee);
  }
  // Codebook pools: the levels as permute tables, K as signed bytes L - 128
  // (the int8 MFMA operand), V as unsigned bytes L (fp16 sub-normals)
  const uint32_t lutK = LUT ? p.codebook[kv] ^ 0x80808080u : 0u;
  const uint32_t lutV = LUT ? p.codebook[Hkv + kv] : 0u;

  float m_run[RT], thr[RT], l_run[RT], zs[RT][NG];
  v4f acc[NJ];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    thr[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) zs[rt][g] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  // One page of this wave: logits, online softmax, P' and PV.
  // `full`: every token of the page is valid (all pages but a sequence's last)
  auto page_step = [&](const PageRegs<D, G> &cur, const int pi, const bool full) __attribute__((always_inline)) {
      const int ntok = full ? kPage : min(kPage, n_hist - pi * kPage);

      // ---- QK^T: logits of heads (rt*4 + r) for tokens 4n + T
      float lg[RT][4];
  #pragma unroll
      for (int T = 0; T < 4; ++T) {
        v4i cacc[RT][NG];
  #pragma unroll
        for (int rt = 0; rt < RT; ++rt)
  #pragma unroll
          for (int g = 0; g < NG; ++g) cacc[rt][g] = v4i{0, 0, 0, 0};
  #pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const uint32_t wv = cur.kc[(T * MI + mi) / 4][(T * MI + mi) % 4];
          v4i B;
          if constexpr (LUT)
            // each byte's code selects its level byte
            B = v4i{(int)__builtin_amdgcn_perm(lutK, lutK, wv & 0x03030303u),
                    (int)__builtin_amdgcn_perm(lutK, lutK, (wv >> 2) & 0x03030303u),
                    (int)__builtin_amdgcn_perm(lutK, lutK, (wv >> 4) & 0x03030303u),
                    (int)__builtin_amdgcn_perm(lutK, lutK, (wv >> 6) & 0x03030303u)};
          else
            B = v4i{(int)(wv & 0x03030303u), (int)(wv & 0x0C0C0C0Cu), (int)(wv & 0x30303030u),
                    (int)((wv >> 6) & 0x03030303u)};
          const int g = NG == 1 ? 0 : mi;
  #pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            cacc[rt][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aq[rt][mi], B, cacc[rt][g], 0, 0, 0);
        }
        const bool tvalid = full || 4 * n + T < ntok;
  #pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          float l = 0.f;
  #pragma unroll
          for (int g = 0; g < NG; ++g) {
            // |dv| < 2^31: the limb sum is exact in wrapping int32 arithmetic
            // (c0 + 2^8 (c1 + 2^8 c2): two shift-and-add instructions)
            const uint32_t hi = ((uint32_t)cacc[rt][g][2] << 8) + (uint32_t)cacc[rt][g][1];
            const float dv = (float)(int)((hi << 8) + (uint32_t)cacc[rt][g][0]);
            const uint32_t sz = cur.kp[(T * NG + g) / 4][(T * NG + g) % 4];
            // the logit in units of kfac (a power of two; the softmax below
            // applies it), so the products are those of kfac * logit exactly
            if constexpr (LUT) {
              // level = (L - 128) / 64 + 2: the zero point gains 2 s
              const float sc = f16lo(sz);
              l = fmaf(sc, dv, fmaf(fmaf(2.f, sc, f16hi(sz)), qsum[rt][g], l));
            } else {
              l = fmaf(f16lo(sz), dv, fmaf(f16hi(sz), qsum[rt][g], l));
            }
          }
          const bool vis = tvalid && (GQ >= 4 || rt * 4 + r < GQ);
          lg[rt][T] = vis ? l : -INFINITY;
        }
      }

      // ---- online softmax over the page (per head: 16 lanes x 4 tokens).
      // The running reference m_run of a head moves only when the page's
      // maximum exceeds it by more than kLazy: weights stay <= 2^kLazy and
      // the PV accumulators are rescaled rarely.  Each lane compares its own
      // maximum with that threshold (kept in logit units, thr = (m_run +
      // kLazy) / kfac, exact: kfac is a power of two); only on the (rare)
      // pages where some lane exceeds it are the row maxima, the new
      // references, their rescale factors and the factors' trip through
      // shared memory computed.
      bool any_jump = false;
      float lmax[RT], alpha[RT];
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        lmax[rt] = fmaxf(fmaxf(lg[rt][0], lg[rt][1]), fmaxf(lg[rt][2], lg[rt][3]));
        any_jump = any_jump || lmax[rt] > thr[rt];
        alpha[rt] = 1.f;
      }
      any_jump = __any(any_jump);
      if (any_jump) {
  #pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float mt = row16_max_dpp(lmax[rt]) * kfac[rt];
          const bool jump = mt > m_run[rt] + kLazy;
          const float mnew = jump ? mt : m_run[rt];
          alpha[rt] = jump ? fast_exp2(m_run[rt] - mnew) : 1.f;
          m_run[rt] = mnew;
          thr[rt] = (mnew + kLazy) * ikfac[rt]; // exact: kfac is a power of two
        }
      }
      // V scale times the token factor of P' (exact: pfac is a power of
      // two), once per token for all row tiles
      float spf[NG][4];
  #pragma unroll
      for (int T = 0; T < 4; ++T)
  #pragma unroll
        for (int g = 0; g < NG; ++g) spf[g][T] = fmaf(f16lo(cur.vp[(T * NG + g) / 4][(T * NG + g) % 4]), pfac[T], 0.f);
  #pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int hrow = rt * 4 + r;
        const float mnew = m_run[rt];
        float psum = 0.f;
        float zadd[NG];
  #pragma unroll
        for (int g = 0; g < NG; ++g) zadd[g] = 0.f;
        float pv[NG][4];
  #pragma unroll
        for (int T = 0; T < 4; ++T) {
          const bool ok = (full && GQ >= 4) || lg[rt][T] != -INFINITY;
          const float pt = ok ? fast_exp2(fmaf(lg[rt][T], kfac[rt], -mnew)) : 0.f;
          psum += pt;
  #pragma unroll
          for (int g = 0; g < NG; ++g) {
            const uint32_t sz = cur.vp[(T * NG + g) / 4][(T * NG + g) % 4];
            zadd[g] = ok ? fmaf(pt, f16hi(sz), zadd[g]) : zadd[g];
            pv[g][T] = ok ? pt * spf[g][T] : 0.f;
          }
        }
        l_run[rt] = fmaf(l_run[rt], alpha[rt], psum);
  #pragma unroll
        for (int g = 0; g < NG; ++g) {
          zs[rt][g] = fmaf(zs[rt][g], alpha[rt], zadd[g]);
          if (hrow < GQ) {
            union {
              _Float16 h[4];
              u32x2 u;
            } hi, lo;
  #pragma unroll
            for (int T = 0; T < 4; ++T) {
              hi.h[T] = (_Float16)pv[g][T];
              // the remainder, exact in fp32, rounded to fp16
              if constexpr (LO) lo.h[T] = (_Float16)(pv[g][T] - (float)hi.h[T]);
            }
            *(u32x2 *)&sm.u.P[w][g][hrow][4 * n] = hi.u;
            if constexpr (LO) *(u32x2 *)&sm.u.P[w][g][GQ + hrow][4 * n] = lo.u;
          }
        }
        if (any_jump && n == 0 && hrow < GQ) {
          sm.alpha[w][hrow] = alpha[rt];
          if constexpr (LO) sm.alpha[w][GQ + hrow] = alpha[rt];
        }
      }
      wave_sync();

      // ---- rescale the PV accumulators when some row's reference moved
      // (rows whose reference stayed have alpha 1)
      if (any_jump) {
        const v4f a4 = *(const v4f *)&sm.alpha[w][4 * r];
  #pragma unroll
        for (int j = 0; j < NJ; ++j) acc[j] *= a4;
      }

      // ---- PV: rows = heads, columns = channels 16 j + n
      v8h Ap[NG][2];
  #pragma unroll
      for (int g = 0; g < NG; ++g)
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb) Ap[g][kb] = *(const v8h *)&sm.u.P[w][g][n][16 * r + 8 * kb];
  #pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint32_t wv = cur.vc[j / 4][j % 4];
        u32x4 b0, b1;
        if constexpr (LUT) {
          // token k's code sits at bit 16 (k & 1) + 2 (k >> 1): one permute
          // per four codes gives x_i, the level bytes of tokens 2i, 8 + 2i,
          // 2i + 1, 9 + 2i; a mask (tokens 2i, 2i + 1) and a second permute
          // (tokens 8 + 2i, 9 + 2i) put each pair in bytes 0 and 2 with zero
          // bytes above: two fp16 sub-normals L * 2^-24
          uint32_t lo4[4], hi4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t x = __builtin_amdgcn_perm(lutV, lutV, (wv >> (2 * i)) & 0x03030303u);
            lo4[i] = x & 0x00FF00FFu;
            hi4[i] = __builtin_amdgcn_perm(x, x, 0x0C030C01u);
          }
          b0 = u32x4{lo4[0], lo4[1], lo4[2], lo4[3]};
          b1 = u32x4{hi4[0], hi4[1], hi4[2], hi4[3]};
        } else {
          const uint32_t w2 = wv >> 10;
          b0 = u32x4{wv & 0x00030003u, wv & 0x000C000Cu, wv & 0x00300030u, wv & 0x00C000C0u};
          b1 = u32x4{wv & 0x03000300u, w2 & 0x00030003u, w2 & 0x000C000Cu, w2 & 0x00300030u};
        }
        const int g = (16 * j) / G;
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ap[g][0], __builtin_bit_cast(v8h, b0), acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ap[g][1], __builtin_bit_cast(v8h, b1), acc[j], 0, 0, 0);
      }
      // the next page rewrites P' and alpha only after every lane read them
      wave_sync();
  };

  // Page stream of a wave.  The split's pages [p0, p1) are cut in segments
  // of up to kIdCache pages whose ids are staged in shared memory.  Inside a
  // segment a wave takes one page at a time from a shared-memory counter
  // (or, deterministic pools, pages w, w + W, ... of the segment), so waves
  // that run ahead take more pages.  NB register buffers rotate: the loads
  // of the page PF steps ahead are in flight while a page is computed; the
  // page for those loads was taken one step earlier.  Every step issues its
  // loads (a page past the segment end loads through an empty resource),
  // so each wait is an exact count of younger loads.  Only a sequence's
  // last page can be partial; it goes to the last wave after the loop.
  for (int s0 = p0; s0 < pf; s0 += kIdCache) {
    const int sf = min(pf, s0 + kIdCache);
    if (s0 != p0) {
      __syncthreads(); // every wave is done with the previous ids
      stage(s0, sf);
      seg0 = s0;
      segf = sf;
      next_static = s0 + w;
    }
    if (!primed) {
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        pg[i] = take();
        load(buf[i], pg[i]);
      }
    }
    primed = false;
    while (pg[0] < sf) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        pg[(j + PF) % NB] = take();
        load(buf[(j + PF) % NB], pg[(j + PF) % NB]);
        if (pg[j] < sf) page_step(buf[j], pg[j], true);
      }
    }
  }
  if (pf < p1 && w == W - 1) {
    int id;
    if (fused_evict) {
      wait_count(&sm.win.app_page_done, 2, p);
      // a page the append took (the evicted token started it, or it is the
      // copy of a shared page): its id may not be in the table yet
      id = b.new_page[e] >= 0 ? b.new_page[e] : ptab[pf];
    } else {
      id = ptab[pf];
    }
    PageRegs<D, G> last;
    load_page<D, G>(last, p.pages + (size_t)id * hstride + hoff, true, p.block_bytes, n, r);
    page_step(last, pf, false);
  }

  // ---- epilogue: per-wave (m, l, acc); each wave weights its accumulators
  // by 2^(m_w - m) (m: the block maximum), the waves are summed, and the sum
  // is de-rotated by R_V^T: the stored partial is in the basis of V itself.
  // R_V^T replaces R_K in shared memory: the first wave out of the page loop
  // copies it (direct to shared memory) while the others finish their last
  // pages; in a fused step's window block only once the appends are done
  // reading R_K.  No page load of this wave is outstanding any more.
  {
    uint32_t order = 0;
    if (lane == 0) order = atomicAdd(&sm.exited, 1u);
    if (__builtin_amdgcn_readlane(order, 0) == 0) {
      if (b.fused && with_window) wait_count(&sm.win.app_page_done, 2, p);
      stage_table<D>(sm.R, p.RVt + (size_t)kv * D * D, 0, 1, lane);
      __builtin_amdgcn_s_waitcnt(0); // the copy has landed before the barrier below
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int hrow = rt * 4 + r;
    const float l = lanes_sum<16>(l_run[rt]);
    float z[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) z[g] = lanes_sum<16>(zs[rt][g]);
    if (n == 0 && hrow < GQ) {
      sm.M[w][hrow] = m_run[rt];
      sm.L[w][hrow] = l;
      __hip_atomic_fetch_max(&sm.Mb[hrow], m_run[rt], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
      for (int g = 0; g < NG; ++g) sm.zsum[w][hrow][g] = z[g];
    }
  }
  __syncthreads(); // every wave has left the loop: P' may be overwritten
  {
    // heads 4 r + i of this lane's accumulator rows: the block maximum and
    // this wave's (two shared-memory reads, not one per wave)
    // (rows GQ .. 2 GQ - 1 hold the remainder part of heads 0 .. GQ - 1)
    float mb[4], mw[4];
    if constexpr (GQ % 4 == 0) {
      const int hb = LO ? (4 * r) % GQ : 4 * r;
      const float4 tb = *(const float4 *)&sm.Mb[hb];
      const float4 tw = *(const float4 *)&sm.M[w][hb];
      mb[0] = tb.x, mb[1] = tb.y, mb[2] = tb.z, mb[3] = tb.w;
      mw[0] = tw.x, mw[1] = tw.y, mw[2] = tw.z, mw[3] = tw.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * r + i, h = LO && row >= GQ ? row - GQ : row;
        mb[i] = h < GQ ? sm.Mb[h] : -INFINITY;
        mw[i] = h < GQ ? sm.M[w][h] : -INFINITY;
      }
    }
    const float unscale = ldexpf(1.f, LUT ? 18 - p.pv_shift : 24 - p.pv_shift); // codebook bytes: 64 x the level
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * r + i;
      const float f = mw[i] == -INFINITY ? 0.f : exp2f(mw[i] - mb[i]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = 16 * j + n;
        if (h < GQ) sm.u.A[w][h][c] = f * fmaf(acc[j][i], unscale, sm.zsum[w][h][c / G]);
      }
    }
    if constexpr (LO) {
      wave_sync(); // the head rows of this wave are written
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * r + i;
        const float f = mw[i] == -INFINITY ? 0.f : exp2f(mw[i] - mb[i]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int c = 16 * j + n;
          if (row >= GQ && row < 2 * GQ) sm.u.A[w][row - GQ][c] += f * (acc[j][i] * unscale);
        }
      }
    }
  }
  __syncthreads();
  float *dst = ws_hist + (size_t)slot * GQ * (D + 2);
  for (int idx = tid; idx < GQ * D; idx += NT) {
    const int h = idx / D, j = idx % D;
    float a = 0.f;
    for (int ww = 0; ww < W; ++ww) a += sm.u.A[ww][h][j];
    sm.mT[j][h] = a;
  }
  // A pair whose only split this is (b.direct: every pair of the launch
  // has one) combines its history and window results here and writes the
  // normalised rows: no merge launch.  dir[0][h] / dir[1][h]: the factors
  // of the history and window sums (their maxima against the joint one),
  // divided by the joint denominator; wf[ww][h]: each window wave's weight.
  static_assert(2 + WW <= W, "the direct-output factors fit in the rescale rows");
  const bool direct = b.direct;
  float(*dir)[16] = sm.alpha; // free after the page loop
  float(*wf)[16] = sm.alpha + 2;
  if (tid < GQ) {
    const float m = sm.Mb[tid];
    float l = 0.f;
    for (int ww = 0; ww < W; ++ww)
      if (sm.M[ww][tid] != -INFINITY) l = fmaf(exp2f(sm.M[ww][tid] - m), sm.L[ww][tid], l);
    if (direct) {
      float mw = -INFINITY, lw = 0.f;
      for (int ww = 0; ww < WW; ++ww) mw = fmaxf(mw, sm.win.M[ww][tid]);
      for (int ww = 0; ww < WW; ++ww) {
        const float f = sm.win.M[ww][tid] == -INFINITY ? 0.f : exp2f(sm.win.M[ww][tid] - mw);
        wf[ww][tid] = f;
        lw += f * sm.win.L[ww][tid];
      }
      const float mm = fmaxf(m, mw); // the window is never empty
      const float fh = m == -INFINITY ? 0.f : exp2f(m - mm), fw = exp2f(mw - mm);
      const float il = 1.f / fmaf(fh, l, fw * lw);
      dir[0][tid] = fh * il;
      dir[1][tid] = fw * il;
    } else {
      dst[(size_t)tid * (D + 2) + D] = m;
      dst[(size_t)tid * (D + 2) + D + 1] = l;
    }
  }
  __syncthreads();
  if (direct) {
    float *o = out + ((size_t)karg_u16(b.row, e) * p.Hq + kv * GQ) * D;
    contract_columns<D, GQ, W>(&sm.mT[0][0], sm.R, w, lane, [&](int h, int c, float y) {
      float aw = 0.f;
#pragma unroll
      for (int ww = 0; ww < WW; ++ww) aw = fmaf(wf[ww][h], sm.win.A[ww][h][c], aw);
      o[(size_t)h * D + c] = fmaf(dir[0][h], y, dir[1][h] * aw);
    });
    return;
  }
  contract_columns<D, GQ, W>(&sm.mT[0][0], sm.R, w, lane,
                             [&](int h, int c, float y) { dst[(size_t)h * (D + 2) + c] = y; });
  // the window waves' results were written before the barriers above
  if (with_window) block_merge_store<D, GQ, WW>(sm.win.M, sm.win.L, sm.win.A, ws_win + ((size_t)e * p.Hq + kv * GQ) * (D + 2));
}


// Merge of one (sequence, kv head): the split partials (already in the
// basis of V; a split without pages holds m = -inf) and the window partial
// -> out = acc / l.  The pair's split partials sit in consecutive slots
// (stride: the batch's largest split count), so the first SB of them are
// read together with the window partial, before the pair's own split count
// is known; slots at or past it are read (in bounds) but never used.  One
// thread per (head, channel) output.
template <int D, int GQ, int NT>
__device__ void merge_pair(const PoolDev &p, const DecodeBatch &b, float *out, const float *ws, int e, int kv,
                           int tid) {
  constexpr int SB = 4; // splits per batch of loads
  const int Hkv = p.Hkv, Hq = p.Hq;
  const float *ws_win = ws;
  const int smax = karg_u8(b.nsplit, 0); // launch order is by split count, descending
  const float *ws_pair = ws + (size_t)b.n * Hq * (D + 2) + (size_t)(e * Hkv + kv) * smax * GQ * (D + 2);
  const int S = karg_u8(b.nsplit, e);
  float *out_pair = out + ((size_t)karg_u16(b.row, e) * Hq + kv * GQ) * D;
  for (int idx = tid; idx < GQ * D; idx += NT) {
    const int h = idx / D, c = idx % D;
    const float *win = ws_win + ((size_t)e * Hq + kv * GQ + h) * (D + 2);
    float m = win[D], l = win[D + 1], a = win[c];
    float hm[SB], hl[SB], ha[SB];
    auto fetch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const float *ph = ws_pair + ((size_t)min(s0 + j, smax - 1) * GQ + h) * (D + 2);
        hm[j] = ph[D];
        hl[j] = ph[D + 1];
        ha[j] = ph[c];
      }
    };
    auto fold = [&](int s0) __attribute__((always_inline)) {
      float mm = m;
#pragma unroll
      for (int j = 0; j < SB; ++j)
        if (s0 + j < S) mm = fmaxf(mm, hm[j]);
      const float f0 = exp2f(m - mm); // the window partial is never empty
      l *= f0;
      a *= f0;
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        // selects, not branches: slots past S hold stale words
        const bool use = s0 + j < S && hm[j] != -INFINITY;
        const float f = exp2f(hm[j] - mm);
        l = use ? fmaf(f, hl[j], l) : l;
        a = use ? fmaf(f, ha[j], a) : a;
      }
      m = mm;
    };
    fetch(0); // every pair has a split
    fold(0);
    for (int s0 = SB; s0 < S; s0 += SB) {
      fetch(s0);
      fold(s0);
    }
    out_pair[idx] = a / l;
  }
}

// One thread per (head, channel) output of the pair, so each thread does a
// single round of loads.
template <int D, int GQ>
constexpr int merge_threads() { return GQ * D < 1024 ? GQ * D : 1024; }

template <int D, int GQ>
__global__ __launch_bounds__((merge_threads<D, GQ>())) void decode_merge_kernel(PoolDev p, DecodeBatch b, float *__restrict__ out,
                                                                     const float *__restrict__ ws) {
  // grid (sequence, kv head): the pair is known before any kernel argument
  // arrives, so all of them load in one round
  merge_pair<D, GQ, merge_threads<D, GQ>()>(p, b, out, ws, blockIdx.x, blockIdx.y, threadIdx.x);
}

template <int D, int G, int GQ, bool LUT = false>
__global__ __launch_bounds__(64 * main_waves(D, G, GQ)) __attribute__((amdgpu_waves_per_eu(main_occupancy(D, G, GQ))))
void decode_main_kernel(PoolDev p, DecodeBatch b, const uint16_t *__restrict__ q, float qscale,
                        float *__restrict__ ws, float *__restrict__ out, AppendIn in) {
  constexpr int W = main_waves(D, G, GQ);
  __shared__ MainSmem<D, G, GQ, W> sm;
  float *ws_win = ws;
  float *ws_hist = ws + (size_t)b.n * p.Hq * (D + 2);
  const int blk = blockIdx.x, Hkv = p.Hkv;
  int s, e, kv;
  block_split(b, Hkv, blk, s, e, kv);
  const int S = karg_u8(b.nsplit, e);
  const int np = (max(b.len[e] - kWindow, 0) + kPage - 1) / kPage;
  int p0, p1;
  split_range(np, S, s, b.win_units, p0, p1);
  // split partial slot: the pair's splits are consecutive, stride the
  // batch's largest split count (launch order is by split count, descending)
  const int slot = (e * Hkv + kv) * karg_u8(b.nsplit, 0) + s;
  if (p0 < p1)
    history_block<D, G, GQ, LUT>(sm.h, p, b, ws_hist, ws_win, out, q, qscale, in, slot, e, kv, p0, p1, s == S - 1);
  else if (s == S - 1) {
    window_block<D, G, GQ>(sm.w, p, b, q, qscale, ws_win, out, in, e, kv);
    if (b.direct) return;
    // this split holds no pages: an empty history partial for the merge
    float *dst = ws_hist + (size_t)slot * GQ * (D + 2);
    for (int idx = threadIdx.x; idx < GQ * (D + 2); idx += 64 * W) dst[idx] = idx % (D + 2) == D ? -INFINITY : 0.f;
  }
}

template <int D, int G, int GQ>
hipError_t decode_impl(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float *out, float scale,
                       float *ws, AppendIn in, hipStream_t s, const KernelTimer &tm, const KernelTimer &tg) {
  const int blocks = b.hist_blocks;
  // Timed launches take their start/stop timestamps from the dispatch itself
  // (no extra packets between kernels).
  if (p.lut)
    hipExtLaunchKernelGGL((decode_main_kernel<D, G, GQ, true>), dim3(blocks), dim3(64 * main_waves(D, G, GQ)), 0,
                          s, tm.on ? tm.ev[0] : nullptr, tm.on ? tm.ev[1] : nullptr, 0, p, b, q, scale * kLog2e, ws,
                          out, in);
  else
    hipExtLaunchKernelGGL((decode_main_kernel<D, G, GQ>), dim3(blocks), dim3(64 * main_waves(D, G, GQ)), 0, s,
                          tm.on ? tm.ev[0] : nullptr, tm.on ? tm.ev[1] : nullptr, 0, p, b, q, scale * kLog2e, ws, out,
                          in);
  // Pairs split over several blocks are merged by a separate launch:
  // merging in the last block of each pair needs device-scope fences, which
  // cost more than this kernel here.  (b.direct: no pair is split, the
  // blocks wrote the rows.)
  if (!b.direct)
    hipExtLaunchKernelGGL((decode_merge_kernel<D, GQ>), dim3(b.n, p.Hkv), dim3(merge_threads<D, GQ>()), 0, s,
                          tg.on ? tg.ev[0] : nullptr, tg.on ? tg.ev[1] : nullptr, 0, p, b, out, (const float *)ws);
  return hipGetLastError();
}

template <int D, int G>
hipError_t decode_g(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float *out, float scale, float *ws,
                    AppendIn in, hipStream_t s, const KernelTimer &tm, const KernelTimer &tg) {
  switch (p.Hq / p.Hkv) {
  case 1: return decode_impl<D, G, 1>(p, b, q, out, scale, ws, in, s, tm, tg);
  case 2: return decode_impl<D, G, 2>(p, b, q, out, scale, ws, in, s, tm, tg);
  case 4: return decode_impl<D, G, 4>(p, b, q, out, scale, ws, in, s, tm, tg);
  case 8: return decode_impl<D, G, 8>(p, b, q, out, scale, ws, in, s, tm, tg);
  case 16: return decode_impl<D, G, 16>(p, b, q, out, scale, ws, in, s, tm, tg);
  }
  return hipErrorInvalidValue;
}

template <int D, int G>
int blocks_per_cu_g(const PoolDev &p) {
  int nb = 0;
  hipError_t e = hipErrorInvalidValue;
  if (p.lut) {
    switch (p.Hq / p.Hkv) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 1, true>, 64 * main_waves(D, G, 1), 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 2, true>, 64 * main_waves(D, G, 2), 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 4, true>, 64 * main_waves(D, G, 4), 0); break;
    case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 8, true>, 64 * main_waves(D, G, 8), 0); break;
    case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 16, true>, 64 * main_waves(D, G, 16), 0); break;
    }
    return e == hipSuccess ? nb : 0;
  }
  switch (p.Hq / p.Hkv) {
  case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 1>, 64 * main_waves(D, G, 1), 0); break;
  case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 2>, 64 * main_waves(D, G, 2), 0); break;
  case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 4>, 64 * main_waves(D, G, 4), 0); break;
  case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 8>, 64 * main_waves(D, G, 8), 0); break;
  case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_main_kernel<D, G, 16>, 64 * main_waves(D, G, 16), 0); break;
  }
  return e == hipSuccess ? nb : 0;
}

} // namespace

int decode_main_blocks_per_cu(const PoolDev &p) {
  if (p.d == 128 && p.G == 128) return blocks_per_cu_g<128, 128>(p);
  if (p.d == 128 && p.G == 64) return blocks_per_cu_g<128, 64>(p);
  if (p.d == 64 && p.G == 64) return blocks_per_cu_g<64, 64>(p);
  return 0;
}

template <int D>
hipError_t merge_d(const PoolDev &p, const DecodeBatch &b, float *out, const float *ws, hipStream_t s,
                   const KernelTimer &tg) {
#define OSCAR_MERGE(GQv)                                                                                            \
  hipExtLaunchKernelGGL((decode_merge_kernel<D, GQv>), dim3(b.n, p.Hkv), dim3(merge_threads<D, GQv>()), 0, s,       \
                        tg.on ? tg.ev[0] : nullptr, tg.on ? tg.ev[1] : nullptr, 0, p, b, out, ws);                   \
  return hipGetLastError();
  switch (p.Hq / p.Hkv) {
  case 1: { OSCAR_MERGE(1) }
  case 2: { OSCAR_MERGE(2) }
  case 4: { OSCAR_MERGE(4) }
  case 8: { OSCAR_MERGE(8) }
  case 16: { OSCAR_MERGE(16) }
  }
#undef OSCAR_MERGE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const PoolDev &p, const DecodeBatch &b, float *out, const float *ws, hipStream_t s,
                               const KernelTimer &tg) {
  if (p.d == 128) return merge_d<128>(p, b, out, ws, s, tg);
  if (p.d == 64) return merge_d<64>(p, b, out, ws, s, tg);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float *out, float scale,
                         float *ws, const uint16_t *k_new, const uint16_t *v_new, hipStream_t s, const KernelTimer &tm,
                         const KernelTimer &tg) {
  const AppendIn in{k_new, v_new};
  if (p.d == 128 && p.G == 128) return decode_g<128, 128>(p, b, q, out, scale, ws, in, s, tm, tg);
  if (p.d == 128 && p.G == 64) return decode_g<128, 64>(p, b, q, out, scale, ws, in, s, tm, tg);
  if (p.d == 64 && p.G == 64) return decode_g<64, 64>(p, b, q, out, scale, ws, in, s, tm, tg);
  return hipErrorInvalidValue;
}

} // namespace oscar
