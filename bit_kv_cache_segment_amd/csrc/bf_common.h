// Device pieces of the VALU split-KV decode kernel of the BF16-history
// baseline: DPP lane sums, kernel-argument readers, the BF16 token loop used
// for a pair's window (sink and recent tokens, stored as they are) and for
// the history pages, and the block epilogue's wave merge.
#pragma once

#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;
constexpr int kBfWaves = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum over aligned groups of N lanes (8 or 16).
template <int N>
__device__ __forceinline__ float lanes_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  if constexpr (N == 16) v += dpp_f<0x140>(v);
  return v;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ int karg_u16(const uint16_t *a, int i) {
  return (int)((((const uint32_t *)a)[i >> 1] >> (16 * (i & 1))) & 0xffffu);
}
__device__ __forceinline__ int karg_u8(const uint8_t *a, int i) {
  return (int)((((const uint32_t *)a)[i >> 2] >> (8 * (i & 3))) & 0xffu);
}

template <int D, int GQ>
struct BfSmem {
  alignas(16) uint32_t q2[GQ][D / 2]; // the pair's query rows as bf16 pairs
  float M[kBfWaves][GQ], L[kBfWaves][GQ];
  float A[kBfWaves][GQ][D];
  uint32_t claim;
};

// Running (m, l, acc) of one wave for the GQ heads; this lane's 8 channels.
template <int GQ>
struct BfState {
  float m[GQ], l[GQ], acc[GQ][8];
};

// Token groups [g0, g1) (step `stride`) of a contiguous block of ntok token
// rows (K at k, V at v), into the wave's state.  WG groups' loads are
// issued together, then computed.
template <int D, int GQ, int WG>
__device__ __forceinline__ void bf_tokens(BfState<GQ> &st, const uint16_t *k, const uint16_t *v, int ntok, int g0,
                                          int stride, const uint32_t (*q2)[D / 2], float qscale, int lane) {
  constexpr int LPT = D / 8, TPI = 64 / LPT;
  const int ts = lane / LPT, cc = lane % LPT;
  const int ngroups = (ntok + TPI - 1) / TPI;
  for (int gb = g0; gb < ngroups; gb += WG * stride) {
    u32x4 kr[WG], vr[WG];
#pragma unroll
    for (int i = 0; i < WG; ++i) {
      const int u = (gb + i * stride) * TPI + ts;
      kr[i] = vr[i] = u32x4{0u, 0u, 0u, 0u};
      if (u < ntok) {
        kr[i] = __builtin_nontemporal_load((const u32x4 *)(k + (size_t)u * D + 8 * cc));
        vr[i] = __builtin_nontemporal_load((const u32x4 *)(v + (size_t)u * D + 8 * cc));
      }
    }
#pragma unroll
    for (int i = 0; i < WG; ++i) {
      const int u = (gb + i * stride) * TPI + ts;
      const bool ok = u < ntok;
      float vf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[2 * j] = __uint_as_float(vr[i][j] << 16);
        vf[2 * j + 1] = __uint_as_float(vr[i][j] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const u32x4 qv = *(const u32x4 *)&q2[h][4 * cc];
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t kw = kr[i][j], qw = qv[j];
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw), __builtin_bit_cast(bf16x2, qw), d, false);
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
}


// The wave's state into shared memory: the TPI token slots of the wave
// (lanes cc, cc + LPT, ...) merged, then (m, l) per head and the wave's
// accumulator row.  The caller synchronises the block afterwards.
template <int D, int GQ>
__device__ __forceinline__ void wave_state_to_smem(BfSmem<D, GQ> &sm, BfState<GQ> &st, int w, int lane) {
  constexpr int LPT = D / 8;
  const int ts = lane / LPT, cc = lane % LPT;
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float m = st.m[h];
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float f = st.m[h] == -INFINITY ? 0.f : exp2f(st.m[h] - m);
    float l = st.l[h] * f;
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) l += __shfl_xor(l, o, 64);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = st.acc[h][j] * f;
#pragma unroll
      for (int o = LPT; o < 64; o <<= 1) a += __shfl_xor(a, o, 64);
      st.acc[h][j] = a;
    }
    if (lane == 0) {
      sm.M[w][h] = m;
      sm.L[w][h] = l;
    }
    if (ts == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.A[w][h][8 * cc + j] = st.acc[h][j];
    }
  }
}

// Weighted sum over the block's waves of head h, channel c: accumulator a,
// maximum m and sum l of the block.
template <int D, int GQ>
__device__ __forceinline__ void block_combine(const BfSmem<D, GQ> &sm, int h, int c, float &a, float &m, float &l) {
  m = -INFINITY;
  for (int ww = 0; ww < kBfWaves; ++ww) m = fmaxf(m, sm.M[ww][h]);
  a = 0.f;
  l = 0.f;
  for (int ww = 0; ww < kBfWaves; ++ww) {
    const float f = sm.M[ww][h] == -INFINITY ? 0.f : exp2f(sm.M[ww][h] - m);
    a += f * sm.A[ww][h][c];
    l += f * sm.L[ww][h];
  }
}

} // namespace
} // namespace oscar
