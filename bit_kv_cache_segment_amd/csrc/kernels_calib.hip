// Offline calibration statistics of one layer (news article on OSCAR,
// section "OSCAR aims the rotation at attention"): per kv head, the query
// covariance Q^T Q, which sets the eigenbasis of the K rotation, and the
// score-weighted value covariance V^T S^T S V = O^T O, O = S V the causal
// attention output of the calibration sequence, which sets the V rotation.
// Both are summed over the query heads that share the kv head.
//
// Two kernels:
//   calib_attn_kernel  O = causal softmax(scale Q K^T) V per query head, fp32
//                      (one wave per eight query rows, sharing their key and
//                      value loads; the sequence is short and this runs once
//                      per layer, so plain VALU code);
//   gram_kernel        C += X^T X per kv head on v_mfma_f32_16x16x4_f32: one
//                      block per 16 x 16 output tile, its 8 waves splitting
//                      the tokens, the contraction running over tokens (and
//                      the kv head's query heads) four tokens per
//                      instruction, four interleaved accumulators per wave.
#include <hip/hip_runtime.h>

#include "oscar_internal.h"

namespace oscar {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Order shared-memory traffic of the lanes of one wave (no block barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// grid (ceil(n / 32), Hq), 256 threads: wave w takes the QW = 8 query rows
// t0 .. t0 + 7 (t0 = 32 x + 8 w) of query head y, so every key and value row
// a lane loads serves eight queries.  Keys are taken 64 at a time, one per
// lane: the lane's eight logits are full dot products of the queries (in
// shared memory, read as broadcasts) with its key row; the chunk then
// updates each query's running max m, sum l and the lane's D/64 output
// channels (online softmax), the chunk's weights passing through shared
// memory (two broadcast reads per key).  Keys past a query's position
// weigh 0.
template <int D>
__global__ __launch_bounds__(256) void calib_attn_kernel(int n, int Hq, int Hkv, const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v, float scale,
                                                         float *__restrict__ o) {
  constexpr int CPL = D / 64, QW = 8; // output channels per lane; queries per wave
  __shared__ float qs[4][QW][D];
  __shared__ float4 ps[4][64][QW / 4]; // the chunk's weights, [key][query]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * (4 * QW) + QW * w, h = blockIdx.y, kvh = h / (Hq / Hkv);
  for (int idx = lane; idx < QW * D; idx += 64) {
    const int r = idx / D, c = idx % D, t = t0 + r;
    qs[w][r][c] = t < n ? bf16_to_f32(q[((size_t)t * Hq + h) * D + c]) : 0.f;
  }
  __syncthreads();
  if (t0 >= n) return;
  const int tlast = min(t0 + QW - 1, n - 1); // the wave's last query
  float m[QW], l[QW], acc[QW][CPL];
#pragma unroll
  for (int r = 0; r < QW; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[r][i] = 0.f;
  }
  for (int j0 = 0; j0 <= tlast; j0 += 64) {
    const int j = j0 + lane;
    float s[QW];
#pragma unroll
    for (int r = 0; r < QW; ++r) s[r] = 0.f;
    if (j <= tlast) {
      const uint4 *kr = (const uint4 *)(k + ((size_t)j * Hkv + kvh) * D);
#pragma unroll 2
      for (int c8 = 0; c8 < D / 8; ++c8) {
        const uint4 u = kr[c8];
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = __uint_as_float(wd[e] << 16), k1 = __uint_as_float(wd[e] & 0xffff0000u);
#pragma unroll
          for (int r = 0; r < QW; ++r) {
            s[r] = fmaf(qs[w][r][8 * c8 + 2 * e], k0, s[r]);
            s[r] = fmaf(qs[w][r][8 * c8 + 2 * e + 1], k1, s[r]);
          }
        }
      }
    }
    float p[QW];
#pragma unroll
    for (int r = 0; r < QW; ++r) {
      const bool vis = j <= t0 + r && t0 + r < n;
      const float logit = vis ? scale * s[r] : -INFINITY;
      const float mx = wave_max(logit);
      const float m_new = fmaxf(m[r], mx);
      // a query whose every key so far is masked (none yet: j0 > its
      // position never happens before its first chunk) keeps m = -inf
      const float alpha = m_new == -INFINITY ? 1.f : expf(m[r] - m_new);
      p[r] = vis ? expf(logit - m_new) : 0.f;
      l[r] = l[r] * alpha + wave_sum(p[r]);
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[r][i] *= alpha;
      m[r] = m_new;
    }
    const int cnt = min(64, tlast + 1 - j0);
#pragma unroll
    for (int r4 = 0; r4 < QW / 4; ++r4) ps[w][lane][r4] = float4{p[4 * r4], p[4 * r4 + 1], p[4 * r4 + 2], p[4 * r4 + 3]};
    wave_sync();
    for (int jj = 0; jj < cnt; ++jj) {
      float pj[QW];
#pragma unroll
      for (int r4 = 0; r4 < QW / 4; ++r4) {
        const float4 t4 = ps[w][jj][r4];
        pj[4 * r4] = t4.x, pj[4 * r4 + 1] = t4.y, pj[4 * r4 + 2] = t4.z, pj[4 * r4 + 3] = t4.w;
      }
      const uint16_t *vr = v + ((size_t)(j0 + jj) * Hkv + kvh) * D + CPL * lane;
      float vv[CPL];
      if constexpr (CPL == 2) {
        const uint32_t u = *(const uint32_t *)vr;
        vv[0] = __uint_as_float(u << 16);
        vv[1] = __uint_as_float(u & 0xffff0000u);
      } else {
        vv[0] = bf16_to_f32(vr[0]);
      }
#pragma unroll
      for (int r = 0; r < QW; ++r)
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc[r][i] = fmaf(pj[r], vv[i], acc[r][i]);
    }
    // the next chunk rewrites the weights only after every lane read them
    wave_sync();
  }
#pragma unroll
  for (int r = 0; r < QW; ++r) {
    const int t = t0 + r;
    if (t < n) {
      float *orow = o + ((size_t)t * Hq + h) * D + CPL * lane;
#pragma unroll
      for (int i = 0; i < CPL; ++i) orow[i] = acc[r][i] / l[r];
    }
  }
}

template <typename T>
__device__ __forceinline__ float load_f(const T *x, size_t i);
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t *x, size_t i) {
  return bf16_to_f32(x[i]);
}
template <>
__device__ __forceinline__ float load_f<float>(const float *x, size_t i) {
  return x[i];
}

// grid ((D/16)^2, Hkv), 64 GW threads.  X is [n][Hin][D] (Hin = Hkv g);
// output kv head y sums input heads y g .. y g + g - 1.  For tile (ti, tj) the
// instruction's A operand (16 x 4) is X^T rows ti, its B operand (4 x 16)
// X rows at tj: lane l loads channel 16 ti + l % 16 (A) and 16 tj + l % 16
// (B) of token t0 + l / 16; the result's lane l holds rows 4 (l / 16) + r,
// r < 4, of column l % 16.  Wave w of the GW waves takes the w-th share of
// the tokens (multiples of 16); the waves' sums are added in wave order in
// shared memory, and C += the total (accumulated into the caller's matrix;
// one writer per element).
constexpr int kGramWaves = 8;
template <int D, typename T>
__global__ __launch_bounds__(64 * kGramWaves) void gram_kernel(int n, int Hin, int g, const T *__restrict__ x,
                                                               float *__restrict__ cov) {
  constexpr int NT = D / 16, GW = kGramWaves;
  __shared__ floatx4 part[GW][64];
  const int ti = blockIdx.x / NT, tj = blockIdx.x % NT, ho = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
  const int share = ((n + GW - 1) / GW + 15) / 16 * 16;
  const int tb = w * share, te = min(n, tb + share);
  floatx4 acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int hh = 0; hh < g; ++hh) {
    const T *xh = x + (size_t)(ho * g + hh) * D;
    const size_t ld = (size_t)Hin * D;
    for (int t0 = tb; t0 < te; t0 += 16) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int t = t0 + 4 * a + kq;
        float va = 0.f, vb = 0.f;
        if (t < te) {
          va = load_f(xh, t * ld + 16 * ti + r);
          vb = load_f(xh, t * ld + 16 * tj + r);
        }
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(va, vb, acc[a], 0, 0, 0);
      }
    }
  }
  part[w][lane] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (w == 0) {
    floatx4 s = part[0][lane];
#pragma unroll
    for (int ww = 1; ww < GW; ++ww) s += part[ww][lane];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float *c = cov + ((size_t)ho * D + 16 * ti + 4 * kq + rr) * D + 16 * tj + r;
      *c += s[rr];
    }
  }
}

template <int D>
hipError_t attn_impl(int n, int Hq, int Hkv, const uint16_t *q, const uint16_t *k, const uint16_t *v, float scale,
                     float *o, hipStream_t s) {
  hipLaunchKernelGGL(calib_attn_kernel<D>, dim3((n + 31) / 32, Hq), dim3(256), 0, s, n, Hq, Hkv, q, k, v, scale, o);
  return hipGetLastError();
}

template <int D>
hipError_t gram_impl(int n, int Hq, int Hkv, const uint16_t *q, const float *o, float *cov_k, float *cov_v,
                     hipStream_t s) {
  const int g = Hq / Hkv;
  if (cov_k)
    hipLaunchKernelGGL((gram_kernel<D, uint16_t>), dim3((D / 16) * (D / 16), Hkv), dim3(64 * kGramWaves), 0, s, n, Hq,
                       g, q, cov_k);
  if (cov_v)
    hipLaunchKernelGGL((gram_kernel<D, float>), dim3((D / 16) * (D / 16), Hkv), dim3(64 * kGramWaves), 0, s, n, Hq,
                       g, o, cov_v);
  return hipGetLastError();
}

} // namespace

hipError_t launch_calib_attn(int n, int Hq, int Hkv, int d, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             float scale, float *o, hipStream_t s) {
  if (d == 128) return attn_impl<128>(n, Hq, Hkv, q, k, v, scale, o, s);
  if (d == 64) return attn_impl<64>(n, Hq, Hkv, q, k, v, scale, o, s);
  return hipErrorInvalidValue;
}

hipError_t launch_calib_gram(int n, int Hq, int Hkv, int d, const uint16_t *q, const float *o, float *cov_k,
                             float *cov_v, hipStream_t s) {
  if (d == 128) return gram_impl<128>(n, Hq, Hkv, q, o, cov_k, cov_v, s);
  if (d == 64) return gram_impl<64>(n, Hq, Hkv, q, o, cov_k, cov_v, s);
  return hipErrorInvalidValue;
}

} // namespace oscar
