// Offline calibration statistics of one layer (news article on OSCAR,
// section "OSCAR aims the rotation at attention"): per kv head, the query
// covariance Q^T Q, which sets the eigenbasis of the K rotation, and the
// score-weighted value covariance V^T S^T S V = O^T O, O = S V the causal
// attention output of the calibration sequence, which sets the V rotation.
// Both are summed over the query heads that share the kv head.
//
// Two kernels:
//   calib_attn_kernel  O = causal softmax(scale Q K^T) V per query head, fp32
//                      (one wave per query row; the sequence is short and
//                      this runs once per layer, so plain VALU code);
//   gram_kernel        C += X^T X per kv head on v_mfma_f32_16x16x4_f32: one
//                      wave per 16 x 16 output tile, the contraction running
//                      over tokens (and the kv head's query heads) four
//                      tokens per instruction, four interleaved accumulators.
#include <hip/hip_runtime.h>

#include "oscar_internal.h"

namespace oscar {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

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

// grid (ceil(n / 4), Hq), 256 threads: wave w takes query row t = 4 x + w of
// query head y.  Keys are taken 64 at a time, one per lane: the lane's logit
// is a full dot product of the query (in shared memory, read as a broadcast)
// with its key row; the chunk then updates the running max m, sum l and the
// lane's D/64 output channels (online softmax).  Masked keys (j > t) weigh 0.
template <int D>
__global__ __launch_bounds__(256) void calib_attn_kernel(int n, int Hq, int Hkv, const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v, float scale,
                                                         float *__restrict__ o) {
  constexpr int CPL = D / 64; // output channels per lane: CPL lane + i
  __shared__ float qs[4][D];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w, h = blockIdx.y, kvh = h / (Hq / Hkv);
  const bool valid = t < n;
  for (int c = lane; c < D; c += 64) qs[w][c] = valid ? bf16_to_f32(q[((size_t)t * Hq + h) * D + c]) : 0.f;
  __syncthreads();
  if (!valid) return;
  float m = -INFINITY, l = 0.f, acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 <= t; j0 += 64) {
    const int j = j0 + lane;
    float logit = -INFINITY;
    if (j <= t) {
      const uint4 *kr = (const uint4 *)(k + ((size_t)j * Hkv + kvh) * D);
      float s = 0.f;
#pragma unroll 4
      for (int c8 = 0; c8 < D / 8; ++c8) {
        const uint4 u = kr[c8];
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = fmaf(qs[w][8 * c8 + 2 * e], __uint_as_float(wd[e] << 16), s);
          s = fmaf(qs[w][8 * c8 + 2 * e + 1], __uint_as_float(wd[e] & 0xffff0000u), s);
        }
      }
      logit = scale * s;
    }
    const float m_new = fmaxf(m, wave_max(logit)); // finite: key j0 <= t is visible
    const float alpha = expf(m - m_new);           // 0 on the first chunk
    const float p = j <= t ? expf(logit - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] *= alpha;
    const int cnt = min(64, t + 1 - j0);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = __shfl(p, jj);
      const uint16_t *vr = v + ((size_t)(j0 + jj) * Hkv + kvh) * D + CPL * lane;
      if constexpr (CPL == 2) {
        const uint32_t u = *(const uint32_t *)vr;
        acc[0] = fmaf(pj, __uint_as_float(u << 16), acc[0]);
        acc[1] = fmaf(pj, __uint_as_float(u & 0xffff0000u), acc[1]);
      } else {
        acc[0] = fmaf(pj, bf16_to_f32(vr[0]), acc[0]);
      }
    }
    m = m_new;
  }
  float *orow = o + ((size_t)t * Hq + h) * D + CPL * lane;
#pragma unroll
  for (int i = 0; i < CPL; ++i) orow[i] = acc[i] / l;
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

// grid ((D/16)^2, Hkv), 64 threads.  X is [n][Hin][D] (Hin = Hkv g); output
// kv head y sums input heads y g .. y g + g - 1.  For tile (ti, tj) the
// instruction's A operand (16 x 4) is X^T rows ti, its B operand (4 x 16)
// X rows at tj: lane l loads channel 16 ti + l % 16 (A) and 16 tj + l % 16
// (B) of token t0 + l / 16; the result's lane l holds rows 4 (l / 16) + r,
// r < 4, of column l % 16.  C += the tile (accumulated into the caller's
// matrix; one writer per element).
template <int D, typename T>
__global__ __launch_bounds__(64) void gram_kernel(int n, int Hin, int g, const T *__restrict__ x,
                                                  float *__restrict__ cov) {
  constexpr int NT = D / 16;
  const int ti = blockIdx.x / NT, tj = blockIdx.x % NT, ho = blockIdx.y, lane = threadIdx.x;
  const int r = lane & 15, kq = lane >> 4;
  floatx4 acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int hh = 0; hh < g; ++hh) {
    const T *xh = x + (size_t)(ho * g + hh) * D;
    const size_t ld = (size_t)Hin * D;
    for (int t0 = 0; t0 < n; t0 += 16) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int t = t0 + 4 * a + kq;
        float va = 0.f, vb = 0.f;
        if (t < n) {
          va = load_f(xh, t * ld + 16 * ti + r);
          vb = load_f(xh, t * ld + 16 * tj + r);
        }
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(va, vb, acc[a], 0, 0, 0);
      }
    }
  }
  const floatx4 s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    float *c = cov + ((size_t)ho * D + 16 * ti + 4 * kq + rr) * D + 16 * tj + r;
    *c += s[rr];
  }
}

template <int D>
hipError_t attn_impl(int n, int Hq, int Hkv, const uint16_t *q, const uint16_t *k, const uint16_t *v, float scale,
                     float *o, hipStream_t s) {
  hipLaunchKernelGGL(calib_attn_kernel<D>, dim3((n + 3) / 4, Hq), dim3(256), 0, s, n, Hq, Hkv, q, k, v, scale, o);
  return hipGetLastError();
}

template <int D>
hipError_t gram_impl(int n, int Hq, int Hkv, const uint16_t *q, const float *o, float *cov_k, float *cov_v,
                     hipStream_t s) {
  const int g = Hq / Hkv;
  if (cov_k)
    hipLaunchKernelGGL((gram_kernel<D, uint16_t>), dim3((D / 16) * (D / 16), Hkv), dim3(64), 0, s, n, Hq, g, q,
                       cov_k);
  if (cov_v)
    hipLaunchKernelGGL((gram_kernel<D, float>), dim3((D / 16) * (D / 16), Hkv), dim3(64), 0, s, n, Hq, g, o,
                       cov_v);
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
