// Prefill attention on matrix cores: many query rows of one kv head attend
// over the three-segment pool.
//
// Method: news article on OSCAR (sanyangsrq.com), section "From offline
// calibration to online inference": the INT2 history is unpacked,
// dequantized with each token's scale and zero point and attended in the
// rotated basis; the BF16 sink and recent tokens are attended in the basis
// of the raw keys; an online softmax merges both.  The query rows of a call
// are (query i, head of the kv head) pairs, flat index i g + hh (g query
// heads per kv head); query i sits at position L - n_q + i and sees the
// positions up to its own.
//
// Launches (one stream), templated on the head dimension D (64 or 128) and
// the scale groups per head row (one, or two for d = 128 and G = 64: then
// the logit sums one QK^T chain per group and P' is formed per group for
// its channel tiles), affine or
// codebook levels (a codebook pool's level is
// z + (L[code] / 64) s: its staged codes are the level bytes L, from one byte
// permute per four codes, and both scales carry the 1/64):
//   prefill_qprep_kernel, one block per (tile of 128 rows, kv head): the
//     rows' queries are rotated by R_K (fp16 MFMAs: the bf16 query is exact
//     in fp16, R_K is staged as hi + lo parts), scaled by
//     scale * log2(e) and 2^E (E per tile: |a| 2^E < 2^14) and split into
//     fp16 hi + lo (~22 bits), laid out as the B operand of
//     v_mfma_f32_32x32x16_f16 with the per-channel factors 4^-e that the K
//     code operand's sub-normal pairs need; the row sums of a (the zero
//     point term) go beside them.
//   prefill_hist_kernel, one block per (two consecutive tiles, kv head,
//     split of their visible history pages), 8 waves of 32 rows, one block
//     per compute unit: the block stages each page once in shared memory
//     as MFMA operands (K and V codes as fp16 sub-normal pairs code 4^e
//     2^-24, per-token scale/zero terms in fp32, the K scale once per tile
//     since E is per tile), for 256 rows; each wave computes
//       S^T = K_codes . (Q_hi + Q_lo)^T        (fp16 MFMA, fp32 accumulate)
//       logit = s_K 2^(24-E) S + z_K sum(a)   (log2 units, exact fp32 terms)
//     runs a lazy online softmax (integer reference m, moved only when a
//     logit exceeds it by more than 8) and accumulates
//       O += P' V_codes,  P' = p s_V 2^pv_shift 4^-e  (fp16 hi + lo)
//     on v_mfma_f32_32x32x16_f16, plus sum p z_V on the VALU.  The token
//     order inside a 32-token tile is chosen so that the S^T accumulators
//     of a lane are the P' operand of the same lane (no data movement).
//     It writes the split's (m, l, O) in the rotated basis.
//   prefill_finish_kernel, one block per (tile, kv head): merges the
//     splits, de-rotates by R_V^T (fp16 MFMAs, the row and R_V^T each split
//     hi + lo, three products), continues the
//     online softmax over the sink and recent tokens with the raw queries
//     (v_mfma_f32_32x32x16_bf16 for both products, P in bf16 hi + lo) and
//     writes the normalised rows.
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 128;       // flat rows per tile (4 waves x 32)
constexpr int kWaves = 4;
constexpr int kPfTilesPerBlock = 2; // tiles whose rows share each staged history page
constexpr int kQBits = 14;       // |a| 2^E < 2^kQBits: fp16 hi/lo parts stay finite
constexpr float kLazyPf = 8.f;   // log2 headroom of the lazy softmax reference
// Per tile, beside the query records: the rows' sums of a for each of up to
// two channel groups (G = 128: one; G = 64: two), then 2^(24 - E).
constexpr int kAux = 2 * kRows + 1;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Token (0..31) of a 32-token tile held in row m of an S^T accumulator: the
// lanes of half h of the wave then hold tokens 16 h .. 16 h + 15, register v
// holding token 16 h + v.
__host__ __device__ inline int tile_token(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
// Row of the S^T accumulator (and A-operand lane) that holds token u.
__host__ __device__ inline int token_row(int u) { return 8 * ((u & 15) >> 2) + 4 * (u >> 4) + (u & 3); }

// Tile geometry shared by the three kernels.
struct TileInfo {
  int f0, nrows;     // first flat row, real rows in the tile
  int pos0, pos1;    // positions of its first and last query
};
__device__ __forceinline__ TileInfo tile_info(const PrefillArgs &a, int T) {
  TileInfo t;
  t.f0 = T * kRows;
  const int rows = a.n_q * a.g;
  t.nrows = min(kRows, rows - t.f0);
  t.pos0 = a.L - a.n_q + t.f0 / a.g;
  t.pos1 = a.L - a.n_q + (t.f0 + t.nrows - 1) / a.g;
  return t;
}

// A d x d fp32 rotation R (row j, column c) as the B operands of
// v_mfma_f32_32x32x16_f16 contractions x . R over j, in shared memory:
// k-step kk, lane (column 32 ct + l % 32, half h = l / 32) holds rows
// (d / 2) h + 8 kk + e, e = 0..7, split into fp16 hi and lo parts (~22 bits).
template <int D>
struct RotB {
  u32x4 b[D / 16][D / 32][2][64]; // [k-step][column tile][hi, lo][lane]  (D^2 4 bytes)
};
template <int D>
__device__ __forceinline__ void stage_rot(RotB<D> &rb, const float *R, int tid) {
  const int lane = tid & 63, ct = tid >> 6, n = lane & 31, h = lane >> 5;
  if (ct >= D / 32) return;
#pragma unroll 2
  for (int kk = 0; kk < D / 16; ++kk) {
    v8h hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y = R[(size_t)(D / 2 * h + 8 * kk + e) * D + 32 * ct + n];
      const _Float16 yh = (_Float16)y;
      hi[e] = yh;
      lo[e] = (_Float16)(y - (float)yh);
    }
    rb.b[kk][ct][0][lane] = __builtin_bit_cast(u32x4, hi);
    rb.b[kk][ct][1][lane] = __builtin_bit_cast(u32x4, lo);
  }
}

// ---------------------------------------------------------------------------
// Query preparation.
// ---------------------------------------------------------------------------
template <int D>
struct QprepSmem {
  RotB<D> rot;                 // R_K as B operands
  float a[kWaves][32][D + 1];  // rotated, scaled rows of each wave
  float up[kWaves][32];        // per row: the power of two its query was scaled down by
  uint32_t amax;               // tile maximum of |a| (bits of a non-negative float)
};

template <int D, int NG>
__global__ __launch_bounds__(256) void prefill_qprep_kernel(PoolDev p, PrefillArgs a, const uint16_t *q,
                                                            u32x4 *qrec, float *qaux) {
  constexpr int KS = D / 16, CT = D / 32; // k-steps of 16 channels, tiles of 32 columns
  __shared__ QprepSmem<D> sm;
  const int T = blockIdx.x, kv = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const TileInfo ti = tile_info(a, T);
  if (tid == 0) sm.amax = 0u;
  // A operand of the rotation: row n of the wave; its half h holds channels
  // (d / 2) h .. (d / 2) h + d / 2 - 1 (8 per k-step)
  const int fr = 32 * w + n; // row in the tile
  const bool real = fr < ti.nrows;
  const int f = ti.f0 + fr;
  u32x4 qv[KS];
  if (real) {
    const int i = f / a.g, head = kv * a.g + f % a.g;
    const u32x4 *src = (const u32x4 *)(q + ((size_t)i * p.Hq + head) * D + D / 2 * h);
#pragma unroll
    for (int k = 0; k < KS; ++k) qv[k] = src[k];
  } else {
#pragma unroll
    for (int k = 0; k < KS; ++k) qv[k] = u32x4{0u, 0u, 0u, 0u};
  }
  // x_rot[c] = sum_j x[j] R_K[j][c]: the query row (bf16, exact in fp16)
  // times R_K's hi and lo parts; k-step kk holds channels (d / 2) h + 8 kk + e
  stage_rot<D>(sm.rot, p.RK + (size_t)kv * D * D, tid);
  __syncthreads();
  // a row whose largest element reaches 2^14 is scaled down by an exact
  // power of two first (fp16 ends at 65504) and scaled back after
  float qm = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qm = fmaxf(qm, fmaxf(fabsf(bf16f((uint16_t)(qv[k][i] & 0xffffu))), fabsf(bf16f((uint16_t)(qv[k][i] >> 16)))));
  qm = fmaxf(qm, __shfl_xor(qm, 32, 64));
  int qe = 0;
  frexpf(qm, &qe);
  const int down = qe > 14 ? qe - 14 : 0;
  if (h == 0) sm.up[w][n] = ldexpf(1.f, down);
  wave_sync();
  v16f acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = v16f{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    v8h A;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wd = qv[kk][e / 2];
      A[e] = (_Float16)ldexpf(bf16f((uint16_t)((e & 1) ? (wd >> 16) : (wd & 0xffffu))), -down);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, __builtin_bit_cast(v8h, sm.rot.b[kk][ct][0][lane]), acc[ct], 0, 0, 0);
      acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, __builtin_bit_cast(v8h, sm.rot.b[kk][ct][1][lane]), acc[ct], 0, 0, 0);
    }
  }
  // scale, tile maximum, transpose through shared memory
  float mx = 0.f;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float y = acc[ct][v] * sm.up[w][8 * (v / 4) + 4 * h + v % 4] * a.qscale;
      mx = fmaxf(mx, fabsf(y));
      sm.a[w][8 * (v / 4) + 4 * h + v % 4][32 * ct + n] = y;
    }
  __syncthreads();
  atomicMax(&sm.amax, __float_as_uint(mx)); // non-negative floats order as their bits
  __syncthreads();
  const float amax = __uint_as_float(sm.amax);
  int ex = 0;
  frexpf(amax, &ex);
  const int E = amax > 0.f ? kQBits - ex : 0; // amax 2^E < 2^kQBits
  // B operand of the QK^T MFMA for lane (row n, half h), k-step ks (the
  // 16 channels 16 ks ..): element e = 2 j + x holds channel
  // 16 ks + 8 x + 4 h + j times 4^-e(4 h + j), e(p) = p <= 4 ? p : p - 5, as
  // fp16 hi and lo parts (the K operand holds code 4^e(p) 2^-24 there)
  u32x4 *dst = qrec + (((size_t)kv * a.NT + T) * kWaves + w) * (KS * 2 * 64);
  float part[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) part[g] = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    v8h hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = e >> 1, pr = 4 * h + j, ef = p.lut ? 0 : (pr <= 4 ? pr : pr - 5);
      const float y = sm.a[w][n][16 * ks + 8 * (e & 1) + pr];
      part[NG == 2 ? ks / (KS / 2) : 0] += y; // k-steps 0 .. KS / 2 - 1 hold the first group
      const float ys = ldexpf(y, E - 2 * ef);
      const _Float16 yh = (_Float16)ys;
      hi[e] = yh;
      lo[e] = (_Float16)(ys - (float)yh);
    }
    dst[(ks * 2 + 0) * 64 + lane] = __builtin_bit_cast(u32x4, hi);
    dst[(ks * 2 + 1) * 64 + lane] = __builtin_bit_cast(u32x4, lo);
  }
  // row sums of a over each channel group (the two halves hold 32 of each)
  float *aux = qaux + ((size_t)kv * a.NT + T) * kAux;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float qsum = part[g] + __shfl_xor(part[g], 32, 64);
    if (h == 0) aux[g * kRows + 32 * w + n] = qsum;
  }
  if (tid == 0) aux[2 * kRows] = ldexpf(1.f, 24 - E);
}

// ---------------------------------------------------------------------------
// History pages.
// ---------------------------------------------------------------------------
// One page (64 tokens of one kv head) as MFMA operands.  The lane slot of
// an operand is XOR-swizzled in bits 1-3 (a constant within each group of 16
// lanes, so a wave's reads stay conflict-free): the staging writes of a wave,
// which would otherwise put four lanes on each bank, spread over all banks.
// K: lane ^ (2 ((lane >> 4) & 1) + 4 ((k-step >> 2) & 1));
// V: lane ^ (4 (channel tile & 1) + 8 ((lane >> 4) & 1)).
template <int D>
struct PageSlot {
  u32x4 K[2][D / 16][64];        // [tile][k-step][lane]: 8 fp16 K code values (A operand)
  u32x4 V[D / 32][2][2][64];     // [channel tile][tile][k-step][lane]: 8 fp16 V code values (B operand)
  float par[8 + 2 * kPfTilesPerBlock][64]; // per token, channel group g: [2g+1] z_K, [4+2g] s_V 2^pv_shift
                                           // 4^-e, [5+2g] z_V; [8+2w+g] s_K 2^(24-E) for tile w of the block
};
template <int D, int NW>
struct HistSmemPf {
  PageSlot<D> slot[2];
  float row[NW][2][32]; // per-wave row broadcast (rescale factors, zero sums)
};

// Raw words of one page a thread of NTH stages: K and V code dwords
// tid + NTH j (4 d of each in a page block), and one parameter dword.
template <int D, int NTH>
struct PageRaw {
  static constexpr int KW = (4 * D + NTH - 1) / NTH;
  uint32_t k[KW], v[KW], par;
};

// npar = 128 NG: the K then V (scale, zero) dwords of the page, token-major
template <int D, int NTH>
__device__ __forceinline__ void load_raw(PageRaw<D, NTH> &r, const uint8_t *blk, int tid, int npar) {
  const uint32_t *w = (const uint32_t *)blk;
#pragma unroll
  for (int j = 0; j < PageRaw<D, NTH>::KW; ++j) {
    const int i = tid + NTH * j;
    const bool in = (4 * D) % NTH == 0 || i < 4 * D;
    r.k[j] = in ? __builtin_nontemporal_load(w + i) : 0u;
    r.v[j] = in ? __builtin_nontemporal_load(w + 4 * D + i) : 0u;
  }
  // K params at byte 32 d + 4 (NG t + g), V params 256 NG bytes later
  r.par = tid < npar ? __builtin_nontemporal_load(w + 8 * D + tid) : 0u;
}

// K code dword i of the pool layout -> (token t, 16-channel group gi): its
// channel pairs (p, p + 8) become fp16 sub-normal pairs code 4^e(p) 2^-24,
// pairs 0..3 in the lanes of half 0 and 4..7 in half 1 of k-step gi.
// Codebook pools (lut != 0): each pair holds the two codes' level bytes L,
// sub-normals L 2^-24 with no 4^e factor.  One byte permute per four codes
// (the codes at bits 2i, 8 + 2i, 16 + 2i, 24 + 2i) gives their level bytes;
// a mask keeps the pair at bits (2i, 16 + 2i) (lo[i]) and a second permute
// moves the pair at bits (8 + 2i, 24 + 2i) into place (hi[i]).
__device__ __forceinline__ void lut_pairs(uint32_t wd, uint32_t lut, u32x4 &lo, u32x4 &hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = __builtin_amdgcn_perm(lut, lut, (wd >> (2 * i)) & 0x03030303u);
    lo[i] = x & 0x00FF00FFu;
    hi[i] = __builtin_amdgcn_perm(x, x, 0x0C030C01u);
  }
}
template <int D>
__device__ __forceinline__ void stage_k(PageSlot<D> &s, int i, uint32_t wd, bool lut, uint32_t lk) {
  const int off = 4 * i;
  const int ls = (off & 1023) >> 4;                 // lane of the share
  const int b = 16 * (off >> 10) + (off & 15);      // byte of the lane's share
  const int t = 4 * (ls & 15) + b / (D / 16);       // token
  const int gi = 4 * ((b % (D / 16)) / 4) + (ls >> 4); // channels 16 gi .. 16 gi + 15
  const uint32_t w2 = wd >> 10;
  const int row = token_row(t & 31);
  const int kz = 2 * ((row >> 4) & 1) + 4 * ((gi >> 2) & 1);
  if (lut) {
    u32x4 lo, hi;
    lut_pairs(wd, lk, lo, hi);
    s.K[t >> 5][gi][row ^ kz] = lo;
    s.K[t >> 5][gi][(row + 32) ^ kz] = hi;
    return;
  }
  s.K[t >> 5][gi][row ^ kz] = u32x4{wd & 0x00030003u, wd & 0x000C000Cu, wd & 0x00300030u, wd & 0x00C000C0u};
  s.K[t >> 5][gi][(row + 32) ^ kz] = u32x4{wd & 0x03000300u, w2 & 0x00030003u, w2 & 0x000C000Cu, w2 & 0x00300030u};
}

// V code dword i -> (channel c, 16-token block r); tokens 8 ks .. 8 ks + 7
// of the block become k-step ks of the B operand (token pairs as fp16
// sub-normals code 4^e 2^-24, e from the pair index).
template <int D>
__device__ __forceinline__ void stage_v(PageSlot<D> &s, int i, uint32_t wd, bool lut, uint32_t lv) {
  const int off = 4 * i;
  const int ls = (off & 1023) >> 4;
  const int b = 16 * (off >> 10) + (off & 15);
  const int r = ls >> 4, c = 16 * (b / 4) + (ls & 15);
  const int lane0 = (c & 31) + 32 * (r & 1);
  const int lane = lane0 ^ (4 * ((c >> 5) & 1) + 8 * ((lane0 >> 4) & 1));
  const uint32_t w2 = wd >> 10;
  if (lut) {
    u32x4 lo, hi;
    lut_pairs(wd, lv, lo, hi);
    s.V[c >> 5][r >> 1][0][lane] = lo;
    s.V[c >> 5][r >> 1][1][lane] = hi;
    return;
  }
  s.V[c >> 5][r >> 1][0][lane] = u32x4{wd & 0x00030003u, wd & 0x000C000Cu, wd & 0x00300030u, wd & 0x00C000C0u};
  s.V[c >> 5][r >> 1][1][lane] = u32x4{wd & 0x03000300u, w2 & 0x00030003u, w2 & 0x000C000Cu, w2 & 0x00300030u};
}

__device__ __forceinline__ float f16lo(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xffffu)); }
__device__ __forceinline__ float f16hi(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(b >> 16)); }

// Codebook pools: a level is z + (L / 64) s, so both scales carry 1/64.
template <int D, int NG, int NTH>
__device__ __forceinline__ void stage_page(PageSlot<D> &s, const PageRaw<D, NTH> &r, int tid, int ntok,
                                           const float (&kscale)[kPfTilesPerBlock], float vscale, bool lut, uint32_t lk,
                                           uint32_t lv) {
#pragma unroll
  for (int j = 0; j < PageRaw<D, NTH>::KW; ++j) {
    const int i = tid + NTH * j;
    if ((4 * D) % NTH == 0 || i < 4 * D) {
      stage_k<D>(s, i, r.k[j], lut, lk);
      stage_v<D>(s, i, r.v[j], lut, lv);
    }
  }
  if (tid < 64 * NG) {
    // tokens past the history hold no data: their terms are zero
    const int t = tid / NG, g = tid % NG;
    const bool ok = t < ntok;
    const float sk = lut ? f16lo(r.par) * 0.015625f : f16lo(r.par);
#pragma unroll
    for (int wt = 0; wt < kPfTilesPerBlock; ++wt) s.par[8 + 2 * wt + g][t] = ok ? sk * kscale[wt] : 0.f;
    s.par[2 * g + 1][t] = ok ? f16hi(r.par) : 0.f;
  } else if (tid < 128 * NG) {
    const int t = (tid - 64 * NG) / NG, g = (tid - 64 * NG) % NG;
    const int pr = (t & 15) >> 1, e = lut ? 3 : (pr <= 4 ? pr : pr - 5); // 4^-3 = 1/64
    const bool ok = t < ntok;
    s.par[4 + 2 * g][t] = ok ? f16lo(r.par) * ldexpf(vscale, -2 * e) : 0.f;
    s.par[5 + 2 * g][t] = ok ? f16hi(r.par) : 0.f;
  }
}

// TW consecutive tiles per block (4 TW waves; a missing last tile's waves
// only stage): every staged page serves 128 TW rows.
template <int D, int NG, int TW>
__global__ __launch_bounds__(256 * TW) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_hist_kernel(
    PoolDev p, PrefillArgs a, const u32x4 *qrec, const float *qaux, float *part_o, float *part_ml) {
  constexpr int KS = D / 16, CT = D / 32; // k-steps of 16 channels, tiles of 32 channels
  constexpr int NTH = 256 * TW;
  static_assert(TW == kPfTilesPerBlock, "the staged K scales are laid out for kPfTilesPerBlock tiles");
  __shared__ HistSmemPf<D, kWaves * TW> sm;
  const int kv = blockIdx.y;
  const int NTP = (a.NT + TW - 1) / TW;
  const int TP = NTP - 1 - (int)blockIdx.x / a.S, s = (int)blockIdx.x % a.S; // later tiles (more pages) first
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int wl = w % kWaves;                 // wave in its tile
  const int T = TW * TP + w / kWaves;        // this wave's tile
  const bool have = T < a.NT;
  const int T0 = TW * TP, T1 = min(TW * TP + TW - 1, a.NT - 1); // the block's first and last tiles
  const TileInfo ti = tile_info(a, have ? T : T0);
  const int n_hist = a.n_hist;
  const int vis_last = prefill_visible_hist(tile_info(a, T1).pos1, n_hist);
  const int pe = (vis_last + kPage - 1) / kPage;                            // pages some row sees
  const int fv = prefill_visible_hist(tile_info(a, T0).pos0, n_hist) / kPage; // pages every row sees whole
  const int p0 = (int)((long)s * pe / a.S), p1 = (int)((long)(s + 1) * pe / a.S);

  // this lane's row (S^T column n)
  const int fr = 32 * wl + n;
  const bool real = have && fr < ti.nrows;
  const int vis = real ? prefill_visible_hist(a.L - a.n_q + (ti.f0 + fr) / a.g, n_hist) : 0;
  const float *aux = qaux + ((size_t)kv * a.NT + (have ? T : T0)) * kAux;
  const float qsum = aux[fr], qsum1 = NG == 2 ? aux[kRows + fr] : 0.f; // per channel group
  // 2^(24 - E) of each tile of the block (E per tile; a missing tile repeats the last)
  float kscale[kPfTilesPerBlock];
#pragma unroll
  for (int wt = 0; wt < kPfTilesPerBlock; ++wt)
    kscale[wt] = qaux[((size_t)kv * a.NT + min(T0 + wt, T1)) * kAux + 2 * kRows];
  const int skr = 8 + 2 * (w / kWaves); // this wave's row of K scales in the staged parameters
  const float vscale = ldexpf(1.f, p.pv_shift);
  const bool lut = p.lut != 0;
  const uint32_t lutK = lut ? p.codebook[kv] : 0u, lutV = lut ? p.codebook[p.Hkv + kv] : 0u;
  v8h Qh[KS], Ql[KS];
  {
    const u32x4 *src = qrec + (((size_t)kv * a.NT + (have ? T : T0)) * kWaves + wl) * (KS * 2 * 64);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Qh[ks] = __builtin_bit_cast(v8h, src[(ks * 2 + 0) * 64 + lane]);
      Ql[ks] = __builtin_bit_cast(v8h, src[(ks * 2 + 1) * 64 + lane]);
    }
  }
  float m = -INFINITY, negm = INFINITY, lsum = 0.f, zsum = 0.f, zsum1 = 0.f;
  v16f O[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) O[ct] = v16f{};

  const int32_t *ptab = p.page_table + (size_t)a.seq * p.maxp;
  const size_t hstride = (size_t)p.Hkv * p.block_bytes, hoff = (size_t)kv * p.block_bytes;
  auto page_ptr = [&](int pi) { return p.pages + (size_t)ptab[pi] * hstride + hoff; };
  auto ntok_of = [&](int pi) { return min(kPage, n_hist - pi * kPage); };

  PageRaw<D, NTH> ra, rb;
  if (p0 < p1) {
    load_raw<D, NTH>(ra, page_ptr(p0), tid, 128 * NG);
    if (p0 + 1 < p1) load_raw<D, NTH>(rb, page_ptr(p0 + 1), tid, 128 * NG);
    stage_page<D, NG, NTH>(sm.slot[0], ra, tid, ntok_of(p0), kscale, vscale, lut, lutK, lutV);
  }
  __syncthreads();

  // One page: nxt holds the raw words of page pi + 1 (loaded one step
  // earlier), fut receives the loads of page pi + 2.  The page's operands
  // are in slot (pi - p0) & 1; page pi + 1 is staged into the other slot
  // after the compute, and one barrier ends the step.
  auto step = [&](int pi, const PageRaw<D, NTH> &nxt, PageRaw<D, NTH> &fut) __attribute__((always_inline)) {
    const int sl = (pi - p0) & 1;
    if (pi + 2 < p1) load_raw<D, NTH>(fut, page_ptr(pi + 2), tid, 128 * NG);
    const PageSlot<D> &S = sm.slot[sl];
    const bool masked = pi >= fv;
    const int tbase = pi * kPage;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (!have) break; // a missing tile's waves only stage
      if constexpr (NG == 2) {
        // two scale groups per token (channels 0..63, 64..127): the logit
        // sums one QK^T chain per group, each with its scale and zero term;
        // it is kept without the reference (lg), which the weights subtract
        const int tok0 = 32 * tt + 16 * h; // token (in the page) of register 0
        float lg[16];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          // the group's per-token logit terms, read before its QK^T chain
          // so that their shared-memory latency overlaps it
          v4f skp[4], zkp[4];
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            skp[J] = *(const v4f *)&S.par[skr + g][tok0 + 4 * J];
            zkp[J] = *(const v4f *)&S.par[2 * g + 1][tok0 + 4 * J];
          }
          v16f acc = v16f{};
#pragma unroll
          for (int k4 = 0; k4 < KS / 2; ++k4) {
            const int ks = KS / 2 * g + k4;
            const v8h A = __builtin_bit_cast(v8h, S.K[tt][ks][lane ^ (2 * ((lane >> 4) & 1) + 4 * ((ks >> 2) & 1))]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, Qh[ks], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, Ql[ks], acc, 0, 0, 0);
          }
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            const v4f sk = skp[J];
            const v4f zk = zkp[J];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int v = 4 * J + i;
              lg[v] = g == 0 ? fmaf(sk[i], acc[v], zk[i] * qsum) : fmaf(sk[i], acc[v], fmaf(zk[i], qsum1, lg[v]));
            }
          }
        }
        float mxl = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (masked) lg[v] = tbase + tok0 + v < vis ? lg[v] : -INFINITY;
          mxl = fmaxf(mxl, lg[v]);
        }
        // lazy reference (as for one group): rows are lanes n and n + 32
        if (__any(mxl > m + kLazyPf)) {
          const float rm = fmaxf(mxl, __shfl_xor(mxl, 32, 64));
          const bool jump = rm > m + kLazyPf;
          const float mn = jump ? ceilf(rm) : m;
          const float alpha = jump ? exp2f(m - mn) : 1.f; // m = -inf: 0
          m = mn;
          lsum *= alpha;
          zsum *= alpha;
          zsum1 *= alpha;
          if (n == lane) sm.row[w][0][n] = alpha;
          wave_sync();
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            const v4f al = *(const v4f *)&sm.row[w][0][8 * J + 4 * h];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
              for (int i = 0; i < 4; ++i) O[ct][4 * J + i] *= al[i];
          }
          wave_sync();
        }
        // a row that has seen no token yet has only masked (-inf) logits
        const float nm = m == -INFINITY ? 0.f : -m;
        float pw[16];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const v4f zv0 = *(const v4f *)&S.par[5][tok0 + 4 * J];
          const v4f zv1 = *(const v4f *)&S.par[7][tok0 + 4 * J];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int v = 4 * J + i;
            const float pv = __builtin_amdgcn_exp2f(lg[v] + nm);
            lsum += pv;
            zsum = fmaf(pv, zv0[i], zsum);
            zsum1 = fmaf(pv, zv1[i], zsum1);
            pw[v] = pv;
          }
        }
        // P' of group g (its V scale) for the channel tiles 2 g, 2 g + 1
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float pp[16];
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            const v4f sp = *(const v4f *)&S.par[4 + 2 * g][tok0 + 4 * J];
#pragma unroll
            for (int i = 0; i < 4; ++i) pp[4 * J + i] = pw[4 * J + i] * sp[i];
          }
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            v8h hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float y = pp[8 * ks + e];
              const _Float16 yh = (_Float16)y;
              hi[e] = yh;
              lo[e] = (_Float16)(y - (float)yh);
            }
#pragma unroll
            for (int c2 = 0; c2 < CT / 2; ++c2) {
              const int ct = CT / 2 * g + c2;
              const v8h B = __builtin_bit_cast(v8h, S.V[ct][tt][ks][lane ^ (4 * (ct & 1) + 8 * ((lane >> 4) & 1))]);
              O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hi, B, O[ct], 0, 0, 0);
              O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(lo, B, O[ct], 0, 0, 0);
            }
          }
        }
      } else {
      const int tok0 = 32 * tt + 16 * h; // token (in the page) of register 0
      // the logits' per-token terms, read before the QK^T chain so that
      // their shared-memory latency overlaps it
      v4f skp[4], zkp[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        skp[J] = *(const v4f *)&S.par[skr][tok0 + 4 * J];
        zkp[J] = *(const v4f *)&S.par[1][tok0 + 4 * J];
      }
      // ---- S^T = K codes . (Q_hi + Q_lo)^T
      v16f acc = v16f{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const v8h A = __builtin_bit_cast(v8h, S.K[tt][ks][lane ^ (2 * ((lane >> 4) & 1) + 4 * ((ks >> 2) & 1))]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, Qh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, Ql[ks], acc, 0, 0, 0);
      }
      // ---- logits (log2 units) of tokens 16 h + v of the tile
      float x[16];
      float mxl = -INFINITY;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const v4f sk = skp[J];
        const v4f zk = zkp[J];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = 4 * J + i;
          float xv = fmaf(sk[i], acc[v], fmaf(zk[i], qsum, negm));
          if (masked) xv = tbase + tok0 + v < vis ? xv : -INFINITY;
          x[v] = xv;
          mxl = fmaxf(mxl, xv);
        }
      }
      // ---- lazy reference: moves (to an integer) only when a logit
      // exceeds it by more than kLazyPf; rows are lanes n and n + 32
      if (__any(mxl > kLazyPf)) {
        float lg = -INFINITY;
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const v4f sk = *(const v4f *)&S.par[skr][tok0 + 4 * J];
          const v4f zk = *(const v4f *)&S.par[1][tok0 + 4 * J];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int v = 4 * J + i;
            const float lv = fmaf(sk[i], acc[v], zk[i] * qsum);
            const bool ok = !masked || tbase + tok0 + v < vis;
            lg = ok ? fmaxf(lg, lv) : lg;
          }
        }
        lg = fmaxf(lg, __shfl_xor(lg, 32, 64));
        const bool jump = lg > m + kLazyPf;
        const float mn = jump ? ceilf(lg) : m;
        const float alpha = jump ? exp2f(m - mn) : 1.f; // m = -inf: 0
        m = mn;
        negm = -mn;
        lsum *= alpha;
        zsum *= alpha;
        if (n == lane) sm.row[w][0][n] = alpha; // lanes 0..31 (both halves agree)
        wave_sync();
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const v4f al = *(const v4f *)&sm.row[w][0][8 * J + 4 * h];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[ct][4 * J + i] *= al[i];
        }
        wave_sync();
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const v4f sk = *(const v4f *)&S.par[skr][tok0 + 4 * J];
          const v4f zk = *(const v4f *)&S.par[1][tok0 + 4 * J];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int v = 4 * J + i;
            const float xv = fmaf(sk[i], acc[v], fmaf(zk[i], qsum, negm));
            x[v] = (!masked || tbase + tok0 + v < vis) ? xv : -INFINITY;
          }
        }
      }
      // ---- weights, sums, P' (fp16 hi + lo) and PV
      float pp[16];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const v4f sp = *(const v4f *)&S.par[4][tok0 + 4 * J];
        const v4f zv = *(const v4f *)&S.par[5][tok0 + 4 * J];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = 4 * J + i;
          const float pv = __builtin_amdgcn_exp2f(x[v]);
          lsum += pv;
          zsum = fmaf(pv, zv[i], zsum);
          pp[v] = pv * sp[i];
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8h hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = pp[8 * ks + e];
          const _Float16 yh = (_Float16)y;
          hi[e] = yh;
          lo[e] = (_Float16)(y - (float)yh);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const v8h B = __builtin_bit_cast(v8h, S.V[ct][tt][ks][lane ^ (4 * (ct & 1) + 8 * ((lane >> 4) & 1))]);
          O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hi, B, O[ct], 0, 0, 0);
          O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(lo, B, O[ct], 0, 0, 0);
        }
      }
      }
    }
    if (pi + 1 < p1) stage_page<D, NG, NTH>(sm.slot[sl ^ 1], nxt, tid, ntok_of(pi + 1), kscale, vscale, lut, lutK, lutV);
    __syncthreads();
  };
  for (int pi = p0; pi < p1; pi += 2) {
    step(pi, rb, ra);
    if (pi + 1 < p1) step(pi + 1, ra, rb);
  }

  // ---- epilogue: (m, l) per row; O in the rotated basis, true units:
  // O 2^(24 - pv_shift) + sum_t p_t z_V(t)
  const float lrow = lsum + __shfl_xor(lsum, 32, 64);
  const float zrow = zsum + __shfl_xor(zsum, 32, 64);
  const float zrow1 = zsum1 + __shfl_xor(zsum1, 32, 64);
  if (lane < 32) {
    sm.row[w][0][n] = zrow;
    sm.row[w][1][n] = zrow1;
  }
  wave_sync();
  if (!have) return;
  const size_t base = (((size_t)kv * a.NT + T) * a.S + s) * kRows + 32 * wl;
  const float k24 = ldexpf(1.f, 24 - p.pv_shift);
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    const v4f zr = *(const v4f *)&sm.row[w][0][8 * J + 4 * h];
    const v4f zr1 = *(const v4f *)&sm.row[w][1][8 * J + 4 * h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 8 * J + 4 * h + i;
      float *dst = part_o + (base + rr) * D + n;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        dst[32 * ct] = fmaf(O[ct][4 * J + i], k24, (NG == 2 && ct >= CT / 2) ? zr1[i] : zr[i]);
    }
  }
  if (lane < 32) {
    part_ml[(base + n) * 2] = m;
    part_ml[(base + n) * 2 + 1] = lrow;
  }
}

// ---------------------------------------------------------------------------
// Merge, de-rotation and the BF16 window.
// ---------------------------------------------------------------------------
template <int D>
struct FinishSmem {
  union {
    RotB<D> rot;               // R_V^T as B operands (de-rotation)
    u32x4 V[2][D / 32][2][64]; // then: [buffer][channel tile][k-step][lane], 8 bf16 window V values
  };
  float row[kWaves][32];
};

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_finish_kernel(PoolDev p, PrefillArgs a, const uint16_t *q,
                                                             const float *part_o, const float *part_ml, float *out) {
  constexpr int KS = D / 16, CT = D / 32;
  constexpr int VW = D / 64; // 16-byte words of a window V row each thread loads (channels D/8 (tid % 8) ..)
  __shared__ FinishSmem<D> sm;
  const int T = blockIdx.x, kv = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const TileInfo ti = tile_info(a, T);
  const int fr = 32 * w + n;
  const bool real = fr < ti.nrows;
  const int f = ti.f0 + fr;
  const int qi = real ? f / a.g : 0, head = kv * a.g + (real ? f % a.g : 0);
  const int rowpos = real ? a.L - a.n_q + qi : -1;

  stage_rot<D>(sm.rot, p.RVt + (size_t)kv * D * D, tid);
  // ---- merge the splits of this lane's row: reference, weights, l
  const size_t base = ((size_t)kv * a.NT + T) * a.S * kRows + fr;
  float M = -INFINITY;
  for (int s = 0; s < a.S; ++s) M = fmaxf(M, part_ml[(base + (size_t)s * kRows) * 2]);
  float L = 0.f;
  // A operand of the de-rotation: O_rot[row][j], j = st + (D / 2) h; the
  // lane keeps its D / 2 merged values
  float orot[D / 2];
#pragma unroll
  for (int j = 0; j < D / 2; ++j) orot[j] = 0.f;
  for (int s = 0; s < a.S; ++s) {
    const float ms = part_ml[(base + (size_t)s * kRows) * 2];
    const float ws = ms == -INFINITY ? 0.f : exp2f(ms - M);
    L = fmaf(ws, part_ml[(base + (size_t)s * kRows) * 2 + 1], L);
    if (ws != 0.f) {
      const v4f *src = (const v4f *)(part_o + (base + (size_t)s * kRows) * D + D / 2 * h);
#pragma unroll
      for (int k = 0; k < D / 8; ++k) {
        const v4f v4 = src[k];
#pragma unroll
        for (int i = 0; i < 4; ++i) orot[4 * k + i] = fmaf(ws, v4[i], orot[4 * k + i]);
      }
    }
  }
  __syncthreads(); // R_V^T staged
  // ---- de-rotation: out[c] = sum_j O_rot[j] R_V^T[j][c].  The row is
  // scaled by 2^-e (|O_rot| / L stays below the largest V value, so the
  // scaled row fits fp16), split into fp16 hi + lo, and multiplied by R_V^T's
  // hi and lo parts (three products; lo x lo is below fp32 rounding); the
  // result is scaled back by 2^e, both exactly.
  int ex = 0;
  frexpf(L, &ex);
  const float sdown = L > 0.f ? ldexpf(1.f, -ex) : 0.f;
  if (lane < 32) sm.row[w][n] = L > 0.f ? ldexpf(1.f, ex) : 0.f;
  v16f O[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) O[ct] = v16f{};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    v8h Ah, Al;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y = orot[8 * kk + e] * sdown;
      const _Float16 yh = (_Float16)y;
      Ah[e] = yh;
      Al[e] = (_Float16)(y - (float)yh);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const v8h Bh = __builtin_bit_cast(v8h, sm.rot.b[kk][ct][0][lane]);
      const v8h Bl = __builtin_bit_cast(v8h, sm.rot.b[kk][ct][1][lane]);
      O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah, Bh, O[ct], 0, 0, 0);
      O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah, Bl, O[ct], 0, 0, 0);
      O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Al, Bh, O[ct], 0, 0, 0);
    }
  }
  wave_sync();
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    const v4f up = *(const v4f *)&sm.row[w][8 * J + 4 * h];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[ct][4 * J + i] *= up[i];
  }
  wave_sync();

  // ---- window: sink and recent tokens, raw queries, bf16 MFMAs
  const int seq = a.seq;
  const int n_sink = min(a.L, kSink), n_rec = min(max(a.L - kSink, 0), kRecent), n_win = n_sink + n_rec;
  const int n_hist = a.n_hist;
  const uint16_t *sinkK = p.sinkK + ((size_t)seq * p.Hkv + kv) * kSink * D;
  const uint16_t *sinkV = p.sinkV + ((size_t)seq * p.Hkv + kv) * kSink * D;
  const uint16_t *recK = p.recentK + ((size_t)seq * p.Hkv + kv) * kRecent * D;
  const uint16_t *recV = p.recentV + ((size_t)seq * p.Hkv + kv) * kRecent * D;
  auto krow = [&](int u) { return u < n_sink ? sinkK + (size_t)u * D : recK + (size_t)(u - n_sink) * D; };
  auto vrow = [&](int u) { return u < n_sink ? sinkV + (size_t)u * D : recV + (size_t)(u - n_sink) * D; };
  // position of window token u (recent slot j holds 64 + n_hist + ((j - n_hist) mod 256))
  auto upos = [&](int u) { return u < n_sink ? u : kSink + n_hist + ((u - n_sink - n_hist) & (kRecent - 1)); };
  // B operand: raw query row n, channels 16 ks + 8 h .. + 7
  v8bf Qw[KS];
  {
    const u32x4 *src = (const u32x4 *)(q + ((size_t)qi * p.Hq + head) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      Qw[ks] = __builtin_bit_cast(v8bf, real ? src[2 * ks + h] : u32x4{0u, 0u, 0u, 0u});
  }
  // online state continues from the merged history (reference M); the
  // row's l is the sum over its two lanes, so the history's L enters once
  float m = M, negm = -M, lsum = h == 0 ? L : 0.f;
  const int nchunk = (n_win + 31) / 32;
  // Chunk c's words are loaded one chunk ahead: the A-operand words of its
  // keys (token tile_token(n) of the chunk, channels 16 ks + 8 h ..) into
  // registers, its V rows (token tid / 8, channels D/8 (tid % 8) ..) into
  // registers and then, transposed to the B operand, into buffer c & 1.
  auto kload = [&](int c, u32x4 (&kr)[KS]) __attribute__((always_inline)) {
    const int u = 32 * c + tile_token(n);
    const bool ok = u < n_win;
    const u32x4 *src = (const u32x4 *)(ok ? krow(u) : sinkK);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kr[ks] = ok ? src[2 * ks + h] : u32x4{0u, 0u, 0u, 0u};
  };
  auto vload = [&](int c, u32x4 (&vr)[VW]) __attribute__((always_inline)) {
    const int u = 32 * c + (tid >> 3);
#pragma unroll
    for (int j = 0; j < VW; ++j) vr[j] = u32x4{0u, 0u, 0u, 0u};
    if (u < n_win) {
      const u32x4 *src = (const u32x4 *)(vrow(u) + D / 8 * (tid & 7));
#pragma unroll
      for (int j = 0; j < VW; ++j) vr[j] = src[j];
    }
  };
  auto vstore = [&](int c, const u32x4 (&vr)[VW]) __attribute__((always_inline)) {
    const int tk = tid >> 3, cb = tid & 7; // token of the chunk, block of D/8 channels
    const int hh = tk >> 4, ks = (tk & 15) >> 3, e = tk & 7;
    uint16_t *V = (uint16_t *)&sm.V[c & 1][0][0][0];
#pragma unroll
    for (int k = 0; k < D / 8; ++k) {
      const uint32_t wd = vr[k / 8][(k % 8) / 2];
      const uint16_t val = (uint16_t)((k & 1) ? (wd >> 16) : (wd & 0xffffu));
      const int c2 = D / 8 * cb + k;
      V[(((c2 >> 5) * 2 + ks) * 64 + (c2 & 31) + 32 * hh) * 8 + e] = val;
    }
  };
  u32x4 kc[KS], kn[KS], vr[VW];
  __syncthreads(); // every wave is done with R_V^T: the window buffers overlay it
  if (nchunk > 0) {
    vload(0, vr);
    vstore(0, vr);
    kload(0, kc);
    if (nchunk > 1) vload(1, vr);
  }
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    if (c + 1 < nchunk) kload(c + 1, kn);
    // S^T = K_win . q^T: A operand token tile_token(n) of the chunk
    v16f S = v16f{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, kc[ks]), Qw[ks], S, 0, 0, 0);
    float x[16], mxl = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int u = 32 * c + 16 * h + v;
      const bool ok = u < n_win && upos(u) <= rowpos;
      x[v] = ok ? fmaf(S[v], a.qscale, negm) : -INFINITY;
      mxl = fmaxf(mxl, x[v]);
    }
    if (__any(mxl > kLazyPf)) {
      float lg = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int u = 32 * c + 16 * h + v;
        const bool ok = u < n_win && upos(u) <= rowpos;
        lg = ok ? fmaxf(lg, S[v] * a.qscale) : lg;
      }
      lg = fmaxf(lg, __shfl_xor(lg, 32, 64));
      const bool jump = lg > m + kLazyPf;
      const float mn = jump ? ceilf(lg) : m;
      const float alpha = jump ? exp2f(m - mn) : 1.f;
      m = mn;
      negm = -mn;
      lsum *= alpha;
      if (n == lane) sm.row[w][n] = alpha;
      wave_sync();
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const v4f al = *(const v4f *)&sm.row[w][8 * J + 4 * h];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[ct][4 * J + i] *= al[i];
      }
      wave_sync();
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int u = 32 * c + 16 * h + v;
        const bool ok = u < n_win && upos(u) <= rowpos;
        x[v] = ok ? fmaf(S[v], a.qscale, negm) : -INFINITY;
      }
    }
    float pp[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      pp[v] = __builtin_amdgcn_exp2f(x[v]);
      lsum += pp[v];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8bf hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = pp[8 * ks + e];
        const __bf16 yh = (__bf16)y;
        hi[e] = yh;
        lo[e] = (__bf16)(y - (float)yh);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const v8bf B = __builtin_bit_cast(v8bf, sm.V[c & 1][ct][ks][lane]);
        O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, B, O[ct], 0, 0, 0);
        O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, B, O[ct], 0, 0, 0);
      }
    }
    if (c + 1 < nchunk) vstore(c + 1, vr);
    if (c + 2 < nchunk) vload(c + 2, vr);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kc[ks] = kn[ks];
  }
  // ---- normalise and store: register (J, i) holds row 8 J + 4 h + i,
  // channel 32 ct + n; the history part was weighted relative to M, the
  // window relative to m >= M (rescales by alpha applied to both)
  const float lrow = lsum + __shfl_xor(lsum, 32, 64);
  if (lane < 32) sm.row[w][n] = lrow > 0.f ? 1.f / lrow : 0.f;
  wave_sync();
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    const v4f il = *(const v4f *)&sm.row[w][8 * J + 4 * h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 8 * J + 4 * h + i;
      const int fo = ti.f0 + 32 * w + rr;
      if (32 * w + rr < ti.nrows) {
        float *dst = out + ((size_t)(fo / a.g) * p.Hq + kv * a.g + fo % a.g) * D + n;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) dst[32 * ct] = O[ct][4 * J + i] * il[i];
      }
    }
  }
}

} // namespace

size_t prefill_mfma_ws_bytes(int Hkv, int NT, int S, int d) {
  const size_t qrec = (size_t)Hkv * NT * kWaves * (d / 16) * 2 * 64 * 16;
  const size_t qaux = (size_t)Hkv * NT * kAux * 4;
  const size_t po = (size_t)Hkv * NT * S * kRows * d * 4;
  const size_t pml = (size_t)Hkv * NT * S * kRows * 2 * 4;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return al(qrec) + al(qaux) + al(po) + al(pml);
}

bool prefill_mfma_supported(const PoolDev &p) {
  return (p.d == 128 || p.d == 64) && (p.G == p.d || (p.d == 128 && p.G == 64)) && !p.bf16_hist;
}

template <int D, int NG>
static void launch_all(const PoolDev &p, const PrefillArgs &a, const uint16_t *q, float *out, u32x4 *qrec,
                       float *qaux, float *po, float *pml, hipStream_t s) {
  constexpr int TW = kPfTilesPerBlock;
  hipLaunchKernelGGL((prefill_qprep_kernel<D, NG>), dim3(a.NT, p.Hkv), dim3(256), 0, s, p, a, q, qrec, qaux);
  hipLaunchKernelGGL((prefill_hist_kernel<D, NG, TW>), dim3((a.NT + TW - 1) / TW * a.S, p.Hkv), dim3(256 * TW), 0, s,
                     p, a, qrec, qaux, po, pml);
  hipLaunchKernelGGL((prefill_finish_kernel<D>), dim3(a.NT, p.Hkv), dim3(256), 0, s, p, a, q, po, pml, out);
}

hipError_t launch_prefill_mfma(const PoolDev &p, const PrefillArgs &a, const uint16_t *q, float *out, void *ws,
                               hipStream_t s) {
  if (!prefill_mfma_supported(p) || a.NT < 1 || a.S < 1) return hipErrorInvalidValue;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  uint8_t *base = (uint8_t *)ws;
  u32x4 *qrec = (u32x4 *)base;
  base += al((size_t)p.Hkv * a.NT * kWaves * (p.d / 16) * 2 * 64 * 16);
  float *qaux = (float *)base;
  base += al((size_t)p.Hkv * a.NT * kAux * 4);
  float *po = (float *)base;
  base += al((size_t)p.Hkv * a.NT * a.S * kRows * p.d * 4);
  float *pml = (float *)base;
  if (p.d == 64)
    launch_all<64, 1>(p, a, q, out, qrec, qaux, po, pml, s);
  else if (p.G == 128)
    launch_all<128, 1>(p, a, q, out, qrec, qaux, po, pml, s);
  else
    launch_all<128, 2>(p, a, q, out, qrec, qaux, po, pml, s);
  return hipGetLastError();
}

} // namespace oscar
