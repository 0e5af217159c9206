// Internal definitions shared by the host library and the HIP kernels:
// the device view of a pool, the byte layout of a history page, and the
// small by-value argument blocks kernels receive.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oscar {

constexpr int kSink = 64;      // BF16 attention sink tokens
constexpr int kRecent = 256;   // BF16 recent window tokens (a ring of slots)
constexpr int kWindow = kSink + kRecent;
constexpr int kPage = 64;      // history tokens per page
constexpr int kMaxBatch = 256; // sequences per kernel launch (by-value metadata)

// Device-side view of a pool.  All arrays live in the caller's pool buffer.
struct PoolDev {
  const float *RK;     // [Hkv][d][d]  x_rot = x . R_K
  const float *RV;     // [Hkv][d][d]
  const float *RVt;    // [Hkv][d][d]  transpose of R_V (de-rotation, coalesced)
  const float *clipK;  // [Hkv][d]
  const float *clipV;  // [Hkv][d]
  int32_t *page_table; // [max_seqs][maxp]
  uint16_t *sinkK;     // [max_seqs][Hkv][64][d] bf16
  uint16_t *sinkV;
  uint16_t *recentK;   // [max_seqs][Hkv][256][d] bf16, slot = (pos - 64) % 256
  uint16_t *recentV;
  uint8_t *pages;      // [num_pages][Hkv][block_bytes]
  int32_t Hq, Hkv, d, G, maxp;
  int32_t block_bytes; // bytes of one (page, kv head) block
  // 2^(pv_shift + 8) * fp16(2 max(clip_V) / 3) <= 65504: the largest power of
  // two by which a softmax weight (<= 2^8) times a V scale may be multiplied
  // and stay finite in fp16.
  int32_t pv_shift;
  // 1: the waves of a decode block take their pages in a fixed order, so
  // results are bitwise reproducible; 0: pages are handed out dynamically.
  int32_t deterministic;
  // Bounded waits inside a decode block (a wave waiting for another wave of
  // the block) poll at most wait_limit times; one that gives up ORs
  // kStatusWaitGaveUp into *status, which the host reports at its next
  // synchronising call.
  int32_t wait_limit;
  uint32_t *status;
  // 1: the history is kept in BF16 (OSCAR_POOL_BF16_HISTORY): a page block
  // is K bf16 [64][d] then V bf16 [64][d], tokens copied, not encoded.
  int32_t bf16_hist;
  // 1: the Lloyd-Max codebook variant (OSCAR_POOL_LLOYD_MAX): a history value
  // is z + (L[code] / 64) s; codebook[kind * Hkv + kv] holds L_0..L_3 of kv
  // head kv, K (kind 0) or V (kind 1), one byte each, L_0 in the low byte.
  // A channel takes the nearest level: u = (y - z) / s against the
  // midpoints (L_k + L_{k+1}) / 128, a midpoint itself taking the lower.
  int32_t lut;
  const uint32_t *codebook;
};

// Code of a clipped rotated value y under codebook dword lw (see lut above).
__host__ __device__ inline uint32_t lut_code(float y, float z, float s, uint32_t lw) {
  if (s == 0.0f) return 0u;
  const float u = (y - z) / s;
  uint32_t c = 0;
  for (int k = 0; k < 3; ++k) {
    const float t = (float)(((lw >> (8 * k)) & 255u) + ((lw >> (8 * k + 8)) & 255u)) / 128.0f;
    c += u > t ? 1u : 0u;
  }
  return c;
}

constexpr uint32_t kStatusWaitGaveUp = 1u;
constexpr int32_t kDefaultWaitLimit = 1 << 22;

// ---------------------------------------------------------------------------
// History page layout.  One page holds 64 consecutive history tokens of one
// sequence for every kv head; the (page, head) block is contiguous:
//
//   [K codes 16d B][V codes 16d B][K params 256 d/G B][V params 256 d/G B]
//
// Code bytes are ordered so that the lanes of a wave read them with
// contiguous 16-byte loads: the code region is a sequence of 1 KB chunks,
// chunk i holding bytes 16 i .. 16 i + 15 of every lane's share, lane l at
// byte 16 l of the chunk (lane l = 16 r + n).
//
// K codes (16d bytes from 0): lane (n, r) owns tokens 4n .. 4n+3 of channel
// quarter r; its share is token-major, d/16 bytes per token.  The 16
// channels {64m + 16r + k : k < 16} of token t form one little-endian dword
// (channel 64m+16r+k in bits 2k..2k+1) at lane-share byte
// b = (t % 4) * (d/16) + 4m of lane (t / 4, r).
//
// V codes (16d bytes from 16d): lane (n, r) owns the 16 tokens
// {16 r + k : k < 16} (a "token block") of the channels {16 j + n}; the
// dword of channel c = 16 j + n sits at lane-share byte b = 4j.  Inside the
// dword, token k sits at bit vbit(k) = 16 (k & 1) + 2 (k >> 1): even tokens
// fill the low half, odd tokens the high half, so one AND with
// 0x00030003 << 2i yields tokens (2i, 2i+1) as a pair of fp16 sub-normals.
//
// Params: fp16 (scale, zero) of token t, group g at byte
//      32d + 4 (t * d/G + g)               (K)
//      32d + 256 d/G + 4 (t * d/G + g)     (V)
// ---------------------------------------------------------------------------
__host__ __device__ inline int block_bytes_for(int d, int G) { return 32 * d + 512 * d / G; }
// (page, head) block of a BF16-history pool: K and V, 64 tokens x d bf16 each
__host__ __device__ inline int bf16_block_bytes(int d) { return 4 * kPage * d; }
__host__ __device__ inline int lane_share_off(int lane, int b) { return (b / 16) * 1024 + lane * 16 + b % 16; }
__host__ __device__ inline int kcode_dword_off(int d, int t, int r, int m) {
  return lane_share_off(16 * r + t / 4, (t % 4) * (d / 16) + 4 * m);
}
__host__ __device__ inline int vcode_dword_off(int d, int tb, int c) {
  return 16 * d + lane_share_off(16 * tb + c % 16, 4 * (c / 16));
}
__host__ __device__ inline int vbit(int k) { return 16 * (k & 1) + 2 * (k >> 1); }
__host__ __device__ inline int kparam_off(int d, int G, int t, int g) {
  return 32 * d + 4 * (t * (d / G) + g);
}
__host__ __device__ inline int vparam_off(int d, int G, int t, int g) {
  return 32 * d + 256 * d / G + 4 * (t * (d / G) + g);
}

// By-value metadata of one append launch (<= kMaxBatch sequences).
// new_page: the page the evicted token goes to when it is not the one the
// page table holds at its index (a fresh page when the token starts one, or
// the copy-on-write page of a shared last page), else -1; the launch writes
// it into the page table.
struct AppendBatch {
  int32_t n;
  int32_t seq[kMaxBatch];
  int32_t len[kMaxBatch];      // length before the append
  int32_t new_page[kMaxBatch];
};

// Copy-on-write copies of one launch: page src[i] to page dst[i], the
// blocks of every kv head.
struct PageCopies {
  int32_t n;
  int32_t src[kMaxBatch];
  int32_t dst[kMaxBatch];
};

// By-value metadata of one decode launch (<= kMaxBatch sequences).  The
// work of a (sequence, kv head) pair is its np history pages plus its BF16
// window, counted as win_units pages; it is cut into nsplit splits of about
// equal work (split_range), the window going to the last split, one block
// per split.  Sequences are ordered by nsplit, descending, and blocks are
// numbered split-major: block = layer_prefix[s] + e * Hkv + kv for split
// s < nsplit[e].
constexpr int kMaxSplits = 32;
constexpr int kIdCache = 1024; // page ids staged in shared memory per segment
struct DecodeBatch {
  int32_t n;
  int32_t hist_blocks;               // blocks of the launch: layer_prefix[kMaxSplits]
  int32_t total_pages;               // history pages of the batch
  int32_t win_units;                 // window work in page units (>= 0)
  int32_t seq[kMaxBatch];            // pool sequence id, launch order
  int32_t len[kMaxBatch];            // its length
  uint16_t row[kMaxBatch];           // its row in q and out
  uint8_t nsplit[kMaxBatch];         // blocks per pair, 1 .. kMaxSplits
  int32_t layer_prefix[kMaxSplits + 1];
  // Fused step (oscar_decode_step): the launch first appends one token per
  // sequence (len is the length after it).  new_page: as in AppendBatch
  // (launch order).
  int32_t fused;
  // Every pair of the launch has one split: its block writes the output
  // rows itself and no merge launch follows (INT2 decode only).
  int32_t direct;
  int32_t new_page[kMaxBatch];
};

// History tokens (from the start of the history) visible to a prefill
// query at position pos: those at positions 64 .. pos.
__host__ __device__ inline int prefill_visible_hist(int pos, int n_hist) {
  const int h = pos + 1 - kSink;
  return h < 0 ? 0 : (h > n_hist ? n_hist : h);
}

// the kernels read row[] and nsplit[] through whole dwords
static_assert(offsetof(DecodeBatch, row) % 4 == 0 && offsetof(DecodeBatch, nsplit) % 4 == 0,
              "row and nsplit must start at 4-byte offsets");

// History pages [p0, p1) of split s of S of a pair with np pages: the pair's
// units [0, np + wu) are cut evenly, pages are units below np.  Only the last
// split can be left without pages when S <= (np + wu) / max(wu, 1).
__host__ __device__ inline void split_range(int np, int S, int s, int wu, int &p0, int &p1) {
  const long U = (long)np + wu;
  p0 = (int)(s * U / S);
  p1 = (int)((s + 1) * U / S);
  p0 = p0 < np ? p0 : np;
  p1 = p1 < np ? p1 : np;
}

// Split layer s, sequence e (launch order) and kv head of decode block blk:
// s is the largest layer with layer_prefix[s] <= blk.  layer_prefix does not
// decrease, so s counts the entries 1..kMaxSplits at or below blk; every
// entry is read at a fixed offset (on the device: one round of scalar loads
// rather than a dependent chain).
__host__ __device__ inline void block_split(const DecodeBatch &b, int Hkv, int blk, int &s, int &e, int &kv) {
  s = 0;
  int base = 0; // layer_prefix[s]
#pragma unroll
  for (int i = 1; i <= kMaxSplits; ++i) {
    const int v = b.layer_prefix[i];
    s += v <= blk ? 1 : 0;
    base = v <= blk ? v : base;
  }
  const int pos = blk - base;
  e = pos / Hkv;
  kv = pos % Hkv;
}

// End of the full pages of a split's page range [p0, p1) of a pair with
// n_hist history tokens: only the sequence's last page can be partial.  The
// partial page, if the split holds it, is page pf (pf < p1, pf = np - 1).
// An empty range gives p0.
__host__ __device__ inline int full_pages_end(int n_hist, int p0, int p1) {
  if (p0 >= p1) return p0;
  const int np = (n_hist + kPage - 1) / kPage; // n_hist > 0: the range is not empty
  const int last = np - 1;
  return (n_hist % kPage == 0 || p1 < np) ? p1 : (last > p0 ? last : p0);
}

// Optional per-kernel timing: when `on`, a launch wrapper records ev[0]
// before and ev[1] after the kernel on its stream.
struct KernelTimer {
  bool on = false;
  hipEvent_t ev[2];
};

hipError_t launch_prefill(const PoolDev &p, int seq, const uint16_t *k, const uint16_t *v,
                          int L, hipStream_t s);
hipError_t launch_append(const PoolDev &p, const AppendBatch &b, const uint16_t *k_new,
                         const uint16_t *v_new, hipStream_t s, const KernelTimer &t);
// Copy-on-write page copies (every kv head of each page).
hipError_t launch_copy_pages(const PoolDev &p, const PageCopies &c, hipStream_t s);
// Fork: sequence src's window (sink and recent ring, all kv heads) and the
// first np entries of its page-table row, copied to sequence dst.
hipError_t launch_fork(const PoolDev &p, int src, int dst, int np, hipStream_t s);
// History entries [0, n_hist) of a sequence in the canonical layout, device
// to device (codes 4-byte aligned: d/4 is a multiple of 4).
hipError_t launch_export(const PoolDev &p, int seq, int n_hist, uint8_t *codes, uint16_t *params, hipStream_t s);
// BF16-history pools: resident decode blocks per compute unit, the history
// launch (partials in the decode workspace layout) and the merge launch.
int bf16_decode_blocks_per_cu(const PoolDev &p);
hipError_t launch_decode_bf16(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float scale, float *ws,
                              hipStream_t s, const KernelTimer &t);
hipError_t launch_decode_merge(const PoolDev &p, const DecodeBatch &b, float *out, const float *ws, hipStream_t s,
                               const KernelTimer &t);
// Resident decode_main blocks per compute unit for this pool's shape.
int decode_main_blocks_per_cu(const PoolDev &p);

// Prefill attention on matrix cores (INT2-history pools, d 64 or 128, one or
// two scale groups per head row, affine or codebook levels): the call's flat rows (query i, head hh of the kv
// head; index i g + hh) are cut in tiles of kPfTileRows, and each tile's
// visible history pages in S splits.
constexpr int kPfTileRows = 128;
struct PrefillArgs {
  int32_t seq, L, n_q, g, n_hist;
  int32_t NT, S;   // tiles per kv head, splits per tile
  float qscale;    // softmax scale * log2(e)
};
// Splits per tile: about 512 (tile, split) pairs per launch, at most 16
// splits; the history kernel takes two tiles per block, so about 256 blocks
// (one per compute unit).
inline int prefill_mfma_splits(int NT, int Hkv) {
  const int tiles = NT * Hkv, want = (512 + tiles - 1) / tiles;
  return want < 1 ? 1 : (want > 16 ? 16 : want);
}
bool prefill_mfma_supported(const PoolDev &p);
size_t prefill_mfma_ws_bytes(int Hkv, int NT, int S, int d);
hipError_t launch_prefill_mfma(const PoolDev &p, const PrefillArgs &a, const uint16_t *q, float *out, void *ws,
                               hipStream_t s);

// k_new, v_new: the appended tokens of a fused step (b.fused), else null.
hipError_t launch_decode(const PoolDev &p, const DecodeBatch &b, const uint16_t *q, float *out,
                         float scale, float *ws, const uint16_t *k_new, const uint16_t *v_new, hipStream_t s,
                         const KernelTimer &t_main, const KernelTimer &t_merge);


// Calibration: O = causal softmax(scale Q K^T) V per query head (fp32
// [n][Hq][d]); then cov_k[h] += sum of Q^T Q and cov_v[h] += sum of O^T O over
// kv head h's query heads (either output may be null).
hipError_t launch_calib_attn(int n, int Hq, int Hkv, int d, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             float scale, float *o, hipStream_t s);
hipError_t launch_calib_gram(int n, int Hq, int Hkv, int d, const uint16_t *q, const float *o, float *cov_k,
                             float *cov_v, hipStream_t s);

// Workspace (4-byte words) of one decode launch: window partials
// [n][Hq][d + 2], then split partials [n][Hkv][smax][g][d + 2], smax the
// launch's largest split count (slot s of a pair holds its split s).
inline size_t decode_ws_floats(int Hq, int d, int n, int Hkv, int smax, int g) {
  return (size_t)n * Hq * (d + 2) + (size_t)n * Hkv * smax * g * (d + 2);
}

// Device address and size of the library's static decode workspace on the
// current device (oscar_decode_step_static).  The address is looked up once
// per device and kept; later calls only read it.
hipError_t static_scratch(void **ptr, size_t *bytes);

} // namespace oscar
