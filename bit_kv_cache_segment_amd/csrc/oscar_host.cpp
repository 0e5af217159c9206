// Host side of the OSCAR pool library: configuration and layout, argument
// validation, the host mirror of lengths / page tables / free list, the
// offline helpers (rotation construction, clip calibration) and the C ABI.
//
// Method source: news article on OSCAR (sanyangsrq.com), sections
// "OSCAR aims the rotation at attention" (R = U . Hadamard . bit-reversal,
// thresholds fixed offline) and "From offline calibration to online
// inference" (three-segment pool, eviction of the oldest recent token,
// paged layout).
#include "../../include/oscar.h"
#include "oscar_internal.h"
#include "decode_plan.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

using namespace oscar;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return OSCAR_OK;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(OSCAR_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t RK, RV, RVt, clipK, clipV, status, codebook, page_table, sinkK, sinkV, recentK, recentV, pages, total;
};

int validate_config(const oscar_pool_config *c) {
  if (!c) return fail(OSCAR_EINVAL, "config is NULL");
  if (c->max_seqs < 1 || c->max_seqs > 65536)
    return fail(OSCAR_EINVAL, "max_seqs %d outside [1, 65536]", c->max_seqs);
  if (c->num_kv_heads < 1 || c->num_kv_heads > 64)
    return fail(OSCAR_EINVAL, "num_kv_heads %d outside [1, 64]", c->num_kv_heads);
  if (c->num_q_heads < 1 || c->num_q_heads % c->num_kv_heads != 0)
    return fail(OSCAR_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                c->num_q_heads, c->num_kv_heads);
  int g = c->num_q_heads / c->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
    return fail(OSCAR_EINVAL, "query heads per kv head (%d) must be 1, 2, 4, 8 or 16", g);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(OSCAR_EINVAL, "head_dim %d must be 64 or 128", c->head_dim);
  if ((c->group_size != 64 && c->group_size != 128) || c->group_size > c->head_dim)
    return fail(OSCAR_EINVAL, "group_size %d must be 64 or 128 and <= head_dim", c->group_size);
  if (c->num_pages < 0 || c->num_pages > (1 << 28))
    return fail(OSCAR_EINVAL, "num_pages %d outside [0, 2^28]", c->num_pages);
  if (c->max_pages_per_seq < 0 || c->max_pages_per_seq > (1 << 20))
    return fail(OSCAR_EINVAL, "max_pages_per_seq %d outside [0, 2^20]", c->max_pages_per_seq);
  if ((int64_t)c->max_seqs * c->max_pages_per_seq > (int64_t)1 << 31)
    return fail(OSCAR_EINVAL, "page table of %d x %d entries is too large", c->max_seqs,
                c->max_pages_per_seq);
  if (c->flags & ~(OSCAR_POOL_HOST_ONLY | OSCAR_POOL_DETERMINISTIC | OSCAR_POOL_BF16_HISTORY | OSCAR_POOL_LLOYD_MAX))
    return fail(OSCAR_EINVAL, "unknown flags 0x%x", c->flags);
  if ((c->flags & OSCAR_POOL_BF16_HISTORY) && (c->flags & OSCAR_POOL_LLOYD_MAX))
    return fail(OSCAR_EINVAL, "a BF16 history has no codebook: OSCAR_POOL_LLOYD_MAX excludes OSCAR_POOL_BF16_HISTORY");
  return OSCAR_OK;
}

Layout layout_of(const oscar_pool_config &c) {
  Layout L;
  size_t d = c.head_dim, H = c.num_kv_heads, S = c.max_seqs;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.RK = take(H * d * d * 4);
  L.RV = take(H * d * d * 4);
  L.RVt = take(H * d * d * 4);
  L.clipK = take(H * d * 4);
  L.clipV = take(H * d * 4);
  L.status = take(4);
  L.codebook = take(2 * H * 4);
  L.page_table = take(S * (size_t)c.max_pages_per_seq * 4);
  L.sinkK = take(S * H * kSink * d * 2);
  L.sinkV = take(S * H * kSink * d * 2);
  L.recentK = take(S * H * kRecent * d * 2);
  L.recentV = take(S * H * kRecent * d * 2);
  L.pages = take((size_t)c.num_pages * H *
                 ((c.flags & OSCAR_POOL_BF16_HISTORY) ? bf16_block_bytes(c.head_dim)
                                                      : block_bytes_for(c.head_dim, c.group_size)));
  L.total = off;
  return L;
}

int pages_for(int64_t n_hist) { return (int)((n_hist + kPage - 1) / kPage); }

} // namespace

// ---------------------------------------------------------------------------
// Static decode workspace, for callers that cannot allocate device memory
// (oscar_decode_step_static): the same partials a caller's workspace holds,
// in a file-scope device array of kStaticScratchBytes on every GPU the
// library runs on, kept until the process ends.  Host code never uses the
// array's name as an address: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and is
// kept per device.  Every call on a GPU shares that GPU's array, so calls
// that overlap on one GPU (on different streams) race; calls on one stream
// are ordered.  Nothing in it needs clearing: each launch writes every
// partial it reads.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

hipError_t oscar::static_scratch(void **ptr, size_t *bytes) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

// Event pairs for per-kernel timing (oscar_profile_begin / _end).
struct Profiler {
  bool on = false;
  int cap = 0, every = 1;
  uint32_t mask = 0;
  std::vector<hipEvent_t> ev[3]; // decode main, decode merge, append: 2 per launch
  int used[3] = {0, 0, 0};
  long calls[3] = {0, 0, 0};
  KernelTimer next(int kind) {
    KernelTimer t;
    if (on && (mask >> kind & 1u) && calls[kind]++ % every == 0 && used[kind] < cap) {
      t.on = true;
      t.ev[0] = ev[kind][2 * used[kind]];
      t.ev[1] = ev[kind][2 * used[kind] + 1];
      ++used[kind];
    }
    return t;
  }
  void release() {
    for (auto &v : ev) {
      for (hipEvent_t e : v) (void)hipEventDestroy(e);
      v.clear();
    }
    on = false;
    cap = 0;
    every = 1;
    used[0] = used[1] = used[2] = 0;
    calls[0] = calls[1] = calls[2] = 0;
  }
};

struct oscar_pool {
  Profiler prof;
  ~oscar_pool() { prof.release(); }
  oscar_pool_config cfg;
  Layout lay;
  PoolDev dev;
  bool host_only;
  // Lloyd-Max pools: the codebook (uint32 per kv head, K then V), once set
  std::vector<uint32_t> codebook;
  int decode_slots = 768; // resident decode blocks on the device
  std::vector<int32_t> len;
  std::vector<std::vector<int32_t>> table;
  std::vector<int32_t> free_list; // pages [free_head, end) are free, front first
  size_t free_head = 0;
  // Page tables holding each page (prefix sharing); 0 for a free page.
  std::vector<int32_t> refs;

  int64_t n_free() const { return (int64_t)free_list.size() - (int64_t)free_head; }
  int32_t pop() { return free_list[free_head++]; }
  void compact() {
    if (free_head > 4096 && free_head * 2 > free_list.size()) {
      free_list.erase(free_list.begin(), free_list.begin() + free_head);
      free_head = 0;
    }
  }
};

// The pool's device status word, read once the work enqueued so far has
// completed (the caller has synchronised): EHIP if a bounded wait inside a
// decode block gave up, which leaves that step's results, and possibly the
// evicted token's codes, undefined.  The word is sticky.
static int check_device_status(oscar_pool *p) {
  if (p->host_only) return OSCAR_OK;
  uint32_t st = 0;
  hipError_t e = hipMemcpy(&st, p->dev.status, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the pool status");
  if (st & kStatusWaitGaveUp)
    return fail(OSCAR_EHIP, "a bounded wait inside a decode step gave up (status 0x%x): the results of the "
                "steps since the pool was created may be wrong", st);
  return OSCAR_OK;
}

extern "C" {

const char *oscar_last_error(void) { return g_err.c_str(); }

int oscar_pool_bytes(const oscar_pool_config *cfg, size_t *device_bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!device_bytes) return fail(OSCAR_EINVAL, "device_bytes is NULL");
  *device_bytes = layout_of(*cfg).total;
  return ok();
}

int oscar_pool_required_bytes(const oscar_pool_config *cfg, size_t *device_bytes, size_t *workspace_bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!device_bytes || !workspace_bytes) return fail(OSCAR_EINVAL, "NULL output");
  size_t ws = 0;
  rc = oscar_decode_workspace_bytes(cfg, std::min(cfg->max_seqs, kMaxBatch), &ws);
  if (rc) return rc;
  *device_bytes = layout_of(*cfg).total;
  *workspace_bytes = ws;
  return ok();
}

int oscar_decode_workspace_bytes(const oscar_pool_config *cfg, int32_t max_batch, size_t *bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!bytes || max_batch < 0) return fail(OSCAR_EINVAL, "bad arguments");
  int n = std::min(max_batch, kMaxBatch);
  int g = cfg->num_q_heads / cfg->num_kv_heads;
  *bytes = decode_ws_floats(cfg->num_q_heads, cfg->head_dim, n, cfg->num_kv_heads, kMaxSplits, g) * sizeof(float);
  return ok();
}

int oscar_pool_create(const oscar_pool_config *cfg, void *device_buf, size_t bytes, const float *R_K,
                      const float *R_V, const float *clip_K, const float *clip_V, void *stream,
                      oscar_pool **out) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!out) return fail(OSCAR_EINVAL, "out is NULL");
  bool host_only = cfg->flags & OSCAR_POOL_HOST_ONLY;
  Layout lay = layout_of(*cfg);
  const int H = cfg->num_kv_heads, d = cfg->head_dim;
  if (!host_only) {
    if (!device_buf || !R_K || !R_V || !clip_K || !clip_V)
      return fail(OSCAR_EINVAL, "NULL buffer or table");
    if ((uintptr_t)device_buf % 256) return fail(OSCAR_EINVAL, "device_buf is not 256-byte aligned");
    if (bytes < lay.total)
      return fail(OSCAR_EINVAL, "device buffer of %zu bytes < %zu required", bytes, lay.total);
    for (size_t i = 0; i < (size_t)H * d * d; ++i)
      if (!std::isfinite(R_K[i]) || !std::isfinite(R_V[i]))
        return fail(OSCAR_EINVAL, "rotation entry %zu is not finite", i);
    for (size_t i = 0; i < (size_t)H * d; ++i) {
      float ck = clip_K[i], cv = clip_V[i];
      // clipped values lie in [-c, c]: the zero point fp16(min) and the scale
      // fp16((max - min) / 3) <= fp16(2c/3) stay finite for c <= 65504.
      if (!(ck > 0.f && ck <= 65504.f) || !(cv > 0.f && cv <= 65504.f))
        return fail(OSCAR_EINVAL, "clip threshold %zu (%g, %g) outside (0, 65504]", i, ck, cv);
    }
  }
  oscar_pool *p = new oscar_pool();
  p->cfg = *cfg;
  p->lay = lay;
  p->host_only = host_only;
  p->len.assign(cfg->max_seqs, 0);
  p->table.assign(cfg->max_seqs, {});
  p->refs.assign(cfg->num_pages, 0);
  // Free list: Fisher-Yates shuffle of [0, num_pages) driven by SplitMix64.
  p->free_list.resize(cfg->num_pages);
  for (int i = 0; i < cfg->num_pages; ++i) p->free_list[i] = i;
  uint64_t state = cfg->page_shuffle_seed;
  auto next = [&state]() {
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  };
  for (int i = cfg->num_pages - 1; i > 0; --i) {
    uint64_t j = next() % (uint64_t)(i + 1);
    std::swap(p->free_list[i], p->free_list[j]);
  }
  PoolDev &D = p->dev;
  std::memset(&D, 0, sizeof D);
  D.Hq = cfg->num_q_heads;
  D.Hkv = H;
  D.d = d;
  D.G = cfg->group_size;
  D.maxp = cfg->max_pages_per_seq;
  D.bf16_hist = (cfg->flags & OSCAR_POOL_BF16_HISTORY) ? 1 : 0;
  D.lut = (cfg->flags & OSCAR_POOL_LLOYD_MAX) ? 1 : 0;
  D.block_bytes = D.bf16_hist ? bf16_block_bytes(d) : block_bytes_for(d, cfg->group_size);
  D.pv_shift = 0;
  D.deterministic = (cfg->flags & OSCAR_POOL_DETERMINISTIC) ? 1 : 0;
  // Polls of a bounded wait inside a decode block before it gives up (and
  // reports it).  OSCAR_WAIT_SPIN_LIMIT overrides the default, so that a
  // test can force a give-up: 0 gives up at once.
  D.wait_limit = kDefaultWaitLimit;
  if (const char *env = std::getenv("OSCAR_WAIT_SPIN_LIMIT")) {
    char *end = nullptr;
    const long v = std::strtol(env, &end, 10);
    if (end != env && v >= 0 && v <= (1L << 30)) D.wait_limit = (int32_t)v;
  }
  if (!host_only) {
    // V scales never exceed fp16(2 c / 3) for the largest V threshold c and
    // the decode's softmax weights never exceed 2^8 (its lazy max); keep
    // weight * scale * 2^pv_shift below 65504 with a margin for fp16 rounding.
    float cmax = 0.f;
    for (size_t i = 0; i < (size_t)H * d; ++i) cmax = std::max(cmax, clip_V[i]);
    double smax = 2.0 * cmax / 3.0 * 1.002;
    int sh = (int)std::floor(std::log2(65504.0 / smax)) - 8;
    D.pv_shift = std::max(-30, std::min(sh, 60));
  }
  if (!host_only) {
    char *b = (char *)device_buf;
    D.RK = (const float *)(b + lay.RK);
    D.RV = (const float *)(b + lay.RV);
    D.RVt = (const float *)(b + lay.RVt);
    D.clipK = (const float *)(b + lay.clipK);
    D.clipV = (const float *)(b + lay.clipV);
    D.page_table = (int32_t *)(b + lay.page_table);
    D.sinkK = (uint16_t *)(b + lay.sinkK);
    D.sinkV = (uint16_t *)(b + lay.sinkV);
    D.recentK = (uint16_t *)(b + lay.recentK);
    D.recentV = (uint16_t *)(b + lay.recentV);
    D.pages = (uint8_t *)(b + lay.pages);
    D.status = (uint32_t *)(b + lay.status);
    D.codebook = (const uint32_t *)(b + lay.codebook);
    std::vector<float> rvt((size_t)H * d * d);
    for (int h = 0; h < H; ++h)
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j)
          rvt[((size_t)h * d + j) * d + i] = R_V[((size_t)h * d + i) * d + j];
    hipStream_t s = (hipStream_t)stream;
    size_t rb = (size_t)H * d * d * 4, cb = (size_t)H * d * 4;
    hipError_t e = hipMemcpyAsync((void *)D.RK, R_K, rb, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync((void *)D.RV, R_V, rb, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync((void *)D.RVt, rvt.data(), rb, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync((void *)D.clipK, clip_K, cb, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync((void *)D.clipV, clip_V, cb, hipMemcpyHostToDevice, s);
    static const uint32_t zero = 0;
    if (e == hipSuccess) e = hipMemcpyAsync((void *)D.status, &zero, 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "copying rotation/clip tables");
    }
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int per_cu = D.bf16_hist ? bf16_decode_blocks_per_cu(D) : decode_main_blocks_per_cu(D);
    if (e != hipSuccess || cus <= 0 || per_cu <= 0) {
      delete p;
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidValue, "querying the decode occupancy");
    }
    p->decode_slots = cus * per_cu;
    // set-up of the static decode workspace on this device (its address is
    // looked up here, once per device, not in the step that uses it)
    void *ws = nullptr;
    size_t ws_bytes = 0;
    e = static_scratch(&ws, &ws_bytes);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "static decode workspace");
    }
  }
  *out = p;
  return ok();
}

int oscar_pool_destroy(oscar_pool *pool) {
  if (!pool) return fail(OSCAR_EINVAL, "pool is NULL");
  delete pool;
  return ok();
}

static int check_seq(const oscar_pool *p, int32_t seq) {
  if (!p) return fail(OSCAR_EINVAL, "pool is NULL");
  if (seq < 0 || seq >= p->cfg.max_seqs)
    return fail(OSCAR_EINVAL, "sequence id %d outside [0, %d)", seq, p->cfg.max_seqs);
  return OSCAR_OK;
}

int oscar_prefill(oscar_pool *p, int32_t seq, const uint16_t *k, const uint16_t *v, int32_t L,
                  void *stream) {
  int rc = check_seq(p, seq);
  if (rc) return rc;
  if (p->len[seq] != 0 || !p->table[seq].empty())
    return fail(OSCAR_EINVAL, "sequence %d is not empty", seq);
  if (L < 0 || L > (1 << 30)) return fail(OSCAR_EINVAL, "prompt length %d is invalid", L);
  if (p->dev.lut && p->codebook.empty())
    return fail(OSCAR_EINVAL, "a Lloyd-Max pool needs its codebook (oscar_pool_set_codebook) first");
  if (L == 0) return ok();
  if (!p->host_only && (!k || !v)) return fail(OSCAR_EINVAL, "NULL k or v");
  int64_t n_hist = std::max(0, L - kWindow);
  int np = pages_for(n_hist);
  if (np > p->cfg.max_pages_per_seq)
    return fail(OSCAR_ERANGE, "sequence %d needs %d pages > max_pages_per_seq %d", seq, np,
                p->cfg.max_pages_per_seq);
  if (np > p->n_free())
    return fail(OSCAR_ENOMEM, "sequence %d needs %d pages, %lld free", seq, np,
                (long long)p->n_free());
  std::vector<int32_t> row(np);
  size_t head0 = p->free_head;
  for (int i = 0; i < np; ++i) row[i] = p->pop();
  if (!p->host_only) {
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (np)
      e = hipMemcpyAsync(p->dev.page_table + (size_t)seq * p->cfg.max_pages_per_seq, row.data(),
                         np * sizeof(int32_t), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = launch_prefill(p->dev, seq, k, v, L, s);
    if (e == hipSuccess && np) e = hipStreamSynchronize(s); // `row` is released on return
    if (e != hipSuccess) {
      p->free_head = head0;
      return hip_fail(e, "prefill");
    }
  }
  for (int32_t pg : row) p->refs[pg] = 1;
  p->table[seq] = std::move(row);
  p->len[seq] = L;
  return ok();
}

// Pages an append of one token to each of seq_ids[0..n) needs, in seq_ids
// order: a fresh page where the evicted token starts one; a page of its own
// where the token lands in a history page that another sequence also holds
// (copy on write: it copies that page first), counting the references the
// call's earlier copies have dropped.  With `a`, the pages are popped from
// the free list (a->taken[i], or -1) and a->cow[i] names the page copied
// (or -1); reference counts change only in commit_append.
struct AppendPages {
  std::vector<int32_t> taken, cow;
};

static int64_t append_pages(oscar_pool *p, const int32_t *seq_ids, int32_t n, AppendPages *a) {
  if (a) {
    a->taken.assign(n, -1);
    a->cow.assign(n, -1);
  }
  std::unordered_map<int32_t, int32_t> dropped;
  int64_t need = 0;
  for (int i = 0; i < n; ++i) {
    const int32_t s = seq_ids[i], L = p->len[s];
    if (L < kWindow) continue;
    const int32_t n_hist = L - kWindow;
    int32_t cow = -1;
    if (n_hist % kPage != 0) {
      const int32_t pg = p->table[s][n_hist / kPage];
      if (p->refs[pg] > 1) {
        int32_t &dr = dropped[pg];
        if (p->refs[pg] - dr > 1) {
          ++dr;
          cow = pg;
        }
      }
      if (cow < 0) continue;
    }
    ++need;
    if (a) {
      a->taken[i] = p->pop();
      a->cow[i] = cow;
    }
  }
  return need;
}

// The host mirror of sequence seq_ids[i]'s append once it is enqueued.
static void commit_append(oscar_pool *p, int32_t s, int32_t taken, int32_t cow) {
  if (taken >= 0) {
    if (cow >= 0) {
      --p->refs[cow];
      p->table[s].back() = taken; // the shared page was the history's last
    } else {
      p->table[s].push_back(taken);
    }
    p->refs[taken] = 1;
  }
  p->len[s] += 1;
}

// Enqueues the copies of the call's copy-on-write pages (before its
// appends).  A failure leaves nothing to undo: the copies only write pages
// that are still free.
static hipError_t launch_cows(oscar_pool *p, const AppendPages &a, hipStream_t stream) {
  PageCopies c;
  c.n = 0;
  for (size_t i = 0; i < a.cow.size(); ++i) {
    if (a.cow[i] < 0) continue;
    c.src[c.n] = a.cow[i];
    c.dst[c.n] = a.taken[i];
    if (++c.n == kMaxBatch) {
      hipError_t e = launch_copy_pages(p->dev, c, stream);
      if (e != hipSuccess) return e;
      c.n = 0;
    }
  }
  return launch_copy_pages(p->dev, c, stream);
}

// After a failed launch of batch `done` (earlier batches are in flight):
// keep the mirror of sequences [0, done * kMaxBatch) and return the pages
// popped for the rest, which were popped after theirs.
static void commit_prefix(oscar_pool *p, const int32_t *seq_ids, const AppendPages &a, size_t head0,
                          size_t done) {
  size_t kept = 0;
  const size_t m = std::min(done * (size_t)kMaxBatch, a.taken.size());
  for (size_t j = 0; j < m; ++j) {
    if (a.taken[j] >= 0) ++kept;
    commit_append(p, seq_ids[j], a.taken[j], a.cow[j]);
  }
  p->free_head = head0 + kept;
}

// Checks of an append of one token to each of seq_ids[0..n) (n > 0): ids
// valid and distinct, lengths below the limit, page-table room, and free
// pages for every eviction that starts a page or copies a shared one.
// Changes nothing.
static int check_append(oscar_pool *p, const int32_t *seq_ids, int32_t n) {
  if (p->dev.lut && p->codebook.empty())
    return fail(OSCAR_EINVAL, "a Lloyd-Max pool needs its codebook (oscar_pool_set_codebook) first");
  std::vector<int32_t> sorted(seq_ids, seq_ids + n);
  std::sort(sorted.begin(), sorted.end());
  for (int i = 0; i < n; ++i) {
    int rc = check_seq(p, sorted[i]);
    if (rc) return rc;
    if (i && sorted[i] == sorted[i - 1])
      return fail(OSCAR_EINVAL, "sequence id %d repeated in one append", sorted[i]);
  }
  for (int i = 0; i < n; ++i) {
    int32_t s = seq_ids[i], L = p->len[s];
    if (L >= (1 << 30)) return fail(OSCAR_ERANGE, "sequence %d is at the length limit", s);
    if (L >= kWindow && (L - kWindow) % kPage == 0) {
      int np = (L - kWindow) / kPage + 1;
      if (np > p->cfg.max_pages_per_seq)
        return fail(OSCAR_ERANGE, "sequence %d would need %d pages > max_pages_per_seq %d", s, np,
                    p->cfg.max_pages_per_seq);
    }
  }
  const int64_t need = append_pages(p, seq_ids, n, nullptr);
  if (need > p->n_free())
    return fail(OSCAR_ENOMEM, "append needs %lld new pages, %lld free", (long long)need,
                (long long)p->n_free());
  return OSCAR_OK;
}

int oscar_append_evict(oscar_pool *p, const int32_t *seq_ids, int32_t n, const uint16_t *k_new,
                       const uint16_t *v_new, void *stream) {
  if (!p) return fail(OSCAR_EINVAL, "pool is NULL");
  if (n < 0) return fail(OSCAR_EINVAL, "n = %d < 0", n);
  if (n == 0) return ok();
  if (!seq_ids) return fail(OSCAR_EINVAL, "seq_ids is NULL");
  if (!p->host_only && (!k_new || !v_new)) return fail(OSCAR_EINVAL, "NULL k_new or v_new");
  {
    int rc = check_append(p, seq_ids, n);
    if (rc) return rc;
  }
  // Take the pages in seq_ids order, then build the launches.
  const size_t head0 = p->free_head;
  AppendPages a;
  append_pages(p, seq_ids, n, &a);
  std::vector<AppendBatch> batches;
  for (int i0 = 0; i0 < n; i0 += kMaxBatch) {
    AppendBatch b;
    b.n = std::min(kMaxBatch, n - i0);
    for (int e = 0; e < b.n; ++e) {
      b.seq[e] = seq_ids[i0 + e];
      b.len[e] = p->len[b.seq[e]];
      b.new_page[e] = a.taken[i0 + e];
    }
    batches.push_back(b);
  }
  if (!p->host_only) {
    hipError_t e = launch_cows(p, a, (hipStream_t)stream);
    if (e != hipSuccess) {
      p->free_head = head0;
      return hip_fail(e, "copy-on-write launch");
    }
    for (size_t i = 0; i < batches.size(); ++i) {
      const AppendBatch &b = batches[i];
      e = launch_append(p->dev, b, k_new + (size_t)i * kMaxBatch * p->cfg.num_kv_heads * p->cfg.head_dim,
                        v_new + (size_t)i * kMaxBatch * p->cfg.num_kv_heads * p->cfg.head_dim,
                        (hipStream_t)stream, p->prof.next(2));
      if (e != hipSuccess) {
        commit_prefix(p, seq_ids, a, head0, i); // earlier launches are in flight
        return hip_fail(e, "append launch");
      }
    }
  }
  for (int i = 0; i < n; ++i) commit_append(p, seq_ids[i], a.taken[i], a.cow[i]);
  p->compact();
  return ok();
}

int oscar_decode_attn(oscar_pool *p, const int32_t *seq_ids, int32_t n, const uint16_t *q, float *out,
                      float softmax_scale, void *workspace, size_t workspace_bytes, void *stream) {
  if (!p) return fail(OSCAR_EINVAL, "pool is NULL");
  if (p->host_only) return fail(OSCAR_EINVAL, "decode on a host-only pool");
  if (n < 0) return fail(OSCAR_EINVAL, "n = %d < 0", n);
  if (n == 0) return ok();
  if (!seq_ids || !q || !out || !workspace) return fail(OSCAR_EINVAL, "NULL argument");
  if (!std::isfinite(softmax_scale)) return fail(OSCAR_EINVAL, "softmax_scale is not finite");
  for (int i = 0; i < n; ++i) {
    int rc = check_seq(p, seq_ids[i]);
    if (rc) return rc;
    if (p->len[seq_ids[i]] < 1) return fail(OSCAR_EINVAL, "sequence %d is empty", seq_ids[i]);
  }
  const int Hq = p->cfg.num_q_heads, Hkv = p->cfg.num_kv_heads, d = p->cfg.head_dim;
  const int g = Hq / Hkv;
  const bool bf16 = p->dev.bf16_hist != 0;
  std::vector<DecodeBatch> batches;
  size_t need = 0;
  for (int i0 = 0; i0 < n; i0 += kMaxBatch) {
    DecodeBatch b;
    b.n = std::min(kMaxBatch, n - i0);
    std::vector<int> len(b.n);
    for (int e = 0; e < b.n; ++e) len[e] = p->len[seq_ids[i0 + e]];
    plan_splits(b, seq_ids + i0, len, Hkv, p->decode_slots,
                bf16 ? window_units_bf16(d) : window_units(d, p->cfg.group_size));
    if (!bf16) set_direct(b);
    need = std::max(need, decode_ws_floats(Hq, d, b.n, Hkv, b.nsplit[0], g) * sizeof(float));
    batches.push_back(b);
  }
  if (workspace_bytes < need)
    return fail(OSCAR_EINVAL, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  for (size_t i = 0; i < batches.size(); ++i) {
    KernelTimer tm = p->prof.next(0), tg = batches[i].direct ? KernelTimer{} : p->prof.next(1);
    const uint16_t *qi = q + i * (size_t)kMaxBatch * Hq * d;
    float *oi = out + i * (size_t)kMaxBatch * Hq * d;
    hipError_t e;
    if (bf16) {
      e = launch_decode_bf16(p->dev, batches[i], qi, softmax_scale, (float *)workspace, (hipStream_t)stream, tm);
      if (e == hipSuccess)
        e = launch_decode_merge(p->dev, batches[i], oi, (const float *)workspace, (hipStream_t)stream, tg);
    } else {
      e = launch_decode(p->dev, batches[i], qi, oi, softmax_scale, (float *)workspace, nullptr, nullptr,
                        (hipStream_t)stream, tm, tg);
    }
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  return ok();
}

} // extern "C"

// The decode step with a given workspace: the caller's (oscar_decode_step)
// or the library's static one (oscar_decode_step_static, `fixed`).
static int decode_step(oscar_pool *p, const int32_t *seq_ids, int32_t n, const uint16_t *k_new,
                       const uint16_t *v_new, const uint16_t *q, float *out, float softmax_scale,
                       void *workspace, size_t workspace_bytes, void *stream, bool fixed) {
  if (!p) return fail(OSCAR_EINVAL, "pool is NULL");
  if (p->host_only) return fail(OSCAR_EINVAL, "decode step on a host-only pool");
  if (n < 0) return fail(OSCAR_EINVAL, "n = %d < 0", n);
  if (n == 0) return ok();
  if (!seq_ids || !k_new || !v_new || !q || !out || !workspace) return fail(OSCAR_EINVAL, "NULL argument");
  if (!std::isfinite(softmax_scale)) return fail(OSCAR_EINVAL, "softmax_scale is not finite");
  {
    int rc = check_append(p, seq_ids, n);
    if (rc) return rc;
  }
  const int Hq = p->cfg.num_q_heads, Hkv = p->cfg.num_kv_heads, d = p->cfg.head_dim;
  const int g = Hq / Hkv;
  // plan on the lengths after the append, then check the workspace: nothing
  // has changed yet.  The append runs inside the decode launch when every
  // block of it is resident at once; a launch that needs several rounds of
  // blocks would wait on the appending blocks round after round, so then
  // the append is its own launch (same results).
  std::vector<DecodeBatch> batches;
  size_t need = 0;
  // (BF16-history pools append in their own launch)
  bool fused = p->dev.bf16_hist == 0;
  for (int pass = fused ? 0 : 1; pass < 2; ++pass) {
    batches.clear();
    need = 0;
    for (int i0 = 0; i0 < n; i0 += kMaxBatch) {
      DecodeBatch b;
      b.n = std::min(kMaxBatch, n - i0);
      std::vector<int> len(b.n);
      for (int e = 0; e < b.n; ++e) len[e] = p->len[seq_ids[i0 + e]] + 1;
      plan_splits(b, seq_ids + i0, len, Hkv, p->decode_slots,
                  p->dev.bf16_hist ? window_units_bf16(d) : window_units(d, p->cfg.group_size, fused), fused);
      if (!p->dev.bf16_hist) set_direct(b);
      need = std::max(need, decode_ws_floats(Hq, d, b.n, Hkv, b.nsplit[0], g) * sizeof(float));
      if (b.hist_blocks > p->decode_slots) fused = false;
      batches.push_back(b);
    }
    if (fused || pass == 1) break;
  }
  if (workspace_bytes < need) {
    if (fixed)
      return fail(OSCAR_EINVAL, "this step needs %zu bytes of decode workspace, more than the %zu bytes of the "
                  "library's static workspace; use oscar_decode_step with a caller workspace", need, workspace_bytes);
    return fail(OSCAR_EINVAL, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  }
  if (!fused) {
    int rc = oscar_append_evict(p, seq_ids, n, k_new, v_new, stream);
    if (rc) return rc;
    return oscar_decode_attn(p, seq_ids, n, q, out, softmax_scale, workspace, workspace_bytes, stream);
  }
  // the append's pages, taken in seq_ids order, then placed in launch
  // order; copies on write first
  const size_t head0 = p->free_head;
  AppendPages a;
  append_pages(p, seq_ids, n, &a);
  for (size_t i = 0; i < batches.size(); ++i) {
    DecodeBatch &b = batches[i];
    for (int e = 0; e < b.n; ++e) b.new_page[e] = a.taken[i * kMaxBatch + b.row[e]];
  }
  {
    hipError_t e = launch_cows(p, a, (hipStream_t)stream);
    if (e != hipSuccess) {
      p->free_head = head0;
      return hip_fail(e, "copy-on-write launch");
    }
  }
  for (size_t i = 0; i < batches.size(); ++i) {
    const size_t r0 = i * (size_t)kMaxBatch;
    KernelTimer tm = p->prof.next(0), tg = batches[i].direct ? KernelTimer{} : p->prof.next(1);
    hipError_t e = launch_decode(p->dev, batches[i], q + r0 * Hq * d, out + r0 * Hq * d, softmax_scale,
                                 (float *)workspace, k_new + r0 * Hkv * d, v_new + r0 * Hkv * d,
                                 (hipStream_t)stream, tm, tg);
    if (e != hipSuccess) {
      commit_prefix(p, seq_ids, a, head0, i); // earlier launches are in flight
      return hip_fail(e, "decode step launch");
    }
  }
  for (int i = 0; i < n; ++i) commit_append(p, seq_ids[i], a.taken[i], a.cow[i]);
  p->compact();
  return ok();
}

extern "C" {

int oscar_decode_step(oscar_pool *p, const int32_t *seq_ids, int32_t n, const uint16_t *k_new,
                      const uint16_t *v_new, const uint16_t *q, float *out, float softmax_scale,
                      void *workspace, size_t workspace_bytes, void *stream) {
  return decode_step(p, seq_ids, n, k_new, v_new, q, out, softmax_scale, workspace, workspace_bytes, stream, false);
}

int oscar_decode_step_static(oscar_pool *p, const int32_t *seq_ids, int32_t n, const uint16_t *k_new,
                             const uint16_t *v_new, const uint16_t *q, float *out, float softmax_scale,
                             void *stream) {
  if (!p) return fail(OSCAR_EINVAL, "pool is NULL");
  if (p->host_only) return fail(OSCAR_EINVAL, "decode step on a host-only pool");
  void *ws = nullptr;
  size_t ws_bytes = 0;
  hipError_t e = static_scratch(&ws, &ws_bytes);
  if (e != hipSuccess) return hip_fail(e, "static decode workspace");
  return decode_step(p, seq_ids, n, k_new, v_new, q, out, softmax_scale, ws, ws_bytes, stream, true);
}

int oscar_pool_check(oscar_pool *p, void *stream) {
  if (!p) return fail(OSCAR_EINVAL, "pool is NULL");
  if (p->host_only) return ok();
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pool check sync");
  const int rc = check_device_status(p);
  return rc ? rc : ok();
}

// The workspace of the matrix-core launches (prefill_mfma_ws_bytes): it
// depends on the configuration and n_q only.
int oscar_prefill_workspace_bytes(const oscar_pool_config *cfg, int32_t n_q, size_t *bytes) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!bytes || n_q < 0) return fail(OSCAR_EINVAL, "bad arguments");
  const int Hkv = cfg->num_kv_heads, g = cfg->num_q_heads / Hkv;
  const int NT = (int)(((int64_t)n_q * g + kPfTileRows - 1) / kPfTileRows);
  *bytes = prefill_mfma_ws_bytes(Hkv, NT, prefill_mfma_splits(NT, Hkv), cfg->head_dim);
  return ok();
}

int oscar_prefill_attn(oscar_pool *p, int32_t seq, int32_t n_q, const uint16_t *q, float *out, float softmax_scale,
                       void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_seq(p, seq);
  if (rc) return rc;
  if (p->host_only) return fail(OSCAR_EINVAL, "prefill attention on a host-only pool");
  if (p->dev.bf16_hist) return fail(OSCAR_EINVAL, "prefill attention runs on INT2-history pools");
  const int32_t L = p->len[seq];
  if (n_q < 1 || n_q > L || (int64_t)n_q * p->cfg.num_q_heads > ((int64_t)1 << 30))
    return fail(OSCAR_EINVAL, "n_q = %d outside [1, L = %d] (or n_q x Hq above 2^30)", n_q, L);
  if (!q || !out || !workspace) return fail(OSCAR_EINVAL, "NULL argument");
  if (!std::isfinite(softmax_scale)) return fail(OSCAR_EINVAL, "softmax_scale is not finite");
  const int Hkv = p->cfg.num_kv_heads, d = p->cfg.head_dim, g = p->cfg.num_q_heads / Hkv;
  if (!prefill_mfma_supported(p->dev)) return fail(OSCAR_EINVAL, "no prefill kernel for d = %d, G = %d", d, p->cfg.group_size);
  // tiles of kPfTileRows (query, head) rows per kv head, S splits each
  PrefillArgs a;
  a.seq = seq;
  a.L = L;
  a.n_q = n_q;
  a.g = g;
  a.n_hist = std::max(0, L - kWindow);
  a.NT = (int)(((int64_t)n_q * g + kPfTileRows - 1) / kPfTileRows);
  a.S = prefill_mfma_splits(a.NT, Hkv);
  a.qscale = softmax_scale * 1.4426950408889634f;
  const size_t need = prefill_mfma_ws_bytes(Hkv, a.NT, a.S, d);
  if (workspace_bytes < need)
    return fail(OSCAR_EINVAL, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  hipError_t e = launch_prefill_mfma(p->dev, a, q, out, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  return ok();
}

int oscar_release_seq(oscar_pool *p, int32_t seq) {
  int rc = check_seq(p, seq);
  if (rc) return rc;
  for (int32_t pg : p->table[seq])
    if (--p->refs[pg] == 0) p->free_list.push_back(pg);
  p->table[seq].clear();
  p->len[seq] = 0;
  return ok();
}

int oscar_fork_seq(oscar_pool *p, int32_t src, int32_t dst, void *stream) {
  int rc = check_seq(p, src);
  if (!rc) rc = check_seq(p, dst);
  if (rc) return rc;
  if (src == dst) return fail(OSCAR_EINVAL, "fork of sequence %d onto itself", src);
  if (p->len[dst] != 0 || !p->table[dst].empty()) return fail(OSCAR_EINVAL, "sequence %d is not empty", dst);
  if (p->len[src] == 0) return ok();
  if (!p->host_only) {
    hipError_t e = launch_fork(p->dev, src, dst, (int)p->table[src].size(), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "fork launch");
  }
  p->table[dst] = p->table[src];
  for (int32_t pg : p->table[dst]) ++p->refs[pg];
  p->len[dst] = p->len[src];
  return ok();
}

int oscar_pool_set_codebook(oscar_pool *p, const uint8_t *levels_k, const uint8_t *levels_v, void *stream) {
  if (!p) return fail(OSCAR_EINVAL, "pool is NULL");
  if (!p->dev.lut) return fail(OSCAR_EINVAL, "not a Lloyd-Max pool (OSCAR_POOL_LLOYD_MAX)");
  if (!levels_k || !levels_v) return fail(OSCAR_EINVAL, "NULL codebook");
  for (int s = 0; s < p->cfg.max_seqs; ++s)
    if (p->len[s] != 0) return fail(OSCAR_EINVAL, "the codebook is set while every sequence is empty (sequence %d is not)", s);
  const int H = p->cfg.num_kv_heads;
  std::vector<uint32_t> cb(2 * H);
  for (int kind = 0; kind < 2; ++kind)
    for (int h = 0; h < H; ++h) {
      const uint8_t *l = (kind ? levels_v : levels_k) + 4 * h;
      if (l[0] > l[1] || l[1] > l[2] || l[2] > l[3])
        return fail(OSCAR_EINVAL, "codebook of kv head %d (%s) is not non-decreasing", h, kind ? "V" : "K");
      cb[kind * H + h] = (uint32_t)l[0] | ((uint32_t)l[1] << 8) | ((uint32_t)l[2] << 16) | ((uint32_t)l[3] << 24);
    }
  if (!p->host_only) {
    hipError_t e = hipMemcpyAsync((void *)p->dev.codebook, cb.data(), cb.size() * 4, hipMemcpyHostToDevice,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "copying the codebook");
  }
  p->codebook = std::move(cb);
  return ok();
}

int oscar_seq_length(const oscar_pool *p, int32_t seq, int32_t *L) {
  int rc = check_seq(p, seq);
  if (rc) return rc;
  if (!L) return fail(OSCAR_EINVAL, "L is NULL");
  *L = p->len[seq];
  return ok();
}

int oscar_page_table(const oscar_pool *p, int32_t seq, int32_t *pages, int32_t capacity,
                     int32_t *n_pages) {
  int rc = check_seq(p, seq);
  if (rc) return rc;
  if (!n_pages) return fail(OSCAR_EINVAL, "n_pages is NULL");
  const auto &row = p->table[seq];
  if ((size_t)capacity < row.size() || (row.size() && !pages))
    return fail(OSCAR_EINVAL, "capacity %d < %zu pages", capacity, row.size());
  std::copy(row.begin(), row.end(), pages);
  *n_pages = (int32_t)row.size();
  return ok();
}

int oscar_free_pages(const oscar_pool *p, int32_t *n_free) {
  if (!p || !n_free) return fail(OSCAR_EINVAL, "NULL argument");
  *n_free = (int32_t)p->n_free();
  return ok();
}

int oscar_export_history(oscar_pool *p, int32_t seq, int32_t first, int32_t count, uint8_t *codes,
                         uint16_t *params, void *stream) {
  int rc = check_seq(p, seq);
  if (rc) return rc;
  if (p->host_only) return fail(OSCAR_EINVAL, "export from a host-only pool");
  if (p->dev.bf16_hist) return fail(OSCAR_EINVAL, "a BF16-history pool has no codes (oscar_export_history_bf16)");
  int64_t n_hist = std::max(0, p->len[seq] - kWindow);
  if (first < 0 || count < 0 || first + (int64_t)count > n_hist)
    return fail(OSCAR_EINVAL, "history range [%d, %d) outside [0, %lld)", first, first + count,
                (long long)n_hist);
  if (count == 0) return ok();
  if (!codes || !params) return fail(OSCAR_EINVAL, "NULL output");
  const int H = p->cfg.num_kv_heads, d = p->cfg.head_dim, G = p->cfg.group_size;
  const int bb = p->dev.block_bytes;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "export sync");
  if ((rc = check_device_status(p))) return rc;
  std::vector<uint8_t> page((size_t)H * bb);
  int cur = -1;
  for (int64_t i = first; i < first + count; ++i) {
    int pg_idx = (int)(i / kPage), t = (int)(i % kPage);
    if (pg_idx != cur) {
      int pg = p->table[seq][pg_idx];
      e = hipMemcpy(page.data(), p->dev.pages + (size_t)pg * H * bb, page.size(), hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, "export copy");
      cur = pg_idx;
    }
    for (int h = 0; h < H; ++h) {
      const uint8_t *blk = page.data() + (size_t)h * bb;
      size_t o = (size_t)(i - first) * H + h;
      uint8_t *ck = codes + (o * 2 + 0) * (d / 4), *cv = codes + (o * 2 + 1) * (d / 4);
      std::memset(ck, 0, d / 4);
      std::memset(cv, 0, d / 4);
      for (int c = 0; c < d; ++c) {
        uint32_t kw, vw;
        std::memcpy(&kw, blk + kcode_dword_off(d, t, (c % 64) / 16, c / 64), 4);
        std::memcpy(&vw, blk + vcode_dword_off(d, t / 16, c), 4);
        uint32_t kc = (kw >> (2 * (c % 16))) & 3, vc = (vw >> vbit(t % 16)) & 3;
        ck[c / 4] |= kc << (2 * (c % 4));
        cv[c / 4] |= vc << (2 * (c % 4));
      }
      for (int gi = 0; gi < d / G; ++gi) {
        std::memcpy(params + ((o * 2 + 0) * (d / G) + gi) * 2, blk + kparam_off(d, G, t, gi), 4);
        std::memcpy(params + ((o * 2 + 1) * (d / G) + gi) * 2, blk + vparam_off(d, G, t, gi), 4);
      }
    }
  }
  return ok();
}

int oscar_export_state(oscar_pool *p, int32_t seq, int32_t *page_table_host, void *codes_dev, void *params_dev,
                       void *stream) {
  int rc = check_seq(p, seq);
  if (rc) return rc;
  if (p->host_only) return fail(OSCAR_EINVAL, "export from a host-only pool");
  if (p->dev.bf16_hist) return fail(OSCAR_EINVAL, "a BF16-history pool has no codes (oscar_export_history_bf16)");
  if (!page_table_host) return fail(OSCAR_EINVAL, "page_table_host is NULL");
  const int64_t n_hist = std::max(0, p->len[seq] - kWindow);
  if (n_hist > 0 && (!codes_dev || !params_dev)) return fail(OSCAR_EINVAL, "NULL output buffer");
  if (n_hist > 0 && ((uintptr_t)codes_dev % 4 || (uintptr_t)params_dev % 4))
    return fail(OSCAR_EINVAL, "output buffers must be 4-byte aligned");
  if (n_hist > 0) {
    hipError_t e = launch_export(p->dev, seq, (int)n_hist, (uint8_t *)codes_dev, (uint16_t *)params_dev,
                                 (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "export launch");
  }
  const auto &row = p->table[seq];
  for (int i = 0; i < p->cfg.max_pages_per_seq; ++i) page_table_host[i] = i < (int)row.size() ? row[i] : -1;
  return ok();
}

int oscar_export_history_bf16(oscar_pool *p, int32_t seq, int32_t first, int32_t count, uint16_t *k, uint16_t *v,
                              void *stream) {
  int rc = check_seq(p, seq);
  if (rc) return rc;
  if (p->host_only || !p->dev.bf16_hist) return fail(OSCAR_EINVAL, "not a device pool with a BF16 history");
  const int64_t n_hist = std::max(0, p->len[seq] - kWindow);
  if (first < 0 || count < 0 || first + (int64_t)count > n_hist)
    return fail(OSCAR_EINVAL, "history range [%d, %d) outside [0, %lld)", first, first + count, (long long)n_hist);
  if (count == 0) return ok();
  if (!k || !v) return fail(OSCAR_EINVAL, "NULL output");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "export sync");
  if ((rc = check_device_status(p))) return rc;
  const int H = p->cfg.num_kv_heads, d = p->cfg.head_dim, bb = p->dev.block_bytes;
  std::vector<uint16_t> page((size_t)H * bb / 2);
  int cur = -1;
  for (int64_t i = first; i < first + count; ++i) {
    const int pg_idx = (int)(i / kPage), t = (int)(i % kPage);
    if (pg_idx != cur) {
      e = hipMemcpy(page.data(), p->dev.pages + (size_t)p->table[seq][pg_idx] * H * bb, (size_t)H * bb,
                    hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, "export copy");
      cur = pg_idx;
    }
    for (int h = 0; h < H; ++h) {
      const uint16_t *blk = page.data() + (size_t)h * bb / 2;
      const size_t o = ((size_t)(i - first) * H + h) * d;
      std::memcpy(k + o, blk + (size_t)t * d, d * 2);
      std::memcpy(v + o, blk + (size_t)(kPage + t) * d, d * 2);
    }
  }
  return ok();
}

int oscar_export_window(oscar_pool *p, int32_t seq, uint16_t *sink_k, uint16_t *sink_v,
                        uint16_t *recent_k, uint16_t *recent_v, void *stream) {
  int rc = check_seq(p, seq);
  if (rc) return rc;
  if (p->host_only) return fail(OSCAR_EINVAL, "export from a host-only pool");
  if (!sink_k || !sink_v || !recent_k || !recent_v) return fail(OSCAR_EINVAL, "NULL output");
  const int H = p->cfg.num_kv_heads, d = p->cfg.head_dim;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "export sync");
  if ((rc = check_device_status(p))) return rc;
  struct Part {
    const uint16_t *src;
    uint16_t *dst;
    int slots;
  } parts[4] = {{p->dev.sinkK, sink_k, kSink},
                {p->dev.sinkV, sink_v, kSink},
                {p->dev.recentK, recent_k, kRecent},
                {p->dev.recentV, recent_v, kRecent}};
  for (const Part &pt : parts) {
    std::vector<uint16_t> tmp((size_t)H * pt.slots * d);
    e = hipMemcpy(tmp.data(), pt.src + (size_t)seq * H * pt.slots * d, tmp.size() * 2,
                  hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "export copy");
    for (int h = 0; h < H; ++h)
      for (int s = 0; s < pt.slots; ++s)
        std::memcpy(pt.dst + ((size_t)s * H + h) * d, tmp.data() + ((size_t)h * pt.slots + s) * d, d * 2);
  }
  return ok();
}

int oscar_profile_begin(oscar_pool *p, int32_t max_calls, uint32_t kernels, int32_t every) {
  if (!p) return fail(OSCAR_EINVAL, "pool is NULL");
  if (kernels == 0 || (kernels & ~7u)) return fail(OSCAR_EINVAL, "bad kernel mask 0x%x", kernels);
  if (every < 1) return fail(OSCAR_EINVAL, "every = %d < 1", every);
  if (max_calls < 1 || max_calls > (1 << 16)) return fail(OSCAR_EINVAL, "max_calls %d outside [1, 65536]", max_calls);
  if (p->host_only) return fail(OSCAR_EINVAL, "profiling a host-only pool");
  p->prof.release();
  for (auto &v : p->prof.ev) {
    v.resize(2 * (size_t)max_calls);
    for (hipEvent_t &e : v) {
      // timing only: without the system-scope fence a timed launch is not
      // preceded by a cache write-back that the interval would count
      hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
      if (r != hipSuccess) {
        e = nullptr;
        p->prof.release();
        return hip_fail(r, "hipEventCreate");
      }
    }
  }
  p->prof.cap = max_calls;
  p->prof.every = every;
  p->prof.mask = kernels;
  p->prof.on = true;
  return ok();
}

int oscar_profile_end(oscar_pool *p, oscar_profile *out) {
  if (!p || !out) return fail(OSCAR_EINVAL, "NULL argument");
  if (!p->prof.on) return fail(OSCAR_EINVAL, "profiling was not started");
  float ms[3] = {0.f, 0.f, 0.f};
  for (int k = 0; k < 3; ++k)
    for (int i = 0; i < p->prof.used[k]; ++i) {
      hipError_t r = hipEventSynchronize(p->prof.ev[k][2 * i + 1]);
      float t = 0.f;
      if (r == hipSuccess) r = hipEventElapsedTime(&t, p->prof.ev[k][2 * i], p->prof.ev[k][2 * i + 1]);
      if (r != hipSuccess) {
        p->prof.release();
        return hip_fail(r, "reading profile events");
      }
      ms[k] += t;
    }
  {
    // the status of every launch so far
    hipError_t r = hipDeviceSynchronize();
    if (r != hipSuccess) {
      p->prof.release();
      return hip_fail(r, "synchronising");
    }
    const int rc = check_device_status(p);
    if (rc) {
      p->prof.release();
      return rc;
    }
  }
  out->n_decode_main = p->prof.used[0];
  out->ms_decode_main = ms[0];
  out->n_decode_merge = p->prof.used[1];
  out->ms_decode_merge = ms[1];
  out->n_append = p->prof.used[2];
  out->ms_append = ms[2];
  p->prof.release();
  return ok();
}

int oscar_build_rotation(int32_t d, const float *U, float *R) {
  if (d < 1 || d > 1024 || (d & (d - 1))) return fail(OSCAR_EINVAL, "d = %d is not a power of two <= 1024", d);
  if (!U || !R) return fail(OSCAR_EINVAL, "NULL argument");
  int bits = 0;
  while ((1 << bits) < d) ++bits;
  std::vector<double> row(d);
  const double sq = std::sqrt((double)d);
  for (int i = 0; i < d; ++i) {
    for (int k = 0; k < d; ++k) row[k] = U[(size_t)i * d + k];
    // row . H (Sylvester order) by the fast Walsh-Hadamard butterflies
    for (int len = 1; len < d; len <<= 1)
      for (int b = 0; b < d; b += 2 * len)
        for (int j = b; j < b + len; ++j) {
          double a = row[j], c = row[j + len];
          row[j] = a + c;
          row[j + len] = a - c;
        }
    // (U H Pi)[i][j] = (U H)[i][bitrev(j)]
    for (int j = 0; j < d; ++j) {
      int r = 0;
      for (int t = 0; t < bits; ++t) r |= ((j >> t) & 1) << (bits - 1 - t);
      R[(size_t)i * d + j] = (float)(row[r] / sq);
    }
  }
  return ok();
}

// ---------------------------------------------------------------------------
// Calibration (news article on OSCAR, section "OSCAR aims the rotation at
// attention"): covariances on the device, eigenbasis on the host.
// ---------------------------------------------------------------------------
static int check_calib_shape(int32_t n, int32_t Hq, int32_t Hkv, int32_t d) {
  if (n < 0 || n > (1 << 24)) return fail(OSCAR_EINVAL, "n = %d outside [0, 2^24]", n);
  if (Hkv < 1 || Hkv > 64 || Hq < 1 || Hq % Hkv != 0 || Hq / Hkv > 64)
    return fail(OSCAR_EINVAL, "heads %d / %d: Hq must be a multiple of Hkv (Hkv <= 64, Hq/Hkv <= 64)", Hq, Hkv);
  if (d != 64 && d != 128) return fail(OSCAR_EINVAL, "head_dim %d must be 64 or 128", d);
  return OSCAR_OK;
}

static int check_calib_inputs(const uint16_t *q, const uint16_t *k, const uint16_t *v, float scale) {
  if (!q || !k || !v) return fail(OSCAR_EINVAL, "NULL q, k or v");
  if (((uintptr_t)k & 15) || ((uintptr_t)v & 3) || ((uintptr_t)q & 1))
    return fail(OSCAR_EINVAL, "k must be 16-byte, v 4-byte and q 2-byte aligned");
  if (!std::isfinite(scale)) return fail(OSCAR_EINVAL, "softmax_scale is not finite");
  return OSCAR_OK;
}

int oscar_calib_workspace_bytes(int32_t n, int32_t num_q_heads, int32_t head_dim, size_t *bytes) {
  if (!bytes || n < 0 || num_q_heads < 1 || head_dim < 1) return fail(OSCAR_EINVAL, "bad arguments");
  *bytes = (size_t)n * num_q_heads * head_dim * sizeof(float);
  return ok();
}

int oscar_calib_attention(int32_t n, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, const uint16_t *q,
                          const uint16_t *k, const uint16_t *v, float softmax_scale, float *out, void *stream) {
  int rc = check_calib_shape(n, num_q_heads, num_kv_heads, head_dim);
  if (rc) return rc;
  if (n == 0) return ok();
  rc = check_calib_inputs(q, k, v, softmax_scale);
  if (rc) return rc;
  if (!out || ((uintptr_t)out & 3)) return fail(OSCAR_EINVAL, "out is NULL or not 4-byte aligned");
  hipError_t e = launch_calib_attn(n, num_q_heads, num_kv_heads, head_dim, q, k, v, softmax_scale, out,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "calibration attention launch");
  return ok();
}

int oscar_calib_covariance(int32_t n, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, const uint16_t *q,
                           const uint16_t *k, const uint16_t *v, float softmax_scale, float *cov_k, float *cov_v,
                           void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_calib_shape(n, num_q_heads, num_kv_heads, head_dim);
  if (rc) return rc;
  if (n == 0) return ok();
  rc = check_calib_inputs(q, k, v, softmax_scale);
  if (rc) return rc;
  if (!cov_k || !cov_v || ((uintptr_t)cov_k & 3) || ((uintptr_t)cov_v & 3))
    return fail(OSCAR_EINVAL, "cov_k or cov_v is NULL or not 4-byte aligned");
  const size_t need = (size_t)n * num_q_heads * head_dim * sizeof(float);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 3))
    return fail(OSCAR_EINVAL, "workspace of %zu bytes < %zu required (or NULL, or not 4-byte aligned)",
                workspace_bytes, need);
  float *o = (float *)workspace;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_calib_attn(n, num_q_heads, num_kv_heads, head_dim, q, k, v, softmax_scale, o, s);
  if (e == hipSuccess) e = launch_calib_gram(n, num_q_heads, num_kv_heads, head_dim, q, o, cov_k, cov_v, s);
  if (e != hipSuccess) return hip_fail(e, "calibration covariance launch");
  return ok();
}

} // extern "C"

// Eigen-decomposition of a symmetric d x d matrix (row-major, fp64) by the
// cyclic Jacobi method (Golub and Van Loan, "Matrix Computations", the
// symmetric Schur decomposition and cyclic Jacobi): sweeps over every
// off-diagonal pair (p, q), each zeroed by a plane rotation J with
// tan = sign(tau) / (|tau| + sqrt(1 + tau^2)), tau = (a_qq - a_pp) / (2 a_pq);
// A <- J^T A J, V <- V J, until the off-diagonal mass is below 1e-30 of the
// diagonal's (a relative Frobenius size of 1e-15).  On return diag(A) holds
// the eigenvalues and the columns of V the eigenvectors.
static void jacobi_eigen(int d, std::vector<double> &A, std::vector<double> &V) {
  V.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) V[(size_t)i * d + i] = 1.0;
  auto a = [&](int i, int j) -> double & { return A[(size_t)i * d + j]; };
  for (int sweep = 0; sweep < 60; ++sweep) {
    double off = 0.0, diag = 0.0;
    for (int i = 0; i < d; ++i) {
      diag += a(i, i) * a(i, i);
      for (int j = i + 1; j < d; ++j) off += a(i, j) * a(i, j);
    }
    if (off == 0.0 || off <= 1e-30 * diag) break;
    for (int p = 0; p < d - 1; ++p)
      for (int q = p + 1; q < d; ++q) {
        const double apq = a(p, q);
        if (apq == 0.0) continue;
        const double tau = (a(q, q) - a(p, p)) / (2.0 * apq);
        const double t = (tau >= 0.0 ? 1.0 : -1.0) / (std::fabs(tau) + std::sqrt(1.0 + tau * tau));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = t * c;
        for (int k = 0; k < d; ++k) { // columns p, q: A J
          const double akp = a(k, p), akq = a(k, q);
          a(k, p) = c * akp - s * akq;
          a(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < d; ++k) { // rows p, q: J^T (A J)
          const double apk = a(p, k), aqk = a(q, k);
          a(p, k) = c * apk - s * aqk;
          a(q, k) = s * apk + c * aqk;
        }
        a(p, q) = a(q, p) = 0.0;
        for (int k = 0; k < d; ++k) {
          double &vkp = V[(size_t)k * d + p], &vkq = V[(size_t)k * d + q];
          const double x = vkp, y = vkq;
          vkp = c * x - s * y;
          vkq = s * x + c * y;
        }
      }
  }
}

extern "C" {

int oscar_calib_rotation(int32_t d, const float *cov, float *U, float *R, double *eigenvalues) {
  if (d < 1 || d > 1024 || (d & (d - 1))) return fail(OSCAR_EINVAL, "d = %d is not a power of two <= 1024", d);
  if (!cov || !R) return fail(OSCAR_EINVAL, "NULL cov or R");
  std::vector<double> A((size_t)d * d), V;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      const float x = cov[(size_t)i * d + j], y = cov[(size_t)j * d + i];
      if (!std::isfinite(x)) return fail(OSCAR_EINVAL, "covariance entry (%d, %d) is not finite", i, j);
      A[(size_t)i * d + j] = 0.5 * ((double)x + (double)y);
    }
  jacobi_eigen(d, A, V);
  // eigenvalues descending (equal ones keep their index order)
  std::vector<int> order(d);
  for (int i = 0; i < d; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return A[(size_t)x * d + x] > A[(size_t)y * d + y]; });
  // columns in that order, each with its first entry of largest magnitude
  // positive, rounded to fp32 and then to the nearest multiple of 2^-40
  // (ties to even), the grid on which U . H . Pi is exact in fp64
  std::vector<float> Ug((size_t)d * d);
  for (int c = 0; c < d; ++c) {
    const int src = order[c];
    int jmax = 0;
    for (int j = 1; j < d; ++j)
      if (std::fabs(V[(size_t)j * d + src]) > std::fabs(V[(size_t)jmax * d + src])) jmax = j;
    const double sign = V[(size_t)jmax * d + src] < 0.0 ? -1.0 : 1.0;
    for (int j = 0; j < d; ++j) {
      const float f = (float)(sign * V[(size_t)j * d + src]);
      Ug[(size_t)j * d + c] = (float)std::ldexp(std::nearbyint(std::ldexp((double)f, 40)), -40);
    }
    if (eigenvalues) eigenvalues[c] = A[(size_t)src * d + src];
  }
  if (U) std::memcpy(U, Ug.data(), Ug.size() * sizeof(float));
  return oscar_build_rotation(d, Ug.data(), R);
}

// Lloyd-Max codebook of one head (offline): the normalised values u = (y - z)
// / s of n tokens (rotation by the eviction's fp32 FMA chain, clip, the
// group's fp16 s and z), taken on the grid of 2^-20 as integers; Lloyd's
// algorithm from the uniform levels 0, 1, 2, 3 (cells split midway between
// levels, a value on a midpoint in the lower cell, each level moved to its
// cell's mean, an empty cell's level kept), then L_k = rint(64 level_k).
int oscar_lloyd_max_codebook(int32_t d, int32_t G, int64_t n, const uint16_t *x, const float *R, const float *clip,
                             int32_t iters, uint8_t *levels) {
  if (d < 1 || d > 1024 || G < 1 || d % G) return fail(OSCAR_EINVAL, "bad d = %d or G = %d", d, G);
  if (n < 1 || !x || !R || !clip || !levels) return fail(OSCAR_EINVAL, "bad arguments");
  if (iters < 0 || iters > 100000) return fail(OSCAR_EINVAL, "iterations %d outside [0, 100000]", iters);
  constexpr double kGrid = 1048576.0; // 2^20
  std::vector<int64_t> U;
  U.reserve((size_t)n * d);
  std::vector<float> y(d);
  for (int64_t t = 0; t < n; ++t) {
    for (int j = 0; j < d; ++j) {
      float acc = 0.0f;
      for (int i = 0; i < d; ++i) {
        uint32_t u = (uint32_t)x[(size_t)t * d + i] << 16;
        float xf;
        std::memcpy(&xf, &u, 4);
        acc = std::fmaf(xf, R[(size_t)i * d + j], acc);
      }
      y[j] = std::fmin(std::fmax(acc, -clip[j]), clip[j]);
    }
    for (int g = 0; g < d / G; ++g) {
      float mn = y[g * G], mx = y[g * G];
      for (int k = 1; k < G; ++k) {
        mn = std::fmin(mn, y[g * G + k]);
        mx = std::fmax(mx, y[g * G + k]);
      }
      const float range = (mx - mn) + 0.0f;
      const float s = (float)(_Float16)(range / 3.0f), z = (float)(_Float16)(mn + 0.0f);
      if (s == 0.0f) continue;
      for (int k = 0; k < G; ++k) {
        const float u = (y[g * G + k] - z) / s;
        U.push_back((int64_t)std::nearbyint((double)u * kGrid));
      }
    }
  }
  double lev[4] = {0.0, 1.0, 2.0, 3.0};
  for (int it = 0; it < iters; ++it) {
    double thr[3];
    for (int k = 0; k < 3; ++k) thr[k] = (lev[k] + lev[k + 1]) * (kGrid / 2);
    int64_t sum[4] = {0, 0, 0, 0}, cnt[4] = {0, 0, 0, 0};
    for (int64_t v : U) {
      const double dv = (double)v;
      const int c = (dv > thr[0]) + (dv > thr[1]) + (dv > thr[2]);
      sum[c] += v;
      ++cnt[c];
    }
    for (int k = 0; k < 4; ++k)
      if (cnt[k]) lev[k] = (double)sum[k] / (double)cnt[k] / kGrid;
  }
  for (int k = 0; k < 4; ++k) levels[k] = (uint8_t)std::min(255.0, std::max(0.0, std::nearbyint(lev[k] * 64.0)));
  return ok();
}

int oscar_calibrate_clip(int32_t d, int64_t n, const uint16_t *x, const float *R, double pct, float *clip) {
  if (d < 1 || d > 1024) return fail(OSCAR_EINVAL, "bad d = %d", d);
  if (n < 1 || !x || !R || !clip) return fail(OSCAR_EINVAL, "bad arguments");
  if (!(pct >= 0.0 && pct <= 100.0)) return fail(OSCAR_EINVAL, "percentile %g outside [0, 100]", pct);
  std::vector<float> y((size_t)n * d);
  for (int64_t t = 0; t < n; ++t)
    for (int j = 0; j < d; ++j) {
      float acc = 0.0f;
      for (int i = 0; i < d; ++i) {
        uint32_t u = (uint32_t)x[(size_t)t * d + i] << 16;
        float xf;
        std::memcpy(&xf, &u, 4);
        acc = std::fmaf(xf, R[(size_t)i * d + j], acc);
      }
      y[(size_t)j * n + t] = std::fabs(acc);
    }
  const double h = (double)(n - 1) * (pct / 100.0);
  const int64_t k = (int64_t)std::floor(h);
  for (int j = 0; j < d; ++j) {
    float *col = y.data() + (size_t)j * n;
    std::sort(col, col + n);
    double lo = col[k], hi = col[std::min<int64_t>(k + 1, n - 1)];
    clip[j] = (float)(lo + (h - (double)k) * (hi - lo));
  }
  return ok();
}

} // extern "C"
