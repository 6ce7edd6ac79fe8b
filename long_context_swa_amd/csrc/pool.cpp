// libswa host side: dual-pool KV metadata, window-safe prefix length, staging of small tables,
// argument checking, work planning and kernel launches behind the C ABI of include/swa.h.
//
// Pool model ([MiMo-review] §潜在力を本番へ, dual-pool KV cache): SWA layers keep a w-slot ring
// per sequence ([SWA-theory] §Rolling Buffer KV Cache, Eq.(7): position t in slot t mod w);
// full layers keep every token in 16-token pages handed out from a per-layer free list, with
// reference counts so that forked sequences share whole pages of a common prefix.

#include "swa.h"
#include "swa_internal.h"
#include "staging_ring.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <new>
#include <string>
#include <vector>

using namespace swa;

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

int hip_fail(hipError_t e, const char *what) {
  return fail(SWA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Landing zone at the end of the arena for per-call metadata of batched commits (sequence list
// and page-table patches), reused in stream order.
constexpr int64_t kMetaBytes = 4 << 20;

// Table cache after the landing zone: device copies of recent per-call tables (sequence lists,
// decode work lists), one per slot.
constexpr int kCacheSlots = 4;
constexpr int64_t kCacheSlotBytes = 2 << 20;

// Pinned host ring used to stage small host tables (page-table rows, decode work lists) for
// stream-ordered copies into device memory.  RingSpace decides where each upload goes and which
// in-flight copies must finish first; each copy is followed by an event that marks its region free.
class Staging {
 public:
  ~Staging() { release(); }
  int init(size_t cap) {
    hipError_t e = hipHostMalloc((void **)&host_, cap, hipHostMallocDefault);
    if (e != hipSuccess) { host_ = nullptr; return hip_fail(e, "hipHostMalloc(staging)"); }
    space_ = RingSpace(cap);
    return SWA_OK;
  }
  void release() {
    if (!host_) return;
    space_.clear([&](uint64_t t) { (void)hipEventSynchronize(events_[t]); });
    for (auto ev : events_) (void)hipEventDestroy(ev);
    events_.clear();
    free_.clear();
    (void)hipHostFree(host_);
    host_ = nullptr;
  }
  // Copy `bytes` from host memory `src` to device `dst` in stream order.
  int upload(void *dst, const void *src, size_t bytes, hipStream_t s) {
    const char *p = static_cast<const char *>(src);
    char *d = static_cast<char *>(dst);
    while (bytes > 0) {
      size_t n = std::min(bytes, space_.capacity() / 2);
      int rc = upload_one(d, p, n, s);
      if (rc) return rc;
      p += n; d += n; bytes -= n;
    }
    return SWA_OK;
  }

 private:
  int upload_one(char *dst, const char *src, size_t n, hipStream_t s) {
    // forget copies that have completed (cheap queries, oldest first)
    space_.retire([&](uint64_t t) { return hipEventQuery(events_[t]) == hipSuccess; },
                  [&](uint64_t t) { free_.push_back((uint32_t)t); });
    const size_t n_al = (size_t)align_up((int64_t)n, 256);
    wait_.clear();
    const size_t b = space_.reserve(n_al, wait_);
    for (uint64_t t : wait_) {  // copies still reading bytes of [b, b + n_al)
      hipError_t he = hipEventSynchronize(events_[t]);
      free_.push_back((uint32_t)t);
      if (he != hipSuccess) return hip_fail(he, "hipEventSynchronize(staging)");
    }
    memcpy(host_ + b, src, n);
    hipError_t he = hipMemcpyAsync(dst, host_ + b, n, hipMemcpyHostToDevice, s);
    if (he != hipSuccess) return hip_fail(he, "hipMemcpyAsync(staging)");
    uint32_t t;
    if (!free_.empty()) { t = free_.back(); free_.pop_back(); }
    else {
      hipEvent_t ev;
      if ((he = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return hip_fail(he, "hipEventCreate");
      t = (uint32_t)events_.size();
      events_.push_back(ev);
    }
    if ((he = hipEventRecord(events_[t], s)) != hipSuccess) return hip_fail(he, "hipEventRecord");
    space_.publish(b, n_al, t);
    return SWA_OK;
  }
  char *host_ = nullptr;
  RingSpace space_;
  std::vector<hipEvent_t> events_;
  std::vector<uint32_t> free_;
  std::vector<uint64_t> wait_;
};

}  // namespace

namespace swa {
// Error reporting for entry points defined in other source files of the library.
int set_error(int code, const char *msg) { return fail(code, "%s", msg); }
}  // namespace swa

struct swa_pool {
  swa_pool_desc desc{};
  std::vector<uint8_t> full;      // per layer
  std::vector<int32_t> kind_idx;  // index among SWA layers or among full layers
  int32_t n_swa = 0, n_full = 0;
  char *arena = nullptr;
  int64_t arena_bytes = 0;
  bool planning = false;
  int32_t n_cu = 256;      // compute units of the arena's device (sizes the decode split)
  int es = 4;              // storage bytes per K/V element (1 for FP8 pools)
  int act_es = 4;          // bytes per element of appended k/v and of attention activations
  bool fp8 = false;
  float k_scale = 1.f, v_scale = 1.f;  // FP8 pools: powers of two
  int64_t tok_bytes = 0;   // K+V bytes of one token, all KV heads
  int64_t ring_bytes = 0;  // one (seq, SWA layer) ring: K then V, each [Hkv][w][d]
  int64_t page_bytes = 0;  // one page: K then V, each [Hkv][16][d]
  int64_t maxp = 0;        // page-table row length
  int64_t off_ring = 0, off_snap = 0, off_pages = 0, off_tables = 0, off_rope = 0, off_meta = 0, total = 0;
  int64_t off_rchunk = 0;  // fused-RoPE pools: rotated keys of the chunk being prefilled
  int64_t rope_hi_rows = 0;  // rows of the high-angle RoPE table (0: pool without RoPE)
  int64_t off_cache = 0;
  // Host copy of what each table-cache slot holds on the device.  A decode step passes the same
  // sequence list to every layer's attention, commit and RoPE call, and the same work list to every
  // layer of a kind, so most calls find their tables already in the arena and copy nothing.
  struct CacheSlot {
    std::vector<char> host;
    uint64_t used = 0;
    bool valid = false;
  };
  CacheSlot cache[kCacheSlots];
  uint64_t cache_tick = 0;

  struct Seq {
    bool open = false;
    std::vector<int64_t> len;                  // per layer
    std::vector<std::vector<int32_t>> pages;   // per full layer
    std::vector<std::vector<int64_t>> tags;    // per SWA layer, w entries
  };
  std::vector<Seq> seqs;
  // Ring snapshots: rings of all SWA layers at length `len` in the arena's snapshot slot, the ring
  // tags, and references on the full-layer pages covering [0, len).
  struct Snap {
    bool used = false;
    int64_t len = 0;
    std::vector<std::vector<int64_t>> tags;     // per SWA layer
    std::vector<std::vector<int32_t>> pages;    // per full layer
  };
  std::vector<Snap> snaps;
  int64_t snap_off(int32_t id) const { return off_snap + (int64_t)id * n_swa * ring_bytes; }
  std::vector<int32_t> free_seqs;                 // stack
  std::vector<std::vector<int32_t>> free_pages;  // per full layer, stack
  std::vector<std::vector<int32_t>> refcnt;      // per full layer, per page
  Staging staging;

  // Rings are laid out layer-major ([SWA layer][sequence]): one layer's rings are contiguous, so
  // a decode call over many sequences reads one dense region of the arena.
  char *ring_ptr(int32_t seq, int32_t swa_i) const { return arena + ring_off(seq, swa_i); }
  int64_t ring_off(int32_t seq, int32_t swa_i) const {
    return off_ring + ((int64_t)swa_i * desc.max_seqs + seq) * ring_bytes;
  }
  int64_t ring_layer_stride() const { return (int64_t)desc.max_seqs * ring_bytes; }
  int64_t page_off(int32_t full_i, int32_t page) const {
    return off_pages + ((int64_t)full_i * desc.pages_per_full_layer + page) * page_bytes;
  }
  int64_t table_off(int32_t full_i, int32_t seq) const {
    return off_tables + (((int64_t)full_i * desc.max_seqs + seq) * maxp) * 4;
  }
  LayerView view(int32_t layer) const {
    LayerView v{};
    int32_t k = kind_idx[layer];
    v.hkv = desc.n_kv_heads;
    v.d = desc.head_dim;
    v.is_full = full[layer];
    v.kv_fp8 = fp8 ? 1 : 0;
    v.k_scale = k_scale;
    v.v_scale = v_scale;
    v.k_inv = 1.f / k_scale;  // exact: powers of two
    v.v_inv = 1.f / v_scale;
    v.rope_fused = desc.rope_fused;
    v.rope_style = desc.rope_style;
    if (rope_hi_rows > 0 && arena) {
      v.rope_lo = reinterpret_cast<const float2 *>(arena + off_rope);
      v.rope_hi = v.rope_lo + kRopeLo * (desc.head_dim / 2);
    }
    if (full[layer]) {
      v.w = 0;
      v.page_base = arena + page_off(k, 0);
      v.tables = reinterpret_cast<const int32_t *>(arena + table_off(k, 0));
      v.table_stride = maxp;
    } else {
      v.w = desc.window;
      v.ring_base = arena + ring_off(0, k);
      v.ring_seq_stride = ring_bytes;
    }
    return v;
  }
  int64_t committed(const Seq &s) const {
    int64_t m = INT64_MAX;
    for (auto l : s.len) m = std::min(m, l);
    return m == INT64_MAX ? 0 : m;
  }
};

namespace {

int check_desc(const swa_pool_desc *d) {
  if (!d) return fail(SWA_EINVAL, "desc is NULL");
  if (d->n_layers < 1) return fail(SWA_EINVAL, "n_layers must be >= 1");
  if (d->window < 1) return fail(SWA_EINVAL, "window must be >= 1");
  if (d->n_kv_heads < 1) return fail(SWA_EINVAL, "n_kv_heads must be >= 1");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(SWA_EINVAL, "head_dim must be 64 or 128");
  if (d->kv_dtype != SWA_F32 && d->kv_dtype != SWA_BF16 && d->kv_dtype != SWA_FP8_E4M3)
    return fail(SWA_EINVAL, "bad kv_dtype");
  if (d->kv_dtype == SWA_FP8_E4M3) {
    for (float sc : {d->k_scale, d->v_scale}) {
      if (sc == 0.f) continue;  // 0 means 1
      int ex = 0;
      const float m = std::frexp(sc, &ex);
      if (!(sc > 0.f) || m != 0.5f || ex < -59 || ex > 61)
        return fail(SWA_EINVAL, "FP8 scales must be powers of two in [2^-60, 2^60] (got %g)", (double)sc);
    }
  }
  if (d->page_tokens != kPageTokens) return fail(SWA_EINVAL, "page_tokens must be 16");
  if (d->pages_per_full_layer < 0 || d->pages_per_full_layer > INT32_MAX)
    return fail(SWA_EINVAL, "pages_per_full_layer out of range");
  if (d->max_seqs < 1) return fail(SWA_EINVAL, "max_seqs must be >= 1");
  if (d->max_snapshots < 0 || d->max_snapshots > (1 << 20)) return fail(SWA_EINVAL, "max_snapshots out of range");
  // work items and the kernels' key indices are 32-bit: a sequence holds at most 2^31 - 1 tokens
  if (d->max_seq_len < 1 || d->max_seq_len > INT32_MAX)
    return fail(SWA_EINVAL, "max_seq_len must be in 1 .. 2^31 - 1");
  if (!(d->rope_base == 0.f || (std::isfinite(d->rope_base) && d->rope_base > 0.f)))
    return fail(SWA_EINVAL, "rope_base must be 0 (no RoPE) or a positive finite number");
  if (d->decode_plan != SWA_PLAN_UNIFORM && d->decode_plan != SWA_PLAN_BUCKETED)
    return fail(SWA_EINVAL, "decode_plan must be SWA_PLAN_UNIFORM or SWA_PLAN_BUCKETED");
  if (d->rope_style != SWA_ROPE_PAIRS && d->rope_style != SWA_ROPE_HALVES)
    return fail(SWA_EINVAL, "rope_style must be SWA_ROPE_PAIRS or SWA_ROPE_HALVES");
  if (d->rope_base > 0.f && d->max_seq_len > ((int64_t)1 << 26))
    return fail(SWA_EINVAL, "RoPE pools need max_seq_len <= 2^26 (angle tables are built at create)");
  if (d->rope_fused != 0 && d->rope_fused != 1) return fail(SWA_EINVAL, "rope_fused must be 0 or 1");
  if (d->max_chunk < 0) return fail(SWA_EINVAL, "max_chunk must be >= 0");
  if (d->rope_fused) {
    if (!(d->rope_base > 0.f)) return fail(SWA_EINVAL, "rope_fused needs rope_base > 0");
    if (d->kv_dtype == SWA_F32) return fail(SWA_EINVAL, "rope_fused needs a bf16 or FP8 pool");
    if (d->max_chunk < 1) return fail(SWA_EINVAL, "rope_fused needs max_chunk >= 1");
  }
  return SWA_OK;
}

bool default_full(int32_t l) { return l % 7 == 6; }

void layout(swa_pool *p) {
  const swa_pool_desc &d = p->desc;
  p->fp8 = d.kv_dtype == SWA_FP8_E4M3;
  p->es = p->fp8 ? 1 : d.kv_dtype == SWA_BF16 ? 2 : 4;
  p->act_es = d.kv_dtype == SWA_F32 ? 4 : 2;
  p->k_scale = (p->fp8 && d.k_scale != 0.f) ? d.k_scale : 1.f;
  p->v_scale = (p->fp8 && d.v_scale != 0.f) ? d.v_scale : 1.f;
  p->tok_bytes = 2LL * d.n_kv_heads * d.head_dim * p->es;
  p->ring_bytes = align_up((int64_t)d.window * p->tok_bytes, 256);
  p->page_bytes = (int64_t)kPageTokens * p->tok_bytes;
  p->maxp = align_up((d.max_seq_len + kPageTokens - 1) / kPageTokens, 64);
  p->off_ring = 0;
  p->off_snap = align_up(p->off_ring + (int64_t)d.max_seqs * p->n_swa * p->ring_bytes, 4096);
  p->off_pages = align_up(p->off_snap + (int64_t)d.max_snapshots * p->n_swa * p->ring_bytes, 4096);
  p->off_tables = align_up(p->off_pages + (int64_t)p->n_full * d.pages_per_full_layer * p->page_bytes, 4096);
  p->off_rope = align_up(p->off_tables + (int64_t)p->n_full * d.max_seqs * p->maxp * 4, 4096);
  p->rope_hi_rows = d.rope_base > 0.f ? (d.max_seq_len + kRopeLo - 1) / kRopeLo : 0;
  const int64_t rope_rows = d.rope_base > 0.f ? kRopeLo + p->rope_hi_rows : 0;
  p->off_rchunk = align_up(p->off_rope + rope_rows * (d.head_dim / 2) * 8, 4096);
  const int64_t rchunk = d.rope_fused ? (int64_t)d.max_chunk * d.n_kv_heads * d.head_dim * 2 : 0;
  p->off_meta = align_up(p->off_rchunk + rchunk, 4096);
  p->off_cache = p->off_meta + kMetaBytes;
  p->total = p->off_cache + kCacheSlots * kCacheSlotBytes;
}

// Device address of a copy of the host table `src` (`bytes` bytes) in the arena's table cache: a
// slot already holding the same bytes is reused, otherwise the least recently used slot is
// overwritten by a stream-ordered copy (work queued earlier that still reads the old contents runs
// first).  nullptr, with rc == SWA_OK, if the table does not fit a slot: the caller then stages it
// elsewhere.
const char *cached_table(swa_pool *p, const void *src, size_t bytes, hipStream_t s, int &rc) {
  rc = SWA_OK;
  if (bytes == 0 || (int64_t)bytes > kCacheSlotBytes) return nullptr;
  int victim = 0;
  for (int i = 0; i < kCacheSlots; ++i) {
    auto &c = p->cache[i];
    if (c.valid && c.host.size() == bytes && std::memcmp(c.host.data(), src, bytes) == 0) {
      c.used = ++p->cache_tick;
      return p->arena + p->off_cache + i * kCacheSlotBytes;
    }
    const auto &v = p->cache[victim];
    if (!c.valid ? v.valid : (v.valid && c.used < v.used)) victim = i;
  }
  char *dst = p->arena + p->off_cache + victim * kCacheSlotBytes;
  auto &c = p->cache[victim];
  c.valid = false;
  if ((rc = p->staging.upload(dst, src, bytes, s))) return nullptr;
  c.host.assign(static_cast<const char *>(src), static_cast<const char *>(src) + bytes);
  c.valid = true;
  c.used = ++p->cache_tick;
  return dst;
}

// RoPE angle tables (RoFormer §3.2-§3.4: theta_i = base^(-2i/d)): (cos, sin) of l * theta_i for
// l < kRopeLo, then of h * kRopeLo * theta_i for h < rope_hi_rows, computed in long double and
// stored as fp32 pairs.
int fill_rope_tables(swa_pool *p) {
  const int half = p->desc.head_dim / 2;
  const int64_t rows = kRopeLo + p->rope_hi_rows;
  std::vector<float> tab((size_t)(rows * half * 2));
  const long double base = p->desc.rope_base;
  for (int i = 0; i < half; ++i) {
    const long double theta = std::pow(base, -2.0L * i / p->desc.head_dim);
    for (int64_t r = 0; r < rows; ++r) {
      const long double pos = r < kRopeLo ? (long double)r : (long double)(r - kRopeLo) * kRopeLo;
      const long double phi = pos * theta;
      tab[(size_t)((r * half + i) * 2)] = (float)std::cos(phi);
      tab[(size_t)((r * half + i) * 2 + 1)] = (float)std::sin(phi);
    }
  }
  hipError_t e = hipMemcpy(p->arena + p->off_rope, tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice);
  return e == hipSuccess ? SWA_OK : hip_fail(e, "hipMemcpy(RoPE tables)");
}

int get_seq(const swa_pool *p, int32_t seq) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  if (seq < 0 || seq >= p->desc.max_seqs) return fail(SWA_ENOSEQ, "sequence %d out of range", seq);
  if (!p->seqs[seq].open) return fail(SWA_ENOSEQ, "sequence %d is not open", seq);
  return SWA_OK;
}

int get_layer(const swa_pool *p, int32_t layer) {
  if (layer < 0 || layer >= p->desc.n_layers) return fail(SWA_EINVAL, "layer %d out of range", layer);
  return SWA_OK;
}

// Upload page-table entries [from, to) of (seq, full layer) to the arena copy.
int upload_table(swa_pool *p, int32_t seq, int32_t full_i, int64_t from, int64_t to, hipStream_t s) {
  if (p->planning || to <= from) return SWA_OK;
  const auto &pg = p->seqs[seq].pages[full_i];
  return p->staging.upload(p->arena + p->table_off(full_i, seq) + from * 4, pg.data() + from,
                           (to - from) * 4, s);
}

// Window-safe length over the ring tags ([MiMo-review] §潜在力を本番へ).  For each SWA layer the
// safe cuts are [0, c] (c = how far [0, c) is still resident, capped at w) plus, if the ring holds
// exactly w consecutive positions [t-w, t), the cut t.  The answer is the largest candidate that
// passes the direct check in every layer.
int64_t window_safe(const swa_pool *p, const swa_pool::Seq &s, int64_t hi) {
  const int64_t w = p->desc.window;
  auto ok = [&](int64_t m) {
    for (const auto &tags : s.tags)
      for (int64_t q = std::max<int64_t>(0, m - w); q < m; ++q)
        if (tags[q % w] != q) return false;
    return true;
  };
  std::vector<int64_t> cand{hi, 0};
  for (const auto &tags : s.tags) {
    int64_t c = 0;
    while (c < w && tags[c % w] == c) ++c;
    cand.push_back(std::min(c, hi));
    int64_t mx = -1, mn = INT64_MAX;
    for (auto t : tags) { mx = std::max(mx, t); if (t >= 0) mn = std::min(mn, t); }
    if (mx >= 0 && mx - mn + 1 == w) cand.push_back(std::min(mx + 1, hi));
  }
  std::sort(cand.begin(), cand.end(), std::greater<int64_t>());
  for (auto m : cand)
    if (m <= hi && m >= 0 && ok(m)) return m;
  return 0;
}

}  // namespace

// =============================================================================================
// C ABI: pool
// =============================================================================================

extern "C" {

const char *swa_last_error(void) { return g_err.c_str(); }

int swa_clock_probe(void *out, int64_t spin_us, void *stream) {
  if (!out) return fail(SWA_EINVAL, "out is NULL");
  if (reinterpret_cast<uintptr_t>(out) % 8) return fail(SWA_EINVAL, "out must be 8-byte aligned");
  if (spin_us < 1 || spin_us > 10000000) return fail(SWA_EINVAL, "spin_us must be in 1 .. 10,000,000");
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return hip_fail(e, "wall clock rate");
  if (khz <= 0) return fail(SWA_EHIP, "device reports no wall clock rate");
  e = launch_clock_probe(static_cast<int64_t *>(out), spin_us * (int64_t)khz / 1000, khz,
                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SWA_OK : hip_fail(e, "clock_probe_kernel");
}

int64_t kvpool_arena_bytes(const swa_pool_desc *d) {
  int rc = check_desc(d);
  if (rc) return rc;
  swa_pool tmp;
  tmp.desc = *d;
  for (int32_t l = 0; l < d->n_layers; ++l) {
    bool f = d->layer_is_full ? d->layer_is_full[l] != 0 : default_full(l);
    (f ? tmp.n_full : tmp.n_swa)++;
  }
  layout(&tmp);
  return tmp.total;
}

int kvpool_create(const swa_pool_desc *d, void *dev_arena, int64_t arena_bytes, swa_pool **out) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!out) return fail(SWA_EINVAL, "out is NULL");
  swa_pool *p = new (std::nothrow) swa_pool();
  if (!p) return fail(SWA_ENOMEM, "host allocation failed");
  p->desc = *d;
  p->desc.layer_is_full = nullptr;
  p->full.resize(d->n_layers);
  p->kind_idx.resize(d->n_layers);
  for (int32_t l = 0; l < d->n_layers; ++l) {
    p->full[l] = (d->layer_is_full ? d->layer_is_full[l] != 0 : default_full(l)) ? 1 : 0;
    p->kind_idx[l] = p->full[l] ? p->n_full++ : p->n_swa++;
  }
  layout(p);
  p->planning = dev_arena == nullptr;
  if (!p->planning) {
    if ((reinterpret_cast<uintptr_t>(dev_arena) & 255) != 0) {
      delete p;
      return fail(SWA_EINVAL, "arena must be 256-byte aligned");
    }
    if (arena_bytes < p->total) {
      int64_t need = p->total;
      delete p;
      return fail(SWA_ENOMEM, "arena has %lld bytes, pool needs %lld", (long long)arena_bytes,
                  (long long)need);
    }
    p->arena = static_cast<char *>(dev_arena);
    p->arena_bytes = arena_bytes;
    if ((rc = p->staging.init(32u << 20))) { delete p; return rc; }
    if (p->rope_hi_rows > 0 && (rc = fill_rope_tables(p))) { delete p; return rc; }
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0)
      p->n_cu = ncu;
  }
  p->seqs.resize(d->max_seqs);
  p->snaps.resize(d->max_snapshots);
  for (int32_t s = d->max_seqs - 1; s >= 0; --s) p->free_seqs.push_back(s);
  p->free_pages.resize(p->n_full);
  p->refcnt.resize(p->n_full);
  for (int32_t f = 0; f < p->n_full; ++f) {
    p->refcnt[f].assign(d->pages_per_full_layer, 0);
    p->free_pages[f].reserve(d->pages_per_full_layer);
    for (int64_t pg = d->pages_per_full_layer - 1; pg >= 0; --pg) p->free_pages[f].push_back((int32_t)pg);
  }
  *out = p;
  return SWA_OK;
}

int kvpool_destroy(swa_pool *p) {
  delete p;
  return SWA_OK;
}

int kvpool_seq_open(swa_pool *p, int32_t *seq) {
  if (!p || !seq) return fail(SWA_EINVAL, "NULL argument");
  if (p->free_seqs.empty()) return fail(SWA_ENOMEM, "no free sequence slot (max_seqs=%d)", p->desc.max_seqs);
  int32_t s = p->free_seqs.back();
  p->free_seqs.pop_back();
  auto &S = p->seqs[s];
  S.open = true;
  S.len.assign(p->desc.n_layers, 0);
  S.pages.assign(p->n_full, {});
  S.tags.assign(p->n_swa, std::vector<int64_t>(p->desc.window, -1));
  *seq = s;
  return SWA_OK;
}

int kvpool_seq_close(swa_pool *p, int32_t seq) {
  int rc = get_seq(p, seq);
  if (rc) return rc;
  auto &S = p->seqs[seq];
  for (int32_t f = 0; f < p->n_full; ++f)
    for (int32_t pg : S.pages[f])
      if (--p->refcnt[f][pg] == 0) p->free_pages[f].push_back(pg);
  S = swa_pool::Seq();
  p->free_seqs.push_back(seq);
  return SWA_OK;
}

int kvpool_seq_len(const swa_pool *p, int32_t seq, int32_t layer, int64_t *len) {
  int rc = get_seq(p, seq);
  if (rc) return rc;
  if ((rc = get_layer(p, layer))) return rc;
  if (!len) return fail(SWA_EINVAL, "len is NULL");
  *len = p->seqs[seq].len[layer];
  return SWA_OK;
}

int kvpool_layer_is_full(const swa_pool *p, int32_t layer) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  int rc = get_layer(p, layer);
  if (rc) return rc;
  return p->full[layer] ? 1 : 0;
}

int kvpool_free_pages(const swa_pool *p, int32_t layer, int64_t *n_free) {
  if (!p || !n_free) return fail(SWA_EINVAL, "NULL argument");
  int rc = get_layer(p, layer);
  if (rc) return rc;
  if (!p->full[layer]) return fail(SWA_EINVAL, "layer %d is not a full-attention layer", layer);
  *n_free = (int64_t)p->free_pages[p->kind_idx[layer]].size();
  return SWA_OK;
}

int kvpool_bytes(const swa_pool *p, int64_t *allocated, int64_t *resident) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  int64_t alloc = 0, res = 0;
  const int64_t ring_logical = (int64_t)p->desc.window * p->tok_bytes;
  for (const auto &S : p->seqs) {
    if (!S.open) continue;
    for (int32_t l = 0; l < p->desc.n_layers; ++l) {
      if (p->full[l]) continue;
      alloc += ring_logical;
      res += std::min<int64_t>(S.len[l], p->desc.window) * p->tok_bytes;
    }
  }
  for (int32_t f = 0; f < p->n_full; ++f) {
    int64_t held = p->desc.pages_per_full_layer - (int64_t)p->free_pages[f].size();
    alloc += held * p->page_bytes;
    res += held * p->page_bytes;
  }
  if (allocated) *allocated = alloc;
  if (resident) *resident = res;
  return SWA_OK;
}

int kvpool_slot_tags(const swa_pool *p, int32_t seq, int32_t layer, int64_t *tags) {
  int rc = get_seq(p, seq);
  if (rc) return rc;
  if ((rc = get_layer(p, layer))) return rc;
  if (p->full[layer]) return fail(SWA_EINVAL, "layer %d is a full-attention layer", layer);
  if (!tags) return fail(SWA_EINVAL, "tags is NULL");
  const auto &t = p->seqs[seq].tags[p->kind_idx[layer]];
  std::copy(t.begin(), t.end(), tags);
  return SWA_OK;
}

int kvpool_locate(const swa_pool *p, int32_t seq, int32_t layer, int64_t pos, int32_t head,
                  int64_t *k_off, int64_t *v_off, int64_t *v_stride) {
  int rc = get_seq(p, seq);
  if (rc) return rc;
  if ((rc = get_layer(p, layer))) return rc;
  if (!k_off || !v_off || !v_stride) return fail(SWA_EINVAL, "NULL argument");
  if (head < 0 || head >= p->desc.n_kv_heads) return fail(SWA_EINVAL, "head out of range");
  const auto &S = p->seqs[seq];
  if (pos < 0 || pos >= S.len[layer]) return fail(SWA_EINVAL, "position %lld not committed", (long long)pos);
  const int64_t d = p->desc.head_dim, es = p->es, hkv = p->desc.n_kv_heads;
  if (!p->full[layer]) {
    const int64_t w = p->desc.window;
    const int32_t a = p->kind_idx[layer];
    if (S.tags[a][pos % w] != pos) return fail(SWA_EINVAL, "position %lld no longer in the ring", (long long)pos);
    int64_t base = p->ring_off(seq, a);
    int64_t slot = pos % w;
    *k_off = base + ((int64_t)head * w + slot) * d * es;
    *v_off = base + hkv * w * d * es + ((int64_t)head * w + slot) * d * es;
    *v_stride = es;
  } else {
    const int32_t f = p->kind_idx[layer];
    int32_t pg = S.pages[f][pos / kPageTokens];
    int64_t r = pos % kPageTokens;
    int64_t base = p->page_off(f, pg);
    *k_off = base + ((int64_t)head * kPageTokens + r) * d * es;
    *v_off = base + hkv * kPageTokens * d * es + ((int64_t)head * kPageTokens + r) * d * es;
    *v_stride = es;
  }
  return SWA_OK;
}

int kvpool_window_safe_len(const swa_pool *p, int32_t donor, int64_t match_len, int64_t *out) {
  int rc = get_seq(p, donor);
  if (rc) return rc;
  if (!out) return fail(SWA_EINVAL, "out is NULL");
  if (match_len < 0) return fail(SWA_EINVAL, "match_len must be >= 0");
  const auto &S = p->seqs[donor];
  *out = window_safe(p, S, std::min(match_len, p->committed(S)));
  return SWA_OK;
}

int kvpool_append(swa_pool *p, int32_t seq, int32_t layer, const void *k, const void *v, int32_t n,
                  void *stream) {
  int rc = get_seq(p, seq);
  if (rc) return rc;
  if ((rc = get_layer(p, layer))) return rc;
  if (n < 1) return fail(SWA_EINVAL, "n must be >= 1");
  if (!p->planning && (!k || !v)) return fail(SWA_EINVAL, "k and v must be device pointers");
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto &S = p->seqs[seq];
  const int64_t L = S.len[layer];
  if (L + n > p->desc.max_seq_len) return fail(SWA_EINVAL, "sequence would exceed max_seq_len");
  const int32_t ki = p->kind_idx[layer];
  if (!p->full[layer]) {
    const int64_t w = p->desc.window;
    const int32_t n_write = (int32_t)std::min<int64_t>(n, w);
    const int32_t row0 = n - n_write;
    if (!p->planning) {
      hipError_t e = launch_append(p->view(layer), seq, k, v, row0, n_write, L, p->act_es, s);
      if (e != hipSuccess) return hip_fail(e, "append kernel");
    }
    auto &tags = S.tags[ki];
    for (int64_t t = row0; t < n; ++t) tags[(L + t) % w] = L + t;
  } else {
    auto &pg = S.pages[ki];
    const int64_t have = (int64_t)pg.size();
    const int64_t need = (L + n + kPageTokens - 1) / kPageTokens;
    auto &fl = p->free_pages[ki];
    if (need - have > (int64_t)fl.size())
      return fail(SWA_ENOMEM, "layer %d: need %lld pages, %zu free", layer, (long long)(need - have), fl.size());
    for (int64_t i = have; i < need; ++i) {
      int32_t id = fl.back();
      fl.pop_back();
      p->refcnt[ki][id] = 1;
      pg.push_back(id);
    }
    if ((rc = upload_table(p, seq, ki, have, need, s))) return rc;
    if (!p->planning) {
      hipError_t e = launch_append(p->view(layer), seq, k, v, 0, n, L, p->act_es, s);
      if (e != hipSuccess) return hip_fail(e, "append kernel");
    }
  }
  S.len[layer] = L + n;
  return SWA_OK;
}

int kvpool_append_batch(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer, const void *k,
                        const void *v, int32_t n, void *stream) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  int rc = get_layer(p, layer);
  if (rc) return rc;
  if (n_seqs < 1 || !seqs) return fail(SWA_EINVAL, "need n_seqs >= 1 and a seqs array");
  if (n < 1) return fail(SWA_EINVAL, "n must be >= 1");
  if (!p->planning && (!k || !v)) return fail(SWA_EINVAL, "k and v must be device pointers");
  std::vector<char> seen(p->desc.max_seqs, 0);
  const bool full = p->full[layer];
  const int32_t ki = p->kind_idx[layer];
  int64_t new_pages = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if ((rc = get_seq(p, seqs[i]))) return rc;
    if (seen[seqs[i]]) return fail(SWA_EINVAL, "sequence %d appears twice", seqs[i]);
    seen[seqs[i]] = 1;
    const int64_t L = p->seqs[seqs[i]].len[layer];
    if (L + n > p->desc.max_seq_len) return fail(SWA_EINVAL, "sequence %d would exceed max_seq_len", seqs[i]);
    if (full) new_pages += (L + n + kPageTokens - 1) / kPageTokens - (int64_t)p->seqs[seqs[i]].pages[ki].size();
  }
  if (full && new_pages > (int64_t)p->free_pages[ki].size())
    return fail(SWA_ENOMEM, "layer %d: need %lld pages, %zu free", layer, (long long)new_pages,
                p->free_pages[ki].size());
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t w = p->desc.window;
  const int32_t n_write = full ? n : (int32_t)std::min<int64_t>(n, w);
  const int32_t row0 = n - n_write;
  const int64_t row_elems = (int64_t)p->desc.n_kv_heads * p->desc.head_dim;
  // metadata for the device, in groups that fit the landing zone
  std::vector<SeqEntry> ent;
  std::vector<TablePatch> patches;
  auto flush = [&](int32_t first) -> int {
    if (ent.empty()) return SWA_OK;
    if (!p->planning) {
      char *zone = p->arena + p->off_meta;
      const int64_t pb = align_up((int64_t)(sizeof(SeqEntry) * ent.size()), 256);
      int r = SWA_OK;
      const char *d_ent = cached_table(p, ent.data(), sizeof(SeqEntry) * ent.size(), s, r);
      if (r) return r;
      if (!d_ent) {
        if ((r = p->staging.upload(zone, ent.data(), sizeof(SeqEntry) * ent.size(), s))) return r;
        d_ent = zone;
      }
      if (!patches.empty()) {
        if ((r = p->staging.upload(zone + pb, patches.data(), sizeof(TablePatch) * patches.size(), s))) return r;
        hipError_t e = launch_table_patch(reinterpret_cast<int32_t *>(p->arena + p->off_tables),
                                          reinterpret_cast<const TablePatch *>(zone + pb), (int32_t)patches.size(), s);
        if (e != hipSuccess) return hip_fail(e, "page-table patch kernel");
      }
      const int es = p->act_es;  // element size of the appended k/v
      hipError_t e = launch_append_batch(p->view(layer), reinterpret_cast<const SeqEntry *>(d_ent), (int32_t)ent.size(),
                                         static_cast<const char *>(k) + (int64_t)first * n * row_elems * es,
                                         static_cast<const char *>(v) + (int64_t)first * n * row_elems * es,
                                         n, row0, n_write, es, s);
      if (e != hipSuccess) return hip_fail(e, "batched append kernel");
    }
    ent.clear();
    patches.clear();
    return SWA_OK;
  };
  int32_t group_first = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto &S = p->seqs[seqs[i]];
    const int64_t L = S.len[layer];
    ent.push_back({seqs[i], 0, L});
    if (full) {
      auto &pg = S.pages[ki];
      const int64_t need = (L + n + kPageTokens - 1) / kPageTokens;
      for (int64_t j = (int64_t)pg.size(); j < need; ++j) {
        int32_t id = p->free_pages[ki].back();
        p->free_pages[ki].pop_back();
        p->refcnt[ki][id] = 1;
        pg.push_back(id);
        const int64_t idx = ((int64_t)ki * p->desc.max_seqs + seqs[i]) * p->maxp + j;
        patches.push_back({idx, id, 0});
      }
    } else {
      auto &tags = S.tags[ki];
      for (int64_t t = row0; t < n; ++t) tags[(L + t) % w] = L + t;
    }
    S.len[layer] = L + n;
    const int64_t bytes = align_up((int64_t)(sizeof(SeqEntry) * ent.size()), 256) +
                          (int64_t)sizeof(TablePatch) * ((int64_t)patches.size() + (n / kPageTokens + 2));
    if (bytes > kMetaBytes - 4096 || i == n_seqs - 1) {
      if ((rc = flush(group_first))) return rc;
      group_first = i + 1;
    }
  }
  return SWA_OK;
}

int kvpool_rope(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer, void *q, int32_t n_q_heads,
                void *k, int32_t n, swa_dtype dt, void *stream) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  if (p->planning) return fail(SWA_EINVAL, "RoPE needs an arena-backed pool");
  if (p->rope_hi_rows == 0) return fail(SWA_EINVAL, "pool was created without RoPE (rope_base 0)");
  int rc = get_layer(p, layer);
  if (rc) return rc;
  if (n_seqs < 1 || !seqs) return fail(SWA_EINVAL, "need n_seqs >= 1 and a seqs array");
  if (n < 1) return fail(SWA_EINVAL, "n must be >= 1");
  if (!q && !k) return fail(SWA_EINVAL, "q and k are both NULL");
  if (q && n_q_heads < 1) return fail(SWA_EINVAL, "n_q_heads must be >= 1");
  const swa_dtype act = p->desc.kv_dtype == SWA_F32 ? SWA_F32 : SWA_BF16;
  if (dt != act) return fail(SWA_EINVAL, "activation dtype must be %s for this pool", act == SWA_F32 ? "fp32" : "bf16");
  if ((int64_t)n_seqs * n > INT32_MAX) return fail(SWA_EINVAL, "too many tokens in one call");
  std::vector<SeqEntry> ent((size_t)n_seqs);
  for (int32_t i = 0; i < n_seqs; ++i) {
    if ((rc = get_seq(p, seqs[i]))) return rc;
    const int64_t L = p->seqs[seqs[i]].len[layer];
    if (L + n > p->desc.max_seq_len) return fail(SWA_EINVAL, "sequence %d: positions would exceed max_seq_len", seqs[i]);
    ent[(size_t)i] = {seqs[i], 0, L};
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int es = p->act_es;
  const int hkv = p->desc.n_kv_heads, d = p->desc.head_dim;
  RopeArgs a{};
  a.lo_tab = reinterpret_cast<const float2 *>(p->arena + p->off_rope);
  a.hi_tab = a.lo_tab + kRopeLo * (d / 2);
  a.n = n;
  a.hq = q ? n_q_heads : 0;
  a.hkv = k ? hkv : 0;
  a.d = d;
  a.style = p->desc.rope_style;
  // one sequence: its first position is a kernel argument; several: the list goes through the
  // landing zone, in groups that fit it
  const int32_t group = n_seqs == 1 ? 1 : (int32_t)((kMetaBytes - 4096) / (int64_t)sizeof(SeqEntry));
  for (int32_t first = 0; first < n_seqs; first += group) {
    const int32_t cnt = std::min(group, n_seqs - first);
    const int64_t tok0 = (int64_t)first * n;
    a.q = q ? static_cast<char *>(q) + tok0 * a.hq * d * es : nullptr;
    a.k = k ? static_cast<char *>(k) + tok0 * a.hkv * d * es : nullptr;
    a.tokens = cnt * n;
    if (n_seqs == 1) {
      a.ent = nullptr;
      a.pos0 = ent[0].prior;
    } else {
      const char *d_ent = cached_table(p, ent.data() + first, sizeof(SeqEntry) * (size_t)cnt, s, rc);
      if (rc) return rc;
      if (!d_ent) {
        char *zone = p->arena + p->off_meta;
        if ((rc = p->staging.upload(zone, ent.data() + first, sizeof(SeqEntry) * (size_t)cnt, s))) return rc;
        d_ent = zone;
      }
      a.ent = reinterpret_cast<const SeqEntry *>(d_ent);
      a.pos0 = 0;
    }
    hipError_t e = launch_rope(a, es, s);
    if (e != hipSuccess) return hip_fail(e, "RoPE kernel");
  }
  return SWA_OK;
}

}  // extern "C"

namespace {

// Open a sequence whose first `reuse_len` tokens are a source's: SWA rings copied from the arena
// bytes at `ring_src` (SWA layer a's ring at ring_src + a * ring_src_stride), ring tags restricted
// to positions below reuse_len, whole pages below reuse_len shared by reference, the partial last
// page copied.
int fork_from(swa_pool *p, int64_t ring_src, int64_t ring_src_stride, const std::vector<std::vector<int64_t>> &src_tags,
              const std::vector<std::vector<int32_t>> &src_pages, int64_t reuse_len, int32_t *seq, void *stream) {
  if (p->free_seqs.empty()) return fail(SWA_ENOMEM, "no free sequence slot");
  const int64_t shared = reuse_len / kPageTokens;
  const bool partial = reuse_len % kPageTokens != 0;
  if (partial)
    for (int32_t f = 0; f < p->n_full; ++f)
      if (p->free_pages[f].empty()) return fail(SWA_ENOMEM, "no free page for the partial page copy");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc;
  int32_t ns;
  kvpool_seq_open(p, &ns);
  auto &N = p->seqs[ns];
  CopyList jobs{};
  auto flush = [&]() -> int {
    if (jobs.n == 0 || p->planning) { jobs.n = 0; return SWA_OK; }
    hipError_t e = launch_copy_list(p->arena, jobs, s);
    jobs.n = 0;
    return e == hipSuccess ? SWA_OK : hip_fail(e, "fork copy kernel");
  };
  for (int32_t a = 0; a < p->n_swa; ++a) {
    jobs.job[jobs.n++] = {ring_src + a * ring_src_stride, p->ring_off(ns, a), p->ring_bytes};
    if (jobs.n == kMaxCopyJobs && (rc = flush())) return rc;
  }
  if (p->n_swa > 0) {
    for (int32_t a = 0; a < p->n_swa; ++a) {
      N.tags[a] = src_tags[a];
      for (auto &t : N.tags[a])
        if (t >= reuse_len) t = -1;
    }
  }
  for (int32_t f = 0; f < p->n_full; ++f) {
    auto &pg = N.pages[f];
    pg.assign(src_pages[f].begin(), src_pages[f].begin() + shared);
    for (int32_t id : pg) p->refcnt[f][id]++;
    if (partial) {
      int32_t id = p->free_pages[f].back();
      p->free_pages[f].pop_back();
      p->refcnt[f][id] = 1;
      jobs.job[jobs.n++] = {p->page_off(f, src_pages[f][shared]), p->page_off(f, id), p->page_bytes};
      pg.push_back(id);
      if (jobs.n == kMaxCopyJobs && (rc = flush())) return rc;
    }
    if ((rc = upload_table(p, ns, f, 0, (int64_t)pg.size(), s))) return rc;
  }
  if ((rc = flush())) return rc;
  for (auto &l : N.len) l = reuse_len;
  *seq = ns;
  return SWA_OK;
}

}  // namespace

extern "C" {

int kvpool_seq_fork(swa_pool *p, int32_t donor, int64_t reuse_len, int32_t *seq, void *stream) {
  int rc = get_seq(p, donor);
  if (rc) return rc;
  if (!seq) return fail(SWA_EINVAL, "seq is NULL");
  if (reuse_len < 0) return fail(SWA_EINVAL, "reuse_len must be >= 0");
  const auto &D = p->seqs[donor];
  const int64_t committed = p->committed(D);
  if (reuse_len > committed)
    return fail(SWA_EINVAL, "reuse_len %lld exceeds the donor's committed length %lld",
                (long long)reuse_len, (long long)committed);
  const int64_t safe = window_safe(p, D, reuse_len);
  if (safe != reuse_len)
    return fail(SWA_EINVAL, "reuse_len %lld is not window-safe (window-safe length is %lld)",
                (long long)reuse_len, (long long)safe);
  return fork_from(p, p->ring_off(donor, 0), p->ring_layer_stride(), D.tags, D.pages, reuse_len, seq, stream);
}

int kvpool_snapshot(swa_pool *p, int32_t seq, int32_t *snap, void *stream) {
  int rc = get_seq(p, seq);
  if (rc) return rc;
  if (!snap) return fail(SWA_EINVAL, "snap is NULL");
  const auto &S = p->seqs[seq];
  const int64_t m = p->committed(S);
  for (int64_t l : S.len)
    if (l != m) return fail(SWA_EINVAL, "sequence %d: layers hold different lengths", seq);
  int32_t id = -1;
  for (int32_t i = 0; i < (int32_t)p->snaps.size(); ++i)
    if (!p->snaps[i].used) { id = i; break; }
  if (id < 0) return fail(SWA_ENOMEM, "no free snapshot slot (max_snapshots = %d)", p->desc.max_snapshots);
  auto &Z = p->snaps[id];
  if (p->n_swa > 0 && !p->planning) {
    // a snapshot keeps its rings contiguous ([SWA layer] within the snapshot's slot)
    CopyList jobs{};
    for (int32_t a = 0; a < p->n_swa; ++a) {
      jobs.job[jobs.n++] = {p->ring_off(seq, a), p->snap_off(id) + a * p->ring_bytes, p->ring_bytes};
      if (jobs.n == kMaxCopyJobs || a == p->n_swa - 1) {
        hipError_t e = launch_copy_list(p->arena, jobs, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_fail(e, "snapshot copy kernel");
        jobs.n = 0;
      }
    }
  }
  Z.tags = S.tags;
  Z.pages.assign(p->n_full, {});
  const int64_t held = (m + kPageTokens - 1) / kPageTokens;
  for (int32_t f = 0; f < p->n_full; ++f) {
    Z.pages[f].assign(S.pages[f].begin(), S.pages[f].begin() + held);
    for (int32_t pg : Z.pages[f]) p->refcnt[f][pg]++;
  }
  Z.len = m;
  Z.used = true;
  *snap = id;
  return SWA_OK;
}

int kvpool_snapshot_len(const swa_pool *p, int32_t snap, int64_t *len) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  if (!len) return fail(SWA_EINVAL, "len is NULL");
  if (snap < 0 || snap >= (int32_t)p->snaps.size() || !p->snaps[snap].used)
    return fail(SWA_EINVAL, "snapshot %d is not held", snap);
  *len = p->snaps[snap].len;
  return SWA_OK;
}

int kvpool_snapshot_release(swa_pool *p, int32_t snap) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  if (snap < 0 || snap >= (int32_t)p->snaps.size() || !p->snaps[snap].used)
    return fail(SWA_EINVAL, "snapshot %d is not held", snap);
  auto &Z = p->snaps[snap];
  for (int32_t f = 0; f < p->n_full; ++f)
    for (int32_t pg : Z.pages[f])
      if (--p->refcnt[f][pg] == 0) p->free_pages[f].push_back(pg);
  Z = swa_pool::Snap{};
  return SWA_OK;
}

int kvpool_seq_fork_snapshot(swa_pool *p, int32_t snap, int32_t *seq, void *stream) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  if (!seq) return fail(SWA_EINVAL, "seq is NULL");
  if (snap < 0 || snap >= (int32_t)p->snaps.size() || !p->snaps[snap].used)
    return fail(SWA_EINVAL, "snapshot %d is not held", snap);
  const auto &Z = p->snaps[snap];
  return fork_from(p, p->snap_off(snap), p->ring_bytes, Z.tags, Z.pages, Z.len, seq, stream);
}

}  // extern "C"

// =============================================================================================
// C ABI: attention
// =============================================================================================

namespace {

struct DecodePlan {
  std::vector<SeqEntry> seqs;
  std::vector<WorkItem> items;
  std::vector<CombineEntry> combine;
  int32_t n_parts = 0, max_split = 0;
  int64_t off_items = 0, off_combine = 0, off_ml = 0, off_o = 0, bytes = 0;
};

// Split of a full layer's prior keys into work items: whole pages, `split` keys per item.
// Keys per split-K item of a full-layer decode call.  One item runs on one 4-wave workgroup (each
// wave takes a quarter of the keys; the waves merge in LDS) and two workgroups run per CU, so
// 2 * n_cu items are in flight at once.  Starting from 4096 keys, the split is shrunk so that the
// items fill a whole number of such rounds: e.g. one 1M-token sequence x 4 KV heads takes 2.03
// rounds at 4096 keys (a nearly empty third round) but 2.96 rounds at 2816.  Multiples of 128 keep
// every wave's first key on a page boundary.
int32_t full_split_keys(const swa_pool *p, int64_t total_key_heads) {
  const int64_t cap = 2LL * p->n_cu;
  const int64_t base = 4096;
  const int64_t rounds = std::max<int64_t>(1, (total_key_heads + base * cap - 1) / (base * cap));
  int64_t split = (total_key_heads + rounds * cap - 1) / (rounds * cap);
  split = (split + 127) / 128 * 128;
  return (int32_t)std::min<int64_t>(base, std::max<int64_t>(512, split));
}

int check_common(const swa_pool *p, int32_t layer, int32_t hq, swa_dtype dt) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  if (p->planning) return fail(SWA_EINVAL, "attention needs an arena-backed pool");
  int rc = get_layer(p, layer);
  if (rc) return rc;
  const swa_dtype act = p->desc.kv_dtype == SWA_F32 ? SWA_F32 : SWA_BF16;
  if (dt != act) return fail(SWA_EINVAL, "activation dtype must be %s for this pool", act == SWA_F32 ? "fp32" : "bf16");
  if (hq < 1 || hq % p->desc.n_kv_heads) return fail(SWA_EINVAL, "n_q_heads must be a positive multiple of n_kv_heads");
  if (dt == SWA_BF16) {
    int g = hq / p->desc.n_kv_heads;
    if (g > 32 || (32 % g) != 0) return fail(SWA_EINVAL, "bf16 path needs Hq/Hkv in {1,2,4,8,16,32}");
  }
  return SWA_OK;
}

int build_plan(const swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer, int32_t q_len,
               int32_t hq, DecodePlan &plan) {
  if (n_seqs < 1 || !seqs) return fail(SWA_EINVAL, "need n_seqs >= 1 and a seqs array");
  if (q_len < 1 || q_len > 4) return fail(SWA_EINVAL, "q_len must be in 1..4");
  std::vector<char> seen(p->desc.max_seqs, 0);
  const int32_t hkv = p->desc.n_kv_heads, d = p->desc.head_dim;
  const bool full = p->full[layer];
  int64_t total = 0;
  plan.seqs.resize(n_seqs);
  for (int32_t i = 0; i < n_seqs; ++i) {
    int rc = get_seq(p, seqs[i]);
    if (rc) return rc;
    if (seen[seqs[i]]) return fail(SWA_EINVAL, "sequence %d appears twice", seqs[i]);
    seen[seqs[i]] = 1;
    int64_t L = p->seqs[seqs[i]].len[layer];
    if (L + q_len > p->desc.max_seq_len) return fail(SWA_EINVAL, "sequence %d would exceed max_seq_len", seqs[i]);
    plan.seqs[i] = {seqs[i], 0, L};
    total += L;
  }
  // Split of the prior keys (full layers).  Uniform: one split for the whole call.  Bucketed: the
  // sequences fall into the length buckets 0-64K, 64K-256K and 256K+ ([MiMo-review] §潜在力を本番へ,
  // length bucketing keeps batches homogeneous), each bucket gets the split that fills whole rounds
  // for its own keys, and the work list runs longest bucket first, whole splits before the shorter
  // tail pieces (longest first), so the last round is filled with the smallest items.
  const bool bucketed = full && p->desc.decode_plan == SWA_PLAN_BUCKETED;
  auto bucket_of = [](int64_t L) { return L < 65536 ? 0 : L < 262144 ? 1 : 2; };
  int32_t split_of[3] = {0, 0, 0};
  if (full) {
    if (bucketed) {
      int64_t tot[3] = {0, 0, 0};
      for (int32_t i = 0; i < n_seqs; ++i) tot[bucket_of(plan.seqs[i].prior)] += plan.seqs[i].prior;
      for (int b = 0; b < 3; ++b) split_of[b] = full_split_keys(p, tot[b] * hkv);
    } else {
      split_of[0] = split_of[1] = split_of[2] = full_split_keys(p, total * hkv);
    }
  }
  plan.combine.assign((size_t)n_seqs * hkv, {0, 0});
  if (!full) {
    for (int32_t i = 0; i < n_seqs; ++i)
      for (int32_t h = 0; h < hkv; ++h)
        plan.items.push_back({i, h, 0, (int32_t)std::min<int64_t>(plan.seqs[i].prior, p->desc.window), -1, 1});
  } else {
    // items of one (sequence, head): whole splits, then the shorter tail piece (or the whole row)
    std::vector<WorkItem> tails;
    auto emit = [&](int32_t i, int32_t h, std::vector<WorkItem> &whole, std::vector<WorkItem> &tail) {
      const int64_t L = plan.seqs[i].prior;
      const int32_t split = split_of[bucket_of(L)];
      const int64_t nsplit = std::max<int64_t>(1, (L + split - 1) / split);
      if (nsplit == 1) {
        tail.push_back({i, h, 0, (int32_t)L, -1, 1});
        return;
      }
      plan.combine[(size_t)i * hkv + h] = {plan.n_parts, (int32_t)nsplit};
      plan.max_split = std::max(plan.max_split, (int32_t)nsplit);
      for (int64_t s = 0; s < nsplit; ++s) {
        const int64_t b = s * split, e = std::min<int64_t>(L, b + split);
        auto &dst = e - b == split ? whole : tail;
        dst.push_back({i, h, (int32_t)b, (int32_t)e, plan.n_parts++, s == nsplit - 1 ? 1 : 0});
      }
    };
    if (!bucketed) {
      for (int32_t i = 0; i < n_seqs; ++i)
        for (int32_t h = 0; h < hkv; ++h) {
          emit(i, h, plan.items, tails);
          plan.items.insert(plan.items.end(), tails.begin(), tails.end());
          tails.clear();
        }
    } else {
      for (int b = 2; b >= 0; --b) {
        for (int32_t i = 0; i < n_seqs; ++i)
          if (bucket_of(plan.seqs[i].prior) == b)
            for (int32_t h = 0; h < hkv; ++h) emit(i, h, plan.items, tails);
        std::stable_sort(tails.begin(), tails.end(), [](const WorkItem &x, const WorkItem &y) {
          return x.k_end - x.k_begin > y.k_end - y.k_begin;
        });
        plan.items.insert(plan.items.end(), tails.begin(), tails.end());
        tails.clear();
      }
    }
  }
  for (WorkItem &w : plan.items) {
    w.seq = plan.seqs[w.si].seq;
    w.prior = plan.seqs[w.si].prior;
  }
  const int64_t rows = (int64_t)(hq / hkv) * q_len;
  if (rows > 32) {  // 32 query rows per item: one copy of every item per further 32-row block
    std::vector<WorkItem> blocks;
    blocks.reserve(plan.items.size() * (size_t)((rows + 31) / 32));
    for (const WorkItem &w : plan.items)
      for (int32_t r0 = 0; r0 < rows; r0 += 32) {
        WorkItem c = w;
        c.row0 = r0;
        blocks.push_back(c);
      }
    plan.items.swap(blocks);
  }
  plan.off_items = align_up((int64_t)sizeof(SeqEntry) * n_seqs, 256);
  plan.off_combine = align_up(plan.off_items + (int64_t)sizeof(WorkItem) * plan.items.size(), 256);
  plan.off_ml = align_up(plan.off_combine + (int64_t)sizeof(CombineEntry) * plan.combine.size(), 256);
  plan.off_o = align_up(plan.off_ml + (int64_t)plan.n_parts * rows * 2 * 4, 256);
  plan.bytes = align_up(plan.off_o + (int64_t)plan.n_parts * rows * d * 4, 256);
  return SWA_OK;
}

int run_decode(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer, const void *q,
               const void *k_new, const void *v_new, int32_t q_len, int32_t hq, swa_dtype dt,
               void *out, void *ws, int64_t ws_bytes, void *stream) {
  DecodePlan plan;
  int rc = build_plan(p, n_seqs, seqs, layer, q_len, hq, plan);
  if (rc) return rc;
  if (!q || !k_new || !v_new || !out) return fail(SWA_EINVAL, "q, k_new, v_new and out must be device pointers");
  if (!ws || ws_bytes < plan.bytes)
    return fail(SWA_ENOMEM, "workspace has %lld bytes, call needs %lld", (long long)ws_bytes, (long long)plan.bytes);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(SWA_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *w = static_cast<char *>(ws);
  // Sequence list and work list (items, then the combine table) from the arena's table cache; if
  // either does not fit a slot, all three go to the head of the workspace in one upload.
  const char *d_seqs, *d_items, *d_comb;
  {
    const int64_t comb_off = plan.off_combine - plan.off_items;
    std::vector<char> work((size_t)(plan.off_ml - plan.off_items), 0);
    std::memcpy(work.data(), plan.items.data(), sizeof(WorkItem) * plan.items.size());
    std::memcpy(work.data() + comb_off, plan.combine.data(), sizeof(CombineEntry) * plan.combine.size());
    d_seqs = cached_table(p, plan.seqs.data(), sizeof(SeqEntry) * plan.seqs.size(), s, rc);
    if (rc) return rc;
    const char *d_work = d_seqs ? cached_table(p, work.data(), work.size(), s, rc) : nullptr;
    if (rc) return rc;
    if (d_seqs && d_work) {
      d_items = d_work;
      d_comb = d_work + comb_off;
    } else {
      std::vector<char> blob((size_t)plan.off_ml, 0);
      std::memcpy(blob.data(), plan.seqs.data(), sizeof(SeqEntry) * plan.seqs.size());
      std::memcpy(blob.data() + plan.off_items, work.data(), work.size());
      if ((rc = p->staging.upload(w, blob.data(), blob.size(), s))) return rc;
      d_seqs = w;
      d_items = w + plan.off_items;
      d_comb = w + plan.off_combine;
    }
  }
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->desc.head_dim));
  if (dt == SWA_F32) {
    F32AttnArgs a{};
    a.L = p->view(layer);
    a.q = static_cast<const float *>(q);
    a.k_new = static_cast<const float *>(k_new);
    a.v_new = static_cast<const float *>(v_new);
    a.out = static_cast<float *>(out);
    a.seqs = reinterpret_cast<const SeqEntry *>(d_seqs);
    a.n_seqs = n_seqs;
    a.q_len = q_len;
    a.hq = hq;
    a.scale_log2 = scale_log2;
    hipError_t e = launch_attn_f32(a, s);
    return e == hipSuccess ? SWA_OK : hip_fail(e, "fp32 decode kernel");
  }
  DecodeArgs a{};
  a.L = p->view(layer);
  a.q = static_cast<const uint16_t *>(q);
  a.k_new = static_cast<const uint16_t *>(k_new);
  a.v_new = static_cast<const uint16_t *>(v_new);
  a.out = static_cast<uint16_t *>(out);
  a.seqs = reinterpret_cast<const SeqEntry *>(d_seqs);
  a.items = reinterpret_cast<const WorkItem *>(d_items);
  a.combine = reinterpret_cast<const CombineEntry *>(d_comb);
  a.part_ml = reinterpret_cast<float *>(w + plan.off_ml);
  a.part_o = reinterpret_cast<float *>(w + plan.off_o);
  a.n_items = (int32_t)plan.items.size();
  a.n_parts = plan.n_parts;
  a.max_split = plan.max_split;
  a.n_seqs = n_seqs;
  a.q_len = q_len;
  a.hq = hq;
  a.scale_log2 = scale_log2;
  hipError_t e = launch_decode_bf16(a, s);
  return e == hipSuccess ? SWA_OK : hip_fail(e, "bf16 decode kernels");
}

int run_prefill(swa_pool *p, int32_t seq, int32_t layer, const void *q, const void *k, const void *v,
                int32_t n, int32_t hq, swa_dtype dt, void *out, void *stream) {
  int rc = get_seq(p, seq);
  if (rc) return rc;
  if (n < 1) return fail(SWA_EINVAL, "n must be >= 1");
  if (!q || !k || !v || !out) return fail(SWA_EINVAL, "q, k, v and out must be device pointers");
  const int64_t L = p->seqs[seq].len[layer];
  if (L + n > p->desc.max_seq_len) return fail(SWA_EINVAL, "chunk would exceed max_seq_len");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->desc.head_dim));
  hipError_t e;
  if (dt == SWA_F32) {
    F32AttnArgs a{};
    a.L = p->view(layer);
    a.q = static_cast<const float *>(q);
    a.k_new = static_cast<const float *>(k);
    a.v_new = static_cast<const float *>(v);
    a.out = static_cast<float *>(out);
    a.seqs = nullptr;
    a.seq = seq;
    a.prior = L;
    a.n_seqs = 1;
    a.q_len = n;
    a.hq = hq;
    a.scale_log2 = scale_log2;
    e = launch_attn_f32(a, s);
  } else {
    PrefillArgs a{};
    a.L = p->view(layer);
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    if (p->desc.rope_fused) {
      // fused RoPE: the chunk's keys turn once, into the arena, before the attention kernel reads
      // them (the kernel turns each query as it loads it); the caller's k stays unrotated
      if (n > p->desc.max_chunk) return fail(SWA_EINVAL, "chunk of %d tokens exceeds max_chunk %d", n, p->desc.max_chunk);
      RopeArgs r{};
      r.k = static_cast<char *>(const_cast<void *>(k));
      r.kout = p->arena + p->off_rchunk;
      r.pos0 = L;
      r.lo_tab = a.L.rope_lo;
      r.hi_tab = a.L.rope_hi;
      r.tokens = n;
      r.n = n;
      r.hkv = p->desc.n_kv_heads;
      r.d = p->desc.head_dim;
      r.style = p->desc.rope_style;
      if ((e = launch_rope(r, 2, s)) != hipSuccess) return hip_fail(e, "RoPE of the chunk's keys");
      a.k = reinterpret_cast<const uint16_t *>(r.kout);
    }
    a.v = static_cast<const uint16_t *>(v);
    a.out = static_cast<uint16_t *>(out);
    a.seq = seq;
    a.prior = L;
    a.n = n;
    a.hq = hq;
    a.scale_log2 = scale_log2;
    a.n_cu = p->n_cu;
    e = launch_prefill_bf16(a, s);
  }
  return e == hipSuccess ? SWA_OK : hip_fail(e, "prefill kernel");
}

}  // namespace

extern "C" {

int swa_attn_prefill(swa_pool *p, int32_t seq, int32_t layer, const void *q, const void *k,
                     const void *v, int32_t n, int32_t n_q_heads, swa_dtype dt, void *out,
                     void *stream) {
  int rc = check_common(p, layer, n_q_heads, dt);
  if (rc) return rc;
  if (p->full[layer]) return fail(SWA_EINVAL, "layer %d is a full-attention layer (use full_attn)", layer);
  return run_prefill(p, seq, layer, q, k, v, n, n_q_heads, dt, out, stream);
}

int swa_attn_decode(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer,
                    const void *q, const void *k_new, const void *v_new, int32_t q_len,
                    int32_t n_q_heads, swa_dtype dt, void *out, void *workspace, int64_t ws_bytes,
                    void *stream) {
  int rc = check_common(p, layer, n_q_heads, dt);
  if (rc) return rc;
  if (p->full[layer]) return fail(SWA_EINVAL, "layer %d is a full-attention layer (use full_attn)", layer);
  return run_decode(p, n_seqs, seqs, layer, q, k_new, v_new, q_len, n_q_heads, dt, out, workspace,
                    ws_bytes, stream);
}

int full_attn(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer, const void *q,
              const void *k_new, const void *v_new, int32_t q_len_or_chunk, int32_t n_q_heads,
              swa_dtype dt, void *out, void *workspace, int64_t ws_bytes, void *stream) {
  int rc = check_common(p, layer, n_q_heads, dt);
  if (rc) return rc;
  if (!p->full[layer]) return fail(SWA_EINVAL, "layer %d is a sliding-window layer", layer);
  if (q_len_or_chunk < 1) return fail(SWA_EINVAL, "q_len_or_chunk must be >= 1");
  if (q_len_or_chunk > 4) {
    if (n_seqs != 1 || !seqs) return fail(SWA_EINVAL, "a full-layer prefill takes exactly one sequence");
    return run_prefill(p, seqs[0], layer, q, k_new, v_new, q_len_or_chunk, n_q_heads, dt, out, stream);
  }
  return run_decode(p, n_seqs, seqs, layer, q, k_new, v_new, q_len_or_chunk, n_q_heads, dt, out,
                    workspace, ws_bytes, stream);
}

int64_t swa_attn_workspace_bytes(const swa_pool *p, int32_t n_seqs, const int32_t *seqs,
                                 int32_t layer, int32_t q_len_or_chunk, int32_t n_q_heads) {
  if (!p) return fail(SWA_EINVAL, "pool is NULL");
  int rc = get_layer(p, layer);
  if (rc) return rc;
  if (n_q_heads < 1 || n_q_heads % p->desc.n_kv_heads) return fail(SWA_EINVAL, "bad n_q_heads");
  if (q_len_or_chunk > 4 && p->full[layer]) return 0;
  DecodePlan plan;
  if ((rc = build_plan(p, n_seqs, seqs, layer, q_len_or_chunk, n_q_heads, plan))) return rc;
  return plan.bytes;
}

}  // extern "C"
