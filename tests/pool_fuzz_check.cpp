// Host-only fuzz of libswa's pool metadata (csrc/pool.cpp) on planning pools, built with g++ and
// AddressSanitizer/UBSan by tests/test_pool_fuzz.py.  No GPU: the HIP runtime entry points and
// the kernel launchers are stubs that abort if reached (planning pools never reach them).
//
// Random sequences of open / append / batched append / window-safe query / fork / snapshot /
// fork-from-snapshot / release / close run against the C ABI and against an independent model:
// ring tags (slot p mod w holds the last committed p, [SWA-theory] §Rolling Buffer KV Cache
// Eq.(7)), page holdings as abstract ids (whole pages below a reuse length shared, a partial last
// page copied), the window-safe length by brute force (every p in [max(0, m-w), m) still in its
// slot in every SWA layer), free pages, byte accounting and the error codes of refused calls.
// Prints "pool_fuzz_mismatches=0" when every check agreed.

#include "swa.h"
#include "swa_internal.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#define DIE(name)                                          \
  do {                                                     \
    std::fprintf(stderr, "stub %s reached\n", name);       \
    std::abort();                                          \
  } while (0)

extern "C" {
hipError_t hipDeviceGetAttribute(int *, hipDeviceAttribute_t, int) { DIE("hipDeviceGetAttribute"); }
hipError_t hipEventCreateWithFlags(hipEvent_t *, unsigned) { DIE("hipEventCreateWithFlags"); }
hipError_t hipEventDestroy(hipEvent_t) { DIE("hipEventDestroy"); }
hipError_t hipEventQuery(hipEvent_t) { DIE("hipEventQuery"); }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { DIE("hipEventRecord"); }
hipError_t hipEventSynchronize(hipEvent_t) { DIE("hipEventSynchronize"); }
hipError_t hipGetDevice(int *) { DIE("hipGetDevice"); }
const char *hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipHostFree(void *) { DIE("hipHostFree"); }
hipError_t hipHostMalloc(void **, size_t, unsigned int) { DIE("hipHostMalloc"); }
hipError_t hipMemcpy(void *, const void *, size_t, hipMemcpyKind) { DIE("hipMemcpy"); }
hipError_t hipMemcpyAsync(void *, const void *, size_t, hipMemcpyKind, hipStream_t) { DIE("hipMemcpyAsync"); }
}

namespace swa {
hipError_t launch_copy_list(char *, const CopyList &, hipStream_t) { DIE("launch_copy_list"); }
hipError_t launch_clock_probe(int64_t *, int64_t, int64_t, hipStream_t) { DIE("launch_clock_probe"); }
hipError_t launch_table_patch(int32_t *, const TablePatch *, int32_t, hipStream_t) { DIE("launch_table_patch"); }
hipError_t launch_append_batch(const LayerView &, const SeqEntry *, int32_t, const void *, const void *, int32_t,
                               int32_t, int32_t, int, hipStream_t) { DIE("launch_append_batch"); }
hipError_t launch_append(const LayerView &, int32_t, const void *, const void *, int32_t, int32_t, int64_t, int,
                         hipStream_t) { DIE("launch_append"); }
hipError_t launch_rope(const RopeArgs &, int, hipStream_t) { DIE("launch_rope"); }
hipError_t launch_attn_f32(const F32AttnArgs &, hipStream_t) { DIE("launch_attn_f32"); }
hipError_t launch_prefill_bf16(const PrefillArgs &, hipStream_t) { DIE("launch_prefill_bf16"); }
hipError_t launch_decode_bf16(const DecodeArgs &, hipStream_t) { DIE("launch_decode_bf16"); }
}  // namespace swa

namespace {

constexpr int NL = 7;   // layers; layer 6 is the full one (default map l % 7 == 6)
constexpr int NSWA = 6;
constexpr int FULL = 6;

struct MSeq {
  bool open = false;
  std::vector<int64_t> len = std::vector<int64_t>(NL, 0);
  std::vector<std::vector<int64_t>> tags;  // per SWA layer, w entries
  std::vector<long> pages;                  // abstract page ids of the full layer
};
struct MSnap {
  bool used = false;
  int64_t len = 0;
  std::vector<std::vector<int64_t>> tags;
  std::vector<long> pages;
};

long mismatches = 0;
void check(bool ok, const char *what, long step) {
  if (!ok) {
    ++mismatches;
    if (mismatches < 20) std::printf("mismatch at step %ld: %s\n", step, what);
  }
}

int swa_index(int layer) { return layer < FULL ? layer : -1; }

}  // namespace

int main() {
  std::mt19937_64 rng(20261203);
  auto uni = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };
  long step = 0;
  for (int trial = 0; trial < 160; ++trial) {
    const int w = (int)uni(1, 20);
    const int max_seqs = 6, max_snaps = 3;
    const int64_t n_pages = uni(8, 96), max_len = 600;
    swa_pool_desc d{};
    d.n_layers = NL;
    d.layer_is_full = nullptr;
    d.window = w;
    d.n_kv_heads = 1;
    d.head_dim = 64;
    d.kv_dtype = SWA_BF16;
    d.page_tokens = 16;
    d.pages_per_full_layer = n_pages;
    d.max_seqs = max_seqs;
    d.max_seq_len = max_len;
    d.max_snapshots = max_snaps;
    swa_pool *p = nullptr;
    if (kvpool_create(&d, nullptr, 0, &p) != SWA_OK) { std::printf("create failed\n"); return 1; }
    std::vector<MSeq> seqs(max_seqs);
    std::vector<MSnap> snaps(max_snaps);
    long next_id = 0;
    const int64_t tok_bytes = 2 * 1 * 64 * 2, page_bytes = 16 * tok_bytes;

    auto held = [&]() {
      std::set<long> h;
      for (auto &s : seqs)
        if (s.open) h.insert(s.pages.begin(), s.pages.end());
      for (auto &z : snaps)
        if (z.used) h.insert(z.pages.begin(), z.pages.end());
      return h;
    };
    auto committed = [](const MSeq &s) { return *std::min_element(s.len.begin(), s.len.end()); };
    auto safe_brute = [&](const std::vector<std::vector<int64_t>> &tags, int64_t hi) {
      for (int64_t m = hi; m >= 0; --m) {
        bool ok = true;
        for (int a = 0; a < NSWA && ok; ++a)
          for (int64_t q = std::max<int64_t>(0, m - w); q < m && ok; ++q) ok = tags[a][q % w] == q;
        if (ok) return m;
      }
      return (int64_t)0;
    };
    auto model_append = [&](MSeq &s, int layer, int64_t n) {
      const int64_t L = s.len[layer];
      if (layer == FULL) {
        const int64_t need = (L + n + 15) / 16;
        while ((int64_t)s.pages.size() < need) s.pages.push_back(next_id++);
      } else {
        const int64_t nw = std::min<int64_t>(n, w);
        for (int64_t t = n - nw; t < n; ++t) s.tags[swa_index(layer)][(L + t) % w] = L + t;
      }
      s.len[layer] = L + n;
    };
    auto new_seq_like = [&](const std::vector<std::vector<int64_t>> &tags, const std::vector<long> &pages,
                            int64_t reuse) {
      MSeq s;
      s.open = true;
      s.len.assign(NL, reuse);
      s.tags = tags;
      for (auto &t : s.tags)
        for (auto &x : t)
          if (x >= reuse) x = -1;
      s.pages.assign(pages.begin(), pages.begin() + reuse / 16);
      if (reuse % 16) s.pages.push_back(next_id++);
      return s;
    };
    auto verify = [&]() {
      ++step;
      int64_t nf = -1;
      check(kvpool_free_pages(p, FULL, &nf) == SWA_OK && nf == n_pages - (int64_t)held().size(), "free pages", step);
      int64_t alloc = 0, res = 0, ea = 0, er = 0;
      for (int i = 0; i < max_seqs; ++i) {
        const MSeq &s = seqs[i];
        if (!s.open) continue;
        for (int l = 0; l < NL; ++l) {
          int64_t len = -1;
          check(kvpool_seq_len(p, i, l, &len) == SWA_OK && len == s.len[l], "length", step);
          if (l == FULL) continue;
          std::vector<int64_t> tg(w);
          check(kvpool_slot_tags(p, i, l, tg.data()) == SWA_OK && tg == s.tags[swa_index(l)], "ring tags", step);
          ea += (int64_t)w * tok_bytes;
          er += std::min<int64_t>(s.len[l], w) * tok_bytes;
        }
        int64_t m = -1;
        const int64_t match = uni(0, committed(s) + 3);
        check(kvpool_window_safe_len(p, i, match, &m) == SWA_OK &&
                  m == safe_brute(s.tags, std::min(match, committed(s))), "window-safe length", step);
      }
      ea += (int64_t)held().size() * page_bytes;
      er += (int64_t)held().size() * page_bytes;
      check(kvpool_bytes(p, &alloc, &res) == SWA_OK && alloc == ea && res == er, "byte accounting", step);
      for (int z = 0; z < max_snaps; ++z) {
        int64_t len = -1;
        const int rc = kvpool_snapshot_len(p, z, &len);
        check(snaps[z].used ? (rc == SWA_OK && len == snaps[z].len) : rc == SWA_EINVAL, "snapshot length", step);
      }
    };
    auto pick_open = [&]() -> int {
      std::vector<int> o;
      for (int i = 0; i < max_seqs; ++i)
        if (seqs[i].open) o.push_back(i);
      return o.empty() ? -1 : o[(size_t)uni(0, (int64_t)o.size() - 1)];
    };
    auto free_slot = [&]() {
      for (auto &s : seqs)
        if (!s.open) return true;
      return false;
    };

    for (int op = 0; op < 400; ++op) {
      const int kind = (int)uni(0, 9);
      if (kind == 0) {  // open
        int32_t s = -1;
        const bool room = free_slot();
        const int rc = kvpool_seq_open(p, &s);
        check(room ? rc == SWA_OK : rc == SWA_ENOMEM, "open", step);
        if (rc == SWA_OK) {
          check(!seqs[s].open, "open returned a live id", step);
          seqs[s] = MSeq{};
          seqs[s].open = true;
          seqs[s].tags.assign(NSWA, std::vector<int64_t>(w, -1));
        }
      } else if (kind <= 3) {  // append to every layer, or (kind 3) to one layer
        const int i = pick_open();
        if (i < 0) continue;
        const int64_t n = uni(1, 40);
        const int lo = kind == 3 ? (int)uni(0, NL - 1) : 0, hi = kind == 3 ? lo : NL - 1;
        for (int l = lo; l <= hi; ++l) {
          MSeq &s = seqs[i];
          const int64_t need = l == FULL ? (s.len[l] + n + 15) / 16 - (int64_t)s.pages.size() : 0;
          const int64_t freep = n_pages - (int64_t)held().size();
          int expect = SWA_OK;
          if (s.len[l] + n > max_len) expect = SWA_EINVAL;
          else if (need > freep) expect = SWA_ENOMEM;
          const int rc = kvpool_append(p, i, l, nullptr, nullptr, (int32_t)n, nullptr);
          check(rc == expect, "append return code", step);
          if (rc == SWA_OK) model_append(s, l, n);
        }
      } else if (kind == 4) {  // batched append of a random subset to one layer
        std::vector<int32_t> ids;
        for (int i = 0; i < max_seqs; ++i)
          if (seqs[i].open && uni(0, 1)) ids.push_back(i);
        if (ids.empty()) continue;
        if (uni(0, 5) == 0) ids.push_back(ids[0]);  // a duplicate: refused
        const int l = (int)uni(0, NL - 1);
        const int64_t n = uni(1, 4);
        int expect = SWA_OK;
        int64_t need = 0;
        std::set<int32_t> uniq(ids.begin(), ids.end());
        if (uniq.size() != ids.size()) expect = SWA_EINVAL;
        for (int32_t i : uniq) {
          if (seqs[i].len[l] + n > max_len) expect = SWA_EINVAL;
          if (l == FULL) need += (seqs[i].len[l] + n + 15) / 16 - (int64_t)seqs[i].pages.size();
        }
        if (expect == SWA_OK && need > n_pages - (int64_t)held().size()) expect = SWA_ENOMEM;
        const int rc = kvpool_append_batch(p, (int32_t)ids.size(), ids.data(), l, nullptr, nullptr, (int32_t)n, nullptr);
        check(rc == expect, "batched append return code", step);
        if (rc == SWA_OK)
          for (int32_t i : ids) model_append(seqs[i], l, n);
      } else if (kind == 5) {  // fork at the window-safe length of a random match (or an unsafe one)
        const int i = pick_open();
        if (i < 0) continue;
        const MSeq &D = seqs[i];
        const int64_t c = committed(D);
        const int64_t match = uni(0, c);
        const int64_t safe = safe_brute(D.tags, match);
        const bool unsafe = uni(0, 4) == 0 && safe < c;
        const int64_t reuse = unsafe ? safe + 1 + uni(0, c - safe - 1) : safe;
        const bool unsafe_real = safe_brute(D.tags, reuse) != reuse;
        int expect = SWA_OK;
        if (unsafe_real) expect = SWA_EINVAL;
        else if (!free_slot() || (reuse % 16 && (int64_t)held().size() >= n_pages)) expect = SWA_ENOMEM;
        int32_t ns = -1;
        const int rc = kvpool_seq_fork(p, i, reuse, &ns, nullptr);
        check(rc == expect, "fork return code", step);
        if (rc == SWA_OK) seqs[ns] = new_seq_like(D.tags, D.pages, reuse);
      } else if (kind == 6) {  // snapshot
        const int i = pick_open();
        if (i < 0) continue;
        const MSeq &s = seqs[i];
        const bool equal = std::all_of(s.len.begin(), s.len.end(), [&](int64_t x) { return x == s.len[0]; });
        int zfree = -1;
        for (int z = 0; z < max_snaps; ++z)
          if (!snaps[z].used) { zfree = z; break; }
        int32_t z = -1;
        const int rc = kvpool_snapshot(p, i, &z, nullptr);
        check(rc == (!equal ? SWA_EINVAL : zfree < 0 ? SWA_ENOMEM : SWA_OK), "snapshot return code", step);
        if (rc == SWA_OK) {
          check(z == zfree, "snapshot slot", step);
          MSnap &Z = snaps[z];
          Z.used = true;
          Z.len = s.len[0];
          Z.tags = s.tags;
          Z.pages.assign(s.pages.begin(), s.pages.begin() + (Z.len + 15) / 16);
        }
      } else if (kind == 7) {  // fork from a snapshot, or release one
        const int z = (int)uni(0, max_snaps - 1);
        if (uni(0, 2) == 0) {
          const int rc = kvpool_snapshot_release(p, z);
          check(rc == (snaps[z].used ? SWA_OK : SWA_EINVAL), "release return code", step);
          if (rc == SWA_OK) snaps[z] = MSnap{};
        } else {
          int expect = SWA_OK;
          if (!snaps[z].used) expect = SWA_EINVAL;
          else if (!free_slot() || (snaps[z].len % 16 && (int64_t)held().size() >= n_pages)) expect = SWA_ENOMEM;
          int32_t ns = -1;
          const int rc = kvpool_seq_fork_snapshot(p, z, &ns, nullptr);
          check(rc == expect, "fork-from-snapshot return code", step);
          if (rc == SWA_OK) seqs[ns] = new_seq_like(snaps[z].tags, snaps[z].pages, snaps[z].len);
        }
      } else {  // close
        const int i = pick_open();
        if (i < 0) continue;
        check(kvpool_seq_close(p, i) == SWA_OK, "close", step);
        seqs[i] = MSeq{};
      }
      verify();
    }
    kvpool_destroy(p);
  }
  std::printf("steps=%ld\npool_fuzz_mismatches=%ld\n", step, mismatches);
  return mismatches == 0 ? 0 : 1;
}
