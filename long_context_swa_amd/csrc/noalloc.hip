// full_attn_noalloc: full_attn for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).  The workspace full_attn
// takes from its caller (split-K partials of a decode / verify call and, when the arena's table
// cache cannot hold them, the call's sequence and work lists) lives instead in `scratch`, a
// file-scope device array of kScratchBytes that every GPU the library runs on holds until the
// process ends.  Host code never passes the array's name to a kernel or copy: on the host it is a
// stand-in, not a device address.  Its address on each device comes from hipGetSymbolAddress, taken
// once per device with that device current, and is kept per device.

#include "swa.h"
#include "swa_internal.h"

#include <mutex>

namespace {

constexpr int64_t kScratchBytes = 32LL << 20;  // 32 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
char *g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device), or nullptr with
// the error recorded.
char *scratch_on_current_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    swa::set_error(SWA_EHIP, "full_attn_noalloc: no usable current device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      swa::set_error(SWA_EHIP, "full_attn_noalloc: hipGetSymbolAddress(scratch) failed");
      return nullptr;
    }
    g_scratch[dev] = static_cast<char *>(ptr);
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int full_attn_noalloc(swa_pool *p, int32_t n_seqs, const int32_t *seqs, int32_t layer,
                                 const void *q, const void *k_new, const void *v_new,
                                 int32_t q_len_or_chunk, int32_t n_q_heads, swa_dtype dt, void *out,
                                 void *stream) {
  const int64_t need = swa_attn_workspace_bytes(p, n_seqs, seqs, layer, q_len_or_chunk, n_q_heads);
  if (need < 0) return (int)need;
  if (need > kScratchBytes)
    return swa::set_error(SWA_ENOMEM, "full_attn_noalloc: call needs more workspace than the 32 MiB "
                                      "device scratch array holds (use full_attn with a workspace)");
  char *ws = scratch_on_current_device();
  if (!ws) return SWA_EHIP;
  return full_attn(p, n_seqs, seqs, layer, q, k_new, v_new, q_len_or_chunk, n_q_heads, dt, out, ws,
                   kScratchBytes, stream);
}
