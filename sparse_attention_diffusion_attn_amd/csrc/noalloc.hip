// mcs_anchor_select_noalloc: the two-pass exact selection with its score
// workspace in a fixed device array of the library instead of caller memory,
// for callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid allocation).
//
// The array `scratch` is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy, MCS_NOALLOC_SCRATCH_BYTES long, from
// the loading of the library's code until the process ends.  Host code never
// uses the array's name as an address (on the host it only names the symbol):
// the first call on a device, with that device current, asks the runtime for
// the device address of that device's copy (hipGetSymbolAddress) and keeps it
// per device; kernels get that pointer as their workspace argument.
//
// Every call on one GPU uses the same array.  The selection writes every
// score and histogram entry it later reads, so nothing has to start at zero
// and leftovers of an earlier call are harmless; two calls whose work overlaps
// on one GPU (different streams, or host threads without ordering) race on
// the array.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/mcs.h"
#include "mcs_internal.h"

static constexpr size_t kScratchBytes = (size_t)MCS_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of each device's copy, once looked up

// Device address of the current device's scratch array (nullptr + error
// recorded on failure).
void* scratch_for_current_device(int32_t* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    *status = mcs::api_fail(MCS_ERR_HIP, "no current HIP device");
    return nullptr;
  }
  if (dev >= kMaxDevices) {
    *status = mcs::api_fail(MCS_ERR_UNSUPPORTED, "device index beyond the scratch table");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      char msg[256];
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      *status = mcs::api_fail(MCS_ERR_HIP, msg);
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int32_t mcs_anchor_select_noalloc(const mcs_dims* dims, const uint16_t* q,
                                             const uint16_t* k, const uint16_t* v,
                                             const int32_t* perm, int32_t topk, float scale,
                                             uint16_t* o_full, float* lse, int32_t* kv_idx,
                                             void* stream) {
  const size_t need = mcs_anchor_select_min_workspace_bytes(dims, topk);
  if (need == 0) {
    // bad dims or topk: the regular call reports which, before any GPU work
    return mcs_anchor_select(dims, q, k, v, perm, topk, scale, o_full, lse, kv_idx, nullptr, 0,
                             stream);
  }
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "one head's scores need %zu bytes; the static scratch holds %zu "
             "(use mcs_anchor_select with a caller workspace)",
             need, kScratchBytes);
    return mcs::api_fail(MCS_ERR_UNSUPPORTED, msg);
  }
  int32_t st = MCS_OK;
  void* ws = scratch_for_current_device(&st);
  if (ws == nullptr) return st;
  return mcs_anchor_select(dims, q, k, v, perm, topk, scale, o_full, lse, kv_idx, ws,
                           kScratchBytes, stream);
}
