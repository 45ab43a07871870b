// ta_tree_attn_rows_noalloc: tree attention for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). It runs the kernels of ta_tree_attn_rows; the
// workspace those kernels need for split partials and hand-off counters is a
// file-scope device array of this library, one copy per GPU, held until the
// process ends.
//
// Host code never passes `scratch` itself to a kernel or a copy: in host code
// that name is a host-side stand-in, not a device address. Its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept in g_scratch[device].
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "launch.h"
#include "plan.h"

namespace ta {
namespace {

constexpr size_t kScratchBytes = TA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes >= kCounterBytes, "the counters must fit");

// Split partials and counters of every no-alloc call on this GPU. A device
// array without an initialiser starts zeroed; the counters must start at zero
// and every completed call leaves them there.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on device `dev` (the current device).
ta_status scratch_on(int dev, void** ptr) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(TA_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return TA_OK;
}

}  // namespace
}  // namespace ta

using namespace ta;

extern "C" ta_status ta_tree_attn_rows_noalloc(const void* q, const ta_kv_cache* cache, int32_t layer,
                                               int32_t prefix_len, const int32_t* parent, int32_t n_tree,
                                               int32_t q_first, int32_t n_q_heads, void* out, void* stream) {
  clear_error();
  // host-side validation first: an invalid call touches no device state
  ta_status st = check_cache(cache, true);
  if (st == TA_OK) st = check_parent(parent, n_tree);
  if (st != TA_OK) return st;
  AttnPlan plan;
  st = plan_tree_attn(cache, n_q_heads, prefix_len, n_tree, q_first, &plan);
  if (st != TA_OK) return st;
  if (plan.ws_bytes > kScratchBytes)
    return fail(TA_ERR_UNSUPPORTED, "this shape needs " + std::to_string(plan.ws_bytes) +
                                        " bytes of workspace, more than the " + std::to_string(kScratchBytes) +
                                        " bytes of static scratch; use ta_tree_attn_rows with a workspace");
  int dev = -1, cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TA_ERR_DEVICE, std::string("device of the stream: ") + hipGetErrorString(e));
  if (dev != cur) return fail(TA_ERR_ARG, "the stream must belong to the current device");
  if (dev < 0 || dev >= kMaxDevices) return fail(TA_ERR_UNSUPPORTED, "device index beyond 63");
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    st = scratch_on(dev, &ws);
    if (st != TA_OK) return st;
  }
  return tree_attn_rows_impl(q, cache, layer, prefix_len, parent, n_tree, q_first, n_q_heads, out, ws,
                             plan.ws_bytes > 0 ? kScratchBytes : 0, stream);
}
