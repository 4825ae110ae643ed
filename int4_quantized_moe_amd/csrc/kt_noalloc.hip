// The inference forward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the same kernels as kt_rawint4_moe_infer, with the workspace in
// a fixed device array of this library instead of a caller's buffer.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy, at its own address, from the code object's load until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it names a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// kept per device.
#include <mutex>
#include <vector>

#include "kt_internal.hpp"

namespace kt {

static __device__ __align__(256) uint8_t scratch[KT_RAWINT4_STATIC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static std::vector<void*> g_scratch_ptr;  // per device ordinal; null until set up

// The current device's copy of the scratch array (set up on its first use).
static hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[(size_t)dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_scratch_ptr[(size_t)dev] = ptr;
  }
  *out = g_scratch_ptr[(size_t)dev];
  return hipSuccess;
}

}  // namespace kt

using namespace kt;

extern "C" int kt_rawint4_moe_infer_static(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                                           const int64_t* expert_ids, const float* route_weights, uint16_t* output,
                                           void* stream) {
  Dims d;
  int rc = check_layer_dims(layer, qlen, &d, true);
  if (rc) return rc;
  d.train = false;
  const size_t need = plan_workspace(d).total;
  if (need > (size_t)KT_RAWINT4_STATIC_SCRATCH_BYTES)
    return set_error(KT_RAWINT4_EWORKSPACE,
                     "the call needs a larger workspace than the static scratch holds "
                     "(kt_rawint4_moe_infer_workspace_bytes > KT_RAWINT4_STATIC_SCRATCH_BYTES)");
  void* ws = nullptr;
  const hipError_t err = scratch_ptr(&ws);
  if (err != hipSuccess) return set_error(KT_RAWINT4_EHIP, "hipGetSymbolAddress of the static scratch failed");
  return run_forward_no_alloc(layer, d, inputs, expert_ids, route_weights, output, ws,
                              (size_t)KT_RAWINT4_STATIC_SCRATCH_BYTES, stream);
}
