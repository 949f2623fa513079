// moe_forward_noalloc: the whole layer forward with its workspace in a
// file-scope device array instead of a caller's buffer, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array lives in the library's code object: every GPU the library runs
// on holds its own copy from module load until the process ends.  Host code
// never uses the array's name as an address (on the host it is a stand-in
// symbol, not device memory): the device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and that pointer is what the kernels receive as their workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe.h"

static_assert(MOE_NOALLOC_MAX_WORKSPACE_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_MAX_WORKSPACE_BYTES];

namespace {

constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_MAX_WORKSPACE_BYTES;  // per GPU
constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// The device address of the current device's copy of `scratch`, looked up
// on the first call on that device.  Returns MOE_ERR_HIP if the device
// cannot be queried or the lookup fails.
moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward_noalloc(const moe_config* cfg, const void* X, const void* Wg, const float* gate_bias,
                               const void* W1, const void* W2, void* out, int32_t* topk_ids, float* topk_w,
                               int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm,
                               void* stream) {
  size_t need = 0;
  if (moe_status s = moe_workspace_size(cfg, MOE_OP_FORWARD, &need); s != MOE_OK) return s;
  if (need > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (moe_status s = scratch_of_current_device(&ws); s != MOE_OK) return s;
  // The forward's kernels write every scratch byte they read, so the array
  // needs no clearing between calls.
  return moe_forward(cfg, X, Wg, gate_bias, W1, W2, out, topk_ids, topk_w, expert_counts, expert_offsets, perm,
                     inv_perm, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
