// ssa_decode_static: the whole decode step with its workspace in a
// file-scope device array instead of a caller-provided buffer, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The entry point allocates nothing: it
// checks that the step's workspace fits the array and runs ssa_decode on it.
//
// The array is a device symbol: its host-side name is only a stand-in, so
// its device address is taken once per device with hipGetSymbolAddress, with
// that device current, and only that address is ever passed to kernels.
// Every call on a device shares that device's array; the step clears what
// must start at zero itself (a kernel, not a memset) and writes everything
// else before reading it, so a call never sees an earlier call's contents.
// Calls that overlap on one device (two streams, two threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssa.h"

namespace {

__device__ __align__(256) unsigned char scratch[SSA_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];

// The device address of this device's array (null if it cannot be had).
void* scratch_address(int dev) {
  std::call_once(g_once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();  // leave no sticky error for the caller's next call
      ptr = nullptr;
    }
    g_scratch[dev] = ptr;
  });
  return g_scratch[dev];
}

}  // namespace

extern "C" int ssa_decode_static(const ssa_params* p, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* topk,
                                 const float* top_p, const int32_t* sample_budget,
                                 const uint64_t* seed, void* out, void* stream) {
  const size_t need = ssa_workspace_bytes(p);
  if (need == 0) return SSA_ERR_INVALID;
  if (need > (size_t)SSA_STATIC_WORKSPACE_BYTES) return SSA_ERR_STATIC_LIMIT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSA_ERR_HIP;
  void* ws = scratch_address(dev);
  if (!ws) return SSA_ERR_HIP;
  return ssa_decode(p, q, k_cache, v_cache, block_table, seq_lens, topk, top_p, sample_budget,
                    seed, out, ws, (size_t)SSA_STATIC_WORKSPACE_BYTES, stream);
}
