// static_fwd.cpp — bdattn_fwd_static: the forward with its scratch in a
// static device buffer instead of a caller workspace, for callers that
// cannot allocate device memory (HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  See include/bdattn.h.
//
// The buffer `scratch` has one copy per GPU, alive until the process ends.
// Host code never passes the array's name as an address (on the host it is
// only a stand-in for the device symbol): its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// that pointer is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abi_internal.h"
#include "bdattn.h"

namespace {

__device__ __align__(256) char scratch[BDATTN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct StaticScratch {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
} g_static;

}  // namespace

namespace bd {

void* static_scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_static.mu);
  if (!g_static.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_static.ptr[dev] = p;
  }
  return g_static.ptr[dev];
}

}  // namespace bd

extern "C" int bdattn_fwd_static(const bdattn_problem* problem, const bdattn_share* share, const bdattn_kv* kv,
                                 bdattn_tensor q_clean, bdattn_tensor q_corr, bdattn_tensor k_clean,
                                 bdattn_tensor v_clean, bdattn_tensor k_corr, bdattn_tensor v_corr,
                                 bdattn_tensor o, int32_t o_dtype, float* lse, void* hip_stream) {
  // the size check needs no device: a problem too large for the buffer is
  // rejected before any HIP call (an invalid one too: the size is then 0
  // and fwd_impl reports it)
  const size_t need = bdattn_workspace_bytes(problem, share, kv, 0);
  if (need > BDATTN_STATIC_SCRATCH_BYTES) return BDATTN_ESCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    ws = bd::static_scratch_ptr();
    if (!ws) return BDATTN_EHIP;
  }
  return bd::fwd_impl(problem, share, kv, q_clean, q_corr, k_clean, v_clean, k_corr, v_corr, o, o_dtype, lse,
                      ws, BDATTN_STATIC_SCRATCH_BYTES, hip_stream);
}
