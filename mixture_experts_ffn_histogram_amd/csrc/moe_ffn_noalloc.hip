// moe_ffn_forward_noalloc: the forward on a workspace the library holds in
// device memory of its own, for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The workspace is the file-scope device array `scratch`, one copy per GPU for
// the life of the process.  In host code its name is not a device address:
// the first call on a device (with that device current) asks the runtime for
// the array's address on that device and keeps it; every launch, copy and
// clear uses that address.  Each call first clears the control block (the
// part of the workspace that must be zero when a call starts) with a
// small kernel on the call's stream (with the barrier counters behind it), then
// runs the ordinary forward.  All calls
// on one GPU share the array, so calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/moe_ffn.h"
#include "moe_ffn_kernel.h"
#include "moe_ffn_layout.h"

static_assert(MOE_FFN_NOALLOC_MAX_WORKSPACE % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) uint8_t scratch[MOE_FFN_NOALLOC_MAX_WORKSPACE];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

__global__ void clear_ctrl_kernel(uint32_t* words) {
  for (int i = threadIdx.x; i < moeffn::kCtrlRegionBytes / 4; i += blockDim.x) words[i] = 0u;
}

// Clears the control block and the barrier counters behind it (the part of
// the workspace that must be zero when a call starts).
hipError_t clear_ctrl(void* workspace, hipStream_t stream) {
  hipLaunchKernelGGL(clear_ctrl_kernel, dim3(1), dim3(256), 0, stream, static_cast<uint32_t*>(workspace));
  return hipGetLastError();
}

// Device address of `scratch` on the current device `dev` (looked up once per device).
void* scratch_on(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" int moe_ffn_forward_noalloc(const moe_ffn_problem* problem, const moe_ffn_args* args, void* stream) {
  size_t need = 0;
  const int rc = moe_ffn_get_workspace_size(problem, &need);
  if (rc != MOE_FFN_OK) return rc;
  if (need > (size_t)MOE_FFN_NOALLOC_MAX_WORKSPACE) return MOE_FFN_ERR_WORKSPACE_TOO_SMALL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_FFN_ERR_HIP;
  void* ws = scratch_on(dev);
  if (!ws) return MOE_FFN_ERR_HIP;
  return moeffn::forward_enqueue(problem, args, ws, (size_t)MOE_FFN_NOALLOC_MAX_WORKSPACE,
                                 static_cast<hipStream_t>(stream), clear_ctrl);
}
