// Test helper: a kernel that holds whole CUs for a bounded time on a side
// stream (the side-stream liveness scenario of the sglang "Reserve SMs for
// DeepGEMM MegaMoE grid barriers" change).  Each of its
// workgroups takes the full 160 KB of LDS of a CU, so no workgroup of another
// kernel can share that CU while it runs.  The wait is bounded by a device
// clock deadline; the kernel always exits.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kLdsBytes = 160 * 1024 - 64;

__global__ __launch_bounds__(64) void hold_cus(uint64_t ticks, uint32_t* done) {
  __shared__ uint8_t lds[kLdsBytes];
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();  // 100 MHz
  uint32_t v = threadIdx.x;
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) {
    lds[(v * 97) % kLdsBytes] = (uint8_t)v;
    v += lds[(v * 31) % kLdsBytes];
    __builtin_amdgcn_s_sleep(20);
  }
  if (threadIdx.x == 0) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    done[1 + blockIdx.x] = xcc & 15u;  // blocks <= 7 (checked on the host)
    atomicAdd(done, v == 0xFFFFFFFFu ? 2u : 1u);
  }
}

struct Side {
  hipStream_t stream;
  uint32_t* done;
  hipEvent_t end;
};

}  // namespace

extern "C" {

// Starts `blocks` (at most 7) workgroups of the holding kernel for
// `ms` milliseconds on a new non-blocking stream.  On an idle MI355X the
// dispatcher places them round-robin over the XCDs, one CU each.  (A CU-masked
// stream is not used: the runtime rejected a mask holding CUs of only some
// XCDs.)  Returns 0 on success and stores an opaque handle.
int side_start(int blocks, int ms, void** handle) {
  if (blocks < 1 || blocks > 7 || ms < 1 || ms > 10000) return -7;
  Side* s = new Side{};
  if (hipStreamCreateWithFlags(&s->stream, hipStreamNonBlocking) != hipSuccess) { delete s; return -1; }
  if (hipMalloc(&s->done, 8 * sizeof(uint32_t)) != hipSuccess) { delete s; return -2; }
  if (hipMemsetAsync(s->done, 0, 8 * sizeof(uint32_t), s->stream) != hipSuccess) return -3;
  if (hipEventCreate(&s->end) != hipSuccess) return -4;
  hipLaunchKernelGGL(hold_cus, dim3(blocks), dim3(64), 0, s->stream, (uint64_t)ms * 100000ull, s->done);
  if (hipGetLastError() != hipSuccess) return -5;
  if (hipEventRecord(s->end, s->stream) != hipSuccess) return -6;
  *handle = s;
  return 0;
}

// 1 while the holding kernel still runs, 0 once it has finished, <0 on error.
int side_running(void* handle) {
  Side* s = static_cast<Side*>(handle);
  const hipError_t e = hipEventQuery(s->end);
  if (e == hipErrorNotReady) return 1;
  return e == hipSuccess ? 0 : -1;
}

// Waits for the holding kernel; returns how many of its workgroups finished
// and stores the XCD of workgroup b in xcc[b] (b < blocks).
int side_finish(void* handle, uint32_t* xcc) {
  Side* s = static_cast<Side*>(handle);
  if (hipEventSynchronize(s->end) != hipSuccess) return -1;
  uint32_t words[8] = {0};
  if (hipMemcpy(words, s->done, sizeof(words), hipMemcpyDeviceToHost) != hipSuccess) return -2;
  const uint32_t done = words[0];
  for (int b = 0; b < 7; b++) xcc[b] = words[1 + b];
  hipEventDestroy(s->end);
  hipFree(s->done);
  hipStreamDestroy(s->stream);
  delete s;
  return (int)done;
}

}  // extern "C"
