// Test helpers: the forward's device helpers applied to lists of floats, so
// that tests can compare them value by value: the hardware pack conversions
// (e4m3x4, bf16x2) with the oracle's encoders, the cross-row lane maximum
// (max_over_rows) with its definition, and the 1x32 block exponent
// (block_scale_exp) with the oracle's scale rule.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../mixture_experts_ffn_histogram_amd/csrc/moe_ffn_device.h"

namespace {

__global__ __launch_bounds__(256) void convert(const float* __restrict__ in, uint32_t* __restrict__ out, int nquads) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < nquads) out[i] = moeffn::e4m3x4(in[4 * i], in[4 * i + 1], in[4 * i + 2], in[4 * i + 3]);
}

__global__ __launch_bounds__(256) void convert_bf16(const float* __restrict__ in, uint32_t* __restrict__ out, int npairs) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < npairs) out[i] = moeffn::bf16x2(in[2 * i], in[2 * i + 1]);
}

__global__ __launch_bounds__(256) void lane_max(const float* __restrict__ in, float* __restrict__ out, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // n is a multiple of 256: every lane of a wave is live
  out[i] = moeffn::max_over_rows(in[i]);
}

__global__ __launch_bounds__(256) void scale_exp(const float* __restrict__ in, int* __restrict__ out, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = moeffn::block_scale_exp(in[i]);
}

}  // namespace

// in: 4 * nquads floats (device), out: nquads dwords (device), byte j of out[i] = code of in[4 i + j].
extern "C" int moe_test_e4m3x4(const float* in, uint32_t* out, int nquads, void* stream) {
  if (nquads <= 0) return 0;
  hipLaunchKernelGGL(convert, dim3((nquads + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), in, out,
                     nquads);
  return (int)hipGetLastError();
}

// in: 2 * npairs floats (device), out: npairs dwords (device), low half of out[i] = bf16 bits of in[2 i],
// high half those of in[2 i + 1].
extern "C" int moe_test_bf16x2(const float* in, uint32_t* out, int npairs, void* stream) {
  if (npairs <= 0) return 0;
  hipLaunchKernelGGL(convert_bf16, dim3((npairs + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), in,
                     out, npairs);
  return (int)hipGetLastError();
}

// in, out: n floats (device), n a positive multiple of 256; out[i] = max over lanes i^16, i^32, i^48 and i
// of its 64-lane wave.
extern "C" int moe_test_max_over_rows(const float* in, float* out, int n, void* stream) {
  if (n <= 0 || n % 256) return 1;
  hipLaunchKernelGGL(lane_max, dim3(n / 256), dim3(256), 0, static_cast<hipStream_t>(stream), in, out, n);
  return (int)hipGetLastError();
}

// in: n floats (device), out: n ints (device), out[i] = the e8m0 exponent the epilogues take for a block
// whose largest magnitude is in[i].
extern "C" int moe_test_block_scale_exp(const float* in, int* out, int n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(scale_exp, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), in, out, n);
  return (int)hipGetLastError();
}
