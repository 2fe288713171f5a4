// Device helpers for the fused MoE forward on gfx950 (CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeffn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Explicit global-address-space accesses.  A pointer that reaches a load
// through LDS or a select is generic (flat) to the compiler, and a pending
// flat load forces a full vmcnt drain before the next use of any load; these
// helpers keep every device-memory access a global_* instruction.
typedef __attribute__((address_space(1))) const v4i gv4i_c;
typedef __attribute__((address_space(1))) v4i gv4i;
typedef __attribute__((address_space(1))) const uint32_t gu32_c;
typedef __attribute__((address_space(1))) uint32_t gu32;
typedef __attribute__((address_space(1))) uint8_t gu8;
typedef __attribute__((address_space(1))) v4f gv4f;
typedef __attribute__((address_space(1))) const v4f gv4f_c;
typedef __attribute__((address_space(1))) uint64_t gu64;

__device__ __forceinline__ v4i ldg16(const void* p) { return *(gv4i_c*)p; }
__device__ __forceinline__ v4i ldg16_nt(const void* p) { return __builtin_nontemporal_load((gv4i_c*)p); }
__device__ __forceinline__ uint32_t ldg4(const void* p) { return *(gu32_c*)p; }
__device__ __forceinline__ v4f ldg16f(const void* p) { return *(gv4f_c*)p; }
__device__ __forceinline__ void stg16f(void* p, v4f v) { *(gv4f*)p = v; }
__device__ __forceinline__ void stg16(void* p, v4i v) { *(gv4i*)p = v; }
__device__ __forceinline__ void stg4(void* p, uint32_t v) { *(gu32*)p = v; }
__device__ __forceinline__ void stg1(void* p, uint8_t v) { *(gu8*)p = v; }
__device__ __forceinline__ void stg8(void* p, uint32_t lo, uint32_t hi) { *(gu64*)p = ((uint64_t)hi << 32) | lo; }

// Buffer resources: a 32-bit byte range of device memory addressed by a
// per-lane VGPR offset plus a wave-uniform SGPR offset.  Reads past the range
// return zero.  The LDS variant writes each lane's bytes straight to LDS at
// the wave-uniform destination + lane * size (no VGPR staging).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// A per-lane offset past any buffer's size: a buffer load from it returns
// zeros without a memory access.
constexpr uint32_t kBufDead = 0x80000000u;
__device__ __forceinline__ v4i buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
#define MOEFFN_LDS(p) ((__attribute__((address_space(3))) void*)(p))
__device__ __forceinline__ void buf_load_lds16(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, MOEFFN_LDS(lds), 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buf_load_lds4(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, MOEFFN_LDS(lds), 4, voff, soff, 0, 0);
}
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define MOEFFN_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// ---------------------------------------------------------------------------
// Number formats
// ---------------------------------------------------------------------------

// fp32 -> bf16 bits, round to nearest even (overflow gives inf, NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two values to bf16 bits packed into a dword (low half = a) with the
// hardware pack conversion, round to nearest even (fp32 denormals kept).
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(moe_f32x2{a, b}, moe_bf16x2));
}

// Largest of a value over lanes l, l^16, l^32 and l^48 (the lanes holding the
// same index of the four 16-lane rows) with the lane-swap moves of gfx950:
// the 32-lane swap pairs each lane with lane l^32, the 16-lane swap with l^16.
// VALU moves, not LDS permutes.
// Maximum of two floats that are not NaN (the NaN-propagating maximum: no
// quieting of its inputs, one instruction).
__device__ __forceinline__ float fmax_nn(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float max_over_rows(float a) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  a = fmax_nn(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return fmax_nn(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Four values to OCP E4M3FN codes packed into a dword (byte j = value j)
// with the hardware pack conversion: round to nearest even, and for values
// in [-464, 464] magnitudes above 448 saturate to 448 (checked on gfx950
// against the oracle's rounding and encoder over every code, every midpoint
// and its neighbours, fp32 denormals, (448, 464] and random values).  The
// block scales keep every scaled value within 448 (the fp32-scale recipe's
// quotient within an ulp of it).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);  // bytes 0, 1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);       // bytes 2, 3
  return (uint32_t)w;
}

// Exponent E of the e8m0 scale of a 1x32 block: the smallest integer with
// amax <= 448 * 2^E (448 = 1.75 * 2^8), clamped to [-127, 127]; 0 for an
// all-zero block.  Exact on the fp32 bit pattern: with amax = f * 2^p,
// f in [1, 2), E = p - 8 when f <= 1.75, else p - 7.
__device__ __forceinline__ int block_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int ef = (int)(b >> 23);  // 0 for a subnormal amax: E below -127, clamped
  const int E = (ef - 127) - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  // at most 255 - 135 + 1 = 121 (infinite amax): no upper clamp; selected, not branched on
  return amax > 0.0f ? (E < -127 ? -127 : E) : 0;
}

// The clamp bound of a call: c, or +infinity with the clamp off, so that the
// clamp is one median-of-three per value and no branch (equal to the clamped
// or unclamped value for every input but NaN).
__device__ __forceinline__ float clamp_bound(bool clamp_on, float c) { return clamp_on ? c : __builtin_inff(); }

// SwiGLU of one (gate, up) pair, both clamped to [-cb, cb] (cb from clamp_bound).
__device__ __forceinline__ float swiglu(float g, float u, float cb) {
  g = __builtin_amdgcn_fmed3f(g, -cb, cb);
  u = __builtin_amdgcn_fmed3f(u, -cb, cb);
  const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  return g * sig * u;
}

// ---------------------------------------------------------------------------
// Agent-scope synchronisation (the 8 XCDs have separate L2s: every hand-off
// between workgroups goes through release/acquire at agent scope).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ uint32_t ld_acquire(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_release(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_acq_rel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }  // 100 MHz

// ---------------------------------------------------------------------------
// Workgroup-wide exclusive scan of one int per thread (256 threads).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// `scratch` needs 4 ints of LDS.  Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    int s = scratch[w];
    base += (w < wave) ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

}  // namespace moeffn
