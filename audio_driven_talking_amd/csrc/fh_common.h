// Device-side helpers shared by the HIP kernels of libfh (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FH_WAVE 64

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// float -> bfloat16 with round to nearest even: gfx950's v_cvt_pk_bf16_f32
// (the compiler emits it for a pair of __bf16 conversions).
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16_t f2bf(float f) { return (bf16_t)(pack2bf(f, 0.f) & 0xffffu); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// tanh-approximated GELU, 0.5 z (1 + tanh(u)) with u = sqrt(2/pi)(z + 0.044715 z^3),
// evaluated as z * sigmoid(2u) = z / (1 + exp(-2u)) (the same function) with the
// hardware exp2 and reciprocal; large |u| saturates to z or -0 correctly.
__device__ __forceinline__ float gelu_tanh(float z) {
  const float c2 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float t = c2 * (z + 0.044715f * z * z * z);
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// ---- LDS DMA (global_load_lds_dwordx4) and explicit waits -------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane;
// lds_base must be wave-uniform.
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void*)g, (lds_void*)lds_base, 16, 0, 0);
}

// wait until at most n vector-memory operations of this wave are outstanding
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// MX-FP8 (OCP microscaling: e4m3 elements, one E8M0 power-of-two scale per 32
// consecutive elements along K). A block with max |x| = a > 0 takes the
// shared exponent floor(log2 a) - 8 (e4m3's largest power of two is 2^8),
// clamped below at -127 (E8M0 byte = exponent + 127); an all-zero block 0.
// Elements are x * 2^-exponent clamped to +-448 and rounded to nearest even.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (amax == 0.f) return 0;
  const int eb = (int)((__float_as_uint(amax) >> 23) & 255);
  return eb == 0 ? -127 : max(eb - 127 - 8, -127);
}
// 2^-e for a shared exponent e in [-127, 119] (exact)
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }
// two scaled values -> two e4m3 bytes (low 16 bits)
__device__ __forceinline__ uint32_t pack2_e4m3(float a, float b) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}
// eight scaled values -> eight e4m3 bytes
__device__ __forceinline__ u32x2 pack8_e4m3(const float* v, float inv) {
  const u32x2 w = {pack2_e4m3(v[0] * inv, v[1] * inv) | (pack2_e4m3(v[2] * inv, v[3] * inv) << 16),
                   pack2_e4m3(v[4] * inv, v[5] * inv) | (pack2_e4m3(v[6] * inv, v[7] * inv) << 16)};
  return w;
}

// wait until every LDS read / write of this wave has completed
__device__ __forceinline__ void wait_lgkm0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  asm volatile("" ::: "memory");
}

// workgroup barrier without the memory fence of __syncthreads (which would
// also wait for every outstanding LDS DMA); callers order DMAs with wait_vm.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait states between the last MFMA of a loop and the first read of its
// accumulator after the loop exit. The compiler's hazard padding does not
// always cover this cross-block case on gfx950 (a 16x16x32 bf16 result was
// read stale without it). The accumulator is an operand of the padding, so its
// reads cannot be scheduled above it; 32 wait states exceed the longest MFMA.
template <typename T>
__device__ __forceinline__ void mfma_drain(T& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}

// Debugging aid for races through LDS: when set (fh_debug_workgroup_order),
// the kernels whose waves share LDS take their work in the reverse order of
// workgroup ids along x, so a scheduling-dependent result shows up as a
// difference between the two orders. Every source file holds its own copy
// of the flag; set_wg_reverse() sets the copy of the file that calls it.
static __constant__ int c_wg_reverse = 0;
__device__ __forceinline__ unsigned wg_x() { return c_wg_reverse ? gridDim.x - 1 - blockIdx.x : blockIdx.x; }
static inline hipError_t set_wg_reverse(int r) { return hipMemcpyToSymbol(HIP_SYMBOL(c_wg_reverse), &r, sizeof r); }
