// Shared device-side helpers for the gfx950 kernels of libgsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <utility>

// pointer qualifier for LDS (local data share) addresses
#define GSA_LDS __attribute__((address_space(3)))

namespace gsa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 bit pattern -> float32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

// Two floats -> a bf16 pair (lo in the low half), each rounded to nearest even:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(bf16)lo, (bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Hardware base-2 exponential (v_exp_f32): exp2(-inf) == 0, exp2(0) == 1 exactly.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Logistic sigmoid 1/(1+e^{-z}): hardware exp2 and hardware reciprocal (within
// one ulp).  z = 0 gives exactly 0.5 and z >= 40 exactly 1.0 (e^{-z} is then
// below half an ulp of 1; reciprocals of 2 and 1 are exact); very negative z
// makes e^{-z} overflow to +inf and gives exactly 0.
__device__ __forceinline__ float sigmoidf(float z) {
  float e = fast_exp2(-z * kLog2e);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// Gate activations ("GatedAttention [2025]" §1.2.2 item (5); NS-sigmoid of
// §1.4.2 (iv)): 0 identity (the raw logits), 1 sigmoid, 2 NS-sigmoid
// 0.5 + 0.5·σ(z), 3 SiLU z·σ(z).
enum : int { kActIdentity = 0, kActSigmoid = 1, kActNsSigmoid = 2, kActSilu = 3 };
__device__ __forceinline__ float gate_act(float z, int act) {
  if (act == kActSigmoid) return sigmoidf(z);
  if (act == kActNsSigmoid) return fmaf(0.5f, sigmoidf(z), 0.5f);
  if (act == kActSilu) return z * sigmoidf(z);
  return z;
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero (the hardware range check), which the kernels use for tails.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

// 16-byte direct global -> LDS load (buffer_load_dwordx4 ... lds): lane l's 16
// bytes land at LDS address lds_addr + 16*l; offsets past the buffer's range
// read as zeros.  Issued through inline assembly so the compiler does not
// track it as a pending LDS write (it would otherwise make every later LDS
// read wait for all such loads, even ones filling a different stage): the
// caller waits for these loads itself (s_waitcnt vmcnt) before the barrier
// that publishes the stage.  lds_addr must be wave-uniform.  Kernels using it
// make no other use of m0.
__device__ __forceinline__ void dma16_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory");
}
// The same with the non-temporal cache policy, for data read once (the decode
// cache stream): a plain read of 4 GiB reaches 6.0-6.5 TB/s, the same read
// with this policy 7.0-7.25 TB/s.
__device__ __forceinline__ void dma16_lds_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1, so
// register-resident arrays are only ever indexed by constants.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename T>
__host__ __device__ __forceinline__ T ceil_div(T a, T b) { return (a + b - 1) / b; }

}  // namespace gsa
