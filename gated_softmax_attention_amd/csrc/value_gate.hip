// G2 value gating: V' = V ⊙ g, with g = σ(X·W_v) per key/value head and dim
// (elementwise, column c·D + d) or per key/value head (headwise, column c) —
// the gate at the value map instead of the SDPA output ("GatedAttention
// [2025]" §1.2.2, position G2; §1.4.2 compares it with G1).  Attention then
// runs on V' with no output gate.  g comes from gsa_gate_logits.
//
// HBM-bound elementwise pass: 16-byte loads of V, the float32 gate read
// alongside, one rounding of V·g to the value dtype.
#include "common.h"

namespace gsa {

template <typename T, bool HEADWISE>
__global__ __launch_bounds__(256)
void value_gate_kernel(const T* __restrict__ V, const float* __restrict__ G, T* __restrict__ Vout, int64_t n16,
                       int Hkv, int D) {
  constexpr int E = 16 / sizeof(T);   // elements per 16-byte chunk
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n16; c += (int64_t)gridDim.x * 256) {
    const int64_t e0 = c * E;                 // first element: ((tok·Hkv + kvh)·D + d0)
    const int64_t row = e0 / D;               // tok·Hkv + kvh
    const u32x4 v = *(const u32x4*)(V + e0);
    float g[E];
    if constexpr (HEADWISE) {
      const float gh = G[row];
#pragma unroll
      for (int e = 0; e < E; ++e) g[e] = gh;
    } else {
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const f32x4 g4 = *(const f32x4*)(G + e0 + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) g[e + k] = g4[k];
      }
    }
    u32x4 out;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        out[w] = pack_bf16x2(bf16_lo(v[w]) * g[2 * w], bf16_hi(v[w]) * g[2 * w + 1]);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) out[w] = __float_as_uint(__uint_as_float(v[w]) * g[w]);
    }
    *(u32x4*)(Vout + e0) = out;
  }
}

// V, Vout: [B·S, Hkv, D] (the layout of K and V); G: [B·S, Hkv·D] (elementwise)
// or [B·S, Hkv] (headwise), float32.
hipError_t launch_value_gate(const void* V, const float* G, void* Vout, int64_t rows, int Hkv, int D,
                             bool headwise, bool bf16_inputs, hipStream_t st) {
  const int64_t n = rows * Hkv * D;
  const int64_t n16 = n / (bf16_inputs ? 8 : 4);
  const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div<int64_t>(n16, 256), 8192);
  if (bf16_inputs) {
    if (headwise)
      hipLaunchKernelGGL((value_gate_kernel<bf16, true>), dim3(blocks), dim3(256), 0, st, (const bf16*)V, G,
                         (bf16*)Vout, n16, Hkv, D);
    else
      hipLaunchKernelGGL((value_gate_kernel<bf16, false>), dim3(blocks), dim3(256), 0, st, (const bf16*)V, G,
                         (bf16*)Vout, n16, Hkv, D);
  } else {
    if (headwise)
      hipLaunchKernelGGL((value_gate_kernel<float, true>), dim3(blocks), dim3(256), 0, st, (const float*)V, G,
                         (float*)Vout, n16, Hkv, D);
    else
      hipLaunchKernelGGL((value_gate_kernel<float, false>), dim3(blocks), dim3(256), 0, st, (const float*)V, G,
                         (float*)Vout, n16, Hkv, D);
  }
  return hipGetLastError();
}

}  // namespace gsa
