// Head-shared gate: the mean over the query heads of the activated
// elementwise gating scores, Gs[m, d] = (1/Hq)·Σ_h G[m, h·D + d].
//
// "GatedAttention [2025]" §1.2.2 item (3) lets every head share one gating
// score; the §1.3.2 Table 1 discussion (observation (ii)) forms it by
// averaging the n×q×d_k scores over the q query heads into n×d_k, and "10 ·
// 门控" §3.2 Table 1 row 12 counts a q·d_k-wide W_θ for it.  The scores are
// the activated values gsa_gate_logits writes (σ by default), so the mean is
// taken after the activation.  The forward and decode variants then apply Gs
// with the shared layout (column d for every head).
//
// HBM-bound pass: each thread owns 4 consecutive dims of one token row and sums
// the Hq heads' 16-byte pieces in head order (float32), then divides by Hq.
// A wave covers whole rows of Gs (D/4 threads per row), so each head's pieces
// of a row are one contiguous read of D·4 bytes.
#include "common.h"

namespace gsa {

__global__ __launch_bounds__(256)
void gate_head_mean_kernel(const float* __restrict__ G, float* __restrict__ Gs, int64_t n4, int Hq, int D4) {
  const float hq = (float)Hq;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / D4;
    const int c = (int)(i - m * D4);
    const f32x4* src = (const f32x4*)G + m * Hq * D4 + c;
    f32x4 acc = src[0];
#pragma unroll 4
    for (int h = 1; h < Hq; ++h) {
      const f32x4 v = src[(int64_t)h * D4];
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    f32x4 out;
    out[0] = acc[0] / hq;
    out[1] = acc[1] / hq;
    out[2] = acc[2] / hq;
    out[3] = acc[3] / hq;
    ((f32x4*)Gs)[i] = out;
  }
}

// G: [M, Hq·D] float32; Gs: [M, D] float32; D a multiple of 4.
hipError_t launch_gate_head_mean(const float* G, float* Gs, int64_t M, int Hq, int D, hipStream_t st) {
  const int D4 = D / 4;
  const int64_t n4 = M * D4;
  const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div<int64_t>(n4, 256), 16384);
  hipLaunchKernelGGL(gate_head_mean_kernel, dim3(blocks), dim3(256), 0, st, G, Gs, n4, Hq, D4);
  return hipGetLastError();
}

}  // namespace gsa
