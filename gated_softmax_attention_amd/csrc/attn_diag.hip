// First-token attention share: for query head h and row i,
//   F[b, h, i] = exp(q_i·k_0/√D − LSE_i),
// the causal softmax probability the row gives token 0 (the F-Attn measure of
// the "GatedAttention [2025]" page, §1.4.3 and Table 4; the average attention
// on the first token in "10 · 门控" §3.4), from the LSE the forward saved.
// Optionally also per-head means over batches and rows, and their mean.
//
// HBM-bound: every Q row is read once (D/8 or D/4 threads per row, 16-byte
// loads, four rows per thread with all loads issued first), key 0 of each
// group is an L2-resident row, and F is written once, contiguously.  The means are reduced in a
// fixed order (no atomics), so repeated calls agree bit for bit.
#include "common.h"

namespace gsa {

template <int D, typename T>
__global__ __launch_bounds__(256)
void first_token_share_kernel(const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ Lse,
                              float* __restrict__ F, int B, int S, int Hq, int Hkv, float scale_log2) {
  constexpr int E = 16 / sizeof(T);          // elements per 16-byte load
  constexpr int TPR = D / E;                 // threads per row
  constexpr int RPB = 256 / TPR;             // rows per block and pass
  constexpr int NR = 4;                      // passes: rows per thread, all loads issued first
  const int tid = threadIdx.x;
  const int64_t nrows = (int64_t)B * S * Hq;
  const int part = tid % TPR;
  u32x4 qv[NR], kv[NR];
  float lse[NR];
  int64_t fo[NR], kofs = -1;
  bool live[NR];
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    // rows in F's order, (b*Hq + h)*S + i: F and LSE are touched contiguously,
    // and each Q row is one full 256-byte (D = 128, bf16) segment
    const int64_t row = ((int64_t)blockIdx.x * NR + n) * RPB + tid / TPR;
    live[n] = row < nrows;
    const int64_t rr = live[n] ? row : nrows - 1;
    const int i = (int)(rr % S);
    const int64_t bh = rr / S;
    const int h = (int)(bh % Hq);
    const int b = (int)(bh / Hq);
    const int c = h / (Hq / Hkv);
    qv[n] = *(const u32x4*)(Q + (((int64_t)b * S + i) * Hq + h) * D + part * E);
    // key 0 of head c: the rows of a block nearly always share (b, c), so it is
    // loaded only when that changes
    const int64_t ko = ((int64_t)b * S * Hkv + c) * D + part * E;
    if (n == 0 || ko != kofs) kv[n] = *(const u32x4*)(K + ko);
    else kv[n] = kv[n - 1];
    kofs = ko;
    fo[n] = rr;
    lse[n] = Lse[rr];
  }
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    float dot = 0.f;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dot = fmaf(bf16_lo(qv[n][w]), bf16_lo(kv[n][w]), dot);
        dot = fmaf(bf16_hi(qv[n][w]), bf16_hi(kv[n][w]), dot);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) dot = fmaf(__uint_as_float(qv[n][w]), __uint_as_float(kv[n][w]), dot);
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) dot += __shfl_xor(dot, o);
    if (live[n] && part == 0) F[fo[n]] = fast_exp2(fmaf(dot, scale_log2, -lse[n] * kLog2e));
  }
}

// head_mean[h] = Σ_{b, i} F[b, h, i] / (B·S): one 1024-thread block per head;
// thread t sums elements t, t + 1024, ... of each batch's row in eight
// independent chains (so eight loads are in flight), the chains are added in a
// fixed order, then a fixed tree over the threads.
__global__ __launch_bounds__(1024)
void first_token_head_mean_kernel(const float* __restrict__ F, float* __restrict__ head_mean, int B, int S,
                                  int Hq) {
  __shared__ float part[1024];
  const int h = blockIdx.x, tid = threadIdx.x;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < B; ++b) {
    const float* f = F + ((int64_t)b * Hq + h) * S;
    int i = tid;
    for (; i + 7 * 1024 < S; i += 8 * 1024) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += f[i + u * 1024];
    }
    for (int u = 0; i < S; i += 1024, ++u) acc[u & 7] += f[i];   // at most 7 more
  }
  float a = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) a += acc[u];
  part[tid] = a;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) head_mean[h] = part[0] / ((float)B * (float)S);
}

// head_mean[Hq] = mean of the Hq per-head means, summed in head order.
__global__ void first_token_overall_mean_kernel(float* __restrict__ head_mean, int Hq) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    float s = 0.f;
    for (int h = 0; h < Hq; ++h) s += head_mean[h];
    head_mean[Hq] = s / (float)Hq;
  }
}

template <int D, typename T>
static hipError_t launch_fts(const void* Q, const void* K, const float* Lse, float* F, float* head_mean, int B,
                             int S, int Hq, int Hkv, hipStream_t st) {
  constexpr int TPR = D / (16 / sizeof(T));
  constexpr int RPB = 256 / TPR * 4;   // rows per block: 4 passes of 256 / TPR
  const int64_t rows = (int64_t)B * S * Hq;
  const float scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((first_token_share_kernel<D, T>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     st, (const T*)Q, (const T*)K, Lse, F, B, S, Hq, Hkv, scale_log2);
  if (head_mean != nullptr) {
    hipLaunchKernelGGL(first_token_head_mean_kernel, dim3(Hq), dim3(1024), 0, st, (const float*)F, head_mean, B,
                       S, Hq);
    hipLaunchKernelGGL(first_token_overall_mean_kernel, dim3(1), dim3(64), 0, st, head_mean, Hq);
  }
  return hipGetLastError();
}

hipError_t launch_first_token_share(const void* Q, const void* K, const float* Lse, float* F, float* head_mean,
                                    int B, int S, int Hq, int Hkv, int D, bool bf16_inputs, hipStream_t st) {
  if (bf16_inputs)
    return D == 128 ? launch_fts<128, bf16>(Q, K, Lse, F, head_mean, B, S, Hq, Hkv, st)
                    : launch_fts<64, bf16>(Q, K, Lse, F, head_mean, B, S, Hq, Hkv, st);
  return D == 128 ? launch_fts<128, float>(Q, K, Lse, F, head_mean, B, S, Hq, Hkv, st)
                  : launch_fts<64, float>(Q, K, Lse, F, head_mean, B, S, Hq, Hkv, st);
}

}  // namespace gsa
