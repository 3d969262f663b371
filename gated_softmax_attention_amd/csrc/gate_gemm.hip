// Gate projection with fused sigmoid: G = σ(X·W_θ)  (bias-free).
//
// Source: "GatedAttention [2025]" page, §1.2.2 gating equation Y' = Y ⊙ σ(X W_θ)
// with σ the logistic sigmoid (default activation, same section); the bias-free
// projection matches the GatedAttentionOutput snippet on the "10 · 门控" page,
// §3.2.  X is [M, K] (token rows × d_model), W_θ is [K, N] (d_model × gate
// width), G is [M, N] float32.
//
// bf16 path: 128×128 output tile per 256-thread workgroup (4 waves in a 2×2
// grid, 64×64 per wave = 2×2 MFMA 32x32x16 tiles), K staged 64 at a time in LDS,
// double-buffered through registers.  The MFMA B operand needs 8 consecutive k
// values of one W column per lane, while W rows are n-contiguous in memory, so
// each thread loads a 4(k)×8(n) block and writes it to LDS transposed
// ([n][k] layout).  The sigmoid is applied in the register epilogue and G is
// written once in float32.
#include "common.h"

namespace gsa {

namespace gemm {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LD = BK + 8;  // LDS row stride in bf16 (144 B: 16-B aligned, rotates banks by 4 per row)
}  // namespace gemm

__global__ __launch_bounds__(256, 2)
void gate_gemm_bf16_kernel(const bf16* __restrict__ X, const bf16* __restrict__ W,
                           float* __restrict__ G, int M, int K, int N, int tiles_n,
                           int apply_sigmoid) {
  using namespace gemm;
  __shared__ __align__(16) bf16 As[2][BM * LD];
  __shared__ __align__(16) bf16 Bs[2][BN * LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hl = lane >> 5;

  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const bool n_vec = (N % 8) == 0;

  // A loader: thread reads 16 B (8 k) of rows (tid>>3) + 32*i, chunk tid&7.
  const int a_row = tid >> 3, a_ch = tid & 7;
  // B loader: thread reads k rows 4*kg .. 4*kg+3 at columns 8*ng .. 8*ng+7.
  const int b_kg = tid & 15, b_ng = tid >> 4;

  u32x4 areg[4], breg[4];

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + a_row + 32 * i;
      const int k = k0 + a_ch * 8;
      if (m < M && k < K)
        areg[i] = *(const u32x4*)(X + m * K + k);
      else
        areg[i] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = k0 + 4 * b_kg + r;
      const int n = n0 + 8 * b_ng;
      if (k < K && n_vec && n + 8 <= N) {
        breg[r] = *(const u32x4*)(W + (int64_t)k * N + n);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          h[e] = (k < K && n + e < N) ? __builtin_bit_cast(uint16_t, W[(int64_t)k * N + n + e]) : 0;
        breg[r] = u32x4{h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16),
                        h[4] | (uint32_t(h[5]) << 16), h[6] | (uint32_t(h[7]) << 16)};
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(u32x4*)(&As[buf][(a_row + 32 * i) * LD + a_ch * 8]) = areg[i];
    // transpose the 4(k) x 8(n) block: column e gets {k0..k3} as 8 bytes
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      const int sh = (e & 1) * 16;
      const uint32_t h0 = (breg[0][w] >> sh) & 0xffffu, h1 = (breg[1][w] >> sh) & 0xffffu;
      const uint32_t h2 = (breg[2][w] >> sh) & 0xffffu, h3 = (breg[3][w] >> sh) & 0xffffu;
      *(u32x2*)(&Bs[buf][(8 * b_ng + e) * LD + 4 * b_kg]) = u32x2{h0 | (h1 << 16), h2 | (h3 << 16)};
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = ceil_div(K, BK);
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *(const bf16x8*)(&As[buf][(wm * 64 + t * 32 + l32) * LD + ks * 16 + 8 * hl]);
        b[t] = *(const bf16x8*)(&Bs[buf][(wn * 64 + t * 32 + l32) * LD + ks * 16 + 8 * hl]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column l32 and rows 8*(r/4) + 4*hl + r%4 of each 32x32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (m < M && n < N) {
          const float z = acc[i][j][r];
          G[m * N + n] = apply_sigmoid ? sigmoidf(z) : z;
        }
      }
    }
}

// float32 gate projection: 64×64 tile per 256 threads, 4×4 outputs per thread.
__global__ __launch_bounds__(256)
void gate_gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                          float* __restrict__ G, int M, int K, int N, int tiles_n,
                          int apply_sigmoid) {
  constexpr int T = 64, TK = 16;
  __shared__ float As[TK][T + 4];
  __shared__ float Bs[TK][T + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * T;
  const int n0 = (blockIdx.x % tiles_n) * T;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
    for (int idx = tid; idx < T * TK; idx += 256) {
      const int r = idx / TK, c = idx % TK;         // A: row r, k c
      const int64_t m = m0 + r;
      As[c][r] = (m < M && k0 + c < K) ? X[m * K + k0 + c] : 0.f;
      const int kr = idx / T, nc = idx % T;         // B: k kr, col nc
      Bs[kr][nc] = (k0 + kr < K && n0 + nc < N) ? W[(int64_t)(k0 + kr) * N + n0 + nc] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = m0 + ty * 4 + i;
      const int n = n0 + tx * 4 + j;
      if (m < M && n < N) G[m * N + n] = apply_sigmoid ? sigmoidf(acc[i][j]) : acc[i][j];
    }
}

hipError_t launch_gate_gemm(const void* X, const void* W, float* G, int64_t M, int64_t K, int64_t N,
                            bool bf16_inputs, bool apply_sigmoid, hipStream_t stream) {
  if (bf16_inputs) {
    const int tiles_n = (int)ceil_div<int64_t>(N, gemm::BN);
    const int64_t tiles = ceil_div<int64_t>(M, gemm::BM) * tiles_n;
    hipLaunchKernelGGL(gate_gemm_bf16_kernel, dim3((unsigned)tiles), dim3(256), 0, stream,
                       (const bf16*)X, (const bf16*)W, G, (int)M, (int)K, (int)N, tiles_n,
                       (int)apply_sigmoid);
  } else {
    const int tiles_n = (int)ceil_div<int64_t>(N, 64);
    const int64_t tiles = ceil_div<int64_t>(M, 64) * tiles_n;
    hipLaunchKernelGGL(gate_gemm_f32_kernel, dim3((unsigned)tiles), dim3(256), 0, stream,
                       (const float*)X, (const float*)W, G, (int)M, (int)K, (int)N, tiles_n,
                       (int)apply_sigmoid);
  }
  return hipGetLastError();
}

}  // namespace gsa
