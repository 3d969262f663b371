// Gated SDPA decode: one query token per batch against a contiguous KV cache.
//
// Sources: "GatedAttention [2025]" page — §1.2.1 SDPA equation, §1.2.2 gating
// equation; the KV cache and its role as the memory-bandwidth bottleneck of
// autoregressive decoding are from the §1.3.1 GQA explainer, and GQA lets a
// group of query heads share each cached key/value head.
//
// Split kernel: workgroup (split s, key/value head c, batch b, quad of query
// heads) streams keys [s*chunk, (s+1)*chunk) of head c once and serves up to 4
// query heads of c's group.  Each wave takes 16-key blocks; per block:
//   S = Q·Kᵀ on v_mfma_f32_16x16x32_bf16 with the (≤4) query rows replicated
//     over the 16 MFMA rows, so every lane ends up holding the 4 heads' scores
//     for "its" key, and K goes from HBM straight into MFMA operand registers
//     (16 B per lane, no LDS);
//   block max over the 16 keys by lane exchanges, online rescale, p = exp2(t − m);
//   O += p·V on the VALU, each lane accumulating its key's contribution for 32
//     of the 128 dims (reduced over the 16 key lanes once, at the end).
// The workgroup merges its 4 waves' (m, l, O) through LDS and writes one
// float32 partial (O, m, l) per query head.  The merge kernel combines the
// splits exactly: m* = max m_s, l* = Σ l_s 2^{m_s − m*}, O* = Σ O_s 2^{m_s − m*},
// then O*/l* times the gate, rounded once to bf16.
#include "common.h"

namespace gsa {

namespace dec {
constexpr int KB = 16;          // keys per MFMA block
constexpr int WAVES = 4;
}  // namespace dec

enum : int { kDecGateNone = 0, kDecGateElem = 1, kDecGateHead = 2 };

template <int D>
__global__ __launch_bounds__(256)
void decode_split_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ Kc,
                              const bf16* __restrict__ Vc, float* __restrict__ part,
                              int L, int Hq, int Hkv, int nsplit, int chunk, float scale_log2) {
  using namespace dec;
  static_assert(D == 128 || D == 64, "head dim");
  constexpr int NKK = D / 32;          // 32-dim MFMA k steps (and 8-dim chunks per lane)
  constexpr int PST = D + 4;           // partial record stride (floats)
  __shared__ float sm_m[WAVES][4], sm_l[WAVES][4];
  __shared__ float sm_o[WAVES][4][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kl = lane & 15, jg = lane >> 4;
  const int s = blockIdx.x;
  const int G = Hq / Hkv;
  const int nquad = (G + 3) / 4;
  const int c = blockIdx.y / nquad, quad = blockIdx.y % nquad;
  const int b = blockIdx.z;
  const int h0 = c * G + quad * 4;
  const int nq = min(4, G - quad * 4);

  const int key_begin = s * chunk;
  const int key_end = min(L, key_begin + chunk);
  const int n_blocks = ceil_div(key_end - key_begin, KB);

  const int64_t kv_row = (int64_t)Hkv * D;
  const bf16* Kb = Kc + (int64_t)b * L * kv_row + (int64_t)c * D;
  const bf16* Vb = Vc + (int64_t)b * L * kv_row + (int64_t)c * D;

  // A operand: MFMA row m = kl holds query slot kl % 4 (rows replicated 4x)
  bf16x8 qa[NKK];
  {
    const int slot = kl & 3;
    const int h = h0 + min(slot, nq - 1);
    const bf16* qp = Q + ((int64_t)b * Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qa[kk] = *(const bf16x8*)(qp + 32 * kk + 8 * jg);
  }

  float m_run[4], l_run[4], o[4][NKK][8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][kk][e] = 0.f;
  }

  u32x4 kreg[NKK], vreg[NKK];
  auto load = [&](int blk) {
    const int key = key_begin + blk * KB + kl;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int64_t off = (int64_t)key * kv_row + 32 * kk + 8 * jg;
      kreg[kk] = key < key_end ? *(const u32x4*)(Kb + off) : u32x4{0, 0, 0, 0};
      vreg[kk] = key < key_end ? *(const u32x4*)(Vb + off) : u32x4{0, 0, 0, 0};
    }
  };

  int blk = wave;
  if (blk < n_blocks) load(blk);
  for (; blk < n_blocks; blk += WAVES) {
    u32x4 kcur[NKK], vcur[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) { kcur[kk] = kreg[kk]; vcur[kk] = vreg[kk]; }
    if (blk + WAVES < n_blocks) load(blk + WAVES);

    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      sacc = mfma16x16x32(qa[kk], __builtin_bit_cast(bf16x8, kcur[kk]), sacc);
    // sacc[r] = score of query slot r against key (key_begin + blk*16 + kl)
    const int key = key_begin + blk * KB + kl;
    float t[4], alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      t[r] = key < key_end ? sacc[r] * scale_log2 : -INFINITY;
      float mx = t[r];
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      mx = fmaxf(mx, __shfl_xor(mx, 8));
      const float m_new = fmaxf(m_run[r], mx);
      alpha[r] = fast_exp2(m_run[r] - m_new);
      m_run[r] = m_new;
    }
    float vf[NKK][8];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vf[kk][2 * w] = bf16_lo(vcur[kk][w]);
        vf[kk][2 * w + 1] = bf16_hi(vcur[kk][w]);
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(t[r] - m_run[r]);
      l_run[r] = l_run[r] * alpha[r] + p;
      if (alpha[r] != 1.0f) {   // uniform across the wave: m_run is a block-wide max
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[r][kk][e] *= alpha[r];
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][kk][e] = fmaf(p, vf[kk][e], o[r][kk][e]);
    }
  }

  // reduce over the 16 key lanes (lanes with equal jg hold the same dims)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float lr = l_run[r];
    lr += __shfl_xor(lr, 1);
    lr += __shfl_xor(lr, 2);
    lr += __shfl_xor(lr, 4);
    lr += __shfl_xor(lr, 8);
    l_run[r] = lr;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = o[r][kk][e];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        o[r][kk][e] = v;
      }
  }
  if (kl == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_o[wave][r][32 * kk + 8 * jg + e] = o[r][kk][e];
      if (jg == 0) {
        sm_m[wave][r] = m_run[r];
        sm_l[wave][r] = l_run[r];
      }
    }
  }
  __syncthreads();

  // merge the 4 waves and write one partial record per (query head, split)
  for (int idx = tid; idx < 4 * D; idx += 256) {
    const int r = idx / D, d = idx % D;
    if (r >= nq) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sm_m[w][r]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float f = fast_exp2(sm_m[w][r] - M);   // waves with no keys: exp2(-inf) = 0
      lsum += sm_l[w][r] * f;
      osum += sm_o[w][r][d] * f;
    }
    float* rec = part + (((int64_t)b * Hq + h0 + r) * nsplit + s) * PST;
    rec[d] = osum;
    if (d == 0) {
      rec[D] = M;
      rec[D + 1] = lsum;
    }
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(D)
void decode_merge_bf16_kernel(const float* __restrict__ part, const float* __restrict__ Gate,
                              bf16* __restrict__ Y, int Hq, int nsplit) {
  constexpr int PST = D + 4;
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* p = part + ((int64_t)b * Hq + h) * nsplit * PST;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, p[s * PST + D]);
  float lsum = 0.f, osum = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float f = fast_exp2(p[s * PST + D] - M);
    lsum += p[s * PST + D + 1] * f;
    osum += p[s * PST + d] * f;
  }
  float y = osum / lsum;
  const int64_t tok = b;
  if constexpr (MODE == kDecGateElem) y *= Gate[tok * Hq * D + (int64_t)h * D + d];
  if constexpr (MODE == kDecGateHead) y *= Gate[tok * Hq + h];
  Y[((int64_t)b * Hq + h) * D + d] = (bf16)y;
}

int64_t decode_auto_splits(int64_t B, int64_t L, int64_t Hq, int64_t Hkv) {
  const int64_t G = Hq / Hkv;
  const int64_t base = B * Hkv * ((G + 3) / 4);
  int64_t ns = (2048 + base - 1) / base;           // aim for >= 2048 workgroups
  const int64_t max_ns = (L + 255) / 256;          // but at least 256 keys per split
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  return ns;
}

int64_t decode_chunk(int64_t L, int64_t nsplit) {
  int64_t chunk = (L + nsplit - 1) / nsplit;
  chunk = (chunk + 15) / 16 * 16;
  return chunk;
}

template <int D>
static void launch_dec(const void* Q, const void* K, const void* V, const float* G, void* Y,
                       float* part, int B, int L, int Hq, int Hkv, int mode, int nsplit,
                       int chunk, float scale_log2, hipStream_t st) {
  const int Gq = Hq / Hkv;
  const int nquad = (Gq + 3) / 4;
  hipLaunchKernelGGL((decode_split_bf16_kernel<D>), dim3(nsplit, Hkv * nquad, B), dim3(256), 0, st,
                     (const bf16*)Q, (const bf16*)K, (const bf16*)V, part, L, Hq, Hkv, nsplit,
                     chunk, scale_log2);
  if (mode == kDecGateElem)
    hipLaunchKernelGGL((decode_merge_bf16_kernel<D, kDecGateElem>), dim3(Hq, B), dim3(D), 0, st,
                       (const float*)part, G, (bf16*)Y, Hq, nsplit);
  else if (mode == kDecGateHead)
    hipLaunchKernelGGL((decode_merge_bf16_kernel<D, kDecGateHead>), dim3(Hq, B), dim3(D), 0, st,
                       (const float*)part, G, (bf16*)Y, Hq, nsplit);
  else
    hipLaunchKernelGGL((decode_merge_bf16_kernel<D, kDecGateNone>), dim3(Hq, B), dim3(D), 0, st,
                       (const float*)part, G, (bf16*)Y, Hq, nsplit);
}

hipError_t launch_decode_bf16(const void* Q, const void* K, const void* V, const float* G, void* Y,
                              void* workspace, int B, int L, int Hq, int Hkv, int D, int mode,
                              int nsplit, hipStream_t stream) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  const int chunk = (int)decode_chunk(L, nsplit);
  float* part = (float*)workspace;
  if (D == 128)
    launch_dec<128>(Q, K, V, G, Y, part, B, L, Hq, Hkv, mode, nsplit, chunk, scale_log2, stream);
  else
    launch_dec<64>(Q, K, V, G, Y, part, B, L, Hq, Hkv, mode, nsplit, chunk, scale_log2, stream);
  return hipGetLastError();
}

}  // namespace gsa
