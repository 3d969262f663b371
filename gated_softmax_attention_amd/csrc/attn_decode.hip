// Gated SDPA decode: one query token per batch against a contiguous KV cache.
//
// Sources: "GatedAttention [2025]" page — §1.2.1 SDPA equation, §1.2.2 gating
// equation; the KV cache and its role as the memory-bandwidth bottleneck of
// autoregressive decoding are from the §1.3.1 GQA explainer, and GQA lets a
// group of query heads share each cached key/value head.
//
// Split kernel: workgroup (split s, key/value heads, batch b, quad of query
// heads) streams keys [s*chunk, (s+1)*chunk) once and serves up to 4 query
// heads of each key/value head's group.  When 4 divides the key/value head
// count a workgroup takes 4 adjacent heads, one per wave, and a stage holds 16
// keys of all 4 (each key's 4-head row is one contiguous 1 KB read at D = 128;
// 7.0 TB/s against 6.7 with one head's 256-byte rows); otherwise it takes one
// head and each wave 16 keys of a 64-key stage.  Either way a stage is 32 KB
// of K and V (D = 128) moving global -> LDS through a ring of 4 stages filled
// by 16-byte direct loads, so ~96 KB per workgroup stay in flight independent
// of the register file.  Per wave and 16 keys:
//   S = Q·Kᵀ on v_mfma_f32_16x16x32_bf16 with the (≤4) query rows replicated
//     over the 16 MFMA rows, so every lane ends up holding the 4 heads' scores
//     for "its" key;
//   block max over the 16 keys by DPP row exchanges, online rescale,
//     p = exp2(t − m);
//   O += p·V on the VALU, each lane accumulating its key's contribution for 32
//     of the 128 dims (reduced over the 16 key lanes once, at the end).
// LDS rows are 16-byte-chunk swizzled (chunk ^= key & 15) so the 16 keys a
// wave reads at one chunk hit distinct banks.
// With one head per workgroup the 4 waves' (m, l, O) are merged through LDS;
// with 4, each wave's own (m, l, O) is final.  Either way one float32 partial
// (O, m, l) is written per query head and split.  The merge kernel combines the
// splits exactly: m* = max m_s, l* = Σ l_s 2^{m_s − m*}, O* = Σ O_s 2^{m_s − m*},
// then O*/l* times the gate, rounded once to bf16.
#include "common.h"

namespace gsa {

namespace dec {
constexpr int KB = 16;          // keys per MFMA block (one wave)
constexpr int WAVES = 4;
constexpr int TK = KB * WAVES;  // keys per LDS stage
constexpr int NS = 4;           // LDS ring depth
}  // namespace dec

// max / sum over the 16 lanes of a DPP row (quad swaps, then half-row and row mirrors)
__device__ __forceinline__ float dpp_f(float x, int ctrl_sel) {
  int v = __float_as_int(x);
  switch (ctrl_sel) {
    case 0: v = __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false); break;   // quad_perm(1,0,3,2)
    case 1: v = __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false); break;   // quad_perm(2,3,0,1)
    case 2: v = __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: v = __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return __int_as_float(v);
}
__device__ __forceinline__ float row16_max(float x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x = fmaxf(x, dpp_f(x, i));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x += dpp_f(x, i);
  return x;
}

enum : int { kDecGateNone = 0, kDecGateElem = 1, kDecGateHead = 2 };

// LDS of one split workgroup: the K/V ring and the wave-merge records.
template <int D>
struct DecSmem {
  bf16 Ks[dec::NS][dec::TK * D];
  bf16 Vs[dec::NS][dec::TK * D];
  float sm_m[dec::WAVES][4], sm_l[dec::WAVES][4];
  float sm_o[dec::WAVES][4][D];
};

// The split workgroup (split s, key/value head group and quad yq, batch b) on
// the LDS sm.  HW = 1: the workgroup takes one key/value head and its 4 waves
// take 16 keys each of a 64-key stage; HW = 4: it takes 4 adjacent key/value
// heads, wave w the (w+1)-th, and a stage holds 16 keys of all 4, so each key's
// cached row of the 4 heads (4·D·2 bytes) is read as one contiguous piece.
template <int D, int HW>
__device__ __forceinline__ void decode_split_body(DecSmem<D>& sm, const bf16* __restrict__ Q,
                                                  const bf16* __restrict__ Kc, const bf16* __restrict__ Vc,
                                                  float* __restrict__ part, int L, int Hq, int Hkv, int nsplit,
                                                  int chunk, float scale_log2, int s, int yq, int b) {
  using namespace dec;
  static_assert(D == 128 || D == 64, "head dim");
  constexpr int NKK = D / 32;          // 32-dim MFMA k steps (and 8-dim chunks per lane)
  constexpr int PST = D + 4;           // partial record stride (floats)
  auto& sm_m = sm.sm_m;
  auto& sm_l = sm.sm_l;
  auto& sm_o = sm.sm_o;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kl = lane & 15, jg = lane >> 4;
  static_assert(HW == 1 || HW == WAVES, "one key/value head per workgroup, or one per wave");
  const int G = Hq / Hkv;
  const int nquad = (G + 3) / 4;
  const int c0 = (yq / nquad) * HW, quad = yq % nquad;   // the workgroup's first key/value head
  const int c = HW == 1 ? c0 : c0 + wave;                 // this wave's key/value head
  const int h0 = c * G + quad * 4;
  const int nq = min(4, G - quad * 4);
  constexpr int TKS = HW == 1 ? TK : KB;                  // keys per stage

  const int key_begin = s * chunk;
  const int key_end = min(L, key_begin + chunk);

  const int64_t kv_row = (int64_t)Hkv * D;
  const bf16* Kb = Kc + (int64_t)b * L * kv_row + (int64_t)c0 * D;
  const bf16* Vb = Vc + (int64_t)b * L * kv_row + (int64_t)c0 * D;

  // A operand: MFMA row m = kl holds query slot kl % 4 (rows replicated 4x)
  bf16x8 qa[NKK];
  {
    const int slot = kl & 3;
    const int h = h0 + min(slot, nq - 1);
    const bf16* qp = Q + ((int64_t)b * Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qa[kk] = *(const bf16x8*)(qp + 32 * kk + 8 * jg);
    // settle the Q loads here: the ring's direct loads are invisible to the
    // compiler's counters, which would otherwise wait for all of them inside the loop
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qa[kk]));
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

  // ---- LDS ring of NS stages, each K[TKS][HW·D] and V[TKS][HW·D]; a stage row
  // is one key of the HW heads, each head's D values chunk-swizzled by key
  constexpr int CHK = D / 8;                         // 16-byte chunks per head and key
  constexpr int RCH = HW * CHK;                      // chunks per stage row
  auto& Ks = sm.Ks;
  auto& Vs = sm.Vs;
  static_assert(TKS * RCH == TK * CHK, "a stage holds the same bytes in either arrangement");
  constexpr int NI = TK * CHK / 64 / WAVES;          // direct loads per wave, stage and tensor
  const uint32_t row_b = (uint32_t)(kv_row * 2);
  const uint32_t kv_bytes = (uint32_t)(((int64_t)L * kv_row - (int64_t)c0 * D) * 2);
  const auto krs = make_rsrc(Kb, kv_bytes);          // keys >= L read as zeros
  const auto vrs = make_rsrc(Vb, kv_bytes);
  uint32_t dma_off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int sl = (wave + WAVES * i) * 64 + lane;
    const int row = sl / RCH, hw = (sl % RCH) / CHK, phys = sl % CHK;
    dma_off[i] = (uint32_t)row * row_b + (uint32_t)(hw * D * 2) + (uint32_t)((phys ^ (row & (CHK - 1))) * 16);
  }
  const int nkeys = key_end - key_begin;
  const int n_st = ceil_div(nkeys, TKS);
  auto dma = [&](int st) {
    const int buf = st % NS;
    const uint32_t base = (uint32_t)(key_begin + st * TKS) * row_b;
    const uint32_t kd = __builtin_amdgcn_readfirstlane(lds_addr(&Ks[buf][0]));
    const uint32_t vd = __builtin_amdgcn_readfirstlane(lds_addr(&Vs[buf][0]));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t ins = (uint32_t)(wave + WAVES * i) * 64 * 16;
      dma16_lds_nt(krs, dma_off[i] + base, kd + ins);   // the cache is read once: streaming policy
      dma16_lds_nt(vrs, dma_off[i] + base, vd + ins);
    }
  };
  // wait until at most n stages of this wave's loads are still in flight
  auto wait_stages = [&](int n) {
    if (n >= 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * 2 * NI) : "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * NI) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  // this lane's key row within a stage, and where this wave's head starts in it
  const int my_row = HW == 1 ? wave * KB + kl : kl;
  const int head_chunk = HW == 1 ? 0 : wave * CHK;

#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < n_st) dma(st);
  for (int t = 0; t < n_st; ++t) {
    wait_stages(min(NS - 2, n_st - 1 - t));
    __syncthreads();                                 // stage t complete; stage t-1 free
    if (t + NS - 1 < n_st) dma(t + NS - 1);
    const int buf = t % NS;
    const int key = key_begin + t * TKS + my_row;
    u32x4 kcur[NKK], vcur[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int ch = head_chunk + ((4 * kk + jg) ^ (my_row & (CHK - 1)));
      kcur[kk] = *(const u32x4*)(&Ks[buf][(my_row * RCH + ch) * 8]);
      vcur[kk] = *(const u32x4*)(&Vs[buf][(my_row * RCH + ch) * 8]);
    }

    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      sacc = mfma16x16x32(qa[kk], __builtin_bit_cast(bf16x8, kcur[kk]), sacc);
    // sacc[r] = score of query slot r against this lane's key
    float tt[4], alpha[4], m_use[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      tt[r] = key < key_end ? sacc[r] * scale_log2 : -INFINITY;
      const float mx = row16_max(tt[r]);
      const float m_new = fmaxf(m_run[r], mx);
      // a wave whose keys so far are all masked keeps m = -inf; exponentiate
      // against 0 then, so that alpha and p come out 0 rather than NaN
      m_use[r] = m_new == -INFINITY ? 0.f : m_new;
      alpha[r] = fast_exp2(m_run[r] - m_use[r]);
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
      const float p = fast_exp2(tt[r] - m_use[r]);
      l_run[r] = l_run[r] * alpha[r] + p;
      if (alpha[r] != 1.0f) {   // uniform within a DPP row: m_run is the 16-key max
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
    l_run[r] = row16_sum(l_run[r]);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][kk][e] = row16_sum(o[r][kk][e]);
  }
  if constexpr (HW != 1) {
    // each wave has its own query heads and saw every key of the split: its
    // (O, m, l) is the record
    if (kl == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r >= nq) continue;
        float* rec = part + (((int64_t)b * Hq + h0 + r) * nsplit + s) * PST;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) rec[32 * kk + 8 * jg + e] = o[r][kk][e];
        if (jg == 0) {
          rec[D] = m_run[r];
          rec[D + 1] = l_run[r];
        }
      }
    }
    return;
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

template <int D, int HW>
__global__ __launch_bounds__(256)
void decode_split_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ Kc,
                              const bf16* __restrict__ Vc, float* __restrict__ part,
                              int L, int Hq, int Hkv, int nsplit, int chunk, float scale_log2) {
  __shared__ __align__(16) DecSmem<D> sm;
  decode_split_body<D, HW>(sm, Q, Kc, Vc, part, L, Hq, Hkv, nsplit, chunk, scale_log2, blockIdx.x, blockIdx.y,
                           blockIdx.z);
}

// Building with -DGSA_DEC_HW=1 keeps one key/value head per split workgroup for
// every head count (the arrangement the 4-head one is compared against).
#ifndef GSA_DEC_HW
#define GSA_DEC_HW 4
#endif
static_assert(GSA_DEC_HW == 4 || GSA_DEC_HW == 1, "GSA_DEC_HW is 4 or 1");
// Key/value heads per split workgroup: 4 when they divide Hkv (each key's row
// of the 4 heads is one contiguous read), else 1.
int decode_heads_per_workgroup(int64_t Hkv) { return (GSA_DEC_HW == 4 && Hkv % 4 == 0) ? 4 : 1; }

template <int D>
static void launch_split(const void* Q, const void* K, const void* V, float* part, int B, int L, int Hq, int Hkv,
                         int nsplit, int chunk, float scale_log2, hipStream_t st) {
  const int nquad = (Hq / Hkv + 3) / 4;
  if (decode_heads_per_workgroup(Hkv) == 4)
    hipLaunchKernelGGL((decode_split_bf16_kernel<D, 4>), dim3(nsplit, (Hkv / 4) * nquad, B), dim3(256), 0, st,
                       (const bf16*)Q, (const bf16*)K, (const bf16*)V, part, L, Hq, Hkv, nsplit, chunk, scale_log2);
  else
    hipLaunchKernelGGL((decode_split_bf16_kernel<D, 1>), dim3(nsplit, Hkv * nquad, B), dim3(256), 0, st,
                       (const bf16*)Q, (const bf16*)K, (const bf16*)V, part, L, Hq, Hkv, nsplit, chunk, scale_log2);
}

// The merge for the whole gated decode step (elementwise gate, bf16): the
// gate's split-K partial logits are added here, in part order, and σ applied,
// so O*/l*·σ(Σ_s gate_part[s]) is rounded once.  The same operations in the
// same order as the part sum of the split-K gate followed by the plain merge.
template <int D>
__global__ __launch_bounds__(D)
void decode_merge_gatesum_bf16_kernel(const float* __restrict__ part, const float* __restrict__ gate_part,
                                      bf16* __restrict__ Y, int B, int Hq, int nsplit, int gsplits) {
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
  const int64_t n = (int64_t)Hq * D, col = (int64_t)h * D + d;
  float z = gate_part[(int64_t)b * n + col];
  for (int s = 1; s < gsplits; ++s) z += gate_part[((int64_t)s * B + b) * n + col];
  float y = osum / lsum;
  y *= sigmoidf(z);
  Y[((int64_t)b * Hq + h) * D + d] = (bf16)y;
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

// Design-space epilogue of the merge ("GatedAttention [2025]" §1.2.2 items
// (3)-(5), §1.4.1 RMSNorm): layout 0 none, 1 elementwise (gate column h·D + d),
// 2 headwise (column h), 3 head-shared (column d); add: Y + g instead of Y ⊙ g;
// rms: the merged head output is first divided by sqrt(mean_d y² + ε) (unit
// weight, ε = 1e-6).  G holds already-activated gate values, [B, N].
struct DecEpi {
  int layout, add, rms;
};
constexpr float kDecRmsEps = 1e-6f;

template <int D>
__global__ __launch_bounds__(D)
void decode_merge_variant_bf16_kernel(const float* __restrict__ part, const float* __restrict__ Gate,
                                      bf16* __restrict__ Y, int Hq, int nsplit, DecEpi ep) {
  constexpr int PST = D + 4;
  __shared__ float red[D / 64];
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
  if (ep.rms) {
    // sum of squares over the head's D values: each wave, then the waves in order
    float ss = y * y;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((d & 63) == 0) red[d >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < D / 64; ++w) tot += red[w];
    y *= 1.0f / sqrtf(tot / (float)D + kDecRmsEps);
  }
  if (ep.layout != kDecGateNone) {
    const float g = ep.layout == kDecGateElem ? Gate[((int64_t)b * Hq + h) * D + d]
                    : ep.layout == kDecGateHead ? Gate[(int64_t)b * Hq + h]
                                                : Gate[(int64_t)b * D + d];
    y = ep.add ? y + g : y * g;
  }
  Y[((int64_t)b * Hq + h) * D + d] = (bf16)y;
}

int64_t decode_auto_splits(int64_t B, int64_t L, int64_t Hq, int64_t Hkv) {
  const int64_t G = Hq / Hkv;
  const int hw = decode_heads_per_workgroup(Hkv);
  const int64_t base = B * (Hkv / hw) * ((G + 3) / 4);
  // One workgroup fits a CU (its LDS ring).  With 4 heads per workgroup aim
  // for one round on the 256 CUs (B 64, L 16384, 8 KV heads: 2 splits, 613 us,
  // against 636 us for 512 workgroups and 661 us for 1024); with one head per
  // workgroup for about 1024 (there 1024 workgroups ran 643 us, 512 ran 661 us).
  const int64_t target = hw == 4 ? 256 : 1024;
  int64_t ns = (target + base - 1) / base;
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
  launch_split<D>(Q, K, V, part, B, L, Hq, Hkv, nsplit, chunk, scale_log2, st);
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

hipError_t launch_decode_variant_bf16(const void* Q, const void* K, const void* V, const float* G, void* Y,
                                      void* workspace, int B, int L, int Hq, int Hkv, int D, int layout, int add,
                                      int rms, int nsplit, hipStream_t st) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  const int chunk = (int)decode_chunk(L, nsplit);
  float* part = (float*)workspace;
  const DecEpi ep{layout, add, rms};
  if (D == 128) {
    launch_split<128>(Q, K, V, part, B, L, Hq, Hkv, nsplit, chunk, scale_log2, st);
    hipLaunchKernelGGL((decode_merge_variant_bf16_kernel<128>), dim3(Hq, B), dim3(128), 0, st, (const float*)part,
                       G, (bf16*)Y, Hq, nsplit, ep);
  } else {
    launch_split<64>(Q, K, V, part, B, L, Hq, Hkv, nsplit, chunk, scale_log2, st);
    hipLaunchKernelGGL((decode_merge_variant_bf16_kernel<64>), dim3(Hq, B), dim3(64), 0, st, (const float*)part,
                       G, (bf16*)Y, Hq, nsplit, ep);
  }
  return hipGetLastError();
}

// Decode with the elementwise gate given as gsplits float32 partial logits
// ([gsplits, B, Hq·D], from the split-K gate): the split kernel, then the merge
// that adds the parts and applies σ.
hipError_t launch_decode_gateparts_bf16(const void* Q, const void* K, const void* V, const float* gate_part,
                                        int gsplits, void* Y, void* workspace, int B, int L, int Hq, int Hkv, int D,
                                        int nsplit, hipStream_t st) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  const int chunk = (int)decode_chunk(L, nsplit);
  float* part = (float*)workspace;
  if (D == 128) {
    launch_split<128>(Q, K, V, part, B, L, Hq, Hkv, nsplit, chunk, scale_log2, st);
    hipLaunchKernelGGL((decode_merge_gatesum_bf16_kernel<128>), dim3(Hq, B), dim3(128), 0, st, (const float*)part,
                       gate_part, (bf16*)Y, B, Hq, nsplit, gsplits);
  } else {
    launch_split<64>(Q, K, V, part, B, L, Hq, Hkv, nsplit, chunk, scale_log2, st);
    hipLaunchKernelGGL((decode_merge_gatesum_bf16_kernel<64>), dim3(Hq, B), dim3(64), 0, st, (const float*)part,
                       gate_part, (bf16*)Y, B, Hq, nsplit, gsplits);
  }
  return hipGetLastError();
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
