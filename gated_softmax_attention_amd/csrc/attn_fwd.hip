// Causal gated SDPA forward: Y' = softmax(Q·Kᵀ/√D, causal) · V ⊙ gate, per head.
//
// Sources: "GatedAttention [2025]" page — §1.2.1 SDPA equation, §1.4.1 per-head
// output equation (causal prefix j = 0..i), §1.2.2 gating equation and
// granularity (elementwise: one score per head dim; headwise: one per head),
// §1.3.1 GQA (a group of query heads shares one key/value head).  The gate is
// applied to each head's SDPA output before concatenation (G1 position, "10 ·
// 门控" page, §3.2 position table), so here it is the output epilogue and the
// ungated SDPA output never reaches HBM.
//
// bf16 kernel (gfx950 MFMA).  One 256-thread workgroup handles 128 query rows
// of one query head (4 waves × 32 rows) and walks the key/value tiles of 64
// keys that its rows can see, staging each K tile ([key][d]) and V tile
// (transposed, [d][key]) in LDS, double-buffered through registers.
// Per wave and tile:
//   Sᵀ = K·Qᵀ  on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the wave's
//              Q rows, held in registers for the whole kernel).  In the 32x32
//              accumulator layout a lane owns ONE query and 16 keys, so the
//              online-softmax max/sum are in-lane with a single exchange
//              between the two wave halves.
//   softmax    t = s·(log2 e/√D); m = max(m_old, max t); p = exp2(t − m), the
//              same rounded t feeding both m and p (so a lone visible key gets
//              p = 1 exactly); l accumulates p; O is rescaled by exp2(m_old − m).
//   Oᵀ += Vᵀ·Pᵀ on MFMA (A = Vᵀ rows from LDS, B = P rounded to bf16, taken
//              straight from the Sᵀ accumulators).  The k order of this product
//              follows the accumulator layout; the Vᵀ tile is stored with keys
//              permuted inside each 16-key block (offset bits 2 and 3 swapped)
//              so each lane's 8 keys are one 16-byte LDS read.
// Epilogue: O/l, times the float32 gate, one round-to-nearest-even to bf16.
#include "common.h"

namespace gsa {

namespace fwd {
constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile
}  // namespace fwd

enum : int { kGateNone = 0, kGateElem = 1, kGateHead = 2 };

// Position of key offset `ko` (0..63) inside a Vᵀ row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int ko) {
  return (ko & ~15) | ((ko & 4) << 1) | ((ko & 8) >> 1) | (ko & 3);
}

template <int D, int MODE>
__global__ __launch_bounds__(256, 2)
void attn_fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                          const bf16* __restrict__ V, const float* __restrict__ Gate,
                          bf16* __restrict__ Y, int B, int S, int Hq, int Hkv, int n_qtiles,
                          float scale_log2) {
  using namespace fwd;
  constexpr int KLD = D + 8;   // K tile row stride (bf16): 16-B aligned, 4-bank rotation per row
  constexpr int VLD = BN + 8;  // Vᵀ tile row stride (bf16)
  __shared__ __align__(16) bf16 Ks[2][BN * KLD];
  __shared__ __align__(16) bf16 Vt[2][D * VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;

  // heaviest (last) query tiles first, then heads, then batches
  const int bid = blockIdx.x;
  const int hb = Hq * B;
  const int qt = n_qtiles - 1 - bid / hb;
  const int head = (bid % hb) % Hq;
  const int b = (bid % hb) / Hq;
  const int kvh = head / (Hq / Hkv);

  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;  // first query row of this wave
  const int my_q = qw0 + l32;      // this lane's query row

  const int64_t q_row = (int64_t)Hq * D;
  const int64_t kv_row = (int64_t)Hkv * D;
  const bf16* Qb = Q + (int64_t)b * S * q_row + (int64_t)head * D;
  const bf16* Kb = K + (int64_t)b * S * kv_row + (int64_t)kvh * D;
  const bf16* Vb = V + (int64_t)b * S * kv_row + (int64_t)kvh * D;

  // Q fragments: B operand of Sᵀ = K·Qᵀ, lane holds Q[my_q][16*kk + 8*hl .. +7]
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (my_q < S) {
      qf[kk] = *(const bf16x8*)(Qb + (int64_t)my_q * q_row + 16 * kk + 8 * hl);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = (bf16)0.0f;
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = min(S, q0 + BM);
  const int n_kv = ceil_div(kv_end, BN);

  // K loader: KCH 16-B chunks per row, KRP rows per pass
  constexpr int KCH = D / 8, KRP = 256 / KCH, KPASS = BN / KRP;
  // V loader: VKR consecutive keys × 8 dims per thread
  constexpr int VKR = BN * D / (256 * 8), VKG = BN / VKR;
  const int k_row = tid / KCH, k_ch = tid % KCH;
  const int v_kg = tid % VKG, v_dg = tid / VKG;
  u32x4 kreg[KPASS], vreg[VKR];

  auto load_kv = [&](int k0) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int key = k0 + k_row + p * KRP;
      kreg[p] = key < S ? *(const u32x4*)(Kb + (int64_t)key * kv_row + k_ch * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < VKR; ++r) {
      const int key = k0 + v_kg * VKR + r;
      vreg[r] = key < S ? *(const u32x4*)(Vb + (int64_t)key * kv_row + v_dg * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_kv = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p)
      *(u32x4*)(&Ks[buf][(k_row + p * KRP) * KLD + k_ch * 8]) = kreg[p];
    const int pos = vt_pos(v_kg * VKR);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1, sh = (e & 1) * 16;
      bf16* dst = &Vt[buf][(v_dg * 8 + e) * VLD + pos];
      if constexpr (VKR == 4) {
        const uint32_t h0 = (vreg[0][w] >> sh) & 0xffffu, h1 = (vreg[1][w] >> sh) & 0xffffu;
        const uint32_t h2 = (vreg[2][w] >> sh) & 0xffffu, h3 = (vreg[3][w] >> sh) & 0xffffu;
        *(u32x2*)dst = u32x2{h0 | (h1 << 16), h2 | (h3 << 16)};
      } else {
        const uint32_t h0 = (vreg[0][w] >> sh) & 0xffffu, h1 = (vreg[1][w] >> sh) & 0xffffu;
        *(uint32_t*)dst = h0 | (h1 << 16);
      }
    }
  };

  const bool wave_rows_valid = qw0 < S;

  load_kv(0);
  store_kv(0);
  __syncthreads();
  for (int it = 0; it < n_kv; ++it) {
    const int buf = it & 1;
    const int k0 = it * BN;
    if (it + 1 < n_kv) load_kv(k0 + BN);

    // a wave whose rows all precede this tile's first key has nothing to do
    if (wave_rows_valid && k0 <= qw0 + 31) {
      f32x16 s[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sub][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 a = *(const bf16x8*)(&Ks[buf][(sub * 32 + l32) * KLD + 16 * kk + 8 * hl]);
          s[sub] = mfma32x32x16(a, qf[kk], s[sub]);
        }
      }
      // scale into the log2 domain and apply the causal / length mask
      const bool need_mask = (k0 + BN - 1 > qw0) || (k0 + BN > S);
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = s[sub][r] * scale_log2;
          if (need_mask) {
            const int key = k0 + sub * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (key > my_q || key >= S) t = -INFINITY;
          }
          s[sub][r] = t;
          mx = fmaxf(mx, t);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      float ps = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(s[sub][r] - m_new);
          s[sub][r] = p;
          ps += p;
        }
      l_run = l_run * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

      bf16x8 pb[2][2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[sub][t][e] = (bf16)s[sub][8 * t + e];

#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8 a = *(const bf16x8*)(&Vt[buf][(dt * 32 + l32) * VLD + sub * 32 + 16 * t + 8 * hl]);
            o[dt] = mfma32x32x16(a, pb[sub][t], o[dt]);
          }
    }

    if (it + 1 < n_kv) store_kv(buf ^ 1);
    __syncthreads();
  }

  if (my_q >= S) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  const int64_t tok = (int64_t)b * S + my_q;
  bf16* yrow = Y + tok * q_row + (int64_t)head * D;
  float gh = 1.0f;
  if constexpr (MODE == kGateHead) gh = Gate[tok * Hq + head];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = dt * 32 + 8 * i + 4 * hl;
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = o[dt][4 * i + j] * inv;
      if constexpr (MODE == kGateElem) {
        const f32x4 g = *(const f32x4*)(Gate + tok * q_row + (int64_t)head * D + d0);
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] *= g[j];
      } else if constexpr (MODE == kGateHead) {
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] *= gh;
      }
      *(u32x2*)(yrow + d0) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    }
}

// float32 kernel, also used for decode in float32: S query rows aligned to the
// END of Skv keys (query i sits at position i + Skv - S).  64 query rows per
// workgroup, 4 lanes per row splitting the head dimension, 32-key tiles in LDS.
template <int D, int MODE>
__global__ __launch_bounds__(256)
void attn_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                         const float* __restrict__ V, const float* __restrict__ Gate,
                         float* __restrict__ Y, int B, int S, int Skv, int Hq, int Hkv,
                         int n_qtiles, float scale_log2) {
  constexpr int BMF = 64, BNF = 32, DPL = D / 4, LDF = D + 4;
  __shared__ float Ks[BNF * LDF];
  __shared__ float Vs[BNF * LDF];
  const int tid = threadIdx.x;
  const int rq = tid >> 2, part = tid & 3;
  const int bid = blockIdx.x;
  const int hb = Hq * B;
  const int qt = n_qtiles - 1 - bid / hb;
  const int head = (bid % hb) % Hq;
  const int b = (bid % hb) / Hq;
  const int kvh = head / (Hq / Hkv);
  const int off = Skv - S;
  const int q = qt * BMF + rq;
  const int pos = q + off;
  const int64_t q_row = (int64_t)Hq * D, kv_row = (int64_t)Hkv * D;
  const float* Kb = K + (int64_t)b * Skv * kv_row + (int64_t)kvh * D;
  const float* Vb = V + (int64_t)b * Skv * kv_row + (int64_t)kvh * D;

  float qv[DPL], acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    qv[e] = q < S ? Q[((int64_t)b * S + q) * q_row + (int64_t)head * D + part * DPL + e] : 0.f;
    acc[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const int kv_end = min(Skv, qt * BMF + BMF + off);
  for (int k0 = 0; k0 < kv_end; k0 += BNF) {
    for (int idx = tid; idx < BNF * D; idx += 256) {
      const int j = idx / D, d = idx % D;
      const bool ok = k0 + j < Skv;
      Ks[j * LDF + d] = ok ? Kb[(int64_t)(k0 + j) * kv_row + d] : 0.f;
      Vs[j * LDF + d] = ok ? Vb[(int64_t)(k0 + j) * kv_row + d] : 0.f;
    }
    __syncthreads();
    float t[BNF];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) dot = fmaf(qv[e], Ks[j * LDF + part * DPL + e], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      float tj = dot * scale_log2;
      if (k0 + j > pos || k0 + j >= Skv) tj = -INFINITY;
      t[j] = tj;
      mx = fmaxf(mx, tj);
    }
    const float m_new = fmaxf(m_run, mx);
    if (m_new != -INFINITY) {
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] *= alpha;
#pragma unroll
      for (int j = 0; j < BNF; ++j) {
        const float p = fast_exp2(t[j] - m_new);
        l_run += p;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(p, Vs[j * LDF + part * DPL + e], acc[e]);
      }
    }
    __syncthreads();
  }
  if (q >= S) return;
  const float inv = 1.0f / l_run;
  const int64_t tok = (int64_t)b * S + q;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const int d = part * DPL + e;
    float y = acc[e] * inv;
    if constexpr (MODE == kGateElem) y *= Gate[tok * q_row + (int64_t)head * D + d];
    if constexpr (MODE == kGateHead) y *= Gate[tok * Hq + head];
    Y[tok * q_row + (int64_t)head * D + d] = y;
  }
}

template <int D, int MODE>
static void launch_bf16(const void* Q, const void* K, const void* V, const float* G, void* Y,
                        int B, int S, int Hq, int Hkv, float scale_log2, hipStream_t st) {
  const int nq = ceil_div(S, fwd::BM);
  const int64_t blocks = (int64_t)nq * Hq * B;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, MODE>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const bf16*)Q, (const bf16*)K, (const bf16*)V, G, (bf16*)Y, B, S, Hq, Hkv,
                     nq, scale_log2);
}

template <int D, int MODE>
static void launch_f32(const void* Q, const void* K, const void* V, const float* G, void* Y,
                       int B, int S, int Skv, int Hq, int Hkv, float scale_log2, hipStream_t st) {
  const int nq = ceil_div(S, 64);
  const int64_t blocks = (int64_t)nq * Hq * B;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, MODE>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const float*)Q, (const float*)K, (const float*)V, G, (float*)Y, B, S, Skv,
                     Hq, Hkv, nq, scale_log2);
}

template <int D>
static void dispatch_mode(int mode, bool bf16_inputs, const void* Q, const void* K, const void* V,
                          const float* G, void* Y, int B, int S, int Skv, int Hq, int Hkv,
                          float scale_log2, hipStream_t st) {
  if (bf16_inputs) {
    if (mode == kGateElem) launch_bf16<D, kGateElem>(Q, K, V, G, Y, B, S, Hq, Hkv, scale_log2, st);
    else if (mode == kGateHead) launch_bf16<D, kGateHead>(Q, K, V, G, Y, B, S, Hq, Hkv, scale_log2, st);
    else launch_bf16<D, kGateNone>(Q, K, V, G, Y, B, S, Hq, Hkv, scale_log2, st);
  } else {
    if (mode == kGateElem) launch_f32<D, kGateElem>(Q, K, V, G, Y, B, S, Skv, Hq, Hkv, scale_log2, st);
    else if (mode == kGateHead) launch_f32<D, kGateHead>(Q, K, V, G, Y, B, S, Skv, Hq, Hkv, scale_log2, st);
    else launch_f32<D, kGateNone>(Q, K, V, G, Y, B, S, Skv, Hq, Hkv, scale_log2, st);
  }
}

// bf16 inputs require Skv == S (prefill); float32 inputs allow Skv >= S.
hipError_t launch_attn_fwd(const void* Q, const void* K, const void* V, const float* G, void* Y,
                           int B, int S, int Skv, int Hq, int Hkv, int D, int mode,
                           bool bf16_inputs, hipStream_t stream) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  if (D == 128)
    dispatch_mode<128>(mode, bf16_inputs, Q, K, V, G, Y, B, S, Skv, Hq, Hkv, scale_log2, stream);
  else
    dispatch_mode<64>(mode, bf16_inputs, Q, K, V, G, Y, B, S, Skv, Hq, Hkv, scale_log2, stream);
  return hipGetLastError();
}

}  // namespace gsa
