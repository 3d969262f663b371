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
//   softmax    in the log2 domain: m = max(m_old, max(s)·(log2 e/√D)),
//              p = exp2(s·(log2 e/√D) − m) as one fused multiply-add and one
//              exp2 per score; l accumulates the bf16-rounded p, the same
//              weights the PV product applies (so a lone visible key, whose p
//              rounds to 1, yields exactly its value row); O is rescaled by
//              exp2(m_old − m).
//   Oᵀ += Vᵀ·Pᵀ on MFMA (A = Vᵀ rows from LDS, B = P rounded to bf16, taken
//              straight from the Sᵀ accumulators).  The k order of this product
//              follows the accumulator layout; the Vᵀ tile is stored with keys
//              permuted inside each 16-key block (offset bits 2 and 3 swapped)
//              so each lane's 8 keys are one 16-byte LDS read.
// Epilogue: O/l, times the float32 gate, one round-to-nearest-even to bf16.
#include <type_traits>

#include "common.h"

namespace gsa {

constexpr float kLn2 = 0.69314718055994531f;

namespace fwd {
constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile
}  // namespace fwd

enum : int { kGateNone = 0, kGateElem = 1, kGateHead = 2, kGateVariant = 3, kValueGateElem = 4, kValueGateHead = 5 };

// G2 value gating ("GatedAttention [2025]" §1.2.2, position G2): modes
// kValueGateElem / kValueGateHead take Gate as σ(X·W_v) per key/value head and
// dim ([B·S, Hkv·D]) or per key/value head ([B·S, Hkv]) and attend over
// V' = V ⊙ g, each product rounded once to bf16.  The gate tile of each key
// tile rides with the V tile's direct loads into LDS, and V' is formed in LDS
// as soon as the V tile lands, before any PV product reads it; there is no
// output gate.

// Epilogue of the design-space variants (MODE == kGateVariant only): the gate
// layout (0 none, 1 elementwise column h·D + d, 2 headwise column h, 3 shared
// column d for every head), additive instead of multiplicative combination,
// and a per-head RMSNorm (unit weight, ε = 1e-6) of the SDPA output first.
// The gate values G arrive already activated (gsa_gate_logits' activation).
struct FwdEpi {
  int layout, add, rms;
};
constexpr float kRmsEps = 1e-6f;

// the gate value of (row tok, head, dim d) for a variant layout
__device__ __forceinline__ float variant_gate(const float* __restrict__ Gate, const FwdEpi& ep, int64_t tok,
                                              int Hq, int D, int head, int d) {
  if (ep.layout == kGateElem) return Gate[(tok * Hq + head) * D + d];
  if (ep.layout == kGateHead) return Gate[tok * Hq + head];
  return Gate[tok * D + d];
}
__device__ __forceinline__ float variant_combine(float y, float g, const FwdEpi& ep) {
  return ep.add ? y + g : y * g;
}

#ifndef GSA_FWD_QB
#define GSA_FWD_QB 1
#endif


// HG > 1 (GQA): the 4 waves take HG query heads of one key/value group, 4/HG
// row blocks each, so one staged K/V tile serves HG heads (HG times fewer K/V
// loads per matrix op, and every wave's rows end at the workgroup's diagonal).
template <int D, int MODE, int QB, int HG = 1>
__global__ __launch_bounds__(256, QB == 1 ? 2 : 1)
void attn_fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                          const bf16* __restrict__ V, const float* __restrict__ Gate,
                          bf16* __restrict__ Y, float* __restrict__ Lse, int B, int S, int Hq,
                          int Hkv, int n_qtiles, float scale_log2, FwdEpi ep) {
  using namespace fwd;
  static_assert(HG == 1 || (QB == 1 && 4 % HG == 0), "head groups of 2 or 4 with 32-row waves");
  constexpr int BMQ = BM * QB / HG;   // query rows per workgroup (QB blocks of 32 per wave)
  constexpr int CH = D / 8;       // 16-byte chunks per K/V row
  constexpr int KSL = CH + 1;     // K row stride in 16-B slots (one pad slot: 4-bank rotation per row)
  constexpr int VSL = CH;         // V rows are unpadded, chunk-swizzled
  constexpr int VSW = CH / 4 - 1; // V swizzle: chunk ^= 4 * (row & VSW)
  // one LDS object per stage: the compiler's alias information then knows a
  // direct load into one stage cannot touch the other, and does not make reads
  // of the current stage wait for loads still filling the next one
  __shared__ __align__(16) bf16 Ks0[BN * KSL * 8];
  __shared__ __align__(16) bf16 Ks1[BN * KSL * 8];
  __shared__ __align__(16) bf16 Vs0[BN * VSL * 8];
  __shared__ __align__(16) bf16 Vs1[BN * VSL * 8];
  // G2 gate tile of the V tile in flight (single-buffered: each one is used up
  // by the pass over its V tile, behind a barrier, before the next is loaded):
  // [BN keys][D] float32 elementwise, BN floats headwise (one 4-byte direct
  // load per lane: 64 slots)
  constexpr bool kG2 = MODE == kValueGateElem || MODE == kValueGateHead;
  constexpr int GFL = MODE == kValueGateElem ? BN * D : MODE == kValueGateHead ? 64 : 4;
  __shared__ __align__(16) float Gst[GFL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
  const int l32 = lane & 31, hl = lane >> 5;

  // Heaviest (last) query tiles first.  Workgroup ids are dealt round-robin
  // over the 8 XCDs; when the (batch, head group) pair count allows, XCD x =
  // id % 8 takes the x-th contiguous eighth of the pairs (pair = b*(Hq/HG) +
  // head group, so the query heads of one GQA group are adjacent), which keeps
  // a key/value head's tiles in one L2.
  const int bid = blockIdx.x;
  const int hb = Hq / HG * B;
  int qt, pair;
  if (hb % 8 == 0) {
    const int pc = hb / 8, j = bid / 8;
    qt = n_qtiles - 1 - j / pc;
    pair = (bid % 8) * pc + j % pc;
  } else {
    qt = n_qtiles - 1 - bid / hb;
    pair = bid % hb;
  }
  const int b = pair / (Hq / HG);
  const int head = (pair % (Hq / HG)) * HG + wave % HG;   // this wave's query head (wave-uniform)
  const int kvh = head / (Hq / Hkv);                       // the same for the HG heads of the group

  const int q0 = qt * BMQ;
  const int qw0 = q0 + (wave / HG) * 32 * QB;  // first query row of this wave
  int my_q[QB];                         // this lane's query row in each 32-row block
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) my_q[qb] = qw0 + 32 * qb + l32;

  const int64_t q_row = (int64_t)Hq * D;
  const int64_t kv_row = (int64_t)Hkv * D;
  const bf16* Qb = Q + (int64_t)b * S * q_row + (int64_t)head * D;
  const bf16* Kb = K + (int64_t)b * S * kv_row + (int64_t)kvh * D;
  const bf16* Vb = V + (int64_t)b * S * kv_row + (int64_t)kvh * D;

  // Q fragments: B operand of Sᵀ = K·Qᵀ, lane holds Q[my_q][16*kk + 8*hl .. +7];
  // rows past the end read zeros (buffer range check) and are never stored
  bf16x8 qf[QB][D / 16];
  {
    const auto qr = make_rsrc(Qb, (uint32_t)(((int64_t)S * q_row - (int64_t)head * D) * 2));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const uint32_t qo = (uint32_t)(((int64_t)my_q[qb] * q_row + 8 * hl) * 2);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        qf[qb][kk] = __builtin_bit_cast(bf16x8, buffer_load16(qr, qo + 32 * kk, 0));
    }
  }

  f32x16 o[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][dt][r] = 0.f;
  // m_run is the reference max of the exp2-domain scores: it only moves when a
  // row's max grows by more than kRescale (then O and l are rescaled), so p may
  // reach 2^kRescale.  O/l does not depend on the reference (exact in real
  // arithmetic); a row's first tile always sets it.
  constexpr float kRescale = 8.0f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  const int kv_end = min(S, q0 + BMQ);
  const int n_kv = ceil_div(kv_end, BN);

  // ---- global -> LDS: 16-byte direct loads (buffer_load ... lds); lane l of a
  // wave instruction lands in slot (instruction base + l).  Keys >= S read as
  // zeros (range check; the whole offset is in the VGPR) and are masked later.
  const uint32_t kv_bytes = (uint32_t)(((int64_t)S * kv_row - (int64_t)kvh * D) * 2);
  const auto krs = make_rsrc(Kb, kv_bytes);
  const auto vrs = make_rsrc(Vb, kv_bytes);
  const uint32_t row_b = (uint32_t)(kv_row * 2);
  // K slot s = row*KSL + chunk (chunk CH is padding: loads from past the end -> 0)
  uint32_t k_off[(KSL + 3) / 4];
#pragma unroll
  for (int j = 0; j < (KSL + 3) / 4; ++j) {
    const int sl = (wave + 4 * j) * 64 + lane;
    const int row = sl / KSL, ch = sl % KSL;
    k_off[j] = ch < CH ? (uint32_t)row * row_b + ch * 16 : 0xfffffff0u;
  }
  // V slot s = row*VSL + phys; phys = chunk ^ 4*(row & VSW)
  uint32_t v_off[VSL / 4];
#pragma unroll
  for (int j = 0; j < VSL / 4; ++j) {
    const int sl = (wave + 4 * j) * 64 + lane;
    const int row = sl / VSL, phys = sl % VSL;
    v_off[j] = (uint32_t)row * row_b + (uint32_t)((phys ^ (4 * (row & VSW))) * 16);
  }
  // a tile that is not needed gets a base past the range check: its loads
  // write zeros to LDS and never touch memory (offsets stay below 2^32:
  // base 2^31 plus at most BN rows of at most 2^20 bytes)
  constexpr uint32_t kNoTile = 0x80000000u;
  auto dma_k = [&](int k0, bool need, bf16* kdst) {
    const uint32_t base = need ? (uint32_t)k0 * row_b : kNoTile;
#pragma unroll
    for (int j = 0; j < (KSL + 3) / 4; ++j) {
      const int ins = wave + 4 * j;
      if (ins < KSL) {
        const uint32_t off = k_off[j] == 0xfffffff0u ? 0xfffffff0u : k_off[j] + base;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (GSA_LDS void*)&kdst[ins * 64 * 8], 16, (int)off, 0, 0, 0);
      }
    }
  };
  auto dma_v = [&](int k0, bool need, bf16* vdst) {
    const uint32_t base = need ? (uint32_t)k0 * row_b : kNoTile;
#pragma unroll
    for (int j = 0; j < VSL / 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (GSA_LDS void*)&vdst[(wave + 4 * j) * 64 * 8], 16,
                                               (int)(v_off[j] + base), 0, 0, 0);
  };

  // G2 gate tiles: rows of key tokens k0 .. k0+63 of key/value head kvh; keys
  // >= S read zeros (range check on the batch's gate rows)
  const float* const Gv = kG2 ? Gate + ((int64_t)b * S * Hkv + kvh) * (MODE == kValueGateElem ? D : 1) : nullptr;
  const uint32_t g_row_b = (uint32_t)(Hkv * (MODE == kValueGateElem ? D : 1) * 4);
  const auto grs = make_rsrc(Gv, kG2 ? (uint32_t)((int64_t)S * g_row_b - (int64_t)kvh * (MODE == kValueGateElem ? D : 1) * 4) : 0u);
  constexpr int GSL = BN * D / 4;                 // 16-B slots of an elementwise gate tile
  constexpr int GIW = GSL / 64 / 4;               // its direct loads per wave
  uint32_t g_off[MODE == kValueGateElem ? GIW : 1];
  if constexpr (MODE == kValueGateElem) {
#pragma unroll
    for (int j = 0; j < GIW; ++j) {
      const int sl = (wave + 4 * j) * 64 + lane;
      g_off[j] = (uint32_t)(sl / (D / 4)) * g_row_b + (uint32_t)(sl % (D / 4)) * 16;
    }
  } else {
    g_off[0] = (uint32_t)lane * g_row_b;          // headwise: lane l = key l of the tile
  }
  auto dma_g = [&](int k0, bool need) {
    if constexpr (kG2) {
      const uint32_t base = need ? (uint32_t)k0 * g_row_b : kNoTile;
      if constexpr (MODE == kValueGateElem) {
#pragma unroll
        for (int j = 0; j < GIW; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(grs, (GSA_LDS void*)&Gst[(wave + 4 * j) * 64 * 4], 16,
                                                   (int)(g_off[j] + base), 0, 0, 0);
      } else {
        if (wave == 0)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(grs, (GSA_LDS void*)&Gst[0], 4, (int)(g_off[0] + base), 0, 0, 0);
      }
    }
  };
  // V' = V ⊙ g in place, one RNE rounding per product: thread t takes V slots
  // t, t + 256, ... (16 bytes: 8 dims of one key; slot phys of row r holds
  // chunk phys ^ 4·(r & VSW))
  auto gate_v = [&](bf16* vbuf) {
    if constexpr (kG2) {
#pragma unroll
      for (int i = 0; i < BN * VSL / 256; ++i) {
        const int sl = tid + 256 * i;
        const int row = sl / VSL, c = (sl % VSL) ^ (4 * (row & VSW));
        u32x4 v = *(u32x4*)&vbuf[sl * 8];
        float g[8];
        if constexpr (MODE == kValueGateElem) {
          const f32x4 g0 = *(const f32x4*)&Gst[row * D + c * 8];
          const f32x4 g1 = *(const f32x4*)&Gst[row * D + c * 8 + 4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            g[e] = g0[e];
            g[4 + e] = g1[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) g[e] = Gst[row];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) v[w] = pack_bf16x2(bf16_lo(v[w]) * g[2 * w], bf16_hi(v[w]) * g[2 * w + 1]);
        *(u32x4*)&vbuf[sl * 8] = v;
      }
    }
  };

  // ---- LDS -> MFMA operands
  // K (A operand of Sᵀ): lane reads row sub*32 + l32, chunk 2*kk + hl (one 16-B read)
  const int ks_lane = (l32 * KSL + hl) * 8;
  // Vᵀ (A operand of Oᵀ += Vᵀ·Pᵀ) via transposed 8-byte reads.  In a 16-lane group
  // g = lane/16, lane i names row 4*(g/2) + i/4 (+ 8*a + 16*t + 32*sub) and dims
  // dt*32 + 16*(g%2) + 4*(i%4) .. +3; the read hands lane i the four rows' values
  // at dim dt*32 + 16*(g%2) + i, i.e. MFMA row l32, k slots 4a..4a+3 = keys
  // 16t + 8a + 4*hl + 0..3 of the subtile, matching the P layout.
  const int vg = lane >> 4, vi = lane & 15;
  const int v_r = 4 * (vg >> 1) + (vi >> 2);           // row within a 16-key block (and r & 3 == vi >> 2)
  const int v_dc = 16 * (vg & 1) + 4 * (vi & 3);       // dim offset within a 32-dim block
  uint32_t vt_base[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int chunk = dt * 4 + (v_dc >> 3);
    const int phys = chunk ^ (4 * (v_r & VSW));
    vt_base[dt] = (uint32_t)(v_r * VSL * 16 + phys * 16 + (v_dc & 7) * 2);
  }

  // Sᵀ tile (64 keys x this wave's 32·QB rows) from the K tile at ksrc; each K
  // fragment serves the QB row blocks; the 2·QB accumulators are independent
  // chains, interleaved
  auto mma_s = [&](const bf16* ksrc, f32x16 (&s)[2][QB]) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sub][qb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const bf16x8 a = *(const bf16x8*)(ksrc + ks_lane + (sub * 32 * KSL + 2 * kk) * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[sub][qb] = mfma32x32x16(a, qf[qb][kk], s[sub][qb]);
      }
  };
  // Online softmax of one Sᵀ tile in two halves (the reference test between
  // them is the only branch of the loop body): row max in-lane, then across the
  // two wave halves, and the reference update; then p = exp2(s·c − m), P
  // packed to bf16 and the row sum folded into l.
  float alpha[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) alpha[qb] = 1.f;
  const bf16x2 kOnes2 = {(bf16)1.0f, (bf16)1.0f};
  // causal / length mask of one Sᵀ tile: key offset within the tile of
  // element (sub, r) is sub*32 + 8*(r/4) + 4*hl + r%4
  auto apply_mask = [&](f32x16 (&s)[2][QB], int k0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int lim = min(my_q[qb], S - 1) - k0 - 4 * hl;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = sub * 32 + 8 * (r >> 2) + (r & 3);
          s[sub][qb][r] = off <= lim ? s[sub][qb][r] : -INFINITY;
        }
    }
  };
  // first half: row max, reference update; returns whether any lane moved
  // its reference (O must then be scaled by alpha)
  auto softmax_max = [&](f32x16 (&s)[2][QB]) -> bool {
    bool moved = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // row max of the raw scores (scaling by a positive constant and rounding
      // are monotonic, so max(s)·c rounds to the max of the rounded s·c)
      float mx = s[0][qb][0];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][qb][r]);
      {
        // max with the other wave half (same query row, the other 32 keys)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
      }
      // move the reference only when the max grew by more than kRescale
      // (always on a row's first tile, where m_run = -inf)
      const float mx_t = mx * scale_log2;
      const bool move = mx_t > m_run[qb] + kRescale;
      const float m_new = move ? mx_t : m_run[qb];
      alpha[qb] = fast_exp2(m_run[qb] - m_new);   // 1 when not moving, 0 on the first tile
      m_run[qb] = m_new;
      moved = moved || move;
    }
    return __any(moved);
  };
  // second half, one 16-key quarter (sub, t) of the tile at a time: p =
  // exp2(s·c − m), P packed to bf16 and summed into ps (l is updated once the
  // four quarters are done), then that quarter's PV product, Oᵀ += Vᵀ·Pᵀ from
  // the V tile at vsrc (the D/32 output blocks are independent accumulation
  // chains).  A quarter's matrix ops depend only on its own probabilities, so
  // the next quarter's exp work can run in their shadow; O still accumulates
  // keys in increasing order.
  auto exp_q = [&](f32x16 (&s)[2][QB], bf16x8 (&pb)[QB][2][2], float (&ps)[QB][2], int sub, int t) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float neg_m = -m_run[qb];
#pragma unroll
      for (int e = 0; e < 8; ++e) s[sub][qb][8 * t + e] = fast_exp2(fmaf(s[sub][qb][8 * t + e], scale_log2, neg_m));
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[qb][sub][t][e] = (bf16)s[sub][qb][8 * t + e];
      // l sums the bf16-rounded p, the very weights the PV product applies
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const bf16x2 pair = {pb[qb][sub][t][2 * w], pb[qb][sub][t][2 * w + 1]};
        ps[qb][w & 1] = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, ps[qb][w & 1], false);
      }
    }
  };
  auto pv_q = [&](const bf16* vsrc, const bf16x8 (&pb)[QB][2][2], int sub, int t) {
    // an LDS pointer derived from the stage array (not from an integer), so
    // the compiler keeps the provenance it needs for its alias information
    GSA_LDS char* const vs = (GSA_LDS char*)(GSA_LDS void*)vsrc;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      GSA_LDS char* const a0 = vs + vt_base[dt] + (sub * 32 + 16 * t) * VSL * 16;
      const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS i16x4*)a0);
      const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS i16x4*)(a0 + 8 * VSL * 16));
      bf16x8 a;
      a.lo = __builtin_bit_cast(bf16x4, lo);
      a.hi = __builtin_bit_cast(bf16x4, hi);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[qb][dt] = mfma32x32x16(a, pb[qb][sub][t], o[qb][dt]);
    }
  };
  auto rescale_o = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][dt][r] *= alpha[qb];
  };
  auto wait_dma_and_sync = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // Pipeline: K runs one tile ahead of V.  At the top of iteration t, K buffer
  // (t+1)&1 holds K(t+1), V buffer t&1 holds V(t) and `cur` holds Sᵀ(t).  The
  // direct loads of K(t+2) and V(t+1) go to K buffer t&1 and V buffer (t+1)&1,
  // both last read in iteration t-1, and are waited for before the barrier.
  // The body is one basic block apart from the mask (diagonal tiles only, at
  // the top) and the rare rescale, so the compiler interleaves the Sᵀ(t+1)
  // matrix ops with the VALU work of softmax(t).  The last tile has a step of
  // its own (last_step), so the loop body never computes an Sᵀ it discards.
  //
  // softmax(t) and PV(t) of the last tile, which has no next tile: no loads
  // and no Sᵀ(t+1).  A wave whose rows all come before the tile's first key
  // (one head per workgroup: the first waves' last tile) skips it: every score
  // would be masked, so its p are 0 and O, l and the reference stay as they are.
  auto last_step = [&](auto parity, int it, f32x16 (&cur)[2][QB]) {
    constexpr int P = decltype(parity)::value;
    bf16* const v_cur = P ? Vs1 : Vs0;   // V(t)
    const int k0 = it * BN;
    if (k0 <= qw0 + 32 * QB - 1) {
      if ((k0 + BN - 1 > qw0) || (k0 + BN > S)) apply_mask(cur, k0);
      const bool move = softmax_max(cur);
      if (move) rescale_o();
      bf16x8 pb[QB][2][2];
      float ps[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) ps[qb][0] = ps[qb][1] = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          exp_q(cur, pb, ps, sub, t);
          pv_q(v_cur, pb, sub, t);
        }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l_run[qb] = l_run[qb] * alpha[qb] + (ps[qb][0] + ps[qb][1]);
    }
    __syncthreads();   // every wave is past its last LDS read: the epilogue reuses the stage arrays
  };
  // iteration `it` (not the last) with compile-time buffer parity P = it & 1
  auto step = [&](auto parity, int it, f32x16 (&cur)[2][QB], f32x16 (&nxt)[2][QB]) {
    constexpr int P = decltype(parity)::value;
    bf16* const k_cur = P ? Ks1 : Ks0;   // held K(t), consumed in iteration t-1: refill with K(t+2)
    bf16* const k_nxt = P ? Ks0 : Ks1;   // K(t+1)
    bf16* const v_cur = P ? Vs1 : Vs0;   // V(t)
    bf16* const v_nxt = P ? Vs0 : Vs1;   // refill with V(t+1)
    const int k0 = it * BN;
    if ((k0 + BN - 1 > qw0) || (k0 + BN > S)) apply_mask(cur, k0);
    dma_k(k0 + 2 * BN, it + 2 < n_kv, k_cur);
    dma_v(k0 + BN, it + 1 < n_kv, v_nxt);
    dma_g(k0 + BN, it + 1 < n_kv);
    mma_s(k_nxt, nxt);
    const bool move = softmax_max(cur);
    // the Sᵀ(t+1) block: LDS latency is several matrix ops long, so keep 8 K
    // fragment reads in flight ahead of the matrix ops and fill their shadow
    // with the row-max VALU work of softmax(t)
    {
      constexpr int NRD = 2 * D / 16;   // K fragment reads, each feeding QB matrix ops
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < NRD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
        if (i + 8 < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2 * QB, 0);
      }
    }
    if (move) rescale_o();
    bf16x8 pb[QB][2][2];
    float ps[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ps[qb][0] = ps[qb][1] = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        exp_q(cur, pb, ps, sub, t);
        pv_q(v_cur, pb, sub, t);
      }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] = l_run[qb] * alpha[qb] + (ps[qb][0] + ps[qb][1]);
    wait_dma_and_sync();
    if constexpr (kG2) {   // V(t+1) and its gate have landed: form V' before iteration t+1 reads it
      gate_v(v_nxt);
      __syncthreads();
    }
  };

  f32x16 sA[2][QB], sB[2][QB];
  dma_k(0, true, Ks0);
  dma_v(0, true, Vs0);
  dma_g(0, true);
  dma_k(BN, n_kv > 1, Ks1);
  // Sᵀ(0) needs only Q and K(0): wait until at most this wave's later loads
  // (V(0), its gate tile, K(1)) are outstanding, then for every wave's K(0),
  // so the first score tile overlaps the rest of the prologue's loads
  {
    constexpr int kAfterK0 = VSL / 4 + (MODE == kValueGateElem ? GIW : 0) + (KSL + 3) / 4 - 1;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAfterK0) : "memory");
    __builtin_amdgcn_s_barrier();
  }
  mma_s(Ks0, sA);
  wait_dma_and_sync();   // V(0), its gate and K(1); K buffer 0 is refilled in the first iteration
  if constexpr (kG2) {
    gate_v(Vs0);
    __syncthreads();     // V' of tile 0 before the first PV product
  }
  // every tile but the last, then the last (its Sᵀ is in sA when its index is even)
  const int n_main = n_kv - 1;
  for (int it = 0; it < n_main; it += 2) {
    step(std::integral_constant<int, 0>{}, it, sA, sB);
    if (it + 1 < n_main) step(std::integral_constant<int, 1>{}, it + 1, sB, sA);
  }
  if (n_main & 1) last_step(std::integral_constant<int, 1>{}, n_main, sB);
  else last_step(std::integral_constant<int, 0>{}, n_main, sA);

  if constexpr (QB == 1) {
    // Epilogue through LDS.  In the accumulator layout a lane holds one row and
    // 16-byte pieces of it 32 bytes apart, so a store (or gate load) there
    // touches 32 rows at once; staged through LDS, each instruction covers
    // whole rows instead (two at D = 128, four at D = 64), with 4-8x fewer
    // cache lines per instruction.  The loop's last barrier came after every
    // wave's last LDS read and direct load, so the stage arrays are free: wave
    // w stages its 32 rows of float32 in the w-th of them (32·D·4 bytes, the
    // size of a V stage), chunk c of row r in slot c ^ (r & 15), so that both
    // the accumulator-layout writes (16 rows per 16 lanes) and the row reads
    // (16 chunks of one row per 16 lanes) fall on distinct banks.  The value
    // stored is still round((o · (1/l)) · g), as in the register epilogue (for
    // the design-space variants round(combine(o · (1/l) · rn, g))).
    const float l_tot = l_run[0] + __shfl_xor(l_run[0], 32);  // the two halves summed different keys
    const bool row_ok = my_q[0] < S;
    if (Lse != nullptr && hl == 0 && row_ok)
      Lse[((int64_t)b * Hq + head) * S + my_q[0]] = (m_run[0] + log2f(l_tot)) * kLn2;
    const float inv = 1.0f / l_tot;
    float rn = 1.0f;   // the variants' RMSNorm factor of the row
    if constexpr (MODE == kGateVariant) {
      if (ep.rms) {
        // the row's D values sit in this lane (half) and in lane ^ 32 (other half)
        float ss = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float y = o[0][dt][r] * inv;
            ss = fmaf(y, y, ss);
          }
        ss += __shfl_xor(ss, 32);
        rn = 1.0f / sqrtf(ss / (float)D + kRmsEps);
      }
    }
    constexpr int LPR = D / 4;       // lanes per row in the row pattern (16 bytes each)
    constexpr int RPI = 64 / LPR;    // rows per instruction
    constexpr int NI = 32 / RPI;     // instructions for the wave's 32 rows
    const int sr = lane / LPR, sc = lane % LPR;
    // elementwise gate: the coalesced row loads go first, before any store
    // (the memory counter the waits use also counts stores); rows past the end
    // read the last row instead and are not stored
    f32x4 gv[NI];
    if constexpr (MODE == kGateElem) {
      const float* const grow = Gate + (int64_t)head * D + 4 * sc;
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int q = min(qw0 + RPI * n + sr, S - 1);
        gv[n] = *(const f32x4*)(grow + ((int64_t)b * S + q) * q_row);
      }
#pragma unroll
      for (int n = 0; n < NI; ++n) asm volatile("" : "+v"(gv[n]));
    }
    if constexpr (MODE == kGateVariant) {
      if (ep.layout != kGateNone) {
#pragma unroll
        for (int n = 0; n < NI; ++n) {
          const int64_t tok = (int64_t)b * S + min(qw0 + RPI * n + sr, S - 1);
          if (ep.layout == kGateHead) {
            const float g = Gate[tok * Hq + head];
            gv[n] = f32x4{g, g, g, g};
          } else {
            gv[n] = *(const f32x4*)(Gate + (ep.layout == kGateElem ? (tok * Hq + head) * D : tok * D) + 4 * sc);
          }
        }
#pragma unroll
        for (int n = 0; n < NI; ++n) asm volatile("" : "+v"(gv[n]));
      }
    }
    float gh = 1.0f;
    if constexpr (MODE == kGateHead) gh = Gate[((int64_t)b * S + min(my_q[0], S - 1)) * Hq + head];
    GSA_LDS char* const stg = wave == 0   ? (GSA_LDS char*)(GSA_LDS void*)Ks0
                              : wave == 1 ? (GSA_LDS char*)(GSA_LDS void*)Ks1
                              : wave == 2 ? (GSA_LDS char*)(GSA_LDS void*)Vs0
                                          : (GSA_LDS char*)(GSA_LDS void*)Vs1;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 8 * dt + 2 * i + hl;   // 16-byte chunk of dims dt*32 + 8i + 4hl .. +3
        f32x4 t;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (MODE == kGateVariant) t[j] = o[0][dt][4 * i + j] * inv * rn;
          else t[j] = o[0][dt][4 * i + j] * inv;
          if constexpr (MODE == kGateHead) t[j] *= gh;
        }
        *(GSA_LDS f32x4*)(stg + l32 * (4 * D) + ((c ^ (l32 & 15)) * 16)) = t;
      }
    // the rows are read back by other lanes of this wave: its LDS writes must
    // have completed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int r = RPI * n + sr;
      f32x4 t = *(GSA_LDS const f32x4*)(stg + r * (4 * D) + ((sc ^ (r & 15)) * 16));
      if constexpr (MODE == kGateElem) {
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] *= gv[n][j];
      }
      if constexpr (MODE == kGateVariant) {
        if (ep.layout != kGateNone) {
#pragma unroll
          for (int j = 0; j < 4; ++j) t[j] = variant_combine(t[j], gv[n][j], ep);
        }
      }
      if (qw0 + r < S)
        *(u32x2*)(Y + ((int64_t)b * S + qw0 + r) * q_row + (int64_t)head * D + 4 * sc) =
            u32x2{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
    }
    return;
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // every lane takes part in the exchange; rows past the end store nothing
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);  // the two halves summed different keys
    if (my_q[qb] >= S) continue;
    // log-sum-exp of the row's scaled scores (natural log): m and l are in the
    // base-2 domain of s·log2(e), so ln Σ e^s = (m + log2 l)·ln 2
    if (Lse != nullptr && hl == 0)
      Lse[((int64_t)b * Hq + head) * S + my_q[qb]] = (m_run[qb] + log2f(l_tot)) * kLn2;
    const float inv = 1.0f / l_tot;
    const int64_t tok = (int64_t)b * S + my_q[qb];
    bf16* yrow = Y + tok * q_row + (int64_t)head * D;
    if constexpr (MODE == kGateVariant) {
      // the row's D values sit in this lane (half) and in lane ^ 32 (other half)
      float rn = 1.0f;
      if (ep.rms) {
        float ss = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float y = o[qb][dt][r] * inv;
            ss = fmaf(y, y, ss);
          }
        ss += __shfl_xor(ss, 32);   // lane ^ 32 holds the same row (same my_q: both take this path)
        rn = 1.0f / sqrtf(ss / (float)D + kRmsEps);
      }
      // the row's gate values, all loaded before the first store of Y (see below)
      f32x4 gv[D / 32][4];
      if (ep.layout != kGateNone) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d0 = dt * 32 + 8 * i + 4 * hl;
            if (ep.layout == kGateHead) {
              const float g = Gate[tok * Hq + head];
              gv[dt][i] = f32x4{g, g, g, g};
            } else {
              gv[dt][i] = *(const f32x4*)(Gate + (ep.layout == kGateElem ? (tok * Hq + head) * D : tok * D) + d0);
            }
          }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(gv[dt][i]));
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = dt * 32 + 8 * i + 4 * hl;
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            y[j] = o[qb][dt][4 * i + j] * inv * rn;
            if (ep.layout != kGateNone) y[j] = variant_combine(y[j], gv[dt][i][j], ep);
          }
          *(u32x2*)(yrow + d0) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
      continue;
    }
    float gh = 1.0f;
    if constexpr (MODE == kGateHead) gh = Gate[tok * Hq + head];
    // elementwise gate: all of the row's gate loads are issued before the first
    // store of Y.  The memory counter the waits use also counts stores, so a
    // gate load issued after a store would wait for that store to complete.
    f32x4 gv[D / 32][4];
    if constexpr (MODE == kGateElem) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          gv[dt][i] = *(const f32x4*)(Gate + tok * q_row + (int64_t)head * D + dt * 32 + 8 * i + 4 * hl);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(gv[dt][i]));
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = dt * 32 + 8 * i + 4 * hl;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = o[qb][dt][4 * i + j] * inv;
        if constexpr (MODE == kGateElem) {
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] *= gv[dt][i][j];
        } else if constexpr (MODE == kGateHead) {
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] *= gh;
        }
        *(u32x2*)(yrow + d0) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      }
  }
}

// float32 kernel, also used for decode in float32: S query rows aligned to the
// END of Skv keys (query i sits at position i + Skv - S).  64 query rows per
// workgroup, 4 lanes per row splitting the head dimension, 32-key tiles in LDS.
template <int D, int MODE>
__global__ __launch_bounds__(256)
void attn_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                         const float* __restrict__ V, const float* __restrict__ Gate,
                         float* __restrict__ Y, float* __restrict__ Lse, int B, int S, int Skv,
                         int Hq, int Hkv, int n_qtiles, float scale_log2, FwdEpi ep) {
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
      float v = ok ? Vb[(int64_t)(k0 + j) * kv_row + d] : 0.f;
      if constexpr (MODE == kValueGateElem)   // G2: V' = V ⊙ g, one float32 product
        v *= ok ? Gate[((int64_t)b * Skv + k0 + j) * kv_row + (int64_t)kvh * D + d] : 0.f;
      if constexpr (MODE == kValueGateHead) v *= ok ? Gate[((int64_t)b * Skv + k0 + j) * Hkv + kvh] : 0.f;
      Vs[j * LDF + d] = v;
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
  // (a row's 4 lanes are adjacent and share q: they leave together)
  if (q >= S) return;
  const float inv = 1.0f / l_run;
  if (Lse != nullptr && part == 0)
    Lse[((int64_t)b * Hq + head) * S + q] = (m_run + log2f(l_run)) * kLn2;
  const int64_t tok = (int64_t)b * S + q;
  if constexpr (MODE == kGateVariant) {
    float rn = 1.0f;
    if (ep.rms) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) ss = fmaf(acc[e] * inv, acc[e] * inv, ss);
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      rn = 1.0f / sqrtf(ss / (float)D + kRmsEps);
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const int d = part * DPL + e;
      float y = acc[e] * inv * rn;
      if (ep.layout != kGateNone) y = variant_combine(y, variant_gate(Gate, ep, tok, Hq, D, head, d), ep);
      Y[tok * q_row + (int64_t)head * D + d] = y;
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const int d = part * DPL + e;
    float y = acc[e] * inv;
    if constexpr (MODE == kGateElem) y *= Gate[tok * q_row + (int64_t)head * D + d];
    if constexpr (MODE == kGateHead) y *= Gate[tok * Hq + head];
    Y[tok * q_row + (int64_t)head * D + d] = y;
  }
}

template <int D, int MODE, int QB, int HG>
static void launch_bf16_hg(const void* Q, const void* K, const void* V, const float* G, void* Y,
                           float* Lse, int B, int S, int Hq, int Hkv, float scale_log2, hipStream_t st,
                           FwdEpi ep) {
  const int nq = ceil_div(S, fwd::BM * QB / HG);
  const int64_t blocks = (int64_t)nq * (Hq / HG) * B;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, MODE, QB, HG>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const bf16*)Q, (const bf16*)K, (const bf16*)V, G, (bf16*)Y, Lse, B, S, Hq,
                     Hkv, nq, scale_log2, ep);
}

// GQA groups of 4 or more query heads share each staged K/V tile among 4 heads
// of a workgroup (groups of 2: among 2)
#ifndef GSA_FWD_HG
#define GSA_FWD_HG 4
#endif
template <int D, int MODE, int QB = GSA_FWD_QB>
static void launch_bf16(const void* Q, const void* K, const void* V, const float* G, void* Y,
                        float* Lse, int B, int S, int Hq, int Hkv, float scale_log2, hipStream_t st,
                        FwdEpi ep = FwdEpi{0, 0, 0}) {
  const int grp = Hq / Hkv;
  if (QB == 1 && GSA_FWD_HG >= 4 && grp % 4 == 0)
    launch_bf16_hg<D, MODE, QB, (QB == 1 && GSA_FWD_HG >= 4) ? 4 : 1>(Q, K, V, G, Y, Lse, B, S, Hq, Hkv,
                                                                        scale_log2, st, ep);
  else if (QB == 1 && GSA_FWD_HG >= 2 && grp % 2 == 0)
    launch_bf16_hg<D, MODE, QB, (QB == 1 && GSA_FWD_HG >= 2) ? 2 : 1>(Q, K, V, G, Y, Lse, B, S, Hq, Hkv,
                                                                        scale_log2, st, ep);
  else
    launch_bf16_hg<D, MODE, QB, 1>(Q, K, V, G, Y, Lse, B, S, Hq, Hkv, scale_log2, st, ep);
}

template <int D, int MODE>
static void launch_f32(const void* Q, const void* K, const void* V, const float* G, void* Y,
                       float* Lse, int B, int S, int Skv, int Hq, int Hkv, float scale_log2,
                       hipStream_t st, FwdEpi ep = FwdEpi{0, 0, 0}) {
  const int nq = ceil_div(S, 64);
  const int64_t blocks = (int64_t)nq * Hq * B;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, MODE>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const float*)Q, (const float*)K, (const float*)V, G, (float*)Y, Lse, B, S,
                     Skv, Hq, Hkv, nq, scale_log2, ep);
}

template <int D>
static void dispatch_mode(int mode, bool bf16_inputs, const void* Q, const void* K, const void* V,
                          const float* G, void* Y, float* Lse, int B, int S, int Skv, int Hq,
                          int Hkv, float scale_log2, hipStream_t st) {
  if (bf16_inputs) {
    if (mode == kGateElem) launch_bf16<D, kGateElem>(Q, K, V, G, Y, Lse, B, S, Hq, Hkv, scale_log2, st);
    else if (mode == kGateHead) launch_bf16<D, kGateHead>(Q, K, V, G, Y, Lse, B, S, Hq, Hkv, scale_log2, st);
    else launch_bf16<D, kGateNone>(Q, K, V, G, Y, Lse, B, S, Hq, Hkv, scale_log2, st);
  } else {
    if (mode == kGateElem) launch_f32<D, kGateElem>(Q, K, V, G, Y, Lse, B, S, Skv, Hq, Hkv, scale_log2, st);
    else if (mode == kGateHead) launch_f32<D, kGateHead>(Q, K, V, G, Y, Lse, B, S, Skv, Hq, Hkv, scale_log2, st);
    else launch_f32<D, kGateNone>(Q, K, V, G, Y, Lse, B, S, Skv, Hq, Hkv, scale_log2, st);
  }
}

// bf16 inputs require Skv == S (prefill); float32 inputs allow Skv >= S.
hipError_t launch_attn_fwd(const void* Q, const void* K, const void* V, const float* G, void* Y,
                           float* Lse, int B, int S, int Skv, int Hq, int Hkv, int D, int mode,
                           bool bf16_inputs, hipStream_t stream) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  if (D == 128)
    dispatch_mode<128>(mode, bf16_inputs, Q, K, V, G, Y, Lse, B, S, Skv, Hq, Hkv, scale_log2, stream);
  else
    dispatch_mode<64>(mode, bf16_inputs, Q, K, V, G, Y, Lse, B, S, Skv, Hq, Hkv, scale_log2, stream);
  return hipGetLastError();
}

// G2 value gating (prefill): attention over V ⊙ g, g per key/value head and dim
// (elementwise) or per key/value head (headwise); no output gate.
hipError_t launch_attn_fwd_value_gated(const void* Q, const void* K, const void* V, const float* Gv, void* Y,
                                       float* Lse, int B, int S, int Hq, int Hkv, int D, bool headwise,
                                       bool bf16_inputs, hipStream_t stream) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  if (bf16_inputs) {
    if (D == 128) {
      if (headwise) launch_bf16<128, kValueGateHead>(Q, K, V, Gv, Y, Lse, B, S, Hq, Hkv, scale_log2, stream);
      else launch_bf16<128, kValueGateElem>(Q, K, V, Gv, Y, Lse, B, S, Hq, Hkv, scale_log2, stream);
    } else {
      if (headwise) launch_bf16<64, kValueGateHead>(Q, K, V, Gv, Y, Lse, B, S, Hq, Hkv, scale_log2, stream);
      else launch_bf16<64, kValueGateElem>(Q, K, V, Gv, Y, Lse, B, S, Hq, Hkv, scale_log2, stream);
    }
  } else {
    if (D == 128) {
      if (headwise) launch_f32<128, kValueGateHead>(Q, K, V, Gv, Y, Lse, B, S, S, Hq, Hkv, scale_log2, stream);
      else launch_f32<128, kValueGateElem>(Q, K, V, Gv, Y, Lse, B, S, S, Hq, Hkv, scale_log2, stream);
    } else {
      if (headwise) launch_f32<64, kValueGateHead>(Q, K, V, Gv, Y, Lse, B, S, S, Hq, Hkv, scale_log2, stream);
      else launch_f32<64, kValueGateElem>(Q, K, V, Gv, Y, Lse, B, S, S, Hq, Hkv, scale_log2, stream);
    }
  }
  return hipGetLastError();
}

// The design-space variants (prefill): the gate layout (kGateNone, kGateElem,
// kGateHead or 3 = shared), additive combination and per-head RMSNorm, on the
// same main loop as launch_attn_fwd.
hipError_t launch_attn_fwd_variant(const void* Q, const void* K, const void* V, const float* G, void* Y,
                                   float* Lse, int B, int S, int Hq, int Hkv, int D, int layout, int add,
                                   int rms, bool bf16_inputs, hipStream_t stream) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  const FwdEpi ep{layout, add, rms};
  if (bf16_inputs) {
    if (D == 128) launch_bf16<128, kGateVariant>(Q, K, V, G, Y, Lse, B, S, Hq, Hkv, scale_log2, stream, ep);
    else launch_bf16<64, kGateVariant>(Q, K, V, G, Y, Lse, B, S, Hq, Hkv, scale_log2, stream, ep);
  } else {
    if (D == 128) launch_f32<128, kGateVariant>(Q, K, V, G, Y, Lse, B, S, S, Hq, Hkv, scale_log2, stream, ep);
    else launch_f32<64, kGateVariant>(Q, K, V, G, Y, Lse, B, S, S, Hq, Hkv, scale_log2, stream, ep);
  }
  return hipGetLastError();
}

// float32 decode with a design-space epilogue: one query row per batch aligned
// to the end of the L-long cache
hipError_t launch_attn_fwd_variant_f32_decode(const void* Q, const void* K, const void* V, const float* G,
                                              void* Y, int B, int L, int Hq, int Hkv, int D, int layout, int add,
                                              int rms, hipStream_t stream) {
  const float scale_log2 = kLog2e / sqrtf((float)D);
  const FwdEpi ep{layout, add, rms};
  if (D == 128) launch_f32<128, kGateVariant>(Q, K, V, G, Y, nullptr, B, 1, L, Hq, Hkv, scale_log2, stream, ep);
  else launch_f32<64, kGateVariant>(Q, K, V, G, Y, nullptr, B, 1, L, Hq, Hkv, scale_log2, stream, ep);
  return hipGetLastError();
}

}  // namespace gsa
