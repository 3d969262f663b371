// Backward of causal gated SDPA (bf16, D in {64, 128}).
//
// The gradients are the chain rule on the forward (see the "Gated Attention如何
// 用1%的参数量…" page, §2.2 gradient analysis, for the gate branch, and the
// derivative of the "GatedAttention [2025]" §1.2.1 SDPA equation, causal per
// §1.4.1, for the attention branch).  For the upstream gradient dY' of the
// gated output Y' = Y ⊙ g:
//   prep:    dY = dY' ⊙ g (bf16), Dᵢ = Σ_d dY'·Y' (= Σ_d dY·Y, the gate cancels),
//            dZ = dY' ⊙ Y' ⊙ (1 − g) (= dY' ⊙ Y ⊙ g(1 − g); headwise:
//            (1 − g_h)·Dᵢ), so no division by g is needed.
//   dQ:      per query tile, over its visible key tiles: S = Q·Kᵀ/√D,
//            P = exp(S − LSE), dP = dY·Vᵀ, dS = P ⊙ (dP − D), dQ += dS·K/√D.
//   dK, dV:  per key tile, over the query heads of its GQA group and the query
//            tiles that see it: dV += Pᵀ·dY, dK += dSᵀ·Q/√D.
// Two kernels recompute S and dP instead of one with atomics, so the result is
// deterministic.
//
// Layout in LDS: every staged tile is [row][d], filled by 16-byte direct loads
// and read both by rows (MFMA operands with 8 consecutive d) and transposed
// (ds_read_b64_tr_b16, operands with 8 consecutive rows).  At D = 128 the rows
// are 256 bytes with an XOR swizzle of their 16-byte chunks that keeps both
// kinds of read free of bank conflicts (Tile below); at D = 64 they are
// padded to 144 bytes.  The transposed-read addressing permutes rows inside
// each 16-row block so a lane's 8 rows match the accumulator layout of S,
// exactly as the forward's PV product does with its probabilities.
#include <type_traits>

#include "common.h"

namespace gsa {

#define GSA_LDS_B __attribute__((address_space(3)))

namespace bwd {
constexpr int QT = 128;   // query rows per dQ workgroup (4 waves x 32)
constexpr int KT = 64;    // key rows per staged tile in the dQ kernel
constexpr int KW = 128;   // key rows per dK/dV workgroup at D = 64 (4 waves x 32)
constexpr int QW = 64;    // query rows per staged tile in the dK/dV kernel
constexpr uint32_t kOOB = 0xfffffff0u;
}  // namespace bwd

enum : int { kBwdGateNone = 0, kBwdGateElem = 1, kBwdGateHead = 2 };

// ---------------------------------------------------------------- prep
// One (token, head) row per D/8 threads, 8 head dims per thread.  Besides dY
// and dZ it writes the per-row statistics both attention kernels read: Stat
// holds [B*Hq][Sp] base-2 LSE values, then [B*Hq][Sp] D values (Sp = S rounded
// up to 64; the padding rows hold zeros and are always masked).
template <int D, int MODE>
__global__ __launch_bounds__(256)
void bwd_prep_kernel(const bf16* __restrict__ dYg, const bf16* __restrict__ Yg,
                     const float* __restrict__ Gate, const float* __restrict__ Lse,
                     bf16* __restrict__ dY, float* __restrict__ Stat, bf16* __restrict__ dZ, int B, int S,
                     int Hq, int Sp) {
  constexpr int TPR = D / 8;                 // threads per row
  constexpr int RPB = 256 / TPR;             // rows per block
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;   // = token * Hq + head
  const int part = tid % TPR;
  const int64_t nrows = (int64_t)B * S * Hq;
  const bool live = row < nrows;
  const int64_t rr = live ? row : nrows - 1;
  const int64_t tok = rr / Hq;
  const int head = (int)(rr % Hq);
  const int64_t e0 = rr * D + part * 8;
  const u32x4 gy = *(const u32x4*)(dYg + e0);
  const u32x4 yy = *(const u32x4*)(Yg + e0);
  float g[8];
  if constexpr (MODE == kBwdGateElem) {
    const f32x4 g0 = *(const f32x4*)(Gate + e0);
    const f32x4 g1 = *(const f32x4*)(Gate + e0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g[e] = g0[e];
      g[e + 4] = g1[e];
    }
  } else {
    const float gh = MODE == kBwdGateHead ? Gate[tok * Hq + head] : 1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = gh;
  }
  float dsum = 0.f, dy[8], z[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a0 = bf16_lo(gy[w]), a1 = bf16_hi(gy[w]);
    const float y0 = bf16_lo(yy[w]), y1 = bf16_hi(yy[w]);
    const float p0 = a0 * y0, p1 = a1 * y1;
    dsum += p0;
    dsum += p1;
    dy[2 * w] = a0 * g[2 * w];
    dy[2 * w + 1] = a1 * g[2 * w + 1];
    z[2 * w] = p0 * (1.0f - g[2 * w]);
    z[2 * w + 1] = p1 * (1.0f - g[2 * w + 1]);
  }
  // row sum over the TPR threads of the row (fixed order)
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) dsum += __shfl_xor(dsum, o);
  if (!live) return;
  if constexpr (MODE != kBwdGateNone) {
    *(u32x4*)(dY + e0) = u32x4{pack_bf16x2(dy[0], dy[1]), pack_bf16x2(dy[2], dy[3]),
                               pack_bf16x2(dy[4], dy[5]), pack_bf16x2(dy[6], dy[7])};
  }
  if constexpr (MODE == kBwdGateElem) {
    *(u32x4*)(dZ + e0) = u32x4{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]),
                               pack_bf16x2(z[4], z[5]), pack_bf16x2(z[6], z[7])};
  }
  if (part == 0) {
    const int64_t b = tok / S, i = tok % S;
    const int64_t bh = b * Hq + head;
    Stat[bh * Sp + i] = Lse[bh * S + i] * kLog2e;
    Stat[((int64_t)B * Hq + bh) * Sp + i] = dsum;
    if (i == S - 1)
      for (int64_t j = S; j < Sp; ++j) {
        Stat[bh * Sp + j] = 0.f;
        Stat[((int64_t)B * Hq + bh) * Sp + j] = 0.f;
      }
    if constexpr (MODE == kBwdGateHead) dZ[tok * Hq + head] = (bf16)((1.0f - g[0]) * dsum);
  }
}

// ---------------------------------------------------------------- shared pieces
// Staged tile: rows of D bf16, each read two ways: 16-byte row reads (8
// consecutive dims of one row: the A operand of S-type products) and
// transposed reads (4 dims of 4 consecutive rows per lane: the A operand of
// products whose k runs over rows).  Both must avoid LDS bank conflicts.
//   D = 64: 144-byte rows, 8 chunks of 16 bytes plus one pad slot.
//   D = 128: 256-byte rows with no pad; chunk c of row r sits in slot
//            c ^ tile_swz(r), tile_swz(r) = 4·(r & 3) + ((r >> 2) & 3).
// tile_swz is a bijection on any 16 consecutive rows, so the 16 rows of a row
// read land in 16 different slots.  A transposed read touches rows R..R+3
// (R a multiple of 4) and chunks 4m..4m+3 over 32 lanes; tile_swz(R + j)
// differs in bits 2..3 for the four j, so those 16 (row, chunk) pairs also
// land in 16 different slots, one per group of four banks.  (A padded 272-byte
// row instead puts neighbouring rows of a transposed read on overlapping banks.)
__host__ __device__ constexpr int tile_swz(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }

template <int D>
struct Tile {
  static constexpr bool SWZ = D == 128;
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int SL = SWZ ? CH : CH + 1;     // slots per row
  static constexpr int RSB = SL * 16;              // row stride in bytes
  // byte offset, within its row, of chunk c of row `row`
  static __device__ __forceinline__ int chunk_off(int row, int c) { return (SWZ ? c ^ tile_swz(row) : c) * 16; }
};

// Direct loads of `rows` rows of a [*, stride] bf16 tensor into a tile by
// WAVES waves; instruction i covers slots 64*i .. 64*i+63 (slot s = row·SL +
// physical chunk).  Rows at or past `row_end` and the pad slot read zeros.
// Every instruction writes all 64 slots, so the LDS buffer must hold kBytes
// (whole instructions), which exceeds ROWS row strides when ROWS * SL is not a
// multiple of 64.
template <int D, int ROWS, int WAVES = 4>
struct TileLoader {
  static constexpr int SL = Tile<D>::SL;
  static constexpr int NI = (ROWS * SL + 64 * WAVES - 1) / (64 * WAVES);   // instructions per wave
  static constexpr int kBytes = (ROWS * SL + 63) / 64 * 1024;
  uint32_t off[NI];
  uint32_t ins_base[NI];
  __device__ void init(int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int ins = wave + WAVES * j;
      const int sl = ins * 64 + lane;
      const int row = sl / SL, ch = sl % SL;
      // the logical chunk stored in physical slot ch (the swizzle is its own inverse)
      const int c = Tile<D>::SWZ ? ch ^ tile_swz(row) : ch;
      off[j] = (ch < Tile<D>::CH && row < ROWS) ? (uint32_t)row * row_bytes + c * 16 : kOOBv();
      ins_base[j] = (uint32_t)ins * 64 * 16;
    }
  }
  static __device__ constexpr uint32_t kOOBv() { return 0xfffffff0u; }
  // rows [r0, r0 + ROWS) of the tensor behind rs; rows >= row_end read zeros
  __device__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, int r0, int row_end,
                       uint32_t lds_base, int wave) const {
    const uint32_t base = (uint32_t)r0 * row_bytes;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int ins = wave + WAVES * j;
      if (ins * 64 < ROWS * SL) {
        const int lane_row = (int)((ins_base[j] / 16 + (threadIdx.x & 63)) / SL);
        const bool ok = off[j] != kOOBv() && r0 + lane_row < row_end;
        dma16_lds(rs, ok ? off[j] + base : kOOBv(), lds_base + ins_base[j]);
      }
    }
  }
};

// Transposed-read addresses of a lane inside a tile for the A operand of an
// MFMA whose k index runs over tile rows: rows 16t + 8a + 4*hl + 0..3 of a
// 16-row block land in k slots 4a..4a+3 of lane half hl (the accumulator layout
// of S), dims dt*32 + (lane within 32).  The lane's first read names row
// r = 4*(g/2) + i/4 (g = lane/16, i = lane%16), the second row r + 8; both
// name dims dt*32 + 16*(g%2) + 4*(i%4) .. +3.  Adding a multiple of 16 rows
// keeps the swizzle, so one pair of offsets serves every 16-row block.
struct TrAddr {
  uint32_t lo, hi;
};
template <int D>
__device__ __forceinline__ TrAddr tr_addr(int lane, int dt) {
  const int vg = lane >> 4, vi = lane & 15;
  const int r = 4 * (vg >> 1) + (vi >> 2);
  const int dc = dt * 32 + 16 * (vg & 1) + 4 * (vi & 3);   // first of the lane's 4 dims
  const int c = dc / 8, in = (dc % 8) * 2;                  // its chunk and byte within the chunk
  return TrAddr{(uint32_t)(r * Tile<D>::RSB + Tile<D>::chunk_off(r, c) + in),
                (uint32_t)((r + 8) * Tile<D>::RSB + Tile<D>::chunk_off(r + 8, c) + in)};
}

__device__ __forceinline__ bf16x8 tr_read(const GSA_LDS_B char* blk, const TrAddr& a) {
  const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS_B i16x4*)(blk + a.lo));
  const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS_B i16x4*)(blk + a.hi));
  bf16x8 r;
  r.lo = __builtin_bit_cast(bf16x4, lo);
  r.hi = __builtin_bit_cast(bf16x4, hi);
  return r;
}

// Row read: row `row`, dims 16*kk + 8*hl .. +7 (the A operand of S-type products).
template <int D>
__device__ __forceinline__ bf16x8 row_read(const GSA_LDS_B char* tile, int row, int kk, int hl) {
  return *(const GSA_LDS_B bf16x8*)(tile + row * Tile<D>::RSB + Tile<D>::chunk_off(row, 2 * kk + hl));
}

// Accumulator pair (2 x 32 rows of a 64-row block, 16 regs each) -> bf16 B
// operands, k order matching tr_addr's row permutation.
__device__ __forceinline__ void pack_b(const f32x16 (&s)[2], bf16x8 (&pb)[2][2]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[sub][t][e] = (bf16)s[sub][8 * t + e];
}

// ---------------------------------------------------------------- dQ
// 256 threads: 128 query rows of one head (4 waves x 32); key tiles of 64.
//   Sᵀ = K·Qᵀ, dPᵀ = V·dYᵀ  (A = K / V rows from LDS, B = Q / dY fragments)
//   dQᵀ += Kᵀ·dSᵀ          (A = K through transposed reads, B = dS in bf16)
// Two workgroups per CU (≤ 256 registers, 68 KB of LDS each): the second
// workgroup's waves hide the first's LDS and barrier waits.
template <int D>
__global__ __launch_bounds__(256, 2)
void bwd_dq_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                   const bf16* __restrict__ dY, const float* __restrict__ Stat,
                   bf16* __restrict__ dQ, int B, int S, int Hq, int Hkv, int n_qtiles, int Sp,
                   float scale) {
  using namespace bwd;
  constexpr int RSB = Tile<D>::RSB;
  static_assert(TileLoader<D, KT>::kBytes == KT * RSB, "key tile is not a whole number of loads");
  __shared__ __align__(16) char Ks[2][KT * RSB];
  __shared__ __align__(16) char Vs[2][KT * RSB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int bid = blockIdx.x;
  const int hb = Hq * B;
  const int qt = n_qtiles - 1 - bid / hb;
  const int pair = bid % hb;
  const int head = pair % Hq, b = pair / Hq;
  const int kvh = head / (Hq / Hkv);
  const int q0 = qt * QT, qw0 = q0 + wave * 32, my_q = qw0 + l32;
  const int64_t q_row = (int64_t)Hq * D, kv_row = (int64_t)Hkv * D;
  const float scale_log2 = scale * kLog2e;

  // Q and dY fragments (B operands), LSE (base 2) and D of this lane's row
  bf16x8 qf[D / 16], yf[D / 16];
  {
    const auto qr = make_rsrc(Q + (int64_t)b * S * q_row + (int64_t)head * D,
                              (uint32_t)(((int64_t)S * q_row - (int64_t)head * D) * 2));
    const auto yr = make_rsrc(dY + (int64_t)b * S * q_row + (int64_t)head * D,
                              (uint32_t)(((int64_t)S * q_row - (int64_t)head * D) * 2));
    const uint32_t o = (uint32_t)(((int64_t)my_q * q_row + 8 * hl) * 2);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = __builtin_bit_cast(bf16x8, buffer_load16(qr, o + 32 * kk, 0));
      yf[kk] = __builtin_bit_cast(bf16x8, buffer_load16(yr, o + 32 * kk, 0));
    }
  }
  const int qc = min(my_q, S - 1);
  float lse2 = Stat[((int64_t)b * Hq + head) * Sp + qc];
  float dval = Stat[((int64_t)(B + b) * Hq + head) * Sp + qc];
  // settle these loads before the loop (see the dK/dV kernel)
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(qf[kk]), "+v"(yf[kk]));
  asm volatile("" : "+v"(lse2), "+v"(dval));

  const uint32_t row_b = (uint32_t)(kv_row * 2);
  const uint32_t kv_bytes = (uint32_t)(((int64_t)S * kv_row - (int64_t)kvh * D) * 2);
  const auto krs = make_rsrc(K + (int64_t)b * S * kv_row + (int64_t)kvh * D, kv_bytes);
  const auto vrs = make_rsrc(V + (int64_t)b * S * kv_row + (int64_t)kvh * D, kv_bytes);
  TileLoader<D, KT> ld;
  ld.init(wave, lane, row_b);
  const uint32_t ks_lds0 = __builtin_amdgcn_readfirstlane(lds_addr(&Ks[0][0]));
  const uint32_t vs_lds0 = __builtin_amdgcn_readfirstlane(lds_addr(&Vs[0][0]));
  TrAddr trb[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) trb[dt] = tr_addr<D>(lane, dt);

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  const int kv_end = min(S, q0 + QT);
  const int n_kv = ceil_div(kv_end, KT);
  ld.load(krs, row_b, 0, S, ks_lds0, wave);
  ld.load(vrs, row_b, 0, S, vs_lds0, wave);
  // one key tile with its stage known at compile time (the loop below is
  // unrolled by two), so every LDS address is a constant offset from the base
  auto one_tile = [&](auto stage, int it) {
    constexpr int buf = decltype(stage)::value;
    const int k0 = it * KT;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < n_kv) {
      ld.load(krs, row_b, k0 + KT, S, ks_lds0 + (buf ^ 1) * (KT * RSB), wave);
      ld.load(vrs, row_b, k0 + KT, S, vs_lds0 + (buf ^ 1) * (KT * RSB), wave);
    }
    const GSA_LDS_B char* kt = (const GSA_LDS_B char*)(GSA_LDS_B void*)&Ks[buf][0];
    const GSA_LDS_B char* vt = (const GSA_LDS_B char*)(GSA_LDS_B void*)&Vs[buf][0];
    f32x16 s[2], dp[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[sub][r] = 0.f;
        dp[sub][r] = 0.f;
      }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        s[sub] = mfma32x32x16(row_read<D>(kt, sub * 32 + l32, kk, hl), qf[kk], s[sub]);
        dp[sub] = mfma32x32x16(row_read<D>(vt, sub * 32 + l32, kk, hl), yf[kk], dp[sub]);
      }
    // element (sub, r) is key k0 + sub*32 + 8*(r/4) + 4*hl + r%4 of query my_q;
    // only tiles reaching past the wave's first query need the causal mask
    // (keys past S hold zeros and only ever meet masked or discarded rows)
    if (k0 + KT - 1 > qw0) {
      const int lim = qc - k0 - 4 * hl;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (sub * 32 + 8 * (r >> 2) + (r & 3) > lim) s[sub][r] = -INFINITY;
    }
    // dS and the dQ product one 16-key quarter (sub, t) at a time: a quarter's
    // matrix ops need only its own dS, so the next quarter's exp work runs in
    // their shadow (dQ still accumulates keys in increasing order)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 ds;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * t + e;
          const float p = fast_exp2(fmaf(s[sub][r], scale_log2, -lse2));
          ds[e] = (bf16)(p * (dp[sub][r] - dval));   // dS
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          acc[dt] = mfma32x32x16(tr_read(kt + (sub * 32 + 16 * t) * RSB, trb[dt]), ds, acc[dt]);
      }
  };
  for (int it = 0; it < n_kv; it += 2) {
    one_tile(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_kv) one_tile(std::integral_constant<int, 1>{}, it + 1);
  }

  // Store through LDS: a lane holds one query row in 16-byte pieces 32 bytes
  // apart, so a direct store would touch 32 rows at once.  Each wave stages
  // its 32 rows of float32 dQ in one of the four tile buffers (free once every
  // wave is past the loop), chunk c of row r in slot c ^ (r & 15) (distinct
  // banks for both access patterns), and reads them back by rows.
  static_assert(KT * RSB >= 32 * 4 * D, "a tile buffer holds one wave's 32 rows of float32");
  __syncthreads();
  char* const stg = wave == 0 ? &Ks[0][0] : wave == 1 ? &Ks[1][0] : wave == 2 ? &Vs[0][0] : &Vs[1][0];
  GSA_LDS_B char* const sg = (GSA_LDS_B char*)(GSA_LDS_B void*)stg;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 8 * dt + 2 * i + hl;   // 16-byte chunk of dims dt*32 + 8i + 4hl .. +3
      *(GSA_LDS_B f32x4*)(sg + l32 * (4 * D) + (c ^ (l32 & 15)) * 16) =
          f32x4{acc[dt][4 * i] * scale, acc[dt][4 * i + 1] * scale, acc[dt][4 * i + 2] * scale,
                acc[dt][4 * i + 3] * scale};
    }
  // the rows are read back by other lanes of this wave
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int LPR = D / 4, RPI = 64 / LPR;
  const int sr = lane / LPR, sc = lane % LPR;
#pragma unroll
  for (int n = 0; n < 32 / RPI; ++n) {
    const int r = RPI * n + sr;
    const f32x4 v = *(const GSA_LDS_B f32x4*)(sg + r * (4 * D) + (sc ^ (r & 15)) * 16);
    if (qw0 + r < S)
      *(u32x2*)(dQ + ((int64_t)b * S + qw0 + r) * q_row + (int64_t)head * D + 4 * sc) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// ---------------------------------------------------------------- dK, dV
// 256 threads: 128 keys of one key/value head (4 waves x 32).  For each query
// head of the workgroup's slice of the group and each 64-row query tile that
// sees these keys:
//   S = Q·Kᵀ, dP = dY·Vᵀ      (A = Q / dY rows from LDS, B = K / V fragments)
//   dVᵀ += dYᵀ·P, dKᵀ += Qᵀ·dS (A through transposed reads, B = P / dS in bf16)
// The query heads of a group may be cut into `nsplit` slices (one workgroup
// each) so small-Hkv shapes still fill the chip; slices then write float32
// partial sums [nsplit][B][S][Hkv][D] that bwd_sum_slices adds in order.
// Launched at D = 64 (two workgroups per CU).  At D = 128 this arrangement
// needs ≈ 360 registers (one workgroup per CU); bwd_dkdv_vlds_kernel replaces it
// there.
template <int D, bool PARTIAL>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1)
void bwd_dkdv_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                     const bf16* __restrict__ dY, const float* __restrict__ Stat,
                     bf16* __restrict__ dK, bf16* __restrict__ dV, float* __restrict__ dKp,
                     float* __restrict__ dVp, int B, int S, int Hq, int Hkv, int Sp, int nsplit,
                     float scale) {
  using namespace bwd;
  constexpr int RSB = Tile<D>::RSB;
  static_assert(TileLoader<D, QW>::kBytes == QW * RSB, "query tile is not a whole number of loads");
  __shared__ __align__(16) char Qs[2][QW * RSB];
  __shared__ __align__(16) char Ys[2][QW * RSB];
  __shared__ __align__(16) float Ss[2][256];   // per stage: base-2 LSE of 64 rows, D of 64 rows, pad
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int bid = blockIdx.x;
  const int hb = Hkv * B * nsplit;
  const int kt_i = bid / hb;                       // early key tiles see the most queries: first
  const int rest = bid % hb;
  const int slice = rest % nsplit, pair = rest / nsplit;
  const int kvh = pair % Hkv, b = pair / Hkv;
  const int G = Hq / Hkv, Gs = G / nsplit;
  const int k0 = kt_i * KW, kw0 = k0 + wave * 32, my_k = kw0 + l32;
  const int64_t q_row = (int64_t)Hq * D, kv_row = (int64_t)Hkv * D;
  const float scale_log2 = scale * kLog2e;

  // K and V fragments (B operands) of this lane's key
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const uint32_t kv_bytes = (uint32_t)(((int64_t)S * kv_row - (int64_t)kvh * D) * 2);
    const auto kr = make_rsrc(K + (int64_t)b * S * kv_row + (int64_t)kvh * D, kv_bytes);
    const auto vr = make_rsrc(V + (int64_t)b * S * kv_row + (int64_t)kvh * D, kv_bytes);
    const uint32_t o = (uint32_t)(((int64_t)my_k * kv_row + 8 * hl) * 2);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kf[kk] = __builtin_bit_cast(bf16x8, buffer_load16(kr, o + 32 * kk, 0));
      vf[kk] = __builtin_bit_cast(bf16x8, buffer_load16(vr, o + 32 * kk, 0));
    }
    // settle these loads here: otherwise the compiler re-waits for them inside
    // the loop, and that wait also drains the next tile's direct loads
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(kf[kk]), "+v"(vf[kk]));
  }
  const uint32_t row_b = (uint32_t)(q_row * 2);
  TileLoader<D, QW> ld;
  ld.init(wave, lane, row_b);
  uint32_t qs_lds[2], ys_lds[2], st_lds[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    qs_lds[i] = __builtin_amdgcn_readfirstlane(lds_addr(&Qs[i][0]));
    ys_lds[i] = __builtin_amdgcn_readfirstlane(lds_addr(&Ys[i][0]));
    st_lds[i] = __builtin_amdgcn_readfirstlane(lds_addr(&Ss[i][0]));
  }
  // statistics loads (wave 0): lanes 0..15 take 4 LSE rows each, lanes 16..31 4 D rows
  const auto srs = make_rsrc(Stat, (uint32_t)((int64_t)2 * B * Hq * Sp * 4));
  const uint32_t st_lane = lane < 16 ? 16u * lane : (uint32_t)((int64_t)B * Hq * Sp * 4) + 16u * (lane - 16);
  TrAddr trb[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) trb[dt] = tr_addr<D>(lane, dt);

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  // query tiles that see keys [k0, k0 + KW): rows >= k0
  const int qt_first = k0 / QW;
  const int n_qt = ceil_div(S, QW) - qt_first;
  const int n_steps = Gs * max(n_qt, 0);
  const int head0 = kvh * G + slice * Gs;
  auto tile_of = [&](int step, int& head, int& qs0) {
    head = head0 + step / n_qt;
    qs0 = (qt_first + step % n_qt) * QW;
  };
  auto issue = [&](int step, int buf) {
    int head, qs0;
    tile_of(step, head, qs0);
    const uint32_t bytes = (uint32_t)(((int64_t)S * q_row - (int64_t)head * D) * 2);
    const auto qr = make_rsrc(Q + (int64_t)b * S * q_row + (int64_t)head * D, bytes);
    const auto yr = make_rsrc(dY + (int64_t)b * S * q_row + (int64_t)head * D, bytes);
    ld.load(qr, row_b, qs0, S, qs_lds[buf], wave);
    ld.load(yr, row_b, qs0, S, ys_lds[buf], wave);
    if (wave == 0)
      dma16_lds(srs, lane < 32 ? st_lane + (uint32_t)(((int64_t)b * Hq + head) * Sp + qs0) * 4u : kOOB,
                st_lds[buf]);
  };
  if (n_steps > 0) issue(0, 0);
  for (int step = 0; step < n_steps; ++step) {
    const int buf = step & 1;
    int head, qs0;
    tile_of(step, head, qs0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (step + 1 < n_steps) issue(step + 1, buf ^ 1);
    const GSA_LDS_B char* qt = (const GSA_LDS_B char*)(GSA_LDS_B void*)&Qs[buf][0];
    const GSA_LDS_B char* yt = (const GSA_LDS_B char*)(GSA_LDS_B void*)&Ys[buf][0];
    const GSA_LDS_B float* st = (const GSA_LDS_B float*)(GSA_LDS_B void*)&Ss[buf][0];
    f32x16 s[2], dp[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[sub][r] = 0.f;
        dp[sub][r] = 0.f;
      }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        s[sub] = mfma32x32x16(row_read<D>(qt, sub * 32 + l32, kk, hl), kf[kk], s[sub]);
        dp[sub] = mfma32x32x16(row_read<D>(yt, sub * 32 + l32, kk, hl), vf[kk], dp[sub]);
      }
    // element (sub, r): query qs0 + 32*sub + 8*(r/4) + 4*hl + r%4, key my_k.
    // A wave needs the mask only where its keys pass the tile's first query or
    // the tile runs past S (rows past S hold zero statistics and must not count).
    if ((qs0 < kw0 + 31) || (qs0 + QW > S)) {
      const int lo = my_k - qs0 - 4 * hl, hi = S - 1 - qs0 - 4 * hl;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * sub + 8 * (r >> 2) + (r & 3);
          if (off < lo || off > hi) s[sub][r] = -INFINITY;
        }
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row4 = 32 * sub + 8 * i + 4 * hl;
        const f32x4 l4 = *(const GSA_LDS_B f32x4*)(st + row4);
        const f32x4 d4 = *(const GSA_LDS_B f32x4*)(st + 64 + row4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * i + j;
          const float p = fast_exp2(fmaf(s[sub][r], scale_log2, -l4[j]));
          dp[sub][r] = p * (dp[sub][r] - d4[j]);   // dS
          s[sub][r] = p;
        }
      }
    bf16x8 pb[2][2], db[2][2];
    pack_b(s, pb);
    pack_b(dp, db);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int ro = (sub * 32 + 16 * t) * RSB;
          dv[dt] = mfma32x32x16(tr_read(yt + ro, trb[dt]), pb[sub][t], dv[dt]);
          dk[dt] = mfma32x32x16(tr_read(qt + ro, trb[dt]), db[sub][t], dk[dt]);
        }
  }

  if (my_k >= S) return;
  const int64_t orow = ((int64_t)b * S + my_k) * kv_row + (int64_t)kvh * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = dt * 32 + 8 * i + 4 * hl;
      if constexpr (PARTIAL) {
        const int64_t o = (int64_t)slice * B * S * kv_row + orow + d0;
        *(f32x4*)(dKp + o) = f32x4{dk[dt][4 * i] * scale, dk[dt][4 * i + 1] * scale,
                                   dk[dt][4 * i + 2] * scale, dk[dt][4 * i + 3] * scale};
        *(f32x4*)(dVp + o) = f32x4{dv[dt][4 * i], dv[dt][4 * i + 1], dv[dt][4 * i + 2], dv[dt][4 * i + 3]};
      } else {
        *(u32x2*)(dK + orow + d0) = u32x2{pack_bf16x2(dk[dt][4 * i] * scale, dk[dt][4 * i + 1] * scale),
                                          pack_bf16x2(dk[dt][4 * i + 2] * scale, dk[dt][4 * i + 3] * scale)};
        *(u32x2*)(dV + orow + d0) = u32x2{pack_bf16x2(dv[dt][4 * i], dv[dt][4 * i + 1]),
                                          pack_bf16x2(dv[dt][4 * i + 2], dv[dt][4 * i + 3])};
      }
    }
}

// ---------------------------------------------------------------- dK, dV at D = 128
// The same products as bwd_dkdv_kernel, arranged to fit two waves per SIMD
// (≤ 256 registers): WAVES = 4 runs two workgroups per CU (66 KB of LDS
// each), so one workgroup's waves cover the other's LDS and barrier waits;
// WAVES = 8 runs one workgroup of 256 keys per CU (98 KB), in which each
// staged query tile feeds twice the matrix ops.
//   * V of the workgroup's keys is staged once in LDS and read back as the
//     B operand of dP (a 16-byte row read per k step) instead of living in
//     registers;
//   * query tiles are 32 rows, halving the S and dP accumulators.
// K fragments and the dK/dV accumulators stay in registers.  Query tiles are
// double-buffered: the next tile's loads fly while one is consumed.
template <int D, bool PARTIAL, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES)
void bwd_dkdv_vlds_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                          const bf16* __restrict__ dY, const float* __restrict__ Stat,
                          bf16* __restrict__ dK, bf16* __restrict__ dV, float* __restrict__ dKp,
                          float* __restrict__ dVp, int B, int S, int Hq, int Hkv, int Sp, int nsplit,
                          float scale) {
  using namespace bwd;
  constexpr int RSB = Tile<D>::RSB;
  constexpr int QR = 32;                 // query rows per staged tile
  constexpr int KWV = 32 * WAVES;        // keys per workgroup
  constexpr int QB = TileLoader<D, QR, WAVES>::kBytes;   // 32 rows, rounded up to whole loads
  __shared__ __align__(16) char Vt[TileLoader<D, KWV, WAVES>::kBytes];
  __shared__ __align__(16) char Qs[2][QB];
  __shared__ __align__(16) char Ys[2][QB];
  __shared__ __align__(16) float Ss[2][256];   // per stage: base-2 LSE of 32 rows, D of 32 rows, pad
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int bid = blockIdx.x;
  const int hb = Hkv * B * nsplit;
  const int kt_i = bid / hb;                       // early key tiles see the most queries: first
  const int rest = bid % hb;
  const int slice = rest % nsplit, pair = rest / nsplit;
  const int kvh = pair % Hkv, b = pair / Hkv;
  const int G = Hq / Hkv, Gs = G / nsplit;
  const int k0 = kt_i * KWV, kw0 = k0 + wave * 32, my_k = kw0 + l32;
  const int64_t q_row = (int64_t)Hq * D, kv_row = (int64_t)Hkv * D;
  const float scale_log2 = scale * kLog2e;

  const uint32_t kv_bytes = (uint32_t)(((int64_t)S * kv_row - (int64_t)kvh * D) * 2);
  const uint32_t kv_row_b = (uint32_t)(kv_row * 2);
  const auto vr = make_rsrc(V + (int64_t)b * S * kv_row + (int64_t)kvh * D, kv_bytes);
  {
    TileLoader<D, KWV, WAVES> vld;
    vld.init(wave, lane, kv_row_b);
    vld.load(vr, kv_row_b, k0, S, __builtin_amdgcn_readfirstlane(lds_addr(&Vt[0])), wave);
  }
  // K fragments (B operands) of this lane's key
  bf16x8 kf[D / 16];
  {
    const auto kr = make_rsrc(K + (int64_t)b * S * kv_row + (int64_t)kvh * D, kv_bytes);
    const uint32_t o = (uint32_t)(((int64_t)my_k * kv_row + 8 * hl) * 2);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kf[kk] = __builtin_bit_cast(bf16x8, buffer_load16(kr, o + 32 * kk, 0));
    // settled here so the loop's waits do not re-wait for them
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(kf[kk]));
  }
  const uint32_t row_b = (uint32_t)(q_row * 2);
  TileLoader<D, QR, WAVES> ld;
  ld.init(wave, lane, row_b);
  // stage i of each array sits i whole stages past stage 0
  const uint32_t qs_lds0 = __builtin_amdgcn_readfirstlane(lds_addr(&Qs[0][0]));
  const uint32_t ys_lds0 = __builtin_amdgcn_readfirstlane(lds_addr(&Ys[0][0]));
  const uint32_t st_lds0 = __builtin_amdgcn_readfirstlane(lds_addr(&Ss[0][0]));
  // statistics loads (wave 0): lanes 0..7 take 4 LSE rows each, lanes 8..15 4 D rows
  const auto srs = make_rsrc(Stat, (uint32_t)((int64_t)2 * B * Hq * Sp * 4));
  const uint32_t st_lane = lane < 8 ? 16u * lane : (uint32_t)((int64_t)B * Hq * Sp * 4) + 16u * (lane - 8);
  TrAddr trb[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) trb[dt] = tr_addr<D>(lane, dt);

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  // query tiles that see keys [k0, k0 + KWV): rows >= k0
  const int qt_first = k0 / QR;
  const int n_qt = ceil_div(S, QR) - qt_first;
  const int n_steps = Gs * max(n_qt, 0);
  const int head0 = kvh * G + slice * Gs;
  auto tile_of = [&](int step, int& head, int& qs0) {
    head = head0 + step / n_qt;
    qs0 = (qt_first + step % n_qt) * QR;
  };
  auto issue = [&](int step, int buf) {
    int head, qs0;
    tile_of(step, head, qs0);
    const uint32_t bytes = (uint32_t)(((int64_t)S * q_row - (int64_t)head * D) * 2);
    const auto qr = make_rsrc(Q + (int64_t)b * S * q_row + (int64_t)head * D, bytes);
    const auto yr = make_rsrc(dY + (int64_t)b * S * q_row + (int64_t)head * D, bytes);
    ld.load(qr, row_b, qs0, S, qs_lds0 + (uint32_t)buf * QB, wave);
    ld.load(yr, row_b, qs0, S, ys_lds0 + (uint32_t)buf * QB, wave);
    if (wave == 0)
      dma16_lds(srs, lane < 16 ? st_lane + (uint32_t)(((int64_t)b * Hq + head) * Sp + qs0) * 4u : kOOB,
                st_lds0 + (uint32_t)buf * 1024u);
  };
  const GSA_LDS_B char* vt = (const GSA_LDS_B char*)(GSA_LDS_B void*)&Vt[0];
  if (n_steps > 0) issue(0, 0);
  // one step with its stage known at compile time (the loop below is unrolled
  // by two), so every LDS address is a constant offset from the stage base
  auto one_step = [&](auto stage, int step) {
    constexpr int buf = decltype(stage)::value;
    int head, qs0;
    tile_of(step, head, qs0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // the stage refilled here was consumed in step - 1, before the barrier
    if (step + 1 < n_steps) issue(step + 1, buf ^ 1);
    // a wave whose keys all come after the tile's last query gets P = dS = 0
    if (kw0 > qs0 + QR - 1) return;
    const GSA_LDS_B char* qt = (const GSA_LDS_B char*)(GSA_LDS_B void*)&Qs[buf][0];
    const GSA_LDS_B char* yt = (const GSA_LDS_B char*)(GSA_LDS_B void*)&Ys[buf][0];
    const GSA_LDS_B float* st = (const GSA_LDS_B float*)(GSA_LDS_B void*)&Ss[buf][0];
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      s = mfma32x32x16(row_read<D>(qt, l32, kk, hl), kf[kk], s);
      dp = mfma32x32x16(row_read<D>(yt, l32, kk, hl), row_read<D>(vt, wave * 32 + l32, kk, hl), dp);
    }
    // element r: query qs0 + 8*(r/4) + 4*hl + r%4, key my_k.  Masked where the
    // wave's keys pass the tile's first query or the tile runs past S (rows
    // past S hold zero statistics and must not count).
    if ((qs0 < kw0 + 31) || (qs0 + QR > S)) {
      const int lo = my_k - qs0 - 4 * hl, hi = S - 1 - qs0 - 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        if (off < lo || off > hi) s[r] = -INFINITY;
      }
    }
    // P, dS and the dV / dK products one 16-row half t at a time: a half's
    // matrix ops need only its own P and dS, so the next half's exp work runs
    // in their shadow (dV and dK still accumulate rows in increasing order)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 pb, db;
#pragma unroll
      for (int i = 2 * t; i < 2 * t + 2; ++i) {
        const int row4 = 8 * i + 4 * hl;
        const f32x4 l4 = *(const GSA_LDS_B f32x4*)(st + row4);
        const f32x4 d4 = *(const GSA_LDS_B f32x4*)(st + QR + row4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * i + j;
          const float p = fast_exp2(fmaf(s[r], scale_log2, -l4[j]));
          pb[r - 8 * t] = (bf16)p;
          db[r - 8 * t] = (bf16)(p * (dp[r] - d4[j]));   // dS
        }
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int ro = 16 * t * RSB;
        dv[dt] = mfma32x32x16(tr_read(yt + ro, trb[dt]), pb, dv[dt]);
        dk[dt] = mfma32x32x16(tr_read(qt + ro, trb[dt]), db, dk[dt]);
      }
    }
  };
  for (int step = 0; step < n_steps; step += 2) {
    one_step(std::integral_constant<int, 0>{}, step);
    if (step + 1 < n_steps) one_step(std::integral_constant<int, 1>{}, step + 1);
  }

  if (my_k >= S) return;
  const int64_t orow = ((int64_t)b * S + my_k) * kv_row + (int64_t)kvh * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = dt * 32 + 8 * i + 4 * hl;
      if constexpr (PARTIAL) {
        const int64_t o = (int64_t)slice * B * S * kv_row + orow + d0;
        *(f32x4*)(dKp + o) = f32x4{dk[dt][4 * i] * scale, dk[dt][4 * i + 1] * scale,
                                   dk[dt][4 * i + 2] * scale, dk[dt][4 * i + 3] * scale};
        *(f32x4*)(dVp + o) = f32x4{dv[dt][4 * i], dv[dt][4 * i + 1], dv[dt][4 * i + 2], dv[dt][4 * i + 3]};
      } else {
        *(u32x2*)(dK + orow + d0) = u32x2{pack_bf16x2(dk[dt][4 * i] * scale, dk[dt][4 * i + 1] * scale),
                                          pack_bf16x2(dk[dt][4 * i + 2] * scale, dk[dt][4 * i + 3] * scale)};
        *(u32x2*)(dV + orow + d0) = u32x2{pack_bf16x2(dv[dt][4 * i], dv[dt][4 * i + 1]),
                                          pack_bf16x2(dv[dt][4 * i + 2], dv[dt][4 * i + 3])};
      }
    }
}

// dK, dV (bf16) = Σ over slices of the float32 partial sums, in slice order;
// 4 elements per thread (n4 = element count / 4).
__global__ __launch_bounds__(256)
void bwd_sum_slices_kernel(const f32x4* __restrict__ dKp, const f32x4* __restrict__ dVp, u32x2* __restrict__ dK,
                           u32x2* __restrict__ dV, int64_t n4, int nsplit) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 a = dKp[i], c = dVp[i];
    for (int z = 1; z < nsplit; ++z) {
      a += dKp[(int64_t)z * n4 + i];
      c += dVp[(int64_t)z * n4 + i];
    }
    dK[i] = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
    dV[i] = u32x2{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
  }
}

// ---------------------------------------------------------------- launch
// Waves (32 keys each) per dK/dV workgroup.  At D = 128 and S >= 8192 one
// eight-wave workgroup per CU (256 keys) halves the query-tile loads per
// matrix op and doubles the time each tile's loads have to arrive (1-2%
// faster there); on shorter sequences its workgroups are short and nothing
// covers one's prologue, so two four-wave workgroups per CU are faster.
static int bwd_dkdv_waves(int S, int D) { return D == 128 && S >= 8192 ? 8 : 4; }

// Query-head slices per key/value head for the dK/dV kernel: the smallest
// divisor of the group size that gives about 1024 four-wave workgroups (or
// the same number of waves in eight-wave ones).
int bwd_kv_slices(int B, int S, int Hq, int Hkv, int D) {
  const int G = Hq / Hkv;
  const int waves = bwd_dkdv_waves(S, D);
  const int64_t base = (int64_t)ceil_div(S, 32 * waves) * Hkv * B;
  const int64_t target = 4096 / waves;
  for (int ns = 1; ns < G; ++ns)
    if (G % ns == 0 && base * ns >= target) return ns;
  return G;
}
int bwd_stat_rows(int S) { return ceil_div(S, 64) * 64; }

template <int D>
static hipError_t launch_bwd_d(const void* Q, const void* K, const void* V, const void* dYg,
                               const void* Yg, const float* G, const float* Lse, void* dQ, void* dK,
                               void* dV, void* dY, float* Stat, void* dZ, float* part, int B, int S,
                               int Hq, int Hkv, int mode, hipStream_t st, hipStream_t dq_st, hipEvent_t fork) {
  const float scale = 1.0f / sqrtf((float)D);
  const int Sp = bwd_stat_rows(S);
  const int64_t rows = (int64_t)B * S * Hq;
  const int rpb = 256 / (D / 8);
  const unsigned pblocks = (unsigned)((rows + rpb - 1) / rpb);
  const bf16* dy_attn = (const bf16*)dY;
  if (mode == kBwdGateElem)
    hipLaunchKernelGGL((bwd_prep_kernel<D, kBwdGateElem>), dim3(pblocks), dim3(256), 0, st, (const bf16*)dYg,
                       (const bf16*)Yg, G, Lse, (bf16*)dY, Stat, (bf16*)dZ, B, S, Hq, Sp);
  else if (mode == kBwdGateHead)
    hipLaunchKernelGGL((bwd_prep_kernel<D, kBwdGateHead>), dim3(pblocks), dim3(256), 0, st, (const bf16*)dYg,
                       (const bf16*)Yg, G, Lse, (bf16*)dY, Stat, (bf16*)dZ, B, S, Hq, Sp);
  else {
    hipLaunchKernelGGL((bwd_prep_kernel<D, kBwdGateNone>), dim3(pblocks), dim3(256), 0, st, (const bf16*)dYg,
                       (const bf16*)Yg, G, Lse, (bf16*)dY, Stat, (bf16*)dZ, B, S, Hq, Sp);
    dy_attn = (const bf16*)dYg;   // no gate: the SDPA output's gradient is dY' itself
  }
  // dQ needs only what the prep pass wrote: on a side stream it runs beside dK/dV
  if (dq_st != st) {
    hipError_t e = hipEventRecord(fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(dq_st, fork, 0);
    if (e != hipSuccess) return e;
  }
  const int nq = ceil_div(S, bwd::QT);
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)((int64_t)nq * Hq * B)), dim3(256), 0, dq_st,
                     (const bf16*)Q, (const bf16*)K, (const bf16*)V, dy_attn, (const float*)Stat, (bf16*)dQ,
                     B, S, Hq, Hkv, nq, Sp, scale);
  constexpr bool vlds = D == 128;
  const int waves = bwd_dkdv_waves(S, D);
  const int nk = ceil_div(S, 32 * waves);
  const int ns = bwd_kv_slices(B, S, Hq, Hkv, D);
  const unsigned grid = (unsigned)((int64_t)nk * Hkv * B * ns);
  auto dkdv = [&](auto partial, bf16* dk, bf16* dv, float* dkp, float* dvp) {
    constexpr bool P = decltype(partial)::value;
    if constexpr (vlds) {
      if (waves == 8)
        hipLaunchKernelGGL((bwd_dkdv_vlds_kernel<D, P, 8>), dim3(grid), dim3(512), 0, st, (const bf16*)Q,
                           (const bf16*)K, (const bf16*)V, dy_attn, (const float*)Stat, dk, dv, dkp, dvp, B, S,
                           Hq, Hkv, Sp, ns, scale);
      else
        hipLaunchKernelGGL((bwd_dkdv_vlds_kernel<D, P, 4>), dim3(grid), dim3(256), 0, st, (const bf16*)Q,
                           (const bf16*)K, (const bf16*)V, dy_attn, (const float*)Stat, dk, dv, dkp, dvp, B, S,
                           Hq, Hkv, Sp, ns, scale);
    } else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, P>), dim3(grid), dim3(256), 0, st, (const bf16*)Q,
                         (const bf16*)K, (const bf16*)V, dy_attn, (const float*)Stat, dk, dv, dkp, dvp, B, S,
                         Hq, Hkv, Sp, ns, scale);
  };
  if (ns == 1) {
    dkdv(std::false_type{}, (bf16*)dK, (bf16*)dV, nullptr, nullptr);
  } else {
    const int64_t n = (int64_t)B * S * Hkv * D;
    float* dKp = part;
    float* dVp = part + ns * n;
    dkdv(std::true_type{}, nullptr, nullptr, dKp, dVp);
    const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div<int64_t>(n / 4, 256), 4096);
    hipLaunchKernelGGL(bwd_sum_slices_kernel, dim3(blocks), dim3(256), 0, st, (const f32x4*)dKp,
                       (const f32x4*)dVp, (u32x2*)dK, (u32x2*)dV, n / 4, ns);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const void* Q, const void* K, const void* V, const void* dYg, const void* Yg,
                           const float* G, const float* Lse, void* dQ, void* dK, void* dV, void* dY,
                           float* Stat, void* dZ, float* part, int B, int S, int Hq, int Hkv, int D,
                           int mode, hipStream_t stream, hipStream_t dq_stream, hipEvent_t fork) {
  if (D == 128)
    return launch_bwd_d<128>(Q, K, V, dYg, Yg, G, Lse, dQ, dK, dV, dY, Stat, dZ, part, B, S, Hq, Hkv, mode,
                             stream, dq_stream, fork);
  return launch_bwd_d<64>(Q, K, V, dYg, Yg, G, Lse, dQ, dK, dV, dY, Stat, dZ, part, B, S, Hq, Hkv, mode,
                          stream, dq_stream, fork);
}

}  // namespace gsa
