// Split-K gate projection for few token rows (the decode gate), used by the
// gate GEMM kernels (gate_gemm.hip).
#pragma once

#include "common.h"


namespace gsa {

// Split-K gate projection for few rows (decode: one token per batch, M <= 128):
// the W_θ stream is the whole cost (33.5 MB at d_model = N = 4096 against a
// 512 KB X), so the design aims at W_θ read once at full HBM speed with as
// little on-chip traffic per byte of it as possible.
//   * Output tiles are 64 rows × 64 columns: every tile re-reads its X rows
//     through L2, and a 64-wide tile halves that (X 32 MB + W_θ 33.5 MB over
//     the chip at M = 64, N = 4096, against 64 + 67 MB with 32×32 tiles).
//   * K is split s ways (s = 4 at that shape: 64 column tiles × 4 = 256
//     workgroups, one per CU), each workgroup's 4 waves taking a quarter of
//     its K range through their own 4-stage LDS rings of 16-byte direct loads
//     (3 stages, 24 KB, in flight per wave; no barrier inside the ring).
//   * The 4 waves' sums are added in wave order through LDS; the s partial
//     tiles go to a float32 workspace, and a second kernel adds them in split
//     order and applies the activation: fixed-order sums, so the result is
//     deterministic (no atomics), with σ taken of the complete logit.
//   X stage: 64 rows × 4 chunks (k 32, 64-byte rows), chunk c of row r in
//            slot c ^ ((r >> 2) & 3): the 16 rows of a row read land on 16
//            distinct bank groups.
//   W stage: 32 k rows × 8 chunks (64 columns, 128-byte rows), chunk c of
//            k row r in slot c ^ (4·((r >> 1) & 1)): the 16 (row, chunk)
//            pairs of a 32-lane transposed read land on distinct bank groups.
namespace gemm_splitk {
constexpr int BM = 64, BN = 64, BK = 32, NS = 4, WAVES = 4;
constexpr int XSLOTS = BM * BK / 8, WSLOTS = BK * BN / 8;   // 16-B slots per stage (256 each)
constexpr uint32_t kOOB = 0xfffffff0u;
__host__ __device__ constexpr int x_slot(int row, int c) { return row * (BK / 8) + (c ^ ((row >> 2) & 3)); }
__host__ __device__ constexpr int w_slot(int krow, int c) { return krow * (BN / 8) + (c ^ (4 * ((krow >> 1) & 1))); }
}  // namespace gemm_splitk

// The workgroup `bid` of the split-K gate on two 64 KB LDS areas, Xs (the
// X rings: [WAVES][NS][XSLOTS·8] bf16) and Ws (the W rings, same shape).
__device__ __forceinline__ void gate_splitk_body(bf16* __restrict__ xs_lds, bf16* __restrict__ ws_lds,
                                                 const bf16* __restrict__ X, const bf16* __restrict__ W,
                                                 float* __restrict__ part, int M, int K, int N, int tiles_n,
                                                 int splits, int nk_split, int bid) {
  using namespace gemm_splitk;
  bf16(*Xs)[NS][XSLOTS * 8] = (bf16(*)[NS][XSLOTS * 8])xs_lds;
  bf16(*Ws)[NS][WSLOTS * 8] = (bf16(*)[NS][WSLOTS * 8])ws_lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  // workgroup -> (output tile, split); the splits of one tile are adjacent ids
  const int ks = bid % splits, tile = bid / splits;
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
  // this wave's k steps: a quarter of the split's range
  const int nk_all = (K + BK - 1) / BK;
  const int s0 = ks * nk_split;
  const int nk_s = max(0, min(nk_all, s0 + nk_split) - s0);
  const int nk_w = (nk_s + WAVES - 1) / WAVES;
  const int kt0 = s0 + wave * nk_w;
  const int nk = max(0, min(s0 + nk_s, kt0 + nk_w) - kt0);

  const auto xr = make_rsrc(X, (uint32_t)((int64_t)M * K * 2));   // rows >= M read zeros
  const auto wr = make_rsrc(W, (uint32_t)((int64_t)K * N * 2));   // k rows >= K read zeros
  // DMA slots: instruction i covers X rows 16i .. 16i+15 and W k rows 8i .. 8i+7
  uint32_t x_off[4], w_off[4];
  int x_k[4], w_n[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sl = i * 64 + lane;
    const int row = sl >> 2, c = (sl & 3) ^ ((row >> 2) & 3);
    x_k[i] = c * 8;
    x_off[i] = (uint32_t)(m0 + row) * (uint32_t)K * 2 + (uint32_t)(c * 16);
    const int krow = sl >> 3, wc = (sl & 7) ^ (4 * ((krow >> 1) & 1));
    w_n[i] = n0 + wc * 8;
    w_off[i] = (uint32_t)krow * (uint32_t)N * 2 + (uint32_t)(n0 + wc * 8) * 2;
  }
  auto dma = [&](int k0, int st) {
    const uint32_t xd = __builtin_amdgcn_readfirstlane(lds_addr(&Xs[wave][st][0]));
    const uint32_t wd = __builtin_amdgcn_readfirstlane(lds_addr(&Ws[wave][st][0]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // a chunk past the end of its row would read the next row: out of range instead
      const uint32_t off = (k0 + x_k[i] < K) ? x_off[i] + (uint32_t)k0 * 2 : kOOB;
      dma16_lds(xr, off, xd + i * 64 * 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (w_n[i] < N) ? w_off[i] + (uint32_t)k0 * (uint32_t)N * 2 : kOOB;
      dma16_lds(wr, off, wd + i * 64 * 16);
    }
  };

  // A operand (X rows): row rb*32 + l32, chunk 2*kk + hl
  const uint32_t xs0 = (uint32_t)(uintptr_t)(GSA_LDS void*)&Xs[wave][0][0];
  const uint32_t ws0 = (uint32_t)(uintptr_t)(GSA_LDS void*)&Ws[wave][0][0];
  uint32_t xa[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) xa[rb][kk] = xs0 + x_slot(rb * 32 + l32, 2 * kk + hl) * 16;
  // B operand: supplier lane (g, si) names k row 8*(g/2) + si/4 (+4 for the
  // second read, +16 for the second k step) and columns nb*32 + 16*(g%2) +
  // 4*(si%4) .. +3; adding 4 or 16 k rows keeps the swizzle
  const int g = lane >> 4, si = lane & 15;
  uint32_t wb[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int krow = 8 * (g >> 1) + (si >> 2);
    const int col = nb * 32 + 16 * (g & 1) + 4 * (si & 3);
    wb[nb] = ws0 + (uint32_t)(w_slot(krow, col >> 3) * 16 + (col & 7) * 2);
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][nb][r] = 0.f;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) dma((kt0 + st) * BK, st);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % NS;
    if (kt + NS - 1 < nk) {
      dma((kt0 + kt + NS - 1) * BK, (kt + NS - 1) % NS);
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(8 * (NS - 1)) : "memory");   // the NS-1 newer stages (8 loads each) may still fly
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        a[rb] = *(const bf16x8*)(GSA_LDS bf16x8*)(uintptr_t)(xa[rb][kk] + st * (XSLOTS * 16));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const uint32_t ad = wb[nb] + st * (WSLOTS * 16) + 16 * kk * (BN / 8) * 16;
        b[nb].lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS i16x4*)(uintptr_t)ad));
        b[nb].hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                  (GSA_LDS i16x4*)(uintptr_t)(ad + 4 * (BN / 8) * 16)));
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[rb][nb] = mfma32x32x16(a[rb], b[nb], acc[rb][nb]);
    }
  }

  // the 4 waves' 64×64 sums added in wave order through LDS (the rings are
  // free once every wave is past its last read): wave w writes its tile into
  // red[w], then thread t adds row t/4, columns 16·(t%4) .. +15 over w = 0..3
  __syncthreads();
  float* const red = (float*)&Xs[0][0][0];   // [4][64][64] floats = 64 KB (the X and W rings hold 128 KB)
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        red[(wave * BM + row) * BN + nb * 32 + l32] = acc[rb][nb][r];
      }
  __syncthreads();
  const int row = tid >> 2, c0 = 16 * (tid & 3);
  if (m0 + row >= M) return;
  float* const dst = part + ((int64_t)ks * M + m0 + row) * N + n0 + c0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 v = *(const f32x4*)&red[row * BN + c0 + 4 * q];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      const f32x4 u = *(const f32x4*)&red[(w * BM + row) * BN + c0 + 4 * q];
      v[0] += u[0];
      v[1] += u[1];
      v[2] += u[2];
      v[3] += u[3];
    }
    if (n0 + c0 + 4 * q < N) *(f32x4*)(dst + 4 * q) = v;   // N % 8 == 0: whole 4-column pieces
  }
}

}  // namespace gsa
