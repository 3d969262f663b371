// Gate projection with fused activation: G = act(X·W_θ)  (bias-free; act is the
// sigmoid by default, or the identity, NS-sigmoid or SiLU: gate_act in common.h).
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
#include "gate_splitk.h"

namespace gsa {

namespace gemm {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LD = BK + 8;  // LDS row stride in bf16 (144 B: 16-B aligned, rotates banks by 4 per row)
}  // namespace gemm

__global__ __launch_bounds__(256, 2)
void gate_gemm_bf16_kernel(const bf16* __restrict__ X, const bf16* __restrict__ W,
                           float* __restrict__ G, int M, int K, int N, int tiles_n,
                           int act) {
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
          G[m * N + n] = gate_act(z, act);
        }
      }
    }
}


// Large-tile bf16 gate projection: a 256×256 output tile per 512-thread
// workgroup (8 waves as 2 (M) × 4 (N), each 128×64 = 4×2 MFMA 32x32x16 tiles),
// K staged 64 at a time, double-buffered.  X and W tiles move global -> LDS
// with 16-byte direct loads (buffer_load ... lds; lane l of an instruction lands
// in slot base + l), so no registers or VALU work are spent staging them.
//   X tile: 256 rows × 8 chunks + 1 pad slot (144-B row stride); the MFMA A
//           operand (row m, 8 consecutive k) is one 16-B read.
//   W tile: 64 rows (k) × 32 chunks (512 B), chunk index XOR 4*(k & 3); the
//           MFMA B operand (column n, 8 consecutive k) comes from two
//           transposed reads (ds_read_b64_tr_b16), 4 k values each.
// Workgroups are mapped so that each XCD (workgroup id mod 8) owns a
// contiguous range of M tiles: an X row block is fetched into one L2 only.
// Every output is one accumulator over 16-wide MFMA steps in increasing k.
namespace gemm_big {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int XSL = BK / 8 + 1;   // 9 slots per X row
constexpr int WSL = BN / 8;       // 32 slots per W row
constexpr uint32_t kOOB = 0xfffffff0u;  // an offset past any buffer: reads zeros
}  // namespace gemm_big

// Where the fused input projection's output columns go: [0, nq) to Q,
// [nq, nq + nkv) to K, [nq + nkv, nq + 2·nkv) to V (bf16, row-major with those
// widths) and the rest to G (σ, float32).
struct ProjOut {
  bf16* q;
  bf16* k;
  bf16* v;
  int nq, nkv;
};

template <bool ROUTE>
__global__ __launch_bounds__(512, 1)
void gate_gemm_bf16_big_kernel(const bf16* __restrict__ X, const bf16* __restrict__ W,
                               float* __restrict__ G, int M, int K, int N, int tiles_m, int tiles_n,
                               int act, ProjOut po) {
  using namespace gemm_big;
  __shared__ __align__(16) bf16 Xs[2][BM * XSL * 8];
  __shared__ __align__(16) bf16 Ws[2][BK * WSL * 8];
  // landing area of the X load rounds that fall past the 36 instructions of a
  // stage (waves 4..7 issue a fifth, out-of-range load so every wave runs the
  // same branch-free code)
  __shared__ __align__(16) bf16 Xpad[64 * 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int l32 = lane & 31, hl = lane >> 5;

  // tile index: XCD x = bid % 8 takes the x-th contiguous eighth of the
  // row-major tile list when the tile count divides evenly.  When that eighth
  // spans more than 8 column tiles (the fused projection), its tiles go in
  // rounds of 4 row tiles x 8 column tiles (32 workgroups, one per CU of the
  // XCD), so a round reads 4 X row blocks and 8 W column blocks and each W
  // column block passes through the XCD's L2 once.
  const int T = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  int tm, tn;
  if (T % 8 == 0 && tiles_m % 32 == 0 && tiles_n % 8 == 0 && tiles_n > 8) {
    const int tm_per = tiles_m / 8, x = bid % 8, j = bid / 8;
    const int in = j % 8, im = (j / 8) % 4, blk = j / 32, nbn = tiles_n / 8;
    tm = x * tm_per + (blk / nbn) * 4 + im;
    tn = (blk % nbn) * 8 + in;
  } else {
    const int t = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
    tm = t / tiles_n;
    tn = t % tiles_n;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  const auto xr = make_rsrc(X, (uint32_t)((int64_t)M * K * 2));
  const auto wr = make_rsrc(W, (uint32_t)((int64_t)K * N * 2));

  // per-lane DMA offsets (the K-step base is added per stage)
  constexpr int XINS = BM * XSL / 64;          // 36 X instructions per stage
  constexpr int XPW = (XINS + 7) / 8;          // per wave (5; the last round is partial)
  uint32_t x_off[XPW];
  int x_kc[XPW];
#pragma unroll
  for (int j = 0; j < XPW; ++j) {
    const int sl = (wave + 8 * j) * 64 + lane;
    const int row = sl / XSL, c = sl % XSL;
    x_kc[j] = c < 8 ? c * 8 : 1 << 30;       // k offset of this chunk within the stage
    x_off[j] = (uint32_t)(m0 + row) * (uint32_t)K * 2 + (uint32_t)(c * 16);
  }
  constexpr int WINS = BK * WSL / 64;          // 32 W instructions per stage
  uint32_t w_off[WINS / 8];
#pragma unroll
  for (int j = 0; j < WINS / 8; ++j) {
    const int sl = (wave + 8 * j) * 64 + lane;
    const int row = sl / WSL, p = sl % WSL;
    const int c = p ^ (4 * (row & 3));
    w_off[j] = (uint32_t)row * (uint32_t)N * 2 + (uint32_t)(n0 + 8 * c) * 2;
  }
  // the load rounds of stage (k0, buf); a stage past the end of K (k0 >= K)
  // loads nothing: every offset is out of range and the rounds write zeros
  const uint32_t xpad = __builtin_amdgcn_readfirstlane(lds_addr(&Xpad[0]));
  auto dma = [&](int k0, int buf) {
    const uint32_t xd = __builtin_amdgcn_readfirstlane(lds_addr(&Xs[buf][0]));
    const uint32_t wd = __builtin_amdgcn_readfirstlane(lds_addr(&Ws[buf][0]));
#pragma unroll
    for (int j = 0; j < XPW; ++j) {
      const int ins = wave + 8 * j;
      const bool real = ins < XINS;
      const uint32_t off = (real && k0 + x_kc[j] < K) ? x_off[j] + (uint32_t)k0 * 2 : kOOB;
      dma16_lds(xr, off, real ? xd + ins * 64 * 16 : xpad);
    }
    const bool live = k0 < K;
#pragma unroll
    for (int j = 0; j < WINS / 8; ++j) {
      const int ins = wave + 8 * j;
      dma16_lds(wr, live ? w_off[j] + (uint32_t)k0 * (uint32_t)N * 2 : kOOB, wd + ins * 64 * 16);
    }
  };

  // operand addresses
  const int xa = ((wm * 128 + l32) * XSL + hl) * 8;
  const int g = lane >> 4, si = lane & 15;
  // B: supplier lane (g, si) names k row 8*(g/2) + si/4 (+4a +16kk) and columns
  // wn*64 + nt*32 + 16*(g%2) + 4*(si%4) .. +3
  uint32_t wb[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = wn * 64 + nt * 32 + 16 * (g & 1) + 4 * (si & 3);
    const int krow = 8 * (g >> 1) + (si >> 2);
    const int phys = (n >> 3) ^ (4 * (krow & 3));
    wb[nt] = (uint32_t)((krow * WSL + phys) * 16 + (n & 7) * 2);
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // MFMA operands of one 16-wide k step: 4 X fragments (A) and 2 W fragments (B)
  struct Frag {
    bf16x8 a[4], b[2];
  };
  auto load_frag = [&](int buf, int kk, Frag& f) {
    const bf16* xs = &Xs[buf][0];
    GSA_LDS char* const wl = (GSA_LDS char*)(GSA_LDS void*)&Ws[buf][0];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) f.a[mt] = *(const bf16x8*)(xs + xa + (mt * 32 * XSL + 2 * kk) * 8);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      GSA_LDS char* const ad = wl + wb[nt] + 16 * kk * WSL * 16;
      f.b[nt].lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS i16x4*)ad));
      f.b[nt].hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS i16x4*)(ad + 4 * WSL * 16)));
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32x32x16(f.a[mt], f.b[nt], acc[mt][nt]);
  };

  // Pipeline: the fragments of k step kk+1 are read while the matrix ops of kk
  // run.  Stage kt+1 is waited for (and every wave is past its reads of stage
  // kt) at a barrier placed before the last k step of stage kt, so the reads of
  // stage kt+1's first k step overlap that step's matrix ops; the direct loads
  // of stage kt+2 then refill the buffer of stage kt.
  const int nk = (K + BK - 1) / BK;
  static_assert(BK / 16 == 4, "four k steps per stage");
  dma(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (nk > 1) dma(BK, 1);
  Frag f0, f1;
  load_frag(0, 0, f0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    load_frag(buf, 1, f1);
    mma(f0);
    load_frag(buf, 2, f0);
    mma(f1);
    load_frag(buf, 3, f1);
    mma(f0);
    // each matrix op takes one of the next step's fragment reads along
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    dma((kt + 2) * BK, buf);          // past the end: out-of-range rounds
    load_frag(buf ^ 1, 0, f0);        // on the last stage: stale, unused
    mma(f1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
  }

  // epilogue: lane holds column l32 of each 32x32 block, rows 8*(r/4) + 4*hl + r%4
  const bool full = (m0 + BM <= M) && (n0 + BN <= N);
  if constexpr (!ROUTE) {
    // one copy of the store loops per activation: no activation switch per element
    auto store_all = [&](auto act_c) {
      constexpr int A = decltype(act_c)::value;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int n = n0 + wn * 64 + nt * 32 + l32;
          const int mb = m0 + wm * 128 + mt * 32 + 4 * hl;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = mb + 8 * (r >> 2) + (r & 3);
            const float v = gate_act(acc[mt][nt][r], A);
            if (full || (m < M && n < N)) G[(int64_t)m * N + n] = v;
          }
        }
    };
    if (act == kActSigmoid) store_all(std::integral_constant<int, kActSigmoid>{});
    else if (act == kActNsSigmoid) store_all(std::integral_constant<int, kActNsSigmoid>{});
    else if (act == kActSilu) store_all(std::integral_constant<int, kActSilu>{});
    else store_all(std::integral_constant<int, kActIdentity>{});
  } else {
    const int ng = N - po.nq - 2 * po.nkv;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int n = n0 + wn * 64 + nt * 32 + l32;
      // this lane's column: destination, its row width and the column within it
      bf16* dst = po.q;
      int ld = po.nq, col = n;
      if (n >= po.nq + 2 * po.nkv) {
        dst = nullptr;
        ld = ng;
        col = n - po.nq - 2 * po.nkv;
      } else if (n >= po.nq + po.nkv) {
        dst = po.v;
        ld = po.nkv;
        col = n - po.nq - po.nkv;
      } else if (n >= po.nq) {
        dst = po.k;
        ld = po.nkv;
        col = n - po.nq;
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int mb = m0 + wm * 128 + mt * 32 + 4 * hl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mb + 8 * (r >> 2) + (r & 3);
          const float z = acc[mt][nt][r];
          if (full || (m < M && n < N)) {
            if (dst != nullptr) dst[(int64_t)m * ld + col] = (bf16)z;
            else G[(int64_t)m * ld + col] = sigmoidf(z);
          }
        }
      }
    }
  }
}

// Narrow / short bf16 gate projection for shapes with few rows (decode: one
// token per batch) or few columns (headwise gate: one per head).  Each
// 4-wave workgroup owns one 32×32 output tile; wave w sums the w-th quarter of
// K, streaming it through its own 4-stage ring of LDS buffers filled by
// 16-byte direct loads (3 stages, 24 KB, in flight per wave).  No barrier is
// needed inside the ring: a wave only reads what its own loads wrote, after
// waiting on them.  At the end the four partial sums are added through LDS in
// wave order and wave 0 applies σ and stores.
//   X stage: 32 rows × 8 chunks (k 64), chunk index XOR (row & 7); the A
//            operand is one 16-B read.
//   W stage: 64 rows (k) × 4 chunks (32 columns, 64 B), unswizzled (eight
//            consecutive rows are 512 contiguous bytes); the B operand comes
//            from two transposed reads.
namespace gemm_narrow {
constexpr int BK = 64, NS = 4, WAVES = 4;
constexpr int XSLOTS = 32 * 8, WSLOTS = 64 * 4;     // 16-B slots per stage
constexpr uint32_t kOOB = 0xfffffff0u;
}  // namespace gemm_narrow

__global__ __launch_bounds__(256)
void gate_gemm_bf16_narrow_kernel(const bf16* __restrict__ X, const bf16* __restrict__ W,
                                  float* __restrict__ G, int M, int K, int N, int tiles_n,
                                  int act, int w_major) {
  using namespace gemm_narrow;
  __shared__ __align__(16) bf16 Xs[WAVES][NS][XSLOTS * 8];
  __shared__ __align__(16) bf16 Ws[WAVES][NS][WSLOTS * 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  // Tile order: workgroup ids go round-robin over the 8 XCDs, and XCD x takes
  // the x-th contiguous eighth of the tile list (when the count allows), so
  // tiles next to each other in the list share an L2.  With w_major the list
  // runs over row tiles first (tiles of one column block, which read the same
  // W_θ columns, are adjacent: for few rows W_θ is the large operand); else
  // over column tiles first (tiles of one row block share their X rows).
  const int tiles = (int)gridDim.x, bid = blockIdx.x;
  const int t = tiles % 8 == 0 ? (bid % 8) * (tiles / 8) + bid / 8 : bid;
  const int tiles_m = tiles / tiles_n;
  const int tm = w_major ? t % tiles_m : t / tiles_n;
  const int tn = w_major ? t / tiles_m : t % tiles_n;
  const int m0 = tm * 32, n0 = tn * 32;

  // this wave's k range: a whole number of BK steps
  const int nk_all = (K + BK - 1) / BK;
  const int nk_w = (nk_all + WAVES - 1) / WAVES;
  const int kt0 = wave * nk_w;
  const int nk = max(0, min(nk_all, kt0 + nk_w) - kt0);

  const auto xr = make_rsrc(X, (uint32_t)((int64_t)M * K * 2));
  const auto wr = make_rsrc(W, (uint32_t)((int64_t)K * N * 2));
  // DMA slots: X instruction i covers rows 8i .. 8i+7; W instruction i rows 16i .. 16i+15
  uint32_t x_off[4], w_off[4];
  int x_k[4], w_n[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sl = i * 64 + lane;
    const int row = sl >> 3, p = sl & 7;
    const int c = p ^ (row & 7);
    x_k[i] = c * 8;
    x_off[i] = (uint32_t)(m0 + row) * (uint32_t)K * 2 + (uint32_t)(c * 16);
    const int krow = sl >> 2, wc = sl & 3;
    w_n[i] = n0 + wc * 8;
    w_off[i] = (uint32_t)krow * (uint32_t)N * 2 + (uint32_t)(n0 + wc * 8) * 2;
  }
  const bool n_ok = (N % 8) == 0;
  auto dma = [&](int k0, int st) {
    const uint32_t xd = __builtin_amdgcn_readfirstlane(lds_addr(&Xs[wave][st][0]));
    const uint32_t wd = __builtin_amdgcn_readfirstlane(lds_addr(&Ws[wave][st][0]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (k0 + x_k[i] < K) ? x_off[i] + (uint32_t)k0 * 2 : kOOB;
      dma16_lds(xr, off, xd + i * 64 * 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = (n_ok && w_n[i] < N) ? w_off[i] + (uint32_t)k0 * (uint32_t)N * 2 : kOOB;
      dma16_lds(wr, off, wd + i * 64 * 16);
    }
  };

  // A operand: row l32, chunk 2*kk + hl, stored at chunk ^ (l32 & 7)
  const uint32_t xs0 = (uint32_t)(uintptr_t)(GSA_LDS void*)&Xs[wave][0][0];
  const uint32_t ws0 = (uint32_t)(uintptr_t)(GSA_LDS void*)&Ws[wave][0][0];
  // B operand: supplier lane (g, si) names k row 8*(g/2) + si/4 (+4a +16kk) and
  // columns 16*(g%2) + 4*(si%4) .. +3 of the 32-column stage
  const int g = lane >> 4, si = lane & 15;
  const uint32_t wb = ws0 + (uint32_t)(((8 * (g >> 1) + (si >> 2)) * 4) * 16 + (16 * (g & 1) + 4 * (si & 3)) * 2);

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // prologue: stages 0 .. NS-2 of this wave's range in flight
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
      const int c = 2 * kk + hl;
      const bf16x8 a = *(const bf16x8*)(GSA_LDS bf16x8*)(uintptr_t)(xs0 + st * (XSLOTS * 16) +
                                                                    (l32 * 8 + (c ^ (l32 & 7))) * 16);
      const uint32_t ad = wb + st * (WSLOTS * 16) + 16 * kk * 4 * 16;
      bf16x8 b;
      b.lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS i16x4*)(uintptr_t)ad));
      b.hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS i16x4*)(uintptr_t)(ad + 4 * 4 * 16)));
      acc = mfma32x32x16(a, b, acc);
    }
  }

  // add the four partial sums in wave order through LDS (the X ring of waves
  // 1..3 is reused once every wave is past its last read)
  __syncthreads();
  float* const red = (float*)&Xs[0][0][0];   // [3][16][64] floats = 12 KB
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wave - 1) * 16 + r) * 64 + lane] = acc[r];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < WAVES - 1; ++w)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += red[(w * 16 + r) * 64 + lane];
  const int n = n0 + l32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 8 * (r >> 2) + 4 * hl + (r & 3);
    if (m < M && n < N) G[(int64_t)m * N + n] = gate_act(acc[r], act);
  }
}

__global__ __launch_bounds__(256)
void gate_gemm_bf16_splitk_kernel(const bf16* __restrict__ X, const bf16* __restrict__ W,
                                  float* __restrict__ part, int M, int K, int N, int tiles_n,
                                  int splits, int nk_split) {
  using namespace gemm_splitk;
  __shared__ __align__(16) bf16 Xs[WAVES][NS][XSLOTS * 8];
  __shared__ __align__(16) bf16 Ws[WAVES][NS][WSLOTS * 8];
  gate_splitk_body(&Xs[0][0][0], &Ws[0][0][0], X, W, part, M, K, N, tiles_n, splits, nk_split, blockIdx.x);
}

// G = act(Σ_{s < splits} part[s]) in split order, 4 values per thread.
__global__ __launch_bounds__(256)
void gate_splitk_sum_kernel(const float* __restrict__ part, float* __restrict__ G, int64_t n4, int64_t stride4,
                            int splits, int act) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 v = ((const f32x4*)part)[i];
  for (int s = 1; s < splits; ++s) {
    const f32x4 u = ((const f32x4*)part)[s * stride4 + i];
    v[0] += u[0];
    v[1] += u[1];
    v[2] += u[2];
    v[3] += u[3];
  }
  f32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = gate_act(v[j], act);
  ((f32x4*)G)[i] = o;
}

// Split count and workspace of the split-K path; 0 splits = not used.
int64_t gate_splitk_splits(int64_t M, int64_t K, int64_t N) {
  using namespace gemm_splitk;
  if (M > 2 * BM || N < BN || N % 8 != 0 || K < 4 * WAVES * BK) return 0;
  if (M * K * 2 >= ((int64_t)1 << 31) || K * N * 2 >= ((int64_t)1 << 31)) return 0;   // 32-bit offsets
  const int64_t tiles = ceil_div<int64_t>(M, BM) * ceil_div<int64_t>(N, BN);
  if (tiles >= 256) return 0;                    // enough tiles already: the narrow kernel's ground
  const int64_t nk_all = ceil_div<int64_t>(K, BK);
  // about one workgroup per CU, at least 4 k steps per wave
  int64_t s = ceil_div<int64_t>(256, tiles);
  s = std::min<int64_t>(s, nk_all / (4 * WAVES));
  return std::max<int64_t>(s, 1);
}
size_t gate_splitk_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  const int64_t s = gate_splitk_splits(M, K, N);
  return s > 0 ? (size_t)(s * M * N) * sizeof(float) : 0;
}

// The split-K partial logits alone ([s, M, N] float32 into part), for a
// consumer that adds them itself (the decode merge).
hipError_t launch_gate_gemm_splitk_parts(const void* X, const void* W, float* part, int64_t M, int64_t K, int64_t N,
                                         hipStream_t stream) {
  using namespace gemm_splitk;
  const int64_t s = gate_splitk_splits(M, K, N);
  const int tiles_n = (int)ceil_div<int64_t>(N, BN);
  const int64_t tiles = ceil_div<int64_t>(M, BM) * tiles_n;
  const int64_t nk_all = ceil_div<int64_t>(K, BK);
  const int nk_split = (int)ceil_div<int64_t>(nk_all, s);
  hipLaunchKernelGGL(gate_gemm_bf16_splitk_kernel, dim3((unsigned)(tiles * s)), dim3(256), 0, stream,
                     (const bf16*)X, (const bf16*)W, part, (int)M, (int)K, (int)N, tiles_n, (int)s, nk_split);
  return hipGetLastError();
}

hipError_t launch_gate_gemm_splitk(const void* X, const void* W, float* G, float* part, int64_t M, int64_t K,
                                   int64_t N, int act, hipStream_t stream) {
  const int64_t s = gate_splitk_splits(M, K, N);
  if (hipError_t e = launch_gate_gemm_splitk_parts(X, W, part, M, K, N, stream); e != hipSuccess) return e;
  const int64_t n4 = M * N / 4;
  hipLaunchKernelGGL(gate_splitk_sum_kernel, dim3((unsigned)ceil_div<int64_t>(n4, 256)), dim3(256), 0, stream,
                     (const float*)part, G, n4, n4, (int)s, act);
  return hipGetLastError();
}

// float32 gate projection: 64×64 tile per 256 threads, 4×4 outputs per thread.
__global__ __launch_bounds__(256)
void gate_gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                          float* __restrict__ G, int M, int K, int N, int tiles_n,
                          int act) {
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
      if (m < M && n < N) G[m * N + n] = gate_act(acc[i][j], act);
    }
}

hipError_t launch_gate_gemm(const void* X, const void* W, float* G, int64_t M, int64_t K, int64_t N,
                            bool bf16_inputs, int act, hipStream_t stream) {
  if (bf16_inputs && M >= 256 && N >= 256 && N % 8 == 0 && M * K * 2 < (int64_t(1) << 31) &&
      K * N * 2 < (int64_t(1) << 31)) {
    const int tiles_n = (int)ceil_div<int64_t>(N, gemm_big::BN);
    const int tiles_m = (int)ceil_div<int64_t>(M, gemm_big::BM);
    hipLaunchKernelGGL(gate_gemm_bf16_big_kernel<false>, dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, stream,
                       (const bf16*)X, (const bf16*)W, G, (int)M, (int)K, (int)N, tiles_m, tiles_n,
                       act, ProjOut{nullptr, nullptr, nullptr, 0, 0});
  } else if (bf16_inputs && N % 8 == 0 && M * K * 2 < (int64_t(1) << 31) && K * N * 2 < (int64_t(1) << 31)) {
    const int tiles_n = (int)ceil_div<int64_t>(N, 32);
    const int64_t tiles = ceil_div<int64_t>(M, 32) * tiles_n;
    // the larger operand is shared within an XCD: W_θ (K·N) when it exceeds X (M·K)
    const int w_major = N > M ? 1 : 0;
    hipLaunchKernelGGL(gate_gemm_bf16_narrow_kernel, dim3((unsigned)tiles), dim3(256), 0, stream,
                       (const bf16*)X, (const bf16*)W, G, (int)M, (int)K, (int)N, tiles_n,
                       act, w_major);
  } else if (bf16_inputs) {
    const int tiles_n = (int)ceil_div<int64_t>(N, gemm::BN);
    const int64_t tiles = ceil_div<int64_t>(M, gemm::BM) * tiles_n;
    hipLaunchKernelGGL(gate_gemm_bf16_kernel, dim3((unsigned)tiles), dim3(256), 0, stream,
                       (const bf16*)X, (const bf16*)W, G, (int)M, (int)K, (int)N, tiles_n,
                       act);
  } else {
    const int tiles_n = (int)ceil_div<int64_t>(N, 64);
    const int64_t tiles = ceil_div<int64_t>(M, 64) * tiles_n;
    hipLaunchKernelGGL(gate_gemm_f32_kernel, dim3((unsigned)tiles), dim3(256), 0, stream,
                       (const float*)X, (const float*)W, G, (int)M, (int)K, (int)N, tiles_n,
                       act);
  }
  return hipGetLastError();
}

// Fused input projection: [Q | K | V | Z] = X · [W_Q | W_K | W_V | W_θ] in one
// pass over X ("GatedAttention [2025]" §1.2.1 QKV projections and §1.2.2 gate
// scores), Q/K/V rounded to bf16, G = σ(Z) in float32.  W is [K, N] with
// N = nq + 2·nkv + ng; the large-tile kernel with the routing epilogue.
hipError_t launch_project_qkvg(const void* X, const void* W, void* Q, void* Kp, void* V, float* G, int64_t M,
                               int64_t K, int64_t nq, int64_t nkv, int64_t ng, hipStream_t stream) {
  const int64_t N = nq + 2 * nkv + ng;
  const int tiles_n = (int)ceil_div<int64_t>(N, gemm_big::BN);
  const int tiles_m = (int)ceil_div<int64_t>(M, gemm_big::BM);
  hipLaunchKernelGGL(gate_gemm_bf16_big_kernel<true>, dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, stream,
                     (const bf16*)X, (const bf16*)W, G, (int)M, (int)K, (int)N, tiles_m, tiles_n, 1,
                     ProjOut{(bf16*)Q, (bf16*)Kp, (bf16*)V, (int)nq, (int)nkv});
  return hipGetLastError();
}

}  // namespace gsa
