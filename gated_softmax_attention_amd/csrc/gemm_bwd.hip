// Gate-branch products of the backward (bf16 operands, fp32 accumulation):
//   dX   = dZ · W_θᵀ     [M, d_model]  (bf16 out)
//   dW_θ = Xᵀ · dZ       [d_model, N]  (fp32 out)
// for the gate-score gradient dZ [M, N] (the "Gated Attention如何用1%的参数量…"
// page, §2.2 gradient analysis: the gate input's gradient times the projection's
// transposes).  X is [M, d_model] and W_θ is [d_model, N], both row-major.
//
// One kernel serves both: out[m][n] = Σ_k L[m][k] · R[k][n] where each operand
// is either k-contiguous in memory or m/n-contiguous.  dX has both operands
// k-contiguous (dZ rows, W_θ rows); dW_θ has both m/n-contiguous (X and dZ read
// down their token columns).  Tiles of 128 (m) x 128 (n) x 64 (k), 4 waves in a
// 2x2 grid of 64x64, double-buffered in LDS by 16-byte direct loads.  A
// k-contiguous operand is staged as [m|n][k] and read row-wise (8 consecutive
// k per lane); an m/n-contiguous one as [k][m|n] and read with transposed LDS
// reads, which hand each lane 4 consecutive k of one column.  Padding keeps
// both read kinds free of bank conflicts.  The MFMA's row index is n, so each
// lane ends with 4 consecutive output columns (one vector store).
//
// dW_θ sums over all M tokens; when its output tiles alone cannot fill the chip
// the token range is cut into equal chunks whose partial sums go to a
// workspace and are added in chunk order by a second kernel (deterministic).
#include "common.h"

namespace gsa {

#define GSA_LDS_G __attribute__((address_space(3)))

namespace bgemm {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr uint32_t kOOB = 0xfffffff0u;

// Staged operand tile.  KC: 128 rows (m or n) of 64 k, 9 slots of 16 B per row
// (one pad slot).  MC: 64 rows (k) of 128 m/n, 20 slots per row (4 pad slots:
// a 320-byte stride puts the four rows of a transposed read 16 banks apart).
template <bool KC>
struct Stage {
  static constexpr int ROWS = KC ? 128 : 64;
  static constexpr int CH = KC ? 8 : 16;
  static constexpr int SL = KC ? 9 : 20;
  static constexpr int RSB = SL * 16;
  static constexpr int SLOTS = ROWS * SL;
  static constexpr int NI = (SLOTS + 255) / 256;   // direct-load instructions per wave
  static constexpr int BYTES = SLOTS * 16;
};

template <bool KC>
struct Loader {
  using St = Stage<KC>;
  int row[St::NI], ch[St::NI];   // ch < 0: pad slot or no slot
  __device__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < St::NI; ++j) {
      const int sl = (wave + 4 * j) * 64 + lane;
      row[j] = sl / St::SL;
      const int c = sl % St::SL;
      ch[j] = (sl < St::SLOTS && c < St::CH) ? c : -1;
    }
  }
  // Tile at (mn0, k0) of an operand with leading dimension ld (elements),
  // valid m/n indices < mn_end and k indices < k_end; the rest reads zeros.
  __device__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t lds, int mn0, int mn_end, int k0, int k_end,
                       uint32_t ld, int wave) const {
#pragma unroll
    for (int j = 0; j < St::NI; ++j) {
      const int ins = wave + 4 * j;
      if (ins * 64 < St::SLOTS) {
        bool ok;
        uint32_t off;
        if constexpr (KC) {
          const int mn = mn0 + row[j], k = k0 + 8 * ch[j];
          ok = ch[j] >= 0 && mn < mn_end && k < k_end;
          off = ((uint32_t)mn * ld + (uint32_t)k) * 2u;
        } else {
          const int k = k0 + row[j], mn = mn0 + 8 * ch[j];
          ok = ch[j] >= 0 && k < k_end && mn < mn_end;
          off = ((uint32_t)k * ld + (uint32_t)mn) * 2u;
        }
        dma16_lds(rs, ok ? off : kOOB, lds + (uint32_t)ins * 1024u);
      }
    }
  }
};

// MFMA operand (32 m/n values at col0 + l32, k = 16*ks + 8*hl .. +7) from a tile.
template <bool KC>
__device__ __forceinline__ bf16x8 frag(const GSA_LDS_G char* tile, int col0, int ks, int lane_off) {
  if constexpr (KC) {
    return *(const GSA_LDS_G bf16x8*)(tile + col0 * Stage<true>::RSB + ks * 32 + lane_off);
  } else {
    const GSA_LDS_G char* p = tile + ks * 16 * Stage<false>::RSB + col0 * 2 + lane_off;
    const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS_G i16x4*)p);
    const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS_G i16x4*)(p + 4 * Stage<false>::RSB));
    bf16x8 a;
    a.lo = __builtin_bit_cast(bf16x4, lo);
    a.hi = __builtin_bit_cast(bf16x4, hi);
    return a;
  }
}

// Lane part of a fragment address.  KC: row l32, chunk hl.  MC: in each 16-lane
// group g, lane i names k row 8*(g/2) + i/4 and columns 16*(g%2) + 4*(i%4) .. +3,
// and receives column 16*(g%2) + i at the four k rows 8*(g/2) + 0..3 (and, from
// the second read 4 rows down, + 4..7): MFMA row l32, k slots 8*hl + 0..7.
template <bool KC>
__device__ __forceinline__ int frag_lane_off(int lane) {
  if constexpr (KC) {
    return (lane & 31) * Stage<true>::RSB + (lane >> 5) * 16;
  } else {
    const int g = lane >> 4, i = lane & 15;
    return (8 * (g >> 1) + (i >> 2)) * Stage<false>::RSB + (16 * (g & 1) + 4 * (i & 3)) * 2;
  }
}
}  // namespace bgemm

template <typename OutT, bool L_KC, bool R_KC>
__global__ __launch_bounds__(256, 2)
void bwd_gemm_kernel(const bf16* __restrict__ L, const bf16* __restrict__ R, OutT* __restrict__ out,
                     int M, int N, int K, uint32_t ldl, uint32_t ldr, uint32_t l_bytes, uint32_t r_bytes,
                     int tiles_m, int tiles_n, int k_chunk) {
  using namespace bgemm;
  __shared__ __align__(16) char Ls[2][Stage<L_KC>::BYTES];
  __shared__ __align__(16) char Rs[2][Stage<R_KC>::BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int hl = lane >> 5, l32 = lane & 31;
  const int tiles = tiles_m * tiles_n;
  const int z = blockIdx.x / tiles, t = blockIdx.x % tiles;
  const int tm = t / tiles_n, tn = t % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb = z * k_chunk, ke = min(K, kb + k_chunk);
  OutT* outz = out + (int64_t)z * M * N;

  const auto lrs = make_rsrc(L, l_bytes);
  const auto rrs = make_rsrc(R, r_bytes);
  Loader<L_KC> lld;
  Loader<R_KC> rld;
  lld.init(wave, lane);
  rld.init(wave, lane);
  uint32_t l_lds[2], r_lds[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    l_lds[i] = __builtin_amdgcn_readfirstlane(lds_addr(&Ls[i][0]));
    r_lds[i] = __builtin_amdgcn_readfirstlane(lds_addr(&Rs[i][0]));
  }
  const int l_off = frag_lane_off<L_KC>(lane), r_off = frag_lane_off<R_KC>(lane);

  f32x16 acc[2][2];   // [n block][m block]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = ke > kb ? ceil_div(ke - kb, BK) : 0;
  if (nk > 0) {
    lld.load(lrs, l_lds[0], m0, M, kb, ke, ldl, wave);
    rld.load(rrs, r_lds[0], n0, N, kb, ke, ldr, wave);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) {
      const int k0 = kb + (kt + 1) * BK;
      lld.load(lrs, l_lds[buf ^ 1], m0, M, k0, ke, ldl, wave);
      rld.load(rrs, r_lds[buf ^ 1], n0, N, k0, ke, ldr, wave);
    }
    const GSA_LDS_G char* lt = (const GSA_LDS_G char*)(GSA_LDS_G void*)&Ls[buf][0];
    const GSA_LDS_G char* rt = (const GSA_LDS_G char*)(GSA_LDS_G void*)&Rs[buf][0];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = frag<R_KC>(rt, wn * 64 + 32 * i, ks, r_off);
        b[i] = frag<L_KC>(lt, wm * 64 + 32 * i, ks, l_off);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  }

  // lane holds output row m0 + wm*64 + 32*j + l32 and columns
  // n0 + wn*64 + 32*i + 8*(r/4) + 4*hl + 0..3 (N is a multiple of 4)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm * 64 + 32 * j + l32;
    if (m >= M) continue;
    OutT* orow = outz + (int64_t)m * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + 32 * i + 8 * q + 4 * hl;
        if (n >= N) continue;
        const f32x16& c = acc[i][j];
        if constexpr (std::is_same<OutT, float>::value) {
          *(f32x4*)(orow + n) = f32x4{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]};
        } else {
          *(u32x2*)(orow + n) = u32x2{pack_bf16x2(c[4 * q], c[4 * q + 1]), pack_bf16x2(c[4 * q + 2], c[4 * q + 3])};
        }
      }
  }
}

// ---------------------------------------------------------------- large tiles
// The same products on 256 (m) x 256 (n) x 64 (k) tiles for shapes whose
// dimensions are all multiples of 256: 8 waves in a 2 (m) x 4 (n) grid, each
// with a 128 x 64 block (eight 32x32 accumulators: six operand fragments feed
// eight matrix ops per 16-wide k step), one workgroup per CU, two LDS stages
// filled by 16-byte direct loads.
//   k-contiguous operand: 256 rows x 8 chunks of 8 k + one pad slot (144-byte
//     stride); the fragment (8 consecutive k of one row) is one 16-byte read.
//   m/n-contiguous operand: 64 k rows x 32 chunks (512 bytes), chunk index XOR
//     4·(k & 3); the fragment (8 consecutive k of one column) comes from two
//     transposed reads of 4 k rows each.
// The fragments of k step s+1 are read while the matrix ops of step s run; a
// stage's barrier sits before its last k step, so the next stage's first
// reads overlap that step's matrix ops.  As in the small-tile kernel the
// matrix op's row index is n, so each lane stores 4 consecutive outputs.
namespace bgbig {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr uint32_t kOOB = 0xfffffff0u;
template <bool KC>
struct St {
  static constexpr int SL = KC ? 9 : 32;              // 16-byte slots per LDS row
  static constexpr int SLOTS = KC ? 256 * 9 : 64 * 32;
  static constexpr int INS = SLOTS / 64;              // direct-load instructions per stage
  static constexpr int PER_WAVE = (INS + 7) / 8;      // per wave (the last round may be partial)
  static constexpr int BYTES = SLOTS * 16;
};
// one operand's direct loads: slot (wave + 8j)*64 + lane of the stage
template <bool KC>
struct BigLoader {
  using S_ = St<KC>;
  uint32_t off[S_::PER_WAVE];   // byte offset within the tile at k0 = 0, or kOOB
  __device__ void init(int wave, int lane, int mn0, uint32_t ld) {
#pragma unroll
    for (int j = 0; j < S_::PER_WAVE; ++j) {
      const int slot = (wave + 8 * j) * 64 + lane;
      if (KC) {
        const int row = slot / 9, c = slot % 9;
        off[j] = (slot < S_::SLOTS && c < 8) ? ((uint32_t)(mn0 + row) * ld + 8u * c) * 2u : kOOB;
      } else {
        const int row = slot / 32, p = slot % 32, c = p ^ (4 * (row & 3));
        off[j] = slot < S_::SLOTS ? ((uint32_t)row * ld + (uint32_t)(mn0 + 8 * c)) * 2u : kOOB;
      }
    }
  }
  // stage at k0 (k0 >= k_end: every slot reads zeros)
  __device__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t pad, int k0, int k_end, uint32_t ld,
                       int wave) const {
    const bool live = k0 < k_end;
    const uint32_t kofs = KC ? (uint32_t)k0 * 2u : (uint32_t)k0 * ld * 2u;
#pragma unroll
    for (int j = 0; j < S_::PER_WAVE; ++j) {
      const int ins = wave + 8 * j;
      const bool real = ins < S_::INS;
      dma16_lds(rs, (live && off[j] != kOOB) ? off[j] + kofs : kOOB, real ? lds + (uint32_t)ins * 1024u : pad);
    }
  }
};
// lane part of a fragment address for the 32-wide block starting at col0
template <bool KC>
__device__ __forceinline__ uint32_t big_frag_base(int lane, int col0) {
  if (KC) {
    return (uint32_t)(((col0 + (lane & 31)) * 9 + (lane >> 5)) * 16);
  } else {
    const int g = lane >> 4, si = lane & 15;
    const int n = col0 + 16 * (g & 1) + 4 * (si & 3);
    const int krow = 8 * (g >> 1) + (si >> 2);
    const int phys = (n >> 3) ^ (4 * (krow & 3));
    return (uint32_t)((krow * 32 + phys) * 16 + (n & 7) * 2);
  }
}
// fragment of k step ks (k = 16 ks + 8 hl .. +7) at a lane base
template <bool KC>
__device__ __forceinline__ bf16x8 big_frag(const GSA_LDS_G char* tile, uint32_t base, int ks) {
  if (KC) {
    return *(const GSA_LDS_G bf16x8*)(tile + base + ks * 32);
  } else {
    const GSA_LDS_G char* p = tile + base + ks * 16 * 32 * 16;
    bf16x8 a;
    a.lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS_G i16x4*)p));
    a.hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((GSA_LDS_G i16x4*)(p + 4 * 32 * 16)));
    return a;
  }
}
}  // namespace bgbig

template <typename OutT, bool L_KC, bool R_KC>
__global__ __launch_bounds__(512, 1)
void bwd_gemm_big_kernel(const bf16* __restrict__ L, const bf16* __restrict__ R, OutT* __restrict__ out,
                         int M, int N, uint32_t ldl, uint32_t ldr, uint32_t l_bytes, uint32_t r_bytes,
                         int tiles_m, int tiles_n, int k_chunk) {
  using namespace bgbig;
  __shared__ __align__(16) char Ls[2][St<L_KC>::BYTES];
  __shared__ __align__(16) char Rs[2][St<R_KC>::BYTES];
  // landing area of the load rounds past a stage's last instruction
  __shared__ __align__(16) char Pad[1024];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int tiles = tiles_m * tiles_n;
  const int z = blockIdx.x / tiles, t0 = blockIdx.x % tiles;
  // workgroup ids are dealt round-robin over the 8 XCDs: XCD x = id % 8 takes
  // the x-th contiguous eighth of the row-major tile list, so an L row block
  // is fetched into one L2 instead of all eight
  const int t = tiles % 8 == 0 ? (t0 % 8) * (tiles / 8) + t0 / 8 : t0;
  const int tm = t / tiles_n, tn = t % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb = z * k_chunk, ke = kb + k_chunk;
  OutT* outz = out + (int64_t)z * M * N;

  const auto lrs = make_rsrc(L, l_bytes);
  const auto rrs = make_rsrc(R, r_bytes);
  BigLoader<L_KC> lld;
  BigLoader<R_KC> rld;
  lld.init(wave, lane, m0, ldl);
  rld.init(wave, lane, n0, ldr);
  const uint32_t pad = __builtin_amdgcn_readfirstlane(lds_addr(&Pad[0]));
  auto dma = [&](int k0, int buf) {
    lld.load(lrs, __builtin_amdgcn_readfirstlane(lds_addr(&Ls[buf][0])), pad, k0, ke, ldl, wave);
    rld.load(rrs, __builtin_amdgcn_readfirstlane(lds_addr(&Rs[buf][0])), pad, k0, ke, ldr, wave);
  };
  uint32_t lb[4], rb[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) lb[i] = big_frag_base<L_KC>(lane, wm * 128 + 32 * i);
#pragma unroll
  for (int i = 0; i < 2; ++i) rb[i] = big_frag_base<R_KC>(lane, wn * 64 + 32 * i);

  f32x16 acc[2][4];   // [n block][m block]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  struct Frag {
    bf16x8 l[4], r[2];
  };
  auto load_frag = [&](int buf, int ks, Frag& f) {
    const GSA_LDS_G char* lt = (const GSA_LDS_G char*)(GSA_LDS_G void*)&Ls[buf][0];
    const GSA_LDS_G char* rt = (const GSA_LDS_G char*)(GSA_LDS_G void*)&Rs[buf][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) f.l[i] = big_frag<L_KC>(lt, lb[i], ks);
#pragma unroll
    for (int i = 0; i < 2; ++i) f.r[i] = big_frag<R_KC>(rt, rb[i], ks);
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(f.r[i], f.l[j], acc[i][j]);
  };

  const int nk = k_chunk / BK;
  static_assert(BK / 16 == 4, "four k steps per stage");
  dma(kb, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  dma(kb + BK, 1);
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
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    dma(kb + (kt + 2) * BK, buf);     // past the chunk: zero rounds
    load_frag(buf ^ 1, 0, f0);        // on the last stage: stale, unused
    mma(f1);
  }

  // lane holds output row m0 + wm*128 + 32*j + l32 and columns
  // n0 + wn*64 + 32*i + 8*(r/4) + 4*hl + 0..3
  const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 128 + 32 * j + l32;
    OutT* orow = outz + (int64_t)m * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + 32 * i + 8 * q + 4 * hl;
        const f32x16& c = acc[i][j];
        if constexpr (std::is_same<OutT, float>::value) {
          *(f32x4*)(orow + n) = f32x4{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]};
        } else {
          *(u32x2*)(orow + n) = u32x2{pack_bf16x2(c[4 * q], c[4 * q + 1]), pack_bf16x2(c[4 * q + 2], c[4 * q + 3])};
        }
      }
  }
}

// Whether the large-tile kernel takes a backward GEMM: every dimension a
// multiple of 256 and every operand addressable with 32-bit byte offsets.
static bool bwd_big_ok(int64_t M, int64_t d_model, int64_t N) {
  return M % 256 == 0 && d_model % 256 == 0 && N % 256 == 0 && M * N * 2 < (int64_t(1) << 31) &&
         M * d_model * 2 < (int64_t(1) << 31) && d_model * N * 2 < (int64_t(1) << 31);
}

// out[i] = Σ_z part[z][i] in z order (float4 granules; n4 = element count / 4).
__global__ __launch_bounds__(256)
void sum_partials_kernel(const f32x4* __restrict__ part, f32x4* __restrict__ out, int64_t n4, int splits) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 s = part[i];
    for (int z = 1; z < splits; ++z) s += part[(int64_t)z * n4 + i];
    out[i] = s;
  }
}

// Token chunks for dW_θ: enough workgroups to fill the chip (about 1024), each
// chunk a multiple of 64 tokens and at least 256 of them.
int64_t bwd_dw_splits(int64_t M, int64_t d_model, int64_t N) {
  if (bwd_big_ok(M, d_model, N)) {
    // large tiles: about one workgroup per CU, chunks a multiple of 256 tokens
    const int64_t tiles = (d_model / 256) * (N / 256);
    int64_t s = std::max<int64_t>(1, 256 / tiles);
    while (s > 1 && (M % (256 * s) != 0)) --s;
    return s;
  }
  const int64_t tiles = ceil_div<int64_t>(d_model, bgemm::BM) * ceil_div<int64_t>(N, bgemm::BN);
  int64_t s = ceil_div<int64_t>(1024, tiles);
  s = std::min<int64_t>(s, std::max<int64_t>(1, M / 256));
  return std::max<int64_t>(s, 1);
}
int64_t bwd_dw_chunk(int64_t M, int64_t splits) {
  return ceil_div<int64_t>(ceil_div<int64_t>(M, splits), bgemm::BK) * bgemm::BK;
}

// dX[M, d_model] = dZ[M, N] · W_θ[d_model, N]ᵀ  (both operands k-contiguous, k = N)
hipError_t launch_bwd_gemm_dx(const void* dZ, const void* W, void* dX, int64_t M, int64_t d_model,
                              int64_t N, hipStream_t st) {
  if (bwd_big_ok(M, d_model, N)) {
    const int tm = (int)(M / 256), tn = (int)(d_model / 256);
    hipLaunchKernelGGL((bwd_gemm_big_kernel<bf16, true, true>), dim3((unsigned)(tm * tn)), dim3(512), 0, st,
                       (const bf16*)dZ, (const bf16*)W, (bf16*)dX, (int)M, (int)d_model, (uint32_t)N,
                       (uint32_t)N, (uint32_t)(M * N * 2), (uint32_t)(d_model * N * 2), tm, tn, (int)N);
    return hipGetLastError();
  }
  const int tm = (int)ceil_div<int64_t>(M, bgemm::BM), tn = (int)ceil_div<int64_t>(d_model, bgemm::BN);
  hipLaunchKernelGGL((bwd_gemm_kernel<bf16, true, true>), dim3((unsigned)(tm * tn)), dim3(256), 0, st,
                     (const bf16*)dZ, (const bf16*)W, (bf16*)dX, (int)M, (int)d_model, (int)N,
                     (uint32_t)N, (uint32_t)N, (uint32_t)(M * N * 2), (uint32_t)(d_model * N * 2), tm, tn,
                     (int)N);
  return hipGetLastError();
}

// dW_θ[d_model, N] = X[M, d_model]ᵀ · dZ[M, N]  (both operands m/n-contiguous, k = M);
// partials: splits * d_model * N floats when splits > 1 (else unused)
hipError_t launch_bwd_gemm_dw(const void* X, const void* dZ, float* dW, float* partials, int64_t M,
                              int64_t d_model, int64_t N, int64_t splits, hipStream_t st) {
  float* dst = splits > 1 ? partials : dW;
  if (bwd_big_ok(M, d_model, N)) {
    const int tm = (int)(d_model / 256), tn = (int)(N / 256);
    hipLaunchKernelGGL((bwd_gemm_big_kernel<float, false, false>), dim3((unsigned)(tm * tn * splits)), dim3(512),
                       0, st, (const bf16*)X, (const bf16*)dZ, dst, (int)d_model, (int)N, (uint32_t)d_model,
                       (uint32_t)N, (uint32_t)(M * d_model * 2), (uint32_t)(M * N * 2), tm, tn,
                       (int)(M / splits));
  } else {
  const int tm = (int)ceil_div<int64_t>(d_model, bgemm::BM), tn = (int)ceil_div<int64_t>(N, bgemm::BN);
  const int64_t chunk = bwd_dw_chunk(M, splits);
  hipLaunchKernelGGL((bwd_gemm_kernel<float, false, false>), dim3((unsigned)(tm * tn * splits)), dim3(256), 0,
                     st, (const bf16*)X, (const bf16*)dZ, dst, (int)d_model, (int)N, (int)M,
                     (uint32_t)d_model, (uint32_t)N, (uint32_t)(M * d_model * 2), (uint32_t)(M * N * 2), tm,
                     tn, (int)chunk);
  }
  if (splits > 1) {
    const int64_t n4 = d_model * N / 4;
    const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div<int64_t>(n4, 256), 4096);
    hipLaunchKernelGGL(sum_partials_kernel, dim3(blocks), dim3(256), 0, st, (const f32x4*)partials, (f32x4*)dW,
                       n4, (int)splits);
  }
  return hipGetLastError();
}

}  // namespace gsa
