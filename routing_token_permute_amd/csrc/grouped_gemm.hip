// Grouped SwiGLU expert GEMMs over expert-major rows.
//
// Algorithm 2 steps 8-9 of "MoE 分布式推理基础（基于 vLLM）" §1.2, in the
// two-GEMM form the same section spells out: gate_up = X_e @ W13[e],
// h = silu(gate) * up, Y_e = h @ W2[e].
//
// bf16 path (fp32 accumulation on MFMA 16x16x32):
//   * One workgroup (4 waves, 2x2) per 128x128 output tile; each wave owns
//     64x64 as 4x4 MFMA tiles. K advances 64 at a time through two LDS
//     stages: the next slice is fetched into registers while the current
//     one feeds the MFMAs.
//   * Row tiles never straddle experts. The tile -> (expert, first row) map
//     is derived on the device from `offsets` (a wave-wide prefix sum of the
//     per-expert tile counts), so no host synchronisation is needed and the
//     grid is sized for the worst split of the rows.
//   * The weights stay in the pages' row-major (H, 2I) and (I, H) layouts,
//     i.e. K-major rows. They are staged in LDS as they come from HBM and
//     turned into MFMA B operands with the gfx950 LDS transpose read
//     (ds_read_b64_tr_b16); A rows are K-contiguous and read with 16-byte
//     LDS loads. Both LDS tiles use XOR swizzles that keep those reads and
//     the 16-byte stores free of bank conflicts.
//   * GEMM1 tiles pair 64 gate columns j with the 64 up columns I + j, so a
//     lane holds gate and up of the same output in registers and the SwiGLU
//     epilogue (fp32, then bf16 round-to-nearest-even) needs no extra pass.
//     Outputs are staged through LDS and written as 16-byte rows.
//
// fp32 path: one thread per output element, fp32 FMA over K. It serves the
// small fp32 workloads, where launch latency dominates.
#include <math.h>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int BN = kGemmBN, BK = kGemmBK;
constexpr int B_BYTES = BK * BN * 2;      // 32 KB per stage
constexpr int B_ROW = BN * 2;             // bytes per staged k-row of B
static_assert(BN == 256 && BK == 64, "LDS layouts below assume 256-column, 64-deep stages");

// Stage geometry for a BM-row tile: A is BM x 64 (BM*128 bytes), B is 64 x 256.
// As many stages as fit in 160 KB of LDS, at most four: BM = 256 gets two
// (128 KB), BM = 128 three (144 KB), BM = 32 four (144 KB).
template <int BM>
struct TileCfg {
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int FIT = (160 * 1024) / STAGE;
  static constexpr int NSTAGE = FIT > 4 ? 4 : FIT;
  static constexpr int EPI_BYTES = BM * 264 * 2;  // staged output tile (GEMM2 is the larger)
  static constexpr int LDS_BYTES = (NSTAGE * STAGE > EPI_BYTES) ? NSTAGE * STAGE : EPI_BYTES;
  static constexpr int REGIONS = STAGE / 1024;  // 1 KB DMA regions per stage
};

// Launch configurations of the bf16 path (BM-row tiles, WM x WN waves):
// large experts use 256-row tiles with 8 waves; when experts average few
// rows (decode-like batches) 32-row tiles with a 4-stage ring keep the
// weight stream deep instead.
constexpr int kBM = 256, kGemmWM = 2, kGemmWN = 4;
constexpr int kSmallBM = 32, kSmallWM = 1, kSmallWN = 4;
constexpr int kSmallRowsPerExpert = 64;  // rows / E at or below this: small tiles

// A tile: 128 rows x 64 k (128 B per row = 8 chunks of 16 B). Chunk c of row r
// sits at slot c ^ ((r / 2) % 8): 16 consecutive rows reading the same chunk
// hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int a_off(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// B tile: 64 k-rows x 256 columns (512 B per row = 32 chunks). Chunk c of row
// k sits at c ^ f(k), f(k) = 2 * ((k % 4) + 4 * ((k / 8) % 2)): the 32 lanes of
// one transpose read (8 k-rows x 4 eight-byte pieces) land on 32 distinct
// 8-byte bank pairs, and 16 lanes storing one row's chunks never collide.
__device__ __forceinline__ int b_swz(int k) { return ((k & 3) + ((k >> 3) & 1) * 4) << 1; }
__device__ __forceinline__ int b_off(int k, int chunk) { return k * B_ROW + ((chunk ^ b_swz(k)) << 4); }

// Direct HBM -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane L's bytes land at LDS byte address lds_base + 16 * L, where lds_base is
// wave-uniform (M0). Issued as inline assembly so that the compiler does not
// treat every later LDS read as dependent on it; completion is awaited
// explicitly with s_waitcnt vmcnt before the barrier that publishes a stage.
// M0 is saved and restored around the copy because the compiler reserves it.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}

struct Tile {
  int e, r0, r1, nb;
  bool valid;
};

// Tiles are ordered expert by expert; within an expert, n-block-major, then
// row tile. Tile t -> (expert, rows [r0, r1), n-block). Every wave computes
// it alike from `offsets` with a wave-wide prefix sum of the per-expert tile
// counts.
template <int BM>
__device__ Tile find_tile(const int32_t* __restrict__ offsets, int E, int rows, int NB, int t) {
  const int lane = lane_id();
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int a = 0, b = 0;
    if (e < E) {
      a = min(max(offsets[e], 0), rows);
      b = min(max(offsets[e + 1], a), rows);
    }
    const int mt = (b - a + BM - 1) / BM;
    const int cnt = mt * NB;
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int excl = incl - cnt;
    const bool hit = (cnt > 0) && (t >= carry + excl) && (t < carry + incl);
    const uint64_t bal = __ballot(hit);
    if (bal != 0) {
      // An expert of n rows gets T = ceil(n / BM) row tiles of nearly equal
      // height (the first n % T of them one row taller), so the last tile is
      // never a sliver; waves skip the 16-row slices a tile does not fill.
      const int L = __ffsll((long long)bal) - 1;
      const int local = t - carry - __shfl(excl, L);
      const int T = __shfl(mt, L);
      const int ah = __shfl(a, L), n = __shfl(b, L) - ah;
      const int m = local % T, q = n / T, rem = n % T;
      const int r0 = ah + m * q + min(m, rem);
      return Tile{e0 + L, r0, r0 + q + (m < rem ? 1 : 0), local / T, true};
    }
    carry += __shfl(incl, 63);
  }
  return Tile{0, 0, 0, 0, false};
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8). Within each round
// of 256 ids, give XCD x the contiguous tiles [32x, 32x + 32) so that the
// workgroups sharing one expert's weight and activation tiles meet in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  constexpr int RS = 256;
  const int full = (G / RS) * RS;
  if (bid >= full) return bid;
  const int w = bid % RS;
  return (bid - w) + (w & 7) * (RS / 8) + (w >> 3);
}

// GATED (GEMM1): the 256 staged columns are 128 gate columns followed by the
// matching 128 up columns; the tile writes 128 columns of h. Otherwise
// (GEMM2): 256 output columns. WM x WN waves split the 128 x 256 tile; each
// wave owns (128/WM) rows and (256/WN) staged columns (for GEMM1, half of
// them gate and the matching half up).
// GATHER: A row r of the expert-major operand is row perm[r] / topk of the
// token matrix A (n_a rows), i.e. the permutation gather is fused into the
// HBM -> LDS copy and no permuted copy of the tokens is materialised.
template <bool GATED, bool GATHER, int BM, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                                    const int32_t* __restrict__ perm, int topk,
                                                                    int n_a, const int32_t* __restrict__ offsets,
                                                                    int E, int rows, int Kdim,
                                                                    const uint16_t* __restrict__ B, int ldb,
                                                                    long long b_expert_stride, int Nout, int up_col,
                                                                    uint16_t* __restrict__ C, int ldc, int NB) {
  using Cfg = TileCfg<BM>;
  constexpr int A_BYTES = Cfg::A_BYTES, STAGE = Cfg::STAGE, NSTAGE = Cfg::NSTAGE;
  constexpr int NW = WM * WN;              // waves
  constexpr int MT = BM / WM / 16;         // 16-row MFMA tiles per wave
  constexpr int NT = BN / WN / 16;         // 16-column MFMA tiles per wave
  constexpr int REG = Cfg::REGIONS / NW;   // 1 KB DMA regions per wave per stage
  constexpr int DMA_PER_STAGE = REG;       // 16-byte loads per thread per stage
  static_assert(NT % 2 == 0 && MT >= 1 && REG * NW == Cfg::REGIONS, "tile split");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4 && 2 * DMA_PER_STAGE <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem_raw[Cfg::LDS_BYTES];
  lds_char_t* smem = (lds_char_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Tile t = find_tile<BM>(offsets, E, rows, NB, xcd_remap(blockIdx.x, gridDim.x));
  if (!t.valid) return;
  const int mrows = __builtin_amdgcn_readfirstlane(t.r1 - t.r0);
  const int nb = t.nb;

  // HBM -> LDS assignment. Each wave-wide DMA fills one 1 KB LDS region in
  // lane order, so the swizzled LDS layout is produced by choosing which
  // global chunk each lane fetches. Regions [0, BM/8) hold A (8 rows each),
  // the next 32 regions hold B (2 k-rows each); wave w fills regions
  // [w*REG, (w+1)*REG). Rows past the tile's last valid row and columns past
  // Nout fetch a valid row/column instead: they only feed outputs that are
  // never stored.
  const uint32_t wave_u = wave;
  constexpr int A_REG = A_BYTES / 1024;
  const uint16_t* src[REG];
#pragma unroll
  for (int j = 0; j < REG; ++j) {
    const int r = wave * REG + j;
    if (r < A_REG) {
      const int row = 8 * r + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      int arow = t.r0 + min(row, mrows - 1);
      if constexpr (GATHER) {
        const int f = perm[arow];
        arow = ((unsigned)f < (unsigned)(n_a * topk)) ? f / topk : 0;
      }
      src[j] = A + (size_t)arow * Kdim + c * 8;
    } else {
      const int k = 2 * (r - A_BYTES / 1024) + (lane >> 5);
      const int c = (lane & 31) ^ b_swz(k);
      int col;
      if constexpr (GATED) {
        int gc = nb * 128 + (c & 15) * 8;
        if (gc >= Nout) gc = 0;
        col = (c < 16) ? gc : up_col + gc;
      } else {
        col = nb * 256 + c * 8;
        if (col >= Nout) col = 0;
      }
      src[j] = B + (size_t)t.e * b_expert_stride + (size_t)k * ldb + col;
    }
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt, int stage) {
    const uint32_t base = lds0 + stage * STAGE + wave_u * REG * 1024;
    const size_t ka = (size_t)kt * BK, kb = (size_t)kt * BK * ldb;
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const int r = (int)(wave_u * REG + j);
      // With a 2-stage ring every wait is vmcnt(0), so A regions wholly past
      // the tile's rows need not be fetched (they are never read).
      if (NSTAGE == 2 && r < A_REG && 8 * r >= mrows) continue;
      dma16(src[j] + (r < A_REG ? ka : kb), base + j * 1024);
    }
  };

  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, li = lane & 15, rr = li >> 2, cc = li & 3;
  // A operand (MFMA tile mt, k-step ks): row wm*(BM/WM) + mt*16 + li, chunk ks*4 + g.
  const int a_sw = (li >> 1) & 7;
  const int a_lane = (wm * (BM / WM) + li) * 128;
  const int a_c0 = (g ^ a_sw) << 4, a_c1 = ((4 + g) ^ a_sw) << 4;
  // B operand (MFMA tile nt, k-step ks, half h): k-row ks*32 + g*8 + h*4 + rr,
  // columns col0(nt) + 4cc..+3; the swizzle depends on the lane only.
  const int bsw = b_swz(g * 8 + rr);
  const int b_lane = (g * 8 + rr) * B_ROW + cc * 8;
  int b_col[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int col0;
    if constexpr (GATED)
      col0 = (nt < NT / 2) ? (wn * (BN / 2 / WN) + nt * 16) : (BN / 2 + wn * (BN / 2 / WN) + (nt - NT / 2) * 16);
    else
      col0 = wn * (BN / WN) + nt * 16;
    b_col[nt] = b_lane + (((col0 >> 3) ^ bsw) << 4);
  }

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // 16-row MFMA slices of this wave that hold at least one valid row
  // (wave-uniform); the rest are skipped.
  const int vm = min(MT, max(0, (mrows - wm * (BM / WM) + 15) / 16));

  // One 64-deep k-step from LDS stage `stage`, as two 32-deep halves. `full`
  // is a constant at each call site: the branch-free body serves waves whose
  // row slab is full, the guarded one the partly filled slab of a short tile.
  auto compute_body = [&](int stage, bool full) {
    const lds_char_t* As = smem + stage * STAGE;
    const lds_char_t* Bs = As + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t a[MT], b[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (full || mt < vm)
          a[mt] = __builtin_bit_cast(bf16x8_t, lds_read_b128(As + a_lane + mt * 16 * 128 + (ks ? a_c1 : a_c0)));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const lds_char_t* p = Bs + b_col[nt] + ks * 32 * B_ROW;
        const bf16x4_t lo = lds_read_tr16(p);
        const bf16x4_t hi = lds_read_tr16(p + 4 * B_ROW);
        b[nt] = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (full || mt < vm) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
        }
    }
  };
  // Pipeline over an NSTAGE-deep LDS ring: while k-step kt is multiplied,
  // k-steps up to kt+NSTAGE-1 are in flight from HBM straight into LDS.
  // Before the barrier that publishes stage kt, each wave waits until only
  // its own loads of the later k-steps remain outstanding. The barrier also
  // guarantees every wave has finished reading k-step kt-1, whose stage the
  // next issue overwrites.
  const int nk = Kdim / BK;
  auto main_loop = [&](bool full) {
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < nk) issue(p, p);
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
      // Stages issued after k-step kt and still allowed in flight.
      const int later = min(NSTAGE - 2, nk - 1 - kt);
      if (later >= 2)
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * DMA_PER_STAGE) : "memory");
      else if (later == 1)
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DMA_PER_STAGE) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      __syncthreads();
      const int nxt = kt + NSTAGE - 1;
      if (nxt < nk) issue(nxt, stage == 0 ? NSTAGE - 1 : stage - 1);
      if (full || vm > 0) compute_body(stage, full);
      stage = (stage == NSTAGE - 1) ? 0 : stage + 1;
    }
  };
  if (vm == MT)
    main_loop(true);
  else
    main_loop(false);
  __syncthreads();

  // Epilogue: lane (g, li) of MFMA tile (mt, nt) holds rows 4g..4g+3, column li.
  // Stage the bf16 tile in LDS, then write 16-byte row pieces.
  uint16_t* Cs = (uint16_t*)smem_raw;
  if constexpr (GATED) {
    constexpr int P = 136;  // 128 h columns + 8 pad
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT / 2; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = wm * (BM / WM) + mt * 16 + 4 * g + j;
          const int hc = wn * (BN / 2 / WN) + nt * 16 + li;
          const float gv = acc[mt][nt][j], uv = acc[mt][nt + NT / 2][j];
          const float hv = gv / (1.f + __expf(-gv)) * uv;
          Cs[row * P + hc] = f32_to_bf16(hv);
        }
    __syncthreads();
    for (int q = tid; q < BM * 16; q += 64 * NW) {
      const int row = q >> 4, c = q & 15;
      const int gc = nb * 128 + c * 8;
      if (row < mrows && gc < Nout)
        *(u32x4_t*)(C + (size_t)(t.r0 + row) * ldc + gc) = *(const u32x4_t*)(Cs + row * P + c * 8);
    }
  } else {
    constexpr int P = 264;  // 256 + 8 pad
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = wm * (BM / WM) + mt * 16 + 4 * g + j;
          const int c = wn * (BN / WN) + nt * 16 + li;
          Cs[row * P + c] = f32_to_bf16(acc[mt][nt][j]);
        }
    __syncthreads();
    for (int q = tid; q < BM * 32; q += 64 * NW) {
      const int row = q >> 5, c = q & 31;
      const int gc = nb * 256 + c * 8;
      if (row < mrows && gc < Nout)
        *(u32x4_t*)(C + (size_t)(t.r0 + row) * ldc + gc) = *(const u32x4_t*)(Cs + row * P + c * 8);
    }
  }
}

// fp32: one thread per output element; lanes run along the output columns.
template <bool GATED, bool GATHER>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                      const int32_t* __restrict__ perm, int topk, int n_a,
                                                      const int32_t* __restrict__ offsets, int E, int rows,
                                                      int Kdim, const float* __restrict__ B, int ldb,
                                                      long long b_expert_stride, int Nout, int up_col,
                                                      float* __restrict__ C, int ldc) {
  const int col = blockIdx.x * 64 + (threadIdx.x & 63);
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (row >= rows || col >= Nout) return;
  // Expert of this row: the last e with offsets[e] <= row (upper bound - 1).
  int lo = 0, hi = E + 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row)
      lo = mid + 1;
    else
      hi = mid;
  }
  const int e = lo - 1;
  if (e < 0 || e >= E) return;
  int arow = row;
  if constexpr (GATHER) {
    const int f = perm[row];
    arow = ((unsigned)f < (unsigned)(n_a * topk)) ? f / topk : 0;
  }
  const float* a = A + (size_t)arow * Kdim;
  const float* b = B + (size_t)e * b_expert_stride + col;
  float gsum = 0.f, usum = 0.f;
  for (int k = 0; k < Kdim; ++k) {
    const float av = a[k];
    gsum = fmaf(av, b[(size_t)k * ldb], gsum);
    if constexpr (GATED) usum = fmaf(av, b[(size_t)k * ldb + up_col], usum);
  }
  if constexpr (GATED)
    C[(size_t)row * ldc + col] = gsum / (1.f + expf(-gsum)) * usum;
  else
    C[(size_t)row * ldc + col] = gsum;
}

}  // namespace

namespace {
template <bool GATED, bool GATHER, int BM, int WM, int WN>
void launch_cfg(const void* a, const int32_t* perm, int topk, int n_a, const int32_t* offsets, int E, int rows,
                int Kdim, const void* B, int ldb, long long bstride, int Nout, int up_col, void* C, int ldc, int NB,
                hipStream_t s) {
  const int mt = max_row_tiles(rows, E, BM);
  gemm_bf16_kernel<GATED, GATHER, BM, WM, WN><<<mt * NB, 64 * WM * WN, 0, s>>>(
      (const uint16_t*)a, perm, topk, n_a, offsets, E, rows, Kdim, (const uint16_t*)B, ldb, bstride, Nout, up_col,
      (uint16_t*)C, ldc, NB);
}

template <bool GATED, bool GATHER>
void launch_bf16(const void* a, const int32_t* perm, int topk, int n_a, const int32_t* offsets, int E, int rows,
                 int Kdim, const void* B, int ldb, long long bstride, int Nout, int up_col, void* C, int ldc, int NB,
                 hipStream_t s) {
  if ((long long)rows <= (long long)kSmallRowsPerExpert * E)
    launch_cfg<GATED, GATHER, kSmallBM, kSmallWM, kSmallWN>(a, perm, topk, n_a, offsets, E, rows, Kdim, B, ldb,
                                                            bstride, Nout, up_col, C, ldc, NB, s);
  else
    launch_cfg<GATED, GATHER, kBM, kGemmWM, kGemmWN>(a, perm, topk, n_a, offsets, E, rows, Kdim, B, ldb, bstride,
                                                     Nout, up_col, C, ldc, NB, s);
}

template <bool GATHER>
hipError_t w13_impl(const void* a, const int32_t* perm, int topk, int n_a, const int32_t* offsets, int rows,
                    const void* W13, int E, int H, int I, moe_dtype dt, void* h, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dt == MOE_BF16) {
    launch_bf16<true, GATHER>(a, perm, topk, n_a, offsets, E, rows, H, W13, 2 * I, (long long)H * 2 * I, I, I, h, I,
                              ceil_div(I, BN / 2), s);
  } else {
    dim3 g1(ceil_div(I, 64), ceil_div(rows, 4));
    gemm_f32_kernel<true, GATHER><<<g1, 256, 0, s>>>((const float*)a, perm, topk, n_a, offsets, E, rows, H,
                                                     (const float*)W13, 2 * I, (long long)H * 2 * I, I, I,
                                                     (float*)h, I);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_w13_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13, int E, int H,
                             int I, moe_dtype dt, void* h, hipStream_t s) {
  return w13_impl<false>(x_perm, nullptr, 1, rows, offsets, rows, W13, E, H, I, dt, h, s);
}

hipError_t launch_w13_swiglu_gather(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                    const void* W13, int E, int H, int I, moe_dtype dt, void* h, hipStream_t s) {
  return w13_impl<true>(x, perm, K, n, offsets, n * K, W13, E, H, I, dt, h, s);
}

hipError_t launch_w2(const void* h, const int32_t* offsets, int rows, const void* W2, int E, int H, int I,
                     moe_dtype dt, void* Y_perm, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dt == MOE_BF16) {
    launch_bf16<false, false>(h, nullptr, 1, rows, offsets, E, rows, I, W2, H, (long long)I * H, H, 0, Y_perm, H,
                              ceil_div(H, BN), s);
  } else {
    dim3 g2(ceil_div(H, 64), ceil_div(rows, 4));
    gemm_f32_kernel<false, false><<<g2, 256, 0, s>>>((const float*)h, nullptr, 1, rows, offsets, E, rows, I,
                                                     (const float*)W2, H, (long long)I * H, H, 0, (float*)Y_perm, H);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13,
                                 const void* W2, int E, int H, int I, moe_dtype dt, void* Y_perm, void* h,
                                 hipStream_t s) {
  const hipError_t e = launch_w13_swiglu(x_perm, offsets, rows, W13, E, H, I, dt, h, s);
  if (e != hipSuccess) return e;
  return launch_w2(h, offsets, rows, W2, E, H, I, dt, Y_perm, s);
}

}  // namespace moe
