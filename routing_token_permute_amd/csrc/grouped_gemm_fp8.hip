// Grouped SwiGLU expert GEMMs with FP8 E4M3 weights (bf16 activations).
//
// "大模型系统中的通算融合" §8.4 asks for low-precision payloads with per-token
// or per-block scales that the GEMM consumes directly, and §4.4 describes Mega
// MoE's first linear with low-precision weights transformed ahead of time. The
// expert weights are stored as OCP FP8 E4M3 codes with one fp32 scale per
// output column, prepared once (moe_quantize_fp8): each output column's K codes
// are contiguous, so the weights arrive in the layout the MFMA wants without a
// transpose. Algorithm 2 steps 8-9 of "MoE 分布式推理基础（基于 vLLM）" §1.2 then
// run as in grouped_gemm.hip, with half the weight bytes: the regime where a
// batch is small and the layer streams its weights (decode) gains most.
//
//   * Stages advance K by 64: A (bf16 rows, 128 bytes each) and B (FP8 rows,
//     64 bytes each) go from HBM into an LDS ring with global_load_lds_dwordx4,
//     both XOR-swizzled by 16-byte chunk.
//   * B fragments are read 8 bytes at a time (ds_read_b64) and widened to bf16
//     in registers with the gfx950 FP8 conversion (exact: E4M3 values fit in
//     bf16), so the products run on bf16 MFMA 16x16x32 with fp32 accumulation.
//   * The column scales multiply the fp32 accumulators in the epilogue (for
//     GEMM1 before SiLU * up).
//
// moe_quantize_fp8 computes the scales (amax / 448 in fp32, 1 for an all-zero
// column) and the codes (nearest E4M3 value of the fp32 quotient w / scale,
// ties to the even mantissa, saturating at 448), written from the format's
// definition rather than taken from a conversion instruction.
#include <math.h>

#include <algorithm>

#include "gemm_tiles.hpp"
#include "place_pairs.hpp"

namespace moe {
namespace {

constexpr int kW8BK = 64;           // k per stage (bytes per B row, elements per A row)
constexpr int kW8ARow = kW8BK * 2;  // bytes per staged A row
constexpr int kW8BRow = kW8BK;      // bytes per staged B row

// At most three stages. The 32-row decode tiles stream 16 KB of codes per
// stage, yet a deeper ring made them slower: at n=32 GEMM1 took 49.9, 50.8,
// 55.4, 59.4 and 62 us with 3, 4, 5, 6 and 8 stages, and 58 us with 2. The
// 256-row tiles fit three 48 KB stages in any case.
constexpr int kW8MaxStages = 3;

template <int BM>
struct W8Cfg {
  static constexpr int A_BYTES = BM * kW8ARow;
  static constexpr int B_BYTES = BN * kW8BRow;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int FIT = (160 * 1024) / STAGE;
  static constexpr int NSTAGE = FIT > kW8MaxStages ? kW8MaxStages : FIT;
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static constexpr int REGIONS = STAGE / 1024;
};

// Chunk c (16 bytes) of A row r sits at slot c ^ ((r / 2) % 8); of B row r at
// slot c ^ ((r / 2) % 4).
__device__ __forceinline__ int w8_a_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int w8_b_swz(int row) { return (row >> 1) & 3; }

// Eight E4M3 codes (k order, little-endian) -> eight bf16 operand values.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(u32x2_t w) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], false);
    const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], true);
    // E4M3 values are exact in bf16: the upper halves of the fp32 values.
    o[2 * q] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
    o[2 * q + 1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
  }
  return __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
}

// GATED (GEMM1): staged B rows 0..127 are gate columns nb*128 + r of the
// (2I, H) code matrix, rows 128..255 the matching up columns I + nb*128 + r;
// the tile writes 128 columns of h. Otherwise (GEMM2) 256 columns of Y.
// GATHER: A row r is token row perm[r] / topk of x.
// IDS (gathered GEMM1 on decode-sized batches, one row tile per expert): no
// perm or offsets yet; every workgroup places the n_a * topk routing ids
// itself in LDS (place_pairs), slot t is expert t / NB and column block
// t % NB, and workgroup 0 writes the metadata for the kernels that follow.
// Bq: codes of expert e at Bq + e * b_stride, N rows of Kdim bytes.
// scale: fp32 column scales of expert e at scale + e * N (N = 2I or H).
template <bool GATED, bool GATHER, int BM, int WM, int WN, bool IDS = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_w8_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm, int topk, int n_a,
    const int32_t* __restrict__ offsets, int E, int rows, int Kdim, const uint8_t* __restrict__ Bq,
    long long b_stride, const float* __restrict__ scale, int N, int Nout, int up_col, uint16_t* __restrict__ C,
    int ldc, int NB, int n_slots, IdsMeta im) {
  static_assert(!IDS || (GATED && GATHER && BM < 256), "placement from ids: gathered decode GEMM1");
  using Cfg = W8Cfg<BM>;
  constexpr int A_BYTES = Cfg::A_BYTES, STAGE = Cfg::STAGE, NSTAGE = Cfg::NSTAGE;
  constexpr int NW = WM * WN;
  constexpr int MT = BM / WM / 16, NT = BN / WN / 16;
  constexpr int REG = Cfg::REGIONS / NW;
  constexpr int A_REG = A_BYTES / 1024;
  constexpr int DMA_PER_STAGE = REG;
  static_assert(REG * NW == Cfg::REGIONS && NT % (GATED ? 4 : 2) == 0, "tile split");
  static_assert(NSTAGE >= 2 && NSTAGE <= 8 && 6 * DMA_PER_STAGE <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem_raw[Cfg::LDS_BYTES];
  lds_char_t* smem = (lds_char_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wave_u = wave;
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, li = lane & 15;
  const int nk = Kdim / kW8BK;

  // IDS: the placement of the pairs, in LDS (one-element arrays otherwise).
  __shared__ int ids_l[IDS ? kIdsMaxPairs : 1];
  __shared__ int perm_l[IDS ? kIdsMaxPairs : 1];
  __shared__ int cnt_l[IDS ? NW : 1][IDS ? kMaxExperts : 1];
  __shared__ int offs_l[IDS ? kMaxExperts + 1 : 1];
  if constexpr (IDS) {
    const int total = n_a * topk;  // <= kIdsMaxPairs (checked by the launcher)
    for (int f = tid; f < total; f += 64 * NW) ids_l[f] = im.ids[f];
    place_pairs<NW>(ids_l, total, E, im.ep, im.id_bits, cnt_l, offs_l, perm_l,
                    PlaceOut{blockIdx.x == 0, im.counts, im.offsets, im.splits, im.perm, im.inv});
    __syncthreads();
  }

  int slot_id = blockIdx.x;
  auto next_tile = [&]() {
    Tile t{0, 0, 0, 0, false};
    while (slot_id < n_slots && !t.valid) {
      if constexpr (IDS) {
        const int tt = xcd_remap(slot_id, n_slots);
        const int e = tt / NB;
        const int r0 = offs_l[e], r1 = offs_l[e + 1];
        t = Tile{e, r0, r1, tt - e * NB, r1 > r0};
      } else {
        t = find_tile<BM>(offsets, E, rows, NB, xcd_remap(slot_id, n_slots));
      }
      slot_id += gridDim.x;
    }
    return t;
  };

  // B row (staged row index) -> column of the code matrix.
  auto b_col_of = [&](int nb, int r) {
    int n;
    if constexpr (GATED) {
      const int j = nb * (BN / 2) + (r & (BN / 2 - 1));
      n = j < Nout ? (r < BN / 2 ? j : up_col + j) : 0;
    } else {
      n = nb * BN + r;
      if (n >= Nout) n = 0;
    }
    return n;
  };

  // Copy sources: regions [0, A_REG) hold A (8 rows of 128 bytes each), the
  // rest hold B (16 rows of 64 bytes each); wave w fills regions
  // [w*REG, (w+1)*REG). Rows past the tile's last row and columns past Nout
  // fetch a valid row; they only feed outputs that are never stored.
  const char* src[REG];
  auto set_sources = [&](const Tile& t) {
    const int mrows = t.r1 - t.r0;
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const int r = wave * REG + j;
      if (r < A_REG) {
        const int row = 8 * r + lane / 8;
        const int c = (lane % 8) ^ w8_a_swz(row);
        int arow = t.r0 + min(row, mrows - 1);
        if constexpr (GATHER) {
          const int f = IDS ? perm_l[arow] : perm[arow];
          arow = ((unsigned)f < (unsigned)(n_a * topk)) ? f / topk : 0;
        }
        src[j] = (const char*)(A + (size_t)arow * Kdim) + c * 16;
      } else {
        const int row = 16 * (r - A_REG) + lane / 4;
        const int c = (lane % 4) ^ w8_b_swz(row);
        src[j] = (const char*)(Bq + (size_t)t.e * b_stride + (size_t)b_col_of(t.nb, row) * Kdim) + c * 16;
      }
    }
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt, int stage) {
    const uint32_t base = lds0 + stage * STAGE + wave_u * REG * 1024;
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const int r = (int)(wave_u * REG + j);
      dma16(src[j] + (size_t)kt * (r < A_REG ? kW8ARow : kW8BRow), base + j * 1024);
    }
  };
  auto issue_first = [&]() {
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < nk) issue(p, p);
  };

  // Fragment addresses: A row (slab + mt*16 + li), chunk 4ks + g; B row
  // (col0(nt) + li), bytes 32ks + 8g .. +7 (chunk 2ks + g/2, half g%2).
  const int a_sw = w8_a_swz(li), b_sw = w8_b_swz(li);
  const int a_lane = (wm * (BM / WM) + li) * kW8ARow;
  int b_row[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int r0;
    if constexpr (GATED)
      r0 = (nt < NT / 2) ? (wn * (BN / 2 / WN) + nt * 16) : (BN / 2 + wn * (BN / 2 / WN) + (nt - NT / 2) * 16);
    else
      r0 = wn * (BN / WN) + nt * 16;
    b_row[nt] = (r0 + li) * kW8BRow;
  }

  f32x4_t acc[MT][NT];
  int vm = 0;
  auto step = [&](int stage, bool full) {
    const lds_char_t* As = smem + stage * STAGE;
    const lds_char_t* Bs = As + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < kW8BK / 32; ++ks) {
      bf16x8_t a[MT], b[NT];
      const int bc = ((2 * ks + (g >> 1)) ^ b_sw) * 16 + (g & 1) * 8;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        b[nt] = fp8x8_to_bf16x8(*(const __attribute__((address_space(3))) u32x2_t*)(Bs + b_row[nt] + bc));
      const int ac = ((4 * ks + g) ^ a_sw) << 4;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (full || mt < vm)
          a[mt] = __builtin_bit_cast(bf16x8_t, lds_read_b128(As + a_lane + mt * 16 * kW8ARow + ac));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (full || mt < vm) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[nt], a[mt], acc[mt][nt], 0, 0, 0);
        }
    }
  };
  // Waits until at most `stages` (<= NSTAGE - 2) of this wave's later stages
  // are still in flight.
  auto wait_dma = [&](int stages) {
    switch (stages) {
      case 0: asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DMA_PER_STAGE) : "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * DMA_PER_STAGE) : "memory"); break;
      case 3: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(3 * DMA_PER_STAGE) : "memory"); break;
      case 4: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(4 * DMA_PER_STAGE) : "memory"); break;
      case 5: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(5 * DMA_PER_STAGE) : "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(%0)" : : "n"(6 * DMA_PER_STAGE) : "memory"); break;
    }
  };
  // The ring discipline of grouped_gemm.hip: wait for this wave's copies of
  // k-step kt, publish it with the barrier (which also frees the slot of
  // k-step kt-1), refill that slot, multiply.
  auto main_loop = [&](bool full) {
    int slot = 0;
    for (int kt = 0; kt < nk; ++kt) {
      wait_dma(min(NSTAGE - 2, nk - 1 - kt));
      __syncthreads();
      if (kt + NSTAGE - 1 < nk) issue(kt + NSTAGE - 1, slot == 0 ? NSTAGE - 1 : slot - 1);
      if (full || vm > 0) step(slot, full);
      slot = (slot == NSTAGE - 1) ? 0 : slot + 1;
    }
  };

  // Epilogue: scale the accumulators by their column scales, then as in
  // grouped_gemm.hip (SwiGLU for GEMM1; lane pairs exchange halves so each
  // lane writes 16 bytes).
  auto pack2 = [](float v0, float v1) {
    return (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
  };
  const bool odd = (g & 1) != 0;
  auto store_pair = [&](uint16_t* crow, bool ok, int colP, u32x2_t pP, u32x2_t pQ) {
    const u32x2_t send = odd ? pP : pQ;
    const u32x2_t got{(uint32_t)__shfl_xor((int)send[0], 16), (uint32_t)__shfl_xor((int)send[1], 16)};
    if (!ok) return;
    if (odd)
      *(u32x4_t*)(crow + colP + 16 + 4 * (g - 1)) = u32x4_t{got[0], got[1], pQ[0], pQ[1]};
    else
      *(u32x4_t*)(crow + colP + 4 * g) = u32x4_t{pP[0], pP[1], got[0], got[1]};
  };
  f32x4_t sc[NT];
  auto load_scales = [&](const Tile& t) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = (b_row[nt] / kW8BRow) - li + 4 * g;  // first of this lane's four staged columns
      int n;
      if constexpr (GATED) {
        const int j = t.nb * (BN / 2) + (r & (BN / 2 - 1));
        n = j < Nout ? (r < BN / 2 ? j : up_col + j) : 0;
      } else {
        n = t.nb * BN + r;
        if (n >= Nout) n = 0;
      }
      sc[nt] = *(const f32x4_t*)(scale + (size_t)t.e * N + n);
    }
  };
  auto store_tile = [&](const Tile& t) {
    if constexpr (BM > 64) load_scales(t);
    const int mrows = t.r1 - t.r0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt >= vm) continue;
      const int row = wm * (BM / WM) + mt * 16 + li;
      const bool row_ok = row < mrows;
      uint16_t* crow = C + (size_t)(t.r0 + min(row, mrows - 1)) * ldc;
      if constexpr (GATED) {
        u32x2_t hp[NT / 2];
#pragma unroll
        for (int nt = 0; nt < NT / 2; ++nt) {
          float hv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gv = acc[mt][nt][j] * sc[nt][j], uv = acc[mt][nt + NT / 2][j] * sc[nt + NT / 2][j];
            hv[j] = swiglu_f32(gv, uv);
          }
          hp[nt] = u32x2_t{pack2(hv[0], hv[1]), pack2(hv[2], hv[3])};
        }
#pragma unroll
        for (int q = 0; q < NT / 2; q += 2) {
          const int colP = t.nb * (BN / 2) + wn * (BN / 2 / WN) + q * 16;
          store_pair(crow, row_ok && colP < Nout, colP, hp[q], hp[q + 1]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < NT; q += 2) {
          const f32x4_t u = acc[mt][q] * sc[q], v = acc[mt][q + 1] * sc[q + 1];
          const int colP = t.nb * BN + wn * (BN / WN) + q * 16;
          store_pair(crow, row_ok && colP < Nout, colP, u32x2_t{pack2(u[0], u[1]), pack2(u[2], u[3])},
                     u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])});
        }
      }
    }
  };

  Tile t = next_tile();
  if (!t.valid) return;
  set_sources(t);
  issue_first();
  for (;;) {
    if constexpr (BM <= 64) load_scales(t);  // few accumulators: prefetch the scales for the epilogue
    const int mrows = __builtin_amdgcn_readfirstlane(t.r1 - t.r0);
    vm = min(MT, max(0, (mrows - wm * (BM / WM) + 15) / 16));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (vm == MT)
      main_loop(true);
    else
      main_loop(false);
    __syncthreads();
    const Tile nt_ = next_tile();
    if (nt_.valid) {
      set_sources(nt_);
      issue_first();
    }
    store_tile(t);
    if (!nt_.valid) break;
    t = nt_;
  }
}

// One workgroup per (64 columns, expert): column amax over K, the scale, then
// the codes, written column-major through an LDS transpose of 64 x 64 blocks.
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const void* __restrict__ W, int Kd, int N,
                                                           uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float red[4][64];
  __shared__ uint8_t tile[64][64 + 4];
  const int tid = threadIdx.x, cl = tid & 63, part = tid >> 6;
  const int n0 = blockIdx.x * 64, e = blockIdx.y;
  const int n = n0 + cl;
  auto ld = [&](int k, int col) {
    const size_t i = ((size_t)e * Kd + k) * N + col;
    return BF16 ? bf16_to_f32(((const uint16_t*)W)[i]) : ((const float*)W)[i];
  };
  float m = 0.f;
  if (n < N)
    for (int k = part; k < Kd; k += 4) m = fmaxf(m, fabsf(ld(k, n)));
  red[part][cl] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0][cl], red[1][cl]), fmaxf(red[2][cl], red[3][cl]));
  const float s = amax > 0.f ? amax / 448.f : 1.f;
  if (part == 0 && n < N) scales[(size_t)e * N + n] = s;
  for (int k0 = 0; k0 < Kd; k0 += 64) {
    // Codes of rows k0..k0+63 of this thread's column into tile[col][k].
    for (int kk = part; kk < 64; kk += 4) {
      const int k = k0 + kk;
      tile[cl][kk] = (n < N && k < Kd) ? (uint8_t)e4m3_nearest(ld(k, n) / s) : 0;
    }
    __syncthreads();
    // Column-major store: thread (c, q) writes 16 codes of column n0 + c.
    const int c = tid >> 2, q = tid & 3;
    if (n0 + c < N && k0 + q * 16 < Kd) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)tile[c][q * 16 + 4 * j] | ((uint32_t)tile[c][q * 16 + 4 * j + 1] << 8) |
               ((uint32_t)tile[c][q * 16 + 4 * j + 2] << 16) | ((uint32_t)tile[c][q * 16 + 4 * j + 3] << 24);
      *(u32x4_t*)(codes + ((size_t)e * N + n0 + c) * Kd + k0 + q * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
    }
    __syncthreads();
  }
}

constexpr int kW8BM = 256, kW8WM = 4, kW8WN = 4;
constexpr int kW8SmallBM = 32, kW8SmallWM = 1, kW8SmallWN = 4;
constexpr int kW8SmallRowsPerExpert = 64;

template <bool GATED, bool GATHER, int BM, int WM, int WN>
void launch_w8_cfg(const void* a, const int32_t* perm, int topk, int n_a, const int32_t* offsets, int E, int rows,
                   int Kdim, const void* Bq, long long bstride, const float* scale, int N, int Nout, int up_col,
                   void* C, int ldc, int NB, hipStream_t s) {
  const int n_slots = max_row_tiles(rows, E, BM) * NB;
  const int grid = std::min(n_slots, stream_cu_count(s));
  gemm_w8_kernel<GATED, GATHER, BM, WM, WN><<<grid, 64 * WM * WN, 0, s>>>(
      (const uint16_t*)a, perm, topk, n_a, offsets, E, rows, Kdim, (const uint8_t*)Bq, bstride, scale, N, Nout,
      up_col, (uint16_t*)C, ldc, NB, n_slots, IdsMeta{});
}

template <bool GATED, bool GATHER>
void launch_w8(const void* a, const int32_t* perm, int topk, int n_a, const int32_t* offsets, int E, int rows,
               int Kdim, const void* Bq, long long bstride, const float* scale, int N, int Nout, int up_col, void* C,
               int ldc, int NB, hipStream_t s) {
  if ((long long)rows <= (long long)kW8SmallRowsPerExpert * E)
    launch_w8_cfg<GATED, GATHER, kW8SmallBM, kW8SmallWM, kW8SmallWN>(a, perm, topk, n_a, offsets, E, rows, Kdim, Bq,
                                                                     bstride, scale, N, Nout, up_col, C, ldc, NB, s);
  else
    launch_w8_cfg<GATED, GATHER, kW8BM, kW8WM, kW8WN>(a, perm, topk, n_a, offsets, E, rows, Kdim, Bq, bstride, scale,
                                                      N, Nout, up_col, C, ldc, NB, s);
}

}  // namespace

hipError_t launch_quantize_fp8(const void* W, int E, int Kd, int N, moe_dtype dt, uint8_t* codes, float* scales,
                               hipStream_t s) {
  if (E == 0 || N == 0) return hipSuccess;
  dim3 grid(ceil_div(N, 64), E);
  if (dt == MOE_BF16)
    quantize_fp8_kernel<true><<<grid, 256, 0, s>>>(W, Kd, N, codes, scales);
  else
    quantize_fp8_kernel<false><<<grid, 256, 0, s>>>(W, Kd, N, codes, scales);
  return hipGetLastError();
}

hipError_t launch_w13_swiglu_gather_fp8(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                        const uint8_t* W13q, const float* s13, int E, int H, int I, void* h,
                                        hipStream_t s) {
  const int rows = n * K;
  if (rows == 0) return hipSuccess;
  launch_w8<true, true>(x, perm, K, n, offsets, E, rows, H, W13q, (long long)2 * I * H, s13, 2 * I, I, I, h, I,
                        ceil_div(I, BN / 2), s);
  return hipGetLastError();
}

bool w13_from_ids_fp8_ok(int n, int K, int E) {
  return n > 0 && n <= kW8SmallBM && (long long)n * K <= kIdsMaxPairs && E <= kMaxExperts &&
         (long long)n * K <= (long long)kW8SmallRowsPerExpert * E;
}

hipError_t launch_w13_swiglu_from_ids_fp8(const void* x, const int32_t* ids, int n, int K, const uint8_t* W13q,
                                          const float* s13, int E, int H, int I, int ep, void* h, int32_t* counts,
                                          int32_t* offsets, int32_t* splits, int32_t* perm, int32_t* inv,
                                          hipStream_t s) {
  if (!w13_from_ids_fp8_ok(n, K, E) || ep <= 0 || E % ep != 0) return hipErrorInvalidValue;
  int id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  const int NB = ceil_div(I, BN / 2);
  const int n_slots = E * NB;
  const int grid = std::min(n_slots, stream_cu_count(s));
  gemm_w8_kernel<true, true, kW8SmallBM, kW8SmallWM, kW8SmallWN, true><<<grid, 64 * kW8SmallWM * kW8SmallWN, 0, s>>>(
      (const uint16_t*)x, nullptr, K, n, nullptr, E, n * K, H, W13q, (long long)2 * I * H, s13, 2 * I, I, I,
      (uint16_t*)h, I, NB, n_slots, IdsMeta{ids, counts, offsets, splits, perm, inv, ep, id_bits});
  return hipGetLastError();
}

hipError_t launch_w2_fp8(const void* h, const int32_t* offsets, int rows, const uint8_t* W2q, const float* s2, int E,
                         int H, int I, void* Y_perm, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  launch_w8<false, false>(h, nullptr, 1, rows, offsets, E, rows, I, W2q, (long long)H * I, s2, H, H, 0, Y_perm, H,
                          ceil_div(H, BN), s);
  return hipGetLastError();
}

}  // namespace moe
