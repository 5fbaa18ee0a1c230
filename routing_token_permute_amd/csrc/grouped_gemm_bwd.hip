// Grouped expert GEMMs of the layer's backward.
//
// The gradient of Algorithm 2 steps 8-9 of "MoE 分布式推理基础（基于 vLLM）"
// §1.2 (gate_up = X_e @ W13[e], h = silu(gate) * up, Y_e = h @ W2[e]) takes
// three kinds of grouped products over the same expert-major rows:
//
//   data gradient through W2, with the SwiGLU derivative in the epilogue:
//       dh = dY_e @ W2[e]^T,  dgate = dh * up * silu'(gate),  dup = dh * silu(gate)
//   data gradient through W13:
//       dX_e = [dgate | dup] @ W13[e]^T
//   weight gradients, contracted over each expert's rows:
//       dW2[e] = h_e^T @ dY_e,  dW13[e] = X_e^T @ [dgate | dup]
//
// One persistent kernel serves all three with the forward GEMM's machinery
// (256 x 256 output tiles, 16 waves of 64 x 64, 32-deep k-steps in a
// five-stage LDS ring filled by global_load_lds_dwordx4, MFMA 16x16x32 bf16
// with fp32 accumulation). Only the operand layouts differ:
//
//   * Data gradients: both operands have K contiguous (the rows of dY or
//     dgate_up, and the weights' rows, since W2[e] is (I, H) and W13[e] is
//     (H, 2I) and the contraction runs over their columns). Both stages use
//     the K-contiguous swizzled layout and ds_read_b128.
//   * Weight gradients: the contraction runs over rows, so both operands are
//     k-rows of 256 contiguous columns. Both stages use the k-row layout and
//     the gfx950 transpose read (ds_read_b64_tr_b16). A k-row past the
//     expert's last row is copied from a zero row, so a ragged tail adds
//     nothing; an expert with no rows gets a zero gradient.
//
// Outputs are rounded to bf16 (nearest even) from the fp32 accumulators. The
// fp32 path computes each output with one thread and fp32 FMAs.
#include <math.h>

#include <algorithm>

#include "gemm_tiles.hpp"

namespace moe {
namespace {

constexpr int kBwdBM = 256, kBwdBK = 32, kBwdWM = 4, kBwdWN = 4;

// kDgradF32 and kWgradF32 are the data- and weight-gradient layouts with fp32
// outputs (for the router's products, whose gradients stay fp32); in
// kDgradF32 the k index of B restarts every `kwrap` columns, so that
// [hi | lo] halves of a split A operand meet the same B values.
// kWgradGather is kWgrad with the A rows gathered: k-row r of A is row
// perm[r] / topk of the (n_a, Mdim) token matrix (dW13 straight from x).
enum BwdMode : int { kDgradSwiglu = 0, kDgrad = 1, kWgrad = 2, kDgradF32 = 3, kWgradF32 = 4, kWgradGather = 5 };

// Source of every k-row copied past the end of an expert's rows (zero at
// program load; nothing writes it).
__device__ __attribute__((aligned(16))) uint16_t kZeroRow[BN];

// Token rows of pair rows r0 .. r0+3 (row perm[r] / topk; -1 from r1 on); r0
// and r1 are wave-uniform, so the loads are scalar.
__device__ __forceinline__ int4 token_rows4(const int32_t* __restrict__ perm, int r0, int r1, int topk, int n_a) {
  int t[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t[q] = -1;
    if (r0 + q < r1) {
      const int f = perm[r0 + q];
      t[q] = ((unsigned)f < (unsigned)(n_a * topk)) ? f / topk : 0;
    }
  }
  return int4{t[0], t[1], t[2], t[3]};
}

struct BTile {
  int e, r0, r1, mb, nb;
  bool valid;
};

// A: for the data gradients the (rows, Kdim) operand, K contiguous, lda; for
//    the weight gradients the (rows, Mdim) operand, lda.
// B: for the data gradients expert e's weight, Ndim rows of Kdim contiguous
//    values at B + e * b_stride (row stride ldb); for the weight gradients the
//    (rows, Ndim) operand, ldb.
// C: data gradients: (rows, ldc) rows; kDgradSwiglu writes dgate at column n
//    and dup at column I + n. Weight gradients: C + e * c_stride, (Mdim, Ndim)
//    with row stride ldc. bf16, or fp32 in the F32 modes.
// gu: kDgradSwiglu only, the saved pre-activations [gate | up], row stride 2I.
template <int MODE>
__global__ __launch_bounds__(64 * kBwdWM * kBwdWN, 1) void gemm_bwd_bf16_kernel(
    const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ B, int ldb, long long b_stride,
    const int32_t* __restrict__ offsets, int E, int rows, int Mdim, int Ndim, int Kdim,
    const uint16_t* __restrict__ gu, int I, void* __restrict__ Cv, int ldc, long long c_stride, int MB, int NB,
    int n_slots, int kwrap, const int32_t* __restrict__ perm, int topk, int n_a) {
  constexpr int BM = kBwdBM, BK = kBwdBK, WM = kBwdWM, WN = kBwdWN;
  constexpr bool WGRAD = MODE == kWgrad || MODE == kWgradF32 || MODE == kWgradGather;
  constexpr bool GATHER_A = MODE == kWgradGather;
  constexpr bool OUTF32 = MODE == kDgradF32 || MODE == kWgradF32;
  uint16_t* __restrict__ C = (uint16_t*)Cv;
  float* __restrict__ Cf = (float*)Cv;
  // A 3-stage ring: measured 1-2% faster than five over the whole backward.
  using Cfg = TileCfg<BM, BK, 3>;
  constexpr int A_BYTES = Cfg::A_BYTES, STAGE = Cfg::STAGE, NSTAGE = Cfg::NSTAGE;
  constexpr int NW = WM * WN;
  constexpr int MT = BM / WM / 16, NT = BN / WN / 16;
  constexpr int REG = Cfg::REGIONS / NW;  // 1 KB DMA regions per wave per stage
  constexpr int HALF_REG = Cfg::REGIONS / 2;
  constexpr int DMA_PER_STAGE = REG;
  constexpr int KROW = BK * 2;  // bytes per staged row in the K-contiguous layout
  static_assert(A_BYTES == Cfg::B_BYTES && REG * NW == Cfg::REGIONS && HALF_REG % REG == 0, "stage split");
  static_assert(NSTAGE >= 2 && NSTAGE <= 5 && 4 * DMA_PER_STAGE <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem_raw[Cfg::LDS_BYTES];
  lds_char_t* smem = (lds_char_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wave_u = wave;
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, li = lane & 15, rr = li >> 2, cc = li & 3;
  // Waves [0, NW/2) fill the A half of every stage, the others the B half.
  const bool a_half = wave * REG < HALF_REG;

  int slot_id = blockIdx.x;
  auto tile_of = [&](int t) __attribute__((always_inline)) {
    BTile b{0, 0, 0, 0, 0, false};
    if constexpr (WGRAD) {
      const int per = MB * NB;
      b.e = t / per;
      const int rem = t - b.e * per;
      b.mb = rem / NB;
      b.nb = rem - b.mb * NB;
      b.r0 = min(max(offsets[b.e], 0), rows);
      b.r1 = min(max(offsets[b.e + 1], b.r0), rows);
      b.valid = true;
    } else {
      const Tile s = find_tile<BM>(offsets, E, rows, NB, t);
      b = BTile{s.e, s.r0, s.r1, 0, s.nb, s.valid};
    }
    return b;
  };
  auto next_tile = [&]() __attribute__((always_inline)) {
    BTile t{0, 0, 0, 0, 0, false};
    while (slot_id < n_slots && !t.valid) {
      t = tile_of(xcd_remap(slot_id, n_slots));
      slot_id += gridDim.x;
    }
    return t;
  };

  // Copy sources of this lane's REG regions for the tile being loaded.
  // K-contiguous layout: region j holds 16 rows of 64 bytes, lane L fetches
  // row 16j + L/4 at the chunk that lands in slot L%4 after the swizzle; the
  // k-step advances the pointer by BK elements.
  // k-row layout: region j holds k-rows 2j and 2j + 1 of 256 columns; lane L
  // fetches k-row 2j + L/32 at the chunk that lands in slot L%32. The row is
  // r0 + kt*BK + k, or the zero row past r1.
  const uint16_t* src[REG];
  const uint16_t* zsrc[REG];
  int srow[REG];
  int ld_rows = 0, kr0 = 0, kr1 = 0, nk = 0;
  // GATHER_A: token rows of the four k-rows an A-half wave copies at the next
  // issued k-step (k-rows 4*wave .. 4*wave+3 of the stage), -1 past the
  // expert's rows. Wave-uniform, loaded with scalar loads one k-step ahead so
  // that the vector-memory count of the copies is not disturbed.
  int4 pf = int4{-1, -1, -1, -1};
  auto load_pf = [&](int kt) __attribute__((always_inline)) {
    pf = token_rows4(perm, __builtin_amdgcn_readfirstlane(kr0 + kt * BK + 4 * wave), kr1, topk, n_a);
  };
  auto set_sources = [&](const BTile& t) __attribute__((always_inline)) {
    // Every lane computes the same tile; readfirstlane makes that visible to
    // the compiler, so the k-loop and the row bounds stay scalar.
    kr0 = __builtin_amdgcn_readfirstlane(t.r0);
    kr1 = __builtin_amdgcn_readfirstlane(t.r1);
    nk = WGRAD ? (kr1 - kr0 + BK - 1) / BK : Kdim / BK;
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const int r = (wave * REG + j) % HALF_REG;  // region within the half
      if constexpr (!WGRAD) {
        const int row = 16 * r + lane / 4;
        const int c = (lane % 4) ^ a_swz<BK>(row);
        if (a_half) {
          const int arow = t.r0 + min(row, t.r1 - t.r0 - 1);
          src[j] = A + (size_t)arow * lda + c * 8;
        } else {
          int n = t.nb * BN + row;
          if (n >= Ndim) n = 0;  // feeds only outputs that are never stored
          src[j] = B + (size_t)t.e * b_stride + (size_t)n * ldb + c * 8;
        }
      } else {
        const int k = 2 * r + (lane >> 5);
        const int c = (lane & 31) ^ b_swz(k);
        int col = (a_half ? t.mb : t.nb) * BN + c * 8;
        if (col >= (a_half ? Mdim : Ndim)) col = 0;
        src[j] = (a_half ? A : B) + col;
        zsrc[j] = kZeroRow + c * 8;
        srow[j] = k;
      }
    }
    ld_rows = a_half ? lda : ldb;
    if constexpr (GATHER_A)
      if (a_half) load_pf(0);
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    const uint32_t base = lds0 + stage * STAGE + wave_u * REG * 1024;
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const uint16_t* p;
      if constexpr (MODE == kDgradF32) {
        p = src[j] + (size_t)(a_half ? kt * BK : (kt * BK) % kwrap);
      } else if constexpr (!WGRAD) {
        p = src[j] + (size_t)kt * BK;
      } else if (GATHER_A && a_half) {
        const int q = srow[j] & 3;  // this lane's k-row among the wave's four
        const int tok = (q & 2) ? ((q & 1) ? pf.w : pf.z) : ((q & 1) ? pf.y : pf.x);
        p = tok >= 0 ? src[j] + (size_t)tok * ld_rows : zsrc[j];
      } else {
        const int row = kr0 + kt * BK + srow[j];
        p = row < kr1 ? src[j] + (size_t)row * ld_rows : zsrc[j];
      }
      dma16(p, base + j * 1024);
    }
    if constexpr (GATHER_A)
      if (a_half) load_pf(kt + 1);
  };
  auto issue_first = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < nk) issue(p, p);
  };

  // Operand reads; every fragment is operand[mn = tile base + li][k = 8g..8g+7].
  // K-contiguous layout: ds_read_b128 of row (base + li), chunk g.
  const int k_sw = a_swz<BK>(li);
  const int k_lane = li * KROW + ((g ^ k_sw) << 4);
  // k-row layout: transpose reads of k-rows 8g + rr and 8g + 4 + rr.
  const int t_sw = b_swz(g * 8 + rr);
  const int t_lane = (g * 8 + rr) * B_ROW + cc * 8;
  int a_off[MT], b_off_[NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m0 = wm * (BM / WM) + mt * 16;
    a_off[mt] = WGRAD ? t_lane + (((m0 >> 3) ^ t_sw) << 4) : m0 * KROW + k_lane;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n0 = wn * (BN / WN) + nt * 16;
    b_off_[nt] = WGRAD ? t_lane + (((n0 >> 3) ^ t_sw) << 4) : n0 * KROW + k_lane;
  }

  f32x4_t acc[MT][NT];
  int vm = MT;  // 16-row slices of this wave holding a valid row (wave-uniform)

  auto frag = [&](const lds_char_t* p) __attribute__((always_inline)) {
    if constexpr (WGRAD) {
      const bf16x4_t lo = lds_read_tr16(p);
      const bf16x4_t hi = lds_read_tr16(p + 4 * B_ROW);
      return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return __builtin_bit_cast(bf16x8_t, lds_read_b128(p));
    }
  };
  auto step = [&](int stage, bool full) __attribute__((always_inline)) {
    const lds_char_t* As = smem + stage * STAGE;
    const lds_char_t* Bs = As + A_BYTES;
    bf16x8_t a[MT], b[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) b[nt] = frag(Bs + b_off_[nt]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (full || mt < vm) a[mt] = frag(As + a_off[mt]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (full || mt < vm) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[nt], a[mt], acc[mt][nt], 0, 0, 0);
      }
  };
  auto wait_dma = [&](int stages) __attribute__((always_inline)) {
    if (stages >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(3 * DMA_PER_STAGE) : "memory");
    else if (stages == 2)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * DMA_PER_STAGE) : "memory");
    else if (stages == 1)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DMA_PER_STAGE) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  };
  // Same ring discipline as the forward GEMM: before the barrier that
  // publishes k-step kt, each wave waits until only its own copies of later
  // k-steps remain in flight; the barrier also frees the slot of k-step kt-1.
  auto main_loop = [&](bool full) __attribute__((always_inline)) {
    int slot = 0;
    for (int kt = 0; kt < nk; ++kt) {
      wait_dma(min(NSTAGE - 2, nk - 1 - kt));
      __syncthreads();
      if (kt + NSTAGE - 1 < nk) issue(kt + NSTAGE - 1, slot == 0 ? NSTAGE - 1 : slot - 1);
      if (full || vm > 0) step(slot, full);
      slot = (slot == NSTAGE - 1) ? 0 : slot + 1;
    }
  };

  // Epilogue: lane (g, li) of accumulator (mt, nt) holds row mt*16 + li of
  // the wave's slab at columns 4g..4g+3 of tile nt. Pairs of adjacent tiles
  // are exchanged between lanes g and g^1 so that each lane writes 8
  // consecutive bf16 with one 16-byte store.
  auto pack2 = [](float v0, float v1) {
    return (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
  };
  auto pack4 = [&](const float* v) __attribute__((always_inline)) { return u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])}; };
  const bool odd = (g & 1) != 0;
  auto store_pair = [&](uint16_t* crow, bool ok, int colP, u32x2_t pP, u32x2_t pQ) __attribute__((always_inline)) {
    const u32x2_t send = odd ? pP : pQ;
    const u32x2_t got{(uint32_t)__shfl_xor((int)send[0], 16), (uint32_t)__shfl_xor((int)send[1], 16)};
    if (!ok) return;
    if (odd)
      *(u32x4_t*)(crow + colP + 16 + 4 * (g - 1)) = u32x4_t{got[0], got[1], pQ[0], pQ[1]};
    else
      *(u32x4_t*)(crow + colP + 4 * g) = u32x4_t{pP[0], pP[1], got[0], got[1]};
  };
  // Inverse of store_pair: pP/pQ receive this lane's columns 4g..4g+3 of tiles
  // P (colP..colP+15) and Q = P + 16 from one 16-byte load per lane.
  auto load_pair = [&](const uint16_t* row, int colP, u32x2_t& pP, u32x2_t& pQ) __attribute__((always_inline)) {
    const u32x4_t v = *(const u32x4_t*)(row + (odd ? colP + 16 + 4 * (g - 1) : colP + 4 * g));
    const u32x2_t keep = odd ? u32x2_t{v[2], v[3]} : u32x2_t{v[0], v[1]};
    const u32x2_t give = odd ? u32x2_t{v[0], v[1]} : u32x2_t{v[2], v[3]};
    const u32x2_t got{(uint32_t)__shfl_xor((int)give[0], 16), (uint32_t)__shfl_xor((int)give[1], 16)};
    pP = odd ? got : keep;
    pQ = odd ? keep : got;
  };
  auto store_tile = [&](const BTile& t) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt >= vm) continue;
      const int row = wm * (BM / WM) + mt * 16 + li;
      if constexpr (OUTF32) {
        // Four consecutive fp32 columns per lane and tile: one 16-byte store.
        bool ok;
        float* crow;
        if constexpr (WGRAD) {
          const int m = t.mb * BM + row;
          ok = m < Mdim;
          crow = Cf + (size_t)t.e * c_stride + (size_t)min(m, Mdim - 1) * ldc;
        } else {
          ok = row < t.r1 - t.r0;
          crow = Cf + (size_t)(t.r0 + min(row, t.r1 - t.r0 - 1)) * ldc;
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = t.nb * BN + wn * (BN / WN) + nt * 16 + 4 * g;
          if (ok && col < Ndim) *(f32x4_t*)(crow + col) = acc[mt][nt];
        }
      } else if constexpr (WGRAD) {
        const int m = t.mb * BM + row;
        uint16_t* crow = C + (size_t)t.e * c_stride + (size_t)min(m, Mdim - 1) * ldc;
#pragma unroll
        for (int q = 0; q < NT; q += 2) {
          const int colP = t.nb * BN + wn * (BN / WN) + q * 16;
          const f32x4_t u = acc[mt][q], v = acc[mt][q + 1];
          store_pair(crow, m < Mdim && colP < Ndim, colP, u32x2_t{pack2(u[0], u[1]), pack2(u[2], u[3])},
                     u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])});
        }
      } else {
        const int mrows = t.r1 - t.r0;
        const bool row_ok = row < mrows;
        const size_t r = (size_t)(t.r0 + min(row, mrows - 1));
        uint16_t* crow = C + r * ldc;
        if constexpr (MODE == kDgradSwiglu) {
          // dgate = dh * up * s * (1 + gate * (1 - s)), dup = dh * gate * s,
          // s = 1 / (1 + exp(-gate)), from the saved bf16 pre-activations.
          // The gate/up values of a pair of adjacent 16-column tiles come in
          // with one 16-byte load per lane, the mirror of store_pair: lane g
          // loads where it would store and swaps halves with lane g^1.
          const uint16_t* grow = gu + r * (size_t)(2 * I);
#pragma unroll
          for (int q = 0; q < NT; q += 2) {
            u32x2_t gv[2], uv[2];
            int colP = t.nb * BN + wn * (BN / WN) + q * 16;
            if (colP >= Ndim) colP = 0;  // feeds only outputs that are never stored
            load_pair(grow, colP, gv[0], gv[1]);
            load_pair(grow + I, colP, uv[0], uv[1]);
            float dg[2][4], du[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t gw = gv[h][j >> 1], uw = uv[h][j >> 1];
                const float ga = __uint_as_float((j & 1) ? (gw & 0xFFFF0000u) : (gw << 16));
                const float ua = __uint_as_float((j & 1) ? (uw & 0xFFFF0000u) : (uw << 16));
                const float dh = acc[mt][q + h][j];
                const float s = 1.f / (1.f + __expf(-ga));
                dg[h][j] = dh * ua * s * (1.f + ga * (1.f - s));
                du[h][j] = dh * ga * s;
              }
            const int colS = t.nb * BN + wn * (BN / WN) + q * 16;
            const bool ok = row_ok && colS < Ndim;
            store_pair(crow, ok, colS, pack4(dg[0]), pack4(dg[1]));
            store_pair(crow + I, ok, colS, pack4(du[0]), pack4(du[1]));
          }
        } else {
#pragma unroll
          for (int q = 0; q < NT; q += 2) {
            const int colP = t.nb * BN + wn * (BN / WN) + q * 16;
            const f32x4_t u = acc[mt][q], v = acc[mt][q + 1];
            store_pair(crow, row_ok && colP < Ndim, colP, u32x2_t{pack2(u[0], u[1]), pack2(u[2], u[3])},
                       u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])});
          }
        }
      }
    }
  };

  BTile t = next_tile();
  if (!t.valid) return;
  set_sources(t);
  issue_first();
  for (;;) {
    if constexpr (!WGRAD) {
      const int mrows = __builtin_amdgcn_readfirstlane(t.r1 - t.r0);
      vm = min(MT, max(0, (mrows - wm * (BM / WM) + 15) / 16));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (vm == MT)
      main_loop(true);
    else
      main_loop(false);
    __syncthreads();
    const BTile nt_ = next_tile();
    if (nt_.valid) {
      set_sources(nt_);
      issue_first();
    }
    store_tile(t);
    if (!nt_.valid) break;
    t = nt_;
  }
}

// fp32: one thread per output element.
template <int MODE>
__global__ __launch_bounds__(256) void gemm_bwd_f32_kernel(const float* __restrict__ A, int lda,
                                                           const float* __restrict__ B, int ldb, long long b_stride,
                                                           const int32_t* __restrict__ offsets, int E, int rows,
                                                           int Mdim, int Ndim, int Kdim, const float* __restrict__ gu,
                                                           int I, float* __restrict__ C, int ldc,
                                                           long long c_stride, const int32_t* __restrict__ perm,
                                                           int topk, int n_a) {
  const int col = blockIdx.x * 64 + (threadIdx.x & 63);
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (col >= Ndim) return;
  if constexpr (MODE == kWgrad || MODE == kWgradGather) {
    const int e = blockIdx.z;
    if (row >= Mdim) return;
    const int r0 = min(max(offsets[e], 0), rows), r1 = min(max(offsets[e + 1], r0), rows);
    float sum = 0.f;
    for (int r = r0; r < r1; ++r) {
      int ar = r;
      if constexpr (MODE == kWgradGather) {
        const int f = perm[r];
        ar = ((unsigned)f < (unsigned)(n_a * topk)) ? f / topk : 0;
      }
      sum = fmaf(A[(size_t)ar * lda + row], B[(size_t)r * ldb + col], sum);
    }
    C[(size_t)e * c_stride + (size_t)row * ldc + col] = sum;
  } else {
    if (row >= rows) return;
    int lo = 0, hi = E + 1;  // expert of this row: last e with offsets[e] <= row
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= row)
        lo = mid + 1;
      else
        hi = mid;
    }
    const int e = lo - 1;
    if (e < 0 || e >= E) return;
    const float* a = A + (size_t)row * lda;
    const float* b = B + (size_t)e * b_stride + (size_t)col * ldb;
    float sum = 0.f;
    for (int k = 0; k < Kdim; ++k) sum = fmaf(a[k], b[k], sum);
    if constexpr (MODE == kDgradSwiglu) {
      const float ga = gu[(size_t)row * 2 * I + col], ua = gu[(size_t)row * 2 * I + I + col];
      const float s = 1.f / (1.f + expf(-ga));
      C[(size_t)row * ldc + col] = sum * ua * s * (1.f + ga * (1.f - s));
      C[(size_t)row * ldc + I + col] = sum * ga * s;
    } else {
      C[(size_t)row * ldc + col] = sum;
    }
  }
}

template <int MODE>
hipError_t launch_bwd(const void* A, int lda, const void* B, int ldb, long long b_stride, const int32_t* offsets,
                      int E, int rows, int Mdim, int Ndim, int Kdim, const void* gu, int I, void* C, int ldc,
                      long long c_stride, moe_dtype dt, hipStream_t s, int kwrap = 0,
                      const int32_t* perm = nullptr, int topk = 1, int n_a = 0) {
  constexpr bool WG = MODE == kWgrad || MODE == kWgradF32 || MODE == kWgradGather;
  if (dt == MOE_BF16) {
    const int NB = ceil_div(Ndim, BN);
    const int MB = WG ? ceil_div(Mdim, kBwdBM) : 1;
    const int n_slots = WG ? E * MB * NB : max_row_tiles(rows, E, kBwdBM) * NB;
    if (n_slots == 0) return hipSuccess;
    const int grid = std::min(n_slots, stream_cu_count(s));
    gemm_bwd_bf16_kernel<MODE><<<grid, 64 * kBwdWM * kBwdWN, 0, s>>>(
        (const uint16_t*)A, lda, (const uint16_t*)B, ldb, b_stride, offsets, E, rows, Mdim, Ndim, Kdim,
        (const uint16_t*)gu, I, C, ldc, c_stride, MB, NB, n_slots, kwrap, perm, topk, n_a);
  } else if constexpr (MODE <= kWgrad || MODE == kWgradGather) {
    dim3 grid(ceil_div(Ndim, 64), ceil_div(WG ? Mdim : rows, 4), WG ? E : 1);
    gemm_bwd_f32_kernel<MODE><<<grid, 256, 0, s>>>((const float*)A, lda, (const float*)B, ldb, b_stride, offsets, E,
                                                   rows, Mdim, Ndim, Kdim, (const float*)gu, I, (float*)C, ldc,
                                                   c_stride, perm, topk, n_a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_dx_mfma(const void* dl_hilo, const int32_t* row_offsets, int n, const void* W_gate, int H,
                                 int E, float* dx_router, hipStream_t s) {
  // dx_router = [dl_hi | dl_lo] . [W_gate | W_gate]^T: K = 2E, B's k index wraps at E.
  return launch_bwd<kDgradF32>(dl_hilo, 2 * E, W_gate, E, 0, row_offsets, 1, n, 0, H, 2 * E, nullptr, 0, dx_router,
                               H, 0, MOE_BF16, s, E);
}

hipError_t launch_router_dw_mfma(const void* x, const void* dl_hilo, const int32_t* chunk_offsets, int S, int n,
                                 int H, int E, float* part, hipStream_t s) {
  // part[g] = x_g^T . [dl_hi | dl_lo]_g for each token chunk g: (S, H, 2E) fp32.
  return launch_bwd<kWgradF32>(x, H, dl_hilo, 2 * E, 0, chunk_offsets, S, n, H, 2 * E, 0, nullptr, 0, part, 2 * E,
                               (long long)H * 2 * E, MOE_BF16, s);
}

hipError_t launch_w2_backward(const void* dY_perm, const int32_t* offsets, int rows, const void* W2,
                              const void* gate_up, int E, int H, int I, moe_dtype dt, void* dgate_up, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // dh = dY_e . W2[e]^T: W2[e] is (I, H), so its rows are the I output columns, H contiguous.
  return launch_bwd<kDgradSwiglu>(dY_perm, H, W2, H, (long long)I * H, offsets, E, rows, 0, I, H, gate_up, I,
                                  dgate_up, 2 * I, 0, dt, s);
}

hipError_t launch_w13_backward(const void* dgate_up, const int32_t* offsets, int rows, const void* W13, int E, int H,
                               int I, moe_dtype dt, void* dX_perm, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // dX_e = dgate_up_e . W13[e]^T: W13[e] is (H, 2I), rows are the H output columns, 2I contiguous.
  return launch_bwd<kDgrad>(dgate_up, 2 * I, W13, 2 * I, (long long)H * 2 * I, offsets, E, rows, 0, H, 2 * I,
                            nullptr, 0, dX_perm, H, 0, dt, s);
}

hipError_t launch_weight_grad(const void* a, const void* b, const int32_t* offsets, int rows, int E, int M, int N,
                              moe_dtype dt, void* dW, hipStream_t s) {
  return launch_bwd<kWgrad>(a, M, b, N, 0, offsets, E, rows, M, N, 0, nullptr, 0, dW, N, (long long)M * N, dt, s);
}

hipError_t launch_weight_grad_gather(const void* x, const int32_t* perm, int n, int K, const void* b,
                                     const int32_t* offsets, int E, int M, int N, moe_dtype dt, void* dW,
                                     hipStream_t s) {
  return launch_bwd<kWgradGather>(x, M, b, N, 0, offsets, E, n * K, M, N, 0, nullptr, 0, dW, N, (long long)M * N, dt,
                                  s, 0, perm, K, n);
}

}  // namespace moe
