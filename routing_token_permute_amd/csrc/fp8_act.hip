// FP8 activations: the per-token FP8 dispatch payload and the FP8 x FP8 first
// expert GEMM that consumes it.
//
// "大模型系统中的通算融合" §8.4 lists MoE dispatch with FP8 data and a
// per-token (or per-block) scale, and asks that the receive buffer feed the
// FP8 GEMM directly rather than being widened back to bf16 first; "0. goin"
// §2.1 notes that the quantized token dispatcher pads each expert's group of
// rows to a multiple of 16 (FP8) so that the quantized grouped GEMM sees
// aligned groups. Here, on one GPU:
//
//   * quantize_rows_kernel: one fp32 scale per token row, s = amax / 448 (1
//     for a zero row), and the nearest E4M3 code of each fp32 quotient x / s.
//   * dispatch_fp8_kernel: the receive buffer, expert-major in Algorithm 2's
//     I_e order (the order moe_permute produced), each expert's group starting
//     at a multiple of 16 rows; a token's K copies share its codes and scale;
//     padding rows hold code 0 and scale 0.
//   * gemm_f8f8_kernel (GEMM1 + SwiGLU of Algorithm 2 step 8 in §1.2 of
//     "MoE 分布式推理基础（基于 vLLM）"): FP8 activation rows times FP8 weight
//     columns (moe_quantize_fp8's column-major codes), both K-contiguous, on
//     the gfx950 FP8 MFMA 32x32x64 with fp32 accumulation; the row and column
//     scales multiply the accumulators in the epilogue before SiLU * up. On one
//     GPU the layer reads each pair's token row in place through perm (GATHER)
//     instead of from the receive buffer, and at n <= 32 places the routing
//     ids itself (IDS); the same kernel without SwiGLU is GEMM2 on FP8 h.
#include <algorithm>

#include "gemm_tiles.hpp"
#include "place_pairs.hpp"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Per-token quantization: one wave per row, 8 elements per lane per chunk.
// ---------------------------------------------------------------------------
// CH > 0: rows of at most 512 * CH elements, whose chunks each lane keeps in
// registers between the amax and the codes (one read of the row); CH = 0:
// any width, the row read twice.
template <bool BF16, int CH>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* __restrict__ x, int n, int H,
                                                            uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  auto load8 = [&](int h0, float* v) {
    if constexpr (BF16) {
      const u32x4_t u = *(const u32x4_t*)((const uint16_t*)x + (size_t)row * H + h0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(u[q] << 16);
        v[2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u);
      }
    } else {
      const f32x4_t a = *(const f32x4_t*)((const float*)x + (size_t)row * H + h0);
      const f32x4_t b = *(const f32x4_t*)((const float*)x + (size_t)row * H + h0 + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = a[q];
        v[4 + q] = b[q];
      }
    }
  };
  auto store8 = [&](int h0, const float* v, float s) {
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = v[j] / s;  // one correctly rounded fp32 division each
    *(u32x2_t*)(codes + (size_t)row * H + h0) =
        u32x2_t{e4m3_pack4(q[0], q[1], q[2], q[3]), e4m3_pack4(q[4], q[5], q[6], q[7])};
  };
  float m = 0.f;
  if constexpr (CH > 0) {
    float v[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int h0 = lane * 8 + c * 512;
      if (h0 < H) {
        load8(h0, v[c]);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[c][j]));
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float s = m > 0.f ? m / 448.f : 1.f;
    if (lane == 0) scales[row] = s;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int h0 = lane * 8 + c * 512;
      if (h0 < H) store8(h0, v[c], s);
    }
  } else {
    for (int h0 = lane * 8; h0 < H; h0 += 512) {
      float v[8];
      load8(h0, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float s = m > 0.f ? m / 448.f : 1.f;
    if (lane == 0) scales[row] = s;
    for (int h0 = lane * 8; h0 < H; h0 += 512) {
      float v[8];
      load8(h0, v);
      store8(h0, v, s);
    }
  }
}

// ---------------------------------------------------------------------------
// The padded FP8 receive buffer. Every block rebuilds the padded group starts
// P[e] from the counts in LDS; one wave then fills one buffer row.
// ---------------------------------------------------------------------------
constexpr int kTokenGroup = 16;

__global__ __launch_bounds__(256) void dispatch_fp8_kernel(const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ perm, int E, int K, int nk,
                                                           int rows_max, const uint8_t* __restrict__ codes_tok,
                                                           const float* __restrict__ s_tok, int H,
                                                           int32_t* __restrict__ offsets_padded,
                                                           uint8_t* __restrict__ x_q, float* __restrict__ x_scale,
                                                           int32_t* __restrict__ perm_padded,
                                                           int32_t* __restrict__ inv_padded) {
  __shared__ int P[kMaxExperts + 1];
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < E ? max(0, counts[e]) : 0;
      const int g = (c + kTokenGroup - 1) / kTokenGroup * kTokenGroup;
      int incl = g;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (e < E) {
        P[e] = carry + incl - g;
        cnt[e] = c;
      }
      carry += __shfl(incl, 63);
    }
    if (lane == 0) P[E] = carry;
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += 256) offsets_padded[e] = P[e];
  const int q = blockIdx.x * 4 + wave;  // buffer row
  if (q >= rows_max || q >= P[E]) return;
  // Expert of row q: the last e with P[e] <= q (groups are non-empty only for hit experts).
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (P[mid] <= q)
      lo = mid;
    else
      hi = mid;
  }
  const int e = lo, j = q - P[e];
  uint8_t* dst = x_q + (size_t)q * H;
  if (j < cnt[e]) {
    const int f = perm[offsets[e] + j];
    const bool ok = (unsigned)f < (unsigned)nk;
    const int tok = ok ? f / K : 0;
    const uint8_t* src = codes_tok + (size_t)tok * H;
    for (int h0 = lane * 16; h0 < H; h0 += 1024) *(u32x4_t*)(dst + h0) = *(const u32x4_t*)(src + h0);
    if (lane == 0) {
      x_scale[q] = ok ? s_tok[tok] : 0.f;
      perm_padded[q] = ok ? f : -1;
      if (ok) inv_padded[f] = q;
    }
  } else {
    for (int h0 = lane * 16; h0 < H; h0 += 1024) *(u32x4_t*)(dst + h0) = u32x4_t{0u, 0u, 0u, 0u};
    if (lane == 0) {
      x_scale[q] = 0.f;
      perm_padded[q] = -1;
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM1 + SwiGLU with FP8 activations and FP8 weights.
// ---------------------------------------------------------------------------
// Stages advance K by BK codes (64 or 128): BM activation rows and 256
// weight columns (128 gate columns then the matching 128 up columns) of BK
// bytes each. Chunk c (16 bytes) of a row r sits at slot c ^ ((r / 2) % (BK /
// 16)): the 16 lanes of one quarter of a wave-wide ds_read_b128 (16 rows at
// one chunk) then run at the full LDS rate (for 64-byte rows this is the
// bf16 tiles' A layout, measured conflict-free).
template <int BM, int BK, int CAP>
struct F8Cfg {
  static_assert(BK == 64 || BK == 128, "k-step");
  static constexpr int ROW = BK;               // bytes per staged row (A and B alike)
  static constexpr int CPR = BK / 16;          // 16-byte chunks per row
  static constexpr int ROWS_PER_REGION = 1024 / ROW;
  static constexpr int A_BYTES = BM * ROW;
  static constexpr int B_BYTES = BN * ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int FIT = (160 * 1024) / STAGE;
  static constexpr int NSTAGE = FIT > CAP ? CAP : FIT;
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static constexpr int REGIONS = STAGE / 1024;
  static constexpr int A_REG = A_BYTES / 1024;
};

template <int BK>
__device__ __forceinline__ int f8_swz(int row) { return (row >> 1) & (BK / 16 - 1); }

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// WM x WN waves split the BM x 256 tile; each wave owns (BM / WM) rows and
// (256 / WN) staged columns, half gate and half the matching up columns, as
// 32 x 32 MFMA tiles.
// GATHER (GEMM1 only): A row r is the token row perm[r] / topk of Aq (n_a
// token rows) and its scale a_scale[perm[r] / topk]: the per-token FP8 rows
// are read in place, with no dispatched copy.
// IDS (gathered GEMM1 on decode-sized batches, one row tile per expert): no
// perm or offsets yet; every workgroup places the n_a * topk routing ids
// itself in LDS (place_pairs), slot t is expert t / NB and column block
// t % NB, and workgroup 0 writes the metadata for the kernels that follow.
template <bool GATED, bool GATHER, int BM, int BK, int CAP, int WM, int WN, bool IDS = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_f8f8_kernel(
    const uint8_t* __restrict__ Aq, const float* __restrict__ a_scale, const int32_t* __restrict__ perm, int topk,
    int n_a, const int32_t* __restrict__ offsets, int E, int rows, int Kdim, const uint8_t* __restrict__ Bq,
    long long b_stride, const float* __restrict__ b_scale, int N, int I, uint16_t* __restrict__ C, int NB,
    int n_slots, IdsMeta im) {
  static_assert(!GATHER || GATED, "the row gather belongs to GEMM1");
  static_assert(!IDS || (GATHER && BM < 256), "placement from ids: gathered decode GEMM1");
  using Cfg = F8Cfg<BM, BK, CAP>;
  constexpr int STAGE = Cfg::STAGE, NSTAGE = Cfg::NSTAGE, A_BYTES = Cfg::A_BYTES, A_REG = Cfg::A_REG;
  constexpr int ROW = Cfg::ROW, CPR = Cfg::CPR, RPR = Cfg::ROWS_PER_REGION;
  constexpr int NW = WM * WN;
  constexpr int MT = BM / WM / 32;        // 32-row MFMA tiles per wave
  constexpr int NQ = BN / WN / 32;         // 32-column MFMA tiles per wave
  constexpr int NTH = NQ / 2;              // GEMM1: as many gate tiles as up tiles
  constexpr int REG = Cfg::REGIONS / NW;  // 1 KB DMA regions per wave per stage
  static_assert(MT >= 1 && NTH >= 1 && REG * NW == Cfg::REGIONS, "tile split");
  static_assert(NSTAGE >= 2 && NSTAGE - 2 <= 2 && 2 * REG <= 63, "vmcnt range (wait_dma covers two later stages)");
  __shared__ __attribute__((aligned(16))) char smem_raw[Cfg::LDS_BYTES];
  lds_char_t* smem = (lds_char_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hi = lane >> 5;
  const int nk = Kdim / BK;

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
  auto pair_at = [&](int r) { return IDS ? perm_l[r] : perm[r]; };

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

  // DMA: region r of a stage holds RPR rows of BK bytes; the first A_REG
  // regions hold A, the rest B. Lane L writes row L / CPR, slot L % CPR, and
  // so fetches chunk (L % CPR) ^ swz(row) of that row.
  const uint8_t* src[REG];
  auto set_sources = [&](const Tile& t) {
    const int mrows = t.r1 - t.r0;
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const int r = wave * REG + j;
      const int rr = (r < A_REG ? r : r - A_REG) * RPR + lane / CPR;
      const int c = (lane % CPR) ^ f8_swz<BK>(rr);
      if (r < A_REG) {
        int arow = t.r0 + min(rr, mrows - 1);
        if constexpr (GATHER) {
          const int f = pair_at(arow);
          arow = ((unsigned)f < (unsigned)(n_a * topk)) ? f / topk : 0;
        }
        src[j] = Aq + (size_t)arow * Kdim + c * 16;
      } else {
        int code_row;
        if constexpr (GATED) {  // 128 gate columns, then the matching 128 up columns
          int gc = t.nb * (BN / 2) + (rr & (BN / 2 - 1));
          if (gc >= I) gc = 0;
          code_row = rr < BN / 2 ? gc : I + gc;
        } else {
          code_row = t.nb * BN + rr;
          if (code_row >= N) code_row = 0;
        }
        src[j] = Bq + (size_t)t.e * b_stride + (size_t)code_row * Kdim + c * 16;
      }
    }
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt, int stage) {
    const uint32_t base = lds0 + stage * STAGE + (uint32_t)wave * REG * 1024;
#pragma unroll
    for (int j = 0; j < REG; ++j) dma16(src[j] + (size_t)kt * BK, base + j * 1024);
  };
  auto issue_first = [&]() {
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < nk) issue(p, p);
  };
  auto wait_dma = [&](int stages) {
    if (stages >= 2)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * REG) : "memory");
    else if (stages == 1)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(REG) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  };

  // Operands of k-substep ks (64 codes): lane l of a 32 x 32 tile reads row
  // (l % 32), chunks 4 ks + 2 (l / 32) and the next. A and B use the same
  // k arrangement, which is all the product needs.
  const int a_row0 = wm * (BM / WM);
  auto rd32 = [&](const lds_char_t* base, int row, int ks) {
    const int c0 = 4 * ks + 2 * hi;
    const int sw = f8_swz<BK>(row);
    const u32x4_t lo = lds_read_b128(base + row * ROW + ((c0 ^ sw) << 4));
    const u32x4_t up = lds_read_b128(base + row * ROW + (((c0 + 1) ^ sw) << 4));
    return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
  };
  f32x16_t acc[MT][NQ];
  // Staged B row of column tile q's lane: GEMM1 pairs gate tile q < NTH with
  // up tile q + NTH; GEMM2 takes the wave's NQ tiles in order.
  auto b_row = [&](int q) {
    if constexpr (GATED)
      return (q / NTH) * (BN / 2) + wn * (BN / 2 / WN) + (q % NTH) * 32 + l32;
    else
      return wn * (BN / WN) + q * 32 + l32;
  };
  int vm = 0;  // 32-row MFMA tiles of this wave that hold a valid row
  auto kstep = [&](int stage) {
    const lds_char_t* As = smem + stage * STAGE;
    const lds_char_t* Bs = As + A_BYTES;
#pragma unroll 1
    for (int ks = 0; ks < BK / 64; ++ks) {
      i32x8_t b[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) b[q] = rd32(Bs, b_row(q), ks);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt >= vm) continue;
        const i32x8_t a = rd32(As, a_row0 + mt * 32 + l32, ks);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          acc[mt][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[q], a, acc[mt][q], 0, 0, 0, 127, 0, 127);
      }
    }
  };

  // Epilogue: weights first, so lane l of tile (mt, q) holds output row
  // mt*32 + (l % 32) at the staged columns 8 (r / 4) + 4 (l / 32) + (r % 4),
  // r = 0..15: four runs of four consecutive columns. The column scales are
  // folded into the accumulators first, one column at a time (every row tile
  // of the wave shares them), so that few values are live at once; then the
  // row scale (and for GEMM1 SwiGLU). Lanes l and l ^ 32 swap runs so that
  // each writes 8 consecutive bf16 values (16 bytes). Output columns: GEMM1
  // I (h), GEMM2 N; row stride alike.
  constexpr int kOutTiles = GATED ? NTH : NQ;
  const int ncols = GATED ? I : N;
  auto out_col0 = [&](const Tile& t, int q) {
    return GATED ? t.nb * (BN / 2) + wn * (BN / 2 / WN) + q * 32 : t.nb * BN + wn * (BN / WN) + q * 32;
  };
  auto store_tile = [&](const Tile& t) {
    const int mrows = t.r1 - t.r0;
    const float* sc = b_scale + (size_t)t.e * N;
#pragma unroll
    for (int q = 0; q < kOutTiles; ++q) {
      const int gcol0 = out_col0(t, q);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int col = gcol0 + 8 * (r / 4) + 4 * hi + (r % 4);
        const int cc = col < ncols ? col : 0;
        if constexpr (GATED) {
          const float sg = sc[cc], su = sc[I + cc];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            acc[mt][q][r] *= sg;
            acc[mt][NTH + q][r] *= su;
          }
        } else {
          const float sn = sc[cc];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][q][r] *= sn;
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = a_row0 + mt * 32 + l32;
      const bool row_ok = mt < vm && row < mrows;
      float sa = 0.f;
      if (row_ok) {
        if constexpr (GATHER) {
          const int f = pair_at(t.r0 + row);
          sa = ((unsigned)f < (unsigned)(n_a * topk)) ? a_scale[f / topk] : 0.f;
        } else {
          sa = a_scale[t.r0 + row];
        }
      }
#pragma unroll
      for (int q = 0; q < kOutTiles; ++q) {
        const int gcol0 = out_col0(t, q);
        uint32_t pk[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float v0, v1;
          if constexpr (GATED) {
            v0 = swiglu_f32(acc[mt][q][r] * sa, acc[mt][NTH + q][r] * sa);
            v1 = swiglu_f32(acc[mt][q][r + 1] * sa, acc[mt][NTH + q][r + 1] * sa);
          } else {
            v0 = acc[mt][q][r] * sa;
            v1 = acc[mt][q][r + 1] * sa;
          }
          pk[r / 2] = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
        }
        // Runs q = 0..3 are pk[2q], pk[2q+1] (columns 8q + 4 hi .. +3). Of the
        // runs 2p and 2p+1, lane half 0 keeps run 2p and receives the
        // partner's run 2p (columns +4); lane half 1 keeps run 2p+1 and
        // receives the partner's run 2p+1 (its first four columns).
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint32_t k0 = hi ? pk[4 * p + 2] : pk[4 * p], k1 = hi ? pk[4 * p + 3] : pk[4 * p + 1];
          const uint32_t s0 = hi ? pk[4 * p] : pk[4 * p + 2], s1 = hi ? pk[4 * p + 1] : pk[4 * p + 3];
          const uint32_t g0 = (uint32_t)__shfl_xor((int)s0, 32);
          const uint32_t g1 = (uint32_t)__shfl_xor((int)s1, 32);
          const int col = gcol0 + 16 * p + 8 * hi;
          if (row_ok && col < ncols) {
            const u32x4_t v = hi ? u32x4_t{g0, g1, k0, k1} : u32x4_t{k0, k1, g0, g1};
            *(u32x4_t*)(C + (size_t)(t.r0 + row) * ncols + col) = v;
          }
        }
      }
    }
  };

  Tile t = next_tile();
  if (!t.valid) return;
  set_sources(t);
  issue_first();
  for (;;) {
    const int mrows = __builtin_amdgcn_readfirstlane(t.r1 - t.r0);
    vm = min(MT, max(0, (mrows - a_row0 + 31) / 32));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][q][r] = 0.f;
    int slot = 0;
    for (int kt = 0; kt < nk; ++kt) {
      wait_dma(min(NSTAGE - 2, nk - 1 - kt));
      __syncthreads();
      if (kt + NSTAGE - 1 < nk) issue(kt + NSTAGE - 1, slot == 0 ? NSTAGE - 1 : slot - 1);
      if (vm > 0) kstep(slot);
      slot = (slot == NSTAGE - 1) ? 0 : slot + 1;
    }
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

// Large batches: 256-row tiles, 16 waves, 128-code stages on a 2-deep ring
// (64 KB each; half the barriers per FLOP of 64-code stages on a 4-deep ring,
// measured 3-4% faster for both GEMMs). Decode-like batches: 32-row tiles, 4
// waves, 128-code stages on a 3-deep ring (36 KB each), which keeps more
// weight bytes in flight.
constexpr int kF8BM = 256, kF8BK = 128, kF8Cap = 2, kF8WM = 4, kF8WN = 4;
constexpr int kF8SmallBM = 32, kF8SmallBK = 128, kF8SmallCap = 3, kF8SmallWM = 1, kF8SmallWN = 4;
constexpr int kF8SmallRowsPerExpert = 64;

// C (rows, ncols) bf16 = (A codes x A row scales) . (B codes x B column
// scales)^T over each expert's rows: GEMM1 (GATED: B = W13 codes (E, 2I, H),
// h = SwiGLU of the paired columns, ncols = I) or GEMM2 (B = W2 codes
// (E, H, I), ncols = H).
template <bool GATED, bool GATHER, int BM, int BK, int CAP, int WM, int WN>
void launch_f8f8_cfg(const uint8_t* Aq, const float* a_scale, const int32_t* perm, int topk, int n_a,
                     const int32_t* offsets, int E, int rows, int Kdim, const uint8_t* Bq, const float* b_scale, int N,
                     int I, void* C, hipStream_t s) {
  const int NB = GATED ? ceil_div(I, BN / 2) : ceil_div(N, BN);
  const int n_slots = max_row_tiles(rows, E, BM) * NB;
  const int grid = std::min(n_slots, stream_cu_count(s));
  gemm_f8f8_kernel<GATED, GATHER, BM, BK, CAP, WM, WN><<<grid, 64 * WM * WN, 0, s>>>(
      Aq, a_scale, perm, topk, n_a, offsets, E, rows, Kdim, Bq, (long long)N * Kdim, b_scale, N, I, (uint16_t*)C, NB,
      n_slots, IdsMeta{});
}

template <bool GATED, bool GATHER = false>
void launch_f8f8(const uint8_t* Aq, const float* a_scale, const int32_t* offsets, int E, int rows, int Kdim,
                 const uint8_t* Bq, const float* b_scale, int N, int I, void* C, hipStream_t s,
                 const int32_t* perm = nullptr, int topk = 1, int n_a = 0) {
  if ((long long)rows <= (long long)kF8SmallRowsPerExpert * E)
    launch_f8f8_cfg<GATED, GATHER, kF8SmallBM, kF8SmallBK, kF8SmallCap, kF8SmallWM, kF8SmallWN>(
        Aq, a_scale, perm, topk, n_a, offsets, E, rows, Kdim, Bq, b_scale, N, I, C, s);
  else
    launch_f8f8_cfg<GATED, GATHER, kF8BM, kF8BK, kF8Cap, kF8WM, kF8WN>(Aq, a_scale, perm, topk, n_a, offsets, E, rows,
                                                                     Kdim, Bq, b_scale, N, I, C, s);
}

}  // namespace

size_t fp8_padded_rows(int n, int E, int K) {
  const long long nk = (long long)n * K;
  return (size_t)(nk + (long long)std::min<long long>(E, nk) * (kTokenGroup - 1));
}

hipError_t launch_quantize_rows_fp8(const void* x, int n, int H, moe_dtype dt, uint8_t* codes, float* scales,
                                    hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int g = ceil_div(n, 4);
  if (dt == MOE_BF16) {
    if (H <= 2048)
      quantize_rows_kernel<true, 4><<<g, 256, 0, s>>>(x, n, H, codes, scales);
    else
      quantize_rows_kernel<true, 0><<<g, 256, 0, s>>>(x, n, H, codes, scales);
  } else {
    if (H <= 2048)
      quantize_rows_kernel<false, 4><<<g, 256, 0, s>>>(x, n, H, codes, scales);
    else
      quantize_rows_kernel<false, 0><<<g, 256, 0, s>>>(x, n, H, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const int32_t* counts, const int32_t* offsets, const int32_t* perm, int n, int E,
                               int K, const uint8_t* codes_tok, const float* s_tok, int H, int32_t* offsets_padded,
                               uint8_t* x_q, float* x_scale, int32_t* perm_padded, int32_t* inv_padded,
                               hipStream_t s) {
  const int rows_max = (int)fp8_padded_rows(n, E, K);
  const int blocks = std::max(1, ceil_div(rows_max, 4));
  dispatch_fp8_kernel<<<blocks, 256, 0, s>>>(counts, offsets, perm, E, K, n * K, rows_max, codes_tok, s_tok, H,
                                             offsets_padded, x_q, x_scale, perm_padded, inv_padded);
  return hipGetLastError();
}

hipError_t launch_w13_swiglu_fp8a(const uint8_t* x_q, const float* x_scale, const int32_t* offsets_padded,
                                  int rows_max, const uint8_t* W13q, const float* s13, int E, int H, int I, void* h,
                                  hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  launch_f8f8<true>(x_q, x_scale, offsets_padded, E, rows_max, H, W13q, s13, 2 * I, I, h, s);
  return hipGetLastError();
}

hipError_t launch_w13_swiglu_gather_fp8a(const uint8_t* codes_tok, const float* s_tok, const int32_t* perm, int n,
                                         int K, const int32_t* offsets, const uint8_t* W13q, const float* s13, int E,
                                         int H, int I, void* h, hipStream_t s) {
  const int rows = n * K;
  if (rows == 0) return hipSuccess;
  launch_f8f8<true, true>(codes_tok, s_tok, offsets, E, rows, H, W13q, s13, 2 * I, I, h, s, perm, K, n);
  return hipGetLastError();
}

bool w13_from_ids_fp8a_ok(int n, int K, int E) {
  return n > 0 && n <= kF8SmallBM && (long long)n * K <= kIdsMaxPairs && E <= kMaxExperts &&
         (long long)n * K <= (long long)kF8SmallRowsPerExpert * E;
}

hipError_t launch_w13_swiglu_from_ids_fp8a(const uint8_t* codes_tok, const float* s_tok, const int32_t* ids, int n,
                                           int K, const uint8_t* W13q, const float* s13, int E, int H, int I, int ep,
                                           void* h, int32_t* counts, int32_t* offsets, int32_t* splits,
                                           int32_t* perm, int32_t* inv, hipStream_t s) {
  if (!w13_from_ids_fp8a_ok(n, K, E) || ep <= 0 || E % ep != 0) return hipErrorInvalidValue;
  int id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  const int NB = ceil_div(I, BN / 2);
  const int n_slots = E * NB;
  const int grid = std::min(n_slots, stream_cu_count(s));
  gemm_f8f8_kernel<true, true, kF8SmallBM, kF8SmallBK, kF8SmallCap, kF8SmallWM, kF8SmallWN, true>
      <<<grid, 64 * kF8SmallWM * kF8SmallWN, 0, s>>>(codes_tok, s_tok, nullptr, K, n, nullptr, E, n * K, H, W13q,
                                                      (long long)2 * I * H, s13, 2 * I, I, (uint16_t*)h, NB, n_slots,
                                                      IdsMeta{ids, counts, offsets, splits, perm, inv, ep, id_bits});
  return hipGetLastError();
}

hipError_t launch_w2_fp8a(const uint8_t* h_q, const float* h_scale, const int32_t* offsets_padded, int rows_max,
                          const uint8_t* W2q, const float* s2, int E, int H, int I, void* Y_perm, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  launch_f8f8<false>(h_q, h_scale, offsets_padded, E, rows_max, I, W2q, s2, H, I, Y_perm, s);
  return hipGetLastError();
}

}  // namespace moe
