// Grouped SwiGLU expert GEMMs over expert-major rows.
//
// Algorithm 2 steps 8-9 of "MoE 分布式推理基础（基于 vLLM）" §1.2, in the
// two-GEMM form the same section spells out: gate_up = X_e @ W13[e],
// h = silu(gate) * up, Y_e = h @ W2[e].
//
// bf16 path (fp32 accumulation on MFMA 16x16x32):
//   * Output tiles of 256 rows x 256 columns, 16 waves (4 x 4, four per SIMD);
//     each wave owns 64 x 64 outputs as 4 x 4 MFMA tiles. Decode-like batches
//     use 32-row tiles with 4 waves instead.
//   * Persistent workgroups, one per compute unit, walk a strided list of
//     tile slots. Row tiles never straddle experts; the slot -> (expert,
//     rows, column block) map is derived on the device from `offsets` (a
//     wave-wide prefix sum of the per-expert tile counts), so no host
//     synchronisation is needed.
//   * Both operands go straight from HBM into a ring of LDS stages with
//     global_load_lds_dwordx4 (GEMM1: 64-deep k-steps, two stages of 64 KB;
//     GEMM2: 32-deep k-steps, three stages of 32 KB),
//     each lane fetching the chunk that lands where the swizzled layout
//     wants it. GEMM1 reads its A rows x[perm[r] / K] in that same copy, so
//     no permuted copy of the tokens is made.
//   * The weights stay in the pages' row-major (H, 2I) and (I, H) layouts,
//     i.e. K-major rows, and become MFMA operands through the gfx950 LDS
//     transpose read (ds_read_b64_tr_b16); A rows are K-contiguous and read
//     with ds_read_b128. Both LDS layouts are XOR-swizzled so those reads run
//     without bank conflicts.
//   * Decode-sized batches (n <= 32 tokens) can skip the permute launch:
//     GEMM1 then places the routing ids itself in LDS (IDS below), each
//     expert being one row tile.
//   * GEMM1 tiles pair 128 gate columns j with the 128 up columns I + j, so a
//     lane holds gate and up of the same output in registers and the SwiGLU
//     epilogue (fp32, then bf16 round-to-nearest-even) needs no extra pass.
//     Outputs are written straight from registers as 16-byte buffer stores
//     while the next tile's first k-steps are already in flight; every wave
//     issues the same number of them, so the waits of those k-steps can let
//     the stores drain behind them.
//
// fp32 path: one thread per output element, fp32 FMA over K. It serves the
// small fp32 workloads, where launch latency dominates.
#include <math.h>

#include <algorithm>

#include "gemm_tiles.hpp"
#include "place_pairs.hpp"

namespace moe {
namespace {

// Launch configurations of the bf16 path (BM-row tiles, WM x WN waves):
// large experts use 256-row tiles with 16 waves; when experts average few
// rows (decode-like batches) 32-row tiles with a 4-stage ring keep the
// weight stream deep instead.
// GEMM1 stages 64-deep k-steps on a 2-deep ring (half the barriers per FLOP;
// measured 2-4% faster), GEMM2 32-deep ones on a 3-deep ring (1-2% faster
// than 64-deep for its 32 k-steps per tile).
constexpr int kBM = 256, kBK = 32, kBK1 = 64, kGemmWM = 4, kGemmWN = 4;
constexpr int kSmallBM = 32, kSmallBK = 64, kSmallWM = 1, kSmallWN = 4;
constexpr int kSmallRowsPerExpert = 64;  // rows / E at or below this: small tiles

// GATED (GEMM1): the 256 staged columns are 128 gate columns followed by the
// matching 128 up columns; the tile writes 128 columns of h. Otherwise
// (GEMM2): 256 output columns. WM x WN waves split the BM x 256 tile; each
// wave owns (BM/WM) rows and (256/WN) staged columns (for GEMM1, half of
// them gate and the matching half up).
// GATHER: A row r of the expert-major operand is row perm[r] / topk of the
// token matrix A (n_a rows), i.e. the permutation gather is fused into the
// HBM -> LDS copy and no permuted copy of the tokens is materialised.
// SCATTER (GEMM2 only): output row r goes to row perm[r] of C (flat pair
// order, n_a rows) scaled by wrow[perm[r]] before the bf16 rounding, i.e. the
// routing weight and the un-permutation are fused into the epilogue.
// SAVE (GEMM1 only): the pre-activations [gate | up] are also written, rounded
// to bf16, to gu_out (row stride 2 * up_col), for the backward pass.
// IDS (gathered GEMM1 with one row tile per expert, i.e. no expert has more
// than BM rows): there is no perm or offsets yet. Every workgroup stages the
// n_a * topk routing ids in LDS and places them itself (place_pairs, the same
// stable placement moe_permute makes), then reads its tiles' rows and
// gathered token indices from LDS; slot t is expert t / NB, column block
// t % NB, and the slots of experts without rows are skipped. Workgroup 0 also
// writes the metadata to memory for the kernels that follow, so no separate
// permute launch runs before this GEMM.
// BPK: B is the packed form of the weights (per expert and 32 K rows, one
// 16 KB unit per 256-column block, each column's 32 values contiguous with the
// A tiles' swizzle; ldb = NB * 256). A stage's B part is then a copy of whole
// units, and B operands are read with ds_read_b128 like A operands; the
// arithmetic, and so every output bit, is that of the plain layout.
template <bool GATED, bool GATHER, bool SCATTER, int BM, int BK, int WM, int WN, bool SAVE = false,
          bool IDS = false, bool BPK = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                                    const int32_t* __restrict__ perm, int topk,
                                                                    int n_a, const float* __restrict__ wrow,
                                                                    const int32_t* __restrict__ offsets,
                                                                    int E, int rows, int Kdim,
                                                                    const uint16_t* __restrict__ B, int ldb,
                                                                    long long b_expert_stride, int Nout, int up_col,
                                                                    uint16_t* __restrict__ C, int ldc, int NB,
                                                                    int n_slots, uint16_t* __restrict__ gu_out,
                                                                    IdsMeta im) {
  // The 256-row tiles run on at most three stages (three of 32 KB for GEMM2;
  // GEMM1's 64 KB stages fit two): measured a little faster than four or five
  // stages, whose deeper copy lead buys nothing.
  using Cfg = TileCfg<BM, BK, (BM == 256) ? 3 : kMaxStages>;
  constexpr int A_BYTES = Cfg::A_BYTES, STAGE = Cfg::STAGE, NSTAGE = Cfg::NSTAGE, A_ROW = Cfg::A_ROW;
  constexpr int KS = BK / 32;              // 32-deep MFMA steps per stage
  constexpr int NW = WM * WN;              // waves
  constexpr int MT = BM / WM / 16;         // 16-row MFMA tiles per wave
  constexpr int NT = BN / WN / 16;         // 16-column MFMA tiles per wave
  constexpr int REG = Cfg::REGIONS / NW;   // 1 KB DMA regions per wave per stage
  constexpr int DMA_PER_STAGE = REG;       // 16-byte loads per thread per stage
  constexpr int A_REG = A_BYTES / 1024;    // regions holding A
  static_assert(NT % (GATED ? 4 : 2) == 0 && MT >= 1 && REG * NW == Cfg::REGIONS, "tile split");
  static_assert(!(SCATTER && (GATED || GATHER)), "the weighted scatter is a GEMM2 epilogue");
  static_assert(!SAVE || GATED, "the pre-activations belong to GEMM1");
  static_assert(!IDS || (GATED && GATHER && !SAVE && BM < 256), "placement from ids: gathered decode GEMM1");
  // Epilogue stores per wave and tile when they go out as buffer stores
  // (every wave issues all of them; lanes without a valid output carry an
  // out-of-range offset, which the hardware drops), so that the waits of the
  // next tile can count them exactly. The weighted scatter keeps plain stores.
  constexpr bool ST_COUNTED = !SCATTER;
  constexpr int ST = !ST_COUNTED ? 0 : GATED ? MT * (NT / 4) * (SAVE ? 3 : 1) : MT * (NT / 2);
  static_assert(NSTAGE >= 2 && NSTAGE <= 5 && (NSTAGE - 2) * DMA_PER_STAGE + ST <= 63, "vmcnt range");
  static_assert(NSTAGE - 2 <= 3, "wait_dma covers up to three later stages");
  __shared__ __attribute__((aligned(16))) char smem_raw[Cfg::LDS_BYTES];
  lds_char_t* smem = (lds_char_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wave_u = wave;
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, li = lane & 15, rr = li >> 2, cc = li & 3;
  const int nk = Kdim / BK;

  // IDS: the placement of the pairs, in LDS (one-element arrays otherwise).
  __shared__ int ids_l[IDS ? kIdsMaxPairs : 1];
  __shared__ int perm_l[IDS ? kIdsMaxPairs : 1];
  __shared__ int cnt_l[IDS ? NW : 1][IDS ? kMaxExperts : 1];
  __shared__ int offs_l[IDS ? kMaxExperts + 1 : 1];
  // Tile slots: this workgroup takes slots blockIdx.x, blockIdx.x + gridDim.x,
  // ... of the n_slots the worst split of the rows can need; a slot past the
  // real tile count comes back invalid.
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

  // HBM -> LDS assignment. Each wave-wide DMA fills one 1 KB LDS region in
  // lane order, so the swizzled LDS layout is produced by choosing which
  // global chunk each lane fetches. The first A_REG regions hold A
  // (1024/A_ROW rows each), the rest hold B (2 k-rows each); wave w fills
  // regions [w*REG, (w+1)*REG). Rows past the tile's last valid row and
  // columns past Nout fetch a valid row/column instead: they only feed
  // outputs that are never stored.
  const uint16_t* src[REG];
  auto set_sources = [&](const Tile& t) {
    const int mrows = t.r1 - t.r0;
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const int r = wave * REG + j;
      if (r < A_REG) {
        constexpr int CPR = A_ROW / 16;  // 16-byte chunks per A row
        const int row = Cfg::A_ROWS_PER_REGION * r + lane / CPR;
        const int c = (lane % CPR) ^ a_swz<BK>(row);
        int arow = t.r0 + min(row, mrows - 1);
        if constexpr (GATHER) {
          const int f = IDS ? perm_l[arow] : perm[arow];
          arow = ((unsigned)f < (unsigned)(n_a * topk)) ? f / topk : 0;
        }
        src[j] = A + (size_t)arow * Kdim + c * 8;
      } else if constexpr (BPK) {
        // Packed weights: the stage's B part is a straight copy of its BK / 32
        // units of column block t.nb, 16 regions of 1 KB each (ldb = NB * 256,
        // so that the k-step advance kt * BK * ldb is BK / 32 unit rows).
        const int rb = r - A_REG;
        src[j] = B + ((size_t)t.e * (Kdim / 32) * NB + t.nb + (size_t)(rb >> 4) * NB) * kPackUnit +
                 (rb & 15) * 512 + lane * 8;
      } else {
        const int k = 2 * (r - A_REG) + (lane >> 5);
        const int c = (lane & 31) ^ b_swz(k);
        int col;
        if constexpr (GATED) {
          int gc = t.nb * 128 + (c & 15) * 8;
          if (gc >= Nout) gc = 0;
          col = (c < 16) ? gc : up_col + gc;
        } else {
          col = t.nb * 256 + c * 8;
          if (col >= Nout) col = 0;
        }
        src[j] = B + (size_t)t.e * b_expert_stride + (size_t)k * ldb + col;
      }
    }
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt, int stage) {
    const uint32_t base = lds0 + stage * STAGE + wave_u * REG * 1024;
    const size_t ka = (size_t)kt * BK, kb = (size_t)kt * BK * ldb;
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const int r = (int)(wave_u * REG + j);
      // Decode-sized tiles read each weight tile once: stream it (nt).
      if (BM < 256 && r >= A_REG)
        dma16_stream(src[j] + kb, base + j * 1024);
      else
        dma16(src[j] + (r < A_REG ? ka : kb), base + j * 1024);
    }
  };
  auto issue_first = [&]() {
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < nk) issue(p, p);
  };

  // A operand (MFMA tile mt, k-step ks): row wm*(BM/WM) + mt*16 + li, chunk
  // ks*4 + g; the swizzle depends on the lane only.
  const int a_sw = a_swz<BK>(li);
  const int a_lane = (wm * (BM / WM) + li) * A_ROW;
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
    if constexpr (BPK)  // column col0 + li of the unit, k-chunk g (the A operand's form)
      b_col[nt] = (col0 + li) * 64 + ((g ^ ((li >> 1) & 3)) << 4);
    else
      b_col[nt] = b_lane + (((col0 >> 3) ^ bsw) << 4);
  }

  f32x4_t acc[MT][NT];
  int vm = 0;  // 16-row MFMA slices of this wave holding a valid row (wave-uniform)

  // Operands of one BK-deep k-step, read from LDS stage `stage`, and the
  // MFMAs over them. `full` is a constant at each call site: the branch-free
  // form serves waves whose row slab is full, the guarded one the partly
  // filled slab of a short tile.
  // Operands of one 32-deep MFMA step ks of a stage are read just before its
  // MFMAs, so a 64-deep stage holds no more operand registers than a 32-deep
  // one.
  using AOps = bf16x8_t[MT];
  using BOps = bf16x8_t[NT];
  auto load_ops = [&](int stage, int ks, bool full, AOps& a, BOps& b) {
    const lds_char_t* As = smem + stage * STAGE;
    const lds_char_t* Bs = As + A_BYTES;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr (BPK) {
        b[nt] = __builtin_bit_cast(bf16x8_t, lds_read_b128(Bs + ks * kPackUnitBytes + b_col[nt]));
      } else {
        const lds_char_t* p = Bs + b_col[nt] + ks * 32 * B_ROW;
        const bf16x4_t lo = lds_read_tr16(p);
        const bf16x4_t hi = lds_read_tr16(p + 4 * B_ROW);
        b[nt] = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (full || mt < vm)
        a[mt] = __builtin_bit_cast(bf16x8_t, lds_read_b128(As + a_lane + mt * 16 * A_ROW + (ks ? a_c1 : a_c0)));
  };
  // The B operand goes first, so each accumulator tile is the transposed
  // product (see the epilogue).
  auto mma = [&](bool full, const AOps& a, const BOps& b) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (full || mt < vm) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[nt], a[mt], acc[mt][nt], 0, 0, 0);
      }
  };
  // Waits until at most `stages` of this wave's later DMA stages are still
  // in flight (every stage is DMA_PER_STAGE loads per lane). Stores still in
  // flight from the previous tile only make the wait longer.
  auto wait_dma = [&](int stages) {
    if (stages >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(3 * DMA_PER_STAGE) : "memory");
    else if (stages == 2)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * DMA_PER_STAGE) : "memory");
    else if (stages == 1)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DMA_PER_STAGE) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  };
  // The same wait for a k-step that was put in flight before the previous
  // tile's ST epilogue stores: those stores are younger than it, so they may
  // stay outstanding too. Vector memory operations retire in issue order, so
  // the count still proves that this k-step has landed, and the stores drain
  // behind the first k-steps instead of holding them up.
  auto wait_dma_st = [&](int stages) {
    if (stages >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(3 * DMA_PER_STAGE + ST) : "memory");
    else if (stages == 2)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * DMA_PER_STAGE + ST) : "memory");
    else if (stages == 1)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DMA_PER_STAGE + ST) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(ST) : "memory");
  };
  // Pipeline over an NSTAGE-deep LDS ring; the first NSTAGE-1 k-steps are
  // already in flight. While k-step kt is multiplied, k-steps up to
  // kt+NSTAGE-1 are in flight from HBM straight into LDS. Before the barrier
  // that publishes stage kt, each wave waits until only its own loads of
  // later k-steps remain outstanding. The barrier also guarantees that every
  // wave has finished reading k-step kt-1 (its MFMAs consumed those reads),
  // whose slot the next issue overwrites.
  // after_st: this wave issued the previous tile's ST epilogue stores right
  // after the first NSTAGE-1 k-steps of this tile.
  auto main_loop = [&](bool full, bool after_st) {
    int slot = 0;  // ring slot of k-step kt
    for (int kt = 0; kt < nk; ++kt) {
      if (ST_COUNTED && after_st && kt <= NSTAGE - 2)
        wait_dma_st(min(NSTAGE - 2, nk - 1 - kt));
      else
        wait_dma(min(NSTAGE - 2, nk - 1 - kt));
      __syncthreads();
      if (kt + NSTAGE - 1 < nk) issue(kt + NSTAGE - 1, slot == 0 ? NSTAGE - 1 : slot - 1);
      if (full || vm > 0) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          AOps a;
          BOps b;
          load_ops(slot, ks, full, a, b);
          mma(full, a, b);
        }
      }
      slot = (slot == NSTAGE - 1) ? 0 : slot + 1;
    }
  };

  // Epilogue. Lane (g, li) of accumulator tile (mt, nt) holds output row
  // mt*16 + li of the wave's slab at the four consecutive columns
  // col0(nt) + 4g .. +3. Values are rounded to bf16 (nearest even); then the
  // lanes g and g^1 of each pair of adjacent 16-column tiles swap halves, so
  // that each lane holds 8 consecutive columns of one tile and writes them
  // with one 16-byte store straight to HBM (a row's 32 columns of the pair go
  // out as one 64-byte piece). The stores drain while the next tile is
  // multiplied.
  auto pack2 = [](float v0, float v1) {
    return (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
  };
  const bool odd = (g & 1) != 0;
  // Tiles P (columns colP..colP+15) and Q = P + 16 of one row: pP/pQ are this
  // lane's packed columns 4g..4g+3 of each. Even g keeps P and receives the
  // partner's P (columns 4g+4..4g+7); odd g keeps Q and receives the
  // partner's Q (columns 4g-4..4g-1). All lanes take part in the exchange.
  auto store_pair = [&](uint16_t* crow, bool ok, int colP, u32x2_t pP, u32x2_t pQ) {
    const u32x2_t send = odd ? pP : pQ;
    const u32x2_t got{(uint32_t)__shfl_xor((int)send[0], 16), (uint32_t)__shfl_xor((int)send[1], 16)};
    if (!ok) return;
    if (odd)
      *(u32x4_t*)(crow + colP + 16 + 4 * (g - 1)) = u32x4_t{got[0], got[1], pQ[0], pQ[1]};
    else
      *(u32x4_t*)(crow + colP + 4 * g) = u32x4_t{pP[0], pP[1], got[0], got[1]};
  };
  // The same exchange, stored through a buffer resource whose base is the
  // tile's first output row: `rowoff` is the byte offset of this lane's row,
  // and a lane without a valid output sends an offset past the resource's
  // range, so the store instruction is issued by every wave (ST per tile) and
  // only the valid lanes write.
  constexpr uint32_t kDropped = 0x80000000u;
  auto store_pair_buf = [&](__amdgpu_buffer_rsrc_t rs, uint32_t rowoff, bool ok, int colP, u32x2_t pP, u32x2_t pQ) {
    const u32x2_t send = odd ? pP : pQ;
    const u32x2_t got{(uint32_t)__shfl_xor((int)send[0], 16), (uint32_t)__shfl_xor((int)send[1], 16)};
    const int col = odd ? colP + 16 + 4 * (g - 1) : colP + 4 * g;
    const u32x4_t v = odd ? u32x4_t{got[0], got[1], pQ[0], pQ[1]} : u32x4_t{pP[0], pP[1], got[0], got[1]};
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, ok ? rowoff + (uint32_t)col * 2u : kDropped, 0, 0);
  };
  // SCATTER: each lane's destination rows and weights, loaded when the tile
  // starts so that the epilogue does not wait for them.
  int sc_row[MT];
  float sc_w[MT];
  auto load_scatter = [&](const Tile& t) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = wm * (BM / WM) + mt * 16 + li;
      const int f = perm[t.r0 + min(row, t.r1 - t.r0 - 1)];
      sc_row[mt] = f;
      sc_w[mt] = ((unsigned)f < (unsigned)n_a) ? wrow[f] : 0.f;
    }
  };
  auto store_tile_plain = [&](const Tile& t) {
    const int mrows = t.r1 - t.r0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt >= vm) continue;
      const int row = wm * (BM / WM) + mt * 16 + li;
      bool row_ok = row < mrows;
      int crow_i = t.r0 + min(row, mrows - 1);
      float wr = 1.f;
      if constexpr (SCATTER) {
        row_ok = row_ok && (unsigned)sc_row[mt] < (unsigned)n_a;
        crow_i = row_ok ? sc_row[mt] : 0;
        wr = sc_w[mt];
      }
      uint16_t* crow = C + (size_t)crow_i * ldc;
      if constexpr (GATED) {
        u32x2_t hp[NT / 2];
#pragma unroll
        for (int nt = 0; nt < NT / 2; ++nt) {
          float hv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gv = acc[mt][nt][j], uv = acc[mt][nt + NT / 2][j];
            hv[j] = swiglu_f32(gv, uv);
          }
          hp[nt] = u32x2_t{pack2(hv[0], hv[1]), pack2(hv[2], hv[3])};
        }
#pragma unroll
        for (int q = 0; q < NT / 2; q += 2) {
          const int colP = t.nb * (BN / 2) + wn * (BN / 2 / WN) + q * 16;
          store_pair(crow, row_ok && colP < Nout, colP, hp[q], hp[q + 1]);
        }
        if constexpr (SAVE) {
          uint16_t* grow = gu_out + (size_t)crow_i * (2 * up_col);
#pragma unroll
          for (int q = 0; q < NT / 2; q += 2) {
            const int colP = t.nb * (BN / 2) + wn * (BN / 2 / WN) + q * 16;
            const f32x4_t g0 = acc[mt][q], g1 = acc[mt][q + 1];
            const f32x4_t u0 = acc[mt][q + NT / 2], u1 = acc[mt][q + 1 + NT / 2];
            store_pair(grow, row_ok && colP < Nout, colP, u32x2_t{pack2(g0[0], g0[1]), pack2(g0[2], g0[3])},
                       u32x2_t{pack2(g1[0], g1[1]), pack2(g1[2], g1[3])});
            store_pair(grow + up_col, row_ok && colP < Nout, colP, u32x2_t{pack2(u0[0], u0[1]), pack2(u0[2], u0[3])},
                       u32x2_t{pack2(u1[0], u1[1]), pack2(u1[2], u1[3])});
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < NT; q += 2) {
          f32x4_t u = acc[mt][q], v = acc[mt][q + 1];
          if constexpr (SCATTER) {
            u *= wr;
            v *= wr;
          }
          const int colP = t.nb * BN + wn * (BN / WN) + q * 16;
          store_pair(crow, row_ok && colP < Nout, colP, u32x2_t{pack2(u[0], u[1]), pack2(u[2], u[3])},
                     u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])});
        }
      }
    }
  };

  // Counted form (every path but the scatter): ST buffer stores per wave,
  // also for the 16-row slices a short tile does not fill.
  auto store_tile_counted = [&](const Tile& t) {
    const int r0 = __builtin_amdgcn_readfirstlane(t.r0);
    const int mrows = __builtin_amdgcn_readfirstlane(t.r1 - t.r0);
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(C + (size_t)r0 * ldc, 0, (int)((uint32_t)mrows * (uint32_t)ldc * 2u),
                                          0x00020000);
    __amdgpu_buffer_rsrc_t rg = rc;
    if constexpr (SAVE)
      rg = __builtin_amdgcn_make_buffer_rsrc(gu_out + (size_t)r0 * (2 * up_col), 0,
                                             (int)((uint32_t)mrows * (uint32_t)(2 * up_col) * 2u), 0x00020000);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = wm * (BM / WM) + mt * 16 + li;
      const bool row_ok = mt < vm && row < mrows;
      const uint32_t coff = (uint32_t)row * (uint32_t)ldc * 2u;
      if constexpr (GATED) {
        u32x2_t hp[NT / 2];
#pragma unroll
        for (int nt = 0; nt < NT / 2; ++nt) {
          float hv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gv = acc[mt][nt][j], uv = acc[mt][nt + NT / 2][j];
            hv[j] = swiglu_f32(gv, uv);
          }
          hp[nt] = u32x2_t{pack2(hv[0], hv[1]), pack2(hv[2], hv[3])};
        }
#pragma unroll
        for (int q = 0; q < NT / 2; q += 2) {
          const int colP = t.nb * (BN / 2) + wn * (BN / 2 / WN) + q * 16;
          store_pair_buf(rc, coff, row_ok && colP < Nout, colP, hp[q], hp[q + 1]);
        }
        if constexpr (SAVE) {
          const uint32_t goff = (uint32_t)row * (uint32_t)(2 * up_col) * 2u;
#pragma unroll
          for (int q = 0; q < NT / 2; q += 2) {
            const int colP = t.nb * (BN / 2) + wn * (BN / 2 / WN) + q * 16;
            const f32x4_t g0 = acc[mt][q], g1 = acc[mt][q + 1];
            const f32x4_t u0 = acc[mt][q + NT / 2], u1 = acc[mt][q + 1 + NT / 2];
            store_pair_buf(rg, goff, row_ok && colP < Nout, colP, u32x2_t{pack2(g0[0], g0[1]), pack2(g0[2], g0[3])},
                           u32x2_t{pack2(g1[0], g1[1]), pack2(g1[2], g1[3])});
            store_pair_buf(rg, goff + (uint32_t)up_col * 2u, row_ok && colP < Nout, colP,
                           u32x2_t{pack2(u0[0], u0[1]), pack2(u0[2], u0[3])},
                           u32x2_t{pack2(u1[0], u1[1]), pack2(u1[2], u1[3])});
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < NT; q += 2) {
          const f32x4_t u = acc[mt][q], v = acc[mt][q + 1];
          const int colP = t.nb * BN + wn * (BN / WN) + q * 16;
          store_pair_buf(rc, coff, row_ok && colP < Nout, colP, u32x2_t{pack2(u[0], u[1]), pack2(u[2], u[3])},
                         u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])});
        }
      }
    }
  };
  auto store_tile = [&](const Tile& t) {
    if constexpr (ST_COUNTED)
      store_tile_counted(t);
    else
      store_tile_plain(t);
  };

  // IDS: stage the ids and place the pairs (every workgroup; workgroup 0 also
  // writes the metadata) before the first tile is looked up.
  if constexpr (IDS) {
    const int total = n_a * topk;  // <= kIdsMaxPairs (checked by the launcher)
    for (int f = tid; f < total; f += 64 * NW) ids_l[f] = im.ids[f];
    place_pairs<NW>(ids_l, total, E, im.ep, im.id_bits, cnt_l, offs_l, perm_l,
                    PlaceOut{blockIdx.x == 0, im.counts, im.offsets, im.splits, im.perm, im.inv});
    __syncthreads();
  }
  // Persistent loop over this workgroup's tiles. Before the epilogue of a
  // tile, the first NSTAGE-1 k-steps of the next one are put in flight (the
  // barrier after the main loop frees the whole ring), so the DMA of the
  // next tile and the stores of this one overlap.
  Tile t = next_tile();
  if (!t.valid) return;
  set_sources(t);
  issue_first();
  bool after_st = false;
  for (;;) {
    if constexpr (SCATTER) load_scatter(t);
    const int mrows = __builtin_amdgcn_readfirstlane(t.r1 - t.r0);
    vm = min(MT, max(0, (mrows - wm * (BM / WM) + 15) / 16));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (vm == MT)
      main_loop(true, after_st);
    else
      main_loop(false, after_st);
    __syncthreads();
    const Tile nt_ = next_tile();
    if (nt_.valid) {
      set_sources(nt_);
      issue_first();
    }
    store_tile(t);
    if (!nt_.valid) break;
    t = nt_;
    after_st = true;
  }
}

// fp32: one thread per output element; lanes run along the output columns.
template <bool GATED, bool GATHER, bool SCATTER, bool SAVE = false>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                      const int32_t* __restrict__ perm, int topk, int n_a,
                                                      const float* __restrict__ wrow,
                                                      const int32_t* __restrict__ offsets, int E, int rows,
                                                      int Kdim, const float* __restrict__ B, int ldb,
                                                      long long b_expert_stride, int Nout, int up_col,
                                                      float* __restrict__ C, int ldc, float* __restrict__ gu_out) {
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
  if constexpr (GATED) {
    C[(size_t)row * ldc + col] = gsum / (1.f + expf(-gsum)) * usum;
    if constexpr (SAVE) {
      gu_out[(size_t)row * 2 * up_col + col] = gsum;
      gu_out[(size_t)row * 2 * up_col + up_col + col] = usum;
    }
  } else if constexpr (SCATTER) {
    const int f = perm[row];
    if ((unsigned)f < (unsigned)n_a) C[(size_t)f * ldc + col] = wrow[f] * gsum;
  } else {
    C[(size_t)row * ldc + col] = gsum;
  }
}

}  // namespace

namespace {

template <bool GATED, bool GATHER, bool SCATTER, int BM, int BK, int WM, int WN, bool SAVE, bool BPK>
void launch_cfg(const void* a, const int32_t* perm, int topk, int n_a, const float* wrow, const int32_t* offsets,
                int E, int rows, int Kdim, const void* B, int ldb, long long bstride, int Nout, int up_col, void* C,
                int ldc, int NB, void* gu_out, hipStream_t s) {
  const int n_slots = max_row_tiles(rows, E, BM) * NB;
  const int grid = std::min(n_slots, stream_cu_count(s));
  gemm_bf16_kernel<GATED, GATHER, SCATTER, BM, BK, WM, WN, SAVE, false, BPK><<<grid, 64 * WM * WN, 0, s>>>(
      (const uint16_t*)a, perm, topk, n_a, wrow, offsets, E, rows, Kdim, (const uint16_t*)B, ldb, bstride, Nout,
      up_col, (uint16_t*)C, ldc, NB, n_slots, (uint16_t*)gu_out, IdsMeta{});
}

// BPK: B is in the packed form (ldb = NB * 256, bstride unused).
template <bool GATED, bool GATHER, bool SCATTER = false, bool SAVE = false, bool BPK = false>
void launch_bf16(const void* a, const int32_t* perm, int topk, int n_a, const int32_t* offsets, int E, int rows,
                 int Kdim, const void* B, int ldb, long long bstride, int Nout, int up_col, void* C, int ldc, int NB,
                 hipStream_t s, const float* wrow = nullptr, void* gu_out = nullptr) {
  if ((long long)rows <= (long long)kSmallRowsPerExpert * E)
    launch_cfg<GATED, GATHER, SCATTER, kSmallBM, kSmallBK, kSmallWM, kSmallWN, SAVE, BPK>(
        a, perm, topk, n_a, wrow, offsets, E, rows, Kdim, B, ldb, bstride, Nout, up_col, C, ldc, NB, gu_out, s);
  else
    launch_cfg<GATED, GATHER, SCATTER, kBM, GATED ? kBK1 : kBK, kGemmWM, kGemmWN, SAVE, BPK>(
        a, perm, topk, n_a, wrow, offsets, E, rows, Kdim, B, ldb, bstride, Nout, up_col, C, ldc, NB, gu_out, s);
}

template <bool GATHER, bool SAVE = false>
hipError_t w13_impl(const void* a, const int32_t* perm, int topk, int n_a, const int32_t* offsets, int rows,
                    const void* W13, int E, int H, int I, moe_dtype dt, void* h, hipStream_t s,
                    void* gu_out = nullptr, bool packed = false) {
  if (rows == 0) return hipSuccess;
  if (packed && dt != MOE_BF16) return hipErrorInvalidValue;
  if (packed) {
    const int NB = ceil_div(I, BN / 2);
    launch_bf16<true, GATHER, false, SAVE, true>(a, perm, topk, n_a, offsets, E, rows, H, W13, NB * 256, 0, I, I, h,
                                                 I, NB, s, nullptr, gu_out);
  } else if (dt == MOE_BF16) {
    launch_bf16<true, GATHER, false, SAVE>(a, perm, topk, n_a, offsets, E, rows, H, W13, 2 * I,
                                           (long long)H * 2 * I, I, I, h, I, ceil_div(I, BN / 2), s, nullptr,
                                           gu_out);
  } else {
    dim3 g1(ceil_div(I, 64), ceil_div(rows, 4));
    gemm_f32_kernel<true, GATHER, false, SAVE><<<g1, 256, 0, s>>>(
        (const float*)a, perm, topk, n_a, nullptr, offsets, E, rows, H, (const float*)W13, 2 * I,
        (long long)H * 2 * I, I, I, (float*)h, I, (float*)gu_out);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_w13_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13, int E, int H,
                             int I, moe_dtype dt, void* h, hipStream_t s) {
  return w13_impl<false>(x_perm, nullptr, 1, rows, offsets, rows, W13, E, H, I, dt, h, s);
}

hipError_t launch_w13_swiglu_gather(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                    const void* W13, int E, int H, int I, moe_dtype dt, void* h, hipStream_t s,
                                    bool packed) {
  return w13_impl<true>(x, perm, K, n, offsets, n * K, W13, E, H, I, dt, h, s, nullptr, packed);
}

hipError_t launch_w13_swiglu_gather_train(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                          const void* W13, int E, int H, int I, moe_dtype dt, void* h, void* gate_up,
                                          hipStream_t s) {
  return w13_impl<true, true>(x, perm, K, n, offsets, n * K, W13, E, H, I, dt, h, s, gate_up);
}

bool w13_from_ids_ok(int n, int K, int E, moe_dtype dt) {
  return dt == MOE_BF16 && n > 0 && n <= kSmallBM && (long long)n * K <= kIdsMaxPairs && E <= kMaxExperts &&
         (long long)n * K <= (long long)kSmallRowsPerExpert * E;
}

hipError_t launch_w13_swiglu_from_ids(const void* x, const int32_t* ids, int n, int K, const void* W13, int E,
                                      int H, int I, int ep, void* h, int32_t* counts, int32_t* offsets,
                                      int32_t* splits, int32_t* perm, int32_t* inv, hipStream_t s, bool packed) {
  if (!w13_from_ids_ok(n, K, E, MOE_BF16) || ep <= 0 || E % ep != 0) return hipErrorInvalidValue;
  int id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  const int NB = ceil_div(I, BN / 2);
  const int n_slots = E * NB;
  const int grid = std::min(n_slots, stream_cu_count(s));
  const IdsMeta im{ids, counts, offsets, splits, perm, inv, ep, id_bits};
  if (packed)
    gemm_bf16_kernel<true, true, false, kSmallBM, kSmallBK, kSmallWM, kSmallWN, false, true, true>
        <<<grid, 64 * kSmallWM * kSmallWN, 0, s>>>((const uint16_t*)x, nullptr, K, n, nullptr, nullptr, E, n * K, H,
                                                   (const uint16_t*)W13, NB * 256, 0, I, I, (uint16_t*)h, I, NB,
                                                   n_slots, nullptr, im);
  else
    gemm_bf16_kernel<true, true, false, kSmallBM, kSmallBK, kSmallWM, kSmallWN, false, true>
        <<<grid, 64 * kSmallWM * kSmallWN, 0, s>>>((const uint16_t*)x, nullptr, K, n, nullptr, nullptr, E, n * K, H,
                                                   (const uint16_t*)W13, 2 * I, (long long)H * 2 * I, I, I,
                                                   (uint16_t*)h, I, NB, n_slots, nullptr, im);
  return hipGetLastError();
}

hipError_t launch_w2(const void* h, const int32_t* offsets, int rows, const void* W2, int E, int H, int I,
                     moe_dtype dt, void* Y_perm, hipStream_t s, bool packed) {
  if (rows == 0) return hipSuccess;
  if (packed && dt != MOE_BF16) return hipErrorInvalidValue;
  if (packed) {
    const int NB = ceil_div(H, BN);
    launch_bf16<false, false, false, false, true>(h, nullptr, 1, rows, offsets, E, rows, I, W2, NB * 256, 0, H, 0,
                                                  Y_perm, H, NB, s);
  } else if (dt == MOE_BF16) {
    launch_bf16<false, false>(h, nullptr, 1, rows, offsets, E, rows, I, W2, H, (long long)I * H, H, 0, Y_perm, H,
                              ceil_div(H, BN), s);
  } else {
    dim3 g2(ceil_div(H, 64), ceil_div(rows, 4));
    gemm_f32_kernel<false, false, false><<<g2, 256, 0, s>>>((const float*)h, nullptr, 1, rows, nullptr, offsets, E,
                                                            rows, I, (const float*)W2, H, (long long)I * H, H, 0,
                                                            (float*)Y_perm, H, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_w2_scatter(const void* h, const int32_t* offsets, int rows, const int32_t* perm,
                             const float* topk_w, const void* W2, int E, int H, int I, moe_dtype dt, void* Y_tok,
                             hipStream_t s, bool packed) {
  if (rows == 0) return hipSuccess;
  if (packed && dt != MOE_BF16) return hipErrorInvalidValue;
  if (packed) {
    const int NB = ceil_div(H, BN);
    launch_bf16<false, false, true, false, true>(h, perm, 1, rows, offsets, E, rows, I, W2, NB * 256, 0, H, 0, Y_tok,
                                                 H, NB, s, topk_w);
  } else if (dt == MOE_BF16) {
    launch_bf16<false, false, true>(h, perm, 1, rows, offsets, E, rows, I, W2, H, (long long)I * H, H, 0, Y_tok, H,
                                    ceil_div(H, BN), s, topk_w);
  } else {
    dim3 g2(ceil_div(H, 64), ceil_div(rows, 4));
    gemm_f32_kernel<false, false, true><<<g2, 256, 0, s>>>((const float*)h, perm, 1, rows, topk_w, offsets, E, rows,
                                                           I, (const float*)W2, H, (long long)I * H, H, 0,
                                                           (float*)Y_tok, H, nullptr);
  }
  return hipGetLastError();
}

namespace {

// One workgroup per 32-deep unit (expert e, unit u, column block nb); thread c
// writes column c of the block: its 32 k-values as four 16-byte chunks at
// their swizzled slots. Gated (half = I > 0): columns 0-127 are the gate
// columns nb * 128 + c, 128-255 the matching up columns I + nb * 128 + c - 128;
// otherwise column nb * 256 + c. Columns past the matrix are zero.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ W, int Kdim, int Ncols,
                                                           int NB, int half, uint16_t* __restrict__ out) {
  const int units = Kdim / 32;
  const int nb = blockIdx.x % NB;
  const int eu = blockIdx.x / NB;  // e * units + u
  const int u = eu % units, e = eu / units;
  const int c = threadIdx.x;
  int col;
  bool ok;
  if (half > 0) {
    const int j = nb * 128 + (c & 127);
    ok = j < half;
    col = (c < 128) ? j : half + j;
  } else {
    col = nb * 256 + c;
    ok = col < Ncols;
  }
  const uint16_t* src = W + (size_t)e * Kdim * Ncols + (size_t)u * 32 * Ncols + (ok ? col : 0);
  uint16_t* dst = out + (size_t)blockIdx.x * kPackUnit + c * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = ok ? src[(size_t)(8 * q + 2 * i) * Ncols] : 0u;
      const uint32_t hi = ok ? src[(size_t)(8 * q + 2 * i + 1) * Ncols] : 0u;
      w[i] = lo | (hi << 16);
    }
    *(u32x4_t*)(dst + ((q ^ ((c >> 1) & 3)) << 3)) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

}  // namespace

size_t packed_weight_bytes(int E, int Kdim, int NB) { return (size_t)E * NB * (Kdim / 32) * kPackUnitBytes; }

hipError_t launch_pack_weights(const void* W, int E, int Kdim, int Ncols, int half, int NB, void* out,
                               hipStream_t s) {
  if (E <= 0 || Kdim % 32 != 0 || Kdim <= 0 || NB <= 0) return hipErrorInvalidValue;
  const long long blocks = (long long)E * NB * (Kdim / 32);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  pack_weights_kernel<<<(int)blocks, 256, 0, s>>>((const uint16_t*)W, Kdim, Ncols, NB, half, (uint16_t*)out);
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
