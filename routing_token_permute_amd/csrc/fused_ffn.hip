// Persistent single-kernel expert FFN: GEMM1 + SwiGLU ("L1") and GEMM2
// ("L2") of Algorithm 2 steps 8-9 ("MoE 分布式推理基础（基于 vLLM）" §1.2) in
// one launch, scheduled the way "大模型系统中的通算融合" §4.4 describes the
// Mega MoE scheduler, restated for one GPU:
//   * Tasks are L1 tiles (a row tile of an expert x 128 gate columns with
//     their 128 up columns) and L2 tiles (the same row tile x 256 output
//     columns). An L2 tile needs every L1 tile of its row tile.
//   * Each XCD has its own task queue (an atomic ticket counter) over a
//     contiguous range of the row tiles; a workgroup takes tickets from the
//     queue of the XCD it was dispatched to and, once that queue is empty,
//     from the others. A queue first hands out the L1 tiles of `warm` row
//     tiles (the warm-up), then alternates the L1 tiles of row tile
//     s + warm with the L2 tiles of row tile s.
//   * h goes to a ring pool of `pool` row-tile slots per queue (0: no ring,
//     h at its expert-major rows): the L1 tiles of a queue's row tile s
//     write slot s % pool once the L2 tiles of row tile s - pool have read
//     it, so h never needs a buffer for all rows.
//   * Readiness is counted per row tile. An L1 tile writes its h rows with
//     device-scope (sc1, write-through) stores, which is how agent-scope
//     atomic stores are made on this chip, so no L2 write-back is needed:
//     once every wave's stores have completed (vmcnt 0) and the workgroup
//     has met at a barrier, one atomic increment of ready[m] publishes them.
//     An L2 tile waits until ready[m] counts every L1 tile of its row tile;
//     then one wave acquires at agent scope (invalidating this CU's L1 and
//     the XCD's L2 of lines that may be stale, for the whole workgroup)
//     before the barrier after which the waves copy h. Measured on the OLMoE
//     layer: a release with L2 write-back per L1 tile and an acquire in every
//     wave cost about a fifth of the kernel; device-scope loads of h in
//     place of the acquire (the copy's cache-policy bits) returned stale
//     rows. Every wait
//     targets a ticket of the same queue taken earlier, and a workgroup
//     publishes its current tile before it waits for the next, so the
//     earliest-taken unfinished ticket can always proceed: no deadlock,
//     whatever the number of resident workgroups. Each wait is bounded all
//     the same; a bound that runs out sets a flag word and the kernel ends
//     (with wrong results) instead of hanging.
// The tiles, operand layouts and the k-step pipeline are those of the bf16
// grouped GEMM (gemm_tiles.hpp): 256 x 256 tiles, 16 waves of 64 x 64, a
// 3-deep ring of 32-deep k-steps copied HBM -> LDS with
// global_load_lds_dwordx4, the row gather of GEMM1 fused into its copy, the
// SwiGLU epilogue in fp32 and bf16 (nearest even) outputs. Each output is the
// same sequence of fp32 operations as in the two-launch path, so the results
// are bitwise equal to it.
#include <algorithm>
#include <type_traits>

#include "gemm_tiles.hpp"

namespace moe {
namespace {

constexpr int kFBM = 256, kFBK = 32, kFWM = 4, kFWN = 4;
constexpr int kQueues = 8;           // one per XCD
constexpr int kSpinLimit = 1 << 20;  // polls of a bounded wait (each with a short sleep)

// Counters (int32, zeroed before each launch): kQueues ticket heads, then
// ready[Mmax], consumed[Mmax], then one flag word.
__host__ __device__ inline int fused_counter_words(int Mmax) { return kQueues + 2 * Mmax + 1; }

struct FTask {
  int kind;  // 0 none, 1 L1, 2 L2
  int q, mloc, m, nb;
};

// Rows [b0, b1) of the row-tile range of queue q.
__device__ __forceinline__ int queue_base(int M, int q) { return (int)((long long)M * q / kQueues); }

__device__ __forceinline__ int queue_tasks(int M, int q, int NB1, int NB2) {
  return (queue_base(M, q + 1) - queue_base(M, q)) * (NB1 + NB2);
}

// Ticket j of queue q -> task. Order: the L1 tiles of the first Wq row tiles,
// then segments s = 0, 1, ...: the L1 tiles of row tile Wq + s (while there is
// one), then the L2 tiles of row tile s.
__device__ FTask decode_task(int q, int j, int M, int NB1, int NB2, int W) {
  const int b0 = queue_base(M, q), Mq = queue_base(M, q + 1) - b0, Wq = min(W, Mq);
  FTask t{0, q, 0, 0, 0};
  if (j < Wq * NB1) {
    t.kind = 1;
    t.mloc = j / NB1;
    t.nb = j % NB1;
  } else {
    const int j2 = j - Wq * NB1, S = NB1 + NB2, nseg = Mq - Wq;
    if (j2 < nseg * S) {
      const int s = j2 / S, o = j2 % S;
      if (o < NB1) {
        t.kind = 1;
        t.mloc = Wq + s;
        t.nb = o;
      } else {
        t.kind = 2;
        t.mloc = s;
        t.nb = o - NB1;
      }
    } else {
      const int j3 = j2 - nseg * S;
      t.kind = 2;
      t.mloc = nseg + j3 / NB2;
      t.nb = j3 % NB2;
    }
  }
  t.m = b0 + t.mloc;
  return t;
}

// Row tiles of all experts (the count find_tile walks), computed by a wave.
template <int BM>
__device__ int count_row_tiles(const int32_t* __restrict__ offsets, int E, int rows) {
  const int lane = lane_id();
  int tot = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int c = 0;
    if (e < E) {
      const int a = min(max(offsets[e], 0), rows);
      const int b = min(max(offsets[e + 1], a), rows);
      c = (b - a + BM - 1) / BM;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
    tot += c;
  }
  return tot;
}

// Thread-level bounded wait until *c >= target; false when the bound ran out.
__device__ bool wait_at_least(int* c, int target) {
  for (int i = 0; i < kSpinLimit; ++i) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// BPK: W13 and W2 in the packed form (per expert and 32 K rows, one 16 KB unit
// per 256-column block; see the grouped GEMM): a stage's B part is one unit,
// read with ds_read_b128; the arithmetic and its order are unchanged.
template <bool BPK>
__global__ __launch_bounds__(64 * kFWM * kFWN, 1) void fused_ffn_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, int topk, int n_a,
    const int32_t* __restrict__ offsets, int E, int rows, const uint16_t* __restrict__ W13,
    const uint16_t* __restrict__ W2, int H, int I, uint16_t* __restrict__ hbuf, int P, uint16_t* __restrict__ Y,
    int* __restrict__ ctr, int Mmax, int W) {
  constexpr int BM = kFBM, BK = kFBK, WM = kFWM, WN = kFWN;
  using Cfg = TileCfg<BM, BK, 3>;
  constexpr int A_BYTES = Cfg::A_BYTES, STAGE = Cfg::STAGE, NSTAGE = Cfg::NSTAGE, A_ROW = Cfg::A_ROW;
  constexpr int KS = BK / 32, NW = WM * WN, MT = BM / WM / 16, NT = BN / WN / 16;
  constexpr int REG = Cfg::REGIONS / NW, DMA_PER_STAGE = REG, A_REG = A_BYTES / 1024;
  constexpr int ST = MT * (NT / 2);  // L2 epilogue buffer stores per wave and tile
  static_assert(NSTAGE == 3 && DMA_PER_STAGE + ST <= 63 && NT == 4, "tile split / vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem_raw[Cfg::LDS_BYTES];
  __shared__ int s_bc[4];
  lds_char_t* smem = (lds_char_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t wave_u = wave;
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, li = lane & 15, rr = li >> 2, cc = li & 3;
  const int NB1 = (I + BN / 2 - 1) / (BN / 2), NB2 = (H + BN - 1) / BN;
  const int M = __builtin_amdgcn_readfirstlane(min(count_row_tiles<BM>(offsets, E, rows), Mmax));
  int* heads = ctr;
  int* ready = ctr + kQueues;
  int* consumed = ready + Mmax;
  int* flag = consumed + Mmax;

  // Ticket fetch (thread 0): the home queue first, then the others.
  const int home = blockIdx.x % kQueues;
  uint32_t exhausted = 0;
  auto fetch = [&]() -> int {
    for (int k = 0; k < kQueues; ++k) {
      const int q = (home + k) % kQueues;
      if ((exhausted >> q) & 1u) continue;
      const int Tq = queue_tasks(M, q, NB1, NB2);
      if (Tq > 0) {
        const int j = __hip_atomic_fetch_add(&heads[q], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (j < Tq) return (q << 24) | j;
      }
      exhausted |= 1u << q;
    }
    return -1;
  };
  auto decode = [&](int tk) {
    if (tk < 0) return FTask{0, 0, 0, 0, 0};
    return decode_task(tk >> 24, tk & 0xFFFFFF, M, NB1, NB2, W);
  };
  auto bounded_wait = [&](int* c, int target) {  // thread 0
    if (!wait_at_least(c, target)) __hip_atomic_fetch_or(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // h rows of a task's row tile: its ring slot, or its expert-major rows.
  auto h_rows = [&](const FTask& t, const Tile& tt) {
    return P > 0 ? hbuf + (size_t)(t.q * P + t.mloc % P) * BM * I : hbuf + (size_t)tt.r0 * I;
  };

  // HBM -> LDS assignment (as in the grouped GEMM): the first A_REG 1 KB
  // regions hold A rows, the rest two k-rows of B each.
  const uint16_t* src[REG];
  int ldb = 0, nk = 0;
  auto set_sources = [&](const FTask& t, const Tile& tt) {
    const int mrows = tt.r1 - tt.r0;
    const bool l1 = t.kind == 1;
    const int nbl = l1 ? (I + BN / 2 - 1) / (BN / 2) : (H + BN - 1) / BN;  // column blocks of the task's weights
    ldb = BPK ? nbl * 256 : (l1 ? 2 * I : H);
    nk = (l1 ? H : I) / BK;
    const uint16_t* hb = l1 ? nullptr : h_rows(t, tt);
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const int r = wave * REG + j;
      if (r < A_REG) {
        constexpr int CPR = A_ROW / 16;
        const int row = Cfg::A_ROWS_PER_REGION * r + lane / CPR;
        const int c = (lane % CPR) ^ a_swz<BK>(row);
        const int lr = min(row, mrows - 1);
        if (l1) {
          const int f = perm[tt.r0 + lr];
          const int arow = ((unsigned)f < (unsigned)(n_a * topk)) ? f / topk : 0;
          src[j] = x + (size_t)arow * H + c * 8;
        } else {
          src[j] = hb + (size_t)lr * I + c * 8;
        }
      } else if constexpr (BPK) {  // one 16 KB unit: a straight copy
        const int rb = r - A_REG;
        const uint16_t* wb = l1 ? W13 + (size_t)tt.e * (H / 32) * nbl * kPackUnit
                                : W2 + (size_t)tt.e * (I / 32) * nbl * kPackUnit;
        src[j] = wb + (size_t)t.nb * kPackUnit + rb * 512 + lane * 8;
      } else {
        const int k = 2 * (r - A_REG) + (lane >> 5);
        const int c = (lane & 31) ^ b_swz(k);
        if (l1) {
          int gc = t.nb * (BN / 2) + (c & 15) * 8;
          if (gc >= I) gc = 0;
          const int col = (c < 16) ? gc : I + gc;
          src[j] = W13 + (size_t)tt.e * H * 2 * I + (size_t)k * ldb + col;
        } else {
          int col = t.nb * BN + c * 8;
          if (col >= H) col = 0;
          src[j] = W2 + (size_t)tt.e * I * H + (size_t)k * ldb + col;
        }
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
      dma16(src[j] + (r < A_REG ? ka : kb), base + j * 1024);
    }
  };
  auto issue_first = [&]() {
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < nk) issue(p, p);
  };

  const int a_sw = a_swz<BK>(li);
  const int a_lane = (wm * (BM / WM) + li) * A_ROW;
  const int a_c0 = (g ^ a_sw) << 4, a_c1 = ((4 + g) ^ a_sw) << 4;
  const int bsw = b_swz(g * 8 + rr);
  const int b_lane = (g * 8 + rr) * B_ROW + cc * 8;
  int b_col[NT];
  auto set_bcol = [&](bool gated) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col0 = gated ? ((nt < NT / 2) ? (wn * (BN / 2 / WN) + nt * 16)
                                              : (BN / 2 + wn * (BN / 2 / WN) + (nt - NT / 2) * 16))
                             : wn * (BN / WN) + nt * 16;
      b_col[nt] = BPK ? (col0 + li) * 64 + ((g ^ ((li >> 1) & 3)) << 4) : b_lane + (((col0 >> 3) ^ bsw) << 4);
    }
  };

  f32x4_t acc[MT][NT];
  int vm = 0;
  using AOps = bf16x8_t[KS][MT];
  using BOps = bf16x8_t[KS][NT];
  auto load_ops = [&](int stage, bool full, AOps& a, BOps& b) {
    const lds_char_t* As = smem + stage * STAGE;
    const lds_char_t* Bs = As + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (BPK) {
          b[ks][nt] = __builtin_bit_cast(bf16x8_t, lds_read_b128(Bs + ks * kPackUnitBytes + b_col[nt]));
        } else {
          const lds_char_t* p = Bs + b_col[nt] + ks * 32 * B_ROW;
          const bf16x4_t lo = lds_read_tr16(p);
          const bf16x4_t hi = lds_read_tr16(p + 4 * B_ROW);
          b[ks][nt] = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (full || mt < vm)
          a[ks][mt] = __builtin_bit_cast(bf16x8_t, lds_read_b128(As + a_lane + mt * 16 * A_ROW + (ks ? a_c1 : a_c0)));
    }
  };
  auto mma = [&](bool full, const AOps& a, const BOps& b) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (full || mt < vm) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[ks][nt], a[ks][mt], acc[mt][nt], 0, 0, 0);
        }
  };
  // Waits: at most `stages` later k-steps of this wave in flight; the _st
  // form also lets the previous L2 tile's ST stores (issued after this tile's
  // first k-steps) stay outstanding.
  auto wait_dma = [&](int stages) {
    if (stages >= 1)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DMA_PER_STAGE) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  };
  auto wait_dma_st = [&](int stages) {
    if (stages >= 1)
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(DMA_PER_STAGE + ST) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(ST) : "memory");
  };
  auto main_loop = [&](bool full, bool after_st) {
    int slot = 0;
    for (int kt = 0; kt < nk; ++kt) {
      if (after_st && kt <= NSTAGE - 2)
        wait_dma_st(min(NSTAGE - 2, nk - 1 - kt));
      else
        wait_dma(min(NSTAGE - 2, nk - 1 - kt));
      __syncthreads();
      if (kt + NSTAGE - 1 < nk) issue(kt + NSTAGE - 1, slot == 0 ? NSTAGE - 1 : slot - 1);
      if (full || vm > 0) {
        AOps a;
        BOps b;
        load_ops(slot, full, a, b);
        mma(full, a, b);
      }
      slot = (slot == NSTAGE - 1) ? 0 : slot + 1;
    }
  };

  // Epilogue stores: lanes g and g^1 of adjacent 16-column tiles swap halves
  // so that each lane writes 8 consecutive bf16 values with one 16-byte
  // buffer store; lanes without a valid output send an offset past the
  // resource, which the hardware drops.
  auto pack2 = [](float v0, float v1) {
    return (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
  };
  const bool odd = (g & 1) != 0;
  constexpr uint32_t kDropped = 0x80000000u;
  // Cache policy of a store: 0, or kDeviceScope (sc1: written through to
  // the device-coherent level before the store completes).
  constexpr int kDeviceScope = 16;
  auto store_pair_buf = [&](__amdgpu_buffer_rsrc_t rs, uint32_t rowoff, bool ok, int colP, u32x2_t pP, u32x2_t pQ,
                            auto policy) {
    const u32x2_t send = odd ? pP : pQ;
    const u32x2_t got{(uint32_t)__shfl_xor((int)send[0], 16), (uint32_t)__shfl_xor((int)send[1], 16)};
    const int col = odd ? colP + 16 + 4 * (g - 1) : colP + 4 * g;
    const u32x4_t v = odd ? u32x4_t{got[0], got[1], pQ[0], pQ[1]} : u32x4_t{pP[0], pP[1], got[0], got[1]};
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, ok ? rowoff + (uint32_t)col * 2u : kDropped, 0, decltype(policy)::value);
  };
  // L1: h = SiLU(gate) * up into the task's h rows (row stride I).
  auto store_l1 = [&](const FTask& t, const Tile& tt) {
    const int mrows = __builtin_amdgcn_readfirstlane(tt.r1 - tt.r0);
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(h_rows(t, tt), 0, (int)((uint32_t)mrows * (uint32_t)I * 2u), 0x00020000);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = wm * (BM / WM) + mt * 16 + li;
      const bool row_ok = mt < vm && row < mrows;
      const uint32_t coff = (uint32_t)row * (uint32_t)I * 2u;
      u32x2_t hp[NT / 2];
#pragma unroll
      for (int nt = 0; nt < NT / 2; ++nt) {
        float hv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) hv[j] = swiglu_f32(acc[mt][nt][j], acc[mt][nt + NT / 2][j]);
        hp[nt] = u32x2_t{pack2(hv[0], hv[1]), pack2(hv[2], hv[3])};
      }
      const int colP = t.nb * (BN / 2) + wn * (BN / 2 / WN);
      store_pair_buf(rc, coff, row_ok && colP < I, colP, hp[0], hp[1], std::integral_constant<int, kDeviceScope>{});
    }
  };
  // L2: Y rows of the row tile (expert-major, row stride H).
  auto store_l2 = [&](const FTask& t, const Tile& tt) {
    const int r0 = __builtin_amdgcn_readfirstlane(tt.r0);
    const int mrows = __builtin_amdgcn_readfirstlane(tt.r1 - tt.r0);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        Y + (size_t)r0 * H, 0, (int)((uint32_t)mrows * (uint32_t)H * 2u), 0x00020000);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = wm * (BM / WM) + mt * 16 + li;
      const bool row_ok = mt < vm && row < mrows;
      const uint32_t coff = (uint32_t)row * (uint32_t)H * 2u;
#pragma unroll
      for (int q = 0; q < NT; q += 2) {
        const f32x4_t u = acc[mt][q], v = acc[mt][q + 1];
        const int colP = t.nb * BN + wn * (BN / WN) + q * 16;
        store_pair_buf(rc, coff, row_ok && colP < H, colP, u32x2_t{pack2(u[0], u[1]), pack2(u[2], u[3])},
                       u32x2_t{pack2(v[0], v[1]), pack2(v[2], v[3])}, std::integral_constant<int, 0>{});
      }
    }
  };
  // Agent-scope acquire for the workgroup: one wave invalidates (the L1 is
  // per CU, the L2 per XCD) and waits for it before the barrier that follows.
  auto acquire = [&]() {
    if (wave == 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    }
  };
  auto row_tile = [&](const FTask& t) {
    Tile r = find_tile<BM>(offsets, E, rows, 1, t.m);
    r.e = __builtin_amdgcn_readfirstlane(r.e);
    r.r0 = __builtin_amdgcn_readfirstlane(r.r0);
    r.r1 = __builtin_amdgcn_readfirstlane(r.r1);
    return r;
  };

  // First task.
  if (tid == 0) s_bc[0] = fetch();
  __syncthreads();
  FTask t = decode(__builtin_amdgcn_readfirstlane(s_bc[0]));
  if (t.kind == 0) return;
  if (t.kind == 2) {
    if (tid == 0) bounded_wait(&ready[t.m], NB1);
    acquire();
    __syncthreads();
  }
  Tile tt = row_tile(t);
  set_bcol(t.kind == 1);
  set_sources(t, tt);
  issue_first();
  bool after_st = false;
  for (;;) {
    // The next ticket, taken while this tile runs (read after the loop's
    // last barrier).
    if (tid == 0) s_bc[1] = fetch();
    const int mrows = __builtin_amdgcn_readfirstlane(tt.r1 - tt.r0);
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
    const FTask nx = decode(__builtin_amdgcn_readfirstlane(s_bc[1]));
    // Thread 0 decides for the workgroup whether the next tile's inputs are
    // ready now; an L2 tile that has copied its h rows releases its slot.
    int ready_now = 1;
    if (tid == 0) {
      if (t.kind == 2 && P > 0) __hip_atomic_fetch_add(&consumed[t.m], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ready_now = nx.kind != 2 ||
                  __hip_atomic_load(&ready[nx.m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= NB1;
      s_bc[2] = ready_now;
    }
    // Wave 0 holds thread 0's decision in its lane 0.
    if (nx.kind == 2 && wave == 0 && __builtin_amdgcn_readfirstlane(ready_now)) acquire();
    __syncthreads();
    const bool early = nx.kind != 0 && __builtin_amdgcn_readfirstlane(s_bc[2]) != 0;
    const int tkind = t.kind;
    Tile ntt{0, 0, 0, 0, false};
    if (early) ntt = row_tile(nx);
    if (tkind == 1) {
      // The ring slot must have been read by every L2 tile of its previous
      // row tile before it is overwritten.
      if (P > 0 && t.mloc >= P) {
        if (tid == 0) bounded_wait(&consumed[t.m - P], NB2);
        __syncthreads();
      }
      if (early) {
        set_bcol(nx.kind == 1);
        set_sources(nx, ntt);
        issue_first();
      }
      store_l1(t, tt);
      // Publish: every wave's write-through stores have completed, then the
      // count.
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(&ready[t.m], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (early) {
        set_bcol(nx.kind == 1);
        set_sources(nx, ntt);
        issue_first();
      }
      store_l2(t, tt);
    }
    if (nx.kind == 0) break;
    if (!early) {
      if (tid == 0) bounded_wait(&ready[nx.m], NB1);
      acquire();
      __syncthreads();
      ntt = row_tile(nx);
      set_bcol(nx.kind == 1);
      set_sources(nx, ntt);
      issue_first();
    }
    // The previous L2 tile's stores are younger than the next tile's first
    // k-steps only when those were issued first.
    after_st = early && tkind == 2;
    t = nx;
    tt = ntt;
  }
}

}  // namespace

int fused_ffn_max_row_tiles(int rows, int E) { return max_row_tiles(rows, E, kFBM); }

size_t fused_ffn_counter_bytes(int rows, int E) {
  return (size_t)fused_counter_words(fused_ffn_max_row_tiles(rows, E)) * 4;
}

size_t fused_ffn_h_bytes(int rows, int E, int I, int pool) {
  if (pool <= 0) return (size_t)rows * I * 2;
  return (size_t)kQueues * pool * kFBM * I * 2;
}

hipError_t launch_fused_ffn(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets, const void* W13,
                            const void* W2, int E, int H, int I, int warm, int pool, void* hbuf, void* Y_perm,
                            int* counters, hipStream_t s, bool packed) {
  const int rows = n * K;
  if (rows == 0) return hipSuccess;
  const int Mmax = fused_ffn_max_row_tiles(rows, E);
  hipError_t e = launch_fill_zero(counters, fused_ffn_counter_bytes(rows, E), s);
  if (e != hipSuccess) return e;
  const long long tasks = (long long)Mmax * (ceil_div(I, BN / 2) + ceil_div(H, BN));
  const int grid = (int)std::min<long long>(tasks, stream_cu_count(s));
  auto kern = packed ? fused_ffn_kernel<true> : fused_ffn_kernel<false>;
  kern<<<grid, 64 * kFWM * kFWN, 0, s>>>((const uint16_t*)x, perm, K, n, offsets, E, rows, (const uint16_t*)W13,
                                         (const uint16_t*)W2, H, I, (uint16_t*)hbuf, pool, (uint16_t*)Y_perm,
                                         counters, Mmax, warm);
  return hipGetLastError();
}

}  // namespace moe
