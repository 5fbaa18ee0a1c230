// Tile machinery shared by the forward and backward bf16 grouped GEMMs:
// LDS stage geometry, the two swizzled LDS layouts (K-contiguous rows read
// with ds_read_b128; k-rows of 256 columns read with the gfx950 transpose
// read), the direct HBM -> LDS copy, the device-side tile map over expert
// segments and the XCD-aware workgroup order.
#pragma once

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int BN = kGemmBN;
constexpr int B_ROW = BN * 2;             // bytes per staged k-row of B
static_assert(BN == 256, "LDS layouts below assume 256-column stages");

constexpr int kMaxStages = 5;

// Packed weights (moe_pack_w13 / moe_pack_w2): the K rows of each expert in
// units of 32 per 256-column output block. A unit is 256 columns x 32 k
// (16 KB), each column's 32 k-values contiguous (64 bytes, four 16-byte
// chunks), chunk q of column c at slot q ^ ((c / 2) % 4): the layout of the
// A tiles of a 32-deep stage, so that a stage's B part is a copy of whole
// units and B operands are read with ds_read_b128. Unit u of block nb of
// expert e starts at element ((e * (Kdim / 32) + u) * NB + nb) * kPackUnit:
// the NB blocks' units of one k-range sit side by side, so the tiles of one
// expert that run at the same time read neighbouring units (one block's units
// laid end to end put those streams exactly 1 MB apart at the OLMoE shape,
// and GEMM1 ran 11% slower).
constexpr int kPackUnit = 256 * 32;           // bf16 elements per unit
constexpr int kPackUnitBytes = kPackUnit * 2;  // 16 KB

// Stage geometry for a BM-row tile advancing BK (32 or 64) along K: A is
// BM x BK, B is BK x 256. As many stages as fit in 160 KB of LDS, at most
// CAP (all but one stay in flight while one is multiplied).
template <int BM, int BK, int CAP = kMaxStages>
struct TileCfg {
  static_assert(BK == 32 || BK == 64, "k-step");
  static constexpr int A_ROW = BK * 2;  // bytes per staged row of A
  static constexpr int A_BYTES = BM * A_ROW;
  static constexpr int B_BYTES = BK * B_ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int FIT = (160 * 1024) / STAGE;
  static constexpr int NSTAGE = FIT > CAP ? CAP : FIT;
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static constexpr int REGIONS = STAGE / 1024;  // 1 KB DMA regions per stage
  static constexpr int A_ROWS_PER_REGION = 1024 / A_ROW;
};

// A tile: BM rows x BK k (2 * BK bytes per row, in 16-byte chunks). Chunk c
// of row r sits at slot c ^ swz(r), swz(r) = (r / 2) % (chunks per row). With
// it, the wave-wide ds_read_b128 of one MFMA A operand (16 rows at the same
// chunk) runs at the full LDS rate of gfx950: 4 cycles per instruction,
// measured with a per-CU timing probe, where the (r / 4) % 4 form of the
// 64-byte rows takes 8. The DMA writes of a row are lane-linear and never
// collide.
template <int BK>
__device__ __forceinline__ int a_swz(int row) { return (row >> 1) & (BK / 8 - 1); }

// B tile: BK k-rows x 256 columns (512 B per row = 32 chunks). Chunk c of row
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

// The same copy with the non-temporal cache policy (nt): for data read once,
// such as the bf16 expert weights of a decode-sized batch, where each weight
// tile feeds a single row tile and each staged k-row is whole 128-byte lines.
// Streaming it past L2 without keeping it measured 11% faster on the decode
// GEMMs. It is slower where weights are reused by several row tiles (the
// large tiles keep the default policy), and where a line is read in two
// stages (the FP8 codes' 64-byte column pieces), whose second half then comes
// from HBM again.
__device__ __forceinline__ void dma16_stream(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
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

// Compute units of the current device (one persistent workgroup each),
// looked up once per device.
inline int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Compute units a launch on stream s can use: the stream's CU mask when it
// has one (hipExtStreamCreateWithCUMask), else the device's count. A
// persistent grid larger than this would leave workgroups waiting for a CU
// while the others hold their whole share of tiles.
inline int stream_cu_count(hipStream_t s) {
  const int dev_cus = device_cu_count();
  if (s == nullptr) return dev_cus;
  uint32_t mask[16] = {};
  if (hipExtStreamGetCUMask(s, 16, mask) != hipSuccess) {
    (void)hipGetLastError();
    return dev_cus;
  }
  int n = 0;
  for (int i = 0; i < 16; ++i) n += __builtin_popcount(mask[i]);
  return (n > 0 && n < dev_cus) ? n : dev_cus;
}

}  // namespace
}  // namespace moe
