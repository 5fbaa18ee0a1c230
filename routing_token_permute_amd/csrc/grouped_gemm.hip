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

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int NTHR = 256;
constexpr int A_BYTES = BM * BK * 2;      // 16 KB
constexpr int B_BYTES = BK * BN * 2;      // 16 KB
constexpr int STAGE = A_BYTES + B_BYTES;  // 32 KB
constexpr int LDS_BYTES = 2 * STAGE;      // 64 KB

// A tile: BM rows x 64 k (128 B per row, 8 chunks of 16 B). Chunk c of row r
// sits at slot c ^ ((r / 2) % 8): 16 consecutive rows reading the same chunk
// hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int a_off(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// B tile: 64 k-rows x 128 columns (256 B per row, 16 chunks). Chunk c of row
// k sits at slot c ^ 2 * ((k % 4) + 4 * ((k / 8) % 2)): the 32 lanes of a
// transpose read (8 k-rows x 4 eight-byte pieces) land on distinct banks.
__device__ __forceinline__ int b_off(int k, int chunk) {
  return k * 256 + ((chunk ^ (((k & 3) + ((k >> 3) & 1) * 4) << 1)) << 4);
}

struct Tile {
  int e, r0, r1;
  bool valid;
};

// Row tile `mb` -> (expert, rows [r0, r1)). Every wave computes it alike.
__device__ Tile find_tile(const int32_t* __restrict__ offsets, int E, int rows, int mb) {
  const int lane = lane_id();
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int a = 0, b = 0;
    if (e < E) {
      a = min(max(offsets[e], 0), rows);
      b = min(max(offsets[e + 1], a), rows);
    }
    const int t = (b - a + BM - 1) / BM;
    int incl = t;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int excl = incl - t;
    const bool hit = (t > 0) && (mb >= carry + excl) && (mb < carry + incl);
    const uint64_t bal = __ballot(hit);
    if (bal != 0) {
      const int L = __ffsll((long long)bal) - 1;
      const int ex = __shfl(excl, L), ah = __shfl(a, L), bh = __shfl(b, L);
      const int r0 = ah + (mb - carry - ex) * BM;
      return Tile{e0 + L, r0, min(r0 + BM, bh), true};
    }
    carry += __shfl(incl, 63);
  }
  return Tile{0, 0, 0, false};
}

template <bool GATED>
__global__ __launch_bounds__(NTHR, 2) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                           const int32_t* __restrict__ offsets, int E, int rows,
                                                           int Kdim, const uint16_t* __restrict__ B, int ldb,
                                                           long long b_expert_stride, int Nout, int up_col,
                                                           uint16_t* __restrict__ C, int ldc, int n_tiles_n) {
  __shared__ __attribute__((aligned(16))) char smem_raw[LDS_BYTES];
  lds_char_t* smem = (lds_char_t*)smem_raw;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int mb = blockIdx.x / n_tiles_n, nb = blockIdx.x % n_tiles_n;
  const Tile t = find_tile(offsets, E, rows, mb);
  if (!t.valid) return;
  const int mrows = t.r1 - t.r0;

  // Global -> register assignment. A: 8 threads per 128-byte row slice.
  const int ca = tid & 7, ra = tid >> 3;
  const uint16_t* a_ptr[4];
  bool a_ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = ra + 32 * j;
    a_ok[j] = r < mrows;
    a_ptr[j] = A + (size_t)(t.r0 + (a_ok[j] ? r : 0)) * Kdim + ca * 8;
  }
  // B: 16 threads per 256-byte k-row (gate half then up half for GEMM1).
  const int cb = tid & 15, kb = tid >> 4;
  int col;
  if constexpr (GATED)
    col = (cb < 8) ? (nb * 64 + cb * 8) : (up_col + nb * 64 + (cb - 8) * 8);
  else
    col = nb * 128 + cb * 8;
  const bool b_ok = GATED ? true : (col < Nout);
  const uint16_t* b_ptr = B + (size_t)t.e * b_expert_stride + (b_ok ? col : 0) + (size_t)kb * ldb;

  u32x4_t ra_reg[4], rb_reg[4];
  const u32x4_t zero4 = u32x4_t{0u, 0u, 0u, 0u};
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) ra_reg[j] = a_ok[j] ? *(const u32x4_t*)(a_ptr[j] + k0) : zero4;
#pragma unroll
    for (int j = 0; j < 4; ++j) rb_reg[j] = b_ok ? *(const u32x4_t*)(b_ptr + (size_t)(k0 + 16 * j) * ldb) : zero4;
  };
  auto sstore = [&](int buf) {
    lds_char_t* As = smem + buf * STAGE;
    lds_char_t* Bs = As + A_BYTES;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_write_b128(As + a_off(ra + 32 * j, ca), ra_reg[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_write_b128(Bs + b_off(kb + 16 * j, cb), rb_reg[j]);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, li = lane & 15, rr = li >> 2, cc = li & 3;
  int a_rd[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a_rd[mt][ks] = a_off(wm * 64 + mt * 16 + li, ks * 4 + g);
  int b_rd[4][2][2];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    int col0;
    if constexpr (GATED)
      col0 = (nt < 2) ? (wn * 32 + nt * 16) : (64 + wn * 32 + (nt - 2) * 16);
    else
      col0 = wn * 64 + nt * 16;
    const int c = col0 + 4 * cc;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) b_rd[nt][ks][h] = b_off(ks * 32 + g * 8 + h * 4 + rr, c >> 3) + (c & 7) * 2;
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = Kdim / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const lds_char_t* As = smem + buf * STAGE;
    const lds_char_t* Bs = As + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a[mt] = __builtin_bit_cast(bf16x8_t, lds_read_b128(As + a_rd[mt][ks]));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x4_t lo = lds_read_tr16(Bs + b_rd[nt][ks][0]);
        const bf16x4_t hi = lds_read_tr16(Bs + b_rd[nt][ks][1]);
        b[nt] = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane (g, li) of MFMA tile (mt, nt) holds rows 4g..4g+3, column li.
  uint16_t* Cs = (uint16_t*)smem_raw;
  if constexpr (GATED) {
    constexpr int P = 72;  // bf16 per staged row (64 + 8 pad)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = wm * 64 + mt * 16 + 4 * g + j;
          const int hc = wn * 32 + nt * 16 + li;
          const float gv = acc[mt][nt][j], uv = acc[mt][nt + 2][j];
          const float hv = gv / (1.f + __expf(-gv)) * uv;
          Cs[row * P + hc] = f32_to_bf16(hv);
        }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (tid >> 3) + 32 * j, c = tid & 7;
      if (row < mrows)
        *(u32x4_t*)(C + (size_t)(t.r0 + row) * ldc + nb * 64 + c * 8) = *(const u32x4_t*)(Cs + row * P + c * 8);
    }
  } else {
    constexpr int P = 136;  // 128 + 8 pad
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = wm * 64 + mt * 16 + 4 * g + j;
          const int c = wn * 64 + nt * 16 + li;
          Cs[row * P + c] = f32_to_bf16(acc[mt][nt][j]);
        }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = (tid >> 4) + 16 * j, c = tid & 15;
      const int gc = nb * 128 + c * 8;
      if (row < mrows && gc < Nout)
        *(u32x4_t*)(C + (size_t)(t.r0 + row) * ldc + gc) = *(const u32x4_t*)(Cs + row * P + c * 8);
    }
  }
}

// fp32: one thread per output element; lanes run along the output columns.
template <bool GATED>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
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
  const float* a = A + (size_t)row * Kdim;
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

hipError_t launch_w13_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13, int E, int H,
                             int I, moe_dtype dt, void* h, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dt == MOE_BF16) {
    const int mt = max_row_tiles(rows, E, BM);
    const int n1 = I / 64;
    gemm_bf16_kernel<true><<<mt * n1, NTHR, 0, s>>>((const uint16_t*)x_perm, offsets, E, rows, H,
                                                    (const uint16_t*)W13, 2 * I, (long long)H * 2 * I, I, I,
                                                    (uint16_t*)h, I, n1);
  } else {
    dim3 g1(ceil_div(I, 64), ceil_div(rows, 4));
    gemm_f32_kernel<true><<<g1, 256, 0, s>>>((const float*)x_perm, offsets, E, rows, H, (const float*)W13, 2 * I,
                                             (long long)H * 2 * I, I, I, (float*)h, I);
  }
  return hipGetLastError();
}

hipError_t launch_w2(const void* h, const int32_t* offsets, int rows, const void* W2, int E, int H, int I,
                     moe_dtype dt, void* Y_perm, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dt == MOE_BF16) {
    const int mt = max_row_tiles(rows, E, BM);
    const int n2 = ceil_div(H, BN);
    gemm_bf16_kernel<false><<<mt * n2, NTHR, 0, s>>>((const uint16_t*)h, offsets, E, rows, I, (const uint16_t*)W2,
                                                     H, (long long)I * H, H, 0, (uint16_t*)Y_perm, H, n2);
  } else {
    dim3 g2(ceil_div(H, 64), ceil_div(rows, 4));
    gemm_f32_kernel<false><<<g2, 256, 0, s>>>((const float*)h, offsets, E, rows, I, (const float*)W2, H,
                                              (long long)I * H, H, 0, (float*)Y_perm, H);
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
