// Weighted top-K combine: y[i] = sum_{k=0..K-1} w[i,k] * Y_perm[inv[i*K+k]].
//
// Algorithm 2 steps 10-11 of "MoE 分布式推理基础（基于 vLLM）" §1.2 (each
// expert output row, times its routing weight, added into its token's row),
// written as a gather per token so that no two workgroups touch the same
// output row: the `_unpermute` plus deterministic weighted scatter-add of
// "0. goin" §2.2 and its top-K slot reduction (§2.3). The K rows are summed
// in slot order with fp32 fused multiply-adds, so the result is bitwise
// reproducible. HBM-bound: every expert row is read once, every token row
// written once, in 16-byte vectors.
#include "moe_internal.hpp"

namespace moe {
namespace {

// One workgroup per token; each thread owns 16-byte column chunks. The K
// rows are fetched in batches of kBatch loads in flight per thread, then
// accumulated in slot order. ADD: the sum starts from an fp32 row of `add`
// (n, row_vecs * EPV) instead of zero, before the single rounding.
constexpr int kBatch = 8;

template <bool BF16, bool ADD = false>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ Y, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int n, int row_vecs, int K,
                                                      void* __restrict__ y, const float* __restrict__ add,
                                                      int total) {
  constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
  const int i = blockIdx.x;
  const u32x4_t* Yv = (const u32x4_t*)Y;
  for (int c = threadIdx.x; c < row_vecs; c += 256) {
    float acc[EPV];
#pragma unroll
    for (int q = 0; q < EPV; ++q) acc[q] = 0.f;
    if constexpr (ADD) {
      const u32x4_t* a = (const u32x4_t*)(add + ((size_t)i * row_vecs + c) * EPV);
#pragma unroll
      for (int q = 0; q < EPV / 4; ++q) {
        const u32x4_t v = a[q];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * q + j] = __uint_as_float(v[j]);
      }
    }
    for (int k0 = 0; k0 < K; k0 += kBatch) {
      u32x4_t v[kBatch];
      float wk[kBatch];
      bool ok[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int k = k0 + j;
        const int r = (k < K) ? inv[(size_t)i * K + k] : -1;
        ok[j] = (unsigned)r < (unsigned)total;  // rows outside Y (total rows) add nothing
        wk[j] = ok[j] ? ((w != nullptr) ? w[(size_t)i * K + k] : 1.f) : 0.f;
        v[j] = ok[j] ? Yv[(size_t)r * row_vecs + c] : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (!ok[j]) continue;
        if constexpr (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] = fmaf(wk[j], __uint_as_float(v[j][q] << 16), acc[2 * q]);
            acc[2 * q + 1] = fmaf(wk[j], __uint_as_float(v[j][q] & 0xFFFF0000u), acc[2 * q + 1]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = fmaf(wk[j], __uint_as_float(v[j][q]), acc[q]);
        }
      }
    }
    u32x4_t out;
    if constexpr (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        out[q] = (uint32_t)f32_to_bf16(acc[2 * q]) | ((uint32_t)f32_to_bf16(acc[2 * q + 1]) << 16);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) out[q] = __float_as_uint(acc[q]);
    }
    ((u32x4_t*)y)[(size_t)i * row_vecs + c] = out;
  }
}

// y[i] = sum_k Y_tok[i*K + k]: the K rows of token i are contiguous (the
// weighted-scatter GEMM2 already applied the routing weights), summed in slot
// order in fp32.
template <bool BF16>
__global__ __launch_bounds__(256) void sum_slots_kernel(const void* __restrict__ Y, int n, int row_vecs, int K,
                                                        void* __restrict__ y) {
  constexpr int EPV = BF16 ? 8 : 4;
  const int i = blockIdx.x;
  const u32x4_t* Yv = (const u32x4_t*)Y + (size_t)i * K * row_vecs;
  for (int c = threadIdx.x; c < row_vecs; c += 256) {
    float acc[EPV];
#pragma unroll
    for (int q = 0; q < EPV; ++q) acc[q] = 0.f;
    for (int k0 = 0; k0 < K; k0 += kBatch) {
      u32x4_t v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        v[j] = (k0 + j < K) ? Yv[(size_t)(k0 + j) * row_vecs + c] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (k0 + j >= K) break;
        if constexpr (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] += __uint_as_float(v[j][q] << 16);
            acc[2 * q + 1] += __uint_as_float(v[j][q] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] += __uint_as_float(v[j][q]);
        }
      }
    }
    u32x4_t out;
    if constexpr (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        out[q] = (uint32_t)f32_to_bf16(acc[2 * q]) | ((uint32_t)f32_to_bf16(acc[2 * q + 1]) << 16);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) out[q] = __float_as_uint(acc[q]);
    }
    ((u32x4_t*)y)[(size_t)i * row_vecs + c] = out;
  }
}

}  // namespace

hipError_t launch_sum_slots(const void* Y_tok, int n, int H, int K, moe_dtype dt, void* y, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dt == MOE_BF16)
    sum_slots_kernel<true><<<n, 256, 0, s>>>(Y_tok, n, H / 8, K, y);
  else
    sum_slots_kernel<false><<<n, 256, 0, s>>>(Y_tok, n, H / 4, K, y);
  return hipGetLastError();
}

hipError_t launch_combine_rows(const void* Y_perm, int y_rows, const int32_t* inv, const float* topk_w, int n, int H,
                               int K, moe_dtype dt, void* y, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dt == MOE_BF16)
    combine_kernel<true><<<n, 256, 0, s>>>(Y_perm, inv, topk_w, n, H / 8, K, y, nullptr, y_rows);
  else
    combine_kernel<false><<<n, 256, 0, s>>>(Y_perm, inv, topk_w, n, H / 4, K, y, nullptr, y_rows);
  return hipGetLastError();
}

hipError_t launch_combine(const void* Y_perm, const int32_t* inv, const float* topk_w, int n, int H, int K,
                          moe_dtype dt, void* y, hipStream_t s) {
  return launch_combine_rows(Y_perm, n * K, inv, topk_w, n, H, K, dt, y, s);
}

hipError_t launch_dispatch_backward(const void* dX_perm, const int32_t* inv, const float* add, int n, int H, int K,
                                    moe_dtype dt, void* dx, hipStream_t s) {
  if (n == 0) return hipSuccess;
  // Unit weights: each token sums the gradients of its K rows (slot order).
  if (add == nullptr) return launch_combine(dX_perm, inv, nullptr, n, H, K, dt, dx, s);
  if (dt == MOE_BF16)
    combine_kernel<true, true><<<n, 256, 0, s>>>(dX_perm, inv, nullptr, n, H / 8, K, dx, add, n * K);
  else
    combine_kernel<false, true><<<n, 256, 0, s>>>(dX_perm, inv, nullptr, n, H / 4, K, dx, add, n * K);
  return hipGetLastError();
}

}  // namespace moe
