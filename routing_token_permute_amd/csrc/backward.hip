// Memory-bound and router pieces of the layer's backward.
//
// The backward of a combine is a dispatch that also yields the routing-score
// gradient, and the backward of a dispatch is a combine ("大模型系统中的通算
// 融合" §6.2.4; "0. goin" §2.3 (d) and the top-K gradient kernels of its
// table (e)). With y[i] = sum_k w[i,k] Y_perm[inv[iK+k]] (Algorithm 2 steps
// 10-11 of "MoE 分布式推理基础（基于 vLLM）" §1.2):
//
//   combine backward:  dY_perm[inv[iK+k]] = w[i,k] dy[i],
//                      dw[i,k] = <dy[i], Y_perm[inv[iK+k]]>
//   router backward:   ds = dw, or (dw - <dw, w>) / S under renormalisation
//                      (w = s / S, S = sum_k s); dp = ds at the selected
//                      experts; dlogits = p * (dp - <p, dp>) (softmax);
//                      dx += dlogits W_gate^T, dW_gate = x^T dlogits,
//                      dbias = sum_i dlogits[i]
//
// (the dispatch backward itself is combine_kernel with unit weights plus the
// router's share, in combine.hip). Every reduction runs in a fixed order in
// fp32, so the results are bitwise reproducible; there are no atomics.
#include <math.h>

#include <algorithm>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kBatch = 8;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One workgroup per token; each thread owns 16-byte column chunks. The K rows
// are visited in batches of kBatch: the dot products are partial sums per
// thread, reduced across the workgroup in a fixed order.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const void* __restrict__ dy, const void* __restrict__ Y,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ w, int n, int row_vecs, int K,
                                                          void* __restrict__ dY, float* __restrict__ dw) {
  constexpr int EPV = BF16 ? 8 : 4;
  __shared__ float red[4][kBatch];
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int total = n * K;
  const u32x4_t* dyv = (const u32x4_t*)dy + (size_t)i * row_vecs;
  const u32x4_t* Yv = (const u32x4_t*)Y;
  u32x4_t* dYv = (u32x4_t*)dY;
  auto unpack = [](const u32x4_t& v, float* f) {
    if constexpr (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(v[q] << 16);
        f[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = __uint_as_float(v[q]);
    }
  };
  for (int k0 = 0; k0 < K; k0 += kBatch) {
    int rk[kBatch];
    float wk[kBatch], part[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int k = k0 + j;
      const int r = (k < K) ? inv[(size_t)i * K + k] : -1;
      rk[j] = ((unsigned)r < (unsigned)total) ? r : -1;
      wk[j] = rk[j] >= 0 ? w[(size_t)i * K + k] : 0.f;
      part[j] = 0.f;
    }
    for (int c = tid; c < row_vecs; c += 256) {
      float g[EPV];
      unpack(dyv[c], g);
      u32x4_t yv[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) yv[j] = rk[j] >= 0 ? Yv[(size_t)rk[j] * row_vecs + c] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (rk[j] < 0) continue;
        float yf[EPV];
        unpack(yv[j], yf);
#pragma unroll
        for (int q = 0; q < EPV; ++q) part[j] = fmaf(g[q], yf[q], part[j]);
        u32x4_t out;
        if constexpr (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            out[q] = (uint32_t)f32_to_bf16(wk[j] * g[2 * q]) | ((uint32_t)f32_to_bf16(wk[j] * g[2 * q + 1]) << 16);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) out[q] = __float_as_uint(wk[j] * g[q]);
        }
        dYv[(size_t)rk[j] * row_vecs + c] = out;
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float v = wave_sum(part[j]);
      if (lane == 0) red[wave][j] = v;
    }
    __syncthreads();
    if (tid < kBatch && k0 + tid < K) dw[(size_t)i * K + k0 + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    __syncthreads();
  }
}

// Router backward, per block of kRbTok tokens. Phase 1 (one wave per token):
// softmax from the saved fp32 logits, the renormalisation and softmax
// backward, dlogits written to HBM and LDS.
// PREP (bf16, E a multiple of 32): the two router products then run on MFMA
// (grouped_gemm_bwd.hip), so phase 1 also writes dlogits split into bf16
// halves, hilo[i] = [hi | lo] with hi = bf16(d) and lo = bf16(d - hi) (their
// sum is d to about 2^-18 relative), the block's column sums of dlogits
// (part_b[block][e], tokens in order) and, from block 0, the row offsets the
// GEMMs group by: row_off = {0, n} and chunk_off[g] = min(n, g * chunk).
// Otherwise phase 2 computes dx_router = dlogits . W_gate^T here, one thread
// per hidden column h over all tokens of the block.
constexpr int kRbTok = 16;

template <bool BF16, bool PREP>
__global__ __launch_bounds__(256) void route_bwd_token_kernel(const float* __restrict__ logits,
                                                              const int32_t* __restrict__ ids,
                                                              const float* __restrict__ w,
                                                              const float* __restrict__ dw, int n, int E, int K,
                                                              int renorm, const void* __restrict__ W_gate, int H,
                                                              float* __restrict__ dlogits,
                                                              float* __restrict__ dx_router,
                                                              uint16_t* __restrict__ hilo, float* __restrict__ part_b,
                                                              int32_t* __restrict__ row_off,
                                                              int32_t* __restrict__ chunk_off, int S, int chunk) {
  __shared__ __attribute__((aligned(16))) float dl[kRbTok][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kRbTok;
  for (int tt = wave; tt < kRbTok; tt += 4) {
    const int i = t0 + tt;
    if (i >= n) {
      for (int e = lane; e < E; e += 64) dl[tt][e] = 0.f;
      continue;
    }
    const float* L = logits + (size_t)i * E;
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, L[e]);
    m = wave_max(m);
    float z = 0.f;
    for (int e = lane; e < E; e += 64) z += __expf(L[e] - m);
    z = wave_sum(z);
    const float rz = 1.f / z;
    int ek = -1;
    float pk = 0.f, dwk = 0.f, wk = 0.f;
    if (lane < K) {
      ek = ids[(size_t)i * K + lane];
      if ((unsigned)ek < (unsigned)E) {
        pk = __expf(L[ek] - m) * rz;
        dwk = dw[(size_t)i * K + lane];
        wk = w[(size_t)i * K + lane];
      } else {
        ek = -1;
      }
    }
    float ds = dwk;
    if (renorm) {
      const float S = wave_sum(pk);
      const float dot = wave_sum(dwk * wk);
      ds = (dwk - dot) / S;
    }
    const float pdp = wave_sum(pk * ds);
    for (int e0 = 0; e0 < E; e0 += 64) {  // every lane takes part in the shuffles
      const int e = e0 + lane;
      float dp = 0.f;
      for (int k = 0; k < K; ++k) {
        const int ekk = __shfl(ek, k);
        const float dsk = __shfl(ds, k);
        if (ekk == e) dp = dsk;
      }
      if (e < E) {
        const float v = __expf(L[e] - m) * rz * (dp - pdp);
        dl[tt][e] = v;
        dlogits[(size_t)i * E + e] = v;
        if constexpr (PREP) {
          const uint16_t hi = f32_to_bf16(v);
          hilo[(size_t)i * 2 * E + e] = hi;
          hilo[(size_t)i * 2 * E + E + e] = f32_to_bf16(v - bf16_to_f32(hi));
        }
      }
    }
  }
  __syncthreads();
  if constexpr (PREP) {
    if (tid < E) {
      float v = 0.f;
      for (int t = 0; t < kRbTok; ++t) v += dl[t][tid];  // rows past n hold zeros
      part_b[(size_t)blockIdx.x * E + tid] = v;
    }
    if (blockIdx.x == 0) {
      if (tid == 0) {
        row_off[0] = 0;
        row_off[1] = n;
      }
      for (int g = tid; g <= S; g += 256) chunk_off[g] = (int)min((long long)n, (long long)g * chunk);
    }
    return;
  }
  if (dx_router == nullptr) return;
  const int nt = min(kRbTok, n - t0);
  for (int h = tid; h < H; h += 256) {
    float acc[kRbTok];
#pragma unroll
    for (int t = 0; t < kRbTok; ++t) acc[t] = 0.f;
    if (BF16 && (E & 7) == 0) {
      const u32x4_t* wr = (const u32x4_t*)((const uint16_t*)W_gate + (size_t)h * E);
      for (int e0 = 0; e0 < E; e0 += 8) {
        const u32x4_t v = wr[e0 / 8];
        float wv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          wv[2 * q] = __uint_as_float(v[q] << 16);
          wv[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
        }
#pragma unroll
        for (int t = 0; t < kRbTok; ++t) {
          const f32x4_t a = *(const f32x4_t*)&dl[t][e0];
          const f32x4_t b = *(const f32x4_t*)&dl[t][e0 + 4];
          float s = acc[t];
          s = fmaf(a[0], wv[0], s);
          s = fmaf(a[1], wv[1], s);
          s = fmaf(a[2], wv[2], s);
          s = fmaf(a[3], wv[3], s);
          s = fmaf(b[0], wv[4], s);
          s = fmaf(b[1], wv[5], s);
          s = fmaf(b[2], wv[6], s);
          s = fmaf(b[3], wv[7], s);
          acc[t] = s;
        }
      }
    } else {
      for (int e = 0; e < E; ++e) {
        const float wv = BF16 ? bf16_to_f32(((const uint16_t*)W_gate)[(size_t)h * E + e])
                              : ((const float*)W_gate)[(size_t)h * E + e];
#pragma unroll
        for (int t = 0; t < kRbTok; ++t) acc[t] = fmaf(dl[t][e], wv, acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < kRbTok; ++t)
      if (t < nt) dx_router[(size_t)(t0 + t) * H + h] = acc[t];
  }
}

// dW_gate partials: workgroup (hb, s) sums x[i][h] * dlogits[i][e] over the
// tokens of chunk s for the 64 columns h of block hb, into part[s][h][e];
// the workgroups of block 0 also sum dlogits over the chunk into
// part_b[s][e]. Thread (h = tid % 64, q = tid / 64) owns experts
// [q * EQ, (q + 1) * EQ), EQ = ceil(E / 4) rounded up to 4.
constexpr int kRwTok = 32;  // tokens staged in LDS at a time
constexpr int kRwMaxEQ = kMaxExperts / 4;

template <bool BF16>
__global__ __launch_bounds__(256) void route_bwd_weight_kernel(const void* __restrict__ x,
                                                               const float* __restrict__ dlogits, int n, int H,
                                                               int E, int chunk, float* __restrict__ part,
                                                               float* __restrict__ part_b) {
  __shared__ float xs[kRwTok][64];
  __shared__ __attribute__((aligned(16))) float ds[kRwTok][kMaxExperts];
  const int tid = threadIdx.x, hl = tid & 63, q = tid >> 6;
  const int h0 = blockIdx.x * 64, s = blockIdx.y;
  const int i0 = s * chunk, i1 = min(n, i0 + chunk);
  const int EQ = ((E + 3) / 4 + 3) & ~3;
  const int e_lo = q * EQ;
  float acc[kRwMaxEQ];
#pragma unroll
  for (int j = 0; j < kRwMaxEQ; ++j) acc[j] = 0.f;
  float bsum = 0.f;  // part_b: thread tid < E owns expert tid
  for (int b0 = i0; b0 < i1; b0 += kRwTok) {
    const int nt = min(kRwTok, i1 - b0);
    for (int idx = tid; idx < kRwTok * 64; idx += 256) {
      const int t = idx / 64, hh = idx % 64;
      float v = 0.f;
      if (t < nt && h0 + hh < H)
        v = BF16 ? bf16_to_f32(((const uint16_t*)x)[(size_t)(b0 + t) * H + h0 + hh])
                 : ((const float*)x)[(size_t)(b0 + t) * H + h0 + hh];
      xs[t][hh] = v;
    }
    for (int idx = tid; idx < kRwTok * 4 * EQ; idx += 256) {
      const int t = idx / (4 * EQ), e = idx % (4 * EQ);
      ds[t][e] = (t < nt && e < E) ? dlogits[(size_t)(b0 + t) * E + e] : 0.f;
    }
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      const float xv = xs[t][hl];
#pragma unroll
      for (int j = 0; j < kRwMaxEQ; j += 4) {
        if (j < EQ) {
          const f32x4_t d = *(const f32x4_t*)&ds[t][e_lo + j];
          acc[j] = fmaf(xv, d[0], acc[j]);
          acc[j + 1] = fmaf(xv, d[1], acc[j + 1]);
          acc[j + 2] = fmaf(xv, d[2], acc[j + 2]);
          acc[j + 3] = fmaf(xv, d[3], acc[j + 3]);
        }
      }
    }
    if (blockIdx.x == 0 && tid < E)
      for (int t = 0; t < nt; ++t) bsum += ds[t][tid];
    __syncthreads();
  }
  const int h = h0 + hl;
  if (h < H) {
    float* out = part + ((size_t)s * H + h) * E;
#pragma unroll
    for (int j = 0; j < kRwMaxEQ; ++j)
      if (j < EQ && e_lo + j < E) out[e_lo + j] = acc[j];
  }
  if (blockIdx.x == 0 && tid < E) part_b[(size_t)s * E + tid] = bsum;
}

// dW_gate[h][e] = sum_s part[s][h][e] and dbias[e] = sum_s part_b[s][e], s ascending.
__global__ __launch_bounds__(256) void route_bwd_reduce_kernel(const float* __restrict__ part,
                                                               const float* __restrict__ part_b, int S, int H, int E,
                                                               float* __restrict__ dW_gate,
                                                               float* __restrict__ dbias) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long HE = (long long)H * E;
  if (idx < HE) {
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += part[(size_t)s * HE + idx];
    if (dW_gate != nullptr) dW_gate[idx] = v;
  } else if (idx < HE + E) {
    const int e = (int)(idx - HE);
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += part_b[(size_t)s * E + e];
    if (dbias != nullptr) dbias[e] = v;
  }
}

// Zero fill of `words` 32-bit words (a kernel rather than a memset, so that
// a caller may capture the call in a HIP graph).
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, long long words) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < words; i += (long long)gridDim.x * 256) p[i] = 0u;
}

// MFMA path: dW_gate[h][e] = sum_g (part[g][h][e] + part[g][h][E + e]) (the hi
// and lo halves of chunk g, chunks in order), one thread per (h, e) in the
// first ceil(H*E / 256) workgroups; dbias[e] = sum_b part_b[b][e], one wave per
// e in the workgroups after them (lane j sums blocks j, j+64, ... in order,
// then a fixed butterfly across the lanes).
__global__ __launch_bounds__(256) void route_bwd_reduce_hilo_kernel(const float* __restrict__ part, int S, int H,
                                                                    int E, const float* __restrict__ part_b, int nb,
                                                                    float* __restrict__ dW_gate,
                                                                    float* __restrict__ dbias) {
  const long long HE = (long long)H * E;
  const int wblocks = (int)((HE + 255) / 256);
  if ((int)blockIdx.x < wblocks) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= HE || dW_gate == nullptr) return;
    const long long h = idx / E, e = idx % E;
    const float* p = part + (size_t)h * 2 * E + e;
    const size_t gs = (size_t)H * 2 * E;
    float v = 0.f;
    // Batches of 8 chunks: 16 loads in flight, then summed in chunk order.
    for (int g0 = 0; g0 < S; g0 += 8) {
      float a[8], b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a[j] = g0 + j < S ? p[(size_t)(g0 + j) * gs] : 0.f;
        b[j] = g0 + j < S ? p[(size_t)(g0 + j) * gs + E] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) v += a[j] + b[j];
    }
    dW_gate[idx] = v;
    return;
  }
  const int e = ((int)blockIdx.x - wblocks) * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E || dbias == nullptr) return;
  float v = 0.f;
  for (int b = lane; b < nb; b += 64) v += part_b[(size_t)b * E + e];
  v = wave_sum(v);
  if (lane == 0) dbias[e] = v;
}

// Token chunks of the MFMA dW_gate product: about one 256-column block of
// H per compute unit, chunks at least 64 tokens long.
int route_mfma_chunks(int n, int H) {
  const int mb = (H + 255) / 256;
  int S = (256 + mb - 1) / mb;
  S = std::min(S, 64);
  S = std::min(S, std::max(1, (n + 63) / 64));
  return S;
}

bool route_mfma_path(moe_dtype dt, int E) { return dt == MOE_BF16 && E % 32 == 0; }

// Workspace pieces of the MFMA path, in bytes, each rounded up to 256.
struct RouteMfmaLayout {
  size_t hilo, part_b, offs, part, total;
};

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

RouteMfmaLayout route_mfma_layout(int n, int H, int E) {
  RouteMfmaLayout L{};
  const int S = route_mfma_chunks(n, H);
  size_t o = 0;
  L.hilo = o;
  o += up256((size_t)n * 2 * E * 2);
  L.part_b = o;
  o += up256((size_t)ceil_div(n, kRbTok) * E * 4);
  L.offs = o;
  o += up256((size_t)(S + 3) * 4);
  L.part = o;
  o += up256((size_t)S * H * 2 * E * 4);
  L.total = o;
  return L;
}

}  // namespace

size_t route_bwd_workspace(int n, int H, int E) {
  const size_t fma = up256((size_t)route_bwd_chunks(n) * (H + 1) * E * 4);
  const size_t mfma = route_mfma_layout(n, H, E).total;
  return std::max(fma, mfma);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const long long words = (long long)(bytes / 4);
  if (words == 0) return hipSuccess;
  const int grid = (int)std::min<long long>(ceil_div(words, 256), 4096);
  fill_zero_kernel<<<grid, 256, 0, s>>>((uint32_t*)p, words);
  return hipGetLastError();
}

int route_bwd_chunks(int n) {
  const int c = (n + 63) / 64;
  return c < 1 ? 1 : (c > kRouteBwdMaxChunks ? kRouteBwdMaxChunks : c);
}

hipError_t launch_combine_backward(const void* dy, const void* Y_perm, const int32_t* inv, const float* topk_w, int n,
                                   int H, int K, moe_dtype dt, void* dY_perm, float* dw, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dt == MOE_BF16)
    combine_bwd_kernel<true><<<n, 256, 0, s>>>(dy, Y_perm, inv, topk_w, n, H / 8, K, dY_perm, dw);
  else
    combine_bwd_kernel<false><<<n, 256, 0, s>>>(dy, Y_perm, inv, topk_w, n, H / 4, K, dY_perm, dw);
  return hipGetLastError();
}

hipError_t launch_route_backward(const void* x, const void* W_gate, const float* logits, const int32_t* ids,
                                 const float* topk_w, const float* dw, int n, int H, int E, int K, int renorm,
                                 moe_dtype dt, float* dlogits, float* dx_router, float* dW_gate, float* dbias,
                                 void* ws, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int nb = ceil_div(n, kRbTok);
  const bool weights = dW_gate != nullptr || dbias != nullptr;
  hipError_t e = hipSuccess;
  if (route_mfma_path(dt, E) && (dx_router != nullptr || weights)) {
    const RouteMfmaLayout L = route_mfma_layout(n, H, E);
    char* base = (char*)ws;
    uint16_t* hilo = (uint16_t*)(base + L.hilo);
    float* part_b = (float*)(base + L.part_b);
    int32_t* row_off = (int32_t*)(base + L.offs);
    int32_t* chunk_off = row_off + 2;
    float* part = (float*)(base + L.part);
    const int S = route_mfma_chunks(n, H);
    const int chunk = ceil_div(n, S);
    route_bwd_token_kernel<true, true><<<nb, 256, 0, s>>>(logits, ids, topk_w, dw, n, E, K, renorm, W_gate, H,
                                                          dlogits, nullptr, hilo, part_b, row_off, chunk_off, S,
                                                          chunk);
    e = hipGetLastError();
    if (e == hipSuccess && dx_router != nullptr) e = launch_router_dx_mfma(hilo, row_off, n, W_gate, H, E, dx_router, s);
    if (e == hipSuccess && weights) e = launch_router_dw_mfma(x, hilo, chunk_off, S, n, H, E, part, s);
    if (e == hipSuccess && weights) {
      const int blocks = ceil_div((long long)H * E, 256) + ceil_div(E, 4);
      route_bwd_reduce_hilo_kernel<<<blocks, 256, 0, s>>>(part, S, H, E, part_b, nb, dW_gate, dbias);
      e = hipGetLastError();
    }
    return e;
  }
  if (dt == MOE_BF16)
    route_bwd_token_kernel<true, false><<<nb, 256, 0, s>>>(logits, ids, topk_w, dw, n, E, K, renorm, W_gate, H,
                                                           dlogits, dx_router, nullptr, nullptr, nullptr, nullptr, 0,
                                                           0);
  else
    route_bwd_token_kernel<false, false><<<nb, 256, 0, s>>>(logits, ids, topk_w, dw, n, E, K, renorm, W_gate, H,
                                                            dlogits, dx_router, nullptr, nullptr, nullptr, nullptr, 0,
                                                            0);
  e = hipGetLastError();
  if (e != hipSuccess || !weights) return e;
  const int S = route_bwd_chunks(n);
  const int chunk = ceil_div(n, S);
  float* part = (float*)ws;
  float* part_b = part + (size_t)S * H * E;
  dim3 g(ceil_div(H, 64), S);
  if (dt == MOE_BF16)
    route_bwd_weight_kernel<true><<<g, 256, 0, s>>>(x, dlogits, n, H, E, chunk, part, part_b);
  else
    route_bwd_weight_kernel<false><<<g, 256, 0, s>>>(x, dlogits, n, H, E, chunk, part, part_b);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  route_bwd_reduce_kernel<<<ceil_div((long long)H * E + E, 256), 256, 0, s>>>(part, part_b, S, H, E, dW_gate,
                                                                             dbias);
  return hipGetLastError();
}

}  // namespace moe
