// Router: logits = x · W_gate (+ bias), softmax, top-K (optional renorm).
//
// Algorithm 2 steps 1-3 of "MoE 分布式推理基础（基于 vLLM）" §1.2 and the
// OlmoeTopKRouter source quoted there. The router product is small and
// HBM-bound (x is read once); each workgroup stages a 64-row slice of W_gate
// in LDS, runs bf16 MFMA 16x16x32 on 16-token groups (one group per wave),
// keeps the fp32 logits in LDS and then does softmax and top-K with one wave
// per token: each lane owns up to four experts, and each of the K passes is a
// wave-wide maximum of a 64-bit key (order-preserving logit bits, then the
// complemented expert index), so ties go to the lowest index.
#include <math.h>

#include "moe_internal.hpp"

namespace moe {
namespace {

// Larger logit -> larger key; among equal logits the lower expert index wins.
// -0.0 is folded into +0.0 so that the two compare equal.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(~(uint32_t)e);
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  uint32_t hi = (uint32_t)(key >> 32);
  uint32_t u = (hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_expert(uint64_t key) { return (int)(~(uint32_t)key); }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

// Butterfly sum: every lane ends with the same, order-fixed value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Softmax + top-K of one row of E fp32 logits, one wave. EPL = experts per lane.
template <int EPL>
__device__ void topk_softmax_row(const float* row, int E, int K, int renorm, int32_t* ids_out, float* w_out) {
  const int lane = lane_id();
  float v[EPL];
  uint64_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      v[j] = row[e];
      key[j] = route_key(v[j], e);
    } else {
      v[j] = -INFINITY;
      key[j] = 0;  // below every real key, including a -inf logit
    }
  }
  float m = 0.f, my_l = 0.f;
  int my_e = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (key[j] == best) key[j] = 0;
    const float lv = key_logit(best);
    if (k == 0) m = lv;
    if (lane == k) {
      my_e = key_expert(best);
      my_l = lv;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (lane + 64 * j < E) s += expf(v[j] - m);
  s = wave_sum(s);
  float wk = expf(my_l - m) / s;
  if (renorm) {
    float t = 0.f;
    for (int k = 0; k < K; ++k) t += __shfl(wk, k);
    wk = wk / t;
  }
  if (lane < K) {
    ids_out[lane] = my_e;
    w_out[lane] = wk;
  }
}

template <int EPL>
__device__ __forceinline__ void topk_dispatch(const float* row, int E, int K, int renorm, int32_t* ids, float* w) {
  topk_softmax_row<EPL>(row, E, K, renorm, ids, w);
}

__device__ void topk_any(const float* row, int E, int K, int renorm, int32_t* ids, float* w) {
  if (E <= 64)
    topk_dispatch<1>(row, E, K, renorm, ids, w);
  else if (E <= 128)
    topk_dispatch<2>(row, E, K, renorm, ids, w);
  else
    topk_dispatch<4>(row, E, K, renorm, ids, w);
}

// ---------------------------------------------------------------------------
// bf16 router: WAVES waves per workgroup, 16 tokens per wave, NT = Epad/16
// expert tiles of 16 columns.
// ---------------------------------------------------------------------------
constexpr int kRouteBK = 64;
constexpr int kRouteLdsBytes = 2 * kRouteBK * kMaxExperts * 2;  // 64 KB: two W_gate slices

template <int WAVES, int NT>
__global__ __launch_bounds__(64 * WAVES) void route_bf16_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ Wg,
                                                                const float* __restrict__ bias, int n, int H,
                                                                int E, int K, int renorm,
                                                                float* __restrict__ logits,
                                                                int32_t* __restrict__ ids,
                                                                float* __restrict__ wout) {
  constexpr int TOK = 16 * WAVES;
  constexpr int EPAD = 16 * NT;
  constexpr int PITCH = EPAD * 2;              // bytes per staged W_gate row
  constexpr int SLICE = kRouteBK * PITCH;      // bytes per staged slice
  constexpr int LPITCH = EPAD + 1;             // floats per logit row in LDS
  static_assert(2 * SLICE <= kRouteLdsBytes, "W_gate slice too large");
  static_assert(TOK * LPITCH * 4 <= kRouteLdsBytes, "logit tile too large");
  __shared__ __attribute__((aligned(16))) char smem_raw[kRouteLdsBytes];
  lds_char_t* smem = (lds_char_t*)smem_raw;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4, li = lane & 15;
  const int t0 = blockIdx.x * TOK;
  const int my_tok = t0 + wave * 16 + li;  // token whose x row this lane feeds to the MFMA
  const bool tok_ok = my_tok < n;
  const uint16_t* xrow = x + (size_t)(tok_ok ? my_tok : 0) * H;

  f32x4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bool vecW = (E % 8) == 0;
  const int nslices = H / kRouteBK;

  auto stage = [&](int s, int buf) {
    // W_gate rows [s*64, s*64+64), columns [0, EPAD): 8 elements per item.
    lds_char_t* dst = smem + buf * SLICE;
    const int k0 = s * kRouteBK;
    for (int it = tid; it < kRouteBK * (EPAD / 8); it += 64 * WAVES) {
      const int kr = it / (EPAD / 8), c = it % (EPAD / 8);
      const int e0 = c * 8;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      const uint16_t* src = Wg + (size_t)(k0 + kr) * E + e0;
      if (vecW && e0 + 8 <= E) {
        v = *(const u32x4_t*)src;
      } else {
        uint16_t tmp[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) tmp[q] = (e0 + q < E) ? src[q] : (uint16_t)0;
        v = u32x4_t{tmp[0] | ((uint32_t)tmp[1] << 16), tmp[2] | ((uint32_t)tmp[3] << 16),
                    tmp[4] | ((uint32_t)tmp[5] << 16), tmp[6] | ((uint32_t)tmp[7] << 16)};
      }
      lds_write_b128(dst + kr * PITCH + c * 16, v);
    }
  };

  stage(0, 0);
  __syncthreads();
  for (int s = 0; s < nslices; ++s) {
    const int buf = s & 1;
    if (s + 1 < nslices) stage(s + 1, buf ^ 1);
    const lds_char_t* wb = smem + buf * SLICE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t a = bf16x8_t{};
      if (tok_ok) {
        u32x4_t av = *(const u32x4_t*)(xrow + s * kRouteBK + ks * 32 + g * 8);
        a = __builtin_bit_cast(bf16x8_t, av);
      }
      const int r = li >> 2, c = li & 3;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = nt * 16 + 4 * c;
        const lds_char_t* p0 = wb + (ks * 32 + g * 8 + r) * PITCH + col * 2;
        bf16x4_t lo = lds_read_tr16(p0);
        bf16x4_t hi = lds_read_tr16(p0 + 4 * PITCH);
        bf16x8_t b = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Logits: lane (g, li) of tile nt holds rows 4g..4g+3 (tokens), column li (expert).
  float* lsm = (float*)smem_raw;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int e = nt * 16 + li;
    const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = wave * 16 + 4 * g + j;
      const float v = acc[nt][j] + b;
      lsm[tl * LPITCH + e] = v;
      const int t = t0 + tl;
      if (e < E && t < n) logits[(size_t)t * E + e] = v;
    }
  }
  __syncthreads();
  for (int q = 0; q < 16; ++q) {
    const int tl = wave * 16 + q;
    const int t = t0 + tl;
    if (t >= n) break;
    topk_any(lsm + tl * LPITCH, E, K, renorm, ids + (size_t)t * K, wout + (size_t)t * K);
  }
}

// ---------------------------------------------------------------------------
// fp32 router: one wave per token, lanes over experts, sequential fp32 FMA
// over the hidden dimension.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_f32_kernel(const float* __restrict__ x, const float* __restrict__ Wg,
                                                        const float* __restrict__ bias, int n, int H, int E,
                                                        int K, int renorm, float* __restrict__ logits,
                                                        int32_t* __restrict__ ids, float* __restrict__ wout) {
  __shared__ float lsm[4][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= n) return;
  const float* xr = x + (size_t)t * H;
  for (int e = lane; e < E; e += 64) {
    float acc = 0.f;
    for (int h = 0; h < H; ++h) acc = fmaf(xr[h], Wg[(size_t)h * E + e], acc);
    if (bias != nullptr) acc += bias[e];
    lsm[wave][e] = acc;
    logits[(size_t)t * E + e] = acc;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  topk_any(lsm[wave], E, K, renorm, ids + (size_t)t * K, wout + (size_t)t * K);
}

// Softmax + top-K only, from caller-supplied logits: one wave per token.
__global__ __launch_bounds__(256) void topk_only_kernel(const float* __restrict__ logits, int n, int E, int K,
                                                        int renorm, int32_t* __restrict__ ids,
                                                        float* __restrict__ wout) {
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= n) return;
  topk_any(logits + (size_t)t * E, E, K, renorm, ids + (size_t)t * K, wout + (size_t)t * K);
}

template <int WAVES>
hipError_t launch_route_bf16(const uint16_t* x, const uint16_t* Wg, const float* bias, int n, int H, int E, int K,
                             int renorm, float* logits, int32_t* ids, float* w, hipStream_t s) {
  const int grid = ceil_div(n, 16 * WAVES);
  const int nt = ceil_div(E, 16);
  if (nt <= 1)
    route_bf16_kernel<WAVES, 1><<<grid, 64 * WAVES, 0, s>>>(x, Wg, bias, n, H, E, K, renorm, logits, ids, w);
  else if (nt <= 2)
    route_bf16_kernel<WAVES, 2><<<grid, 64 * WAVES, 0, s>>>(x, Wg, bias, n, H, E, K, renorm, logits, ids, w);
  else if (nt <= 4)
    route_bf16_kernel<WAVES, 4><<<grid, 64 * WAVES, 0, s>>>(x, Wg, bias, n, H, E, K, renorm, logits, ids, w);
  else if (nt <= 8)
    route_bf16_kernel<WAVES, 8><<<grid, 64 * WAVES, 0, s>>>(x, Wg, bias, n, H, E, K, renorm, logits, ids, w);
  else
    route_bf16_kernel<WAVES, 16><<<grid, 64 * WAVES, 0, s>>>(x, Wg, bias, n, H, E, K, renorm, logits, ids, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const void* x, const void* W_gate, const float* bias, int n, int H, int E, int K,
                        int renorm, moe_dtype dt, float* logits, int32_t* topk_ids, float* topk_w,
                        hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (x == nullptr) {
    topk_only_kernel<<<ceil_div(n, 4), 256, 0, s>>>(logits, n, E, K, renorm, topk_ids, topk_w);
    return hipGetLastError();
  }
  if (dt == MOE_BF16)
    return launch_route_bf16<2>((const uint16_t*)x, (const uint16_t*)W_gate, bias, n, H, E, K, renorm, logits,
                                topk_ids, topk_w, s);
  route_f32_kernel<<<ceil_div(n, 4), 256, 0, s>>>((const float*)x, (const float*)W_gate, bias, n, H, E, K, renorm,
                                                   logits, topk_ids, topk_w);
  return hipGetLastError();
}

}  // namespace moe
