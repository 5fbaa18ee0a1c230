// Router: logits = x · W_gate (+ bias), softmax, top-K (optional renorm).
//
// Algorithm 2 steps 1-3 of "MoE 分布式推理基础（基于 vLLM）" §1.2 and the
// OlmoeTopKRouter source quoted there (linear layer, softmax, topk, and the
// optional division of the K weights by their sum).
//
// bf16 path. One workgroup serves 16 tokens; its WK waves split the hidden
// dimension. Each wave streams its own 64-row slices of W_gate through a
// private double buffer in LDS (the next slice is fetched into registers
// while the current one feeds the MFMAs) and turns them into MFMA B operands
// with the gfx950 LDS transpose read; the token rows are the A operands,
// loaded from HBM one slice ahead. bf16 MFMA 16x16x32 accumulates in fp32.
// The WK partial logit tiles are summed in LDS in wave order, so the result
// does not depend on timing.
//
// Top-K. One wave per token, one expert per lane (more for E > 64): the row
// maximum and the softmax denominator are wave reductions over DPP lane
// moves in a fixed order; then K rounds each take the largest remaining order
// key (logit descending) and, among equal keys, the lowest expert index (a
// ballot of the lanes that hold it), and clear it. Slot k is written by lane k.
#include <math.h>

#include "moe_internal.hpp"

namespace moe {
namespace {

// Order key of a logit: larger logit -> larger key; -0.0 is folded into +0.0
// so that the two compare equal; -inf maps above 0, which marks "no expert".
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide reductions over the 64 lanes with DPP lane moves: two quad
// swaps, the half-row and row mirrors (every lane of a 16-lane row then
// holds the row's result), then the row-15 and row-31 broadcasts into the
// upper rows; lane 63 ends with the total, read back as a wave constant.
// The order of the fp32 additions is fixed, so the sum is deterministic.
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, int ctrl_sel) {
  switch (ctrl_sel) {
    case 0: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false);  // row half mirror
    case 3: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false);  // row mirror
    case 4: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false);  // row bcast 15
    default: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false); // row bcast 31
  }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const uint32_t o = dpp_u32(v, i);
    v = o > v ? o : v;
  }
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    // Rows that a broadcast step leaves out add nothing.
    const uint32_t o = dpp_u32(__float_as_uint(v), i);
    const bool take = i < 4 || (i == 4 ? ((lane_id() >> 4) & 1) : (lane_id() >> 5));
    v += take ? __uint_as_float(o) : 0.f;
  }
  return __uint_as_float(__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

// Softmax + top-K of one token whose E logits (fp32) and order keys sit in
// LDS; one wave, EPL experts per lane (EPL * 64 >= E). The K experts are
// taken one at a time: the largest remaining order key over the wave, and
// among equal keys the lowest expert index (a ballot of the lanes holding
// it); that expert's key is then cleared. The first round's maximum is the
// softmax's row maximum. `ex` (wave-private LDS scratch) is not needed here.
template <int EPL>
__device__ __forceinline__ void topk_token(const float* lg, const uint32_t* keys, int E, int K, int renorm, float* ex,
                                           int32_t* ids_out, float* w_out) {
  (void)ex;
  const int lane = lane_id();
  uint32_t key[EPL];
  float exv[EPL];
  uint32_t lmax = 0u;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? keys[e] : 0u;
    lmax = key[j] > lmax ? key[j] : lmax;
  }
  const uint32_t kmax = wave_max_u32(lmax);
  const float m = key_value(kmax);
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    exv[j] = e < E ? expf(lg[e] - m) : 0.f;
    part += exv[j];
  }
  const float s = wave_sum_f32(part);
  int my_id = 0;
  float my_w = 0.f, t = 0.f;
  for (int k = 0; k < K; ++k) {
    uint32_t mx = kmax;
    if (k > 0) {
      lmax = 0u;
#pragma unroll
      for (int j = 0; j < EPL; ++j) lmax = key[j] > lmax ? key[j] : lmax;
      mx = wave_max_u32(lmax);
    }
    int win = -1;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const uint64_t b = __ballot(key[j] == mx);
      if (win < 0 && b != 0) win = 64 * j + __ffsll((long long)b) - 1;
    }
    win = __builtin_amdgcn_readfirstlane(win);
    const int wl = win & 63, wj = win >> 6;
    float ev = exv[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j)
      if (j == wj) ev = exv[j];
    const float w = __uint_as_float(__builtin_amdgcn_readlane((int)__float_as_uint(ev), wl)) / s;
    t += w;
    if (lane == k) {
      my_id = win;
      my_w = w;
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j == win) key[j] = 0u;
  }
  if (lane < K) {
    ids_out[lane] = my_id;
    w_out[lane] = renorm ? my_w / t : my_w;
  }
}

// `scratch`: kMaxExperts + kMaxTopK floats of LDS private to the calling wave.
// Inlined, so that the LDS arrays keep their address space (a call would pass
// them as generic pointers and read them with flat loads).
__device__ __forceinline__ void topk_token_any(const float* lg, const uint32_t* keys, int E, int K, int renorm, float* scratch,
                               int32_t* ids, float* w) {
  if (E <= 64)
    topk_token<1>(lg, keys, E, K, renorm, scratch, ids, w);
  else if (E <= 128)
    topk_token<2>(lg, keys, E, K, renorm, scratch, ids, w);
  else
    topk_token<4>(lg, keys, E, K, renorm, scratch, ids, w);
}

constexpr int kScratch = kMaxExperts + kMaxTopK;  // floats of top-K scratch per wave

// ---------------------------------------------------------------------------
// bf16 router: 16 tokens per workgroup, WK waves split H, NT expert tiles.
// ---------------------------------------------------------------------------
constexpr int kTok = 16;
constexpr int kSliceRows = 64;

template <int NT, int WK>
struct RouteCfg {
  static constexpr int EPAD = 16 * NT;
  static constexpr int PITCH = EPAD * 2;                  // bytes per staged W_gate row
  static constexpr int SLICE = kSliceRows * PITCH;        // bytes per staged slice
  static constexpr int STAGING = WK * 2 * SLICE;          // per-wave double buffers
  static constexpr int LPITCH = EPAD + 4;                 // floats per logit row (16-byte rows)
  static constexpr int PARTIAL = WK * kTok * EPAD * 4;    // per-wave partial tiles
  static constexpr int LOGITS = kTok * LPITCH * 8;        // logits + order keys
  static constexpr int SLOTS = WK * kScratch * 4;         // top-K scratch, one row per wave
  static constexpr int AFTER = PARTIAL + LOGITS + SLOTS;
  static constexpr int LDS = STAGING > AFTER ? STAGING : AFTER;
  static constexpr int CHUNKS = kSliceRows * EPAD / 8;    // 16-byte pieces per slice
  static constexpr int CPL = (CHUNKS + 63) / 64;          // pieces per lane
};

template <int NT, int WK>
__global__ __launch_bounds__(64 * WK) void route_bf16_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ Wg,
                                                             const float* __restrict__ bias, int n, int H, int E,
                                                             int K, int renorm, float* __restrict__ logits,
                                                             int32_t* __restrict__ ids, float* __restrict__ wout) {
  using C = RouteCfg<NT, WK>;
  constexpr int EPAD = C::EPAD, PITCH = C::PITCH, SLICE = C::SLICE;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::LDS];
  lds_char_t* smem = (lds_char_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int t0 = blockIdx.x * kTok;
  const int my_tok = t0 + li;
  const bool tok_ok = my_tok < n;
  const uint16_t* xrow = x + (size_t)(tok_ok ? my_tok : 0) * H + g * 8;
  const bool vecW = (E % 8) == 0;
  const int nslices = H / kSliceRows;
  const int rounds = (nslices + WK - 1) / WK;
  lds_char_t* mybuf = smem + wave * 2 * SLICE;

  f32x4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t wreg[C::CPL];
  u32x4_t xa[2];
  auto fetch = [&](int s) {  // W_gate slice s into registers, x operands of slice s
    const int k0 = s * kSliceRows;
#pragma unroll
    for (int q = 0; q < C::CPL; ++q) {
      const int it = lane + 64 * q;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (it < C::CHUNKS) {
        const int kr = it / (EPAD / 8), e0 = (it % (EPAD / 8)) * 8;
        const uint16_t* src = Wg + (size_t)(k0 + kr) * E + e0;
        if (vecW && e0 + 8 <= E) {
          v = *(const u32x4_t*)src;
        } else {
          uint32_t p[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e0 + e < E) p[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
          v = u32x4_t{p[0], p[1], p[2], p[3]};
        }
      }
      wreg[q] = v;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      xa[ks] = tok_ok ? *(const u32x4_t*)(xrow + k0 + ks * 32) : u32x4_t{0u, 0u, 0u, 0u};
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int q = 0; q < C::CPL; ++q) {
      const int it = lane + 64 * q;
      if (it < C::CHUNKS) {
        const int kr = it / (EPAD / 8), c = it % (EPAD / 8);
        lds_write_b128(mybuf + buf * SLICE + kr * PITCH + c * 16, wreg[q]);
      }
    }
  };

  // Round r: wave w handles slice r*WK + w. Every wave runs the same number
  // of rounds so the barriers match; waves past the last slice idle.
  const int s0 = wave;
  if (s0 < nslices) fetch(s0);
  for (int r = 0; r < rounds; ++r) {
    const int s = r * WK + wave;
    const bool active = s < nslices;
    u32x4_t xcur[2] = {xa[0], xa[1]};
    if (active) stash(r & 1);
    if (active && s + WK < nslices) fetch(s + WK);
    __syncthreads();
    if (active) {
      const lds_char_t* wb = mybuf + (r & 1) * SLICE;
      const int rr = li >> 2, cc = li & 3;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xcur[ks]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const lds_char_t* p0 = wb + (ks * 32 + g * 8 + rr) * PITCH + (nt * 16 + 4 * cc) * 2;
          const bf16x4_t lo = lds_read_tr16(p0);
          const bf16x4_t hi = lds_read_tr16(p0 + 4 * PITCH);
          const bf16x8_t b = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // Partial tiles: lane (g, li) of tile nt holds tokens 4g..4g+3, expert nt*16+li.
  float* part = (float*)smem_raw;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int j = 0; j < 4; ++j) part[(wave * kTok + 4 * g + j) * EPAD + nt * 16 + li] = acc[nt][j];
  __syncthreads();
  float* lg = part + WK * kTok * EPAD;                      // [kTok][LPITCH] logits
  uint32_t* keys = (uint32_t*)(lg + kTok * C::LPITCH);     // [kTok][LPITCH] order keys
  float* slots = (float*)(keys + kTok * C::LPITCH);        // [WK][kScratch]
  for (int q = tid; q < kTok * EPAD; q += 64 * WK) {
    const int tl = q / EPAD, e = q % EPAD;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < WK; ++w) v += part[(w * kTok + tl) * EPAD + e];
    if (e < E) {
      if (bias != nullptr) v += bias[e];
      lg[tl * C::LPITCH + e] = v;
      keys[tl * C::LPITCH + e] = order_key(v);
      if (t0 + tl < n) logits[(size_t)(t0 + tl) * E + e] = v;
    }
  }
  __syncthreads();
  for (int tl = wave; tl < kTok; tl += WK) {
    const int t = t0 + tl;
    if (t >= n) break;
    topk_token_any(lg + tl * C::LPITCH, keys + tl * C::LPITCH, E, K, renorm, slots + wave * kScratch,
                   ids + (size_t)t * K, wout + (size_t)t * K);
  }
}

// ---------------------------------------------------------------------------
// bf16 router for small batches: one workgroup of 1024 threads per token.
// With CH = E / 8 chunks of 8 experts per W_gate row, thread i reads chunk
// i % CH of rows i / CH, i / CH + 1024 / CH, ... (each wave's 16-byte loads
// cover whole consecutive rows; eight rows' loads of every thread are in
// flight together, 128 KB per workgroup) and accumulates its 8 experts in
// fp32 (bf16 products are exact in fp32). The partial sums meet in LDS and
// each expert's are added in thread order, so the result does not depend on
// timing; then one wave runs the same softmax/top-K as the batched router.
// Many workgroups stream W_gate from L2 at once, where the batched router's
// two workgroups at n = 32 walk it in four dependent rounds each (11.2 against
// 6.9 us at the decode shape; with 256 threads per workgroup, 14.4 us).
// ---------------------------------------------------------------------------
constexpr int kRowsThreads = 1024;
constexpr int kRowsMaxTokens = 256;  // the batched router takes over above this

template <int CH>
__global__ __launch_bounds__(kRowsThreads) void route_bf16_rows_kernel(const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ Wg,
                                                                       const float* __restrict__ bias, int H, int K,
                                                                       int renorm, float* __restrict__ logits,
                                                                       int32_t* __restrict__ ids,
                                                                       float* __restrict__ wout) {
  constexpr int E = CH * 8;
  constexpr int RPS = kRowsThreads / CH;  // rows per step
  constexpr int U = 8;                    // steps whose loads are in flight together
  __shared__ float part[kRowsThreads][9];  // 8 partial sums per thread (+1: bank spread)
  __shared__ float lg[E];
  __shared__ uint32_t keys[E];
  __shared__ float scratch[kScratch];
  const int tid = threadIdx.x, t = blockIdx.x;
  const int c = tid % CH, r0 = tid / CH;
  const uint16_t* xr = x + (size_t)t * H;
  const uint16_t* wr = Wg + c * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int rb = r0; rb < H; rb += U * RPS) {
    u32x4_t w[U];
    uint16_t xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * RPS;
      w[u] = r < H ? *(const u32x4_t*)(wr + (size_t)r * E) : u32x4_t{0u, 0u, 0u, 0u};
      xv[u] = r < H ? xr[r] : (uint16_t)0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float xf = bf16_to_f32(xv[u]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(xf, __uint_as_float(w[u][q] << 16), acc[2 * q]);
        acc[2 * q + 1] = fmaf(xf, __uint_as_float(w[u][q] & 0xFFFF0000u), acc[2 * q + 1]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[tid][j] = acc[j];
  __syncthreads();
  // Expert e = 8c + j: the partial sums of threads c, c + CH, c + 2 CH, ...,
  // added in that order.
  for (int e = tid; e < E; e += kRowsThreads) {
    const int ce = e >> 3, j = e & 7;
    float v = 0.f;
    for (int i = 0; i < RPS; ++i) v += part[ce + CH * i][j];
    if (bias != nullptr) v += bias[e];
    lg[e] = v;
    keys[e] = order_key(v);
    logits[(size_t)t * E + e] = v;
  }
  __syncthreads();
  if (tid < 64) topk_token_any(lg, keys, E, K, renorm, scratch, ids + (size_t)t * K, wout + (size_t)t * K);
}

template <int CH>
void launch_rows(const uint16_t* x, const uint16_t* Wg, const float* bias, int n, int H, int K, int renorm,
                 float* logits, int32_t* ids, float* w, hipStream_t s) {
  route_bf16_rows_kernel<CH><<<n, kRowsThreads, 0, s>>>(x, Wg, bias, H, K, renorm, logits, ids, w);
}

// ---------------------------------------------------------------------------
// fp32 router: one wave per token, lanes over experts, sequential fp32 FMA
// over the hidden dimension. Also the softmax/top-K-only entry (x == NULL).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_f32_kernel(const float* __restrict__ x, const float* __restrict__ Wg,
                                                        const float* __restrict__ bias,
                                                        const float* __restrict__ logits_in, int n, int H, int E,
                                                        int K, int renorm, float* __restrict__ logits,
                                                        int32_t* __restrict__ ids, float* __restrict__ wout) {
  __shared__ __attribute__((aligned(16))) float lg[4][kMaxExperts];
  __shared__ __attribute__((aligned(16))) uint32_t keys[4][kMaxExperts];
  __shared__ __attribute__((aligned(16))) float slots[4][kScratch];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= n) return;
  for (int e = lane; e < E; e += 64) {
    float v;
    if (x != nullptr) {
      const float* xr = x + (size_t)t * H;
      v = 0.f;
      for (int h = 0; h < H; ++h) v = fmaf(xr[h], Wg[(size_t)h * E + e], v);
      if (bias != nullptr) v += bias[e];
      logits[(size_t)t * E + e] = v;
    } else {
      v = logits_in[(size_t)t * E + e];
    }
    lg[wave][e] = v;
    keys[wave][e] = order_key(v);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  topk_token_any(lg[wave], keys[wave], E, K, renorm, slots[wave], ids + (size_t)t * K, wout + (size_t)t * K);
}

template <int NT, int WK>
void launch_bf16(const uint16_t* x, const uint16_t* Wg, const float* bias, int n, int H, int E, int K, int renorm,
                 float* logits, int32_t* ids, float* w, hipStream_t s) {
  static_assert(RouteCfg<NT, WK>::LDS <= 160 * 1024, "router LDS budget");
  route_bf16_kernel<NT, WK><<<ceil_div(n, kTok), 64 * WK, 0, s>>>(x, Wg, bias, n, H, E, K, renorm, logits, ids, w);
}

}  // namespace

hipError_t launch_route(const void* x, const void* W_gate, const float* bias, int n, int H, int E, int K,
                        int renorm, moe_dtype dt, float* logits, int32_t* topk_ids, float* topk_w,
                        hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (x != nullptr && dt == MOE_BF16) {
    const uint16_t* xb = (const uint16_t*)x;
    const uint16_t* wb = (const uint16_t*)W_gate;
    if (n <= kRowsMaxTokens) {  // small batches: one workgroup per token (E = 8 * 2^k)
      switch (E) {
        case 8: launch_rows<1>(xb, wb, bias, n, H, K, renorm, logits, topk_ids, topk_w, s); return hipGetLastError();
        case 16: launch_rows<2>(xb, wb, bias, n, H, K, renorm, logits, topk_ids, topk_w, s); return hipGetLastError();
        case 32: launch_rows<4>(xb, wb, bias, n, H, K, renorm, logits, topk_ids, topk_w, s); return hipGetLastError();
        case 64: launch_rows<8>(xb, wb, bias, n, H, K, renorm, logits, topk_ids, topk_w, s); return hipGetLastError();
        case 128: launch_rows<16>(xb, wb, bias, n, H, K, renorm, logits, topk_ids, topk_w, s); return hipGetLastError();
        case 256: launch_rows<32>(xb, wb, bias, n, H, K, renorm, logits, topk_ids, topk_w, s); return hipGetLastError();
        default: break;
      }
    }
    const int nt = ceil_div(E, 16);
    if (nt <= 1)
      launch_bf16<1, 8>(xb, wb, bias, n, H, E, K, renorm, logits, topk_ids, topk_w, s);
    else if (nt <= 2)
      launch_bf16<2, 8>(xb, wb, bias, n, H, E, K, renorm, logits, topk_ids, topk_w, s);
    else if (nt <= 4)
      launch_bf16<4, 8>(xb, wb, bias, n, H, E, K, renorm, logits, topk_ids, topk_w, s);
    else if (nt <= 8)
      launch_bf16<8, 4>(xb, wb, bias, n, H, E, K, renorm, logits, topk_ids, topk_w, s);
    else
      launch_bf16<16, 2>(xb, wb, bias, n, H, E, K, renorm, logits, topk_ids, topk_w, s);
    return hipGetLastError();
  }
  // fp32 router, or softmax/top-K from caller-supplied logits (x == NULL).
  route_f32_kernel<<<ceil_div(n, 4), 256, 0, s>>>((const float*)x, (const float*)W_gate, bias,
                                                   x == nullptr ? logits : nullptr, n, H, E, K, renorm, logits,
                                                   topk_ids, topk_w);
  return hipGetLastError();
}

}  // namespace moe
