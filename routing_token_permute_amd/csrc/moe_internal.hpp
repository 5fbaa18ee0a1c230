// Internal declarations shared by the HIP kernels and the C-ABI layer.
// Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Largest expert count the kernels accept (LDS histograms and the router's
// accumulators are sized for it) and the largest top-K (one lane per slot).
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 64;

// moe_permute: threads per count/place block; at most kPermMaxBlocks blocks.
constexpr int kPermThreads = 256;
constexpr int kPermMaxBlocks = 128;

// Router backward: dW_gate is summed over at most this many token chunks.
constexpr int kRouteBwdMaxChunks = 32;

// bf16 grouped GEMM tile.
constexpr int kGemmBM = 128;
constexpr int kGemmBN = 256;
constexpr int kGemmBK = 64;

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Number of BM-row tiles covering any split of `rows` rows into E segments:
// sum_e ceil(c_e / BM) <= (rows + min(E, rows) * (BM - 1)) / BM.
inline int max_row_tiles(int rows, int E, int BM) {
  long long nonempty = rows < E ? rows : E;
  return (int)(((long long)rows + nonempty * (BM - 1)) / BM);
}

// ---- host launchers (each returns hipGetLastError() after its launches) ----

hipError_t launch_route(const void* x, const void* W_gate, const float* bias, int n, int H, int E, int K,
                        int renorm, moe_dtype dt, float* logits, int32_t* topk_ids, float* topk_w,
                        hipStream_t s);

// block_counts: workspace of kPermMaxBlocks * E int32.
hipError_t launch_permute(const int32_t* topk_ids, const void* x, int n, int H, int E, int K, int ep,
                          moe_dtype dt, int32_t* counts, int32_t* offsets, int32_t* splits, int32_t* perm,
                          int32_t* inv, void* x_perm, int32_t* block_counts, hipStream_t s);

// h: workspace of rows * I elements of dt.
hipError_t launch_grouped_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13,
                                 const void* W2, int E, int H, int I, moe_dtype dt, void* Y_perm, void* h,
                                 hipStream_t s);

// The two GEMMs separately (launch_grouped_swiglu runs both).
hipError_t launch_w13_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13, int E, int H,
                             int I, moe_dtype dt, void* h, hipStream_t s);
// GEMM1 reading token rows x[perm[r] / K] directly (no permuted copy of x).
// packed: the weights are in the packed form of launch_pack_weights (bf16).
hipError_t launch_w13_swiglu_gather(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                    const void* W13, int E, int H, int I, moe_dtype dt, void* h, hipStream_t s,
                                    bool packed = false);
hipError_t launch_w2(const void* h, const int32_t* offsets, int rows, const void* W2, int E, int H, int I,
                     moe_dtype dt, void* Y_perm, hipStream_t s, bool packed = false);

// bf16 weights of E experts, each Kdim x Ncols row-major, rewritten in the
// GEMMs' tile order: per expert, per 32 K rows, one 16 KB unit for each of the
// NB 256-column output blocks (the layout is described where the GEMM tiles
// are defined). half > 0: W13 with gate columns [0, half) and up columns
// [half, 2 * half), block nb holding gate columns nb * 128 + [0, 128) and the
// matching up columns; half == 0: W2, block nb holding columns nb * 256 +
// [0, 256). Columns past the matrix are zero. Kdim % 32 == 0.
size_t packed_weight_bytes(int E, int Kdim, int NB);
hipError_t launch_pack_weights(const void* W, int E, int Kdim, int Ncols, int half, int NB, void* out,
                               hipStream_t s);

// GEMM2 with the routing weight and the un-permutation in its epilogue:
// Y_tok[perm[p]] = topk_w[perm[p]] * (h[p] . W2[e(p)]), rows in flat pair order.
hipError_t launch_w2_scatter(const void* h, const int32_t* offsets, int rows, const int32_t* perm,
                             const float* topk_w, const void* W2, int E, int H, int I, moe_dtype dt, void* Y_tok,
                             hipStream_t s,
                             bool packed = false);
// y[i] = sum_k Y_tok[i*K + k] in slot order (fp32 accumulation).
hipError_t launch_sum_slots(const void* Y_tok, int n, int H, int K, moe_dtype dt, void* y, hipStream_t s);
hipError_t launch_combine(const void* Y_perm, const int32_t* inv, const float* topk_w, int n, int H, int K,
                          moe_dtype dt, void* y, hipStream_t s);
// The same over a Y of y_rows rows (a padded buffer): inv entries in [0, y_rows) are gathered.
hipError_t launch_combine_rows(const void* Y_perm, int y_rows, const int32_t* inv, const float* topk_w, int n, int H,
                               int K, moe_dtype dt, void* y, hipStream_t s);

// Persistent single-kernel GEMM1 + SwiGLU + GEMM2 (bf16): route and permute
// metadata as for launch_w13_swiglu_gather, h in `hbuf` (a ring of `pool`
// row-tile slots per XCD queue, or all rows when pool is 0), Y_perm expert-
// major. `counters`: fused_ffn_counter_bytes(n*K, E) bytes, zeroed by the
// launcher; its last int32 becomes nonzero if a bounded wait ran out.
int fused_ffn_max_row_tiles(int rows, int E);
size_t fused_ffn_counter_bytes(int rows, int E);
size_t fused_ffn_h_bytes(int rows, int E, int I, int pool);
hipError_t launch_fused_ffn(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets, const void* W13,
                            const void* W2, int E, int H, int I, int warm, int pool, void* hbuf, void* Y_perm,
                            int* counters, hipStream_t s,
                            bool packed = false);

// Decode-sized GEMM1 (bf16, n <= 32 tokens, n * K <= 1024 pairs, E <= 256):
// the GEMM places the routing ids itself (the placement moe_permute makes) and
// also writes counts, offsets, splits, perm and inv, so no permute launch
// precedes it. w13_from_ids_ok says whether a shape qualifies.
bool w13_from_ids_ok(int n, int K, int E, moe_dtype dt);
hipError_t launch_w13_swiglu_from_ids(const void* x, const int32_t* ids, int n, int K, const void* W13, int E,
                                      int H, int I, int ep, void* h, int32_t* counts, int32_t* offsets,
                                      int32_t* splits, int32_t* perm, int32_t* inv, hipStream_t s,
                                      bool packed = false);

// ---- backward ----

// GEMM1 that also writes the pre-activations [gate | up] (rows, 2I) for the backward.
hipError_t launch_w13_swiglu_gather_train(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                          const void* W13, int E, int H, int I, moe_dtype dt, void* h, void* gate_up,
                                          hipStream_t s);
// x_perm[p] = x[perm[p] / K] for all n*K rows.
hipError_t launch_gather_rows(const void* x, const int32_t* perm, int n, int H, int K, moe_dtype dt, void* x_perm,
                              hipStream_t s);
// dY_perm[inv[iK+k]] = w[i,k] dy[i]; dw[i,k] = <dy[i], Y_perm[inv[iK+k]]>.
hipError_t launch_combine_backward(const void* dy, const void* Y_perm, const int32_t* inv, const float* topk_w, int n,
                                   int H, int K, moe_dtype dt, void* dY_perm, float* dw, hipStream_t s);
// dx[i] = (add[i] if add) + sum_k dX_perm[inv[iK+k]], slot order, one rounding.
hipError_t launch_dispatch_backward(const void* dX_perm, const int32_t* inv, const float* add, int n, int H, int K,
                                    moe_dtype dt, void* dx, hipStream_t s);
// dgate_up = SwiGLU'(gate_up) applied to dY_perm . W2[e]^T.
hipError_t launch_w2_backward(const void* dY_perm, const int32_t* offsets, int rows, const void* W2,
                              const void* gate_up, int E, int H, int I, moe_dtype dt, void* dgate_up, hipStream_t s);
// dX_perm = dgate_up . W13[e]^T.
hipError_t launch_w13_backward(const void* dgate_up, const int32_t* offsets, int rows, const void* W13, int E, int H,
                               int I, moe_dtype dt, void* dX_perm, hipStream_t s);
// dW[e] = a_e^T . b_e over each expert's rows; a (rows, M), b (rows, N), dW (E, M, N).
hipError_t launch_weight_grad(const void* a, const void* b, const int32_t* offsets, int rows, int E, int M, int N,
                              moe_dtype dt, void* dW, hipStream_t s);
// Zero `bytes` (a multiple of 4) with a kernel.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// dW[e] = x_e^T . b_e with the rows of x gathered: row r of x_e is x[perm[r] / K].
hipError_t launch_weight_grad_gather(const void* x, const int32_t* perm, int n, int K, const void* b,
                                     const int32_t* offsets, int E, int M, int N, moe_dtype dt, void* dW,
                                     hipStream_t s);
// Token chunks of the dW_gate reduction for n tokens.
int route_bwd_chunks(int n);
// Workspace bytes of launch_route_backward.
size_t route_bwd_workspace(int n, int H, int E);
// ws: route_bwd_workspace(n, H, E) bytes (only used when dx_router, dW_gate
// or dbias is wanted).
hipError_t launch_route_backward(const void* x, const void* W_gate, const float* logits, const int32_t* ids,
                                 const float* topk_w, const float* dw, int n, int H, int E, int K, int renorm,
                                 moe_dtype dt, float* dlogits, float* dx_router, float* dW_gate, float* dbias,
                                 void* ws, hipStream_t s);
// The router's two products on MFMA (bf16 path, E a multiple of 32), from the
// split dlogits [hi | lo] (n, 2E) bf16:
//   dx_router (n, H) fp32 = hilo . [W_gate | W_gate]^T, rows grouped by row_offsets = {0, n};
//   part (S, H, 2E) fp32 = x_g^T . hilo_g per token chunk g of chunk_offsets (S+1).
hipError_t launch_router_dx_mfma(const void* dl_hilo, const int32_t* row_offsets, int n, const void* W_gate, int H,
                                 int E, float* dx_router, hipStream_t s);
hipError_t launch_router_dw_mfma(const void* x, const void* dl_hilo, const int32_t* chunk_offsets, int S, int n,
                                 int H, int E, float* part, hipStream_t s);

// ---- FP8 E4M3 expert weights ----

// codes (E, N, Kd) = nearest E4M3 codes of W (E, Kd, N) / scales (E, N),
// scales = column amax / 448 (1 for a zero column).
hipError_t launch_quantize_fp8(const void* W, int E, int Kd, int N, moe_dtype dt, uint8_t* codes, float* scales,
                               hipStream_t s);
// GEMM1 + SwiGLU with W13 codes (E, 2I, H) and scales (E, 2I), rows gathered through perm.
hipError_t launch_w13_swiglu_gather_fp8(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                        const uint8_t* W13q, const float* s13, int E, int H, int I, void* h,
                                        hipStream_t s);
// The same from the routing ids on decode-sized batches (n <= 32, n * K <=
// 1024, E <= 256): the GEMM places the pairs itself and writes counts,
// offsets, splits, perm and inv.
bool w13_from_ids_fp8_ok(int n, int K, int E);
hipError_t launch_w13_swiglu_from_ids_fp8(const void* x, const int32_t* ids, int n, int K, const uint8_t* W13q,
                                          const float* s13, int E, int H, int I, int ep, void* h, int32_t* counts,
                                          int32_t* offsets, int32_t* splits, int32_t* perm, int32_t* inv,
                                          hipStream_t s);
// GEMM2 with W2 codes (E, H, I) and scales (E, H).
hipError_t launch_w2_fp8(const void* h, const int32_t* offsets, int rows, const uint8_t* W2q, const float* s2, int E,
                         int H, int I, void* Y_perm, hipStream_t s);

// ---- FP8 activations ----

// Rows of the padded FP8 receive buffer for n tokens, top-K: n*K plus at most
// 15 padding rows per expert that received rows.
size_t fp8_padded_rows(int n, int E, int K);
// codes (n, H) = nearest E4M3 codes of x / scales, scales (n) = row amax / 448 (1 for a zero row).
hipError_t launch_quantize_rows_fp8(const void* x, int n, int H, moe_dtype dt, uint8_t* codes, float* scales,
                                    hipStream_t s);
// The padded receive buffer from moe_permute's counts, offsets and perm and the per-token codes/scales.
hipError_t launch_dispatch_fp8(const int32_t* counts, const int32_t* offsets, const int32_t* perm, int n, int E,
                               int K, const uint8_t* codes_tok, const float* s_tok, int H, int32_t* offsets_padded,
                               uint8_t* x_q, float* x_scale, int32_t* perm_padded, int32_t* inv_padded,
                               hipStream_t s);
// GEMM1 + SwiGLU with FP8 activation rows (padded groups) and FP8 W13 codes (E, 2I, H).
hipError_t launch_w13_swiglu_fp8a(const uint8_t* x_q, const float* x_scale, const int32_t* offsets_padded,
                                  int rows_max, const uint8_t* W13q, const float* s13, int E, int H, int I, void* h,
                                  hipStream_t s);
// GEMM1 + SwiGLU with FP8 activations read in place: row r of the expert-major
// order is token perm[r] / K of the per-token codes (n, H) and scales (n);
// h (n*K, I) bf16 over the unpadded offsets.
hipError_t launch_w13_swiglu_gather_fp8a(const uint8_t* codes_tok, const float* s_tok, const int32_t* perm, int n,
                                         int K, const int32_t* offsets, const uint8_t* W13q, const float* s13, int E,
                                         int H, int I, void* h, hipStream_t s);
// The same from the routing ids on decode-sized batches (n <= 32, n * K <=
// 1024, E <= 256): the GEMM places the pairs itself and writes counts,
// offsets, splits, perm and inv. w13_from_ids_fp8a_ok says whether it serves
// a shape.
bool w13_from_ids_fp8a_ok(int n, int K, int E);
hipError_t launch_w13_swiglu_from_ids_fp8a(const uint8_t* codes_tok, const float* s_tok, const int32_t* ids, int n,
                                           int K, const uint8_t* W13q, const float* s13, int E, int H, int I, int ep,
                                           void* h, int32_t* counts, int32_t* offsets, int32_t* splits,
                                           int32_t* perm, int32_t* inv, hipStream_t s);
// GEMM2 with FP8 activations: Y_perm (rows_max, H) bf16 = (h codes x per-row
// scales) . (W2 codes x column scales) over the padded receive buffer's rows.
hipError_t launch_w2_fp8a(const uint8_t* h_q, const float* h_scale, const int32_t* offsets_padded, int rows_max,
                          const uint8_t* W2q, const float* s2, int E, int H, int I, void* Y_perm, hipStream_t s);

}  // namespace moe

// ---- device helpers ----
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_char_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// SwiGLU of one output: SiLU(g) * u = g * u / (1 + e^-g), with e^-g from the
// hardware base-2 exponential and the quotient from the hardware reciprocal
// (each about 1 ulp of fp32, far below the bf16 rounding that follows). For
// g -> -inf, e^-g overflows to +inf and the reciprocal to 0, the exact limit.
__device__ __forceinline__ float swiglu_f32(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.f + e) * u;
}

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lanes 4r..4r+3 together supply row r (16 consecutive 16-bit elements, 4
// per lane); lane c of the group receives column c of those 4 rows.
__device__ __forceinline__ bf16x4_t lds_read_tr16(const lds_char_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)p);
}

// Nearest E4M3 code of x (ties to the even mantissa, magnitudes saturated at
// 448; NaN is not expected), from the format: 1 sign, 4 exponent bits (bias
// 7), 3 mantissa bits, subnormals m * 2^-9, largest finite 1.75 * 2^8.
__device__ __forceinline__ uint32_t e4m3_nearest(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: steps of 2^-9 (m = 8 is the smallest normal, code 8)
    code = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t b = __float_as_uint(a);
    int ex = (int)(b >> 23) - 127 + 7;                             // biased E4M3 exponent, 1..15
    const float f = __uint_as_float((b & 0x007FFFFFu) | 0x3F800000u);  // 1.m in [1, 2)
    int m = (int)rintf((f - 1.f) * 8.f);                           // exact scaling, then RNE
    if (m == 8) {
      m = 0;
      ++ex;
    }
    code = ((uint32_t)ex << 3) | (uint32_t)m;
  }
  return code == 0 ? 0u : (sign | code);
}

// Four nearest E4M3 codes packed little-endian, by the gfx950 conversion
// (v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even, subnormals kept), with a
// negative zero mapped to code 0 as e4m3_nearest does. For |v| < 464, where
// nearest-with-saturation and the plain nearest value agree (the callers'
// quotients x / s are at most 448 (1 + 2^-23)).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  const uint32_t w = (uint32_t)r;
  // bit 7 of each byte: set where the byte's magnitude is nonzero
  const uint32_t nz = ((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;
  return w & (0x7F7F7F7Fu | nz);
}

__device__ __forceinline__ u32x4_t lds_read_b128(const lds_char_t* p) {
  return *(const __attribute__((address_space(3))) u32x4_t*)p;
}

__device__ __forceinline__ void lds_write_b128(lds_char_t* p, u32x4_t v) {
  *(__attribute__((address_space(3))) u32x4_t*)p = v;
}

}  // namespace moe
#endif
