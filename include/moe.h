/*
 * moe.h — C ABI of the single-GPU MoE expert layer on MI355X (gfx950): the
 * forward, its pieces, the backward (training) pass and FP8 expert weights.
 *
 * The layer is Algorithm 2 "Single-GPU MoE Forward" of the page
 * "MoE 分布式推理基础（基于 vLLM）" (cnblogs, §1.2 MoE Forward), with the
 * router and experts as in the Hugging Face OlmoeTopKRouter /
 * OlmoeExperts.forward source that section quotes:
 *
 *   logits = x · W_gate (+ bias)            (n, E)
 *   p      = softmax(logits)                 (n, E)
 *   (w_top, e_top) = TopK(p, K)              (n, K) each, optional renorm
 *   for each expert e: X_e = rows of x routed to e,
 *       Y_e = (SiLU(X_e·W13[e][:, :I]) * (X_e·W13[e][:, I:])) · W2[e]
 *   y[i] = sum over the K slots of w_top[i,k] · Y_{e_top[i,k]}[row of (i,k)]
 *
 * Notation follows the page: n tokens, hidden size H, expert intermediate
 * size I, E experts, top-K. Shapes are row-major:
 *   x (n, H); W_gate (H, E); W13 (E, H, 2I) with gate = columns [0, I) and
 *   up = columns [I, 2I); W2 (E, I, H); y (n, H).
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers owned by the caller; the
 *     library allocates no memory and keeps no per-call state (moe_backward
 *     keeps one auxiliary stream per device, see there). Scratch memory is a
 *     caller-supplied workspace whose size the *_workspace_size functions
 *     return.
 *   - Calls are asynchronous on the given HIP stream (0 = the null stream)
 *     and never synchronise the host. Results are valid once the stream has
 *     reached the end of the call.
 *   - Arguments are validated on the host before anything is enqueued:
 *     MOE_EINVAL for null required pointers, negative or zero sizes where a
 *     size must be positive, K outside [1, min(E, 64)], E outside
 *     [1, 256], ep not dividing E, a workspace smaller than required, or
 *     shapes the kernels do not cover (bf16: H and I multiples of 64;
 *     fp32: H and I multiples of 4; H and I at most 2^20);
 *     MOE_EUNSUPPORTED for a dtype value
 *     that is not built. Nothing is enqueued when a call returns an error.
 *   - Alignment: every row matrix (x, x_perm, h, gate_up, Y_perm, y and
 *     their gradients), every weight array (W_gate, W13, W2, FP8 codes and
 *     scales), the fp32 router-gradient buffers, the `add` addend and every
 *     workspace must be 16-byte aligned (the kernels move them with 16-byte
 *     vector loads, LDS DMA and buffer stores); the per-pair and per-expert
 *     int32/fp32 arrays (topk_ids, topk_w, logits, bias, counts, offsets,
 *     splits, perm, inv, dw, dlogits, dbias) 4-byte aligned. A misaligned
 *     pointer gives MOE_EINVAL before anything is enqueued.
 *   - MOE_EHIP reports a kernel launch failure (hipGetLastError after each
 *     launch); the stream may then hold part of the call's work.
 *   - n == 0 (or rows == 0) is valid: outputs that have one entry per expert
 *     or rank are still written (zeros), nothing else is touched; the
 *     layer calls (moe_forward, moe_forward_fp8) then need no workspace.
 *   - Calls on different streams may run concurrently when their outputs
 *     and workspaces do not overlap.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs on every run (no floating-point atomics).
 *   - Expert ids handed to the library must lie in [0, E); a pair whose id
 *     lies outside is skipped (not counted, not placed; its perm/inv
 *     entries are undefined) and never causes an out-of-bounds access.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* bad argument, detected on the host before any launch */
  MOE_EUNSUPPORTED = 2, /* dtype or shape combination not built */
  MOE_EWORKSPACE = 3,   /* workspace pointer null or smaller than required */
  MOE_EHIP = 4,         /* a HIP launch failed */
  MOE_ETOOLARGE = 5     /* moe_forward_noalloc: the problem needs more than its fixed scratch */
} moe_status;

/* Element type of x, W_gate, W13, W2, x_perm, Y_perm and y.
 * MOE_BF16: bfloat16 storage, fp32 accumulation (MFMA), the intermediate h
 *           rounded to bf16 (round-to-nearest-even) before the second GEMM.
 * MOE_F32:  fp32 storage and arithmetic throughout.
 * Router logits, routing weights and the bias are fp32 in both cases. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Static description of a status code; never NULL. */
const char* moe_status_string(moe_status s);

/* Library version as major*10000 + minor*100 + patch. */
int moe_version(void);

/* Properties of the current HIP device that the roofline figures are derived
 * from: compute units, peak shader clock (kHz), peak memory clock (kHz) and
 * memory bus width (bits), from hipDeviceGetAttribute. Any pointer may be
 * NULL. Returns MOE_EHIP when a query fails. */
moe_status moe_device_info(int* compute_units, int* sclk_khz, int* mem_clk_khz, int* mem_bus_bits);

/* ---------------------------------------------------------------------------
 * moe_route — router GEMM, softmax and top-K (Algorithm 2 steps 1-3; the
 * OlmoeTopKRouter source of the same section: F.linear, softmax, topk, and
 * the optional division of the K weights by their sum).
 *
 *   x       (n, H) dtype, or NULL: then `logits` is an INPUT the caller filled
 *           (fp32, (n, E)) and only softmax/top-K run.
 *   W_gate  (H, E) dtype; ignored when x == NULL.
 *   bias    (E) fp32 added to each logit after the product, or NULL. -inf
 *           entries are allowed: such experts get probability 0 and are
 *           only selected when fewer than K finite logits remain.
 *   renorm  nonzero: w_top[i,:] /= sum_k w_top[i,k].
 *   logits  (n, E) fp32: written when x != NULL, read when x == NULL.
 *   topk_ids (n, K) int32 out: slot 0 holds the largest logit; experts are
 *           ranked by (fp32 logit descending, expert index ascending), which
 *           is the softmax order with ties to the lowest index, decided on
 *           the fp32 logits (-0.0 counts as +0.0).
 *   topk_w  (n, K) fp32 out: softmax probability of each selected expert
 *           (max-subtracted, fp32), renormalised if asked.
 * The router product accumulates in fp32 (bf16: MFMA; for at most 256 tokens
 * and E a power of two times 8, one workgroup per token with fp32 FMA, the
 * partial sums added in a fixed order). NaN logits are not supported (the
 * selection is then unspecified, still in bounds).
 * ------------------------------------------------------------------------- */
moe_status moe_route(const void* x, const void* W_gate, const float* bias, int n, int H, int E, int K,
                     int renorm, moe_dtype dt, float* logits, int32_t* topk_ids, float* topk_w,
                     hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_permute — per-expert counts, offsets and per-rank splits, the stable
 * expert-major permutation of the n*K (token, slot) pairs, and the row
 * gather x_perm[p] = x[perm[p] / K].
 *
 * Defines: n_e = sum 1[e_top = e] (hit statistics under Algorithm 2);
 * Algorithm 2 step 5/7 (the set I_e and the gather X_e); the expert-sorted
 * order of moe_align_block_size in §2.3 of the same page (pairs sorted by
 * expert, ascending flat index i*K+k within an expert, without padding);
 * the per-rank send sizes of Algorithm 5 step 3 (§2.4); and the torchtitan
 * `_local_reorder` of the page "0. goin" (§2.2).
 *
 *   topk_ids (n, K) int32, each in [0, E).
 *   x        (n, H) dtype, or NULL to compute the metadata only.
 *   ep       number of expert-parallel ranks (>= 1, divides E): rank j owns
 *            experts [j*E/ep, (j+1)*E/ep).
 *   counts   (E) int32 out: n_e.
 *   offsets  (E+1) int32 out: offsets[0] = 0, offsets[e+1] = offsets[e] + n_e.
 *   splits   (ep) int32 out: splits[j] = offsets[(j+1)E/ep] - offsets[jE/ep].
 *   perm     (n*K) int32 out: perm[p] = flat pair index i*K+k at permuted row p.
 *   inv      (n*K) int32 out: inv[perm[p]] = p.
 *   x_perm   (n*K, H) dtype out, or NULL (required when x != NULL).
 *   ws       workspace of at least moe_permute_workspace_size(n, E, K) bytes.
 * ------------------------------------------------------------------------- */
size_t moe_permute_workspace_size(int n, int E, int K);
moe_status moe_permute(const int32_t* topk_ids, const void* x, int n, int H, int E, int K, int ep,
                       moe_dtype dt, int32_t* counts, int32_t* offsets, int32_t* splits, int32_t* perm,
                       int32_t* inv, void* x_perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_swiglu — every expert's SwiGLU FFN on its contiguous segment of
 * expert-major rows (Algorithm 2 steps 8-9; "SwiGLU expert 的两段 GEMM" of
 * the same section: gate_up = X_e @ W13[e]; gate, up = chunk(2); h =
 * silu(gate) * up; Y_e = h @ W2[e]).
 *
 *   x_perm   (rows, H) dtype: row r belongs to expert e when
 *            offsets[e] <= r < offsets[e+1].
 *   offsets  (E+1) int32, DEVICE memory, nondecreasing, offsets[E] <= rows
 *            (rows past offsets[E] are left untouched in Y_perm).
 *   W13      (E, H, 2I) dtype; W2 (E, I, H) dtype.
 *   Y_perm   (rows, H) dtype out.
 *   ws       workspace of at least moe_grouped_swiglu_workspace_size(rows, I, dt)
 *            bytes (it holds h, (rows, I)).
 * ------------------------------------------------------------------------- */
size_t moe_grouped_swiglu_workspace_size(int rows, int I, moe_dtype dt);
moe_status moe_grouped_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13,
                              const void* W2, int E, int H, int I, moe_dtype dt, void* Y_perm, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* The two halves of moe_grouped_swiglu, for callers that schedule or time
 * them separately (same arguments and rules as above).
 *
 * moe_expert_w13_swiglu — Algorithm 2 step 8: for every expert segment,
 *   h = SiLU(X_e · W13[e][:, :I]) * (X_e · W13[e][:, I:]), h (rows, I) dtype out
 *   (bf16: fp32 accumulation, SiLU and product in fp32, then rounded to bf16).
 * moe_expert_w2 — Algorithm 2 step 9: Y_perm = h · W2[e] per segment,
 *   h (rows, I) dtype in, Y_perm (rows, H) dtype out.
 * Neither needs a workspace. */
moe_status moe_expert_w13_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13, int E, int H,
                                 int I, moe_dtype dt, void* h, hipStream_t stream);
/* moe_expert_w13_swiglu_gather — Algorithm 2 steps 7-8 fused: the gather
 * X_e = x[{i : (i,k) in I_e}] happens inside the GEMM's operand loads, so no
 * permuted copy of x is written. Row r of h belongs to pair perm[r] = i*K+k
 * and uses token row x[perm[r] / K].
 *   x (n, H) dtype; perm (n*K) int32 from moe_permute; offsets (E+1) int32;
 *   h (n*K, I) dtype out. perm entries outside [0, n*K) read token row 0. */
moe_status moe_expert_w13_swiglu_gather(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                        const void* W13, int E, int H, int I, moe_dtype dt, void* h,
                                        hipStream_t stream);
moe_status moe_expert_w2(const void* h, const int32_t* offsets, int rows, const void* W2, int E, int H, int I,
                         moe_dtype dt, void* Y_perm, hipStream_t stream);

/* moe_expert_w13_swiglu_from_ids — Algorithm 2 steps 5-8 in one launch for a
 * decode-sized batch: moe_permute's metadata (no x_perm) and
 * moe_expert_w13_swiglu_gather's h, computed straight from the routing ids.
 * Every workgroup places the pairs itself in on-chip memory; one of them also
 * writes counts, offsets, splits, perm and inv, with the values (and the
 * meaning) moe_permute gives them, for the kernels that follow. h is bit for
 * bit what moe_permute + moe_expert_w13_swiglu_gather give.
 *   x (n, H) bf16; topk_ids (n, K) int32 with K distinct experts per token in
 *   [0, E) (as moe_route writes them); W13 (E, H, 2I) bf16; ep as moe_permute;
 *   h (n*K, I) bf16 out; counts (E), offsets (E+1), splits (ep), perm (n*K),
 *   inv (n*K) int32 out.
 * Shapes it serves: dt = MOE_BF16, n <= 32, n*K <= 1024, E <= 256; others
 * return MOE_EUNSUPPORTED (use moe_permute and moe_expert_w13_swiglu_gather).
 * An id outside [0, E) is neither counted nor placed; ids repeated within a
 * token give unspecified h rows (still in bounds). n == 0 writes zero counts,
 * offsets and splits. */
moe_status moe_expert_w13_swiglu_from_ids(const void* x, const int32_t* topk_ids, int n, int K, const void* W13,
                                          int E, int H, int I, int ep, moe_dtype dt, void* h, int32_t* counts,
                                          int32_t* offsets, int32_t* splits, int32_t* perm, int32_t* inv,
                                          hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_w2_scatter — Algorithm 2 steps 9-11 with the weight and the
 * un-permutation in GEMM2's epilogue: the second MoE layer of "大模型系统中的
 * 通算融合" §4.2.5 (expert GEMM, gather back to token order, weighted top-K
 * reduce) with its gather and weighting folded into the GEMM, and the output
 * landing in the layout its consumer reads (§8.5 of the same page):
 *
 *   Y_tok[perm[p]] = topk_w[perm[p]] * (h[p] · W2[e])   for every row p of
 *   expert e's segment, the product accumulated in fp32 and rounded to dt
 *   after the scaling.
 *
 *   h (rows, I) dtype; offsets (E+1) int32; perm (rows) int32 from
 *   moe_permute (perm[p] = i*K+k, rows = n*K); topk_w (rows) fp32, indexed by
 *   the flat pair index (the (n, K) routing weights); Y_tok (rows, H) dtype
 *   out, row i*K+k holding token i's slot k. perm entries outside [0, rows)
 *   write nothing. No workspace.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_w2_scatter(const void* h, const int32_t* offsets, int rows, const int32_t* perm,
                                 const float* topk_w, const void* W2, int E, int H, int I, moe_dtype dt,
                                 void* Y_tok, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_sum_slots — the top-K reduction over rows that moe_expert_w2_scatter
 * already weighted and placed in token order (Algorithm 2 step 11):
 *
 *   y[i] = sum_{k=0..K-1} Y_tok[i*K+k]
 *
 * in slot order with fp32 accumulation, then stored in dt.
 *   Y_tok (n*K, H) dtype; y (n, H) dtype out.
 * ------------------------------------------------------------------------- */
moe_status moe_sum_slots(const void* Y_tok, int n, int H, int K, moe_dtype dt, void* y, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_unpermute_combine — weighted top-K reduction back to token order
 * (Algorithm 2 steps 10-11, the scatter-add y[i] += Y_e[idx] * w_top[i,k];
 * the `_unpermute` + weighted deterministic scatter-add of "0. goin" §2.2
 * and its top-K slot reduction kernel, §2.3):
 *
 *   y[i] = sum_{k=0..K-1} w[i,k] * Y_perm[inv[i*K+k]]
 *
 * summed in slot order k = 0..K-1 with fp32 accumulation, then stored in dt.
 *   Y_perm  (n*K, H) dtype; inv (n*K) int32 in [0, n*K);
 *   topk_w  (n, K) fp32, or NULL for unit weights (with K = 1 this is a plain
 *           un-permute back to arrival order);
 *   y       (n, H) dtype out.
 * ------------------------------------------------------------------------- */
moe_status moe_unpermute_combine(const void* Y_perm, const int32_t* inv, const float* topk_w, int n, int H,
                                 int K, moe_dtype dt, void* y, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_forward — the whole layer, Algorithm 2: moe_route, the metadata part
 * of moe_permute (ep=1), moe_expert_w13_swiglu_gather, moe_expert_w2 and
 * moe_unpermute_combine enqueued back to back on one stream, with no host
 * synchronisation. For shapes moe_expert_w13_swiglu_from_ids serves (bf16,
 * n <= 32) that call replaces the permute and the gathered GEMM1 (same
 * results, one launch fewer).
 *
 *   y            (n, H) dtype out.
 *   logits_out   (n, E) fp32 out, or NULL.
 *   topk_ids_out (n, K) int32 out, or NULL.
 *   topk_w_out   (n, K) fp32 out, or NULL.
 *   counts_out   (E) int32 out, or NULL.
 *   ws           workspace of at least moe_forward_workspace_size(...) bytes.
 * ------------------------------------------------------------------------- */
size_t moe_forward_workspace_size(int n, int H, int I, int E, int K, moe_dtype dt);

/* The same size under the name of the layer's planned interface
 * (workspace of moe_forward). */
size_t moe_workspace_size(int n, int H, int I, int E, int K, moe_dtype dt);
moe_status moe_forward(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2,
                       int n, int H, int I, int E, int K, int renorm, moe_dtype dt, void* y, float* logits_out,
                       int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* moe_forward_timed — moe_forward that also records two caller-created HIP
 * events on `stream`, right before and right after the layer's GEMM1 launch
 * (the gathered GEMM1 + SwiGLU, or at n <= 32 the GEMM1 from the ids), so
 * that a caller can time the layer's dominant kernel inside the layer call.
 * Either event may be NULL (then it is not recorded); with both NULL this is
 * moe_forward. The events stay the caller's. With n == 0 nothing is recorded. */
moe_status moe_forward_timed(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2,
                             int n, int H, int I, int E, int K, int renorm, moe_dtype dt, void* y,
                             float* logits_out, int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                             void* ws, size_t ws_bytes, hipEvent_t gemm1_begin, hipEvent_t gemm1_end,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Packed expert weights. "大模型系统中的通算融合" §4.4 describes a fused MoE
 * kernel that takes its weights converted once, ahead of time, into the
 * kernel's own layout, and §8.5 counts such pre-converted weights among the
 * ways to keep layout copies off the critical path. moe_pack_w13 and
 * moe_pack_w2 make that conversion for the bf16 GEMMs here: for each expert
 * and each 32 rows of K, one 16 KB unit per 256-column output block (the
 * blocks' units side by side), each column's 32 values contiguous and
 * swizzled as the GEMM's on-chip tiles want them, so that a GEMM stage copies
 * whole contiguous units and reads its weight operands like its token
 * operands. Unit u of block nb of expert e starts at element
 * ((e * K/32 + u) * NB + nb) * 8192; within a unit, column c's 16-byte chunk q
 * (its k-values 8q .. 8q+7) sits at element c * 32 + 8 * (q ^ ((c / 2) % 4)).
 * GEMM1's blocks hold 128 gate columns followed by the matching 128 up
 * columns. Columns past the matrix (I or H
 * not a multiple of 128 / 256) are stored as zeros. The values are the
 * weights' own: moe_forward_packed gives bit for bit what moe_forward gives.
 *
 *   moe_packed_w13_bytes / moe_packed_w2_bytes: bytes of the packed form
 *     (E * ceil(I/128) * 256 * H * 2, E * ceil(H/256) * 256 * I * 2); 0 for
 *     shapes outside the bf16 GEMMs' range (1 <= E <= 256, H and I positive
 *     multiples of 64).
 *   moe_pack_w13: W13 (E, H, 2I) bf16 -> W13p; moe_pack_w2: W2 (E, I, H) bf16
 *     -> W2p. Both buffers device memory, 16-byte aligned, the caller's; W13p /
 *     W2p must hold the bytes above and must not overlap the input. One
 *     launch, stream-ordered. MOE_EINVAL for a bad shape or pointer.
 * ------------------------------------------------------------------------- */
size_t moe_packed_w13_bytes(int E, int H, int I);
size_t moe_packed_w2_bytes(int E, int H, int I);
moe_status moe_pack_w13(const void* W13, int E, int H, int I, void* W13p, hipStream_t stream);
moe_status moe_pack_w2(const void* W2, int E, int H, int I, void* W2p, hipStream_t stream);

/* The layer's GEMMs over packed weights, staged as their plain-layout
 * counterparts (bf16 only; every other argument, the validation and the
 * results, bit for bit, as moe_expert_w13_swiglu_gather,
 * moe_expert_w13_swiglu_from_ids and moe_expert_w2 with dt = MOE_BF16). */
moe_status moe_expert_w13_swiglu_gather_packed(const void* x, const int32_t* perm, int n, int K,
                                               const int32_t* offsets, const void* W13p, int E, int H, int I,
                                               void* h, hipStream_t stream);
moe_status moe_expert_w13_swiglu_from_ids_packed(const void* x, const int32_t* topk_ids, int n, int K,
                                                 const void* W13p, int E, int H, int I, int ep, void* h,
                                                 int32_t* counts, int32_t* offsets, int32_t* splits, int32_t* perm,
                                                 int32_t* inv, hipStream_t stream);
moe_status moe_expert_w2_packed(const void* h, const int32_t* offsets, int rows, const void* W2p, int E, int H,
                                int I, void* Y_perm, hipStream_t stream);
/* moe_expert_w2_scatter over packed W2 (bf16; as moe_expert_w2_scatter otherwise, bit for bit). */
moe_status moe_expert_w2_scatter_packed(const void* h, const int32_t* offsets, int rows, const int32_t* perm,
                                        const float* topk_w, const void* W2p, int E, int H, int I, void* Y_tok,
                                        hipStream_t stream);

/* moe_forward_packed — moe_forward (bf16 only) over packed weights: W13p and
 * W2p as moe_pack_w13 / moe_pack_w2 write them; every other argument, the
 * workspace size (moe_forward_workspace_size with MOE_BF16) and the results
 * as moe_forward's, bit for bit. gemm1_begin / gemm1_end: optional events,
 * as in moe_forward_timed. */
moe_status moe_forward_packed(const void* x, const void* W_gate, const float* bias, const void* W13p,
                              const void* W2p, int n, int H, int I, int E, int K, int renorm, void* y,
                              float* logits_out, int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                              void* ws, size_t ws_bytes, hipEvent_t gemm1_begin, hipEvent_t gemm1_end,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_forward_noalloc — moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and bitwise the same outputs. Its scratch is a fixed device array
 * of moe_forward_noalloc_max_bytes() bytes (64 MiB) that the library holds on
 * every device it runs on until the process ends; a problem whose
 * moe_forward_workspace_size exceeds it returns MOE_ETOOLARGE before anything
 * is enqueued (at the OLMoE layer shape, H = 2048, I = 1024, E = 64, K = 8,
 * that is n above about 1300 tokens). The call allocates nothing. Every call
 * on a device shares that one scratch array: calls that overlap on one
 * device (other streams, other threads) race and must be ordered by the
 * caller. Nothing in the scratch needs clearing between calls.
 * ------------------------------------------------------------------------- */
size_t moe_forward_noalloc_max_bytes(void);
moe_status moe_forward_noalloc(const void* x, const void* W_gate, const float* bias, const void* W13,
                               const void* W2, int n, int H, int I, int E, int K, int renorm, moe_dtype dt, void* y,
                               float* logits_out, int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_forward_persistent — moe_forward with GEMM1 + SwiGLU and GEMM2 in ONE
 * persistent kernel, scheduled as "大模型系统中的通算融合" §4.4 describes
 * DeepGEMM's Mega MoE scheduler (restated for one GPU): L1 tiles (GEMM1 +
 * SwiGLU) and L2 tiles (GEMM2) of each row tile are handed out from one task
 * queue per XCD, the L1 tiles of `warmup_row_tiles` row tiles first, then
 * alternating L1 tiles of later row tiles with L2 tiles of earlier ones; an
 * L2 tile starts once every L1 tile of its rows has published h (per-row-
 * tile counters with agent-scope release/acquire); h lives in a ring pool of
 * `pool_row_tiles` row-tile slots per queue (0: one buffer for all rows).
 * Outputs are bitwise equal to moe_forward's. bf16 only, and at most 2^24
 * tasks per queue (MOE_EUNSUPPORTED otherwise); warmup_row_tiles >= 1, and pool_row_tiles either 0 or larger
 * than warmup_row_tiles (MOE_EINVAL otherwise), so that every wait targets
 * a task handed out earlier and the schedule cannot deadlock. Each wait is
 * bounded nonetheless: if one runs out (a scheduling fault, never expected)
 * the kernel finishes with wrong outputs and sets the workspace's last int32
 * to nonzero instead of hanging.
 *
 *   arguments as moe_forward; ws at least
 *   moe_forward_persistent_workspace_size(n, H, I, E, K, pool_row_tiles)
 *   bytes (the last 4 bytes are the flag word above).
 * ------------------------------------------------------------------------- */
size_t moe_forward_persistent_workspace_size(int n, int H, int I, int E, int K, int pool_row_tiles);
moe_status moe_forward_persistent(const void* x, const void* W_gate, const float* bias, const void* W13,
                                  const void* W2, int n, int H, int I, int E, int K, int renorm, moe_dtype dt,
                                  int warmup_row_tiles, int pool_row_tiles, void* y, float* logits_out,
                                  int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* moe_forward_persistent_packed — moe_forward_persistent over weights packed
 * by moe_pack_w13 / moe_pack_w2 (bf16); the same workspace, schedule
 * arguments and results, bit for bit (and bit for bit moe_forward_packed's). */
moe_status moe_forward_persistent_packed(const void* x, const void* W_gate, const float* bias, const void* W13p,
                                         const void* W2p, int n, int H, int I, int E, int K, int renorm,
                                         int warmup_row_tiles, int pool_row_tiles, void* y, float* logits_out,
                                         int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, void* ws,
                                         size_t ws_bytes, hipStream_t stream);

/* ===========================================================================
 * Backward (training) pass of the same layer.
 *
 * The pages name the pieces of the training backward without formulas: the
 * backward of a dispatch is a combine, and the backward of a combine is a
 * dispatch that also yields the routing-score gradient ("大模型系统中的通算
 * 融合" §6.2.4; "0. goin" §2.3 (d), and its kernel table (e), which lists a
 * top-K gradient expansion and a routing-score gradient kernel). What is
 * computed is the gradient of the forward above for an upstream dy, with the
 * top-K selection held fixed:
 *
 *   dY_perm[inv[iK+k]] = w[i,k] dy[i];     dw[i,k] = <dy[i], Y_perm[inv[iK+k]]>
 *   dh = dY_e · W2[e]^T;                   dW2[e] = h_e^T · dY_e
 *   dgate = dh * up * s * (1 + gate * (1 - s)),  dup = dh * gate * s,
 *           s = 1 / (1 + e^-gate)
 *   dX_e = [dgate | dup] · W13[e]^T;       dW13[e] = X_e^T · [dgate | dup]
 *   dx[i] = sum_k dX_perm[inv[iK+k]] + dlogits[i] · W_gate^T
 *   ds = dw, or (dw - <dw, w>) / S with S = sum_k s under renormalisation;
 *   dp = ds at the selected experts, 0 elsewhere;
 *   dlogits = p * (dp - <p, dp>);  dW_gate = x^T · dlogits;  dbias = sum_i dlogits
 *
 * bf16: every product accumulates in fp32; gradients with the shape of a
 * bf16 tensor (dx, dY_perm, dgate_up, dX_perm, dW13, dW2) are rounded to bf16
 * once; the router gradients (dw, dlogits, dW_gate, dbias) stay fp32.
 * ========================================================================= */

/* ---------------------------------------------------------------------------
 * moe_expert_w13_swiglu_gather_train — moe_expert_w13_swiglu_gather that also
 * stores the pre-activations the backward needs.
 *   gate_up (n*K, 2I) dtype out: [gate | up] = X_e · W13[e] per row, rounded
 *           to dt (bf16: from the same fp32 accumulators as h).
 * Other arguments as moe_expert_w13_swiglu_gather.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_w13_swiglu_gather_train(const void* x, const int32_t* perm, int n, int K,
                                              const int32_t* offsets, const void* W13, int E, int H, int I,
                                              moe_dtype dt, void* h, void* gate_up, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_forward_train — moe_forward that keeps what the backward reads. Every
 * saved buffer is caller-owned and written:
 *   logits (n, E) fp32; topk_ids (n, K) int32; topk_w (n, K) fp32;
 *   offsets (E+1) int32; perm, inv (n*K) int32;
 *   gate_up (n*K, 2I) dtype; h (n*K, I) dtype; Y_perm (n*K, H) dtype.
 *   y (n, H) dtype out.
 *   ws  at least moe_forward_train_workspace_size(n, E, K) bytes (counts,
 *       splits and the permutation's block counts).
 * ------------------------------------------------------------------------- */
size_t moe_forward_train_workspace_size(int n, int E, int K);
moe_status moe_forward_train(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2,
                             int n, int H, int I, int E, int K, int renorm, moe_dtype dt, void* y, float* logits,
                             int32_t* topk_ids, float* topk_w, int32_t* offsets, int32_t* perm, int32_t* inv,
                             void* gate_up, void* h, void* Y_perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_combine_backward — gradient of moe_unpermute_combine (a dispatch of dy
 * plus the routing-score gradient):
 *   dY_perm[inv[i*K+k]] = w[i,k] * dy[i]      (n*K, H) dtype out
 *   dw[i,k] = <dy[i], Y_perm[inv[i*K+k]]>     (n, K) fp32 out, fp32 sums in a
 *                                             fixed order
 *   dy (n, H) dtype; Y_perm (n*K, H) dtype; inv (n*K) int32; topk_w (n, K) fp32.
 * ------------------------------------------------------------------------- */
moe_status moe_combine_backward(const void* dy, const void* Y_perm, const int32_t* inv, const float* topk_w, int n,
                                int H, int K, moe_dtype dt, void* dY_perm, float* dw, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_w2_backward — data gradient through GEMM2 and SwiGLU, per expert
 * segment of the expert-major rows:
 *   dh = dY_perm[p] · W2[e]^T, then
 *   dgate_up[p] = [dh * up * s * (1 + gate*(1 - s)) | dh * gate * s]
 * with [gate | up] = gate_up[p] (the saved pre-activations).
 *   dY_perm (rows, H), gate_up (rows, 2I), W2 (E, I, H) dtype;
 *   dgate_up (rows, 2I) dtype out.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_w2_backward(const void* dY_perm, const int32_t* offsets, int rows, const void* W2,
                                  const void* gate_up, int E, int H, int I, moe_dtype dt, void* dgate_up,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_w13_backward — data gradient through GEMM1:
 *   dX_perm[p] = dgate_up[p] · W13[e]^T     (rows, H) dtype out
 *   dgate_up (rows, 2I), W13 (E, H, 2I) dtype.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_w13_backward(const void* dgate_up, const int32_t* offsets, int rows, const void* W13, int E,
                                   int H, int I, moe_dtype dt, void* dX_perm, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_weight_grad — weight gradient of a grouped product
 * out_e = a_e · W[e], contracted over each expert's rows:
 *   dW[e] = a[offsets[e]:offsets[e+1]]^T · b[offsets[e]:offsets[e+1]]
 *   a (rows, M), b (rows, N) dtype; dW (E, M, N) dtype out. An expert with no
 *   rows gets zeros. dW2 is (a, b) = (h, dY_perm) with (M, N) = (I, H); dW13
 *   is (x_perm, dgate_up) with (H, 2I). M and N follow the rules for H.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_weight_grad(const void* a, const void* b, const int32_t* offsets, int rows, int E, int M, int N,
                                  moe_dtype dt, void* dW, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_weight_grad_gather — moe_expert_weight_grad with the rows of a
 * read through the permutation: row r of a_e is x[perm[r] / K], so dW13 is
 * formed straight from the token matrix without a permuted copy of it:
 *   dW[e] = sum over rows r of expert e of x[perm[r] / K]^T b[r]
 *   x (n, M) dtype; perm (n*K) int32 from moe_permute; b (n*K, N) dtype;
 *   dW (E, M, N) dtype out (zeros for an expert without rows).
 * It saves the (n*K, M) permuted copy of x; at the OLMoE shape it measured
 * slower than moe_permute's gather plus moe_expert_weight_grad (410 us
 * against 31 + 337 us), so moe_backward uses the latter.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_weight_grad_gather(const void* x, const int32_t* perm, int n, int K, const void* b,
                                         const int32_t* offsets, int E, int M, int N, moe_dtype dt, void* dW,
                                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_dispatch_backward — gradient of the row gather x_perm[p] = x[perm[p]/K]
 * (a combine with unit weights), plus an optional fp32 addend:
 *   dx[i] = add[i] + sum_{k=0..K-1} dX_perm[inv[i*K+k]]
 * summed in fp32 (add first, then slot order) and rounded once.
 *   dX_perm (n*K, H) dtype; inv (n*K) int32; add (n, H) fp32 or NULL;
 *   dx (n, H) dtype out.
 * ------------------------------------------------------------------------- */
moe_status moe_dispatch_backward(const void* dX_perm, const int32_t* inv, const float* add, int n, int H, int K,
                                 moe_dtype dt, void* dx, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_route_backward — gradient through routing (top-K weights, softmax and
 * the router product) given dw = dL/dtopk_w:
 *   dlogits (n, E) fp32 out (always);
 *   dx_router (n, H) fp32 out = dlogits · W_gate^T, or NULL to skip;
 *   dW_gate (H, E) fp32 out = x^T · dlogits, or NULL;
 *   dbias (E) fp32 out = sum_i dlogits[i], or NULL.
 *   x (n, H), W_gate (H, E) dtype (x unused when dW_gate and dbias are NULL;
 *   W_gate unused when dx_router is NULL; H is only checked when one of
 *   dx_router, dW_gate, dbias is wanted); logits (n, E) fp32 as written by
 *   moe_route; topk_ids, topk_w (n, K) as written by moe_route; dw (n, K) fp32.
 *   The softmax is recomputed from the logits in fp32. For bf16 with E a
 *   multiple of 32 the two router products run on MFMA with dlogits split
 *   into bf16 halves hi + lo (their sum is dlogits to about 2^-18 relative);
 *   otherwise with fp32 FMAs. dW_gate and dbias are sums of per-chunk partial
 *   sums taken in a fixed order.
 *   ws  moe_route_backward_workspace_size(n, H, E) bytes when any of
 *       dx_router, dW_gate, dbias is wanted (else unused and may be NULL).
 * ------------------------------------------------------------------------- */
size_t moe_route_backward_workspace_size(int n, int H, int E);
moe_status moe_route_backward(const void* x, const void* W_gate, const float* logits, const int32_t* topk_ids,
                              const float* topk_w, const float* dw, int n, int H, int E, int K, int renorm,
                              moe_dtype dt, float* dlogits, float* dx_router, float* dW_gate, float* dbias, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_backward — the whole layer's backward: combine backward, route
 * backward, GEMM2 + SwiGLU data gradient, dW2, GEMM1 data gradient, dispatch
 * backward (with the router's share of dx), row gather of x, dW13. The route
 * backward, dW2, the gather and dW13 run on a second HIP stream (one per
 * device, default priority, created on the first call and kept for the
 * process), forked from and joined back into `stream` with events, so that
 * they overlap the main chain; when that stream cannot be created everything
 * runs on `stream`. The second stream is shared by all calls on the device
 * (their enqueue sequences are serialised by a mutex, so backward calls on
 * different streams share its queue); while it belongs to a graph capture
 * other than `stream`'s (another thread's capture that forked into it and has
 * not ended), the call runs every branch on `stream` instead, in the same
 * order. All work is ordered after earlier work on `stream`, and later work
 * on `stream` sees every output. The call can be captured in a HIP graph (the
 * fork and join are events), except the first call on a device, which
 * creates the second stream.
 *   dy (n, H) dtype; x, W_gate, W13, W2 as given to moe_forward_train;
 *   logits ... Y_perm: the buffers moe_forward_train saved;
 *   dx (n, H) dtype out; dW_gate (H, E) fp32 out; dbias (E) fp32 out or NULL;
 *   dW13 (E, H, 2I), dW2 (E, I, H) dtype out.
 *   ws  at least moe_backward_workspace_size(...) bytes.
 * ------------------------------------------------------------------------- */
size_t moe_backward_workspace_size(int n, int H, int I, int E, int K, moe_dtype dt);
moe_status moe_backward(const void* dy, const void* x, const void* W_gate, const void* W13, const void* W2, int n,
                        int H, int I, int E, int K, int renorm, moe_dtype dt, const float* logits,
                        const int32_t* topk_ids, const float* topk_w, const int32_t* offsets, const int32_t* perm,
                        const int32_t* inv, const void* gate_up, const void* h, const void* Y_perm, void* dx,
                        float* dW_gate, float* dbias, void* dW13, void* dW2, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* ===========================================================================
 * FP8 expert weights.
 *
 * "大模型系统中的通算融合" §8.4 asks for low-precision payloads with per-token
 * or per-block scales that the GEMM consumes directly; §4.4 describes Mega
 * MoE's first linear with low-precision weights prepared ahead of time. Here
 * W13 and W2 are stored as OCP FP8 E4M3 codes (1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, largest finite 448) with one fp32
 * scale per output column; activations stay bf16 and the products accumulate
 * in fp32 on bf16 MFMA (E4M3 values are exact in bf16). The layer is
 * otherwise the one above; dt must be MOE_BF16 (else MOE_EUNSUPPORTED).
 * ========================================================================= */

/* ---------------------------------------------------------------------------
 * moe_quantize_fp8 — FP8 codes and column scales of a stack of weights
 * W (E, Kd, N) row-major (W13: Kd = H, N = 2I; W2: Kd = I, N = H):
 *   scales[e, n] = max_k |W[e, k, n]| / 448 (fp32; 1 for an all-zero column);
 *   codes[e, n, k] = nearest E4M3 value of the fp32 quotient W[e, k, n] /
 *                    scales[e, n], ties to the even mantissa, magnitudes
 *                    beyond 448 saturated to 448.
 * codes are column-major per expert: each output column's Kd codes are
 * contiguous (the layout the GEMMs read). Kd must be a multiple of 64, N of 4.
 *   W dtype (bf16 or fp32); codes (E, N, Kd) uint8 out; scales (E, N) fp32 out.
 * ------------------------------------------------------------------------- */
moe_status moe_quantize_fp8(const void* W, int E, int Kd, int N, moe_dtype dt, uint8_t* codes, float* scales,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_w13_swiglu_gather_fp8 — moe_expert_w13_swiglu_gather with FP8
 * W13: gate_up[r] = (x[perm[r]/K] · W13'[e]) where W13'[e][k, n] =
 * decode(W13q[e, n, k]) * s13[e, n], accumulated in fp32, the column scale
 * applied to the accumulator, then h = SiLU(gate) * up rounded to bf16.
 *   W13q (E, 2I, H) uint8; s13 (E, 2I) fp32; other arguments as the bf16 call.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_w13_swiglu_gather_fp8(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                            const uint8_t* W13q, const float* s13, int E, int H, int I, moe_dtype dt,
                                            void* h, hipStream_t stream);

/* moe_expert_w13_swiglu_from_ids_fp8 — moe_expert_w13_swiglu_gather_fp8 for a
 * decode-sized batch straight from the routing ids, as
 * moe_expert_w13_swiglu_from_ids does it for bf16 weights: the GEMM places the
 * pairs itself and also writes counts, offsets, splits, perm and inv
 * (moe_permute's values). x (n, H) bf16; topk_ids (n, K) int32 with K distinct
 * experts per token; ep as moe_permute. Shapes it serves: n <= 32,
 * n*K <= 1024, E <= 256, else MOE_EUNSUPPORTED; n == 0 writes zero counts,
 * offsets and splits. */
moe_status moe_expert_w13_swiglu_from_ids_fp8(const void* x, const int32_t* topk_ids, int n, int K,
                                              const uint8_t* W13q, const float* s13, int E, int H, int I, int ep,
                                              void* h, int32_t* counts, int32_t* offsets, int32_t* splits,
                                              int32_t* perm, int32_t* inv, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_w2_fp8 — moe_expert_w2 with FP8 W2: Y_perm[p] = h[p] · W2'[e],
 * W2'[e][k, n] = decode(W2q[e, n, k]) * s2[e, n].
 *   W2q (E, H, I) uint8; s2 (E, H) fp32.
 * ------------------------------------------------------------------------- */
moe_status moe_expert_w2_fp8(const void* h, const int32_t* offsets, int rows, const uint8_t* W2q, const float* s2,
                             int E, int H, int I, moe_dtype dt, void* Y_perm, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_forward_fp8 — moe_forward with FP8 expert weights (route, permute
 * metadata, FP8 GEMM1 with the gather fused, FP8 GEMM2, combine; at n <= 32
 * moe_expert_w13_swiglu_from_ids_fp8 in place of the first two). Workspace:
 * moe_forward_workspace_size(n, H, I, E, K, MOE_BF16) bytes.
 * ------------------------------------------------------------------------- */
moe_status moe_forward_fp8(const void* x, const void* W_gate, const float* bias, const uint8_t* W13q,
                           const float* s13, const uint8_t* W2q, const float* s2, int n, int H, int I, int E, int K,
                           int renorm, moe_dtype dt, void* y, float* logits_out, int32_t* topk_ids_out,
                           float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * FP8 activations. "大模型系统中的通算融合" §8.4 lists MoE dispatch with FP8
 * data and a per-token scale, the receive buffer feeding the FP8 GEMM directly;
 * "0. goin" §2.1 pads each expert's group of rows to a multiple of 16 for FP8.
 *
 * moe_quantize_rows_fp8 — per-token FP8: scales[i] = max_h |x[i,h]| / 448 in
 * fp32 (1 for a zero row), codes[i,h] = the nearest OCP E4M3 code of the fp32
 * quotient x[i,h] / scales[i] (ties to even, saturating at 448).
 *   x (n, H) dtype; codes (n, H) uint8 out; scales (n) fp32 out; H a multiple
 *   of 8.
 *
 * moe_fp8_padded_rows — rows of the padded receive buffer for n tokens, top-K:
 * n*K + 15 * min(E, n*K) (each expert that receives rows pads fewer than 16).
 *
 * moe_dispatch_fp8 — the padded FP8 receive buffer from moe_permute's counts,
 * offsets and perm (ep = 1) and the per-token codes/scales: expert e's rows,
 * in moe_permute's order, start at offsets_padded[e] = sum over e' < e of
 * 16 * ceil(counts[e'] / 16); a token's K copies share its codes and scale;
 * padding rows hold code 0, scale 0 and perm_padded -1. Rows past
 * offsets_padded[E] are not written.
 *   counts (E), offsets (E+1), perm (n*K) int32 from moe_permute;
 *   codes_tok (n, H) uint8 and s_tok (n) fp32 from moe_quantize_rows_fp8;
 *   offsets_padded (E+1) int32 out; x_q (rows, H) uint8 out and x_scale (rows)
 *   fp32 out with rows = moe_fp8_padded_rows(n, E, K); perm_padded (rows)
 *   int32 out: the flat pair index i*K+k of each row or -1; inv_padded (n*K)
 *   int32 out: the buffer row of each pair. H a multiple of 16.
 *
 * moe_expert_w13_swiglu_fp8a — Algorithm 2 step 8 on the receive buffer:
 * h[r] = SiLU(g) * u with [g | u] = (x_scale[r] * decode(x_q[r])) .
 * (s13 * decode(W13q)) over expert e's columns, on the gfx950 FP8 MFMA with
 * fp32 accumulation; h (rows_max, I) bf16 out (padding rows give 0; rows past
 * offsets_padded[E] are not written). W13q (E, 2I, H) and s13 (E, 2I) as from
 * moe_quantize_fp8 on W13; rows_max = moe_fp8_padded_rows(n, E, K) (an upper
 * bound; the tile map comes from offsets_padded). H a multiple of 128.
 *
 * moe_expert_w2_fp8a — GEMM2 with FP8 activations: Y_perm row r (bf16) =
 * (h_scale[r] * decode(h_q[r])) . (s2 * decode(W2q)) over the expert of row r
 * (offsets_padded), on the FP8 MFMA with fp32 accumulation. h_q (rows_max, I)
 * uint8 and h_scale (rows_max) fp32 are h quantized per row as
 * moe_quantize_rows_fp8 does it ("大模型系统中的通算融合" §8.4 lists FP8
 * activations among the low-precision forms); W2q (E, H, I) and s2 (E, H) as
 * from moe_quantize_fp8 on W2; Y_perm (rows_max, H) bf16 out (rows past
 * offsets_padded[E] not written). I a multiple of 128.
 *
 * moe_expert_w13_swiglu_gather_fp8a — moe_expert_w13_swiglu_fp8a with the
 * activations read in place instead of from a receive buffer: row r of the
 * expert-major order (offsets, unpadded) is token perm[r] / K of codes_tok
 * (n, H) uint8 with scale s_tok[perm[r] / K] (moe_quantize_rows_fp8 of x);
 * perm as from moe_permute; h (n*K, I) bf16 out. H a multiple of 128.
 *
 * moe_expert_w13_swiglu_from_ids_fp8a — moe_expert_w13_swiglu_gather_fp8a for
 * a decode-sized batch straight from the routing ids, as
 * moe_expert_w13_swiglu_from_ids does it for bf16: the GEMM places the pairs
 * itself and also writes counts, offsets, splits, perm and inv (moe_permute's
 * values). topk_ids (n, K) int32 with K distinct experts per token; ep as
 * moe_permute. Shapes it serves: n <= 32, n*K <= 1024, E <= 256, else
 * MOE_EUNSUPPORTED; n == 0 writes zero counts, offsets and splits.
 *
 * moe_forward_fp8a — the layer with FP8 activations and FP8 weights: moe_route
 * on x (bf16), the moe_permute metadata, moe_quantize_rows_fp8 of x,
 * moe_expert_w13_swiglu_gather_fp8a (at n <= 32:
 * moe_expert_w13_swiglu_from_ids_fp8a in place of both), moe_quantize_rows_fp8 of h,
 * moe_expert_w2_fp8a and moe_unpermute_combine. On one GPU the per-token FP8
 * rows are read in place through perm, as moe_forward reads x; the padded
 * receive buffer of moe_dispatch_fp8 is the form an expert-parallel exchange
 * delivers, which moe_expert_w13_swiglu_fp8a and moe_expert_w2_fp8a take as
 * well. Arguments as moe_forward_fp8 (dt must be MOE_BF16, H and I multiples
 * of 128); ws of at least moe_forward_fp8a_workspace_size(n, H, I, E, K)
 * bytes.
 * ------------------------------------------------------------------------- */
moe_status moe_quantize_rows_fp8(const void* x, int n, int H, moe_dtype dt, uint8_t* codes, float* scales,
                                 hipStream_t stream);
size_t moe_fp8_padded_rows(int n, int E, int K);
moe_status moe_dispatch_fp8(const int32_t* counts, const int32_t* offsets, const int32_t* perm, int n, int E, int K,
                            const uint8_t* codes_tok, const float* s_tok, int H, int32_t* offsets_padded,
                            uint8_t* x_q, float* x_scale, int32_t* perm_padded, int32_t* inv_padded,
                            hipStream_t stream);
moe_status moe_expert_w13_swiglu_fp8a(const uint8_t* x_q, const float* x_scale, const int32_t* offsets_padded,
                                      int rows_max, const uint8_t* W13q, const float* s13, int E, int H, int I,
                                      void* h, hipStream_t stream);
moe_status moe_expert_w13_swiglu_gather_fp8a(const uint8_t* codes_tok, const float* s_tok, const int32_t* perm,
                                             int n, int K, const int32_t* offsets, const uint8_t* W13q,
                                             const float* s13, int E, int H, int I, void* h, hipStream_t stream);
moe_status moe_expert_w13_swiglu_from_ids_fp8a(const uint8_t* codes_tok, const float* s_tok,
                                               const int32_t* topk_ids, int n, int K, const uint8_t* W13q,
                                               const float* s13, int E, int H, int I, int ep, void* h,
                                               int32_t* counts, int32_t* offsets, int32_t* splits, int32_t* perm,
                                               int32_t* inv, hipStream_t stream);
moe_status moe_expert_w2_fp8a(const uint8_t* h_q, const float* h_scale, const int32_t* offsets_padded, int rows_max,
                              const uint8_t* W2q, const float* s2, int E, int H, int I, void* Y_perm,
                              hipStream_t stream);
size_t moe_forward_fp8a_workspace_size(int n, int H, int I, int E, int K);
moe_status moe_forward_fp8a(const void* x, const void* W_gate, const float* bias, const uint8_t* W13q,
                            const float* s13, const uint8_t* W2q, const float* s2, int n, int H, int I, int E, int K,
                            int renorm, moe_dtype dt, void* y, float* logits_out, int32_t* topk_ids_out,
                            float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* MOE_H_ */
