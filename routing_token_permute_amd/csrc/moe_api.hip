// C ABI of the MoE expert layer (forward and backward): argument checks,
// workspace layouts and the order in which the kernels are enqueued.
// Everything numeric runs in the kernels of route.hip, permute.hip,
// grouped_gemm.hip, combine.hip, grouped_gemm_bwd.hip and backward.hip.
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "moe_internal.hpp"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t elt_size(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }

bool dtype_ok(moe_dtype dt) { return dt == MOE_BF16 || dt == MOE_F32; }

// Shape rules the kernels rely on: bf16 GEMMs and the router advance K in
// steps of 64; every row copy moves 16-byte vectors. The GEMM epilogues
// address a tile's outputs with 32-bit byte offsets (at most 256 rows of up
// to 2 * kMaxHidden bf16 values), so hidden sizes are bounded.
constexpr int kMaxHidden = 1 << 20;
bool hidden_ok(int H, moe_dtype dt) {
  return H > 0 && H <= kMaxHidden && (dt == MOE_BF16 ? H % 64 == 0 : H % 4 == 0);
}

bool experts_ok(int E, int K) { return E >= 1 && E <= kMaxExperts && K >= 1 && K <= E && K <= kMaxTopK; }

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Pointer alignment the kernels rely on: row matrices, weights, workspaces
// and fp32 row buffers are moved with 16-byte vector loads, 16-byte LDS DMA
// and 16-byte buffer stores; per-pair int32/fp32 arrays with 4-byte accesses.
// A null pointer passes (optional arguments are checked for presence apart).
bool aligned(std::initializer_list<const void*> ps, uintptr_t a) {
  for (const void* p : ps)
    if (((uintptr_t)p & (a - 1)) != 0) return false;
  return true;
}
bool vec_ok(std::initializer_list<const void*> ps) { return aligned(ps, 16); }
bool word_ok(std::initializer_list<const void*> ps) { return aligned(ps, 4); }

size_t permute_ws(int n, int E, int K) {
  (void)n;
  (void)K;
  return align_up((size_t)kPermMaxBlocks * E * sizeof(int32_t));
}

// moe_forward workspace, in order.
struct ForwardLayout {
  size_t logits, ids, w, counts, offsets, splits, perm, inv, pscratch, h, Y_perm, total;
};

ForwardLayout forward_layout(int n, int H, int I, int E, int K, moe_dtype dt) {
  ForwardLayout L{};
  const size_t nk = (size_t)n * K;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes > 0 ? bytes : 1);
    return at;
  };
  L.logits = take((size_t)n * E * 4);
  L.ids = take(nk * 4);
  L.w = take(nk * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.splits = take(4);
  L.perm = take(nk * 4);
  L.inv = take(nk * 4);
  L.pscratch = take(permute_ws(n, E, K));
  L.h = take(nk * I * elt_size(dt));
  L.Y_perm = take(nk * H * elt_size(dt));
  L.total = o;
  return L;
}

// moe_forward_fp8a workspace, in order: routing, dispatch metadata, the
// per-token FP8 rows, h and its per-row FP8 form, and Y_perm (nK rows each).
struct Fp8aLayout {
  size_t logits, ids, w, counts, offsets, splits, perm, inv, pscratch, codes_tok, s_tok, h, h_q, h_scale, Y_perm,
      total;
};
Fp8aLayout fp8a_layout(int n, int H, int I, int E, int K) {
  Fp8aLayout L{};
  const size_t nk = (size_t)n * K;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes > 0 ? bytes : 1);
    return at;
  };
  L.logits = take((size_t)n * E * 4);
  L.ids = take(nk * 4);
  L.w = take(nk * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.splits = take(4);
  L.perm = take(nk * 4);
  L.inv = take(nk * 4);
  L.pscratch = take(permute_ws(n, E, K));
  L.codes_tok = take((size_t)n * H);
  L.s_tok = take((size_t)n * 4);
  L.h = take(nk * I * 2);
  L.h_q = take(nk * I);
  L.h_scale = take(nk * 4);
  L.Y_perm = take(nk * H * 2);
  L.total = o;
  return L;
}

// moe_forward_train workspace: what the forward uses but does not save.
struct TrainLayout {
  size_t counts, splits, pscratch, total;
};

TrainLayout train_layout(int n, int E, int K) {
  TrainLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes > 0 ? bytes : 1);
    return at;
  };
  L.counts = take((size_t)E * 4);
  L.splits = take(4);
  L.pscratch = take(permute_ws(n, E, K));
  L.total = o;
  return L;
}

size_t route_bwd_ws(int n, int H, int E) { return align_up(route_bwd_workspace(n, H, E)); }

// moe_backward workspace, in order. rows_a holds dY_perm, then dX_perm (dY_perm
// is dead once dgate_up and dW2 are done); rows_b the gathered x_perm. (dW13
// straight from x through perm, moe_expert_weight_grad_gather, needs no
// rows_b but measured slower than the gather plus the plain weight gradient.)
struct BackwardLayout {
  size_t rows_a, rows_b, dgu, dw, dlogits, dx_router, rws, total;
};

BackwardLayout backward_layout(int n, int H, int I, int E, int K, moe_dtype dt) {
  BackwardLayout L{};
  const size_t nk = (size_t)n * K;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes > 0 ? bytes : 1);
    return at;
  };
  L.rows_a = take(nk * H * elt_size(dt));
  L.rows_b = take(nk * H * elt_size(dt));
  L.dgu = take(nk * 2 * I * elt_size(dt));
  L.dw = take(nk * 4);
  L.dlogits = take((size_t)n * E * 4);
  L.dx_router = take((size_t)n * H * 4);
  L.rws = take(route_bwd_ws(n, H, E));
  L.total = o;
  return L;
}

// A second stream per device for the backward's independent branches, with
// its fork/join events; created on first use and kept for the process. The
// mutex keeps each call's record/wait sequence in one piece when several host
// threads enqueue at once.
struct AuxStream {
  hipStream_t s = nullptr;
  hipEvent_t ev[4] = {};
  bool ok = false;
  bool tried = false;
};

std::mutex g_aux_mutex;

AuxStream* aux_stream() {
  constexpr int kMaxDevices = 64;
  static AuxStream aux[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  AuxStream& a = aux[dev];
  if (!a.tried) {
    a.tried = true;
    bool ok = hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; i < 4 && ok; ++i) ok = hipEventCreateWithFlags(&a.ev[i], hipEventDisableTiming) == hipSuccess;
    a.ok = ok;
    if (!ok) (void)hipGetLastError();
  }
  return a.ok ? &a : nullptr;
}

// Argument checks of the layer call (everything
// but the workspace).
moe_status check_forward(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2,
                         int n, int H, int I, int E, int K, moe_dtype dt, const void* y, const float* logits_out,
                         const int32_t* topk_ids_out, const float* topk_w_out, const int32_t* counts_out) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || !experts_ok(E, K) || !hidden_ok(H, dt) || !hidden_ok(I, dt)) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (n > 0 && (x == nullptr || W_gate == nullptr || W13 == nullptr || W2 == nullptr || y == nullptr))
    return MOE_EINVAL;
  if (!vec_ok({x, W_gate, W13, W2, y}) || !word_ok({bias, logits_out, topk_ids_out, topk_w_out, counts_out}))
    return MOE_EINVAL;
  return MOE_OK;
}

// The layer's launches over a workspace laid out by forward_layout at `base`
// (n > 0, arguments checked).
// g1_begin / g1_end: optional events recorded right before and after GEMM1.
moe_status forward_enqueue(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2,
                           int n, int H, int I, int E, int K, int renorm, moe_dtype dt, void* y, float* logits_out,
                           int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, char* base,
                           hipStream_t stream, hipEvent_t g1_begin = nullptr, hipEvent_t g1_end = nullptr,
                           bool packed = false) {
  const ForwardLayout L = forward_layout(n, H, I, E, K, dt);
  float* logits = logits_out ? logits_out : (float*)(base + L.logits);
  int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(base + L.ids);
  float* w = topk_w_out ? topk_w_out : (float*)(base + L.w);
  int32_t* counts = counts_out ? counts_out : (int32_t*)(base + L.counts);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* splits = (int32_t*)(base + L.splits);
  int32_t* perm = (int32_t*)(base + L.perm);
  int32_t* inv = (int32_t*)(base + L.inv);

  hipError_t e = launch_route(x, W_gate, bias, n, H, E, K, renorm, dt, logits, ids, w, stream);
  if (e != hipSuccess) return MOE_EHIP;
  if (w13_from_ids_ok(n, K, E, dt)) {
    // Decode-sized batch: GEMM1 places the pairs itself and writes the
    // metadata for GEMM2 and the combine (one launch fewer).
    if (g1_begin != nullptr && hipEventRecord(g1_begin, stream) != hipSuccess) return MOE_EHIP;
    e = launch_w13_swiglu_from_ids(x, ids, n, K, W13, E, H, I, 1, base + L.h, counts, offsets, splits, perm, inv,
                                   stream, packed);
  } else {
    // Metadata only: GEMM1 gathers the token rows itself through perm.
    e = launch_permute(ids, nullptr, n, H, E, K, 1, dt, counts, offsets, splits, perm, inv, nullptr,
                       (int32_t*)(base + L.pscratch), stream);
    if (e != hipSuccess) return MOE_EHIP;
    if (g1_begin != nullptr && hipEventRecord(g1_begin, stream) != hipSuccess) return MOE_EHIP;
    e = launch_w13_swiglu_gather(x, perm, n, K, offsets, W13, E, H, I, dt, base + L.h, stream, packed);
  }
  if (e != hipSuccess) return MOE_EHIP;
  if (g1_end != nullptr && hipEventRecord(g1_end, stream) != hipSuccess) return MOE_EHIP;
  // Expert-major GEMM2, then the gathered weighted combine: measured a little
  // faster here than moe_expert_w2_scatter + moe_sum_slots, whose scattered
  // row stores cost GEMM2 more than the contiguous sum saves.
  e = launch_w2(base + L.h, offsets, n * K, W2, E, H, I, dt, base + L.Y_perm, stream, packed);
  if (e != hipSuccess) return MOE_EHIP;
  return from_hip(launch_combine(base + L.Y_perm, inv, w, n, H, K, dt, y, stream));
}

// moe_forward_persistent workspace: routing and metadata as in
// forward_layout, h (ring pool or all rows), Y_perm, and the scheduler's
// counters last, so that its flag word is the workspace's last int32.
struct PersistentLayout {
  size_t logits, ids, w, counts, offsets, splits, perm, inv, pscratch, h, Y_perm, counters, total;
};
PersistentLayout persistent_layout(int n, int H, int I, int E, int K, int pool) {
  PersistentLayout L{};
  const size_t nk = (size_t)n * K;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes > 0 ? bytes : 1);
    return at;
  };
  L.logits = take((size_t)n * E * 4);
  L.ids = take(nk * 4);
  L.w = take(nk * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.splits = take(4);
  L.perm = take(nk * 4);
  L.inv = take(nk * 4);
  L.pscratch = take(permute_ws(n, E, K));
  L.h = take(fused_ffn_h_bytes((int)nk, E, I, pool));
  L.Y_perm = take(nk * H * 2);
  L.counters = o;
  L.total = o + fused_ffn_counter_bytes((int)nk, E);
  return L;
}

// Scratch of moe_forward_noalloc: the workspace of moe_forward, in a static
// device array that every device the library runs on holds from the first
// call to the end of the process. Every call on a device shares it (calls
// that overlap on one device race); no part needs to start at zero, since
// every region is written by the call before it is read.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; the array's name itself is a
// host-side stand-in that must never reach a kernel.
char* scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static char* ptrs[kMaxDevices] = {};
  static std::once_flag once[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr)
      ptrs[dev] = (char*)p;
    else
      (void)hipGetLastError();
  });
  return ptrs[dev];
}

// Capture state of a stream: 0 when it is not being captured, else the id of
// the capture it belongs to; ~0 when the query fails (treated as busy).
unsigned long long capture_id(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  unsigned long long id = 0;
  if (hipStreamGetCaptureInfo(s, &st, &id) != hipSuccess) {
    (void)hipGetLastError();
    return ~0ull;
  }
  return st == hipStreamCaptureStatusNone ? 0ull : (id == 0 ? ~1ull : id);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK:
      return "MOE_OK: success";
    case MOE_EINVAL:
      return "MOE_EINVAL: invalid argument (null pointer, size or shape outside the supported range)";
    case MOE_EUNSUPPORTED:
      return "MOE_EUNSUPPORTED: dtype not built";
    case MOE_EWORKSPACE:
      return "MOE_EWORKSPACE: workspace missing or smaller than required";
    case MOE_EHIP:
      return "MOE_EHIP: a HIP kernel launch failed";
    case MOE_ETOOLARGE:
      return "MOE_ETOOLARGE: the problem needs more scratch than moe_forward_noalloc holds "
             "(moe_forward_noalloc_max_bytes); use moe_forward with a workspace";
  }
  return "unknown moe_status";
}

int moe_version(void) { return 100; }

moe_status moe_device_info(int* compute_units, int* sclk_khz, int* mem_clk_khz, int* mem_bus_bits) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  const struct {
    int* out;
    hipDeviceAttribute_t attr;
  } q[] = {{compute_units, hipDeviceAttributeMultiprocessorCount},
           {sclk_khz, hipDeviceAttributeClockRate},
           {mem_clk_khz, hipDeviceAttributeMemoryClockRate},
           {mem_bus_bits, hipDeviceAttributeMemoryBusWidth}};
  for (const auto& e : q)
    if (e.out != nullptr && hipDeviceGetAttribute(e.out, e.attr, dev) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

moe_status moe_route(const void* x, const void* W_gate, const float* bias, int n, int H, int E, int K, int renorm,
                     moe_dtype dt, float* logits, int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || !experts_ok(E, K)) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  if (logits == nullptr || topk_ids == nullptr || topk_w == nullptr) return MOE_EINVAL;
  if (x != nullptr && (W_gate == nullptr || !hidden_ok(H, dt))) return MOE_EINVAL;
  if (!vec_ok({x, W_gate}) || !word_ok({bias, logits, topk_ids, topk_w})) return MOE_EINVAL;
  return from_hip(launch_route(x, W_gate, bias, n, H, E, K, renorm, dt, logits, topk_ids, topk_w, stream));
}

size_t moe_permute_workspace_size(int n, int E, int K) {
  if (n < 0 || E < 1 || K < 1) return 0;
  return permute_ws(n, E, K);
}

moe_status moe_permute(const int32_t* topk_ids, const void* x, int n, int H, int E, int K, int ep, moe_dtype dt,
                       int32_t* counts, int32_t* offsets, int32_t* splits, int32_t* perm, int32_t* inv,
                       void* x_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || !experts_ok(E, K) || ep < 1 || E % ep != 0) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (counts == nullptr || offsets == nullptr || splits == nullptr) return MOE_EINVAL;
  if (n > 0 && (topk_ids == nullptr || perm == nullptr || inv == nullptr)) return MOE_EINVAL;
  if (x != nullptr && (x_perm == nullptr || !hidden_ok(H, dt))) return MOE_EINVAL;
  if (ws == nullptr || ws_bytes < permute_ws(n, E, K)) return MOE_EWORKSPACE;
  if (!vec_ok({x, x_perm, ws}) || !word_ok({topk_ids, counts, offsets, splits, perm, inv})) return MOE_EINVAL;
  return from_hip(launch_permute(topk_ids, x, n, H, E, K, ep, dt, counts, offsets, splits, perm, inv, x_perm,
                                 (int32_t*)ws, stream));
}

size_t moe_grouped_swiglu_workspace_size(int rows, int I, moe_dtype dt) {
  if (rows < 0 || I < 1 || !dtype_ok(dt)) return 0;
  return align_up((size_t)rows * I * elt_size(dt));
}

moe_status moe_grouped_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13, const void* W2,
                              int E, int H, int I, moe_dtype dt, void* Y_perm, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (rows < 0 || E < 1 || E > kMaxExperts || !hidden_ok(H, dt) || !hidden_ok(I, dt)) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  if (x_perm == nullptr || offsets == nullptr || W13 == nullptr || W2 == nullptr || Y_perm == nullptr)
    return MOE_EINVAL;
  if (ws == nullptr || ws_bytes < (size_t)rows * I * elt_size(dt)) return MOE_EWORKSPACE;
  if (!vec_ok({x_perm, W13, W2, Y_perm, ws}) || !word_ok({offsets})) return MOE_EINVAL;
  return from_hip(launch_grouped_swiglu(x_perm, offsets, rows, W13, W2, E, H, I, dt, Y_perm, ws, stream));
}

static moe_status check_expert_gemm(const void* a, const int32_t* offsets, int rows, const void* w, int E, int H,
                                    int I, moe_dtype dt, const void* out) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (rows < 0 || E < 1 || E > kMaxExperts || !hidden_ok(H, dt) || !hidden_ok(I, dt)) return MOE_EINVAL;
  if (rows > 0 && (a == nullptr || offsets == nullptr || w == nullptr || out == nullptr)) return MOE_EINVAL;
  if (!vec_ok({a, w, out}) || !word_ok({offsets})) return MOE_EINVAL;
  return MOE_OK;
}

moe_status moe_expert_w13_swiglu(const void* x_perm, const int32_t* offsets, int rows, const void* W13, int E, int H,
                                 int I, moe_dtype dt, void* h, hipStream_t stream) {
  const moe_status st = check_expert_gemm(x_perm, offsets, rows, W13, E, H, I, dt, h);
  if (st != MOE_OK) return st;
  return from_hip(launch_w13_swiglu(x_perm, offsets, rows, W13, E, H, I, dt, h, stream));
}

namespace {
moe_status w13_gather_call(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                           const void* W13, int E, int H, int I, moe_dtype dt, void* h, hipStream_t stream,
                           bool packed) {
  if (n < 0 || K < 1 || K > kMaxTopK || (long long)n * K > INT32_MAX) return MOE_EINVAL;
  if ((n > 0 && perm == nullptr) || !word_ok({perm})) return MOE_EINVAL;
  const moe_status st = check_expert_gemm(x, offsets, n * K, W13, E, H, I, dt, h);
  if (st != MOE_OK) return st;
  return from_hip(launch_w13_swiglu_gather(x, perm, n, K, offsets, W13, E, H, I, dt, h, stream, packed));
}

moe_status w13_from_ids_call(const void* x, const int32_t* topk_ids, int n, int K, const void* W13, int E, int H,
                             int I, int ep, moe_dtype dt, void* h, int32_t* counts, int32_t* offsets,
                             int32_t* splits, int32_t* perm, int32_t* inv, hipStream_t stream, bool packed) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || !experts_ok(E, K) || ep < 1 || E % ep != 0 || !hidden_ok(H, dt) || !hidden_ok(I, dt))
    return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (counts == nullptr || offsets == nullptr || splits == nullptr) return MOE_EINVAL;
  if (!word_ok({topk_ids, counts, offsets, splits, perm, inv})) return MOE_EINVAL;
  if (n == 0)
    return from_hip(launch_permute(nullptr, nullptr, 0, H, E, K, ep, dt, counts, offsets, splits, nullptr, nullptr,
                                   nullptr, nullptr, stream));
  if (!w13_from_ids_ok(n, K, E, dt)) return MOE_EUNSUPPORTED;
  if (x == nullptr || topk_ids == nullptr || W13 == nullptr || h == nullptr || perm == nullptr || inv == nullptr)
    return MOE_EINVAL;
  if (!vec_ok({x, W13, h})) return MOE_EINVAL;
  return from_hip(launch_w13_swiglu_from_ids(x, topk_ids, n, K, W13, E, H, I, ep, h, counts, offsets, splits, perm,
                                             inv, stream, packed));
}
}  // namespace

moe_status moe_expert_w13_swiglu_gather(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                        const void* W13, int E, int H, int I, moe_dtype dt, void* h,
                                        hipStream_t stream) {
  return w13_gather_call(x, perm, n, K, offsets, W13, E, H, I, dt, h, stream, false);
}

moe_status moe_expert_w13_swiglu_gather_packed(const void* x, const int32_t* perm, int n, int K,
                                               const int32_t* offsets, const void* W13p, int E, int H, int I,
                                               void* h, hipStream_t stream) {
  return w13_gather_call(x, perm, n, K, offsets, W13p, E, H, I, MOE_BF16, h, stream, true);
}

moe_status moe_expert_w13_swiglu_from_ids(const void* x, const int32_t* topk_ids, int n, int K, const void* W13,
                                          int E, int H, int I, int ep, moe_dtype dt, void* h, int32_t* counts,
                                          int32_t* offsets, int32_t* splits, int32_t* perm, int32_t* inv,
                                          hipStream_t stream) {
  return w13_from_ids_call(x, topk_ids, n, K, W13, E, H, I, ep, dt, h, counts, offsets, splits, perm, inv, stream,
                           false);
}

moe_status moe_expert_w13_swiglu_from_ids_packed(const void* x, const int32_t* topk_ids, int n, int K,
                                                 const void* W13p, int E, int H, int I, int ep, void* h,
                                                 int32_t* counts, int32_t* offsets, int32_t* splits, int32_t* perm,
                                                 int32_t* inv, hipStream_t stream) {
  return w13_from_ids_call(x, topk_ids, n, K, W13p, E, H, I, ep, MOE_BF16, h, counts, offsets, splits, perm, inv,
                           stream, true);
}

moe_status moe_expert_w2(const void* h, const int32_t* offsets, int rows, const void* W2, int E, int H, int I,
                         moe_dtype dt, void* Y_perm, hipStream_t stream) {
  const moe_status st = check_expert_gemm(h, offsets, rows, W2, E, H, I, dt, Y_perm);
  if (st != MOE_OK) return st;
  return from_hip(launch_w2(h, offsets, rows, W2, E, H, I, dt, Y_perm, stream));
}

moe_status moe_expert_w2_packed(const void* h, const int32_t* offsets, int rows, const void* W2p, int E, int H,
                                int I, void* Y_perm, hipStream_t stream) {
  const moe_status st = check_expert_gemm(h, offsets, rows, W2p, E, H, I, MOE_BF16, Y_perm);
  if (st != MOE_OK) return st;
  return from_hip(launch_w2(h, offsets, rows, W2p, E, H, I, MOE_BF16, Y_perm, stream, true));
}

moe_status moe_expert_w2_scatter(const void* h, const int32_t* offsets, int rows, const int32_t* perm,
                                 const float* topk_w, const void* W2, int E, int H, int I, moe_dtype dt,
                                 void* Y_tok, hipStream_t stream) {
  const moe_status st = check_expert_gemm(h, offsets, rows, W2, E, H, I, dt, Y_tok);
  if (st != MOE_OK) return st;
  if (rows > 0 && (perm == nullptr || topk_w == nullptr)) return MOE_EINVAL;
  if (!word_ok({perm, topk_w})) return MOE_EINVAL;
  return from_hip(launch_w2_scatter(h, offsets, rows, perm, topk_w, W2, E, H, I, dt, Y_tok, stream));
}

moe_status moe_expert_w2_scatter_packed(const void* h, const int32_t* offsets, int rows, const int32_t* perm,
                                        const float* topk_w, const void* W2p, int E, int H, int I, void* Y_tok,
                                        hipStream_t stream) {
  const moe_status st = check_expert_gemm(h, offsets, rows, W2p, E, H, I, MOE_BF16, Y_tok);
  if (st != MOE_OK) return st;
  if (rows > 0 && (perm == nullptr || topk_w == nullptr)) return MOE_EINVAL;
  if (!word_ok({perm, topk_w})) return MOE_EINVAL;
  return from_hip(launch_w2_scatter(h, offsets, rows, perm, topk_w, W2p, E, H, I, MOE_BF16, Y_tok, stream, true));
}

moe_status moe_sum_slots(const void* Y_tok, int n, int H, int K, moe_dtype dt, void* y, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || K < 1 || K > kMaxTopK || !hidden_ok(H, dt)) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  if (Y_tok == nullptr || y == nullptr || !vec_ok({Y_tok, y})) return MOE_EINVAL;
  return from_hip(launch_sum_slots(Y_tok, n, H, K, dt, y, stream));
}

moe_status moe_unpermute_combine(const void* Y_perm, const int32_t* inv, const float* topk_w, int n, int H, int K,
                                 moe_dtype dt, void* y, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || K < 1 || K > kMaxTopK || !hidden_ok(H, dt)) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  if (Y_perm == nullptr || inv == nullptr || y == nullptr) return MOE_EINVAL;
  if (!vec_ok({Y_perm, y}) || !word_ok({inv, topk_w})) return MOE_EINVAL;
  return from_hip(launch_combine(Y_perm, inv, topk_w, n, H, K, dt, y, stream));
}

size_t moe_forward_workspace_size(int n, int H, int I, int E, int K, moe_dtype dt) {
  if (n < 0 || H < 1 || I < 1 || E < 1 || K < 1 || !dtype_ok(dt)) return 0;
  return forward_layout(n, H, I, E, K, dt).total;
}

size_t moe_workspace_size(int n, int H, int I, int E, int K, moe_dtype dt) {
  return moe_forward_workspace_size(n, H, I, E, K, dt);
}

moe_status moe_forward_timed(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2,
                             int n, int H, int I, int E, int K, int renorm, moe_dtype dt, void* y,
                             float* logits_out, int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                             void* ws, size_t ws_bytes, hipEvent_t gemm1_begin, hipEvent_t gemm1_end,
                             hipStream_t stream) {
  const moe_status st = check_forward(x, W_gate, bias, W13, W2, n, H, I, E, K, dt, y, logits_out, topk_ids_out,
                                      topk_w_out, counts_out);
  if (st != MOE_OK) return st;
  if (!vec_ok({ws})) return MOE_EINVAL;
  if (n == 0)  // no tokens: nothing to compute; the optional counts are all zero
    return counts_out ? from_hip(launch_fill_zero(counts_out, (size_t)E * 4, stream)) : MOE_OK;
  if (ws == nullptr || ws_bytes < forward_layout(n, H, I, E, K, dt).total) return MOE_EWORKSPACE;
  return forward_enqueue(x, W_gate, bias, W13, W2, n, H, I, E, K, renorm, dt, y, logits_out, topk_ids_out,
                         topk_w_out, counts_out, (char*)ws, stream, gemm1_begin, gemm1_end);
}

size_t moe_packed_w13_bytes(int E, int H, int I) {
  if (E < 1 || E > kMaxExperts || !hidden_ok(H, MOE_BF16) || !hidden_ok(I, MOE_BF16)) return 0;
  return packed_weight_bytes(E, H, ceil_div(I, 128));
}

size_t moe_packed_w2_bytes(int E, int H, int I) {
  if (E < 1 || E > kMaxExperts || !hidden_ok(H, MOE_BF16) || !hidden_ok(I, MOE_BF16)) return 0;
  return packed_weight_bytes(E, I, ceil_div(H, 256));
}

moe_status moe_pack_w13(const void* W13, int E, int H, int I, void* W13p, hipStream_t stream) {
  if (E < 1 || E > kMaxExperts || !hidden_ok(H, MOE_BF16) || !hidden_ok(I, MOE_BF16)) return MOE_EINVAL;
  if (W13 == nullptr || W13p == nullptr || !vec_ok({W13, W13p})) return MOE_EINVAL;
  return from_hip(launch_pack_weights(W13, E, H, 2 * I, I, ceil_div(I, 128), W13p, stream));
}

moe_status moe_pack_w2(const void* W2, int E, int H, int I, void* W2p, hipStream_t stream) {
  if (E < 1 || E > kMaxExperts || !hidden_ok(H, MOE_BF16) || !hidden_ok(I, MOE_BF16)) return MOE_EINVAL;
  if (W2 == nullptr || W2p == nullptr || !vec_ok({W2, W2p})) return MOE_EINVAL;
  return from_hip(launch_pack_weights(W2, E, I, H, 0, ceil_div(H, 256), W2p, stream));
}

moe_status moe_forward_packed(const void* x, const void* W_gate, const float* bias, const void* W13p,
                              const void* W2p, int n, int H, int I, int E, int K, int renorm, void* y,
                              float* logits_out, int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                              void* ws, size_t ws_bytes, hipEvent_t gemm1_begin, hipEvent_t gemm1_end,
                              hipStream_t stream) {
  const moe_status st = check_forward(x, W_gate, bias, W13p, W2p, n, H, I, E, K, MOE_BF16, y, logits_out,
                                      topk_ids_out, topk_w_out, counts_out);
  if (st != MOE_OK) return st;
  if (!vec_ok({ws})) return MOE_EINVAL;
  if (n == 0)  // no tokens: nothing to compute; the optional counts are all zero
    return counts_out ? from_hip(launch_fill_zero(counts_out, (size_t)E * 4, stream)) : MOE_OK;
  if (ws == nullptr || ws_bytes < forward_layout(n, H, I, E, K, MOE_BF16).total) return MOE_EWORKSPACE;
  return forward_enqueue(x, W_gate, bias, W13p, W2p, n, H, I, E, K, renorm, MOE_BF16, y, logits_out, topk_ids_out,
                         topk_w_out, counts_out, (char*)ws, stream, gemm1_begin, gemm1_end, true);
}

moe_status moe_forward(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2, int n,
                       int H, int I, int E, int K, int renorm, moe_dtype dt, void* y, float* logits_out,
                       int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  return moe_forward_timed(x, W_gate, bias, W13, W2, n, H, I, E, K, renorm, dt, y, logits_out, topk_ids_out,
                           topk_w_out, counts_out, ws, ws_bytes, nullptr, nullptr, stream);
}

size_t moe_forward_persistent_workspace_size(int n, int H, int I, int E, int K, int pool_row_tiles) {
  if (n < 0 || H < 1 || I < 1 || E < 1 || K < 1 || pool_row_tiles < 0) return 0;
  if ((long long)n * K > INT32_MAX) return 0;
  return persistent_layout(n, H, I, E, K, pool_row_tiles).total;
}

namespace {
moe_status persistent_call(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2,
                           int n, int H, int I, int E, int K, int renorm, moe_dtype dt, int warmup_row_tiles,
                           int pool_row_tiles, void* y, float* logits_out, int32_t* topk_ids_out, float* topk_w_out,
                           int32_t* counts_out, void* ws, size_t ws_bytes, hipStream_t stream, bool packed) {
  const moe_status st = check_forward(x, W_gate, bias, W13, W2, n, H, I, E, K, dt, y, logits_out, topk_ids_out,
                                      topk_w_out, counts_out);
  if (st != MOE_OK) return st;
  if (dt != MOE_BF16) return MOE_EUNSUPPORTED;
  // The ring must hold the warm-up row tiles and one more, so that an L1 tile
  // only ever waits for L2 tiles taken before it.
  if (warmup_row_tiles < 1 || pool_row_tiles < 0 || (pool_row_tiles > 0 && pool_row_tiles <= warmup_row_tiles))
    return MOE_EINVAL;
  if (!vec_ok({ws})) return MOE_EINVAL;
  if (n == 0) return counts_out ? from_hip(launch_fill_zero(counts_out, (size_t)E * 4, stream)) : MOE_OK;
  // A ticket packs its queue into the top byte: at most 2^24 tasks per queue.
  const long long tasks_per_queue =
      ((long long)fused_ffn_max_row_tiles(n * K, E) / 8 + 1) * (ceil_div(I, 128) + ceil_div(H, 256));
  if (tasks_per_queue >= (1LL << 24)) return MOE_EUNSUPPORTED;
  const PersistentLayout L = persistent_layout(n, H, I, E, K, pool_row_tiles);
  if (ws == nullptr || ws_bytes < L.total) return MOE_EWORKSPACE;
  char* base = (char*)ws;
  float* logits = logits_out ? logits_out : (float*)(base + L.logits);
  int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(base + L.ids);
  float* w = topk_w_out ? topk_w_out : (float*)(base + L.w);
  int32_t* counts = counts_out ? counts_out : (int32_t*)(base + L.counts);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* perm = (int32_t*)(base + L.perm);
  int32_t* inv = (int32_t*)(base + L.inv);
  hipError_t e = launch_route(x, W_gate, bias, n, H, E, K, renorm, dt, logits, ids, w, stream);
  if (e == hipSuccess)
    e = launch_permute(ids, nullptr, n, H, E, K, 1, dt, counts, offsets, (int32_t*)(base + L.splits), perm, inv,
                       nullptr, (int32_t*)(base + L.pscratch), stream);
  if (e == hipSuccess)
    e = launch_fused_ffn(x, perm, n, K, offsets, W13, W2, E, H, I, warmup_row_tiles, pool_row_tiles, base + L.h,
                         base + L.Y_perm, (int*)(base + L.counters), stream, packed);
  if (e == hipSuccess) e = launch_combine(base + L.Y_perm, inv, w, n, H, K, dt, y, stream);
  return from_hip(e);
}
}  // namespace

moe_status moe_forward_persistent(const void* x, const void* W_gate, const float* bias, const void* W13,
                                  const void* W2, int n, int H, int I, int E, int K, int renorm, moe_dtype dt,
                                  int warmup_row_tiles, int pool_row_tiles, void* y, float* logits_out,
                                  int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  return persistent_call(x, W_gate, bias, W13, W2, n, H, I, E, K, renorm, dt, warmup_row_tiles, pool_row_tiles, y,
                         logits_out, topk_ids_out, topk_w_out, counts_out, ws, ws_bytes, stream, false);
}

moe_status moe_forward_persistent_packed(const void* x, const void* W_gate, const float* bias, const void* W13p,
                                         const void* W2p, int n, int H, int I, int E, int K, int renorm,
                                         int warmup_row_tiles, int pool_row_tiles, void* y, float* logits_out,
                                         int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  return persistent_call(x, W_gate, bias, W13p, W2p, n, H, I, E, K, renorm, MOE_BF16, warmup_row_tiles,
                         pool_row_tiles, y, logits_out, topk_ids_out, topk_w_out, counts_out, ws, ws_bytes, stream,
                         true);
}

size_t moe_forward_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

moe_status moe_forward_noalloc(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2,
                               int n, int H, int I, int E, int K, int renorm, moe_dtype dt, void* y,
                               float* logits_out, int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                               hipStream_t stream) {
  const moe_status st = check_forward(x, W_gate, bias, W13, W2, n, H, I, E, K, dt, y, logits_out, topk_ids_out,
                                      topk_w_out, counts_out);
  if (st != MOE_OK) return st;
  if (n == 0)
    return counts_out ? from_hip(launch_fill_zero(counts_out, (size_t)E * 4, stream)) : MOE_OK;
  if (forward_layout(n, H, I, E, K, dt).total > kNoAllocScratchBytes) return MOE_ETOOLARGE;
  char* base = scratch_ptr();
  if (base == nullptr) return MOE_EHIP;
  return forward_enqueue(x, W_gate, bias, W13, W2, n, H, I, E, K, renorm, dt, y, logits_out, topk_ids_out,
                         topk_w_out, counts_out, base, stream);
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------

moe_status moe_expert_w13_swiglu_gather_train(const void* x, const int32_t* perm, int n, int K,
                                              const int32_t* offsets, const void* W13, int E, int H, int I,
                                              moe_dtype dt, void* h, void* gate_up, hipStream_t stream) {
  if (n < 0 || K < 1 || K > kMaxTopK || (long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (n > 0 && (perm == nullptr || gate_up == nullptr)) return MOE_EINVAL;
  if (!vec_ok({gate_up}) || !word_ok({perm})) return MOE_EINVAL;
  const moe_status st = check_expert_gemm(x, offsets, n * K, W13, E, H, I, dt, h);
  if (st != MOE_OK) return st;
  return from_hip(launch_w13_swiglu_gather_train(x, perm, n, K, offsets, W13, E, H, I, dt, h, gate_up, stream));
}

size_t moe_forward_train_workspace_size(int n, int E, int K) {
  if (n < 0 || E < 1 || K < 1) return 0;
  return train_layout(n, E, K).total;
}

moe_status moe_forward_train(const void* x, const void* W_gate, const float* bias, const void* W13, const void* W2,
                             int n, int H, int I, int E, int K, int renorm, moe_dtype dt, void* y, float* logits,
                             int32_t* topk_ids, float* topk_w, int32_t* offsets, int32_t* perm, int32_t* inv,
                             void* gate_up, void* h, void* Y_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || !experts_ok(E, K) || !hidden_ok(H, dt) || !hidden_ok(I, dt)) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (offsets == nullptr) return MOE_EINVAL;
  if (n > 0 && (x == nullptr || W_gate == nullptr || W13 == nullptr || W2 == nullptr || y == nullptr ||
                logits == nullptr || topk_ids == nullptr || topk_w == nullptr || perm == nullptr || inv == nullptr ||
                gate_up == nullptr || h == nullptr || Y_perm == nullptr))
    return MOE_EINVAL;
  if (!vec_ok({x, W_gate, W13, W2, y, gate_up, h, Y_perm, ws}) ||
      !word_ok({bias, logits, topk_ids, topk_w, offsets, perm, inv}))
    return MOE_EINVAL;
  const TrainLayout L = train_layout(n, E, K);
  if (ws == nullptr || ws_bytes < L.total) return MOE_EWORKSPACE;
  char* base = (char*)ws;
  hipError_t e = launch_route(x, W_gate, bias, n, H, E, K, renorm, dt, logits, topk_ids, topk_w, stream);
  if (e != hipSuccess) return MOE_EHIP;
  e = launch_permute(topk_ids, nullptr, n, H, E, K, 1, dt, (int32_t*)(base + L.counts), offsets,
                     (int32_t*)(base + L.splits), perm, inv, nullptr, (int32_t*)(base + L.pscratch), stream);
  if (e != hipSuccess) return MOE_EHIP;
  if (n == 0) return MOE_OK;
  e = launch_w13_swiglu_gather_train(x, perm, n, K, offsets, W13, E, H, I, dt, h, gate_up, stream);
  if (e != hipSuccess) return MOE_EHIP;
  e = launch_w2(h, offsets, n * K, W2, E, H, I, dt, Y_perm, stream);
  if (e != hipSuccess) return MOE_EHIP;
  return from_hip(launch_combine(Y_perm, inv, topk_w, n, H, K, dt, y, stream));
}

moe_status moe_combine_backward(const void* dy, const void* Y_perm, const int32_t* inv, const float* topk_w, int n,
                                int H, int K, moe_dtype dt, void* dY_perm, float* dw, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || K < 1 || K > kMaxTopK || !hidden_ok(H, dt)) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  if (dy == nullptr || Y_perm == nullptr || inv == nullptr || topk_w == nullptr || dY_perm == nullptr ||
      dw == nullptr)
    return MOE_EINVAL;
  if (!vec_ok({dy, Y_perm, dY_perm}) || !word_ok({inv, topk_w, dw})) return MOE_EINVAL;
  return from_hip(launch_combine_backward(dy, Y_perm, inv, topk_w, n, H, K, dt, dY_perm, dw, stream));
}

moe_status moe_expert_w2_backward(const void* dY_perm, const int32_t* offsets, int rows, const void* W2,
                                  const void* gate_up, int E, int H, int I, moe_dtype dt, void* dgate_up,
                                  hipStream_t stream) {
  const moe_status st = check_expert_gemm(dY_perm, offsets, rows, W2, E, H, I, dt, dgate_up);
  if (st != MOE_OK) return st;
  if ((rows > 0 && gate_up == nullptr) || !vec_ok({gate_up})) return MOE_EINVAL;
  return from_hip(launch_w2_backward(dY_perm, offsets, rows, W2, gate_up, E, H, I, dt, dgate_up, stream));
}

moe_status moe_expert_w13_backward(const void* dgate_up, const int32_t* offsets, int rows, const void* W13, int E,
                                   int H, int I, moe_dtype dt, void* dX_perm, hipStream_t stream) {
  const moe_status st = check_expert_gemm(dgate_up, offsets, rows, W13, E, H, I, dt, dX_perm);
  if (st != MOE_OK) return st;
  return from_hip(launch_w13_backward(dgate_up, offsets, rows, W13, E, H, I, dt, dX_perm, stream));
}

moe_status moe_expert_weight_grad(const void* a, const void* b, const int32_t* offsets, int rows, int E, int M, int N,
                                  moe_dtype dt, void* dW, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (rows < 0 || E < 1 || E > kMaxExperts || !hidden_ok(M, dt) || !hidden_ok(N, dt)) return MOE_EINVAL;
  if (offsets == nullptr || dW == nullptr) return MOE_EINVAL;
  if (rows > 0 && (a == nullptr || b == nullptr)) return MOE_EINVAL;
  if (!vec_ok({a, b, dW}) || !word_ok({offsets})) return MOE_EINVAL;
  return from_hip(launch_weight_grad(a, b, offsets, rows, E, M, N, dt, dW, stream));
}

moe_status moe_expert_weight_grad_gather(const void* x, const int32_t* perm, int n, int K, const void* b,
                                         const int32_t* offsets, int E, int M, int N, moe_dtype dt, void* dW,
                                         hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || K < 1 || K > kMaxTopK || (long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (E < 1 || E > kMaxExperts || !hidden_ok(M, dt) || !hidden_ok(N, dt)) return MOE_EINVAL;
  if (offsets == nullptr || dW == nullptr) return MOE_EINVAL;
  if (n > 0 && (x == nullptr || perm == nullptr || b == nullptr)) return MOE_EINVAL;
  if (!vec_ok({x, b, dW}) || !word_ok({perm, offsets})) return MOE_EINVAL;
  return from_hip(launch_weight_grad_gather(x, perm, n, K, b, offsets, E, M, N, dt, dW, stream));
}

moe_status moe_dispatch_backward(const void* dX_perm, const int32_t* inv, const float* add, int n, int H, int K,
                                 moe_dtype dt, void* dx, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || K < 1 || K > kMaxTopK || !hidden_ok(H, dt)) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  if (dX_perm == nullptr || inv == nullptr || dx == nullptr) return MOE_EINVAL;
  if (!vec_ok({dX_perm, add, dx}) || !word_ok({inv})) return MOE_EINVAL;
  return from_hip(launch_dispatch_backward(dX_perm, inv, add, n, H, K, dt, dx, stream));
}

size_t moe_route_backward_workspace_size(int n, int H, int E) {
  if (n < 0 || H < 0 || E < 1) return 0;
  return route_bwd_ws(n, H, E);
}

moe_status moe_route_backward(const void* x, const void* W_gate, const float* logits, const int32_t* topk_ids,
                              const float* topk_w, const float* dw, int n, int H, int E, int K, int renorm,
                              moe_dtype dt, float* dlogits, float* dx_router, float* dW_gate, float* dbias, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || !experts_ok(E, K)) return MOE_EINVAL;
  const bool weights = dW_gate != nullptr || dbias != nullptr;
  if ((dx_router != nullptr || weights) && !hidden_ok(H, dt)) return MOE_EINVAL;
  if (n == 0) {  // no tokens: the weight gradients are zero
    if (dW_gate != nullptr && launch_fill_zero(dW_gate, (size_t)H * E * 4, stream) != hipSuccess) return MOE_EHIP;
    if (dbias != nullptr && launch_fill_zero(dbias, (size_t)E * 4, stream) != hipSuccess) return MOE_EHIP;
    return MOE_OK;
  }
  if (logits == nullptr || topk_ids == nullptr || topk_w == nullptr || dw == nullptr || dlogits == nullptr)
    return MOE_EINVAL;
  if (dx_router != nullptr && W_gate == nullptr) return MOE_EINVAL;
  if (weights && x == nullptr) return MOE_EINVAL;
  if (!vec_ok({x, W_gate, dx_router, dW_gate, ws}) || !word_ok({logits, topk_ids, topk_w, dw, dlogits, dbias}))
    return MOE_EINVAL;
  if ((weights || dx_router != nullptr) && (ws == nullptr || ws_bytes < route_bwd_ws(n, H, E)))
    return MOE_EWORKSPACE;
  return from_hip(launch_route_backward(x, W_gate, logits, topk_ids, topk_w, dw, n, H, E, K, renorm, dt, dlogits,
                                        dx_router, dW_gate, dbias, ws, stream));
}

size_t moe_backward_workspace_size(int n, int H, int I, int E, int K, moe_dtype dt) {
  if (n < 0 || H < 1 || I < 1 || E < 1 || K < 1 || !dtype_ok(dt)) return 0;
  return backward_layout(n, H, I, E, K, dt).total;
}

moe_status moe_backward(const void* dy, const void* x, const void* W_gate, const void* W13, const void* W2, int n,
                        int H, int I, int E, int K, int renorm, moe_dtype dt, const float* logits,
                        const int32_t* topk_ids, const float* topk_w, const int32_t* offsets, const int32_t* perm,
                        const int32_t* inv, const void* gate_up, const void* h, const void* Y_perm, void* dx,
                        float* dW_gate, float* dbias, void* dW13, void* dW2, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || !experts_ok(E, K) || !hidden_ok(H, dt) || !hidden_ok(I, dt)) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (offsets == nullptr || dW_gate == nullptr || dW13 == nullptr || dW2 == nullptr) return MOE_EINVAL;
  if (n > 0 && (dy == nullptr || x == nullptr || W_gate == nullptr || W13 == nullptr || W2 == nullptr ||
                logits == nullptr || topk_ids == nullptr || topk_w == nullptr || perm == nullptr || inv == nullptr ||
                gate_up == nullptr || h == nullptr || Y_perm == nullptr || dx == nullptr))
    return MOE_EINVAL;
  if (!vec_ok({dy, x, W_gate, W13, W2, gate_up, h, Y_perm, dx, dW_gate, dW13, dW2, ws}) ||
      !word_ok({logits, topk_ids, topk_w, offsets, perm, inv, dbias}))
    return MOE_EINVAL;
  const BackwardLayout L = backward_layout(n, H, I, E, K, dt);
  if (ws == nullptr || ws_bytes < L.total) return MOE_EWORKSPACE;
  char* base = (char*)ws;
  void* rows_a = base + L.rows_a;
  void* dgu = base + L.dgu;
  float* dw = (float*)(base + L.dw);
  float* dlogits = (float*)(base + L.dlogits);
  float* dx_router = (float*)(base + L.dx_router);
  const int rows = n * K;

  hipError_t e = hipSuccess;
  if (n == 0) {  // no rows: every weight gradient is zero
    e = launch_fill_zero(dW13, (size_t)E * H * 2 * I * elt_size(dt), stream);
    if (e == hipSuccess) e = launch_fill_zero(dW2, (size_t)E * I * H * elt_size(dt), stream);
    if (e == hipSuccess) e = launch_fill_zero(dW_gate, (size_t)H * E * 4, stream);
    if (e == hipSuccess && dbias != nullptr) e = launch_fill_zero(dbias, (size_t)E * 4, stream);
    return from_hip(e);
  }
  void* rows_b = base + L.rows_b;
  // Two branches run beside the main chain on a second stream:
  //   main: combine bwd -> dgate_up ------(join 1)-> dX_perm -> dispatch bwd -(join 2)
  //   aux:             \-> route bwd -> dW2 -/   \-> gather x_perm -> dW13 ----/
  // dW2 and dgate_up both read dY_perm, which dX_perm overwrites after join 1.
  // The second stream is shared by every call on this device, so it is used
  // only when it is free of other work's graph capture: when it is being
  // captured into another capture than the caller's stream (a capture on
  // another thread that forked into it and has not ended yet), the branches
  // run on the caller's stream instead, in the same order as above.
  std::lock_guard<std::mutex> lock(g_aux_mutex);
  AuxStream* aux = aux_stream();
  if (aux != nullptr) {
    const unsigned long long aux_cap = capture_id(aux->s);
    if (aux_cap == ~0ull || (aux_cap != 0 && aux_cap != capture_id(stream))) aux = nullptr;
  }
  hipStream_t side = aux ? aux->s : stream;
  auto fork = [&](int i, hipStream_t from, hipStream_t to) {
    if (from == to) return hipSuccess;
    hipError_t r = hipEventRecord(aux->ev[i], from);
    return r == hipSuccess ? hipStreamWaitEvent(to, aux->ev[i], 0) : r;
  };
  e = launch_combine_backward(dy, Y_perm, inv, topk_w, n, H, K, dt, rows_a, dw, stream);
  if (e == hipSuccess) e = fork(0, stream, side);
  if (e == hipSuccess)
    e = launch_route_backward(x, W_gate, logits, topk_ids, topk_w, dw, n, H, E, K, renorm, dt, dlogits, dx_router,
                              dW_gate, dbias, base + L.rws, side);
  if (e == hipSuccess) e = launch_weight_grad(h, rows_a, offsets, rows, E, I, H, dt, dW2, side);
  if (e == hipSuccess) e = launch_w2_backward(rows_a, offsets, rows, W2, gate_up, E, H, I, dt, dgu, stream);
  if (e == hipSuccess) e = fork(1, side, stream);    // join 1: dW2 and the router gradients are done
  if (e == hipSuccess) e = fork(2, stream, side);    // dgate_up is ready for dW13
  if (e == hipSuccess) e = launch_gather_rows(x, perm, n, H, K, dt, rows_b, side);
  if (e == hipSuccess) e = launch_weight_grad(rows_b, dgu, offsets, rows, E, H, 2 * I, dt, dW13, side);
  if (e == hipSuccess) e = launch_w13_backward(dgu, offsets, rows, W13, E, H, I, dt, rows_a, stream);
  if (e == hipSuccess) e = launch_dispatch_backward(rows_a, inv, dx_router, n, H, K, dt, dx, stream);
  if (e == hipSuccess) e = fork(3, side, stream);    // join 2: dW13 is done
  return from_hip(e);
}

// ---------------------------------------------------------------------------
// FP8 expert weights
// ---------------------------------------------------------------------------

moe_status moe_quantize_fp8(const void* W, int E, int Kd, int N, moe_dtype dt, uint8_t* codes, float* scales,
                            hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (E < 0 || !hidden_ok(Kd, MOE_BF16) || N < 1 || N % 4 != 0) return MOE_EINVAL;
  if (E == 0) return MOE_OK;
  if (W == nullptr || codes == nullptr || scales == nullptr || !vec_ok({W, codes, scales})) return MOE_EINVAL;
  return from_hip(launch_quantize_fp8(W, E, Kd, N, dt, codes, scales, stream));
}

static moe_status check_fp8_gemm(const void* a, const int32_t* offsets, int rows, const void* wq, const float* sc,
                                 int E, int H, int I, moe_dtype dt, const void* out) {
  if (dt != MOE_BF16) return MOE_EUNSUPPORTED;  // FP8 weights pair with bf16 activations
  if (rows < 0 || E < 1 || E > kMaxExperts || !hidden_ok(H, dt) || !hidden_ok(I, dt)) return MOE_EINVAL;
  if (rows > 0 && (a == nullptr || offsets == nullptr || wq == nullptr || sc == nullptr || out == nullptr))
    return MOE_EINVAL;
  if (!vec_ok({a, wq, sc, out}) || !word_ok({offsets})) return MOE_EINVAL;
  return MOE_OK;
}

moe_status moe_expert_w13_swiglu_gather_fp8(const void* x, const int32_t* perm, int n, int K, const int32_t* offsets,
                                            const uint8_t* W13q, const float* s13, int E, int H, int I, moe_dtype dt,
                                            void* h, hipStream_t stream) {
  if (n < 0 || K < 1 || K > kMaxTopK || (long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (n > 0 && perm == nullptr) return MOE_EINVAL;
  const moe_status st = check_fp8_gemm(x, offsets, n * K, W13q, s13, E, H, I, dt, h);
  if (st != MOE_OK) return st;
  return from_hip(launch_w13_swiglu_gather_fp8(x, perm, n, K, offsets, W13q, s13, E, H, I, h, stream));
}

moe_status moe_expert_w13_swiglu_from_ids_fp8(const void* x, const int32_t* topk_ids, int n, int K,
                                              const uint8_t* W13q, const float* s13, int E, int H, int I, int ep,
                                              void* h, int32_t* counts, int32_t* offsets, int32_t* splits,
                                              int32_t* perm, int32_t* inv, hipStream_t stream) {
  if (n < 0 || !experts_ok(E, K) || ep < 1 || E % ep != 0 || !hidden_ok(H, MOE_BF16) || !hidden_ok(I, MOE_BF16))
    return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (counts == nullptr || offsets == nullptr || splits == nullptr) return MOE_EINVAL;
  if (!word_ok({topk_ids, counts, offsets, splits, perm, inv})) return MOE_EINVAL;
  if (n == 0)
    return from_hip(launch_permute(nullptr, nullptr, 0, H, E, K, ep, MOE_BF16, counts, offsets, splits, nullptr,
                                   nullptr, nullptr, nullptr, stream));
  if (!w13_from_ids_fp8_ok(n, K, E)) return MOE_EUNSUPPORTED;
  if (x == nullptr || topk_ids == nullptr || W13q == nullptr || s13 == nullptr || h == nullptr || perm == nullptr ||
      inv == nullptr)
    return MOE_EINVAL;
  if (!vec_ok({x, W13q, s13, h})) return MOE_EINVAL;
  return from_hip(launch_w13_swiglu_from_ids_fp8(x, topk_ids, n, K, W13q, s13, E, H, I, ep, h, counts, offsets,
                                                 splits, perm, inv, stream));
}

moe_status moe_expert_w2_fp8(const void* h, const int32_t* offsets, int rows, const uint8_t* W2q, const float* s2,
                             int E, int H, int I, moe_dtype dt, void* Y_perm, hipStream_t stream) {
  const moe_status st = check_fp8_gemm(h, offsets, rows, W2q, s2, E, H, I, dt, Y_perm);
  if (st != MOE_OK) return st;
  return from_hip(launch_w2_fp8(h, offsets, rows, W2q, s2, E, H, I, Y_perm, stream));
}

moe_status moe_forward_fp8(const void* x, const void* W_gate, const float* bias, const uint8_t* W13q,
                           const float* s13, const uint8_t* W2q, const float* s2, int n, int H, int I, int E, int K,
                           int renorm, moe_dtype dt, void* y, float* logits_out, int32_t* topk_ids_out,
                           float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (dt != MOE_BF16) return MOE_EUNSUPPORTED;
  if (n < 0 || !experts_ok(E, K) || !hidden_ok(H, dt) || !hidden_ok(I, dt)) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (n > 0 && (x == nullptr || W_gate == nullptr || W13q == nullptr || s13 == nullptr || W2q == nullptr ||
                s2 == nullptr || y == nullptr))
    return MOE_EINVAL;
  if (!vec_ok({x, W_gate, W13q, s13, W2q, s2, y, ws}) ||
      !word_ok({bias, logits_out, topk_ids_out, topk_w_out, counts_out}))
    return MOE_EINVAL;
  if (n == 0)  // no tokens: nothing to compute; the optional counts are all zero
    return counts_out ? from_hip(launch_fill_zero(counts_out, (size_t)E * 4, stream)) : MOE_OK;
  const ForwardLayout L = forward_layout(n, H, I, E, K, dt);
  if (ws == nullptr || ws_bytes < L.total) return MOE_EWORKSPACE;
  char* base = (char*)ws;
  float* logits = logits_out ? logits_out : (float*)(base + L.logits);
  int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(base + L.ids);
  float* w = topk_w_out ? topk_w_out : (float*)(base + L.w);
  int32_t* counts = counts_out ? counts_out : (int32_t*)(base + L.counts);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* perm = (int32_t*)(base + L.perm);
  int32_t* inv = (int32_t*)(base + L.inv);
  hipError_t e = launch_route(x, W_gate, bias, n, H, E, K, renorm, dt, logits, ids, w, stream);
  if (e != hipSuccess) return MOE_EHIP;
  if (w13_from_ids_fp8_ok(n, K, E)) {
    // Decode-sized batch: GEMM1 places the pairs itself and writes the
    // metadata for GEMM2 and the combine (no permute launch).
    e = launch_w13_swiglu_from_ids_fp8(x, ids, n, K, W13q, s13, E, H, I, 1, base + L.h, counts, offsets,
                                       (int32_t*)(base + L.splits), perm, inv, stream);
  } else {
    e = launch_permute(ids, nullptr, n, H, E, K, 1, dt, counts, offsets, (int32_t*)(base + L.splits), perm, inv,
                       nullptr, (int32_t*)(base + L.pscratch), stream);
    if (e != hipSuccess) return MOE_EHIP;
    e = launch_w13_swiglu_gather_fp8(x, perm, n, K, offsets, W13q, s13, E, H, I, base + L.h, stream);
  }
  if (e != hipSuccess) return MOE_EHIP;
  e = launch_w2_fp8(base + L.h, offsets, n * K, W2q, s2, E, H, I, base + L.Y_perm, stream);
  if (e != hipSuccess) return MOE_EHIP;
  return from_hip(launch_combine(base + L.Y_perm, inv, w, n, H, K, dt, y, stream));
}


// ---------------------------------------------------------------------------
// FP8 activations: per-token FP8 dispatch into a padded receive buffer and
// the FP8 x FP8 first expert GEMM
// ---------------------------------------------------------------------------

size_t moe_fp8_padded_rows(int n, int E, int K) {
  if (n < 0 || E < 1 || K < 1) return 0;
  return fp8_padded_rows(n, E, K);
}

moe_status moe_quantize_rows_fp8(const void* x, int n, int H, moe_dtype dt, uint8_t* codes, float* scales,
                                 hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (n < 0 || !hidden_ok(H, dt) || H % 8 != 0) return MOE_EINVAL;  // eight elements per lane step
  if (n == 0) return MOE_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return MOE_EINVAL;
  if (!vec_ok({x, codes}) || !word_ok({scales})) return MOE_EINVAL;
  return from_hip(launch_quantize_rows_fp8(x, n, H, dt, codes, scales, stream));
}

moe_status moe_dispatch_fp8(const int32_t* counts, const int32_t* offsets, const int32_t* perm, int n, int E, int K,
                            const uint8_t* codes_tok, const float* s_tok, int H, int32_t* offsets_padded,
                            uint8_t* x_q, float* x_scale, int32_t* perm_padded, int32_t* inv_padded,
                            hipStream_t stream) {
  if (n < 0 || !experts_ok(E, K) || H <= 0 || H > kMaxHidden || H % 16 != 0) return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX / 2) return MOE_EINVAL;
  if (counts == nullptr || offsets == nullptr || offsets_padded == nullptr) return MOE_EINVAL;
  if (n > 0 && (perm == nullptr || codes_tok == nullptr || s_tok == nullptr || x_q == nullptr ||
                x_scale == nullptr || perm_padded == nullptr || inv_padded == nullptr))
    return MOE_EINVAL;
  if (!vec_ok({codes_tok, x_q}) || !word_ok({counts, offsets, perm, s_tok, offsets_padded, x_scale, perm_padded,
                                             inv_padded}))
    return MOE_EINVAL;
  return from_hip(launch_dispatch_fp8(counts, offsets, perm, n, E, K, codes_tok, s_tok, H, offsets_padded, x_q,
                                      x_scale, perm_padded, inv_padded, stream));
}

moe_status moe_expert_w13_swiglu_fp8a(const uint8_t* x_q, const float* x_scale, const int32_t* offsets_padded,
                                      int rows_max, const uint8_t* W13q, const float* s13, int E, int H, int I,
                                      void* h, hipStream_t stream) {
  if (rows_max < 0 || E < 1 || E > kMaxExperts || !hidden_ok(H, MOE_BF16) || H % 128 != 0 ||
      !hidden_ok(I, MOE_BF16))
    return MOE_EINVAL;
  if (rows_max == 0) return MOE_OK;
  if (x_q == nullptr || x_scale == nullptr || offsets_padded == nullptr || W13q == nullptr || s13 == nullptr ||
      h == nullptr)
    return MOE_EINVAL;
  if (!vec_ok({x_q, W13q, s13, h}) || !word_ok({x_scale, offsets_padded})) return MOE_EINVAL;
  return from_hip(launch_w13_swiglu_fp8a(x_q, x_scale, offsets_padded, rows_max, W13q, s13, E, H, I, h, stream));
}

moe_status moe_expert_w13_swiglu_gather_fp8a(const uint8_t* codes_tok, const float* s_tok, const int32_t* perm,
                                             int n, int K, const int32_t* offsets, const uint8_t* W13q,
                                             const float* s13, int E, int H, int I, void* h, hipStream_t stream) {
  if (n < 0 || !experts_ok(E, K) || !hidden_ok(H, MOE_BF16) || H % 128 != 0 || !hidden_ok(I, MOE_BF16))
    return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  if (codes_tok == nullptr || s_tok == nullptr || perm == nullptr || offsets == nullptr || W13q == nullptr ||
      s13 == nullptr || h == nullptr)
    return MOE_EINVAL;
  if (!vec_ok({codes_tok, W13q, s13, h}) || !word_ok({s_tok, perm, offsets})) return MOE_EINVAL;
  return from_hip(
      launch_w13_swiglu_gather_fp8a(codes_tok, s_tok, perm, n, K, offsets, W13q, s13, E, H, I, h, stream));
}

moe_status moe_expert_w13_swiglu_from_ids_fp8a(const uint8_t* codes_tok, const float* s_tok,
                                               const int32_t* topk_ids, int n, int K, const uint8_t* W13q,
                                               const float* s13, int E, int H, int I, int ep, void* h,
                                               int32_t* counts, int32_t* offsets, int32_t* splits, int32_t* perm,
                                               int32_t* inv, hipStream_t stream) {
  if (n < 0 || !experts_ok(E, K) || ep < 1 || E % ep != 0 || !hidden_ok(H, MOE_BF16) || H % 128 != 0 ||
      !hidden_ok(I, MOE_BF16) || I % 128 != 0)
    return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX) return MOE_EINVAL;
  if (counts == nullptr || offsets == nullptr || splits == nullptr) return MOE_EINVAL;
  if (!word_ok({topk_ids, counts, offsets, splits, perm, inv, s_tok})) return MOE_EINVAL;
  if (n == 0)
    return from_hip(launch_permute(nullptr, nullptr, 0, H, E, K, ep, MOE_BF16, counts, offsets, splits, nullptr,
                                   nullptr, nullptr, nullptr, stream));
  if (!w13_from_ids_fp8a_ok(n, K, E)) return MOE_EUNSUPPORTED;
  if (codes_tok == nullptr || s_tok == nullptr || topk_ids == nullptr || W13q == nullptr || s13 == nullptr ||
      h == nullptr || perm == nullptr || inv == nullptr)
    return MOE_EINVAL;
  if (!vec_ok({codes_tok, W13q, s13, h})) return MOE_EINVAL;
  return from_hip(launch_w13_swiglu_from_ids_fp8a(codes_tok, s_tok, topk_ids, n, K, W13q, s13, E, H, I, ep, h,
                                                  counts, offsets, splits, perm, inv, stream));
}

moe_status moe_expert_w2_fp8a(const uint8_t* h_q, const float* h_scale, const int32_t* offsets_padded, int rows_max,
                              const uint8_t* W2q, const float* s2, int E, int H, int I, void* Y_perm,
                              hipStream_t stream) {
  if (rows_max < 0 || E < 1 || E > kMaxExperts || !hidden_ok(H, MOE_BF16) || !hidden_ok(I, MOE_BF16) ||
      I % 128 != 0)
    return MOE_EINVAL;
  if (rows_max == 0) return MOE_OK;
  if (h_q == nullptr || h_scale == nullptr || offsets_padded == nullptr || W2q == nullptr || s2 == nullptr ||
      Y_perm == nullptr)
    return MOE_EINVAL;
  if (!vec_ok({h_q, W2q, s2, Y_perm}) || !word_ok({h_scale, offsets_padded})) return MOE_EINVAL;
  return from_hip(launch_w2_fp8a(h_q, h_scale, offsets_padded, rows_max, W2q, s2, E, H, I, Y_perm, stream));
}

size_t moe_forward_fp8a_workspace_size(int n, int H, int I, int E, int K) {
  if (n < 0 || H < 1 || I < 1 || E < 1 || K < 1) return 0;
  return fp8a_layout(n, H, I, E, K).total;
}

moe_status moe_forward_fp8a(const void* x, const void* W_gate, const float* bias, const uint8_t* W13q,
                            const float* s13, const uint8_t* W2q, const float* s2, int n, int H, int I, int E, int K,
                            int renorm, moe_dtype dt, void* y, float* logits_out, int32_t* topk_ids_out,
                            float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dt)) return MOE_EUNSUPPORTED;
  if (dt != MOE_BF16) return MOE_EUNSUPPORTED;
  if (n < 0 || !experts_ok(E, K) || !hidden_ok(H, dt) || H % 128 != 0 || !hidden_ok(I, dt) || I % 128 != 0)
    return MOE_EINVAL;
  if ((long long)n * K > INT32_MAX / 2) return MOE_EINVAL;
  if (n > 0 && (x == nullptr || W_gate == nullptr || W13q == nullptr || s13 == nullptr || W2q == nullptr ||
                s2 == nullptr || y == nullptr))
    return MOE_EINVAL;
  if (!vec_ok({x, W_gate, W13q, s13, W2q, s2, y, ws}) ||
      !word_ok({bias, logits_out, topk_ids_out, topk_w_out, counts_out}))
    return MOE_EINVAL;
  if (n == 0)
    return counts_out ? from_hip(launch_fill_zero(counts_out, (size_t)E * 4, stream)) : MOE_OK;
  const Fp8aLayout L = fp8a_layout(n, H, I, E, K);
  if (ws == nullptr || ws_bytes < L.total) return MOE_EWORKSPACE;
  char* base = (char*)ws;
  float* logits = logits_out ? logits_out : (float*)(base + L.logits);
  int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(base + L.ids);
  float* w = topk_w_out ? topk_w_out : (float*)(base + L.w);
  int32_t* counts = counts_out ? counts_out : (int32_t*)(base + L.counts);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* perm = (int32_t*)(base + L.perm);
  int32_t* inv = (int32_t*)(base + L.inv);
  uint8_t* codes_tok = (uint8_t*)(base + L.codes_tok);
  float* s_tok = (float*)(base + L.s_tok);
  const int nk = n * K;
  // On one GPU the per-token FP8 rows are read in place through perm (as the
  // bf16 layer reads x): the padded receive buffer of moe_dispatch_fp8 is what
  // an expert-parallel exchange would deliver, and not needed here.
  hipError_t e = launch_route(x, W_gate, bias, n, H, E, K, renorm, dt, logits, ids, w, stream);
  if (w13_from_ids_fp8a_ok(n, K, E)) {
    // Decode-sized batch: GEMM1 places the pairs itself and writes the
    // metadata for GEMM2 and the combine (no permute launch).
    if (e == hipSuccess) e = launch_quantize_rows_fp8(x, n, H, dt, codes_tok, s_tok, stream);
    if (e == hipSuccess)
      e = launch_w13_swiglu_from_ids_fp8a(codes_tok, s_tok, ids, n, K, W13q, s13, E, H, I, 1, base + L.h, counts,
                                          offsets, (int32_t*)(base + L.splits), perm, inv, stream);
  } else {
    if (e == hipSuccess)
      e = launch_permute(ids, nullptr, n, H, E, K, 1, dt, counts, offsets, (int32_t*)(base + L.splits), perm, inv,
                         nullptr, (int32_t*)(base + L.pscratch), stream);
    if (e == hipSuccess) e = launch_quantize_rows_fp8(x, n, H, dt, codes_tok, s_tok, stream);
    if (e == hipSuccess)
      e = launch_w13_swiglu_gather_fp8a(codes_tok, s_tok, perm, n, K, offsets, W13q, s13, E, H, I, base + L.h,
                                        stream);
  }
  // h per row in FP8, then GEMM2 on the FP8 MFMA.
  if (e == hipSuccess)
    e = launch_quantize_rows_fp8(base + L.h, nk, I, MOE_BF16, (uint8_t*)(base + L.h_q), (float*)(base + L.h_scale),
                                 stream);
  if (e == hipSuccess)
    e = launch_w2_fp8a((uint8_t*)(base + L.h_q), (float*)(base + L.h_scale), offsets, nk, W2q, s2, E, H, I,
                       base + L.Y_perm, stream);
  if (e == hipSuccess) e = launch_combine(base + L.Y_perm, inv, w, n, H, K, dt, y, stream);
  return from_hip(e);
}

}  // extern "C"
