// Dispatch metadata and row gather: counts, offsets, splits, the stable
// expert-major permutation of the n*K (token, slot) pairs, and
// x_perm[p] = x[perm[p] / K].
//
// What is computed: the per-expert hit counts n_e and the sets I_e of
// Algorithm 2 ("MoE 分布式推理基础（基于 vLLM）" §1.2), laid out in the
// expert-sorted order of that page's moe_align_block_size example (§2.3)
// without padding, with the per-rank send sizes of its Algorithm 5 step 3
// (§2.4); the torchtitan `_local_reorder` / `_permute` and the index
// inversion kernel of "0. goin" (§2.2, §2.3) are the same operation.
//
// How: up to 4096 pairs, one workgroup with the ids staged in LDS
// (permute_single_kernel). Beyond that, two launches over blocks of P pairs
// (at most 128 blocks):
//   1. count:  per-block histogram in LDS (integer atomics: the result does
//              not depend on their order).
//   2. place:  every block reads all block histograms (a few KB from L2) and
//              derives the per-expert totals, the exclusive offsets and its
//              own starting row per expert, so no separate scan launch is
//              needed; then each wave walks its part of the block in 64-pair
//              steps. Lanes with the same expert are found with ballots over
//              the id bits and ranked by a popcount of the lower lanes, so
//              pairs keep ascending flat order inside every expert segment.
// When x is given, a row gather follows: one wave per destination row copies
// 16-byte vectors.
#include "place_pairs.hpp"

namespace moe {
namespace {

constexpr int kWaves = kPermThreads / 64;  // 4
constexpr int kMaxBlocks = kPermMaxBlocks;
constexpr int kStepBatch = 8;              // 64-pair steps whose ids are loaded together

// Pairs per block of the count + place launches: a multiple of 256 (whole
// 64-pair steps for each of the 4 waves), at least 512, and large enough that
// there are at most kMaxBlocks.
inline int pairs_per_block(int total) {
  int p = ceil_div(ceil_div(total, kMaxBlocks), 256) * 256;
  return p < 512 ? 512 : p;
}

__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(const int32_t* __restrict__ ids, int total,
                                                                     int E, int P,
                                                                     int32_t* __restrict__ block_counts) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kPermThreads) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * P;
  const int end = min(base + P, total);
  for (int f = base + (int)threadIdx.x; f < end; f += kPermThreads) {
    const int e = ids[f];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) block_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Block b places its P pairs. Each wave first counts its quarter of the
// block per expert; then the block derives, from every block's counts, the
// per-expert totals, the exclusive offsets and the number of pairs of each
// expert in the blocks before it (block 0 also writes counts, offsets and
// splits); finally each wave walks its quarter in 64-pair steps and places
// pairs in ascending flat order.
__global__ __launch_bounds__(kPermThreads) void permute_place_kernel(const int32_t* __restrict__ ids, int total,
                                                                     int E, int ep, int P, int nblk, int id_bits,
                                                                     const int32_t* __restrict__ block_counts,
                                                                     int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ splits,
                                                                     int32_t* __restrict__ perm,
                                                                     int32_t* __restrict__ inv) {
  __shared__ int scan[kMaxExperts];
  __shared__ int offs[kMaxExperts + 1];
  __shared__ int next[kWaves][kMaxExperts];  // next free row per (wave, expert)
  __shared__ int part_before[kPermThreads], part_tot[kPermThreads];  // [g * E + e]
  __shared__ int wave_tot[kWaves];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x;
  for (int i = tid; i < kWaves * kMaxExperts; i += kPermThreads) (&next[0][0])[i] = 0;
  __syncthreads();
  // Pass 1: this wave's pairs per expert.
  const int per_wave = P / kWaves;
  const int wbase = b * P + wave * per_wave;
  const int steps = per_wave / 64;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s0 = 0; s0 < steps; s0 += kStepBatch) {
    int eid[kStepBatch];
#pragma unroll
    for (int q = 0; q < kStepBatch; ++q) {
      const int f = wbase + (s0 + q) * 64 + lane;
      eid[q] = (s0 + q < steps && f < total) ? ids[f] : -1;
    }
#pragma unroll
    for (int q = 0; q < kStepBatch; ++q) {
      const int e = eid[q];
      const bool valid = (unsigned)e < (unsigned)E;
      const uint64_t same = same_expert_lanes(e, valid, id_bits);
      if (valid && (same & below) == 0) next[wave][e] += __popcll(same);
      wave_sync_lds();
    }
  }
  __syncthreads();
  // Per-expert totals and the pairs of each expert in earlier blocks. The G =
  // kPermThreads / E threads of expert e split the block histograms (thread
  // (g, e) reads blocks g, g + G, ...), so their loads are in flight together;
  // the partial sums meet in LDS.
  const int G = kPermThreads / E;  // >= 1: E <= kMaxExperts = kPermThreads
  {
    const int e = tid % E, g = tid / E;
    int pb = 0, pt = 0;
    if (g < G) {
      for (int b0 = g; b0 < nblk; b0 += 16 * G) {
        int c[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int bb = b0 + q * G;
          c[q] = (bb < nblk) ? block_counts[(size_t)bb * E + e] : 0;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          pb += (b0 + q * G < b) ? c[q] : 0;
          pt += c[q];
        }
      }
      part_before[g * E + e] = pb;
      part_tot[g * E + e] = pt;
    }
  }
  __syncthreads();
  int before = 0, tot = 0;
  if (tid < E) {
    for (int g = 0; g < G; ++g) {
      before += part_before[g * E + tid];
      tot += part_tot[g * E + tid];
    }
  }
  // Inclusive scan of the totals over the experts: a shuffle scan within each
  // wave's 64 experts, then the totals of the lower waves.
  int incl = (tid < E) ? tot : 0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wave_tot[w];
  if (tid < kMaxExperts) scan[tid] = incl;
  if (tid < E) {
    const int excl = scan[tid] - tot;
    offs[tid] = excl;
    if (tid == E - 1) offs[E] = scan[tid];
    if (b == 0) {
      counts[tid] = tot;
      offsets[tid] = excl;
      if (tid == E - 1) offsets[E] = scan[tid];
    }
  }
  __syncthreads();
  if (b == 0 && tid < ep) {
    const int El = E / ep;
    splits[tid] = offs[(tid + 1) * El] - offs[tid * El];
  }
  // Each wave's first row per expert: offset + earlier blocks + lower waves.
  if (tid < E) {
    int run = offs[tid] + before;
    for (int w = 0; w < kWaves; ++w) {
      const int c = next[w][tid];
      next[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  // Pass 2: stable placement.
  for (int s0 = 0; s0 < steps; s0 += kStepBatch) {
    int eid[kStepBatch];
#pragma unroll
    for (int q = 0; q < kStepBatch; ++q) {
      const int f = wbase + (s0 + q) * 64 + lane;
      eid[q] = (s0 + q < steps && f < total) ? ids[f] : -1;
    }
#pragma unroll
    for (int q = 0; q < kStepBatch; ++q) {
      const int f = wbase + (s0 + q) * 64 + lane;
      const int e = eid[q];
      const bool valid = (unsigned)e < (unsigned)E;
      const uint64_t same = same_expert_lanes(e, valid, id_bits);
      const int rank = __popcll(same & below);
      int pos = 0;
      if (valid) pos = next[wave][e] + rank;
      wave_sync_lds();
      if (valid) {
        perm[pos] = f;
        inv[f] = pos;
        if (rank == 0) next[wave][e] = pos + __popcll(same);
      }
      wave_sync_lds();
    }
  }
}

// Up to kSingleMaxPairs pairs: one workgroup of 16 waves stages the ids in
// LDS (one round trip to memory) and places them (place_pairs).
constexpr int kSingleWaves = 16;
// Up to here one workgroup beats the count + place launches (4 steps per
// wave; at 32768 pairs the walks take about 37 us against 14 us for them).
constexpr int kSingleMaxPairs = 4096;

__global__ __launch_bounds__(64 * kSingleWaves) void permute_single_kernel(const int32_t* __restrict__ ids, int total,
                                                                         int E, int ep, int id_bits,
                                                                         int32_t* __restrict__ counts,
                                                                         int32_t* __restrict__ offsets,
                                                                         int32_t* __restrict__ splits,
                                                                         int32_t* __restrict__ perm,
                                                                         int32_t* __restrict__ inv) {
  __shared__ __attribute__((aligned(16))) int sid[kSingleMaxPairs];
  __shared__ int cnt[kSingleWaves][kMaxExperts];
  __shared__ int offs[kMaxExperts + 1];
  const int tid = threadIdx.x;
  // Stage the ids: 16-byte pieces where the source is aligned, the rest one by one.
  const int vec = ((uintptr_t)ids % 16 == 0) ? total / 4 : 0;
  {
    constexpr int kPer = (kSingleMaxPairs / 4 + 64 * kSingleWaves - 1) / (64 * kSingleWaves);  // pieces per thread
    u32x4_t v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int c = tid + q * 64 * kSingleWaves;
      v[q] = (c < vec) ? ((const u32x4_t*)ids)[c] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int c = tid + q * 64 * kSingleWaves;
      if (c < vec) *(u32x4_t*)&sid[4 * c] = v[q];
    }
    for (int f = 4 * vec + tid; f < total; f += 64 * kSingleWaves) sid[f] = ids[f];
  }
  place_pairs<kSingleWaves>(sid, total, E, ep, id_bits, cnt, offs, nullptr,
                            PlaceOut{true, counts, offsets, splits, perm, inv});
}

// No pairs: counts, offsets and splits are all zero.
__global__ __launch_bounds__(kMaxExperts) void permute_empty_kernel(int E, int ep, int32_t* __restrict__ counts,
                                                                    int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ splits) {
  const int t = threadIdx.x;
  if (t < E) counts[t] = 0;
  if (t < E) offsets[t] = 0;
  if (t == 0) offsets[E] = 0;
  if (t < ep) splits[t] = 0;
}

// x_perm[p] = x[perm[p] / K]: one wave per row, 16-byte vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ x, int row_vecs,
                                                          const int32_t* __restrict__ perm, int K, int total,
                                                          char* __restrict__ x_perm) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= total) return;
  const int f = perm[p];
  if ((unsigned)f >= (unsigned)total) return;
  const u32x4_t* src = (const u32x4_t*)x + (size_t)(f / K) * row_vecs;
  u32x4_t* dst = (u32x4_t*)x_perm + (size_t)p * row_vecs;
  // Four 16-byte loads in flight per lane, then their stores.
  int c = lane;
  for (; c + 192 < row_vecs; c += 256) {
    const u32x4_t v0 = src[c], v1 = src[c + 64], v2 = src[c + 128], v3 = src[c + 192];
    dst[c] = v0;
    dst[c + 64] = v1;
    dst[c + 128] = v2;
    dst[c + 192] = v3;
  }
  for (; c < row_vecs; c += 64) dst[c] = src[c];
}

}  // namespace

hipError_t launch_gather_rows(const void* x, const int32_t* perm, int n, int H, int K, moe_dtype dt, void* x_perm,
                              hipStream_t s) {
  const int total = n * K;
  if (total == 0) return hipSuccess;
  const int row_vecs = H * (dt == MOE_BF16 ? 2 : 4) / 16;
  gather_rows_kernel<<<ceil_div(total, 4), 256, 0, s>>>((const char*)x, row_vecs, perm, K, total, (char*)x_perm);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* topk_ids, const void* x, int n, int H, int E, int K, int ep,
                          moe_dtype dt, int32_t* counts, int32_t* offsets, int32_t* splits, int32_t* perm,
                          int32_t* inv, void* x_perm, int32_t* block_counts, hipStream_t s) {
  const int total = n * K;
  const int P = pairs_per_block(total);
  const int nblk = total > 0 ? ceil_div(total, P) : 0;
  int id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  if (total > 0 && total <= kSingleMaxPairs) {
    permute_single_kernel<<<1, 64 * kSingleWaves, 0, s>>>(topk_ids, total, E, ep, id_bits, counts, offsets, splits,
                                                          perm, inv);
  } else if (total > 0) {
    permute_count_kernel<<<nblk, kPermThreads, 0, s>>>(topk_ids, total, E, P, block_counts);
    permute_place_kernel<<<nblk, kPermThreads, 0, s>>>(topk_ids, total, E, ep, P, nblk, id_bits, block_counts,
                                                       counts, offsets, splits, perm, inv);
  } else {
    permute_empty_kernel<<<1, kMaxExperts, 0, s>>>(E, ep, counts, offsets, splits);
  }
  if (x != nullptr && total > 0) {
    const int elt = (dt == MOE_BF16) ? 2 : 4;
    const int row_vecs = H * elt / 16;
    gather_rows_kernel<<<ceil_div(total, 4), 256, 0, s>>>((const char*)x, row_vecs, perm, K, total,
                                                          (char*)x_perm);
  }
  return hipGetLastError();
}

}  // namespace moe
