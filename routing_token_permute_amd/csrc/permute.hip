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
// How: three small kernels over blocks of 2048 pairs, then a row gather.
//   1. count:   per-block histogram in LDS (integer atomics: the result does
//               not depend on their order).
//   2. scan:    one workgroup turns the per-block histograms into counts,
//               offsets, splits and each block's starting row per expert.
//   3. place:   each wave walks its 512 pairs in 64-pair steps; lanes with
//               the same expert are found with ballots over the id bits, and
//               a lane's rank among them is a popcount of the lower lanes, so
//               pairs keep ascending flat order inside every expert segment.
//   4. gather:  one wave per destination row copies 16-byte vectors.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kPairsPerThread = kPermChunk / kPermThreads;  // 8
constexpr int kWaves = kPermThreads / 64;                   // 4
constexpr int kPairsPerWave = kPermChunk / kWaves;          // 512

__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(const int32_t* __restrict__ ids, int total,
                                                                     int E, int32_t* __restrict__ block_counts) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kPermThreads) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kPermChunk;
#pragma unroll
  for (int j = 0; j < kPairsPerThread; ++j) {
    const int f = base + j * kPermThreads + (int)threadIdx.x;
    if (f < total) {
      const int e = ids[f];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) block_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup of 256 threads (E <= 256): thread e owns expert e.
// In: block_counts[b][e]. Out: block_counts[b][e] becomes the first row of
// block b's pairs for expert e; counts, offsets, splits.
__global__ __launch_bounds__(kMaxExperts) void permute_scan_kernel(int32_t* __restrict__ block_counts, int nblk,
                                                                   int E, int ep, int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ splits) {
  __shared__ int scan[kMaxExperts];
  __shared__ int offs[kMaxExperts + 1];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    for (int b = 0; b < nblk; ++b) {
      const int c = block_counts[(size_t)b * E + e];
      block_counts[(size_t)b * E + e] = total;
      total += c;
    }
    counts[e] = total;
  }
  scan[e] = (e < E) ? total : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 256 slots.
  for (int d = 1; d < kMaxExperts; d <<= 1) {
    const int v = (e >= d) ? scan[e - d] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  const int excl = scan[e] - ((e < E) ? total : 0);
  if (e < E) {
    offs[e] = excl;
    offsets[e] = excl;
    if (e == E - 1) {
      offs[E] = scan[e];
      offsets[E] = scan[e];
    }
    for (int b = 0; b < nblk; ++b) block_counts[(size_t)b * E + e] += excl;
  }
  __syncthreads();
  if (e < ep) {
    const int El = E / ep;
    splits[e] = offs[(e + 1) * El] - offs[e * El];
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_place_kernel(const int32_t* __restrict__ ids, int total,
                                                                     int E, int id_bits,
                                                                     const int32_t* __restrict__ block_base,
                                                                     int32_t* __restrict__ perm,
                                                                     int32_t* __restrict__ inv) {
  __shared__ int next[kWaves][kMaxExperts];  // next free row per (wave, expert)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kWaves * kMaxExperts; i += kPermThreads) (&next[0][0])[i] = 0;
  __syncthreads();
  const int wbase = blockIdx.x * kPermChunk + wave * kPairsPerWave;
  // Pass 1: how many of this wave's pairs go to each expert.
  for (int s = 0; s < kPairsPerWave / 64; ++s) {
    const int f = wbase + s * 64 + lane;
    const int e = (f < total) ? ids[f] : -1;
    if ((unsigned)e < (unsigned)E) atomicAdd(&next[wave][e], 1);
  }
  __syncthreads();
  // Each wave's first row per expert: the block's first row plus the
  // pairs of the lower waves.
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    int run = block_base[(size_t)blockIdx.x * E + e];
    for (int w = 0; w < kWaves; ++w) {
      const int c = next[w][e];
      next[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  // Pass 2: place pairs in ascending flat order.
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s = 0; s < kPairsPerWave / 64; ++s) {
    const int f = wbase + s * 64 + lane;
    const int e = (f < total) ? ids[f] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & below);
    int pos = 0;
    if (valid) pos = next[wave][e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      perm[pos] = f;
      inv[f] = pos;
      if (rank == 0) next[wave][e] = pos + __popcll(same);
    }
    __builtin_amdgcn_wave_barrier();
  }
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
  for (int c = lane; c < row_vecs; c += 64) dst[c] = src[c];
}

}  // namespace

hipError_t launch_permute(const int32_t* topk_ids, const void* x, int n, int H, int E, int K, int ep,
                          moe_dtype dt, int32_t* counts, int32_t* offsets, int32_t* splits, int32_t* perm,
                          int32_t* inv, void* x_perm, int32_t* block_counts, hipStream_t s) {
  const int total = n * K;
  const int nblk = ceil_div(total, kPermChunk);
  int id_bits = 0;
  while ((1 << id_bits) < E) ++id_bits;
  if (nblk > 0) permute_count_kernel<<<nblk, kPermThreads, 0, s>>>(topk_ids, total, E, block_counts);
  permute_scan_kernel<<<1, kMaxExperts, 0, s>>>(block_counts, nblk, E, ep, counts, offsets, splits);
  if (nblk > 0)
    permute_place_kernel<<<nblk, kPermThreads, 0, s>>>(topk_ids, total, E, id_bits, block_counts, perm, inv);
  if (x != nullptr && total > 0) {
    const int elt = (dt == MOE_BF16) ? 2 : 4;
    const int row_vecs = H * elt / 16;
    gather_rows_kernel<<<ceil_div(total, 4), 256, 0, s>>>((const char*)x, row_vecs, perm, K, total,
                                                          (char*)x_perm);
  }
  return hipGetLastError();
}

}  // namespace moe
