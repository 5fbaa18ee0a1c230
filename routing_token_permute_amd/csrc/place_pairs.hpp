// Stable expert-major placement of the (token, slot) pairs by one workgroup,
// the ids already staged in LDS: the per-expert counts n_e, the exclusive
// offsets, the per-rank splits and the permutation with its inverse.
//
// What is computed: the sets I_e of Algorithm 2 ("MoE 分布式推理基础（基于
// vLLM）" §1.2) in ascending flat order, laid out expert-major as in that
// page's moe_align_block_size example (§2.3) without padding, and the send
// sizes of its Algorithm 5 step 3 (§2.4).
//
// How: wave w owns pairs [w * chunk, (w + 1) * chunk) in 64-pair steps. Pass
// 1 counts them per (wave, expert): the first lane of each group of
// same-expert lanes (found with ballots over the id bits) adds the group's
// size with an LDS atomic. Wave 0 then sums the waves, scans over the experts
// and derives each wave's first row per expert. Pass 2 repeats the walk: the
// group leader reserves its group's rows with an atomic add that returns the
// old count, and every lane places its pair at the leader's old count + its
// rank among the lower lanes of its group. Each wave's adds to one counter run
// in program order, so pairs keep ascending flat order inside every expert
// segment, whatever the number of waves. Pairs whose id is outside [0, E) are
// neither counted nor placed (their inverse entry is not written).
#pragma once

#include "moe_internal.hpp"

namespace moe {

// Lanes of this wave whose expert id equals this lane's (ballots over the id
// bits); `valid` lanes only match valid lanes.
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool valid, int id_bits) {
  uint64_t same = __ballot(valid);
  for (int b = 0; b < id_bits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  return same;
}

// Where place_pairs writes. The global outputs are written only when `global`
// is set; perm_lds (LDS, `total` entries) and offs (LDS, E + 1 entries) are
// always written when given.
struct PlaceOut {
  bool global;
  int32_t* counts;   // (E)
  int32_t* offsets;  // (E + 1)
  int32_t* splits;   // (ep)
  int32_t* perm;     // (total)
  int32_t* inv;      // (total)
};

// A GEMM that places the routing ids itself (decode-sized batches): at most
// this many (token, slot) pairs, staged in LDS.
constexpr int kIdsMaxPairs = 1024;

// Such a GEMM's ids, and where its workgroup 0 writes the dispatch metadata
// (counts, offsets, splits, perm, inv) for the kernels that follow.
struct IdsMeta {
  const int32_t* ids;
  int32_t* counts;
  int32_t* offsets;
  int32_t* splits;
  int32_t* perm;
  int32_t* inv;
  int ep, id_bits;
};

// NW waves of the calling workgroup run this together; every thread of the
// workgroup must call it (it contains barriers). sid: the `total` ids in LDS.
// cnt: an LDS array of NW x kMaxExperts counters. offs: an LDS array of
// kMaxExperts + 1 entries, holding the exclusive offsets on return. E <=
// kMaxExperts; ep divides E.
template <int NW>
__device__ __forceinline__ void place_pairs(const int* sid, int total, int E, int ep, int id_bits,
                                            int (*cnt)[kMaxExperts], int* offs, int* perm_lds,
                                            const PlaceOut& out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < NW * kMaxExperts; i += 64 * NW) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int chunk = ((total + NW * 64 - 1) / (NW * 64)) * 64;
  const int f0 = wave * chunk, f1 = min(total, f0 + chunk);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // Pass 1: counts per (wave, expert).
#pragma unroll 4
  for (int base = f0; base < f1; base += 64) {
    const int f = base + lane;
    const int e = (f < f1) ? sid[f] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    const uint64_t same = same_expert_lanes(e, valid, id_bits);
    if (valid && (same & below) == 0) atomicAdd(&cnt[wave][e], (int)__popcll(same));
  }
  __syncthreads();
  // Totals, exclusive offsets (wave 0: 4 consecutive experts per lane, then a
  // shuffle scan).
  if (wave == 0) {
    int t4[4], run = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      int tt = 0;
      if (e < E)
        for (int w = 0; w < NW; ++w) tt += cnt[w][e];
      t4[j] = tt;
      run += tt;
    }
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int ex = incl - run;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      if (e < E) {
        offs[e] = ex;
        if (out.global) {
          out.counts[e] = t4[j];
          out.offsets[e] = ex;
        }
      }
      ex += t4[j];
    }
    if (lane == 63) {
      offs[E] = incl;
      if (out.global) out.offsets[E] = incl;
    }
  }
  __syncthreads();
  if (out.global && tid < ep) {
    const int El = E / ep;
    out.splits[tid] = offs[(tid + 1) * El] - offs[tid * El];
  }
  // Each wave's first row per expert: offset + the lower waves' counts.
  for (int e = tid; e < E; e += 64 * NW) {
    int run = offs[e];
    for (int w = 0; w < NW; ++w) {
      const int c = cnt[w][e];
      cnt[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  // Pass 2: stable placement.
#pragma unroll 4
  for (int base = f0; base < f1; base += 64) {
    const int f = base + lane;
    const int e = (f < f1) ? sid[f] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    const uint64_t same = same_expert_lanes(e, valid, id_bits);
    const int rank = __popcll(same & below);
    int old = 0;
    if (valid && rank == 0) old = atomicAdd(&cnt[wave][e], (int)__popcll(same));
    const int leader = valid ? (__ffsll((long long)same) - 1) : lane;
    const int pos = __shfl(old, leader) + rank;
    if (valid) {
      if (perm_lds != nullptr) perm_lds[pos] = f;
      if (out.global) {
        out.perm[pos] = f;
        out.inv[f] = pos;
      }
    }
  }
}

}  // namespace moe
