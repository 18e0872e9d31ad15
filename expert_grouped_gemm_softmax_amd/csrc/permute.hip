// Local-pair filter and expert-contiguous permutation for gfx950.
//
// "Systems engineering playbook: optimizing Qwen 3.5-397B MoE on Ironwood (TPU7x)", section 3
// (option B): each device keeps only the token-expert pairs routed to its own experts.  They are
// grouped by expert with a stable counting sort: histogram, exclusive prefix scan, scatter.
//
// One workgroup of NW wavefronts.  Wave w owns a contiguous range of pairs (a multiple of 64), so
// the stable order inside a group is: by wave, then by 64-pair step, then by lane.  Inside a
// step, lanes carrying the same local expert are found with one ballot per bit of the local id
// (a match-any built from ballots); the lowest such lane updates the wave's LDS counter for that
// expert, so no atomics are needed and the result is deterministic.
#include "common.h"

namespace moe {
namespace {

constexpr int kUnroll = 8;

struct Match {
  uint64_t same;   // lanes holding the same valid local id as this lane
  bool valid;
};

__device__ __forceinline__ Match match_local(int le, bool valid, int nbits) {
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (le >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    same &= bit ? bb : ~bb;
  }
  return {same, valid};
}

__global__ __launch_bounds__(1024) void k_permute(const int32_t* __restrict__ blob, int P, int e_first,
                                                  int e_local, int nbits, int32_t* __restrict__ sorted_pairs,
                                                  int32_t* __restrict__ group_offsets,
                                                  int32_t* __restrict__ pair_pos) {
  extern __shared__ int32_t lds[];
  const int NW = blockDim.x >> 6;
  int32_t* cnt = lds;                         // [NW][e_local]: counts, then running row bases
  int32_t* tot = lds + NW * e_local;          // [e_local]
  int32_t* wsum = tot + e_local;              // [16]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  for (int i = threadIdx.x; i < NW * e_local; i += blockDim.x) cnt[i] = 0;
  __syncthreads();

  const int per = ((P + NW * 64 - 1) / (NW * 64)) * 64;
  const int beg = min(P, wv * per), end = min(P, beg + per);
  int32_t* mine = cnt + wv * e_local;

  // Pass 1: per-wave histogram of local ids.
  for (int base = beg; base < end; base += 64 * kUnroll) {
    int le[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + 64 * u + lane;
      le[u] = (p < end) ? blob[p] - e_first : -1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool valid = le[u] >= 0 && le[u] < e_local;
      const Match m = match_local(le[u], valid, nbits);
      if (valid && lane == __ffsll((unsigned long long)m.same) - 1) mine[le[u]] += __popcll(m.same);
    }
  }
  __syncthreads();

  // Per expert: exclusive prefix over waves, and the expert's total.
  for (int e = threadIdx.x; e < e_local; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int c = cnt[w * e_local + e];
      cnt[w * e_local + e] = run;
      run += c;
    }
    tot[e] = run;
  }
  __syncthreads();

  // Exclusive scan of the totals over experts, in chunks of blockDim.x.
  int carry = 0;
  for (int c0 = 0; c0 < e_local; c0 += blockDim.x) {
    const int e = c0 + threadIdx.x;
    const int v = (e < e_local) ? tot[e] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    if (wv == 0) {
      int s = (lane < NW) ? wsum[lane] : 0;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int o = __shfl_up(s, off);
        if (lane >= off) s += o;
      }
      if (lane < NW) wsum[lane] = s;                      // inclusive over waves
    }
    __syncthreads();
    const int wave_base = (wv == 0) ? 0 : wsum[wv - 1];
    const int chunk_total = wsum[NW - 1];
    __syncthreads();                                       // wsum reused by the next chunk
    if (e < e_local) {
      const int off = carry + wave_base + incl - v;
      group_offsets[e] = off;
      for (int w = 0; w < NW; ++w) cnt[w * e_local + e] += off;
    }
    carry += chunk_total;
  }
  if (threadIdx.x == 0) group_offsets[e_local] = carry;
  __syncthreads();

  // Pass 2: stable scatter.
  for (int base = beg; base < end; base += 64 * kUnroll) {
    int le[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + 64 * u + lane;
      le[u] = (p < end) ? blob[p] - e_first : -1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + 64 * u + lane;
      const bool valid = le[u] >= 0 && le[u] < e_local;
      const Match m = match_local(le[u], valid, nbits);
      int row = -1;
      if (valid) row = mine[le[u]] + __popcll(m.same & below);
      if (valid && lane == __ffsll((unsigned long long)m.same) - 1) mine[le[u]] += __popcll(m.same);
      if (p < end) {
        pair_pos[p] = row;
        if (valid) sorted_pairs[row] = p;
      }
    }
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* blob, int T, int k, int e_first, int e_local,
                          int32_t* sorted_pairs, int32_t* group_offsets, int32_t* pair_pos,
                          hipStream_t s) {
  const int P = T * k;
  const int NW = (e_local <= 512) ? 16 : 8;
  int nbits = 1;
  while ((1 << nbits) < e_local) ++nbits;
  const size_t lds = sizeof(int32_t) * ((size_t)NW * e_local + e_local + 16);
  k_permute<<<dim3(1), dim3(NW * 64), lds, s>>>(blob, P, e_first, e_local, nbits, sorted_pairs,
                                                group_offsets, pair_pos);
  return hipGetLastError();
}

}  // namespace moe
