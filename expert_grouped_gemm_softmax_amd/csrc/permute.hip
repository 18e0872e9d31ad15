// Local-pair filter and expert-contiguous permutation for gfx950.
//
// "Systems engineering playbook: optimizing Qwen 3.5-397B MoE on Ironwood (TPU7x)", section 3
// (option B): each device keeps only the token-expert pairs routed to its own experts.  They are
// grouped by expert with a stable counting sort: histogram, exclusive prefix scan, scatter.
//
// Up to kSmallPairs pairs: one launch, one workgroup of 16 wavefronts (k_perm_small).  With at
// most 64 local experts and 2048 tokens it ranks pairs with an LDS bit per (expert, token) (see
// the kernel); otherwise it counts per wavefront in LDS, scans over experts, recounts and writes.
// Larger inputs: two launches over chunks
// of kChunk consecutive pairs (one workgroup of 4 wavefronts per chunk, 128 pairs per wavefront):
//   k_perm_count    per-chunk histogram of local expert ids -> workspace counts[chunk][e];
//   k_perm_scatter  every workgroup sums the counts of the chunks before it (its row base per
//                   expert) and of all chunks (the group offsets), recounts its own chunk per
//                   wavefront, and writes each local pair to its row.
// Inside a 64-pair step, lanes carrying the same local expert are found with one ballot per bit
// of the local id (a match-any built from ballots); the lowest such lane updates the wavefront's
// LDS counter for that expert.  Stable order = (chunk, wavefront, step, lane) = ascending pair
// index.  The only atomics are the token-bit path's OR into LDS, whose result does not depend on
// their order, so every output is deterministic.
#include "common.h"

namespace moe {
namespace {

constexpr int kWavesPerChunk = 4;
constexpr int kSteps = 2;                                  // 64-pair steps per wavefront
constexpr int kWavePairs = 64 * kSteps;
constexpr int kChunk = kWavesPerChunk * kWavePairs;        // 512 pairs per workgroup
constexpr int kSmallWaves = 16;                            // single-workgroup path
constexpr int kSmallSteps = 16;                            // 64-pair steps per wavefront at most
constexpr int kSmallPairs = kSmallWaves * kSmallSteps * 64;   // 16384
constexpr int kBitsMaxExperts = 64;                       // token-bit path: one lane per expert
constexpr int kBitsMaxWords = 64;                         // and at most 2048 tokens

__device__ __forceinline__ uint64_t match_local(int le, bool valid, int nbits) {
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (le >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    same &= bit ? bb : ~bb;
  }
  return same;
}

// Inclusive prefix sum over the 64 lanes of a wavefront: four row shifts inside each 16-lane row,
// then the row broadcasts of lanes 15 and 31 (lanes whose DPP source is outside the row or whose
// row is masked off add 0).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
  return x;
}

// Local expert id of pair p (-1 outside [0, e_local) or p >= end).
__device__ __forceinline__ int local_id(const int32_t* __restrict__ blob, int p, int end, int e_first, int e_local) {
  const int id = (p < end) ? blob[min(p, end - 1)] : e_first - 1;
  return (id >= e_first && id - e_first < e_local) ? id - e_first : -1;
}

// Local expert ids of this wavefront's pairs (-1 outside [0, e_local) or past the end).
__device__ __forceinline__ void load_local_ids(const int32_t* __restrict__ blob, int beg, int end, int e_first,
                                               int e_local, int lane, int (&le)[kSteps]) {
#pragma unroll
  for (int u = 0; u < kSteps; ++u) le[u] = local_id(blob, beg + 64 * u + lane, end, e_first, e_local);
}

// Counts of this wavefront's pairs per local expert, accumulated into mine[0..e_local).
__device__ __forceinline__ void count_wave(const int (&le)[kSteps], int nbits, int lane, int32_t* mine) {
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    const bool valid = le[u] >= 0;
    const uint64_t same = match_local(le[u], valid, nbits);
    if (valid && lane == __ffsll((unsigned long long)same) - 1) mine[le[u]] += __popcll(same);
  }
}

__global__ __launch_bounds__(256) void k_perm_count(const int32_t* __restrict__ blob, int P, int e_first,
                                                    int e_local, int nbits, int32_t* __restrict__ counts) {
  extern __shared__ int32_t lds[];                         // [4][e_local]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int beg = blockIdx.x * kChunk + wv * kWavePairs;
  int le[kSteps];
  load_local_ids(blob, beg, min(P, beg + kWavePairs), e_first, e_local, lane, le);
  for (int i = threadIdx.x; i < kWavesPerChunk * e_local; i += blockDim.x) lds[i] = 0;
  __syncthreads();
  count_wave(le, nbits, lane, lds + wv * e_local);
  __syncthreads();
  for (int e = threadIdx.x; e < e_local; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerChunk; ++w) c += lds[w * e_local + e];
    counts[(size_t)blockIdx.x * e_local + e] = c;
  }
}

// all_in_lds: the counts of every chunk fit in LDS (loaded with independent, coalesced loads);
// otherwise each thread walks the chunks of its experts in global memory.
template <bool ALL_IN_LDS>
__global__ __launch_bounds__(256) void k_perm_scatter(const int32_t* __restrict__ blob, int P, int e_first,
                                                      int e_local, int nbits, int nchunks,
                                                      const int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ sorted_pairs,
                                                      int32_t* __restrict__ group_offsets,
                                                      int32_t* __restrict__ pair_pos) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;                                      // [4][e_local] wave counts -> row bases
  int32_t* base = lds + kWavesPerChunk * e_local;          // [e_local] chunk base per expert
  int32_t* wsum = base + e_local;                          // [4]
  int32_t* allc = wsum + kWavesPerChunk;                   // [nchunks][e_local] when ALL_IN_LDS
  int32_t* pbef = allc + (size_t)nchunks * e_local;        // [parts][e_local] when ALL_IN_LDS
  const int parts = ALL_IN_LDS ? max(1, (int)blockDim.x / e_local) : 1;
  int32_t* ptot = pbef + parts * e_local;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int chunk = blockIdx.x;
  const int beg = chunk * kChunk + wv * kWavePairs;
  const int end = min(P, beg + kWavePairs);

  // One round trip: this wavefront's ids and (when they fit) every chunk's counts.
  int le[kSteps];
  load_local_ids(blob, beg, end, e_first, e_local, lane, le);
  if constexpr (ALL_IN_LDS) {
    // 16-byte loads, eight in flight per thread (the host checks the workspace is 16-byte
    // aligned; a tail of fewer than four counts is copied one by one)
    const int n = nchunks * e_local, n4 = n / 4;
    const int4* c4 = reinterpret_cast<const int4*>(counts);
    for (int i0 = threadIdx.x; i0 < n4; i0 += 8 * blockDim.x) {
      int4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * blockDim.x;
        v[u] = c4[min(i, n4 - 1)];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * blockDim.x;
        if (i < n4) {
          allc[4 * i] = v[u].x; allc[4 * i + 1] = v[u].y; allc[4 * i + 2] = v[u].z; allc[4 * i + 3] = v[u].w;
        }
      }
    }
    for (int i = 4 * n4 + threadIdx.x; i < n; i += blockDim.x) allc[i] = counts[i];
  }
  for (int i = threadIdx.x; i < kWavesPerChunk * e_local; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  count_wave(le, nbits, lane, cnt + wv * e_local);
  if constexpr (ALL_IN_LDS) {
    // thread (part, e) sums chunks [part, part+1) * nchunks / parts of expert e
    for (int i = threadIdx.x; i < parts * e_local; i += blockDim.x) {
      const int part = i / e_local, e = i % e_local;
      int bsum = 0, tsum = 0;
      for (int c = part * nchunks / parts; c < (part + 1) * nchunks / parts; ++c) {
        const int v = allc[c * e_local + e];
        bsum += (c < chunk) ? v : 0;
        tsum += v;
      }
      pbef[i] = bsum;
      ptot[i] = tsum;
    }
    __syncthreads();
  }

  // Per expert: pairs in earlier chunks and in all chunks; then the offsets (scan over experts).
  int carry = 0;
  for (int c0 = 0; c0 < e_local; c0 += blockDim.x) {
    const int e = c0 + threadIdx.x;
    int before = 0, total = 0;
    if (e < e_local) {
      if constexpr (ALL_IN_LDS) {
        for (int part = 0; part < parts; ++part) {
          before += pbef[part * e_local + e];
          total += ptot[part * e_local + e];
        }
      } else {
        int c = 0;
        for (; c + 8 <= nchunks; c += 8) {
          int v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = counts[(size_t)(c + u) * e_local + e];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            before += (c + u < chunk) ? v[u] : 0;
            total += v[u];
          }
        }
        for (; c < nchunks; ++c) {
          const int v = counts[(size_t)c * e_local + e];
          before += (c < chunk) ? v : 0;
          total += v;
        }
      }
    }
    const int incl = wave_incl_scan(total);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int wave_base = 0;
    for (int w = 0; w < wv; ++w) wave_base += wsum[w];
    const int chunk_total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (e < e_local) {
      const int off = carry + wave_base + incl - total;
      if (chunk == 0) group_offsets[e] = off;
      base[e] = off + before;
    }
    carry += chunk_total;
    __syncthreads();                                       // wsum reused by the next chunk of experts
  }
  if (chunk == 0 && threadIdx.x == 0) group_offsets[e_local] = carry;

  // Row base of each wavefront: chunk base plus the counts of the earlier wavefronts.
  for (int e = threadIdx.x; e < e_local; e += blockDim.x) {
    int run = base[e];
#pragma unroll
    for (int w = 0; w < kWavesPerChunk; ++w) {
      const int c = cnt[w * e_local + e];
      cnt[w * e_local + e] = run;
      run += c;
    }
  }
  __syncthreads();

  int32_t* mine = cnt + wv * e_local;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    const int p = beg + 64 * u + lane;
    const bool valid = le[u] >= 0;
    const uint64_t same = match_local(le[u], valid, nbits);
    int row = -1;
    if (valid) row = mine[le[u]] + __popcll(same & below);
    if (valid && lane == __ffsll((unsigned long long)same) - 1) mine[le[u]] += __popcll(same);
    if (p < end) {
      pair_pos[p] = row;
      if (valid) sorted_pairs[row] = p;
    }
  }
}

// Whole permutation in one workgroup of kSmallWaves wavefronts; wavefront w owns the consecutive
// pairs [w * span, (w + 1) * span), span a multiple of 64.
//
// Token-bit path (words > 0: at most 64 local experts and 32 * words >= T tokens): bit t of row e
// of an LDS bit matrix is set when token t has a pair routed to local expert e.  When no token
// routes two of its pairs to one expert (the bit was never set twice), the rank of pair (t, e)
// inside group e is the number of bits of row e below t: one wavefront turns the rows into
// per-word prefix counts and the group offsets (one lane per expert), and every pair then finds
// its row with three LDS reads.  Stable order within a group is ascending token, which is
// ascending pair index.
//
// Otherwise (or if some token repeats an expert): pass 1 counts per wavefront with the match-any
// ballots, the offsets and per-wavefront row bases come from one scan over the experts, pass 2
// recounts in the same order and writes the rows.
__global__ __launch_bounds__(64 * kSmallWaves) void k_perm_small(const int32_t* __restrict__ blob, int P, int k,
                                                                 int e_first, int e_local, int nbits, int span,
                                                                 int words, int32_t* __restrict__ sorted_pairs,
                                                                 int32_t* __restrict__ group_offsets,
                                                                 int32_t* __restrict__ pair_pos) {
  extern __shared__ int32_t lds[];                         // [kSmallWaves][e_local] counts -> row bases
  int32_t* wsum = lds + kSmallWaves * e_local;             // [kSmallWaves]
  uint32_t* bits = reinterpret_cast<uint32_t*>(wsum + kSmallWaves);   // [words][64]
  int32_t* pre = reinterpret_cast<int32_t*>(bits + words * 64);       // [words][64] bits of row e below word w
  int32_t* goff = pre + words * 64;                        // [64] group offsets
  int32_t* repeat = goff + 64;                             // [1] some token repeats an expert
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int beg = wv * span, end = min(P, beg + span);
  // all of this wavefront's ids in registers, loaded at once (span <= 64 * kSmallSteps)
  int le[kSmallSteps];
#pragma unroll
  for (int u = 0; u < kSmallSteps; ++u) le[u] = local_id(blob, beg + 64 * u + lane, end, e_first, e_local);
  for (int i = threadIdx.x; i < kSmallWaves * e_local; i += blockDim.x) lds[i] = 0;
  for (int i = threadIdx.x; i < words * 64; i += blockDim.x) bits[i] = 0u;
  if (threadIdx.x == 0) *repeat = 0;
  __syncthreads();

  if (words > 0) {
    bool rep = false;
#pragma unroll
    for (int u = 0; u < kSmallSteps; ++u) {
      if (beg + 64 * u >= end) break;                      // wavefront-uniform
      if (le[u] >= 0) {
        const uint32_t t = (uint32_t)(beg + 64 * u + lane) / (uint32_t)k;
        const uint32_t bit = 1u << (t & 31);
        rep |= (atomicOr(&bits[(t >> 5) * 64 + le[u]], bit) & bit) != 0u;
      }
    }
    if (rep) *repeat = 1;
    __syncthreads();
    if (*repeat == 0) {                                    // workgroup-uniform
      if (wv == 0) {                                       // lane e: row e of the bit matrix
        int run = 0;
        for (int w0 = 0; w0 < words; w0 += 8) {
          uint32_t v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = bits[min(w0 + j, words - 1) * 64 + lane];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (w0 + j < words) {
              pre[(w0 + j) * 64 + lane] = run;
              run += __popc(v[j]);
            }
        }
        const int incl = wave_incl_scan(run);             // lanes >= e_local have run = 0
        goff[lane] = incl - run;
        if (lane < e_local) group_offsets[lane] = incl - run;
        if (lane == 63) group_offsets[e_local] = incl;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kSmallSteps; ++u) {
        if (beg + 64 * u >= end) break;                    // wavefront-uniform
        const int p = beg + 64 * u + lane;
        int row = -1;
        if (le[u] >= 0) {
          const uint32_t t = (uint32_t)p / (uint32_t)k;
          const int cell = (int)(t >> 5) * 64 + le[u];
          row = goff[le[u]] + pre[cell] + __popc(bits[cell] & ((1u << (t & 31)) - 1u));
          sorted_pairs[row] = p;
        }
        if (p < end) pair_pos[p] = row;
      }
      return;
    }
  }

  int32_t* mine = lds + wv * e_local;
#pragma unroll
  for (int u = 0; u < kSmallSteps; ++u) {
    if (beg + 64 * u >= end) break;                        // wavefront-uniform
    const uint64_t same = match_local(le[u], le[u] >= 0, nbits);
    if (le[u] >= 0 && lane == __ffsll((unsigned long long)same) - 1) mine[le[u]] += __popcll(same);
  }
  __syncthreads();

  // experts in blocks of blockDim.x: totals, exclusive scan, per-wavefront bases
  int carry = 0;
  for (int c0 = 0; c0 < e_local; c0 += blockDim.x) {
    const int e = c0 + threadIdx.x;
    int total = 0;
    if (e < e_local)
      for (int w = 0; w < kSmallWaves; ++w) total += lds[w * e_local + e];
    const int incl = wave_incl_scan(total);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int wave_base = 0, block_total = 0;
    for (int w = 0; w < kSmallWaves; ++w) {
      wave_base += (w < wv) ? wsum[w] : 0;
      block_total += wsum[w];
    }
    if (e < e_local) {
      int run = carry + wave_base + incl - total;
      group_offsets[e] = run;
      for (int w = 0; w < kSmallWaves; ++w) {
        const int c = lds[w * e_local + e];
        lds[w * e_local + e] = run;
        run += c;
      }
    }
    carry += block_total;
    __syncthreads();                                       // wsum reused by the next block
  }
  if (threadIdx.x == 0) group_offsets[e_local] = carry;

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int u = 0; u < kSmallSteps; ++u) {
    if (beg + 64 * u >= end) break;                        // wavefront-uniform
    const int p = beg + 64 * u + lane;
    const uint64_t same = match_local(le[u], le[u] >= 0, nbits);
    int row = -1;
    if (le[u] >= 0) row = mine[le[u]] + __popcll(same & below);
    if (le[u] >= 0 && lane == __ffsll((unsigned long long)same) - 1) mine[le[u]] += __popcll(same);
    if (p < end) {
      pair_pos[p] = row;
      if (le[u] >= 0) sorted_pairs[row] = p;
    }
  }
}

}  // namespace

size_t permute_workspace_bytes(int T, int k, int e_local) {
  const long long P = (long long)T * k;
  if (P <= kSmallPairs) return 0;
  const long long nchunks = (P + kChunk - 1) / kChunk;
  return (size_t)(nchunks * e_local * (long long)sizeof(int32_t));
}

hipError_t launch_permute(const int32_t* blob, int T, int k, int e_first, int e_local,
                          int32_t* sorted_pairs, int32_t* group_offsets, int32_t* pair_pos,
                          void* workspace, hipStream_t s) {
  const int P = T * k;
  const int nchunks = (P + kChunk - 1) / kChunk;
  int nbits = 1;
  while ((1 << nbits) < e_local) ++nbits;
  if (P <= kSmallPairs) {
    const int span = ((P + kSmallWaves - 1) / kSmallWaves + 63) / 64 * 64;
    const int words = (e_local <= kBitsMaxExperts && T <= 32 * kBitsMaxWords) ? (T + 31) / 32 : 0;
    const size_t lds = sizeof(int32_t) * ((size_t)kSmallWaves * e_local + kSmallWaves + 2 * 64 * (size_t)words + 65);
    k_perm_small<<<dim3(1), dim3(64 * kSmallWaves), lds, s>>>(blob, P, k, e_first, e_local, nbits, span, words,
                                                              sorted_pairs, group_offsets, pair_pos);
    return hipGetLastError();
  }
  int32_t* counts = static_cast<int32_t*>(workspace);
  const size_t lds_count = sizeof(int32_t) * kWavesPerChunk * e_local;
  k_perm_count<<<dim3(nchunks), dim3(256), lds_count, s>>>(blob, P, e_first, e_local, nbits, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds_scatter = sizeof(int32_t) * ((kWavesPerChunk + 1) * e_local + kWavesPerChunk);
  const size_t lds_all = sizeof(int32_t) * ((size_t)nchunks * e_local + 2 * (size_t)max(256, e_local));
  if (lds_scatter + lds_all <= 96 * 1024)
    k_perm_scatter<true><<<dim3(nchunks), dim3(256), lds_scatter + lds_all, s>>>(
        blob, P, e_first, e_local, nbits, nchunks, counts, sorted_pairs, group_offsets, pair_pos);
  else
    k_perm_scatter<false><<<dim3(nchunks), dim3(256), lds_scatter, s>>>(
        blob, P, e_first, e_local, nbits, nchunks, counts, sorted_pairs, group_offsets, pair_pos);
  return hipGetLastError();
}

}  // namespace moe
