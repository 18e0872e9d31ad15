// Softmax top-k routing and routing-blob packing for gfx950.
//
// Routing follows "Systems engineering playbook: optimizing Qwen 3.5-397B MoE on Ironwood
// (TPU7x)", section 1 (sparse MoE: softmax over the experts, top-k selected), with the
// renormalised weight sequence stated in moe.h.  The blob layout follows section 3 (3-to-2
// all-gather: ids and weight bits stacked on a new leading axis in one int32 array).
//
// One 64-lane wavefront owns one token: lane l holds logits l, l+64, l+128, ... in registers as
// order-mapped value bits with their ids, sorted once per lane; each of the k rounds is a 6-step
// DPP max of the lane heads' value bits (4 steps inside each 16-lane row, 2 row broadcasts) read
// from lane 63, a ballot of the heads holding that value, and (only when several do) a second
// max over their ids.  The weights need no E-term reduction: slot j's weight only involves the
// k selected logits.
#include "common.h"

namespace moe {
namespace {

// e^d for d <= 0 from correctly rounded fp32 operations: multiply, rint, fma, and an exact
// scaling by 2^n.  Steps and constants as declared for moe_route in moe.h.
__device__ __forceinline__ float exp_neg(float d) {
#pragma clang fp contract(off)
  constexpr double kLn2 = 0.693147180559945309417232121458176568;
  constexpr float kLog2e = (float)(1.0 / kLn2);
  constexpr float kLn2Hi = (float)kLn2;
  constexpr float kLn2Lo = (float)(kLn2 - (double)kLn2Hi);
  constexpr float kC2 = (float)(1.0 / 2.0), kC3 = (float)(1.0 / 6.0), kC4 = (float)(1.0 / 24.0);
  constexpr float kC5 = (float)(1.0 / 120.0), kC6 = (float)(1.0 / 720.0);
  constexpr float kC7 = (float)(1.0 / 5040.0);
  if (d < -86.0f) return 0.0f;
  const float n = __builtin_rintf(d * kLog2e);            // in [-124, 0]
  float r = __builtin_fmaf(-n, kLn2Hi, d);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = kC7;
  p = __builtin_fmaf(p, r, kC6);
  p = __builtin_fmaf(p, r, kC5);
  p = __builtin_fmaf(p, r, kC4);
  p = __builtin_fmaf(p, r, kC3);
  p = __builtin_fmaf(p, r, kC2);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  const float two_n = __uint_as_float((uint32_t)((int)n + 127) << 23);  // 2^n, a normal number
  return p * two_n;                                        // exact: the product stays normal
}

// Selection order of (logit v, expert id): larger value first, then lower id.  A logit is held as
// its fp32 bits mapped to an unsigned order (-0 folded onto +0) and its id as ~id, so "selected
// first" is the larger (bits, ~id) pair.  Bits 0 mark an empty slot (every finite logit maps
// above it).
__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;                            // -0 equals +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_value(uint32_t b) {
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}

// DPP controls (gfx9 encoding): quad permutations, reverse within 8 lanes, reverse within 16,
// and the wave64 row broadcasts of lane 15 (to the next row) and lane 31 (to rows 2 and 3).
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// max(x, x of the DPP source lane); lanes outside ROW_MASK keep x (their DPP result is 0).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_max(uint32_t x) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, false);
  return o > x ? o : x;
}

// Largest x over the wavefront (all 64 lanes active), wave-uniform: the maximum of each 16-lane
// row in four steps, then rows 1 and 3 take rows 0 and 2, row 3 takes row 1; lane 63 holds it.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = dpp_max<kQuadXor1>(x);
  x = dpp_max<kQuadXor2>(x);
  x = dpp_max<kRowHalfMirror>(x);
  x = dpp_max<kRowMirror>(x);
  x = dpp_max<kRowBcast15, 0xa>(x);
  x = dpp_max<kRowBcast31, 0xc>(x);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// ids / w / blob: outputs (a NULL pointer is not written; ids and w are NULL together).
template <int PER_LANE>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ w,
                                               int32_t* __restrict__ blob) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                     // uniform per wave
  const float* row = logits + (size_t)t * E;
  // Lane l owns experts l, l+64, ...: value bits vb and ~id ib, sorted once (descending value;
  // insertion sort with strict comparisons is stable, so equal values keep ascending id), so each
  // round only compares the heads of the 64 lists and the winning lane drops its head.  Loads are
  // unconditional (clamped index): none waits behind a branch.
  uint32_t vb[PER_LANE], ib[PER_LANE];
  float x[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) x[i] = __builtin_nontemporal_load(row + min(lane + 64 * i, E - 1));
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    vb[i] = (e < E) ? order_bits(x[i]) : 0u;
    ib[i] = ~(uint32_t)e;
  }
#pragma unroll
  for (int i = 1; i < PER_LANE; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = vb[j] > vb[j - 1];
      const uint32_t v0 = vb[j - 1], v1 = vb[j], i0 = ib[j - 1], i1 = ib[j];
      vb[j - 1] = sw ? v1 : v0;
      vb[j] = sw ? v0 : v1;
      ib[j - 1] = sw ? i1 : i0;
      ib[j] = sw ? i0 : i1;
    }
  uint32_t sel_v = 0, sel_i = 0;                          // slot `lane` (lanes < k)
  for (int j = 0; j < k; ++j) {
    const uint32_t best_v = wave_max(vb[0]);
    const uint64_t tied = __ballot(vb[0] == best_v);
    int win;
    if (__popcll(tied) == 1) {
      win = __ffsll((unsigned long long)tied) - 1;
    } else {                                              // equal values at several heads: lowest id
      const uint32_t best_i = wave_max(vb[0] == best_v ? ib[0] : 0u);
      win = __ffsll((unsigned long long)__ballot(vb[0] == best_v && ib[0] == best_i)) - 1;
    }
    const uint32_t best_i = (uint32_t)__builtin_amdgcn_readlane((int)ib[0], win);
    if (lane == win) {                                     // the winner's list advances
#pragma unroll
      for (int i = 0; i + 1 < PER_LANE; ++i) {
        vb[i] = vb[i + 1];
        ib[i] = ib[i + 1];
      }
      vb[PER_LANE - 1] = 0u;
    }
    if (lane == j) {
      sel_v = best_v;
      sel_i = best_i;
    }
  }
  const float sel_x = order_value(sel_v);
  const int sel_id = (int)~sel_i;
  const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_x), 0));
  const float e = (lane < k) ? exp_neg(sel_x - m) : 0.0f;
  float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), 0));
  for (int j = 1; j < k; ++j) s = s + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), j));
  if (lane < k) {
    const float wt = e / s;                              // correctly rounded division
    const size_t q = (size_t)t * k + lane;
    if (ids) {
      ids[q] = sel_id;
      w[q] = wt;
    }
    if (blob) {                                          // the packed form: ids, then weight bits
      blob[q] = sel_id;
      blob[(size_t)T * k + q] = __float_as_int(wt);
    }
  }
}

__global__ __launch_bounds__(256) void k_pack(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                              int64_t P, int32_t* __restrict__ blob) {
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < P;
       p += (int64_t)gridDim.x * blockDim.x) {
    blob[p] = ids[p];
    blob[P + p] = __float_as_int(w[p]);
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* blob,
                        hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64) k_route<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, blob);
  else if (E <= 128) k_route<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, blob);
  else if (E <= 256) k_route<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, blob);
  else if (E <= 512) k_route<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, blob);
  else k_route<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w, blob);
  return hipGetLastError();
}

hipError_t launch_pack(const int32_t* ids, const float* w, int T, int k, int32_t* blob, hipStream_t s) {
  const int64_t P = (int64_t)T * k;
  int64_t blocks = (P + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_pack<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(ids, w, P, blob);
  return hipGetLastError();
}

}  // namespace moe
