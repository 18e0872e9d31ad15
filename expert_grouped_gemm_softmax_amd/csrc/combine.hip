// Weighted combine back to token order for gfx950.
//
// "Systems engineering playbook: optimizing Qwen 3.5-397B MoE on Ironwood (TPU7x)": the unpermute
// building block (executive summary) returns expert-ordered rows to token order, and the
// always-executed shared expert joins the routed output (section 1).  The sum over a token's
// slots is a gather in ascending slot order with fp32 accumulation, so the result is bitwise
// reproducible (no atomics).
//
// One workgroup per token; each lane owns 8 consecutive hidden elements (one 16-byte bf16 or two
// 16-byte fp32 accesses per row), so every gathered row is read with fully coalesced loads.  Rows
// are read once and y is written once, so both go through nontemporal accesses: the caches are
// left to the weights that the next GEMMs stream (skewed combine 335 -> 305 us; the prefill gate/up
// launch after it no longer pays for evicting y, 259 -> 241 us).
#include "common.h"

namespace moe {
namespace {

template <typename T> struct Vec8;
template <> struct Vec8<u16> {
  __device__ static void load(const u16* p, float* v) {
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  }
  __device__ static void store(u16* p, const float* v) {
    u32x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(p));
  }
};
template <> struct Vec8<_Float16> {
  // halves taken with integer shifts: hipcc (ROCm 7.2) miscompiles element reads of a 16-bit
  // vector bitcast from one dword of a 16-byte load (every element came from the same dword)
  __device__ static void load(const _Float16* p, float* v) {
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (float)__builtin_bit_cast(_Float16, (u16)(q[i] & 0xffffu));
      v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (u16)(q[i] >> 16));
    }
  }
};
template <> struct Vec8<float> {
  __device__ static void load(const float* p, float* v) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  __device__ static void store(float* p, const float* v) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(p + 4));
  }
};

template <typename TA, typename TY>
__global__ __launch_bounds__(512) void k_combine(const TA* __restrict__ o, const int32_t* __restrict__ blob,
                                                 const int32_t* __restrict__ pair_pos,
                                                 const TA* __restrict__ shared, int T, int k, int H,
                                                 int rows, TY* __restrict__ y) {
  __shared__ int s_pos[64];
  __shared__ float s_w[64];
  __shared__ int s_n;
  const int t = blockIdx.x;
  const int64_t P = (int64_t)T * k;
  if (threadIdx.x < 64) {                                // wave 0 compacts the token's valid slots in order
    const int j = threadIdx.x;
    int pos = -1;
    float wj = 0.f;
    if (j < k) {
      pos = pair_pos[(int64_t)t * k + j];
      wj = __int_as_float(blob[P + (int64_t)t * k + j]);
    }
    const bool valid = j < k && pos >= 0 && pos < rows;
    const uint64_t m = __ballot(valid);
    if (valid) {
      const int slot = __popcll(m & ((1ull << j) - 1ull));
      s_pos[slot] = pos;
      s_w[slot] = wj;
    }
    if (j == 0) s_n = __popcll(m);
  }
  __syncthreads();
  const int n = s_n;
  for (int h = threadIdx.x * 8; h < H; h += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // rows in batches of four: the loads of a batch are in flight together, the sum keeps slot order
    for (int j0 = 0; j0 < n; j0 += 4) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u < n) Vec8<TA>::load(o + (size_t)s_pos[j0 + u] * H + h, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + u < n) {
          const float wj = s_w[j0 + u];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[u][i], acc[i]);
        }
    }
    if (shared) {
      float v[8];
      Vec8<TA>::load(shared + (size_t)t * H + h, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    Vec8<TY>::store(y + (size_t)t * H + h, acc);
  }
}

template <typename TA, typename TY>
hipError_t run(const void* o, const int32_t* blob, const int32_t* pair_pos, const void* shared, int T,
               int k, int H, int rows, void* y, hipStream_t s) {
  int threads = H / 8;
  if (threads > 512) threads = 512;
  threads = ((threads + 63) / 64) * 64;
  k_combine<TA, TY><<<dim3(T), dim3(threads), 0, s>>>(static_cast<const TA*>(o), blob, pair_pos,
                                                      static_cast<const TA*>(shared), T, k, H, rows,
                                                      static_cast<TY*>(y));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* o, int act, const int32_t* blob, const int32_t* pair_pos,
                          const void* shared, int T, int k, int H, int rows, void* y, int y_dtype,
                          hipStream_t s) {
  if (act == MOE_DT_BF16)
    return y_dtype == MOE_DT_BF16 ? run<u16, u16>(o, blob, pair_pos, shared, T, k, H, rows, y, s)
                                  : run<u16, float>(o, blob, pair_pos, shared, T, k, H, rows, y, s);
  if (act == MOE_DT_F16)
    return y_dtype == MOE_DT_BF16 ? run<_Float16, u16>(o, blob, pair_pos, shared, T, k, H, rows, y, s)
                                  : run<_Float16, float>(o, blob, pair_pos, shared, T, k, H, rows, y, s);
  return y_dtype == MOE_DT_BF16 ? run<float, u16>(o, blob, pair_pos, shared, T, k, H, rows, y, s)
                                : run<float, float>(o, blob, pair_pos, shared, T, k, H, rows, y, s);
}

}  // namespace moe
