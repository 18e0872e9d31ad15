// One-time weight preparation for gfx950: dense expert matrices as the layer states them,
// W[e][k][n] (x·W), are stored transposed as W[e][n][k] -- the [out][in] orientation in which the
// grouped GEMM reads each output column's K weights as one contiguous row -- in their own dtype, or
// from bf16 to fp16 holding 2^8 * W for the fp16 down projection.
//
// 64 x 64 tiles through LDS: a workgroup reads 64 rows of 64 consecutive n (coalesced), and
// writes 64 rows of 64 consecutive k (coalesced); the LDS tile is padded by one element per row so
// both the row writes and the column reads are free of bank conflicts.
#include "common.h"

namespace moe {
namespace {

// Element conversions: identity, or bf16 bits -> fp16 bits of 2^8 times the value.
struct Same {
  template <typename T> __device__ static T cvt(T v) { return v; }
};
struct Bf16ToF16Scaled {
  __device__ static u16 cvt(u16 b) {
    return __builtin_bit_cast(u16, (_Float16)(__uint_as_float((uint32_t)b << 16) * kF16WeightScale));
  }
};

template <typename T, class Cvt>
__global__ __launch_bounds__(256) void k_prepare(const T* __restrict__ w, int K, int N, T* __restrict__ out) {
  __shared__ T tile[64][64 + 1];
  const int e = blockIdx.z;
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const T* src = w + (size_t)e * K * N;
  T* dst = out + (size_t)e * N * K;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 64 x 4
  for (int r = ty; r < 64; r += 4) {
    const int k = k0 + r, n = n0 + tx;
    if (k < K && n < N) tile[r][tx] = src[(size_t)k * N + n];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int n = n0 + r, k = k0 + tx;
    if (n < N && k < K) dst[(size_t)n * K + k] = Cvt::cvt(tile[tx][r]);
  }
}

// Router weights: W_r fp32 [H][E] -> two bf16 planes [2][E][H] (hi = bf16(W), lo = bf16(W - hi)),
// each expert's H weights contiguous.  hi + lo keeps 16 significant bits of W: |W - hi - lo| <=
// 2^-18 |W|, and W - hi is exact in fp32.
__global__ __launch_bounds__(256) void k_prepare_router(const float* __restrict__ w, int H, int E, u16* __restrict__ out) {
  __shared__ float tile[64][64 + 1];
  const int h0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int h = h0 + r, e = e0 + tx;
    if (h < H && e < E) tile[r][tx] = w[(size_t)h * E + e];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int e = e0 + r, h = h0 + tx;
    if (e < E && h < H) {
      const float v = tile[tx][r];
      const u16 hi = f32_to_bf16(v);
      out[(size_t)e * H + h] = hi;
      out[((size_t)E + e) * H + h] = f32_to_bf16(v - bf16_to_f32(hi));
    }
  }
}

}  // namespace

hipError_t launch_prepare_router(const float* w, int H, int E, void* out, hipStream_t s) {
  k_prepare_router<<<dim3((E + 63) / 64, (H + 63) / 64), dim3(256), 0, s>>>(w, H, E, static_cast<u16*>(out));
  return hipGetLastError();
}

hipError_t launch_prepare(const void* w, int E, int K, int N, int dtype, void* out, hipStream_t s) {
  const dim3 grid((N + 63) / 64, (K + 63) / 64, E), block(256);
  if (dtype == MOE_DT_F16)                         // bf16 in, fp16 (x 2^8) out
    k_prepare<u16, Bf16ToF16Scaled><<<grid, block, 0, s>>>(static_cast<const u16*>(w), K, N, static_cast<u16*>(out));
  else if (dtype == MOE_DT_BF16)
    k_prepare<u16, Same><<<grid, block, 0, s>>>(static_cast<const u16*>(w), K, N, static_cast<u16*>(out));
  else
    k_prepare<float, Same><<<grid, block, 0, s>>>(static_cast<const float*>(w), K, N, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace moe
