// Internal definitions shared by the HIP sources of libmoe_mi355x.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 pair packed into one dword (lo in bits 0..15): one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(u16, a) | ((uint32_t)__builtin_bit_cast(u16, b) << 16);
}

__device__ __forceinline__ u16 f32_to_bf16(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

// Round-to-nearest-even fp32 -> fp16 pair packed into one dword (lo in bits 0..15): one
// v_cvt_pk_f16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// fp16 operands of the grouped GEMM carry weights scaled by 2^8 (int4 dequantisation and the
// prepared fp16 dense weights), which centres fp16's exact range on weight magnitudes; outputs
// are multiplied by 2^-8 (exact).
constexpr float kF16WeightScale = 256.0f;

// Host-side launchers (one per source file); each returns hipSuccess or the launch error.
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* blob,
                        hipStream_t s);
hipError_t launch_pack(const int32_t* ids, const float* w, int T, int k, int32_t* blob,
                       hipStream_t s);
size_t permute_workspace_bytes(int T, int k, int e_local);
hipError_t launch_permute(const int32_t* blob, int T, int k, int e_first, int e_local,
                          int32_t* sorted_pairs, int32_t* group_offsets, int32_t* pair_pos,
                          void* workspace, hipStream_t s);
hipError_t launch_grouped_gemm(const moe_gemm_args& a, hipStream_t s);
hipError_t launch_prepare(const void* w, int E, int K, int N, int dtype, void* out, hipStream_t s);
hipError_t launch_prepare_router(const float* w, int H, int E, void* out, hipStream_t s);
hipError_t launch_router_logits(const void* x, int x_dtype, const void* w_split, const float* bias, int T, int H,
                                int E, float* logits, hipStream_t s);
hipError_t launch_combine(const void* o, int act, const int32_t* blob, const int32_t* pair_pos,
                          const void* shared, int T, int k, int H, int rows, void* y,
                          int y_dtype, hipStream_t s);

// Number of compute units of the current device (cached per device id).
int device_cu_count();

}  // namespace moe
