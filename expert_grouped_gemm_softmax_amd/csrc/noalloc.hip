// Allocation-free permutation for callers that cannot allocate device memory (code under HIP graph
// capture, serving loops, harnesses that forbid allocation).  moe_permute keeps its per-chunk
// expert counts in a workspace the caller allocates; moe_permute_noalloc keeps them in `scratch`,
// a file-scope device array of MOE_PERMUTE_NOALLOC_SCRATCH_BYTES that every GPU the library runs on
// holds until the process ends.  The kernels are moe_permute's, given the array's device address.
//
// In host code `scratch` is a host-side stand-in, not a device address: its address on the
// current device comes from hipGetSymbolAddress, looked up once per device on the first call there
// (with that device current) and kept.  The array needs no clearing: the count kernel writes every
// count it later reads.  All calls on one GPU share the array, so calls that overlap on one GPU
// (on different streams, or from different threads) race.
#include <atomic>
#include <climits>
#include <mutex>

#include "common.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {

static __device__ __align__(256) int32_t scratch[MOE_PERMUTE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace {

constexpr int kMaxDevices = 64;

// Device address of the current device's copy of `scratch`, or nullptr if the lookup fails.
void* scratch_ptr() {
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = ptrs[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    ptrs[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

inline bool fits_i32(long long v) { return v >= 0 && v < (long long)INT_MAX; }

}  // namespace
}  // namespace moe

MOE_API moe_status moe_permute_noalloc(const int32_t* blob, int T, int k, int e_first, int e_local,
                                       int32_t* sorted_pairs, int32_t* group_offsets, int32_t* pair_pos,
                                       void* stream) {
  using moe::fits_i32;
  if (!blob || !sorted_pairs || !group_offsets || !pair_pos) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)blob | (uintptr_t)sorted_pairs | (uintptr_t)group_offsets | (uintptr_t)pair_pos) & 3)
    return MOE_ERR_INVALID_ARG;                    // int32 arrays: 4-byte aligned
  if (T < 1 || k < 1 || k > 64 || !fits_i32((long long)T * k)) return MOE_ERR_INVALID_ARG;
  if (e_local < 1 || e_local > 1024 || e_first < 0 || !fits_i32((long long)e_first + e_local))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe::permute_workspace_bytes(T, k, e_local);
  if (need > MOE_PERMUTE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0) {
    ws = moe::scratch_ptr();
    if (ws == nullptr) return MOE_ERR_HIP;
  }
  (void)hipGetLastError();                         // report only this call's launch errors
  return moe::launch_permute(blob, T, k, e_first, e_local, sorted_pairs, group_offsets, pair_pos, ws,
                             static_cast<hipStream_t>(stream)) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}
