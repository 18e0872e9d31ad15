// C ABI of libmoe_mi355x.so: host-side validation and dispatch.  Every entry point validates its
// arguments before making any HIP call, so invalid calls are rejected without a GPU and without
// enqueueing work.
#include <atomic>
#include <climits>

#include "common.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace moe

namespace {

inline bool fits_i32(long long v) { return v >= 0 && v < (long long)INT_MAX; }

// Alignment of device pointers (NULL passes; required arguments are checked separately): index,
// routing and fp32 vector arrays to 4 bytes, matrices that kernels move 16 bytes at a time to 16.
inline bool al4(const void* p) { return ((uintptr_t)p & 3) == 0; }
inline bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Status of one enqueue: the runtime's last-error slot is cleared first, so an error left there by
// an earlier, unrelated call of the caller is not reported as this call's failure.
template <class F>
inline moe_status enqueue(F&& launch) {
  (void)hipGetLastError();
  return launch() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

MOE_API int moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_SCRATCH_TOO_SMALL:
      return "input needs more scratch than the allocation-free entry point holds "
             "(MOE_PERMUTE_NOALLOC_SCRATCH_BYTES per GPU); call moe_permute with a workspace";
    default: return "unknown status";
  }
}

MOE_API moe_status moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                             void* stream) {
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!al4(logits) || !al4(topk_ids) || !al4(topk_w)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || E < 1 || E > 1024 || k < 1 || k > 64 || k > E) return MOE_ERR_INVALID_ARG;
  if (!fits_i32((long long)T * E)) return MOE_ERR_INVALID_ARG;
  return enqueue([&] { return moe::launch_route(logits, T, E, k, topk_ids, topk_w, nullptr, as_stream(stream)); });
}

MOE_API moe_status moe_route_packed(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                                    int32_t* blob, void* stream) {
  if (!logits || !blob || (topk_ids == nullptr) != (topk_w == nullptr)) return MOE_ERR_INVALID_ARG;
  if (!al4(logits) || !al4(blob) || !al4(topk_ids) || !al4(topk_w)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || E < 1 || E > 1024 || k < 1 || k > 64 || k > E) return MOE_ERR_INVALID_ARG;
  if (!fits_i32((long long)T * E) || !fits_i32((long long)T * k)) return MOE_ERR_INVALID_ARG;
  return enqueue([&] { return moe::launch_route(logits, T, E, k, topk_ids, topk_w, blob, as_stream(stream)); });
}

MOE_API moe_status moe_pack_routing(const int32_t* topk_ids, const float* topk_w, int T, int k,
                                    int32_t* blob, void* stream) {
  if (!topk_ids || !topk_w || !blob) return MOE_ERR_INVALID_ARG;
  if (!al4(topk_ids) || !al4(topk_w) || !al4(blob)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || k < 1 || k > 64 || !fits_i32((long long)T * k)) return MOE_ERR_INVALID_ARG;
  return enqueue([&] { return moe::launch_pack(topk_ids, topk_w, T, k, blob, as_stream(stream)); });
}

MOE_API moe_status moe_prepare_router_weights(const float* wr, int H, int E, void* out, void* stream) {
  if (!wr || !out) return MOE_ERR_INVALID_ARG;
  if (!al4(wr) || !al16(out)) return MOE_ERR_INVALID_ARG;
  if (H < 1 || E < 1 || E > 1024 || H > (1 << 22) || !fits_i32((long long)H * E)) return MOE_ERR_INVALID_ARG;
  return enqueue([&] { return moe::launch_prepare_router(wr, H, E, out, as_stream(stream)); });
}

namespace {
moe_status check_router(const void* x, int x_dtype, const void* w_split, int T, int H, int E) {
  if (!x || !w_split) return MOE_ERR_INVALID_ARG;
  if (!al16(x) || !al16(w_split)) return MOE_ERR_INVALID_ARG;
  if (x_dtype != MOE_DT_F32 && x_dtype != MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
  if (T < 1 || H < 1 || E < 1 || E > 1024 || H > (1 << 22)) return MOE_ERR_INVALID_ARG;
  const long long esz = x_dtype == MOE_DT_F32 ? 4 : 2;
  if (!fits_i32((long long)T * E) || (long long)T * H * esz >= (1LL << 31) || !fits_i32((long long)H * E))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}
}  // namespace

MOE_API moe_status moe_router_logits(const void* x, int x_dtype, const void* w_split, const float* bias, int T,
                                     int H, int E, float* logits, void* stream) {
  if (!logits || !al4(logits) || !al4(bias)) return MOE_ERR_INVALID_ARG;
  const moe_status st = check_router(x, x_dtype, w_split, T, H, E);
  if (st != MOE_OK) return st;
  return enqueue([&] { return moe::launch_router_logits(x, x_dtype, w_split, bias, T, H, E, logits, as_stream(stream)); });
}

MOE_API moe_status moe_route_hidden(const void* x, int x_dtype, const void* w_split, const float* bias, int T, int H,
                                    int E, int k, float* logits, int32_t* topk_ids, float* topk_w, int32_t* blob,
                                    void* stream) {
  if (!logits || !blob || (topk_ids == nullptr) != (topk_w == nullptr)) return MOE_ERR_INVALID_ARG;
  if (!al4(logits) || !al4(bias) || !al4(blob) || !al4(topk_ids) || !al4(topk_w)) return MOE_ERR_INVALID_ARG;
  const moe_status st = check_router(x, x_dtype, w_split, T, H, E);
  if (st != MOE_OK) return st;
  if (k < 1 || k > 64 || k > E || !fits_i32((long long)T * k)) return MOE_ERR_INVALID_ARG;
  return enqueue([&] {
    const hipError_t e = moe::launch_router_logits(x, x_dtype, w_split, bias, T, H, E, logits, as_stream(stream));
    if (e != hipSuccess) return e;
    return moe::launch_route(logits, T, E, k, topk_ids, topk_w, blob, as_stream(stream));
  });
}

MOE_API size_t moe_permute_workspace_bytes(int T, int k, int e_local) {
  if (T < 1 || k < 1 || k > 64 || e_local < 1 || e_local > 1024 || !fits_i32((long long)T * k)) return 0;
  return moe::permute_workspace_bytes(T, k, e_local);
}

MOE_API moe_status moe_permute(const int32_t* blob, int T, int k, int e_first, int e_local,
                               int32_t* sorted_pairs, int32_t* group_offsets, int32_t* pair_pos,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!blob || !sorted_pairs || !group_offsets || !pair_pos) return MOE_ERR_INVALID_ARG;
  if (!al4(blob) || !al4(sorted_pairs) || !al4(group_offsets) || !al4(pair_pos)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || k < 1 || k > 64 || !fits_i32((long long)T * k)) return MOE_ERR_INVALID_ARG;
  if (e_local < 1 || e_local > 1024 || e_first < 0 || !fits_i32((long long)e_first + e_local))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe::permute_workspace_bytes(T, k, e_local);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15) != 0))
    return MOE_ERR_INVALID_ARG;
  return enqueue([&] { return moe::launch_permute(blob, T, k, e_first, e_local, sorted_pairs, group_offsets,
                                      pair_pos, workspace, as_stream(stream)); });
}

inline bool is_dtype(int d) { return d == MOE_DT_F32 || d == MOE_DT_BF16 || d == MOE_DT_F16; }

MOE_API moe_status moe_grouped_gemm(const moe_gemm_args* a, void* stream) {
  if (!a) return MOE_ERR_INVALID_ARG;
  if (a->op != MOE_OP_GATE_UP_SWIGLU && a->op != MOE_OP_DOWN) return MOE_ERR_INVALID_ARG;
  if (!is_dtype(a->act_dtype) || !is_dtype(a->out_dtype)) return MOE_ERR_UNSUPPORTED;
  if (a->wfmt != MOE_W_DENSE && a->wfmt != MOE_W_INT4_SYM_GROUP && a->wfmt != MOE_W_DENSE_NK &&
      a->wfmt != MOE_W_DENSE_NK_F16 && a->wfmt != MOE_W_FP8_E4M3)
    return MOE_ERR_UNSUPPORTED;
  const bool gu = a->op == MOE_OP_GATE_UP_SWIGLU;
  const bool q4 = a->wfmt == MOE_W_INT4_SYM_GROUP;
  const bool w8 = a->wfmt == MOE_W_FP8_E4M3;
  if (!a->a || !a->group_offsets || !a->w0 || !a->out) return MOE_ERR_INVALID_ARG;
  if (gu ? !a->w1 : a->w1 != nullptr) return MOE_ERR_INVALID_ARG;
  if (!al16(a->a) || !al16(a->w0) || !al16(a->w1) || !al16(a->s0) || !al16(a->s1) || !al16(a->out) ||
      !al4(a->group_offsets) || !al4(a->row_index))
    return MOE_ERR_INVALID_ARG;
  if (a->K < 64 || a->K % 64 != 0 || a->N < 64) return MOE_ERR_INVALID_ARG;
  if (a->N % (gu ? 64 : 128) != 0) return MOE_ERR_INVALID_ARG;
  if (a->n_groups < 1 || a->n_groups > 1024) return MOE_ERR_INVALID_ARG;
  if (a->rows_cap < 1 || a->a_rows < 1 || a->row_div < 1 || a->m_hint < 0) return MOE_ERR_INVALID_ARG;
  if (!a->row_index && a->a_rows < a->rows_cap) return MOE_ERR_INVALID_ARG;
  if (q4 || w8) {
    if (!a->s0 || (gu ? !a->s1 : a->s1 != nullptr)) return MOE_ERR_INVALID_ARG;
  } else if (a->group_size != 0 || a->s0 || a->s1) {
    return MOE_ERR_INVALID_ARG;
  }
  // dtype combinations (see moe.h): an output dtype the op never writes is an invalid argument,
  // a well-formed combination that is not implemented is unsupported
  if (a->act_dtype == MOE_DT_F32) {
    if (a->out_dtype != MOE_DT_F32) return MOE_ERR_INVALID_ARG;
    if (a->wfmt != MOE_W_DENSE && a->wfmt != MOE_W_DENSE_NK) return MOE_ERR_UNSUPPORTED;
  } else if (gu) {
    if (a->out_dtype == MOE_DT_F32) return MOE_ERR_INVALID_ARG;
    if (a->act_dtype != MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
    if (q4 ? a->out_dtype != MOE_DT_F16 : (a->wfmt == MOE_W_DENSE_NK_F16)) return MOE_ERR_UNSUPPORTED;
  } else {
    if (a->out_dtype != MOE_DT_F32 && a->out_dtype != a->act_dtype) return MOE_ERR_INVALID_ARG;
    if (!w8 && (a->act_dtype == MOE_DT_BF16 ? (a->wfmt != MOE_W_DENSE_NK && a->wfmt != MOE_W_DENSE)
                                            : (a->wfmt != MOE_W_DENSE_NK_F16 && !q4)))
      return MOE_ERR_UNSUPPORTED;
  }
  if (w8 && a->group_size != a->K) return MOE_ERR_UNSUPPORTED;   // one scale per output channel
  // 32-bit byte offsets inside a (below 2^31: offsets from 2^31 up mark rows that load nothing)
  // and inside one expert's weight matrix
  const long long esz = a->act_dtype == MOE_DT_F32 ? 4 : 2;
  if ((long long)a->a_rows * a->K * esz >= (1LL << 31) || (long long)a->K * a->N * (w8 ? 1 : esz) >= (1LL << 32))
    return MOE_ERR_UNSUPPORTED;
  if (q4 && (a->group_size < 8 || (a->group_size % 64 != 0 && 64 % a->group_size != 0) ||
             a->K % a->group_size != 0))
    return MOE_ERR_UNSUPPORTED;
  return enqueue([&] { return moe::launch_grouped_gemm(*a, as_stream(stream)); });
}

MOE_API moe_status moe_prepare_dense_weights(const void* w, int E, int K, int N, int dtype, void* out,
                                             void* stream) {
  if (!w || !out || !al16(w) || !al16(out)) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
  if (E < 1 || K < 1 || N < 1 || E > 65535 || K > (1 << 22) || (long long)E * K * N >= (1LL << 40))
    return MOE_ERR_INVALID_ARG;
  return enqueue([&] { return moe::launch_prepare(w, E, K, N, dtype, out, as_stream(stream)); });
}

MOE_API moe_status moe_prepare_dense_weights_f16(const void* w, int E, int K, int N, void* out, void* stream) {
  if (!w || !out || !al16(w) || !al16(out)) return MOE_ERR_INVALID_ARG;
  if (E < 1 || K < 1 || N < 1 || E > 65535 || K > (1 << 22) || (long long)E * K * N >= (1LL << 40))
    return MOE_ERR_INVALID_ARG;
  return enqueue([&] { return moe::launch_prepare(w, E, K, N, MOE_DT_F16, out, as_stream(stream)); });
}

MOE_API moe_status moe_combine(const void* expert_out, int expert_rows, int act_dtype, const int32_t* blob,
                               const int32_t* pair_pos, const void* shared_out, int T, int k, int H,
                               void* y, int y_dtype, void* stream) {
  if (!expert_out || !blob || !pair_pos || !y) return MOE_ERR_INVALID_ARG;
  if (!al16(expert_out) || !al16(shared_out) || !al16(y) || !al4(blob) || !al4(pair_pos)) return MOE_ERR_INVALID_ARG;
  if (!is_dtype(act_dtype)) return MOE_ERR_UNSUPPORTED;
  if (y_dtype != MOE_DT_F32 && y_dtype != MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
  if (expert_rows < 1 || T < 1 || k < 1 || k > 64 || H < 8 || H % 8 != 0) return MOE_ERR_INVALID_ARG;
  if (!fits_i32((long long)T * k)) return MOE_ERR_INVALID_ARG;
  return enqueue([&] { return moe::launch_combine(expert_out, act_dtype, blob, pair_pos, shared_out, T, k, H,
                                      expert_rows, y, y_dtype, as_stream(stream)); });
}
