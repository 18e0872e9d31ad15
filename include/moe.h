/*
 * moe.h -- C ABI of libmoe_mi355x.so: one device's share of a routed sparse mixture-of-experts
 * feed-forward layer on AMD MI355X (gfx950).
 *
 * The layer (as stated in "Systems engineering playbook: optimizing Qwen 3.5-397B MoE on Ironwood
 * (TPU7x)", sections 1 and 3, and "vLLM TPU Inference v0.31.0", 4-bit weight scope):
 *   1. moe_route         softmax top-k routing of each token over E experts, renormalised weights;
 *   2. moe_pack_routing  ids and weight bits packed into one int32 routing blob;
 *   3. moe_permute       the pairs routed to this device's experts, grouped expert by expert;
 *   4. moe_grouped_gemm  per-expert SwiGLU FFN: fused gate/up projection + SwiGLU, then the down
 *                        projection, with bf16 or symmetric int4 group-quantised (W4A16) weights;
 *   5. moe_combine       weighted sum of each token's expert outputs back in token order.
 * Also: moe_route_packed (steps 1 and 2 in one launch); moe_router_logits and moe_route_hidden
 * (the router projection x W_r before step 1, and with steps 1-2 after it); moe_permute_noalloc
 * (step 3 without a workspace); one-time, load-time weight preparation (moe_prepare_dense_weights,
 * moe_prepare_dense_weights_f16, moe_prepare_router_weights).
 *
 * Conventions shared by every entry point:
 *   - Every array argument is a DEVICE pointer owned by the caller.  The library never allocates,
 *     frees or synchronises; each call only enqueues kernels on `stream` (a hipStream_t; NULL is
 *     the null stream) and returns.  Results are valid once the stream reaches that point.
 *   - Arguments are validated on the host before anything is enqueued; an invalid call returns
 *     MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED and enqueues nothing.  A failed launch returns
 *     MOE_ERR_HIP.  Validation needs no GPU.
 *   - Alignment: int32 arrays (ids, blob, sorted_pairs, group_offsets, pair_pos, row_index) and
 *     fp32 vectors and logits (topk_w, logits, bias) 4-byte aligned; matrices that kernels move 16
 *     bytes at a time (activations x and h, expert and router weights and their scales, the
 *     outputs of moe_grouped_gemm, expert_out, shared_out and y of moe_combine, prepared weight
 *     copies, workspaces) 16-byte aligned.  A misaligned pointer is MOE_ERR_INVALID_ARG.
 *     hipMalloc and PyTorch allocations satisfy both.
 *   - Data-dependent preconditions are not checked on the device: logits are finite, blob ids are
 *     in [0, E).  Kernels clamp every index they read, so violating them gives wrong values, not
 *     out-of-bounds accesses.
 *   - Row-major layouts; "bf16" is IEEE bfloat16 stored in 16 bits; conversions to bf16 round to
 *     nearest even.  No call depends on the number of local pairs being known on the host.
 *   - The library's global state is a per-device cache of the compute-unit count and the
 *     per-device scratch array of moe_permute_noalloc; calls on different streams may run
 *     concurrently, except moe_permute_noalloc calls on one GPU (see its declaration).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null pointer, size out of range, inconsistent sizes */
  MOE_ERR_UNSUPPORTED = 2,   /* well-formed request outside what the library implements */
  MOE_ERR_HIP = 3,           /* a HIP runtime call or kernel launch failed */
  MOE_ERR_SCRATCH_TOO_SMALL = 4  /* moe_permute_noalloc: the input needs more than its fixed scratch */
} moe_status;

/* MOE_DT_F16 (IEEE binary16) is the dtype of the SwiGLU output h between the two grouped GEMMs of
 * a bf16 layer: its 11-bit significand keeps the rounding of h 8x smaller than bf16's, which the
 * layer's error bar needs on heavy-tailed outputs. */
typedef enum moe_dtype { MOE_DT_F32 = 0, MOE_DT_BF16 = 1, MOE_DT_F16 = 2 } moe_dtype;

/* Expert weight formats for a K x N matrix W of expert e (output n = sum_k a[k] W[k][n]).
 * MOE_W_DENSE: W[e][k][n] in the activation dtype, the layout the layer is stated in.
 * MOE_W_DENSE_NK: the same values stored [e][n][k] (row n = the K weights of output n), as
 * moe_prepare_dense_weights writes them; the bf16 grouped GEMM's fastest tiles read this layout.
 * MOE_W_DENSE_NK_F16: fp16 [e][n][k] holding 2^8 * W (moe_prepare_dense_weights_f16 writes it
 * from bf16 MOE_W_DENSE weights), the weights of a down projection over fp16 h.  The conversion
 * is exact for 2^-22 <= |W| <= 255 (fp16's normal range shifted by 2^8); smaller magnitudes keep
 * an absolute error below 2^-33.
 * MOE_W_INT4_SYM_GROUP: symmetric int4 with one bf16 scale per group of
 * `group_size` consecutive K rows per output column ("vLLM TPU Inference v0.31.0", 4-bit weight
 * scope: symmetric int4, group-wise scales, activations not quantised; asymmetric, 8-bit and
 * activation-order variants are not supported there and are not representable here).
 * Layout for a [K][N] matrix of expert e: words int32 [E][K/8][N], the two's-complement nibble at
 * bits 4i..4i+3 of word [e][kb][n] is q[8*kb+i][n]; scales bf16 [E][K/group_size][N];
 * weight = q * scale.  Channel-wise scales are group_size == K.
 * MOE_W_FP8_E4M3: 8-bit floating-point weights (the FP8-served models of "vLLM TPU Inference
 * v0.31.0", inter-chip transfer split), read as OCP E4M3 (bias 7, no infinities, S.1111.111 NaN)
 * bytes stored [E][N][K] (each output column's K weights contiguous, the [out][in] orientation of
 * a linear layer) with one bf16 scale per output column, [E][N]; weight = e4m3(q) * scale;
 * group_size must be K. */
typedef enum moe_wfmt {
  MOE_W_DENSE = 0,
  MOE_W_INT4_SYM_GROUP = 1,
  MOE_W_DENSE_NK = 2,
  MOE_W_DENSE_NK_F16 = 3,
  MOE_W_FP8_E4M3 = 4
} moe_wfmt;

typedef enum moe_gemm_op {
  MOE_OP_GATE_UP_SWIGLU = 0,  /* out = silu(A Wg) * (A Wu), silu(z) = z / (1 + e^-z) */
  MOE_OP_DOWN = 1             /* out = A Wd */
} moe_gemm_op;

/* ABI version of the loaded library (MOE_ABI_VERSION at build time). */
int moe_abi_version(void);

/* Static description of a status code; never NULL. */
const char* moe_status_string(int status);

/*
 * moe_route -- softmax top-k routing ("Systems engineering playbook ...", section 1, sparse MoE:
 * the router projects the token and picks the top experts of a softmax over all experts).
 *   logits    fp32 [T][E]   router logits (finite).
 *   topk_ids  int32 [T][k]  out: global expert ids, slot order by descending logit, ties to the
 *                           lower expert id (-0 equals +0).
 *   topk_w    fp32 [T][k]   out: weights renormalised over the k selected experts, evaluated as
 *                           m = logit of slot 0, e_j = exp_ref(l_j - m), S = e_0 + e_1 + ... (left to
 *                           right), w_j = e_j / S with correctly rounded fp32 operations and no
 *                           contraction; exp_ref(d) = p(r) * 2^n with n = rint(d * fl(log2 e)),
 *                           r = d - n*ln2 (two fma with the fp32 high and low parts of ln 2),
 *                           p = degree-7 Taylor polynomial with fp32 coefficients 1/i! in Horner
 *                           form (fma), and 0 for d < -86.  Equal in exact arithmetic to a softmax
 *                           over all E experts restricted to the selected ones and renormalised.
 *   Limits: 1 <= T, 1 <= E <= 1024, 1 <= k <= min(E, 64); T * E < 2^31.
 */
moe_status moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                     void* stream);

/*
 * moe_prepare_router_weights -- one-time preparation of the router weight for the projections
 * below: W_r fp32 [H][E] (logits = x W_r) -> two bf16 planes out [2][E][H], hi = bf16(W_r) and
 * lo = bf16(W_r - hi), each expert's H weights contiguous.  hi + lo keeps 16 significant bits of
 * every weight (|W_r - hi - lo| <= 2^-18 |W_r|).  wr and out must not overlap.
 *   Limits: 1 <= E <= 1024, 1 <= H <= 2^22, H * E < 2^31.
 */
moe_status moe_prepare_router_weights(const float* wr, int H, int E, void* out, void* stream);

/*
 * moe_router_logits -- the router projection ("Systems engineering playbook ...", section 1,
 * sparse MoE: the router gate projects each token's representation before the softmax over the
 * experts): logits[t][e] = sum_h x[t][h] (hi[e][h] + lo[e][h]) (+ bias[e]) in fp32.
 *   x        [T][H] bf16 (MOE_DT_BF16) or fp32 (MOE_DT_F32), row-major.
 *   w_split  bf16 [2][E][H] from moe_prepare_router_weights.
 *   bias     fp32 [E] added to every token's logits, or NULL.
 *   logits   fp32 [T][E] out.
 * bf16 x with H and E multiples of 64 runs on bf16 MFMA (each product x * hi and x * lo exact,
 * fp32 accumulation in a fixed order); otherwise an fp32 vector loop over h in order.  Against
 * the exact sum with W_r the error is at most (2^-18 + n_acc 2^-24) * sum_h |x[t][h] W_r[h][e]|
 * with n_acc = H + 2 (fp32 path) or H / 32 + 34 (MFMA path), plus the rounding of the bias addition.
 *   Limits: 1 <= T, 1 <= H <= 2^22, 1 <= E <= 1024, T * H * sizeof(x) < 2^31, T * E < 2^31.
 */
moe_status moe_router_logits(const void* x, int x_dtype, const void* w_split, const float* bias, int T, int H,
                             int E, float* logits, void* stream);

/*
 * moe_route_hidden -- the router projection followed by moe_route_packed, from the hidden states:
 * logits (written to `logits`, fp32 [T][E]) then ids, weights and blob exactly as moe_route_packed
 * computes them from those logits.  topk_ids / topk_w: both written, or both NULL.
 *   Limits: those of moe_router_logits and moe_route_packed.
 */
moe_status moe_route_hidden(const void* x, int x_dtype, const void* w_split, const float* bias, int T, int H, int E,
                            int k, float* logits, int32_t* topk_ids, float* topk_w, int32_t* blob, void* stream);

/*
 * moe_pack_routing -- routing blob ("Systems engineering playbook ...", section 3, 3-to-2
 * all-gather: ids and weights share their shape, are stacked on a new axis, bitcast and packed
 * into one dense int32 array, to be unpacked locally after one collective).
 *   blob int32 [2][T][k] out: blob[0][t][j] = topk_ids[t][j]; blob[1][t][j] = bits of topk_w[t][j].
 *   Limits: 1 <= T, 1 <= k <= 64, T * k < 2^31.
 */
moe_status moe_pack_routing(const int32_t* topk_ids, const float* topk_w, int T, int k,
                            int32_t* blob, void* stream);

/*
 * moe_route_packed -- moe_route followed by moe_pack_routing in one launch: blob [2][T][k] as
 * moe_pack_routing would build it from moe_route's outputs (bit for bit).  topk_ids and topk_w
 * are written when both are non-NULL and skipped when both are NULL.
 *   Limits: those of moe_route, and T * k < 2^31.
 */
moe_status moe_route_packed(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                            int32_t* blob, void* stream);

/*
 * moe_permute -- keep the pairs routed to this device's experts and group them by expert
 * ("Systems engineering playbook ...", section 3, option B: each device filters and computes only
 * the inputs of its local experts).  Pair p = t*k + j is local iff
 * e_first <= blob[0][t][j] < e_first + e_local.
 *   sorted_pairs  int32 [T*k]        out: rows [0, n_loc) hold the local pairs grouped by local
 *                                    expert, ascending p within a group (stable counting sort);
 *                                    rows >= n_loc are left untouched.
 *   group_offsets int32 [e_local+1]  out: group e owns rows [off[e], off[e+1]); off[0] = 0,
 *                                    off[e_local] = n_loc.
 *   pair_pos      int32 [T*k]        out: row of pair p in sorted_pairs, or -1 if p is not local.
 *   workspace     device scratch of at least moe_permute_workspace_bytes(T, k, e_local) bytes,
 *                 16-byte aligned (per-chunk expert counts); its contents on entry do not matter.  Calls that
 *                 may run concurrently need separate workspaces.  When that size is 0 (T*k <=
 *                 16384: one workgroup does the whole permutation) workspace may be NULL.
 *   Limits: 1 <= T, 1 <= k <= 64, 1 <= e_local <= 1024, e_first >= 0, T * k < 2^31.
 *   Deterministic: the output does not depend on scheduling.
 */
size_t moe_permute_workspace_bytes(int T, int k, int e_local);

moe_status moe_permute(const int32_t* blob, int T, int k, int e_first, int e_local,
                       int32_t* sorted_pairs, int32_t* group_offsets, int32_t* pair_pos,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_permute_noalloc -- moe_permute for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same arguments,
 * outputs and limits as moe_permute, without the workspace: the per-chunk counts live in a
 * library-owned static device array of MOE_PERMUTE_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held
 * until the process ends.  Allocates nothing.  Inputs whose moe_permute_workspace_bytes exceeds
 * that size return MOE_ERR_SCRATCH_TOO_SMALL (e.g. 64 local experts: up to 8,388,608 pairs; 1024
 * local experts: up to 524,288 pairs).  Every call on a GPU shares its array, which keeps the last
 * call's contents (no call reads them): calls that overlap on one GPU (different streams or
 * threads) race and must be serialised by the caller.
 */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (4u << 20)

moe_status moe_permute_noalloc(const int32_t* blob, int T, int k, int e_first, int e_local,
                               int32_t* sorted_pairs, int32_t* group_offsets, int32_t* pair_pos,
                               void* stream);

/*
 * moe_grouped_gemm -- one grouped GEMM over the experts of this device ("Systems engineering
 * playbook ...", executive summary: the grouped GEMM building block; section 1: experts of
 * intermediate size 1024, read here as SwiGLU FFNs without biases; "vLLM TPU Inference v0.31.0",
 * 4-bit weight scope: int4 weights stay packed in HBM and only the tiles in use are dequantised on
 * chip).  Group e covers output rows [group_offsets[e], group_offsets[e+1]); output row r uses
 * A row a[row_index[r] / row_div] (or a[r] when row_index is NULL) and expert e's weights.
 * GATE_UP_SWIGLU: out[r][n] = silu(sum_k A[k] Wg(e)[k][n]) * (sum_k A[k] Wu(e)[k][n]).
 * DOWN:           out[r][n] = sum_k A[k] Wd(e)[k][n].
 * Supported combinations (anything else is MOE_ERR_UNSUPPORTED):
 *   fp32:     a, weights (MOE_W_DENSE or MOE_W_DENSE_NK) and out fp32; vector-ALU fp32 arithmetic.
 *   GATE_UP:  a = x bf16; MOE_W_DENSE or MOE_W_DENSE_NK bf16 or MOE_W_FP8_E4M3 weights (bf16 MFMA
 *             operands) with out (h) bf16 or fp16, or MOE_W_INT4_SYM_GROUP with out fp16.
 *   DOWN:     a = h bf16 with MOE_W_DENSE or MOE_W_DENSE_NK bf16 weights (bf16 operands), or a = h fp16 with
 *             MOE_W_DENSE_NK_F16 or MOE_W_INT4_SYM_GROUP weights (fp16 operands), or a = h bf16 or
 *             fp16 with MOE_W_FP8_E4M3 weights (operands in h's dtype); out fp32 or a's dtype.
 * fp8 weights convert exactly to bf16 and to fp16 (4 significant bits; exponents 2^-9..2^8) on
 * their way to LDS; their per-column scales multiply the fp32 accumulators in the epilogue.
 * Bf16 weights in the stated MOE_W_DENSE [e][K][N] layout are read as they are (K rows staged in
 * LDS, operands read transposed; same results, bit for bit, as MOE_W_DENSE_NK); the prepared
 * MOE_W_DENSE_NK copy (moe_prepare_dense_weights) takes the faster tile paths.
 * Accumulation is fp32 throughout.  int4 weights run on fp16 operands: each weight q * s is
 * dequantised exactly to fp16 in LDS (q * s has at most 11 significant bits, which bf16 would
 * round), as 2^8 * q * s, exact for scales 2^-22 <= s < 32; their bf16 activations x are converted
 * to fp16 on the way to LDS (exact for |x| in [2^-14, 65504]; smaller magnitudes keep an absolute
 * error below 2^-25).  fp16 outputs (h) are rounded to nearest even and overflow to infinity above
 * 65504.  A 16-bit DOWN output is the round-to-nearest-even of the fp32 one (the same
 * accumulators); fp32 is the output meant for partial sums.  fp32 path: fp32 throughout.  Rows >= group_offsets[n_groups] are
 * not written.  Limits (32-bit byte offsets): a_rows * K * sizeof(act) < 2^31 and
 * K * N * sizeof(act) < 2^32, else MOE_ERR_UNSUPPORTED.
 */
typedef struct moe_gemm_args {
  int32_t op;          /* moe_gemm_op */
  int32_t act_dtype;   /* moe_dtype of a (and of dense MOE_W_DENSE / MOE_W_DENSE_NK weights) */
  int32_t wfmt;        /* moe_wfmt of w0 / w1 (int4 requires MOE_DT_BF16) */
  int32_t group_size;  /* int4: K rows per scale, dividing K: 8, 16, 32 or a multiple of 64
                          (K: channel-wise).  fp8: K.  Dense: 0 */
  int32_t K;           /* contraction length: H for GATE_UP, I for DOWN; multiple of 64 */
  int32_t N;           /* output columns: I for GATE_UP (multiple of 64), H for DOWN (multiple
                          of 128) */
  int32_t n_groups;    /* experts in this call, 1..1024 */
  int32_t rows_cap;    /* rows of out; group_offsets[n_groups] <= rows_cap */
  int32_t a_rows;      /* rows of a (tokens for GATE_UP, rows_cap for DOWN) */
  int32_t row_div;     /* >= 1; divisor applied to row_index (k for GATE_UP after moe_permute) */
  int32_t m_hint;      /* expected rows per group, a launch-shape hint only (0: unknown) */
  int32_t out_dtype;   /* moe_dtype of out (see the combinations above) */
  const void* a;                 /* [a_rows][K] act dtype */
  const int32_t* row_index;      /* [rows_cap] (e.g. sorted_pairs) or NULL for identity rows */
  const int32_t* group_offsets;  /* [n_groups+1] non-decreasing, [0] = 0 (e.g. from moe_permute) */
  const void* w0;      /* GATE_UP: Wg; DOWN: Wd, in format wfmt (see moe_wfmt) */
  const void* w1;      /* GATE_UP: Wu (same layout as w0); DOWN: NULL */
  const void* s0;      /* int4: bf16 scales of w0 [n_groups][K/group_size][N]; fp8: bf16 [n_groups][N];
                          dense: NULL */
  const void* s1;      /* int4, fp8 GATE_UP: scales of w1 (as s0); otherwise NULL */
  void* out;           /* [rows_cap][N] out_dtype */
} moe_gemm_args;

moe_status moe_grouped_gemm(const moe_gemm_args* args, void* stream);

/*
 * moe_prepare_dense_weights -- one-time weight preparation (not part of the per-batch path):
 * out[e][n][k] = w[e][k][n] for E matrices of K x N in dtype (MOE_DT_F32 or MOE_DT_BF16), i.e.
 * MOE_W_DENSE -> MOE_W_DENSE_NK.  w and out must not overlap.
 *   Limits: 1 <= E <= 65535, 1 <= K <= 2^22, 1 <= N, E * K * N < 2^40.
 */
moe_status moe_prepare_dense_weights(const void* w, int E, int K, int N, int dtype, void* out, void* stream);

/*
 * moe_prepare_dense_weights_f16 -- one-time weight preparation for a down projection over fp16 h:
 * out[e][n][k] = fp16(2^8 * w[e][k][n]) from bf16 MOE_W_DENSE weights, i.e. MOE_W_DENSE_NK_F16
 * (exact for 2^-22 <= |w| <= 255; rounded to nearest even otherwise).  w and out must not overlap.
 *   Limits: as moe_prepare_dense_weights.
 */
moe_status moe_prepare_dense_weights_f16(const void* w, int E, int K, int N, void* out, void* stream);

/*
 * moe_combine -- weighted sum back to token order ("Systems engineering playbook ...",
 * executive summary: the unpermute building block; section 1: the always-executed shared expert
 * is added to the routed output, its formula being read as plain addition).
 *   expert_out  [expert_rows][H] act dtype   rows indexed by pair_pos (e.g. the DOWN output).
 *   blob        int32 [2][T][k]              weights are read from plane 1.
 *   pair_pos    int32 [T*k]                  from moe_permute; -1 (or any value outside
 *                                            [0, expert_rows)) marks a pair without a row.
 *   shared_out  [T][H] act dtype or NULL (same dtype as expert_out).
 *   y           [T][H] y_dtype               out: y[t] = sum_{j ascending, valid pair_pos}
 *                                            w[t][j] * expert_out[pair_pos[t*k+j]]
 *                                            (+ shared_out[t]), accumulated in fp32 in that
 *                                            order (deterministic, no atomics); a token with no
 *                                            local pair gets 0 (+ shared_out[t]).
 *   Limits: 1 <= T, 1 <= k <= 64, H a multiple of 8, 1 <= expert_rows, T * k < 2^31; act_dtype
 *   in {MOE_DT_F32, MOE_DT_BF16, MOE_DT_F16}, y_dtype in {MOE_DT_F32, MOE_DT_BF16}.
 */
moe_status moe_combine(const void* expert_out, int expert_rows, int act_dtype, const int32_t* blob,
                       const int32_t* pair_pos, const void* shared_out, int T, int k, int H,
                       void* y, int y_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
