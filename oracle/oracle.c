/*
 * oracle.c -- plain, slow CPU oracle for one device's share of a routed sparse MoE
 * feed-forward layer.  TEST INFRASTRUCTURE ONLY: it is called by the tests, by the smoke check
 * and by the benchmark's CPU-baseline leg, never by the library's product path.  It shares no
 * code, header or constant with the HIP library.
 *
 * What it computes (sources are the pages' titles and sections):
 *  - Routing: "Systems engineering playbook: optimizing Qwen 3.5-397B MoE on Ironwood (TPU7x)",
 *    section 1 (sparse MoE): the router projects each token, takes a softmax over the 512 experts
 *    and selects the top 10.  Readings taken here: selection on the logits (same order as on the
 *    probabilities, exp being monotone), ties toward the lower expert id, -0 equal to +0, slots in
 *    descending order, and the selected weights renormalised to sum to one.  The renormalised
 *    weight of slot j equals exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected slots, which
 *    is evaluated in a fixed fp32 sequence with exp_ref so a GPU implementation can match bits.
 *  - Routing blob: same page, section 3 (3-to-2 all-gather): the top-k ids and weights share a
 *    shape, are stacked on a new leading axis, bitcast to 32-bit integers and packed into one
 *    dense int32 array that is unpacked locally.  Layout [2][T][k]: plane 0 ids, plane 1 the
 *    fp32 weight bits.
 *  - Local filter and grouping: same page, section 3 (option B): each device keeps only the pairs
 *    routed to its own experts; grouping them by expert for a grouped GEMM is done here as a
 *    stable counting sort by definition.
 *  - Expert FFN: same page, section 1 (FFN split into 512 experts of intermediate size 1024),
 *    taken as SwiGLU without biases: h = silu(a Wg) * (a Wu), o = h Wd, silu(z) = z / (1 + e^-z).
 *  - Combine: y[t] = sum over the token's local slots j (ascending) of w_j * o_j, plus the
 *    always-executed shared expert's output when present (section 1; the page's formula image is
 *    missing, so the merge is read as plain addition).
 *  - int4 weights: "vLLM TPU Inference v0.31.0" (4-bit weight scope): symmetric int4,
 *    group-wise scales, only the needed tiles restored on chip.  Reading taken here: word
 *    [e][K/8][N] int32, two's-complement nibble i (bits 4i..4i+3) holds K-row 8*kb+i, bf16
 *    scales [e][K/gs][N]; the oracle dequantises exactly (q * s in double).
 *
 * All FFN arithmetic is in double from exactly converted inputs; nothing is rounded to bf16.
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math): the routing sequence relies on
 * every fp32 operation being rounded on its own.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* exp_ref: e^d for d <= 0 in fp32, from basic IEEE operations only (multiply, rint, fma, exact  */
/* power-of-two scaling), so that any implementation of the same steps returns the same bits.   */
/*   n = rint(d * log2(e));  r = d - n*ln2 (two-part ln2, each step one fma);                    */
/*   p = sum_{i<=7} r^i / i!  (Horner, fma);  result = p * 2^n.   Returns 0 for d < -86.         */
/* Constants are the fp32 roundings of the mathematical values, computed here from ln 2.        */
/* ------------------------------------------------------------------------------------------ */
static float orc_c_log2e, orc_c_ln2_hi, orc_c_ln2_lo, orc_c_coef[8];

__attribute__((constructor)) static void orc_init_constants(void) {
  const double ln2 = 0.693147180559945309417232121458176568; /* ln 2 */
  orc_c_log2e = (float)(1.0 / ln2);
  orc_c_ln2_hi = (float)ln2;
  orc_c_ln2_lo = (float)(ln2 - (double)orc_c_ln2_hi);
  double fact = 1.0;
  for (int i = 0; i < 8; ++i) {
    if (i > 0) fact *= (double)i;
    orc_c_coef[i] = (float)(1.0 / fact);
  }
}

float orc_exp_ref(float d) {
  if (d < -86.0f) return 0.0f;
  float t = d * orc_c_log2e;
  float n = rintf(t);
  float r = fmaf(-n, orc_c_ln2_hi, d);
  r = fmaf(-n, orc_c_ln2_lo, r);
  float p = orc_c_coef[7];
  for (int i = 6; i >= 0; --i) p = fmaf(p, r, orc_c_coef[i]);
  return ldexpf(p, (int)n);
}

void orc_exp_ref_array(const float* d, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_exp_ref(d[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* Routing: top-k of a full sort by (logit descending, expert id ascending), then weights.     */
/* ------------------------------------------------------------------------------------------ */
typedef struct { float v; int32_t id; } orc_key;

static int orc_key_cmp(const void* pa, const void* pb) {
  const orc_key* a = (const orc_key*)pa;
  const orc_key* b = (const orc_key*)pb;
  if (a->v > b->v) return -1;        /* larger logit first; -0 == +0 compares equal */
  if (a->v < b->v) return 1;
  return (a->id > b->id) - (a->id < b->id);   /* tie: lower expert id first */
}

/* logits [T][E] fp32 (finite) -> ids [T][k] int32 (global expert ids), w [T][k] fp32. */
void orc_route(const float* logits, int T, int E, int k, int32_t* ids, float* w) {
  orc_key* keys = (orc_key*)malloc(sizeof(orc_key) * (size_t)E);
  float* e = (float*)malloc(sizeof(float) * (size_t)k);
  for (int t = 0; t < T; ++t) {
    const float* row = logits + (size_t)t * E;
    for (int i = 0; i < E; ++i) { keys[i].v = row[i]; keys[i].id = i; }
    qsort(keys, (size_t)E, sizeof(orc_key), orc_key_cmp);
    const float m = keys[0].v;
    float s = 0.0f;
    for (int j = 0; j < k; ++j) {
      float dj = keys[j].v - m;                /* <= 0 */
      e[j] = orc_exp_ref(dj);
      s = (j == 0) ? e[0] : s + e[j];          /* left-to-right fp32 sum */
    }
    for (int j = 0; j < k; ++j) {
      ids[(size_t)t * k + j] = keys[j].id;
      w[(size_t)t * k + j] = e[j] / s;         /* IEEE division */
    }
  }
  free(e);
  free(keys);
}

/* ------------------------------------------------------------------------------------------ */
/* Router projection ("Systems engineering playbook ...", section 1, sparse MoE: the router gate */
/* projects each token's representation before the softmax over the experts):                  */
/*   logits[t][e] = fp32( sum_h x[t][h] * wr[h][e] ) (+ bias[e] in fp32),                        */
/* every product and the sum taken in double from exactly converted inputs, rounded once.       */
/* x is bf16 (act = 1) or fp32 (act = 0) [T][H]; wr fp32 [H][E]; bias fp32 [E] or NULL.          */
/* ------------------------------------------------------------------------------------------ */
static double orc_bf16_bits_to_double(uint16_t b);

void orc_router_logits(const void* x, int act, const float* wr, const float* bias, int T, int H, int E,
                       float* logits) {
  double* acc = (double*)malloc(sizeof(double) * (size_t)E);
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    for (int h = 0; h < H; ++h) {
      const double xv = act ? orc_bf16_bits_to_double(((const uint16_t*)x)[(size_t)t * H + h])
                            : (double)((const float*)x)[(size_t)t * H + h];
      const float* row = wr + (size_t)h * E;
      for (int e = 0; e < E; ++e) acc[e] += xv * (double)row[e];
    }
    for (int e = 0; e < E; ++e) {
      float v = (float)acc[e];
      if (bias) v = v + bias[e];
      logits[(size_t)t * E + e] = v;
    }
  }
  free(acc);
}

/* ------------------------------------------------------------------------------------------ */
/* Routing blob [2][T][k] int32: plane 0 ids, plane 1 bit pattern of the fp32 weights.         */
/* ------------------------------------------------------------------------------------------ */
void orc_pack(const int32_t* ids, const float* w, int T, int k, int32_t* blob) {
  const size_t P = (size_t)T * k;
  for (size_t p = 0; p < P; ++p) {
    blob[p] = ids[p];
    memcpy(&blob[P + p], &w[p], 4);
  }
}

void orc_unpack(const int32_t* blob, int T, int k, int32_t* ids, float* w) {
  const size_t P = (size_t)T * k;
  for (size_t p = 0; p < P; ++p) {
    ids[p] = blob[p];
    memcpy(&w[p], &blob[P + p], 4);
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Permutation: pair p = t*k + j is local iff e_first <= id < e_first + e_local.                 */
/* group_offsets[e] = number of local pairs with a smaller local id; group_offsets[e_local] =   */
/* n_loc.  sorted_pairs[off[e] + rank] = p where rank counts earlier local pairs with the same  */
/* id (stable).  pair_pos[p] = that row, or -1.  Returns n_loc.                                 */
/* ------------------------------------------------------------------------------------------ */
int orc_permute(const int32_t* blob, int T, int k, int e_first, int e_local,
                int32_t* sorted_pairs, int32_t* group_offsets, int32_t* pair_pos) {
  const int64_t P = (int64_t)T * k;
  int64_t* cnt = (int64_t*)calloc((size_t)e_local, sizeof(int64_t));
  for (int64_t p = 0; p < P; ++p) {
    int32_t id = blob[p];
    if (id >= e_first && id < e_first + e_local) cnt[id - e_first] += 1;
  }
  int64_t run = 0;
  for (int e = 0; e < e_local; ++e) { group_offsets[e] = (int32_t)run; run += cnt[e]; }
  group_offsets[e_local] = (int32_t)run;
  int64_t* fill = (int64_t*)calloc((size_t)e_local, sizeof(int64_t));
  for (int64_t p = 0; p < P; ++p) {
    int32_t id = blob[p];
    if (id >= e_first && id < e_first + e_local) {
      int le = id - e_first;
      int64_t row = group_offsets[le] + fill[le];
      fill[le] += 1;
      sorted_pairs[row] = (int32_t)p;
      pair_pos[p] = (int32_t)row;
    } else {
      pair_pos[p] = -1;
    }
  }
  free(fill);
  free(cnt);
  return (int)run;
}

/* ------------------------------------------------------------------------------------------ */
/* Exact conversions of stored values to double.                                               */
/* ------------------------------------------------------------------------------------------ */
static double orc_bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Signed nibble i of an int32 word (two's complement, bits 4i..4i+3). */
int orc_int4_nibble(int32_t word, int i) {
  int v = (int)(((uint32_t)word >> (4 * i)) & 0xFu);
  return v >= 8 ? v - 16 : v;
}

/* OCP FP8 E4M3 ("FN": no infinities) byte -> exact value: sign bit 7, exponent bits 3..6 with
 * bias 7, mantissa bits 0..2; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN.  The
 * FP8-served models of "vLLM TPU Inference v0.31.0" (inter-chip transfer split) carry their
 * weights in 8-bit floating point; this reading takes OCP E4M3 with one scale per output
 * channel. */
double orc_fp8_e4m3_to_double(uint8_t c) {
  const int e = (c >> 3) & 0xF, m = c & 7;
  const double sign = (c & 0x80) ? -1.0 : 1.0;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) return sign * ldexp((double)m / 8.0, -6);
  return sign * ldexp(1.0 + (double)m / 8.0, e - 7);
}

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_DENSE = 0, ORC_INT4 = 1, ORC_FP8 = 2 };

/* Row kk of matrix `e` of a stack of [K][N] matrices, converted exactly to double. */
typedef struct {
  const void* w;            /* dense: f32/bf16 [E][K][N]; int4: int32 words [E][K/8][N];
                               fp8: e4m3 bytes [E][N][K] (output channel major) */
  const uint16_t* scale;    /* int4: bf16 [E][K/gs][N]; fp8: bf16 [E][N] per output channel */
  int fmt, act, K, N, gs;
} orc_mat;

static void orc_row(const orc_mat* m, int e, int kk, double* out) {
  const size_t N = (size_t)m->N;
  if (m->fmt == ORC_FP8) {
    const uint8_t* q = (const uint8_t*)m->w + (size_t)e * N * m->K;
    const uint16_t* s = m->scale + (size_t)e * N;
    for (size_t n = 0; n < N; ++n)
      out[n] = orc_fp8_e4m3_to_double(q[n * (size_t)m->K + kk]) * orc_bf16_to_double(s[n]);
  } else if (m->fmt == ORC_INT4) {
    const int32_t* words = (const int32_t*)m->w + ((size_t)e * (m->K / 8) + kk / 8) * N;
    const uint16_t* s = m->scale + ((size_t)e * (m->K / m->gs) + kk / m->gs) * N;
    for (size_t n = 0; n < N; ++n)
      out[n] = (double)orc_int4_nibble(words[n], kk % 8) * orc_bf16_to_double(s[n]);
  } else if (m->act == ORC_BF16) {
    const uint16_t* r = (const uint16_t*)m->w + ((size_t)e * m->K + kk) * N;
    for (size_t n = 0; n < N; ++n) out[n] = orc_bf16_to_double(r[n]);
  } else {
    const float* r = (const float*)m->w + ((size_t)e * m->K + kk) * N;
    for (size_t n = 0; n < N; ++n) out[n] = (double)r[n];
  }
}

/* Dequantise (or convert) matrix e of a stack to double [K][N]. */
void orc_expand_matrix(const void* w, const uint16_t* scale, int fmt, int act, int K, int N, int gs,
                       int e, double* out) {
  orc_mat m = {w, scale, fmt, act, K, N, gs};
  for (int kk = 0; kk < K; ++kk) orc_row(&m, e, kk, out + (size_t)kk * N);
}

static double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* One SwiGLU expert on one input row a[H] (double): out[H] = (silu(a Wg) * (a Wu)) Wd. */
static void orc_swiglu(const double* a, const orc_mat* g, const orc_mat* u, const orc_mat* d,
                       int e, int H, int I, double* gacc, double* uacc, double* row, double* out) {
  for (int n = 0; n < I; ++n) { gacc[n] = 0.0; uacc[n] = 0.0; }
  for (int kk = 0; kk < H; ++kk) {
    orc_row(g, e, kk, row);
    for (int n = 0; n < I; ++n) gacc[n] += a[kk] * row[n];
    orc_row(u, e, kk, row);
    for (int n = 0; n < I; ++n) uacc[n] += a[kk] * row[n];
  }
  for (int n = 0; n < H; ++n) out[n] = 0.0;
  for (int i = 0; i < I; ++i) {
    double h = orc_silu(gacc[i]) * uacc[i];
    orc_row(d, e, i, row);
    for (int n = 0; n < H; ++n) out[n] += h * row[n];
  }
}

typedef struct {
  int T, H, I, k, e_first, e_local;
  int act;          /* ORC_F32 or ORC_BF16: x, dense weights, shared weights */
  int wfmt;         /* ORC_DENSE, ORC_INT4 or ORC_FP8 for the routed experts */
  int group_size;   /* int4 group along K; <= 0: channel-wise (all K rows of a matrix) */
  int shared_I;     /* 0: no shared expert */
  const void* x;    /* [T][H] */
  const int32_t* ids;   /* [T][k] global expert ids */
  const float* w;       /* [T][k] routing weights */
  const void* wg; const void* wu; const void* wd;       /* [e_local][H][I], [e_local][H][I], [e_local][I][H] */
  const uint16_t* sg; const uint16_t* su; const uint16_t* sd;   /* int4 scales */
  const void* shg; const void* shu; const void* shd;    /* shared [H][Is], [H][Is], [Is][H] */
} orc_layer_args;

/* y[i][:] (double [n_tokens][H]) for token tokens[i]: the routed-expert combine over the
 * token's local slots in ascending j, plus the shared expert. */
void orc_layer(const orc_layer_args* A, const int32_t* tokens, int n_tokens, double* y) {
  const int H = A->H, I = A->I, k = A->k;
  const int Imax = (A->shared_I > I) ? A->shared_I : I;
  const int wide = (H > Imax) ? H : Imax;
  double* a = (double*)malloc(sizeof(double) * (size_t)H);
  double* gacc = (double*)malloc(sizeof(double) * (size_t)Imax);
  double* uacc = (double*)malloc(sizeof(double) * (size_t)Imax);
  double* row = (double*)malloc(sizeof(double) * (size_t)wide);
  double* o = (double*)malloc(sizeof(double) * (size_t)H);
  /* group_size <= 0: channel-wise scales, one group of all K rows of a matrix */
  const int gs_in = A->group_size > 0 ? A->group_size : H, gs_out = A->group_size > 0 ? A->group_size : I;
  orc_mat g = {A->wg, A->sg, A->wfmt, A->act, H, I, gs_in};
  orc_mat u = {A->wu, A->su, A->wfmt, A->act, H, I, gs_in};
  orc_mat d = {A->wd, A->sd, A->wfmt, A->act, I, H, gs_out};
  orc_mat sg = {A->shg, NULL, ORC_DENSE, A->act, H, A->shared_I, 1};
  orc_mat su = {A->shu, NULL, ORC_DENSE, A->act, H, A->shared_I, 1};
  orc_mat sd = {A->shd, NULL, ORC_DENSE, A->act, A->shared_I, H, 1};
  for (int i = 0; i < n_tokens; ++i) {
    const int t = tokens[i];
    double* yt = y + (size_t)i * H;
    for (int n = 0; n < H; ++n) {
      a[n] = (A->act == ORC_BF16) ? orc_bf16_to_double(((const uint16_t*)A->x)[(size_t)t * H + n])
                                  : (double)((const float*)A->x)[(size_t)t * H + n];
      yt[n] = 0.0;
    }
    for (int j = 0; j < k; ++j) {
      const int id = A->ids[(size_t)t * k + j];
      if (id < A->e_first || id >= A->e_first + A->e_local) continue;
      const double wj = (double)A->w[(size_t)t * k + j];
      orc_swiglu(a, &g, &u, &d, id - A->e_first, H, I, gacc, uacc, row, o);
      for (int n = 0; n < H; ++n) yt[n] += wj * o[n];
    }
    if (A->shared_I > 0) {
      orc_swiglu(a, &sg, &su, &sd, 0, H, A->shared_I, gacc, uacc, row, o);
      for (int n = 0; n < H; ++n) yt[n] += o[n];
    }
  }
  free(o); free(row); free(uacc); free(gacc); free(a);
}
