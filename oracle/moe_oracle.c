/*
 * moe_oracle.c -- plain, slow, fp64 reference of the fused MoE layer forward
 * and of the routed expert layer's backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under grouped_gemm_amd/) never calls, links or includes it, and
 * this file includes nothing from there.
 *
 * What it computes, step by step, and where the pages describe it:
 *
 *  - top-k routing: per token, the k experts with the largest router score,
 *    ties to the lower expert index, gate weights renormalised over the k
 *    (Alpha-MoE news page, "How the megakernel works": routing and gating are
 *    stages of the layer; LightMoE README, "MoE inference": top_k_ids are
 *    int32 and distinct per token, top_k_weights are fp32);
 *  - deterministic expert-major dispatch: per-expert counts, their exclusive
 *    prefix sum m_indptr of length E+1 (zero-row experts allowed), and the
 *    stable permutation of the T*k (token, slot) pairs into contiguous expert
 *    row groups (LightMoE README, API table and "Grouped GEMM";
 *    "MoE training": gather indices and inverse slots);
 *  - the block-id -> (expert, row offset) table that lets one launch cover
 *    variable-size expert groups without padding (pure-Triton MoE
 *    commentary, second paragraph);
 *  - dynamic activation quantisation before each expert GEMM and the
 *    requantisation of the gated intermediate (LightMoE README, "MoE
 *    inference": input quantisation and requantisation; Alpha-MoE news page,
 *    "The MoE bottleneck": FP8 W8A8);
 *  - per expert, out = A * B^T against [N, K] weights (LightMoE README,
 *    "Dense GEMM"/"Grouped GEMM"), gate and up from the same input, SiLU(gate)
 *    times up (pure-Triton MoE commentary, second paragraph), then the down
 *    projection;
 *  - routing-weight application and combine in a fixed order (LightMoE
 *    README, "MoE inference");
 *  - the gradients of the routed expert layer with respect to its input,
 *    its expert weights and its routing weights, and of the routing weights
 *    with respect to the router scores (LightMoE README, "MoE training" and
 *    "Highlights"), as the derivatives of the forward written out.
 *
 * Everything is accumulated in double over exactly dequantised operands.
 * Where the activations are quantised on the fly, the oracle applies the
 * same rule the layer does (stated at oracle_quant_group) so that both
 * sides multiply the same codes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SCORE_SOFTMAX 0
#define SCORE_SIGMOID 1
#define SCORE_PROBS 2
#define W_BF16 0
#define W_FP8_CHANNEL 1
#define W_FP8_BLOCK128 2
#define W_MXFP4 3
#define A_BF16 0
#define A_FP8_TOKEN 1
#define A_FP8_G128 2
#define A_MXFP8_G32 3
#define ACT_SWIGLU 0
#define ACT_SWIGLU_BOUNDED 1
#define ACT_SWIGLU_OAI 2
#define ACT_GEGLU 3
#define ACT_REGLU 4
#define ACT_RELU2 5

/* ------------------------------------------------------------------ codecs */

/* bf16: the top 16 bits of an IEEE binary32. */
double oracle_bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even (finite inputs). */
double oracle_bf16_round(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  frexp(v, &e);                 /* |v| in [2^(e-1), 2^e) */
  int emin = -126;              /* bf16 shares binary32's exponent range */
  int q = (e - 1 < emin ? emin : e - 1) - 7;   /* 8 significant bits */
  double ulp = ldexp(1.0, q);
  double r = nearbyint(v / ulp); /* default rounding mode: ties to even */
  return r * ulp;
}

/* OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 * no infinities, 0x7f/0xff are NaN, largest finite 448. */
double oracle_e4m3_decode(uint8_t c) {
  int s = c >> 7, ex = (c >> 3) & 0xF, m = c & 7;
  double mag;
  if (ex == 0xF && m == 7) return NAN;
  if (ex == 0)
    mag = ldexp((double)m, -9);            /* subnormal: m * 2^-6 / 8 */
  else
    mag = ldexp(1.0 + m / 8.0, ex - 7);
  return s ? -mag : mag;
}

/* Nearest E4M3 value to v, ties to the even mantissa, saturating at +-448.
 * Brute force over the 127 non-negative finite codes.  The sign bit is the
 * input's sign, also when the magnitude rounds to zero (IEEE-style -0). */
uint8_t oracle_e4m3_encode(double v) {
  double a = fabs(v);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 127; ++c) {
    double d = fabs(oracle_e4m3_decode((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

/* OCP E8M0 scale: 2^(c-127); 0xff is NaN. */
double oracle_e8m0_decode(uint8_t c) {
  if (c == 0xFF) return NAN;
  return ldexp(1.0, (int)c - 127);
}

/* OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit. */
double oracle_e2m1_decode(uint8_t nib) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double m = mag[nib & 7];
  return (nib & 8) ? -m : m;
}

/* --------------------------------------------------- activation quantisation
 * One group of n values (a token row, or a 1x128 or 1x32 slice of it):
 *  FP8 with an fp32 scale (per-token and 1x128 groups):
 *    a = max |v| ; s = fp32(a / 448), or 1 when a == 0 ;
 *    q_i = e4m3_rne(clamp(fp32(v_i / s), -448, 448)) ; value = q_i * s.
 *  MXFP8 (OCP MX v1.0, 32-element blocks with E4M3 elements):
 *    X = 2^(floor(log2 a) - 8)  (8 = largest exponent of E4M3), X = 2^-127
 *    when a == 0 ; q_i = e4m3_rne_saturating(v_i / X) ; value = q_i * X.
 * Returns the scale as a double (exact: an fp32 value or a power of two);
 * for MX groups *e8m0 receives the biased exponent.
 */
double oracle_quant_group(const double* v, int n, int a_format, uint8_t* q, uint8_t* e8m0) {
  double a = 0.0;
  for (int i = 0; i < n; ++i)
    if (fabs(v[i]) > a) a = fabs(v[i]);
  if (a_format == A_MXFP8_G32) {
    int ex;
    if (a == 0.0) {
      ex = -127;
    } else {
      int e;
      frexp(a, &e);            /* a in [2^(e-1), 2^e) => floor(log2 a) = e-1 */
      ex = (e - 1) - 8;
      if (ex < -127) ex = -127;
      if (ex > 127) ex = 127;
    }
    double X = ldexp(1.0, ex);
    for (int i = 0; i < n; ++i) q[i] = oracle_e4m3_encode((double)(float)(v[i] / X));
    if (e8m0) *e8m0 = (uint8_t)(ex + 127);
    return X;
  }
  float s = (a == 0.0) ? 1.0f : (float)((double)(float)a / 448.0);
  for (int i = 0; i < n; ++i) {
    float r = (float)(v[i] / (double)s);
    if (r > 448.0f) r = 448.0f;
    if (r < -448.0f) r = -448.0f;
    q[i] = oracle_e4m3_encode((double)r);
  }
  return (double)s;
}

static int group_len(int a_format, int n) {
  switch (a_format) {
    case A_FP8_TOKEN: return n;
    case A_FP8_G128: return 128;
    case A_MXFP8_G32: return 32;
    default: return 1;
  }
}

/* Replace v[0..n) by its dequantised image under the activation format. */
static void quant_dequant_row(double* v, int n, int a_format) {
  if (a_format == A_BF16) {
    for (int i = 0; i < n; ++i) v[i] = oracle_bf16_round(v[i]);
    return;
  }
  int g = group_len(a_format, n);
  uint8_t* q = (uint8_t*)malloc((size_t)g);
  for (int i0 = 0; i0 < n; i0 += g) {
    double s = oracle_quant_group(v + i0, g, a_format, q, NULL);
    for (int i = 0; i < g; ++i) v[i0 + i] = oracle_e4m3_decode(q[i]) * s;
  }
  free(q);
}

/* Activation quantisation exposed for the test suite: row-major [rows, n]. */
void oracle_quant_rows(const double* v, int rows, int n, int a_format, uint8_t* q,
                       double* scales) {
  int g = group_len(a_format, n);
  for (int r = 0; r < rows; ++r)
    for (int i0 = 0; i0 < n; i0 += g)
      scales[(size_t)r * (n / g) + i0 / g] =
          oracle_quant_group(v + (size_t)r * n + i0, g, a_format, q + (size_t)r * n + i0, NULL);
}

/* ------------------------------------------------------------------ routing
 * Per token: repeatedly take the highest remaining score, the lower expert
 * index winning a tie (scores are compared as given, fp32, +0 == -0).
 * Gate weights are renormalised over the k chosen experts:
 *   softmax: w_j = exp(l_j - l_max) / sum_sel exp(l_i - l_max)
 *   sigmoid: w_j = sig(l_j) / sum_sel sig(l_i)
 *   probs:   w_j = p_j / sum_sel p_i
 */
void oracle_route(const float* scores, int T, int E, int k, int score_fn, int32_t* ids,
                  double* w) {
  char* taken = (char*)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const float* row = scores + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || (double)row[e] > (double)row[best]) best = e;
      }
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
    }
    double sum = 0.0, top = (double)row[ids[(size_t)t * k]];
    double* wt = w + (size_t)t * k;
    for (int j = 0; j < k; ++j) {
      double l = (double)row[ids[(size_t)t * k + j]];
      double v;
      if (score_fn == SCORE_SOFTMAX)
        v = exp(l - top);
      else if (score_fn == SCORE_SIGMOID)
        v = 1.0 / (1.0 + exp(-l));
      else
        v = l;
      wt[j] = v;
      sum += v;
    }
    for (int j = 0; j < k; ++j) wt[j] /= sum;
  }
  free(taken);
}

/* ----------------------------------------------------------------- dispatch
 * counts[e] = number of (t, j) with ids[t, j] == e; m_indptr = exclusive
 * prefix sum (length E+1).  Slots are ordered by expert, then by the flat
 * index t*k + j (a stable counting sort).  gather[slot] = t*k + j and
 * inv[t*k + j] = slot.
 */
void oracle_dispatch(const int32_t* ids, int T, int k, int E, int32_t* counts,
                     int32_t* m_indptr, int32_t* gather, int32_t* inv) {
  int S = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int p = 0; p < S; ++p) counts[ids[p]]++;
  m_indptr[0] = 0;
  for (int e = 0; e < E; ++e) m_indptr[e + 1] = m_indptr[e] + counts[e];
  int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int e = 0; e < E; ++e) next[e] = m_indptr[e];
  for (int p = 0; p < S; ++p) {
    int slot = next[ids[p]]++;
    gather[slot] = p;
    inv[p] = slot;
  }
  free(next);
}

/* Block table for row blocks of height bm: for each expert in ascending
 * order, ceil(counts[e] / bm) entries (e, r * bm).  Returns the entry count;
 * writes at most cap entries as pairs into table. */
int oracle_tile_table(const int32_t* counts, int E, int bm, int32_t* table, int cap) {
  int n = 0;
  for (int e = 0; e < E; ++e)
    for (int r = 0; r * bm < counts[e]; ++r) {
      if (n < cap) {
        table[2 * n] = e;
        table[2 * n + 1] = r * bm;
      }
      ++n;
    }
  return n;
}

/* ------------------------------------------------------------------ experts */
/* Decoded values of every e4m3 and e8m0 code, filled once when the library
 * loads from oracle_e4m3_decode / oracle_e8m0_decode (a lookup in place of
 * recomputing the same value per element). */
static double e4m3_tab[256], e8m0_tab[256];
__attribute__((constructor)) static void oracle_tables(void) {
  for (int c = 0; c < 256; ++c) {
    e4m3_tab[c] = oracle_e4m3_decode((uint8_t)c);
    e8m0_tab[c] = oracle_e8m0_decode((uint8_t)c);
  }
}

typedef struct {
  int w_format;
  const void* codes;   /* one expert's [N, K] matrix */
  const void* scales;  /* per format, or NULL */
  int N, K;
} oracle_mat;

static void dequant_row(const oracle_mat* m, int n, double* out) {
  int K = m->K;
  if (m->w_format == W_BF16) {
    const uint16_t* c = (const uint16_t*)m->codes + (size_t)n * K;
    for (int i = 0; i < K; ++i) out[i] = oracle_bf16_decode(c[i]);
  } else if (m->w_format == W_FP8_CHANNEL) {
    const uint8_t* c = (const uint8_t*)m->codes + (size_t)n * K;
    double s = ((const float*)m->scales)[n];
    for (int i = 0; i < K; ++i) out[i] = e4m3_tab[c[i]] * s;
  } else if (m->w_format == W_FP8_BLOCK128) {
    const uint8_t* c = (const uint8_t*)m->codes + (size_t)n * K;
    const float* s = (const float*)m->scales + (size_t)(n / 128) * (K / 128);
    for (int i = 0; i < K; ++i) out[i] = e4m3_tab[c[i]] * (double)s[i / 128];
  } else { /* W_MXFP4: two e2m1 codes per byte, element 2i in the low nibble */
    const uint8_t* c = (const uint8_t*)m->codes + (size_t)n * (K / 2);
    const uint8_t* s = (const uint8_t*)m->scales + (size_t)n * (K / 32);
    for (int i = 0; i < K; ++i) {
      uint8_t nib = (i & 1) ? (c[i / 2] >> 4) : (c[i / 2] & 0xF);
      out[i] = oracle_e2m1_decode(nib) * e8m0_tab[s[i / 32]];
    }
  }
}

/* out[n] = sum_k a[k] * W[n, k] for every row n of an expert matrix, each
 * sum in ascending k.  Rows are split over threads when `par` is set
 * (callers that already run one token or row per thread pass 0); the split
 * does not change any sum. */
static void matvec(const oracle_mat* m, const double* a, double* out, int par) {
#pragma omp parallel if (par)
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)m->K);
#pragma omp for schedule(static)
    for (int n = 0; n < m->N; ++n) {
      dequant_row(m, n, row);
      double acc = 0.0;
      for (int i = 0; i < m->K; ++i) acc += a[i] * row[i];
      out[n] = acc;
    }
    free(row);
  }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

static double clampd(double v, double lo, double hi) { return v < lo ? lo : (v > hi ? hi : v); }

/*
 * The expert's activation of its gate value g and up value u (LightMoE
 * README, "Compatibility" and "MoE inference": SwiGLU, bounded SwiGLU with
 * an activation clamp, SwiGLU-OAI, GeGLU, ReGLU, and ReLU^2 in the
 * two-weight form).  The pages name these without formulas; the readings:
 *   SwiGLU          SiLU(g) * u
 *   bounded SwiGLU  SiLU(min(g, L)) * clamp(u, -L, L)         (L = limit)
 *   SwiGLU-OAI      g' sigma(1.702 g') (clamp(u, -L, L) + 1), g' = min(g, L)
 *   GeGLU           GELU(g) * u, GELU(z) = z (1 + erf(z / sqrt 2)) / 2
 *   ReGLU           max(g, 0) * u
 *   ReLU^2          max(u, 0)^2 (no gate projection; g is unused)
 */
double oracle_activation(int act, double limit, double g, double u) {
  switch (act) {
    case ACT_SWIGLU_BOUNDED:
      return silu(g < limit ? g : limit) * clampd(u, -limit, limit);
    case ACT_SWIGLU_OAI: {
      double gc = g < limit ? g : limit;
      return gc / (1.0 + exp(-1.702 * gc)) * (clampd(u, -limit, limit) + 1.0);
    }
    case ACT_GEGLU:
      return 0.5 * g * (1.0 + erf(g / sqrt(2.0))) * u;
    case ACT_REGLU:
      return (g > 0.0 ? g : 0.0) * u;
    case ACT_RELU2:
      return u > 0.0 ? u * u : 0.0;
    default:
      return silu(g) * u;
  }
}

/* One expert on one (already dequantised) token row: gated MLP with the
 * intermediate requantised under the activation format.  o has H entries.
 * g is NULL for the two-weight ReLU^2 form. */
static void expert_forward(const oracle_mat* g, const oracle_mat* u, const oracle_mat* d,
                           const double* xq, int a_format, int act, double limit, double* o,
                           int par) {
  int I = u->N;
  double* gv = (double*)malloc(sizeof(double) * (size_t)I);
  double* uv = (double*)malloc(sizeof(double) * (size_t)I);
  if (act == ACT_RELU2) {
    for (int n = 0; n < I; ++n) gv[n] = 0.0;
  } else {
    matvec(g, xq, gv, par);
  }
  matvec(u, xq, uv, par);
  for (int n = 0; n < I; ++n) gv[n] = oracle_activation(act, limit, gv[n], uv[n]);
  quant_dequant_row(gv, I, a_format);
  matvec(d, gv, o, par);
  free(gv);
  free(uv);
}

static size_t code_bytes(int w_format, int N, int K) {
  if (w_format == W_BF16) return (size_t)N * K * 2;
  if (w_format == W_MXFP4) return (size_t)N * K / 2;
  return (size_t)N * K;
}

static size_t scale_bytes(int w_format, int N, int K) {
  if (w_format == W_FP8_CHANNEL) return (size_t)N * 4;
  if (w_format == W_FP8_BLOCK128) return (size_t)(N / 128) * (K / 128) * 4;
  if (w_format == W_MXFP4) return (size_t)N * (K / 32);
  return 0;
}

static oracle_mat expert_mat(int w_format, const void* codes, const void* scales, int e, int N,
                             int K) {
  oracle_mat m;
  m.w_format = w_format;
  m.N = N;
  m.K = K;
  m.codes = (const char*)codes + code_bytes(w_format, N, K) * (size_t)e;
  m.scales = scales ? (const char*)scales + scale_bytes(w_format, N, K) * (size_t)e : NULL;
  return m;
}

/*
 * Layer output for a list of tokens.
 *   x_bits  [T, H] bf16 activations
 *   ids, w  [T, k] routing (from oracle_route, or any valid routing)
 *   w_*     codes [E, N, K] and scales of the routed experts
 *   sh_*    the always-on shared expert (weight 1, outside renormalisation)
 *           when has_shared != 0
 *   tokens  which rows of y to compute; y is [ntok, H] (fp64)
 * y_t = sum_j w[t,j] * expert_{ids[t,j]}(x_t) (+ shared(x_t)), j ascending.
 * Tokens are independent: with several tokens each thread takes whole
 * tokens (every sum is formed exactly as for one token on its own).
 */
void oracle_layer_forward(int H, int I, int E, int k, int w_format, int a_format, int act,
                          double limit, const void* wg, const void* sg, const void* wu, const void* su,
                          const void* wd, const void* sd, int has_shared, int Is,
                          const void* shg, const void* shsg, const void* shu, const void* shsu,
                          const void* shd, const void* shsd, const uint16_t* x_bits,
                          const int32_t* ids, const double* w, const int32_t* tokens, int ntok,
                          double* y) {
  const int tok_par = ntok >= 4;
#pragma omp parallel if (tok_par)
  {
  double* xq = (double*)malloc(sizeof(double) * (size_t)H);
  double* o = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
  for (int i = 0; i < ntok; ++i) {
    int t = tokens[i];
    for (int h = 0; h < H; ++h) xq[h] = oracle_bf16_decode(x_bits[(size_t)t * H + h]);
    if (a_format != A_BF16) quant_dequant_row(xq, H, a_format);
    double* yt = y + (size_t)i * H;
    for (int h = 0; h < H; ++h) yt[h] = 0.0;
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)t * k + j];
      oracle_mat g = expert_mat(w_format, wg, sg, e, I, H);
      oracle_mat u = expert_mat(w_format, wu, su, e, I, H);
      oracle_mat d = expert_mat(w_format, wd, sd, e, H, I);
      expert_forward(&g, &u, &d, xq, a_format, act, limit, o, !tok_par);
      double wj = w[(size_t)t * k + j];
      for (int h = 0; h < H; ++h) yt[h] += wj * o[h];
    }
    if (has_shared) {
      oracle_mat g = expert_mat(w_format, shg, shsg, 0, Is, H);
      oracle_mat u = expert_mat(w_format, shu, shsu, 0, Is, H);
      oracle_mat d = expert_mat(w_format, shd, shsd, 0, H, Is);
      expert_forward(&g, &u, &d, xq, a_format, act, limit, o, !tok_par);
      for (int h = 0; h < H; ++h) yt[h] += o[h];
    }
  }
  free(xq);
  free(o);
  }
}

/* ------------------------------------------------------------ grouped GEMM
 * The grouped projection on its own (LightMoE README, "Grouped GEMM":
 * contiguous expert-major rows delimited by m_indptr; out = A * B^T per
 * expert).  Row r of group e (m_indptr[e] <= r < m_indptr[e+1]) reads
 * activation row a_gather ? a_gather[r] / gather_div : r, dequantised under
 * a_format (codes times the row's, group's or block's scale).
 *   op 0: out[r, n] = sum_k a[r, k] * B0[e, n, k]
 *   op 1: out[r, n] = act(sum_k a B0, sum_k a B1) (oracle_activation), not
 *         requantised; ReLU^2 reads only B1 (B0 may be NULL).
 * out is fp64 [m_indptr[E], N]. */
void oracle_grouped_gemm(int w_format, int a_format, int op, int act, double limit,
                         const void* a, const void* a_scale,
                         const int32_t* a_gather, int gather_div, const int32_t* m_indptr, int E,
                         int N, int K, const void* b0, const void* b0s, const void* b1,
                         const void* b1s, double* out) {
  const int R = m_indptr[E];
#pragma omp parallel
  {
  double* arow = (double*)malloc(sizeof(double) * (size_t)K);
  double* g = (double*)malloc(sizeof(double) * (size_t)N);
  double* u = (double*)malloc(sizeof(double) * (size_t)N);
  /* rows are independent: each thread takes whole rows */
#pragma omp for schedule(dynamic, 4)
  for (int r = 0; r < R; ++r) {
    int e = 0;
    while (m_indptr[e + 1] <= r) ++e;
    const int relu2 = op == 1 && act == ACT_RELU2;
    oracle_mat B0 = expert_mat(w_format, relu2 ? b1 : b0, relu2 ? b1s : b0s, e, N, K);
    oracle_mat B1 = expert_mat(w_format, b1 ? b1 : b0, b1 ? b1s : b0s, e, N, K);
    {
      long src = a_gather ? a_gather[r] / gather_div : r;
      for (int k = 0; k < K; ++k) {
        if (a_format == A_BF16) {
          arow[k] = oracle_bf16_decode(((const uint16_t*)a)[src * K + k]);
          continue;
        }
        double q = oracle_e4m3_decode(((const uint8_t*)a)[src * K + k]);
        double s;
        if (a_format == A_FP8_TOKEN)
          s = ((const float*)a_scale)[src];
        else if (a_format == A_FP8_G128)
          s = ((const float*)a_scale)[src * (K / 128) + k / 128];
        else
          s = oracle_e8m0_decode(((const uint8_t*)a_scale)[src * (K / 32) + k / 32]);
        arow[k] = q * s;
      }
      if (op == 1 && relu2) {
        for (int n = 0; n < N; ++n) g[n] = 0.0;
      } else {
        matvec(&B0, arow, g, 0);
      }
      if (op == 1) {
        matvec(&B1, arow, u, 0);
        for (int n = 0; n < N; ++n) out[(size_t)r * N + n] = oracle_activation(act, limit, g[n], u[n]);
      } else {
        for (int n = 0; n < N; ++n) out[(size_t)r * N + n] = g[n];
      }
    }
  }
  free(arow);
  free(g);
  free(u);
  }
}

/* ---------------------------------------------------------------- backward
 * Gradients of the routed expert layer (LightMoE README, "MoE training" and
 * "Highlights": deterministic dispatch, combine, input-gradient,
 * weight-gradient and router-gradient kernels).  The pages name the
 * gradients but give no formulas; these are the derivatives of the forward
 * above, written out.
 *
 * Partial derivatives of oracle_activation with respect to g and u.  At a
 * clamp boundary the derivative of the branch the forward takes: min(g, L)
 * passes g only for g < L, clamp(u, -L, L) passes u for -L <= u <= L.
 *   SwiGLU          dg = SiLU'(g) u,     du = SiLU(g)
 *                   SiLU'(z) = s(z) (1 + z (1 - s(z))), s the logistic
 *   GeGLU           dg = GELU'(g) u,     du = GELU(g)
 *                   GELU'(z) = Phi(z) + z phi(z) (standard normal cdf, pdf)
 *   ReLU^2          dg = 0,              du = 2 max(u, 0)
 * ReGLU has no backward here (the pages' training set excludes it).
 */
static double sigm(double z) { return 1.0 / (1.0 + exp(-z)); }

void oracle_activation_grad(int act, double limit, double g, double u, double* dg, double* du) {
  switch (act) {
    case ACT_SWIGLU_BOUNDED: {
      const int gin = g < limit, uin = u >= -limit && u <= limit;
      const double gc = gin ? g : limit, uc = clampd(u, -limit, limit);
      const double s = sigm(gc);
      *dg = gin ? s * (1.0 + gc * (1.0 - s)) * uc : 0.0;
      *du = uin ? gc * s : 0.0;
      return;
    }
    case ACT_SWIGLU_OAI: {
      const int gin = g < limit, uin = u >= -limit && u <= limit;
      const double gc = gin ? g : limit, uc = clampd(u, -limit, limit);
      const double s = sigm(1.702 * gc);
      *dg = gin ? (s + 1.702 * gc * s * (1.0 - s)) * (uc + 1.0) : 0.0;
      *du = uin ? gc * s : 0.0;
      return;
    }
    case ACT_GEGLU: {
      const double Phi = 0.5 * (1.0 + erf(g / sqrt(2.0)));
      const double phi = exp(-0.5 * g * g) / sqrt(2.0 * acos(-1.0));
      *dg = (Phi + g * phi) * u;
      *du = g * Phi;
      return;
    }
    case ACT_RELU2:
      *dg = 0.0;
      *du = u > 0.0 ? 2.0 * u : 0.0;
      return;
    default: {
      const double s = sigm(g);
      *dg = s * (1.0 + g * (1.0 - s)) * u;
      *du = g * s;
      return;
    }
  }
}

static double bf16_read(const uint16_t* p, size_t i) { return oracle_bf16_decode(p[i]); }

/*
 * Expert-layer backward for bf16 weights (gate, up [E, I, H]; down
 * [E, H, I]), activations x and upstream gradient dy bf16 [T, H], routing
 * ids and weights w [T, k].  Forward per slot (t, j), e = ids[t, j]:
 *   g = Wg[e] x_t, u = Wu[e] x_t, h = act(g, u), o = Wd[e] h,
 *   y_t = sum_j w[t, j] o.
 * Backward:
 *   r  = Wd[e]^T dy_t                  (gradient at h before the weight)
 *   dw[t, j] = <r, h>                  (= <dy_t, o>: the router's input)
 *   dWd[e] += (w dy_t) h^T
 *   dg = w r * dact/dg, du = w r * dact/du
 *   dWg[e] += dg x_t^T,  dWu[e] += du x_t^T
 *   dx_t = sum_j (Wg[e]^T dg + Wu[e]^T du), j ascending
 * With round_bf16 set, h, w dy_t, dg and du are rounded to bf16 before they
 * multiply anything else (they are the operands of the layer's bf16
 * products); otherwise every quantity stays fp64.  ReLU^2 ignores Wg (may
 * be NULL; dWg is then left untouched).  Outputs fp64: dx [T, H],
 * dwg/dwu [E, I, H], dwd [E, H, I], dw [T, k]; the dW arrays are zeroed
 * here.  Experts are independent: each thread owns whole experts and adds
 * their slots in ascending (t, j) order.
 */
void oracle_expert_backward(int H, int I, int E, int k, int act, double limit,
                            const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                            const uint16_t* x_bits, const int32_t* ids, const double* w, int T,
                            const uint16_t* dy_bits, int round_bf16, double* dx, double* dwg,
                            double* dwu, double* dwd, double* dw) {
  const size_t S = (size_t)T * k;
  const int relu2 = act == ACT_RELU2;
  double* da = (double*)calloc(S * (size_t)H, sizeof(double));   /* per-slot input gradient */
  if (!relu2) memset(dwg, 0, sizeof(double) * (size_t)E * I * H);
  memset(dwu, 0, sizeof(double) * (size_t)E * I * H);
  memset(dwd, 0, sizeof(double) * (size_t)E * H * I);
#pragma omp parallel
  {
  double* xt = (double*)malloc(sizeof(double) * (size_t)H);
  double* dyt = (double*)malloc(sizeof(double) * (size_t)H);
  double* dot = (double*)malloc(sizeof(double) * (size_t)H);
  double* g = (double*)malloc(sizeof(double) * (size_t)I);
  double* u = (double*)malloc(sizeof(double) * (size_t)I);
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  double* r = (double*)malloc(sizeof(double) * (size_t)I);
  double* dg = (double*)malloc(sizeof(double) * (size_t)I);
  double* du = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
  for (int e = 0; e < E; ++e) {
    const uint16_t* Wg = relu2 ? NULL : wg + (size_t)e * I * H;
    const uint16_t* Wu = wu + (size_t)e * I * H;
    const uint16_t* Wd = wd + (size_t)e * H * I;
    double* dWg = relu2 ? NULL : dwg + (size_t)e * I * H;
    double* dWu = dwu + (size_t)e * I * H;
    double* dWd = dwd + (size_t)e * H * I;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j) {
        if (ids[(size_t)t * k + j] != e) continue;
        const size_t slot = (size_t)t * k + j;
        const double wj = w[slot];
        for (int c = 0; c < H; ++c) {
          xt[c] = bf16_read(x_bits, (size_t)t * H + c);
          dyt[c] = bf16_read(dy_bits, (size_t)t * H + c);
          dot[c] = round_bf16 ? oracle_bf16_round(wj * dyt[c]) : wj * dyt[c];
        }
        /* forward of this slot */
        for (int n = 0; n < I; ++n) {
          double ag = 0.0, au = 0.0;
          for (int c = 0; c < H; ++c) {
            if (!relu2) ag += bf16_read(Wg, (size_t)n * H + c) * xt[c];
            au += bf16_read(Wu, (size_t)n * H + c) * xt[c];
          }
          g[n] = ag;
          u[n] = au;
          const double hv = oracle_activation(act, limit, ag, au);
          h[n] = round_bf16 ? oracle_bf16_round(hv) : hv;
          r[n] = 0.0;
        }
        /* r = Wd^T dy_t, and dWd += (w dy_t) h^T */
        for (int c = 0; c < H; ++c) {
          const uint16_t* wrow = Wd + (size_t)c * I;
          double* drow = dWd + (size_t)c * I;
          for (int n = 0; n < I; ++n) {
            r[n] += bf16_read(wrow, n) * dyt[c];
            drow[n] += dot[c] * h[n];
          }
        }
        double acc = 0.0;
        for (int n = 0; n < I; ++n) acc += r[n] * h[n];
        dw[slot] = acc;
        for (int n = 0; n < I; ++n) {
          double pg, pu;
          oracle_activation_grad(act, limit, g[n], u[n], &pg, &pu);
          const double dh = wj * r[n];
          dg[n] = round_bf16 ? oracle_bf16_round(dh * pg) : dh * pg;
          du[n] = round_bf16 ? oracle_bf16_round(dh * pu) : dh * pu;
        }
        double* dat = da + slot * (size_t)H;
        for (int n = 0; n < I; ++n) {
          for (int c = 0; c < H; ++c) {
            if (!relu2) {
              dWg[(size_t)n * H + c] += dg[n] * xt[c];
              dat[c] += dg[n] * bf16_read(Wg, (size_t)n * H + c);
            }
            dWu[(size_t)n * H + c] += du[n] * xt[c];
            dat[c] += du[n] * bf16_read(Wu, (size_t)n * H + c);
          }
        }
      }
  }
  free(xt); free(dyt); free(dot); free(g); free(u); free(h); free(r); free(dg); free(du);
  }
  /* dispatch backward: each token's input gradient, j ascending */
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += da[((size_t)t * k + j) * H + c];
      dx[(size_t)t * H + c] = acc;
    }
  free(da);
}

/*
 * Router backward: gradient of a loss with respect to the router scores
 * [T, E], given its gradient dw [T, k] with respect to the renormalised
 * top-k weights (the selection itself is piecewise constant).  With
 * m = sum_j w_j dw_j over the token's k slots, for a selected expert i:
 *   softmax  w_i = exp(l_i) / sum_sel exp(l):  dl_i = w_i (dw_i - m)
 *   sigmoid  w_i = s_i / S, S = sum_sel s:     dl_i = s_i (1 - s_i) (dw_i - m) / S
 *   probs    w_i = p_i / P, P = sum_sel p:     dp_i = (dw_i - m) / P
 * Unselected scores get 0.  w is the oracle's fp64 routing weights.
 */
void oracle_router_backward(const float* scores, const int32_t* ids, const double* w,
                            const double* dw, int T, int E, int k, int score_fn, double* dscores) {
  memset(dscores, 0, sizeof(double) * (size_t)T * E);
  for (int t = 0; t < T; ++t) {
    double m = 0.0, den = 0.0;
    for (int j = 0; j < k; ++j) m += w[(size_t)t * k + j] * dw[(size_t)t * k + j];
    for (int j = 0; j < k; ++j) {
      const double l = scores[(size_t)t * E + ids[(size_t)t * k + j]];
      den += score_fn == SCORE_SIGMOID ? sigm(l) : l;
    }
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      const double l = scores[(size_t)t * E + e];
      const double d = dw[(size_t)t * k + j] - m;
      double v;
      if (score_fn == SCORE_SOFTMAX) v = w[(size_t)t * k + j] * d;
      else if (score_fn == SCORE_SIGMOID) v = sigm(l) * (1.0 - sigm(l)) * d / den;
      else v = d / den;
      dscores[(size_t)t * E + e] = v;
    }
  }
}
