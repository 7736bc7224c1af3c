/*
 * moe_oracle.c -- plain, slow CPU oracle for the fused Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this file.  Only the
 * test-suite, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no source with the GPU path.
 *
 * What is computed (a fused MoE layer: token routing, data shuffling, the
 * expert network and expert aggregation as one batched operation):
 *   - readmex.ai, "AWS details fused MoE kernel optimizations on SageMaker, up
 *     to 10% throughput gain", summary paragraphs: the fused MoE op merges
 *     token routing, data shuffling and the expert computation;
 *   - codebridge-ai.com, "aws-moe-kernel-wgmma-triton-ttft", section
 *     "2. Backend routing": scaling, matmul and aggregation are the steps that
 *     the fused FP8 pass combines;
 *   - agentic-affairs.com, section "Triton improves the FP8 execution path":
 *     FP8 tensor scaling, matrix multiplication and expert aggregation.
 * The pages name the pieces but give no formulas.  The layer specification
 * fixes them: renormalised top-k softmax gating, a SwiGLU expert FFN with
 * gate/up packed in w13 followed by w2, bf16 or FP8 e4m3 weights with fp32
 * per-tensor scales, dynamic per-tensor activation quantisation in FP8 mode.
 * Every place where a reading had to be chosen is marked "Reading:".
 *
 * Precision: all sums, the SiLU and the combine are done in double.  Values
 * are rounded only where the method stores a tensor in a narrower type
 * (h and out in the activation type, fp32 scales, e4m3 codes).  Decisions
 * that pick an integer (an e4m3 code) are taken on the fp32 product x*r,
 * which is the precision the layer defines for the scale.
 *
 * Parallelism: OpenMP over independent output elements only; every reduction
 * runs in one thread in ascending index order.
 *
 * Data types (wdtype): 0 = fp32, 1 = bf16, 2 = FP8 e4m3 (OCP e4m3fn).
 *   fp32 mode : x, w13, w2, h, out are fp32.
 *   bf16 mode : x, w13, w2, h, out are bf16 (passed as raw uint16 bits).
 *   FP8 mode  : x, h, out are bf16 bits; w13, w2 are e4m3 codes with one fp32
 *               scale per expert and matrix.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MOE_F32 0
#define MOE_BF16 1
#define MOE_FP8 2

/* ------------------------------------------------------------------------ */
/* bf16: 1 sign, 8 exponent, 7 fraction bits; the upper half of an fp32.     */
/* ------------------------------------------------------------------------ */

/* Exact value of a bf16 bit pattern. */
double oracle_bf16_decode(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/*
 * Round a double to the nearest bf16 value, ties to even, and return its bit
 * pattern.  bf16 keeps 8 significant bits; for |v| >= 2^-126 the spacing of
 * bf16 values in the binade [2^(e-1), 2^e) is 2^(e-8), below it the fixed
 * subnormal spacing 2^-133.  v/q is exact in double (power-of-two scaling) and
 * rint() rounds it to an integer with ties to even (default rounding mode).
 * Overflow past the largest finite bf16 gives infinity (IEEE round to
 * nearest); it does not occur in this layer.
 */
uint16_t oracle_bf16_round(double v) {
  if (isnan(v)) return 0x7fc0;
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  int e;
  frexp(v, &e); /* |v| in [2^(e-1), 2^e) */
  int qexp = (e - 1 >= -126) ? e - 8 : -133;
  double r = rint(ldexp(v, -qexp));
  double rv = ldexp(r, qexp);
  /* rv is a bf16 value (or overflowed); convert via float exactly. */
  float f = (float)rv;
  if (isinf(f) || fabs(rv) > 3.3895313892515355e38) f = (rv > 0) ? INFINITY : -INFINITY;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* FP8 e4m3 in the OCP "e4m3fn" form: 1 sign, 4 exponent (bias 7), 3 fraction */
/* bits; no infinities; S.1111.111 is NaN; largest finite 448; subnormals    */
/* m * 2^-9.                                                                  */
/* Reading: the layer's FP8 is this format (the pages only say "FP8").       */
/* ------------------------------------------------------------------------ */

/* Exact value of an e4m3 code (closed form of the format). */
double oracle_e4m3_decode(uint8_t c) {
  int s = (c >> 7) & 1, ex = (c >> 3) & 15, m = c & 7;
  double v;
  if (ex == 15 && m == 7) return NAN;
  if (ex == 0)
    v = ldexp((double)m, -9); /* subnormal: m/8 * 2^-6 */
  else
    v = ldexp(1.0 + m / 8.0, ex - 7);
  return s ? -v : v;
}

/*
 * Nearest e4m3 value to v, ties to even, saturating to +-448 ("satfinite"):
 * values beyond the largest finite magnitude become +-448, never NaN.
 * Reading: round-to-nearest-even and saturation are the conversion rules of
 * the quantiser; the pages do not state them.
 */
uint8_t oracle_e4m3_encode(float vf) {
  double v = (double)vf;
  if (isnan(v)) return 0x7f;
  uint8_t sign = (signbit(v) ? 0x80 : 0x00);
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int qexp = (e - 1 >= -6) ? e - 4 : -9; /* 4 significant bits, else subnormal step */
  double r = rint(ldexp(a, -qexp));
  double q = ldexp(r, qexp);
  if (q > 448.0) q = 448.0;
  if (q == 0.0) return sign;
  /* encode the exactly representable magnitude q */
  int qe;
  frexp(q, &qe);
  int ex = qe - 1 + 7; /* biased exponent if normal */
  uint8_t code;
  if (ex <= 0) {
    int m = (int)ldexp(q, 9); /* subnormal: q = m * 2^-9 */
    code = (uint8_t)m;
  } else {
    double frac = ldexp(q, -(qe - 1)) - 1.0; /* in [0, 1) with step 1/8 */
    int m = (int)(frac * 8.0);
    code = (uint8_t)((ex << 3) | m);
  }
  return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------ */
/* element access for the three storage types                               */
/* ------------------------------------------------------------------------ */

static double g_e4m3_table[256];
static int g_table_ready = 0;

static void ensure_table(void) {
  if (!g_table_ready) {
    for (int i = 0; i < 256; i++) g_e4m3_table[i] = oracle_e4m3_decode((uint8_t)i);
    g_table_ready = 1;
  }
}

/* Value of element i of a weight matrix stored in dtype dt (unscaled). */
static inline double wval(const void* w, int dt, size_t i) {
  if (dt == MOE_F32) return (double)((const float*)w)[i];
  if (dt == MOE_BF16) return oracle_bf16_decode(((const uint16_t*)w)[i]);
  return g_e4m3_table[((const uint8_t*)w)[i]];
}

/* Value of element i of an activation (x or h): fp32 in fp32 mode, else bf16. */
static inline double aval(const void* a, int dt, size_t i) {
  if (dt == MOE_F32) return (double)((const float*)a)[i];
  return oracle_bf16_decode(((const uint16_t*)a)[i]);
}

/* Store an activation value: fp32 in fp32 mode, else bf16 (RNE). */
static inline void astore(void* a, int dt, size_t i, double v) {
  if (dt == MOE_F32)
    ((float*)a)[i] = (float)v;
  else
    ((uint16_t*)a)[i] = oracle_bf16_round(v);
}

/* ------------------------------------------------------------------------ */
/* Step 0 (optional): the router's logits.                                    */
/* Token routing starts from a score of every expert for every token          */
/* (readmex.ai summary: routing is the first stage of the fused op).  The     */
/* pages give no formula; Reading: a bias-free linear router, logits[t][e] =  */
/* sum_h x[t][h] * wg[e][h], with wg stored in the activation type (bf16, or  */
/* fp32 in fp32 mode) as one row per expert, summed exactly (double,          */
/* ascending h) and rounded once to fp32.                                     */
/* ------------------------------------------------------------------------ */
void oracle_router_logits(int adt, int T, int H, int E, const void* x, const void* wg,
                          float* logits) {
#pragma omp parallel for schedule(static)
  for (long te = 0; te < (long)T * E; te++) {
    const long t = te / E, e = te % E;
    double acc = 0.0;
    for (int h = 0; h < H; h++)
      acc += aval(x, adt, (size_t)t * H + h) * aval(wg, adt, (size_t)e * H + h);
    logits[te] = (float)acc;
  }
}

/* ------------------------------------------------------------------------ */
/* Step 1: top-k softmax gating.                                             */
/* Token routing is the first stage of the fused op (readmex.ai summary;     */
/* agentic-affairs.com "Swap-AB targets matrix execution on Hopper").        */
/* Selection: experts ordered by logit descending, ties to the lower expert  */
/* index (Reading: the pages give no tie rule).  -0 and +0 compare equal.    */
/* renormalize=1: w_j = exp(l_j - m) / sum over the k selected of exp(. - m) */
/* with m the largest selected logit; this equals the full softmax           */
/* restricted to the selected experts and rescaled to sum to one.            */
/* renormalize=0: w_j = full softmax probability of the selected expert.     */
/* ------------------------------------------------------------------------ */
void oracle_topk_gating(const float* logits, int T, int E, int k, int renormalize,
                        int32_t* topk_ids, float* topk_weights) {
  for (int t = 0; t < T; t++) {
    const float* l = logits + (size_t)t * E;
    /* selection: k passes, each taking the best not-yet-taken expert */
    for (int j = 0; j < k; j++) {
      int best = -1;
      for (int e = 0; e < E; e++) {
        int taken = 0;
        for (int q = 0; q < j; q++)
          if (topk_ids[(size_t)t * k + q] == e) taken = 1;
        if (taken) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep lower index */
      }
      topk_ids[(size_t)t * k + j] = best;
    }
    double m = (double)l[topk_ids[(size_t)t * k]];
    if (renormalize) {
      double s = 0.0;
      for (int j = 0; j < k; j++) s += exp((double)l[topk_ids[(size_t)t * k + j]] - m);
      for (int j = 0; j < k; j++)
        topk_weights[(size_t)t * k + j] =
            (float)(exp((double)l[topk_ids[(size_t)t * k + j]] - m) / s);
    } else {
      /* m is the row maximum: the first selected expert has the largest logit */
      double s = 0.0;
      for (int e = 0; e < E; e++) s += exp((double)l[e] - m);
      for (int j = 0; j < k; j++)
        topk_weights[(size_t)t * k + j] =
            (float)(exp((double)l[topk_ids[(size_t)t * k + j]] - m) / s);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Step 2: grouping ("data shuffling", readmex.ai summary).                   */
/* A pair is (t, j), flat index f = t*k + j.  counts[e] = #pairs routed to e, */
/* offsets = exclusive prefix sum (offsets[E] = T*k).  sorted_ids lists the   */
/* pairs grouped by expert ascending and, inside an expert, by f ascending    */
/* (Reading: the pages leave the order inside an expert open; the stable     */
/* order is the one that is unique).  inv_perm[f] = position of f.           */
/* ------------------------------------------------------------------------ */
void oracle_align_sort(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_ids, int32_t* inv_perm) {
  long n = (long)T * k;
  for (int e = 0; e < E; e++) counts[e] = 0;
  for (long f = 0; f < n; f++) counts[topk_ids[f]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
  long pos = 0;
  for (int e = 0; e < E; e++)
    for (long f = 0; f < n; f++)
      if (topk_ids[f] == e) {
        sorted_ids[pos] = (int32_t)f;
        if (inv_perm) inv_perm[f] = (int32_t)pos;
        pos++;
      }
}

/* ------------------------------------------------------------------------ */
/* Step 3: dynamic per-tensor FP8 quantisation of an activation tensor.       */
/* FP8 tensor scaling is part of the fused pass (agentic-affairs.com,        */
/* "Triton improves the FP8 execution path").                                */
/* Reading: A = max |a| over the whole tensor; s = fl32(A / 448) is the      */
/* dequantisation scale; the codes use r = fl32(448 / A); A = 0 gives        */
/* s = r = 1.  code_i = e4m3(fl32(a_i * r)).  Writes codes (if non-NULL) and */
/* returns s.  The two divisions and the product are single fp32 operations. */
/* ------------------------------------------------------------------------ */
float oracle_act_quant(const void* a, int adt, long n, uint8_t* codes, float* r_out) {
  double A = 0.0;
  for (long i = 0; i < n; i++) {
    double v = fabs(aval(a, adt, i));
    if (v > A) A = v;
  }
  float Af = (float)A; /* exact: A is a bf16 value */
  volatile float s = 1.0f, r = 1.0f;
  if (Af > 0.0f) {
    s = Af / 448.0f;
    r = 448.0f / Af;
  }
  if (codes) {
    for (long i = 0; i < n; i++) {
      volatile float p = (float)aval(a, adt, i) * r;
      codes[i] = oracle_e4m3_encode(p);
    }
  }
  if (r_out) *r_out = r;
  return s;
}

/* expert owning sorted position p (offsets is the exclusive scan of counts) */
static int expert_of_position(const int32_t* offsets, int E, long p) {
  int e = 0;
  while (e < E - 1 && offsets[e + 1] <= p) e++;
  return e;
}

/* ------------------------------------------------------------------------ */
/* Step 4: expert gate/up projection with SwiGLU, for the pairs in sorted     */
/* order ("specialized network calculations", readmex.ai summary; "matrix    */
/* multiplication", agentic-affairs.com FP8 section).                         */
/* Layout (Reading): w13 is [E, 2I, H], rows 0..I-1 the gate projection,      */
/* rows I..2I-1 the up projection, H contiguous.  For sorted position p with  */
/* pair f = sorted_ids[p], token t = f / k, expert e (from offsets):         */
/*   g_n = sum_h xa[t,h] * W13[e,n,h],   u_n = sum_h xa[t,h] * W13[e,I+n,h]    */
/*   FP8: c = fl32(s_x * s_w13[e]), g_n *= c, u_n *= c                        */
/*   h[p,n] = silu(g_n) * u_n, silu(z) = z / (1 + exp(-z)),                   */
/* stored in the activation type.  xa is x in fp32/bf16 mode and the decoded  */
/* e4m3 codes of x in FP8 mode (scale applied in c, not to xa).              */
/* positions == NULL: all T*k positions; else only the listed ones (rows of  */
/* h not listed are left untouched).                                          */
/* Writes s_x (FP8 mode) to *s_x_out and returns nothing else; the scale of   */
/* h is computed separately by oracle_act_quant over the finished h.         */
/* ------------------------------------------------------------------------ */
void oracle_w13_swiglu(int wdtype, int T, int H, int E, int k, int I, const void* x,
                       const void* w13, const float* w13_scale, const int32_t* sorted_ids,
                       const int32_t* offsets, const int32_t* positions, long n_positions,
                       void* h, float* s_x_out) {
  ensure_table();
  long n_pairs = (long)T * k;
  double* xa = (double*)malloc(sizeof(double) * (size_t)T * H);
  float s_x = 1.0f;
  if (wdtype == MOE_FP8) {
    uint8_t* xq = (uint8_t*)malloc((size_t)T * H);
    s_x = oracle_act_quant(x, MOE_BF16, (long)T * H, xq, NULL);
    for (long i = 0; i < (long)T * H; i++) xa[i] = g_e4m3_table[xq[i]];
    free(xq);
  } else {
    for (long i = 0; i < (long)T * H; i++) xa[i] = aval(x, wdtype, i);
  }
  if (s_x_out) *s_x_out = s_x;
  long np = positions ? n_positions : n_pairs;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (long q = 0; q < np; q++) {
    for (int n = 0; n < I; n++) {
      long p = positions ? positions[q] : q;
      int f = sorted_ids[p];
      int t = f / k;
      int e = expert_of_position(offsets, E, p);
      size_t wg = ((size_t)e * 2 * I + n) * H;
      size_t wu = ((size_t)e * 2 * I + I + n) * H;
      double g = 0.0, u = 0.0;
      for (int hh = 0; hh < H; hh++) g += xa[(size_t)t * H + hh] * wval(w13, wdtype, wg + hh);
      for (int hh = 0; hh < H; hh++) u += xa[(size_t)t * H + hh] * wval(w13, wdtype, wu + hh);
      if (wdtype == MOE_FP8) {
        volatile float c = s_x * w13_scale[e];
        g *= (double)c;
        u *= (double)c;
      }
      double hv = g / (1.0 + exp(-g)) * u;
      astore(h, wdtype, (size_t)p * I + n, hv);
    }
  }
  free(xa);
}

/* ------------------------------------------------------------------------ */
/* Step 5: expert down projection.  w2 is [E, H, I] (Reading), I contiguous.  */
/* For sorted position p of expert e:                                         */
/*   y[p,m] = sum_n ha[p,n] * W2[e,m,n]                                       */
/*   FP8: ha = decoded e4m3 codes of h under the per-tensor scale s_h (step 3 */
/*   applied to all of h), and y *= fl32(s_h * s_w2[e]).                      */
/* Reading: h is quantised in FP8 mode (dynamic, per tensor), like x.         */
/* y is kept in double (the fp32 intermediate of the layer is not rounded    */
/* here; the oracle keeps full precision until the output is stored).        */
/* h must hold all T*k rows: the FP8 scale of h is a maximum over all of it. */
/* positions: as in step 4; y row q belongs to positions[q].                  */
/* ------------------------------------------------------------------------ */
void oracle_w2(int wdtype, int T, int H, int E, int k, int I, const void* h, const void* w2,
               const float* w2_scale, const int32_t* offsets, const int32_t* positions,
               long n_positions, double* y, float* s_h_out) {
  ensure_table();
  long n_pairs = (long)T * k;
  double* ha = (double*)malloc(sizeof(double) * (size_t)n_pairs * I);
  float s_h = 1.0f;
  if (wdtype == MOE_FP8) {
    uint8_t* hq = (uint8_t*)malloc((size_t)n_pairs * I);
    s_h = oracle_act_quant(h, MOE_BF16, n_pairs * I, hq, NULL);
    for (long i = 0; i < n_pairs * I; i++) ha[i] = g_e4m3_table[hq[i]];
    free(hq);
  } else {
    for (long i = 0; i < n_pairs * I; i++) ha[i] = aval(h, wdtype, i);
  }
  if (s_h_out) *s_h_out = s_h;
  long np = positions ? n_positions : n_pairs;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (long q = 0; q < np; q++) {
    for (int m = 0; m < H; m++) {
      long p = positions ? positions[q] : q;
      int e = expert_of_position(offsets, E, p);
      size_t wr = ((size_t)e * H + m) * I;
      double acc = 0.0;
      for (int n = 0; n < I; n++) acc += ha[(size_t)p * I + n] * wval(w2, wdtype, wr + n);
      if (wdtype == MOE_FP8) {
        volatile float c = s_h * w2_scale[e];
        acc *= (double)c;
      }
      y[(size_t)q * H + m] = acc;
    }
  }
  free(ha);
}

/* ------------------------------------------------------------------------ */
/* Step 6: expert aggregation (codebridge-ai.com "2. Backend routing";        */
/* agentic-affairs.com FP8 section).                                          */
/*   out[t,m] = sum_{j<k} w[t,j] * y[inv_perm[t*k+j], m], in slot order,      */
/* rounded once to the output type.                                           */
/* y is indexed by sorted position and given in double.  out_exact (may be   */
/* NULL) receives the same sums before that final rounding.                  */
/* ------------------------------------------------------------------------ */
void oracle_combine(int wdtype, int T, int H, int k, const double* y, const int32_t* inv_perm,
                    const float* topk_weights, void* out, double* out_exact) {
#pragma omp parallel for collapse(2)
  for (int t = 0; t < T; t++) {
    for (int m = 0; m < H; m++) {
      double acc = 0.0;
      for (int j = 0; j < k; j++) {
        long p = inv_perm[(size_t)t * k + j];
        acc += (double)topk_weights[(size_t)t * k + j] * y[(size_t)p * H + m];
      }
      astore(out, wdtype, (size_t)t * H + m, acc);
      if (out_exact) out_exact[(size_t)t * H + m] = acc;
    }
  }
}

/* Same as oracle_combine but y is fp32 (the step interface of the layer). */
void oracle_combine_f32(int wdtype, int T, int H, int k, const float* y, const int32_t* inv_perm,
                        const float* topk_weights, void* out) {
#pragma omp parallel for collapse(2)
  for (int t = 0; t < T; t++) {
    for (int m = 0; m < H; m++) {
      double acc = 0.0;
      for (int j = 0; j < k; j++) {
        long p = inv_perm[(size_t)t * k + j];
        acc += (double)topk_weights[(size_t)t * k + j] * (double)y[(size_t)p * H + m];
      }
      astore(out, wdtype, (size_t)t * H + m, acc);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* The whole layer: routing, grouping, gate/up + SwiGLU, (FP8: h scale),      */
/* down projection, aggregation.  Because the FP8 scale of h is a maximum    */
/* over every routed pair, all of h is finished before any down projection. */
/* Optional outputs (may be NULL): topk ids/weights, counts, offsets,         */
/* sorted ids, inverse permutation, h (sorted order), scales[2] = s_x, s_h,  */
/* out_exact = out before its rounding to the output type (double).          */
/* Returns 0, or -1 if an allocation fails.                                   */
/* ------------------------------------------------------------------------ */
int oracle_forward(int wdtype, int T, int H, int E, int k, int I, int renormalize,
                   const void* x, const float* logits, const void* w13, const float* w13_scale,
                   const void* w2, const float* w2_scale, void* out, int32_t* ids_out,
                   float* w_out, int32_t* counts_out, int32_t* offsets_out,
                   int32_t* sorted_out, int32_t* inv_out, void* h_out, float* scales_out,
                   double* out_exact) {
  long n_pairs = (long)T * k;
  size_t abytes = (wdtype == MOE_F32) ? 4 : 2;
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_pairs + 1));
  float* w = (float*)malloc(sizeof(float) * (size_t)(n_pairs + 1));
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* sorted_ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_pairs + 1));
  int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_pairs + 1));
  void* h = malloc(abytes * (size_t)(n_pairs * I + 1));
  double* y = (double*)malloc(sizeof(double) * (size_t)(n_pairs * H + 1));
  if (!ids || !w || !counts || !offsets || !sorted_ids || !inv || !h || !y) return -1;

  oracle_topk_gating(logits, T, E, k, renormalize, ids, w);
  oracle_align_sort(ids, T, k, E, counts, offsets, sorted_ids, inv);
  float s_x = 1.0f, s_h = 1.0f;
  oracle_w13_swiglu(wdtype, T, H, E, k, I, x, w13, w13_scale, sorted_ids, offsets, NULL, 0, h,
                    &s_x);
  oracle_w2(wdtype, T, H, E, k, I, h, w2, w2_scale, offsets, NULL, 0, y, &s_h);
  oracle_combine(wdtype, T, H, k, y, inv, w, out, out_exact);

  if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)n_pairs);
  if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)n_pairs);
  if (counts_out) memcpy(counts_out, counts, sizeof(int32_t) * (size_t)E);
  if (offsets_out) memcpy(offsets_out, offsets, sizeof(int32_t) * (size_t)(E + 1));
  if (sorted_out) memcpy(sorted_out, sorted_ids, sizeof(int32_t) * (size_t)n_pairs);
  if (inv_out) memcpy(inv_out, inv, sizeof(int32_t) * (size_t)n_pairs);
  if (h_out) memcpy(h_out, h, abytes * (size_t)n_pairs * I);
  if (scales_out) {
    scales_out[0] = s_x;
    scales_out[1] = s_h;
  }
  free(ids); free(w); free(counts); free(offsets); free(sorted_ids); free(inv); free(h); free(y);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The second fused kernel of the pages: inverse rotary position embedding   */
/* followed by per-head FP8 quantisation, over a token count that changes    */
/* from call to call (codebridge-ai.com, "aws-moe-kernel-wgmma-triton-ttft", */
/* section "3. Kill JIT recompilation": a fused rotary-embedding plus FP8    */
/* quantisation kernel; agentic-affairs.com, "Removing recompilation         */
/* improves the first-token result": the kernel's variable-length            */
/* parameters; modelsatwork.news, "The three changes").  The pages give no   */
/* formula; Readings:                                                         */
/*  - x [T, n_heads, head_dim] bf16, one position per token (int32);          */
/*  - the rotary embedding rotates coordinate pairs of the first rot_dim     */
/*    values of each head by the angle of the token's position; the angle's  */
/*    cosine and sine come from a table cos_sin [max_pos, rot_dim] fp32,     */
/*    row p = cos of the rot_dim/2 pair angles, then their sines;             */
/*  - pairs are (i, i + rot_dim/2) ("rotate half"), or (2i, 2i+1) when       */
/*    interleaved = 1; values past rot_dim pass through;                      */
/*  - "inverse" is the rotation by the negative angle (the transpose of the  */
/*    forward rotation), which undoes a forward rotary embedding:            */
/*      y_a = x_a c + x_b s,   y_b = x_b c - x_a s   for pair (a, b);        */
/*    each product and the sum are single fp32 operations (no fused          */
/*    multiply-add), since the codes are decided on y;                        */
/*  - "per head" quantisation: one dynamic scale per (token, head), the      */
/*    same rule as the layer's activations: A = max |y| over the head,       */
/*    s = fl32(A / 448), codes e4m3(fl32(y * fl32(448 / A))), A = 0 giving    */
/*    s = 1 and multiplier 1.                                                 */
/* A position outside [0, max_pos) breaks the contract; it is clamped into   */
/* the table.  Writes codes [T, n_heads, head_dim], scales [T, n_heads] and,  */
/* if y_out is non-NULL, the rotated values y (fp32) before quantisation.    */
/* ------------------------------------------------------------------------ */
void oracle_inv_rope_fp8(const uint16_t* x, const int32_t* positions, const float* cos_sin,
                         int T, int n_heads, int head_dim, int rot_dim, int max_pos,
                         int interleaved, float* y_out, uint8_t* codes, float* scales) {
  const int half = rot_dim / 2;
  float* y = (float*)malloc(sizeof(float) * (size_t)(head_dim > 0 ? head_dim : 1));
  for (long th = 0; th < (long)T * n_heads; th++) {
    const long t = th / n_heads;
    long p = positions[t];
    if (p < 0) p = 0;
    if (p >= max_pos) p = max_pos - 1;
    const float* cs = cos_sin + (size_t)p * rot_dim;
    const uint16_t* xh = x + (size_t)th * head_dim;
    for (int d = 0; d < head_dim; d++) y[d] = (float)oracle_bf16_decode(xh[d]);
    for (int i = 0; i < half; i++) {
      const int a = interleaved ? 2 * i : i;
      const int b = interleaved ? 2 * i + 1 : i + half;
      const float xa = (float)oracle_bf16_decode(xh[a]);
      const float xb = (float)oracle_bf16_decode(xh[b]);
      volatile float c = cs[i], s = cs[half + i];
      volatile float p1 = xa * c, p2 = xb * s, p3 = xb * c, p4 = xa * s;
      volatile float ya = p1 + p2, yb = p3 - p4;
      y[a] = ya;
      y[b] = yb;
    }
    double A = 0.0;
    for (int d = 0; d < head_dim; d++)
      if (fabs((double)y[d]) > A) A = fabs((double)y[d]);
    float Af = (float)A; /* exact: A is an fp32 value */
    volatile float sc = 1.0f, r = 1.0f;
    if (Af > 0.0f) {
      sc = Af / 448.0f;
      r = 448.0f / Af;
    }
    for (int d = 0; d < head_dim; d++) {
      volatile float q = y[d] * r;
      codes[(size_t)th * head_dim + d] = oracle_e4m3_encode(q);
      if (y_out) y_out[(size_t)th * head_dim + d] = y[d];
    }
    scales[th] = sc;
  }
  free(y);
}

/* ------------------------------------------------------------------------ */
/* array forms of the codecs (for exhaustive checks)                         */
/* ------------------------------------------------------------------------ */
void oracle_e4m3_encode_array(const float* v, long n, uint8_t* out) {
  for (long i = 0; i < n; i++) out[i] = oracle_e4m3_encode(v[i]);
}
void oracle_e4m3_decode_array(const uint8_t* c, long n, double* out) {
  for (long i = 0; i < n; i++) out[i] = oracle_e4m3_decode(c[i]);
}
void oracle_bf16_round_array(const double* v, long n, uint16_t* out) {
  for (long i = 0; i < n; i++) out[i] = oracle_bf16_round(v[i]);
}
