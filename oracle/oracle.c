/*
 * oracle.c -- plain, slow CPU reference of the routed MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  The GPU library never links, loads or calls this
 * file; only the test suite, the package smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or table with the GPU path
 * or with the input generators: it reads the same input bytes and decodes
 * them with its own code.
 *
 * Everything is scalar C in double precision, written as the definitions
 * read, with no blocking, fusion or reordering.
 *
 * What the layer computes, and where it comes from:
 *  - Routing.  Each token wakes only a handful of experts (10 of the 512 in a
 *    layer; 10 of 24,576 across the 48 layers of the 125B model): Strata
 *    feature, tech.hub77a.com, summary table row "핵심 기법" and section
 *    "2. 왜 대단한가" (1); the router's choice decides which experts run,
 *    ibid. (2).  The selection is the k largest router logits, ties going to
 *    the lower expert id; the gate weights are the softmax of the k selected
 *    logits, so they sum to one.
 *  - Expert FFN.  SwiGLU: y = Wd (silu(Wg x) * (Wu x)), silu(z) = z/(1+e^-z),
 *    no biases; Wg, Wu are [I x H], Wd is [H x I].
 *  - Weights.  The engine's fast size is a 2-bit class quantization (Q2_0)
 *    (same page, speed table in section "3. 바로 써먹기"); the format used here
 *    is blocks of 32 weights along each row with an fp16 scale s and fp16 min
 *    m and b-bit unsigned codes (b = 2, 3 or 4), weight = s*q + m.  Bytes per
 *    weight = b/8 + 4/32, the same block-32 accounting that gives the 0.5625
 *    bytes/value printed for Q4_0 on the KATANA page (trawling.dev/post/3323,
 *    section "실행 환경과 메모리 구성").
 *  - Combine.  out[t] = residual[t] + sum_j w[t,j] * y[t,j], j ascending.
 *
 * Byte layout (decoded here from its description, not from any other code):
 *   code plane of a [R x K] matrix: per row K*b/32 little-endian 32-bit words;
 *   b = 2, 4: word w holds columns w*(32/b) .. w*(32/b) + 32/b - 1; column c of
 *   the word is at bit 16*(c mod 2) + b*floor(c/2).  b = 3 (3-bit size classes
 *   are ranked on the same page; their layout is not given there, so this one
 *   is a reading): three words per 32-column block, the low two bits of each
 *   code in words 0-1 laid out as for b = 2, the high bit of block column j in
 *   word 2 at bit 16*(j mod 2) + floor(j/2).
 *   scale/min plane: per row K/32 words; low half = scale, high half = min
 *   (IEEE binary16 each).
 *   expert blob: Wg codes, Wg s/m, Wu codes, Wu s/m, Wd codes, Wd s/m, each
 *   plane starting at the next multiple of 256 bytes; blob size = end of the
 *   last plane rounded up to a multiple of 256.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- number formats ------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 0x1F, f = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-10 * 2^-14 */
  else if (e == 31)
    v = (f == 0) ? INFINITY : NAN;
  else
    v = ldexp(1.0 + (double)f / 1024.0, e - 15);
  return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16(uint16_t b) {
  int sign = (b >> 15) & 1, e = (b >> 7) & 0xFF, f = b & 0x7F;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133); /* f * 2^-7 * 2^-126 */
  else if (e == 255)
    v = (f == 0) ? INFINITY : NAN;
  else
    v = ldexp(1.0 + (double)f / 128.0, e - 127);
  return sign ? -v : v;
}

/* ---- weight format -------------------------------------------------------- */

static int64_t round_up_256(int64_t v) { return (v + 255) / 256 * 256; }

/* Start of each plane and the blob size: off[0..5] = Wg codes, Wg s/m, Wu codes,
 * Wu s/m, Wd codes, Wd s/m; off[6] = blob bytes. */
void oracle_blob_layout(int H, int I, int bits, int64_t off[7]) {
  int64_t rows[3] = {I, I, H}, cols[3] = {H, H, I};
  int64_t pos = 0;
  for (int m = 0; m < 3; ++m) {
    off[2 * m] = pos;
    pos = round_up_256(pos + rows[m] * cols[m] * bits / 8);
    off[2 * m + 1] = pos;
    pos = round_up_256(pos + rows[m] * (cols[m] / 32) * 4);
  }
  off[6] = pos;
}

static uint32_t read_u32_le(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* W[r][c] of a matrix with K columns, from its code plane and s/m plane:
 * s*q + m.  Exact in double: an fp16 times a code below 16 has at most 15
 * significant bits, and the sum with an fp16 spans far fewer than 53 bits. */
static double weight_at(const uint8_t* codes, const uint8_t* sm, int K, int bits, int r, int c) {
  int64_t row_words = (int64_t)K * bits / 32;
  uint32_t q;
  if (bits == 3) {
    /* three words per 32-column block: the low two bits of the codes laid out
     * as in the 2-bit format (16 columns per word), then one word of high bits,
     * block column j at bit 16*(j%2) + j/2 */
    const uint8_t* blk = codes + 4 * ((int64_t)r * row_words + 3 * (c / 32));
    int j = c % 32, cw = j % 16;
    uint32_t lo = (read_u32_le(blk + 4 * (j / 16)) >> (16 * (cw % 2) + 2 * (cw / 2))) & 3u;
    uint32_t hi = (read_u32_le(blk + 8) >> (16 * (j % 2) + j / 2)) & 1u;
    q = lo + 4u * hi;
  } else {
    int per_word = 32 / bits;
    uint32_t word = read_u32_le(codes + 4 * ((int64_t)r * row_words + c / per_word));
    int cw = c % per_word;
    int shift = 16 * (cw % 2) + bits * (cw / 2);
    q = (word >> shift) & ((1u << bits) - 1u);
  }
  uint32_t smw = read_u32_le(sm + 4 * ((int64_t)r * (K / 32) + c / 32));
  double s = oracle_f16((uint16_t)(smw & 0xFFFF));
  double m = oracle_f16((uint16_t)(smw >> 16));
  return s * (double)q + m;
}

/* Decoded weight W[r][c] of matrix mat (0 = Wg, 1 = Wu, 2 = Wd) of an expert blob. */
double oracle_weight(const uint8_t* blob, int H, int I, int bits, int mat, int r, int c) {
  int64_t off[7];
  oracle_blob_layout(H, I, bits, off);
  int K = (mat < 2) ? H : I;
  return weight_at(blob + off[2 * mat], blob + off[2 * mat + 1], K, bits, r, c);
}

/* Whole matrix [R x K] decoded into out (row-major). */
void oracle_dequant_matrix(const uint8_t* blob, int H, int I, int bits, int mat, double* out) {
  int64_t off[7];
  oracle_blob_layout(H, I, bits, off);
  int R = (mat < 2) ? I : H, K = (mat < 2) ? H : I;
  for (int r = 0; r < R; ++r)
    for (int c = 0; c < K; ++c)
      out[(int64_t)r * K + c] = weight_at(blob + off[2 * mat], blob + off[2 * mat + 1], K, bits, r, c);
}

/* ---- routing -------------------------------------------------------------- */

/* Expert a ranks above expert b: larger logit, or equal logits and lower id.
 * C's == treats -0.0 and +0.0 as equal, as the ranking requires. */
static int ranks_above(const float* row, int a, int b) {
  double la = row[a], lb = row[b];
  if (la > lb) return 1;
  if (la < lb) return 0;
  return a < b;
}

/* For each token: ids[t][0..k) = the k highest-ranked experts in descending
 * rank; w[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected.
 * Returns 0, or -1 on bad sizes. */
int oracle_route(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
  if (T < 0 || E < 1 || k < 1 || k > E) return -1;
  char* taken = (char*)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const float* row = logits + (int64_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || ranks_above(row, e, best))) best = e;
      taken[best] = 1;
      ids[(int64_t)t * k + j] = best;
    }
    double l0 = row[ids[(int64_t)t * k]], den = 0.0;
    for (int j = 0; j < k; ++j) den += exp((double)row[ids[(int64_t)t * k + j]] - l0);
    for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = exp((double)row[ids[(int64_t)t * k + j]] - l0) / den;
  }
  free(taken);
  return 0;
}

/* ---- dispatch ------------------------------------------------------------- */

/* Group the n = T*k assignments (a = t*k + j) by expert, keeping ascending a
 * inside each expert:
 *   offsets[e] = number of assignments with expert < e (offsets[E] = n),
 *   sorted_assign[p] = the assignment at sorted position p,
 *   assign_pos[a] = its sorted position (the inverse permutation),
 *   active[0..n_active) = experts with at least one assignment, ascending.
 * Returns 0, or -1 if an id is out of range. */
int oracle_dispatch(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_assign,
                    int32_t* assign_pos, int32_t* active, int32_t* n_active) {
  int64_t n = (int64_t)T * k;
  for (int64_t a = 0; a < n; ++a)
    if (ids[a] < 0 || ids[a] >= E) return -1;
  int32_t pos = 0, na = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = pos;
    int32_t start = pos;
    for (int64_t a = 0; a < n; ++a)
      if (ids[a] == e) {
        sorted_assign[pos] = (int32_t)a;
        assign_pos[a] = pos;
        ++pos;
      }
    if (pos > start) active[na++] = e;
  }
  offsets[E] = pos;
  *n_active = na;
  return 0;
}

/* ---- expert FFN ------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert with decoded matrices on one input row x[H]:
 * g = Wg x, u = Wu x, h = silu(g) * u, y = Wd h.  h_out (length I) may be NULL. */
void oracle_ffn_decoded(const double* wg, const double* wu, const double* wd, int H, int I, const double* x,
                        double* h_out, double* y) {
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int c = 0; c < H; ++c) {
      g += wg[(int64_t)i * H + c] * x[c];
      u += wu[(int64_t)i * H + c] * x[c];
    }
    h[i] = silu(g) * u;
    if (h_out) h_out[i] = h[i];
  }
  for (int n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += wd[(int64_t)n * I + i] * h[i];
    y[n] = acc;
  }
  free(h);
}

/* The same from the encoded blob. */
void oracle_expert_ffn(const uint8_t* blob, int H, int I, int bits, const double* x, double* h_out, double* y) {
  size_t n = (size_t)H * (size_t)I;
  double* wg = (double*)malloc(sizeof(double) * n);
  double* wu = (double*)malloc(sizeof(double) * n);
  double* wd = (double*)malloc(sizeof(double) * n);
  oracle_dequant_matrix(blob, H, I, bits, 0, wg);
  oracle_dequant_matrix(blob, H, I, bits, 1, wu);
  oracle_dequant_matrix(blob, H, I, bits, 2, wd);
  oracle_ffn_decoded(wg, wu, wd, H, I, x, h_out, y);
  free(wg);
  free(wu);
  free(wd);
}

/* ---- combine -------------------------------------------------------------- */

/* out[t][c] = residual[t][c] (0 if residual is NULL) + sum_{j=0}^{k-1} w[t][j] * y[t][j][c]. */
void oracle_combine(const double* y, const double* w, int T, int k, int H, const double* residual, double* out) {
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < H; ++c) {
      double acc = residual ? residual[(int64_t)t * H + c] : 0.0;
      for (int j = 0; j < k; ++j) acc += w[(int64_t)t * k + j] * y[((int64_t)t * k + j) * H + c];
      out[(int64_t)t * H + c] = acc;
    }
}

/* ---- whole layer -------------------------------------------------------------- */

static double x_value(const void* x, int x_is_bf16, int64_t i) {
  return x_is_bf16 ? oracle_bf16(((const uint16_t*)x)[i]) : (double)((const float*)x)[i];
}

/* ---- router projection ------------------------------------------------------ */

/* The router scores every expert from the token's hidden state (Strata feature,
 * tech.hub77a.com, section "2. 왜 대단한가" (2): the router's choice decides which
 * experts run).  The pages give no formula; the reading taken is a bias-free
 * linear map: logits[t][e] = sum_c x[t][c] * Wr[e][c].
 * x: [T x H] fp32 values (x_is_bf16 = 0) or raw bf16 bits (x_is_bf16 = 1);
 * wr: [E x H] raw bf16 bits; logits: [T x E] doubles. */
void oracle_router_logits(const void* x, int x_is_bf16, const uint16_t* wr, int T, int H, int E, double* logits) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int c = 0; c < H; ++c)
        acc += x_value(x, x_is_bf16, (int64_t)t * H + c) * oracle_bf16(wr[(int64_t)e * H + c]);
      logits[(int64_t)t * E + e] = acc;
    }
}


/* x: [T x H] fp32 values (x_is_bf16 = 0) or raw bf16 bits (x_is_bf16 = 1).
 * experts: expert e's blob at experts + e * stride.
 * residual: NULL or [T x H] doubles.
 * Outputs: ids, w [T x k]; y [T x k x H] (may be NULL); out [T x H].
 * Each selected expert is decoded once and applied to every row routed to it.
 * Returns 0, or -1 on bad arguments. */
int oracle_layer(const void* x, int x_is_bf16, const float* logits, const uint8_t* experts, int64_t stride, int T,
                 int E, int k, int H, int I, int bits, const double* residual, int32_t* ids, double* w, double* y,
                 double* out) {
  if (H % 32 || I % 32 || bits < 2 || bits > 4) return -1;
  if (oracle_route(logits, T, E, k, ids, w) != 0) return -1;
  size_t n = (size_t)H * (size_t)I;
  double* wg = (double*)malloc(sizeof(double) * n);
  double* wu = (double*)malloc(sizeof(double) * n);
  double* wd = (double*)malloc(sizeof(double) * n);
  double* xr = (double*)malloc(sizeof(double) * (size_t)H);
  double* yall = (double*)malloc(sizeof(double) * ((size_t)T * (size_t)k * (size_t)H + 1));
  for (int e = 0; e < E; ++e) {
    int used = 0;
    for (int64_t a = 0; a < (int64_t)T * k; ++a) used |= (ids[a] == e);
    if (!used) continue;
    const uint8_t* blob = experts + (int64_t)e * stride;
    oracle_dequant_matrix(blob, H, I, bits, 0, wg);
    oracle_dequant_matrix(blob, H, I, bits, 1, wu);
    oracle_dequant_matrix(blob, H, I, bits, 2, wd);
    for (int64_t a = 0; a < (int64_t)T * k; ++a) {
      if (ids[a] != e) continue;
      int64_t t = a / k;
      for (int c = 0; c < H; ++c) xr[c] = x_value(x, x_is_bf16, t * H + c);
      oracle_ffn_decoded(wg, wu, wd, H, I, xr, NULL, yall + a * H);
    }
  }
  oracle_combine(yall, w, T, k, H, residual, out);
  if (y) memcpy(y, yall, sizeof(double) * (size_t)T * (size_t)k * (size_t)H);
  free(yall);
  free(xr);
  free(wd);
  free(wu);
  free(wg);
  return 0;
}

/* ---- the same layer on several threads (full-size checks and CPU timing) ---- */

/* oracle_layer_mt computes what oracle_layer computes, with the same
 * functions applied to the same rows, so its outputs equal oracle_layer's bit
 * for bit whatever the thread count.  Only the order in which independent
 * rows are visited changes:
 *   1. routing: oracle_route on disjoint slices of tokens;
 *   2. experts: work items of (expert, up to MT_ROWS of its assignments in
 *      ascending order); each item decodes its expert with
 *      oracle_dequant_matrix and runs oracle_ffn_decoded on each of its rows;
 *      threads take items from a shared counter;
 *   3. combine: oracle_combine on disjoint slices of tokens.
 * y may be NULL.  Returns 0, or -1 on bad arguments or memory exhaustion. */

#define MT_ROWS 256

typedef struct {
  /* shared inputs */
  const void* x;
  int x_is_bf16;
  const float* logits;
  const uint8_t* experts;
  int64_t stride;
  int T, E, k, H, I, bits, nthreads;
  const double* residual;
  /* shared outputs and schedule */
  int32_t* ids;
  double* w;
  double* yall;
  double* out;
  const int32_t* order;  /* assignments grouped by expert, ascending inside */
  const int64_t* item_first;
  const int32_t* item_count;
  int64_t n_items;
  int64_t next_item;
  int failed;
} mt_job;

typedef struct {
  mt_job* job;
  int rank;
} mt_arg;

static void mt_slice(int T, int nthreads, int rank, int* t0, int* t1) {
  *t0 = (int)((int64_t)T * rank / nthreads);
  *t1 = (int)((int64_t)T * (rank + 1) / nthreads);
}

static void* mt_route(void* p) {
  mt_arg* a = (mt_arg*)p;
  mt_job* j = a->job;
  int t0, t1;
  mt_slice(j->T, j->nthreads, a->rank, &t0, &t1);
  if (t1 > t0 && oracle_route(j->logits + (int64_t)t0 * j->E, t1 - t0, j->E, j->k, j->ids + (int64_t)t0 * j->k,
                              j->w + (int64_t)t0 * j->k) != 0)
    j->failed = 1;
  return NULL;
}

static void* mt_ffn(void* p) {
  mt_arg* a = (mt_arg*)p;
  mt_job* j = a->job;
  size_t n = (size_t)j->H * (size_t)j->I;
  double* wg = (double*)malloc(sizeof(double) * n);
  double* wu = (double*)malloc(sizeof(double) * n);
  double* wd = (double*)malloc(sizeof(double) * n);
  double* xr = (double*)malloc(sizeof(double) * (size_t)j->H);
  if (!wg || !wu || !wd || !xr) {
    j->failed = 1;
  } else {
    for (;;) {
      int64_t it = __atomic_fetch_add(&j->next_item, 1, __ATOMIC_RELAXED);
      if (it >= j->n_items) break;
      const int32_t* rows = j->order + j->item_first[it];
      int e = j->ids[rows[0]];
      const uint8_t* blob = j->experts + (int64_t)e * j->stride;
      oracle_dequant_matrix(blob, j->H, j->I, j->bits, 0, wg);
      oracle_dequant_matrix(blob, j->H, j->I, j->bits, 1, wu);
      oracle_dequant_matrix(blob, j->H, j->I, j->bits, 2, wd);
      for (int r = 0; r < j->item_count[it]; ++r) {
        int64_t asg = rows[r], t = asg / j->k;
        for (int c = 0; c < j->H; ++c) xr[c] = x_value(j->x, j->x_is_bf16, t * j->H + c);
        oracle_ffn_decoded(wg, wu, wd, j->H, j->I, xr, NULL, j->yall + asg * j->H);
      }
    }
  }
  free(xr);
  free(wd);
  free(wu);
  free(wg);
  return NULL;
}

static void* mt_combine(void* p) {
  mt_arg* a = (mt_arg*)p;
  mt_job* j = a->job;
  int t0, t1;
  mt_slice(j->T, j->nthreads, a->rank, &t0, &t1);
  if (t1 > t0)
    oracle_combine(j->yall + (int64_t)t0 * j->k * j->H, j->w + (int64_t)t0 * j->k, t1 - t0, j->k, j->H,
                   j->residual ? j->residual + (int64_t)t0 * j->H : NULL, j->out + (int64_t)t0 * j->H);
  return NULL;
}

static int mt_run(mt_job* j, void* (*fn)(void*)) {
  pthread_t th[256];
  mt_arg args[256];
  int started = 0;
  for (int r = 0; r < j->nthreads; ++r) {
    args[r].job = j;
    args[r].rank = r;
    if (r == 0) continue;
    if (pthread_create(&th[r], NULL, fn, &args[r]) != 0) break;
    started = r;
  }
  if (started < j->nthreads - 1) {
    /* fewer threads than asked: the started ones and this one share the work
     * only where the work is a shared queue; slices need every rank */
    j->failed = 1;
  }
  fn(&args[0]);
  for (int r = 1; r <= started; ++r) pthread_join(th[r], NULL);
  return j->failed ? -1 : 0;
}

int oracle_layer_mt(const void* x, int x_is_bf16, const float* logits, const uint8_t* experts, int64_t stride, int T,
                    int E, int k, int H, int I, int bits, const double* residual, int32_t* ids, double* w, double* y,
                    double* out, int nthreads) {
  if (H % 32 || I % 32 || bits < 2 || bits > 4 || T < 0 || E < 1 || k < 1 || k > E) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  const int64_t n = (int64_t)T * k;
  mt_job j;
  memset(&j, 0, sizeof j);
  j.x = x;
  j.x_is_bf16 = x_is_bf16;
  j.logits = logits;
  j.experts = experts;
  j.stride = stride;
  j.T = T;
  j.E = E;
  j.k = k;
  j.H = H;
  j.I = I;
  j.bits = bits;
  j.nthreads = nthreads;
  j.residual = residual;
  j.ids = ids;
  j.w = w;
  j.out = out;
  if (mt_run(&j, mt_route) != 0) return -1;
  /* group the assignments by expert (ascending inside) and cut the groups into items */
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n + 1));
  int64_t* count = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
  int64_t* item_first = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n / MT_ROWS + E + 1));
  int32_t* item_count = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n / MT_ROWS + E + 1));
  double* yall = y ? y : (double*)malloc(sizeof(double) * ((size_t)n * (size_t)H + 1));
  int rc = -1;
  if (order && count && item_first && item_count && yall) {
    for (int64_t a = 0; a < n; ++a) ++count[ids[a] + 1];
    for (int e = 0; e < E; ++e) count[e + 1] += count[e];
    int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
    if (fill) {
      memcpy(fill, count, sizeof(int64_t) * (size_t)E);
      for (int64_t a = 0; a < n; ++a) order[fill[ids[a]]++] = (int32_t)a;
      free(fill);
      int64_t ni = 0;
      for (int e = 0; e < E; ++e)
        for (int64_t p = count[e]; p < count[e + 1]; p += MT_ROWS) {
          item_first[ni] = p;
          item_count[ni] = (int32_t)((count[e + 1] - p) < MT_ROWS ? (count[e + 1] - p) : MT_ROWS);
          ++ni;
        }
      j.order = order;
      j.item_first = item_first;
      j.item_count = item_count;
      j.n_items = ni;
      j.yall = yall;
      if (mt_run(&j, mt_ffn) == 0 && mt_run(&j, mt_combine) == 0) rc = 0;
    }
  }
  if (!y) free(yall);
  free(item_count);
  free(item_first);
  free(count);
  free(order);
  return rc;
}
