/*
 * synth.c -- seeded synthetic inputs for the routed MoE FFN layer.
 *
 * This module only *produces* input bytes: random streams, router logits with
 * a Zipf-shaped popularity bias, bf16 activations, and expert weights drawn
 * from N(0, std) and encoded in the block-32 scale+min format.  It holds none
 * of the layer's arithmetic (no decoding, routing, FFN or combine); both the
 * CPU oracle and the GPU path consume the bytes it writes.
 *
 * Random numbers: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: element i of a stream with key K is mix(K + (i+1)*gamma).
 * Normals use the Box-Muller transform (cosine branch) on two uniforms.
 *
 * Weight encoding (the format the layer decodes):
 *   a matrix [R x K] (rows K-contiguous, K % 32 == 0) is cut into blocks of 32
 *   weights along K.  Each block has an IEEE binary16 scale s and min m and
 *   b-bit unsigned codes q (b = 2, 3 or 4); the weight it stands for is s*q + m.
 *   Code plane: each row is K*b/32 little-endian 32-bit words.  b = 2, 4: word
 *   w holds columns [w*32/b, (w+1)*32/b); column c of the word (0 <= c < 32/b)
 *   sits at bit 16*(c % 2) + b*(c / 2).  Even columns fill the low halfword,
 *   odd columns the high halfword.  b = 3: three words per 32-column block, the
 *   low two bits of the codes in words 0-1 as for b = 2, the high bits in word
 *   2 (block column j at bit 16*(j % 2) + j / 2).
 *   Scale/min plane: one 32-bit word per block, row-major [R][K/32]; low
 *   halfword = scale, high halfword = min.
 *   Expert blob: Wg codes, Wg s/m, Wu codes, Wu s/m, Wd codes, Wd s/m, each
 *   starting on a 256-byte boundary; Wg, Wu are [I x H], Wd is [H x I].  The
 *   blob size is the end of the last plane rounded up to 256 bytes.
 *
 * Quantizer (input side only): m = fp16_rne(min w), s = fp16_rne((max w -
 * min w) / (2^b - 1)), q = clamp(rne((w - m)/s), 0, 2^b - 1) evaluated in
 * double from the decoded s and m; s == 0 gives q = 0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of a named stream: (seed, tag, a, b, c) -> 64-bit key. */
uint64_t synth_stream_key(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, uint64_t c) {
  uint64_t k = sm_mix(seed + SM_GAMMA);
  k = sm_mix(k ^ (tag + 1) * SM_GAMMA);
  k = sm_mix(k ^ (a + 1) * 0xD1B54A32D192ED03ULL);
  k = sm_mix(k ^ (b + 1) * 0xAEF17502108EF2D9ULL);
  k = sm_mix(k ^ (c + 1) * 0xF1357AEA2E62A9C5ULL);
  return k;
}

static inline uint64_t draw_u64(uint64_t key, uint64_t i) { return sm_mix(key + (i + 1) * SM_GAMMA); }

/* Uniform in the open interval (0, 1). */
static inline double draw_uniform(uint64_t key, uint64_t i) {
  return ((double)(draw_u64(key, i) >> 11) + 0.5) * 0x1.0p-53;
}

static inline double draw_normal(uint64_t key, uint64_t i) {
  double u1 = draw_uniform(key, 2 * i), u2 = draw_uniform(key, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

void synth_u64(uint64_t key, uint64_t first, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = draw_u64(key, first + (uint64_t)i);
}
void synth_uniform(uint64_t key, uint64_t first, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = draw_uniform(key, first + (uint64_t)i);
}
void synth_normal(uint64_t key, uint64_t first, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = draw_normal(key, first + (uint64_t)i);
}

/* ---- rounding helpers (encoders only) ---------------------------------- */

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* double -> IEEE binary16 bits, round to nearest even; overflow saturates to inf. */
uint16_t synth_f64_to_f16(double x) {
  uint16_t sign = 0;
  if (signbit(x)) { sign = 0x8000; x = -x; }
  if (x == 0.0) return sign;
  if (isnan(x)) return 0x7E00;
  if (x >= 65520.0) return sign | 0x7C00; /* rounds past the largest finite value */
  int e;
  (void)frexp(x, &e);        /* x = fr * 2^e with fr in [0.5, 1) */
  int exp16 = e - 1 + 15;   /* biased exponent if normal */
  double scaled;
  if (exp16 >= 1) {
    scaled = ldexp(x, 10 - (e - 1)); /* in [1024, 2048) */
  } else {
    scaled = ldexp(x, 24);           /* subnormal: units of 2^-24 */
    exp16 = 0;
  }
  double fl = floor(scaled);
  double rem = scaled - fl;
  uint32_t m = (uint32_t)fl;
  if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m += 1;
  if (exp16 == 0) {
    return sign | (uint16_t)m; /* m == 1024 becomes the smallest normal, which is correct */
  }
  if (m == 2048) { m = 1024; exp16 += 1; }
  if (exp16 >= 31) return sign | 0x7C00;
  return sign | (uint16_t)(exp16 << 10) | (uint16_t)(m - 1024);
}

/* binary16 bits -> double, used only to evaluate the quantizer from the stored values. */
static double f16_bits_value(uint16_t h) {
  int e = (h >> 10) & 31, f = h & 1023;
  double v = (e == 0) ? ldexp((double)f, -24) : ldexp((double)(f + 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}

/* ---- activations and logits -------------------------------------------- */

/* out[i] = fp32(N(0,1)) for i < n. */
void synth_normal_f32(uint64_t key, int64_t n, float scale, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(draw_normal(key, (uint64_t)i) * (double)scale);
}

/* out[i] = bf16_rne(fp32(N(0,1))) as raw bits. */
void synth_normal_bf16(uint64_t key, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)draw_normal(key, (uint64_t)i));
}

/* out[i] = bf16_rne(fp32(scale * N(0,1))) as raw bits. */
void synth_normal_bf16_scaled(uint64_t key, int64_t n, double scale, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)(draw_normal(key, (uint64_t)i) * scale));
}

/* Seeded permutation of ranks 1..E (Fisher-Yates driven by the stream). */
void synth_ranks(uint64_t key, int E, int32_t* rank) {
  for (int e = 0; e < E; ++e) rank[e] = e + 1;
  for (int i = E - 1; i > 0; --i) {
    uint64_t j = draw_u64(key, (uint64_t)i) % (uint64_t)(i + 1);
    int32_t t = rank[i];
    rank[i] = rank[j];
    rank[j] = t;
  }
}

/* Zipf(s) popularity bias: bias[e] = fp32(-s * ln(rank[e])). */
void synth_zipf_bias(uint64_t key, int E, double s, float* bias) {
  int32_t* rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  synth_ranks(key, E, rank);
  for (int e = 0; e < E; ++e) bias[e] = (float)(-s * log((double)rank[e]));
  free(rank);
}

/* logits[t,e] = fp32(N(0,1)) + bias[e] (an fp32 add); bias may be NULL. */
void synth_logits(uint64_t key, int T, int E, const float* bias, float* out) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      float n = (float)draw_normal(key, (uint64_t)t * (uint64_t)E + (uint64_t)e);
      out[(size_t)t * E + e] = bias ? n + bias[e] : n;
    }
}

/* ---- weight encoding ----------------------------------------------------- */

static size_t align256(size_t v) { return (v + 255u) & ~(size_t)255u; }

/* Plane offsets of the expert blob: off[0..5] = Wg codes, Wg sm, Wu codes, Wu sm,
 * Wd codes, Wd sm; off[6] = blob bytes. */
void synth_blob_layout(int H, int I, int bits, int64_t* off) {
  size_t gu_codes = (size_t)I * (size_t)H * (size_t)bits / 8, gu_sm = (size_t)I * (size_t)(H / 32) * 4;
  size_t d_codes = (size_t)H * (size_t)I * (size_t)bits / 8, d_sm = (size_t)H * (size_t)(I / 32) * 4;
  size_t o = 0;
  off[0] = (int64_t)o; o = align256(o + gu_codes);
  off[1] = (int64_t)o; o = align256(o + gu_sm);
  off[2] = (int64_t)o; o = align256(o + gu_codes);
  off[3] = (int64_t)o; o = align256(o + gu_sm);
  off[4] = (int64_t)o; o = align256(o + d_codes);
  off[5] = (int64_t)o; o = align256(o + d_sm);
  off[6] = (int64_t)o;
}

/* Encode a [R x K] matrix of doubles into the code plane and the s/m plane.
 * bits 2 and 4: word w of a row holds columns w*(32/bits) .., column c of the
 * word at bit 16*(c%2) + bits*(c/2).  bits 3: three words per 32-column block;
 * words 0 and 1 hold the low two bits of each code as the 2-bit layout does,
 * word 2 the high bit, block column j at bit 16*(j%2) + j/2. */
void synth_quantize_matrix(const double* w, int R, int K, int bits, uint32_t* codes, uint32_t* sm) {
  const int qmax = (1 << bits) - 1, nb = K / 32;
  const int per_word = bits == 3 ? 16 : 32 / bits;
  const size_t row_words = (size_t)K * (size_t)bits / 32;
  for (int r = 0; r < R; ++r) {
    const double* row = w + (size_t)r * K;
    uint32_t* crow = codes + (size_t)r * row_words;
    memset(crow, 0, sizeof(uint32_t) * row_words);
    for (int b = 0; b < nb; ++b) {
      const double* blk = row + 32 * b;
      double mn = blk[0], mx = blk[0];
      for (int j = 1; j < 32; ++j) { if (blk[j] < mn) mn = blk[j]; if (blk[j] > mx) mx = blk[j]; }
      uint16_t mh = synth_f64_to_f16(mn), sh = synth_f64_to_f16((mx - mn) / (double)qmax);
      double md = f16_bits_value(mh), sd = f16_bits_value(sh);
      sm[(size_t)r * nb + b] = (uint32_t)sh | ((uint32_t)mh << 16);
      for (int j = 0; j < 32; ++j) {
        int q = 0;
        if (sd > 0.0) {
          double v = nearbyint((blk[j] - md) / sd); /* default rounding mode: ties to even */
          q = v < 0.0 ? 0 : (v > (double)qmax ? qmax : (int)v);
        }
        if (bits == 3) {
          const int c = j % 16;
          crow[3 * b + j / 16] |= (uint32_t)(q & 3) << (16 * (c & 1) + 2 * (c >> 1));
          crow[3 * b + 2] |= (uint32_t)(q >> 2) << (16 * (j & 1) + (j >> 1));
        } else {
          int col = 32 * b + j, word = col / per_word, c = col % per_word;
          crow[word] |= (uint32_t)q << (16 * (c & 1) + bits * (c >> 1));
        }
      }
    }
  }
}

/* Stream tags. */
enum { TAG_LOGITS = 1, TAG_X = 2, TAG_WEIGHT = 3, TAG_RANK = 4, TAG_DRIFT = 5, TAG_ROUTER = 6 };

/* One expert: Wg, Wu [I x H] and Wd [H x I] from N(0, std), encoded into blob. */
void synth_expert(uint64_t seed, int layer, int expert, int H, int I, int bits, double std, uint8_t* blob) {
  int64_t off[7];
  synth_blob_layout(H, I, bits, off);
  memset(blob, 0, (size_t)off[6]);
  size_t n = (size_t)H * (size_t)I;
  double* w = (double*)malloc(sizeof(double) * n);
  for (int mat = 0; mat < 3; ++mat) {
    uint64_t key = synth_stream_key(seed, TAG_WEIGHT, (uint64_t)layer, (uint64_t)expert, (uint64_t)mat);
    for (size_t i = 0; i < n; ++i) w[i] = std * draw_normal(key, (uint64_t)i);
    int R = mat < 2 ? I : H, K = mat < 2 ? H : I;
    synth_quantize_matrix(w, R, K, bits, (uint32_t*)(blob + off[2 * mat]), (uint32_t*)(blob + off[2 * mat + 1]));
  }
  free(w);
}

typedef struct {
  uint64_t seed;
  int layer, E, H, I, bits, nthreads, tid;
  double std;
  uint8_t* out;
  int64_t stride;
  const int32_t* which; /* optional subset of experts */
  int n_which;
} layer_job;

static void* layer_worker(void* p) {
  layer_job* j = (layer_job*)p;
  int n = j->which ? j->n_which : j->E;
  for (int i = j->tid; i < n; i += j->nthreads) {
    int e = j->which ? j->which[i] : i;
    synth_expert(j->seed, j->layer, e, j->H, j->I, j->bits, j->std, j->out + (size_t)e * (size_t)j->stride);
  }
  return NULL;
}

/* All E experts of a layer (or the listed subset) at out + e*stride, on nthreads threads. */
int synth_layer(uint64_t seed, int layer, int E, int H, int I, int bits, double std, uint8_t* out, int64_t stride,
                const int32_t* which, int n_which, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  pthread_t th[64];
  layer_job jobs[64];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (layer_job){seed, layer, E, H, I, bits, nthreads, t, std, out, stride, which, n_which};
    if (t > 0 && pthread_create(&th[t], NULL, layer_worker, &jobs[t]) != 0) return -1;
  }
  layer_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}
