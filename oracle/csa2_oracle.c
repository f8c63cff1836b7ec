/*
 * CPU ORACLE for the CSA2 global-attention path — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load or call this library. The HIP library never does, and shares no code,
 * header, table or constant with it.
 *
 * Plain, slow, obviously-correct C in fp64. Each function names the passage
 * it follows. Pages:
 *   [ATLAS]  "An infra-oriented diagram of the DeepSeek-V4.1-Flash
 *            architecture" — Reading notes (KV-latent bullet, Full-layer cache
 *            bullet, indexer bullet, role bullet) and section "The KV cache".
 *   [HELIX]  "DeepSeek V4.1 Flash: Why Its Encoder, Engram and KV Cache
 *            Matter" — section "CSA2 makes long context cheaper to retain".
 *   [PERCHY] "DeepSeek V4.1 Flash" model guide — "A closer look: Full.
 *            Reindex. Reuse."
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   R1 code byte j holds channel 2j in the low nibble, 2j+1 in the high one;
 *      codes precede scales inside an entry.
 *   R2 the E4M3 flavour is OCP E4M3FN (bias 7, no inf, S.1111.111 = NaN).
 *   R3 the indexer query is MXFP4 like the keys (E2M1, E8M0 per 32).
 *   R4 indexer score = sum_h w_h * max(q_h . k, 0): no extra constant factor.
 *   R5 top-k ranks candidates by (score descending, entry index ascending),
 *      -0 == +0, NaN below every number; the selected set is returned in
 *      ascending entry index (the pages fix the set, not an order).
 *   R6 Reindex pools are aligned blocks: block b covers entries 8b..8b+7.
 *   R7 attention runs over the selected entries followed by the SWA rows, one
 *      softmax over the joint set, no de-duplication, no sink, no bias; the
 *      latent is both key and value; RoPE is outside this path.
 *   R8 selected ids outside [0, n_entries) (the -1 padding) are skipped; an
 *      empty joint set gives a zero output and lse = -inf.
 *   R13 writing a new entry (fp32 in): a main block's E4M3 scale is the
 *       E4M3FN value nearest to amax/6 (ties to the even code, saturating at
 *       448); an indexer block's E8M0 scale is 2^e for the smallest e in
 *       [-127, 127] with 6 * 2^e >= amax (e = 0 for an all-zero block); each
 *       element takes the E2M1 magnitude nearest to |x| / scale (ties to the
 *       even code, saturating at 6) and the sign bit of x; a block whose scale
 *       is zero (main) or whose amax is zero (indexer) gets all-zero codes.
 *       NaN counts as a zero magnitude, +-inf as the largest one.
 *   R14 a window row in FP8 (528 bytes, [ATLAS] "The KV cache") is OCP
 *       MXFP8: 512 E4M3FN codes, then 16 E8M0 scales, one per 32 channels.
 *   R15 RoPE un-rotation of the output ([ATLAS] KV-latent bullet): the rotary
 *       channels are 448..511 in adjacent pairs (448+2i, 449+2i); a caller
 *       table gives each query's (cos, sin) per pair; the pair (a, b) of the
 *       normalised output becomes (a c + b s, b c - a s).
 *   R16 a Reindex pool ([ATLAS] indexer bullet: a 16,384-entry pool that
 *       layer 20 chose by blocks of 8) is built from that layer's own scores:
 *       a block scores the best of its entries inside the causal limit (rank
 *       order of R5); the n_pool best blocks by (block score descending, block
 *       id ascending) are kept and listed in ascending block id, -1 padded.
 *   R17 m=2 pooling ([ATLAS] Full-layer cache bullet: two consecutive tokens
 *       pooled into one entry with a learned softmax gate): entry i is
 *       p x_{2i} + (1 - p) x_{2i+1} with p = 1 / (1 + exp(g_{2i+1} - g_{2i})),
 *       the two-way softmax of the gate logits, taken per channel (or one
 *       logit per token); the logits are inputs (their projection needs
 *       trained weights); the pooled row is then quantised as in R13.
 *   R18 Reuse layers ([HELIX] CSA2 section: they share the global KV and the
 *       selected positions of an earlier layer) attend over the same
 *       selection with their own queries; the selected entries may first be
 *       copied into a dense per-query list (slot j = the j-th selected id;
 *       skipped ids keep a slot whose dense id is -1), and attention over
 *       that list with dense ids equals attention over the cache with the
 *       original ids.
 *   (R9-R12 concern the workload and its generator; they are listed with the
 *   design notes.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ O1 --- */
/* Element formats named in [ATLAS] Full-layer cache bullet ("E2M1, one E4M3
 * scale per 16 channels") and "The KV cache" ("one E8M0 scale per 32"). The
 * value definitions are those of the OCP Microscaling (MX) formats spec. */

/* FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf/NaN. */
ORC_API double orc_e2m1(unsigned code) {
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

/* FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa; S.1111.111 is NaN. */
ORC_API double orc_e4m3(unsigned byte) {
  unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* E8M0: unsigned power of two 2^(b-127); 0xFF is NaN. */
ORC_API double orc_e8m0(unsigned byte) {
  if ((byte & 0xFFu) == 0xFFu) return NAN;
  return ldexp(1.0, (int)(byte & 0xFFu) - 127);
}

static double nib(const uint8_t* codes, int ch) { /* R1 */
  unsigned b = codes[ch >> 1];
  return orc_e2m1((ch & 1) ? (b >> 4) : (b & 15u));
}

/* Main entry: 256 code bytes then 32 E4M3 scales ([ATLAS] "The KV cache":
 * 512 FP4 values with an E4M3 scale per 16 channels, 288 bytes). */
static void main_entry_f64(const uint8_t* entry, double* out512) {
  for (int c = 0; c < 512; ++c) out512[c] = nib(entry, c) * orc_e4m3(entry[256 + c / 16]);
}

/* Indexer key: 64 code bytes + 4 E8M0 scales (68 bytes, [ATLAS] "The KV cache"). */
static void index_row_f64(const uint8_t* codes, const uint8_t* scales, double* out128) {
  for (int c = 0; c < 128; ++c) out128[c] = nib(codes, c) * orc_e8m0(scales[c / 32]);
}

ORC_API int orc_main_entry_bytes(void) { return 512 / 2 + 512 / 16; }  /* 288 */
ORC_API int orc_index_entry_bytes(void) { return 128 / 2 + 128 / 32; } /* 68 */

/* fp64 -> bf16 (1 sign, 8 exponent bits with bias 127, 7 mantissa bits) in
 * ONE round-to-nearest-even step, on the integer fields of the fp64 value, so
 * that no intermediate fp32 rounding can move a value that lies just off a
 * bf16 midpoint onto it. bf16 subnormals (|v| < 2^-126) keep 7 fraction bits
 * of 2^-126; overflow gives +-inf; NaN stays a (quiet) NaN. */
ORC_API uint16_t orc_f64_to_bf16(double v) {
  uint64_t u;
  memcpy(&u, &v, 8);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const int e = (int)((u >> 52) & 0x7FF);
  const uint64_t frac = u & ((1ull << 52) - 1);
  if (e == 0x7FF) return (uint16_t)(sign | (frac ? 0x7FC0u : 0x7F80u));
  if (e == 0) return sign; /* fp64 zero or subnormal: below half the least bf16 subnormal */
  /* |v| = full * 2^(e - 1075), full = 2^52 + frac (53 bits). The bf16
   * result counts units of 2^(eb - 134) for a normal result (eb = e - 896,
   * the bf16 biased exponent) and of 2^-133 for a subnormal one; shift is
   * the number of low bits of full below that unit. */
  const uint64_t full = (1ull << 52) | frac;
  const int eb = e - 1023 + 127;
  const int shift = (eb >= 1) ? 45 : 45 + (1 - eb);
  if (shift > 54) return sign; /* |v| < 2^-134: below half the least subnormal */
  uint64_t keep = full >> shift;
  const uint64_t rem = full & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1))) ++keep;
  /* normal: keep = 2^7 + mantissa (a carry to 2^8 moves into the exponent);
   * subnormal: keep is the bf16 bit pattern itself (2^7 = least normal) */
  uint32_t bits = (eb >= 1) ? ((uint32_t)eb << 7) + (uint32_t)(keep - 128) : (uint32_t)keep;
  if (bits >= 0x7F80u) bits = 0x7F80u;
  return (uint16_t)(sign | bits);
}

static uint16_t f64_to_bf16(double v) { return orc_f64_to_bf16(v); }

static double bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Dequantise n main entries to fp32 [n][512] and/or bf16 [n][512]. */
ORC_API void orc_dequant_main(const uint8_t* entries, int64_t n, float* out_f32, uint16_t* out_bf16) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double v[512];
    main_entry_f64(entries + (size_t)i * 288, v);
    for (int c = 0; c < 512; ++c) {
      if (out_f32) out_f32[(size_t)i * 512 + c] = (float)v[c];
      if (out_bf16) out_bf16[(size_t)i * 512 + c] = f64_to_bf16(v[c]);
    }
  }
}

/* Dequantise n indexer keys to fp32 [n][128] and/or bf16. */
ORC_API void orc_dequant_index(const uint8_t* codes, const uint8_t* scales, int64_t n, float* out_f32,
                               uint16_t* out_bf16) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double v[128];
    index_row_f64(codes + (size_t)i * 64, scales + (size_t)i * 4, v);
    for (int c = 0; c < 128; ++c) {
      if (out_f32) out_f32[(size_t)i * 128 + c] = (float)v[c];
      if (out_bf16) out_bf16[(size_t)i * 128 + c] = f64_to_bf16(v[c]);
    }
  }
}

/* ------------------------------------------------------------------ O7 --- */
/* Cache write: quantise new fp32 entries into the two stored formats
 * ([ATLAS] "The KV cache" and Full-layer cache bullet give the formats; the
 * rounding rule is reading R13). Brute force: every candidate code is tried
 * and the nearest kept, so the result is the definition itself. */

static int e2m1_is_better(double d, unsigned m, double best_d, unsigned best_m) {
  return d < best_d || (d == best_d && (m & 1u) == 0 && (best_m & 1u) == 1);
}

/* Nearest E2M1 magnitude code (0..7) to |x| / s, s > 0; compared as
 * |x| against s * value so that no quotient is rounded. Magnitudes above the
 * largest value 6 are first brought down to it (saturation). */
static unsigned e2m1_nearest_mag(double ax, double s) {
  if (isnan(ax)) return 0;
  if (ax > 6.0 * s) ax = 6.0 * s;
  unsigned best = 0;
  double best_d = INFINITY;
  for (unsigned m = 0; m < 8; ++m) {
    double d = fabs(ax - s * orc_e2m1(m));
    if (e2m1_is_better(d, m, best_d, best)) { best = m; best_d = d; }
  }
  return best;
}

/* Nearest finite non-negative E4M3FN code (0..0x7E) to amax / 6, after
 * bringing amax / 6 down to the largest finite value 448 (saturation). */
static unsigned e4m3_scale_code(double amax) {
  if (amax > 6.0 * 448.0) amax = 6.0 * 448.0;
  unsigned best = 0;
  double best_d = INFINITY;
  for (unsigned c = 0; c <= 0x7E; ++c) {
    double d = fabs(amax - 6.0 * orc_e4m3(c));
    if (e2m1_is_better(d, c, best_d, best)) { best = c; best_d = d; }
  }
  return best;
}

static double abs_or_zero(float x) { return isnan(x) ? 0.0 : fabs((double)x); }

static void put_code(uint8_t* codes, int ch, float x, unsigned mag) { /* R1 */
  unsigned code = mag | (signbit(x) ? 8u : 0u);
  codes[ch >> 1] |= (uint8_t)(code << ((ch & 1) ? 4 : 0));
}

/* n main latents [n][512] fp32 -> n entries of 288 bytes. */
ORC_API void orc_quantize_main(const float* x, int64_t n, uint8_t* entries) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const float* xi = x + (size_t)i * 512;
    uint8_t* out = entries + (size_t)i * 288;
    memset(out, 0, 288);
    for (int g = 0; g < 32; ++g) {
      double amax = 0.0;
      for (int c = 0; c < 16; ++c) {
        double a = abs_or_zero(xi[16 * g + c]);
        if (a > amax) amax = a;
      }
      unsigned sc = e4m3_scale_code(amax);
      out[256 + g] = (uint8_t)sc;
      double s = orc_e4m3(sc);
      if (s == 0.0) continue;
      for (int c = 0; c < 16; ++c) {
        int ch = 16 * g + c;
        put_code(out, ch, xi[ch], e2m1_nearest_mag(fabs((double)xi[ch]), s));
      }
    }
  }
}

/* n indexer keys [n][128] fp32 -> codes [n][64] and E8M0 scales [n][4]. */
ORC_API void orc_quantize_index(const float* x, int64_t n, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const float* xi = x + (size_t)i * 128;
    uint8_t* co = codes + (size_t)i * 64;
    memset(co, 0, 64);
    for (int g = 0; g < 4; ++g) {
      double amax = 0.0;
      for (int c = 0; c < 32; ++c) {
        double a = abs_or_zero(xi[32 * g + c]);
        if (a > amax) amax = a;
      }
      int e = 0;
      if (amax > 0.0) {
        e = -127;
        while (e < 127 && 6.0 * ldexp(1.0, e) < amax) ++e;
      }
      scales[(size_t)i * 4 + g] = (uint8_t)(e + 127);
      if (amax == 0.0) continue;
      double s = ldexp(1.0, e);
      for (int c = 0; c < 32; ++c) {
        int ch = 32 * g + c;
        put_code(co, ch, xi[ch], e2m1_nearest_mag(fabs((double)xi[ch]), s));
      }
    }
  }
}

/* m=2 pooling (R17): x [2n][512] token latents, gate [2n][gate_width] logits
 * (gate_width 512: per channel; 1: per token). out [n][512] pooled, fp64. */
ORC_API void orc_pool_latents(const float* x, const float* gate, int gate_width, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const float* xa = x + (size_t)(2 * i) * 512;
    const float* xb = xa + 512;
    for (int c = 0; c < 512; ++c) {
      int gc = gate_width == 1 ? 0 : c;
      double ga = gate[(size_t)(2 * i) * gate_width + gc], gb = gate[(size_t)(2 * i + 1) * gate_width + gc];
      double pa = 1.0 / (1.0 + exp(gb - ga)), pb = 1.0 / (1.0 + exp(ga - gb));
      out[(size_t)i * 512 + c] = pa * (double)xa[c] + pb * (double)xb[c];
    }
  }
}

/* ------------------------------------------------------------------ O3 --- */
/* Candidate set. Full layers score every cache entry ([HELIX] CSA2 section:
 * Full layers "search the full sparse index"); Reindex layers score only a
 * pool built from blocks of 8 ([ATLAS] indexer bullet). Position p of the
 * candidate list maps to a global entry id; n_valid (if given) excludes ids
 * >= n_valid[q] (causal limit). */
static int64_t cand_entry(const int32_t* blocks_q, int64_t p) {
  if (!blocks_q) return p;
  return 8 * (int64_t)blocks_q[p / 8] + p % 8; /* R6 */
}

/* ------------------------------------------------------------------ O2 --- */
/* Lightning indexer, [ATLAS] indexer bullet: 32 FP4 query heads of 128 dims
 * against one shared key per entry, ReLU'd scores summed with per-head
 * weights. d_h = q_h . k is exact in fp64 for these formats; the weighted sum
 * is formed in fp64 and rounded once to fp32. Entries outside the candidate
 * set get -inf. dots_out (optional) receives d as [Q][32][n_cand] fp64. */
ORC_API void orc_index_score(int Q, int64_t n_entries, int64_t cache_q_stride, const uint8_t* key_codes,
                             const uint8_t* key_scales, const uint8_t* iq_codes, const uint8_t* iq_scales,
                             const float* w, const int32_t* cand_blocks, int n_blocks, const int32_t* n_valid,
                             float* scores, double* dots_out) {
  int64_t n_cand = cand_blocks ? 8 * (int64_t)n_blocks : n_entries;
#pragma omp parallel for schedule(dynamic, 1)
  for (int q = 0; q < Q; ++q) {
    double qv[32][128];
    for (int h = 0; h < 32; ++h)
      index_row_f64(iq_codes + ((size_t)q * 32 + h) * 64, iq_scales + ((size_t)q * 32 + h) * 4, qv[h]);
    const int32_t* blk = cand_blocks ? cand_blocks + (size_t)q * n_blocks : NULL;
    int64_t limit = n_valid ? (int64_t)n_valid[q] : n_entries;
    if (limit > n_entries) limit = n_entries;
    for (int64_t p = 0; p < n_cand; ++p) {
      int64_t e = cand_entry(blk, p);
      if (e < 0 || e >= limit) {
        scores[(size_t)q * n_cand + p] = -INFINITY;
        continue;
      }
      int64_t row = (int64_t)q * cache_q_stride + e;
      double kv[128];
      index_row_f64(key_codes + (size_t)row * 64, key_scales + (size_t)row * 4, kv);
      double acc = 0.0;
      for (int h = 0; h < 32; ++h) {
        double d = 0.0;
        for (int c = 0; c < 128; ++c) d += qv[h][c] * kv[c];
        if (dots_out) dots_out[((size_t)q * 32 + h) * n_cand + p] = d;
        double r = d > 0.0 ? d : 0.0; /* ReLU before the head weighting */
        acc += (double)w[q * 32 + h] * r;
      }
      scores[(size_t)q * n_cand + p] = (float)acc;
    }
  }
}

/* ------------------------------------------------------------------ O4 --- */
/* Top-k per query ([PERCHY] "Main sparse selection: 512 entries"; [ATLAS]
 * indexer bullet "top-512"). Sort the candidates by the R5 ranking, keep the
 * first min(k, n), and list them by ascending entry id. idx gets entry ids,
 * padded with -1; top_scores (optional) gets their scores, padded with -inf. */
typedef struct {
  float s;
  int64_t e;
} orc_pair;

static int rank_cmp(const void* a, const void* b) {
  const orc_pair* x = (const orc_pair*)a;
  const orc_pair* y = (const orc_pair*)b;
  int xn = isnan(x->s), yn = isnan(y->s);
  if (xn != yn) return xn ? 1 : -1;
  if (!xn && x->s != y->s) return (x->s > y->s) ? -1 : 1; /* -0 == +0 here */
  return (x->e < y->e) ? -1 : (x->e > y->e) ? 1 : 0;
}

static int id_cmp(const void* a, const void* b) {
  int64_t ea = ((const orc_pair*)a)->e, eb = ((const orc_pair*)b)->e;
  if (ea == eb) return 0;
  return ea < eb ? -1 : 1;
}

ORC_API void orc_topk(const float* scores, int Q, int64_t n_cand, const int32_t* n_valid, int64_t n_entries,
                      const int32_t* cand_blocks, int n_blocks, int k, int32_t* idx, float* top_scores) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int q = 0; q < Q; ++q) {
    const int32_t* blk = cand_blocks ? cand_blocks + (size_t)q * n_blocks : NULL;
    int64_t limit = n_valid ? (int64_t)n_valid[q] : n_entries;
    if (limit > n_entries) limit = n_entries;
    orc_pair* v = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)(n_cand > 0 ? n_cand : 1));
    int64_t m = 0;
    for (int64_t p = 0; p < n_cand; ++p) {
      int64_t e = cand_entry(blk, p);
      if (e < 0 || e >= limit) continue;
      v[m].s = scores[(size_t)q * n_cand + p];
      v[m].e = e;
      ++m;
    }
    qsort(v, (size_t)m, sizeof(orc_pair), rank_cmp);
    int64_t keep = m < k ? m : k;
    qsort(v, (size_t)keep, sizeof(orc_pair), id_cmp);
    for (int j = 0; j < k; ++j) {
      idx[(size_t)q * k + j] = (j < m) ? (int32_t)v[j].e : -1;
      if (top_scores) top_scores[(size_t)q * k + j] = (j < m) ? v[j].s : -INFINITY;
    }
    free(v);
  }
}

/* FP8 window row (R14): value = E4M3(code_c) * E8M0(scale_{c/32}). */
static void swa_fp8_row_f64(const uint8_t* row, double* out512) {
  for (int c = 0; c < 512; ++c) out512[c] = orc_e4m3(row[c]) * orc_e8m0(row[512 + c / 32]);
}

ORC_API void orc_dequant_swa_fp8(const uint8_t* rows, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) swa_fp8_row_f64(rows + (size_t)i * 528, out + (size_t)i * 512);
}

/* ------------------------------------------------------------------ O8 --- */
/* Reindex pool construction (R16): block b covers entries 8b..8b+7 (R6); its
 * score is the best valid entry score in the top-k order (NaN below every
 * number, -0 == +0); the n_pool best blocks are chosen exactly as O4 chooses
 * entries. out: [Q][n_pool] ascending block ids, -1 padded. */
static int score_better(float x, float y) { /* x ranks above y */
  if (isnan(x)) return 0;
  if (isnan(y)) return 1;
  return x > y;
}

ORC_API void orc_pool_blocks(const float* scores, int Q, int64_t n_entries, const int32_t* n_valid, int n_pool,
                             int32_t* out) {
  int64_t nb = (n_entries + 7) / 8;
  float* bs = (float*)malloc(sizeof(float) * (size_t)(Q > 0 ? Q : 1) * (size_t)(nb > 0 ? nb : 1));
  int32_t* nvb = (int32_t*)malloc(sizeof(int32_t) * (size_t)(Q > 0 ? Q : 1));
  for (int q = 0; q < Q; ++q) {
    int64_t lim = n_entries;
    if (n_valid && n_valid[q] < lim) lim = n_valid[q] < 0 ? 0 : n_valid[q];
    nvb[q] = (int32_t)((lim + 7) / 8);
    for (int64_t b = 0; b < nb; ++b) {
      float best = NAN;
      for (int64_t e = 8 * b; e < 8 * b + 8 && e < lim; ++e) {
        float x = scores[(size_t)q * (size_t)n_entries + (size_t)e];
        if (e == 8 * b || score_better(x, best)) best = x;
      }
      bs[(size_t)q * (size_t)nb + (size_t)b] = best;
    }
  }
  orc_topk(bs, Q, nb, nvb, nb, NULL, 0, n_pool, out, NULL);
  free(nvb);
  free(bs);
}

/* Gather of the selected entries (R18): out [Q][k][288], dense_idx [Q][k] = j
 * for a valid id (copied), -1 for a skipped one (its slot left zero). */
ORC_API void orc_gather_selected(const uint8_t* main_cache, int64_t n_entries, int64_t cache_q_stride,
                                 const int32_t* idx, int Q, int k, uint8_t* out, int32_t* dense_idx) {
  for (int q = 0; q < Q; ++q)
    for (int j = 0; j < k; ++j) {
      int64_t e = idx[(size_t)q * k + j];
      uint8_t* dst = out + ((size_t)q * k + j) * 288;
      int ok = e >= 0 && e < n_entries;
      if (ok)
        memcpy(dst, main_cache + (size_t)((int64_t)q * cache_q_stride + e) * 288, 288);
      else
        memset(dst, 0, 288);
      dense_idx[(size_t)q * k + j] = ok ? j : -1;
    }
}

/* ------------------------------------------------------------------ O5 --- */
/* Sparse attention, [ATLAS] role bullet (every non-SWA-only layer attends
 * over the 128-token window plus 512 selected entries) and KV-latent bullet
 * (one 512-wide latent per entry, k = v, shared by all 64 query heads).
 * J = valid selected ids in idx order, then the n_swa window rows (R7, R8).
 * logits l_hj = scale * q_h . K_j; p = softmax_j(l) in max-subtracted form;
 * o_h = sum_j p_hj V_j, all in fp64. Outputs: bf16 (RNE) and/or fp32 of the
 * fp64 result, and optional lse_h = m_h + log(sum_j exp(l_hj - m_h)).
 * probs_out (optional, for tests): [Q][64][k_sel + n_swa] softmax weights in
 * joint-list order, with skipped slots left at 0. Window rows are bf16
 * [..][512], or FP8 [..][528] (R14) when swa_fp8; rope_cs ([Q][32][2] or
 * NULL) rotates the output's rotary pairs back (R15) before the rounding. */
ORC_API void orc_sparse_attn(int Q, int64_t n_entries, int64_t cache_q_stride, const uint8_t* main_cache,
                             const int32_t* idx, int k_sel, const uint16_t* q_bf16, const void* swa,
                             int64_t swa_q_stride, int n_swa, double scale, uint16_t* out_bf16, float* out_f32,
                             float* lse, double* probs_out, int swa_fp8, const float* rope_cs) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int qi = 0; qi < Q; ++qi) {
    int jmax = k_sel + n_swa;
    double* kv = (double*)malloc(sizeof(double) * (size_t)(jmax > 0 ? jmax : 1) * 512);
    int* slot = (int*)malloc(sizeof(int) * (size_t)(jmax > 0 ? jmax : 1));
    int nj = 0;
    for (int j = 0; j < k_sel; ++j) {
      int64_t e = idx[(size_t)qi * k_sel + j];
      if (e < 0 || e >= n_entries) continue; /* R8 */
      main_entry_f64(main_cache + (size_t)((int64_t)qi * cache_q_stride + e) * 288, kv + (size_t)nj * 512);
      slot[nj++] = j;
    }
    for (int r = 0; r < n_swa; ++r) {
      if (swa_fp8) {
        swa_fp8_row_f64((const uint8_t*)swa + (size_t)((int64_t)qi * swa_q_stride + r) * 528, kv + (size_t)nj * 512);
      } else {
        const uint16_t* row = (const uint16_t*)swa + (size_t)((int64_t)qi * swa_q_stride + r) * 512;
        for (int c = 0; c < 512; ++c) kv[(size_t)nj * 512 + c] = bf16_to_f64(row[c]);
      }
      slot[nj++] = k_sel + r;
    }
    double* lg = (double*)malloc(sizeof(double) * (size_t)(nj > 0 ? nj : 1));
    for (int h = 0; h < 64; ++h) {
      double qh[512];
      for (int c = 0; c < 512; ++c) qh[c] = bf16_to_f64(q_bf16[((size_t)qi * 64 + h) * 512 + c]);
      double o[512];
      for (int c = 0; c < 512; ++c) o[c] = 0.0;
      double mx = -INFINITY, z = 0.0;
      for (int j = 0; j < nj; ++j) {
        double d = 0.0;
        for (int c = 0; c < 512; ++c) d += qh[c] * kv[(size_t)j * 512 + c];
        lg[j] = scale * d;
        if (lg[j] > mx) mx = lg[j];
      }
      for (int j = 0; j < nj; ++j) z += exp(lg[j] - mx);
      if (probs_out)
        for (int j = 0; j < jmax; ++j) probs_out[((size_t)qi * 64 + h) * jmax + j] = 0.0;
      for (int j = 0; j < nj; ++j) {
        double p = exp(lg[j] - mx) / z;
        if (probs_out) probs_out[((size_t)qi * 64 + h) * jmax + slot[j]] = p;
        for (int c = 0; c < 512; ++c) o[c] += p * kv[(size_t)j * 512 + c];
      }
      if (rope_cs) { /* R15 */
        for (int i = 0; i < 32; ++i) {
          double cs = rope_cs[((size_t)qi * 32 + i) * 2], sn = rope_cs[((size_t)qi * 32 + i) * 2 + 1];
          double a = o[448 + 2 * i], b = o[449 + 2 * i];
          o[448 + 2 * i] = a * cs + b * sn;
          o[449 + 2 * i] = b * cs - a * sn;
        }
      }
      for (int c = 0; c < 512; ++c) {
        size_t at = ((size_t)qi * 64 + h) * 512 + c;
        if (out_bf16) out_bf16[at] = f64_to_bf16(o[c]);
        if (out_f32) out_f32[at] = (float)o[c];
      }
      if (lse) lse[qi * 64 + h] = (nj > 0) ? (float)(mx + log(z)) : -INFINITY;
    }
    free(lg);
    free(slot);
    free(kv);
  }
}

/* ------------------------------------------------------------------ O6 --- */
/* Fused decode: O2 -> O4 -> O5 ([PERCHY] "shared KV -> candidate pool ->
 * top 512 -> attention"). scores_out/idx_out (optional) expose the stages. */
ORC_API void orc_decode(int Q, int64_t n_entries, int64_t cache_q_stride, const uint8_t* key_codes,
                        const uint8_t* key_scales, const uint8_t* iq_codes, const uint8_t* iq_scales,
                        const float* w, const int32_t* cand_blocks, int n_blocks, const int32_t* n_valid, int k,
                        const uint8_t* main_cache, const uint16_t* q_bf16, const void* swa,
                        int64_t swa_q_stride, int n_swa, double scale, uint16_t* out_bf16, float* out_f32,
                        float* lse, int32_t* idx_out, float* scores_out, int swa_fp8, const float* rope_cs) {
  int64_t n_cand = cand_blocks ? 8 * (int64_t)n_blocks : n_entries;
  float* sc = scores_out ? scores_out : (float*)malloc(sizeof(float) * (size_t)Q * (size_t)(n_cand > 0 ? n_cand : 1));
  int32_t* id = idx_out ? idx_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)Q * (size_t)(k > 0 ? k : 1));
  orc_index_score(Q, n_entries, cache_q_stride, key_codes, key_scales, iq_codes, iq_scales, w, cand_blocks, n_blocks,
                  n_valid, sc, NULL);
  orc_topk(sc, Q, n_cand, n_valid, n_entries, cand_blocks, n_blocks, k, id, NULL);
  orc_sparse_attn(Q, n_entries, cache_q_stride, main_cache, id, k, q_bf16, swa, swa_q_stride, n_swa, scale, out_bf16,
                  out_f32, lse, NULL, swa_fp8, rope_cs);
  if (!scores_out) free(sc);
  if (!idx_out) free(id);
}

ORC_API void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

ORC_API int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
