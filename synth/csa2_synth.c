/*
 * Seeded synthetic inputs for the CSA2 global-attention path.
 *
 * This module only MAKES inputs: random numbers, the storage quantisation that
 * turns N(0,1) vectors into cache entries, and candidate-pool block lists. It
 * holds none of the scoring, selection or attention arithmetic; the CPU oracle
 * and the HIP library both consume the bytes it writes.
 *
 * Random stream: a counter-based generator. Each value is the SplitMix64
 * finaliser (Steele, Lea & Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) applied to
 *     seed ^ (tensor_id << 56) ^ (seq << 40) ^ counter
 * so any element of any tensor can be produced independently and in parallel.
 * Normals come in Box-Muller pairs: element 2j uses the cosine and 2j+1 the
 * sine branch of the transform of counters 2j and 2j+1.
 *
 * Storage formats follow "An infra-oriented diagram of the DeepSeek-V4.1-Flash
 * architecture" (Reading notes, the Full-layer cache bullet; section "The KV
 * cache"): a main entry is 512 FP4 E2M1 codes plus one E4M3 scale per 16
 * channels (288 bytes); an indexer key is 128 FP4 codes plus one E8M0 scale per
 * 32 channels (68 bytes). Code byte j packs channel 2j in its low nibble and
 * channel 2j+1 in its high nibble.
 *
 * Quantisation recipe (synthetic-workload definition):
 *   main   : per 16 channels, scale = E4M3 round-to-nearest-even of amax/6
 *            (saturating at 448), code = E2M1 RNE of x/scale (saturating at 6).
 *   index  : per 32 channels, scale = 2^ceil(log2(amax/6)) as E8M0,
 *            code = E2M1 RNE of x/scale (never saturates).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYN_API __attribute__((visibility("default")))

enum { TID_MAIN = 0, TID_IKEY = 1, TID_IQ = 2, TID_W = 3, TID_Q = 4, TID_SWA = 5, TID_POOL = 6 };

static uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t ctr_bits(uint64_t seed, uint64_t tid, uint64_t seq, uint64_t ctr) {
  return splitmix64(seed ^ (tid << 56) ^ (seq << 40) ^ ctr);
}

/* uniform in [0,1) with 53 random bits */
static double ctr_uniform(uint64_t seed, uint64_t tid, uint64_t seq, uint64_t ctr) {
  return (double)(ctr_bits(seed, tid, seq, ctr) >> 11) * (1.0 / 9007199254740992.0);
}

static void ctr_normal_pair(uint64_t seed, uint64_t tid, uint64_t seq, uint64_t pair, double* z) {
  double u1 = 1.0 - ctr_uniform(seed, tid, seq, 2 * pair); /* (0,1] */
  double u2 = ctr_uniform(seed, tid, seq, 2 * pair + 1);
  double r = sqrt(-2.0 * log(u1)), t = 6.283185307179586476925 * u2;
  z[0] = r * cos(t);
  z[1] = r * sin(t);
}

static double ctr_normal(uint64_t seed, uint64_t tid, uint64_t seq, uint64_t elem) {
  double z[2];
  ctr_normal_pair(seed, tid, seq, elem >> 1, z);
  return z[elem & 1];
}

/* n (even) consecutive normals starting at an even element */
static void ctr_normals(uint64_t seed, uint64_t tid, uint64_t seq, uint64_t first, int n, double* out) {
  for (int i = 0; i < n; i += 2) ctr_normal_pair(seed, tid, seq, (first >> 1) + (uint64_t)(i >> 1), out + i);
}

SYN_API double syn_normal(uint64_t seed, int tid, uint64_t seq, uint64_t elem) {
  return ctr_normal(seed, (uint64_t)tid, seq, elem);
}

SYN_API uint64_t syn_bits(uint64_t seed, int tid, uint64_t seq, uint64_t ctr) {
  return ctr_bits(seed, (uint64_t)tid, seq, ctr);
}

/* ---- storage encoders (input construction only) ------------------------ */

/* E2M1 magnitude code for v >= 0, round to nearest, ties to the even code,
 * saturating at 6. Magnitudes by code: 0, .5, 1, 1.5, 2, 3, 4, 6. */
static unsigned enc_e2m1_mag(double v) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  if (!(v > 0.0)) return 0;
  if (v >= 6.0) return 7;
  unsigned lo = 0;
  while (lo < 7 && mag[lo + 1] <= v) lo++;
  if (lo == 7) return 7;
  double dlo = v - mag[lo], dhi = mag[lo + 1] - v;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return lo + 1;
  return (lo & 1u) ? lo + 1 : lo; /* tie: even code */
}

static unsigned enc_e2m1(double x) {
  unsigned c = enc_e2m1_mag(fabs(x));
  return (x < 0.0) ? (c | 8u) : c;
}

/* E4M3 (OCP E4M3FN) code for v >= 0, RNE, saturating at 448. */
static unsigned enc_e4m3_pos(double v) {
  if (!(v > 0.0)) return 0;
  if (v >= 448.0) return 0x7E;
  int E;
  frexp(v, &E); /* v = f * 2^E, f in [0.5,1) -> leading bit exponent E-1 */
  int ex = E - 1;
  if (ex < -6) { /* subnormal range: step 2^-9 */
    double m = nearbyint(v * 512.0);
    return (unsigned)m; /* m == 8 is exactly the smallest normal, code 0x08 */
  }
  double q = nearbyint(ldexp(v, 3 - ex)); /* in [8,16] */
  if (q >= 16.0) { q = 8.0; ex += 1; }
  int field = ex + 7;
  unsigned code = ((unsigned)field << 3) | ((unsigned)q - 8u);
  if (code > 0x7E) code = 0x7E;
  return code;
}

static double dec_e4m3_pos(unsigned b) { /* encoder-side helper: value of a positive finite code */
  unsigned e = (b >> 3) & 15u, m = b & 7u;
  return e ? ldexp(1.0 + m / 8.0, (int)e - 7) : ldexp(m / 8.0, -6);
}

static void quant_main_entry(const double* x, uint8_t* out) {
  memset(out, 0, 288);
  for (int g = 0; g < 32; ++g) {
    double amax = 0.0;
    for (int c = 0; c < 16; ++c) amax = fmax(amax, fabs(x[16 * g + c]));
    unsigned sc = enc_e4m3_pos(amax / 6.0);
    out[256 + g] = (uint8_t)sc;
    double s = dec_e4m3_pos(sc);
    for (int c = 0; c < 16; ++c) {
      int ch = 16 * g + c;
      unsigned code = (s > 0.0) ? enc_e2m1(x[ch] / s) : 0u;
      out[ch >> 1] |= (uint8_t)(code << ((ch & 1) ? 4 : 0));
    }
  }
}

static void quant_mx_row(const double* x, int n, uint8_t* codes, uint8_t* scales) {
  memset(codes, 0, (size_t)n / 2);
  for (int g = 0; g < n / 32; ++g) {
    double amax = 0.0;
    for (int c = 0; c < 32; ++c) amax = fmax(amax, fabs(x[32 * g + c]));
    int ex = 0;
    if (amax > 0.0) {
      int E;
      double f = frexp(amax / 6.0, &E);
      ex = (f == 0.5) ? E - 1 : E; /* ceil(log2(amax/6)) */
    }
    if (ex < -127) ex = -127;
    if (ex > 127) ex = 127;
    scales[g] = (uint8_t)(ex + 127);
    for (int c = 0; c < 32; ++c) {
      int ch = 32 * g + c;
      unsigned code = (amax > 0.0) ? enc_e2m1(ldexp(x[ch], -ex)) : 0u;
      codes[ch >> 1] |= (uint8_t)(code << ((ch & 1) ? 4 : 0));
    }
  }
}

/* ---- tensors ------------------------------------------------------------ */

/* Main latents of sequence `seq`, entries [first, first+n): entry e uses
 * elements e*512 + c of stream TID_MAIN. out: [n][288]. */
SYN_API void syn_main_latents(uint64_t seed, uint64_t seq, int64_t first, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double x[512];
    uint64_t e = (uint64_t)(first + i);
    ctr_normals(seed, TID_MAIN, seq, e * 512u, 512, x);
    quant_main_entry(x, out + (size_t)i * 288);
  }
}

/* Main latents for an explicit list of entry ids (pool entries of a sparse
 * cache). out: [n][288] in list order. */
SYN_API void syn_main_latents_list(uint64_t seed, uint64_t seq, const int64_t* ids, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double x[512];
    uint64_t e = (uint64_t)ids[i];
    ctr_normals(seed, TID_MAIN, seq, e * 512u, 512, x);
    quant_main_entry(x, out + (size_t)i * 288);
  }
}

/* Indexer keys: entry e uses elements e*128 + c of TID_IKEY.
 * codes [n][64], scales [n][4]. */
SYN_API void syn_index_keys(uint64_t seed, uint64_t seq, int64_t first, int64_t n, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double x[128];
    uint64_t e = (uint64_t)(first + i);
    ctr_normals(seed, TID_IKEY, seq, e * 128u, 128, x);
    quant_mx_row(x, 128, codes + (size_t)i * 64, scales + (size_t)i * 4);
  }
}

SYN_API void syn_index_keys_list(uint64_t seed, uint64_t seq, const int64_t* ids, int64_t n, uint8_t* codes,
                                 uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double x[128];
    uint64_t e = (uint64_t)ids[i];
    ctr_normals(seed, TID_IKEY, seq, e * 128u, 128, x);
    quant_mx_row(x, 128, codes + (size_t)i * 64, scales + (size_t)i * 4);
  }
}

/* Indexer queries for queries [first, first+n): query i is sequence i, head h
 * uses elements h*128 + c of TID_IQ. codes [n][32][64], scales [n][32][4]. */
SYN_API void syn_index_queries(uint64_t seed, int64_t first, int64_t n, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    for (int h = 0; h < 32; ++h) {
      double x[128];
      ctr_normals(seed, TID_IQ, (uint64_t)(first + i), (uint64_t)(h * 128), 128, x);
      quant_mx_row(x, 128, codes + ((size_t)i * 32 + h) * 64, scales + ((size_t)i * 32 + h) * 4);
    }
  }
}

/* Head weights N(0, 1/32) (variance 1/32): w [n][32] fp32. */
SYN_API void syn_head_weights(uint64_t seed, int64_t first, int64_t n, float* w) {
  const double sd = sqrt(1.0 / 32.0);
  for (int64_t i = 0; i < n; ++i)
    for (int h = 0; h < 32; ++h) w[i * 32 + h] = (float)(sd * ctr_normal(seed, TID_W, (uint64_t)(first + i), (uint64_t)h));
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* FP8 window rows (512 channels, 528 bytes each): rows [first_row, +n_rows)
 * of stream (tid, seq), row r using elements r*512 + c, quantised as OCP
 * MXFP8: per 32 channels an E8M0 scale 2^e with e the smallest integer in
 * [-127, 127] such that 448 * 2^e >= amax (0 for an all-zero block), codes
 * E4M3FN(x / 2^e) rounded to nearest even, saturating at 448. Layout: 512
 * codes (byte c = channel c), then the 16 scale bytes. */
SYN_API void syn_fp8_rows(uint64_t seed, int tid, uint64_t seq, int64_t first_row, int64_t n_rows, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    double x[512];
    ctr_normals(seed, (uint64_t)tid, seq, (uint64_t)(first_row + r) * 512u, 512, x);
    uint8_t* o = out + (size_t)r * 528;
    for (int b = 0; b < 16; ++b) {
      double amax = 0.0;
      for (int c = 0; c < 32; ++c) amax = fmax(amax, fabs(x[32 * b + c]));
      int e = 0;
      if (amax > 0.0) {
        e = -127;
        while (e < 127 && 448.0 * ldexp(1.0, e) < amax) ++e;
      }
      o[512 + b] = (uint8_t)(e + 127);
      for (int c = 0; c < 32; ++c) {
        double v = ldexp(x[32 * b + c], -e);
        unsigned code = enc_e4m3_pos(fabs(v));
        o[32 * b + c] = (uint8_t)(code | (v < 0.0 ? 0x80u : 0u));
      }
    }
  }
}

/* fp32 N(0,1) rows: rows [first_row, first_row + n_rows) of width `width`
 * (even) of stream (tid, seq), row r using elements r*width + c. On the
 * main-latent and indexer-key streams these are the unquantised values the
 * stored cache entries were made from, rounded to fp32. */
SYN_API void syn_f32_rows(uint64_t seed, int tid, uint64_t seq, int64_t first_row, int64_t n_rows, int width,
                          float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    double x[1024];
    for (int c0 = 0; c0 < width; c0 += 1024) {
      int n = width - c0 < 1024 ? width - c0 : 1024;
      ctr_normals(seed, (uint64_t)tid, seq, (uint64_t)(first_row + r) * (uint64_t)width + (uint64_t)c0, n, x);
      for (int c = 0; c < n; ++c) out[(size_t)r * (size_t)width + (size_t)(c0 + c)] = (float)x[c];
    }
  }
}

/* bf16 N(0,1) values: element `first + i` of stream (tid, seq). */
SYN_API void syn_bf16_normal(uint64_t seed, int tid, uint64_t seq, int64_t first, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne((float)ctr_normal(seed, (uint64_t)tid, seq, (uint64_t)(first + i)));
}

/* bf16 N(0,1) rows: rows [first_row, first_row + n_rows) of width `width`
 * (even) of stream (tid, seq); row r uses elements r*width + c. */
SYN_API void syn_bf16_rows(uint64_t seed, int tid, uint64_t seq, int64_t first_row, int64_t n_rows, int width,
                           uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    double z[2];
    for (int c = 0; c < width; c += 2) {
      ctr_normal_pair(seed, (uint64_t)tid, seq, ((uint64_t)(first_row + r) * (uint64_t)width + (uint64_t)c) >> 1, z);
      out[r * width + c] = f32_to_bf16_rne((float)z[0]);
      out[r * width + c + 1] = f32_to_bf16_rne((float)z[1]);
    }
  }
}

/* Candidate pool: n_pick distinct block ids out of [0, n_total), ascending,
 * by selection sampling (Knuth, TAOCP vol. 2, Algorithm S) driven by the
 * counter stream TID_POOL of sequence `seq`. */
SYN_API void syn_pool_blocks(uint64_t seed, uint64_t seq, int64_t n_pick, int64_t n_total, int32_t* out) {
  int64_t picked = 0;
  for (int64_t t = 0; t < n_total && picked < n_pick; ++t) {
    double u = ctr_uniform(seed, TID_POOL, seq, (uint64_t)t);
    if ((double)(n_total - t) * u < (double)(n_pick - picked)) out[picked++] = (int32_t)t;
  }
}
