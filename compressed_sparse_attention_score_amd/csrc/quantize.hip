// csa2_quantize kernels: new fp32 / bf16 values -> stored FP4 cache entries.
//
// Formats ("An infra-oriented diagram of the DeepSeek-V4.1-Flash architecture",
// Full-layer cache bullet and "The KV cache"): a main latent is 512 E2M1 codes
// with one E4M3 scale per 16 channels (288 bytes); an indexer key is 128 E2M1
// codes with one E8M0 scale per 32 channels (64 + 4 bytes). The pages fix the
// formats, not the rounding; the rule implemented here is:
//   main scale   E4M3FN value nearest to amax/6, ties to the even code,
//                saturating at 448;
//   index scale  2^e, e the smallest integer in [-127, 127] with 6*2^e >= amax
//                (e = 0 for an all-zero block);
//   element      E2M1 magnitude nearest to |x|/scale, ties to the even code,
//                saturating at 6, with the sign bit of x; all codes are zero
//                when the main scale is zero or the index block is all zero;
//   NaN counts as a zero magnitude, +-inf as the largest one.
//
// Every decision is an exact fp32 comparison: thresholds such as scale * 1.25
// or 3 * (two adjacent E4M3 values) have at most 7 significant bits, so no
// quotient is ever rounded and the result is the exact nearest code.
//
// Thread layout: each lane encodes 16 consecutive channels (a main scale
// group, or half of an indexer scale block), so the scale and its thresholds
// are worked out once per 16 values; waves stream tiles of 64 such groups
// through LDS so that the HBM reads stay fully coalesced (see k_quantize).
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

// Workgroup cap of a quantiser launch. One tile per wave measured fastest (a
// 131072-row write fills 16384 workgroups); only larger writes loop.
constexpr int64_t kQuantGroups = 65536;

namespace {

// |x| as ordered bits, NaN -> 0 (so that integer max is the float max).
__device__ __forceinline__ unsigned mag_bits(float x) {
  unsigned u = __float_as_uint(x) & 0x7FFFFFFFu;
  return u > 0x7F800000u ? 0u : u;
}

// Largest magnitude of a block, NaNs counting as zero. The plain integer max
// of the magnitude bits is a NaN pattern only when the block holds a NaN;
// only then is the block scanned again without them.
template <int G>
__device__ __forceinline__ float block_amax(const float (&f)[G]) {
  unsigned m = 0;
#pragma unroll
  for (int i = 0; i < G; ++i) m = max(m, __float_as_uint(f[i]) & 0x7FFFFFFFu);
  if (m > 0x7F800000u) {
    m = 0;
#pragma unroll
    for (int i = 0; i < G; ++i) m = max(m, mag_bits(f[i]));
  }
  return __uint_as_float(m);
}

// Non-negative E4M3FN code -> value, codes 0..0x7E: c * 2^-9 below 8, else
// bits (c << 20) + (120 << 23) (exponent field c >> 3, mantissa c & 7).
__device__ __forceinline__ float e4m3_pos_value(int c) {
  float sub = (float)c * 0x1p-9f;
  float nrm = __uint_as_float(((unsigned)c << 20) + 0x3C000000u);
  return c < 8 ? sub : nrm;
}

// Largest float below t when `odd`, else t: comparing y > result is y >= t
// for an odd lower code (a tie rounds up to the even neighbour) and y > t for
// an even one. t is a positive float (inf gives FLT_MAX).
__device__ __forceinline__ float tie_nudge(float t, bool odd) {
  return __uint_as_float(__float_as_uint(t) - (odd ? 1u : 0u));
}

// E4M3 code of the scale of a main block with largest magnitude a (a >= 0,
// not NaN): nearest to a/6, ties to the even code, saturating at 448 (0x7E).
// The floor code c of an approximate a/6 is off by at most one (the quotient
// is within a few ulp and the E4M3 grid is 2^-3 relative, 2^-9 absolute
// below 2^-6), so the answer lies in [c-1, c+2]: counting the exact
// midpoints 6 * (val(k) + val(k+1)) / 2 that a passes from lo = c-1 gives it.
// 3 * (val(k) + val(k+1)) has at most 7 significant bits, so is exact.
__device__ __forceinline__ unsigned e4m3_scale_code(float a) {
  float v = a * (1.0f / 6.0f);
  int cn = (int)(__float_as_uint(v) >> 20) - 960;  // v >= 2^-6 (inf: large)
  int cs = (int)(v * 512.0f);                      // v < 2^-6
  int c = v < 0x1p-6f ? cs : cn;
  int lo = min(max(c - 1, 0), 0x7B);
  float w0 = 3.0f * e4m3_pos_value(lo), w1 = 3.0f * e4m3_pos_value(lo + 1);
  float w2 = 3.0f * e4m3_pos_value(lo + 2), w3 = 3.0f * e4m3_pos_value(lo + 3);
  bool odd = lo & 1;
  unsigned r = (unsigned)lo;
  r += a > tie_nudge(w0 + w1, odd) ? 1u : 0u;
  r += a > tie_nudge(w1 + w2, !odd) ? 1u : 0u;
  r += a > tie_nudge(w2 + w3, odd) ? 1u : 0u;
  return r;
}

// Exponent e of the E8M0 scale of an index block with largest magnitude a:
// the smallest e in [-127, 127] with a * 2^-e <= 6 (0 when a == 0). The
// estimate from the bits of an approximate a/6 is off by at most one; two
// exact tests on a * 2^-e (a power-of-two scaling, exact here) settle it.
__device__ __forceinline__ int e8m0_scale_exp(float a) {
  unsigned vb = __float_as_uint(a * (1.0f / 6.0f));
  int e = (int)(vb >> 23) - 127 + ((vb & 0x7FFFFFu) != 0u ? 1 : 0);
  e = min(max(e, -127), 127);
  e += (e < 127 && __builtin_amdgcn_ldexpf(a, -e) > 6.0f) ? 1 : 0;
  e -= (e > -127 && __builtin_amdgcn_ldexpf(a, 1 - e) <= 6.0f) ? 1 : 0;
  return a == 0.0f ? 0 : e;
}

// E2M1 thresholds: the midpoints between consecutive E2M1 magnitudes
// (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) in the block's units, nudged for the
// tie rule. An element's magnitude code is the number of thresholds below
// |x| (NaN: 0; beyond the last: 7, the saturated code).
struct Thresholds {
  float t[7];
};

// Main blocks: scale s is an E4M3 value (>= 2^-9, <= 448); s * midpoint has
// at most 7 significant bits and is a normal float, hence exact.
__device__ __forceinline__ Thresholds thresholds_e4m3(float s) {
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  Thresholds r;
#pragma unroll
  for (int k = 0; k < 7; ++k) r.t[k] = tie_nudge(s * mids[k], k & 1);
  return r;
}

// Index blocks: scale 2^e. midpoint * 2^e is exact (subnormal included) or
// overflows to inf, which only happens for e = 127 (an inf in the block):
// there the even thresholds are brought down to FLT_MAX and the nudged odd
// ones are FLT_MAX already, so inf still passes every threshold while no
// finite value passes one beyond the float range.
__device__ __forceinline__ Thresholds thresholds_e8m0(int e) {
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  Thresholds r;
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    float t = __builtin_amdgcn_ldexpf(mids[k], e);
    r.t[k] = (k & 1) ? tie_nudge(t, true) : fminf(t, 0x1.fffffep127f);
  }
  return r;
}

// E2M1 magnitude code of y: the number of thresholds below y, found by a
// three-level binary search over the sorted thresholds (is it above t3? then
// above t5 or t1? then above the one threshold left between the two codes).
__device__ __forceinline__ unsigned e2m1_mag(float y, const Thresholds& th) {
  bool b2 = y > th.t[3];
  bool b1 = y > (b2 ? th.t[5] : th.t[1]);
  float lo = b1 ? th.t[2] : th.t[0];
  float hi = b1 ? th.t[6] : th.t[4];
  bool b0 = y > (b2 ? hi : lo);
  return (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
}

// Eight E2M1 codes in one word: nibble i (bits 4i..4i+3) is channel i, i.e.
// byte j holds channel 2j in its low nibble and 2j+1 in its high one. Each
// code is the magnitude code with the sign bit of x on bit 3.
__device__ __forceinline__ unsigned encode8(const float* f, const Thresholds& th) {
  unsigned w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    unsigned sgn = (__float_as_uint(f[i]) >> (28 - 4 * i)) & (8u << (4 * i));
    w |= (e2m1_mag(fabsf(f[i]), th) << (4 * i)) | sgn;
  }
  return w;
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Largest of a and the value of the neighbouring lane (lane ^ 1), for
// non-negative floats compared as bits (quad_perm [1,0,3,2]).
__device__ __forceinline__ float pair_max(float a) {
  unsigned u = __float_as_uint(a);
  return __uint_as_float(max(u, (unsigned)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, false)));
}

// One kernel for both formats and input types. The unit of work is a
// half-block of 16 channels: a main scale group, or half of an indexer scale
// block (the two halves are neighbouring lanes and share their maximum).
//
// Each wave streams tiles of 64 consecutive half-blocks (4 KiB of fp32, 2 KiB
// of bf16): the tile is read with coalesced 16-B loads (lane l takes chunks
// l, l+64, ...), written to a wave-private, padded LDS area and read back so
// that lane l holds half-block l; reading 64 B per lane straight from HBM
// instead would touch every cache line four times per load instruction and
// cost a third of the bandwidth. The next tile's loads are issued before the
// current one is encoded.
// Softmax-gated mean of two tokens' channel values (m=2 pooling): weights
// 1/(1+e) and e/(1+e) with e = exp(-|g_b - g_a|), the larger going to the
// token with the larger logit, so nothing overflows.
__device__ __forceinline__ float gated_pair(float xa, float xb, float ga, float gb) {
  const float d = gb - ga;
  const float e = expf(-fabsf(d));
  const float big = 1.0f / (1.0f + e), small = e * big;
  const float pa = d <= 0.0f ? big : small, pb = d <= 0.0f ? small : big;
  return pa * xa + pb * xb;
}

// GATE = 0: rows quantised as given. GATE = 1 / 512 (main latents, fp32 only):
// row i of the output is the m=2 pooling of input rows 2i and 2i+1 under one
// gate logit per token / per channel, optionally stored as fp32 in `pooled`.
template <bool BF16, bool INDEX, int GATE>
__global__ __launch_bounds__(256) void k_quantize(const void* __restrict__ x, int64_t n,
                                                  const int64_t* __restrict__ rows, int64_t n_rows,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  const float* __restrict__ gate, float* __restrict__ pooled) {
  static_assert(GATE == 0 || (!BF16 && !INDEX), "pooling takes fp32 main latents");
  constexpr int C = BF16 ? 2 : 4;  // 16-B chunks per half-block
  constexpr int S = C + 1;         // padded stride: lanes read distinct LDS banks
  constexpr int SHIFT = INDEX ? 3 : 5;  // half-blocks per entry: 8 (index), 32 (main)
  __shared__ v4u lds[4][64 * S];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nhb = n << SHIFT, nchunk = nhb * C;
  const int64_t ntile = (nhb + 63) >> 6, wstride = (int64_t)gridDim.x * 4;
  int64_t tile = (int64_t)blockIdx.x * 4 + w;
  if (tile >= ntile) return;
  const v4u* src = (const v4u*)x;
  v4u reg[C];
  // pooling: the second token's chunks and both tokens' gates (per token: x
  // lane of ga/gb holds the logit)
  v4u xb[GATE ? C : 1], ga[GATE ? C : 1], gb[GATE ? C : 1];
  int64_t row_next;
  // Loads of tile t; indexes past the end are clamped to the last chunk (their
  // half-blocks are never stored), so no load sits behind a branch. The
  // destination row is loaded first and checked only at the store, so that
  // nothing waits on these loads before the tile is needed.
  auto fetch = [&](int64_t t) {
    const int64_t e = min(t * 64 + lane, nhb - 1) >> SHIFT;
    row_next = rows ? rows[e] : e;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      int64_t c = min(t * 64 * C + lane + 64 * j, nchunk - 1);
      if constexpr (GATE == 0) {
        reg[j] = __builtin_nontemporal_load(src + c);
      } else {
        // output chunk c = entry c/128, channels 4(c%128)..+3; token rows 2e, 2e+1
        const int64_t ca = c + (c >> 7) * 128;
        reg[j] = __builtin_nontemporal_load(src + ca);
        xb[j] = __builtin_nontemporal_load(src + ca + 128);
        if constexpr (GATE == 512) {
          ga[j] = __builtin_nontemporal_load((const v4u*)gate + ca);
          gb[j] = __builtin_nontemporal_load((const v4u*)gate + ca + 128);
        } else {
          ga[j][0] = __float_as_uint(gate[2 * (c >> 7)]);
          gb[j][0] = __float_as_uint(gate[2 * (c >> 7) + 1]);
        }
      }
    }
  };
  fetch(tile);
  for (;;) {
    if constexpr (GATE != 0) {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        v4u p;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int kg = GATE == 512 ? k : 0;
          p[k] = __float_as_uint(gated_pair(__uint_as_float(reg[j][k]), __uint_as_float(xb[j][k]),
                                            __uint_as_float(ga[j][kg]), __uint_as_float(gb[j][kg])));
        }
        reg[j] = p;
        const int64_t c = tile * 64 * C + lane + 64 * j;
        if (pooled && c < nchunk) *((v4u*)pooled + c) = p;
      }
    }
#pragma unroll
    for (int j = 0; j < C; ++j) {
      int c = lane + 64 * j;
      lds[w][(c / C) * S + (c % C)] = reg[j];
    }
    const int64_t row = row_next;
    __builtin_amdgcn_wave_barrier();
    const int64_t next = tile + wstride;
    if (next < ntile) fetch(next);
    float f[16];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      v4u v = lds[w][lane * S + i];
      if (BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[8 * i + 2 * j] = __uint_as_float(v[j] << 16);
          f[8 * i + 2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[4 * i + j] = __uint_as_float(v[j]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    const int64_t hb = tile * 64 + lane;
    const int h = (int)(hb & ((1 << SHIFT) - 1));
    if (INDEX) {
      float a = pair_max(block_amax(f));  // both lanes of the pair run this
      int ex = e8m0_scale_exp(a);
      v2u cw = {0u, 0u};
      if (a != 0.0f) {
        Thresholds th = thresholds_e8m0(ex);
        cw = v2u{encode8(f, th), encode8(f + 8, th)};
      }
      if (hb < nhb && row >= 0 && row < n_rows) {
        *(v2u*)(codes + row * 64 + 8 * h) = cw;
        if ((h & 1) == 0) scales[row * 4 + (h >> 1)] = (uint8_t)(ex + 127);
      }
    } else {
      unsigned sc = e4m3_scale_code(block_amax(f));
      v2u cw = {0u, 0u};
      if (sc != 0u) {
        Thresholds th = thresholds_e4m3(e4m3_pos_value((int)sc));
        cw = v2u{encode8(f, th), encode8(f + 8, th)};
      }
      if (hb < nhb && row >= 0 && row < n_rows) {
        uint8_t* ent = codes + row * kMainBytes;
        *(v2u*)(ent + 8 * h) = cw;
        ent[256 + h] = (uint8_t)sc;
      }
    }
    if (next >= ntile) break;
    tile = next;
  }
}

}  // namespace

hipError_t launch_quantize(int kind, const void* x, int in_bf16, int64_t n, const int64_t* rows, int64_t n_rows,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t nhb = n * (kind == 0 ? 32 : 8), ntile = (nhb + 63) / 64;
  // Four waves per workgroup, one tile per wave at a time; large writes cap
  // the grid at kQuantGroups workgroups and loop.
  const int64_t groups = (ntile + 3) / 4;
  dim3 grid((unsigned)(groups < kQuantGroups ? groups : kQuantGroups));
  if (kind == 0) {
    if (in_bf16)
      k_quantize<true, false, 0><<<grid, 256, 0, s>>>(x, n, rows, n_rows, codes, scales, nullptr, nullptr);
    else
      k_quantize<false, false, 0><<<grid, 256, 0, s>>>(x, n, rows, n_rows, codes, scales, nullptr, nullptr);
  } else {
    if (in_bf16)
      k_quantize<true, true, 0><<<grid, 256, 0, s>>>(x, n, rows, n_rows, codes, scales, nullptr, nullptr);
    else
      k_quantize<false, true, 0><<<grid, 256, 0, s>>>(x, n, rows, n_rows, codes, scales, nullptr, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_pool_quantize(const float* x, const float* gate, int gate_width, int64_t n, const int64_t* rows,
                                int64_t n_rows, uint8_t* cache, float* pooled, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t ntile = (n * 32 + 63) / 64, groups = (ntile + 3) / 4;
  dim3 grid((unsigned)(groups < kQuantGroups ? groups : kQuantGroups));
  if (gate_width == 1)
    k_quantize<false, false, 1><<<grid, 256, 0, s>>>(x, n, rows, n_rows, cache, nullptr, gate, pooled);
  else
    k_quantize<false, false, 512><<<grid, 256, 0, s>>>(x, n, rows, n_rows, cache, nullptr, gate, pooled);
  return hipGetLastError();
}

}  // namespace csa2
