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
// Thread layout: one thread per 4 consecutive channels (one 16-B fp32 load or
// one 8-B bf16 load), so a wave reads 1 KiB (fp32) of contiguous input. A
// main scale group is a quad of lanes, an index scale block 8 lanes; the block
// maximum is combined with DPP lane moves. Each lane stores its two code bytes
// and the first lane of a group stores the scale byte.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {
namespace {

// |x| as ordered bits, NaN -> 0 (so that integer max is the float max).
__device__ __forceinline__ unsigned mag_bits(float x) {
  unsigned u = __float_as_uint(x) & 0x7FFFFFFFu;
  return u > 0x7F800000u ? 0u : u;
}

template <int CTRL>
__device__ __forceinline__ unsigned umax_dpp(unsigned x) {
  return max(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false));
}

// Maximum over lanes 4i..4i+3 (quad_perm [1,0,3,2] then [2,3,0,1]).
__device__ __forceinline__ unsigned quad_umax(unsigned x) { return umax_dpp<0x4E>(umax_dpp<0xB1>(x)); }

// Maximum over lanes 8i..8i+7: quad maximum, then the mirrored quad of the
// same half-row (row_half_mirror maps lane j of a half-row to lane 7-j).
__device__ __forceinline__ unsigned oct_umax(unsigned x) { return umax_dpp<0x141>(quad_umax(x)); }

// Non-negative E4M3FN code -> value (codes 0..0x7E; subnormals step 2^-9).
__device__ __forceinline__ float e4m3_pos_value(unsigned c) {
  return (c < 8u) ? (float)c * 0x1p-9f : __uint_as_float(((c >> 3) + 120u) << 23 | (c & 7u) << 20);
}

// E4M3 code of the scale for a main block with maximum magnitude a (a >= 0,
// not NaN): nearest to a/6, ties to even, saturating at 448 (code 0x7E).
__device__ __forceinline__ unsigned e4m3_scale_code(float a) {
  if (a >= 2688.0f) return 0x7Eu;  // 6 * 448 and above (including inf)
  // Floor code of an approximate a/6, then corrected by exact comparisons.
  float v = a * (1.0f / 6.0f);
  unsigned vb = __float_as_uint(v);
  int c;
  if (v < 0x1p-6f) {
    c = (int)(v * 512.0f);
    c = c > 8 ? 8 : c;
  } else {
    c = (int)(((vb >> 23) - 120u) << 3 | ((vb >> 20) & 7u));
    c = c > 0x7E ? 0x7E : c;
  }
  // v is within a few ulp of a/6 and the E4M3 grid is 2^-3 relative (2^-9
  // absolute below 2^-6), so the floor code is off by at most one.
  if (c > 0 && 6.0f * e4m3_pos_value((unsigned)c) > a) --c;
  if (c < 0x7E && 6.0f * e4m3_pos_value((unsigned)c + 1u) <= a) ++c;
  if (c < 0x7E) {
    float mid6 = 3.0f * (e4m3_pos_value((unsigned)c) + e4m3_pos_value((unsigned)c + 1u));
    if (a > mid6 || (a == mid6 && (c & 1))) ++c;
  }
  return (unsigned)c;
}

// Exponent e of the E8M0 scale for an index block with maximum magnitude a:
// the smallest e in [-127, 127] with a * 2^-e <= 6 (0 when a == 0).
__device__ __forceinline__ int e8m0_scale_exp(float a) {
  if (a == 0.0f) return 0;
  float v = a * (1.0f / 6.0f);
  // ceil(log2(v)) from the bits of the approximate quotient (subnormal v: the
  // clamp below takes over), then exact corrections on a * 2^-e.
  unsigned vb = __float_as_uint(v);
  int e = (int)(vb >> 23) - 127 + ((vb & 0x7FFFFFu) != 0u);
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  if (e < 127 && __builtin_amdgcn_ldexpf(a, -e) > 6.0f) ++e;
  if (e > -127 && __builtin_amdgcn_ldexpf(a, -(e - 1)) <= 6.0f) --e;
  return e;
}

// E2M1 magnitude code of y against thresholds t[0..6] (the midpoints of the
// E2M1 values scaled to y's units; the odd ones lowered by one ulp so that a
// tie there rounds up to the even code): the count of thresholds below y.
// NaN gives 0, anything above the last threshold 7.
struct Thresholds {
  float t[7];
};

__device__ __forceinline__ Thresholds make_thresholds(float s) {
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  Thresholds r;
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    float t = s * mids[k];  // exact: <= 4 significant bits times <= 3
    r.t[k] = (k & 1) ? __uint_as_float(__float_as_uint(t) - 1u) : t;
  }
  return r;
}

__device__ __forceinline__ unsigned e2m1_code(float x, const Thresholds& th) {
  float y = fabsf(x);
  unsigned c = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) c += (y > th.t[k]) ? 1u : 0u;
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Channels 4t..4t+3 of the input as fp32 (bf16 widens exactly).
template <bool BF16>
__device__ __forceinline__ v4f load4(const void* x, int64_t t) {
  if (BF16) {
    v2u h = __builtin_nontemporal_load((const v2u*)x + t);
    return v4f{__uint_as_float(h.x << 16), __uint_as_float(h.x & 0xFFFF0000u), __uint_as_float(h.y << 16),
               __uint_as_float(h.y & 0xFFFF0000u)};
  } else {
    return __builtin_nontemporal_load((const v4f*)x + t);
  }
}

// Destination row of entry e, or -1 when it is out of range.
__device__ __forceinline__ int64_t dst_row(const int64_t* rows, int64_t e, int64_t n_rows) {
  int64_t r = rows ? rows[e] : e;
  return (r >= 0 && r < n_rows) ? r : -1;
}

// Main latents: thread t covers channels 4q..4q+3 of entry t/128 (q = t%128).
template <bool BF16>
__global__ __launch_bounds__(256) void k_quantize_main(const void* __restrict__ x, int64_t n,
                                                       const int64_t* __restrict__ rows, int64_t n_rows,
                                                       uint8_t* __restrict__ cache) {
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // Every lane of a group runs the DPP steps; a grid tail of whole groups
  // (n * 128 is a multiple of 64) never splits a wave's active quads.
  if (t >= n * 128) return;
  v4f v = load4<BF16>(x, t);
  unsigned m = max(max(mag_bits(v.x), mag_bits(v.y)), max(mag_bits(v.z), mag_bits(v.w)));
  float a = __uint_as_float(quad_umax(m));
  unsigned sc = e4m3_scale_code(a);
  unsigned codes = 0;
  if (sc != 0u) {
    Thresholds th = make_thresholds(e4m3_pos_value(sc));
    codes = e2m1_code(v.x, th) | e2m1_code(v.y, th) << 4 | e2m1_code(v.z, th) << 8 | e2m1_code(v.w, th) << 12;
  }
  int64_t e = t >> 7;
  int q = (int)(t & 127);
  int64_t r = dst_row(rows, e, n_rows);
  if (r < 0) return;
  uint8_t* ent = cache + r * kMainBytes;
  *(uint16_t*)(ent + 2 * q) = (uint16_t)codes;
  if ((q & 3) == 0) ent[256 + (q >> 2)] = (uint8_t)sc;
}

// Indexer keys: thread t covers channels 4q..4q+3 of key t/32 (q = t%32).
template <bool BF16>
__global__ __launch_bounds__(256) void k_quantize_index(const void* __restrict__ x, int64_t n,
                                                        const int64_t* __restrict__ rows, int64_t n_rows,
                                                        uint8_t* __restrict__ codes_out,
                                                        uint8_t* __restrict__ scales_out) {
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n * 32) return;  // n * 32 is a multiple of 8: groups stay whole
  v4f v = load4<BF16>(x, t);
  unsigned m = max(max(mag_bits(v.x), mag_bits(v.y)), max(mag_bits(v.z), mag_bits(v.w)));
  float a = __uint_as_float(oct_umax(m));
  int ex = e8m0_scale_exp(a);
  unsigned codes = 0;
  if (a != 0.0f) {
    // Compare |x| * 2^-e (exact: the result is <= 6 or the block saturates)
    // with the unit-scale thresholds.
    Thresholds th = make_thresholds(1.0f);
    codes = e2m1_code(__builtin_amdgcn_ldexpf(v.x, -ex), th) | e2m1_code(__builtin_amdgcn_ldexpf(v.y, -ex), th) << 4 |
            e2m1_code(__builtin_amdgcn_ldexpf(v.z, -ex), th) << 8 |
            e2m1_code(__builtin_amdgcn_ldexpf(v.w, -ex), th) << 12;
  }
  int64_t e = t >> 5;
  int q = (int)(t & 31);
  int64_t r = dst_row(rows, e, n_rows);
  if (r < 0) return;
  *(uint16_t*)(codes_out + r * 64 + 2 * q) = (uint16_t)codes;
  if ((q & 7) == 0) scales_out[r * 4 + (q >> 3)] = (uint8_t)(ex + 127);
}

}  // namespace

hipError_t launch_quantize(int kind, const void* x, int in_bf16, int64_t n, const int64_t* rows, int64_t n_rows,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t threads = n * (kind == 0 ? 128 : 32);
  dim3 grid((unsigned)((threads + 255) / 256));
  if (kind == 0) {
    if (in_bf16)
      k_quantize_main<true><<<grid, 256, 0, s>>>(x, n, rows, n_rows, codes);
    else
      k_quantize_main<false><<<grid, 256, 0, s>>>(x, n, rows, n_rows, codes);
  } else {
    if (in_bf16)
      k_quantize_index<true><<<grid, 256, 0, s>>>(x, n, rows, n_rows, codes, scales);
    else
      k_quantize_index<false><<<grid, 256, 0, s>>>(x, n, rows, n_rows, codes, scales);
  }
  return hipGetLastError();
}

}  // namespace csa2
