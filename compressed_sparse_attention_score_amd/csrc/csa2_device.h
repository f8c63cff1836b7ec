// Device-side helpers of the CSA2 HIP library (gfx950 only).
//
// Storage formats ("An infra-oriented diagram of the DeepSeek-V4.1-Flash
// architecture", Full-layer cache bullet and section "The KV cache"): FP4 E2M1
// codes, two per byte (even channel in the low nibble), with E4M3 scales per
// 16 channels (main latents) or E8M0 scales per 32 channels (indexer keys).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kMainBytes = 288;
constexpr int kIdxCodeBytes = 64;
constexpr int kIHeads = 32;
constexpr int kHeads = 64;
constexpr int kDim = 512;

// ---- element decode ---------------------------------------------------------

// E2M1 magnitude code (3 bits) -> fp32 value. The code placed at bit 22 is an
// fp32 with exponent field e and mantissa MSB m; scaling by 2^126 rebiases it
// to 2^(e-1) * (1 + m/2), and maps e == 0 (an fp32 subnormal) to m/2.
__device__ __forceinline__ float e2m1_to_f32(unsigned code) {
  unsigned bits = ((code & 7u) << 22) | ((code & 8u) << 28);
  return __uint_as_float(bits) * 0x1p126f;
}

// OCP E4M3FN byte -> fp32 (bias 7, subnormals 2^-6 * m/8, S.1111.111 = NaN).
__device__ __forceinline__ float e4m3_to_f32(unsigned b) {
  unsigned e = (b >> 3) & 15u, m = b & 7u;
  float mag;
  if (e == 0)
    mag = (float)m * 0x1p-9f;
  else
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15u && m == 7u) mag = __uint_as_float(0x7FC00000u);
  return (b & 0x80u) ? -mag : mag;
}

// The same decode by the gfx950 fp8 convert (OCP E4M3FN), one instruction.
// Equal to e4m3_to_f32 for every byte (NaN codes give a NaN).
__device__ __forceinline__ float e4m3_to_f32_hw(unsigned b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// E8M0 byte -> fp32 2^(b-127); b == 0 is the subnormal 2^-127, 0xFF is NaN.
__device__ __forceinline__ float e8m0_to_f32(unsigned b) {
  b &= 0xFFu;
  if (b == 0xFFu) return __uint_as_float(0x7FC00000u);
  if (b == 0u) return __uint_as_float(0x00400000u);
  return __uint_as_float(b << 23);
}

__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  // Round to nearest even; callers only pass values exact in bf16 or NaN.
  unsigned u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (unsigned short)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short h) { return __uint_as_float((unsigned)h << 16); }

// Eight E2M1 codes of one 32-bit word (byte j = channel 2j low nibble, 2j+1
// high nibble) times a scale s. The gfx950 convert takes its scale's exponent
// only, so it is given 1.0 and the (exact) product with s is a plain fp32
// multiply: E2M1 has 2 significant bits, E4M3 4, the product at most 6.
__device__ __forceinline__ void decode_e2m1x8_scaled(unsigned word, float s, float* v) {
  v2f f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
  v2f f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
  v2f f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
  v2f f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
  v[0] = f0[0] * s; v[1] = f0[1] * s;
  v[2] = f1[0] * s; v[3] = f1[1] * s;
  v[4] = f2[0] * s; v[5] = f2[1] * s;
  v[6] = f3[0] * s; v[7] = f3[1] * s;
}

// Pack two fp32 values that are exact in bf16 (or NaN) into bf16x2 by keeping
// their high halves: lo -> bits 15:0, hi -> bits 31:16.
__device__ __forceinline__ unsigned pack_bf16x2_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

__device__ __forceinline__ v4u pack_bf16x8(const float* v) {
  v4u r;
  r[0] = pack_bf16x2_exact(v[0], v[1]);
  r[1] = pack_bf16x2_exact(v[2], v[3]);
  r[2] = pack_bf16x2_exact(v[4], v[5]);
  r[3] = pack_bf16x2_exact(v[6], v[7]);
  return r;
}

// ---- ordered keys for selection ---------------------------------------------
// Larger key = larger score. -0 maps like +0; every NaN maps to 1 (below
// -inf, whose key is 0x007FFFFF); 0 is reserved for "not a candidate".
__device__ __forceinline__ unsigned score_key(float s) {
  unsigned u = __float_as_uint(s);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 1u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(unsigned k) {
  if (k <= 1u) return __uint_as_float(0x7FC00000u);
  unsigned u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// max(x, 0) on the bit pattern: every value with the sign bit set (-0
// included) becomes +0, the rest pass unchanged. Equal to fmaxf(x, 0) for
// every non-NaN x, in one integer max and without NaN canonicalisation.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ---- cross-lane helpers (wave64) -------------------------------------------
// Maximum over the 16 lanes of a row (lanes 16r..16r+15), left in every lane
// of the row: DPP row rotations by 8 and 4, then quad permutations.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false)));  // row_ror:8
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false)));  // row_ror:4
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)));   // [2,3,0,1]
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)));   // [1,0,3,2]
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave in six DPP adds, no LDS:
// row_shr 1, 2, 4, 8 scan each row of 16 lanes, then row_bcast:15 adds the
// last lane of rows 0 and 2 to rows 1 and 3, and row_bcast:31 the last lane
// of row 1 to rows 2 and 3. Every lane must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned dpp_add_u32(unsigned x) {
  return x + (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}

__device__ __forceinline__ unsigned wave_incl_scan(unsigned x) {
  x = dpp_add_u32<0x111, 0xF>(x);  // row_shr:1
  x = dpp_add_u32<0x112, 0xF>(x);  // row_shr:2
  x = dpp_add_u32<0x114, 0xF>(x);  // row_shr:4
  x = dpp_add_u32<0x118, 0xF>(x);  // row_shr:8
  x = dpp_add_u32<0x142, 0xA>(x);  // row_bcast:15 into rows 1, 3
  x = dpp_add_u32<0x143, 0xC>(x);  // row_bcast:31 into rows 2, 3
  return x;
}

// x + x[lane ^ 32] and x + x[lane ^ 16] with gfx950 lane swaps (no LDS).
__device__ __forceinline__ float add_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ unsigned umax_xor32(unsigned x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] > r[1] ? r[0] : r[1];
}
__device__ __forceinline__ unsigned umax_xor16(unsigned x) {
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return r[0] > r[1] ? r[0] : r[1];
}

// Unsigned maximum / minimum over the 64 lanes of a wave, left in every lane:
// quad permutations and row rotations by 4 and 8 (DPP), then the two lane
// swaps. No LDS traffic, unlike a shuffle.
__device__ __forceinline__ unsigned wave_umax(unsigned x) {
  x = max(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
  x = max(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
  x = max(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xF, 0xF, false));  // row_ror:4
  x = max(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false));  // row_ror:8
  return umax_xor32(umax_xor16(x));
}
__device__ __forceinline__ unsigned wave_umin(unsigned x) {
  x = min(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));
  x = min(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));
  x = min(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xF, 0xF, false));
  x = min(x, (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false));
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = r[0] < r[1] ? r[0] : r[1];
  auto t = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return t[0] < t[1] ? t[0] : t[1];
}

}  // namespace csa2
