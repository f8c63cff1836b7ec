// csa2_dequant kernels: stored FP4 entries -> fp32 / bf16 values.
// Main latents: 512 E2M1 codes times an E4M3 scale per 16 channels; indexer
// keys: 128 E2M1 codes times an E8M0 scale per 32 channels ("An infra-oriented
// diagram of the DeepSeek-V4.1-Flash architecture", Full-layer cache bullet and
// "The KV cache"). Both products are exact in fp32 and in bf16.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

// One thread per (entry, 16-channel scale group): 8 code bytes + 1 scale byte in,
// 16 values out.
template <bool BF16>
__global__ __launch_bounds__(256) void k_dequant_main(const uint8_t* __restrict__ cache, int64_t n,
                                                      void* __restrict__ out) {
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n * 32) return;
  int64_t e = t >> 5;
  int g = (int)(t & 31);
  const uint8_t* ent = cache + e * kMainBytes;
  uint2 codes = *(const uint2*)(ent + g * 8);
  float s = e4m3_to_f32(ent[256 + g]);
  float v[16];
  decode_e2m1x8_scaled(codes.x, s, v);
  decode_e2m1x8_scaled(codes.y, s, v + 8);
  if (BF16) {
    v4u* o = (v4u*)((uint16_t*)out + e * kDim + g * 16);
    o[0] = pack_bf16x8(v);
    o[1] = pack_bf16x8(v + 8);
  } else {
    float4* o = (float4*)((float*)out + e * kDim + g * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

// One thread per (entry, 32-channel scale block): 16 code bytes + 1 scale byte.
template <bool BF16>
__global__ __launch_bounds__(256) void k_dequant_index(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales, int64_t n,
                                                       void* __restrict__ out) {
  int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n * 4) return;
  int64_t e = t >> 2;
  int b = (int)(t & 3);
  v4u c = *(const v4u*)(codes + e * 64 + b * 16);
  float s = e8m0_to_f32(scales[e * 4 + b]);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) decode_e2m1x8_scaled(c[i], s, v + 8 * i);
  if (BF16) {
    v4u* o = (v4u*)((uint16_t*)out + e * 128 + b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x8(v + 8 * i);
  } else {
    float4* o = (float4*)((float*)out + e * 128 + b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

hipError_t launch_dequant(int kind, const uint8_t* codes, const uint8_t* scales, int64_t n, int out_bf16, void* out,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (kind == 0) {
    int64_t threads = n * 32;
    dim3 grid((unsigned)((threads + 255) / 256));
    if (out_bf16)
      k_dequant_main<true><<<grid, 256, 0, s>>>(codes, n, out);
    else
      k_dequant_main<false><<<grid, 256, 0, s>>>(codes, n, out);
  } else {
    int64_t threads = n * 4;
    dim3 grid((unsigned)((threads + 255) / 256));
    if (out_bf16)
      k_dequant_index<true><<<grid, 256, 0, s>>>(codes, scales, n, out);
    else
      k_dequant_index<false><<<grid, 256, 0, s>>>(codes, scales, n, out);
  }
  return hipGetLastError();
}

}  // namespace csa2
