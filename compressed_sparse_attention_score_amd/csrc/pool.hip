// Reindex pool construction, the block half: the score of each block of 8
// entries, from the scores of a Full layer's indexer over its whole cache.
//
// The pages say that Reindex layers score only a 16,384-entry pool that layer
// 20 chose by blocks of 8 ("An infra-oriented diagram of the DeepSeek-V4.1-
// Flash architecture", indexer bullet), not how the blocks are ranked. Here a
// block scores the best of its entries inside the causal limit, in the same
// order as top-k (NaN below every number, -0 == +0); the best blocks are then
// chosen by the top-k selection itself, with block ids as entry ids.
//
// One thread per half block (4 consecutive scores, one 16-B load when the
// rows allow it, so a wave reads 1 KiB contiguously); the two halves of a
// block are neighbouring lanes and combine their best key with one DPP swap.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {
namespace {

template <bool VEC>
__global__ __launch_bounds__(256) void k_block_max(const float* __restrict__ scores, int64_t n,
                                                   const int32_t* __restrict__ n_valid, int64_t nb,
                                                   float* __restrict__ bmax, int32_t* __restrict__ nvb) {
  const int q = blockIdx.y;
  const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;  // half block: entries 4h..4h+3
  int64_t lim = n;
  if (n_valid) lim = min(lim, (int64_t)max(n_valid[q], 0));
  const float* row = scores + (int64_t)q * n;
  const int64_t e0 = 4 * h;
  float v[4];
  if (VEC) {  // n % 4 == 0 and the rows 16-B aligned: clamp to the last whole vector
    const v4f x = *(const v4f*)(row + min(e0, n - 4));
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = row[min(e0 + j, n - 1)];
  }
  unsigned k = 0u;  // 0: no valid entry
#pragma unroll
  for (int j = 0; j < 4; ++j) k = max(k, (e0 + j < lim) ? score_key(v[j]) : 0u);
  // every lane of the wave is active here (no early exit): lanes past the end
  // carry key 0 and store nothing
  k = max(k, (unsigned)__builtin_amdgcn_mov_dpp((int)k, 0xB1, 0xF, 0xF, false));  // lane ^ 1
  const int64_t b = h >> 1;
  if ((h & 1) == 0 && b < nb) bmax[(int64_t)q * nb + b] = key_score(k);
  if (h == 0) nvb[q] = (int32_t)((lim + 7) / 8);
}

}  // namespace

hipError_t launch_block_max(const float* scores, int Q, int64_t n, const int32_t* n_valid, float* bmax, int32_t* nvb,
                            hipStream_t s) {
  if (Q <= 0 || n <= 0) return hipSuccess;
  const int64_t nb = (n + 7) / 8;
  dim3 grid((unsigned)((2 * nb + 255) / 256), (unsigned)Q);
  const bool vec = (n % 4) == 0 && ((uintptr_t)scores % 16) == 0;
  if (vec)
    k_block_max<true><<<grid, 256, 0, s>>>(scores, n, n_valid, nb, bmax, nvb);
  else
    k_block_max<false><<<grid, 256, 0, s>>>(scores, n, n_valid, nb, bmax, nvb);
  return hipGetLastError();
}

}  // namespace csa2
