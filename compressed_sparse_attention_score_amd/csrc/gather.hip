// Dense copy of each query's selected main entries, for the Reuse layers:
// they share the global KV and the selected positions of an earlier layer
// ("DeepSeek V4.1 Flash: Why Its Encoder, Engram and KV Cache Matter", CSA2
// section), so the selection can be gathered once and every later layer's
// attention then reads contiguous rows instead of scattered ones.
//
// One thread per 16-B chunk of a destination slot (18 per 288-byte entry):
// consecutive threads write consecutive bytes, and the 18 threads of a slot
// read one contiguous source row.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {
namespace {

__global__ __launch_bounds__(256) void k_gather_selected(const uint8_t* __restrict__ cache, int64_t n_entries,
                                                         int64_t cache_q_stride, const int32_t* __restrict__ idx,
                                                         int64_t n_slots, int k, uint8_t* __restrict__ out,
                                                         int32_t* __restrict__ dense) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_slots * 18) return;
  const int64_t slot = t / 18;
  const int c = (int)(t - slot * 18);
  const int64_t q = slot / k;
  const int j = (int)(slot - q * k);
  const int32_t e = idx[slot];
  const bool ok = e >= 0 && (int64_t)e < n_entries;
  v4u v = {0u, 0u, 0u, 0u};
  if (ok) v = *(const v4u*)(cache + (q * cache_q_stride + e) * kMainBytes + 16 * c);
  *(v4u*)(out + slot * kMainBytes + 16 * c) = v;
  if (c == 0) dense[slot] = ok ? j : -1;
}

}  // namespace

hipError_t launch_gather_selected(const uint8_t* cache, int64_t n_entries, int64_t cache_q_stride, const int32_t* idx,
                                  int Q, int k, uint8_t* out, int32_t* dense, hipStream_t s) {
  const int64_t n_slots = (int64_t)Q * k;
  if (n_slots <= 0) return hipSuccess;
  k_gather_selected<<<dim3((unsigned)((n_slots * 18 + 255) / 256)), 256, 0, s>>>(cache, n_entries, cache_q_stride,
                                                                                 idx, n_slots, k, out, dense);
  return hipGetLastError();
}

}  // namespace csa2
