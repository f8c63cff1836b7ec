// Top-k selection of indexer scores ("DeepSeek V4.1 Flash" guide, "A closer
// look": main sparse selection of 512 entries; "An infra-oriented diagram of
// the DeepSeek-V4.1-Flash architecture", indexer bullet: top-512).
//
// Order: score descending, entry id ascending (-0 == +0, NaN lowest). Each
// candidate is a 64-bit composite (order-preserving score key << 32 | ~id), so
// the exact top-k is simply the k largest composites, which are unique.
//
// Three steps, no host round trip and no full sort:
//  1. The scoring pass records the largest key of every sub-chunk of the
//     candidate list (>= 2k sub-chunks when the list is long enough).
//  2. theta = the k-th largest of those sub-chunk maxima is a lower bound on
//     the k-th largest score: k distinct sub-chunks each hold an element
//     >= theta. Every selection workgroup recomputes theta for its query,
//     then appends the composites of its chunk with key >= theta to a
//     per-query candidate list (typically ~k(1 + small) entries in all).
//  3. The last workgroup of each query (atomic ticket) radix-selects the k
//     largest composites of that list and bitonic-sorts them.
// With fewer than k non-empty sub-chunks theta falls back to "every valid
// candidate", so the result is exact for any input; degenerate inputs (huge
// tie sets) only make the list longer.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {
constexpr int NT = 256;
constexpr int kRadixBits = 11;
constexpr int kBins = 1 << kRadixBits;  // 2048
constexpr int kChunk = 4096;            // scores per selection workgroup
constexpr int kLdsCand = 4096;          // composites kept in LDS for the final select
constexpr int kSortMax = 1024;          // CSA2_MAX_K

struct SelShared {
  unsigned hist[kBins];
  unsigned red[8];
  unsigned res[4];
  unsigned long long buf[kLdsCand];
  unsigned long long sortbuf[kSortMax];
  unsigned n_buf;
  unsigned base;
  unsigned is_last;
};
}  // namespace

// k-th largest of the non-zero values src[0..n) (values may repeat), by MSB-first
// radix passes of 11 bits with an LDS histogram. Returns 0 when fewer than k
// non-zero values exist. If the bucket holding the k-th value is taken whole,
// the returned threshold T has that bucket's lower bits cleared: exactly the
// values >= T are then "the k largest" (or a superset when values repeat).
// All NT threads must call it.
template <typename T>
__device__ T radix_kth_largest(const T* src, int64_t n, unsigned k, SelShared& sh) {
  constexpr int W = (int)(sizeof(T) * 8);
  const int tid = threadIdx.x;
  T prefix = 0;
  unsigned remaining = k;
  int hi = W;  // bits >= hi are fixed in prefix
  while (hi > 0) {
    const int bits = (hi >= kRadixBits) ? kRadixBits : hi;
    const int shift = hi - bits;
    const unsigned mask = (1u << bits) - 1u;
    for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < n; i += NT) {
      T v = src[i];
      if (v == 0) continue;
      if (hi < W && (v >> hi) != (prefix >> hi)) continue;
      atomicAdd(&sh.hist[(unsigned)(v >> shift) & mask], 1u);
    }
    __syncthreads();
    // suffix sums: thread t owns bins [t*8, t*8+8)
    constexpr int PER = kBins / NT;
    unsigned local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) local += sh.hist[tid * PER + j];
    // inclusive suffix scan over threads (higher thread ids = larger digits)
    const int lane = tid & 63, wv = tid >> 6;
    unsigned x = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      unsigned y = (unsigned)__shfl_down((int)x, off, 64);
      if (lane + off < 64) x += y;
    }
    if (lane == 0) sh.red[wv] = x;
    __syncthreads();
    unsigned higher_waves = 0;
    for (int w2 = wv + 1; w2 < NT / 64; ++w2) higher_waves += sh.red[w2];
    const unsigned incl = x + higher_waves;  // sum over bins >= t*PER
    const unsigned above = incl - local;     // sum over bins >= (t+1)*PER
    if (tid == 0) {
      unsigned total = 0;
      for (int w2 = 0; w2 < NT / 64; ++w2) total += sh.red[w2];
      sh.res[3] = total;
    }
    if (above < remaining && remaining <= incl) {
      unsigned acc = above;
      for (int j = PER - 1; j >= 0; --j) {
        unsigned h = sh.hist[tid * PER + j];
        if (acc + h >= remaining) {
          sh.res[0] = (unsigned)(tid * PER + j);
          sh.res[1] = acc;
          sh.res[2] = h;
          break;
        }
        acc += h;
      }
    }
    __syncthreads();
    if (sh.res[3] < remaining) {  // fewer than k values in total (first pass only)
      __syncthreads();
      return (T)0;
    }
    const unsigned d = sh.res[0], acc = sh.res[1], h = sh.res[2];
    __syncthreads();
    prefix |= ((T)d) << shift;
    remaining -= acc;
    hi = shift;
    if (h == remaining) break;  // the whole bucket is taken
  }
  return prefix;
}

// Selection workgroup: grid (n_chunks, Q).
__global__ __launch_bounds__(NT) void k_select(const float* __restrict__ scores, int Q, int64_t n_cand,
                                               int64_t n_entries, const int32_t* __restrict__ cand_blocks,
                                               int n_blocks, const int32_t* __restrict__ n_valid, int k, int chunk,
                                               int n_chunks, const unsigned* __restrict__ gmax, int64_t n_groups,
                                               unsigned* __restrict__ ctrl, unsigned long long* __restrict__ cand,
                                               int32_t* __restrict__ idx, float* __restrict__ top_scores) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  SelShared& sh = *reinterpret_cast<SelShared*>(smem);
  const int q = blockIdx.y, tid = threadIdx.x;
  unsigned* qcount = ctrl;
  unsigned* ticket = ctrl + Q;
  int64_t limit = n_entries;
  if (n_valid) limit = min(limit, (int64_t)n_valid[q]);

  // ---- 1. theta from the sub-chunk maxima
  unsigned theta = 1u;
  if (n_groups >= k) theta = radix_kth_largest<unsigned>(gmax + (int64_t)q * n_groups, n_groups, (unsigned)k, sh);
  if (theta < 1u) theta = 1u;

  // ---- 2. compact this chunk's candidates with key >= theta
  if (tid == 0) sh.n_buf = 0u;
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * chunk, c1 = min(c0 + chunk, n_cand);
  const float* srow = scores + (int64_t)q * n_cand;
  for (int64_t p = c0 + tid; p < c1; p += NT) {
    int64_t e = p;
    if (cand_blocks) {
      int32_t b = cand_blocks[(int64_t)q * n_blocks + (p >> 3)];
      e = (b < 0) ? -1 : 8 * (int64_t)b + (p & 7);
    }
    if (e < 0 || e >= limit) continue;
    unsigned key = score_key(srow[p]);
    if (key >= theta) {
      unsigned pos = atomicAdd(&sh.n_buf, 1u);
      sh.buf[pos] = ((unsigned long long)key << 32) | (unsigned long long)(~(unsigned)e);
    }
  }
  __syncthreads();
  const unsigned nb = sh.n_buf;
  if (tid == 0) sh.base = nb ? atomicAdd(&qcount[q], nb) : 0u;
  __syncthreads();
  unsigned long long* qc = cand + (int64_t)q * n_cand;
  for (unsigned i = tid; i < nb; i += NT) qc[sh.base + i] = sh.buf[i];
  __threadfence();
  __syncthreads();
  if (tid == 0) sh.is_last = (atomicAdd(&ticket[q], 1u) == (unsigned)(n_chunks - 1)) ? 1u : 0u;
  __syncthreads();
  if (!sh.is_last) return;

  // ---- 3. last workgroup of query q: exact top-k of the candidate list
  __threadfence();
  const unsigned m = atomicAdd(&qcount[q], 0u);
  const unsigned long long* src = qc;
  if (m <= (unsigned)kLdsCand) {
    for (unsigned i = tid; i < m; i += NT) sh.buf[i] = qc[i];
    __syncthreads();
    src = sh.buf;
  }
  unsigned long long T = 0ull;
  if (m > (unsigned)k) T = radix_kth_largest<unsigned long long>(src, m, (unsigned)k, sh);
  if (tid == 0) sh.n_buf = 0u;
  __syncthreads();
  for (unsigned i = tid; i < m; i += NT) {
    unsigned long long v = src[i];
    if (v >= T) {
      unsigned pos = atomicAdd(&sh.n_buf, 1u);
      if (pos < (unsigned)kSortMax) sh.sortbuf[pos] = v;
    }
  }
  __syncthreads();
  const unsigned cnt = min(sh.n_buf, (unsigned)k);
  int P = 1;
  while (P < (int)cnt) P <<= 1;
  for (int i = tid; i < P; i += NT)
    if (i >= (int)cnt) sh.sortbuf[i] = 0ull;
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += NT) {
        int i = 2 * t - (t & (stride - 1));
        int j = i + stride;
        bool desc = ((i & size) == 0);
        unsigned long long x = sh.sortbuf[i], y = sh.sortbuf[j];
        if ((x < y) == desc) {
          sh.sortbuf[i] = y;
          sh.sortbuf[j] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < k; j += NT) {
    int32_t id = -1;
    float sc = -__builtin_inff();
    if (j < (int)cnt) {
      unsigned long long v = sh.sortbuf[j];
      id = (int32_t)(~(unsigned)(v & 0xFFFFFFFFull));
      sc = key_score((unsigned)(v >> 32));
    }
    idx[(int64_t)q * k + j] = id;
    if (top_scores) top_scores[(int64_t)q * k + j] = sc;
  }
}

SelectPlan plan_select(int64_t n_cand) {
  SelectPlan p;
  p.chunk = kChunk;
  p.n_chunks = (int)((n_cand + kChunk - 1) / kChunk);
  if (p.n_chunks < 1) p.n_chunks = 1;
  return p;
}

hipError_t launch_select(const float* scores, int Q, int64_t n_cand, int64_t n_entries, const int32_t* cand_blocks,
                         int n_blocks, const int32_t* n_valid, int k, const ScorePlan& sp, const unsigned* gmax,
                         unsigned* ctrl, unsigned long long* cand, int32_t* idx, float* top_scores, hipStream_t s) {
  if (Q <= 0) return hipSuccess;
  SelectPlan pl = plan_select(n_cand);
  dim3 grid((unsigned)pl.n_chunks, (unsigned)Q);
  k_select<<<grid, NT, sizeof(SelShared), s>>>(scores, Q, n_cand, n_entries, cand_blocks, n_blocks, n_valid, k,
                                               pl.chunk, pl.n_chunks, gmax, sp.n_groups, ctrl, cand, idx, top_scores);
  return hipGetLastError();
}

__global__ void k_zero_u32(unsigned* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_u32(unsigned* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_zero_u32<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace csa2
