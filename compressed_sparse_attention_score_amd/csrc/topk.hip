// Top-k selection of indexer scores ("DeepSeek V4.1 Flash" guide, "A closer
// look": main sparse selection of 512 entries; "An infra-oriented diagram of
// the DeepSeek-V4.1-Flash architecture", indexer bullet: top-512).
//
// Ranking: score descending, entry id ascending (-0 == +0, NaN lowest). Each
// candidate is a 64-bit composite (order-preserving score key << 32 | ~id),
// so the exact top-k is the set of the k largest composites, which are
// unique. The set is returned in ascending entry id.
//
// No sort is needed:
//  1. The scoring pass records the largest key of every sub-chunk of the
//     candidate list (>= 2k sub-chunks when the list is long enough).
//  2. The k-th largest of those sub-chunk maxima is a lower bound on the
//     k-th largest score: k distinct sub-chunks each hold an element >= it.
//     theta is that key with its low 16 bits cleared (a lower bound still,
//     found by two radix passes). Each compaction workgroup finds theta and
//     writes its chunk's composites with key >= theta, in position order
//     (block prefix sum), to a fixed region of the candidate list.
//  3. One workgroup per query gathers the regions in chunk order, finds the
//     k-th largest composite T by radix select and writes every candidate
//     >= T in list order, which is ascending entry id.
// With fewer than k non-empty sub-chunks theta falls back to "every valid
// candidate", so the result is exact for any input; heavy ties only make the
// candidate list longer. Steps 2 and 3 are separate kernels: handing the list
// over at a kernel boundary is cheaper on this multi-XCD part than an
// in-kernel hand-off between workgroups.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {
constexpr int NT = 256;
constexpr int kChunk = 4096;  // scores per compaction workgroup (16 per thread)
constexpr int kPer = kChunk / NT;
constexpr int kRegCand = 16;  // candidates per thread held in registers by the final pass
constexpr int kRadixBits = 8;
constexpr int kBins = 1 << kRadixBits;

// Score staging of the compaction: thread t's 16 scores at 20t (4 pad
// floats per 16 keep its 16-B reads on distinct banks).
constexpr int kStageStride = kPer + 4;

struct SelShared {
  alignas(16) unsigned hist[2][kBins];
  alignas(16) unsigned wsum[NT / 64];
  unsigned res[4];
  unsigned off[NT + 1];  // exclusive offsets of the chunk regions in the joined list
  alignas(16) float stage[NT * kStageStride];
};
}  // namespace

// Inclusive prefix sum of x over the workgroup (thread order); *total gets the
// sum of all. Uses wsum (NT/64 entries, 16-B aligned); contains barriers.
__device__ __forceinline__ unsigned block_incl_scan(unsigned x, unsigned* wsum, unsigned* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  x = wave_incl_scan(x);
  __syncthreads();
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  const v4u s = *(const v4u*)wsum;  // NT / 64 == 4
  unsigned before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    before += (w < wv) ? s[w] : 0u;
    all += s[w];
  }
  *total = all;
  return x + before;
}


// Digit pick of one radix pass, run by wave 0 alone. Lane l holds bins
// 255-4l .. 252-4l (the digits from the top); a wave prefix sum over the lanes
// counts the values in the bins above each lane's, and the lane whose four
// bins hold the `remaining`-th largest value walks them. res gets the digit,
// the count in the bins above it, the count in its bin, and the histogram's
// total (lane 63's inclusive sum).
__device__ __forceinline__ void pick_digit_wave0(const unsigned* hist, unsigned remaining, unsigned* res) {
  const int lane = threadIdx.x & 63;
  const v4u h = *(const v4u*)(hist + (kBins - 4) - 4 * lane);  // bins 252-4l .. 255-4l
  const unsigned s = h[0] + h[1] + h[2] + h[3];
  const unsigned incl = wave_incl_scan(s);  // values in bins >= 252 - 4l
  unsigned above = incl - s;                // values in bins > 255 - 4l
  if (above < remaining && remaining <= incl) {
#pragma unroll
    for (int r = 3; r >= 0; --r) {
      if (above < remaining && remaining <= above + h[r]) {
        res[0] = (unsigned)(kBins - 4 - 4 * lane + r);
        res[1] = above;
        res[2] = h[r];
      }
      above += h[r];
    }
  }
  if (lane == 63) res[3] = incl;
}

// k-th largest of a multiset of non-zero values (zeros are ignored), by
// MSB-first radix passes of 8 bits over an LDS histogram, NTH threads. count(h,
// hi, shift, prefix) adds to h every value whose bits above `hi` equal those of
// prefix, binned by bits shift..shift+7 (all values when hi is the width).
// Two histograms alternate: the one a pass fills was cleared during the pass
// before, so a pass costs two barriers (histogram complete; digit picked).
// Returns 0 when fewer than k non-zero values exist. When the bucket holding
// the k-th value is taken whole, or after max_passes passes, the remaining low
// bits are left at zero: the result is then a lower bound on the k-th value
// and the values >= it are a superset of the k largest (exactly them when the
// bucket was taken whole and no value repeats).
template <int NTH, typename T, typename Count>
__device__ __forceinline__ T radix_kth(Count count, unsigned k, unsigned (*hist)[kBins], unsigned* res, int max_passes) {
  constexpr int W = (int)(sizeof(T) * 8);
  for (int i = threadIdx.x; i < 2 * kBins; i += NTH) hist[i / kBins][i % kBins] = 0u;
  __syncthreads();
  T prefix = 0;
  unsigned remaining = k;
  int b = 0, pass = 0;
  for (int hi = W; hi > 0 && pass < max_passes; hi -= kRadixBits, ++pass, b ^= 1) {
    const int shift = hi - kRadixBits;
    count(hist[b], hi, shift, prefix);
    // the other histogram was last read before the previous pass's second
    // barrier, and the next pass fills it after this pass's second barrier
    if (pass > 0)
      for (int i = threadIdx.x; i < kBins; i += NTH) hist[b ^ 1][i] = 0u;
    __syncthreads();
    if (threadIdx.x < 64) pick_digit_wave0(hist[b], remaining, res);
    __syncthreads();
    const unsigned d = res[0], above = res[1], cnt = res[2], total = res[3];
    if (total < remaining) return (T)0;
    prefix |= ((T)d) << shift;
    remaining -= above;
    if (cnt == remaining) break;
  }
  return prefix;
}

// The same over PER values per thread held in registers.
template <int NTH, typename T, int PER>
__device__ __forceinline__ T radix_kth_regs(const T (&v)[PER], unsigned k, unsigned (*hist)[kBins], unsigned* res,
                            int max_passes = 64) {
  constexpr int W = (int)(sizeof(T) * 8);
  auto count = [&](unsigned* h, int hi, int shift, T prefix) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const T x = v[j];
      if (x == 0) continue;
      if (hi < W && (x >> hi) != (prefix >> hi)) continue;
      atomicAdd(&h[(unsigned)(x >> shift) & (kBins - 1)], 1u);
    }
  };
  return radix_kth<NTH, T>(count, k, hist, res, max_passes);
}

// The same over n values streamed from memory (lists too long for registers).
template <int NTH, typename T>
__device__ __forceinline__ T radix_kth_stream(const T* src, int64_t n, unsigned k, unsigned (*hist)[kBins], unsigned* res,
                              int max_passes = 64) {
  constexpr int W = (int)(sizeof(T) * 8);
  auto count = [&](unsigned* h, int hi, int shift, T prefix) {
    for (int64_t i = threadIdx.x; i < n; i += NTH) {
      const T x = src[i];
      if (x == 0) continue;
      if (hi < W && (x >> hi) != (prefix >> hi)) continue;
      atomicAdd(&h[(unsigned)(x >> shift) & (kBins - 1)], 1u);
    }
  };
  return radix_kth<NTH, T>(count, k, hist, res, max_passes);
}

// theta needs only to be a lower bound on the k-th largest score: two passes
// fix the sign, exponent and top 7 mantissa bits of the k-th sub-chunk
// maximum, which lowers the bound by less than 2^-7 of its value and adds a
// few percent of survivors, and saves the passes over the low 16 bits.
constexpr int kThetaPasses = 2;

// Threshold + compaction: grid (n_chunks, Q). Writes cand[q][c0 .. c0+cnt) in
// position order and counts[q][chunk] = cnt.
__global__ __launch_bounds__(NT) void k_select_compact(const float* __restrict__ scores, int64_t n_cand,
                                                       int64_t n_entries, const int32_t* __restrict__ cand_blocks,
                                                       int n_blocks, const int32_t* __restrict__ n_valid, int k,
                                                       const unsigned* __restrict__ gmax, int64_t n_groups,
                                                       int n_chunks, unsigned* __restrict__ counts,
                                                       unsigned long long* __restrict__ cand) {
  __shared__ SelShared sh;
  const int q = blockIdx.y, tid = threadIdx.x;
  int64_t limit = n_entries;
  if (n_valid) limit = min(limit, (int64_t)n_valid[q]);

  // this thread's 16 consecutive positions. The chunk's scores are read with
  // coalesced 16-B loads (lane l takes vector l of each 4-KiB slice; a list
  // whose rows are not 16-B aligned takes 4-B loads in the same order) and
  // staged in LDS before the threshold work; the thread picks its 16 up after
  // it, whose barriers order the stores before the reads.
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  const int64_t p0 = c0 + (int64_t)tid * kPer;
  const float* srow = scores + (int64_t)q * n_cand;
  {
    const bool vec = ((uintptr_t)srow & 15) == 0;  // rows 16-B aligned (base and length)
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const int v = i * NT + tid;  // float4 index inside the chunk
      const int64_t f0 = c0 + 4 * (int64_t)v;
      v4f x;
      if (vec && f0 + 4 <= n_cand) {
        x = *(const v4f*)(srow + f0);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = srow[min(f0 + u, n_cand - 1)];
      }
      *(v4f*)(sh.stage + (v >> 2) * kStageStride + 4 * (v & 3)) = x;
    }
  }
  float sc[kPer];
  int64_t ent[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = p0 + j;
    int64_t e = p;
    if (cand_blocks) {
      const int32_t b = (p < n_cand) ? cand_blocks[(int64_t)q * n_blocks + (p >> 3)] : -1;
      e = (b < 0) ? -1 : 8 * (int64_t)b + (p & 7);
    }
    ent[j] = (p < n_cand && e >= 0 && e < limit) ? e : -1;
  }

  // ---- theta = k-th largest sub-chunk maximum
  unsigned theta = 1u;
  if (n_groups >= k) {
    const unsigned* gq = gmax + (int64_t)q * n_groups;
    unsigned t;
    if (n_groups <= (int64_t)NT * 16) {
      unsigned g[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t i = (int64_t)j * NT + tid;
        g[j] = (i < n_groups) ? gq[i] : 0u;
      }
      t = radix_kth_regs<NT, unsigned, 16>(g, (unsigned)k, sh.hist, sh.res, kThetaPasses);
    } else {
      t = radix_kth_stream<NT, unsigned>(gq, n_groups, (unsigned)k, sh.hist, sh.res, kThetaPasses);
    }
    theta = t > 1u ? t : 1u;
  }

  if (n_groups < k) __syncthreads();  // no threshold pass ran: order the staging
#pragma unroll
  for (int i = 0; i < kPer / 4; ++i) {
    const v4f x = *(const v4f*)(sh.stage + tid * kStageStride + 4 * i);
    sc[4 * i] = x[0]; sc[4 * i + 1] = x[1]; sc[4 * i + 2] = x[2]; sc[4 * i + 3] = x[3];
  }

  // ---- keep key >= theta, in position order
  unsigned long long comp[kPer];
  unsigned cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const unsigned key = score_key(sc[j]);
    const bool keep = ent[j] >= 0 && key >= theta;
    comp[j] = keep ? (((unsigned long long)key << 32) | (unsigned long long)(~(unsigned)ent[j])) : 0ull;
    cnt += keep ? 1u : 0u;
  }
  unsigned total;
  const unsigned incl = block_incl_scan(cnt, sh.wsum, &total);
  unsigned pos = incl - cnt;
  unsigned long long* dst = cand + (int64_t)q * n_cand + c0;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (comp[j]) dst[pos++] = comp[j];
  if (tid == 0) counts[(int64_t)q * n_chunks + blockIdx.x] = total;
}

// Exact top-k of the non-zero composites held kRegCand per thread, thread
// order being list order: the k-th largest T (when there are more than k),
// then every composite >= T written in list order. Returns the count written.
__device__ __forceinline__ unsigned select_write(const unsigned long long (&v)[kRegCand], unsigned m, int k,
                                                 SelShared& sh, int32_t* iq, float* tq) {
  const unsigned long long T =
      (m > (unsigned)k) ? radix_kth_regs<NT, unsigned long long, kRegCand>(v, (unsigned)k, sh.hist, sh.res) : 0ull;
  unsigned c = 0;
#pragma unroll
  for (int j = 0; j < kRegCand; ++j) c += (v[j] != 0ull && v[j] >= T) ? 1u : 0u;
  unsigned all;
  unsigned pos = block_incl_scan(c, sh.wsum, &all) - c;
#pragma unroll
  for (int j = 0; j < kRegCand; ++j) {
    if (v[j] != 0ull && v[j] >= T && pos < (unsigned)k) {
      iq[pos] = (int32_t)(~(unsigned)(v[j] & 0xFFFFFFFFull));
      if (tq) tq[pos] = key_score((unsigned)(v[j] >> 32));
      ++pos;
    }
  }
  return min(all, (unsigned)k);
}

// Exact top-k of each query's candidate list: grid (Q). Output in list order.
__global__ __launch_bounds__(NT) void k_select_final(const unsigned* __restrict__ counts, int n_chunks,
                                                     int64_t n_cand, int k, const unsigned long long* __restrict__ cand,
                                                     int32_t* __restrict__ idx, float* __restrict__ top_scores) {
  __shared__ SelShared sh;
  const int q = blockIdx.x, tid = threadIdx.x;
  const unsigned* cq = counts + (int64_t)q * n_chunks;
  const unsigned long long* lq = cand + (int64_t)q * n_cand;
  int32_t* iq = idx + (int64_t)q * k;
  float* tq = top_scores ? top_scores + (int64_t)q * k : nullptr;

  unsigned written = 0;
  bool done = false;
  unsigned m = 0, cnt_c = 0, incl_c = 0;
  if (n_chunks <= NT && n_cand > 0) {
    // Chunk c's region starts at c*kChunk whatever the counts, so each thread
    // loads kRegCand fixed slots of one chunk (threads c*tpc .. c*tpc+tpc-1
    // take chunk c in order, so thread order is list order) together with
    // the counts, and masks the slots past its chunk's count afterwards.
    // When some chunk holds more survivors than its threads' slots, the
    // offset-table pass below runs instead.
    const int tpc = NT / n_chunks;
    const int c_t = tid / tpc, sub = tid - c_t * tpc;
    const bool own = c_t < n_chunks;
    const unsigned slot0 = (unsigned)sub * kRegCand;
    cnt_c = (tid < n_chunks) ? cq[tid] : 0u;
    const unsigned my_cnt = own ? cq[c_t] : 0u;
    const int64_t rb = (own ? (int64_t)c_t * kChunk : 0) + slot0;
    unsigned long long v[kRegCand];
#pragma unroll
    for (int j = 0; j < kRegCand; ++j) v[j] = lq[min(rb + j, n_cand - 1)];  // slots past the list: dropped below
    incl_c = block_incl_scan(cnt_c, sh.wsum, &m);
    const bool fits = __syncthreads_and(!own || my_cnt <= (unsigned)tpc * kRegCand) != 0;
    if (fits) {
#pragma unroll
      for (int j = 0; j < kRegCand; ++j) v[j] = (own && slot0 + j < my_cnt) ? v[j] : 0ull;
      written = select_write(v, m, k, sh, iq, tq);
      done = true;
    }
  } else {
    for (int c0 = 0; c0 < n_chunks; c0 += NT) {
      const unsigned x = (c0 + tid < n_chunks) ? cq[c0 + tid] : 0u;
      unsigned tot;
      const unsigned incl = block_incl_scan(x, sh.wsum, &tot);
      if (c0 == 0) {
        cnt_c = x;
        incl_c = incl;
      }
      m += tot;
    }
  }
  if (done) {
  } else if (m <= (unsigned)(NT * kRegCand) && n_chunks <= NT) {
    // The joined list is the chunk regions in chunk order; thread t takes its
    // elements t*kRegCand .. +kRegCand-1, locating their chunk through the
    // offset table (one binary search, then a forward walk).
    if (tid < n_chunks) sh.off[tid] = incl_c - cnt_c;
    if (tid == 0) sh.off[n_chunks] = m;
    __syncthreads();
    const unsigned e0 = (unsigned)tid * kRegCand;
    int ch = 0;
    if (e0 < m) {
      int lo = 0, hi = n_chunks - 1;  // largest c with off[c] <= e0
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sh.off[mid] <= e0) lo = mid; else hi = mid - 1;
      }
      ch = lo;
    }
    // addresses first (the walk reads LDS only), then every load at once: a
    // load inside the walk would wait for the previous one each time
    int64_t at[kRegCand];
#pragma unroll
    for (int j = 0; j < kRegCand; ++j) {
      const unsigned e = e0 + j;
      at[j] = 0;
      if (e < m) {
        while (e >= sh.off[ch + 1]) ++ch;  // e < m = off[n_chunks] bounds the walk
        at[j] = (int64_t)ch * kChunk + (e - sh.off[ch]);
      }
    }
    unsigned long long v[kRegCand];
#pragma unroll
    for (int j = 0; j < kRegCand; ++j) {
      const unsigned long long x = lq[at[j]];  // at[j] = 0 past the end: a valid slot, dropped
      v[j] = (e0 + j < m) ? x : 0ull;
    }
    written = select_write(v, m, k, sh, iq, tq);
  } else {
    // long lists (heavy ties or huge candidate sets): stream the chunk regions
    unsigned long long T = 0ull;
    if (m > (unsigned)k) {
      auto count = [&](unsigned* h, int hi, int shift, unsigned long long prefix) {
        for (int c = 0; c < n_chunks; ++c) {
          const unsigned n_c = cq[c];
          for (unsigned i = tid; i < n_c; i += NT) {
            const unsigned long long x = lq[(int64_t)c * kChunk + i];
            if (hi < 64 && (x >> hi) != (prefix >> hi)) continue;
            atomicAdd(&h[(unsigned)(x >> shift) & (kBins - 1)], 1u);
          }
        }
      };
      T = radix_kth<NT, unsigned long long>(count, (unsigned)k, sh.hist, sh.res, 64);
    }
    // ordered write: chunk by chunk, NT elements at a time
    for (int c = 0; c < n_chunks; ++c) {
      const unsigned n_c = cq[c];
      for (unsigned i0 = 0; i0 < n_c; i0 += NT) {
        const unsigned i = i0 + tid;
        const unsigned long long x = (i < n_c) ? lq[(int64_t)c * kChunk + i] : 0ull;
        const unsigned sel = (x != 0ull && x >= T) ? 1u : 0u;
        unsigned tot;
        const unsigned pos = written + block_incl_scan(sel, sh.wsum, &tot) - sel;
        if (sel && pos < (unsigned)k) {
          iq[pos] = (int32_t)(~(unsigned)(x & 0xFFFFFFFFull));
          if (tq) tq[pos] = key_score((unsigned)(x >> 32));
        }
        written += tot;
      }
    }
    written = min(written, (unsigned)k);
  }
  for (int j = (int)written + tid; j < k; j += NT) {
    iq[j] = -1;
    if (tq) tq[j] = -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// One workgroup per query (lists up to kQMaxCand candidates). Same method as
// the two kernels above, in one launch: theta from the sub-chunk maxima,
// compaction of the candidates >= theta in position order (ascending entry
// id: pools list their blocks in ascending order), then the exact k-th
// composite among the survivors and the ordered write.
namespace {
constexpr int NQ = 1024;            // threads
constexpr int kQPer = 16;           // consecutive positions per thread per pass
constexpr int kQCap = 8192;         // survivors held in LDS (8 per thread)
constexpr int64_t kQMaxCand = 1 << 18;

struct QSelShared {
  alignas(16) unsigned hist[2][kBins];
  alignas(16) unsigned wsum[NQ / 64];
  unsigned res[4];
  unsigned long long cand[kQCap + kQCap / 16];  // survivor i at q_slot(i)
};

// LDS slot of survivor i: one pad slot after every 16. A thread writes its
// survivors as a run, and with everything kept the runs of neighbouring
// lanes start 16 composites (128 bytes) apart, i.e. in the same banks; the
// pad shifts each run by one composite so a store spreads over the banks.
__device__ __forceinline__ unsigned q_slot(unsigned i) { return i + (i >> 4); }

// Inclusive prefix sum over the NQ threads; *total = sum of all. Barriers inside.
__device__ __forceinline__ unsigned q_scan(unsigned x, QSelShared& sh, unsigned* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  x = wave_incl_scan(x);
  __syncthreads();
  if (lane == 63) sh.wsum[wv] = x;
  __syncthreads();
  const v4u* w4 = (const v4u*)sh.wsum;
  unsigned before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NQ / 256; ++i) {
    const v4u v = w4[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      before += (4 * i + j < wv) ? v[j] : 0u;
      all += v[j];
    }
  }
  *total = all;
  return x + before;
}

}  // namespace

__global__ __launch_bounds__(NQ) void k_select_query(const float* __restrict__ scores, int64_t n_cand,
                                                     int64_t n_entries, const int32_t* __restrict__ cand_blocks,
                                                     int n_blocks, const int32_t* __restrict__ n_valid, int k,
                                                     const unsigned* __restrict__ gmax, int64_t n_groups,
                                                     unsigned long long* __restrict__ gcand, int32_t* __restrict__ idx,
                                                     float* __restrict__ top_scores) {
  __shared__ QSelShared sh;
  const int q = blockIdx.x, tid = threadIdx.x;
  int64_t limit = n_entries;
  if (n_valid) limit = min(limit, (int64_t)n_valid[q]);
  int32_t* iq = idx + (int64_t)q * k;
  float* tq = top_scores ? top_scores + (int64_t)q * k : nullptr;
  const float* srow = scores + (int64_t)q * n_cand;
  unsigned long long* gq = gcand + (int64_t)q * n_cand;

  // Positions are taken in passes of NQ*kQPer; thread t owns positions
  // 16t..16t+15 of each pass. Full passes (rows 16-byte aligned) load with
  // aligned vectors and no per-thread conditions, the next pass's scores
  // in flight while this one is compacted; a ragged last pass is guarded.
  constexpr int64_t kStep = (int64_t)NQ * kQPer;
  const int64_t n_full = ((n_cand & 3) == 0) ? n_cand / kStep : 0;
  auto load_full = [&](float* sc, int32_t* blk, int64_t p0) {
    const int64_t pb = p0 + (int64_t)tid * kQPer;
#pragma unroll
    for (int j = 0; j < kQPer; j += 4) {
      const v4f v = *(const v4f*)(srow + pb + j);
      sc[j] = v[0]; sc[j + 1] = v[1]; sc[j + 2] = v[2]; sc[j + 3] = v[3];
    }
#pragma unroll
    for (int j = 0; j < kQPer / 8; ++j) blk[j] = cand_blocks ? cand_blocks[(int64_t)q * n_blocks + ((pb >> 3) + j)] : 0;
  };
  float scA[kQPer], scB[kQPer];
  int32_t bkA[kQPer / 8], bkB[kQPer / 8];
  if (n_full > 0) load_full(scA, bkA, 0);  // in flight during the threshold search

  // ---- theta = k-th largest sub-chunk maximum (1 = keep every valid candidate)
  unsigned theta = 1u;
  if (gmax && n_groups >= k) {
    const unsigned* gm = gmax + (int64_t)q * n_groups;
    unsigned t;
    if (n_groups <= 4 * NQ) {
      unsigned g[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t i = (int64_t)j * NQ + tid;
        g[j] = (i < n_groups) ? gm[i] : 0u;
      }
      t = radix_kth_regs<NQ, unsigned, 4>(g, (unsigned)k, sh.hist, sh.res, kThetaPasses);
    } else {
      t = radix_kth_stream<NQ, unsigned>(gm, n_groups, (unsigned)k, sh.hist, sh.res, kThetaPasses);
    }
    theta = t > 1u ? t : 1u;
  }

  // ---- keep key >= theta, in position order
  unsigned m = 0;  // survivors so far (block-uniform)
  auto process = [&](const float* sc, const int32_t* blk, int64_t p0) {
    const int64_t pb = p0 + (int64_t)tid * kQPer;
    unsigned long long comp[kQPer];
    unsigned cnt = 0;
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      const int64_t p = pb + j;
      int64_t e = p;
      if (cand_blocks) e = (blk[j >> 3] < 0) ? -1 : 8 * (int64_t)blk[j >> 3] + (p & 7);
      const bool valid = p < n_cand && e >= 0 && e < limit;
      const unsigned key = score_key(sc[j]);
      const bool keep = valid && key >= theta;
      comp[j] = keep ? (((unsigned long long)key << 32) | (unsigned long long)(~(unsigned)e)) : 0ull;
      cnt += keep ? 1u : 0u;
    }
    unsigned total;
    unsigned pos = m + q_scan(cnt, sh, &total) - cnt;
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      if (comp[j]) {
        if (pos < (unsigned)kQCap) sh.cand[q_slot(pos)] = comp[j];
        else gq[pos] = comp[j];
        ++pos;
      }
    }
    m += total;
  };
  for (int64_t i = 0; i < n_full; i += 2) {
    if (i + 1 < n_full) load_full(scB, bkB, (i + 1) * kStep);
    process(scA, bkA, i * kStep);
    if (i + 1 >= n_full) break;
    if (i + 2 < n_full) load_full(scA, bkA, (i + 2) * kStep);
    process(scB, bkB, (i + 1) * kStep);
  }
  for (int64_t p0 = n_full * kStep; p0 < n_cand; p0 += kStep) {  // ragged or unaligned passes
    // positions past the end load the last score (clamped, so every load is
    // issued at once instead of one guarded round trip after another) and
    // are dropped by process()
    const int64_t pb = p0 + (int64_t)tid * kQPer;
#pragma unroll
    for (int j = 0; j < kQPer; ++j) scA[j] = srow[min(pb + j, n_cand - 1)];
#pragma unroll
    for (int j = 0; j < kQPer / 8; ++j)
      bkA[j] = cand_blocks ? cand_blocks[(int64_t)q * n_blocks + min((pb >> 3) + j, (int64_t)n_blocks - 1)] : 0;
    process(scA, bkA, p0);
  }
  __syncthreads();

  unsigned written = 0;
  if (m <= (unsigned)kQCap) {
    // ---- survivors in LDS: thread t holds list elements 8t..8t+7
    constexpr int PER = kQCap / NQ;
    unsigned long long v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const unsigned e = (unsigned)tid * PER + j;
      v[j] = (e < m) ? sh.cand[q_slot(e)] : 0ull;
    }
    const unsigned long long T = (m > (unsigned)k) ? radix_kth_regs<NQ, unsigned long long, PER>(v, (unsigned)k, sh.hist, sh.res) : 0ull;
    unsigned c = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) c += (v[j] != 0ull && v[j] >= T) ? 1u : 0u;
    unsigned all;
    unsigned pos = q_scan(c, sh, &all) - c;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (v[j] != 0ull && v[j] >= T && pos < (unsigned)k) {
        iq[pos] = (int32_t)(~(unsigned)(v[j] & 0xFFFFFFFFull));
        if (tq) tq[pos] = key_score((unsigned)(v[j] >> 32));
        ++pos;
      }
    }
    written = min(all, (unsigned)k);
  } else {
    // ---- long survivor lists (heavy ties): move the LDS part to global and
    // select from there
    for (int i = tid; i < kQCap; i += NQ) gq[i] = sh.cand[q_slot((unsigned)i)];
    __syncthreads();
    const unsigned long long T = radix_kth_stream<NQ, unsigned long long>(gq, m, (unsigned)k, sh.hist, sh.res);
    for (unsigned i0 = 0; i0 < m; i0 += NQ) {
      const unsigned i = i0 + tid;
      const unsigned long long x = (i < m) ? gq[i] : 0ull;
      const unsigned sel = (x != 0ull && x >= T) ? 1u : 0u;
      unsigned tot;
      const unsigned pos = written + q_scan(sel, sh, &tot) - sel;
      if (sel && pos < (unsigned)k) {
        iq[pos] = (int32_t)(~(unsigned)(x & 0xFFFFFFFFull));
        if (tq) tq[pos] = key_score((unsigned)(x >> 32));
      }
      written += tot;
    }
    written = min(written, (unsigned)k);
  }
  for (int j = (int)written + tid; j < k; j += NQ) {
    iq[j] = -1;
    if (tq) tq[j] = -__builtin_inff();
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
                         unsigned* counts, unsigned long long* cand, int32_t* idx, float* top_scores, hipStream_t s) {
  if (Q <= 0) return hipSuccess;
  // one workgroup per query when that fills the chip or the lists are short
  // (a single CU compacts ~20 vector ops per candidate)
  if (n_cand <= kQMaxCand && (Q >= 64 || n_cand <= 16384)) {
    k_select_query<<<(unsigned)Q, NQ, 0, s>>>(scores, n_cand, n_entries, cand_blocks, n_blocks, n_valid, k, gmax,
                                             sp.n_groups, cand, idx, top_scores);
    return hipGetLastError();
  }
  SelectPlan pl = plan_select(n_cand);
  k_select_compact<<<dim3((unsigned)pl.n_chunks, (unsigned)Q), NT, 0, s>>>(
      scores, n_cand, n_entries, cand_blocks, n_blocks, n_valid, k, gmax, sp.n_groups, pl.n_chunks, counts, cand);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_select_final<<<(unsigned)Q, NT, 0, s>>>(counts, pl.n_chunks, n_cand, k, cand, idx, top_scores);
  return hipGetLastError();
}

}  // namespace csa2
