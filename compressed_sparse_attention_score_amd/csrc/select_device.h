// Workgroup-level building blocks of the top-k selection, shared by the
// selection kernels and by the attention kernel that finishes a query's
// selection itself ("DeepSeek V4.1 Flash" guide, "A closer look": 512 entries
// selected per query; "An infra-oriented diagram of the DeepSeek-V4.1-Flash
// architecture", indexer bullet: top-512).
//
// Ranking: score descending, entry id ascending. A candidate is a 64-bit
// composite (order-preserving score key << 32 | ~id), so the exact top-k is
// the set of the k largest composites, which are unique; 0 marks "no
// candidate". Everything here is templated on the workgroup size NTH (a
// multiple of 256) and every function must be reached by the whole workgroup.
#pragma once

#include "csa2_device.h"

namespace csa2 {

constexpr int kRadixBits = 8;
constexpr int kBins = 1 << kRadixBits;
constexpr int kRegCand = 16;  // default candidates per thread held in registers by the final selection
// Candidates per thread once the final selection has spread a short joined
// list evenly over the workgroup (lists of at most NTH * kBalCand).
constexpr int kBalCand = 4;

// LDS scratch of the selection steps below.
template <int NTH>
struct SelScratch {
  alignas(16) unsigned hist[2][kBins];
  alignas(16) unsigned wsum[2 * (NTH / 64)];
  unsigned res[4];
  unsigned off[NTH + 1];  // exclusive offsets of the chunk regions in the joined list
  unsigned ext[2 * (NTH / 64)];  // per-wave largest and smallest key
};

// Inclusive prefix sum of x over the workgroup (thread order); *total gets the
// sum of all. Uses wsum (NTH/64 entries, 16-B aligned); contains barriers.
template <int NTH>
__device__ __forceinline__ unsigned block_incl_scan(unsigned x, unsigned* wsum, unsigned* total) {
  static_assert(NTH % 256 == 0, "wave sums are read four at a time");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  x = wave_incl_scan(x);
  __syncthreads();
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  unsigned before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NTH / 256; ++i) {
    const v4u s = *(const v4u*)(wsum + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      before += (4 * i + j < wv) ? s[j] : 0u;
      all += s[j];
    }
  }
  *total = all;
  return x + before;
}

// Two inclusive prefix sums at once (x0 and x1 scanned independently, one
// barrier pair for both). wsum holds 2*(NTH/64) entries, 16-B aligned.
template <int NTH>
__device__ __forceinline__ void block_incl_scan2(unsigned& x0, unsigned& x1, unsigned* wsum, unsigned* total0,
                                                 unsigned* total1) {
  static_assert(NTH % 256 == 0, "wave sums are read four at a time");
  constexpr int W = NTH / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  x0 = wave_incl_scan(x0);
  x1 = wave_incl_scan(x1);
  __syncthreads();
  if (lane == 63) {
    wsum[wv] = x0;
    wsum[W + wv] = x1;
  }
  __syncthreads();
  unsigned b0 = 0, b1 = 0, a0 = 0, a1 = 0;
#pragma unroll
  for (int i = 0; i < W / 4; ++i) {
    const v4u s0 = *(const v4u*)(wsum + 4 * i);
    const v4u s1 = *(const v4u*)(wsum + W + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b0 += (4 * i + j < wv) ? s0[j] : 0u;
      b1 += (4 * i + j < wv) ? s1[j] : 0u;
      a0 += s0[j];
      a1 += s1[j];
    }
  }
  *total0 = a0;
  *total1 = a1;
  x0 += b0;
  x1 += b1;
}

// Digit pick of one radix pass, run by wave 0 alone. Lane l holds bins
// 255-4l .. 252-4l (the digits from the top); a wave prefix sum over the lanes
// counts the values in the bins above each lane's, and the lane whose four
// bins hold the `remaining`-th largest value walks them. res gets the digit,
// the count in the bins above it, the count in its bin, and the histogram's
// total (lane 63's inclusive sum).
template <int CP = 1>
__device__ __forceinline__ void pick_digit_wave0(const unsigned* hist, unsigned remaining, unsigned* res) {
  const int lane = threadIdx.x & 63;
  v4u h = *(const v4u*)(hist + (kBins - 4) - 4 * lane);  // bins 252-4l .. 255-4l
#pragma unroll
  for (int c = 1; c < CP; ++c) h += *(const v4u*)(hist + c * kBins + (kBins - 4) - 4 * lane);
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
//
// top and prefix0 let a caller that knows every value shares its bits above
// `top` (those of prefix0) start there: the passes over bits that are the same
// in every value, which would put everything in one bin, are skipped.
//
// CP copies per histogram: hist then holds 2*CP rows, histogram b being rows
// b*CP .. b*CP+CP-1; count() spreads its atomics over them (by lane, in the
// callers below) so that lanes adding to one bin in the same instruction
// meet CP times less often, and the digit pick sums the copies.
template <int NTH, typename T, int CP = 1, typename Count>
__device__ __forceinline__ T radix_kth(Count count, unsigned k, unsigned (*hist)[kBins], unsigned* res, int max_passes,
                                       int top = (int)(sizeof(T) * 8), T prefix0 = 0) {
  constexpr int W = (int)(sizeof(T) * 8);
  for (int i = threadIdx.x; i < 2 * CP * kBins; i += NTH) hist[i / kBins][i % kBins] = 0u;
  __syncthreads();
  T prefix = prefix0;
  unsigned remaining = k;
  int b = 0, pass = 0;
  for (int hi = top; hi > 0 && pass < max_passes; hi -= kRadixBits, ++pass, b ^= 1) {
    const int shift = max(hi - kRadixBits, 0);
    count(hist[b * CP], hi, shift, prefix);
    // the other histogram was last read before the previous pass's second
    // barrier, and the next pass fills it after this pass's second barrier
    if (pass > 0)
      for (int i = threadIdx.x; i < CP * kBins; i += NTH) hist[(b ^ 1) * CP + i / kBins][i % kBins] = 0u;
    __syncthreads();
    if (threadIdx.x < 64) pick_digit_wave0<CP>(hist[b * CP], remaining, res);
    __syncthreads();
    const unsigned d = res[0], above = res[1], cnt = res[2], total = res[3];
    if (total < remaining) return (T)0;
    prefix |= ((T)(d & ((1u << (hi - shift)) - 1u))) << shift;
    remaining -= above;
    if (cnt == remaining) break;
  }
  return prefix;
}

// The same over PER values per thread held in registers.
template <int NTH, typename T, int PER, int CP = 1>
__device__ __forceinline__ T radix_kth_regs(const T (&v)[PER], unsigned k, unsigned (*hist)[kBins], unsigned* res,
                                            int max_passes = 64, int top = (int)(sizeof(T) * 8), T prefix0 = 0) {
  constexpr int W = (int)(sizeof(T) * 8);
  auto count = [&](unsigned* h, int hi, int shift, T prefix) {
    const unsigned dmask = (1u << (hi - shift)) - 1u;
    if (CP > 1) h += (threadIdx.x & (CP - 1)) * kBins;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const T x = v[j];
      if (x == 0) continue;
      if (hi < W && (x >> hi) != (prefix >> hi)) continue;
      atomicAdd(&h[(unsigned)(x >> shift) & dmask], 1u);
    }
  };
  return radix_kth<NTH, T, CP>(count, k, hist, res, max_passes, top, prefix0);
}

// The same over n values streamed from memory (lists too long for registers).
template <int NTH, typename T>
__device__ __forceinline__ T radix_kth_stream(const T* src, int64_t n, unsigned k, unsigned (*hist)[kBins],
                                              unsigned* res, int max_passes = 64) {
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

// The bits every non-zero value shares. Each lies between the smallest and
// the largest, so all agree above the highest bit where those two differ;
// 64-bit composites are ranged by their score keys (the top 32 bits), below
// which they may differ anywhere. *top gets that bit (the width when there are
// no values or they differ in the top bit, and at least 1) and *prefix the
// shared bits above it. ext: 2*(NTH/64) words of LDS. One barrier.
template <int NTH, typename T, int REG>
__device__ __forceinline__ void shared_top_bits(const T (&v)[REG], unsigned* ext, int* top, T* prefix) {
  constexpr int W = (int)(sizeof(T) * 8), S = W - 32;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  unsigned kmax = 0u, kmin = ~0u;
#pragma unroll
  for (int j = 0; j < REG; ++j) {
    if (v[j] != 0) {
      const unsigned key = (unsigned)(v[j] >> S);
      kmax = max(kmax, key);
      kmin = min(kmin, key);
    }
  }
  kmax = wave_umax(kmax);
  kmin = wave_umin(kmin);
  if (lane == 0) {
    ext[2 * wv] = kmax;
    ext[2 * wv + 1] = kmin;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    kmax = max(kmax, ext[2 * w]);
    kmin = min(kmin, ext[2 * w + 1]);
  }
  const unsigned diff = kmax ^ kmin;
  int t = (kmax == 0u || (diff >> 31)) ? W : S + (diff ? 32 - __clz((int)diff) : 0);
  // All values equal (32-bit values: t would be 0): start one bit up, so that
  // radix_kth still runs one pass, whose total tells whether k values exist
  // at all (with none run it would return the common value even when fewer
  // than k are present, e.g. a causal limit inside the first sub-chunk).
  if (t < 1) t = 1;
  *top = t;
  *prefix = (t >= W) ? (T)0 : ((((T)kmax) << S) >> t) << t;
}

// Exact top-k of the non-zero composites held REG per thread, thread order
// being list order: the k-th largest T (when there are more than m > k),
// then every composite >= T in list order; emit(pos, composite) for the list
// positions pos in [lo, hi) (hi <= k). Returns the number selected. With CP
// > 1 the radix passes count into CP copies per histogram held at hist
// (2*CP rows of LDS) instead of sc.hist.
template <int NTH, int REG, int CP = 1, typename Emit>
__device__ __forceinline__ unsigned select_regs(const unsigned long long (&v)[REG], unsigned m, int k,
                                                SelScratch<NTH>& sc, int lo, int hi, Emit emit,
                                                unsigned (*hist)[kBins] = nullptr) {
  unsigned long long T = 0ull;
  if (m > (unsigned)k) {
    int top;
    unsigned long long prefix;
    shared_top_bits<NTH, unsigned long long, REG>(v, sc.ext, &top, &prefix);
    T = radix_kth_regs<NTH, unsigned long long, REG, CP>(v, (unsigned)k, CP > 1 ? hist : sc.hist, sc.res, 64, top, prefix);
  }
  unsigned c = 0;
#pragma unroll
  for (int j = 0; j < REG; ++j) c += (v[j] != 0ull && v[j] >= T) ? 1u : 0u;
  unsigned all;
  unsigned pos = block_incl_scan<NTH>(c, sc.wsum, &all) - c;
#pragma unroll
  for (int j = 0; j < REG; ++j) {
    if (v[j] != 0ull && v[j] >= T) {
      if (pos >= (unsigned)lo && pos < (unsigned)hi) emit(pos, v[j]);
      ++pos;
    }
  }
  return min(all, (unsigned)k);
}

// Exact top-k of one query from the compacted candidate list: chunk c of the
// list holds cq[c] composites from position c*chunk on (in position order,
// which is ascending entry id), and the joined list is the chunks in order.
// emit(pos, composite) receives every selected composite whose rank in the
// output (list order) lies in [lo, hi), hi <= k, and emit(pos, 0) every
// position of [lo, hi) past the number selected.
//
// Three paths, by what fits: (1) each chunk's survivors fit the threads'
// register slots of that chunk: the slots are loaded together with the
// counts (one memory round trip) and masked by the counts; a joined list of
// at most NTH * kBalCand is then spread evenly over the threads through
// `list` (LDS, that many composites), so that every radix pass and the
// ordered write loop over kBalCand values instead of REG; (2) the joined list
// fits the registers: each thread locates its elements through an offset
// table; (3) otherwise the chunk regions are streamed.
template <int NTH, int REG = kRegCand, typename Emit>
__device__ __forceinline__ void select_from_regions(const unsigned* __restrict__ cq, int n_chunks, int chunk,
                                                    int64_t n_cand, int k, const unsigned long long* __restrict__ lq,
                                                    SelScratch<NTH>& sc, unsigned long long* list, int lo, int hi,
                                                    Emit emit) {
  const int tid = threadIdx.x;
  unsigned written = 0;
  bool done = false;
  unsigned m = 0, cnt_c = 0, incl_c = 0;
  if (n_chunks <= NTH && n_cand > 0) {
    // Chunk c's region starts at c*chunk whatever the counts, so each thread
    // loads REG fixed slots of one chunk (threads c*tpc .. c*tpc+tpc-1
    // take chunk c in order, so thread order is list order) together with
    // its chunk's count, and masks the slots past that count afterwards.
    const int tpc = NTH / n_chunks;
    const int c_t = tid / tpc, sub = tid - c_t * tpc;
    const bool own = c_t < n_chunks;
    const unsigned slot0 = (unsigned)sub * REG;
    const unsigned my_cnt = own ? cq[c_t] : 0u;
    const int64_t rb = (own ? (int64_t)c_t * chunk : 0) + slot0;
    unsigned long long v[REG];
#pragma unroll
    for (int j = 0; j < REG; ++j) v[j] = lq[min(rb + j, n_cand - 1)];  // slots past the list: dropped below
    // survivors this thread holds, and whether its chunk has more than its
    // threads' slots: one scan gives every thread its list position and the
    // list length, and tells whether the registers hold the whole list
    const unsigned held = (own && my_cnt > slot0) ? min(my_cnt - slot0, (unsigned)REG) : 0u;
    unsigned incl = held, over = (own && sub == 0 && my_cnt > (unsigned)tpc * REG) ? 1u : 0u, n_over;
    block_incl_scan2<NTH>(incl, over, sc.wsum, &m, &n_over);
    if (n_over == 0) {
#pragma unroll
      for (int j = 0; j < REG; ++j) v[j] = ((unsigned)j < held) ? v[j] : 0ull;
      if (m <= (unsigned)(NTH * kBalCand)) {
        const unsigned p = incl - held;
#pragma unroll
        for (int j = 0; j < REG; ++j)
          if ((unsigned)j < held) list[p + j] = v[j];
        __syncthreads();
        unsigned long long b[kBalCand];
#pragma unroll
        for (int j = 0; j < kBalCand; ++j) {
          const unsigned e = (unsigned)(tid * kBalCand + j);
          b[j] = (e < m) ? list[e] : 0ull;
        }
        written = select_regs<NTH, kBalCand>(b, m, k, sc, lo, hi, emit);
      } else {
        written = select_regs<NTH, REG>(v, m, k, sc, lo, hi, emit);
      }
      done = true;
    }
  }
  if (done) {
  } else if (n_chunks <= NTH && n_cand > 0) {
    cnt_c = (tid < n_chunks) ? cq[tid] : 0u;
    incl_c = block_incl_scan<NTH>(cnt_c, sc.wsum, &m);
  } else {
    for (int c0 = 0; c0 < n_chunks; c0 += NTH) {
      const unsigned x = (c0 + tid < n_chunks) ? cq[c0 + tid] : 0u;
      unsigned tot;
      const unsigned incl = block_incl_scan<NTH>(x, sc.wsum, &tot);
      if (c0 == 0) {
        cnt_c = x;
        incl_c = incl;
      }
      m += tot;
    }
  }
  if (done) {
  } else if (m <= (unsigned)(NTH * REG) && n_chunks <= NTH) {
    // The joined list is the chunk regions in chunk order; thread t takes its
    // elements t*REG .. +REG-1, locating their chunk through the
    // offset table (one binary search, then a forward walk).
    if (tid < n_chunks) sc.off[tid] = incl_c - cnt_c;
    if (tid == 0) sc.off[n_chunks] = m;
    __syncthreads();
    const unsigned e0 = (unsigned)tid * REG;
    int ch = 0;
    if (e0 < m) {
      int l = 0, h = n_chunks - 1;  // largest c with off[c] <= e0
      while (l < h) {
        const int mid = (l + h + 1) >> 1;
        if (sc.off[mid] <= e0) l = mid; else h = mid - 1;
      }
      ch = l;
    }
    // addresses first (the walk reads LDS only), then every load at once: a
    // load inside the walk would wait for the previous one each time
    int64_t at[REG];
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const unsigned e = e0 + j;
      at[j] = 0;
      if (e < m) {
        while (e >= sc.off[ch + 1]) ++ch;  // e < m = off[n_chunks] bounds the walk
        at[j] = (int64_t)ch * chunk + (e - sc.off[ch]);
      }
    }
    unsigned long long v[REG];
#pragma unroll
    for (int j = 0; j < REG; ++j) {
      const unsigned long long x = lq[at[j]];  // at[j] = 0 past the end: a valid slot, dropped
      v[j] = (e0 + j < m) ? x : 0ull;
    }
    written = select_regs<NTH, REG>(v, m, k, sc, lo, hi, emit);
  } else {
    // long lists (heavy ties or huge candidate sets): stream the chunk regions
    unsigned long long T = 0ull;
    if (m > (unsigned)k) {
      auto count = [&](unsigned* h, int hbit, int shift, unsigned long long prefix) {
        for (int c = 0; c < n_chunks; ++c) {
          const unsigned n_c = cq[c];
          for (unsigned i = tid; i < n_c; i += NTH) {
            const unsigned long long x = lq[(int64_t)c * chunk + i];
            if (hbit < 64 && (x >> hbit) != (prefix >> hbit)) continue;
            atomicAdd(&h[(unsigned)(x >> shift) & (kBins - 1)], 1u);
          }
        }
      };
      T = radix_kth<NTH, unsigned long long>(count, (unsigned)k, sc.hist, sc.res, 64);
    }
    // ordered write: chunk by chunk, NTH elements at a time, until the
    // requested range is covered (written is uniform over the workgroup)
    for (int c = 0; c < n_chunks && written < (unsigned)hi; ++c) {
      const unsigned n_c = cq[c];
      for (unsigned i0 = 0; i0 < n_c && written < (unsigned)hi; i0 += NTH) {
        const unsigned i = i0 + tid;
        const unsigned long long x = (i < n_c) ? lq[(int64_t)c * chunk + i] : 0ull;
        const unsigned sel = (x != 0ull && x >= T) ? 1u : 0u;
        unsigned tot;
        const unsigned pos = written + block_incl_scan<NTH>(sel, sc.wsum, &tot) - sel;
        if (sel && pos >= (unsigned)lo && pos < (unsigned)hi) emit(pos, x);
        written += tot;
      }
    }
    written = min(written, (unsigned)k);
  }
  for (int j = max((int)written, lo) + tid; j < hi; j += NTH) emit((unsigned)j, 0ull);
}


// Exact top-k of a plain candidate range straight from its scores: position
// p (< n_cand) is a candidate when p < limit; thread t takes positions
// PER*t .. PER*t+PER-1 (thread order is list order) as composites, and the
// selection and ordered write are those of select_regs. emit as for
// select_from_regions, including emit(pos, 0) past the number selected.
// hist4: 2*4 histogram rows of LDS. Normal scores put most of the 4,096 keys
// of the first radix pass into a few exponent bins, so the passes count
// into four copies (a step of 21.7 -> 21.1 us for one query over 4,096
// entries; eight copies: 21.8 us).
template <int NTH, int PER, typename Emit>
__device__ __forceinline__ void select_from_scores(const float* __restrict__ sq, int64_t n_cand, int64_t limit, int k,
                                                   SelScratch<NTH>& sc, int lo, int hi, Emit emit,
                                                   unsigned (*hist4)[kBins]) {
  const int tid = threadIdx.x;
  const int64_t p0 = (int64_t)tid * PER;
  const int64_t vlim = min(n_cand, limit);
  unsigned long long v[PER];
  unsigned cnt = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t p = p0 + j;
    // a load without a condition (the last score stands in past the list)
    const float s = sq[n_cand > 0 ? min(p, n_cand - 1) : 0];
    const bool ok = p < vlim;
    v[j] = ok ? (((unsigned long long)score_key(s) << 32) | (unsigned long long)(~(unsigned)p)) : 0ull;
    cnt += ok ? 1u : 0u;
  }
  unsigned m;
  block_incl_scan<NTH>(cnt, sc.wsum, &m);
  const unsigned written = select_regs<NTH, PER, 4>(v, m, k, sc, lo, hi, emit, hist4);
  for (int j = max((int)written, lo) + tid; j < hi; j += NTH) emit((unsigned)j, 0ull);
}

}  // namespace csa2
