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
//     theta is that key with its low bits cleared (a lower bound still):
//     radix passes fix the 8 (compaction) or 16 (per-query kernel) bits
//     below those every maximum shares. Each compaction workgroup finds
//     theta and writes its chunk's composites with key >= theta, in position
//     order (block prefix sum), to a fixed region of the candidate list.
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
#include "select_device.h"

#include <type_traits>

namespace csa2 {

namespace {
constexpr int NT = 256;
constexpr int kChunk = 4096;  // scores per compaction workgroup (16 per thread)
constexpr int kPer = kChunk / NT;

// Score staging of the compaction: part p (4 scores) of thread t's 16 at
// float 16t + 4 (p ^ ((t / 4) & 3)), so that each run of 8 lanes storing
// writes one 128-byte half of a bank row and each run of 16 lanes reading
// part p covers the 16 granules of one.
// (The earlier padded layout, 20 floats per thread, spread each run of 8
// stores over both halves: config 4's step 74.1 -> 73.8 us, config 1's 37.6
// -> 37.4 us, A/B.)
__device__ __forceinline__ int stage_at(int t, int p) { return 16 * t + 4 * (p ^ ((t >> 2) & 3)); }
// Buffer resource word 3 for untyped dword access on gfx9-family parts.
constexpr int kBufWord3 = 0x00020000;

struct SelShared {
  SelScratch<NT> sel;
  alignas(16) float stage[NT * kPer];
};
}  // namespace

// theta needs only to be a lower bound on the k-th largest score: two passes,
// starting at the highest bit where the sub-chunk maxima differ, fix 16 bits
// of the k-th sub-chunk maximum below the bits all maxima share (at least its
// sign, exponent and top 7 mantissa bits), which lowers the bound by less
// than 2^-7 of its value and adds a few percent of survivors, and saves the
// passes over the remaining low bits.
constexpr int kThetaPasses = 2;
// The chunk compaction takes one pass (8 bits below the shared ones): its
// survivors only pass through LDS and a final selection, and one pass fewer
// shortened the batch-16 x 65,536 decode step by about 0.6 us. The per-query
// kernel keeps two: it reads only the sub-chunks whose maximum reaches theta,
// and the coarser bound let enough more through to cost the 4,096-query
// prefill selection over 100 us.
constexpr int kCompactThetaPasses = 1;
// The per-query kernel of small batches (1,024 threads) also takes one: each
// pass costs it about 2,000 cycles of barrier-bound work, and the coarser
// bound adds a few hundred survivors to a final selection whose cost hardly
// depends on their number.
constexpr int kSmallThetaPasses = 1;

// Threshold + compaction: grid (n_chunks, Q), or with qx a 1-D grid of
// n_chunks * Q whose workgroups of query q sit 8 ids apart from q & 7 on, so
// that they share an XCD with the query's scan and attention workgroups (Q a
// multiple of 8). Writes cand[q][c0 .. c0+cnt) in position order and
// counts[q][chunk] = cnt.
__global__ __launch_bounds__(NT) void k_select_compact(const float* __restrict__ scores, int64_t n_cand,
                                                       int64_t n_entries, const int32_t* __restrict__ cand_blocks,
                                                       int n_blocks, const int32_t* __restrict__ n_valid, int k,
                                                       const unsigned* __restrict__ gmax, int64_t n_groups,
                                                       int n_chunks, unsigned* __restrict__ counts,
                                                       unsigned long long* __restrict__ cand, int qx) {
  __shared__ SelShared sh;
  int q = blockIdx.y, cx = blockIdx.x;  // query, chunk
  if (qx) {
    const int lin = blockIdx.x;
    q = ((lin / (8 * n_chunks)) << 3) | (lin & 7);
    cx = (lin >> 3) % n_chunks;
  }
  const int tid = threadIdx.x;
  int64_t limit = n_entries;
  if (n_valid) limit = min(limit, (int64_t)n_valid[q]);

  // this thread's 16 consecutive positions. The query's sub-chunk maxima are
  // requested first and the chunk's scores after them (lane l takes vector l
  // of each 4-KiB slice, coalesced), all without a condition, and the scores
  // stay in registers until the threshold is known: the threshold then waits
  // for the maxima alone while the scores are in flight. The scores go
  // through LDS afterwards so that each thread picks up its own 16. (The
  // maxima's wait used to cover the scores too: config 1's step 38.2 ->
  // 36.9 us, config 4's 74.9 -> 74.2 us.)
  const int64_t c0 = (int64_t)cx * kChunk;
  const int64_t p0 = c0 + (int64_t)tid * kPer;
  const float* srow = scores + (int64_t)q * n_cand;
  unsigned g[16];
  {
    // through a buffer resource that ends at the last sub-chunk: lanes past
    // it read zeros (the empty key) without touching memory
    const int gbytes = (int)min(n_groups, (int64_t)NT * 16) * 4;
    const __amdgpu_buffer_rsrc_t grs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(gmax + (int64_t)q * n_groups), 0, gbytes, kBufWord3);
#pragma unroll
    for (int j = 0; j < 16; ++j) g[j] = __builtin_amdgcn_raw_buffer_load_b32(grs, 4 * (j * NT + tid), 0, 0);
  }
  v4u xs[kPer / 4];
  {
    // coalesced 16-B loads through a buffer resource that ends at the list's
    // end: the range check is per dword, so a load straddling the end returns
    // its dwords inside and zeros past it (positions never kept)
    const int nrec = (int)min(n_cand - c0, (int64_t)kChunk) * 4;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc((void*)(srow + c0), 0, nrec, kBufWord3);
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) xs[i] = __builtin_amdgcn_raw_buffer_load_b128(srs, 16 * (i * NT + tid), 0, 0);
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
      int top;
      unsigned prefix;
      shared_top_bits<NT, unsigned, 16>(g, sh.sel.ext, &top, &prefix);
      t = radix_kth_regs<NT, unsigned, 16>(g, (unsigned)k, sh.sel.hist, sh.sel.res, kCompactThetaPasses, top,
                                            prefix);
    } else {
      t = radix_kth_stream<NT, unsigned>(gq, n_groups, (unsigned)k, sh.sel.hist, sh.sel.res, kThetaPasses);
    }
    theta = t > 1u ? t : 1u;
  }

  // the scores to LDS, then each thread picks up its 16 consecutive ones
#pragma unroll
  for (int i = 0; i < kPer / 4; ++i) {
    const int v = i * NT + tid;  // float4 index inside the chunk
    *(v4u*)(sh.stage + stage_at(v >> 2, v & 3)) = xs[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer / 4; ++i) {
    const v4f x = *(const v4f*)(sh.stage + stage_at(tid, i));
    sc[4 * i] = x[0]; sc[4 * i + 1] = x[1]; sc[4 * i + 2] = x[2]; sc[4 * i + 3] = x[3];
  }

  // ---- keep key >= theta, in position order. Above the key of +0 and on a
  // plain range, the same one-compare filter as the per-query kernel below
  // (a score passes exactly when theta' <= its bits <= those of +inf).
  unsigned long long comp[kPer];
  unsigned cnt = 0;
  if (cand_blocks == nullptr && theta > 0x80000000u) {
    const unsigned tlo = theta & 0x7FFFFFFFu, tspan = 0x7F800000u - tlo;
    const int nv = (int)max((int64_t)0, min(min(n_cand, limit) - p0, (int64_t)kPer));
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const unsigned u = __float_as_uint(sc[j]);
      const bool keep = j < nv && u - tlo <= tspan;
      comp[j] = keep ? (((unsigned long long)(u | 0x80000000u) << 32) | (unsigned long long)(~(unsigned)(p0 + j)))
                     : 0ull;
      cnt += keep ? 1u : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const unsigned key = score_key(sc[j]);
      const bool keep = ent[j] >= 0 && key >= theta;
      comp[j] = keep ? (((unsigned long long)key << 32) | (unsigned long long)(~(unsigned)ent[j])) : 0ull;
      cnt += keep ? 1u : 0u;
    }
  }
  unsigned total;
  const unsigned incl = block_incl_scan<NT>(cnt, sh.sel.wsum, &total);
  unsigned pos = incl - cnt;
  unsigned long long* dst = cand + (int64_t)q * n_cand + c0;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (comp[j]) dst[pos++] = comp[j];
  if (tid == 0) counts[(int64_t)q * n_chunks + cx] = total;
}

// Exact top-k of each query's candidate list: grid (Q). Output in list order.
__global__ __launch_bounds__(NT) void k_select_final(const unsigned* __restrict__ counts, int n_chunks,
                                                     int64_t n_cand, int k, const unsigned long long* __restrict__ cand,
                                                     int32_t* __restrict__ idx, float* __restrict__ top_scores) {
  __shared__ SelScratch<NT> sc;
  __shared__ __attribute__((aligned(16))) unsigned long long list[NT * kBalCand];
  const int q = blockIdx.x;
  int32_t* iq = idx + (int64_t)q * k;
  float* tq = top_scores ? top_scores + (int64_t)q * k : nullptr;
  select_from_regions<NT>(counts + (int64_t)q * n_chunks, n_chunks, kChunk, n_cand, k, cand + (int64_t)q * n_cand, sc,
                          list, 0, k, [&](unsigned pos, unsigned long long x) {
                            iq[pos] = x ? (int32_t)(~(unsigned)(x & 0xFFFFFFFFull)) : -1;
                            if (tq) tq[pos] = x ? key_score((unsigned)(x >> 32)) : -__builtin_inff();
                          });
}

// ---------------------------------------------------------------------------
// One workgroup per query (lists up to kQMaxCand candidates). Same method as
// the two kernels above, in one launch: theta from the sub-chunk maxima,
// compaction of the candidates >= theta in position order (ascending entry
// id: pools list their blocks in ascending order), then the exact k-th
// composite among the survivors and the ordered write.
namespace {
// The workgroup size is a template parameter. Large batches take 256-thread
// workgroups limited to 128 VGPRs, four to a CU, so that some stream their
// query's scores while others run their barrier-bound radix passes; small
// batches take 1,024 threads, so that their few queries still spread over
// the CU's waves.
constexpr int kQPer = 16;           // positions per thread per pass
constexpr int64_t kQMaxCand = 1 << 18;
constexpr int kQSmallBatch = 1024;  // queries from which the 256-thread workgroup is used

// Survivors held in LDS: 8 per thread at 1,024 threads, 15 per thread below
// (a selection keeps k and a few percent more).
template <int NQ>
constexpr int q_cap() { return NQ >= 1024 ? 8192 : 15 * NQ; }
// Sub-chunk maxima held per thread for the threshold search and the
// sub-chunk skipping (lists of up to kQMaxPer * NQ sub-chunks).
constexpr int kQMaxPer = 8;

template <int NQ>
struct QSelShared {
  alignas(16) unsigned hist[2][kBins];
  alignas(16) unsigned wsum[2 * (NQ / 64)];
  unsigned res[4];
  unsigned ext[2 * (NQ / 64)];
  unsigned short glist[kQMaxPer * NQ];  // sub-chunks that can hold survivors, ascending
  unsigned long long cand[q_cap<NQ>() + q_cap<NQ>() / 16];  // survivor i at q_slot(i)
};

// LDS slot of survivor i: one pad slot after every 16, so that the runs of
// survivors that neighbouring lanes write spread over the banks.
__device__ __forceinline__ unsigned q_slot(unsigned i) { return i + (i >> 4); }

}  // namespace

// POOL: the lists are pools of blocks of 8 (cand_blocks given); otherwise
// the plain range [0, n_cand) (cand_blocks NULL).
template <int NQ, int RUN, bool POOL>
__global__ __launch_bounds__(NQ) __attribute__((amdgpu_waves_per_eu(NQ >= 1024 ? 1 : 4))) void k_select_query(const float* __restrict__ scores, int64_t n_cand,
                                                     int64_t n_entries, const int32_t* __restrict__ cand_blocks,
                                                     int n_blocks, const int32_t* __restrict__ n_valid, int k,
                                                     const unsigned* __restrict__ gmax, int64_t n_groups, int group,
                                                     unsigned long long* __restrict__ gcand, int32_t* __restrict__ idx,
                                                     float* __restrict__ top_scores) {
  constexpr int kQCap = q_cap<NQ>();
  constexpr int kQGrp = kQPer / RUN;  // groups per pass
  static_assert(RUN == 4 || RUN == 8 || RUN == 16, "a run is 4, 8 or 16 positions");
  __shared__ QSelShared<NQ> sh;
  const int q = blockIdx.x, tid = threadIdx.x;
  int64_t limit = n_entries;
  if (n_valid) limit = min(limit, (int64_t)n_valid[q]);
  int32_t* iq = idx + (int64_t)q * k;
  float* tq = top_scores ? top_scores + (int64_t)q * k : nullptr;
  const float* srow = scores + (int64_t)q * n_cand;
  unsigned long long* gq = gcand + (int64_t)q * n_cand;

  // Positions are taken in passes of NQ*kQPer, split into kQGrp groups of
  // NQ*RUN consecutive positions; thread t owns positions RUN*t..RUN*t+RUN-1
  // of each group (with RUN = 4 every load instruction of the workgroup
  // reads one contiguous NQ*16-byte span). Survivors keep position order:
  // group g's go after those of the groups before it, within a group in
  // thread order. Full passes (rows 16-byte aligned) load with aligned
  // vectors and no per-thread conditions, the next pass's scores in flight
  // while this one is compacted; a ragged last pass is guarded. (These
  // "groups" are the pass's thread layout; the "sub-chunks" below are the
  // ranges whose maxima the scan wrote.)
  constexpr int64_t kGrpLen = (int64_t)NQ * RUN;
  constexpr int kBlk = (RUN + 7) / 8;  // pool blocks a run touches
  constexpr int64_t kStep = kGrpLen * kQGrp;
  const int64_t n_full = ((n_cand & 3) == 0) ? n_cand / kStep : 0;
  auto load_full = [&](float* sc, int32_t* blk, int64_t p0) {
#pragma unroll
    for (int g = 0; g < kQGrp; ++g) {
      const int64_t pb = p0 + g * kGrpLen + RUN * tid;
#pragma unroll
      for (int j = 0; j < RUN; j += 4) {
        const v4f v = *(const v4f*)(srow + pb + j);
        sc[RUN * g + j] = v[0]; sc[RUN * g + j + 1] = v[1]; sc[RUN * g + j + 2] = v[2]; sc[RUN * g + j + 3] = v[3];
      }
#pragma unroll
      for (int b = 0; b < kBlk; ++b)
        blk[kBlk * g + b] = POOL ? cand_blocks[(int64_t)q * n_blocks + (pb >> 3) + b] : 0;
    }
  };
  float scA[kQPer], scB[kQPer];
  int32_t bkA[kQGrp * kBlk], bkB[kQGrp * kBlk];
  // Sub-chunk skipping (plain ranges, maxima held in registers): a sub-chunk
  // whose maximum key lies below theta holds no survivor, so only the others
  // are read. The maxima pass over NaN and give an all-invalid or all -inf
  // sub-chunk key 0, so they bound every key above that of -inf; skipping is
  // taken only with theta above the key of +0, where NaN and -inf cannot pass.
  // A list read in one pass is read whole, its loads in flight during the
  // threshold search; skipping pays when it saves passes.
  const bool can_skip = !POOL && gmax && n_cand > kStep && n_groups >= k && n_groups <= kQMaxPer * NQ && group >= RUN &&
                        (group & (group - 1)) == 0;
  const bool pre = n_full > 0 && !can_skip;
  // Ragged or unaligned passes: positions past the end load the last score
  // (clamped, so every load is issued at once instead of one guarded round
  // trip after another) and are dropped by process(). A list that is one such
  // pass is requested before the threshold search, like the full passes.
  auto load_ragged = [&](float* sc, int32_t* blk, int64_t p0) {
#pragma unroll
    for (int g = 0; g < kQGrp; ++g) {
      const int64_t pb = p0 + g * kGrpLen + RUN * tid;
#pragma unroll
      for (int i = 0; i < RUN; ++i) sc[RUN * g + i] = srow[min(pb + i, n_cand - 1)];
#pragma unroll
      for (int b = 0; b < kBlk; ++b)
        blk[kBlk * g + b] = POOL ? cand_blocks[(int64_t)q * n_blocks + min((pb >> 3) + b, (int64_t)n_blocks - 1)] : 0;
    }
  };
  const bool pre_ragged = n_full == 0 && n_cand > 0 && n_cand <= kStep && !can_skip;

  // ---- theta = k-th largest sub-chunk maximum (1 = keep every valid candidate)
  unsigned theta = 1u;
  unsigned g[kQMaxPer];  // maxima of sub-chunks j*NQ + tid
#pragma unroll
  for (int j = 0; j < kQMaxPer; ++j) g[j] = 0u;
  const bool theta_regs = gmax && n_groups >= k && n_groups <= kQMaxPer * NQ;
  if (theta_regs) {  // requested first: the threshold search waits on these, not on the scores
    const unsigned* gm = gmax + (int64_t)q * n_groups;
#pragma unroll
    for (int j = 0; j < kQMaxPer; ++j) {
      const int64_t i = (int64_t)j * NQ + tid;
      g[j] = (i < n_groups) ? gm[i] : 0u;
    }
  }
  if (pre) load_full(scA, bkA, 0);  // in flight during the threshold search
  if (pre_ragged) load_ragged(scA, bkA, 0);
  if (gmax && n_groups >= k) {
    const unsigned* gm = gmax + (int64_t)q * n_groups;
    unsigned t;
    if (theta_regs) {
      int top;
      unsigned prefix;
      shared_top_bits<NQ, unsigned, kQMaxPer>(g, sh.ext, &top, &prefix);
      t = radix_kth_regs<NQ, unsigned, kQMaxPer>(g, (unsigned)k, sh.hist, sh.res,
                                                 NQ >= 1024 ? kSmallThetaPasses : kThetaPasses, top, prefix);
    } else {
      t = radix_kth_stream<NQ, unsigned>(gm, n_groups, (unsigned)k, sh.hist, sh.res, kThetaPasses);
    }
    theta = t > 1u ? t : 1u;
  }

  // ---- keep key >= theta, in position order
  unsigned m = 0;  // survivors so far (block-uniform)
  // Fast filter. When theta lies above the key of +0 and the list is the
  // plain range [0, n_cand), a score passes exactly when its bit pattern u
  // satisfies theta' <= u <= 0x7F800000 (+inf), theta' being theta without
  // its sign bit: a non-negative score's key is u + 2^31, and every negative
  // score, -0 and NaN has u > 0x7F800000 and a key below theta. One subtract
  // and one unsigned compare per score; the composite is built for the
  // survivors only.
  const bool fast = theta > 0x80000000u;
  const unsigned tlo = theta & 0x7FFFFFFFu, tspan = 0x7F800000u - tlo;
  const int64_t vlim = min(n_cand, limit);  // valid positions of the plain range
  // Each group's count (at most RUN per thread, NQ*RUN <= 16,384 per
  // workgroup) takes 16 bits of a scanned word: one word for one or two
  // groups, two words (one scan) for four.
  static_assert(NQ * RUN <= 65535, "a group's count fits 16 bits");
  auto place = [&](const unsigned (&cnt)[kQGrp], unsigned (&pos)[kQGrp]) {
    if constexpr (kQGrp == 4) {
      unsigned w0 = cnt[0] | (cnt[1] << 16), w1 = cnt[2] | (cnt[3] << 16);
      const unsigned e0 = w0, e1 = w1;
      unsigned t0, t1;
      block_incl_scan2<NQ>(w0, w1, sh.wsum, &t0, &t1);
      w0 -= e0;  // exclusive
      w1 -= e1;
      const unsigned T0 = t0 & 0xFFFFu, T1 = t0 >> 16, T2 = t1 & 0xFFFFu;
      pos[0] = m + (w0 & 0xFFFFu);
      pos[1] = m + T0 + (w0 >> 16);
      pos[2] = m + T0 + T1 + (w1 & 0xFFFFu);
      pos[3] = m + T0 + T1 + T2 + (w1 >> 16);
      m += T0 + T1 + T2 + (t1 >> 16);
    } else {
      const unsigned w = kQGrp == 2 ? (cnt[0] | (cnt[kQGrp - 1] << 16)) : cnt[0];
      unsigned t;
      const unsigned x = block_incl_scan<NQ>(w, sh.wsum, &t) - w;  // exclusive
      const unsigned T0 = kQGrp == 2 ? (t & 0xFFFFu) : t;
      pos[0] = m + (kQGrp == 2 ? (x & 0xFFFFu) : x);
      pos[kQGrp - 1] = kQGrp == 2 ? m + T0 + (x >> 16) : pos[0];
      m += kQGrp == 2 ? T0 + (t >> 16) : t;
    }
  };
  auto put = [&](unsigned pos, unsigned long long comp) {
    if (pos < (unsigned)kQCap) sh.cand[q_slot(pos)] = comp;
    else gq[pos] = comp;
  };
  // The survivors of a pass are marked in a bit mask (bit 4g+i: position
  // 4t+i of group g) and their composites rebuilt at the store, so no
  // per-position composite is held across the scan.
  // entry of position p = RUN*t + i of group g
  auto entry_of = [&](const int32_t* blk, int g, int i, int64_t p) -> int64_t {
    if constexpr (!POOL) return p;
    const int32_t b = blk[kBlk * g + (RUN >= 8 ? i >> 3 : 0)];
    return (b < 0) ? -1 : 8 * (int64_t)b + (p & 7);
  };
  // run_pos(g): first position of this thread's run in group g (runs hold
  // consecutive positions)
  auto process_at = [&](const float* sc, const int32_t* blk, auto&& run_pos) {
    unsigned cnt[kQGrp], pos[kQGrp];
    unsigned keep = 0;  // bit RUN*g+i: position RUN*t+i of group g survives
    // Pools with one group (runs of 16), without the fast filter: the
    // composites are built once, before the scan, and held (32 VGPRs, which
    // that variant has to spare); otherwise they are rebuilt at the store.
    constexpr bool kHold = POOL && kQGrp == 1;
    unsigned long long comp[kHold ? kQPer : 1];
#pragma unroll
    for (int g = 0; g < kQGrp; ++g) {
      const int64_t pb = run_pos(g);
      unsigned kg = 0;
      if (fast) {
        const int nv = (int)max((int64_t)0, min((POOL ? n_cand : vlim) - pb, (int64_t)RUN));
#pragma unroll
        for (int i = 0; i < RUN; ++i)
          kg |= (i < nv && __float_as_uint(sc[RUN * g + i]) - tlo <= tspan) ? (1u << i) : 0u;
        if constexpr (POOL) {
          // a pool position holds a candidate when its block id is valid and
          // the entry lies below the limit: checked for the few that pass
          for (unsigned rest = kg; rest; rest &= rest - 1) {
            const int i = __builtin_ctz(rest);
            const int64_t e = entry_of(blk, g, i, pb + i);
            if (e < 0 || e >= limit) kg &= ~(1u << i);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < RUN; ++i) {
          const int64_t e = entry_of(blk, g, i, pb + i);
          const bool valid = pb + i < n_cand && e >= 0 && e < limit;
          const unsigned key = score_key(sc[RUN * g + i]);
          const bool kp = valid && key >= theta;
          if constexpr (kHold) comp[i] = kp ? (((unsigned long long)key << 32) | (unsigned long long)(~(unsigned)e)) : 0ull;
          kg |= kp ? (1u << i) : 0u;
        }
      }
      cnt[g] = __builtin_popcount(kg);
      keep |= kg << (RUN * g);
    }
    place(cnt, pos);
    if (kHold && !fast) {
#pragma unroll
      for (int i = 0; i < kQPer; ++i)
        if (comp[i]) put(pos[0]++, comp[i]);
      return;
    }
#pragma unroll
    for (int g = 0; g < kQGrp; ++g) {
      const int64_t pb = run_pos(g);
#pragma unroll
      for (int i = 0; i < RUN; ++i) {
        if (keep & (1u << (RUN * g + i))) {
          // in the fast filter every survivor is a non-negative score: key =
          // bits with the sign bit set
          const unsigned key = fast ? (__float_as_uint(sc[RUN * g + i]) | 0x80000000u) : score_key(sc[RUN * g + i]);
          const unsigned e = (unsigned)entry_of(blk, g, i, pb + i);
          put(pos[g]++, ((unsigned long long)key << 32) | (unsigned long long)(~e));
        }
      }
    }
  };
  auto process = [&](const float* sc, const int32_t* blk, int64_t p0) {
    process_at(sc, blk, [&](int g) { return p0 + g * kGrpLen + RUN * tid; });
  };
  if (can_skip && fast) {
    // ordered list of the sub-chunks with maximum >= theta (sub-chunk
    // j*NQ + t is this thread's g[j]; at most NQ per j, so 16-bit fields,
    // two to a scanned word)
    const int lg = __builtin_ctz((unsigned)group);
    static_assert(kQMaxPer % 4 == 0, "maxima are listed four at a time");
    unsigned base = 0;  // listed sub-chunks of the rounds before
#pragma unroll
    for (int r = 0; r < kQMaxPer; r += 4) {
      unsigned f[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) f[j] = ((int64_t)(r + j) * NQ + tid < n_groups && g[r + j] >= theta) ? 1u : 0u;
      unsigned w0 = f[0] | (f[1] << 16), w1 = f[2] | (f[3] << 16);
      const unsigned e0 = w0, e1 = w1;
      unsigned t0, t1;
      block_incl_scan2<NQ>(w0, w1, sh.wsum, &t0, &t1);
      w0 -= e0;
      w1 -= e1;
      const unsigned T0 = t0 & 0xFFFFu, T1 = t0 >> 16, T2 = t1 & 0xFFFFu;
      const unsigned at[4] = {w0 & 0xFFFFu, T0 + (w0 >> 16), T0 + T1 + (w1 & 0xFFFFu), T0 + T1 + T2 + (w1 >> 16)};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (f[j]) sh.glist[base + at[j]] = (unsigned short)((r + j) * NQ + tid);
      base += T0 + T1 + T2 + (t1 >> 16);
    }
    __syncthreads();
    const int64_t V = (int64_t)base << lg;  // positions of the listed sub-chunks
    const bool vec = (n_cand & 3) == 0;
    // virtual position v -> position: listed sub-chunk v >> lg, offset
    // v & (group-1); a run never crosses a sub-chunk (group >= RUN, both
    // powers of two)
    auto load_v = [&](float* sc, int64_t* pbs, int64_t v0) {
#pragma unroll
      for (int gg = 0; gg < kQGrp; ++gg) {
        const int64_t v = v0 + gg * kGrpLen + RUN * tid;
        int64_t pb = n_cand;  // past the list: dropped by the filter
        if (v < V) pb = ((int64_t)sh.glist[v >> lg] << lg) + (v & (group - 1));
        pbs[gg] = pb;
        if (vec && pb + RUN <= n_cand) {
#pragma unroll
          for (int jj = 0; jj < RUN; jj += 4) {
            const v4f x = *(const v4f*)(srow + pb + jj);
            sc[RUN * gg + jj] = x[0]; sc[RUN * gg + jj + 1] = x[1];
            sc[RUN * gg + jj + 2] = x[2]; sc[RUN * gg + jj + 3] = x[3];
          }
        } else {
#pragma unroll
          for (int i = 0; i < RUN; ++i) sc[RUN * gg + i] = srow[min(pb + i, n_cand - 1)];
        }
      }
    };
    int64_t pA[kQGrp], pB[kQGrp];
    const int64_t n_pass = (V + kStep - 1) / kStep;
    if (n_pass > 0) load_v(scA, pA, 0);
    for (int64_t i = 0; i < n_pass; i += 2) {
      if (i + 1 < n_pass) load_v(scB, pB, (i + 1) * kStep);
      process_at(scA, bkA, [&](int gg) { return pA[gg]; });
      if (i + 1 >= n_pass) break;
      if (i + 2 < n_pass) load_v(scA, pA, (i + 2) * kStep);
      process_at(scB, bkB, [&](int gg) { return pB[gg]; });
    }
  } else {
    if (n_full > 0 && !pre) load_full(scA, bkA, 0);
    for (int64_t i = 0; i < n_full; i += 2) {
      if (i + 1 < n_full) load_full(scB, bkB, (i + 1) * kStep);
      process(scA, bkA, i * kStep);
      if (i + 1 >= n_full) break;
      if (i + 2 < n_full) load_full(scA, bkA, (i + 2) * kStep);
      process(scB, bkB, (i + 1) * kStep);
    }
    for (int64_t p0 = n_full * kStep; p0 < n_cand; p0 += kStep) {  // ragged or unaligned passes
      if (!(pre_ragged && p0 == 0)) load_ragged(scA, bkA, p0);
      process(scA, bkA, p0);
    }
  }
  __syncthreads();

  unsigned written = 0;
  // ---- survivors in LDS: thread t takes list elements P*t..P*t+P-1, P the
  // fewest per thread that hold the list (2, 4 or all kQCap/NQ), so that the
  // radix passes and the ordered write loop over no more slots than needed
  auto final_select = [&](auto p_tag) {
    constexpr int P = decltype(p_tag)::value;
    unsigned long long v[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const unsigned e = (unsigned)tid * P + j;
      v[j] = (e < m) ? sh.cand[q_slot(e)] : 0ull;
    }
    unsigned long long T = 0ull;
    if (m > (unsigned)k) {
      int top;
      unsigned long long prefix;
      shared_top_bits<NQ, unsigned long long, P>(v, sh.ext, &top, &prefix);
      T = radix_kth_regs<NQ, unsigned long long, P>(v, (unsigned)k, sh.hist, sh.res, 64, top, prefix);
    }
    unsigned c = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) c += (v[j] != 0ull && v[j] >= T) ? 1u : 0u;
    unsigned all;
    unsigned pos = block_incl_scan<NQ>(c, sh.wsum, &all) - c;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      if (v[j] != 0ull && v[j] >= T && pos < (unsigned)k) {
        iq[pos] = (int32_t)(~(unsigned)(v[j] & 0xFFFFFFFFull));
        if (tq) tq[pos] = key_score((unsigned)(v[j] >> 32));
        ++pos;
      }
    }
    written = min(all, (unsigned)k);
  };
  constexpr int kPerAll = kQCap / NQ;
  if (m <= (unsigned)(2 * NQ)) {
    final_select(std::integral_constant<int, 2>{});
  } else if (kPerAll > 4 && m <= (unsigned)(4 * NQ)) {
    final_select(std::integral_constant<int, (kPerAll > 4 ? 4 : kPerAll)>{});
  } else if (m <= (unsigned)kQCap) {
    final_select(std::integral_constant<int, kPerAll>{});
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
      const unsigned pos = written + block_incl_scan<NQ>(sel, sh.wsum, &tot) - sel;
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

// One workgroup per query when that fills the chip or the lists are short
// (a single CU compacts ~20 vector ops per candidate); otherwise compaction
// chunks in parallel, then a per-query final selection.
bool select_is_chunked(int Q, int64_t n_cand) { return !(n_cand <= kQMaxCand && (Q >= 64 || n_cand <= 16384)); }

hipError_t launch_select_compact(const float* scores, int Q, int64_t n_cand, int64_t n_entries,
                                 const int32_t* cand_blocks, int n_blocks, const int32_t* n_valid, int k,
                                 const ScorePlan& sp, const unsigned* gmax, unsigned* counts, unsigned long long* cand,
                                 hipStream_t s) {
  if (Q <= 0) return hipSuccess;
  SelectPlan pl = plan_select(n_cand);
  const bool qx = Q % 8 == 0 && (int64_t)pl.n_chunks * Q * NT < ((int64_t)1 << 31);  // 1-D grid size
  const dim3 cg = qx ? dim3((unsigned)(pl.n_chunks * Q)) : dim3((unsigned)pl.n_chunks, (unsigned)Q);
  k_select_compact<<<cg, NT, 0, s>>>(
      scores, n_cand, n_entries, cand_blocks, n_blocks, n_valid, k, gmax, sp.n_groups, pl.n_chunks, counts, cand, qx ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_select(const float* scores, int Q, int64_t n_cand, int64_t n_entries, const int32_t* cand_blocks,
                         int n_blocks, const int32_t* n_valid, int k, const ScorePlan& sp, const unsigned* gmax,
                         unsigned* counts, unsigned long long* cand, int32_t* idx, float* top_scores, hipStream_t s) {
  if (Q <= 0) return hipSuccess;
  if (!select_is_chunked(Q, n_cand)) {
    // Small batches: 1,024 threads, pools in runs of 16 (composites held),
    // plain ranges in runs of 4 (coalesced loads); large batches: 256
    // threads in runs of 4.
    const bool pool = cand_blocks != nullptr;
    const dim3 g((unsigned)Q);
    if (Q >= kQSmallBatch && pool)
      k_select_query<256, 4, true><<<g, 256, 0, s>>>(scores, n_cand, n_entries, cand_blocks, n_blocks, n_valid, k, gmax,
                                                     sp.n_groups, sp.group, cand, idx, top_scores);
    else if (Q >= kQSmallBatch)
      k_select_query<256, 4, false><<<g, 256, 0, s>>>(scores, n_cand, n_entries, nullptr, n_blocks, n_valid, k, gmax,
                                                      sp.n_groups, sp.group, cand, idx, top_scores);
    else if (pool)
      k_select_query<1024, 16, true><<<g, 1024, 0, s>>>(scores, n_cand, n_entries, cand_blocks, n_blocks, n_valid, k,
                                                        gmax, sp.n_groups, sp.group, cand, idx, top_scores);
    else
      k_select_query<1024, 4, false><<<g, 1024, 0, s>>>(scores, n_cand, n_entries, nullptr, n_blocks, n_valid, k,
                                                        gmax, sp.n_groups, sp.group, cand, idx, top_scores);
    return hipGetLastError();
  }
  hipError_t e = launch_select_compact(scores, Q, n_cand, n_entries, cand_blocks, n_blocks, n_valid, k, sp, gmax,
                                       counts, cand, s);
  if (e != hipSuccess) return e;
  SelectPlan pl = plan_select(n_cand);
  k_select_final<<<(unsigned)Q, NT, 0, s>>>(counts, pl.n_chunks, n_cand, k, cand, idx, top_scores);
  return hipGetLastError();
}

}  // namespace csa2
