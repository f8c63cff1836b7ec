// Lightning-indexer scoring on gfx950 scaled-FP4 matrix cores.
//
// Method ("An infra-oriented diagram of the DeepSeek-V4.1-Flash architecture",
// Reading notes, indexer bullet): 32 FP4 query heads of 128 dims against one
// shared FP4 key per cache entry; the ReLU'd head scores are summed with
// per-head weights. Full layers score every entry; Reindex layers score a pool
// built from blocks of 8 entries.
//
// Mapping: one V_MFMA_SCALE_F32_16X16X128_F8F6F4 computes a full 128-dim dot
// product for 16 heads x 16 entries, with the E8M0 block scales applied by the
// matrix core (the format's native MX scaling). Lane l holds row/column l%16
// and the 32-channel block l/16 (16 bytes of codes plus that block's scale),
// which is exactly one stored scale block of a query head or key. The two
// MFMAs per 16 entries (heads 0-15 and 16-31) leave, in each lane, 8 head dots
// of one entry; ReLU and the weighted sum run in fp32 on the vector unit and
// two lane swaps finish the sum over heads. Keys stream from HBM once, in
// 1 KiB-per-wave contiguous loads.
#include "csa2_device.h"
#include "csa2_internal.h"

#include <type_traits>

namespace csa2 {

namespace {
constexpr int kUnroll = 4;  // 16-entry groups per load batch
constexpr int kScanRing = 2;  // load batches in flight per wave
// Plain ranges: the four waves of a workgroup take the 64-entry batches of
// its range in turn (wave w: batches w, w+4, ...), so that at any time they
// read one contiguous stretch of the cache; the scores meet in LDS. (This
// took about 2 us off the 4 x 1,048,576 decode scan; pools, whose rows are
// scattered anyway, keep one contiguous range per wave.)
constexpr bool kScanInterleave = true;
// Buffer resource word 3 for untyped dword access on gfx9-family parts, the
// nontemporal cache-policy bit of a buffer access, and an offset that is
// past every resource these kernels build (their sizes stay below 2 GiB).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;
constexpr unsigned kStoreDrop = 0x80000000u;
constexpr int kMaxWaveSpan = 512;  // entries per wave (the plan picks 64..512)

struct ScoreArgs {
  const uint8_t* key_codes;
  const uint8_t* key_scales;
  const uint8_t* iq_codes;
  const uint8_t* iq_scales;
  const float* w;
  const int32_t* cand_blocks;
  const int32_t* n_valid;
  int64_t n_entries, cache_q_stride, n_cand, n_groups;
  int n_blocks, Q, wave_span, group;
  // Placement of the workgroups on the XCDs (each run of 8 consecutive ids
  // goes round the 8 XCDs): qmaj set, a 1-D grid whose workgroups of query q
  // sit 8 ids apart from q & 7 on (n_wg per query), so the query's scores
  // stay in the L2 that its selection, attention and merge workgroups read
  // through; else xw > 0, the xw workgroups that score one compaction chunk
  // c share XCD c % 8, the compaction workgroup's.
  int xw, qmaj, n_wg;
  float* scores;
  unsigned* gmax;
};
}  // namespace

// Position p of a candidate list -> entry id, or -1 when p is not a valid
// candidate (beyond the list, out-of-range block id, causal limit). blk holds
// the block ids of the wave's range, from position p0 on (pools only).
template <bool POOL>
__device__ __forceinline__ int64_t cand_entry(const ScoreArgs& a, const int32_t* blk, int64_t p0, int64_t p,
                                              int64_t limit) {
  if (p >= a.n_cand) return -1;
  int64_t e;
  if (POOL) {
    const int32_t b = blk[(p - p0) >> 3];
    e = (b < 0) ? -1 : 8 * (int64_t)b + (p & 7);
  } else {
    e = p;
  }
  return (e >= 0 && e < limit) ? e : -1;
}

// BUF (plain ranges): the keys are read through buffer resources that span
// the workgroup's positions up to the query's last valid entry, so one
// 32-bit offset per lane, stepped by the batch, addresses every load (the
// group's 1 KiB and 64 B strides are instruction offsets) and the hardware
// returns zeros past the end instead of a clamped row. Pools (BUF false)
// take per-entry addresses and clamp to row 0.
// NB: batches of 64 entries per wave (the wave span is 64*NB); the batch
// loop is unrolled in full, so every wait names the exact load it needs.
template <bool POOL, bool BUF, int NB, int UNROLL = kUnroll>
__global__ __launch_bounds__(256) void k_index_score(ScoreArgs a) {
  static_assert(!(POOL && BUF), "pools take per-entry addresses");
  static_assert(NB >= 1 && 64 * NB <= kMaxWaveSpan, "wave span");
  static_assert(UNROLL == 4, "a batch is 64 entries: one staged score per lane");
  constexpr bool IL = kScanInterleave && !POOL;  // pools keep one range per wave
  int q = blockIdx.y, xb = blockIdx.x;  // query, workgroup within the query
  if (a.qmaj) {
    const int lin = blockIdx.x;
    q = ((lin / (8 * a.n_wg)) << 3) | (lin & 7);
    xb = (lin >> 3) % a.n_wg;
  } else if (a.xw > 0) {
    const int r = xb % (8 * a.xw);
    xb = xb - r + (r & 7) * a.xw + (r >> 3);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kb = lane >> 4;
  // Scores are staged in LDS and written once per wave after the loop, so the
  // loop's only vector-memory operations are loads; the sub-chunk maxima are
  // formed from the staged scores at that point.
  __shared__ __attribute__((aligned(16))) float s_score[4][kMaxWaveSpan];
  // A pool's block ids for the wave's range, read once: a key load then
  // waits on an LDS read instead of a global one.
  __shared__ int32_t s_blk[4][POOL ? kMaxWaveSpan / 8 : 1];

  // A operands: query heads r16 and 16+r16, scale block kb.
  const uint8_t* iqc = a.iq_codes + (int64_t)q * kIHeads * 64;
  const v4u qa0 = *(const v4u*)(iqc + r16 * 64 + kb * 16);
  const v4u qa1 = *(const v4u*)(iqc + (16 + r16) * 64 + kb * 16);
  const int sa0 = a.iq_scales[(int64_t)q * 128 + r16 * 4 + kb];
  const int sa1 = a.iq_scales[(int64_t)q * 128 + (16 + r16) * 4 + kb];
  v8i A0 = {(int)qa0[0], (int)qa0[1], (int)qa0[2], (int)qa0[3], 0, 0, 0, 0};
  v8i A1 = {(int)qa1[0], (int)qa1[1], (int)qa1[2], (int)qa1[3], 0, 0, 0, 0};
  // Output rows of this lane: heads 4*kb + r (first MFMA) and 16 + 4*kb + r.
  float w0[4], w1[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    w0[r] = a.w[q * kIHeads + 4 * kb + r];
    w1[r] = a.w[q * kIHeads + 16 + 4 * kb + r];
  }
  int64_t limit = a.n_entries;
  if (a.n_valid) limit = min(limit, (int64_t)a.n_valid[q]);
  const int64_t base_row = (int64_t)q * a.cache_q_stride;
  float* out = a.scores + (int64_t)q * a.n_cand;

  constexpr int kSpan = 64 * NB;  // entries per wave
  const int64_t wg0 = (int64_t)xb * 4 * kSpan;
  if (wg0 >= a.n_cand) return;  // uniform over the workgroup
  const int64_t wg1 = min(wg0 + 4 * kSpan, a.n_cand);
  // the wave's share of the scores to write and reduce: [w0p, w1p)
  const int64_t w0p = wg0 + (int64_t)wave * kSpan;
  const int64_t w1p = max(w0p, min(w0p + kSpan, a.n_cand));
  // the positions the wave scores: batch b at bpos(b), inside [r0, r1)
  const int64_t r0 = IL ? wg0 : w0p, r1 = IL ? wg1 : w1p;
  auto bpos = [&](int b) -> int64_t {
    return IL ? wg0 + (int64_t)(4 * b + wave) * 64 : w0p + (int64_t)b * 64;
  };
  // LDS rows: staged score of position p at s_flat[p - r0 + soff]; the
  // wave's share starts at s_flat[sown]
  float* s_flat = &s_score[0][0];
  const int soff = IL ? 0 : wave * kMaxWaveSpan;
  const int sown = IL ? wave * kSpan : wave * kMaxWaveSpan;

  // Key loads run kScanRing - 1 batches of UNROLL groups ahead of the matrix
  // cores (statically indexed buffers). Loads are unconditional so that the
  // compiler keeps the second batch in flight: lanes without a valid
  // candidate read nothing (buffer resources) or row 0 of their cache, and
  // are masked at compute time.
  if (limit <= 0) {  // no valid candidate in this query's list
    for (int64_t p = w0p + lane; p < w1p; p += 64) out[p] = -__builtin_inff();
    if (a.gmax && lane == 0)
      for (int64_t g = w0p / a.group; g * a.group < w1p; ++g) a.gmax[(int64_t)q * a.n_groups + g] = 0u;
    return;
  }
  int32_t* s_blkp = &s_blk[0][0] + wave * (kMaxWaveSpan / 8);
  if (POOL) {  // the range starts on a block boundary (spans are multiples of 64)
    const int nb = (int)((r1 - r0 + 7) >> 3);
    const int32_t* src = a.cand_blocks + (int64_t)q * a.n_blocks + (r0 >> 3);
    for (int i = lane; i < nb; i += 64) s_blkp[i] = src[i];
    // read back by other lanes of this wave only: its LDS accesses complete
    // in order, and this keeps the compiler from moving the reads above
    __builtin_amdgcn_wave_barrier();
  }
  v4u bcr[kScanRing][UNROLL];
  unsigned bsr[kScanRing][UNROLL];
  bool okr[kScanRing][UNROLL];
  __amdgpu_buffer_rsrc_t crs, srs;
  int64_t lim_w = 0;  // BUF: valid positions of the wave's range end here
  if constexpr (BUF) {
    // resources based at the start of this workgroup's positions, so that
    // their sizes and offsets stay small whatever the list length
    const int64_t lim = min(limit, a.n_cand);
    lim_w = min(lim, r1);
    const int nrec = (int)max((int64_t)0, lim_w - r0);  // valid positions from r0 on (at most 2,048)
    crs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.key_codes + (base_row + r0) * 64), 0, nrec * 64, kBufferWord3);
    srs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.key_scales + (base_row + r0) * 4), 0, nrec * 4, kBufferWord3);
  }
  auto issue = [&](v4u* bc, unsigned* bs, bool* ok, int64_t g0) {
    if constexpr (BUF) {
      // a batch past the range (the one the loop issues after its last)
      // reads nothing: its offsets are past every resource
      const unsigned p = (unsigned)(g0 - r0) + (unsigned)r16;
      const bool in = g0 < r1;
      const unsigned co = in ? 64u * p + 16u * (unsigned)kb : kStoreDrop;
      const unsigned so = in ? 4u * p : kStoreDrop;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        ok[u] = g0 + 16 * u + r16 < lim_w;
        bc[u] = __builtin_amdgcn_raw_buffer_load_b128(crs, (int)(co + 1024u * u), 0, kNonTemporal);
        bs[u] = __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(so + 64u * u), 0, kNonTemporal);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t p = g0 + 16 * u + r16;
      const int64_t e = (p < r1) ? cand_entry<POOL>(a, s_blkp, r0, p, limit) : -1;
      ok[u] = e >= 0;
      const int64_t row = base_row + (e >= 0 ? e : 0);
      bc[u] = __builtin_nontemporal_load((const v4u*)(a.key_codes + row * 64 + kb * 16));
      bs[u] = __builtin_nontemporal_load((const unsigned*)(a.key_scales + row * 4));
    }
  };
  // Both MFMAs of one 16-entry group. A lane without a valid candidate
  // holds the codes of a clamped row with a unit scale: FP4 codes are all
  // finite, each entry is its own MFMA column, and the column's score is
  // replaced by -inf below, so those bytes never reach a valid score.
  auto mfma2 = [&](const v4u& bcu, unsigned bsu, bool oku, v4f& c0, v4f& c1) {
    const int sb = oku ? (int)((bsu >> (8 * kb)) & 0xFFu) : 127;
    const v8i B = {(int)bcu[0], (int)bcu[1], (int)bcu[2], (int)bcu[3], 0, 0, 0, 0};
    c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, B, v4f{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, sa0, 0, sb);
    c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, B, v4f{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, sa1, 0, sb);
  };
  // One batch of UNROLL groups, software-pipelined: the MFMAs of group u+1
  // are issued before the vector epilogue of group u (the scheduling
  // barriers keep that order), so the matrix core and the vector unit work
  // at the same time. Groups past the wave's range are computed on masked
  // lanes and land in staging slots past the range, which the flush skips
  // (the range is a multiple of 64 entries except at the list end, and the
  // slots stay inside the wave's row).
  auto compute = [&](const v4u* bc, const unsigned* bs, const bool* ok, int64_t g0) {
    v4f c0, c1, n0, n1;
    float sv[UNROLL];
    mfma2(bc[0], bs[0], ok[0], c0, c1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (u + 1 < UNROLL) mfma2(bc[u + 1], bs[u + 1], ok[u + 1], n0, n1);
      __builtin_amdgcn_sched_barrier(0);
      float sc = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) sc = fmaf(w0[r], relu_bits(c0[r]), sc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc = fmaf(w1[r], relu_bits(c1[r]), sc);
      sc = add_xor16(sc);
      sc = add_xor32(sc);
      // every lane now holds the score of entry r16 of group u
      sv[u] = ok[u] ? sc : -__builtin_inff();
      __builtin_amdgcn_sched_barrier(0);
      c0 = n0;
      c1 = n1;
    }
    // lane (kb, r16) stages entry r16 of group kb: one conflict-free store
    float mine = sv[0];
#pragma unroll
    for (int u = 1; u < UNROLL; ++u) mine = (kb == u) ? sv[u] : mine;
    s_flat[soff + (int)(g0 - r0) + lane] = mine;
  };
  // Both batches are issued without conditions (a batch past the range is
  // masked: no bytes through the buffer resources, row 0 of the cache
  // otherwise), so that the wait before each group counts only the loads
  // issued after it and the other batch stays in flight meanwhile; a load
  // under a condition would make those waits cover both batches.
  // Each buffer is refilled right after its batch is computed. Batches past
  // the range (a wave at the list end) are computed on masked lanes too.
#pragma unroll
  for (int b = 0; b < kScanRing && b < NB; ++b) issue(bcr[b], bsr[b], okr[b], bpos(b));
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    constexpr int R = kScanRing;
    compute(bcr[b % R], bsr[b % R], okr[b % R], bpos(b));
    if (b + R < NB) issue(bcr[b % R], bsr[b % R], okr[b % R], bpos(b + R));
  }
  if (IL) __syncthreads();  // every wave's staged scores in LDS
  // flush this wave's share of the staged scores: 16-byte stores of 4 scores
  // when the row allows (config 4's isolated scan 50.8 -> 50.6 us, config
  // 1's 11.8 -> 11.6 us against one 4-byte store per score), then the tail
  const float* srow = s_flat + sown;
  const int span = (int)(w1p - w0p);
  {
    float* orow = out + w0p;
    int i0 = 0;
    if ((((uintptr_t)orow) & 15) == 0) {
      const int nv4 = span >> 2;
      for (int i = lane; i < nv4; i += 64) *(v4f*)(orow + 4 * i) = *(const v4f*)(srow + 4 * i);
      i0 = 4 * nv4;
    }
    for (int i = i0 + lane; i < span; i += 64) orow[i] = srow[i];
  }
  if (a.gmax) {
    // Sub-chunk maxima (sub-chunks of 4 to 512 entries start at multiples of
    // the group size, and so does the wave's range). In each pass over 256
    // staged scores lane l takes scores 4l..4l+3, and the group/4 lanes of a
    // sub-chunk reduce into its first lane; a 512-entry sub-chunk spans two
    // passes. Invalid entries
    // are -inf and a NaN score is passed over by the maximum, which can only
    // lower it and so keeps the selection bound valid. Order key 0 = empty.
    const int lpg = a.group >> 2;
    const int64_t grow = (int64_t)q * a.n_groups;
    float carry = -__builtin_inff();
    for (int base = 0; base < span; base += 256) {
      const int i = base + 4 * lane;
      float m = -__builtin_inff();
      if (i < span) {
        const v4f x = *(const v4f*)&srow[i];
        m = x[0];
#pragma unroll
        for (int e = 1; e < 4; ++e) m = (i + e < span) ? fmaxf(m, x[e]) : m;
      }
      if (lpg >= 2) m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, false)));  // lane ^ 1
      if (lpg >= 4) m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, false)));  // lane ^ 2
      // row rotations: the first lane of each 8- or 16-lane group collects it
      if (lpg >= 8) m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x124, 0xF, 0xF, false)));
      if (lpg >= 16) m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x128, 0xF, 0xF, false)));
      if (lpg >= 32) m = max_xor16(m);
      if (lpg >= 64) m = max_xor32(m);
      bool emit = true;
      if (lpg > 64) {  // 512-entry sub-chunk: finish it on its second pass (or at the range end)
        carry = fmaxf(carry, m);
        m = carry;
        emit = ((base + 256) & (a.group - 1)) == 0 || base + 256 >= span;
        if (emit) carry = -__builtin_inff();
      }
      const int first = (lpg > 64) ? base - (base & (a.group - 1)) : i;  // first score of the sub-chunk
      if (emit && (lane & (min(lpg, 64) - 1)) == 0 && i < span)
        a.gmax[grow + (w0p + first) / a.group] = (m == -__builtin_inff()) ? 0u : score_key(m);
    }
  }
}

// Many queries over one shared cache (a prefill chunk): the contraction is
// dense, so queries are tiled instead of streaming the keys once per query.
// MFMA rows are (query, head) pairs, 4 queries x 4 heads; the eight MFMAs of
// one 16-entry key block cover 32 heads of 4 queries, and the output layout
// (lane l holds rows 4*(l/16)..+3 of column l%16) leaves each lane with heads
// 4hb..4hb+3 of query l/16 for entry l%16. So ReLU and the weighted head sum
// stay inside the lane, with no cross-lane step. Each wave keeps 8 queries'
// operands and weights in registers; the workgroup walks an entry range in
// batches of 64 keys that all four waves share: each batch is loaded once,
// cooperatively, one batch ahead into registers and then into a
// double-buffered LDS stage (one barrier per batch), and every wave reads its
// B fragments from LDS (64 lanes read one contiguous 1 KiB). The range index
// runs fastest in the grid, so with a multiple of 8 ranges each XCD's L2
// serves 1/8 of the key cache.
namespace {
constexpr int kQSets = 2;  // 4-query sets per wave
constexpr int kTileUnroll = 4;  // 16-entry steps per load batch
}  // namespace

template <bool GMAX, int QSETS = kQSets, int BB = kTileUnroll>
__global__ __launch_bounds__(256) void k_index_score_qtile(ScoreArgs a, int range) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[2][BB * 16 * 64];
  __shared__ unsigned s_scl[2][BB * 16];
  constexpr int kQPerWave = 4 * QSETS;
  constexpr int kQPerWg = 4 * kQPerWave;
  // the wave index is uniform across the wave; saying so keeps the output
  // buffer resources in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kb = lane >> 4;
  const int q0 = blockIdx.y * kQPerWg + wave * kQPerWave;
  const int64_t e_begin = (int64_t)blockIdx.x * range;
  const int64_t e_end = min(e_begin + range, a.n_cand);
  // Every wave takes part in the batch loads and barriers below, also one
  // whose queries are past Q (its operands are zero and it stores nothing).
  if (e_begin >= e_end) return;

  // A operands: set s, head block hb -> row r16 = query q0+4s+r16/4, head 4hb+r16%4
  v8i A[QSETS][8];
  int sA[QSETS][8];
#pragma unroll
  for (int s = 0; s < QSETS; ++s) {
    const int qa = q0 + 4 * s + (r16 >> 2);
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
      const int h = 4 * hb + (r16 & 3);
      v4u c = v4u{0u, 0u, 0u, 0u};
      int sc = 127;
      if (qa < a.Q) {
        c = *(const v4u*)(a.iq_codes + ((int64_t)qa * kIHeads + h) * 64 + kb * 16);
        sc = a.iq_scales[((int64_t)qa * kIHeads + h) * 4 + kb];
      }
      A[s][hb] = v8i{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
      sA[s][hb] = sc;
    }
  }
  // this lane's output rows: query q0+4s+kb, heads 4hb+r. Positions inside
  // the range are 32-bit offsets from e_begin; the output row of set s is a
  // wave-uniform base plus kb*n_cand.
  const int span = (int)(e_end - e_begin);
  float wt[QSETS][32];
  int lim[QSETS];
  bool qok[QSETS];
  // Score stores go through a buffer resource per set whose base is the
  // set's first output row at e_begin (wave-uniform) and whose size is what
  // remains of the score array from there. A lane with nothing to store
  // passes an offset past that size and the hardware drops the store, so a
  // step has no branches and the scheduler can interleave its MFMAs with the
  // vector epilogue.
  __amdgpu_buffer_rsrc_t orsrc[QSETS];
#pragma unroll
  for (int s = 0; s < QSETS; ++s) {
    const int qo = q0 + 4 * s + kb;
    qok[s] = qo < a.Q;
#pragma unroll
    for (int h = 0; h < 32; ++h) wt[s][h] = qok[s] ? a.w[(int64_t)qo * kIHeads + h] : 0.f;
    int64_t l = a.n_entries;
    if (a.n_valid && qok[s]) l = min(l, (int64_t)a.n_valid[qo]);
    lim[s] = (int)max((int64_t)0, min(l - e_begin, (int64_t)span));
    const int64_t first = (int64_t)(q0 + 4 * s) * a.n_cand + e_begin;
    const int64_t room = max((int64_t)0, min((int64_t)a.Q * a.n_cand - first, (int64_t)kStoreDrop / 4 - 1));
    orsrc[s] = __builtin_amdgcn_make_buffer_rsrc(a.scores + first, 0, (int)(room * 4), kBufferWord3);
  }
  const unsigned orow_off = (unsigned)kb * (unsigned)a.n_cand + (unsigned)r16;
  // running maximum score of the current sub-chunk (invalid entries as -inf;
  // a NaN score can only lower it, which keeps the selection bound valid)
  const float ninf = -__builtin_inff();
  float gm[QSETS];
#pragma unroll
  for (int s = 0; s < QSETS; ++s) gm[s] = ninf;
  const int steps_per_group = a.group >> 4;
  int step_in_group = 0;
  int64_t gidx = e_begin / a.group;
  constexpr int kBatch = 16 * BB;  // entries per batch (compute() call)
  const bool batch_groups = a.group >= kBatch;
  // the sub-chunk maximum of each of this lane's query sets, over the 16
  // entries of its row group, to gmax[query][g]; then restart
  auto flush_max = [&](int64_t g) {
#pragma unroll
    for (int s = 0; s < QSETS; ++s) {
      const float m = row16_max(gm[s]);
      if (r16 == 0 && qok[s]) a.gmax[(int64_t)(q0 + 4 * s + kb) * a.n_groups + g] = (m == ninf) ? 0u : score_key(m);
      gm[s] = ninf;
    }
  };

  // cooperative batch loads: batch = BB*16 entries; thread t loads code chunks
  // t and t+256 (16 B each: entry c/4, quarter c%4) and, t < BB*16, one scale dword
  constexpr int kEnt = BB * 16;
  constexpr int kChunks = kEnt * 4;
  v4u pf[kChunks / 256];
  unsigned pfs = 0u;
  const int tid = threadIdx.x;
  auto gload = [&](int off0) {
#pragma unroll
    for (int i = 0; i < kChunks / 256; ++i) {
      const int c = tid + 256 * i;
      const int64_t e = e_begin + min(off0 + (c >> 2), span - 1);
      pf[i] = *(const v4u*)(a.key_codes + e * 64 + (c & 3) * 16);
    }
    if (tid < kEnt) {
      const int64_t e = e_begin + min(off0 + tid, span - 1);
      pfs = *(const unsigned*)(a.key_scales + e * 4);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < kChunks / 256; ++i) *(v4u*)(&s_codes[st][(tid + 256 * i) * 16]) = pf[i];
    if (tid < kEnt) s_scl[st][tid] = pfs;
  };
  auto compute = [&](int st, int off0) {
#pragma unroll
    for (int u = 0; u < BB; ++u) {
      const int off = off0 + 16 * u;
      if (off >= span) break;
      const v4u bc = *(const v4u*)(&s_codes[st][(16 * u + r16) * 64 + kb * 16]);
      const unsigned bs = s_scl[st][16 * u + r16];
      const v8i B = {(int)bc[0], (int)bc[1], (int)bc[2], (int)bc[3], 0, 0, 0, 0};
      const int sb = (int)((bs >> (8 * kb)) & 0xFFu);
      const int p = off + r16;
      const bool in_range = p < span;
      // Software pipeline: the MFMAs of head block hb+1 are issued before the
      // vector epilogue of block hb, so the matrix core and the vector unit
      // work at the same time within one wave.
      float acc[QSETS];
      v4f cur[QSETS], nxt[QSETS];
#pragma unroll
      for (int s = 0; s < QSETS; ++s) {
        acc[s] = 0.f;
        cur[s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[s][0], B, v4f{0.f, 0.f, 0.f, 0.f}, 4, 4, 0,
                                                                  sA[s][0], 0, sb);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hb = 0; hb < 8; ++hb) {
        if (hb + 1 < 8) {
#pragma unroll
          for (int s = 0; s < QSETS; ++s)
            nxt[s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[s][hb + 1], B, v4f{0.f, 0.f, 0.f, 0.f}, 4,
                                                                      4, 0, sA[s][hb + 1], 0, sb);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < QSETS; ++s)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[s] = fmaf(wt[s][4 * hb + r], relu_bits(cur[s][r]), acc[s]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < QSETS; ++s) cur[s] = nxt[s];
      }
#pragma unroll
      for (int s = 0; s < QSETS; ++s) {
        const float sv = (p < lim[s]) ? acc[s] : ninf;
        // scores stream out past L2 (the selection pass reads them much later)
        const unsigned boff = (qok[s] && in_range) ? 4u * (orow_off + (unsigned)off) : kStoreDrop;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv), orsrc[s], boff, 0, kNonTemporal);
        if (GMAX) gm[s] = fmaxf(gm[s], sv);  // lim <= span, so sv is -inf outside the range
      }
      if (GMAX && !batch_groups) {  // sub-chunks shorter than a batch: flushed by step
        ++step_in_group;
        if (step_in_group == steps_per_group || off + 16 >= span) {
          flush_max(gidx);
          step_in_group = 0;
          ++gidx;
        }
      }
    }
    // Sub-chunks of a batch or more (ranges start on sub-chunk boundaries):
    // flushed after the batch that ends one, outside the step loop, so that
    // no branch splits the steps' interleaved MFMA and vector work.
    if (GMAX && batch_groups && (((off0 + kBatch) & (a.group - 1)) == 0 || off0 + kBatch >= span))
      flush_max((e_begin + off0) / a.group);
  };
  constexpr int kStep = 16 * BB;
  gload(0);
  lstore(0);
  if (kStep < span) gload(kStep);
  int st = 0;
  for (int g0 = 0; g0 < span; g0 += kStep) {
    __syncthreads();  // stage st holds this batch; stage st^1 is free
    if (g0 + kStep < span) lstore(st ^ 1);
    if (g0 + 2 * kStep < span) gload(g0 + 2 * kStep);
    compute(st, g0);
    st ^= 1;
  }
}

// Sub-chunk maximum keys computed from an existing score array (standalone
// top-k). One wave per sub-chunk.
__global__ __launch_bounds__(256) void k_score_maxima(const float* __restrict__ scores, int Q, int64_t n_cand,
                                                      int64_t n_entries, const int32_t* __restrict__ cand_blocks,
                                                      int n_blocks, const int32_t* __restrict__ n_valid, int group,
                                                      int64_t n_groups, unsigned* __restrict__ gmax) {
  const int q = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gi = (int64_t)blockIdx.x * 4 + wave;
  if (gi >= n_groups) return;
  int64_t limit = n_entries;
  if (n_valid) limit = min(limit, (int64_t)n_valid[q]);
  unsigned m = 0u;
  const int64_t p0 = gi * group, p1 = min(p0 + group, n_cand);
  for (int64_t p = p0 + lane; p < p1; p += 64) {
    int64_t e = p;
    if (cand_blocks) {
      int32_t b = cand_blocks[(int64_t)q * n_blocks + (p >> 3)];
      e = (b < 0) ? -1 : 8 * (int64_t)b + (p & 7);
    }
    if (e >= 0 && e < limit) m = max(m, score_key(scores[(int64_t)q * n_cand + p]));
  }
  m = wave_umax(m);
  if (lane == 0) gmax[(int64_t)q * n_groups + gi] = m;
}

static int64_t floor_pow2(int64_t x) {
  int64_t p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

ScorePlan plan_score(int64_t n_cand, int Q, int k) {
  ScorePlan p;
  int W = 512;
  while (W > 64 && (int64_t)Q * ((n_cand + 4 * W - 1) / (4 * W)) < 1024) W /= 2;
  p.wave_span = W;
  // Sub-chunks of about n / 2k entries, so that at least k of them exist
  // and the threshold is informative; n / 4k for 1,024 queries or more,
  // whose selection reads only the sub-chunks that reach the threshold
  // (about k of them, so half the scores of n / 2k). The query-tiled scan
  // (32 queries or more over a shared cache) forms maxima per 16-entry step,
  // so there the smallest sub-chunk is 16; the per-query scan goes down to 4.
  const int64_t kk = k > 0 ? k : 1;
  int64_t g = floor_pow2(n_cand / ((Q >= 1024 ? 4 : 2) * kk));
  const int64_t gmin = (Q >= 16 * kQSets) ? 16 : 4;
  if (g < gmin) g = gmin;
  if (g > W) g = W;
  p.group = (int)g;
  p.n_groups = (n_cand + g - 1) / g;
  p.n_wg = (int)((n_cand + 4 * (int64_t)W - 1) / (4 * (int64_t)W));
  return p;
}

// The query-tiled kernel applies when all queries share one cache (prefill).
static bool use_query_tiles(const IndexLaunch& L) {
  // store offsets (up to 4 rows of 4-byte scores) stay below 2 GiB: 16*n_cand < 2^31
  return L.cache_q_stride == 0 && L.cand_blocks == nullptr && L.Q >= 16 * kQSets && L.n_cand < (1ll << 27);
}

hipError_t launch_index_score(const IndexLaunch& L, const ScorePlan& plan, float* scores, unsigned* gmax,
                              hipStream_t s) {
  if (L.Q <= 0) return hipSuccess;
  ScoreArgs a;
  a.key_codes = L.key_codes;
  a.key_scales = L.key_scales;
  a.iq_codes = L.iq_codes;
  a.iq_scales = L.iq_scales;
  a.w = L.w;
  a.cand_blocks = L.cand_blocks;
  a.n_valid = L.n_valid;
  a.n_entries = L.n_entries;
  a.cache_q_stride = L.cache_q_stride;
  a.n_cand = L.n_cand;
  a.n_groups = plan.n_groups;
  a.n_blocks = L.n_blocks;
  a.Q = L.Q;
  a.wave_span = plan.wave_span;
  a.group = plan.group;
  a.scores = scores;
  a.gmax = gmax;
  // XCD placement: query-major when the queries fill the 8 XCDs evenly;
  // otherwise by compaction chunk. (Config 1, 16 queries: 39.0 -> 38.2 us
  // per step with the compaction placed alike; config 4, 4 queries, by
  // chunk: 76.8 -> 75.3 us.)
  a.xw = 0;
  a.n_wg = plan.n_wg;
  a.qmaj = (L.Q % 8 == 0 && (int64_t)plan.n_wg * L.Q * 256 < ((int64_t)1 << 31)) ? 1 : 0;  // 1-D grid size
  if (!a.qmaj) {
    const int wpc = plan_select(L.n_cand).chunk / (4 * plan.wave_span);
    if (!L.cand_blocks && wpc >= 1 && plan.n_wg % (8 * wpc) == 0) a.xw = wpc;
  }
  if (L.n_cand <= 0) return hipSuccess;
  if (use_query_tiles(L)) {
    const int qb = (L.Q + 16 * kQSets - 1) / (16 * kQSets);
    const int64_t align = plan.group > 64 ? plan.group : 64;
    int64_t want = (2048 + qb - 1) / qb;
    want = (want + 7) / 8 * 8;
    int64_t range = (L.n_cand + want - 1) / want;
    range = (range + align - 1) / align * align;
    const int64_t n_ranges = (L.n_cand + range - 1) / range;
    const dim3 grid((unsigned)n_ranges, (unsigned)qb);
    if (gmax)
      k_index_score_qtile<true><<<grid, 256, 0, s>>>(a, (int)range);
    else
      k_index_score_qtile<false><<<grid, 256, 0, s>>>(a, (int)range);
    return hipGetLastError();
  }
  dim3 grid = a.qmaj ? dim3((unsigned)(plan.n_wg * L.Q)) : dim3((unsigned)plan.n_wg, (unsigned)L.Q);
  auto go = [&](auto nb_tag) {
    constexpr int NB = decltype(nb_tag)::value;
    if (L.cand_blocks)
      k_index_score<true, false, NB><<<grid, 256, 0, s>>>(a);
    else
      k_index_score<false, true, NB><<<grid, 256, 0, s>>>(a);
  };
  switch (plan.wave_span) {
    case 64: go(std::integral_constant<int, 1>{}); break;
    case 128: go(std::integral_constant<int, 2>{}); break;
    case 256: go(std::integral_constant<int, 4>{}); break;
    case 512: go(std::integral_constant<int, 8>{}); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_maxima(const float* scores, int Q, int64_t n_cand, int64_t n_entries,
                               const int32_t* cand_blocks, int n_blocks, const int32_t* n_valid,
                               const ScorePlan& plan, unsigned* gmax, hipStream_t s) {
  if (Q <= 0 || n_cand <= 0) return hipSuccess;
  dim3 grid((unsigned)((plan.n_groups + 3) / 4), (unsigned)Q);
  k_score_maxima<<<grid, 256, 0, s>>>(scores, Q, n_cand, n_entries, cand_blocks, n_blocks, n_valid, plan.group,
                                      plan.n_groups, gmax);
  return hipGetLastError();
}

}  // namespace csa2
