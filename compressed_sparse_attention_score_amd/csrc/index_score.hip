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

namespace csa2 {

namespace {
constexpr int kUnroll = 4;  // 16-entry groups per load batch (two batches in flight per wave)
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
  float* scores;
  unsigned* gmax;
};
}  // namespace

// Position p of query q's candidate list -> entry id, or -1 when p is not a
// valid candidate (beyond the list, out-of-range block id, causal limit).
template <bool POOL>
__device__ __forceinline__ int64_t cand_entry(const ScoreArgs& a, int q, int64_t p, int64_t limit) {
  if (p >= a.n_cand) return -1;
  int64_t e;
  if (POOL) {
    int32_t b = a.cand_blocks[(int64_t)q * a.n_blocks + (p >> 3)];
    e = (b < 0) ? -1 : 8 * (int64_t)b + (p & 7);
  } else {
    e = p;
  }
  return (e >= 0 && e < limit) ? e : -1;
}

template <bool POOL, int UNROLL = kUnroll>
__global__ __launch_bounds__(256) void k_index_score(ScoreArgs a) {
  const int q = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kb = lane >> 4;
  // Scores and sub-chunk maxima are staged in LDS and written once per wave
  // after the loop, so the loop's only vector-memory operations are loads.
  __shared__ float s_score[4][kMaxWaveSpan];
  __shared__ unsigned s_gmax[4][kMaxWaveSpan / 16];

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

  const int64_t w0p = ((int64_t)blockIdx.x * 4 + wave) * a.wave_span;
  if (w0p >= a.n_cand) return;
  const int64_t w1p = min(w0p + a.wave_span, a.n_cand);
  unsigned gm = 0u;

  // Key loads run one batch of UNROLL groups ahead of the matrix cores (two
  // statically indexed buffers, alternated by a 2x unrolled loop). Loads are
  // unconditional so that the compiler keeps the second batch in flight:
  // lanes without a valid candidate read row 0 of their cache and are masked
  // at compute time.
  if (limit <= 0) {  // no valid candidate in this query's list
    for (int64_t p = w0p + lane; p < w1p; p += 64) out[p] = -__builtin_inff();
    if (a.gmax && lane == 0)
      for (int64_t g = w0p / a.group; g * a.group < w1p; ++g) a.gmax[(int64_t)q * a.n_groups + g] = 0u;
    return;
  }
  v4u bcA[UNROLL], bcB[UNROLL];
  unsigned bsA[UNROLL], bsB[UNROLL];
  bool okA[UNROLL], okB[UNROLL];
  auto issue = [&](v4u* bc, unsigned* bs, bool* ok, int64_t g0) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t p = g0 + 16 * u + r16;
      const int64_t e = (p < w1p) ? cand_entry<POOL>(a, q, p, limit) : -1;
      ok[u] = e >= 0;
      const int64_t row = base_row + (e >= 0 ? e : 0);
      bc[u] = __builtin_nontemporal_load((const v4u*)(a.key_codes + row * 64 + kb * 16));
      bs[u] = __builtin_nontemporal_load((const unsigned*)(a.key_scales + row * 4));
    }
  };
  auto compute = [&](const v4u* bc, const unsigned* bs, const bool* ok, int64_t g0) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t gp = g0 + 16 * u;
      if (gp >= w1p) break;
      const v4u c = ok[u] ? bc[u] : v4u{0u, 0u, 0u, 0u};
      const int sb = ok[u] ? (int)((bs[u] >> (8 * kb)) & 0xFFu) : 127;
      v8i B = {(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
      v4f c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
      c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, B, c0, 4, 4, 0, sa0, 0, sb);
      c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, B, c1, 4, 4, 0, sa1, 0, sb);
      float sc = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) sc = fmaf(w0[r], fmaxf(c0[r], 0.f), sc);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc = fmaf(w1[r], fmaxf(c1[r], 0.f), sc);
      sc = add_xor16(sc);
      sc = add_xor32(sc);
      // every lane now holds the score of entry r16 of this group
      if (kb == 0) s_score[wave][gp - w0p + r16] = ok[u] ? sc : -__builtin_inff();
      if (a.gmax) {
        gm = max(gm, ok[u] ? score_key(sc) : 0u);
        const int64_t gend = gp + 16;
        if ((gend & (a.group - 1)) == 0 || gend >= w1p) {
          unsigned v = gm;
          v = max(v, (unsigned)__shfl_xor((int)v, 1, 64));
          v = max(v, (unsigned)__shfl_xor((int)v, 2, 64));
          v = max(v, (unsigned)__shfl_xor((int)v, 4, 64));
          v = max(v, (unsigned)__shfl_xor((int)v, 8, 64));
          if (lane == 0) s_gmax[wave][(gp - w0p) / a.group] = v;
          gm = 0u;
        }
      }
    }
  };
  constexpr int64_t kStep = 16 * UNROLL;
  issue(bcA, bsA, okA, w0p);
  for (int64_t g0 = w0p; g0 < w1p; g0 += 2 * kStep) {
    if (g0 + kStep < w1p) issue(bcB, bsB, okB, g0 + kStep);
    compute(bcA, bsA, okA, g0);
    if (g0 + kStep >= w1p) break;
    if (g0 + 2 * kStep < w1p) issue(bcA, bsA, okA, g0 + 2 * kStep);
    compute(bcB, bsB, okB, g0 + kStep);
  }
  // flush this wave's staged scores and maxima (wave-private LDS rows)
  const int span = (int)(w1p - w0p);
  for (int i = lane; i < span; i += 64) out[w0p + i] = s_score[wave][i];
  if (a.gmax) {
    const int ng = (span + a.group - 1) / a.group;
    for (int i = lane; i < ng; i += 64) a.gmax[(int64_t)q * a.n_groups + w0p / a.group + i] = s_gmax[wave][i];
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
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, o, 64));
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
  int64_t g = floor_pow2(n_cand / (2 * (int64_t)(k > 0 ? k : 1)));
  if (g < 16) g = 16;
  if (g > W) g = W;
  p.group = (int)g;
  p.n_groups = (n_cand + g - 1) / g;
  p.n_wg = (int)((n_cand + 4 * (int64_t)W - 1) / (4 * (int64_t)W));
  return p;
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
  if (L.n_cand <= 0) return hipSuccess;
  dim3 grid((unsigned)plan.n_wg, (unsigned)L.Q);
  if (L.cand_blocks)
    k_index_score<true><<<grid, 256, 0, s>>>(a);
  else
    k_index_score<false><<<grid, 256, 0, s>>>(a);
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
