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
constexpr int kUnroll = 4;  // 16-entry groups in flight per wave

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
  unsigned* ctrl;
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

template <bool POOL>
__global__ __launch_bounds__(256) void k_index_score(ScoreArgs a) {
  const int q = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kb = lane >> 4;

  if (a.ctrl && blockIdx.x == 0 && threadIdx.x < 3) a.ctrl[(int64_t)threadIdx.x * a.Q + q] = 0u;

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

  for (int64_t g0 = w0p; g0 < w1p; g0 += 16 * kUnroll) {
    v4u bc[kUnroll];
    int bs[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t p = g0 + 16 * u + r16;
      const int64_t e = (p < w1p) ? cand_entry<POOL>(a, q, p, limit) : -1;
      ok[u] = e >= 0;
      bc[u] = v4u{0u, 0u, 0u, 0u};
      bs[u] = 127;
      if (ok[u]) {
        const int64_t row = base_row + e;
        bc[u] = __builtin_nontemporal_load((const v4u*)(a.key_codes + row * 64 + kb * 16));
        bs[u] = (int)((__builtin_nontemporal_load((const unsigned*)(a.key_scales + row * 4)) >> (8 * kb)) & 0xFFu);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t gp = g0 + 16 * u;
      if (gp >= w1p) break;
      v8i B = {(int)bc[u][0], (int)bc[u][1], (int)bc[u][2], (int)bc[u][3], 0, 0, 0, 0};
      v4f c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
      c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, B, c0, 4, 4, 0, sa0, 0, bs[u]);
      c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, B, c1, 4, 4, 0, sa1, 0, bs[u]);
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) s = fmaf(w0[r], fmaxf(c0[r], 0.f), s);
#pragma unroll
      for (int r = 0; r < 4; ++r) s = fmaf(w1[r], fmaxf(c1[r], 0.f), s);
      s = add_xor16(s);
      s = add_xor32(s);
      // every lane now holds the score of entry r16 of this group
      const int64_t p = gp + r16;
      if (kb == 0 && p < w1p) out[p] = ok[u] ? s : -__builtin_inff();
      if (a.gmax) {
        gm = max(gm, ok[u] ? score_key(s) : 0u);
        const int64_t gend = gp + 16;
        if ((gend & (a.group - 1)) == 0 || gend >= w1p) {
          unsigned v = gm;
          v = max(v, (unsigned)__shfl_xor((int)v, 1, 64));
          v = max(v, (unsigned)__shfl_xor((int)v, 2, 64));
          v = max(v, (unsigned)__shfl_xor((int)v, 4, 64));
          v = max(v, (unsigned)__shfl_xor((int)v, 8, 64));
          if (lane == 0) a.gmax[(int64_t)q * a.n_groups + gp / a.group] = v;
          gm = 0u;
        }
      }
    }
  }
}

// Sub-chunk maximum keys computed from an existing score array (standalone
// top-k). One wave per sub-chunk.
__global__ __launch_bounds__(256) void k_score_maxima(const float* __restrict__ scores, int Q, int64_t n_cand,
                                                      int64_t n_entries, const int32_t* __restrict__ cand_blocks,
                                                      int n_blocks, const int32_t* __restrict__ n_valid, int group,
                                                      int64_t n_groups, unsigned* __restrict__ gmax,
                                                      unsigned* __restrict__ ctrl) {
  const int q = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (ctrl && blockIdx.x == 0 && threadIdx.x < 3) ctrl[(int64_t)threadIdx.x * Q + q] = 0u;
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
                              unsigned* ctrl, hipStream_t s) {
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
  a.ctrl = ctrl;
  if (L.n_cand <= 0) {
    if (ctrl) return launch_zero_u32(ctrl, 3 * (int64_t)L.Q, s);
    return hipSuccess;
  }
  dim3 grid((unsigned)plan.n_wg, (unsigned)L.Q);
  if (L.cand_blocks)
    k_index_score<true><<<grid, 256, 0, s>>>(a);
  else
    k_index_score<false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_score_maxima(const float* scores, int Q, int64_t n_cand, int64_t n_entries,
                               const int32_t* cand_blocks, int n_blocks, const int32_t* n_valid,
                               const ScorePlan& plan, unsigned* gmax, unsigned* ctrl, hipStream_t s) {
  if (Q <= 0) return hipSuccess;
  if (n_cand <= 0) return launch_zero_u32(ctrl, 3 * (int64_t)Q, s);
  dim3 grid((unsigned)((plan.n_groups + 3) / 4), (unsigned)Q);
  k_score_maxima<<<grid, 256, 0, s>>>(scores, Q, n_cand, n_entries, cand_blocks, n_blocks, n_valid, plan.group,
                                      plan.n_groups, gmax, ctrl);
  return hipGetLastError();
}

}  // namespace csa2
