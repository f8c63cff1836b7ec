// Internal launch interface between the C-ABI front end (capi.hip) and the
// kernels. Host code only; every launcher enqueues on `stream` and returns the
// hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// Largest number of selected entries per query the kernels hold on chip
// (equal to CSA2_MAX_K; checked where the public header is included).
constexpr int kMaxSelected = 1024;

struct IndexLaunch {
  int Q;
  int64_t n_entries, cache_q_stride, n_cand;
  const uint8_t *key_codes, *key_scales, *iq_codes, *iq_scales;
  const float* w;
  const int32_t* cand_blocks;
  int n_blocks;
  const int32_t* n_valid;
};

// Work decomposition of the scoring pass, shared by the selection pass.
struct ScorePlan {
  int wave_span;    // entries per wave (power of two, multiple of 16)
  int group;        // sub-chunk size whose maximum key is recorded (4..wave_span)
  int64_t n_groups; // sub-chunks per query
  int n_wg;         // scoring workgroups per query
};
ScorePlan plan_score(int64_t n_cand, int Q, int k);

// Selection pass layout.
struct SelectPlan {
  int chunk;        // scores per selection workgroup
  int n_chunks;     // selection workgroups per query
};
SelectPlan plan_select(int64_t n_cand);

// Attention layout: the joint list in 32-slot tiles (window rows and
// selected latents tiled apart), split into n_splits ranges of
// tiles_per_split tiles per query.
struct AttnPlan {
  int n_tiles;
  int tiles_per_split;
  int n_splits;
};
AttnPlan plan_attn(int Q, int k_sel, int n_swa);

// Attention split plan bounds: a split launch holds at most kAttnTargetWgs
// (query, range) pairs, each with one partial record of kAttnPartialFloats
// floats (the 64 heads' maxima and sums, then their normalised outputs as
// bf16, written by the pair's two head-half workgroups), so no call's
// partials exceed kAttnPartialMaxBytes.
constexpr int kAttnTargetWgs = 128;
constexpr size_t kAttnPartialFloats = 2 * 64 + 64 * 512 / 2;
constexpr size_t kAttnPartialMaxBytes = (size_t)kAttnTargetWgs * kAttnPartialFloats * sizeof(float);

hipError_t launch_dequant(int kind, const uint8_t* codes, const uint8_t* scales, int64_t n, int out_bf16, void* out,
                          hipStream_t s);

// Quantise n fp32 (or bf16) rows into main entries (kind 0, cache [rows][288])
// or indexer keys (kind 1, codes [rows][64] + scales [rows][4]); row i goes to
// cache row rows[i] (i when rows == NULL), skipped outside [0, n_rows).
hipError_t launch_quantize(int kind, const void* x, int in_bf16, int64_t n, const int64_t* rows, int64_t n_rows,
                           uint8_t* codes, uint8_t* scales, hipStream_t s);

// m=2 pooling then main-entry quantisation: x [2n][512] fp32 token latents,
// gate [2n][gate_width] logits (gate_width 1 or 512); entry i pools rows 2i
// and 2i+1 and goes to cache row rows[i] (i when rows == NULL); pooled
// (optional) [n][512] receives the fp32 pooled rows.
hipError_t launch_pool_quantize(const float* x, const float* gate, int gate_width, int64_t n, const int64_t* rows,
                                int64_t n_rows, uint8_t* cache, float* pooled, hipStream_t s);

// Scores [Q][n_cand] and, if gmax != NULL, the maximum selection key of each
// sub-chunk [Q][plan.n_groups].
hipError_t launch_index_score(const IndexLaunch& a, const ScorePlan& plan, float* scores, unsigned* gmax,
                              hipStream_t s);

// Sub-chunk maxima straight from a score array (standalone top-k).
hipError_t launch_score_maxima(const float* scores, int Q, int64_t n_cand, int64_t n_entries,
                               const int32_t* cand_blocks, int n_blocks, const int32_t* n_valid,
                               const ScorePlan& plan, unsigned* gmax, hipStream_t s);

// Threshold + compaction kernel, then the exact selection kernel.
// counts: [Q][plan_select(n_cand).n_chunks]; cand: [Q][n_cand] composites.
hipError_t launch_select(const float* scores, int Q, int64_t n_cand, int64_t n_entries, const int32_t* cand_blocks,
                         int n_blocks, const int32_t* n_valid, int k, const ScorePlan& sp, const unsigned* gmax,
                         unsigned* counts, unsigned long long* cand, int32_t* idx, float* top_scores, hipStream_t s);

// Whether launch_select takes the chunk-parallel form (compaction, then a
// per-query final selection) for these sizes, and that form's compaction
// kernel alone (its final selection then runs inside the attention kernel).
bool select_is_chunked(int Q, int64_t n_cand);
hipError_t launch_select_compact(const float* scores, int Q, int64_t n_cand, int64_t n_entries,
                                 const int32_t* cand_blocks, int n_blocks, const int32_t* n_valid, int k,
                                 const ScorePlan& sp, const unsigned* gmax, unsigned* counts, unsigned long long* cand,
                                 hipStream_t s);

// Largest number of compaction chunks per query for which the attention
// kernel finishes the selection (one workgroup of that many threads).
constexpr int kFusedSelectMaxChunks = 256;

// Reindex pool construction: bmax [Q][ceil(n/8)] = best score of each block
// of 8 inside the causal limit (as a score whose key is the block's best
// key), nvb [Q] = blocks holding at least one valid entry.
hipError_t launch_block_max(const float* scores, int Q, int64_t n, const int32_t* n_valid, float* bmax, int32_t* nvb,
                            hipStream_t s);

// Dense copies out [Q][k][288] of the selected entries and dense ids [Q][k]
// (j for a valid id, -1 for a skipped one, whose slot is zeroed).
hipError_t launch_gather_selected(const uint8_t* cache, int64_t n_entries, int64_t cache_q_stride, const int32_t* idx,
                                  int Q, int k, uint8_t* out, int32_t* dense, hipStream_t s);

struct AttnLaunch {
  int Q;
  int64_t n_entries, cache_q_stride;
  const uint8_t* main_cache;
  const int32_t* idx;
  int k_sel;
  const uint16_t* q;
  const void* swa;  // bf16 rows [..][512], or FP8 rows [..][528] when swa_fp8
  int64_t swa_q_stride;
  int n_swa;
  float scale;
  uint16_t* out;
  float* lse;
  int swa_fp8;
  const float* rope;  // [Q][32][2] (cos, sin) or nullptr
  // Selection finished by the attention kernel (decode): the compaction's
  // counts [Q][sel_chunks] and composites [Q][sel_n_cand], or (sel_scores
  // given) the plain range's raw scores [Q][sel_n_cand] with the causal
  // limits sel_n_valid (or nullptr); with neither the ids are read from idx.
  // idx_out receives the ids (or nullptr).
  const unsigned* sel_counts;
  const unsigned long long* sel_cand;
  int64_t sel_n_cand;
  int sel_chunks, sel_chunk;
  int32_t* idx_out;
  const float* sel_scores;
  const int32_t* sel_n_valid;
};

// Longest plain candidate list whose selection the attention kernel makes
// straight from the scores (16 per thread).
constexpr int kRawSelectMax = 4096;

// partial: workspace for the per-range records (plan.n_splits > 1); the
// merge runs as a second kernel.
hipError_t launch_attn(const AttnLaunch& a, const AttnPlan& plan, float* partial, hipStream_t s);

size_t attn_partial_bytes(int Q, const AttnPlan& plan);

}  // namespace csa2
