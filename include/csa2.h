/*
 * csa2.h — C ABI of the CSA2 global-attention hot path on AMD Instinct MI355X
 * (gfx950): lightning-indexer scoring, top-k selection and sparse attention
 * over FP4 latents plus a sliding window.
 *
 * Source of the method: "An infra-oriented diagram of the DeepSeek-V4.1-Flash
 * architecture" (Reading notes: KV-latent bullet, Full-layer cache bullet,
 * indexer bullet, role bullet; section "The KV cache"), "DeepSeek V4.1 Flash:
 * Why Its Encoder, Engram and KV Cache Matter" (section "CSA2 makes long
 * context cheaper to retain") and the "DeepSeek V4.1 Flash" model guide
 * ("A closer look": shared KV -> candidate pool -> top 512 -> attention).
 *
 * Conventions for every entry point
 *  - All data pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors),
 *    C-contiguous, owned by the caller. The library allocates nothing, keeps no
 *    pointer after a call returns and holds no mutable global state (apart
 *    from the static device scratch of csa2_sparse_attn_noalloc, below); calls
 *    are thread-safe and reentrant.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued asynchronously on it; outputs are valid once it synchronises.
 *    A call only enqueues kernels (and the event records a caller asks for;
 *    no allocation, memset or synchronisation), so it can be captured in a
 *    HIP graph on that stream; replays reproduce the eager results bit for
 *    bit (csa2_decode is tested that way).
 *  - Arguments are validated on the host before anything is enqueued: a
 *    non-zero status means no work was launched. Data contents (NaN scores,
 *    unsorted block lists) are preconditions and are not checked on the host;
 *    kernels never read outside the buffers the arguments describe (selected
 *    ids outside [0, n_entries) are skipped, out-of-range block ids are treated
 *    as absent). Launch failures surface as CSA2_ERR_HIP.
 *  - Argument structs begin with `struct_size` (set it to sizeof the struct).
 *
 * Storage layouts (one "row" = one cache entry)
 *  main cache   uint8 [rows][288]: bytes 0..255 hold 512 FP4 E2M1 codes, byte j
 *               = channel 2j (low nibble) and 2j+1 (high nibble); bytes 256..287
 *               hold 32 E4M3 (OCP E4M3FN) scales, scale g for channels 16g..16g+15.
 *  index codes  uint8 [rows][64]: 128 FP4 E2M1 codes, same nibble order.
 *  index scales uint8 [rows][4]:  E8M0 scales, scale b for channels 32b..32b+31.
 *  Query i's cache is rows [i*cache_q_stride, i*cache_q_stride + n_entries)
 *  (cache_q_stride = n_entries for independent per-sequence caches, 0 for one
 *  cache shared by all queries, as in a prefill chunk). Entry ids returned and
 *  consumed by the library are relative to the query's cache.
 */
#ifndef CSA2_H_
#define CSA2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef CSA2_API
#define CSA2_API __attribute__((visibility("default")))
#endif

/* ---------------------------------------------------------------- status */
enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,      /* a required pointer is NULL                        */
  CSA2_ERR_SHAPE = 2,     /* unsupported size (k, counts, ranges)               */
  CSA2_ERR_ALIGN = 3,     /* a pointer is not aligned as documented             */
  CSA2_ERR_WORKSPACE = 4, /* workspace NULL or smaller than csa2_workspace_size */
  CSA2_ERR_HIP = 5,       /* a HIP launch or runtime call failed                */
  CSA2_ERR_ARG = 6,       /* struct_size mismatch or bad enum value             */
  CSA2_ERR_SCRATCH = 7    /* the call needs more than the library's static scratch */
};

/* Fixed shapes of the method ("An infra-oriented diagram ...", Reading notes). */
#define CSA2_MAIN_ENTRY_BYTES 288  /* 256 B codes + 32 E4M3 scales               */
#define CSA2_INDEX_CODE_BYTES 64   /* 128 FP4 codes                              */
#define CSA2_INDEX_SCALE_BYTES 4   /* 4 E8M0 scales                              */
#define CSA2_INDEX_HEADS 32        /* indexer query heads                        */
#define CSA2_INDEX_DIM 128         /* indexer head dim                           */
#define CSA2_HEADS 64              /* attention query heads                      */
#define CSA2_LATENT_DIM 512        /* shared k = v latent width                  */
#define CSA2_POOL_BLOCK 8          /* Reindex pools are built from blocks of 8   */
#define CSA2_MAX_K 1024            /* largest supported top-k                    */
#define CSA2_MAX_SWA 128           /* sliding-window rows per query              */
#define CSA2_SWA_FP8_ROW_BYTES 528 /* 512 E4M3 codes + 16 E8M0 scales            */
#define CSA2_ROPE_PAIRS 32         /* RoPE covers channels 448..511 in 32 pairs  */

/* ------------------------------------------------------------- dequant */
enum { CSA2_KIND_MAIN = 0, CSA2_KIND_INDEX = 1 };
enum { CSA2_OUT_F32 = 0, CSA2_OUT_BF16 = 1 };

/* csa2_dequant — decode stored entries to real values (FP4 E2M1 times its
 * block scale: E4M3 per 16 channels for main entries, E8M0 per 32 for indexer
 * keys; "An infra-oriented diagram ...", Full-layer cache bullet and "The KV
 * cache"). The result is the exact product (it fits both fp32 and bf16; E8M0
 * extremes may give fp32 subnormals or inf, NaN scale codes give NaN).
 *   kind      CSA2_KIND_MAIN:  codes = main cache [n][288], scales ignored;
 *                              out = [n][512].
 *             CSA2_KIND_INDEX: codes = [n][64], scales = [n][4]; out = [n][128].
 *   out_dtype CSA2_OUT_F32 (float) or CSA2_OUT_BF16 (bf16 bits, uint16).
 *   Alignment: codes and out 16 B; scales 4 B. n_entries >= 0 (0 = no-op). */
CSA2_API int csa2_dequant(int kind, const void* codes, const void* scales, int64_t n_entries, int out_dtype, void* out,
                 void* stream);

/* ------------------------------------------------------------ quantize */
enum { CSA2_IN_F32 = 0, CSA2_IN_BF16 = 1 };

/* csa2_quantize — write new cache entries: encode real rows into the stored
 * formats that csa2_dequant decodes ("An infra-oriented diagram ...",
 * Full-layer cache bullet and "The KV cache" fix the formats; the pages do not
 * give the rounding, which is fixed here as follows).
 *   main scale (per 16 channels): the E4M3FN value nearest to amax/6, ties to
 *     the even code, saturating at 448;
 *   index scale (per 32 channels): E8M0 2^e with e the smallest integer in
 *     [-127, 127] such that 6 * 2^e >= amax (byte 127, i.e. 2^0, when the
 *     block is all zero);
 *   element: the E2M1 magnitude nearest to |x| / scale, ties to the even code,
 *     saturating at 6, with the sign bit of x; every code of a block is 0 when
 *     its main scale is 0 or its index block is all zero.
 * NaN inputs count as zero magnitudes (keeping their sign bit), +-inf as the
 * largest. All decisions are exact (no rounded quotient takes part), so the
 * result is the nearest code, not an approximation of it.
 *   kind       CSA2_KIND_MAIN:  x = [n][512]; codes = main cache [n_cache_rows][288];
 *                               scales ignored.
 *              CSA2_KIND_INDEX: x = [n][128]; codes = [n_cache_rows][64],
 *                               scales = [n_cache_rows][4].
 *   in_dtype   CSA2_IN_F32 (float, 16-B aligned) or CSA2_IN_BF16 (bf16 bits, 8-B aligned).
 *   dst_rows   [n] int64 cache row of each input row (8-B aligned), or NULL for
 *              row i -> cache row i (then n_cache_rows >= n). Rows outside
 *              [0, n_cache_rows) are skipped; duplicate rows race.
 *   Alignment: codes 16 B, scales 4 B. n_entries >= 0 (0 = no-op). */
CSA2_API int csa2_quantize(int kind, const void* x, int in_dtype, int64_t n_entries, const int64_t* dst_rows,
                           int64_t n_cache_rows, void* codes, void* scales, void* stream);

/* csa2_pool_quantize — the encoder's cache write: m=2 pooling then the main
 * entry encoding of csa2_quantize ("An infra-oriented diagram ...",
 * Full-layer cache bullet: in the encoder two consecutive tokens are pooled
 * into one entry with a learned softmax gate). Entry i is
 *     p * x[2i] + (1 - p) * x[2i+1],  p = 1 / (1 + exp(g[2i+1] - g[2i])),
 * the two-way softmax of the pair's gate logits, per channel (gate_width
 * 512) or once per token (gate_width 1); the logits come from the caller
 * (their projection needs trained weights). Computed in fp32 (exp to about an ulp),
 * then encoded exactly as csa2_quantize encodes that fp32 row.
 *   x          [2n][512] fp32 token latents, 16-B aligned
 *   gate       [2n][gate_width] fp32 logits, 16-B (512) or 4-B (1) aligned
 *   dst_rows / n_cache_rows / cache   as csa2_quantize (CSA2_KIND_MAIN)
 *   pooled     [n][512] fp32 out (the pooled rows, for the index-key
 *              projection), 16-B aligned, or NULL
 * n_entries = n >= 0 (0 = no-op). */
CSA2_API int csa2_pool_quantize(const float* x, const float* gate, int gate_width, int64_t n_entries,
                                const int64_t* dst_rows, int64_t n_cache_rows, void* cache, float* pooled,
                                void* stream);

/* ---------------------------------------------------- pool construction */
#define CSA2_MAX_POOL_BLOCKS 8192  /* largest pool, in blocks of 8 (the method: 2048) */

typedef struct csa2_pool_args {
  size_t struct_size;
  int32_t n_queries;          /* Q >= 0                                          */
  int64_t n_entries;          /* scores per query (the whole cache), < 2^31      */
  const float* scores;        /* [Q][n_entries] a Full layer's indexer scores, 4-B aligned */
  const int32_t* n_valid;     /* [Q] causal limit (entries >= n_valid[q] ignored) or NULL */
  int32_t n_pool_blocks;      /* blocks to keep, 1..CSA2_MAX_POOL_BLOCKS          */
  int32_t* pool_blocks;       /* out [Q][n_pool_blocks], 4-B aligned             */
} csa2_pool_args;

/* csa2_build_pool — the candidate pool of the Reindex layers ("An
 * infra-oriented diagram ...", indexer bullet: a 16,384-entry pool chosen by
 * layer 20 by blocks of 8; "DeepSeek V4.1 Flash: Why Its Encoder, Engram and
 * KV Cache Matter", CSA2 section: a hierarchical index narrows later searches
 * to a pool chosen earlier). The pages do not give the block ranking; here
 * block b (entries 8b..8b+7) scores the best of its entries below the causal
 * limit, in the csa2_topk order (NaN lowest, -0 == +0), and the
 * n_pool_blocks best blocks by (block score descending, block id ascending)
 * are written in ascending block id, -1 padded when fewer blocks hold a valid
 * entry: exactly the cand_blocks input of a Reindex csa2_index_score.
 * Workspace: csa2_workspace_size(CSA2_WS_POOL, args) bytes, 256-B aligned. */
CSA2_API int csa2_build_pool(const csa2_pool_args* args, void* workspace, size_t ws_bytes, void* stream);

/* --------------------------------------------------------- index score */
typedef struct csa2_index_args {
  size_t struct_size;
  int32_t n_queries;          /* Q >= 0                                         */
  int64_t n_entries;          /* entries per query cache, 0 <= N < 2^31         */
  int64_t cache_q_stride;     /* rows between consecutive queries' caches       */
  const uint8_t* key_codes;   /* [rows][64]   16-B aligned                       */
  const uint8_t* key_scales;  /* [rows][4]    4-B aligned                        */
  const uint8_t* iq_codes;    /* [Q][32][64]  indexer query, MXFP4, 16-B aligned */
  const uint8_t* iq_scales;   /* [Q][32][4]   E8M0, 4-B aligned                  */
  const float* head_weights;  /* [Q][32]      per-head weights                   */
  const int32_t* cand_blocks; /* [Q][n_blocks] Reindex pool block ids, or NULL  */
  int32_t n_blocks;           /* pool blocks per query (0 when cand_blocks NULL) */
  const int32_t* n_valid;     /* [Q] causal limit (ids >= n_valid[q] excluded) or NULL */
} csa2_index_args;

/* csa2_index_score — lightning-indexer scores ("An infra-oriented diagram ...",
 * indexer bullet): for query q and candidate entry e,
 *     score = sum_{h<32} w[q][h] * max(0, iq_h . key_e)
 * over 32 MXFP4 heads of 128 dims against the entry's one shared MXFP4 key.
 * Candidates (Full layer, "search the full sparse index"): entries 0..N-1;
 * (Reindex layer, pool of blocks of 8): position p -> entry
 * 8*cand_blocks[q][p/8] + p%8, with block ids ascending and distinct
 * (precondition). Entries outside [0, min(N, n_valid[q])) score -inf.
 *   scores: [Q][n_cand] float, n_cand = N (Full) or 8*n_blocks (Reindex); 4-B aligned.
 * The dot products are exact (FP4 products, power-of-two scales); the weighted
 * sum is accumulated in fp32. */
CSA2_API int csa2_index_score(const csa2_index_args* args, float* scores, void* stream);

/* ---------------------------------------------------------------- topk */
typedef struct csa2_topk_args {
  size_t struct_size;
  int32_t n_queries;          /* Q >= 0                                          */
  int64_t n_cand;             /* scores per query, < 2^31                        */
  int64_t n_entries;          /* cache size; candidate ids >= n_entries excluded */
  const float* scores;        /* [Q][n_cand]                                     */
  const int32_t* cand_blocks; /* [Q][n_blocks] or NULL (then id = position)      */
  int32_t n_blocks;           /* n_cand == 8*n_blocks when cand_blocks != NULL   */
  const int32_t* n_valid;     /* [Q] causal limit or NULL                        */
  int32_t k;                  /* 1 <= k <= CSA2_MAX_K (the method uses 512)      */
  int32_t* idx;               /* out [Q][k] entry ids, -1 padded                 */
  float* top_scores;          /* out [Q][k] scores (-inf padded), or NULL        */
} csa2_topk_args;

/* csa2_topk — per-query top-k of the candidate scores ("DeepSeek V4.1 Flash"
 * guide, "A closer look": main sparse selection of 512 entries). The k best
 * candidates by (score descending, entry id ascending) are kept: equal scores
 * go to the lower id, -0 equals +0, NaN ranks below every number. The kept set
 * is written in ascending entry id (the selection fixes a set, not an order);
 * top_scores[q][j] is the score of idx[q][j], as ranked: a selected -0 is
 * reported as +0, the two being one value for the ranking; a selected NaN is
 * reported as the quiet NaN 0x7FC00000. When fewer than k candidates are
 * valid the tail is -1 / -inf. Needs a workspace of
 * csa2_workspace_size(CSA2_WS_TOPK, args) bytes, 256-B aligned, contents
 * ignored on entry. */
CSA2_API int csa2_topk(const csa2_topk_args* args, void* workspace, size_t ws_bytes, void* stream);

/* --------------------------------------------------------- sparse attn */
typedef struct csa2_attn_args {
  size_t struct_size;
  int32_t n_queries;          /* Q >= 0                                          */
  int64_t n_entries;          /* entries per query cache                         */
  int64_t cache_q_stride;     /* rows between consecutive queries' caches        */
  const uint8_t* main_cache;  /* [rows][288], 16-B aligned                       */
  const int32_t* idx;         /* [Q][k_sel] selected ids; ids outside [0,N) skipped */
  int32_t k_sel;              /* 0 <= k_sel <= CSA2_MAX_K                        */
  const uint16_t* q;          /* [Q][64][512] bf16, 16-B aligned                 */
  const void* swa;            /* window rows, 16-B aligned (NULL iff n_swa == 0): bf16 [..][512]
                                 or FP8 [..][528], as swa_format says          */
  int64_t swa_q_stride;       /* query i's window = rows i*swa_q_stride + 0..n_swa-1 */
  int32_t n_swa;              /* 0 <= n_swa <= 128                               */
  float softmax_scale;        /* e.g. 1/sqrt(512)                                */
  uint16_t* out;              /* out [Q][64][512] bf16, 16-B aligned             */
  float* lse;                 /* out [Q][64] natural-log sum-exp of scaled logits, or NULL */
  int32_t swa_format;         /* CSA2_SWA_BF16 or CSA2_SWA_FP8                   */
  const float* rope_cos_sin;  /* [Q][32][2] (cos, sin) of each query's RoPE angles, 8-B
                                 aligned, or NULL: no un-rotation of the output */
} csa2_attn_args;

/* Window row formats. The pages give the window cache as 128 entries of 528
 * FP8 bytes ("An infra-oriented diagram ...", "The KV cache") without its
 * scale layout; CSA2_SWA_FP8 reads it as OCP MXFP8: bytes 0..511 are E4M3FN
 * codes of channels 0..511, bytes 512..527 are E8M0 scales, scale b for
 * channels 32b..32b+31; value = E4M3(code) * 2^(scale - 127). */
enum { CSA2_SWA_BF16 = 0, CSA2_SWA_FP8 = 1 };

/* csa2_sparse_attn — attention of 64 query heads over one shared k = v latent
 * per entry ("An infra-oriented diagram ...", KV-latent bullet), for the joint
 * set J = selected entries (in idx order) followed by the n_swa window rows
 * (role bullet: the 128-token window plus 512 selected entries):
 *     o_h = sum_{j in J} softmax_j(scale * q_h . x_j) x_j
 * with x_j the dequantised latent (exact in bf16) or the window row (bf16, or
 * FP8 decoded exactly to bf16 while the scaled value stays in bf16's normal
 * range). bf16 matrix-core products, fp32 accumulation and softmax, bf16
 * output. An empty J gives zeros and lse = -inf. Also the whole path of a
 * Reuse layer (given ids) and of an SWA-only layer (k_sel = 0).
 * RoPE un-rotation (KV-latent bullet: RoPE touches 64 of the 512 dims and is
 * un-rotated on the attention output): with rope_cos_sin set, channels
 * 448 + 2i and 449 + 2i of every head's normalised output (a, b) become
 * (a c + b s, b c - a s) with (c, s) = rope_cos_sin[q][i], i < 32, before
 * the bf16 rounding; lse is unchanged. Workspace:
 * csa2_workspace_size(CSA2_WS_ATTN, args) bytes, 256-B aligned. */
CSA2_API int csa2_sparse_attn(const csa2_attn_args* args, void* workspace, size_t ws_bytes, void* stream);

/* csa2_sparse_attn_noalloc — csa2_sparse_attn for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, results and kernels, no workspace: the
 * partial records of small batches (the only scratch csa2_sparse_attn uses)
 * go to a device array the library holds on every GPU it runs on, of
 * CSA2_ATTN_SCRATCH_BYTES, until the process ends. Any valid args fit in it
 * (a split launch has at most 128 partial records of 66,048 B); a call that
 * would need more returns CSA2_ERR_SCRATCH before any work is enqueued. The
 * call allocates nothing; the array's address on the current device is
 * looked up once per device (hipGetSymbolAddress) on the first call there,
 * so the stream must belong to the current device. Calls that overlap on one
 * GPU (several streams, or host threads) share the array and race; the array
 * keeps the last call's contents, and every record a call reads it wrote
 * itself. */
#define CSA2_ATTN_SCRATCH_BYTES 8454144
CSA2_API int csa2_sparse_attn_noalloc(const csa2_attn_args* args, void* stream);

/* csa2_gather_selected — for the Reuse layers, which share the global KV and
 * the selected positions of an earlier layer ("DeepSeek V4.1 Flash: Why Its
 * Encoder, Engram and KV Cache Matter", CSA2 section): copy each query's
 * selected main entries once into a dense list, so that every later layer
 * attends over contiguous rows.
 *   main_cache, n_entries, cache_q_stride, idx [Q][k_sel]: as csa2_attn_args
 *   out        [Q][k_sel][288], 16-B aligned: slot j = entry idx[q][j], or
 *              zeros when that id is skipped (outside [0, n_entries))
 *   dense_idx  [Q][k_sel] out: j, or -1 for a skipped id
 * csa2_sparse_attn with main_cache = out, n_entries = cache_q_stride = k_sel
 * and idx = dense_idx gives the same result as over the original cache. */
CSA2_API int csa2_gather_selected(const uint8_t* main_cache, int64_t n_entries, int64_t cache_q_stride,
                                  const int32_t* idx, int32_t n_queries, int32_t k_sel, uint8_t* out,
                                  int32_t* dense_idx, void* stream);

/* -------------------------------------------------------- fused decode */
typedef struct csa2_decode_args {
  size_t struct_size;
  csa2_index_args index;      /* struct_size inside must also be set             */
  int32_t k;                  /* top-k, 1..CSA2_MAX_K                            */
  const uint8_t* main_cache;  /* [rows][288], same row indexing as the keys      */
  const uint16_t* q;          /* [Q][64][512] bf16                               */
  const void* swa;            /* window rows, format swa_format                  */
  int64_t swa_q_stride;
  int32_t n_swa;
  float softmax_scale;
  uint16_t* out;              /* out [Q][64][512] bf16                           */
  float* lse;                 /* out [Q][64] or NULL                             */
  int32_t* idx_out;           /* out [Q][k] selected ids, or NULL                */
  void* stage_events[4];      /* optional hipEvent_t (as void*) recorded on the stream
                                 before scoring [0], after scoring [1], after the
                                 selection kernels that precede attention [2]
                                 and after attention [3]; NULL = skip. For few
                                 long lists the last selection step runs inside
                                 the attention kernel, and for few short plain
                                 lists (< 64 queries, <= 4,096 candidates) the
                                 whole selection does, so [2]..[3] includes it. */
  int32_t swa_format;         /* CSA2_SWA_BF16 or CSA2_SWA_FP8                   */
  const float* rope_cos_sin;  /* [Q][32][2] or NULL, as in csa2_attn_args        */
} csa2_decode_args;

/* csa2_decode — the whole path for one batch: csa2_index_score ->
 * csa2_topk -> csa2_sparse_attn ("DeepSeek V4.1 Flash" guide: shared KV ->
 * candidate pool -> top 512 -> attention), enqueued back to back with
 * no host round trip; scores and ids live in the workspace. Same results as
 * the three calls in sequence. Workspace: csa2_workspace_size(CSA2_WS_DECODE,
 * args) bytes, 256-B aligned. */
CSA2_API int csa2_decode(const csa2_decode_args* args, void* workspace, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------- utilities */
enum { CSA2_WS_TOPK = 0, CSA2_WS_ATTN = 1, CSA2_WS_DECODE = 2, CSA2_WS_POOL = 3 };

/* Bytes of workspace the call `which` needs for `args` (a csa2_topk_args*,
 * csa2_attn_args*, csa2_decode_args* or csa2_pool_args*); 0 if none;
 * SIZE_MAX if the args are invalid. */
CSA2_API size_t csa2_workspace_size(int which, const void* args);

/* Static, human-readable text for a status code. */
CSA2_API const char* csa2_status_string(int status);

/* ABI version of this header (major*10000 + minor*100 + patch). */
CSA2_API int csa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H_ */
