// C-ABI front end: argument validation (host-side, before any launch),
// workspace layout and the launch sequence of every entry point in csa2.h.
#include "../../include/csa2.h"
#include "csa2_internal.h"

static_assert(CSA2_MAX_K == csa2::kMaxSelected, "on-chip selected-id capacity must match the ABI limit");
static_assert(CSA2_ATTN_SCRATCH_BYTES == csa2::kAttnPartialMaxBytes, "static scratch must hold the largest partials");

// Device scratch of csa2_sparse_attn_noalloc (the attention partials), one
// copy per GPU, held until the process ends. Host code never uses this name
// as an address: it passes the address hipGetSymbolAddress returns for the
// current device (scratch_on_current_device below).
static __device__ __align__(256) unsigned char scratch[CSA2_ATTN_SCRATCH_BYTES];

#include <limits.h>
#include <stdint.h>

#include <atomic>

using namespace csa2;

namespace {

constexpr int64_t kMaxI32 = 2147483647LL;
constexpr int kMaxQ = 65535;  // grid.y limit

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carve {  // bump allocator over the caller's workspace
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off = up256(off + count * sizeof(T));
    return p;
  }
};

int check_index(const csa2_index_args* a, int64_t* n_cand_out) {
  if (!a) return CSA2_ERR_NULL;
  if (a->struct_size != sizeof(csa2_index_args)) return CSA2_ERR_ARG;
  if (a->n_queries < 0 || a->n_queries > kMaxQ) return CSA2_ERR_SHAPE;
  if (a->n_entries < 0 || a->n_entries > kMaxI32 || a->cache_q_stride < 0) return CSA2_ERR_SHAPE;
  int64_t n_cand = a->n_entries;
  if (a->cand_blocks) {
    if (a->n_blocks < 0 || 8LL * a->n_blocks > kMaxI32) return CSA2_ERR_SHAPE;
    n_cand = 8LL * a->n_blocks;
  } else if (a->n_blocks != 0) {
    return CSA2_ERR_SHAPE;
  }
  *n_cand_out = n_cand;
  if (a->n_queries == 0) return CSA2_OK;
  if (!a->iq_codes || !a->iq_scales || !a->head_weights) return CSA2_ERR_NULL;
  if (a->n_entries > 0 && n_cand > 0 && (!a->key_codes || !a->key_scales)) return CSA2_ERR_NULL;
  if (!aligned(a->key_codes, 16) || !aligned(a->iq_codes, 16) || !aligned(a->key_scales, 4) ||
      !aligned(a->iq_scales, 4) || !aligned(a->head_weights, 4) || !aligned(a->cand_blocks, 4) ||
      !aligned(a->n_valid, 4))
    return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

int check_topk(const csa2_topk_args* a) {
  if (!a) return CSA2_ERR_NULL;
  if (a->struct_size != sizeof(csa2_topk_args)) return CSA2_ERR_ARG;
  if (a->n_queries < 0 || a->n_queries > kMaxQ) return CSA2_ERR_SHAPE;
  if (a->k < 1 || a->k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (a->n_cand < 0 || a->n_cand > kMaxI32 || a->n_entries < 0 || a->n_entries > kMaxI32) return CSA2_ERR_SHAPE;
  if (a->cand_blocks) {
    if (a->n_blocks < 0 || 8LL * a->n_blocks != a->n_cand) return CSA2_ERR_SHAPE;
  } else if (a->n_blocks != 0) {
    return CSA2_ERR_SHAPE;
  }
  if (a->n_queries == 0) return CSA2_OK;
  if (!a->idx || (a->n_cand > 0 && !a->scores)) return CSA2_ERR_NULL;
  if (!aligned(a->scores, 4) || !aligned(a->idx, 4) || !aligned(a->top_scores, 4) || !aligned(a->cand_blocks, 4) ||
      !aligned(a->n_valid, 4))
    return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

int check_attn_fields(int Q, int64_t n_entries, int64_t cache_q_stride, const uint8_t* main_cache,
                      const int32_t* idx, int k_sel, const uint16_t* q, const void* swa, int64_t swa_q_stride,
                      int n_swa, const uint16_t* out, const float* lse, int swa_format, const float* rope,
                      bool idx_internal) {
  if (swa_format != CSA2_SWA_BF16 && swa_format != CSA2_SWA_FP8) return CSA2_ERR_ARG;
  if (Q < 0 || Q > kMaxQ) return CSA2_ERR_SHAPE;
  if (n_entries < 0 || n_entries > kMaxI32 || cache_q_stride < 0) return CSA2_ERR_SHAPE;
  if (k_sel < 0 || k_sel > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (n_swa < 0 || n_swa > CSA2_MAX_SWA || swa_q_stride < 0) return CSA2_ERR_SHAPE;
  if (Q == 0) return CSA2_OK;
  if (!q || !out) return CSA2_ERR_NULL;
  if (k_sel > 0 && ((!idx && !idx_internal) || (n_entries > 0 && !main_cache))) return CSA2_ERR_NULL;
  if (n_swa > 0 && !swa) return CSA2_ERR_NULL;
  if (!aligned(main_cache, 16) || !aligned(q, 16) || !aligned(swa, 16) || !aligned(out, 16) || !aligned(idx, 4) ||
      !aligned(lse, 4) || !aligned(rope, 8))
    return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

int check_attn(const csa2_attn_args* a) {
  if (!a) return CSA2_ERR_NULL;
  if (a->struct_size != sizeof(csa2_attn_args)) return CSA2_ERR_ARG;
  return check_attn_fields(a->n_queries, a->n_entries, a->cache_q_stride, a->main_cache, a->idx, a->k_sel, a->q,
                           a->swa, a->swa_q_stride, a->n_swa, a->out, a->lse, a->swa_format, a->rope_cos_sin, false);
}

int check_decode(const csa2_decode_args* a, int64_t* n_cand) {
  if (!a) return CSA2_ERR_NULL;
  if (a->struct_size != sizeof(csa2_decode_args)) return CSA2_ERR_ARG;
  int st = check_index(&a->index, n_cand);
  if (st) return st;
  if (a->k < 1 || a->k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  st = check_attn_fields(a->index.n_queries, a->index.n_entries, a->index.cache_q_stride, a->main_cache, a->idx_out,
                         a->k, a->q, a->swa, a->swa_q_stride, a->n_swa, a->out, a->lse, a->swa_format,
                         a->rope_cos_sin, true);
  if (st) return st;
  if (!aligned(a->idx_out, 4)) return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

// Workspace layouts (each region 256-byte aligned).
struct TopkWs {
  unsigned* counts;          // [Q][n_chunks] candidates kept per compaction chunk
  unsigned* gmax;            // [Q][n_groups] sub-chunk maximum keys
  unsigned long long* cand;  // [Q][n_cand] kept composites
  size_t bytes;
};

TopkWs carve_topk(void* ws, int Q, int64_t n_cand, const ScorePlan& sp, Carve& c) {
  TopkWs w;
  w.counts = c.take<unsigned>((size_t)Q * (size_t)plan_select(n_cand).n_chunks);
  w.gmax = c.take<unsigned>((size_t)Q * (size_t)(sp.n_groups > 0 ? sp.n_groups : 1));
  w.cand = c.take<unsigned long long>((size_t)Q * (size_t)(n_cand > 0 ? n_cand : 1));
  w.bytes = c.off;
  (void)ws;
  return w;
}

size_t ws_topk(const csa2_topk_args* a) {
  if (a->n_queries == 0) return 0;
  ScorePlan sp = plan_score(a->n_cand, a->n_queries, a->k);
  Carve c(nullptr);
  return carve_topk(nullptr, a->n_queries, a->n_cand, sp, c).bytes;
}

// Pool construction: block scores, valid-block counts, then a top-k workspace
// over the blocks.
struct PoolWs {
  float* bmax;    // [Q][nb]
  int32_t* nvb;   // [Q]
  TopkWs tk;
  size_t bytes;
};

PoolWs carve_pool(void* ws, int Q, int64_t n_entries, int n_pool) {
  const int64_t nb = (n_entries + 7) / 8;
  ScorePlan sp = plan_score(nb, Q, n_pool);
  Carve c(ws);
  PoolWs w;
  w.bmax = c.take<float>((size_t)Q * (size_t)(nb > 0 ? nb : 1));
  w.nvb = c.take<int32_t>((size_t)Q);
  w.tk = carve_topk(ws, Q, nb, sp, c);
  w.bytes = c.off;
  return w;
}

int check_pool(const csa2_pool_args* a) {
  if (!a) return CSA2_ERR_NULL;
  if (a->struct_size != sizeof(csa2_pool_args)) return CSA2_ERR_ARG;
  if (a->n_queries < 0 || a->n_queries > kMaxQ) return CSA2_ERR_SHAPE;
  if (a->n_entries < 0 || a->n_entries > kMaxI32) return CSA2_ERR_SHAPE;
  if (a->n_pool_blocks < 1 || a->n_pool_blocks > CSA2_MAX_POOL_BLOCKS) return CSA2_ERR_SHAPE;
  if (a->n_queries == 0) return CSA2_OK;
  if (!a->pool_blocks || (a->n_entries > 0 && !a->scores)) return CSA2_ERR_NULL;
  if (!aligned(a->scores, 4) || !aligned(a->n_valid, 4) || !aligned(a->pool_blocks, 4)) return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

size_t ws_attn(int Q, int k_sel, int n_swa) {
  if (Q == 0) return 0;
  AttnPlan ap = plan_attn(Q, k_sel, n_swa);
  if (ap.n_splits <= 1) return 0;
  Carve c(nullptr);
  c.take<char>(attn_partial_bytes(Q, ap));
  return c.off;
}

struct DecodeWs {
  TopkWs tk;
  float* scores;
  int32_t* idx;
  float* partial;
  size_t bytes;
};

DecodeWs carve_decode(void* ws, const csa2_decode_args* a, int64_t n_cand) {
  const int Q = a->index.n_queries;
  ScorePlan sp = plan_score(n_cand, Q, a->k);
  AttnPlan ap = plan_attn(Q, a->k, a->n_swa);
  Carve c(ws);
  DecodeWs d;
  d.tk = carve_topk(ws, Q, n_cand, sp, c);
  d.scores = c.take<float>((size_t)Q * (size_t)(n_cand > 0 ? n_cand : 1));
  d.idx = a->idx_out ? a->idx_out : c.take<int32_t>((size_t)Q * a->k);
  size_t pb = attn_partial_bytes(Q, ap);
  d.partial = pb ? c.take<float>(pb / sizeof(float)) : nullptr;
  d.bytes = c.off;
  return d;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

// Address of `scratch` on the current device, looked up on the first call
// there and kept per device (each GPU holds its own copy at its own address).
constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];

int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA2_ERR_HIP;
  uintptr_t p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == 0) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return CSA2_ERR_HIP;
    p = (uintptr_t)ptr;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = (void*)p;
  return CSA2_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return CSA2_OK;
  if (!ws || have < need) return CSA2_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

}  // namespace

extern "C" {

int csa2_version(void) { return 200; }

const char* csa2_status_string(int s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "required pointer is NULL";
    case CSA2_ERR_SHAPE: return "unsupported size or range";
    case CSA2_ERR_ALIGN: return "pointer not aligned as required";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP runtime or launch error";
    case CSA2_ERR_ARG: return "bad struct_size or enum value";
    case CSA2_ERR_SCRATCH: return "call needs more than the library's static scratch";
    default: return "unknown status";
  }
}

int csa2_dequant(int kind, const void* codes, const void* scales, int64_t n_entries, int out_dtype, void* out,
                 void* stream) {
  if (kind != CSA2_KIND_MAIN && kind != CSA2_KIND_INDEX) return CSA2_ERR_ARG;
  if (out_dtype != CSA2_OUT_F32 && out_dtype != CSA2_OUT_BF16) return CSA2_ERR_ARG;
  if (n_entries < 0 || n_entries > kMaxI32) return CSA2_ERR_SHAPE;
  if (n_entries == 0) return CSA2_OK;
  if (!codes || !out || (kind == CSA2_KIND_INDEX && !scales)) return CSA2_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(scales, 4)) return CSA2_ERR_ALIGN;
  return hip_status(launch_dequant(kind, (const uint8_t*)codes, (const uint8_t*)scales, n_entries,
                                   out_dtype == CSA2_OUT_BF16, out, (hipStream_t)stream));
}

int csa2_quantize(int kind, const void* x, int in_dtype, int64_t n_entries, const int64_t* dst_rows,
                  int64_t n_cache_rows, void* codes, void* scales, void* stream) {
  if (kind != CSA2_KIND_MAIN && kind != CSA2_KIND_INDEX) return CSA2_ERR_ARG;
  if (in_dtype != CSA2_IN_F32 && in_dtype != CSA2_IN_BF16) return CSA2_ERR_ARG;
  if (n_entries < 0 || n_entries > kMaxI32 || n_cache_rows < 0) return CSA2_ERR_SHAPE;
  if (!dst_rows && n_cache_rows < n_entries) return CSA2_ERR_SHAPE;
  if (n_entries == 0) return CSA2_OK;
  if (!x || !codes || (kind == CSA2_KIND_INDEX && !scales)) return CSA2_ERR_NULL;
  if (!aligned(x, in_dtype == CSA2_IN_F32 ? 16 : 8) || !aligned(codes, 16) || !aligned(scales, 4) ||
      !aligned(dst_rows, 8))
    return CSA2_ERR_ALIGN;
  return hip_status(launch_quantize(kind, x, in_dtype == CSA2_IN_BF16, n_entries, dst_rows, n_cache_rows,
                                    (uint8_t*)codes, (uint8_t*)scales, (hipStream_t)stream));
}

int csa2_pool_quantize(const float* x, const float* gate, int gate_width, int64_t n_entries,
                       const int64_t* dst_rows, int64_t n_cache_rows, void* cache, float* pooled, void* stream) {
  if (gate_width != 1 && gate_width != 512) return CSA2_ERR_ARG;
  if (n_entries < 0 || n_entries > kMaxI32 / 2 || n_cache_rows < 0) return CSA2_ERR_SHAPE;
  if (!dst_rows && n_cache_rows < n_entries) return CSA2_ERR_SHAPE;
  if (n_entries == 0) return CSA2_OK;
  if (!x || !gate || !cache) return CSA2_ERR_NULL;
  if (!aligned(x, 16) || !aligned(gate, gate_width == 1 ? 4 : 16) || !aligned(cache, 16) || !aligned(pooled, 16) ||
      !aligned(dst_rows, 8))
    return CSA2_ERR_ALIGN;
  return hip_status(launch_pool_quantize(x, gate, gate_width, n_entries, dst_rows, n_cache_rows, (uint8_t*)cache,
                                         pooled, (hipStream_t)stream));
}

int csa2_gather_selected(const uint8_t* main_cache, int64_t n_entries, int64_t cache_q_stride, const int32_t* idx,
                         int32_t n_queries, int32_t k_sel, uint8_t* out, int32_t* dense_idx, void* stream) {
  if (n_queries < 0 || n_queries > kMaxQ || k_sel < 0 || k_sel > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (n_entries < 0 || n_entries > kMaxI32 || cache_q_stride < 0) return CSA2_ERR_SHAPE;
  if (n_queries == 0 || k_sel == 0) return CSA2_OK;
  if (!idx || !out || !dense_idx || (n_entries > 0 && !main_cache)) return CSA2_ERR_NULL;
  if (!aligned(main_cache, 16) || !aligned(out, 16) || !aligned(idx, 4) || !aligned(dense_idx, 4))
    return CSA2_ERR_ALIGN;
  return hip_status(launch_gather_selected(main_cache, n_entries, cache_q_stride, idx, n_queries, k_sel, out,
                                           dense_idx, (hipStream_t)stream));
}

int csa2_build_pool(const csa2_pool_args* a, void* ws, size_t ws_bytes, void* stream) {
  int st = check_pool(a);
  if (st) return st;
  if (a->n_queries == 0) return CSA2_OK;
  const int Q = a->n_queries;
  const int64_t nb = (a->n_entries + 7) / 8;
  PoolWs w = carve_pool(nullptr, Q, a->n_entries, a->n_pool_blocks);
  st = check_ws(ws, ws_bytes, w.bytes);
  if (st) return st;
  w = carve_pool(ws, Q, a->n_entries, a->n_pool_blocks);
  hipStream_t s = (hipStream_t)stream;
  ScorePlan sp = plan_score(nb, Q, a->n_pool_blocks);
  hipError_t e = launch_block_max(a->scores, Q, a->n_entries, a->n_valid, w.bmax, w.nvb, s);
  // an empty cache leaves no block: the selection pads every row with -1
  if (e == hipSuccess && nb > 0) e = launch_score_maxima(w.bmax, Q, nb, nb, nullptr, 0, w.nvb, sp, w.tk.gmax, s);
  if (e == hipSuccess)
    e = launch_select(w.bmax, Q, nb, nb, nullptr, 0, nb > 0 ? w.nvb : nullptr, a->n_pool_blocks, sp,
                      nb > 0 ? w.tk.gmax : nullptr, w.tk.counts, w.tk.cand, a->pool_blocks, nullptr, s);
  return hip_status(e);
}

int csa2_index_score(const csa2_index_args* a, float* scores, void* stream) {
  int64_t n_cand = 0;
  int st = check_index(a, &n_cand);
  if (st) return st;
  if (a->n_queries == 0 || n_cand == 0) return CSA2_OK;
  if (!scores) return CSA2_ERR_NULL;
  if (!aligned(scores, 4)) return CSA2_ERR_ALIGN;
  IndexLaunch L{a->n_queries, a->n_entries, a->cache_q_stride, n_cand,       a->key_codes, a->key_scales,
                a->iq_codes,  a->iq_scales, a->head_weights,   a->cand_blocks, a->n_blocks, a->n_valid};
  ScorePlan sp = plan_score(n_cand, a->n_queries, 512);
  return hip_status(launch_index_score(L, sp, scores, nullptr, (hipStream_t)stream));
}

int csa2_topk(const csa2_topk_args* a, void* ws, size_t ws_bytes, void* stream) {
  int st = check_topk(a);
  if (st) return st;
  if (a->n_queries == 0) return CSA2_OK;
  st = check_ws(ws, ws_bytes, ws_topk(a));
  if (st) return st;
  const int Q = a->n_queries;
  ScorePlan sp = plan_score(a->n_cand, Q, a->k);
  Carve c(ws);
  TopkWs w = carve_topk(ws, Q, a->n_cand, sp, c);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_score_maxima(a->scores, Q, a->n_cand, a->n_entries, a->cand_blocks, a->n_blocks, a->n_valid,
                                     sp, w.gmax, s);
  if (e != hipSuccess) return CSA2_ERR_HIP;
  e = launch_select(a->scores, Q, a->n_cand, a->n_entries, a->cand_blocks, a->n_blocks, a->n_valid, a->k, sp, w.gmax,
                    w.counts, w.cand, a->idx, a->top_scores, s);
  return hip_status(e);
}

int csa2_sparse_attn(const csa2_attn_args* a, void* ws, size_t ws_bytes, void* stream) {
  int st = check_attn(a);
  if (st) return st;
  if (a->n_queries == 0) return CSA2_OK;
  const int Q = a->n_queries;
  st = check_ws(ws, ws_bytes, ws_attn(Q, a->k_sel, a->n_swa));
  if (st) return st;
  AttnPlan ap = plan_attn(Q, a->k_sel, a->n_swa);
  hipStream_t s = (hipStream_t)stream;
  float* partial = nullptr;
  if (ap.n_splits > 1) {
    Carve c(ws);
    partial = c.take<float>(attn_partial_bytes(Q, ap) / sizeof(float));
  }
  AttnLaunch L{Q,        a->n_entries,     a->cache_q_stride, a->main_cache,
               a->idx,   a->k_sel,         a->q,              a->swa,
               a->swa_q_stride, a->n_swa,  a->softmax_scale,  a->out,
               a->lse,   a->swa_format == CSA2_SWA_FP8, a->rope_cos_sin};
  return hip_status(launch_attn(L, ap, partial, s));
}

int csa2_sparse_attn_noalloc(const csa2_attn_args* a, void* stream) {
  int st = check_attn(a);
  if (st) return st;
  if (a->n_queries == 0) return CSA2_OK;
  const int Q = a->n_queries;
  const size_t need = ws_attn(Q, a->k_sel, a->n_swa);
  if (need > sizeof(scratch)) return CSA2_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_on_current_device(&ws);
    if (st) return st;
  }
  AttnPlan ap = plan_attn(Q, a->k_sel, a->n_swa);
  AttnLaunch L{Q,        a->n_entries,     a->cache_q_stride, a->main_cache,
               a->idx,   a->k_sel,         a->q,              a->swa,
               a->swa_q_stride, a->n_swa,  a->softmax_scale,  a->out,
               a->lse,   a->swa_format == CSA2_SWA_FP8, a->rope_cos_sin};
  return hip_status(launch_attn(L, ap, (float*)ws, (hipStream_t)stream));
}

int csa2_decode(const csa2_decode_args* a, void* ws, size_t ws_bytes, void* stream) {
  int64_t n_cand = 0;
  int st = check_decode(a, &n_cand);
  if (st) return st;
  const int Q = a->index.n_queries;
  if (Q == 0) return CSA2_OK;
  DecodeWs need = carve_decode(nullptr, a, n_cand);
  st = check_ws(ws, ws_bytes, need.bytes);
  if (st) return st;
  DecodeWs w = carve_decode(ws, a, n_cand);
  hipStream_t s = (hipStream_t)stream;
  ScorePlan sp = plan_score(n_cand, Q, a->k);
  IndexLaunch L{Q,
                a->index.n_entries,
                a->index.cache_q_stride,
                n_cand,
                a->index.key_codes,
                a->index.key_scales,
                a->index.iq_codes,
                a->index.iq_scales,
                a->index.head_weights,
                a->index.cand_blocks,
                a->index.n_blocks,
                a->index.n_valid};
  auto mark = [&](int i) {
    return a->stage_events[i] ? hipEventRecord((hipEvent_t)a->stage_events[i], s) : hipSuccess;
  };
  // Few queries over a short plain list: the attention kernel selects
  // straight from the scores (no selection launch, no sub-chunk maxima).
  const bool raw = a->index.cand_blocks == nullptr && n_cand <= kRawSelectMax && Q < 64;
  // 1. scores + sub-chunk maxima
  hipError_t e = mark(0);
  if (e == hipSuccess) e = launch_index_score(L, sp, w.scores, raw ? nullptr : w.tk.gmax, s);
  if (e == hipSuccess) e = mark(1);
  if (e != hipSuccess) return CSA2_ERR_HIP;
  // 2. threshold + compaction, exact top-k. In the chunk-parallel form the
  // final selection runs inside the attention kernel, whose every split
  // finishes its query's selection from the compacted candidates: one kernel
  // boundary and one id round trip fewer. In the raw form the attention
  // kernel makes the whole selection from the scores.
  const SelectPlan pl = plan_select(n_cand);
  const bool fused = !raw && select_is_chunked(Q, n_cand) && pl.n_chunks <= kFusedSelectMaxChunks;
  if (raw)
    e = hipSuccess;
  else if (fused)
    e = launch_select_compact(w.scores, Q, n_cand, a->index.n_entries, a->index.cand_blocks, a->index.n_blocks,
                              a->index.n_valid, a->k, sp, w.tk.gmax, w.tk.counts, w.tk.cand, s);
  else
    e = launch_select(w.scores, Q, n_cand, a->index.n_entries, a->index.cand_blocks, a->index.n_blocks,
                      a->index.n_valid, a->k, sp, w.tk.gmax, w.tk.counts, w.tk.cand, w.idx, nullptr, s);
  if (e == hipSuccess) e = mark(2);
  if (e != hipSuccess) return CSA2_ERR_HIP;
  // 3. attention over the selection + window
  AttnPlan ap = plan_attn(Q, a->k, a->n_swa);
  AttnLaunch A{Q,      a->index.n_entries, a->index.cache_q_stride, a->main_cache,
               w.idx,  a->k,               a->q,                    a->swa,
               a->swa_q_stride, a->n_swa, a->softmax_scale,        a->out,
               a->lse, a->swa_format == CSA2_SWA_FP8, a->rope_cos_sin};
  if (raw) {
    A.sel_scores = w.scores;
    A.sel_n_valid = a->index.n_valid;
    A.sel_n_cand = n_cand;
    A.idx_out = a->idx_out;
  } else if (fused) {
    A.sel_counts = w.tk.counts;
    A.sel_cand = w.tk.cand;
    A.sel_n_cand = n_cand;
    A.sel_chunks = pl.n_chunks;
    A.sel_chunk = pl.chunk;
    A.idx_out = a->idx_out;
  }
  e = launch_attn(A, ap, w.partial, s);
  if (e == hipSuccess) e = mark(3);
  return hip_status(e);
}

size_t csa2_workspace_size(int which, const void* args) {
  if (!args) return SIZE_MAX;
  if (which == CSA2_WS_TOPK) {
    const csa2_topk_args* a = (const csa2_topk_args*)args;
    if (a->struct_size != sizeof(csa2_topk_args)) return SIZE_MAX;
    if (a->n_queries < 0 || a->n_queries > kMaxQ || a->k < 1 || a->k > CSA2_MAX_K || a->n_cand < 0 ||
        a->n_cand > kMaxI32)
      return SIZE_MAX;
    return ws_topk(a);
  }
  if (which == CSA2_WS_ATTN) {
    const csa2_attn_args* a = (const csa2_attn_args*)args;
    if (a->struct_size != sizeof(csa2_attn_args)) return SIZE_MAX;
    if (a->n_queries < 0 || a->n_queries > kMaxQ || a->k_sel < 0 || a->k_sel > CSA2_MAX_K || a->n_swa < 0 ||
        a->n_swa > CSA2_MAX_SWA)
      return SIZE_MAX;
    return ws_attn(a->n_queries, a->k_sel, a->n_swa);
  }
  if (which == CSA2_WS_POOL) {
    const csa2_pool_args* a = (const csa2_pool_args*)args;
    if (a->struct_size != sizeof(csa2_pool_args)) return SIZE_MAX;
    if (a->n_queries < 0 || a->n_queries > kMaxQ || a->n_entries < 0 || a->n_entries > kMaxI32 ||
        a->n_pool_blocks < 1 || a->n_pool_blocks > CSA2_MAX_POOL_BLOCKS)
      return SIZE_MAX;
    if (a->n_queries == 0) return 0;
    return carve_pool(nullptr, a->n_queries, a->n_entries, a->n_pool_blocks).bytes;
  }
  if (which == CSA2_WS_DECODE) {
    const csa2_decode_args* a = (const csa2_decode_args*)args;
    if (a->struct_size != sizeof(csa2_decode_args) || a->index.struct_size != sizeof(csa2_index_args))
      return SIZE_MAX;
    if (a->index.n_entries < 0 || a->index.n_entries > kMaxI32 || a->index.n_blocks < 0 ||
        8LL * a->index.n_blocks > kMaxI32)
      return SIZE_MAX;
    const int64_t n_cand = a->index.cand_blocks ? 8LL * a->index.n_blocks : a->index.n_entries;
    if (a->index.n_queries < 0 || a->index.n_queries > kMaxQ || a->k < 1 || a->k > CSA2_MAX_K || a->n_swa < 0 ||
        a->n_swa > CSA2_MAX_SWA || n_cand < 0)
      return SIZE_MAX;
    if (a->index.n_queries == 0) return 0;
    return carve_decode(nullptr, a, n_cand).bytes;
  }
  return SIZE_MAX;
}

}  // extern "C"
