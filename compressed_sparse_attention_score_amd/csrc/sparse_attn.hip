// Sparse attention over the selected FP4 latents plus the sliding window.
//
// Method ("An infra-oriented diagram of the DeepSeek-V4.1-Flash architecture",
// Reading notes): one 512-wide latent per cache entry, shared by all 64 query
// heads, serving as both key and value; each layer attends over the 128-token
// window plus the 512 selected entries.
//
// Mapping (one workgroup = one query x one split of the joint slot list,
// 4 waves, wave w owns heads 16w..16w+15):
//  * Tiles of 32 joint slots are gathered and dequantised ONCE into LDS as
//    bf16 (exact), in two layouts: Kt[slot][channel] feeds S^T = K q^T, and
//    a blocked V^T (16 channels x 4 slots per 128-byte block, chunks rotated
//    by the writer's lane so stores and loads are bank-conflict free) feeds
//    O^T = V^T P^T. One tile serves as K and V; MFMA operand fragments are
//    loaded from LDS four ahead of their use.
//  * q stays in registers (16 fragments per lane). S^T comes out with one
//    head per lane column, so the online-softmax max/sum over the tile's
//    entries is 8 in-lane values plus two lane swaps, and the P^T fragments
//    are already in the B-operand layout of the PV product (the k-slot order
//    of the PV MFMA is permuted to match, and V^T is read in that order).
//  * O^T accumulates in 32 fp32 4-vectors per lane; softmax in fp32 (exp2
//    with the scale folded into log2 units). The running max is a reference
//    that only moves when a head's tile max exceeds it by more than 2^8, so
//    the accumulators are rescaled a handful of times per query instead of
//    every tile (p <= 256 is exact enough in bf16 and safe in fp32). The
//    hardware exp2 is used as is: terms below 2^-126 of the reference do not
//    matter to the sum.
//  * Small batches split the slot list over workgroups; each writes
//    (reference max, sum, unnormalised O) and a second kernel, one workgroup
//    per (query, 16 heads), merges them in split order. Handing the partials
//    over at a kernel boundary is cheaper on this multi-XCD part than any
//    in-kernel hand-off between workgroups.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {
constexpr int TILE = 32;
constexpr int KT_LD = kDim + 8;  // bf16 per Kt row (16-byte pad)
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const uint8_t* main_cache;
  const int32_t* idx;
  const uint16_t* q;
  const uint16_t* swa;
  uint16_t* out;
  float* lse;
  float* partial;
  int64_t n_entries, cache_q_stride, swa_q_stride;
  int k_sel, n_swa, nj, n_tiles, tiles_per_split, n_splits;
  float scale_log2;
};

// Per-split partial record: m[64], l[64], O[64][512] (fp32, O unnormalised).
constexpr int64_t kPartialFloats = 64 + 64 + 64 * 512;
constexpr int kMaxSplits = 64;
}  // namespace

__device__ __forceinline__ void finalize_head(const AttnArgs& a, int q, int head, int g, const v4f* o, float m,
                                              float l) {
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  uint16_t* orow = a.out + ((int64_t)q * kHeads + head) * kDim;
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) {
    const int ch = ct * 16 + 4 * g;
    __bf16 b0 = (__bf16)(o[ct][0] * inv), b1 = (__bf16)(o[ct][1] * inv);
    __bf16 b2 = (__bf16)(o[ct][2] * inv), b3 = (__bf16)(o[ct][3] * inv);
    uint2 pk;
    pk.x = (unsigned)__builtin_bit_cast(uint16_t, b0) | ((unsigned)__builtin_bit_cast(uint16_t, b1) << 16);
    pk.y = (unsigned)__builtin_bit_cast(uint16_t, b2) | ((unsigned)__builtin_bit_cast(uint16_t, b3) << 16);
    *(uint2*)(orow + ch) = pk;
  }
  if (a.lse && g == 0) a.lse[(int64_t)q * kHeads + head] = (l > 0.f) ? (m + __log2f(l)) * kLn2 : -__builtin_inff();
}

// One staged slot of 16 channels: FP4 codes (8 bytes) + E4M3 scale byte of a
// selected latent (kind 1), a window row to be read at decode time (kind 2),
// or nothing (kind 0).
struct RawSlot {
  uint2 c;
  unsigned sc;
  int kind;
};

// Selected ids of the 4 slots (4eg..4eg+3) of tile t; -1 marks a non-latent slot.
__device__ __forceinline__ void load_ids(const AttnArgs& a, int q, int t, int eg, int* e) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = t * TILE + 4 * eg + i;
    e[i] = (slot < a.k_sel) ? a.idx[(int64_t)q * a.k_sel + slot] : -1;
  }
}

__device__ __forceinline__ void issue_raw(const AttnArgs& a, int q, int t, int eg, int cg, const int* e,
                                          RawSlot* r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = t * TILE + 4 * eg + i;
    r[i].kind = 0;
    r[i].c = uint2{0u, 0u};
    r[i].sc = 0u;
    if (slot < a.k_sel) {
      if (e[i] >= 0 && (int64_t)e[i] < a.n_entries) {
        const uint8_t* ent = a.main_cache + ((int64_t)q * a.cache_q_stride + e[i]) * kMainBytes;
        r[i].c = *(const uint2*)(ent + cg * 8);
        r[i].sc = ent[256 + cg];
        r[i].kind = 1;
      }
    } else if (slot < a.nj) {
      r[i].kind = 2;
    }
  }
}

__device__ __forceinline__ void decode_raw(const AttnArgs& a, int q, int t, int eg, int cg, int i, const RawSlot& r,
                                           unsigned* kw, bool& ok) {
  ok = r.kind != 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) kw[j] = 0u;
  if (r.kind == 1) {
    const float sc = e4m3_to_f32(r.sc);
    float f[8];
    decode_e2m1x8_scaled(r.c.x, sc, f);
#pragma unroll
    for (int j = 0; j < 4; ++j) kw[j] = pack_bf16x2_exact(f[2 * j], f[2 * j + 1]);
    decode_e2m1x8_scaled(r.c.y, sc, f);
#pragma unroll
    for (int j = 0; j < 4; ++j) kw[4 + j] = pack_bf16x2_exact(f[2 * j], f[2 * j + 1]);
  } else if (r.kind == 2) {
    // window rows are already bf16 pairs
    const int slot = t * TILE + 4 * eg + i;
    const uint16_t* row = a.swa + ((int64_t)q * a.swa_q_stride + (slot - a.k_sel)) * kDim + cg * 16;
    const v4u r0 = *(const v4u*)row, r1 = *(const v4u*)(row + 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kw[j] = r0[j];
      kw[4 + j] = r1[j];
    }
  }
}

// V^T block of (channel group cg, slot group sg): 16 channels x 4 slots, chunk
// c (channel c of the group, 4 slots = 8 bytes) stored at chunk (c + rot) & 15
// where rot = (cg*8 + sg) & 15 is the writer lane's index mod 16.
__device__ __forceinline__ int vb_offset(int cg, int sg, int c) {
  return ((cg * 8 + sg) * 16 + ((c + ((cg * 8 + sg) & 15)) & 15)) * 4;
}

__global__ __launch_bounds__(256, 1) void k_sparse_attn(AttnArgs a) {
  const int q = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int head = 16 * wave + r16;

  __shared__ __attribute__((aligned(16))) uint16_t Kt[TILE * KT_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vb[TILE * kDim];
  __shared__ unsigned char slot_ok[TILE];

  // q fragments: head, channels kk*32 + 8g .. +7
  v8bf qf[16];
  {
    const uint16_t* qrow = a.q + ((int64_t)q * kHeads + head) * kDim + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      v4u raw = *(const v4u*)(qrow + kk * 32);
      qf[kk] = __builtin_bit_cast(v8bf, raw);
    }
  }
  v4f o[32];
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) o[ct] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff(), l_run = 0.f;

  const int t0 = split * a.tiles_per_split;
  const int t1 = min(t0 + a.tiles_per_split, a.n_tiles);
  const int eg = tid & 7, cg = tid >> 3;  // staging: slots 4eg..4eg+3, channels 16cg..16cg+15

  // Software pipeline: while tile t is multiplied, the FP4 latents of tile
  // t+1 and the selected ids of tile t+2 are in flight.
  int e_nxt[4];
  RawSlot raw[4];
  if (t0 < t1) {
    int e0[4];
    load_ids(a, q, t0, eg, e0);
    issue_raw(a, q, t0, eg, cg, e0, raw);
    if (t0 + 1 < t1) load_ids(a, q, t0 + 1, eg, e_nxt);
  }

  for (int t = t0; t < t1; ++t) {
    // ---- this thread's 4 slots x 16 channels as bf16 pairs
    // kw[i][j] = channels 16cg+2j (bits 15:0) and 16cg+2j+1 (bits 31:16) of slot 4eg+i
    unsigned kw[4][8];
    bool okf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) decode_raw(a, q, t, eg, cg, i, raw[i], kw[i], okf[i]);
    __syncthreads();  // previous tile's LDS reads are complete
    if (cg == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) slot_ok[4 * eg + i] = okf[i] ? 1 : 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v4u* kp = (v4u*)(Kt + (4 * eg + i) * KT_LD + cg * 16);
      kp[0] = v4u{kw[i][0], kw[i][1], kw[i][2], kw[i][3]};
      kp[1] = v4u{kw[i][4], kw[i][5], kw[i][6], kw[i][7]};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // channel 2j: low halves; channel 2j+1: high halves; slots 4eg..4eg+3
      uint2 lo, hi;
      lo.x = __builtin_amdgcn_perm(kw[1][j], kw[0][j], 0x05040100u);
      lo.y = __builtin_amdgcn_perm(kw[3][j], kw[2][j], 0x05040100u);
      hi.x = __builtin_amdgcn_perm(kw[1][j], kw[0][j], 0x07060302u);
      hi.y = __builtin_amdgcn_perm(kw[3][j], kw[2][j], 0x07060302u);
      *(uint2*)(Vb + vb_offset(cg, eg, 2 * j)) = lo;
      *(uint2*)(Vb + vb_offset(cg, eg, 2 * j + 1)) = hi;
    }
    // ---- prefetch the next tile's latents and the ids after it
    if (t + 1 < t1) {
      issue_raw(a, q, t + 1, eg, cg, e_nxt, raw);
      if (t + 2 < t1) load_ids(a, q, t + 2, eg, e_nxt);
    }
    __syncthreads();

    // ---- S^T[entry][head] for entries et*16 + 4g + r
    v4f s[2];
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      s[et] = v4f{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = Kt + (et * 16 + r16) * KT_LD + 8 * g;
      v4u fr[4], nx[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) fr[j] = *(const v4u*)(kr + j * 32);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (kb < 3) {
#pragma unroll
          for (int j = 0; j < 4; ++j) nx[j] = *(const v4u*)(kr + (4 * (kb + 1) + j) * 32);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          s[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, fr[j]), qf[4 * kb + j], s[et],
                                                          0, 0, 0);
        if (kb < 3) {
#pragma unroll
          for (int j = 0; j < 4; ++j) fr[j] = nx[j];
        }
      }
    }
    // ---- online softmax in log2 units with a lazily moved reference max
    float x[8];
    float mt = -__builtin_inff();
#pragma unroll
    for (int et = 0; et < 2; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + 4 * g + r;
        x[et * 4 + r] = slot_ok[e] ? s[et][r] * a.scale_log2 : -__builtin_inff();
        mt = fmaxf(mt, x[et * 4 + r]);
      }
    mt = max_xor16(mt);
    mt = max_xor32(mt);
    const bool move = mt > m_ref + kRescaleSlack;  // also true when m_ref = -inf and mt is finite
    if (__any(move)) {
      const float m_new = move ? mt : m_ref;
      const float alpha = (m_ref == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      if (move) l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) o[ct] = move ? o[ct] * alpha : o[ct];
      m_ref = m_new;
    }
    float p[8], ps = 0.f;
    const bool live = m_ref != -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = live ? __builtin_amdgcn_exp2f(x[i] - m_ref) : 0.f;
      ps += p[i];
    }
    ps = add_xor16(ps);
    ps = add_xor32(ps);
    l_run += ps;
    v8bf pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = (__bf16)p[i];
    // ---- O^T[channel][head] += V^T P^T; this lane's k-slots: slots 4g..4g+3, 16+4g..16+4g+3
    {
      v4u fr[4], nx[4];
      // lane-constant parts of vb_offset(ct, sg, r16): the rotation only
      // depends on ct's parity, the rest is ct * 512 elements
      const uint16_t* vlo[2] = {Vb + vb_offset(0, g, r16), Vb + vb_offset(1, g, r16) - 512};
      const uint16_t* vhi[2] = {Vb + vb_offset(0, 4 + g, r16), Vb + vb_offset(1, 4 + g, r16) - 512};
      auto vfrag = [&](int ct) {
        const uint2 lo = *(const uint2*)(vlo[ct & 1] + ct * 512);
        const uint2 hi = *(const uint2*)(vhi[ct & 1] + ct * 512);
        return v4u{lo.x, lo.y, hi.x, hi.y};
      };
#pragma unroll
      for (int j = 0; j < 4; ++j) fr[j] = vfrag(j);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        if (cb < 7) {
#pragma unroll
          for (int j = 0; j < 4; ++j) nx[j] = vfrag(4 * (cb + 1) + j);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[4 * cb + j] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, fr[j]), pb, o[4 * cb + j], 0, 0, 0);
        if (cb < 7) {
#pragma unroll
          for (int j = 0; j < 4; ++j) fr[j] = nx[j];
        }
      }
    }
  }

  if (a.n_splits == 1) {
    finalize_head(a, q, head, g, o, m_ref, l_run);
    return;
  }
  // ---- write this split's partial (merged by k_attn_combine)
  float* part = a.partial + ((int64_t)q * a.n_splits + split) * kPartialFloats;
  if (g == 0) {
    part[head] = m_ref;
    part[64 + head] = l_run;
  }
  float* po = part + 128 + (int64_t)head * kDim;
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) *(v4f*)(po + ct * 16 + 4 * g) = o[ct];
}

// Merge the splits of one query: out = sum_s O_s 2^(m_s - M) /
// sum_s l_s 2^(m_s - M), in split order. grid (16, Q), 256 threads:
// thread -> head blockIdx.x*4 + tid/64, channels (tid%64)*8 .. +7.
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ partial, int n_splits,
                                                      uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int q = blockIdx.y, tid = threadIdx.x;
  const int h = blockIdx.x * 4 + (tid >> 6), c0 = (tid & 63) * 8;
  const float* base = partial + (int64_t)q * n_splits * kPartialFloats;
  float M = -__builtin_inff();
  for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, base[sp * kPartialFloats + h]);
  float L = 0.f;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  if (M != -__builtin_inff()) {
    for (int sp = 0; sp < n_splits; ++sp) {
      const float* ps = base + sp * kPartialFloats;
      const float ms = ps[h];
      const float f = (ms == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      L += ps[64 + h] * f;
      const v4f* src = (const v4f*)(ps + 128 + (int64_t)h * kDim + c0);
      const v4f x0 = src[0], x1 = src[1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[c] += x0[c] * f;
        acc[4 + c] += x1[c] * f;
      }
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  v4u pk;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    __bf16 lo = (__bf16)(acc[2 * j] * inv), hi = (__bf16)(acc[2 * j + 1] * inv);
    pk[j] = (unsigned)__builtin_bit_cast(uint16_t, lo) | ((unsigned)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  *(v4u*)(out + ((int64_t)q * kHeads + h) * kDim + c0) = pk;
  if (lse && (tid & 63) == 0)
    lse[(int64_t)q * kHeads + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

AttnPlan plan_attn(int Q, int nj) {
  // Aim for one workgroup per CU, with at least 4 tiles per split so the
  // software pipeline has work to overlap and the merge reads few partials.
  AttnPlan p;
  p.n_tiles = (nj + TILE - 1) / TILE;
  if (p.n_tiles < 1) p.n_tiles = 1;
  const int want = (Q > 0) ? (256 + Q - 1) / Q : 1;
  int tps = (p.n_tiles + want - 1) / want;
  if (tps < 4) tps = 4;
  p.tiles_per_split = tps;
  p.n_splits = (p.n_tiles + tps - 1) / tps;
  if (p.n_splits > kMaxSplits) {
    p.tiles_per_split = (p.n_tiles + kMaxSplits - 1) / kMaxSplits;
    p.n_splits = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  }
  return p;
}

size_t attn_partial_bytes(int Q, const AttnPlan& plan) {
  if (plan.n_splits <= 1) return 0;
  return (size_t)Q * plan.n_splits * kPartialFloats * sizeof(float);
}

hipError_t launch_attn(const AttnLaunch& L, const AttnPlan& plan, float* partial, hipStream_t s) {
  if (L.Q <= 0) return hipSuccess;
  AttnArgs a;
  a.main_cache = L.main_cache;
  a.idx = L.idx;
  a.q = L.q;
  a.swa = L.swa;
  a.out = L.out;
  a.lse = L.lse;
  a.partial = partial;
  a.n_entries = L.n_entries;
  a.cache_q_stride = L.cache_q_stride;
  a.swa_q_stride = L.swa_q_stride;
  a.k_sel = L.k_sel;
  a.n_swa = L.n_swa;
  a.nj = L.k_sel + L.n_swa;
  a.n_tiles = plan.n_tiles;
  a.tiles_per_split = plan.tiles_per_split;
  a.n_splits = plan.n_splits;
  a.scale_log2 = L.scale * kLog2e;
  dim3 grid((unsigned)plan.n_splits, (unsigned)L.Q);
  k_sparse_attn<<<grid, 256, 0, s>>>(a);
  if (plan.n_splits > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_attn_combine<<<dim3(16, (unsigned)L.Q), 256, 0, s>>>(partial, plan.n_splits, L.out, L.lse);
  }
  return hipGetLastError();
}

}  // namespace csa2
