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
//    Vt[channel][slot] feeds O^T = V^T P^T, so every 16x16x32 bf16 MFMA
//    operand is a contiguous 16-byte LDS read. One tile serves as K and V.
//  * q stays in registers (16 fragments per lane). S^T comes out with one
//    head per lane column, so the online-softmax max/sum over the tile's
//    entries is 8 in-lane values plus two lane swaps, and the P^T fragments
//    are already in the B-operand layout of the PV product (the k-slot order
//    of the PV MFMA is permuted to match, and V^T is read in that order).
//  * O^T accumulates in 32 fp32 4-vectors per lane; softmax in fp32 (exp2
//    with the scale folded into log2 units).
//  * Small batches split the slot list over workgroups; each writes
//    (max, sum, unnormalised O) and the last one per query (atomic ticket)
//    merges them in split order.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

namespace {
constexpr int TILE = 32;
constexpr int KT_LD = kDim + 8;  // bf16 per Kt row (16-byte pad)
constexpr int VT_LD = TILE + 8;  // bf16 per Vt row (16-byte pad)
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
  unsigned* ticket;
  int64_t n_entries, cache_q_stride, swa_q_stride;
  int k_sel, n_swa, nj, n_tiles, tiles_per_split, n_splits;
  float scale_log2;
};

// Per-split partial record: m[64], l[64], O[64][512] (fp32, O unnormalised).
constexpr int64_t kPartialFloats = 64 + 64 + 64 * 512;
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

__global__ __launch_bounds__(256, 2) void k_sparse_attn(AttnArgs a) {
  const int q = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int head = 16 * wave + r16;

  __shared__ __attribute__((aligned(16))) uint16_t Kt[TILE * KT_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kDim * VT_LD];
  __shared__ unsigned char slot_ok[TILE];
  __shared__ unsigned is_last;

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
  float m_run = -__builtin_inff(), l_run = 0.f;

  const int t0 = split * a.tiles_per_split;
  const int t1 = min(t0 + a.tiles_per_split, a.n_tiles);
  const int eg = tid >> 5, cg = tid & 31;  // staging: slots 4eg..4eg+3, channels 16cg..16cg+15

  for (int t = t0; t < t1; ++t) {
    // ---- gather + dequantise 32 slots into registers as bf16 pairs
    // kw[i][j] = channels 16cg+2j (bits 15:0) and 16cg+2j+1 (bits 31:16) of slot 4eg+i
    unsigned kw[4][8];
    bool okf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = t * TILE + 4 * eg + i;
      bool ok = false;
#pragma unroll
      for (int j = 0; j < 8; ++j) kw[i][j] = 0u;
      if (slot < a.k_sel) {
        const int32_t e = a.idx[(int64_t)q * a.k_sel + slot];
        if (e >= 0 && (int64_t)e < a.n_entries) {
          ok = true;
          const uint8_t* ent = a.main_cache + ((int64_t)q * a.cache_q_stride + e) * kMainBytes;
          const uint2 c = *(const uint2*)(ent + cg * 8);
          const float sc = e4m3_to_f32(ent[256 + cg]);
          float f[8];
          decode_e2m1x8_scaled(c.x, sc, f);
#pragma unroll
          for (int j = 0; j < 4; ++j) kw[i][j] = pack_bf16x2_exact(f[2 * j], f[2 * j + 1]);
          decode_e2m1x8_scaled(c.y, sc, f);
#pragma unroll
          for (int j = 0; j < 4; ++j) kw[i][4 + j] = pack_bf16x2_exact(f[2 * j], f[2 * j + 1]);
        }
      } else if (slot < a.nj) {
        ok = true;
        const uint16_t* row = a.swa + ((int64_t)q * a.swa_q_stride + (slot - a.k_sel)) * kDim + cg * 16;
        const v4u r0 = *(const v4u*)row, r1 = *(const v4u*)(row + 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kw[i][j] = r0[j];
          kw[i][4 + j] = r1[j];
        }
      }
      okf[i] = ok;
    }
    __syncthreads();  // previous tile's LDS reads are complete
    if (cg == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) slot_ok[4 * eg + i] = okf[i] ? 1 : 0;
    }
    // ---- write Kt rows and Vt columns
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
      *(uint2*)(Vt + (cg * 16 + 2 * j) * VT_LD + 4 * eg) = lo;
      *(uint2*)(Vt + (cg * 16 + 2 * j + 1) * VT_LD + 4 * eg) = hi;
    }
    __syncthreads();

    // ---- S^T[entry][head] for entries et*16 + 4g + r
    v4f s[2];
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      s[et] = v4f{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = Kt + (et * 16 + r16) * KT_LD + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        v8bf A = __builtin_bit_cast(v8bf, *(const v4u*)(kr + kk * 32));
        s[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qf[kk], s[et], 0, 0, 0);
      }
    }
    // ---- online softmax (log2 units)
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
    const float m_new = fmaxf(m_run, mt);
    const bool none = (m_new == -__builtin_inff());
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = none ? 0.f : exp2f(x[i] - m_new);
      ps += p[i];
    }
    ps = add_xor16(ps);
    ps = add_xor32(ps);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    v8bf pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = (__bf16)p[i];
    // ---- O^T[channel][head] += V^T P^T; this lane's k-slots: slots 4g..4g+3, 16+4g..16+4g+3
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
      const uint16_t* vr = Vt + (ct * 16 + r16) * VT_LD + 4 * g;
      const uint2 lo = *(const uint2*)vr, hi = *(const uint2*)(vr + 16);
      v4u raw = {lo.x, lo.y, hi.x, hi.y};
      v8bf A = __builtin_bit_cast(v8bf, raw);
      o[ct] = o[ct] * alpha;
      o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, pb, o[ct], 0, 0, 0);
    }
  }

  if (a.n_splits == 1) {
    finalize_head(a, q, head, g, o, m_run, l_run);
    return;
  }
  // ---- write this split's partial, then the last split merges
  float* part = a.partial + ((int64_t)q * a.n_splits + split) * kPartialFloats;
  if (g == 0) {
    part[head] = m_run;
    part[64 + head] = l_run;
  }
  float* po = part + 128 + (int64_t)head * kDim;
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) *(float4*)(po + ct * 16 + 4 * g) = make_float4(o[ct][0], o[ct][1], o[ct][2], o[ct][3]);
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = (atomicAdd(&a.ticket[q], 1u) == (unsigned)(a.n_splits - 1)) ? 1u : 0u;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  // thread -> head tid/4, channels (tid%4)*128 .. +127, in passes of 32
  const int h = tid >> 2, c0 = (tid & 3) * 128;
  const float* base = a.partial + (int64_t)q * a.n_splits * kPartialFloats;
  float M = -__builtin_inff();
  for (int sp = 0; sp < a.n_splits; ++sp) M = fmaxf(M, __builtin_nontemporal_load(base + sp * kPartialFloats + h));
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int sp = 0; sp < a.n_splits; ++sp) {
      const float ms = __builtin_nontemporal_load(base + sp * kPartialFloats + h);
      if (ms != -__builtin_inff()) L += __builtin_nontemporal_load(base + sp * kPartialFloats + 64 + h) * exp2f(ms - M);
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  uint16_t* orow = a.out + ((int64_t)q * kHeads + h) * kDim + c0;
  for (int pass = 0; pass < 4; ++pass) {
    float acc[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) acc[c] = 0.f;
    if (M != -__builtin_inff()) {
      for (int sp = 0; sp < a.n_splits; ++sp) {
        const float* ps = base + sp * kPartialFloats;
        const float ms = __builtin_nontemporal_load(ps + h);
        if (ms == -__builtin_inff()) continue;
        const float f = exp2f(ms - M);
        const v4f* src = (const v4f*)(ps + 128 + (int64_t)h * kDim + c0 + pass * 32);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          v4f x4 = __builtin_nontemporal_load(src + c);
          acc[4 * c] += x4[0] * f;
          acc[4 * c + 1] += x4[1] * f;
          acc[4 * c + 2] += x4[2] * f;
          acc[4 * c + 3] += x4[3] * f;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 32; c += 8) {
      v4u pk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __bf16 lo = (__bf16)(acc[c + 2 * j] * inv), hi = (__bf16)(acc[c + 2 * j + 1] * inv);
        pk[j] = (unsigned)__builtin_bit_cast(uint16_t, lo) | ((unsigned)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *(v4u*)(orow + pass * 32 + c) = pk;
    }
  }
  if (a.lse && (tid & 3) == 0)
    a.lse[(int64_t)q * kHeads + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

AttnPlan plan_attn(int Q, int nj) {
  AttnPlan p;
  p.n_tiles = (nj + TILE - 1) / TILE;
  if (p.n_tiles < 1) p.n_tiles = 1;
  int want = (Q > 0) ? (512 + Q - 1) / Q : 1;
  int max_splits = (p.n_tiles + 1) / 2;  // at least two tiles per split
  if (max_splits < 1) max_splits = 1;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  p.tiles_per_split = (p.n_tiles + want - 1) / want;
  p.n_splits = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

size_t attn_partial_bytes(int Q, const AttnPlan& plan) {
  if (plan.n_splits <= 1) return 0;
  return (size_t)Q * plan.n_splits * kPartialFloats * sizeof(float);
}

hipError_t launch_attn(const AttnLaunch& L, const AttnPlan& plan, float* partial, unsigned* ticket, hipStream_t s) {
  if (L.Q <= 0) return hipSuccess;
  AttnArgs a;
  a.main_cache = L.main_cache;
  a.idx = L.idx;
  a.q = L.q;
  a.swa = L.swa;
  a.out = L.out;
  a.lse = L.lse;
  a.partial = partial;
  a.ticket = ticket;
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
  return hipGetLastError();
}

}  // namespace csa2
