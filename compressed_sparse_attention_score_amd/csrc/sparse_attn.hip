// Sparse attention over the selected FP4 latents plus the sliding window.
//
// Method ("An infra-oriented diagram of the DeepSeek-V4.1-Flash architecture",
// Reading notes): one 512-wide latent per cache entry, shared by all 64 query
// heads, serving as both key and value; each layer attends over the 128-token
// window plus the 512 selected entries.
//
// Mapping (one workgroup of 8 waves = one query x one split of the joint slot
// list):
//  * Tiles of 32 joint slots are gathered and dequantised ONCE into LDS as
//    bf16 (exact), in two layouts: Kt[slot][channel] (16-byte chunks XOR-
//    swizzled by slot) feeds S^T = K q^T, and a blocked V^T (16 channels x 4
//    slots per 128-byte block, chunks rotated by the writer's lane) feeds
//    O^T = V^T P^T. Reads of both are bank-conflict free.
//  * Wave (hh, cc) owns heads 32hh..32hh+31 and channels 128cc..128cc+127
//    for the matrix products: every LDS fragment it reads feeds two MFMAs
//    (two 16-head blocks), and q for its heads and channels stays in
//    registers. Each wave forms S^T over its channel quarter; the softmax is
//    then done once per (slot, head): wave w owns heads 8w..8w+7 over all 32
//    slots of the tile (4 values per lane), adds the four partial sums from
//    LDS, and writes P^T (bf16, laid out as the PV B operand) and the
//    per-head rescale factor back to LDS for the product waves.
//  * Per tile t, three barrier-separated phases: (1) S^T of tile t and
//    O^T += V^T P^T of tile t-1 back to back on the matrix cores; (2) the
//    softmax of tile t, and tile t+1 dequantised into LDS (V^T
//    double-buffered, K single-buffered) with the latents of tile t+2
//    requested; (3) P^T of tile t picked up and O^T rescaled if a head's
//    reference moved.
//  * The PV product's k-slot order is permuted (slots 4g..4g+3 and
//    16+4g..16+4g+3 for lane group g) so that S^T fragments, P^T fragments
//    and V^T reads line up without shuffles.
//  * Softmax in fp32 with exp2 (the scale folded into log2 units). The
//    running max is a reference that only moves when a head's tile max
//    exceeds it by more than 2^8, so the accumulators are rescaled a handful
//    of times per query instead of every tile (p <= 256 is exact enough in
//    bf16 and safe in fp32). The hardware exp2 is used as is: terms below
//    2^-126 of the reference do not matter to the sum.
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
constexpr int NT = 512;  // threads per workgroup
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

struct AttnShared {
  uint16_t kt[TILE * kDim];         // [slot][channel], 16-byte chunks swizzled
  uint16_t vb[2][TILE * kDim];      // blocked V^T, double-buffered
  v4f sx[8][4][64];                 // partial S^T per wave: [wave][2*sb+hb][lane]
  uint2 pl[kHeads][TILE / 4];       // P^T as bf16: [head][slot quad] = 4 slots
  float alpha[kHeads];              // per-head rescale of O for this tile (1 = none)
  float fin_m[kHeads], fin_l[kHeads];
  unsigned ok[2][TILE / 4];         // slot validity bytes per tile (double-buffered)
};
}  // namespace

// One staged slot of 8 channels: 4 bytes of FP4 codes + the E4M3 scale byte
// of a selected latent (kind 1), 8 bf16 of a window row (kind 2), or nothing.
struct RawSlot {
  v4u a;
  unsigned sc;  // bits 7:0 scale byte, bits 9:8 kind
};

// Selected ids of the 4 slots (4eg..4eg+3) of tile t; -1 marks a non-latent
// slot. Tiles wholly inside the selected part read their ids unconditionally
// (a per-slot branch around a load makes the compiler wait for it).
__device__ __forceinline__ void load_ids(const AttnArgs& a, int q, int t, int eg, int* e) {
  const int s0 = t * TILE + 4 * eg;
  if (t * TILE + TILE <= a.k_sel) {
    const int32_t* ip = a.idx + (int64_t)q * a.k_sel + s0;
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = ip[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = (s0 + i < a.k_sel) ? a.idx[(int64_t)q * a.k_sel + s0 + i] : -1;
  }
}

// Channels 8c8..8c8+7 of the 4 slots of tile t. A tile holds only selected
// latents or only window rows unless k_sel is not a multiple of the tile:
// those two cases issue every load unconditionally (invalid slots read row 0
// of the query's cache or window and are flagged empty), so all loads of the
// tile stay in flight together; a mixed tile takes the per-slot path.
__device__ __forceinline__ void issue_raw(const AttnArgs& a, int q, int t, int eg, int c8, const int* e,
                                          RawSlot* r) {
  const int s0 = t * TILE;
  if (s0 + TILE <= a.k_sel && a.n_entries > 0) {
    const uint8_t* base = a.main_cache + (int64_t)q * a.cache_q_stride * kMainBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = e[i] >= 0 && (int64_t)e[i] < a.n_entries;
      const uint8_t* ent = base + (int64_t)(ok ? e[i] : 0) * kMainBytes;
      r[i].a = v4u{*(const unsigned*)(ent + c8 * 4), 0u, 0u, 0u};
      r[i].sc = (unsigned)ent[256 + (c8 >> 1)] | (ok ? (1u << 8) : 0u);
    }
    return;
  }
  if (s0 >= a.k_sel) {  // window rows only (this tile exists, so n_swa >= 1)
    const uint16_t* base = a.swa + (int64_t)q * a.swa_q_stride * kDim + c8 * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = s0 + 4 * eg + i;
      const bool ok = slot < a.nj;
      r[i].a = *(const v4u*)(base + (int64_t)(ok ? slot - a.k_sel : 0) * kDim);
      r[i].sc = ok ? (2u << 8) : 0u;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = s0 + 4 * eg + i;
    r[i].a = v4u{0u, 0u, 0u, 0u};
    r[i].sc = 0u;
    if (slot < a.k_sel) {
      if (e[i] >= 0 && (int64_t)e[i] < a.n_entries) {
        const uint8_t* ent = a.main_cache + ((int64_t)q * a.cache_q_stride + e[i]) * kMainBytes;
        r[i].a = v4u{*(const unsigned*)(ent + c8 * 4), 0u, 0u, 0u};
        r[i].sc = ent[256 + (c8 >> 1)] | (1u << 8);
      }
    } else if (slot < a.nj) {
      r[i].a = *(const v4u*)(a.swa + ((int64_t)q * a.swa_q_stride + (slot - a.k_sel)) * kDim + c8 * 8);
      r[i].sc = 2u << 8;
    }
  }
}

// kw[j] = channels 8c8+2j (bits 15:0) and 8c8+2j+1 (bits 31:16) as bf16.
// Branch-free: a latent is decoded, a window row passed through, an empty
// slot gives zeros (its loaded bytes may be anything, NaN included).
__device__ __forceinline__ void decode_raw(const RawSlot& r, unsigned* kw) {
  float f[8];
  decode_e2m1x8_scaled(r.a[0], e4m3_to_f32_hw(r.sc & 0xFFu), f);
  const unsigned kind = r.sc >> 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned dec = pack_bf16x2_exact(f[2 * j], f[2 * j + 1]);
    kw[j] = (kind == 1u) ? dec : (kind == 2u) ? r.a[j] : 0u;
  }
}

// Validity bytes of the 4 staged slots (byte i = slot 4eg+i holds data).
__device__ __forceinline__ unsigned raw_ok(const RawSlot* r) {
  unsigned okb = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) okb |= ((r[i].sc >> 8) != 0u ? 1u : 0u) << (8 * i);
  return okb;
}

// Element offset of channel chunk `chunk` (8 channels, 16 bytes) of Kt row
// `slot`; chunks are XOR-swizzled by the row so that a store of one row by 64
// lanes and a fragment read of 16 rows at one chunk both touch 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int kt_offset(int slot, int chunk) { return slot * kDim + ((chunk ^ (slot & 15)) << 3); }

// V^T block of (channel group cg, slot group sg): 16 channels x 4 slots, 128
// bytes. Block order within a channel group alternates with cg's parity and
// chunk c (channel c of the group, 4 slots = 8 bytes) sits at (c + cg) & 15:
// a fragment read (16 channels of 4 consecutive slot groups) covers 512
// contiguous bytes, and a store of one slot group by 64 lanes (32 channel
// groups) spreads over every bank twice.
__device__ __forceinline__ int vb_offset(int cg, int sg, int c) {
  return ((cg * 8 + (sg ^ (cg & 1))) * 16 + ((c + cg) & 15)) * 4;
}

// Store this thread's 4 dequantised slots (8 channels each) as tile data:
// Kt rows, V^T buffer vbuf, validity flags okbuf.
__device__ __forceinline__ void store_tile(AttnShared& sh, int vbuf, int eg, int c8, const unsigned (*kw)[4],
                                           unsigned okb) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *(v4u*)(sh.kt + kt_offset(4 * eg + i, c8)) = v4u{kw[i][0], kw[i][1], kw[i][2], kw[i][3]};
  const int cg = c8 >> 1, cbase = (c8 & 1) * 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // channel cbase+2j: low halves; channel cbase+2j+1: high halves; slots 4eg..4eg+3
    uint2 lo, hi;
    lo.x = __builtin_amdgcn_perm(kw[1][j], kw[0][j], 0x05040100u);
    lo.y = __builtin_amdgcn_perm(kw[3][j], kw[2][j], 0x05040100u);
    hi.x = __builtin_amdgcn_perm(kw[1][j], kw[0][j], 0x07060302u);
    hi.y = __builtin_amdgcn_perm(kw[3][j], kw[2][j], 0x07060302u);
    *(uint2*)(sh.vb[vbuf] + vb_offset(cg, eg, cbase + 2 * j)) = lo;
    *(uint2*)(sh.vb[vbuf] + vb_offset(cg, eg, cbase + 2 * j + 1)) = hi;
  }
  if (c8 == 0) sh.ok[vbuf][eg] = okb;  // one lane per slot group
}

__global__ __launch_bounds__(NT, 1) void k_sparse_attn(AttnArgs a) {
  const int q = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int hh = wave & 1, cc = wave >> 1;

  __shared__ AttnShared sh;

  // q fragments: head 32hh + 16hb + r16, channels 128cc + 32ks + 8g .. +7
  v8bf qf[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const uint16_t* qrow = a.q + ((int64_t)q * kHeads + 32 * hh + 16 * hb + r16) * kDim + 128 * cc + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[hb][ks] = __builtin_bit_cast(v8bf, *(const v4u*)(qrow + ks * 32));
  }
  // O^T accumulators: channels 128cc + 16cb + 4g + r, head 32hh + 16hb + r16
  v4f o[8][2];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) o[cb][hb] = v4f{0.f, 0.f, 0.f, 0.f};
  v8bf pb[2];  // P^T of the last softmaxed tile, B-operand layout

  // softmax ownership: head sh_head = 8*wave + (lane & 7), slots 4*quad..+3
  const int quad = lane >> 3;
  const int sh_head = 8 * wave + (lane & 7);
  const int s_hh = sh_head >> 5, s_hb = (sh_head >> 4) & 1, s_r16 = sh_head & 15;
  const int s_sb = quad >> 2, s_g = quad & 3;
  float m_ref = -__builtin_inff(), l_run = 0.f;

  const int t0 = split * a.tiles_per_split;
  const int t1 = min(t0 + a.tiles_per_split, a.n_tiles);
  const int eg = wave, c8 = lane;  // staging: slots 4eg..4eg+3, channels 8c8..8c8+7

  auto pv_product = [&](int vbuf) {
    const uint16_t* vb = sh.vb[vbuf];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int cg = 8 * cc + cb;
      const uint2 lo = *(const uint2*)(vb + vb_offset(cg, g, r16));
      const uint2 hi = *(const uint2*)(vb + vb_offset(cg, 4 + g, r16));
      const v8bf vf = __builtin_bit_cast(v8bf, v4u{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) o[cb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[hb], o[cb][hb], 0, 0, 0);
    }
  };

  RawSlot raw[4];
  int e_nxt[4];
  if (t0 < t1) {
    int e0[4];
    load_ids(a, q, t0, eg, e0);
    issue_raw(a, q, t0, eg, c8, e0, raw);
    unsigned kw[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) decode_raw(raw[i], kw[i]);
    store_tile(sh, 0, eg, c8, kw, raw_ok(raw));
    if (t0 + 1 < t1) {
      load_ids(a, q, t0 + 1, eg, e0);
      issue_raw(a, q, t0 + 1, eg, c8, e0, raw);
    }
    if (t0 + 2 < t1) load_ids(a, q, t0 + 2, eg, e_nxt);
  }

  for (int t = t0; t < t1; ++t) {
    const int b = (t - t0) & 1;
    __syncthreads();  // tile t is in Kt and vb[b]; sx is free

    // ---- phase 1: S^T(t) over this wave's channel quarter; O^T += V^T(t-1) P^T(t-1)
    {
      v4f s[2][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) s[sb][hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const v8bf kf =
              __builtin_bit_cast(v8bf, *(const v4u*)(sh.kt + kt_offset(16 * sb + r16, 16 * cc + 4 * ks + g)));
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
            s[sb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[hb][ks], s[sb][hb], 0, 0, 0);
        }
      if (t > t0) pv_product(b ^ 1);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) sh.sx[wave][2 * sb + hb][lane] = s[sb][hb];
    }
    __syncthreads();  // partial sums written; Kt and vb[b^1] are no longer read

    // ---- phase 2: softmax of this lane's head over slots 4quad..4quad+3
    {
      v4f tot = sh.sx[s_hh][2 * s_sb + s_hb][16 * s_g + s_r16];
#pragma unroll
      for (int c = 1; c < 4; ++c) tot += sh.sx[s_hh + 2 * c][2 * s_sb + s_hb][16 * s_g + s_r16];
      const unsigned okw = sh.ok[b][quad];
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = ((okw >> (8 * r)) & 1u) ? tot[r] * a.scale_log2 : -__builtin_inff();
      float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mt = fmaxf(mt, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mt), 0x128, 0xF, 0xF, false)));  // lane ^ 8
      mt = max_xor16(mt);
      mt = max_xor32(mt);
      float al = 1.f;
      if (mt > m_ref + kRescaleSlack) {  // also true when m_ref = -inf and mt is finite
        al = (m_ref == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m_ref - mt);
        l_run *= al;
        m_ref = mt;
      }
      const bool live = m_ref != -__builtin_inff();
      float p[4], ps = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = live ? __builtin_amdgcn_exp2f(x[r] - m_ref) : 0.f;
        ps += p[r];
      }
      ps += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ps), 0x128, 0xF, 0xF, false));
      ps = add_xor16(ps);
      ps = add_xor32(ps);
      l_run += ps;
      uint2 pk;
      pk.x = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)p[0]) |
             ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)p[1]) << 16);
      pk.y = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)p[2]) |
             ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)p[3]) << 16);
      sh.pl[sh_head][quad] = pk;
      if (quad == 0) sh.alpha[sh_head] = al;
    }
    // ---- tile t+1 to LDS, latents of tile t+2 and ids of tile t+3 requested
    if (t + 1 < t1) {
      unsigned kw[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) decode_raw(raw[i], kw[i]);
      store_tile(sh, b ^ 1, eg, c8, kw, raw_ok(raw));
    }
    if (t + 2 < t1) {
      issue_raw(a, q, t + 2, eg, c8, e_nxt, raw);
      if (t + 3 < t1) load_ids(a, q, t + 3, eg, e_nxt);
    }
    __syncthreads();  // P^T and the rescale factors of tile t are written

    // ---- phase 3: pick up P^T(t); rescale O^T where a reference moved
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int head = 32 * hh + 16 * hb + r16;
      const uint2 lo = sh.pl[head][g], hi = sh.pl[head][4 + g];
      pb[hb] = __builtin_bit_cast(v8bf, v4u{lo.x, lo.y, hi.x, hi.y});
      const float al = sh.alpha[head];
      if (__any(al != 1.f)) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) o[cb][hb] *= al;
      }
    }
  }
  // O^T += V^T P^T of the last tile (its V^T buffer is no longer written)
  if (t0 < t1) pv_product((t1 - 1 - t0) & 1);
  if (quad == 0) {
    sh.fin_m[sh_head] = m_ref;
    sh.fin_l[sh_head] = l_run;
  }
  __syncthreads();

  // ---- epilogue: this wave's heads x channel quarter
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = 32 * hh + 16 * hb + r16;
    const float mh = sh.fin_m[head], lh = sh.fin_l[head];
    if (a.n_splits == 1) {
      const float inv = (lh > 0.f) ? 1.f / lh : 0.f;
      uint16_t* orow = a.out + ((int64_t)q * kHeads + head) * kDim + 128 * cc;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const int ch = cb * 16 + 4 * g;
        __bf16 b0 = (__bf16)(o[cb][hb][0] * inv), b1 = (__bf16)(o[cb][hb][1] * inv);
        __bf16 b2 = (__bf16)(o[cb][hb][2] * inv), b3 = (__bf16)(o[cb][hb][3] * inv);
        uint2 pk;
        pk.x = (unsigned)__builtin_bit_cast(uint16_t, b0) | ((unsigned)__builtin_bit_cast(uint16_t, b1) << 16);
        pk.y = (unsigned)__builtin_bit_cast(uint16_t, b2) | ((unsigned)__builtin_bit_cast(uint16_t, b3) << 16);
        *(uint2*)(orow + ch) = pk;
      }
      if (a.lse && cc == 0 && g == 0)
        a.lse[(int64_t)q * kHeads + head] = (lh > 0.f) ? (mh + __log2f(lh)) * kLn2 : -__builtin_inff();
    } else {
      // this split's partial record, merged by k_attn_combine
      float* part = a.partial + ((int64_t)q * a.n_splits + split) * kPartialFloats;
      if (cc == 0 && g == 0) {
        part[head] = mh;
        part[64 + head] = lh;
      }
      float* po = part + 128 + (int64_t)head * kDim + 128 * cc;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) *(v4f*)(po + cb * 16 + 4 * g) = o[cb][hb];
    }
  }
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
  k_sparse_attn<<<grid, NT, 0, s>>>(a);
  if (plan.n_splits > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_attn_combine<<<dim3(16, (unsigned)L.Q), 256, 0, s>>>(partial, plan.n_splits, L.out, L.lse);
  }
  return hipGetLastError();
}

}  // namespace csa2
