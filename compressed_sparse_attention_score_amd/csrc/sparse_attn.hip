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
//  * Per tile t, two barrier-separated phases: (1) P^T of tile t-1 picked
//    up (O^T rescaled if a head's reference moved), then S^T of tile t and
//    O^T += V^T P^T of tile t-1 back to back on the matrix cores; (2) the
//    softmax of tile t, and tile t+1 dequantised into LDS (V^T
//    double-buffered, K single-buffered), with the latents of tile t+2
//    requested at the start of the step.
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
//  * Window rows are bf16, or FP8 (MXFP8: 512 E4M3 codes + 16 E8M0 scales,
//    528 bytes, the pages' window entry size) decoded to bf16 at staging like
//    the latents. With a RoPE table, the 64 rotary channels of the output are
//    rotated back by each query's angles in the epilogue that writes it.
#include "csa2_device.h"
#include "csa2_internal.h"
#include "select_device.h"

namespace csa2 {

namespace {
constexpr int TILE = 32;
constexpr int NT = 512;  // threads per workgroup
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kSwa8Bytes = 528;  // FP8 window row: 512 E4M3 codes + 16 E8M0 scales
constexpr int kStageRow = kDim + 8;  // epilogue LDS row (bf16): 16 B of pad spreads the banks
constexpr int kRopeFirst = 448;  // first rotary channel; pairs (448+2i, 449+2i), i < 32
// Compacted candidates per thread when a split finishes the selection: 8 x
// 512 threads give each of up to 512 chunks at least 8 slots (a decode chunk
// keeps a few dozen survivors at most for random scores; more take the
// offset-table or streaming path).
constexpr int kSelReg = 8;

struct AttnArgs {
  const uint8_t* main_cache;
  const int32_t* idx;
  const uint16_t* q;
  const uint16_t* swa;   // bf16 window rows
  const uint8_t* swa8;   // FP8 window rows
  const float* rope;     // [Q][32][2] (cos, sin) or nullptr
  uint16_t* out;
  float* lse;
  float* partial;
  // Selection finished here (decode): chunk c of query q's compacted list
  // holds sel_counts[q][c] composites from sel_cand[q][c*sel_chunk] on.
  const unsigned* sel_counts;
  const unsigned long long* sel_cand;
  int64_t sel_n_cand;
  int sel_chunks, sel_chunk;
  int32_t* idx_out;  // selected ids [Q][k_sel] written by the split that holds them, or nullptr
  int64_t n_entries, cache_q_stride, swa_q_stride;
  int k_sel, n_swa, nj, n_tiles, tiles_per_split, n_splits;
  float scale_log2;
};

// Per-split partial record: fp32 m[64], fp32 l[64], then O[64][512] as bf16
// normalised by the split's own l (an average of V rows, so of the output's
// magnitude; one bf16 rounding). Sized in floats.
constexpr int64_t kPartialFloats = 64 + 64 + 64 * 512 / 2;
constexpr int kMaxSplits = 32;

struct AttnShared {
  union {
    struct {
      uint16_t kt[TILE * kDim];     // [slot][channel], 16-byte chunks swizzled
      uint16_t vb[2][TILE * kDim];  // blocked V^T, double-buffered
    };
    uint16_t ostage[kHeads * kStageRow];  // epilogue: the 64 output rows (bf16)
    SelScratch<NT> sel;                   // prologue: finishing the selection
  };
  v4f sx[8][4][64];                 // partial S^T per wave: [wave][2*sb+hb][lane]
  // P^T as bf16, 4 slots per entry: [slot quad][head], head h of quad q at
  // column h ^ (8 * (q >> 1)) of a 640-byte row (pl_col). A reader's 32
  // lanes take 16 consecutive heads of two quads (two 128-byte runs, 128
  // bytes apart modulo the 256-byte bank width); a writer's 32 lanes store 8
  // heads of four quads (four 64-byte runs, moved apart by the swizzle).
  uint2 pl[TILE / 4][kHeads + 16];
  float alpha[kHeads];              // per-head rescale of O for this tile (1 = none)
  float fin_m[kHeads], fin_l[kHeads];
  unsigned ok[2][TILE / 4];         // slot validity bytes per tile (double-buffered)
  int32_t ids[kMaxSelected];        // this split's selected ids, from slot t0*TILE on
};
}  // namespace

// The staged raw data of one slot for this lane's 8 channels: a selected
// latent keeps its 4 code bytes in x and its E4M3 scale byte in y with bit 8
// set when the id is valid; a bf16 window row keeps its 8 bf16 in x..w; an
// FP8 window row keeps its 8 E4M3 codes in x, y and its E8M0 scale byte in z.
// Which of these a slot is follows from its index and the window format.
typedef v4u RawSlot;

// This lane's 8 channels of FP8 window row `row` (codes 8c8..8c8+7, scale of
// their 32-channel block).
__device__ __forceinline__ RawSlot load_swa8(const uint8_t* rowp, int c8) {
  const uint2 c = *(const uint2*)(rowp + 8 * c8);
  return v4u{c.x, c.y, (unsigned)rowp[512 + (c8 >> 2)], 0u};
}

// Channels 8c8..8c8+7 of the 4 slots of tile t (slot group eg), ids from LDS.
// A tile holds only selected latents or only window rows unless k_sel is not
// a multiple of the tile: those two cases issue every load unconditionally
// (invalid slots read row 0 of the query's cache or window and are flagged),
// so all loads stay in flight together; a mixed tile takes a per-slot path.
template <bool SWA8>
__device__ __forceinline__ void issue_raw(const AttnArgs& a, const AttnShared& sh, int q, int t, int t0, int eg,
                                          int c8, RawSlot* r) {
  const int s0 = t * TILE;
  const int32_t* ids = sh.ids + (s0 - t0 * TILE) + 4 * eg;
  if (s0 + TILE <= a.k_sel && a.n_entries > 0) {
    const uint8_t* base = a.main_cache + (int64_t)q * a.cache_q_stride * kMainBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = ids[i];
      const bool ok = e >= 0 && (int64_t)e < a.n_entries;
      const uint8_t* ent = base + (int64_t)(ok ? e : 0) * kMainBytes;
      r[i] = v4u{*(const unsigned*)(ent + c8 * 4), (unsigned)ent[256 + (c8 >> 1)] | (ok ? 0x100u : 0u), 0u, 0u};
    }
    return;
  }
  if (s0 >= a.k_sel) {  // window rows only (this tile exists, so n_swa >= 1)
    if (SWA8) {
      const uint8_t* base = a.swa8 + (int64_t)q * a.swa_q_stride * kSwa8Bytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = s0 + 4 * eg + i;
        r[i] = load_swa8(base + (int64_t)(slot < a.nj ? slot - a.k_sel : 0) * kSwa8Bytes, c8);
      }
    } else {
      const uint16_t* base = a.swa + (int64_t)q * a.swa_q_stride * kDim + c8 * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = s0 + 4 * eg + i;
        r[i] = *(const v4u*)(base + (int64_t)(slot < a.nj ? slot - a.k_sel : 0) * kDim);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = s0 + 4 * eg + i;
    r[i] = v4u{0u, 0u, 0u, 0u};
    if (slot < a.k_sel) {
      const int e = ids[i];
      if (e >= 0 && (int64_t)e < a.n_entries) {
        const uint8_t* ent = a.main_cache + ((int64_t)q * a.cache_q_stride + e) * kMainBytes;
        r[i] = v4u{*(const unsigned*)(ent + c8 * 4), (unsigned)ent[256 + (c8 >> 1)] | 0x100u, 0u, 0u};
      }
    } else if (slot < a.nj) {
      const int64_t row = (int64_t)q * a.swa_q_stride + (slot - a.k_sel);
      if (SWA8)
        r[i] = load_swa8(a.swa8 + row * kSwa8Bytes, c8);
      else
        r[i] = *(const v4u*)(a.swa + row * kDim + c8 * 8);
    }
  }
}

// Window row of a slot as 4 bf16 pairs: passed through (bf16) or decoded
// (FP8: E4M3 times a power of two, exact in bf16 inside its normal range).
template <bool SWA8>
__device__ __forceinline__ void window_pairs(const RawSlot& r, unsigned* win) {
  if (SWA8) {
    const float ws = e8m0_to_f32(r[2]);
    const v2f v[4] = {__builtin_amdgcn_cvt_pk_f32_fp8((int)r[0], false), __builtin_amdgcn_cvt_pk_f32_fp8((int)r[0], true),
                      __builtin_amdgcn_cvt_pk_f32_fp8((int)r[1], false), __builtin_amdgcn_cvt_pk_f32_fp8((int)r[1], true)};
#pragma unroll
    for (int j = 0; j < 4; ++j) win[j] = pack_bf16x2_exact(v[j].x * ws, v[j].y * ws);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) win[j] = r[j];
  }
}

// kw[i][j] = channels 8c8+2j (bits 15:0) and 8c8+2j+1 (bits 31:16) of slot
// 4eg+i of tile t as bf16: a latent decoded, a window row passed through or
// decoded, an empty slot zeros (its loaded bytes may be anything, NaN
// included). A tile of latents only or of window rows only (all but at most
// one tile per query) decodes only its own kind; the test is uniform over the
// workgroup. *okb gets the validity byte of each slot.
template <bool SWA8>
__device__ __forceinline__ void decode_tile(const AttnArgs& a, int t, int eg, const RawSlot* r, unsigned (*kw)[4],
                                            unsigned* okb) {
  const int s0 = t * TILE;
  const bool all_lat = s0 + TILE <= a.k_sel, all_win = s0 >= a.k_sel;
  unsigned ob = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = s0 + 4 * eg + i;
    const bool latent = slot < a.k_sel, window = !latent && slot < a.nj;
    const bool lat_ok = latent && (r[i][1] & 0x100u);
    unsigned dec[4] = {0u, 0u, 0u, 0u}, win[4] = {0u, 0u, 0u, 0u};
    if (!all_win) {
      float f[8];
      decode_e2m1x8_scaled(r[i][0], e4m3_to_f32_hw(r[i][1] & 0xFFu), f);
#pragma unroll
      for (int j = 0; j < 4; ++j) dec[j] = pack_bf16x2_exact(f[2 * j], f[2 * j + 1]);
    }
    if (!all_lat) window_pairs<SWA8>(r[i], win);
#pragma unroll
    for (int j = 0; j < 4; ++j) kw[i][j] = lat_ok ? dec[j] : window ? win[j] : 0u;
    ob |= ((lat_ok || window) ? 1u : 0u) << (8 * i);
  }
  *okb = ob;
}

// Element offset of channel chunk `chunk` (8 channels, 16 bytes) of Kt row
// `slot`; chunks are XOR-swizzled by the row so that a store of one row by 64
// lanes and a fragment read of 16 rows at one chunk both touch 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int kt_offset(int slot, int chunk) { return slot * kDim + ((chunk ^ (slot & 15)) << 3); }

// V^T block of (channel group cg, slot group sg): 16 channels x 4 slots, 128
// bytes. Block order within a channel group alternates with the parity of
// cg ^ (cg >> 3), and chunk c (channel c of the group, 4 slots = 8 bytes)
// sits at (c + cg) & 15: a fragment read (16 channels of 4 consecutive slot
// groups) covers 512 contiguous bytes, and in a store of one slot group by 64
// lanes (32 channel groups) each 32 lanes served together touch 32 distinct
// 8-byte bank pairs (groups cg and cg + 8, which share a chunk position, sit
// in opposite 128-byte halves).
__device__ __forceinline__ int vb_offset(int cg, int sg, int c) {
  return ((cg * 8 + (sg ^ ((cg ^ (cg >> 3)) & 1))) * 16 + ((c + cg) & 15)) * 4;
}

// Slot of element e (a lane's partial S^T fragment) in a wave's row of the
// partial-sum exchange: bit 3 flipped in the upper half, so that a softmax
// read (8 consecutive elements from each of two halves) touches 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int sx_slot(int e) { return e ^ ((e & 16) >> 1); }

// Column of head h in row q of the P^T exchange (see AttnShared::pl).
__device__ __forceinline__ int pl_col(int q, int h) { return h ^ (8 * (q >> 1)); }

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

// Channels (a, b) of one rotary pair rotated back by the angle whose cosine
// and sine are cs: (a c + b s, b c - a s).
__device__ __forceinline__ void unrotate(float& x, float& y, float2 cs) {
  const float a = x, b = y;
  x = a * cs.x + b * cs.y;
  y = b * cs.x - a * cs.y;
}

template <bool SWA8, bool FUSED>
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

  // The split's selected ids, into LDS once: read from the id list, or
  // (FUSED) taken from the exact selection over the query's compacted
  // candidates, which every split holding selected slots finishes for itself
  // (the same result in each) and writes its own range of to idx_out.
  {
    const int sbeg = t0 * TILE, send = min(t1 * TILE, a.k_sel);
    if (FUSED) {
      if (sbeg < send) {  // uniform over the workgroup
        int32_t* io = a.idx_out ? a.idx_out + (int64_t)q * a.k_sel : nullptr;
        select_from_regions<NT, kSelReg>(a.sel_counts + (int64_t)q * a.sel_chunks, a.sel_chunks, a.sel_chunk, a.sel_n_cand,
                                a.k_sel, a.sel_cand + (int64_t)q * a.sel_n_cand, sh.sel, sbeg, send,
                                [&](unsigned pos, unsigned long long x) {
                                  const int32_t id = x ? (int32_t)(~(unsigned)(x & 0xFFFFFFFFull)) : -1;
                                  sh.ids[pos - sbeg] = id;
                                  if (io) io[pos] = id;
                                });
      }
    } else {
      for (int sl = sbeg + tid; sl < send; sl += NT) sh.ids[sl - sbeg] = a.idx[(int64_t)q * a.k_sel + sl];
    }
  }
  __syncthreads();  // ids in LDS; the selection scratch (over the tile area) is free

  // Pipeline: tile t is multiplied from LDS while tile t+1 (raw data already
  // in registers) is dequantised into the other buffer and the latents of
  // tile t+2 are in flight; the two raw buffers alternate by a 2x unrolled
  // loop so no loaded register is copied before it is consumed.
  RawSlot rawA[4], rawB[4];
  if (t0 < t1) {
    issue_raw<SWA8>(a, sh, q, t0, t0, eg, c8, rawA);
    unsigned kw[4][4], okb;
    decode_tile<SWA8>(a, t0, eg, rawA, kw, &okb);
    store_tile(sh, 0, eg, c8, kw, okb);
    if (t0 + 1 < t1) issue_raw<SWA8>(a, sh, q, t0 + 1, t0, eg, c8, rawA);
  }

  // Pick up P^T of the last softmaxed tile; rescale O^T where a head's
  // reference moved. Runs after the barrier that follows that softmax, and
  // before the barrier after which the next softmax rewrites pl and alpha.
  auto pickup = [&]() {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int head = 32 * hh + 16 * hb + r16;
      const uint2 lo = sh.pl[g][pl_col(g, head)], hi = sh.pl[4 + g][pl_col(4 + g, head)];
      pb[hb] = __builtin_bit_cast(v8bf, v4u{lo.x, lo.y, hi.x, hi.y});
      const float al = sh.alpha[head];
      if (__any(al != 1.f)) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) o[cb][hb] *= al;
      }
    }
  };

  // One tile: nxt holds the raw data of tile t+1, fut receives tile t+2's.
  // Two barriers per tile: the P^T pickup of tile t-1 opens the step.
  auto step = [&](int t, RawSlot* nxt, RawSlot* fut) {
    const int b = (t - t0) & 1;
    __syncthreads();  // tile t is in Kt and vb[b]; P^T(t-1) and its rescale factors are written; sx is free
    if (t + 2 < t1) issue_raw<SWA8>(a, sh, q, t + 2, t0, eg, c8, fut);
    if (t > t0) pickup();

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
        for (int hb = 0; hb < 2; ++hb) sh.sx[wave][2 * sb + hb][sx_slot(lane)] = s[sb][hb];
    }
    __syncthreads();  // partial sums written; Kt and vb[b^1] are no longer read

    // ---- phase 2: softmax of this lane's head over slots 4quad..4quad+3
    {
      const int sxe = sx_slot(16 * s_g + s_r16);
      v4f tot = sh.sx[s_hh][2 * s_sb + s_hb][sxe];
#pragma unroll
      for (int c = 1; c < 4; ++c) tot += sh.sx[s_hh + 2 * c][2 * s_sb + s_hb][sxe];
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
      sh.pl[quad][pl_col(quad, sh_head)] = pk;
      if (quad == 0) sh.alpha[sh_head] = al;
    }
    // ---- tile t+1 to LDS
    if (t + 1 < t1) {
      unsigned kw[4][4], okb;
      decode_tile<SWA8>(a, t + 1, eg, nxt, kw, &okb);
      store_tile(sh, b ^ 1, eg, c8, kw, okb);
    }
  };
  for (int t = t0; t < t1; t += 2) {
    step(t, rawA, rawB);
    if (t + 1 < t1) step(t + 1, rawB, rawA);
  }
  // O^T += V^T P^T of the last tile (its V^T buffer is no longer written)
  __syncthreads();  // P^T of the last tile and its rescale factors are written
  if (t0 < t1) {
    pickup();
    pv_product((t1 - 1 - t0) & 1);
  }
  if (quad == 0) {
    sh.fin_m[sh_head] = m_ref;
    sh.fin_l[sh_head] = l_run;
  }
  __syncthreads();

  // ---- epilogue: O / l as bf16 (rotary channels rotated back when a table is
  // given and this is the only split; a split's partial record is rotated
  // after the merge), staged in LDS over the free Kt / V^T area as 64 padded
  // rows, then written as whole 1-KiB rows: one row per wave store instead of
  // sixteen 32-byte pieces of different rows.
  const float* rope = (a.n_splits == 1 && a.rope && cc == 3) ? a.rope + (int64_t)q * 64 : nullptr;
  uint16_t* stage = sh.ostage;  // over kt / vb, no longer read
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = 32 * hh + 16 * hb + r16;
    const float mh = sh.fin_m[head], lh = sh.fin_l[head];
    const float inv = (lh > 0.f) ? 1.f / lh : 0.f;
    if (a.n_splits == 1) {
      if (a.lse && cc == 0 && g == 0)
        a.lse[(int64_t)q * kHeads + head] = (lh > 0.f) ? (mh + __log2f(lh)) * kLn2 : -__builtin_inff();
    } else if (cc == 0 && g == 0) {
      float* part = a.partial + ((int64_t)q * a.n_splits + split) * kPartialFloats;
      part[head] = mh;
      part[64 + head] = lh;
    }
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int ch = cb * 16 + 4 * g;
      float v0 = o[cb][hb][0] * inv, v1 = o[cb][hb][1] * inv, v2 = o[cb][hb][2] * inv, v3 = o[cb][hb][3] * inv;
      if (cb >= 4 && rope) {  // channels 384 + ch >= 448: pairs (384 + ch - 448) / 2 and +1
        unrotate(v0, v1, *(const float2*)(rope + (ch - 64)));  // the table is 8-B aligned
        unrotate(v2, v3, *(const float2*)(rope + (ch - 62)));
      }
      __bf16 b0 = (__bf16)v0, b1 = (__bf16)v1, b2 = (__bf16)v2, b3 = (__bf16)v3;
      uint2 pk;
      pk.x = (unsigned)__builtin_bit_cast(uint16_t, b0) | ((unsigned)__builtin_bit_cast(uint16_t, b1) << 16);
      pk.y = (unsigned)__builtin_bit_cast(uint16_t, b2) | ((unsigned)__builtin_bit_cast(uint16_t, b3) << 16);
      *(uint2*)(stage + head * kStageRow + 128 * cc + ch) = pk;
    }
  }
  __syncthreads();
  uint16_t* obase = (a.n_splits == 1)
                        ? a.out + (int64_t)q * kHeads * kDim
                        : (uint16_t*)(a.partial + ((int64_t)q * a.n_splits + split) * kPartialFloats + 128);
#pragma unroll
  for (int k = 0; k < kHeads * kDim / 8 / NT; ++k) {  // 16-B chunks; a wave covers one head row
    const int i = k * NT + tid, head = i >> 6, chunk = i & 63;
    __builtin_nontemporal_store(*(const v4u*)(stage + head * kStageRow + chunk * 8), (v4u*)(obase + head * kDim + chunk * 8));
  }
}

// Merge the splits of one query: with O_s stored as O_s / l_s,
// out = sum_s (O_s / l_s) l_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), in split
// order. grid (16, Q), 256 threads:
// thread -> head blockIdx.x*4 + tid/64, channels (tid%64)*8 .. +7. MS is the
// split capacity of the instantiation (n_splits <= MS): every split's (m, l)
// and O row are requested together (clamped indices, zero weight past the
// last split), so the merge costs one memory round trip.
template <int MS>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ partial, int n_splits,
                                                      const float* __restrict__ rope, uint16_t* __restrict__ out,
                                                      float* __restrict__ lse) {
  const int q = blockIdx.y, tid = threadIdx.x;
  const int h = blockIdx.x * 4 + (tid >> 6), c0 = (tid & 63) * 8;
  const float* base = partial + (int64_t)q * n_splits * kPartialFloats;
  float ms[MS], ls[MS];
  v4u x[MS];
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    const int ss = min(sp, n_splits - 1);
    ms[sp] = base[ss * kPartialFloats + h];
    ls[sp] = base[ss * kPartialFloats + 64 + h];
    x[sp] = *(const v4u*)((const uint16_t*)(base + ss * kPartialFloats + 128) + (int64_t)h * kDim + c0);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load above issued before any use
  float M = -__builtin_inff();
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) M = (sp < n_splits) ? fmaxf(M, ms[sp]) : M;
  // every weight is 0 when no split holds a slot (M = -inf), so no branch
  float L = 0.f;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    const float f =  // weight of split sp: l 2^(m - M)
        (sp < n_splits && ms[sp] != -__builtin_inff()) ? ls[sp] * __builtin_amdgcn_exp2f(ms[sp] - M) : 0.f;
    L += f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[2 * c] += __uint_as_float(x[sp][c] << 16) * f;
      acc[2 * c + 1] += __uint_as_float(x[sp][c] & 0xFFFF0000u) * f;
    }
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] *= inv;
  if (rope && c0 >= kRopeFirst) {  // pairs (c0 - 448) / 2 .. +3
    const float* cs = rope + (int64_t)q * 64 + (c0 - kRopeFirst);
#pragma unroll
    for (int j = 0; j < 4; ++j) unrotate(acc[2 * j], acc[2 * j + 1], *(const float2*)(cs + 2 * j));
  }
  v4u pk;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    __bf16 lo = (__bf16)acc[2 * j], hi = (__bf16)acc[2 * j + 1];
    pk[j] = (unsigned)__builtin_bit_cast(uint16_t, lo) | ((unsigned)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  *(v4u*)(out + ((int64_t)q * kHeads + h) * kDim + c0) = pk;
  if (lse && (tid & 63) == 0)
    lse[(int64_t)q * kHeads + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

AttnPlan plan_attn(int Q, int nj) {
  // As many splits as keep every workgroup of the launch resident at once
  // (one per CU): one tile per split when that fits, else at least 2 tiles
  // per split so the gather of the next tile overlaps the current one; at
  // most kMaxSplits splits.
  AttnPlan p;
  p.n_tiles = (nj + TILE - 1) / TILE;
  if (p.n_tiles < 1) p.n_tiles = 1;
  const int want = (Q > 0) ? 256 / Q : 1;
  int tps = (want > 0) ? (p.n_tiles + want - 1) / want : p.n_tiles;
  if (tps < 2 && !(tps == 1 && p.n_tiles <= kMaxSplits)) tps = 2;
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
  a.swa = (const uint16_t*)L.swa;
  a.swa8 = (const uint8_t*)L.swa;
  a.rope = L.rope;
  a.out = L.out;
  a.lse = L.lse;
  a.partial = partial;
  a.sel_counts = L.sel_counts;
  a.sel_cand = L.sel_cand;
  a.sel_n_cand = L.sel_n_cand;
  a.sel_chunks = L.sel_chunks;
  a.sel_chunk = L.sel_chunk;
  a.idx_out = L.idx_out;
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
  const bool fused = L.sel_counts != nullptr;
  if (L.swa_fp8) {
    if (fused)
      k_sparse_attn<true, true><<<grid, NT, 0, s>>>(a);
    else
      k_sparse_attn<true, false><<<grid, NT, 0, s>>>(a);
  } else {
    if (fused)
      k_sparse_attn<false, true><<<grid, NT, 0, s>>>(a);
    else
      k_sparse_attn<false, false><<<grid, NT, 0, s>>>(a);
  }
  if (plan.n_splits > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid(16, (unsigned)L.Q);
    if (plan.n_splits <= 4)
      k_attn_combine<4><<<grid, 256, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 8)
      k_attn_combine<8><<<grid, 256, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 12)  // 640 slots over 16 queries: 10 splits
      k_attn_combine<12><<<grid, 256, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 16)
      k_attn_combine<16><<<grid, 256, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 24)  // 640 slots over 4 or fewer queries: 20 splits
      k_attn_combine<24><<<grid, 256, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
    else
      k_attn_combine<kMaxSplits><<<grid, 256, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
  }
  return hipGetLastError();
}

}  // namespace csa2
