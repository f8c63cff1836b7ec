// Sparse attention over the selected FP4 latents plus the sliding window.
//
// Method ("An infra-oriented diagram of the DeepSeek-V4.1-Flash architecture",
// Reading notes): one 512-wide latent per cache entry, shared by all 64 query
// heads, serving as both key and value; each layer attends over the 128-token
// window plus the 512 selected entries.
//
// Mapping: one workgroup of 4 waves = one query, one half of the 64 heads
// (32), one range of the joint slot list (the whole list for large batches;
// small batches split it so that the launch fills the chip, and a second
// kernel merges the (max, sum, O) partials). Two workgroups share a CU (56
// KB of LDS, at most 256 VGPRs each). Wave w owns channels 128w..128w+127
// throughout. A query's workgroups are dispatched to one XCD, whose L2 then
// serves the second head half's reads of each slot. Window rows come first
// (their bytes do not wait for the selection), then the selected latents, in
// tiles of 32 slots of one kind. Per tile, between two barriers:
//  * QK: wave w decodes the 32 slots' channels 128w.. straight from the
//    loaded bytes into MFMA operands (lane = slot, 8 channels per k-step;
//    lane group g takes channels 128w+32g..+31, so each lane loads 16
//    contiguous code bytes) and forms the partial S^T[32 slots x 32 heads]
//    over its channels with q in registers (the same channel order).
//    Latents decode to fp16: E2M1 times the power-of-two part of the E4M3
//    scale in one convert, then the scale's mantissa in one packed multiply
//    (the product has at most 6 significant bits, so both steps are exact);
//    q enters those products as fp16 times a per-head power of two that
//    keeps it in fp16's range, taken back out of the logits. Window rows stay
//    bf16 (exact). The decoded values also go to LDS (the tile's rows,
//    swizzled) as the values, and the partial sums go to LDS.
//  * Softmax: each wave takes 8 heads, adds the four partial sums and runs
//    the online softmax for those heads over the 32 slots (lane = head, one
//    run of 4 slots); P^T goes to LDS in the layout the PV product takes
//    (lane = head, slots 4g..4g+3 and 16+4g..16+4g+3). The running maximum
//    is a reference that moves only when a head's tile maximum exceeds it
//    by more than 2^8 (log2 units), so O is rescaled a handful of times per
//    query; the factor goes to LDS with P.
//  * PV: wave w owns channels 128w..128w+127 of the 32 heads:
//    O^T[128 x 32] += V^T P^T, the V^T operand read back from the rows it
//    decoded itself by gfx950's transposing LDS read (ds_read_b64_tr_b16:
//    within each 16-lane group, lanes 4j..4j+3 each point at 4 consecutive
//    elements of row j and lane i receives element i of rows 0..3).
// The bytes of the next two latent tiles are in flight meanwhile.
// Window rows are bf16, or FP8 (MXFP8: 512 E4M3 codes + 16 E8M0 scales, 528
// bytes, the pages' window entry size) decoded to bf16 like the latents. With
// a RoPE table, the 64 rotary channels of the output are rotated back by each
// query's angles before the bf16 rounding.
#include "csa2_device.h"
#include "csa2_internal.h"
#include "select_device.h"
#include "../../include/csa2.h"

#include <type_traits>

namespace csa2 {

namespace {
constexpr int TILE = 32;
constexpr int NT = 256;     // threads per workgroup (4 waves)
constexpr int kWaves = NT / 64;
constexpr int kHalves = 2;                 // workgroups per (query, slot range)
constexpr int kHeadsWg = kHeads / kHalves;  // heads per workgroup
constexpr int kHB = kHeadsWg / 16;          // head blocks of 16 (MFMA columns)
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr float kRefFloor = -0x1p126f;  // initial reference max (log2 units)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kSwa8Bytes = 528;  // FP8 window row: 512 E4M3 codes + 16 E8M0 scales
constexpr int kRopeFirst = 448;  // first rotary channel; pairs (448+2i, 449+2i), i < 32
// Compacted candidates per thread when the workgroup finishes the selection:
// 16 x 256 threads give each of up to 256 chunks at least 16 slots (a decode
// chunk keeps a few dozen survivors at most for random scores; more take the
// offset-table or streaming path).
constexpr int kSelReg = 16;
// Partial record of one (query, slot range): reference max m[64] and sum
// l[64] (log2 units), then O[64][512] normalised by the range's own l, as
// bf16 (an average of value rows, so of the output's magnitude; one bf16
// rounding). Sized in floats.
constexpr int kPartFloats = 2 * kHeads + kHeads * kDim / 2;
static_assert(kPartFloats == (int)kAttnPartialFloats, "partial record size");
// Slot ranges a launch aims at (two workgroups each, one per CU) when it
// splits the list, the fewest tiles a range may hold, and the most ranges.
constexpr int kTargetWgs = kAttnTargetWgs;
constexpr int kMinTilesPerSplit = 2;
constexpr int kMaxSplits = 32;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

struct AttnArgs {
  const uint8_t* main_cache;
  const int32_t* idx;
  const uint16_t* q;
  const uint16_t* swa;   // bf16 window rows
  const uint8_t* swa8;   // FP8 window rows
  const float* rope;     // [Q][32][2] (cos, sin) or nullptr
  uint16_t* out;
  float* lse;
  float* partial;        // [Q][n_split][kPartFloats] when n_split > 1
  // Selection finished here (decode): chunk c of query q's compacted list
  // holds sel_counts[q][c] composites from sel_cand[q][c*sel_chunk] on.
  const unsigned* sel_counts;
  const unsigned long long* sel_cand;
  int64_t sel_n_cand;
  int sel_chunks, sel_chunk;
  int32_t* idx_out;  // selected ids [Q][k_sel], or nullptr
  // or straight from the raw scores of a short plain range (sel_scores)
  const float* sel_scores;
  const int32_t* sel_n_valid;
  int64_t n_entries, cache_q_stride, swa_q_stride;
  int Q, k_sel, n_swa, n_split, tps;
  float scale_log2;
};

struct AttnShared {
  union {
    uint16_t v[TILE * kDim];  // the tile's rows (16-bit), swizzled (v_offset)
    struct {
      SelScratch<NT> sc;
      alignas(16) unsigned long long list[NT * kBalCand];
    } sel;                    // prologue: finishing the selection
  };
  v4f sx[kWaves][kHB][2][64];   // partial S^T: [channel quarter][head block][slot block][sx_idx]
  v4u px[kHB][64];              // P^T operands: [head block][lane]
  float alpha[kHB][16];         // O rescale factor per head (1 when unchanged)
  unsigned resc[kHB][2];        // nonzero when some head of the block's half rescales
  alignas(16) float mask[TILE];  // per slot of the tile: 0 (valid) or -inf, added to its logits
  unsigned qmax[kWaves][kHeadsWg];  // per channel quarter, each head's largest |q| (bf16 bits)
  float ml[2][kHeadsWg];        // end: each head's reference max and sum
  alignas(16) float rope[64];   // the query's (cos, sin) table (final outputs with a table)
  int32_t ids[kMaxSelected];    // the query's selected ids (by list position)
};

// Raw bytes of this lane's two slots (tile slots r16 and 16 + r16) for its 32
// channels 128w+32g.., as loaded. A selected latent: 16 code bytes and 2 E4M3
// scale bytes per slot. A window row: 64 bytes of bf16 per slot (FP8 rows: 32
// code bytes in w.[0..1] and the E8M0 scale bytes in s0, s1). ok: the slot holds a
// valid latent or window row.
// Each loaded value stays in a register of its own until it is decoded: a
// value combined from two loads right away would make the compiler wait for
// the newest loads there, and the tiles in flight would gain nothing.
struct RawLat {
  v4u c0, c1;
  unsigned s0, s1;  // scale dwords of slot r16, of slot 16 + r16 (the lane's two bytes at 16*(g&1))
  bool ok0, ok1;
};
struct RawWin {
  v4u w0[4], w1[4];
  unsigned s0, s1;
  bool ok0, ok1;
};
// x + x[lane ^ 8] and max(x, x[lane ^ 8]): a rotation by 8 within each row
// of 16 lanes (DPP row_ror:8).
__device__ __forceinline__ float add_xor8(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float max_xor8(float x) {
  return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false)));
}

// Latent tiles whose bytes are in flight ahead of the one being processed
// (register ring; the loop is unrolled by this so every index is static).
constexpr int kRing = 2;
}  // namespace

// Element offset of (slot, channel) in a tile: rows of 512 channels (1 KB),
// each row 64 granules of 16 bytes (8 channels). Channel chunk C = c/16
// (32 bytes) and half h = (c/8) & 1 go to granule
// 16*(C/8) + 8*h + ((C & 7) ^ (s & 7)). Measured with bank-conflict counters
// on this part: a 16-byte LDS store is conflict-free when each run of 8
// consecutive lanes writes 8 distinct granules of one 128-byte half of a
// 256-byte bank row, a 16-byte load when each run of 16 lanes covers the 16
// granules of a bank row, and the transposing 8-byte load when each run of
// 32 lanes covers the 64 banks. Here a row store (lanes r..r+7: rows
// s..s+7, one chunk half) fills one half, and a transposing read (8 rows x
// the 32 bytes of one chunk) fills a whole bank row. (The previous layout,
// chunk C at C ^ (s & 7), spread each run of 8 row stores over both halves:
// every row store took two passes, with no measurable change in time.)
__device__ __forceinline__ int v_offset(int s, int c) {
  const int C = c >> 4;
  return s * kDim + ((16 * (C >> 3) + 8 * ((c >> 3) & 1) + ((C & 7) ^ (s & 7))) << 3) + (c & 7);
}

// Selected latents at list positions tile*32 + r16 and +16 (none past
// k_sel), channels 128w + 32g .. +31.
__device__ __forceinline__ void load_latent(const AttnArgs& a, const AttnShared& sh, int q, int tile, int w, int g,
                                            int r16, RawLat& r) {
  const int s0 = tile * TILE + r16, s1 = s0 + 16;
  const int e0 = s0 < a.k_sel ? sh.ids[s0] : -1;
  const int e1 = s1 < a.k_sel ? sh.ids[s1] : -1;
  r.ok0 = e0 >= 0 && (int64_t)e0 < a.n_entries;
  r.ok1 = e1 >= 0 && (int64_t)e1 < a.n_entries;
  const int64_t base = (int64_t)q * a.cache_q_stride;
  const uint8_t* p0 = a.main_cache + (base + (r.ok0 ? e0 : 0)) * kMainBytes;
  const uint8_t* p1 = a.main_cache + (base + (r.ok1 ? e1 : 0)) * kMainBytes;
  r.c0 = *(const v4u*)(p0 + 64 * w + 16 * g);
  r.c1 = *(const v4u*)(p1 + 64 * w + 16 * g);
  // whole aligned dwords (two 16-bit loads could share a register, and
  // then neither could be used before both arrived)
  r.s0 = *(const unsigned*)(p0 + 256 + 8 * w + 4 * (g >> 1));
  r.s1 = *(const unsigned*)(p1 + 256 + 8 * w + 4 * (g >> 1));
}

// Window rows tile*32 + r16 and +16 (valid below n_swa), channels
// 128w + 32g .. +31.
template <bool SWA8>
__device__ __forceinline__ void load_window(const AttnArgs& a, int q, int tile, int w, int g, int r16, RawWin& r) {
  const int j0 = tile * TILE + r16, j1 = j0 + 16;
  r.ok0 = j0 < a.n_swa;
  r.ok1 = j1 < a.n_swa;
  const int64_t row0 = (int64_t)q * a.swa_q_stride + (r.ok0 ? j0 : 0);
  const int64_t row1 = (int64_t)q * a.swa_q_stride + (r.ok1 ? j1 : 0);
  if (SWA8) {
    const uint8_t* p0 = a.swa8 + row0 * kSwa8Bytes;
    const uint8_t* p1 = a.swa8 + row1 * kSwa8Bytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      r.w0[i] = *(const v4u*)(p0 + 128 * w + 32 * g + 16 * i);
      r.w1[i] = *(const v4u*)(p1 + 128 * w + 32 * g + 16 * i);
    }
    r.s0 = p0[512 + 4 * w + g];
    r.s1 = p1[512 + 4 * w + g];
  } else {
    const uint16_t* p0 = a.swa + row0 * kDim + 128 * w + 32 * g;
    const uint16_t* p1 = a.swa + row1 * kDim + 128 * w + 32 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.w0[i] = *(const v4u*)(p0 + 8 * i);
      r.w1[i] = *(const v4u*)(p1 + 8 * i);
    }
  }
}

// E4M3 scale byte -> (power-of-two part as f32, mantissa in [1, 2) as an
// fp16 pair). Byte 0 (taken for an invalid slot, an integer select, so that
// no branch separates the loads from their uses) gives zero, so that slot's
// codes, whatever they are, decode to zeros.
struct LatScale {
  float p2;
  v2h m2;
};
__device__ __forceinline__ LatScale lat_scale(unsigned sbyte) {
  const unsigned sb = __float_as_uint(e4m3_to_f32_hw(sbyte));
  LatScale s;
  s.p2 = __uint_as_float(sb & 0x7F800000u);
  const _Float16 mh = (_Float16)__uint_as_float((sb & 0x007FFFFFu) | 0x3F800000u);
  s.m2 = v2h{mh, mh};
  return s;
}

// One k-step (8 channels, one code dword) of a latent as fp16: E2M1 x 2^E by
// the scaled convert, times the E4M3 scale's mantissa m by one packed
// multiply (scale = 2^E m; both steps exact).
__device__ __forceinline__ v4u decode_latent(unsigned w, const LatScale& s) {
  v2h h[4];
  h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 0) * s.m2;
  h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 1) * s.m2;
  h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 2) * s.m2;
  h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 3) * s.m2;
  return v4u{__builtin_bit_cast(unsigned, h[0]), __builtin_bit_cast(unsigned, h[1]), __builtin_bit_cast(unsigned, h[2]),
             __builtin_bit_cast(unsigned, h[3])};
}

// k-step ks of a window row (slot block sb) as bf16: passed through, or
// E4M3 x 2^(E8M0-127) (FP8), exact while it stays a normal bf16.
template <bool SWA8>
__device__ __forceinline__ v4u decode_window(const RawWin& r, int sb, int ks) {
  const v4u* wv = sb ? r.w1 : r.w0;
  const bool ok = sb ? r.ok1 : r.ok0;
  v4u out;
  if (SWA8) {
    const float ws = e8m0_to_f32(sb ? r.s1 : r.s0);
    const unsigned c0 = wv[ks >> 1][2 * (ks & 1)], c1 = wv[ks >> 1][2 * (ks & 1) + 1];
    const v2f v[4] = {__builtin_amdgcn_cvt_pk_f32_fp8((int)c0, false), __builtin_amdgcn_cvt_pk_f32_fp8((int)c0, true),
                      __builtin_amdgcn_cvt_pk_f32_fp8((int)c1, false), __builtin_amdgcn_cvt_pk_f32_fp8((int)c1, true)};
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = pack_bf16x2_exact(v[j].x * ws, v[j].y * ws);
  } else {
    out = wv[ks];
  }
  return ok ? out : v4u{0u, 0u, 0u, 0u};
}

// Channels (a, b) of one rotary pair rotated back by the angle whose cosine
// and sine are cs: (a c + b s, b c - a s).
__device__ __forceinline__ void unrotate(float& x, float& y, float2 cs) {
  const float a = x, b = y;
  x = a * cs.x + b * cs.y;
  y = b * cs.x - a * cs.y;
}

// bf16 pair -> the pair times f (a power of two) as fp16.
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned u, float f) {
  const v2h h = {(_Float16)(__uint_as_float(u << 16) * f), (_Float16)(__uint_as_float(u & 0xFFFF0000u) * f)};
  return __builtin_bit_cast(unsigned, h);
}

// Two fp32 values rounded (to nearest even) into bf16x2, lo in bits 15:0:
// one paired conversion (two single conversions, a shift and an or when
// written as two scalar casts).
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((v2f){lo, hi}, v2bf16));
}

template <bool SWA8, bool FUSED>
__global__ __launch_bounds__(NT, 2) void k_sparse_attn(AttnArgs a) {
  // workgroup -> (query, slot range, head half): the workgroups of a query
  // are 8 ids apart, so they land on one XCD, whose L2 serves both head
  // halves' reads of each latent
  const int ns = a.n_split;
  const int per_q = kHalves * ns;
  const int lin = blockIdx.x;
  const int q = ((lin / (8 * per_q)) << 3) | (lin & 7);
  const int w_in = (lin >> 3) % per_q;
  const int split = w_in >> 1, hh = w_in & 1;
  if (q >= a.Q) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int h0 = kHeadsWg * hh;  // first head of this workgroup

  __shared__ AttnShared sh;

  // this workgroup's tiles: window tiles [w0, w1), then latent tiles [l0, l1)
  const int n_wt = (a.n_swa + TILE - 1) / TILE;
  const int n_lt = (a.k_sel + TILE - 1) / TILE;
  const int T0 = split * a.tps, T1 = min(T0 + a.tps, n_wt + n_lt);
  const int w0 = min(T0, n_wt), w1 = min(T1, n_wt);
  const int l0 = max(T0, n_wt) - n_wt, l1 = max(T1, n_wt) - n_wt;

  // q^T operands: head h0 + 16*hb + r16, channels 128w + 32g + 8ks .. +7
  // (bf16 while the window tiles run, then fp16 scaled)
  v4u qr[kHB][4];
  {
    const uint16_t* qrow = a.q + ((int64_t)q * kHeads + h0 + r16) * kDim + 128 * w + 32 * g;
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qr[hb][ks] = *(const v4u*)(qrow + (int64_t)16 * hb * kDim + 8 * ks);
  }
  // the query's RoPE table, for the epilogue (a load without a condition:
  // the first floats of q stand in when there is no table)
  const float rope_v = (a.rope ? a.rope + (int64_t)q * 64 : (const float*)a.q)[lane];
  RawWin rwA, rwB;
  if (w1 > w0) load_window<SWA8>(a, q, w0, w, g, r16, rwA);
  if (w1 > w0 + 1) load_window<SWA8>(a, q, w0 + 1, w, g, r16, rwB);
  // each head's largest |q| over this wave's channels (bf16 magnitude bits
  // order like the values): the lane's 32, then over the 4 lane groups
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    unsigned qm = 0u;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) qm = max(qm, max(qr[hb][ks][j] & 0x7FFFu, (qr[hb][ks][j] >> 16) & 0x7FFFu));
    qm = umax_xor16(qm);
    qm = umax_xor32(qm);
    if (g == 0) sh.qmax[w][16 * hb + r16] = qm;
  }

  // The selected ids of this workgroup's latent tiles, into LDS: read from
  // the id list, or (FUSED) taken from the exact selection over the query's
  // compacted candidates, which every workgroup holding latent tiles
  // finishes for itself (the same result in each).
  const int sbeg = l0 * TILE, send = min(l1 * TILE, a.k_sel);
  if (FUSED) {
    if (sbeg < send) {  // uniform over the workgroup
      int32_t* io = (a.idx_out && hh == 0) ? a.idx_out + (int64_t)q * a.k_sel : nullptr;
      auto emit = [&](unsigned pos, unsigned long long x) {
        const int32_t id = x ? (int32_t)(~(unsigned)(x & 0xFFFFFFFFull)) : -1;
        sh.ids[pos] = id;
        if (io) io[pos] = id;
      };
      if (a.sel_scores) {
        int64_t limit = a.n_entries;
        if (a.sel_n_valid) limit = min(limit, (int64_t)a.sel_n_valid[q]);
        select_from_scores<NT, kRawSelectMax / NT>(a.sel_scores + (int64_t)q * a.sel_n_cand, a.sel_n_cand, limit,
                                                   a.k_sel, sh.sel.sc, sbeg, send, emit,
                                                   (unsigned (*)[kBins])sh.sel.list);  // unused on this path
      } else {
        select_from_regions<NT, kSelReg>(a.sel_counts + (int64_t)q * a.sel_chunks, a.sel_chunks, a.sel_chunk,
                                         a.sel_n_cand, a.k_sel, a.sel_cand + (int64_t)q * a.sel_n_cand, sh.sel.sc,
                                         sh.sel.list, sbeg, send, emit);
      }
    }
  } else {
    for (int sl = sbeg + tid; sl < send; sl += NT) sh.ids[sl] = a.idx[(int64_t)q * a.k_sel + sl];
  }
  __syncthreads();  // ids and q maxima in LDS; the selection scratch (over the tile area) is free
  if (w == 0) sh.rope[lane] = rope_v;  // read after the barrier that ends the tiles

  // q scaled into fp16's range for the latent products: 2^k with the head's
  // largest |q| times 2^k in [2^14, 2^15) (k clamped to +-100); logits of
  // latent tiles are multiplied back by 2^-k. (h: head within the workgroup)
  auto head_k2 = [&](int h) {
    const unsigned qmh = max(max(sh.qmax[0][h], sh.qmax[1][h]), max(sh.qmax[2][h], sh.qmax[3][h]));
    const int qe = (qmh == 0u) ? 127 : (int)(qmh >> 7);  // bf16 biased exponent
    return min(100, max(-100, 14 - (qe - 127)));
  };
  // softmax role: wave w takes heads h0 + 16*shb + 8*shalf .. +7 (shb = w/2,
  // shalf = w%2); lane (sr8, sgq, ssb) holds head shead's slots
  // 16*ssb + 4*sgq .. +3, and the 8 lanes of a head reduce by lane swaps.
  // (Two waves of 16 heads each left the other two idle between the
  // barriers: prefill attention took 652 us against 623 us.)
  const int shb = w >> 1, shalf = w & 1;
  const int sr8 = lane & 7, sgq = (lane >> 3) & 3, ssb = lane >> 5;
  const int shead = 16 * shb + 8 * shalf + sr8;
  const bool slead = (lane >> 3) == 0;
  const float lat_log2 = a.scale_log2 * __uint_as_float((unsigned)(127 - head_k2(shead)) << 23);
  // position in a [head block][slot block] row of sx of the MFMA output of
  // lane (g, r16 = 8*half + r8): the 8 heads of a softmax wave's lane group
  // sit together, XOR-swizzled so that 16 consecutive lanes of either side
  // touch 16 distinct 16-byte bank groups
  auto sx_idx = [](int half, int gg, int r8) { return (32 * half + 8 * gg + r8) ^ (8 * half); };

  // O^T accumulators: channels 128w + 16cb + 4g + j, head h0 + 16hb + r16
  v4f o[kHB][8];
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) o[hb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
  // softmax role: reference max (log2 units; a finite floor below any
  // logit until the first valid slot, so that no -inf - -inf arises) and sum
  float m_ref = kRefFloor, l_run = 0.f;

  // transposing-read addresses (element offsets, cb = 0) of the PV operand:
  // lanes 4j..4j+3 of a 16-lane group point at row 4*g + j (then 16 + 4*g + j)
  // and channels 128w + 4*(lane & 3) ..
  const int tr_row = 4 * g + ((lane & 15) >> 2), tr_c = 128 * w + 4 * (lane & 3);

  // Per tile, between two barriers:
  //  qk: decode + partial S^T of this wave's channels -> sx, rows -> v
  //  softmax (8 heads per wave) over the tile -> px, alpha, resc
  //  pv: O rescale (when flagged) and O += V^T P^T
  // Each buffer is single: a wave rewrites its own rows of v only after its
  // pv has read them, sx only after the barrier that ends every softmax
  // read, and px, alpha, resc and ok are rewritten only after the barrier
  // that follows every wave's pv.
  using Bf16Tag = std::integral_constant<bool, false>;
  using F16Tag = std::integral_constant<bool, true>;
  auto qk = [&](bool ok0, bool ok1, auto f16_tag, auto&& kstep) {
    constexpr bool F16 = decltype(f16_tag)::value;
    v4f s[2][kHB];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) s[sb][hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const v4u kf = kstep(sb, ks);
        *(v4u*)(sh.v + v_offset(16 * sb + r16, 128 * w + 32 * g + 8 * ks)) = kf;
#pragma unroll
        for (int hb = 0; hb < kHB; ++hb) {
          if constexpr (F16)
            s[sb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, kf),
                                                               __builtin_bit_cast(v8h, qr[hb][ks]), s[sb][hb], 0, 0, 0);
          else
            s[sb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(v8bf, kf), __builtin_bit_cast(v8bf, qr[hb][ks]), s[sb][hb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) sh.sx[w][hb][sb][sx_idx(r16 >> 3, g, r16 & 7)] = s[sb][hb];
    if (w == 0 && g == 0) {
      sh.mask[r16] = ok0 ? 0.f : -__builtin_inff();
      sh.mask[16 + r16] = ok1 ? 0.f : -__builtin_inff();
    }
  };
  auto softmax = [&](auto f16_tag) {
    constexpr bool F16 = decltype(f16_tag)::value;
    // lane: head h0 + shead, slots 16*ssb + 4*sgq .. +3
    const float sl2 = F16 ? lat_log2 : a.scale_log2;
    const int si = sx_idx(shalf, sgq, sr8);
    v4f s0 = sh.sx[0][shb][ssb][si];
#pragma unroll
    for (int c = 1; c < kWaves; ++c) s0 += sh.sx[c][shb][ssb][si];
    const v4f mk0 = *(const v4f*)&sh.mask[16 * ssb + 4 * sgq];
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = fmaf(s0[j], sl2, mk0[j]);
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = max_xor8(mt);
    mt = max_xor16(mt);
    mt = max_xor32(mt);
    // the reference moves (also from the floor, when the first valid slot
    // comes): O and l are scaled by al, 0 from the floor (both are still 0
    // then)
    const bool moved = mt > m_ref + kRescaleSlack;
    float al = 1.f;
    if (moved) {
      al = __builtin_amdgcn_exp2f(m_ref - mt);
      l_run *= al;
      m_ref = mt;
    }
    float p[4], ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = __builtin_amdgcn_exp2f(x[j] - m_ref);
      ps += p[j];
    }
    ps = add_xor8(ps);
    ps = add_xor16(ps);
    ps = add_xor32(ps);
    l_run += ps;
    v2u pk;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (F16)
        pk[j] = __builtin_bit_cast(unsigned, v2h{(_Float16)p[2 * j], (_Float16)p[2 * j + 1]});
      else
        pk[j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
    }
    *((v2u*)&sh.px[shb][16 * sgq + 8 * shalf + sr8] + ssb) = pk;
    if (slead) sh.alpha[shb][8 * shalf + sr8] = al;
    const bool any = __builtin_amdgcn_ballot_w64(moved) != 0ull;
    if (lane == 0) sh.resc[shb][shalf] = any ? 1u : 0u;
  };
  auto pv = [&](auto f16_tag) {
    constexpr bool F16 = decltype(f16_tag)::value;
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      if (__builtin_amdgcn_readfirstlane(sh.resc[hb][0] | sh.resc[hb][1])) {
        const float al = sh.alpha[hb][r16];
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) o[hb][cb] *= al;
      }
    }
    v4u pk[kHB];
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) pk[hb] = sh.px[hb][lane];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(sh.v + v_offset(tr_row, tr_c + 16 * cb)));
      const v4s hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(sh.v + v_offset(16 + tr_row, tr_c + 16 * cb)));
      const auto vt = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) {
        if constexpr (F16)
          o[hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, vt),
                                                             __builtin_bit_cast(v8h, pk[hb]), o[hb][cb], 0, 0, 0);
        else
          o[hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, vt),
                                                              __builtin_bit_cast(v8bf, pk[hb]), o[hb][cb], 0, 0, 0);
      }
    }
  };
  auto rest = [&](auto f16_tag) {  // after qk: the two barriers, softmax and pv
    __syncthreads();
    softmax(f16_tag);
    __syncthreads();
    pv(f16_tag);
  };
  auto qk_win = [&](const RawWin& r) {
    qk(r.ok0, r.ok1, Bf16Tag{}, [&](int sb, int ks) { return decode_window<SWA8>(r, sb, ks); });
  };
  auto qk_lat = [&](const RawLat& r) {
    LatScale ls[2][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const bool ok = sb ? r.ok1 : r.ok0;
#pragma unroll
      for (int h = 0; h < 2; ++h) ls[sb][h] = lat_scale(ok ? ((sb ? r.s1 : r.s0) >> (16 * (g & 1) + 8 * h)) & 0xFFu : 0u);
    }
    qk(r.ok0, r.ok1, F16Tag{}, [&](int sb, int ks) { return decode_latent(sb ? r.c1[ks] : r.c0[ks], ls[sb][ks >> 1]); });
  };

  // tiles: window n = 0..nw-1 (at most four, straight-line code), then
  // latent i = 0..nl-1 (latent tile l0 + i in ring slot i % kRing). Ring
  // loads past the list are issued all the same (positions past it flagged
  // invalid).
  static_assert(CSA2_MAX_SWA <= 4 * TILE, "at most four window tiles");
  const int nw = w1 - w0, nl = l1 - l0;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    if (n < nw) {
      qk_win((n & 1) ? rwB : rwA);
      if (n + 2 < nw) load_window<SWA8>(a, q, w0 + n + 2, w, g, r16, (n & 1) ? rwB : rwA);
      rest(Bf16Tag{});
    }
  }
  // The first latent tiles' bytes are requested only now: with no load
  // issued under a condition between these and the loop, every wait in the
  // loop counts exactly the loads issued after the slot it needs.
  RawLat ring[kRing];
#pragma unroll
  for (int j = 0; j < kRing; ++j) load_latent(a, sh, q, l0 + j, w, g, r16, ring[j]);
  if (nl > 0) {
    // q to fp16, scaled per head
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      const float qs = __uint_as_float((unsigned)(head_k2(16 * hb + r16) + 127) << 23);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) qr[hb][ks][j] = bf16x2_to_f16x2(qr[hb][ks][j], qs);
    }
  }
  // Whole groups of kRing tiles run without conditions, so that each wait
  // for a ring slot counts exactly the loads issued after it (a load under a
  // condition makes the wait at the next join count conservatively, which
  // here means waiting for every tile in flight); the last nl % kRing tiles
  // follow.
  int i0 = 0;
  for (; i0 + kRing <= nl; i0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      qk_lat(ring[j]);
      load_latent(a, sh, q, l0 + i0 + j + kRing, w, g, r16, ring[j]);
      rest(F16Tag{});
    }
  }
#pragma unroll
  for (int j = 0; j < kRing - 1; ++j) {
    if (i0 + j < nl) {
      qk_lat(ring[j]);
      rest(F16Tag{});
    }
  }

  // ---- every head's reference max and sum to all waves
  if (slead) {
    sh.ml[0][shead] = m_ref;
    sh.ml[1][shead] = l_run;
  }
  __syncthreads();
  // ---- epilogue: O / l rounded once to bf16 (the rotary channels of a
  // final output rotated back first), staged by each wave in its own
  // quarter of the tile rows (which every wave has finished reading) as
  // [32 heads][its 128 channels], so that each store then writes 256
  // contiguous bytes of four rows instead of 32 bytes of sixteen. Lane
  // (head h0 + 16hb + r16, g) holds channels 128w + 16cb + 4g .. +3; the
  // rotary pairs (448 + 2i, 449 + 2i) lie in wave 3's cb >= 4. A row's
  // sixteen 16-byte granules sit XOR-swizzled by the row (bank spread).
  uint16_t* stg = sh.v + w * (kHeadsWg * 128);
  auto stg_at = [](int row, int gran) { return row * 128 + ((gran ^ (row & 15)) << 3); };
  const bool split_out = a.n_split > 1;
  const bool rot = !split_out && a.rope != nullptr && w == kWaves - 1;
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    const float lh = sh.ml[1][16 * hb + r16];
    const float inv = (lh > 0.f) ? 1.f / lh : 0.f;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      float v0 = o[hb][cb][0] * inv, v1 = o[hb][cb][1] * inv, v2 = o[hb][cb][2] * inv, v3 = o[hb][cb][3] * inv;
      if (cb >= 4 && rot) {  // pairs (16*cb + 4*g - 64) / 2 and +1
        const int c0 = 16 * cb + 4 * g - 64;
        unrotate(v0, v1, *(const float2*)&sh.rope[c0]);
        unrotate(v2, v3, *(const float2*)&sh.rope[c0 + 2]);
      }
      v2u pk;
      pk.x = pack_bf16x2(v0, v1);
      pk.y = pack_bf16x2(v2, v3);
      *(v2u*)(stg + stg_at(16 * hb + r16, 2 * cb + (g >> 1)) + 4 * (g & 1)) = pk;
    }
  }
  uint16_t* dst;
  if (split_out) {
    // partial record (shared by the two head halves): m, l and O / l of
    // this slot range, with nontemporal stores (the merge, in the next
    // kernel, is the only reader; at 16 queries x 65,536 entries these
    // stores took about 2 us off the step against ordinary ones)
    float* part = a.partial + ((int64_t)q * ns + split) * kPartFloats;
    if (w == 0 && lane < kHeadsWg) {
      __builtin_nontemporal_store(sh.ml[0][lane], part + h0 + lane);
      __builtin_nontemporal_store(sh.ml[1][lane], part + kHeads + h0 + lane);
    }
    dst = (uint16_t*)(part + 2 * kHeads) + h0 * kDim;
  } else {
    if (a.lse && slead)
      a.lse[(int64_t)q * kHeads + h0 + shead] =
          (l_run > 0.f) ? (m_ref + __log2f(l_run)) * kLn2 : -__builtin_inff();
    dst = a.out + ((int64_t)q * kHeads + h0) * kDim;
  }
  // the staged block is read back by lanes of the same wave only (its LDS
  // accesses complete in order): lane l takes granule l & 15 of row
  // 4i + l/16
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < kHeadsWg / 4; ++i) {
    const int row = 4 * i + (lane >> 4), gran = lane & 15;
    const v4u x = *(const v4u*)(stg + stg_at(row, gran));
    __builtin_nontemporal_store(x, (v4u*)(dst + row * kDim + 128 * w + 8 * gran));
  }
}

// Merge the slot ranges of one query's head: with partial (m_s, l_s,
// P_s = O_s / l_s), out = sum_s P_s l_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// M = max_s m_s, in range order. grid (Q rounded up to 8, times 64):
// workgroup -> (query, head), the workgroups of query q 8 ids apart from
// q & 7 on, so that they run on the XCD whose workgroups wrote its records
// (the attention kernel's mapping; each batch of 8 ids goes round the 8
// XCDs), 64 threads -> 8 channels each. Every range's record is requested
// before any is used. (Against one query per run of 64 ids: config 1's step
// 40.7 -> 39.2 us, config 4's 76.8 -> 75.9 us, config 2's 54.1 -> 53.5 us.)
template <int MS>
__global__ __launch_bounds__(64) void k_attn_merge(const float* __restrict__ partial, int n_split, int n_q,
                                                   const float* __restrict__ rope, uint16_t* __restrict__ out,
                                                   float* __restrict__ lse) {
  const int lin = blockIdx.x;
  const int q = ((lin >> 9) << 3) | (lin & 7), h = (lin >> 3) & 63;
  if (q >= n_q) return;
  const int c0 = threadIdx.x * 8;
  const float* base = partial + (int64_t)q * n_split * kPartFloats;
  // the (cos, sin) of this thread's four rotary pairs, requested with the
  // records (a load without a condition: another thread's or the first
  // pairs stand in where they are not needed)
  const bool rot = rope != nullptr && c0 >= kRopeFirst;
  const float* csp = (rope ? rope : partial) + (rope ? (int64_t)q * 64 + max(c0 - kRopeFirst, 0) : 0);
  float2 cs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cs[j] = *(const float2*)(csp + 2 * j);
  float ms[MS], ls[MS];
  v4u x[MS];
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    const float* pr = base + (int64_t)min(sp, n_split - 1) * kPartFloats;
    ms[sp] = pr[h];
    ls[sp] = pr[kHeads + h];
    x[sp] = *(const v4u*)((const uint16_t*)(pr + 2 * kHeads) + h * kDim + c0);
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) M = (sp < n_split) ? fmaxf(M, ms[sp]) : M;
  float L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    // weight of range sp: l 2^(m - M); 0 past the last range or for a range
    // without a valid slot (every weight is 0 when no range holds one)
    const float f =
        (sp < n_split && ms[sp] != -__builtin_inff()) ? ls[sp] * __builtin_amdgcn_exp2f(ms[sp] - M) : 0.f;
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
  if (rot) {  // pairs (c0 - 448) / 2 .. +3
#pragma unroll
    for (int j = 0; j < 4; ++j) unrotate(acc[2 * j], acc[2 * j + 1], cs[j]);
  }
  v4u pk;
#pragma unroll
  for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
  __builtin_nontemporal_store(pk, (v4u*)(out + ((int64_t)q * kHeads + h) * kDim + c0));
  if (lse && threadIdx.x == 0)
    lse[(int64_t)q * kHeads + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

AttnPlan plan_attn(int Q, int k_sel, int n_swa) {
  // Window rows and selected latents are tiled apart. The slot list is split
  // only when the launch would hold fewer workgroups than CUs: into as many
  // ranges as bring it to about kTargetWgs workgroups, each of at least
  // kMinTilesPerSplit tiles.
  AttnPlan p;
  p.n_tiles = (k_sel + TILE - 1) / TILE + (n_swa + TILE - 1) / TILE;
  int ns = 1;
  if (Q > 0 && Q < kTargetWgs) ns = kTargetWgs / Q;
  ns = max(1, min(ns, min(kMaxSplits, p.n_tiles / kMinTilesPerSplit)));
  p.tiles_per_split = p.n_tiles > 0 ? (p.n_tiles + ns - 1) / ns : 1;
  p.n_splits = p.n_tiles > 0 ? (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split : 1;
  return p;
}

size_t attn_partial_bytes(int Q, const AttnPlan& plan) {
  if (plan.n_splits <= 1) return 0;
  // a split launch has Q * n_splits <= kTargetWgs workgroups, so this stays
  // within kAttnPartialMaxBytes
  return (size_t)Q * plan.n_splits * kPartFloats * sizeof(float);
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
  a.sel_scores = L.sel_scores;
  a.sel_n_valid = L.sel_n_valid;
  a.n_entries = L.n_entries;
  a.cache_q_stride = L.cache_q_stride;
  a.swa_q_stride = L.swa_q_stride;
  a.Q = L.Q;
  a.k_sel = L.k_sel;
  a.n_swa = L.n_swa;
  a.n_split = plan.n_splits;
  a.tps = plan.tiles_per_split;
  a.scale_log2 = L.scale * kLog2e;
  // The kernel issues its loads unconditionally (invalid slots flagged and
  // clamped to row 0): with no cache or no window rows it reads the first
  // row of q instead, a valid address, and every such slot stays invalid.
  if (L.main_cache == nullptr || L.n_entries <= 0) {
    a.main_cache = (const uint8_t*)L.q;
    a.n_entries = 0;
    a.cache_q_stride = 0;
  }
  if (L.swa == nullptr || L.n_swa <= 0) {
    a.swa = L.q;
    a.swa8 = (const uint8_t*)L.q;
    a.swa_q_stride = 0;
    a.n_swa = 0;
  }
  if (plan.n_splits > 1 && partial == nullptr) return hipErrorInvalidValue;
  const int q8 = (L.Q + 7) / 8 * 8;
  const dim3 grid((unsigned)(kHalves * plan.n_splits * q8));
  const bool fused = L.sel_counts != nullptr || L.sel_scores != nullptr;
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
    const dim3 mg((unsigned)(q8 * kHeads));
    if (plan.n_splits <= 2)
      k_attn_merge<2><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.Q, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 4)
      k_attn_merge<4><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.Q, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 8)
      k_attn_merge<8><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.Q, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 12)
      k_attn_merge<12><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.Q, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 16)
      k_attn_merge<16><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.Q, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 24)
      k_attn_merge<24><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.Q, L.rope, L.out, L.lse);
    else
      k_attn_merge<kMaxSplits><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.Q, L.rope, L.out, L.lse);
  }
  return hipGetLastError();
}

}  // namespace csa2
