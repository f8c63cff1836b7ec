// Sparse attention over the selected FP4 latents plus the sliding window.
//
// Method ("An infra-oriented diagram of the DeepSeek-V4.1-Flash architecture",
// Reading notes): one 512-wide latent per cache entry, shared by all 64 query
// heads, serving as both key and value; each layer attends over the 128-token
// window plus the 512 selected entries.
//
// Mapping: one workgroup of 4 waves = one query x one block of 16 heads x
// one range of the joint slot list (the whole list for large batches; small
// batches split it so that the launch fills the chip, and a second kernel
// merges the (max, sum, O) partials). A query's workgroups are dispatched to
// one XCD, whose L2 then serves the repeated reads of its latents. Window
// rows come first (their bytes do not wait for the selection), then the
// selected latents, in tiles of 32 slots of one kind. Per tile:
//  * QK: wave w = (slot block sb = w/2, channel half ch = w%2) decodes its 16
//    slots x 256 channels straight from the loaded bytes into MFMA operands
//    (lane = slot, 8 channels per k-step) and forms the partial S^T[16 slots
//    x 16 heads] with q for its channel half in registers. Latents decode to
//    fp16: E2M1 times the power-of-two part of the E4M3 scale in one convert,
//    then the scale's mantissa in one packed multiply (the product has at
//    most 6 significant bits, so both steps are exact); q enters those
//    products as fp16 times a per-head power of two that keeps it in fp16's
//    range, taken back out of the logits. Window rows stay bf16 (exact). The
//    decoded rows also go to LDS (one copy of the tile, swizzled) as the
//    values, and the four partial sums are exchanged through LDS.
//  * Softmax: every wave adds the four partial sums and runs the same online
//    softmax for the 16 heads over the 32 slots, so P^T stays in registers
//    in the layout the PV product takes (lane = head, slots 4g..4g+3 and
//    16+4g..16+4g+3), with no exchange. The running maximum is a reference
//    that moves only when a head's tile maximum exceeds it by more than 2^8
//    (log2 units), so O is rescaled a handful of times per query.
//  * PV: wave w owns channels 128w..128w+127: O^T[128 x 16] += V^T P^T, the
//    V^T operand read from the row-major tile by gfx950's transposing LDS
//    read (ds_read_b64_tr_b16: within each 16-lane group, lanes 4j..4j+3
//    each point at 4 consecutive elements of row j and lane i receives
//    element i of rows 0..3).
//  * One barrier per tile: the LDS tile and the partial sums are double
//    buffered; the bytes of the next four latent tiles are in flight.
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
constexpr int HEADS_WG = 16;
constexpr int kHeadBlocks = kHeads / HEADS_WG;
constexpr float kRescaleSlack = 8.f;  // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kSwa8Bytes = 528;  // FP8 window row: 512 E4M3 codes + 16 E8M0 scales
constexpr int kRopeFirst = 448;  // first rotary channel; pairs (448+2i, 449+2i), i < 32
// Compacted candidates per thread when the workgroup finishes the selection:
// 16 x 256 threads give each of up to 256 chunks at least 16 slots (a decode
// chunk keeps a few dozen survivors at most for random scores; more take the
// offset-table or streaming path).
constexpr int kSelReg = 16;
// Partial record of one (query, head block, slot range): reference max m[16]
// and sum l[16] (log2 units), then O[16][512] normalised by the range's own
// l, as bf16 (an average of value rows, so of the output's magnitude; one
// bf16 rounding). Sized in floats.
constexpr int kPartFloats = 2 * HEADS_WG + HEADS_WG * kDim / 2;
static_assert(kPartFloats == (int)kAttnPartialFloats, "partial record size");
// Workgroups a launch aims at (two per CU) when it splits slot ranges, and
// the fewest tiles a split may hold.
constexpr int kTargetWgs = kAttnTargetWgs;
constexpr int kMinTilesPerSplit = 2;
constexpr int kMaxSplits = 16;

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
  float* partial;        // [Q][4][n_split][kPartFloats] when n_split > 1
  // Selection finished here (decode): chunk c of query q's compacted list
  // holds sel_counts[q][c] composites from sel_cand[q][c*sel_chunk] on.
  const unsigned* sel_counts;
  const unsigned long long* sel_cand;
  int64_t sel_n_cand;
  int sel_chunks, sel_chunk;
  int32_t* idx_out;  // selected ids [Q][k_sel] (written by head block 0), or nullptr
  int64_t n_entries, cache_q_stride, swa_q_stride;
  int Q, k_sel, n_swa, n_split, tps;
  float scale_log2;
};

struct AttnShared {
  union {
    uint16_t v[2][TILE * kDim];  // the tile's rows (16-bit), double-buffered, swizzled (v_offset)
    SelScratch<NT> sel;          // prologue: finishing the selection
  };
  v4f sx[2][2][2][64];           // partial S^T: [buffer][slot block][channel half][lane]
  unsigned char ok[2][TILE];     // slot validity per tile (double-buffered)
  unsigned qmax[2][HEADS_WG];    // per channel half, each head's largest |q| (bf16 bits)
  int32_t ids[kMaxSelected];     // the query's selected ids (by list position)
};

// Raw bytes of this lane's slot (16 slots x 4 lane groups per wave) for its
// 256-channel half, as loaded. A selected latent: its 32 code bytes and 4
// E4M3 scale bytes. A window row: its 64 bf16 channels (FP8 rows: 64 codes
// in w[0..3] and the two E8M0 scale bytes in s). ok: the slot holds a valid
// latent or window row.
struct RawLat {
  v4u c0, c1;
  unsigned s;
  bool ok;
};
struct RawWin {
  v4u w[8];
  unsigned s;
  bool ok;
};
// Latent tiles whose bytes are in flight ahead of the one being processed
// (register ring; the loop is unrolled by this so every index is static).
constexpr int kRing = 4;
}  // namespace

// Element offset of (slot, channel) in a tile: rows of 512 channels; the
// 32-byte chunk c/16 of row s sits at chunk (c/16) ^ (s & 7), its 16-byte
// halves swapped when s & 8. A transposing read (8 rows x 32 bytes per 32
// lanes) and a row store (16 rows x 16 bytes per 16 lanes) both touch
// distinct banks.
__device__ __forceinline__ int v_offset(int s, int c) {
  return s * kDim + ((2 * ((c >> 4) ^ (s & 7)) + (((c >> 3) & 1) ^ ((s >> 3) & 1))) << 3) + (c & 7);
}

// Selected latent at list position `slot` (none past k_sel), channels
// 256*ch + 64*g .. +63.
__device__ __forceinline__ void load_latent(const AttnArgs& a, const AttnShared& sh, int q, int slot, int ch, int g,
                                            RawLat& r) {
  const int e = slot < a.k_sel ? sh.ids[slot] : -1;
  r.ok = e >= 0 && (int64_t)e < a.n_entries;
  const uint8_t* ent = a.main_cache + ((int64_t)q * a.cache_q_stride + (r.ok ? e : 0)) * kMainBytes;
  r.c0 = *(const v4u*)(ent + 128 * ch + 32 * g);
  r.c1 = *(const v4u*)(ent + 128 * ch + 32 * g + 16);
  r.s = *(const unsigned*)(ent + 256 + 16 * ch + 4 * g);
}

// Window row j (valid when j < n_swa), channels 256*ch + 64*g .. +63.
template <bool SWA8>
__device__ __forceinline__ void load_window(const AttnArgs& a, int q, int j, int ch, int g, RawWin& r) {
  r.ok = j < a.n_swa;
  const int64_t row = (int64_t)q * a.swa_q_stride + (r.ok ? j : 0);
  if (SWA8) {
    const uint8_t* p = a.swa8 + row * kSwa8Bytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = *(const v4u*)(p + 256 * ch + 64 * g + 16 * i);
    r.s = *(const unsigned short*)(p + 512 + 8 * ch + 2 * g);
  } else {
    const uint16_t* p = a.swa + row * kDim + 256 * ch + 64 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.w[i] = *(const v4u*)(p + 8 * i);
  }
}

// k-step ks (channels 256*ch + 64*g + 8*ks .. +7) of a latent as fp16:
// E2M1 x 2^E by the scaled convert, times the E4M3 scale's mantissa m in
// [1, 2) by one packed multiply (scale = 2^E m; both steps exact). An
// invalid slot takes scale byte 0, an integer select, so that no branch
// separates the loads from their uses; its bytes may be anything, and the
// zero scale gives zeros.
__device__ __forceinline__ v4u decode_latent(const RawLat& r, int ks) {
  const unsigned sbyte = r.ok ? (r.s >> (8 * (ks >> 1))) & 0xFFu : 0u;
  const unsigned sb = __float_as_uint(e4m3_to_f32_hw(sbyte));
  const float p2 = __uint_as_float(sb & 0x7F800000u);
  const _Float16 mh = (_Float16)__uint_as_float((sb & 0x007FFFFFu) | 0x3F800000u);
  const v2h m2 = {mh, mh};
  const unsigned w = (ks < 4) ? r.c0[ks] : r.c1[ks - 4];
  v2h h[4];
  h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 0) * m2;
  h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 1) * m2;
  h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 2) * m2;
  h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, p2, 3) * m2;
  return v4u{__builtin_bit_cast(unsigned, h[0]), __builtin_bit_cast(unsigned, h[1]), __builtin_bit_cast(unsigned, h[2]),
             __builtin_bit_cast(unsigned, h[3])};
}

// The same for a window row, as bf16: passed through, or E4M3 x
// 2^(E8M0-127) (FP8), exact while it stays a normal bf16.
template <bool SWA8>
__device__ __forceinline__ v4u decode_window(const RawWin& r, int ks) {
  v4u out;
  if (SWA8) {
    const float ws = e8m0_to_f32((r.s >> (8 * (ks >> 2))) & 0xFFu);
    const unsigned c0 = r.w[ks >> 1][2 * (ks & 1)], c1 = r.w[ks >> 1][2 * (ks & 1) + 1];
    const v2f v[4] = {__builtin_amdgcn_cvt_pk_f32_fp8((int)c0, false), __builtin_amdgcn_cvt_pk_f32_fp8((int)c0, true),
                      __builtin_amdgcn_cvt_pk_f32_fp8((int)c1, false), __builtin_amdgcn_cvt_pk_f32_fp8((int)c1, true)};
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = pack_bf16x2_exact(v[j].x * ws, v[j].y * ws);
  } else {
    out = r.w[ks];
  }
  return r.ok ? out : v4u{0u, 0u, 0u, 0u};
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

template <bool SWA8, bool FUSED>
__global__ __launch_bounds__(NT, 2) void k_sparse_attn(AttnArgs a) {
  // workgroup -> (query, head block, slot range): the workgroups of a query
  // are 8 ids apart, so they land on one XCD
  const int per_q = kHeadBlocks * a.n_split;
  const int lin = blockIdx.x;
  const int q = ((lin / (8 * per_q)) << 3) | (lin & 7);
  const int w_in = (lin >> 3) % per_q;
  const int hb = w_in / a.n_split, split = w_in - hb * a.n_split;
  if (q >= a.Q) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int sb = wave >> 1, ch = wave & 1;  // QK role
  const int cq = wave;                      // PV role: channels 128*cq ..
  const int my_slot = 16 * sb + r16;        // QK role: this lane's slot within a tile

  __shared__ AttnShared sh;

  // this workgroup's tiles: window tiles [w0, w1), then latent tiles [l0, l1)
  const int n_wt = (a.n_swa + TILE - 1) / TILE;
  const int n_lt = (a.k_sel + TILE - 1) / TILE;
  const int T0 = split * a.tps, T1 = min(T0 + a.tps, n_wt + n_lt);
  const int w0 = min(T0, n_wt), w1 = min(T1, n_wt);
  const int l0 = max(T0, n_wt) - n_wt, l1 = max(T1, n_wt) - n_wt;

  // q^T operand: head 16*hb + r16, channels 256*ch + 64*g + 8*ks .. +7
  v8bf qf[8];
  {
    const uint16_t* qrow = a.q + ((int64_t)q * kHeads + HEADS_WG * hb + r16) * kDim + 256 * ch + 64 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(v8bf, *(const v4u*)(qrow + 8 * ks));
  }
  RawWin rwA, rwB;
  if (w1 > w0) load_window<SWA8>(a, q, w0 * TILE + my_slot, ch, g, rwA);
  if (w1 > w0 + 1) load_window<SWA8>(a, q, (w0 + 1) * TILE + my_slot, ch, g, rwB);
  // this lane's largest |q| (bf16 magnitude bits order like the values),
  // over the 4 lane groups, then the two channel halves through LDS
  unsigned qm = 0u;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const v4u u = __builtin_bit_cast(v4u, qf[ks]);
#pragma unroll
    for (int j = 0; j < 4; ++j) qm = max(qm, max(u[j] & 0x7FFFu, (u[j] >> 16) & 0x7FFFu));
  }
  qm = umax_xor16(qm);
  qm = umax_xor32(qm);
  if (sb == 0 && g == 0) sh.qmax[ch][r16] = qm;

  // The selected ids of this workgroup's latent tiles, into LDS: read from
  // the id list, or (FUSED) taken from the exact selection over the query's
  // compacted candidates, which every workgroup holding latent tiles
  // finishes for itself (the same result in each).
  const int sbeg = l0 * TILE, send = min(l1 * TILE, a.k_sel);
  if (FUSED) {
    if (sbeg < send) {  // uniform over the workgroup
      int32_t* io = (a.idx_out && hb == 0) ? a.idx_out + (int64_t)q * a.k_sel : nullptr;
      select_from_regions<NT, kSelReg>(a.sel_counts + (int64_t)q * a.sel_chunks, a.sel_chunks, a.sel_chunk,
                                       a.sel_n_cand, a.k_sel, a.sel_cand + (int64_t)q * a.sel_n_cand, sh.sel, sbeg,
                                       send, [&](unsigned pos, unsigned long long x) {
                                         const int32_t id = x ? (int32_t)(~(unsigned)(x & 0xFFFFFFFFull)) : -1;
                                         sh.ids[pos] = id;
                                         if (io) io[pos] = id;
                                       });
    }
  } else {
    for (int sl = sbeg + tid; sl < send; sl += NT) sh.ids[sl] = a.idx[(int64_t)q * a.k_sel + sl];
  }
  __syncthreads();  // ids and q maxima in LDS; the selection scratch (over the tile area) is free
  RawLat ring[kRing];
#pragma unroll
  for (int j = 0; j < kRing; ++j) load_latent(a, sh, q, (l0 + j) * TILE + my_slot, ch, g, ring[j]);

  // q scaled into fp16's range for the latent products: 2^k with the head's
  // largest |q| times 2^k in [2^14, 2^15) (k clamped to +-100); logits of
  // latent tiles are multiplied back by 2^-k. lane (head r16, g): its head.
  const unsigned qmh = max(sh.qmax[0][r16], sh.qmax[1][r16]);
  const int qe = (qmh == 0u) ? 127 : (int)(qmh >> 7);  // bf16 biased exponent
  const int k2 = min(100, max(-100, 14 - (qe - 127)));
  const float qscale = __uint_as_float((unsigned)(k2 + 127) << 23);
  const float lat_log2 = a.scale_log2 * __uint_as_float((unsigned)(127 - k2) << 23);
  // (formed when the first latent tile comes, so that the bf16 and fp16
  // copies of q are not both held through the window tiles)
  v8h qh[8];
  auto make_qh = [&]() {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const v4u u = __builtin_bit_cast(v4u, qf[ks]);
      qh[ks] = __builtin_bit_cast(v8h, v4u{bf16x2_to_f16x2(u[0], qscale), bf16x2_to_f16x2(u[1], qscale),
                                           bf16x2_to_f16x2(u[2], qscale), bf16x2_to_f16x2(u[3], qscale)});
    }
  };

  // O^T accumulators: channels 128*cq + 16*cb + 4*g + j, head 16*hb + r16
  v4f o[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) o[cb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff(), l_run = 0.f;

  // transposing-read addresses (element offsets, cb = 0) of the PV operand:
  // lanes 4j..4j+3 of a 16-lane group point at row 4*g + j (then 16 + 4*g + j)
  // and channels 128*cq + 4*(lane & 3) ..
  const int tr_row = 4 * g + ((lane & 15) >> 2), tr_c = 128 * cq + 4 * (lane & 3);

  // The n-th tile of this workgroup uses LDS buffer n & 1. qk(): the tile's
  // QK with the k-step operands from `kstep` (fp16 latents or bf16 window
  // rows), its rows to LDS, the partial sums and slot flags; sv(): after
  // the barrier that follows qk(), the softmax and PV in the same type. The
  // latent loop is software-pipelined: qk() of tile n+1 comes before sv() of
  // tile n, so the decoding and matrix products of the next tile overlap the
  // softmax and value products of this one; one barrier per tile (buffers
  // n & 1 are next written by qk() of tile n+2, after the barrier that ends
  // sv() of tile n in every wave).
  using Bf16Tag = std::integral_constant<bool, false>;
  using F16Tag = std::integral_constant<bool, true>;
  auto qk = [&](int n, bool ok, auto f16_tag, auto&& kstep) {
    constexpr bool F16 = decltype(f16_tag)::value;
    const int b = n & 1;
    v4f s = v4f{0.f, 0.f, 0.f, 0.f};
    uint16_t* vb = sh.v[b];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const v4u kf = kstep(ks);
      *(v4u*)(vb + v_offset(my_slot, 256 * ch + 64 * g + 8 * ks)) = kf;
      if constexpr (F16)
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, kf), qh[ks], s, 0, 0, 0);
      else
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kf), qf[ks], s, 0, 0, 0);
    }
    sh.sx[b][sb][ch][lane] = s;
    if (ch == 0 && g == 0) sh.ok[b][my_slot] = ok ? 1 : 0;
  };
  auto sv = [&](int n, auto f16_tag) {
    constexpr bool F16 = decltype(f16_tag)::value;
    const int b = n & 1;
    const uint16_t* vb = sh.v[b];
    // softmax of the 16 heads over the tile (same in every wave): lane
    // (head r16, g) holds slots 4g..4g+3 and 16+4g..16+4g+3
    const float sl2 = F16 ? lat_log2 : a.scale_log2;
    const v4f s0 = sh.sx[b][0][0][lane] + sh.sx[b][0][1][lane];
    const v4f s1 = sh.sx[b][1][0][lane] + sh.sx[b][1][1][lane];
    const unsigned ok0 = *(const unsigned*)&sh.ok[b][4 * g], ok1 = *(const unsigned*)&sh.ok[b][16 + 4 * g];
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = ((ok0 >> (8 * j)) & 1u) ? s0[j] * sl2 : -__builtin_inff();
      x[4 + j] = ((ok1 >> (8 * j)) & 1u) ? s1[j] * sl2 : -__builtin_inff();
    }
    float mt = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
    mt = max_xor16(mt);
    mt = max_xor32(mt);
    if (mt > m_ref + kRescaleSlack) {  // also true when m_ref = -inf and mt is finite
      const float al = (m_ref == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m_ref - mt);
      l_run *= al;
      m_ref = mt;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) o[cb] *= al;
    }
    const bool live = m_ref != -__builtin_inff();
    float p[8], ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = live ? __builtin_amdgcn_exp2f(x[j] - m_ref) : 0.f;
      ps += p[j];
    }
    ps = add_xor16(ps);
    ps = add_xor32(ps);
    l_run += ps;
    v4u pk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (F16)
        pk[j] = __builtin_bit_cast(unsigned, v2h{(_Float16)p[2 * j], (_Float16)p[2 * j + 1]});
      else
        pk[j] = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)p[2 * j]) |
                ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)p[2 * j + 1]) << 16);
    }
    // PV: O^T[128 channels x 16 heads] += V^T P^T
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + v_offset(tr_row, tr_c + 16 * cb)));
      const v4s hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + v_offset(16 + tr_row, tr_c + 16 * cb)));
      const auto vt = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      if constexpr (F16)
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, vt), __builtin_bit_cast(v8h, pk), o[cb],
                                                        0, 0, 0);
      else
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, vt), __builtin_bit_cast(v8bf, pk),
                                                         o[cb], 0, 0, 0);
    }
  };
  auto qk_win = [&](int n, const RawWin& r) {
    qk(n, r.ok, Bf16Tag{}, [&](int ks) { return decode_window<SWA8>(r, ks); });
  };
  auto qk_lat = [&](int n, const RawLat& r) {
    qk(n, r.ok, F16Tag{}, [&](int ks) { return decode_latent(r, ks); });
  };

  // tiles: window n = 0..nw-1 (at most four, straight-line code, qk() then
  // sv() per tile: the two 128-byte window buffers per lane leave no room
  // for a second tile's state), then latent n = nw + i, i = 0..nl-1 (latent
  // tile l0 + i in ring slot i & 3), software-pipelined. Every ring load is
  // issued unconditionally (positions past the list flagged invalid), so
  // each wait counts exactly the loads it needs.
  static_assert(CSA2_MAX_SWA <= 4 * TILE, "at most four window tiles");
  const int nw = w1 - w0, nl = l1 - l0;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    if (n < nw) {
      qk_win(n, (n & 1) ? rwB : rwA);
      if (n + 2 < nw) load_window<SWA8>(a, q, (w0 + n + 2) * TILE + my_slot, ch, g, (n & 1) ? rwB : rwA);
      __syncthreads();
      sv(n, Bf16Tag{});
    }
  }
  if (nl > 0) {
    make_qh();
    qk_lat(nw, ring[0]);
    load_latent(a, sh, q, (l0 + kRing) * TILE + my_slot, ch, g, ring[0]);
    __syncthreads();
  }
  for (int i0 = 0; i0 < nl; i0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int i = i0 + j;
      if (i < nl) {
        if (i + 1 < nl) qk_lat(nw + i + 1, ring[(j + 1) & (kRing - 1)]);
        load_latent(a, sh, q, (l0 + i + 1 + kRing) * TILE + my_slot, ch, g, ring[(j + 1) & (kRing - 1)]);
        sv(nw + i, F16Tag{});
        __syncthreads();
      }
    }
  }

  const int head = HEADS_WG * hb + r16;
  if (a.n_split > 1) {
    // ---- partial record: m, l and O / l of this slot range
    float* part = a.partial + (((int64_t)q * kHeadBlocks + hb) * a.n_split + split) * kPartFloats;
    if (cq == 0 && g == 0) {
      part[r16] = m_ref;
      part[HEADS_WG + r16] = l_run;
    }
    const float pinv = (l_run > 0.f) ? 1.f / l_run : 0.f;
    uint16_t* orow = (uint16_t*)(part + 2 * HEADS_WG) + r16 * kDim + 128 * cq + 4 * g;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      v2u pk;
      pk.x = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)(o[cb][0] * pinv)) |
             ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)(o[cb][1] * pinv)) << 16);
      pk.y = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)(o[cb][2] * pinv)) |
             ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)(o[cb][3] * pinv)) << 16);
      *(v2u*)(orow + 16 * cb) = pk;
    }
    return;
  }

  // ---- epilogue: O / l as bf16 (rotary channels rotated back when a table
  // is given); lane (head r16, g) holds channels 128*cq + 16*cb + 4*g .. +3
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  if (a.lse && cq == 0 && g == 0)
    a.lse[(int64_t)q * kHeads + head] = (l_run > 0.f) ? (m_ref + __log2f(l_run)) * kLn2 : -__builtin_inff();
  const float* rope = (a.rope && cq == 3) ? a.rope + (int64_t)q * 64 : nullptr;
  uint16_t* orow = a.out + ((int64_t)q * kHeads + head) * kDim + 128 * cq + 4 * g;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    float v0 = o[cb][0] * inv, v1 = o[cb][1] * inv, v2 = o[cb][2] * inv, v3 = o[cb][3] * inv;
    if (cb >= 4 && rope) {  // channels 384 + 16*cb + 4*g >= 448: pairs (16*cb + 4*g - 64) / 2 and +1
      const int c0 = 16 * cb + 4 * g - 64;
      unrotate(v0, v1, *(const float2*)(rope + c0));  // the table is 8-B aligned
      unrotate(v2, v3, *(const float2*)(rope + c0 + 2));
    }
    v2u pk;
    pk.x = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)v0) | ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)v1) << 16);
    pk.y = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)v2) | ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)v3) << 16);
    __builtin_nontemporal_store(pk, (v2u*)(orow + 16 * cb));
  }
}

// Merge the slot ranges of one (query, head block): with partial (m_s, l_s,
// P_s = O_s / l_s), out = sum_s P_s l_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// M = max_s m_s, in range order. grid (Q * 64): workgroup -> (query, head),
// 64 threads -> 8 channels each. Every range's record is requested before
// any is used.
template <int MS>
__global__ __launch_bounds__(64) void k_attn_merge(const float* __restrict__ partial, int n_split,
                                                   const float* __restrict__ rope, uint16_t* __restrict__ out,
                                                   float* __restrict__ lse) {
  const int q = blockIdx.x >> 6, h = blockIdx.x & 63;
  const int hb = h >> 4, hl = h & 15, c0 = threadIdx.x * 8;
  const float* base = partial + ((int64_t)q * kHeadBlocks + hb) * n_split * kPartFloats;
  float ms[MS], ls[MS];
  v4u x[MS];
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    const float* pr = base + (int64_t)min(sp, n_split - 1) * kPartFloats;
    ms[sp] = pr[hl];
    ls[sp] = pr[HEADS_WG + hl];
    x[sp] = *(const v4u*)((const uint16_t*)(pr + 2 * HEADS_WG) + hl * kDim + c0);
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
  __builtin_nontemporal_store(pk, (v4u*)(out + ((int64_t)q * kHeads + h) * kDim + c0));
  if (lse && threadIdx.x == 0)
    lse[(int64_t)q * kHeads + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

AttnPlan plan_attn(int Q, int k_sel, int n_swa) {
  // Window rows and selected latents are tiled apart. The slot list is split
  // only when the launch would hold fewer than two workgroups per CU: into as
  // many ranges as bring it to about kTargetWgs workgroups, each of at least
  // kMinTilesPerSplit tiles.
  AttnPlan p;
  p.n_tiles = (k_sel + TILE - 1) / TILE + (n_swa + TILE - 1) / TILE;
  int ns = 1;
  if (Q > 0 && kHeadBlocks * Q < kTargetWgs) ns = kTargetWgs / (kHeadBlocks * Q);
  ns = max(1, min(ns, min(kMaxSplits, p.n_tiles / kMinTilesPerSplit)));
  p.tiles_per_split = p.n_tiles > 0 ? (p.n_tiles + ns - 1) / ns : 1;
  p.n_splits = p.n_tiles > 0 ? (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split : 1;
  return p;
}

size_t attn_partial_bytes(int Q, const AttnPlan& plan) {
  if (plan.n_splits <= 1) return 0;
  // a split launch has kHeadBlocks * Q * n_splits <= kTargetWgs workgroups,
  // so this stays within kAttnPartialMaxBytes
  return (size_t)Q * kHeadBlocks * plan.n_splits * kPartFloats * sizeof(float);
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
  const dim3 grid((unsigned)(kHeadBlocks * plan.n_splits * q8));
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
    const dim3 mg((unsigned)(L.Q * kHeads));
    if (plan.n_splits <= 2)
      k_attn_merge<2><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 4)
      k_attn_merge<4><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 8)
      k_attn_merge<8><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
    else if (plan.n_splits <= 12)
      k_attn_merge<12><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
    else
      k_attn_merge<kMaxSplits><<<mg, 64, 0, s>>>(partial, plan.n_splits, L.rope, L.out, L.lse);
  }
  return hipGetLastError();
}

}  // namespace csa2
