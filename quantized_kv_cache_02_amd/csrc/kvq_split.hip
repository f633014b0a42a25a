// kvq_split.hip -- split-KV decode attention over a quantized (int8 / packed
// int4 / fp8 E4M3FN) cache, or an unquantized bf16 one, for gfx950.  Compiled
// once per (KVQ_DTYPE, KVQ_MODE, KVQ_VROW); each translation unit instantiates
// head_dim x row-block variants.
//
// Method (kernel page "kv-quant-attn", "Method"; ORT PR "[CUDA] PagedAttention:
// quantized KV cache ...", "CUDA kernels": split-KV, block-table-aware decode
// with on-the-fly dequantization):
//   * one workgroup owns (sequence b, KV head, split s) and serves every query
//     row of that KV head -- the G grouped query heads times the Tq query
//     tokens -- from a single pass over the split's cached rows (past 768
//     accumulator columns, two workgroups share the rows, reading the split
//     through one L2);
//   * its 4 wavefronts take interleaved 16-token tiles and keep private
//     online-softmax state (max, sum, accumulator) with no barrier or atomic in
//     the loop; the wavefronts merge once at the end in a fixed order and the
//     split's normalized partial goes to the workspace;
//   * scales: a per-channel K scale is folded into q and the per-channel /
//     per-tensor V scale is applied to the output by the combine ("[CUDA] Add
//     INT4 paged KV cache with per-channel scales": exact because
//     dequantization is linear, the channel index being contracted for K and
//     free for V).  Per-row scales multiply the logit (K) or the softmax weight
//     (V) of their token.
//
// gfx950 mapping:
//   S^T = K . Q^T  int8 / int4 caches: on v_mfma_i32_16x16x64_i8 with the K
//                 codes as loaded (int4: each nibble moved to a byte's high
//                 half) and the query as a fixed-point vector in 2 or 3 int8
//                 slices (exact int32 dot products); fp8: on
//                 v_mfma_f32_16x16x32_f16, A = 16 tokens x 32 channels of K
//                 codes unpacked to fp16, B = q rows in fp16 after a
//                 power-of-two row normalization.
//   O  += P . V    on v_mfma_f32_16x16x16_f16: A = the softmax weights, which
//                 sit in exactly the lanes the S^T result left them in; B = V
//                 codes, transposed token-major -> channel-major in registers
//                 with byte permutes and unpacked to fp16.
//   The softmax weights are fp16 in [0, 2^8] (a lazily moved reference,
//   relative rounding 2^-11); the accumulators are fp32.
//   An unquantized bf16 cache (the baseline the kernel page compares against,
//   "Performance") takes the same path with the bf16 MFMAs: K rows and q rows
//   enter v_mfma_f32_16x16x32_bf16 as they are; for P . V each weight is split
//   into two bf16 terms hi + lo (hi = bf16(p), lo = bf16(p - hi), together
//   within 2^-17 of p) and both go through v_mfma_f32_16x16x16_bf16.

#include <utility>

#include "kvq_quant.h"
#include "kvq_sched.h"

#ifndef KVQ_DTYPE
#error "KVQ_DTYPE must be defined"
#endif
#ifndef KVQ_VROW
#error "KVQ_VROW must be defined (1: V scales per row, 0: static)"
#endif
#ifndef KVQ_MODE
#error "KVQ_MODE must be defined"
#endif
#ifndef KVQ_WIDE
#define KVQ_WIDE 0  // 1: the unit holds the wide-row-set variants only
#endif

namespace kvq {
namespace {

// The translation unit's V scale kind: per-row scales ride with the tiles; a
// static V scale (per tensor or per channel) is applied by the combine.  The
// template MODE is the K side's scale mode.
constexpr bool kVRow = KVQ_VROW != 0;

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int DT, int D>
struct Geo {
  // bytes per cached row
  static constexpr int ROWB = (DT == kInt4) ? D / 2 : (DT == kBf16) ? 2 * D : D;
  // K tile, lane (token i = l%16, group g = l/16): the lane's quarter of the row
  // is read as chunks of KCH bytes at row offsets KCH*(4c+g), so the 4 lanes of
  // a row read one contiguous 4*KCH-byte span per load instruction.
  static constexpr int KLB = ROWB / 4;
  static constexpr int KCH = KLB < 16 ? KLB : 16;
  static constexpr int KNCH = KLB / KCH;
  static constexpr int KDW = KLB / 4;      // dwords of K codes per lane
  static constexpr int KSTEPS = D / 32;    // 16x16x32 MFMAs per row block
  // The integer caches take S^T on the int8 MFMA: the K codes are its A operand
  // as loaded (int4 nibbles moved to the high half of a byte, 16 * code), q the
  // B operand in two int8 halves.  16x16x64 steps per row block (and half):
  static constexpr bool IQK = DT == kInt8 || DT == kInt4;
  static constexpr int ISTEPS = D / 64;
  // V tile, lane (column j = l%16, group g = l/16): rows 4g..4g+3, VLB bytes
  // of each row, read as VNCH chunks of VCH bytes at row offsets VCH*(j+16c);
  // a load instruction covers 4 whole rows (or 4 whole 256-byte spans).
  static constexpr int VLB = ROWB / 16;
  static constexpr int VCH = VLB < 16 ? VLB : 16;
  static constexpr int VNCH = VLB / VCH;
  static constexpr int VDW = VLB >= 4 ? VLB / 4 : 1;
  static constexpr int NCOL = D / 16;      // 16x16x16 MFMAs per row block
};

// Query slices of the integer S^T (see q_slice_bytes): three for a per-channel K
// scale, whose folded query spans the table's range, two otherwise.  The q
// operand array holds NSL slices per integer k-step (integer caches) or one
// fp16 / bf16 operand per k-step.
template <int DT, int MODE>
constexpr int kQSlices = (MODE == kPerChannel) ? 3 : 2;
template <int DT, int MODE, int D>
constexpr int kQOps = Geo<DT, D>::IQK ? kQSlices<DT, MODE> * Geo<DT, D>::ISTEPS : Geo<DT, D>::KSTEPS;

// Channel d that element e (0..7) of k-step `ks` holds in lane group g, for both
// MFMA operands of S^T (the K codes and the q rows use the same map).
template <int DT, int D>
__device__ __forceinline__ int k_channel(int ks, int g, int e) {
  using G_ = Geo<DT, D>;
  constexpr int DPC = G_::KCH / 4;  // dwords per chunk
  if constexpr (DT == kInt4) {
    const int w = ks;
    const int byteoff = G_::KCH * (4 * (w / DPC) + g) + 4 * (w % DPC);
    const int nib = e < 4 ? 2 * e : 2 * (e - 4) + 1;
    return 2 * byteoff + nib;
  } else if constexpr (DT == kBf16) {  // two channels per dword
    const int w = 4 * ks + (e >> 1);
    const int byteoff = G_::KCH * (4 * (w / DPC) + g) + 4 * (w % DPC);
    return byteoff / 2 + (e & 1);
  } else {
    const int w = 2 * ks + (e >> 2);
    return G_::KCH * (4 * (w / DPC) + g) + 4 * (w % DPC) + (e & 3);
  }
}

// Channel d that byte p (0..15) of integer k-step s holds in lane group g, for
// both operands of the int8 S^T MFMA.  int8: the 16 bytes are the lane's K
// dwords 4s..4s+3; int4: the even and odd nibbles of dwords 2s and 2s+1, as
// (even 2s, odd 2s, even 2s+1, odd 2s+1).  Either way 16 consecutive channels.
template <int DT, int D>
__device__ __forceinline__ int k_channel_i8(int s, int g, int p) {
  using G_ = Geo<DT, D>;
  constexpr int DPC = G_::KCH / 4;  // dwords per chunk
  if constexpr (DT == kInt4) {
    const int j = p / 4, w = 2 * s + j / 2;
    const int byteoff = G_::KCH * (4 * (w / DPC) + g) + 4 * (w % DPC) + p % 4;
    return 2 * byteoff + (j & 1);
  } else {
    const int w = 4 * s + p / 4;
    return G_::KCH * (4 * (w / DPC) + g) + 4 * (w % DPC) + p % 4;
  }
}

// k_channel_i8(s, g, p) - k_channel_i8(s, g, 0), which depends on p alone:
// int8 0..15 in order; int4 the even channels 0, 2, 4, 6, the odd ones, then
// the same 8 higher.
template <int DT>
__device__ __forceinline__ constexpr int k_offset_i8(int p) {
  return DT == kInt4 ? 8 * (p / 8) + 2 * (p % 4) + ((p / 4) & 1) : p;
}

// Channel d of column c (0..NCOL-1) of the P.V MFMA in lane column j.
template <int DT, int D>
__device__ __forceinline__ int v_channel(int c, int j) {
  using G_ = Geo<DT, D>;
  if constexpr (DT == kInt4) {
    constexpr int nb = G_::VLB >= 4 ? 4 : G_::VLB;  // valid bytes per dword
    const int w = c / (2 * nb), r = c % (2 * nb);
    const int k = r % nb, odd = r / nb;
    return 2 * G_::VLB * j + 2 * (4 * w + k) + odd;
  } else if constexpr (DT == kBf16) {
    constexpr int CPC = G_::VCH / 2;  // channels per chunk
    return CPC * (j + 16 * (c / CPC)) + c % CPC;
  } else {
    return G_::VLB * j + c;
  }
}

// Inverse of v_channel within a lane: the column c holding channel
// NCOL * j + o (every lane covers NCOL consecutive channels).
template <int DT, int D>
__device__ __forceinline__ constexpr int col_of(int o) {
  using G_ = Geo<DT, D>;
  if constexpr (DT == kInt4) {
    constexpr int nb = G_::VLB >= 4 ? 4 : G_::VLB;
    const int w = o / 8, within = o % 8;  // 8 channels per dword of nibbles
    const int k = within / 2, odd = within % 2;
    return 2 * nb * w + odd * nb + k;
  } else {
    return o;
  }
}

// The merge writes each lane's accumulator columns in groups of 4 consecutive
// channels: group k of lane column n holds columns col_of(4k) .. col_of(4k+3),
// which are channels NCOL*n + 4k .. +3 (bf16: v_channel(4k, n) .. +3).
// group_owner is the inverse: the lane column and group of channel d (a
// multiple of 4).
template <int DT, int D>
__device__ __forceinline__ void group_owner(int d, int& n, int& k) {
  using G_ = Geo<DT, D>;
  if constexpr (DT == kBf16) {
    constexpr int CPC = G_::VCH / 2;
    const int q = d / CPC;
    n = q % 16;
    k = (q / 16) * (CPC / 4) + (d % CPC) / 4;
  } else {
    n = d / G_::NCOL;
    k = (d % G_::NCOL) / 4;
  }
}

// Cache codes and row scales are read with buffer loads through a descriptor
// that covers exactly the valid rows of the tile: rows past the sequence end,
// tiles past the split's last one and blocks outside the pool read as zero
// without a memory access (the descriptor's record count is 0 or the valid
// bytes).  So every wavefront runs one unconditional load sequence -- the
// compiler's waits stay exact -- and ragged tails never see stale bytes.  All
// offsets go in the per-lane offset, which is the part the range check covers.
// The loads are non-temporal: each byte is read once per decode (measured on
// MI355X: the same read pattern goes from 5.7 to 6.2 TB/s).
constexpr int kBufWord3 = 0x00020000;  // gfx9 raw-buffer descriptor format word
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufWord3);
}

template <int N>
__device__ __forceinline__ void load_bytes(__amdgpu_buffer_rsrc_t r, int off, uint32_t* out) {
  if constexpr (N == 16) {
    u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  } else if constexpr (N == 8) {
    u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNonTemporal);
    out[0] = v[0]; out[1] = v[1];
  } else if constexpr (N == 4) {
    out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNonTemporal);
  } else {
    static_assert(N == 2, "unsupported chunk");
    out[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kNonTemporal);
  }
}

// Unpack the lane's K codes of k-step ks into the A operand (8 halves).
template <int DT, int D>
__device__ __forceinline__ half8_t k_operand(const uint32_t* kw, int ks) {
  uint32_t h[4];
  if constexpr (DT == kBf16) {  // the bf16 values themselves (a bit container here)
    return u4_to_h8(kw[4 * ks], kw[4 * ks + 1], kw[4 * ks + 2], kw[4 * ks + 3]);
  } else if constexpr (DT == kInt4) {
    int4x8_to_h(kw[ks], h);
  } else if constexpr (DT == kInt8) {
    int8x4_to_h(kw[2 * ks], h[0], h[1]);
    int8x4_to_h(kw[2 * ks + 1], h[2], h[3]);
  } else {
    fp8x4_to_h(kw[2 * ks], h[0], h[1]);
    fp8x4_to_h(kw[2 * ks + 1], h[2], h[3]);
  }
  return u4_to_h8(h[0], h[1], h[2], h[3]);
}

// The lane's K codes of integer k-step s as the int8 A operand: int8 codes as
// they are; int4 nibbles n as the bytes 16 n (two's complement nibble in the
// high half), even nibbles then odd ones of each dword.
template <int DT, int D>
__device__ __forceinline__ i32x4_t k_operand_i8(const uint32_t* kw, int s) {
  if constexpr (DT == kInt4) {
    const uint32_t x = kw[2 * s], y = kw[2 * s + 1];
    return i32x4_t{(int)((x << 4) & 0xF0F0F0F0u), (int)(x & 0xF0F0F0F0u),
                   (int)((y << 4) & 0xF0F0F0F0u), (int)(y & 0xF0F0F0F0u)};
  } else {
    return i32x4_t{(int)kw[4 * s], (int)kw[4 * s + 1], (int)kw[4 * s + 2], (int)kw[4 * s + 3]};
  }
}

// Codes and scales of one 16-token tile as this lane holds them.
template <int DT, int D>
struct Tile {
  uint32_t kw[Geo<DT, D>::KDW];     // K: token n, the lane's quarter of the row
  uint32_t vw[4][Geo<DT, D>::VDW];  // V: tokens 4g..4g+3, the lane's column bytes
  float4_t ks4, vs4;                // per-row scales of tokens 4g..4g+3
  int ok;                           // block-table entry inside the pool
};

// First cache row of each of a wavefront's tiles, in units of 16 rows (a
// tile's 16 rows are consecutive: block sizes are multiples of 16), or -1 for a
// tile whose block-table entry lies outside the pool.  The wavefront's k-th
// tile is t0 + kWaves * k; its value sits in lane k % 64 of register k / 64.
// Computed once before the first tile (the block-table reads included), so
// the tile loop neither waits on a table read nor does row arithmetic beyond
// one shift.  The host bounds the pool so that every value fits an int.
struct TableRegs {
  int e0, e1, e2, e3;  // kTableRegs == 4 (named, not an array: stays in registers)
};
static_assert(kTableRegs == 4, "TableRegs holds four registers");

// The block-table reads of a wavefront's tiles are issued first (TableLoads:
// the block of each tile and its 16-row group inside the block), the rows
// computed once they land (finish), so that other loads can be issued in
// between.  All in 32 bits: the host bounds the pool to 2^31 groups of 16
// rows, and tile indices stay below 2^27.
struct TableLoads {
  int blk[kTableRegs];  // the tile's block (contiguous: the sequence's)
  int in[kTableRegs];   // its 16-row group inside the block
};

__device__ __forceinline__ TableLoads table_issue(const SplitArgs& a, int b, int t0, int waves, int lane) {
  TableLoads tl;
  const uint32_t bs16 = (uint32_t)a.c.block_size >> 4;
#pragma unroll
  for (int j = 0; j < kTableRegs; ++j) {
    const uint32_t t = (uint32_t)t0 + (uint32_t)(waves * (64 * j + lane));
    if (a.c.block_table != nullptr) {
      uint32_t idx = t / bs16;
      tl.in[j] = (int)(t - idx * bs16);
      idx = idx < (uint32_t)a.c.max_blocks ? idx : (uint32_t)a.c.max_blocks - 1;  // dead tiles stay in range
      tl.blk[j] = a.c.block_table[(size_t)b * a.c.max_blocks + idx];
    } else {
      tl.blk[j] = b;
      tl.in[j] = t < bs16 ? (int)t : 0;  // (tiles past a contiguous sequence read nothing)
    }
  }
  return tl;
}

__device__ __forceinline__ TableRegs table_finish(const SplitArgs& a, int hkv, const TableLoads& tl) {
  const uint32_t bs16 = (uint32_t)a.c.block_size >> 4;
  int e[kTableRegs];
#pragma unroll
  for (int j = 0; j < kTableRegs; ++j) {
    const uint32_t blk = (uint32_t)tl.blk[j];
    e[j] = blk >= (uint32_t)a.c.num_blocks
               ? -1
               : (int)((blk * (uint32_t)a.c.Hkv + (uint32_t)hkv) * bs16 + (uint32_t)tl.in[j]);
  }
  return TableRegs{e[0], e[1], e[2], e[3]};
}

// Value of the wavefront's k-th tile (k wave-uniform, k < kTableRegs * 64 for
// every live tile; larger k only occurs for dead tiles, which read nothing).
__device__ __forceinline__ int table_entry(const TableRegs& r, int k) {
  const int j = k >> 6;
  const int v = j == 0 ? r.e0 : j == 1 ? r.e1 : j == 2 ? r.e2 : r.e3;
  return __builtin_amdgcn_readlane(v, k & 63);
}

// Issue the loads of tile t (tokens 16t..16t+15), whose first cache row is
// 16 * row16 (row16 < 0: outside the pool).  `live` is false for the tiles a
// wavefront loads past the end of its split; those read nothing.
template <int DT, int MODE, int D>
__device__ __forceinline__ void load_tile(const SplitArgs& a, int t, bool live, int row16, int L,
                                          int n, int g, Tile<DT, D>& T) {
  using G_ = Geo<DT, D>;
  constexpr int ROWB = G_::ROWB;
  const int tok0 = t * kTile;
  const int ok = row16 >= 0;
  T.ok = ok;
  const int rows = (live && ok) ? min(kTile, L - tok0) : 0;
  const size_t row0 = (size_t)(uint32_t)(ok ? row16 : 0) * kTile;
  const auto kr = make_rsrc(a.c.k_codes + row0 * ROWB, rows * ROWB);
  const auto vr = make_rsrc(a.c.v_codes + row0 * ROWB, rows * ROWB);
  const int koff = n * ROWB + G_::KCH * g;
#pragma unroll
  for (int c = 0; c < G_::KNCH; ++c)
    load_bytes<G_::KCH>(kr, koff + c * 4 * G_::KCH, T.kw + c * (G_::KCH / 4));
  const int voff = 4 * g * ROWB + G_::VCH * n;
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int c = 0; c < G_::VNCH; ++c)
      load_bytes<G_::VCH>(vr, voff + e * ROWB + c * 16 * G_::VCH, T.vw[e] + c * (G_::VCH / 4));
  if constexpr (MODE == kPerRow) {
    uint32_t w[4];
    load_bytes<16>(make_rsrc(a.c.k_scales + row0, rows * 4), 16 * g, w);
    T.ks4 = float4_t{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                     __uint_as_float(w[3])};
  }
  if constexpr (kVRow) {
    uint32_t w[4];
    load_bytes<16>(make_rsrc(a.c.v_scales + row0, rows * 4), 16 * g, w);
    T.vs4 = float4_t{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                     __uint_as_float(w[3])};
  }
}

// Query rows staged in LDS as bf16, one row every kQStride elements: the 16
// bytes of padding put the 16 rows of a k-step read in different banks.
template <int D>
constexpr int kQStride = D + 8;


// Per-wavefront online-softmax state over its tiles.
template <int DT, int D, int RB>
struct WaveState {
  float m[RB];                         // reference logit of row rb*16+n (log2 units)
  float l[RB];                         // this lane's share of the running sum
  float4_t acc[RB][Geo<DT, D>::NCOL];  // O rows rb*16+4g+e, column c of lane n
  float vref;                          // per-row V: weights carry 1/vref, a power of two
  float ivref;                         // 1 / vref (exact)
};

// Per-row V scales: keep vref a power of two >= every scale seen, so the
// weights p * s / vref stay at most p.  The reduction runs only on the rare
// tiles where some scale exceeds the current reference; then vfac = old vref /
// new vref (exact) multiplies the accumulators.
__device__ __forceinline__ void v_reference(const float4_t& vs4, float& vref, float& ivref, float& vfac,
                                            bool& rescale, float (&vsn)[4]) {
  const float vmax4 = fmaxf(fmaxf(vs4[0], vs4[1]), fmaxf(vs4[2], vs4[3]));
  if (__builtin_amdgcn_ballot_w64(vmax4 > vref) != 0) {
    const float vmax = group_max4(vmax4);
    int en;
    (void)frexpf(vmax, &en);  // vmax < 2^en
    ivref = ldexpf(1.0f, -en);
    vfac = vref * ivref;  // both powers of two: exact
    vref = ldexpf(1.0f, en);
    rescale = true;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) vsn[e] = vs4[e] * ivref;
}

// S^T of one tile for one 16-row block: this lane's 4 dot products (tokens
// 4g..4g+3 of the tile, query row n) of the K codes with the row block's q
// operand (qop(k): the operand of k-step k), in the operand's units.
template <int DT, int MODE, int D, class QOp>
__device__ __forceinline__ void tile_dots(const uint32_t* kw, QOp qop, float (&dot)[4]) {
  using G_ = Geo<DT, D>;
  // S^T: two independent accumulation chains over the k-steps
  float4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (G_::IQK) {
    // exact integer dot products with each query slice (operand NSL st + k
    // is slice k of integer step st), combined into one float per logit
    constexpr int NSL = kQSlices<DT, MODE>;
    i32x4_t acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < G_::ISTEPS; ++st) {
      const i32x4_t ka = k_operand_i8<DT, D>(kw, st);
      if constexpr (NSL == 3)
        acc2 = mfma64_i8(ka, __builtin_bit_cast(i32x4_t, qop(NSL * st + 2)), acc2);
      acc1 = mfma64_i8(ka, __builtin_bit_cast(i32x4_t, qop(NSL * st + 1)), acc1);
      acc0 = mfma64_i8(ka, __builtin_bit_cast(i32x4_t, qop(NSL * st)), acc0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (NSL == 3) {
        const int dd[3] = {acc0[e], acc1[e], acc2[e]};
        dot[e] = q_dot<3>(dd);
      } else {
        const int dd[2] = {acc0[e], acc1[e]};
        dot[e] = q_dot<2>(dd);
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < G_::KSTEPS; ks += 2) {
      if constexpr (DT == kBf16) {
        s0 = mfma32_bf16(k_operand<DT, D>(kw, ks), qop(ks), s0);
        if (ks + 1 < G_::KSTEPS) s1 = mfma32_bf16(k_operand<DT, D>(kw, ks + 1), qop(ks + 1), s1);
      } else {
        s0 = mfma32(k_operand<DT, D>(kw, ks), qop(ks), s0);
        if (ks + 1 < G_::KSTEPS) s1 = mfma32(k_operand<DT, D>(kw, ks + 1), qop(ks + 1), s1);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) dot[e] = s0[e] + s1[e];
  }
}

// Logits (log2 units) of this lane's 4 tokens tbase..tbase+3 from their dot
// products: the row multiplier, a per-row K scale, the soft cap, and -inf for
// tokens outside the row's visible range lo <= t < lim (or a tile outside the
// pool).  Rows past the sequence and tiles outside the pool were read as zero
// by the bounded loads (codes and scales), so only the logits need masking:
// those tokens then get weight 0 and add nothing.
template <int MODE, bool CAP>
__device__ __forceinline__ void tile_logits(const float (&dot)[4], const float4_t& ks4, bool ok, int tbase,
                                            float rowmul, int lim, int lo, float cap2, float icap2,
                                            float (&z)[4]) {
  // token tbase + e is visible to this lane's row iff lo <= it < lim
  const unsigned span = ok ? (unsigned)(lim - lo) : 0u;
  const int rel = tbase - lo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float zz = dot[e] * rowmul;
    if constexpr (MODE == kPerRow) zz *= ks4[e];
    // soft cap in log2 units: with x = z / softcap, z2 = z log2(e), cap2 =
    // softcap log2(e): cap2 tanh(x) = cap2 (1 - 2 / (1 + 2^(2 z2 / softcap)))
    // (icap2 = 2 / softcap); the hardware exp2 and reciprocal, 1 ulp each
    if constexpr (CAP) {
      const float ex = __builtin_amdgcn_exp2f(zz * icap2);
      zz = cap2 - 2.0f * cap2 * __builtin_amdgcn_rcpf(ex + 1.0f);
    }
    z[e] = (unsigned)(rel + e) < span ? zz : -INFINITY;
  }
}

// One tile's logits and softmax weights for one 16-row block: S^T, the
// logits, the lazily moved reference m, the running sum l and the P operand
// (bf16 cache: its hi and lo parts).  alpha is the factor the row's
// accumulators take when m moved (1 otherwise), and `rescale` is set then.
template <int DT, int MODE, bool CAP>
__device__ __forceinline__ void row_block_softmax(const float (&dot)[4], const float4_t& ks4, bool ok,
                                                  int tbase, float rowmul, int lim, int lo, float cap2,
                                                  float icap2, const float (&vsn)[4], float& m, float& l,
                                                  float& alpha, bool& rescale, half4_t& pa, u32x2_t& phi,
                                                  u32x2_t& plo) {
  float z[4];
  tile_logits<MODE, CAP>(dot, ks4, ok, tbase, rowmul, lim, lo, cap2, icap2, z);
  bool up = false;
#pragma unroll
  for (int e = 0; e < 4; ++e) up |= z[e] > m + kLazyHeadroom;
  // The reference m moves only when a logit exceeds it by more than
  // kLazyHeadroom (a factor 2^8 in the weights); the cross-lane reduction and
  // the accumulator rescale run only then.  m stays a logit of the row, so
  // m <= the row's max logit <= m + kLazyHeadroom.
  alpha = 1.0f;
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
    const float tmax = group_max4(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    if (tmax > m + kLazyHeadroom) {
      // hardware exp2 (results below 2^-126 flush to 0: such weights vanish
      // in the fp16 operand anyway); 0 when the old reference was -inf
      alpha = __builtin_amdgcn_exp2f(m - tmax);
      l *= alpha;
      m = tmax;
      rescale = true;
    }
  }
  const float msafe = (m == -INFINITY) ? 0.0f : m;
  half4_t ph;
  float pf[4];
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p = __builtin_amdgcn_exp2f(z[e] - msafe);
    psum += p;
    float pv = p;
    if constexpr (kVRow) pv = p * vsn[e];
    ph[e] = (_Float16)pv;
    pf[e] = pv;
  }
  l += psum;
  pa = ph;
  if constexpr (DT == kBf16) {
    uint16_t h[4], lw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = f32_to_bf16(pf[e]);
      lw[e] = f32_to_bf16(pf[e] - bf16_to_f32(h[e]));  // exact difference
    }
    phi = u32x2_t{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
    plo = u32x2_t{lw[0] | ((uint32_t)lw[1] << 16), lw[2] | ((uint32_t)lw[3] << 16)};
  }
}

// The B operands of the P . V MFMA from dword w of the lane's V codes (tokens
// 4g..4g+3 of the tile): vb[k] feeds accumulator column v_column(w, k), for k
// < 8 (int4: both nibbles of the bytes of the dword, nb of them valid) or
// k < 4 (the 8-bit caches).
template <int DT, int VD>
__device__ __forceinline__ void v_block(const uint32_t (&vw)[4][Geo<DT, VD>::VDW], int w, half4_t (&vb)[8]) {
  if constexpr (DT == kInt4) {
    uint32_t ev4[4], od4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = vw[e][w] ^ 0x88888888u;
      ev4[e] = (x << 4) & 0xF0F0F0F0u;
      od4[e] = x & 0xF0F0F0F0u;
    }
    v_transpose4<0>(ev4[0], ev4[1], ev4[2], ev4[3], vb);
    v_transpose4<0>(od4[0], od4[1], od4[2], od4[3], vb + 4);
  } else if constexpr (DT == kInt8) {
    v_transpose4<0>(vw[0][w] ^ 0x80808080u, vw[1][w] ^ 0x80808080u, vw[2][w] ^ 0x80808080u,
                    vw[3][w] ^ 0x80808080u, vb);
  } else {
    static_assert(DT == kFp8, "v_block: quantized caches");
    v_transpose4<1>(vw[0][w], vw[1][w], vw[2][w], vw[3][w], vb);
  }
}

// Operands of dword block w: how many, and the accumulator column of vb[k].
template <int DT, int VD>
constexpr int v_block_ops() {
  return DT == kInt4 ? 2 * (Geo<DT, VD>::VLB >= 4 ? 4 : Geo<DT, VD>::VLB) : 4;
}
template <int DT, int VD>
__device__ __forceinline__ constexpr int v_column(int w, int k) {
  if constexpr (DT == kInt4) {
    constexpr int nb = Geo<DT, VD>::VLB >= 4 ? 4 : Geo<DT, VD>::VLB;
    return 2 * nb * w + (k < nb ? k : nb + (k - 4));
  } else {
    return 4 * w + k;
  }
}

template <int DT, int MODE, int D, bool CAP, class QOp>
__device__ __forceinline__ void row_block_weights(const uint32_t* kw, const float4_t& ks4, bool ok,
                                                  int tbase, QOp qop, float rowmul, int lim, int lo,
                                                  float cap2, float icap2, const float (&vsn)[4],
                                                  float& m, float& l, float& alpha, bool& rescale,
                                                  half4_t& pa, u32x2_t& phi, u32x2_t& plo) {
  float dot[4];
  tile_dots<DT, MODE, D>(kw, qop, dot);
  row_block_softmax<DT, MODE, CAP>(dot, ks4, ok, tbase, rowmul, lim, lo, cap2, icap2, vsn, m, l, alpha,
                                   rescale, pa, phi, plo);
}

// S^T accumulators of one tile for all RB row blocks: exact int32 per query
// slice for the integer caches, fp32 otherwise.
template <int DT, int MODE, int D, int RB>
struct QKAcc {
  static constexpr bool IQK = Geo<DT, D>::IQK;
  static constexpr int NSL = IQK ? kQSlices<DT, MODE> : 1;
  i32x4_t ia[RB][IQK ? NSL : 1];
  float4_t fa[RB];
};

// S^T of one tile for all RB row blocks at once, their q operands read from
// the lane-linear LDS copy (operand k of row block rb at qlds[(rb * QO + k) *
// 64]).  The reads of every block's operands of k-step st + 1 are interleaved
// with the MFMAs of step st (scheduling group barriers), so the LDS latency
// hides under the MFMAs instead of stalling one wavefront per SIMD before
// each of them.  Only issues the MFMAs: qk_dots reads the results.
template <int DT, int MODE, int D, int RB>
__device__ __forceinline__ void qk_issue(const uint32_t* kw, const half8_t* qlds, QKAcc<DT, MODE, D, RB>& A) {
  using G_ = Geo<DT, D>;
  constexpr int QO = kQOps<DT, MODE, D>;
  // opaque base: keeps the reads inside the tile loop (in registers the
  // operands of every block would not fit)
  int qb = 0;
  asm volatile("" : "+v"(qb));
  const half8_t* q = qlds + qb;
  if constexpr (G_::IQK) {
    constexpr int NSL = kQSlices<DT, MODE>;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int k = 0; k < NSL; ++k) A.ia[rb][k] = i32x4_t{0, 0, 0, 0};
    half8_t qv[2][RB][NSL];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int k = 0; k < NSL; ++k) qv[0][rb][k] = q[(rb * QO + k) * 64];
#pragma unroll
    for (int st = 0; st < G_::ISTEPS; ++st) {
      const i32x4_t ka = k_operand_i8<DT, D>(kw, st);
      if (st + 1 < G_::ISTEPS) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int k = 0; k < NSL; ++k) qv[(st + 1) & 1][rb][k] = q[(rb * QO + NSL * (st + 1) + k) * 64];
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int k = 0; k < NSL; ++k)
          A.ia[rb][k] = mfma64_i8(ka, __builtin_bit_cast(i32x4_t, qv[st & 1][rb][k]), A.ia[rb][k]);
    }
    // schedule: step 0's reads, then each MFMA of step st after one read of
    // step st + 1, so a step's reads complete under the previous step's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, RB * NSL, 0);
#pragma unroll
    for (int st = 0; st < G_::ISTEPS; ++st)
#pragma unroll
      for (int j = 0; j < RB * NSL; ++j) {
        if (st + 1 < G_::ISTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) A.fa[rb] = float4_t{0.f, 0.f, 0.f, 0.f};
    half8_t qv[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) qv[0][rb] = q[(rb * QO) * 64];
#pragma unroll
    for (int ks = 0; ks < G_::KSTEPS; ++ks) {
      const half8_t ka = k_operand<DT, D>(kw, ks);
      if (ks + 1 < G_::KSTEPS) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) qv[(ks + 1) & 1][rb] = q[(rb * QO + ks + 1) * 64];
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (DT == kBf16)
          A.fa[rb] = mfma32_bf16(ka, qv[ks & 1][rb], A.fa[rb]);
        else
          A.fa[rb] = mfma32(ka, qv[ks & 1][rb], A.fa[rb]);
      }
    }
    // the same schedule as the integer path
    __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);
#pragma unroll
    for (int ks = 0; ks < G_::KSTEPS; ++ks)
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        if (ks + 1 < G_::KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
  }
}

// The dot products of qk_issue's accumulators (in the q operand's units).
template <int DT, int MODE, int D, int RB>
__device__ __forceinline__ void qk_dots(const QKAcc<DT, MODE, D, RB>& A, float (&dot)[RB][4]) {
  if constexpr (Geo<DT, D>::IQK) {
    constexpr int NSL = kQSlices<DT, MODE>;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (NSL == 3) {
          const int dd[3] = {A.ia[rb][0][e], A.ia[rb][1][e], A.ia[rb][2][e]};
          dot[rb][e] = q_dot<3>(dd);
        } else {
          const int dd[2] = {A.ia[rb][0][e], A.ia[rb][1][e]};
          dot[rb][e] = q_dot<2>(dd);
        }
      }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) dot[rb][e] = A.fa[rb][e];
  }
}

template <int DT, int MODE, int D, int RB>
__device__ __forceinline__ void tile_dots_lds(const uint32_t* kw, const half8_t* qlds, float (&dot)[RB][4]) {
  QKAcc<DT, MODE, D, RB> A;
  qk_issue<DT, MODE, D, RB>(kw, qlds, A);
  qk_dots<DT, MODE, D, RB>(A, dot);
}

// O += P . V for one tile: unpack the lane's V column blocks (VD channels) and
// accumulate every row block's weights into them.
template <int DT, int VD, int RB>
__device__ __forceinline__ void accumulate_pv(const uint32_t (&vw)[4][Geo<DT, VD>::VDW],
                                              const half4_t (&pa)[RB], const u32x2_t (&phi)[RB],
                                              const u32x2_t (&plo)[RB],
                                              float4_t (&acc)[RB][Geo<DT, VD>::NCOL]) {
  using GV = Geo<DT, VD>;
#pragma unroll
  for (int w = 0; w < GV::VDW; ++w) {
    if constexpr (DT == kBf16) {
      // dword w of the lane's span holds channel columns 2w (low half) and 2w+1
      const u32x2_t b0 = {perm(vw[1][w], vw[0][w], 0x05040100u), perm(vw[3][w], vw[2][w], 0x05040100u)};
      const u32x2_t b1 = {perm(vw[1][w], vw[0][w], 0x07060302u), perm(vw[3][w], vw[2][w], 0x07060302u)};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb][2 * w] = mfma16_bf16(phi[rb], b0, acc[rb][2 * w]);
        acc[rb][2 * w] = mfma16_bf16(plo[rb], b0, acc[rb][2 * w]);
        acc[rb][2 * w + 1] = mfma16_bf16(phi[rb], b1, acc[rb][2 * w + 1]);
        acc[rb][2 * w + 1] = mfma16_bf16(plo[rb], b1, acc[rb][2 * w + 1]);
      }
    } else {
      half4_t vb[8];
      v_block<DT, VD>(vw, w, vb);
      constexpr int NO = v_block_ops<DT, VD>();
#pragma unroll
      for (int k0 = 0; k0 < NO; ++k0) {
        // int4: the even-nibble operand k and its odd partner, as before
        const int k = DT == kInt4 ? (k0 % 2 == 0 ? k0 / 2 : 4 + k0 / 2) : k0;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][v_column<DT, VD>(w, k)] = mfma16(pa[rb], vb[k], acc[rb][v_column<DT, VD>(w, k)]);
      }
    }
  }
}

// The same P . V in two parts for the quantized caches: the whole tile's V
// operands unpacked first (so the unpack can run beside the tile's S^T
// MFMAs), then the MFMAs.
template <int DT, int VD>
struct VTile {
  half4_t vb[Geo<DT, VD>::VDW][8];
};

template <int DT, int VD>
__device__ __forceinline__ void unpack_v(const uint32_t (&vw)[4][Geo<DT, VD>::VDW], VTile<DT, VD>& V) {
  static_assert(DT != kBf16, "unpack_v: quantized caches");
#pragma unroll
  for (int w = 0; w < Geo<DT, VD>::VDW; ++w) v_block<DT, VD>(vw, w, V.vb[w]);
}

template <int DT, int VD, int RB>
__device__ __forceinline__ void pv_unpacked(const VTile<DT, VD>& V, const half4_t (&pa)[RB],
                                            float4_t (&acc)[RB][Geo<DT, VD>::NCOL]) {
  constexpr int NO = v_block_ops<DT, VD>();
#pragma unroll
  for (int w = 0; w < Geo<DT, VD>::VDW; ++w)
#pragma unroll
    for (int k0 = 0; k0 < NO; ++k0) {
      const int k = DT == kInt4 ? (k0 % 2 == 0 ? k0 / 2 : 4 + k0 / 2) : k0;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][v_column<DT, VD>(w, k)] = mfma16(pa[rb], V.vb[w][k], acc[rb][v_column<DT, VD>(w, k)]);
    }
}

// One tile's softmax weights for every row block (pa, or phi + plo for the
// bf16 cache), with the factors alpha (per row) and vfac (V reference) that
// the accumulators take before its P . V.  Returns whether they must be
// applied (wave-uniform): some row's reference or the V reference moved.  For
// wide row sets it is also false while no weight of the wavefront has been
// nonzero yet (l = 0 everywhere), as the accumulators are then still zero.
template <int DT, int MODE, int D, int RB, bool CAP, bool QLDS>
__device__ __forceinline__ bool tile_weights(const Tile<DT, D>& T, int t, int n, int g,
                                             const half8_t (&qb)[RB][kQOps<DT, MODE, D>],
                                             const half8_t* qlds, const float (&rowmul)[RB],
                                             const int (&lim)[RB], const int (&lo)[RB], float cap2,
                                             float icap2, WaveState<DT, D, RB>& W, half4_t (&pa)[RB],
                                             u32x2_t (&phi)[RB], u32x2_t (&plo)[RB], float (&alpha)[RB],
                                             float& vfac) {
  const int tok0 = t * kTile;
  const int tbase = tok0 + 4 * g;
  const bool ok = T.ok != 0;
  (void)n;

  vfac = 1.0f;
  bool rescale = false;
  float vsn[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (kVRow) v_reference(T.vs4, W.vref, W.ivref, vfac, rescale, vsn);

  bool live = false;
  if constexpr (RB * D > kSplitMaxAccColumns) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) live |= W.l[rb] != 0.0f;
  }
  if constexpr (RB * D > kSplitMaxAccColumns) {
    float dot[RB][4];
    tile_dots_lds<DT, MODE, D, RB>(T.kw, qlds, dot);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      row_block_softmax<DT, MODE, CAP>(dot[rb], T.ks4, ok, tbase, rowmul[rb], lim[rb], lo[rb], cap2, icap2,
                                       vsn, W.m[rb], W.l[rb], alpha[rb], rescale, pa[rb], phi[rb], plo[rb]);
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // the q operand of k-step k: registers, or this wavefront's LDS copy
      // (lane-linear, so conflict-free).  The LDS offset is made opaque so the
      // compiler cannot hoist those reads out of the tile loop back into
      // registers.
      int qo = rb * kQOps<DT, MODE, D> * 64;
      if constexpr (QLDS) asm volatile("" : "+v"(qo));
      auto qop = [&](int k) { return QLDS ? qlds[qo + 64 * k] : qb[rb][k]; };
      row_block_weights<DT, MODE, D, CAP>(T.kw, T.ks4, ok, tbase, qop, rowmul[rb], lim[rb], lo[rb],
                                          cap2, icap2, vsn, W.m[rb], W.l[rb], alpha[rb], rescale,
                                          pa[rb], phi[rb], plo[rb]);
    }
  }
  if constexpr (RB * D > kSplitMaxAccColumns)
    return __builtin_amdgcn_ballot_w64(rescale) != 0 && __builtin_amdgcn_ballot_w64(live) != 0;
  else
    return __builtin_amdgcn_ballot_w64(rescale) != 0;
}

// The tile loop's common case for wide row sets, free of branches so the
// scheduler can interleave its vector work with the MFMAs: from the tile's
// S^T dot products, the logits, and -- when no logit exceeds its row's
// reference by more than kLazyHeadroom and (per-row V) no V scale exceeds the
// V reference -- the weights and running sums.  Otherwise it returns true and
// changes nothing; the caller then takes the tile through weights_general,
// which moves the references.
template <int DT, int MODE, int RB, bool CAP, class WS>
__device__ __forceinline__ bool weights_fast(const float (&dot)[RB][4], const float4_t& ks4, const float4_t& vs4,
                                             bool ok, int t, int g, const float (&rowmul)[RB],
                                             const int (&lim)[RB], const int (&lo)[RB], float cap2, float icap2,
                                             WS& W, half4_t (&pa)[RB], u32x2_t (&phi)[RB], u32x2_t (&plo)[RB]) {
  const int tbase = t * kTile + 4 * g;
  bool slow = false;
  float vsn[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (kVRow) {
    slow = fmaxf(fmaxf(vs4[0], vs4[1]), fmaxf(vs4[2], vs4[3])) > W.vref;
#pragma unroll
    for (int e = 0; e < 4; ++e) vsn[e] = vs4[e] * W.ivref;  // exact: ivref is a power of two
  }
  float z[RB][4];
  // largest logit over reference (m = -inf: +inf for a finite logit; NaN
  // for -inf - -inf, which fmaxf drops)
  float over = -INFINITY;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    tile_logits<MODE, CAP>(dot[rb], ks4, ok, tbase, rowmul[rb], lim[rb], lo[rb], cap2, icap2, z[rb]);
    over = fmaxf(over, fmaxf(fmaxf(z[rb][0], z[rb][1]), fmaxf(z[rb][2], z[rb][3])) - W.m[rb]);
  }
  slow |= over > kLazyHeadroom;
  if (__builtin_amdgcn_ballot_w64(slow) != 0) return true;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // m is finite here unless every logit so far, these included, was -inf
    const float msafe = (W.m[rb] == -INFINITY) ? 0.0f : W.m[rb];
    float psum = 0.0f;
    float pf[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __builtin_amdgcn_exp2f(z[rb][e] - msafe);
      psum += p;
      pf[e] = kVRow ? p * vsn[e] : p;
      pa[rb][e] = (_Float16)pf[e];
    }
    W.l[rb] += psum;
    if constexpr (DT == kBf16) {
      uint16_t h[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = f32_to_bf16(pf[e]);
        lw[e] = f32_to_bf16(pf[e] - bf16_to_f32(h[e]));  // exact difference
      }
      phi[rb] = u32x2_t{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
      plo[rb] = u32x2_t{lw[0] | ((uint32_t)lw[1] << 16), lw[2] | ((uint32_t)lw[3] << 16)};
    }
  }
  return false;
}

template <int DT, int MODE, int D, int RB, bool CAP>
__device__ __forceinline__ bool tile_fast(const Tile<DT, D>& T, int t, int g, const half8_t* qlds,
                                          const float (&rowmul)[RB], const int (&lim)[RB], const int (&lo)[RB],
                                          float cap2, float icap2, WaveState<DT, D, RB>& W, half4_t (&pa)[RB],
                                          u32x2_t (&phi)[RB], u32x2_t (&plo)[RB]) {
  float dot[RB][4];
  tile_dots_lds<DT, MODE, D, RB>(T.kw, qlds, dot);
  return weights_fast<DT, MODE, RB, CAP>(dot, T.ks4, T.vs4, T.ok != 0, t, g, rowmul, lim, lo, cap2, icap2, W, pa,
                                         phi, plo);
}

// The accumulators' rescale when the tile's reference moved: accumulator rows
// 4g+e belong to the P rows held by lanes 4g+e.
template <int DT, int D, int RB>
__device__ __forceinline__ void rescale_acc(WaveState<DT, D, RB>& W, const float (&alpha)[RB], float vfac,
                                            int g) {
  if constexpr (RB * D > kSplitMaxAccColumns) {
    // Wide row sets: their accumulators sit in the accumulation registers,
    // which vector ALU instructions cannot multiply (a multiply made the
    // compiler copy all of them out and spill).  The rows are scaled on the
    // fp32 MFMA instead, which writes the accumulation registers directly:
    // register e of a 16 x 16 block is the B operand (k = lane group) of
    // v_mfma_f32_16x16x4_f32, and A_e holds row i's factor at k = (i - e) / 4
    // when i = e (mod 4), so the sum over e gives every element its factor
    // times itself plus exact zeros -- one rounding, as the multiply.  A
    // scheduling barrier after each block keeps its operand copies to 4
    // registers at a time.
    const int n = __lane_id() & 15;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float fi = alpha[rb] * vfac;  // row n's factor
      float ae[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ae[e] = n == 4 * g + e ? fi : 0.0f;
#pragma unroll
      for (int c = 0; c < Geo<DT, D>::NCOL; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        float4_t d = __builtin_amdgcn_mfma_f32_16x16x4f32(ae[0], W.acc[rb][c][0], float4_t{0.f, 0.f, 0.f, 0.f},
                                                          0, 0, 0);
#pragma unroll
        for (int e = 1; e < 4; ++e) d = __builtin_amdgcn_mfma_f32_16x16x4f32(ae[e], W.acc[rb][c][e], d, 0, 0, 0);
        W.acc[rb][c] = d;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    return;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float f[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __shfl(alpha[rb], 4 * g + e) * vfac;
#pragma unroll
    for (int c = 0; c < Geo<DT, D>::NCOL; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) W.acc[rb][c][e] *= f[e];
  }
}

// The general step of a wide row set's tile from its S^T dot products: moves
// the references (row maxima, V reference) as tile_weights does and rescales
// the accumulators when it moved one and some weight of the wavefront has
// been nonzero.
template <int DT, int MODE, int D, int RB, bool CAP>
__device__ __forceinline__ void weights_general(const float (&dot)[RB][4], const float4_t& ks4,
                                                const float4_t& vs4, bool ok, int t, int g,
                                                const float (&rowmul)[RB], const int (&lim)[RB],
                                                const int (&lo)[RB], float cap2, float icap2,
                                                WaveState<DT, D, RB>& W, half4_t (&pa)[RB],
                                                u32x2_t (&phi)[RB], u32x2_t (&plo)[RB]) {
  const int tbase = t * kTile + 4 * g;
  float vfac = 1.0f;
  bool rescale = false;
  float vsn[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (kVRow) v_reference(vs4, W.vref, W.ivref, vfac, rescale, vsn);
  bool live = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) live |= W.l[rb] != 0.0f;
  float alpha[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    row_block_softmax<DT, MODE, CAP>(dot[rb], ks4, ok, tbase, rowmul[rb], lim[rb], lo[rb], cap2, icap2, vsn,
                                     W.m[rb], W.l[rb], alpha[rb], rescale, pa[rb], phi[rb], plo[rb]);
  if (__builtin_amdgcn_ballot_w64(rescale) != 0 && __builtin_amdgcn_ballot_w64(live) != 0)
    rescale_acc<DT, D, RB>(W, alpha, vfac, g);
}

// One tile: weights, the rescale when needed (rare after the first tiles),
// then O += P . V.
template <int DT, int MODE, int D, int RB, bool CAP, bool QLDS>
__device__ __forceinline__ void process_tile(const Tile<DT, D>& T, int t, int n, int g,
                                             const half8_t (&qb)[RB][kQOps<DT, MODE, D>],
                                             const half8_t* qlds, const float (&rowmul)[RB],
                                             const int (&lim)[RB], const int (&lo)[RB], float cap2,
                                             float icap2, WaveState<DT, D, RB>& W) {
  half4_t pa[RB];
  u32x2_t phi[RB], plo[RB];  // bf16 cache: p = hi + lo, each a bf16 A operand
  float alpha[RB], vfac;
  if (tile_weights<DT, MODE, D, RB, CAP, QLDS>(T, t, n, g, qb, qlds, rowmul, lim, lo, cap2, icap2, W, pa,
                                               phi, plo, alpha, vfac))
    rescale_acc<DT, D, RB>(W, alpha, vfac, g);
  accumulate_pv<DT, D, RB>(T.vw, pa, phi, plo, W.acc);
}

// B operands of S^T for the workgroup's RB row blocks, computed once per
// workgroup (every wavefront needs the same ones) into the lane-linear LDS
// array qop: operand k of row block rb for lane l at qop[(rb * QO + k) * 64 + l].
// Each row is taken in this lane's channel order from the staged rows qs (bf16,
// kQStride apart), times a per-channel K scale, and normalized by a power of
// two: the integer caches get a fixed-point integer vector in NSL int8 slices
// (see q_slice_bytes: 15 bits of the row's largest element, 23 with a per-channel
// K scale folded in), fp8 an fp16 vector with every element in (-1, 1), bf16
// the row as it is (bf16 products are exact in the fp32 accumulation).
// Wavefront w folds the k-steps st = w, w + 4, ...: their row maxima meet in
// s_pmax ([kWaves][16 RB]) across a barrier, the operands in qop across a
// second one.  rowmul[rb] restores the power of two (logit in log2 units =
// dot * rowmul * per-row K scale).  Every wavefront must call it.
// The static K scales come in kst_lds, staged in LDS by the caller: the KV
// head's D per-channel scales, or the per-tensor one.
template <int DT, int MODE, int D, int RB>
__device__ __forceinline__ void fold_q_shared(const SplitArgs& a, const uint16_t* qs, int hkv, int wave,
                                              int n, int g, int lane, half8_t* qop, float* s_pmax,
                                              const float* kst_lds, float (&rowmul)[RB]) {
  using G_ = Geo<DT, D>;
  constexpr int QO = kQOps<DT, MODE, D>;
  constexpr int RP = 16 * RB;
  (void)hkv;
  float mul = a.sm_scale * 1.4426950408889634f;  // natural -> log2 units
  if constexpr (MODE == kPerTensor) mul *= kst_lds[0];
  if constexpr (DT == kInt4) mul *= 0.0625f;  // K operand holds 16 * code
  if constexpr (G_::IQK) {
    constexpr int NSL = kQSlices<DT, MODE>;
    constexpr int NS = G_::ISTEPS;
    constexpr int MY = (NS + kWaves - 1) / kWaves;  // steps per wavefront
    float qv[RB][MY][16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rb * 16 + n;
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < MY; ++j) {
        const int st = wave + kWaves * j;
        if (st >= NS) continue;
        const int base = k_channel_i8<DT, D>(st, g, 0);
        const u32x4_t r0 = *reinterpret_cast<const u32x4_t*>(qs + r * kQStride<D> + base);
        const u32x4_t r1 = *reinterpret_cast<const u32x4_t*>(qs + r * kQStride<D> + base + 8);
        float x16[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x16[2 * i] = __uint_as_float(r0[i] << 16);
          x16[2 * i + 1] = __uint_as_float(r0[i] & 0xFFFF0000u);
          x16[8 + 2 * i] = __uint_as_float(r1[i] << 16);
          x16[8 + 2 * i + 1] = __uint_as_float(r1[i] & 0xFFFF0000u);
        }
#pragma unroll
        for (int p = 0; p < 16; ++p) {
          const int off = k_offset_i8<DT>(p);  // 0..15
          float x = x16[off];
          if constexpr (MODE == kPerChannel) x *= kst_lds[base + off];
          qv[rb][j][p] = x;
          amax = fmaxf(amax, fabsf(x));
        }
      }
      amax = group_max4(amax);
      if (g == 0) s_pmax[wave * RP + r] = amax;
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rb * 16 + n;
      float amax = s_pmax[r];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, s_pmax[w * RP + r]);
      int ex = 0;
      if (amax > 0.0f) (void)frexpf(amax, &ex);  // amax < 2^ex
      rowmul[rb] = ldexpf(mul, ex - (8 * NSL - 2));
#pragma unroll
      for (int j = 0; j < MY; ++j) {
        const int st = wave + kWaves * j;
        if (st >= NS) continue;
        uint32_t wb[16];
#pragma unroll
        for (int p = 0; p < 16; ++p) wb[p] = q_slice_bytes<NSL>(qv[rb][j][p], ex);
        u32x4_t w4[NSL];
#pragma unroll
        for (int k = 0; k < NSL; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w4[k][i] = slice_dword(wb[4 * i], wb[4 * i + 1], wb[4 * i + 2], wb[4 * i + 3], k);
#pragma unroll
        for (int k = 0; k < NSL; ++k)
          qop[(rb * QO + NSL * st + k) * 64 + lane] = __builtin_bit_cast(half8_t, w4[k]);
      }
    }
    __syncthreads();
  } else {
    constexpr int NS = G_::KSTEPS;
    constexpr int MY = (NS + kWaves - 1) / kWaves;
    float qv[RB][MY][8];
    u32x4_t raw[RB][MY];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rb * 16 + n;
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < MY; ++j) {
        const int ks = wave + kWaves * j;
        if (ks >= NS) continue;
        // the 8 channels of a k-step are 8 consecutive channels
        const int base = k_channel<DT, D>(ks, g, 0);
        raw[rb][j] = *reinterpret_cast<const u32x4_t*>(qs + r * kQStride<D> + base);
        if constexpr (DT != kBf16) {
          float x8[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x8[2 * i] = __uint_as_float(raw[rb][j][i] << 16);
            x8[2 * i + 1] = __uint_as_float(raw[rb][j][i] & 0xFFFF0000u);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int off = k_channel<DT, D>(ks, g, e) - base;  // 0..7
            float x = x8[off];
            if constexpr (MODE == kPerChannel) x *= kst_lds[base + off];
            qv[rb][j][e] = x;
            amax = fmaxf(amax, fabsf(x));
          }
        }
      }
      if constexpr (DT != kBf16) {
        amax = group_max4(amax);
        if (g == 0) s_pmax[wave * RP + r] = amax;
      }
    }
    if constexpr (DT != kBf16) __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rb * 16 + n;
      int ex = 0;
      if constexpr (DT != kBf16) {
        float amax = s_pmax[r];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, s_pmax[w * RP + r]);
        if (amax > 0.0f) (void)frexpf(amax, &ex);  // amax < 2^ex
      }
      rowmul[rb] = DT == kBf16 ? mul : ldexpf(mul, ex);
#pragma unroll
      for (int j = 0; j < MY; ++j) {
        const int ks = wave + kWaves * j;
        if (ks >= NS) continue;
        half8_t h;
        if constexpr (DT == kBf16) {
          h = __builtin_bit_cast(half8_t, raw[rb][j]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = (_Float16)ldexpf(qv[rb][j][e], -ex);
        }
        qop[(rb * QO + ks) * 64 + lane] = h;
      }
    }
    __syncthreads();
  }
}

// Tokens visible to query row `row` (of the sequence's R rows; `live` false
// for padding rows, which see none): lo <= t < lim.
__device__ __forceinline__ void row_window(const SplitArgs& a, int L, int row, bool live, int& lim, int& lo) {
  lim = live ? (L - a.Tq + row / a.G + 1) : 0;
  if (lim > L) lim = L;
  lo = a.window > 0 ? lim - a.window : 0;
  if (lim < lo) lim = lo;  // a query before the first token sees none
}

// This workgroup's chunk under the balanced schedule -- sequence b (length L)
// and its tiles [tb, te) -- the same for every wavefront; false for an idle
// slot.  With one sequence load_q(0) issues the query loads at once (chunk =
// slot: they go out before the length arrives); with several the caller
// issues them once the sequence is known, after the block-table reads.
// `record`: this wavefront also writes every sequence's chunk slots for the
// combine.
template <class LoadQ>
__device__ __forceinline__ bool workgroup_chunk(const SplitArgs& a, int slot, bool record, int lane,
                                                LoadQ&& load_q, int& b, int& L, int& tb, int& te) {
  if (a.B == 1) {
    b = 0;
    load_q(0);
    L = clamp_len(a.seq_lens[0], a.max_seq_len);
    const Span sp = visible_tiles(L, a.Tq, a.window);
    const int C = max((sp.end - sp.first + a.NW - 1) / a.NW, kMinTilesPerSplit);
    tb = sp.first + slot * C;
    te = min(tb + C, sp.end);
    return tb < sp.end;
  }
  const Chunk ch = find_chunk(a.seq_lens, a.B, a.max_seq_len, a.NW, a.Tq, a.window, slot, -1, lane,
                              record ? a.ws_chunks : nullptr);
  if (ch.b < 0) return false;
  b = ch.b;
  L = ch.L;
  tb = ch.first;
  te = ch.end;
  return true;
}

// Fused append: the new K and V rows of the query tokens j with mine[j]
// (position L - Tq + j), loaded from the bf16 inputs, then quantized and
// stored into the cache with the same arithmetic as kvq_append.  store() waits
// until the stores are acknowledged, so the wavefront's later loads of those
// rows see them.
template <int DT, int MODE, int D>
struct NewRows {
  using RG = RowGeo<DT, D>;
  uint16_t rk[kMaxQTokens][RG::EPL], rv[kMaxQTokens][RG::EPL];
  int rblk[kMaxQTokens];

  __device__ __forceinline__ void load(const SplitArgs& a, const bool (&mine)[kMaxQTokens], int b, int hkv,
                                       int L, int lane) {
#pragma unroll
    for (int j = 0; j < kMaxQTokens; ++j) {
      if (!mine[j]) continue;
      const int p = L - a.Tq + j;
      const size_t xi = (((size_t)b * a.Tq + j) * a.c.Hkv + hkv) * D;
      load_row<DT, D>(a.k_new + xi, lane, rk[j]);
      load_row<DT, D>(a.v_new + xi, lane, rv[j]);
      rblk[j] = a.c.block_table != nullptr
                    ? a.c.block_table[(size_t)b * a.c.max_blocks + p / a.c.block_size]
                    : b;
    }
  }

  __device__ __forceinline__ void store(const SplitArgs& a, const bool (&mine)[kMaxQTokens], int hkv, int L,
                                        int lane) {
#pragma unroll
    for (int j = 0; j < kMaxQTokens; ++j) {
      if (!mine[j] || (unsigned)rblk[j] >= (unsigned)a.c.num_blocks) continue;
      const int p = L - a.Tq + j;
      const size_t ri =
          ((size_t)rblk[j] * a.c.Hkv + hkv) * a.c.block_size + (size_t)(p % a.c.block_size);
      quantize_store_row<DT, MODE, D>(rk[j], lane, a.c.k_codes + ri * RG::ROWB, a.c.k_scales + ri,
                                      MODE == kPerChannel ? a.c.k_scales + (size_t)hkv * D : a.c.k_scales);
      if constexpr (kVRow)  // V per row: known at compile time
        quantize_store_row<DT, kPerRow, D>(rv[j], lane, a.c.v_codes + ri * RG::ROWB, a.c.v_scales + ri,
                                           a.c.v_scales);
      else
        quantize_store_row_mode<DT, D>(a.vmode, rv[j], lane, a.c.v_codes + ri * RG::ROWB,
                                       a.c.v_scales + ri,
                                       a.vmode == kPerChannel ? a.c.v_scales + (size_t)hkv * D : a.c.v_scales);
    }
    __builtin_amdgcn_s_waitcnt(0);  // stores acknowledged before any load of those rows
  }
};

// NB tiles of codes are held per wavefront: while one is processed, the loads
// of the next NB-1 are in flight.
template <int DT, int MODE, int D, int RB, int WPE = kSplitWavesPerSimd>
struct Knobs {
  // q operand from LDS instead of registers: the bf16 tiles need those
  // registers, and so do the three query slices of an int8 cache with a
  // per-channel K scale once the accumulators fill a wavefront (RB * D = 256:
  // in registers they spilled 13-45 of them to scratch).  (For the 8-bit
  // caches with two slices this measured slower on MI355X: 64K int8
  // 28.9 -> 30.5 us, and 3 tiles in flight with it 33.6 us, with spills.)
  // Wide row sets (RB * D above kSplitMaxAccColumns) always read it from LDS.
  static constexpr bool WIDE = RB * D > kSplitMaxAccColumns;
  static constexpr bool QLDS =
      WIDE || DT == kBf16 || (DT == kInt8 && MODE == kPerChannel && RB * D >= kSplitMaxAccColumns);
  // Wide row sets of the quantized caches pipeline the tile loop by one tile
  // -- except where the accumulators fill the accumulation registers (RB * D
  // = 768), whose pipelined loop spilled.  The pipelined loop keeps two tiles
  // in flight (a third spilled in some variants), the other wide loops three.
  static constexpr bool PIPE = WIDE && DT != kBf16 && RB * D < kSplitMaxWideColumns;
  static constexpr int NB = !WIDE || PIPE ? kSplitTilesInFlight : kSplitWideTilesInFlight;
  static constexpr int WAVES_PER_EU = WPE;
  static_assert(!WIDE || WPE == 1, "wide row sets need one wavefront per SIMD");
  // merge buffers: one per wavefront, MRB row blocks at a time (64 KiB)
  static constexpr int MERGE_BUFS = kWaves;
  static constexpr int MRB = WIDE ? kSplitMaxAccColumns / D : RB;
  static constexpr int MPASS = (RB + MRB - 1) / MRB;
  static_assert(MERGE_BUFS * 16 * MRB * D * 4 <= 65536, "merge buffers exceed 64 KiB");
};

// Variants whose accumulators fill a wavefront and whose rows exceed 128 bytes
// sit at the 256-register budget of two wavefronts per SIMD (a spill there is a
// scratch reload in the tile loop, which waits for every tile load before it).
// Launches that place one workgroup per CU run them with WPE = 1 instead: up to 512 registers, the MFMA
// accumulators in ordinary VGPRs (the units build with -amdgpu-mfma-vgpr-form)
// and any excess held in the accumulation registers, not in memory.
template <int DT, int D, int RB>
constexpr bool kHeavy = Geo<DT, D>::ROWB > 128 && RB * D >= kSplitMaxAccColumns;

template <int DT, int MODE, int D, int RB, bool CAP, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void
split_decode_kernel(SplitArgs a) {
  using G_ = Geo<DT, D>;
  using K_ = Knobs<DT, MODE, D, RB, WPE>;
  constexpr int RP = 16 * RB;  // padded query rows
  constexpr int NB = K_::NB;

  // q rows staged as bf16 and the workgroup's q operand after them, then the
  // merge buffers
  constexpr int kQStageBytes = (RP * kQStride<D> * 2 + 255) / 256 * 256;
  constexpr int kQOpBytes = RB * kQOps<DT, MODE, D> * 64 * 16;  // the workgroup's q operand
  constexpr int kMergeFloats = K_::MERGE_BUFS * 16 * K_::MRB * D;
  constexpr int kSmemFloats = kMergeFloats > (kQStageBytes + kQOpBytes) / 4 ? kMergeFloats
                                                                            : (kQStageBytes + kQOpBytes) / 4;
  __shared__ __attribute__((aligned(16))) float smem[kSmemFloats];
  static_assert(kSmemFloats * 4 <= 65536, "the q operand does not fit 64 KiB");
  __shared__ float s_pmax[kWaves * RP];  // row maxima of each wavefront's k-steps
  __shared__ float s_m[kWaves][RP];
  __shared__ float s_l[kWaves][RP];
  __shared__ float s_vref[kWaves];
  __shared__ float s_f[K_::MPASS > 1 ? kWaves : 1][RP];  // merge weights (several passes)
  __shared__ float s_kst[MODE == kPerChannel ? D : 1];  // static K scales (per channel / tensor)

  const int hkv = blockIdx.y;
  // Row-split launches (RBN > 1) share a chunk's query rows out over RBN
  // workgroups of RB 16-row blocks each.  The x index packs (chunk slot, row
  // set) so that the RBN workgroups of one chunk are 8 dispatch positions
  // apart: the dispatcher deals workgroups to the 8 XCDs in turn, so they
  // share one L2 and read the chunk's bytes from HBM once.  (With a fused
  // append, each of them quantizes and stores the same new rows before it
  // reads them: identical bytes, so no workgroup waits for another.)
  int slot = blockIdx.x, rbi = 0;
  if (a.RBN > 1) {
    const int grp = slot / (8 * a.RBN), rem = slot % (8 * a.RBN);
    rbi = rem / 8;
    slot = grp * 8 + rem % 8;
    if (slot >= a.S) return;
  }
  const int row0 = rbi * RP;               // first query row of this workgroup
  const int Rw = min(RP, a.R - row0);      // its query rows
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;  // S^T column / P row / V column index
  const int g = lane >> 4;  // lane group

  constexpr int QU = D / 8;                           // 16-byte units per q row
  constexpr int QPT = (RP * QU + 255) / 256;          // units per thread
  // Query rows of sequence bq: unconditional loads, clamped to row 0, so no
  // branch joins on their data (padding rows are zeroed when staged).  Issued
  // before the tiles: loads retire in order, so staging them later waits only
  // for them.
  u32x4_t qreg[QPT];
  auto load_q = [&](int bq) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int u = (tid + 256 * i) % (RP * QU);
      const int r = u / QU, cu = u % QU;
      const int rr = row0 + (r < Rw ? r : 0);
      const int jq = rr / a.G, gh = rr % a.G;
      const uint16_t* src = a.q + ((((size_t)bq * a.Tq + jq) * a.Hq) + (size_t)hkv * a.G + gh) * D;
      qreg[i] = *reinterpret_cast<const u32x4_t*>(src + cu * 8);
    }
  };

  // ---- this workgroup's chunk under the balanced schedule (every wavefront
  // derives the same one; an idle slot leaves as a whole before any barrier).
  // The first wavefront of slot 0, KV head 0, row block 0 also records every
  // sequence's chunk slots for the combine.
  int b, L, tb, te;
  if (!workgroup_chunk(a, slot, slot == 0 && hkv == 0 && rbi == 0 && wave == 0, lane, load_q, b, L, tb,
                       te))
    return;
  const int t0 = tb + wave;  // the wavefront's tiles are t0, t0 + 4, ...
  // The block-table reads of its tiles go out first: loads return in order,
  // so the first tile loads, which need them, wait for nothing issued after
  // them (a batch's query rows, the new rows, the scales).
  const TableLoads tl = table_issue(a, b, t0, kWaves, lane);
  if (a.B > 1) load_q(b);

  // ---- fused append: the wavefront that will read the tile holding a new
  // position quantizes and stores that row (the same arithmetic as
  // kvq_append) and waits for its stores before it issues the load of that
  // tile.  No other wavefront of the workgroup reads those rows.  Position
  // L - Tq + j holds query token j's row.
  bool mine[kMaxQTokens];    // wave-uniform
  bool any_mine = false, early_hit = false;
#pragma unroll
  for (int j = 0; j < kMaxQTokens; ++j) {
    const int p = L - a.Tq + j;
    const int t = p / kTile;
    mine[j] = a.k_new != nullptr && j < a.Tq && p >= 0 && t >= tb && t < te && (t - tb) % kWaves == wave;
    any_mine |= mine[j];
    early_hit |= mine[j] && t < t0 + NB * kWaves;  // among the first NB tiles
  }
  // The static K scales of this head (per channel: one per thread), loaded
  // before the tile loads: loads return in order, so the query fold would
  // otherwise wait for the first tiles (measured on MI355X, workload 5: the
  // fold ended 8.2 us after the workgroup started).
  float kst_v = 0.0f;
  if constexpr (MODE == kPerChannel) {
    static_assert(D <= 256, "one scale per thread");
    kst_v = tid < D ? a.c.k_scales[(size_t)hkv * D + tid] : 0.0f;
  } else if constexpr (MODE == kPerTensor) {
    kst_v = a.c.k_scales[0];
  }
  NewRows<DT, MODE, D> nr;
  if (any_mine) nr.load(a, mine, b, hkv, L, lane);  // first, so their latency overlaps the tile loads
  auto append_rows = [&]() { nr.store(a, mine, hkv, L, lane); };

  // ---- start the loads of the wavefront's first NB tiles now so their
  // latency overlaps the query prologue (and the append).  Every load is
  // issued unconditionally (tiles past the split read nothing).  A wavefront
  // whose first tiles hold a new row appends first; any other appends after
  // issuing them, so the stores overlap the loads.
  const TableRegs tbl = table_finish(a, hkv, tl);
  Tile<DT, D> buf[NB];
  // (the loads stay at one program point, so the compiler's waits for them
  // remain exact on the path every wavefront but one takes)
  if (early_hit) append_rows();
#pragma unroll
  for (int i = 0; i < NB; ++i)
    load_tile<DT, MODE, D>(a, t0 + i * kWaves, t0 + i * kWaves < te, table_entry(tbl, i), L, n, g,
                           buf[i]);
  if (any_mine && !early_hit) append_rows();

  // ---- stage the query rows in LDS (bf16), zero padding rows
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int u = tid + 256 * i;
    if (u < RP * QU) {
      const u32x4_t v = (u / QU < Rw) ? qreg[i] : u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(qs + (u / QU) * kQStride<D> + (u % QU) * 8) = v;
    }
  }
  if constexpr (MODE == kPerChannel) {
    if (tid < D) s_kst[tid] = kst_v;
  } else if constexpr (MODE == kPerTensor) {
    if (tid == 0) s_kst[0] = kst_v;
  }
  __syncthreads();

  // ---- B operands of S^T, folded once for the workgroup into LDS (lane-
  // linear, after the staged rows); the QLDS variants read them from there in
  // the tile loop, the others copy them into registers
  constexpr int QO = kQOps<DT, MODE, D>;
  half8_t* qop = reinterpret_cast<half8_t*>(reinterpret_cast<char*>(smem) + kQStageBytes);
  float rowmul[RB];  // logit (log2 units) = dot * rowmul * per-row K scale
  fold_q_shared<DT, MODE, D, RB>(a, qs, hkv, wave, n, g, lane, qop, s_pmax, s_kst, rowmul);
  const half8_t* qlds = qop + lane;
  half8_t qb[RB][QO];
  if constexpr (!K_::QLDS) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int k = 0; k < QO; ++k) qb[rb][k] = qlds[(rb * QO + k) * 64];
    // every wavefront holds its copy before any overwrites the area (the
    // merge writes its accumulators there as soon as its loop ends)
    __syncthreads();
  }
  int lim[RB];  // tokens visible to this lane's row n: lo <= t < lim
  int lo[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + n;
    row_window(a, L, row0 + r, r < Rw, lim[rb], lo[rb]);
  }

  // soft cap in log2 units (the CAP variant is launched when softcap > 0)
  const float cap2 = CAP ? a.softcap * 1.4426950408889634f : 0.0f;
  const float icap2 = CAP ? 2.0f / a.softcap : 0.0f;
  WaveState<DT, D, RB> W;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    W.m[rb] = -INFINITY;
    W.l[rb] = 0.0f;
#pragma unroll
    for (int c = 0; c < G_::NCOL; ++c) W.acc[rb][c] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  W.vref = 0x1p-126f;  // smallest normal: any nonzero scale above it raises the reference
  W.ivref = 0x1p126f;

  if constexpr (!K_::WIDE) {
    for (int t = t0, k = 0; t < te;) {
      // Two workgroups per CU share each SIMD, and the issue arbiter favours
      // the older wavefront: left alone, the workgroup dispatched first ran
      // ahead and the other finished its last tiles alone (int4 at 64K on
      // MI355X: loops ended at 11.8 us against 15.2 us, by dispatch order).
      // A wavefront's priority follows the share of its tiles it has left, so
      // the one behind is served first (the two halves' loops then ended
      // 0.8 us apart instead of 3.4; the kernel 18.45 -> 18.2 us).
      if constexpr (WPE > 1) {
        const int left = te - t, all = te - t0;
        if (4 * left > 3 * all)
          __builtin_amdgcn_s_setprio(3);
        else if (2 * left > all)
          __builtin_amdgcn_s_setprio(2);
        else if (4 * left > all)
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_s_setprio(0);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (t < te)
          process_tile<DT, MODE, D, RB, CAP, K_::QLDS>(buf[i], t, n, g, qb, qlds, rowmul, lim, lo, cap2,
                                                       icap2, W);
        load_tile<DT, MODE, D>(a, t + NB * kWaves, t + NB * kWaves < te, table_entry(tbl, k + NB), L, n,
                               g, buf[i]);
        t += kWaves;
        ++k;
      }
    }
    if constexpr (WPE > 1) __builtin_amdgcn_s_setprio(0);
  } else if constexpr (K_::PIPE) {
    // Wide row sets of the quantized caches: the accumulators live in the
    // accumulation registers, which vector ALU instructions cannot multiply,
    // so the rare reference moves and their rescales run outside the tile
    // loop, and the loop is pipelined by one tile so that one wavefront per
    // SIMD keeps both units busy: while tile t's logits and weights are
    // computed, tile t + 1's S^T MFMAs run; while tile t's P . V MFMAs run,
    // tile t + 1's V is unpacked.  A tile's slot is free once its S^T and V
    // unpack are done, so its next load is issued at the start of the tile's
    // step.  A tile whose references must move leaves the ring: it and the
    // rest of the ring take the general weights, and the ring restarts at its
    // first slot.
    QKAcc<DT, MODE, D, RB> qa;  // S^T of the next tile
    VTile<DT, D> vc;            // V operands of the current tile
    float4_t nks, nvs;          // scales and pool flag of the next tile
    int nok;
    float cdot[RB][4];          // the current tile's
    float4_t cks, cvs;
    int cok;
    half4_t pa[RB];
    u32x2_t phi[RB], plo[RB];
    int t = t0, k = 0;
    if (t0 < te) {
      qk_issue<DT, MODE, D, RB>(buf[0].kw, qlds, qa);
      nks = buf[0].ks4;
      nvs = buf[0].vs4;
      nok = buf[0].ok;
      unpack_v<DT, D>(buf[0].vw, vc);
      // the references start at the first tile's row maxima (and, per-row
      // V, its largest V scale); the accumulators are still zero
      float dot[RB][4];
      qk_dots<DT, MODE, D, RB>(qa, dot);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float z[4];
        tile_logits<MODE, CAP>(dot[rb], nks, nok != 0, t0 * kTile + 4 * g, rowmul[rb], lim[rb], lo[rb], cap2,
                               icap2, z);
        W.m[rb] = group_max4(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
      }
      if constexpr (kVRow) {
        float vfac, vsn[4];
        bool moved = false;
        v_reference(nvs, W.vref, W.ivref, vfac, moved, vsn);
      }
    }
    // the first half of tile t's step in slot S: the slot's next load, the
    // tile's dot products, the next tile's S^T
    auto front = [&](auto S) {
      constexpr int sl = decltype(S)::value, s1 = (sl + 1) % NB;
      load_tile<DT, MODE, D>(a, t + NB * kWaves, t + NB * kWaves < te, table_entry(tbl, k + NB), L, n, g,
                             buf[sl]);
      qk_dots<DT, MODE, D, RB>(qa, cdot);
      cks = nks;
      cvs = nvs;
      cok = nok;
      qk_issue<DT, MODE, D, RB>(buf[s1].kw, qlds, qa);
      nks = buf[s1].ks4;
      nvs = buf[s1].vs4;
      nok = buf[s1].ok;
    };
    // the second half: P . V, the next tile's V operands
    auto back = [&](auto S) {
      constexpr int s1 = (decltype(S)::value + 1) % NB;
      pv_unpacked<DT, D, RB>(vc, pa, W.acc);
      unpack_v<DT, D>(buf[s1].vw, vc);
      t += kWaves;
      ++k;
    };
    while (t < te) {
      int hit = -1;
      bool stop = false;
      do {
        static_for<NB>([&](auto S) {
          if (stop) return;
          if (t >= te) {
            stop = true;
            return;
          }
          front(S);
          if (weights_fast<DT, MODE, RB, CAP>(cdot, cks, cvs, cok != 0, t, g, rowmul, lim, lo, cap2, icap2, W,
                                              pa, phi, plo)) {
            hit = decltype(S)::value;
            stop = true;
            return;
          }
          back(S);
        });
      } while (!stop);
      if (hit < 0) break;
      // the tile that left the ring (its front half done) and the rest of
      // the ring through the general weights
      static_for<NB>([&](auto S) {
        constexpr int sl = decltype(S)::value;
        if (sl < hit || t >= te) return;
        if (sl > hit) front(S);
        weights_general<DT, MODE, D, RB, CAP>(cdot, cks, cvs, cok != 0, t, g, rowmul, lim, lo, cap2, icap2, W, pa,
                                              phi, plo);
        back(S);
      });
    }
  } else {
    // Wide row sets: the accumulators live in the accumulation registers,
    // which vector ALU instructions cannot multiply, so the rare reference
    // moves and rescales run outside the tile loop (inside it, the compiler
    // copied every accumulator out and back on every tile).  The loop runs
    // tile_fast and leaves at a tile that needs a move, before its P . V and
    // its slot's next load; the tail below takes that tile and the rest of the
    // ring through the general step, so the loop always resumes at the ring's
    // first slot with the usual loads in flight.
    static_assert(!K_::WIDE || K_::QLDS, "wide row sets read q from LDS");
    // The references start at the first tile's row maxima (and, per-row V,
    // its largest V scale), so that tile and the many like it stay in the
    // loop; the accumulators are still zero, so nothing is rescaled.
    if (t0 < te) {
      float dot[RB][4];
      tile_dots_lds<DT, MODE, D, RB>(buf[0].kw, qlds, dot);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float z[4];
        tile_logits<MODE, CAP>(dot[rb], buf[0].ks4, buf[0].ok != 0, t0 * kTile + 4 * g, rowmul[rb], lim[rb],
                               lo[rb], cap2, icap2, z);
        W.m[rb] = group_max4(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
      }
      if constexpr (kVRow) {
        float vfac, vsn[4];
        bool moved = false;
        v_reference(buf[0].vs4, W.vref, W.ivref, vfac, moved, vsn);
      }
    }
    int t = t0, k = 0;
    while (t < te) {
      int hit = -1;
      do {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (t >= te) break;
          half4_t pa[RB];
          u32x2_t phi[RB], plo[RB];
          if constexpr (DT == kBf16) {
            if (tile_fast<DT, MODE, D, RB, CAP>(buf[i], t, g, qlds, rowmul, lim, lo, cap2, icap2, W, pa, phi,
                                                plo)) {
              hit = i;
              break;
            }
            accumulate_pv<DT, D, RB>(buf[i].vw, pa, phi, plo, W.acc);
          } else {
            VTile<DT, D> V;
            unpack_v<DT, D>(buf[i].vw, V);
            if (tile_fast<DT, MODE, D, RB, CAP>(buf[i], t, g, qlds, rowmul, lim, lo, cap2, icap2, W, pa, phi,
                                                plo)) {
              hit = i;
              break;
            }
            pv_unpacked<DT, D, RB>(V, pa, W.acc);
          }
          load_tile<DT, MODE, D>(a, t + NB * kWaves, t + NB * kWaves < te, table_entry(tbl, k + NB), L, n,
                                 g, buf[i]);
          t += kWaves;
          ++k;
        }
      } while (hit < 0 && t < te);
      if (hit < 0) break;
      // the tile that left the loop and the rest of the ring through the
      // general step (references moved, accumulators rescaled)
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (i >= hit) {
          if (t < te)
            process_tile<DT, MODE, D, RB, CAP, true>(buf[i], t, n, g, qb, qlds, rowmul, lim, lo, cap2, icap2,
                                                     W);
          load_tile<DT, MODE, D>(a, t + NB * kWaves, t + NB * kWaves < te, table_entry(tbl, k + NB), L, n,
                                 g, buf[i]);
          t += kWaves;
          ++k;
        }
      }
    }
  }

  // ---- merge the 4 wavefronts in fixed order, write the split partial.
  // Each wavefront publishes its row statistics and its raw accumulator rows
  // (to its own LDS buffer).  Where the loop read q from registers the LDS is
  // free by then, so a wavefront writes them as soon as its own loop ends,
  // while slower ones are still loading, and one barrier is left.  The
  // readback weighs each wavefront's rows by exp2(m_w - M) / L and sums the
  // buffers in wave order.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float lsum = group_sum4(W.l[rb]);
    if (g == 0) {
      s_m[wave][rb * 16 + n] = W.m[rb];
      s_l[wave][rb * 16 + n] = lsum;
    }
  }
  if constexpr (kVRow)
    if (lane == 0) s_vref[wave] = W.vref;

  // Lane column n owns NCOL channels, NCOL / 4 groups of 4 consecutive ones
  // (see group_owner); they go to the lane's NCOL-float LDS slot as 16-byte
  // chunks whose order is rotated by n / (64 / NCOL) so the 16 lanes of a pass
  // hit distinct banks.
  constexpr int NCH = G_::NCOL / 4;                 // 16-byte chunks per lane and row
  constexpr int ROT = G_::NCOL >= 16 ? 4 : (G_::NCOL == 8 ? 8 : 16);
  // Wide row sets merge MRB row blocks per pass (the buffers hold 64 KiB).
  constexpr int MRB = K_::MRB;
  constexpr int MR = 16 * MRB;  // rows per pass
  constexpr bool kEarly = !K_::QLDS && K_::MPASS == 1;
  auto write_rows = [&](int p) {
    float* ob = smem + (size_t)wave * MR * D;
#pragma unroll
    for (int rr = 0; rr < MRB; ++rr) {
      const int rb = p * MRB + rr;
      if (rb < RB) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rb * 16 + 4 * g + e;
          if (r < Rw) {
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
              float4_t v;
#pragma unroll
              for (int i = 0; i < 4; ++i) v[i] = W.acc[rb][col_of<DT, D>(4 * k + i)][e];
              const int slot = (k + n / ROT) % NCH;
              *reinterpret_cast<float4_t*>(ob + (r - p * MR) * D + G_::NCOL * n + 4 * slot) = v;
            }
          }
        }
      }
    }
  };
  if constexpr (kEarly) write_rows(0);
  __syncthreads();

  // the chunk's statistics of row r (log2 units) and the weight of each
  // wavefront's rows: exp2(m_w - M) / L, times its V reference (1/16 more for
  // int4, whose V operand holds 16 * code); the partial's m and l stored
  auto row_weights = [&](int r, float (&f)[kWaves]) {
    float M = s_m[0][r];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][r]);
    float Lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      // the hardware exp2, as in the tile loop (results below 2^-126 flush to 0)
      f[w] = M != -INFINITY ? __builtin_amdgcn_exp2f(s_m[w][r] - M) : 0.0f;
      Lt += s_l[w][r] * f[w];
    }
    const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      f[w] *= inv;
      if constexpr (kVRow) f[w] *= s_vref[w];
      if constexpr (DT == kInt4) f[w] *= 0.0625f;
    }
    return std::pair<float, float>(M, Lt);
  };
  // Several passes (wide row sets): one thread per row turns the statistics
  // into weights once, for every pass (its barriers publish them); one pass:
  // each thread takes its own row's.
  constexpr bool kRowTable = K_::MPASS > 1;
  if constexpr (kRowTable) {
    if (tid < Rw) {
      float f[kWaves];
      const auto ml = row_weights(tid, f);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s_f[w][tid] = f[w];
      const size_t ri = ((size_t)hkv * a.R + row0 + tid) * a.S + slot;
      a.ws_m[ri] = ml.first;
      a.ws_l[ri] = ml.second;
    }
  }
#pragma unroll
  for (int p = 0; p < K_::MPASS; ++p) {
    if constexpr (!kEarly) {
      if (p > 0) __syncthreads();  // the previous pass's readback is done
      write_rows(p);
      __syncthreads();
    }
    const int rn = min(MR, Rw - p * MR);  // rows of this pass
    for (int idx = tid * 4; idx < rn * D; idx += 256 * 4) {
      const int lr = idx / D, d = idx % D, r = p * MR + lr;
      const size_t ri = ((size_t)hkv * a.R + row0 + r) * a.S + slot;
      float f[kWaves];
      if constexpr (kRowTable) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) f[w] = s_f[w][r];
      } else {
        const auto ml = row_weights(r, f);
        if (d == 0) {
          a.ws_m[ri] = ml.first;
          a.ws_l[ri] = ml.second;
        }
      }
      int jn, k;
      group_owner<DT, D>(d, jn, k);
      const int off = lr * D + G_::NCOL * jn + 4 * ((k + jn / ROT) % NCH);
      float4_t v = f[0] * *reinterpret_cast<const float4_t*>(smem + off);
#pragma unroll
      for (int w = 1; w < kWaves; ++w)
        v += f[w] * *reinterpret_cast<const float4_t*>(smem + (size_t)w * MR * D + off);
      *reinterpret_cast<float4_t*>(a.ws_o + ri * D + d) = v;
    }
  }
}

#define KVQ_CAT2(a, b, c, d) a##b##_##c##_##d
#define KVQ_CAT(a, b, c, d) KVQ_CAT2(a, b, c, d)

#if !KVQ_WIDE
template <int DT, int MODE, int D, int RB>
hipError_t launch_one(const SplitArgs& a, int B, hipStream_t st) {
  // Row sets whose accumulators exceed a two-wavefronts-per-SIMD budget run in
  // the unit's wide variants; the host gives wider ones one workgroup per
  // 16-row block instead.
  (void)B;
  if constexpr (RB * D > kSplitMaxWideColumns) {
    (void)a;
    (void)st;
    return hipErrorInvalidValue;
  } else if constexpr (RB * D > kSplitMaxAccColumns) {
    return KVQ_CAT(launch_split_wide_, KVQ_DTYPE, KVQ_MODE, KVQ_VROW)(D, RB, a, st);
  } else {
    const int gx = a.RBN > 1 ? (a.S + 7) / 8 * 8 * a.RBN : a.S;
    dim3 grid(gx, a.c.Hkv, 1);
    constexpr int W2 = kSplitWavesPerSimd;
    if constexpr (kHeavy<DT, D, RB>) {
      if (a.one_per_cu) {
        if (a.softcap > 0.0f)
          hipLaunchKernelGGL((split_decode_kernel<DT, MODE, D, RB, true, 1>), grid, dim3(256), 0, st, a);
        else
          hipLaunchKernelGGL((split_decode_kernel<DT, MODE, D, RB, false, 1>), grid, dim3(256), 0, st, a);
        return hipGetLastError();
      }
    }
    if (a.softcap > 0.0f)
      hipLaunchKernelGGL((split_decode_kernel<DT, MODE, D, RB, true, W2>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((split_decode_kernel<DT, MODE, D, RB, false, W2>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
}

template <int DT, int MODE, int D>
hipError_t launch_d(int RB, const SplitArgs& a, int B, hipStream_t st) {
  switch (RB) {
    case 1: return launch_one<DT, MODE, D, 1>(a, B, st);
    case 2: return launch_one<DT, MODE, D, 2>(a, B, st);
    case 3: return launch_one<DT, MODE, D, 3>(a, B, st);
    case 4: return launch_one<DT, MODE, D, 4>(a, B, st);
    default: return hipErrorInvalidValue;
  }
}
#else
// A wide row set: one workgroup per chunk slot (RBN of them when the row
// blocks are shared out), one wavefront per SIMD.
template <int DT, int MODE, int D, int RB>
hipError_t launch_wide(const SplitArgs& a, hipStream_t st) {
  static_assert(RB * D > kSplitMaxAccColumns && RB * D <= kSplitMaxWideColumns, "not a wide row set");
  const int gx = a.RBN > 1 ? (a.S + 7) / 8 * 8 * a.RBN : a.S;
  dim3 grid(gx, a.c.Hkv, 1);
  if (a.softcap > 0.0f)
    hipLaunchKernelGGL((split_decode_kernel<DT, MODE, D, RB, true, 1>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((split_decode_kernel<DT, MODE, D, RB, false, 1>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}
#endif

}  // namespace

#if !KVQ_WIDE
hipError_t KVQ_CAT(launch_split_, KVQ_DTYPE, KVQ_MODE, KVQ_VROW)(int D, int RB, const SplitArgs& a,
                                                                  int B, hipStream_t st) {
  switch (D) {
    case 64: return launch_d<KVQ_DTYPE, KVQ_MODE, 64>(RB, a, B, st);
    case 128: return launch_d<KVQ_DTYPE, KVQ_MODE, 128>(RB, a, B, st);
    case 256: return launch_d<KVQ_DTYPE, KVQ_MODE, 256>(RB, a, B, st);
    default: return hipErrorInvalidValue;
  }
}
#else
hipError_t KVQ_CAT(launch_split_wide_, KVQ_DTYPE, KVQ_MODE, KVQ_VROW)(int D, int RB, const SplitArgs& a,
                                                                       hipStream_t st) {
  if (D == 128 && RB == 3) return launch_wide<KVQ_DTYPE, KVQ_MODE, 128, 3>(a, st);
  if (D == 128 && RB == 4) return launch_wide<KVQ_DTYPE, KVQ_MODE, 128, 4>(a, st);
  if (D == 256 && RB == 2) return launch_wide<KVQ_DTYPE, KVQ_MODE, 256, 2>(a, st);
  if (D == 256 && RB == 3) return launch_wide<KVQ_DTYPE, KVQ_MODE, 256, 3>(a, st);
  return hipErrorInvalidValue;
}
#endif

}  // namespace kvq
