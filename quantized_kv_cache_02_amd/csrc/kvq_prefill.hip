// kvq_prefill.hip -- chunked prefill: the Tq tokens of a chunk (already
// quantized into the cache at positions seq_len - Tq .. seq_len - 1) attend
// causally to every cached token up to their own, on gfx950.  Compiled once per
// (KVQ_DTYPE, KVQ_MODE, KVQ_VROW) like the decode kernel.
//
// Kernel page "kv-quant-attn", "Requirements and limits": prefill is a tiled
// attention kernel whose keys and values are then handed to the append; ORT
// PR "[CUDA] Add INT4 paged KV cache ...", "Testing": prefill and chunked
// prefill over the paged quantized cache.  Here the chunk is appended first
// (the same quantize-on-write as every other row) and then attended through
// the cache, so a chunk sees exactly the cache a later decode sees.
//
// Work assignment: one workgroup per (sequence, KV head, 128 query rows), the
// rows being the G grouped heads times the chunk's tokens (row = token * G +
// head).  Below D = 256 each of 4 wavefronts owns 32 rows (two 16-row MFMA
// blocks, so every operand read from LDS feeds two MFMAs); at D = 256 each of
// 8 wavefronts owns 16.  The workgroup walks the 64-token tiles its rows can
// see; per tile all its threads load the codes and unpack them once into LDS
// -- K as fp16 rows, V transposed to channel-major --
// into one of two buffers, so the next tile is loaded and unpacked while this
// one is used (one barrier per tile), and every wavefront runs
//   S^T = K . Q^T   v_mfma_f32_16x16x32_f16 (A: K rows from LDS, B: its q rows),
//   online softmax over the tile's 64 tokens per row,
//   O  += P . V     v_mfma_f32_16x16x32_f16 over two 16-token sub-tiles (A: the
//                   weights where S^T left them, B: the same 8 tokens of one
//                   channel read from the transposed V).
// Scales enter as in the decode kernel: a per-row K scale multiplies the
// logit, a per-row V scale the weight (over a power-of-two reference),
// per-channel K is folded into q, static V scales are applied at the output.
// A bf16 cache runs on the bf16 MFMAs with the weights split hi + lo.

#include "kvq_device.h"
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

namespace kvq {
namespace {

constexpr bool kVRow = KVQ_VROW != 0;
constexpr int kPT = 64;  // tokens per KV tile
// 16-row blocks per wavefront: two (every operand read from LDS feeds two
// MFMAs) where the accumulators fit the registers beside the q operands; at
// D = 256 two blocks pushed the accumulators into the accumulation registers
// and the compiler copied them back and forth every tile.
template <int D>
constexpr int kPRowBlocks = D >= 256 ? 1 : 2;
// Wavefronts per workgroup (W): 4, or at D = 256 also 8 (one row block each,
// so the tile's unpack is shared by 128 rows and two wavefronts per SIMD hide
// each other's stalls; the two tile buffers still fit the LDS) when that still
// gives every CU a workgroup.
template <int D, int W>
constexpr int kPRows = 16 * kPRowBlocks<D> * W;  // query rows per workgroup

template <int DT, int D, int W>
struct PGeo {
  static constexpr int ROWB = (DT == kInt4) ? D / 2 : (DT == kBf16) ? 2 * D : D;
  // The integer caches take S^T on the int8 MFMA: their K tile holds the codes
  // as bytes (int4: 16 n), rows of D + 16 bytes; the others hold fp16 rows of
  // D + 8 elements.  KST is the row stride in 16-bit elements either way.
  static constexpr bool IQK = DT == kInt8 || DT == kInt4;
  static constexpr int KST = IQK ? (D + 16) / 2 : D + 8;
  static constexpr int ISTEPS = D / 64;  // 16x16x64 int8 MFMAs per S^T sub-tile (and q half)
  // transposed V row stride (16-bit elements): 42 dwords.  Measured on MI355X
  // (chunked prefill, 1-2K tokens after 16-32K): 84 beats 72 by 12 % for int8
  // and 22 % for bf16 and ties the best int4 stride; 76 does about as well,
  // 72 and 80 (multiples of 4 dwords) are slow, and 68 was fast for int4 only.
  static constexpr int VST = kPT + 20;
  static constexpr int KSTEPS = D / 32;  // 16x16x32 MFMAs per S^T sub-tile
  static constexpr int NCOL = D / 16;    // 16-channel output column blocks
  static constexpr int NT = 64 * W;
  // K load: thread -> token tid / KP, bytes [KQB * (tid % KP), +KQB) of its row
  static constexpr int KP = NT / kPT;    // threads per K row
  static constexpr int KQB = ROWB / KP;
  // V load: thread -> channel chunk tid / 16 (VNC chunks of D / VNC channels),
  // tokens 4 * (tid % 16) + 0..3
  static constexpr int VNC = NT / 16;
  static constexpr int VCB = ROWB / VNC;  // bytes of one token in one chunk
  static constexpr int VCW = VCB >= 4 ? VCB / 4 : 1;
  static constexpr int CPD = (DT == kInt4) ? 8 : (DT == kBf16) ? 2 : 4;  // channels per dword
};

// Load N (2, 4, 8 or 16) bytes from a device address into dwords.
template <int N>
__device__ __forceinline__ void gload(const uint8_t* p, uint32_t* out) {
  if constexpr (N >= 16) {
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i);
      out[4 * i] = v[0]; out[4 * i + 1] = v[1]; out[4 * i + 2] = v[2]; out[4 * i + 3] = v[3];
    }
  } else if constexpr (N == 8) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    out[0] = v[0]; out[1] = v[1];
  } else if constexpr (N == 4) {
    out[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  } else {
    static_assert(N == 2, "unsupported load");
    out[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
  }
}

// Codes (and per-row scales) of one tile as this thread loads them.  Rows
// that cannot be read are loaded from row 0 and flagged; the flags are applied
// when the tile is unpacked, so nothing between the loads and that point waits
// for the loaded values (the next tile's loads stay in flight under this
// tile's math).
template <int DT, int D, int W>
struct PTile {
  uint32_t k[PGeo<DT, D, W>::KQB / 4];
  uint32_t v[4][PGeo<DT, D, W>::VCW];
  float ks, vs;  // per-row scales of token tid (threads 0..63)
  bool kok, vok[4], sok;
};

// Cache rows of one 64-token tile: block sizes are multiples of 16, so each
// aligned group of 16 tokens lies in one block; r16[sg] is the cache row of
// token 16 * sg of the tile over 16 (-1: past the length or outside the pool;
// the host bounds the pool so that it fits an int).  Computed once per tile
// from uniform values.
struct TileRows {
  int r16[4];
};

// In units of 16 rows throughout (block sizes are multiples of 16, and the host
// bounds the pool to 2^31 such groups), so every step is 32-bit and wave-uniform.
__device__ __forceinline__ TileRows tile_rows(const PrefillArgs& a, int b, int hkv, int kt, int L) {
  TileRows tr;
  const int bs16 = a.c.block_size >> 4;
#pragma unroll
  for (int sg = 0; sg < 4; ++sg) {
    const int p = kt * kPT + 16 * sg;
    int r16 = -1;
    if (p < L) {
      if (a.c.block_table == nullptr) {
        r16 = (b * a.c.Hkv + hkv) * bs16 + (p >> 4);  // contiguous: p < L <= block_size
      } else {
        // a wave-uniform index, so the entry comes through a scalar load: a
        // vector load here would make its wait wait for the tile loads in
        // flight before it
        const unsigned q = (unsigned)p / (unsigned)a.c.block_size;
        const int col = __builtin_amdgcn_readfirstlane((int)q);
        const int blk = a.c.block_table[(size_t)__builtin_amdgcn_readfirstlane(b) * a.c.max_blocks + col];
        if ((unsigned)blk < (unsigned)a.c.num_blocks)
          r16 = (blk * a.c.Hkv + hkv) * bs16 + ((p - col * a.c.block_size) >> 4);
      }
    }
    tr.r16[sg] = __builtin_amdgcn_readfirstlane(r16);  // uniform: scalar registers
  }
  return tr;
}

// r16 of group sg (0..3) by masked xors on its two bits (a select chain here
// is turned into a table in scratch memory)
__device__ __forceinline__ int group_r16(const TileRows& tr, int sg) {
  const int m1 = -(sg & 1), m2 = -((sg >> 1) & 1);
  const int lo = tr.r16[0] ^ ((tr.r16[0] ^ tr.r16[1]) & m1);
  const int hi = tr.r16[2] ^ ((tr.r16[2] ^ tr.r16[3]) & m1);
  return lo ^ ((lo ^ hi) & m2);
}

// Loads read row 0 (always present) in place of a row they may not read; the
// flags say which rows are real, and the unpack zeroes the others.  Rows past
// the length inside a present group are read and flagged the same way.
template <int DT, int MODE, int D, int W>
__device__ __forceinline__ void load_ptile(const PrefillArgs& a, int b, int hkv, int kt, int L, int tid,
                                           PTile<DT, D, W>& T) {
  using P = PGeo<DT, D, W>;
  const TileRows tr = tile_rows(a, b, hkv, kt, L);
  const int lrem = L - kt * kPT;  // tokens of the tile before the length
  // K: one row part per thread; a wavefront's tokens share one group
  {
    const int tk = tid / P::KP;
    const int r16 = group_r16(tr, __builtin_amdgcn_readfirstlane(tk) >> 4);
    T.kok = r16 >= 0 && tk < lrem;
    const size_t row = T.kok ? (size_t)(uint32_t)r16 * 16 + (tk & 15) : 0;
    gload<P::KQB>(a.c.k_codes + row * P::ROWB + P::KQB * (tid % P::KP), T.k);
  }
  // V: 4 consecutive tokens (one group) of one channel chunk
  {
    const int tv = 4 * (tid % 16);
    const int r16 = group_r16(tr, tv >> 4);
    const size_t row = r16 >= 0 ? (size_t)(uint32_t)r16 * 16 + (tv & 15) : 0;
    const uint8_t* src = a.c.v_codes + row * P::ROWB + P::VCB * (tid / 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      T.vok[e] = r16 >= 0 && tv + e < lrem;
      if constexpr (P::VCB < 4) T.v[e][0] = 0u;  // the load fills the low bytes only
      gload<P::VCB>(src + e * P::ROWB, T.v[e]);
    }
  }
  // per-row scales of token tid % 64 (every thread loads; threads 0..63 store)
  {
    const int ts = tid % kPT;
    const int r16 = group_r16(tr, ts >> 4);
    T.sok = r16 >= 0 && ts < lrem;
    const size_t rs = T.sok ? (size_t)(uint32_t)r16 * 16 + (ts & 15) : 0;
    T.ks = 0.0f;
    T.vs = 0.0f;
    if constexpr (MODE == kPerRow) T.ks = __builtin_nontemporal_load(a.c.k_scales + rs);
    if constexpr (kVRow) T.vs = __builtin_nontemporal_load(a.c.v_scales + rs);
  }
}

// Unpack a loaded tile into LDS: K rows as int8 bytes (int8, int4 as 16 n) or
// fp16 (fp8; bf16 as is), V transposed to [channel][token] as fp16 (bf16),
// per-row scales.
template <int DT, int MODE, int D, int W>
__device__ __forceinline__ void stage_ptile(const PTile<DT, D, W>& T, int tid, uint16_t* ks_lds,
                                            uint16_t* vt_lds, float* ksc, float* vsc) {
  using P = PGeo<DT, D, W>;
  {
    // this thread's part of its row: channels (D / KP) * (tid % KP) .. + D / KP
    uint16_t* dst = ks_lds + (tid / P::KP) * P::KST + (P::IQK ? (D / P::KP) / 2 : (D / P::KP)) * (tid % P::KP);
    constexpr int NW = P::KQB / 4;  // dwords loaded
    // the thread's part of the row as dwords, then 16-byte LDS writes
    constexpr int OW = (DT == kInt4 || DT == kFp8) ? 2 * NW : NW;
    static_assert(OW % 4 == 0, "whole 16-byte writes");
    uint32_t ow[OW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint32_t kw = T.kok ? T.k[i] : 0u;
      if constexpr (DT == kInt8 || DT == kBf16) {
        ow[i] = kw;  // the codes (bf16 values) as they are
      } else if constexpr (P::IQK) {
        // 8 nibbles -> the bytes 16 n in channel order
        const uint32_t ev = (kw << 4) & 0xF0F0F0F0u, od = kw & 0xF0F0F0F0u;
        ow[2 * i] = perm(od, ev, 0x05010400u);
        ow[2 * i + 1] = perm(od, ev, 0x07030602u);
      } else {  // fp8 -> fp16
        fp8x4_to_h(kw, ow[2 * i], ow[2 * i + 1]);
      }
    }
#pragma unroll
    for (int j = 0; j < OW / 4; ++j)
      reinterpret_cast<u32x4_t*>(dst)[j] = u32x4_t{ow[4 * j], ow[4 * j + 1], ow[4 * j + 2], ow[4 * j + 3]};
  }
  {
    // channels [cb0, cb0 + D / 16) of tokens t0 .. t0 + 3
    constexpr int NCH = D / P::VNC;  // channels of this thread
    const int cb0 = NCH * (tid / 16), t0 = 4 * (tid % 16);
    uint32_t vv[4][P::VCW];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < P::VCW; ++i) vv[e][i] = T.vok[e] ? T.v[e][i] : 0u;
#pragma unroll
    for (int w = 0; w < P::VCW; ++w) {
      if constexpr (DT == kBf16) {
        // dword w holds channels 2w, 2w + 1
        const u32x2_t lo = {perm(vv[1][w], vv[0][w], 0x05040100u), perm(vv[3][w], vv[2][w], 0x05040100u)};
        const u32x2_t hi = {perm(vv[1][w], vv[0][w], 0x07060302u), perm(vv[3][w], vv[2][w], 0x07060302u)};
        *reinterpret_cast<u32x2_t*>(vt_lds + (cb0 + 2 * w) * P::VST + t0) = lo;
        *reinterpret_cast<u32x2_t*>(vt_lds + (cb0 + 2 * w + 1) * P::VST + t0) = hi;
      } else if constexpr (DT == kInt4) {
        // dword w holds channels 8w .. 8w + 7 (even in the low nibbles)
        uint32_t ev4[4], od4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = vv[e][w] ^ 0x88888888u;
          ev4[e] = (x << 4) & 0xF0F0F0F0u;
          od4[e] = x & 0xF0F0F0F0u;
        }
        half4_t ve[4], vo[4];
        v_transpose4<0>(ev4[0], ev4[1], ev4[2], ev4[3], ve);
        v_transpose4<0>(od4[0], od4[1], od4[2], od4[3], vo);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (8 * w + 2 * q < NCH)
            *reinterpret_cast<half4_t*>(vt_lds + (cb0 + 8 * w + 2 * q) * P::VST + t0) = ve[q];
          if (8 * w + 2 * q + 1 < NCH)
            *reinterpret_cast<half4_t*>(vt_lds + (cb0 + 8 * w + 2 * q + 1) * P::VST + t0) = vo[q];
        }
      } else {
        half4_t vb[4];
        if constexpr (DT == kInt8)
          v_transpose4<0>(vv[0][w] ^ 0x80808080u, vv[1][w] ^ 0x80808080u, vv[2][w] ^ 0x80808080u,
                          vv[3][w] ^ 0x80808080u, vb);
        else
          v_transpose4<1>(vv[0][w], vv[1][w], vv[2][w], vv[3][w], vb);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * w + q < NCH) *reinterpret_cast<half4_t*>(vt_lds + (cb0 + 4 * w + q) * P::VST + t0) = vb[q];
      }
    }
  }
  // (every thread writes the scales of token tid % 64: the same values)
  ksc[tid % kPT] = T.sok ? T.ks : 0.0f;
  vsc[tid % kPT] = T.sok ? T.vs : 0.0f;
}

template <int DT, int MODE, int D, int W, bool CAP>
__global__ __launch_bounds__(64 * W) void prefill_kernel(
    PrefillArgs a) {
  using P = PGeo<DT, D, W>;
  constexpr int KSTEPS = P::KSTEPS;
  constexpr int NCOL = P::NCOL;
  constexpr int RBW = kPRowBlocks<D>;
  constexpr int kRows = kPRows<D, W>;
  constexpr int KTILE_ELEMS = kPT * P::KST;
  constexpr int VTILE_ELEMS = D * P::VST;
  constexpr int BUF_ELEMS = KTILE_ELEMS + VTILE_ELEMS;
  // two tile buffers (K rows, transposed V): one is read while the next tile
  // is unpacked into the other; after the loop the output staging reuses them
  constexpr int OUT_ELEMS = W * 16 * RBW * (D + 4) * 2;  // the output staging, fp32
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BUF_ELEMS > OUT_ELEMS ? 2 * BUF_ELEMS : OUT_ELEMS];
  __shared__ float ksc[2][kPT], vsc[2][kPT];
  __shared__ float rowf[W][16 * RBW], rowsink[W][16 * RBW];
  static_assert(W * 16 * RBW * (D + 4) * 4 <= (int)sizeof(lds), "output staging does not fit");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  // The workgroups of sequence b (x: row group and context part, y: KV head)
  // in dispatch order are taken as (row group, KV head, part) with the part
  // fastest and the row groups in reverse: later rows see more of the causal
  // context, so the longest workgroups start first and the shortest fill the
  // last round; and the dispatcher, dealing workgroups to the 8 XCDs in turn,
  // gives each XCD the same (KV head, part) again and again when KS * Hkv
  // divides 8 (the tiles they share stay in that XCD's L2).
  const int lin = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  const int b = blockIdx.z;
  const int part = lin % a.KS;                 // context part (KS > 1: split launch)
  const int hkv = lin / a.KS % (int)gridDim.y;
  const int rbase = ((int)gridDim.x / a.KS - 1 - lin / (a.KS * (int)gridDim.y)) * kRows;  // first row
  const int rwave = rbase + 16 * RBW * wave;   // first row of this wavefront
  const int L = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int pos0 = L - a.Tq;                   // position of query token 0

  // rows rwave + 16 rb + n of this lane: visible tokens lo <= t < lim
  int lim[RBW], lo[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = rwave + 16 * rb + n;
    lim[rb] = 0;
    lo[rb] = 0;
    if (r < a.R) {
      lim[rb] = min(pos0 + r / a.G + 1, L);
      lo[rb] = a.window > 0 ? lim[rb] - a.window : 0;
    }
  }

  // the wavefront's tightest bounds over its rows (rows past R are never
  // written, so they do not constrain it): a tile inside [wlo_max, wlim_min)
  // needs no mask
  int wlim_min = 0x7FFFFFFF, wlo_max = 0;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const bool valid = rwave + 16 * rb + n < a.R;
    wlim_min = min(wlim_min, valid ? lim[rb] : 0x7FFFFFFF);
    wlo_max = max(wlo_max, valid ? lo[rb] : 0);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    wlim_min = min(wlim_min, __shfl_xor(wlim_min, o));
    wlo_max = max(wlo_max, __shfl_xor(wlo_max, o));
  }
  wlim_min = __builtin_amdgcn_readfirstlane(wlim_min);
  wlo_max = __builtin_amdgcn_readfirstlane(wlo_max);

  // q operand: row r, channels 32 ks + 8 g + 0..7 (zero rows past R).
  // Integer caches: channels 64 st + 16 g + 0..15 of the row as a fixed-point
  // integer vector in NSL int8 slices (q_slice_bytes: 15 bits of the row's largest
  // element, 23 with a per-channel K scale folded in); qb[rb][NSL st + k]
  // holds slice k.
  constexpr int NSL = MODE == kPerChannel ? 3 : 2;
  constexpr int QOPS = P::IQK ? NSL * P::ISTEPS : KSTEPS;
  half8_t qb[RBW][QOPS];
  float rowmul[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = rwave + 16 * rb + n;
    const int rr = r < a.R ? r : 0;
    const uint16_t* src = a.q + (((size_t)b * a.Tq + rr / a.G) * a.Hq + (size_t)hkv * a.G + rr % a.G) * D;
    if constexpr (P::IQK) {
      float qv[P::ISTEPS][16];
      float amax = 0.0f;
#pragma unroll
      for (int st = 0; st < P::ISTEPS; ++st) {
        const int c0 = 64 * st + 16 * g;
        u32x4_t r0 = *reinterpret_cast<const u32x4_t*>(src + c0);
        u32x4_t r1 = *reinterpret_cast<const u32x4_t*>(src + c0 + 8);
        if (r >= a.R) r0 = r1 = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qv[st][2 * i] = __uint_as_float(r0[i] << 16);
          qv[st][2 * i + 1] = __uint_as_float(r0[i] & 0xFFFF0000u);
          qv[st][8 + 2 * i] = __uint_as_float(r1[i] << 16);
          qv[st][8 + 2 * i + 1] = __uint_as_float(r1[i] & 0xFFFF0000u);
        }
#pragma unroll
        for (int p = 0; p < 16; ++p) {
          if constexpr (MODE == kPerChannel) qv[st][p] *= a.c.k_scales[(size_t)hkv * D + c0 + p];
          amax = fmaxf(amax, fabsf(qv[st][p]));
        }
      }
      amax = group_max4(amax);
      int ex = 0;
      if (amax > 0.0f) (void)frexpf(amax, &ex);
#pragma unroll
      for (int st = 0; st < P::ISTEPS; ++st) {
        uint32_t wb[16];
#pragma unroll
        for (int p = 0; p < 16; ++p) wb[p] = q_slice_bytes<NSL>(qv[st][p], ex);
        u32x4_t wq[NSL];
#pragma unroll
        for (int k = 0; k < NSL; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            wq[k][i] = slice_dword(wb[4 * i], wb[4 * i + 1], wb[4 * i + 2], wb[4 * i + 3], k);
#pragma unroll
        for (int k = 0; k < NSL; ++k) qb[rb][NSL * st + k] = __builtin_bit_cast(half8_t, wq[k]);
      }
      float mul = a.sm_scale * 1.4426950408889634f;  // natural -> log2 units
      if constexpr (MODE == kPerTensor) mul *= a.c.k_scales[0];
      if constexpr (DT == kInt4) mul *= 0.0625f;  // K tile holds 16 * code
      rowmul[rb] = ldexpf(mul, ex - (8 * NSL - 2));
      continue;
    }
    u32x4_t raw[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      raw[ks] = *reinterpret_cast<const u32x4_t*>(src + 32 * ks + 8 * g);
      if (r >= a.R) raw[ks] = u32x4_t{0u, 0u, 0u, 0u};
    }
    float mul = a.sm_scale * 1.4426950408889634f;  // natural -> log2 units
    if constexpr (DT == kBf16) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) qb[rb][ks] = __builtin_bit_cast(half8_t, raw[ks]);
    } else {
      // fp16 after a power-of-two row normalization (every element in (-1, 1))
      float qv[KSTEPS][8];
      float amax = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x0 = __uint_as_float(raw[ks][i] << 16), x1 = __uint_as_float(raw[ks][i] & 0xFFFF0000u);
          if constexpr (MODE == kPerChannel) {
            const float* kst = a.c.k_scales + (size_t)hkv * D + 32 * ks + 8 * g + 2 * i;
            x0 *= kst[0];
            x1 *= kst[1];
          }
          qv[ks][2 * i] = x0;
          qv[ks][2 * i + 1] = x1;
          amax = fmaxf(amax, fmaxf(fabsf(x0), fabsf(x1)));
        }
      amax = group_max4(amax);
      int ex = 0;
      if (amax > 0.0f) (void)frexpf(amax, &ex);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        half8_t h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (_Float16)ldexpf(qv[ks][e], -ex);
        qb[rb][ks] = h;
      }
      if constexpr (MODE == kPerTensor) mul *= a.c.k_scales[0];
      if constexpr (DT == kInt4) mul *= 0.0625f;  // K tile holds 16 * code
      mul = ldexpf(mul, ex);
    }
    rowmul[rb] = mul;
  }

  // tiles any row of the workgroup can see
  const int rlast = min(rbase + kRows, a.R) - 1;
  const int pos_hi = min(pos0 + rlast / a.G, L - 1);
  int kt_end = pos_hi >= 0 ? pos_hi / kPT + 1 : 0;
  int kt_begin = 0;
  if (a.window > 0) {
    const int first = pos0 + rbase / a.G - a.window + 1;
    kt_begin = first > 0 ? first / kPT : 0;
  }
  if (kt_begin > kt_end) kt_begin = kt_end;
  if (a.KS > 1) {
    // this workgroup's part: consecutive tiles, as even as whole tiles allow
    const int nt = kt_end - kt_begin;
    const int C = (nt + a.KS - 1) / a.KS;
    kt_begin = min(kt_begin + part * C, kt_end);
    kt_end = min(kt_begin + C, kt_end);
  }
  // uniform, in scalar registers (the divisions above run on the vector
  // unit), so the tile index and each tile's row arithmetic stay scalar
  kt_begin = __builtin_amdgcn_readfirstlane(kt_begin);
  kt_end = __builtin_amdgcn_readfirstlane(kt_end);

  const float cap2 = CAP ? a.softcap * 1.4426950408889634f : 0.0f;
  const float icap2 = CAP ? 2.0f / a.softcap : 0.0f;
  float m[RBW], l[RBW];
  float vref = 0x1p-126f;
  float ivref = 0x1p126f;  // 1 / vref, exact (vref is a power of two)
  float4_t acc[RBW][NCOL];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.0f;
#pragma unroll
    for (int c = 0; c < NCOL; ++c) acc[rb][c] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  PTile<DT, D, W> T;
  if (kt_begin < kt_end) {
    load_ptile<DT, MODE, D, W>(a, b, hkv, kt_begin, L, tid, T);
    stage_ptile<DT, MODE, D, W>(T, tid, lds, lds + KTILE_ELEMS, ksc[0], vsc[0]);
  }
  __syncthreads();
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = (kt - kt_begin) & 1;
    // the next tile's loads (past the last tile they read rows that exist and
    // are never used)
    load_ptile<DT, MODE, D, W>(a, b, hkv, kt + 1, L, tid, T);
    const uint16_t* ks_lds = lds + cur * BUF_ELEMS;
    const uint16_t* vt_lds = ks_lds + KTILE_ELEMS;

    // ---- S^T for the 4 sub-tiles of 16 tokens: lane (n, g) gets tokens 4g + e
    // of its rows.  The K operands of sub-tile s + 1 are read from LDS before
    // sub-tile s's MFMAs in source order (the compiler schedules them).
    // z: logits in log2 units relative to the row's reference, z - msafe
    // (msafe = m, or 0 before the first visible token), folded into one fma
    // (with a soft cap the capped logit comes first, then the subtraction)
    float msafe[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) msafe[rb] = m[rb] == -INFINITY ? 0.0f : m[rb];
    float z[RBW][4][4];
    bool up = false;
    // (one sub-tile's K operands at a time at D = 256: two in flight cost 32
    // more registers than two wavefronts per SIMD leave)
    constexpr int KB = W > 4 ? 1 : 2;
    half8_t kop[KB][KSTEPS];
    auto kread = [&](int s, half8_t (&dst)[KSTEPS]) {
      if constexpr (P::IQK) {
        // 16 code bytes of channels 64 st + 16 g .. + 15 per integer step
        const uint8_t* krow = reinterpret_cast<const uint8_t*>(ks_lds + (16 * s + n) * P::KST) + 16 * g;
#pragma unroll
        for (int st = 0; st < P::ISTEPS; ++st)
          dst[st] = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4_t*>(krow + 64 * st));
      } else {
        const uint16_t* krow = ks_lds + (16 * s + n) * P::KST + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          dst[ks] = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4_t*>(krow + 32 * ks));
      }
    };
    if constexpr (KB == 2) kread(0, kop[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (KB == 2) {
        if (s + 1 < 4) kread(s + 1, kop[(s + 1) & 1]);
      } else {
        kread(s, kop[0]);
      }
      float4_t s0[RBW], s1[RBW];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        s0[rb] = float4_t{0.f, 0.f, 0.f, 0.f};
        s1[rb] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
      if constexpr (P::IQK) {
        // exact integer dot products with each q slice, combined into one
        // float per logit in s0
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          i32x4_t acc[NSL];
#pragma unroll
          for (int k = 0; k < NSL; ++k) acc[k] = i32x4_t{0, 0, 0, 0};
#pragma unroll
          for (int st = 0; st < P::ISTEPS; ++st) {
            const i32x4_t ka = __builtin_bit_cast(i32x4_t, kop[s % KB][st]);
#pragma unroll
            for (int k = NSL - 1; k >= 0; --k)
              acc[k] = mfma64_i8(ka, __builtin_bit_cast(i32x4_t, qb[rb][NSL * st + k]), acc[k]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            int dd[NSL];
#pragma unroll
            for (int k = 0; k < NSL; ++k) dd[k] = acc[k][e];
            s0[rb][e] = q_dot<NSL>(dd);
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < (P::IQK ? 0 : KSTEPS); ks += 2) {
        const half8_t k0 = kop[s % KB][ks];
        const half8_t k1 = kop[s % KB][ks + 1 < KSTEPS ? ks + 1 : ks];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          if constexpr (DT == kBf16) {
            s0[rb] = mfma32_bf16(k0, qb[rb][ks], s0[rb]);
            if (ks + 1 < KSTEPS) s1[rb] = mfma32_bf16(k1, qb[rb][ks + 1], s1[rb]);
          } else {
            s0[rb] = mfma32(k0, qb[rb][ks], s0[rb]);
            if (ks + 1 < KSTEPS) s1[rb] = mfma32(k1, qb[rb][ks + 1], s1[rb]);
          }
        }
      }
      const float4_t ks4 = MODE == kPerRow ? *reinterpret_cast<const float4_t*>(&ksc[cur][16 * s + 4 * g])
                                           : float4_t{1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float d = s0[rb][e] + s1[rb][e];
          if constexpr (MODE == kPerRow) d *= ks4[e];
          if constexpr (CAP) {
            float zz = d * rowmul[rb];
            const float ex = __builtin_amdgcn_exp2f(zz * icap2);
            zz = cap2 - 2.0f * cap2 * __builtin_amdgcn_rcpf(ex + 1.0f);
            z[rb][s][e] = zz - msafe[rb];
          } else {
            z[rb][s][e] = __builtin_fmaf(d, rowmul[rb], -msafe[rb]);
          }
        }
    }
    // causal / window / length mask, skipped on tiles every row of the
    // wavefront sees whole
    if (!(kt * kPT + kPT <= wlim_min && kt * kPT >= wlo_max)) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = kt * kPT + 16 * s + 4 * g + e;
            if (!(t < lim[rb] && t >= lo[rb])) z[rb][s][e] = -INFINITY;
          }
    }
    // one comparison of the largest relative logit instead of one per logit
    {
      float zmax = -INFINITY;
      bool noref = false;
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          zmax = fmaxf(zmax, fmaxf(fmaxf(z[rb][s][0], z[rb][s][1]), fmaxf(z[rb][s][2], z[rb][s][3])));
        noref |= m[rb] == -INFINITY;
      }
      up = zmax > kLazyHeadroom || noref;
    }

    // ---- online softmax over the tile's 64 tokens (row n: lanes n, n+16, n+32,
    // n+48), with the lazily moved reference of the decode kernel: m moves only
    // when a logit exceeds it by more than kLazyHeadroom
    float alpha[RBW];
    float vfac = 1.0f;
    bool rescale = false;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) alpha[rb] = 1.0f;
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          tmax = fmaxf(tmax, fmaxf(fmaxf(z[rb][s][0], z[rb][s][1]), fmaxf(z[rb][s][2], z[rb][s][3])));
        tmax = group_max4(tmax);  // relative to msafe
        if (tmax > kLazyHeadroom || (m[rb] == -INFINITY && tmax > -INFINITY)) {
          // hardware exp2; 0 when there was no reference yet
          alpha[rb] = m[rb] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(-tmax);
          l[rb] *= alpha[rb];
          m[rb] = msafe[rb] + tmax;
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) z[rb][s][e] -= tmax;
          rescale = true;
        }
      }
    }
    float vsn[4][4] = {};
    if constexpr (kVRow) {
      // weights carry v_scale / vref with vref a power of two >= every scale seen
      bool vup = false;
      float4_t vs4[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        vs4[s] = *reinterpret_cast<const float4_t*>(&vsc[cur][16 * s + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) vup |= vs4[s][e] > vref;
      }
      if (__builtin_amdgcn_ballot_w64(vup) != 0) {
        float vmax = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) vmax = fmaxf(vmax, vs4[s][e]);
        vmax = wave_max(vmax);
        int en;
        (void)frexpf(vmax, &en);
        const float nref = ldexpf(1.0f, en);
        if (nref > vref) {
          // powers of two: both products are exact, no division per tile
          ivref = ldexpf(1.0f, -en);
          vfac = vref * ivref;
          vref = nref;
          rescale = true;
        }
      }
      const float inv = ivref;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) vsn[s][e] = vs4[s][e] * inv;
    }
    if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = __shfl(alpha[rb], 4 * g + e) * vfac;
#pragma unroll
        for (int c = 0; c < NCOL; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rb][c][e] *= f[e];
      }
    }

    // ---- unpack the next tile into the other buffer (nobody reads it during
    // this tile; past the last tile it writes what nobody reads), ahead of the
    // P . V MFMAs so that its VALU work and LDS writes interleave with them
    stage_ptile<DT, MODE, D, W>(T, tid, lds + (cur ^ 1) * BUF_ELEMS, lds + (cur ^ 1) * BUF_ELEMS + KTILE_ELEMS,
                                ksc[cur ^ 1], vsc[cur ^ 1]);

    // ---- O += P . V, two sub-tiles (32 tokens) per 16x16x32 MFMA: lane group
    // g's A operand holds tokens 16s + 4g + 0..3 then 16s + 16 + 4g + 0..3 of its
    // row, and the B operand the same tokens of its channel (two 8-byte reads
    // of the transposed V)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      half8_t ph[RBW];
      half8_t phi[RBW], plo[RBW];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        float pf[8];
        float psum = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = 2 * sp + h;
            const float p = __builtin_amdgcn_exp2f(z[rb][s][e]);
            psum += p;
            if constexpr (kVRow)
              pf[4 * h + e] = p * vsn[s][e];
            else
              pf[4 * h + e] = p;
          }
        l[rb] += psum;
        if constexpr (DT == kBf16) {
          uint16_t hh[8], ll[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            hh[e] = f32_to_bf16(pf[e]);
            ll[e] = f32_to_bf16(pf[e] - bf16_to_f32(hh[e]));
          }
          u32x4_t wh, wl;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            wh[i] = hh[2 * i] | ((uint32_t)hh[2 * i + 1] << 16);
            wl[i] = ll[2 * i] | ((uint32_t)ll[2 * i + 1] << 16);
          }
          phi[rb] = __builtin_bit_cast(half8_t, wh);
          plo[rb] = __builtin_bit_cast(half8_t, wl);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) ph[rb][e] = (_Float16)pf[e];
        }
      }
      // the pair's V operands in groups read ahead of their MFMAs, so their
      // LDS latencies overlap (all at once with 4 wavefronts; two halves with
      // 8, whose registers are shared by two wavefronts per SIMD)
      const uint16_t* vcol = vt_lds + 32 * sp + 4 * g;
      constexpr int VG = W > 4 ? NCOL / 2 : NCOL;
#pragma unroll
      for (int c0 = 0; c0 < NCOL; c0 += VG) {
        u32x4_t vop[VG];
#pragma unroll
        for (int c = 0; c < VG; ++c) {
          const uint16_t* src = vcol + (16 * (c0 + c) + n) * P::VST;
          const u32x2_t a0 = *reinterpret_cast<const u32x2_t*>(src);
          const u32x2_t a1 = *reinterpret_cast<const u32x2_t*>(src + 16);
          vop[c] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
        }
#pragma unroll
        for (int c = 0; c < VG; ++c) {
          const half8_t vb = __builtin_bit_cast(half8_t, vop[c]);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) {
            if constexpr (DT == kBf16) {
              acc[rb][c0 + c] = mfma32_bf16(phi[rb], vb, acc[rb][c0 + c]);
              acc[rb][c0 + c] = mfma32_bf16(plo[rb], vb, acc[rb][c0 + c]);
            } else {
              acc[rb][c0 + c] = mfma32(ph[rb], vb, acc[rb][c0 + c]);
            }
          }
        }
      }
    }

    // one barrier: the next tile is unpacked, and this tile's buffer is free
    __syncthreads();
  }

  // ---- epilogue: per row 1 / l (with the V reference and the int4 factor),
  // the head sink, then the static V scale per channel, bf16 out; a split
  // launch's part writes its normalized rows and (m, l) for the combine
  // instead, which applies the sink and the static V scale
  const bool split = a.KS > 1;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const float lt = group_sum4(l[rb]);
    if (g == 0) {
      const int r = rwave + 16 * rb + n;
      float f = 0.0f, sk = 1.0f;
      if (split && r < a.R) {
        float* ml = a.ws_ml + (((size_t)b * a.c.Hkv + hkv) * a.R + r) * a.KS * 2 + 2 * part;
        ml[0] = lt > 0.0f ? m[rb] : -INFINITY;
        ml[1] = lt;
      }
      if (lt > 0.0f) {
        f = 1.0f / lt;
        if constexpr (kVRow) f *= vref;           // weights carried v_scale / vref
        if constexpr (DT == kInt4) f *= 0.0625f;  // V tile holds 16 * code
        if (!split && a.sink != nullptr && r < a.R) {
          const int h = hkv * a.G + r % a.G;
          const float lse = 0.6931471805599453f * (m[rb] + log2f(lt));
          sk = 1.0f / (1.0f + expf(a.sink[h] - lse));
        }
      }
      rowf[wave][16 * rb + n] = f;
      rowsink[wave][16 * rb + n] = sk;
    }
  }
  // stage this wavefront's rows as fp32 (row stride D + 4); the loop ended
  // with a barrier, so the tile buffers are free
  float* ob = reinterpret_cast<float*>(lds) + wave * 16 * RBW * (D + 4);
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int c = 0; c < NCOL; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) ob[(16 * rb + 4 * g + e) * (D + 4) + 16 * c + n] = acc[rb][c][e];
  __syncthreads();
  constexpr int QPR = D / 4;  // float4 per row
  for (int i = lane; i < 16 * RBW * QPR; i += 64) {
    const int rr = i / QPR, d = 4 * (i % QPR);
    const int row = rwave + rr;
    if (row >= a.R) continue;
    const float f = rowf[wave][rr] * rowsink[wave][rr];
    const float4_t v = *reinterpret_cast<const float4_t*>(ob + rr * (D + 4) + d);
    if (split) {
      *reinterpret_cast<float4_t*>(a.ws_o + ((((size_t)b * a.c.Hkv + hkv) * a.R + row) * a.KS + part) * D +
                                   d) = v * f;
      continue;
    }
    uint16_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = v[e] * f;
      if (!kVRow && a.v_static != nullptr)
        x *= a.vmode == kPerTensor ? a.v_static[0] : a.v_static[(size_t)hkv * D + d + e];
      o[e] = f32_to_bf16(x);
    }
    const int jq = row / a.G, h = hkv * a.G + row % a.G;
    *reinterpret_cast<u32x2_t*>(a.out + (((size_t)b * a.Tq + jq) * a.Hq + h) * D + d) =
        u32x2_t{(uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
  }
}

template <int DT, int MODE, int D, int W>
hipError_t launch_w(const PrefillArgs& a, int B, hipStream_t st) {
  const long nx = ((long)a.R + kPRows<D, W> - 1) / kPRows<D, W> * a.KS;
  if (nx > 0x7FFFFFFFL || a.KS < 1) return hipErrorInvalidValue;
  dim3 grid((unsigned)nx, a.c.Hkv, B);
  if (a.softcap > 0.0f)
    hipLaunchKernelGGL((prefill_kernel<DT, MODE, D, W, true>), grid, dim3(64 * W), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<DT, MODE, D, W, false>), grid, dim3(64 * W), 0, st, a);
  return hipGetLastError();
}

// The host picks the workgroup size (prefill_plan in kvq_host.cpp): 8
// wavefronts only at D = 256.
template <int DT, int MODE, int D>
hipError_t launch_d(const PrefillArgs& a, int B, hipStream_t st) {
  if constexpr (D == 256) {
    if (a.W == 8) return launch_w<DT, MODE, D, 8>(a, B, st);
  }
  if (a.W != 4) return hipErrorInvalidValue;
  return launch_w<DT, MODE, D, 4>(a, B, st);
}

}  // namespace

#define KVQ_PCAT2(a, b, c, d) a##b##_##c##_##d
#define KVQ_PCAT(a, b, c, d) KVQ_PCAT2(a, b, c, d)

hipError_t KVQ_PCAT(launch_prefill_, KVQ_DTYPE, KVQ_MODE, KVQ_VROW)(int D, const PrefillArgs& a, int B,
                                                                    hipStream_t st) {
  switch (D) {
    case 64: return launch_d<KVQ_DTYPE, KVQ_MODE, 64>(a, B, st);
    case 128: return launch_d<KVQ_DTYPE, KVQ_MODE, 128>(a, B, st);
    case 256: return launch_d<KVQ_DTYPE, KVQ_MODE, 256>(a, B, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
