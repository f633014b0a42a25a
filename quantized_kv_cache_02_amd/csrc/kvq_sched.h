// kvq_sched.h -- the balanced split schedule shared by the decode and combine
// kernels.  GPU code only.
//
// Kernel page "kv-quant-attn", "Method": the cached sequence is cut into
// splits that separate workgroups reduce, and the partials are merged in a
// fixed order.  With a batch of ragged lengths, a fixed number of splits per
// sequence leaves the workgroups of the longest sequence on the critical path
// while the others idle, so the cut is made over the whole batch instead:
//
//   n_b = ceil(L_b / 16) - f_b          16-token tiles sequence b's queries see
//                                        (f_b: the first tile inside a sliding
//                                        window, 0 without one)
//   T   = sum_b n_b                      tiles of one KV head
//   C   = max(ceil(T / NW), kMinTilesPerSplit)   tiles per chunk
//   S_b = ceil(n_b / C)                  chunks of sequence b (never straddling two)
//   P_b = sum_{b' < b} S_b'              first chunk slot of sequence b
//
// NW is the host's nominal workgroup count per KV head.  Since
// sum_b S_b < T / C + B <= NW + B, the NW + B - 1 slots per KV head cover every
// chunk; slots past the last chunk are idle.  Every workgroup derives the same
// integers from the same seq_lens with wave-level sums, so the decode kernel
// and the combine agree on where each partial lives.  The schedule depends on
// the lengths only, so repeated calls cut identically and stay bitwise equal.
#pragma once

#include "kvq_device.h"

namespace kvq {

__device__ __forceinline__ int clamp_len(int L, int max_seq_len) {
  return L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_scan_i(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Tiles [first, end) of a sequence of length L that its Tq queries can see: a
// sliding window hides every token before L - Tq - window + 1 (the first
// query's window) ([P] "CUDA kernels": sliding-window decode).
struct Span {
  int first, end;
};
__device__ __forceinline__ Span visible_tiles(int L, int Tq, int window) {
  const int end = (L + kTile - 1) / kTile;
  int lo = window > 0 ? L - Tq - window + 1 : 0;
  lo = lo < 0 ? 0 : lo;
  const int first = lo / kTile;
  return Span{first < end ? first : end, end};
}

struct Chunk {
  int b;       // sequence (-1: idle slot)
  int first;   // first tile of the chunk
  int end;     // one past its last tile
  int L;       // the sequence's length (clamped)
  int P;       // first slot of the sequence
  int S;       // chunks of the sequence
};

// Tiles per chunk over the whole batch (every lane gets the same value).
__device__ __forceinline__ int chunk_tiles(const int32_t* seq_lens, int B, int max_seq_len, int NW,
                                           int Tq, int window, int lane) {
  int T = 0;
  for (int base = 0; base < B; base += 64) {
    const int i = base + lane;
    const int L = i < B ? clamp_len(seq_lens[i], max_seq_len) : 0;
    const Span sp = visible_tiles(L, Tq, window);
    T += wave_sum_i(sp.end - sp.first);
  }
  const int C = (T + NW - 1) / NW;
  return C > kMinTilesPerSplit ? C : kMinTilesPerSplit;
}

// The chunk of workgroup `slot`, or, with slot < 0, just P_b and S_b of
// sequence `want_b`.  Wave-uniform results.
// With `table` non-null, also writes every sequence's (P_b, S_b) there.
__device__ __forceinline__ Chunk find_chunk(const int32_t* seq_lens, int B, int max_seq_len, int NW,
                                            int Tq, int window, int slot, int want_b, int lane,
                                            int32_t* table = nullptr) {
  Chunk ch{-1, 0, 0, 0, 0, 0};
  int P = 0;  // chunks of the sequences before this pass
  // one pass: lane l holds sequence base + l (length L); true once done
  auto pass = [&](int base, int L, int C) {
    const int i = base + lane;
    const Span sp = visible_tiles(L, Tq, window);
    const int n = sp.end - sp.first;
    const int Sb = (n + C - 1) / C;
    const int incl = wave_scan_i(Sb, lane);
    const int Pb = P + incl - Sb;
    if (table != nullptr && i < B) {
      table[2 * i] = Pb;
      table[2 * i + 1] = Sb;
    }
    const bool hit = (i < B) && (slot >= 0 ? (Sb > 0 && Pb <= slot && slot < Pb + Sb) : i == want_b);
    const uint64_t m = __ballot(hit);
    bool done = false;
    if (m != 0 && ch.b < 0) {
      const int l = __builtin_ctzll(m);
      ch.b = base + l;
      ch.L = __shfl(L, l);
      ch.P = __shfl(Pb, l);
      ch.S = __shfl(Sb, l);
      const int c = slot >= 0 ? slot - ch.P : 0;
      const int f0 = __shfl(sp.first, l);
      const int nb = __shfl(sp.end, l);
      ch.first = f0 + c * C;
      ch.end = min(ch.first + C, nb);
      done = table == nullptr;  // the table needs every pass
    }
    P += __shfl(incl, 63);
    return done;
  };
  if (B <= 64) {
    // one read of the lengths serves both the tile count and the search
    const int L = lane < B ? clamp_len(seq_lens[lane], max_seq_len) : 0;
    const Span sp = visible_tiles(L, Tq, window);
    const int T = wave_sum_i(sp.end - sp.first);
    const int C = (T + NW - 1) / NW;
    pass(0, L, C > kMinTilesPerSplit ? C : kMinTilesPerSplit);
  } else {
    const int C = chunk_tiles(seq_lens, B, max_seq_len, NW, Tq, window, lane);
    for (int base = 0; base < B; base += 64) {
      const int i = base + lane;
      if (pass(base, i < B ? clamp_len(seq_lens[i], max_seq_len) : 0, C)) break;
    }
  }
  ch.b = __builtin_amdgcn_readfirstlane(ch.b);
  ch.first = __builtin_amdgcn_readfirstlane(ch.first);
  ch.end = __builtin_amdgcn_readfirstlane(ch.end);
  ch.L = __builtin_amdgcn_readfirstlane(ch.L);
  ch.P = __builtin_amdgcn_readfirstlane(ch.P);
  ch.S = __builtin_amdgcn_readfirstlane(ch.S);
  return ch;
}

}  // namespace kvq
