// kvq_quant.h -- quantize-on-write of one K or V row by one wavefront, shared
// by the append kernel and the decode kernel's fused append.  GPU code only.
//
// Kernel page "kv-quant-attn", "Method": every key and value row carries its
// own absmax scale, computed when the row is written, so appending never
// rewrites earlier rows.  ORT PR "[CUDA] PagedAttention: quantized KV cache
// ...", "CUDA kernels": ReshapeAndCache quantizes on write under static
// PER_TENSOR / PER_CHANNEL scales.  Packed int4: "[CUDA] Add INT4 paged KV
// cache with per-channel scales", two signed values per byte.
//
// Per element:
//   y = x / s                        IEEE fp32 division (never x * (1/s))
//   int:  c = clamp(rint(y), -Qmax, Qmax)   rint rounds half to even
//   fp8:  c = E4M3FN(clamp(y, -448, 448))   hardware RNE convert; the clamp
//                                           gives saturation, signed zero kept
//   s == 0 -> c = 0.
// Per-row mode: s = max|x| / Qmax (fp32 division), written next to the row.
// An unquantized bf16 cache stores the row's bf16 values as they are.
#pragma once

#include "kvq_device.h"

namespace kvq {

template <int DT>
struct QMax;
template <>
struct QMax<kInt8> {
  static constexpr float v = 127.0f;
};
template <>
struct QMax<kInt4> {
  static constexpr float v = 7.0f;
};
template <>
struct QMax<kFp8> {
  static constexpr float v = 448.0f;
};

template <int DT>
__device__ __forceinline__ int int_code(float y) {
  constexpr float qm = QMax<DT>::v;
  float r = __builtin_rintf(y);
  r = fminf(fmaxf(r, -qm), qm);
  return (int)r;
}

__device__ __forceinline__ uint32_t fp8_code(float y) {
  y = fminf(fmaxf(y, -448.0f), 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFFu;
}

// Lane layout of a row: lane l owns elements [l*EPL, (l+1)*EPL); int4 lanes
// always own whole bytes, so for D = 64 only 32 lanes are active.
template <int DT, int D>
struct RowGeo {
  static constexpr int EPL = (DT == kInt4 && D / 64 < 2) ? 2 : D / 64;
  static constexpr int ACTIVE = D / EPL;
  static constexpr int ROWB = (DT == kInt4) ? D / 2 : (DT == kBf16) ? 2 * D : D;
};

// Load the lane's bf16 elements of a row (unconditional; idle lanes read
// element 0) as one 4- or 8-byte load.
template <int DT, int D>
__device__ __forceinline__ void load_row(const uint16_t* x, int lane,
                                         uint16_t (&raw)[RowGeo<DT, D>::EPL]) {
  using R = RowGeo<DT, D>;
  static_assert(R::EPL == 1 || R::EPL == 2 || R::EPL == 4, "row elements per lane");
  const int i = lane < R::ACTIVE ? lane * R::EPL : 0;
  if constexpr (R::EPL == 4) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(x + i);
    raw[0] = (uint16_t)v[0]; raw[1] = (uint16_t)(v[0] >> 16);
    raw[2] = (uint16_t)v[1]; raw[3] = (uint16_t)(v[1] >> 16);
  } else if constexpr (R::EPL == 2) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(x + i);
    raw[0] = (uint16_t)v; raw[1] = (uint16_t)(v >> 16);
  } else {
    raw[0] = x[i];
  }
}

// Quantize the row held in `raw` and store its codes (and, per-row, its scale).
//   codes        row_bytes of this row in the cache
//   scale_out    per-row: where the row's scale goes (written by lane 0)
//   static_s     per-tensor: [1]; per-channel: this KV head's [D] table
// Every lane of the wavefront must call this (the per-row max is a wave reduction).
template <int DT, int MODE, int D>
__device__ __forceinline__ void quantize_store_row_q(const uint16_t (&raw)[RowGeo<DT, D>::EPL], int lane,
                                                     uint8_t* codes, float* scale_out,
                                                     const float* static_s) {
  using R = RowGeo<DT, D>;
  constexpr int EPL = R::EPL;
  const bool active = lane < R::ACTIVE;
  float xv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) xv[e] = active ? bf16_to_f32(raw[e]) : 0.0f;

  float s_row = 0.0f;
  if constexpr (MODE == kPerRow) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(xv[e]));
    amax = wave_max(amax);
    s_row = amax / QMax<DT>::v;
    if (lane == 0) *scale_out = s_row;
  }
  if (!active) return;

  uint32_t c[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float s;
    if constexpr (MODE == kPerRow)
      s = s_row;
    else if constexpr (MODE == kPerTensor)
      s = static_s[0];
    else
      s = static_s[lane * EPL + e];
    if (s == 0.0f) {
      c[e] = 0u;
    } else {
      const float y = xv[e] / s;
      if constexpr (DT == kFp8)
        c[e] = fp8_code(y);
      else
        c[e] = (uint32_t)int_code<DT>(y);
    }
  }
  if constexpr (DT == kInt4) {
#pragma unroll
    for (int e = 0; e < EPL; e += 2)
      codes[(lane * EPL + e) / 2] = (uint8_t)((c[e] & 0xFu) | ((c[e + 1] & 0xFu) << 4));
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) codes[lane * EPL + e] = (uint8_t)c[e];
  }
}

template <int DT, int MODE, int D>
__device__ __forceinline__ void quantize_store_row(const uint16_t (&raw)[RowGeo<DT, D>::EPL], int lane,
                                                   uint8_t* codes, float* scale_out,
                                                   const float* static_s) {
  if constexpr (DT == kBf16) {  // unquantized: the row itself, no scale
    (void)scale_out;
    (void)static_s;
    uint16_t* dst = reinterpret_cast<uint16_t*>(codes);
#pragma unroll
    for (int e = 0; e < RowGeo<DT, D>::EPL; ++e) dst[lane * RowGeo<DT, D>::EPL + e] = raw[e];
  } else {
    quantize_store_row_q<DT, MODE, D>(raw, lane, codes, scale_out, static_s);
  }
}

// The same with the scale mode chosen at run time (uniform over the wavefront).
template <int DT, int D>
__device__ __forceinline__ void quantize_store_row_mode(int mode,
                                                        const uint16_t (&raw)[RowGeo<DT, D>::EPL],
                                                        int lane, uint8_t* codes, float* scale_out,
                                                        const float* static_s) {
  if constexpr (DT == kBf16)
    quantize_store_row<DT, kNoScale, D>(raw, lane, codes, scale_out, static_s);
  else if (mode == kPerRow)
    quantize_store_row<DT, kPerRow, D>(raw, lane, codes, scale_out, static_s);
  else if (mode == kPerTensor)
    quantize_store_row<DT, kPerTensor, D>(raw, lane, codes, scale_out, static_s);
  else
    quantize_store_row<DT, kPerChannel, D>(raw, lane, codes, scale_out, static_s);
}

}  // namespace kvq
