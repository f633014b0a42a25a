// kvq_append.hip -- quantize-on-write of newly appended K/V rows.
//
// Kernel page "kv-quant-attn", "Method": every key and value row carries its
// own absmax scale, computed when the row is written, so appending never
// rewrites earlier rows.  ORT PR "[CUDA] PagedAttention: quantized KV cache
// ...", "CUDA kernels": ReshapeAndCache quantizes on write under static
// PER_TENSOR / PER_CHANNEL scales.  Packed int4: "[CUDA] Add INT4 paged KV
// cache with per-channel scales", two signed values per byte.
//
// One wavefront per (sequence, token, KV head, K|V) row.  Per element:
//   y = x / s                        IEEE fp32 division (never x * (1/s))
//   int:  c = clamp(rint(y), -Qmax, Qmax)   rint rounds half to even
//   fp8:  c = E4M3FN(clamp(y, -448, 448))   hardware RNE convert; the clamp
//                                           gives saturation, signed zero kept
//   s == 0 -> c = 0.
// Per-row mode: s = max|x| / Qmax (fp32 division), written next to the row.

#include "kvq_device.h"

namespace kvq {
namespace {

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

template <int DT, int MODE, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  // elements per lane; int4 lanes always own whole bytes
  constexpr int EPL = (DT == kInt4 && D / 64 < 2) ? 2 : D / 64;
  constexpr int ACTIVE = D / EPL;
  constexpr int ROWB = (DT == kInt4) ? D / 2 : D;
  const int lane = threadIdx.x & 63;
  const long row_id = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int Hkv = a.c.Hkv;
  const long nrows = (long)a.B * a.Tn * Hkv * 2;
  if (row_id >= nrows) return;  // whole wavefront leaves together
  const int side = (int)(row_id & 1);
  long rest = row_id >> 1;
  const int h = (int)(rest % Hkv);
  rest /= Hkv;
  const int j = (int)(rest % a.Tn);
  const int b = (int)(rest / a.Tn);

  // the row load does not depend on the position: issue it first so the two
  // memory round trips overlap (unconditional, clamped for idle lanes)
  const uint16_t* x = (side ? a.v : a.k) + (((size_t)b * a.Tn + j) * Hkv + h) * D;
  const bool active = lane < ACTIVE;
  uint16_t raw[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) raw[e] = x[active ? lane * EPL + e : 0];

  const int pos = a.positions[b] + j;
  if (pos < 0 || pos >= a.capacity) return;
  const int bs = a.c.block_size;
  int blk = b;
  if (a.c.block_table != nullptr) {
    blk = a.c.block_table[(size_t)b * a.c.max_blocks + pos / bs];
    if (blk < 0 || blk >= a.c.num_blocks) return;
  }
  const size_t ri = ((size_t)blk * Hkv + h) * bs + (size_t)(pos % bs);
  uint8_t* codes = (side ? a.c.v_codes : a.c.k_codes) + ri * ROWB;
  float* scales = side ? a.c.v_scales : a.c.k_scales;

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
    if (lane == 0) scales[ri] = s_row;
  }
  if (!active) return;

  uint32_t c[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float s;
    if constexpr (MODE == kPerRow)
      s = s_row;
    else if constexpr (MODE == kPerTensor)
      s = scales[0];
    else
      s = scales[(size_t)h * D + lane * EPL + e];
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

template <int DT, int MODE>
hipError_t launch_dm(int D, const AppendArgs& a, hipStream_t st) {
  const long nrows = (long)a.B * a.Tn * a.c.Hkv * 2;
  const long nblk = (nrows + 3) / 4;
  if (nblk > 0x7FFFFFFFL) return hipErrorInvalidValue;
  dim3 grid((unsigned)nblk);
  switch (D) {
    case 64: hipLaunchKernelGGL((append_kernel<DT, MODE, 64>), grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL((append_kernel<DT, MODE, 128>), grid, dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL((append_kernel<DT, MODE, 256>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(int mode, int D, const AppendArgs& a, hipStream_t st) {
  switch (mode) {
    case kPerRow: return launch_dm<DT, kPerRow>(D, a, st);
    case kPerTensor: return launch_dm<DT, kPerTensor>(D, a, st);
    case kPerChannel: return launch_dm<DT, kPerChannel>(D, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_append(int dtype, int mode, int D, const AppendArgs& a, hipStream_t st) {
  switch (dtype) {
    case kInt8: return launch_dt<kInt8>(mode, D, a, st);
    case kInt4: return launch_dt<kInt4>(mode, D, a, st);
    case kFp8: return launch_dt<kFp8>(mode, D, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
