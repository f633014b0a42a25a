// kvq_append.hip -- quantize-on-write of newly appended K/V rows: one
// wavefront per (sequence, token, KV head, K|V) row; the arithmetic of a row
// is in kvq_quant.h.  A bf16 cache stores the rows unchanged.

#include "kvq_quant.h"

namespace kvq {
namespace {

template <int DT, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  using R = RowGeo<DT, D>;
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
  // memory round trips overlap
  uint16_t raw[R::EPL];
  load_row<DT, D>((side ? a.v : a.k) + (((size_t)b * a.Tn + j) * Hkv + h) * D, lane, raw);

  // with seq_lens, the length is clamped to the host bound exactly as the
  // attention that follows clamps it, so the rows land where it reads them
  int base;
  if (a.positions != nullptr) {
    base = a.positions[b];
  } else {
    const int L = a.seq_lens[b];
    base = (L < 0 ? 0 : L > a.max_len ? a.max_len : L) - a.Tn;
  }
  const int pos = base + j;
  if (pos < 0 || pos >= a.capacity) return;
  const int bs = a.c.block_size;
  int blk = b;
  if (a.c.block_table != nullptr) {
    blk = a.c.block_table[(size_t)b * a.c.max_blocks + pos / bs];
    if (blk < 0 || blk >= a.c.num_blocks) return;
  }
  const size_t ri = ((size_t)blk * Hkv + h) * bs + (size_t)(pos % bs);
  float* scales = side ? a.c.v_scales : a.c.k_scales;
  const int mode = side ? a.vmode : a.kmode;
  quantize_store_row_mode<DT, D>(mode, raw, lane, (side ? a.c.v_codes : a.c.k_codes) + ri * R::ROWB,
                                 scales + ri, mode == kPerChannel ? scales + (size_t)h * D : scales);
}

template <int DT>
hipError_t launch_dt(int D, const AppendArgs& a, hipStream_t st) {
  const long nrows = (long)a.B * a.Tn * a.c.Hkv * 2;
  const long nblk = (nrows + 3) / 4;
  if (nblk > 0x7FFFFFFFL) return hipErrorInvalidValue;
  dim3 grid((unsigned)nblk);
  switch (D) {
    case 64: hipLaunchKernelGGL((append_kernel<DT, 64>), grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL((append_kernel<DT, 128>), grid, dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL((append_kernel<DT, 256>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int dtype, int kmode, int vmode, int D, const AppendArgs& a,
                         hipStream_t st) {
  auto ok = [](int m) { return m == kPerRow || m == kPerTensor || m == kPerChannel; };
  if (a.kmode != kmode || a.vmode != vmode) return hipErrorInvalidValue;
  if (dtype == kBf16)  // unquantized rows, no scales
    return (kmode == kNoScale && vmode == kNoScale) ? launch_dt<kBf16>(D, a, st) : hipErrorInvalidValue;
  if (!ok(kmode) || !ok(vmode)) return hipErrorInvalidValue;
  switch (dtype) {
    case kInt8: return launch_dt<kInt8>(D, a, st);
    case kInt4: return launch_dt<kInt4>(D, a, st);
    case kFp8: return launch_dt<kFp8>(D, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
