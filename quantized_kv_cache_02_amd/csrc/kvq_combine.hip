// kvq_combine.hip -- fixed-order merge of the split partials, static V scale,
// head sink, bf16 output.
//
// Kernel page "kv-quant-attn", "Method": the sequence is split across
// workgroups and the partials are merged in a fixed order, so repeated decodes
// are bitwise identical.  ORT PR "[CUDA] PagedAttention: quantized KV cache
// ...", "CUDA kernels" (ApplyHeadSink): the output of head h is rescaled by
// 1 / (1 + exp(s_h - lse)) after the quantized branch.
//
// One wavefront per (sequence, KV head, query row, 64 channels).  With split s
// holding (m_s in log2 units, l_s, o_s normalized):
//   M = max_s m_s,  w_s = l_s 2^(m_s - M),  L = sum_s w_s,  o = sum_s w_s o_s / L,
//   lse = ln 2 (M + log2 L).
// Every sum runs in the same order on every call.

#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kMaxSplits = 4096;

template <int MODE>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a, int D) {
  __shared__ float w_s[kMaxSplits];
  const int lane = threadIdx.x;
  const int d = blockIdx.x * 64 + lane;
  const int r = blockIdx.y;
  const int head = blockIdx.z;  // b * Hkv + hkv
  const int b = head / a.Hkv, hkv = head % a.Hkv;
  const int S = a.S;
  const float* ms = a.ws_m + ((size_t)head * a.R + r) * S;
  const float* ls = a.ws_l + ((size_t)head * a.R + r) * S;

  // M: each lane scans splits lane, lane+64, ...; then a fixed butterfly
  float M = -INFINITY;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, ms[s]);
  M = wave_max(M);
  float part = 0.0f;
  for (int s = lane; s < S; s += 64) {
    const float w = (M == -INFINITY || ls[s] == 0.0f) ? 0.0f : ls[s] * exp2f(ms[s] - M);
    w_s[s] = w;
    part += w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
  const float Lsum = part;
  __syncthreads();

  float o = 0.0f;
  if (Lsum > 0.0f) {
    const float* os = a.ws_o + (((size_t)head * a.R + r) * S) * D + d;
    for (int s = 0; s < S; ++s) o += w_s[s] * os[(size_t)s * D];
    o /= Lsum;
  }
  if constexpr (MODE == kPerTensor) o *= a.v_static[0];
  if constexpr (MODE == kPerChannel) o *= a.v_static[(size_t)hkv * D + d];
  const int jq = r / a.G, gh = r % a.G;
  const int h = hkv * a.G + gh;
  if (a.sink != nullptr && Lsum > 0.0f) {
    const float lse = 0.6931471805599453f * (M + log2f(Lsum));
    o *= 1.0f / (1.0f + expf(a.sink[h] - lse));
  }
  a.out[(((size_t)b * a.Tq + jq) * a.Hq + h) * D + d] = f32_to_bf16(o);
}

}  // namespace

hipError_t launch_combine(int mode, int D, const CombineArgs& a, int B, hipStream_t st) {
  if (a.S > kMaxSplits || D % 64 != 0) return hipErrorInvalidValue;
  dim3 grid(D / 64, a.R, B * a.Hkv);
  switch (mode) {
    case kPerRow: hipLaunchKernelGGL(combine_kernel<kPerRow>, grid, dim3(64), 0, st, a, D); break;
    case kPerTensor: hipLaunchKernelGGL(combine_kernel<kPerTensor>, grid, dim3(64), 0, st, a, D); break;
    case kPerChannel: hipLaunchKernelGGL(combine_kernel<kPerChannel>, grid, dim3(64), 0, st, a, D); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
