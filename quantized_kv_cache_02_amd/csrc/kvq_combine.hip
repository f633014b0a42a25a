// kvq_combine.hip -- fixed-order merge of the split partials, static V scale,
// head sink, bf16 output: the decode's chunks and a split prefill's context
// parts.
//
// Kernel page "kv-quant-attn", "Method": the sequence is split across
// workgroups and the partials are merged in a fixed order, so repeated decodes
// are bitwise identical.  ORT PR "[CUDA] PagedAttention: quantized KV cache
// ...", "CUDA kernels" (ApplyHeadSink): the output of head h is rescaled by
// 1 / (1 + exp(s_h - lse)) after the quantized branch.
//
// With split s holding (m_s in log2 units, l_s, o_s normalized):
//   M = max_s m_s,  w_s = l_s 2^(m_s - M),  L = sum_s w_s,  o = sum_s w_s o_s / L,
//   lse = ln 2 (M + log2 L).
//
// One workgroup per (sequence, KV head, query row, 64 channels) of W = 1 or 4
// wavefronts: 16 channel quads x 4 W split groups.  It first locates the
// sequence's chunk slots (recorded by the decode kernel); then every thread
// issues the loads of its splits' m and l and of the first batch of partial
// outputs before using any (one round trip to the cache hierarchy), the
// weights follow, and the split groups are summed in group order -- across
// lanes, and with 4 wavefronts through LDS.  Every sum runs in the same order
// on every call.  The batch loads stay unconditional (clamped to slot 0).
// One wavefront has no barrier but covers 64 splits per round trip, 4 cover
// 128.  A third form (combine16_kernel) gives one wavefront 16 channels, for
// grids too small to fill the CUs; launch_mode picks among them.

#include "kvq_device.h"
#include "kvq_sched.h"  // clamp_len

namespace kvq {
namespace {

constexpr int kMaxSplits = 4096;
constexpr int kQuads = 16;  // 4-channel columns per workgroup (64 channels)

template <int MODE, int D, int W>
__global__ __launch_bounds__(64 * W) void combine_kernel(CombineArgs a) {
  constexpr int kGroups = 4 * W;           // split groups
  constexpr int kBatch = W == 1 ? 16 : 8;  // loads issued back to back per thread
  extern __shared__ float w_s[];           // [SMAX] chunk weights
  __shared__ float red[W];
  __shared__ float4_t part[W > 1 ? kGroups : 1][kQuads];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int quad = tid % kQuads, grp = tid / kQuads;
  const int d = blockIdx.x * 64 + quad * 4;
  const int r = blockIdx.y;
  const int head = blockIdx.z;  // b * Hkv + hkv
  const int b = head / a.Hkv, hkv = head % a.Hkv;
  // The chunk slots [P, P + S) that hold sequence b's partials.  With one
  // sequence P = 0, and every slot that may hold one (Sld) is loaded at once,
  // beside the length that says how many do (S, computed once the loads are
  // out); the others are never used.
  const int L0 = a.seq_lens[0];
  int P, Sld;
  if (a.B == 1) {
    P = 0;
    Sld = min(a.S, a.SMAX);
  } else {
    // the split kernel recorded the sequence's chunk slots in the workspace
    const int Sb = a.chunks[2 * b + 1];
    Sld = min(Sb, a.SMAX);  // the host bounds every S_b by SMAX
    // an empty sequence owns no slot; its (unused) loads read slot 0
    P = Sld > 0 ? a.chunks[2 * b] : 0;
  }
  const size_t rowbase = ((size_t)hkv * a.R + r) * a.S + P;
  const float* ms = a.ws_m + rowbase;
  const float* ls = a.ws_l + rowbase;

  // Split tid's m and l, then the first batch of partial outputs (which does
  // not depend on the split maxima): all in one round trip.
  constexpr int NT = 64 * W;
  const int sm = tid < Sld ? tid : 0;
  const float m0 = ms[sm], l0 = ls[sm];
  const float* os = a.ws_o + rowbase * D + d;
  float4_t v0[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int s = grp + i * kGroups;
    v0[i] = *reinterpret_cast<const float4_t*>(os + (size_t)(s < Sld ? s : 0) * D);
  }
  int S = Sld;
  if (a.B == 1) {
    const Span sp = visible_tiles(clamp_len(L0, a.max_seq_len), a.Tq, a.window);
    const int nt = sp.end - sp.first;
    const int C = max((nt + a.NW - 1) / a.NW, kMinTilesPerSplit);
    S = min((nt + C - 1) / C, Sld);
  }

  // M: per-thread max over s = tid, tid + NT, ..., then waves, then in wave order
  float M = tid < S ? m0 : -INFINITY;
  for (int s = tid + NT; s < S; s += NT) M = fmaxf(M, ms[s]);
  M = wave_max(M);
  if constexpr (W > 1) {
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, red[w]);
    __syncthreads();
  }
  float part_l = 0.0f;
  for (int s = tid; s < S; s += NT) {
    const float m = s == tid ? m0 : ms[s], l = s == tid ? l0 : ls[s];
    const float w = (M == -INFINITY || l == 0.0f) ? 0.0f : l * exp2f(m - M);
    w_s[s] = w;
    part_l += w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part_l += __shfl_xor(part_l, o);
  float Lsum = part_l;
  if constexpr (W > 1) {
    if (lane == 0) red[wave] = part_l;
    __syncthreads();  // (also publishes w_s to the other wavefronts)
    Lsum = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) Lsum += red[w];
  }

  // weighted sum of this thread's splits s = grp, grp + kGroups, ... in order
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int s = grp + i * kGroups;
    if (s < S) acc += w_s[s] * v0[i];
  }
  for (int s0 = grp + kGroups * kBatch; s0 < S; s0 += kGroups * kBatch) {
    float4_t v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int s = s0 + i * kGroups;
      v[i] = *reinterpret_cast<const float4_t*>(os + (size_t)(s < S ? s : 0) * D);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int s = s0 + i * kGroups;
      if (s < S) acc += w_s[s] * v[i];
    }
  }
  float4_t o;
  if constexpr (W == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = group_sum4(acc[e]);  // the 4 groups, across lanes
    if (grp != 0) return;
  } else {
    part[grp][quad] = acc;
    __syncthreads();
    if (grp != 0) return;
    o = part[0][quad];
#pragma unroll
    for (int g2 = 1; g2 < kGroups; ++g2) o += part[g2][quad];
  }

  float f = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  const int jq = r / a.G, gh = r % a.G;
  const int h = hkv * a.G + gh;
  if (a.sink != nullptr && Lsum > 0.0f) {
    const float lse = 0.6931471805599453f * (M + log2f(Lsum));
    f *= 1.0f / (1.0f + expf(a.sink[h] - lse));
  }
  uint16_t ob[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = o[e] * f;
    if constexpr (MODE == kPerTensor) x *= a.v_static[0];
    if constexpr (MODE == kPerChannel) x *= a.v_static[(size_t)hkv * D + d + e];
    ob[e] = f32_to_bf16(x);
  }
  u32x2_t packed = {(uint32_t)ob[0] | ((uint32_t)ob[1] << 16), (uint32_t)ob[2] | ((uint32_t)ob[3] << 16)};
  *reinterpret_cast<u32x2_t*>(a.out + (((size_t)b * a.Tq + jq) * a.Hq + h) * D + d) = packed;
}

// One wavefront per (sequence, KV head, query row, 16 channels): its lanes are
// 4 channel quads x 16 split groups.  Every lane loads the m, l and partial
// output of its splits s = group + 16 i (all of them in one round trip for up
// to 128 partials), and the split groups are summed across lanes in a fixed
// order: no LDS and no barrier.
template <int MODE, int D>
__global__ __launch_bounds__(64) void combine16_kernel(CombineArgs a) {
  constexpr int kG = 16;  // split groups
  constexpr int kB = 8;   // partials per lane in the first round trip
  const int lane = threadIdx.x;
  const int quad = lane & 3, grp = lane >> 2;
  const int d = blockIdx.x * 16 + quad * 4;
  const int r = blockIdx.y;
  const int head = blockIdx.z;  // b * Hkv + hkv
  const int b = head / a.Hkv, hkv = head % a.Hkv;
  const int L0 = a.seq_lens[0];
  int P, Sld;
  if (a.B == 1) {
    P = 0;
    Sld = min(a.S, a.SMAX);
  } else {
    const int Sb = a.chunks[2 * b + 1];
    Sld = min(Sb, a.SMAX);  // the host bounds every S_b by SMAX
    P = Sld > 0 ? a.chunks[2 * b] : 0;
  }
  const size_t rowbase = ((size_t)hkv * a.R + r) * a.S + P;
  const float* ms = a.ws_m + rowbase;
  const float* ls = a.ws_l + rowbase;
  const float* os = a.ws_o + rowbase * D + d;
  float mv[kB], lv[kB];
  float4_t v0[kB];
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    const int s = grp + kG * i;
    const int sc = s < Sld ? s : 0;
    mv[i] = ms[sc];
    lv[i] = ls[sc];
    v0[i] = *reinterpret_cast<const float4_t*>(os + (size_t)sc * D);
  }
  int S = Sld;
  if (a.B == 1) {
    const Span sp = visible_tiles(clamp_len(L0, a.max_seq_len), a.Tq, a.window);
    const int nt = sp.end - sp.first;
    const int C = max((nt + a.NW - 1) / a.NW, kMinTilesPerSplit);
    S = min((nt + C - 1) / C, Sld);
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kB; ++i)
    if (grp + kG * i < S) M = fmaxf(M, mv[i]);
  for (int s = grp + kG * kB; s < S; s += kG) M = fmaxf(M, ms[s]);
  M = wave_max(M);
  float lsum = 0.0f;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    if (grp + kG * i < S) {
      const float w = (M == -INFINITY || lv[i] == 0.0f) ? 0.0f : lv[i] * exp2f(mv[i] - M);
      lsum += w;
      acc += w * v0[i];
    }
  }
  for (int s = grp + kG * kB; s < S; s += kG) {
    const float l = ls[s];
    const float w = (M == -INFINITY || l == 0.0f) ? 0.0f : l * exp2f(ms[s] - M);
    lsum += w;
    acc += w * *reinterpret_cast<const float4_t*>(os + (size_t)s * D);
  }
  // the 16 split groups (lane bits 2..5); the 4 quads hold the same weights
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) {
    lsum += __shfl_xor(lsum, o);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], o);
  }
  if (grp != 0) return;
  const float Lsum = lsum;
  float f = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  const int jq = r / a.G, gh = r % a.G;
  const int h = hkv * a.G + gh;
  if (a.sink != nullptr && Lsum > 0.0f) {
    const float lse = 0.6931471805599453f * (M + log2f(Lsum));
    f *= 1.0f / (1.0f + expf(a.sink[h] - lse));
  }
  uint16_t ob[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = acc[e] * f;
    if constexpr (MODE == kPerTensor) x *= a.v_static[0];
    if constexpr (MODE == kPerChannel) x *= a.v_static[(size_t)hkv * D + d + e];
    ob[e] = f32_to_bf16(x);
  }
  u32x2_t packed = {(uint32_t)ob[0] | ((uint32_t)ob[1] << 16), (uint32_t)ob[2] | ((uint32_t)ob[3] << 16)};
  *reinterpret_cast<u32x2_t*>(a.out + (((size_t)b * a.Tq + jq) * a.Hq + h) * D + d) = packed;
}

template <int MODE, int W>
hipError_t launch_waves(int D, const CombineArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  switch (D) {
    case 64: hipLaunchKernelGGL((combine_kernel<MODE, 64, W>), grid, dim3(64 * W), lds, st, a); break;
    case 128: hipLaunchKernelGGL((combine_kernel<MODE, 128, W>), grid, dim3(64 * W), lds, st, a); break;
    case 256: hipLaunchKernelGGL((combine_kernel<MODE, 256, W>), grid, dim3(64 * W), lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_16(int D, const CombineArgs& a, dim3 grid, hipStream_t st) {
  const dim3 g16(D / 16, grid.y, grid.z);
  switch (D) {
    case 64: hipLaunchKernelGGL((combine16_kernel<MODE, 64>), g16, dim3(64), 0, st, a); break;
    case 128: hipLaunchKernelGGL((combine16_kernel<MODE, 128>), g16, dim3(64), 0, st, a); break;
    case 256: hipLaunchKernelGGL((combine16_kernel<MODE, 256>), g16, dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int D, const CombineArgs& a, dim3 grid, hipStream_t st) {
  if (a.SMAX < 1 || a.SMAX > kMaxSplits) return hipErrorInvalidValue;
  const size_t lds = (size_t)a.SMAX * sizeof(float);
  // Rows with at most 64 partials: one wavefront per 16 channels where the
  // 64-channel grid leaves CUs idle, one per 64 where it fills them; more
  // partials: four wavefronts per 64 channels.  Measured on MI355X, step us:
  // int8 at 64K (96 workgroups of 64 channels) 29.34 with four wavefronts,
  // 29.10 with one per 16 channels; workload 5 (3,072) 73.8 with one per 64,
  // 76.7 with one per 16; int4 at 64K (128 partials) 22.16 with four, 22.45
  // with one per 16, 24.4 with one per 64.
  const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
  if (a.SMAX <= 64 && wgs < kNumCUs) return launch_16<MODE>(D, a, grid, st);
  if (a.SMAX <= 64) return launch_waves<MODE, 1>(D, a, grid, lds, st);
  return launch_waves<MODE, 4>(D, a, grid, lds, st);
}


// Merge of a split prefill's KS context parts, one thread per (sequence, KV
// head, query row, 4 channels): with part p holding (m_p in log2 units, l_p,
// o_p normalized), M = max_p m_p, w_p = l_p 2^(m_p - M), L = sum_p w_p and
// o = sum_p w_p o_p / L in part order; then the head sink and the static V
// scale as in the decode combine, bf16 out.
template <int MODE, int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillCombineArgs a) {
  constexpr int Q = D / 4;  // channel quads per row
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)a.R * Q) return;
  const int r = (int)(i / Q), d = 4 * (int)(i % Q);
  const int head = blockIdx.y;  // b * Hkv + hkv
  const int b = head / a.Hkv, hkv = head % a.Hkv;
  const size_t row = (size_t)head * a.R + r;
  const float* ml = a.ws_ml + row * a.KS * 2;
  float M = -INFINITY;
  for (int p = 0; p < a.KS; ++p) M = fmaxf(M, ml[2 * p]);
  float Lsum = 0.0f;
  float4_t o = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.KS; ++p) {
    const float l = ml[2 * p + 1];
    const float w = (M == -INFINITY || l == 0.0f) ? 0.0f : l * exp2f(ml[2 * p] - M);
    Lsum += w;
    o += w * *reinterpret_cast<const float4_t*>(a.ws_o + (row * a.KS + p) * D + d);
  }
  float f = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  const int jq = r / a.G, gh = r % a.G;
  const int h = hkv * a.G + gh;
  if (a.sink != nullptr && Lsum > 0.0f) {
    const float lse = 0.6931471805599453f * (M + log2f(Lsum));
    f *= 1.0f / (1.0f + expf(a.sink[h] - lse));
  }
  uint16_t ob[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = o[e] * f;
    if constexpr (MODE == kPerTensor) x *= a.v_static[0];
    if constexpr (MODE == kPerChannel) x *= a.v_static[(size_t)hkv * D + d + e];
    ob[e] = f32_to_bf16(x);
  }
  u32x2_t packed = {(uint32_t)ob[0] | ((uint32_t)ob[1] << 16), (uint32_t)ob[2] | ((uint32_t)ob[3] << 16)};
  *reinterpret_cast<u32x2_t*>(a.out + (((size_t)b * a.Tq + jq) * a.Hq + h) * D + d) = packed;
}

template <int MODE>
hipError_t launch_prefill_mode(int D, const PrefillCombineArgs& a, int B, hipStream_t st) {
  if (a.KS < 2 || a.R < 1) return hipErrorInvalidValue;
  const long n = (long)a.R * (D / 4);
  dim3 grid((unsigned)((n + 255) / 256), (unsigned)(B * a.Hkv), 1);
  switch (D) {
    case 64: hipLaunchKernelGGL((prefill_combine_kernel<MODE, 64>), grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL((prefill_combine_kernel<MODE, 128>), grid, dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL((prefill_combine_kernel<MODE, 256>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(int mode, int D, const CombineArgs& a, int B, hipStream_t st) {
  dim3 grid(D / 64, a.R, B * a.Hkv);
  switch (mode) {
    case kNoScale:  // unquantized cache: nothing to apply
    case kPerRow: return launch_mode<kPerRow>(D, a, grid, st);
    case kPerTensor: return launch_mode<kPerTensor>(D, a, grid, st);
    case kPerChannel: return launch_mode<kPerChannel>(D, a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_combine(int mode, int D, const PrefillCombineArgs& a, int B, hipStream_t st) {
  switch (mode) {
    case kNoScale:  // unquantized cache: nothing to apply
    case kPerRow: return launch_prefill_mode<kPerRow>(D, a, B, st);
    case kPerTensor: return launch_prefill_mode<kPerTensor>(D, a, B, st);
    case kPerChannel: return launch_prefill_mode<kPerChannel>(D, a, B, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
