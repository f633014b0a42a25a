// kvq_params.h -- parameter blocks passed by value from the host launcher to
// the HIP kernels, and the launcher entry points of each kernel family.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// kBf16: an unquantized cache whose rows are the bf16 values themselves (the
// baseline of the quantized ones); it has no scales (scale mode kNoScale).
enum : int { kInt8 = 1, kInt4 = 2, kFp8 = 3, kBf16 = 4 };
enum : int { kNoScale = 0, kPerRow = 1, kPerTensor = 2, kPerChannel = 3 };

// Tokens per decode tile: one MFMA M dimension (16 rows of K) per wavefront step.
constexpr int kTile = 16;
// Wavefronts per decode workgroup; each owns a private online-softmax state.
constexpr int kWaves = 4;
constexpr int kNumCUs = 256;  // compute units of an MI355X

// Block-table entries of a paged cache are read once per decode workgroup, in
// its prologue, and held in registers: a wavefront keeps the entries of up to
// kTableRegs * 64 of its tiles, so a split spans at most kMaxTilesPerSplit
// tiles (the host sizes the split count accordingly).
constexpr int kTableRegs = 4;
constexpr int kMaxTilesPerSplit = kWaves * 64 * kTableRegs;
// Query tokens per sequence and step (1 + up to 7 speculative drafts).
constexpr int kMaxQTokens = 8;
// Smallest chunk of the balanced split schedule, in tiles.
constexpr int kMinTilesPerSplit = 8;
// Most context parts a prefill workgroup's tiles are cut into.
constexpr int kPrefillMaxParts = 8;

// Decode-kernel register budget: two wavefronts per SIMD (<= 256 registers
// per lane).  The kernel is built for row-block counts RB (16 query rows each)
// with RB * D <= 256, whose accumulators fit that budget beside the q operand
// and the tiles in flight.  Wider row sets up to kSplitMaxWideColumns run as
// one workgroup per chunk with one wavefront per SIMD, the accumulators in the
// accumulation registers (the "wide" units); wider ones share their row blocks
// out over several such workgroups per chunk.
constexpr int kSplitWavesPerSimd = 2;
constexpr int kSplitMaxAccColumns = 256;   // RB * D
constexpr int kSplitMaxWideColumns = 768;  // RB * D
// Tiles of codes held in registers per wavefront (one in use, one loading).
constexpr int kSplitTilesInFlight = 2;
// ... and for the wide-row-set variants (one wavefront per SIMD)
constexpr int kSplitWideTilesInFlight = 3;

struct CacheArgs {
  uint8_t* k_codes;
  uint8_t* v_codes;
  float* k_scales;  // per-row array, or static table
  float* v_scales;
  int32_t Hkv;
  int32_t block_size;
  int32_t num_blocks;
  const int32_t* block_table;  // nullptr: contiguous, sequence b owns block b
  int32_t max_blocks;
};

struct AppendArgs {
  CacheArgs c;
  const uint16_t* k;  // bf16 [B, Tn, Hkv, D]
  const uint16_t* v;
  const int32_t* positions;  // [B], or nullptr: position min(seq_lens[b], max_len) - Tn
  const int32_t* seq_lens;   // used when positions is nullptr
  int32_t max_len;           // bound on seq_lens (as the attention clamps it)
  int32_t B;
  int32_t Tn;
  int32_t capacity;  // tokens addressable per sequence
  int32_t kmode, vmode;  // scale modes of the K and V rows
};

struct SplitArgs {
  CacheArgs c;
  const uint16_t* q;  // bf16 [B, Tq, Hq, D]
  const int32_t* seq_lens;
  int32_t Hq, Tq, G, R;  // R = G * Tq query rows per (sequence, KV head)
  int32_t max_seq_len;
  int32_t B;   // sequences
  int32_t NW;  // nominal workgroups per KV head (the schedule's divisor)
  int32_t S;   // chunk slots per KV head: NW + B - 1
  int32_t RBN; // workgroups per chunk, each serving the kernel's RB 16-row blocks
               // of query rows (1: one workgroup serves every row)
  int32_t one_per_cu;  // the grid holds at most one workgroup per CU, so a variant
                       // may use one wavefront per SIMD's register budget
  float sm_scale;
  int32_t vmode;   // V scale mode (the K mode is the kernel's template mode)
  float softcap;   // > 0: logits z -> softcap * tanh(z / softcap)
  int32_t window;  // > 0: a query at position p sees tokens p - window + 1 .. p
  // fused append (both null when not fused): bf16 [B, Tq, Hkv, D] rows of the
  // query tokens, written at positions seq_len - Tq + j before they are read
  const uint16_t* k_new;
  const uint16_t* v_new;
  float* ws_o;  // [Hkv, R, S, D]  normalized chunk outputs, slot-major per row
  float* ws_m;  // [Hkv, R, S]     chunk max logit (log2 units)
  float* ws_l;  // [Hkv, R, S]     chunk normalizer
  int32_t* ws_chunks;  // [B][2] first chunk slot and chunk count of each sequence
                       // (written when B > 1 by the workgroup of slot 0, KV head 0)
};

struct CombineArgs {
  const float* ws_o;
  const float* ws_m;
  const float* ws_l;
  const float* v_static;  // per-tensor [1] / per-channel [Hkv, D] / nullptr (per-row)
  const float* sink;      // [Hq] or nullptr
  uint16_t* out;          // bf16 [B, Tq, Hq, D]
  const int32_t* seq_lens;
  const int32_t* chunks;  // [B][2] as written by the split kernel (used when B > 1)
  int32_t max_seq_len, B, NW;
  int32_t SMAX;           // most chunks one sequence can have
  int32_t window;         // the split's sliding window (it shapes the chunks)
  int32_t Hkv, Hq, Tq, G, R, S;
};

// Chunked prefill: Tq query tokens per sequence (the chunk, already appended
// at positions seq_len - Tq + j) attend causally to the cache.
struct PrefillArgs {
  CacheArgs c;
  const uint16_t* q;  // bf16 [B, Tq, Hq, D]
  const int32_t* seq_lens;
  int32_t Hq, Tq, G, R;  // R = G * Tq query rows per (sequence, KV head)
  int32_t max_seq_len;
  float sm_scale;
  int32_t vmode;          // V scale mode
  float softcap;          // > 0: logits z -> softcap * tanh(z / softcap)
  int32_t window;         // > 0: a query at position p sees tokens p - window + 1 .. p
  const float* v_static;  // per-tensor [1] / per-channel [Hkv, D] / nullptr
  const float* sink;      // [Hq] or nullptr
  uint16_t* out;          // bf16 [B, Tq, Hq, D]
  int32_t W;              // wavefronts per workgroup (4, or 8 at D = 256)
  // Context split: each workgroup's visible tiles are cut into KS parts, one
  // workgroup each; with KS > 1 the parts write their normalized partial
  // outputs and (m, l) to the workspace and a combine merges them.
  int32_t KS;
  float* ws_o;   // [B, Hkv, R, KS, D]
  float* ws_ml;  // [B, Hkv, R, KS, 2]: max logit (log2 units), normalizer
};

// The merge of a split prefill's parts (kvq_combine.hip).
struct PrefillCombineArgs {
  const float* ws_o;
  const float* ws_ml;
  const float* v_static;  // per-tensor [1] / per-channel [Hkv, D] / nullptr (per-row)
  const float* sink;      // [Hq] or nullptr
  uint16_t* out;          // bf16 [B, Tq, Hq, D]
  int32_t Hkv, Hq, Tq, G, R, KS;
};

hipError_t launch_append(int dtype, int kmode, int vmode, int D, const AppendArgs& a,
                         hipStream_t st);
hipError_t launch_split(int dtype, int mode, int D, int RB, const SplitArgs& a, int B,
                        hipStream_t st);
hipError_t launch_combine(int mode, int D, const CombineArgs& a, int B, hipStream_t st);
hipError_t launch_prefill_combine(int mode, int D, const PrefillCombineArgs& a, int B, hipStream_t st);

// translation units of the split kernel per (dtype, K scale mode, V scale per
// row or static): launch_split_<dtype>_<K mode>_<V per row>
#define KVQ_DECLARE_SPLIT(DT, MD)                                                                  \
  hipError_t launch_split_##DT##_##MD##_0(int D, int RB, const SplitArgs& a, int B, hipStream_t st); \
  hipError_t launch_split_##DT##_##MD##_1(int D, int RB, const SplitArgs& a, int B, hipStream_t st);
KVQ_DECLARE_SPLIT(1, 1)
KVQ_DECLARE_SPLIT(1, 2)
KVQ_DECLARE_SPLIT(1, 3)
KVQ_DECLARE_SPLIT(2, 1)
KVQ_DECLARE_SPLIT(2, 2)
KVQ_DECLARE_SPLIT(2, 3)
KVQ_DECLARE_SPLIT(3, 1)
KVQ_DECLARE_SPLIT(3, 2)
KVQ_DECLARE_SPLIT(3, 3)
#undef KVQ_DECLARE_SPLIT
hipError_t launch_split_4_0_0(int D, int RB, const SplitArgs& a, int B, hipStream_t st);
// their wide-row-set variants (kSplitMaxAccColumns < RB * D <= kSplitMaxWideColumns),
// built in units of their own; called by the units above
#define KVQ_DECLARE_WIDE(DT, MD)                                                                 \
  hipError_t launch_split_wide_##DT##_##MD##_0(int D, int RB, const SplitArgs& a, hipStream_t st); \
  hipError_t launch_split_wide_##DT##_##MD##_1(int D, int RB, const SplitArgs& a, hipStream_t st);
KVQ_DECLARE_WIDE(1, 1)
KVQ_DECLARE_WIDE(1, 2)
KVQ_DECLARE_WIDE(1, 3)
KVQ_DECLARE_WIDE(2, 1)
KVQ_DECLARE_WIDE(2, 2)
KVQ_DECLARE_WIDE(2, 3)
KVQ_DECLARE_WIDE(3, 1)
KVQ_DECLARE_WIDE(3, 2)
KVQ_DECLARE_WIDE(3, 3)
#undef KVQ_DECLARE_WIDE
hipError_t launch_split_wide_4_0_0(int D, int RB, const SplitArgs& a, hipStream_t st);

// prefill translation units, the same split by (dtype, K mode, V per row)
#define KVQ_DECLARE_PREFILL(DT, MD)                                                             \
  hipError_t launch_prefill_##DT##_##MD##_0(int D, const PrefillArgs& a, int B, hipStream_t st); \
  hipError_t launch_prefill_##DT##_##MD##_1(int D, const PrefillArgs& a, int B, hipStream_t st);
KVQ_DECLARE_PREFILL(1, 1)
KVQ_DECLARE_PREFILL(1, 2)
KVQ_DECLARE_PREFILL(1, 3)
KVQ_DECLARE_PREFILL(2, 1)
KVQ_DECLARE_PREFILL(2, 2)
KVQ_DECLARE_PREFILL(2, 3)
KVQ_DECLARE_PREFILL(3, 1)
KVQ_DECLARE_PREFILL(3, 2)
KVQ_DECLARE_PREFILL(3, 3)
#undef KVQ_DECLARE_PREFILL
hipError_t launch_prefill_4_0_0(int D, const PrefillArgs& a, int B, hipStream_t st);

}  // namespace kvq
