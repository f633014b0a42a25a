// kvq_host.cpp -- the C ABI of libkvq (include/kvq.h): host-side validation,
// static grid / workspace sizing, kernel launches.  Never synchronizes, never
// allocates, never reads device memory, so every entry point can be captured
// into a HIP graph.

#include <algorithm>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "kvq.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvq_params.h"

namespace {

using kvq::CacheArgs;

constexpr int kMaxGroup = 8;     // query heads per KV head
constexpr int kMaxSplits = 4096;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_cache(const kvq_cache* c) {
  if (c == nullptr) return KVQ_EINVAL;
  if (c->dtype != KVQ_INT8 && c->dtype != KVQ_INT4 && c->dtype != KVQ_FP8_E4M3FN &&
      c->dtype != KVQ_BF16)
    return KVQ_EUNSUPPORTED;
  const bool scaled = c->dtype != KVQ_BF16;
  if (!scaled) {
    // unquantized: no scale of either side
    if (c->scale_mode != KVQ_NO_SCALE || c->v_scale_mode != KVQ_NO_SCALE) return KVQ_EUNSUPPORTED;
  } else {
    if (c->scale_mode != KVQ_PER_ROW && c->scale_mode != KVQ_PER_TENSOR &&
        c->scale_mode != KVQ_PER_CHANNEL)
      return KVQ_EUNSUPPORTED;
    if (c->v_scale_mode != 0 && c->v_scale_mode != KVQ_PER_ROW &&
        c->v_scale_mode != KVQ_PER_TENSOR && c->v_scale_mode != KVQ_PER_CHANNEL)
      return KVQ_EUNSUPPORTED;
  }
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return KVQ_EUNSUPPORTED;
  if (c->num_kv_heads < 1 || c->block_size < 16 || c->block_size % 16 != 0 || c->num_blocks < 1)
    return KVQ_EINVAL;
  if (c->k_codes == nullptr || c->v_codes == nullptr) return KVQ_EINVAL;
  if (!aligned16(c->k_codes) || !aligned16(c->v_codes)) return KVQ_EINVAL;
  if (scaled) {
    if (c->k_scales == nullptr || c->v_scales == nullptr) return KVQ_EINVAL;
    if (!aligned16(c->k_scales) || !aligned16(c->v_scales)) return KVQ_EINVAL;
  }
  return KVQ_OK;
}

// Bytes of one cached row of codes (int4: two per byte; bf16: two bytes each).
int64_t row_bytes(const kvq_cache* c) {
  return c->dtype == KVQ_INT4 ? c->head_dim / 2 : c->dtype == KVQ_BF16 ? 2 * c->head_dim : c->head_dim;
}

int v_mode_of(const kvq_cache* c) { return c->v_scale_mode != 0 ? c->v_scale_mode : c->scale_mode; }

CacheArgs cache_args(const kvq_cache* c, const int32_t* table, int32_t max_blocks) {
  CacheArgs a;
  const bool scaled = c->dtype != KVQ_BF16;  // an unquantized cache's scales are never read
  a.k_codes = static_cast<uint8_t*>(c->k_codes);
  a.v_codes = static_cast<uint8_t*>(c->v_codes);
  a.k_scales = scaled ? c->k_scales : nullptr;
  a.v_scales = scaled ? c->v_scales : nullptr;
  a.Hkv = c->num_kv_heads;
  a.block_size = c->block_size;
  a.num_blocks = c->num_blocks;
  a.block_table = table;
  a.max_blocks = table ? max_blocks : 0;
  return a;
}

struct DecodeShape {
  int G, R, RB, S;  // S: reported by kvq_num_splits (= NW)
  int NW;           // nominal workgroups per KV head, batch * S
  int RBN;          // workgroups per chunk (row-split launches), 1 otherwise
  int RBK;          // row blocks per workgroup (the kernel variant)
  int SMAX;         // most chunks one sequence can get
  int NSLOT;        // chunk slots per KV head, NW + batch - 1
  int one_per_cu;   // at most one live workgroup per CU (NW not doubled)
};

// Static decode shape: grouping, query rows, row blocks and the split count S,
// a pure function of (batch, Hkv, max_seq_len) so that graphs and workspaces
// sized once stay valid.  Independent of the cache layout.
int decode_shape(const kvq_cache* c, int32_t batch, int32_t hq, int32_t tq, int32_t max_seq_len,
                 DecodeShape* sh) {
  int st = check_cache(c);
  if (st != KVQ_OK) return st;
  if (batch < 1 || hq < 1 || tq < 1 || max_seq_len < 1) return KVQ_EINVAL;
  if (hq % c->num_kv_heads != 0) return KVQ_EINVAL;
  const int G = hq / c->num_kv_heads;
  if (G > kMaxGroup || tq > kvq::kMaxQTokens) return KVQ_EUNSUPPORTED;
  if (batch > 65535 || c->num_kv_heads > 65535) return KVQ_EUNSUPPORTED;
  // the split kernel addresses a tile by its first pool row over 16 in an int
  if ((int64_t)c->num_blocks * c->num_kv_heads * c->block_size / 16 > INT32_MAX) return KVQ_EUNSUPPORTED;
  const int64_t ntiles = ((int64_t)max_seq_len + 15) / 16;
  const int64_t Hkv = c->num_kv_heads;
  // Balanced schedule: the tiles of all sequences of a KV head are cut into
  // chunks of C = max(ceil(T / NW), kMinTilesPerSplit) tiles, sequence by
  // sequence, so at most NW + batch - 1 chunk workgroups per KV head.  NW is
  // sized so that the whole grid fits one workgroup per CU (measured on
  // MI355X at 64K tokens, B1 Hkv4 D256 int8: 256 workgroups, 16 tiles per
  // wavefront, beat 512, 28.1 vs 29.4 us), with at least kMinTilesPerSplit
  // tiles per chunk for a full-length sequence, and few enough tiles per chunk
  // for the block-table registers.
  // More than 256 accumulator columns (row blocks x head_dim) do not fit the
  // registers of two wavefronts per SIMD with the q operand and the tiles in
  // flight.  Up to kSplitMaxWideColumns the chunk keeps one workgroup, built
  // for one wavefront per SIMD with the accumulators in the accumulation
  // registers, so every tile is unpacked once for all its rows; beyond that
  // the row blocks are shared out evenly over RBN such workgroups per chunk
  // (49-64 rows at D 256: two of 2 blocks), which read the chunk's bytes
  // through L2.
  // At exactly kSplitMaxWideColumns (33-48 rows at D 256) the one-workgroup
  // loop is not pipelined, and with per-row V scales (multiplied into the
  // weights: more live registers) it measured slower on MI355X than two
  // pipelined workgroups of 2 row blocks (64K int8 per-row, 48 rows:
  // 56.5 -> 45.7 us; fp8 K per-channel + V per-row 57.6 -> 48.9 us); with
  // static V scales one workgroup stays (int4 per-channel 68.3 vs 81.4 us).
  const int RB = (G * tq + 15) / 16;
  const int rb_max = std::max(kvq::kSplitMaxWideColumns / c->head_dim, 1);
  const bool vrow_768 = RB * c->head_dim == kvq::kSplitMaxWideColumns && RB > 2 &&
                        c->dtype != KVQ_BF16 && v_mode_of(c) == KVQ_PER_ROW;
  const int RBN = vrow_768 ? 2 : (RB + rb_max - 1) / rb_max;
  const int RBK = (RB + RBN - 1) / RBN;  // row blocks per workgroup
  const bool wide = RBK * c->head_dim > kvq::kSplitMaxAccColumns;
  // Compute-bound variants of at most 256 accumulator columns (rows of at
  // most 128 bytes, whose tiles carry less data per instruction: packed int4
  // at D 256, the 8-bit caches at D 128 and below) run two workgroups per
  // CU -- two wavefronts per SIMD hide each other's dependency stalls
  // (measured on MI355X: int4 at 256K tokens 78.1 -> 68.6 us, paged fp8 at
  // D 128 28.9 -> 27.9 us per step) -- as long as a chunk keeps at least
  // 2 * kMinTilesPerSplit tiles.  (Every row-split launch is wide.)
  const int64_t per_head = std::max<int64_t>(kvq::kNumCUs / (Hkv * RBN), 1);
  const int64_t all_tiles = (int64_t)batch * ntiles;
  int64_t NW = per_head - (batch - 1);
  bool doubled = false;
  if (!wide && row_bytes(c) <= 128 &&
      2 * per_head - (batch - 1) <= all_tiles / (2 * kvq::kMinTilesPerSplit)) {
    NW = 2 * per_head - (batch - 1);
    doubled = true;
  }
  NW = std::min<int64_t>(NW, all_tiles / kvq::kMinTilesPerSplit);
  NW = std::max<int64_t>(NW, 1);
  const int64_t need = ((int64_t)batch * ntiles + kvq::kMaxTilesPerSplit - 1) / kvq::kMaxTilesPerSplit;
  NW = std::max(NW, need);
  // chunks of one sequence: at most NW + 1, and at most one per
  // kMinTilesPerSplit tiles; the combine merges up to kMaxSplits
  const int64_t most = std::min<int64_t>(NW + 1, (ntiles + kvq::kMinTilesPerSplit - 1) /
                                                     kvq::kMinTilesPerSplit);
  if (most > kMaxSplits || NW + batch - 1 > INT32_MAX / 2) return KVQ_EUNSUPPORTED;
  sh->G = G;
  sh->R = G * tq;
  sh->RB = (sh->R + 15) / 16;
  sh->S = (int)NW;
  sh->NW = (int)NW;
  sh->RBN = RBN;
  sh->SMAX = (int)std::min<int64_t>(most, NW + batch - 1);
  sh->RBK = RBK;
  sh->NSLOT = (int)(NW + batch - 1);
  // (the need-based minimum below can exceed the CU count for very long
  // batches; then the grid holds more than one workgroup per CU)
  sh->one_per_cu = !doubled && (int64_t)sh->NSLOT * Hkv * RBN <= kvq::kNumCUs;
  return KVQ_OK;
}

// Layout of the sequences in the cache: contiguous (no table) or paged.
int check_layout(const kvq_cache* c, int32_t batch, int32_t max_seq_len, const int32_t* table,
                 int32_t max_blocks) {
  if (table == nullptr) {
    if (c->num_blocks < batch || max_seq_len > c->block_size) return KVQ_EINVAL;
  } else {
    if (max_blocks < 1) return KVQ_EINVAL;
    if ((int64_t)max_seq_len > (int64_t)max_blocks * c->block_size) return KVQ_EINVAL;
  }
  return KVQ_OK;
}

size_t workspace_size(const kvq_cache* c, int32_t batch, const DecodeShape& sh) {
  const size_t rows = (size_t)c->num_kv_heads * sh.R * sh.NSLOT;
  // o [rows, D], m [rows], l [rows], then the chunk table [batch] (first slot,
  // chunk count), each region 256-byte aligned
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return up(rows * c->head_dim * 4) + 2 * up(rows * 4) + up((size_t)batch * 8);
}

void workspace_ptrs(void* ws, const kvq_cache* c, int32_t batch, const DecodeShape& sh, float** o,
                    float** m, float** l, int32_t** chunks) {
  (void)batch;
  const size_t rows = (size_t)c->num_kv_heads * sh.R * sh.NSLOT;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* base = static_cast<char*>(ws);
  *o = reinterpret_cast<float*>(base);
  *m = reinterpret_cast<float*>(base + up(rows * c->head_dim * 4));
  *l = reinterpret_cast<float*>(base + up(rows * c->head_dim * 4) + up(rows * 4));
  *chunks = reinterpret_cast<int32_t*>(base + up(rows * c->head_dim * 4) + 2 * up(rows * 4));
}

hipError_t dispatch_split(int dt, int md, bool vrow, int D, int RB, const kvq::SplitArgs& a, int B,
                          hipStream_t st) {
#define KVQ_CASE(DT, MD)                                                                        \
  if (dt == DT && md == MD)                                                                     \
    return vrow ? kvq::launch_split_##DT##_##MD##_1(D, RB, a, B, st)                            \
                : kvq::launch_split_##DT##_##MD##_0(D, RB, a, B, st);
  KVQ_CASE(1, 1)
  KVQ_CASE(1, 2)
  KVQ_CASE(1, 3)
  KVQ_CASE(2, 1)
  KVQ_CASE(2, 2)
  KVQ_CASE(2, 3)
  KVQ_CASE(3, 1)
  KVQ_CASE(3, 2)
  KVQ_CASE(3, 3)
#undef KVQ_CASE
  if (dt == KVQ_BF16 && md == KVQ_NO_SCALE && !vrow) return kvq::launch_split_4_0_0(D, RB, a, B, st);
  return hipErrorInvalidValue;
}

// Chunked prefill: workgroup size W and context split KS.  A workgroup owns
// 16 * W query rows (32 * W below D = 256) of one KV head and walks the
// 64-token tiles they see; workgroups run one per CU.  An 8-wavefront
// workgroup (D = 256 only) gets through 128 rows in 1 / 0.8 of the time a
// 4-wavefront one takes for 64 (measured on MI355X at 32K + 1K tokens: 1.66x
// the row rate for int4, 1.63x for bf16).  When the workgroups do not fill
// whole rounds of 256 CUs (384 for 2K query tokens at 24 / 4 heads: a second
// round half empty), the tiles of each are cut into KS parts, one workgroup
// each, and a combine merges the parts.  Cost model per (W, KS): a
// workgroup costs its part's tiles + 4 tiles of per-workgroup overhead, times
// 0.8 for W = 4, and the kernel the makespan of the workgroups dealt longest
// first to the least loaded of 256 CUs, as the kernel orders them (causal
// rows see different tile counts: with no cached context a 2,048-token chunk
// ran 330 TFLOP/s in two parts and 417 in one, which a model of whole rounds
// of the longest workgroup had ranked the other way); past 16 rounds, rounds
// of the longest workgroup.  KS only where the workspace is given, each part
// keeping at least 8 tiles; a larger KS must beat a smaller one by 3 % per
// step, and one that breaks the kernel's XCD grouping (below) by 10 %.  A
// pure function of the shape, so workspaces sized once stay valid.
struct PrefillPlan {
  int W, KS;
};

PrefillPlan prefill_plan(const kvq_cache* c, int32_t batch, int G, int32_t tq, int32_t max_seq_len,
                         int32_t window, bool split) {
  const int D = c->head_dim;
  const int64_t R = (int64_t)G * tq;
  const int64_t L = max_seq_len, pos0 = L - tq;  // position of the chunk's first token
  int64_t tiles = (L + 63) / 64;  // a workgroup sees at most these
  PrefillPlan best{4, 1};
  double best_cost = 0.0;
  bool first = true;
  std::vector<double> work;
  for (int W : {4, 8}) {
    if (W == 8 && D != 256) continue;
    const int64_t rows = 16 * (D >= 256 ? 1 : 2) * W;
    const int64_t nrg = (R + rows - 1) / rows;
    const double wgf = W == 4 ? 0.8 : 1.0;
    int64_t t = tiles;
    if (window > 0) t = std::min<int64_t>(t, ((int64_t)window + rows / G + 63) / 64 + 1);
    for (int ks = 1; ks <= (split ? kvq::kPrefillMaxParts : 1); ++ks) {
      if (ks > 1 && t < (int64_t)ks * 8) break;
      const int64_t copies = (int64_t)c->num_kv_heads * batch;
      const int64_t items = nrg * copies * ks;
      double cost;
      if (items > 16 * (int64_t)kvq::kNumCUs) {
        const int64_t rounds = (items + kvq::kNumCUs - 1) / kvq::kNumCUs;
        cost = (double)rounds * ((double)t / ks + 4.0) * wgf;
      } else {
        // the tiles each row group's rows see (as the kernel bounds them)
        work.clear();
        for (int64_t g = 0; g < nrg; ++g) {
          const int64_t rlast = std::min((g + 1) * rows, R) - 1;
          const int64_t hi = std::min(pos0 + rlast / G, L - 1);
          const int64_t end = hi >= 0 ? hi / 64 + 1 : 0;
          int64_t begin = 0;
          if (window > 0) begin = std::max<int64_t>(pos0 + g * rows / G - window + 1, 0) / 64;
          const int64_t tg = std::max<int64_t>(end - begin, 0);
          const int64_t C = (tg + ks - 1) / ks;
          for (int p = 0; p < ks; ++p) {
            const int64_t tp = std::min(std::max<int64_t>(tg - p * C, 0), C);
            for (int64_t k = 0; k < copies; ++k) work.push_back(((double)tp + 4.0) * wgf);
          }
        }
        std::sort(work.begin(), work.end(), std::greater<double>());
        std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
        for (int i = 0; i < kvq::kNumCUs; ++i) cu.push(0.0);
        double span = 0.0;
        for (double w : work) {
          const double e = cu.top() + w;
          cu.pop();
          cu.push(e);
          span = std::max(span, e);
        }
        cost = span;
      }
      cost *= 1.0 + 0.03 * (ks - 1);
      // the kernel keeps each XCD on the same (KV head, part) pairs only when
      // KS * Hkv divides 8 or 8 divides it; other splits lose that L2 reuse
      const int64_t hp = (int64_t)ks * c->num_kv_heads;
      if (ks > 1 && 8 % hp != 0 && hp % 8 != 0) cost *= 1.1;
      if (first || cost < best_cost) {
        best = PrefillPlan{W, ks};
        best_cost = cost;
        first = false;
      }
    }
  }
  return best;
}

size_t prefill_workspace_size(const kvq_cache* c, int32_t batch, int32_t R, int KS) {
  if (KS <= 1) return 0;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)batch * c->num_kv_heads * R * KS;
  return up(rows * c->head_dim * 4) + up(rows * 2 * 4);
}

// Shape checks shared by the prefill entry points.
int prefill_check(const kvq_cache* cache, int32_t batch, int32_t num_q_heads, int32_t q_tokens,
                  int32_t max_seq_len, int* G) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (batch < 1 || num_q_heads < 1 || q_tokens < 1 || max_seq_len < 1) return KVQ_EINVAL;
  if (num_q_heads % cache->num_kv_heads != 0) return KVQ_EINVAL;
  *G = num_q_heads / cache->num_kv_heads;
  if (*G > kMaxGroup) return KVQ_EUNSUPPORTED;
  if (batch > 65535 || cache->num_kv_heads > 65535) return KVQ_EUNSUPPORTED;
  if ((int64_t)*G * q_tokens > INT32_MAX / 2) return KVQ_EUNSUPPORTED;
  // the prefill kernel addresses a 16-row group by its first pool row over 16 in an int
  if ((int64_t)cache->num_blocks * cache->num_kv_heads * cache->block_size / 16 > INT32_MAX)
    return KVQ_EUNSUPPORTED;
  return KVQ_OK;
}


hipError_t dispatch_prefill(int dt, int md, bool vrow, int D, const kvq::PrefillArgs& a, int B,
                            hipStream_t st) {
#define KVQ_CASE(DT, MD)                                                                        \
  if (dt == DT && md == MD)                                                                     \
    return vrow ? kvq::launch_prefill_##DT##_##MD##_1(D, a, B, st)                              \
                : kvq::launch_prefill_##DT##_##MD##_0(D, a, B, st);
  KVQ_CASE(1, 1)
  KVQ_CASE(1, 2)
  KVQ_CASE(1, 3)
  KVQ_CASE(2, 1)
  KVQ_CASE(2, 2)
  KVQ_CASE(2, 3)
  KVQ_CASE(3, 1)
  KVQ_CASE(3, 2)
  KVQ_CASE(3, 3)
#undef KVQ_CASE
  if (dt == KVQ_BF16 && md == KVQ_NO_SCALE && !vrow) return kvq::launch_prefill_4_0_0(D, a, B, st);
  return hipErrorInvalidValue;
}

int prefill_impl(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                 int32_t batch, int32_t num_q_heads, int32_t q_tokens, const int32_t* seq_lens,
                 int32_t max_seq_len, float softmax_scale, const float* head_sink,
                 const int32_t* block_table, int32_t max_blocks, const kvq_attn_options* options,
                 void* out, void* workspace, size_t workspace_bytes, bool split, void* stream) {
  int G = 0;
  int st = prefill_check(cache, batch, num_q_heads, q_tokens, max_seq_len, &G);
  if (st != KVQ_OK) return st;
  st = check_layout(cache, batch, max_seq_len, block_table, max_blocks);
  if (st != KVQ_OK) return st;
  if (q == nullptr || seq_lens == nullptr || out == nullptr || !aligned16(q) || !aligned16(out))
    return KVQ_EINVAL;
  if ((k_new == nullptr) != (v_new == nullptr)) return KVQ_EINVAL;
  if (k_new != nullptr && (!aligned16(k_new) || !aligned16(v_new))) return KVQ_EINVAL;
  if (options != nullptr) {
    const float cap = options->softcap;
    if (!(cap >= 0.0f) || cap > 3.0e38f || options->window < 0) return KVQ_EINVAL;
  }
  const int32_t window = options ? options->window : 0;
  const PrefillPlan plan = prefill_plan(cache, batch, G, q_tokens, max_seq_len, window, split);
  const size_t need = prefill_workspace_size(cache, batch, G * q_tokens, plan.KS);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return KVQ_EINVAL;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (k_new != nullptr) {
    // the chunk's rows first, at positions seq_lens[b] - q_tokens + j
    kvq::AppendArgs ap;
    ap.c = cache_args(cache, block_table, max_blocks);
    ap.k = static_cast<const uint16_t*>(k_new);
    ap.v = static_cast<const uint16_t*>(v_new);
    ap.positions = nullptr;
    ap.seq_lens = seq_lens;
    ap.max_len = max_seq_len;
    ap.B = batch;
    ap.Tn = q_tokens;
    const int64_t capacity =
        block_table == nullptr ? cache->block_size : (int64_t)max_blocks * cache->block_size;
    if (capacity > INT32_MAX) return KVQ_EUNSUPPORTED;
    ap.capacity = (int32_t)capacity;
    ap.kmode = cache->scale_mode;
    ap.vmode = v_mode_of(cache);
    hipError_t e = kvq::launch_append(cache->dtype, ap.kmode, ap.vmode, cache->head_dim, ap, hs);
    if (e != hipSuccess) return KVQ_EHIP;
  }
  kvq::PrefillArgs a;
  a.c = cache_args(cache, block_table, max_blocks);
  a.q = static_cast<const uint16_t*>(q);
  a.seq_lens = seq_lens;
  a.Hq = num_q_heads;
  a.Tq = q_tokens;
  a.G = G;
  a.R = G * q_tokens;
  a.max_seq_len = max_seq_len;
  a.sm_scale = softmax_scale;
  a.vmode = v_mode_of(cache);
  a.softcap = options ? options->softcap : 0.0f;
  a.window = window;
  a.v_static = (a.vmode == KVQ_PER_TENSOR || a.vmode == KVQ_PER_CHANNEL) ? cache->v_scales : nullptr;
  a.sink = head_sink;
  a.out = static_cast<uint16_t*>(out);
  a.W = plan.W;
  a.KS = plan.KS;
  a.ws_o = nullptr;
  a.ws_ml = nullptr;
  if (plan.KS > 1) {
    const size_t rows = (size_t)batch * cache->num_kv_heads * a.R * plan.KS;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       ((rows * cache->head_dim * 4 + 255) & ~(size_t)255));
  }
  hipError_t e = dispatch_prefill(cache->dtype, cache->scale_mode, a.vmode == KVQ_PER_ROW,
                                  cache->head_dim, a, batch, hs);
  if (e != hipSuccess) return KVQ_EHIP;
  if (plan.KS > 1) {
    kvq::PrefillCombineArgs cb;
    cb.ws_o = a.ws_o;
    cb.ws_ml = a.ws_ml;
    cb.v_static = a.v_static;
    cb.sink = head_sink;
    cb.out = a.out;
    cb.Hkv = cache->num_kv_heads;
    cb.Hq = num_q_heads;
    cb.Tq = q_tokens;
    cb.G = G;
    cb.R = a.R;
    cb.KS = plan.KS;
    e = kvq::launch_prefill_combine(a.vmode, cache->head_dim, cb, batch, hs);
    if (e != hipSuccess) return KVQ_EHIP;
  }
  return KVQ_OK;
}

int split_impl(const kvq_cache* c, const void* q, int32_t batch, int32_t hq, int32_t tq,
               const int32_t* seq_lens, int32_t max_seq_len, float scale, const int32_t* table,
               int32_t max_blocks, void* ws, size_t ws_bytes, void* stream,
               const void* k_new = nullptr, const void* v_new = nullptr,
               const kvq_attn_options* opts = nullptr) {
  DecodeShape sh;
  int st = decode_shape(c, batch, hq, tq, max_seq_len, &sh);
  if (st != KVQ_OK) return st;
  st = check_layout(c, batch, max_seq_len, table, max_blocks);
  if (st != KVQ_OK) return st;
  if (q == nullptr || seq_lens == nullptr || ws == nullptr || !aligned16(q) || !aligned16(ws))
    return KVQ_EINVAL;
  if (ws_bytes < workspace_size(c, batch, sh)) return KVQ_EINVAL;
  kvq::SplitArgs a;
  a.c = cache_args(c, table, max_blocks);
  a.q = static_cast<const uint16_t*>(q);
  a.seq_lens = seq_lens;
  a.Hq = hq;
  a.Tq = tq;
  a.G = sh.G;
  a.R = sh.R;
  a.max_seq_len = max_seq_len;
  a.B = batch;
  a.NW = sh.NW;
  a.S = sh.NSLOT;
  a.RBN = sh.RBN;
  a.one_per_cu = sh.one_per_cu;
  a.sm_scale = scale;
  a.softcap = opts ? opts->softcap : 0.0f;
  a.window = opts ? opts->window : 0;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  workspace_ptrs(ws, c, batch, sh, &a.ws_o, &a.ws_m, &a.ws_l, &a.ws_chunks);
  a.vmode = v_mode_of(c);
  hipError_t e = dispatch_split(c->dtype, c->scale_mode, a.vmode == KVQ_PER_ROW, c->head_dim, sh.RBK, a,
                                batch,
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

int combine_impl(const kvq_cache* c, int32_t batch, int32_t hq, int32_t tq, const int32_t* seq_lens,
                 int32_t max_seq_len, const float* sink, void* out, const void* ws, size_t ws_bytes,
                 void* stream, int32_t window = 0) {
  DecodeShape sh;
  int st = decode_shape(c, batch, hq, tq, max_seq_len, &sh);
  if (st != KVQ_OK) return st;
  if (seq_lens == nullptr || out == nullptr || ws == nullptr || !aligned16(out) || !aligned16(ws))
    return KVQ_EINVAL;
  if (ws_bytes < workspace_size(c, batch, sh)) return KVQ_EINVAL;
  kvq::CombineArgs a;
  float *o, *m, *l;
  int32_t* chunks;
  workspace_ptrs(const_cast<void*>(ws), c, batch, sh, &o, &m, &l, &chunks);
  a.chunks = chunks;
  a.SMAX = sh.SMAX;
  a.window = window;
  a.ws_o = o;
  a.ws_m = m;
  a.ws_l = l;
  const int vmode = v_mode_of(c);
  a.v_static = (vmode == KVQ_PER_TENSOR || vmode == KVQ_PER_CHANNEL) ? c->v_scales : nullptr;
  a.sink = sink;
  a.out = static_cast<uint16_t*>(out);
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.B = batch;
  a.NW = sh.NW;
  a.Hkv = c->num_kv_heads;
  a.Hq = hq;
  a.Tq = tq;
  a.G = sh.G;
  a.R = sh.R;
  a.S = sh.NSLOT;
  hipError_t e = kvq::launch_combine(vmode, c->head_dim, a, batch,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

// Scratch of kvq_attend_ex_noalloc: the decode workspace of callers that
// cannot allocate.  One array per GPU (the runtime places a copy on every
// device the library runs on); host code uses only the device address that
// hipGetSymbolAddress returns for the current device, never the name.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The scratch address on the device the call's kernels run on (the stream's
// device; the current one for the null stream), looked up once per device
// with that device current.
int scratch_for_stream(hipStream_t stream, void** ptr) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return KVQ_EHIP;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return KVQ_EHIP;
    dev = static_cast<int>(sd);
  }
  if (dev < 0 || dev >= kMaxDevices) return KVQ_EHIP;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return KVQ_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return KVQ_EHIP;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return KVQ_OK;
}

}  // namespace

extern "C" {

int kvq_append(const kvq_cache* cache, const void* k, const void* v, int32_t batch, int32_t tokens,
               const int32_t* positions, const int32_t* block_table, int32_t max_blocks,
               void* stream) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (k == nullptr || v == nullptr || positions == nullptr || batch < 1 || tokens < 1)
    return KVQ_EINVAL;
  if (!aligned16(k) || !aligned16(v)) return KVQ_EINVAL;
  int64_t capacity;
  if (block_table == nullptr) {
    if (cache->num_blocks < batch) return KVQ_EINVAL;
    capacity = cache->block_size;
  } else {
    if (max_blocks < 1) return KVQ_EINVAL;
    capacity = (int64_t)max_blocks * cache->block_size;
  }
  if (capacity > INT32_MAX) return KVQ_EUNSUPPORTED;
  kvq::AppendArgs a;
  a.c = cache_args(cache, block_table, max_blocks);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.positions = positions;
  a.seq_lens = nullptr;
  a.max_len = 0;
  a.B = batch;
  a.Tn = tokens;
  a.capacity = (int32_t)capacity;
  a.kmode = cache->scale_mode;
  a.vmode = v_mode_of(cache);
  hipError_t e = kvq::launch_append(cache->dtype, cache->scale_mode, v_mode_of(cache), cache->head_dim, a,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

int32_t kvq_num_splits(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                       int32_t q_tokens, int32_t max_seq_len) {
  DecodeShape sh;
  int st = decode_shape(cache, batch, num_q_heads, q_tokens, max_seq_len, &sh);
  return st == KVQ_OK ? sh.S : st;
}

size_t kvq_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                           int32_t q_tokens, int32_t max_seq_len) {
  DecodeShape sh;
  if (decode_shape(cache, batch, num_q_heads, q_tokens, max_seq_len, &sh) != KVQ_OK) return 0;
  return workspace_size(cache, batch, sh);
}

int kvq_split_decode(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                     int32_t q_tokens, const int32_t* seq_lens, int32_t max_seq_len,
                     float softmax_scale, const int32_t* block_table, int32_t max_blocks,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return split_impl(cache, q, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, softmax_scale,
                    block_table, max_blocks, workspace, workspace_bytes, stream);
}

int kvq_combine(const kvq_cache* cache, int32_t batch, int32_t num_q_heads, int32_t q_tokens,
                const int32_t* seq_lens, int32_t max_seq_len, const float* head_sink, void* out,
                const void* workspace, size_t workspace_bytes, void* stream) {
  return combine_impl(cache, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, head_sink, out,
                      workspace, workspace_bytes, stream);
}

int kvq_decode_attend(const kvq_cache* cache, const void* q, int32_t batch, int32_t num_q_heads,
                      int32_t q_tokens, const int32_t* seq_lens, int32_t max_seq_len,
                      float softmax_scale, const float* head_sink, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (out == nullptr || !aligned16(out)) return KVQ_EINVAL;
  int st = split_impl(cache, q, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, softmax_scale,
                      nullptr, 0, workspace, workspace_bytes, stream);
  if (st != KVQ_OK) return st;
  return kvq_combine(cache, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, head_sink, out,
                     workspace, workspace_bytes, stream);
}

int kvq_paged_decode_attend(const kvq_cache* cache, const void* q, int32_t batch,
                            int32_t num_q_heads, int32_t q_tokens, const int32_t* seq_lens,
                            int32_t max_seq_len, float softmax_scale, const float* head_sink,
                            const int32_t* block_table, int32_t max_blocks, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (block_table == nullptr) return KVQ_EINVAL;
  if (out == nullptr || !aligned16(out)) return KVQ_EINVAL;
  int st = split_impl(cache, q, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, softmax_scale,
                      block_table, max_blocks, workspace, workspace_bytes, stream);
  if (st != KVQ_OK) return st;
  return kvq_combine(cache, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, head_sink, out,
                     workspace, workspace_bytes, stream);
}

int kvq_append_decode_attend(const kvq_cache* cache, const void* k_new, const void* v_new,
                             const void* q, int32_t batch, int32_t num_q_heads, int32_t q_tokens,
                             const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                             const float* head_sink, const int32_t* block_table,
                             int32_t max_blocks, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (k_new == nullptr || v_new == nullptr || !aligned16(k_new) || !aligned16(v_new))
    return KVQ_EINVAL;
  if (out == nullptr || !aligned16(out)) return KVQ_EINVAL;
  int st = split_impl(cache, q, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, softmax_scale,
                      block_table, max_blocks, workspace, workspace_bytes, stream, k_new, v_new);
  if (st != KVQ_OK) return st;
  return kvq_combine(cache, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, head_sink, out,
                     workspace, workspace_bytes, stream);
}

int kvq_attend_ex(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                  int32_t batch, int32_t num_q_heads, int32_t q_tokens, const int32_t* seq_lens,
                  int32_t max_seq_len, float softmax_scale, const float* head_sink,
                  const int32_t* block_table, int32_t max_blocks, const kvq_attn_options* options,
                  void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if ((k_new == nullptr) != (v_new == nullptr)) return KVQ_EINVAL;
  if (k_new != nullptr && (!aligned16(k_new) || !aligned16(v_new))) return KVQ_EINVAL;
  if (out == nullptr || !aligned16(out)) return KVQ_EINVAL;
  if (options != nullptr) {
    const float cap = options->softcap;
    if (!(cap >= 0.0f) || cap > 3.0e38f || options->window < 0) return KVQ_EINVAL;
  }
  int st = split_impl(cache, q, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, softmax_scale,
                      block_table, max_blocks, workspace, workspace_bytes, stream, k_new, v_new,
                      options);
  if (st != KVQ_OK) return st;
  return combine_impl(cache, batch, num_q_heads, q_tokens, seq_lens, max_seq_len, head_sink, out,
                      workspace, workspace_bytes, stream, options ? options->window : 0);
}

int kvq_attend_ex_noalloc(const kvq_cache* cache, const void* k_new, const void* v_new,
                          const void* q, int32_t batch, int32_t num_q_heads, int32_t q_tokens,
                          const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                          const float* head_sink, const int32_t* block_table, int32_t max_blocks,
                          const kvq_attn_options* options, void* out, void* stream) {
  // the shape's workspace must fit the scratch: checked on the host first
  DecodeShape sh;
  int st = decode_shape(cache, batch, num_q_heads, q_tokens, max_seq_len, &sh);
  if (st != KVQ_OK) return st;
  if (workspace_size(cache, batch, sh) > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ESCRATCH;
  void* ws = nullptr;
  st = scratch_for_stream(static_cast<hipStream_t>(stream), &ws);
  if (st != KVQ_OK) return st;
  return kvq_attend_ex(cache, k_new, v_new, q, batch, num_q_heads, q_tokens, seq_lens, max_seq_len,
                       softmax_scale, head_sink, block_table, max_blocks, options, out, ws,
                       KVQ_NOALLOC_SCRATCH_BYTES, stream);
}

int kvq_prefill_attend(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                       int32_t batch, int32_t num_q_heads, int32_t q_tokens, const int32_t* seq_lens,
                       int32_t max_seq_len, float softmax_scale, const float* head_sink,
                       const int32_t* block_table, int32_t max_blocks,
                       const kvq_attn_options* options, void* out, void* stream) {
  return prefill_impl(cache, k_new, v_new, q, batch, num_q_heads, q_tokens, seq_lens, max_seq_len,
                      softmax_scale, head_sink, block_table, max_blocks, options, out, nullptr, 0, false,
                      stream);
}

size_t kvq_prefill_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t num_q_heads,
                                   int32_t q_tokens, int32_t max_seq_len, const kvq_attn_options* options) {
  int G = 0;
  if (prefill_check(cache, batch, num_q_heads, q_tokens, max_seq_len, &G) != KVQ_OK) return 0;
  const int32_t window = options ? options->window : 0;
  const PrefillPlan plan = prefill_plan(cache, batch, G, q_tokens, max_seq_len, window, true);
  return prefill_workspace_size(cache, batch, G * q_tokens, plan.KS);
}

int kvq_prefill_attend_ws(const kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                          int32_t batch, int32_t num_q_heads, int32_t q_tokens, const int32_t* seq_lens,
                          int32_t max_seq_len, float softmax_scale, const float* head_sink,
                          const int32_t* block_table, int32_t max_blocks,
                          const kvq_attn_options* options, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return prefill_impl(cache, k_new, v_new, q, batch, num_q_heads, q_tokens, seq_lens, max_seq_len,
                      softmax_scale, head_sink, block_table, max_blocks, options, out, workspace,
                      workspace_bytes, true, stream);
}

size_t kvq_cache_bytes(int32_t dtype, int32_t scale_mode, int32_t num_kv_heads, int32_t head_dim,
                       int64_t tokens) {
  if (num_kv_heads < 1 || head_dim < 1 || tokens < 0) return 0;
  size_t row;
  switch (dtype) {
    case KVQ_INT8:
    case KVQ_FP8_E4M3FN: row = (size_t)head_dim; break;
    case KVQ_INT4: row = (size_t)(head_dim + 1) / 2; break;
    case KVQ_BF16:
      if (scale_mode != KVQ_NO_SCALE) return 0;
      return 2 * (size_t)num_kv_heads * (2 * (size_t)head_dim) * (size_t)tokens;
    default: return 0;
  }
  if (scale_mode == KVQ_PER_ROW)
    row += 4;
  else if (scale_mode != KVQ_PER_TENSOR && scale_mode != KVQ_PER_CHANNEL)
    return 0;
  return 2 * (size_t)num_kv_heads * row * (size_t)tokens;
}

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_EINVAL: return "KVQ_EINVAL: invalid argument";
    case KVQ_EUNSUPPORTED: return "KVQ_EUNSUPPORTED: unsupported shape or type";
    case KVQ_EHIP: return "KVQ_EHIP: HIP runtime error";
    case KVQ_ESCRATCH:
      return "KVQ_ESCRATCH: the call needs more workspace than the library's static scratch "
             "(KVQ_NOALLOC_SCRATCH_BYTES); pass a workspace to kvq_attend_ex instead";
    default: return "unknown kvq status";
  }
}

}  // extern "C"
