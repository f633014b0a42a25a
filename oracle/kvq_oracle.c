/*
 * kvq_oracle.c -- plain, slow, obviously-correct CPU oracle for quantized-KV
 * decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file's library: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or table with the HIP
 * library; the two see only the same seeded inputs.
 *
 * What it computes, and where the pages define it:
 *   - per-row absmax quantization on write: every K and V row gets its own
 *     scale when it is written; appending never touches earlier rows
 *     (kv-quant-attn page, "Method"; ORT issue "Feature request: quantized
 *     (int8/fp8) KV cache in GroupQueryAttention ...", "Motivation").
 *   - static per-tensor and per-channel scales (ORT PR "[CUDA] PagedAttention:
 *     quantized KV cache, XQA decode, MLA, QK-Norm and head sink", "Summary of
 *     Changes", the k_scale / v_scale inputs and k_quant_type / v_quant_type).
 *   - cache element types int8, float8e4m3fn (same PR, T_CACHE constraint) and
 *     signed int4 packed two per byte in uint8 ("[CUDA] Add INT4 paged KV cache
 *     with per-channel scales", opening description).
 *   - dequantize on read, then exact softmax attention with grouped-query heads
 *     (kv-quant-attn page, "Method" and "Correctness": the reference is fp32
 *     attention on the dequantized cache).
 *   - head sink: the output is rescaled by 1/(1+exp(s_h - lse)) (PagedAttention
 *     PR, "CUDA kernels", ApplyHeadSink).
 *   - an unquantized bf16 cache, the baseline the kernel page's crossover is
 *     measured against (kv-quant-attn page, "Performance"): its "codes" are the
 *     bf16 values themselves (two bytes, little-endian) and it has no scales.
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
 *   integer codes round half to even and clamp symmetrically to [-Qmax, Qmax]
 *   (Qmax 127 int8, 7 int4, 448 fp8); the code is computed from y = x / s with
 *   one IEEE fp32 division; s = 0 gives all-zero codes; fp8 encodes y with
 *   round-to-nearest-even and saturates to +-448; the even element of an int4
 *   pair sits in the low nibble; the dequantized value is float(c) * s with one
 *   fp32 multiply; query j of Tq sits at position len - Tq + j and sees tokens
 *   at or before it; a sequence with no visible token outputs zeros.
 *
 * Build: gcc -std=c11 -O2 -fopenmp -ffp-contract=off -fPIC -shared (no
 * -ffast-math: the quantizer depends on IEEE division and rint).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define KVO_INT8 1
#define KVO_INT4 2
#define KVO_FP8 3
#define KVO_BF16 4
#define KVO_PER_ROW 1
#define KVO_PER_TENSOR 2
#define KVO_PER_CHANNEL 3

/* ---------------------------------------------------------------- bf16 */

/* A bf16 value is the upper 16 bits of the fp32 with the same value. */
float kvo_bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* ------------------------------------------------- OCP FP8 E4M3FN codec */
/*
 * E4M3FN (the float8e4m3fn element type named by the PagedAttention PR):
 * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * the all-ones exponent-and-mantissa pattern (S.1111.111) is NaN, the largest
 * finite magnitude is 1.75 * 2^8 = 448, exponent field 0 holds subnormals
 * m * 2^-9.  This follows the OCP 8-bit floating point specification.
 */
double kvo_fp8_decode(uint8_t c) {
  int sign = c >> 7;
  int e = (c >> 3) & 0xF;
  int m = c & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Nearest E4M3FN value to the fp32 y, ties to even mantissa, |y| >= 448
 * saturates to 448.  The sign of y is kept, so a negative y that rounds to
 * zero encodes as 0x80.  y must not be NaN. */
uint8_t kvo_fp8_encode(float y) {
  int sign = signbit(y) ? 1 : 0;
  double a = fabs((double)y);
  int code;
  if (a >= 448.0) {
    code = 0x7E;
  } else if (a < ldexp(1.0, -6)) {
    /* subnormal grid: multiples of 2^-9; q == 8 is the smallest normal, whose
       code happens to be 8 as well */
    double q = rint(ldexp(a, 9));
    code = (int)q;
  } else {
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;         /* a in [2^e, 2^(e+1)) */
    double q = rint(ldexp(a, 3 - e)); /* in [8, 16] */
    if (q >= 16.0) {
      q = 8.0;
      e += 1;
    }
    code = ((e + 7) << 3) | ((int)q - 8);
  }
  return (uint8_t)(code | (sign << 7));
}

/* ------------------------------------------------------ row quantizer */

static float qmax_of(int dtype) {
  return dtype == KVO_INT8 ? 127.0f : dtype == KVO_INT4 ? 7.0f : 448.0f;
}

int kvo_row_bytes(int dtype, int D) {
  return dtype == KVO_INT4 ? D / 2 : dtype == KVO_BF16 ? 2 * D : D;
}

/* Code of one element from y = x / s. */
static int encode_int(float y, float qmax) {
  float r = rintf(y); /* round half to even (default rounding mode) */
  if (r > qmax) r = qmax;
  if (r < -qmax) r = -qmax;
  return (int)r;
}

/*
 * Quantize one row of D bf16 values.
 *   PER_ROW:     s = max_d |x_d| / Qmax (fp32 division), stored in *row_scale.
 *   PER_TENSOR:  s = static_scale[0] for every element.
 *   PER_CHANNEL: s_d = static_scale[d] (this KV head's table row).
 * Codes: int8 -> D bytes; fp8 -> D bytes; int4 -> D/2 bytes, element 2i in the
 * low nibble and 2i+1 in the high nibble, two's complement.
 * bf16 (unquantized): the 2D bytes of the input itself, element d at bytes
 * 2d (low) and 2d+1 (high); mode, scales and row_scale are not used.
 */
void kvo_quantize_row(const uint16_t* x, int D, int dtype, int mode, const float* static_scale,
                      uint8_t* codes, float* row_scale) {
  if (dtype == KVO_BF16) {
    for (int d = 0; d < D; ++d) {
      codes[2 * d] = (uint8_t)(x[d] & 0xFF);
      codes[2 * d + 1] = (uint8_t)(x[d] >> 8);
    }
    return;
  }
  float qmax = qmax_of(dtype);
  float s_row = 0.0f;
  if (mode == KVO_PER_ROW) {
    float a = 0.0f;
    for (int d = 0; d < D; ++d) {
      float v = fabsf(kvo_bf16_to_float(x[d]));
      if (v > a) a = v;
    }
    s_row = a / qmax;
    if (row_scale) *row_scale = s_row;
  }
  if (dtype == KVO_INT4) memset(codes, 0, (size_t)D / 2);
  for (int d = 0; d < D; ++d) {
    float s = mode == KVO_PER_ROW ? s_row : mode == KVO_PER_TENSOR ? static_scale[0] : static_scale[d];
    float xv = kvo_bf16_to_float(x[d]);
    if (dtype == KVO_FP8) {
      codes[d] = (s == 0.0f) ? 0 : kvo_fp8_encode(xv / s);
    } else {
      int c = (s == 0.0f) ? 0 : encode_int(xv / s, qmax);
      if (dtype == KVO_INT8) {
        codes[d] = (uint8_t)(int8_t)c;
      } else {
        uint8_t nib = (uint8_t)(c & 0xF);
        codes[d / 2] |= (d % 2 == 0) ? nib : (uint8_t)(nib << 4);
      }
    }
  }
}

/* Integer or fp8 value of element d of a code row (before scaling). */
static double code_value(const uint8_t* codes, int d, int dtype) {
  if (dtype == KVO_INT8) return (double)(int8_t)codes[d];
  if (dtype == KVO_FP8) return kvo_fp8_decode(codes[d]);
  uint8_t byte = codes[d / 2];
  int nib = (d % 2 == 0) ? (byte & 0xF) : (byte >> 4);
  return (double)(nib >= 8 ? nib - 16 : nib);
}

/* Dequantize one row: xhat_d = float(c_d) * s_d, one fp32 multiply.  A bf16
 * row is read back as its values (no scale). */
void kvo_dequantize_row(const uint8_t* codes, int D, int dtype, int mode, float row_scale,
                        const float* static_scale, float* out) {
  if (dtype == KVO_BF16) {
    for (int d = 0; d < D; ++d)
      out[d] = kvo_bf16_to_float((uint16_t)(codes[2 * d] | (codes[2 * d + 1] << 8)));
    return;
  }
  for (int d = 0; d < D; ++d) {
    float s = mode == KVO_PER_ROW ? row_scale : mode == KVO_PER_TENSOR ? static_scale[0] : static_scale[d];
    float c = (float)code_value(codes, d, dtype);
    out[d] = c * s;
  }
}

/* ------------------------------------------------------- cache layout */
/*
 * Codes:  [num_blocks, Hkv, block_size, row_bytes]
 * Scales: [num_blocks, Hkv, block_size] fp32 (PER_ROW only)
 * Token p of sequence b lives in block block_table[b * max_blocks + p / block_size]
 * (block b when block_table is NULL, the contiguous [B, Hkv, T, D] layout) at
 * row p % block_size.
 */
static size_t row_index(int b, int p, int h, int Hkv, int block_size, const int32_t* table,
                        int max_blocks) {
  int blk = table ? table[(size_t)b * max_blocks + p / block_size] : b;
  return ((size_t)blk * Hkv + h) * block_size + (size_t)(p % block_size);
}

/*
 * Append Tn new tokens per sequence: k, v are bf16 [B, Tn, Hkv, D]; token j of
 * sequence b is written at position positions[b] + j.  Only those rows (and
 * their scales) are written.  K rows use k_mode, V rows v_mode ([P]: separate
 * k_scale and v_scale inputs, each per-tensor or per-channel).
 */
void kvo_append(int dtype, int k_mode, int v_mode, int Hkv, int D, int block_size, uint8_t* k_codes,
                uint8_t* v_codes, float* k_scales, float* v_scales, const float* k_static,
                const float* v_static, const uint16_t* k, const uint16_t* v, int B, int Tn,
                const int32_t* positions, const int32_t* block_table, int max_blocks) {
  int rb = kvo_row_bytes(dtype, D);
  for (int b = 0; b < B; ++b)
    for (int j = 0; j < Tn; ++j)
      for (int h = 0; h < Hkv; ++h) {
        int p = positions[b] + j;
        size_t ri = row_index(b, p, h, Hkv, block_size, block_table, max_blocks);
        size_t xi = (((size_t)b * Tn + j) * Hkv + h) * (size_t)D;
        const float* ks = k_mode == KVO_PER_CHANNEL ? k_static + (size_t)h * D : k_static;
        const float* vs = v_mode == KVO_PER_CHANNEL ? v_static + (size_t)h * D : v_static;
        kvo_quantize_row(k + xi, D, dtype, k_mode, ks, k_codes + ri * rb,
                         k_mode == KVO_PER_ROW ? k_scales + ri : NULL);
        kvo_quantize_row(v + xi, D, dtype, v_mode, vs, v_codes + ri * rb,
                         v_mode == KVO_PER_ROW ? v_scales + ri : NULL);
      }
}

/*
 * Materialize the dequantized cache of every sequence as dense fp32
 * [B, Hkv, Lmax, D] (positions >= lens[b] are left as zero).
 */
void kvo_dequantize(int dtype, int k_mode, int v_mode, int Hkv, int D, int block_size,
                    const uint8_t* k_codes,
                    const uint8_t* v_codes, const float* k_scales, const float* v_scales,
                    const float* k_static, const float* v_static, int B, const int32_t* lens,
                    const int32_t* block_table, int max_blocks, int Lmax, float* k_out,
                    float* v_out) {
  int rb = kvo_row_bytes(dtype, D);
  memset(k_out, 0, sizeof(float) * (size_t)B * Hkv * Lmax * D);
  memset(v_out, 0, sizeof(float) * (size_t)B * Hkv * Lmax * D);
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hkv; ++h)
      for (int p = 0; p < lens[b]; ++p) {
        size_t ri = row_index(b, p, h, Hkv, block_size, block_table, max_blocks);
        size_t oi = (((size_t)b * Hkv + h) * Lmax + p) * (size_t)D;
        const float* ks = k_mode == KVO_PER_CHANNEL ? k_static + (size_t)h * D : k_static;
        const float* vs = v_mode == KVO_PER_CHANNEL ? v_static + (size_t)h * D : v_static;
        kvo_dequantize_row(k_codes + ri * rb, D, dtype, k_mode,
                           k_mode == KVO_PER_ROW ? k_scales[ri] : 0.0f, ks, k_out + oi);
        kvo_dequantize_row(v_codes + ri * rb, D, dtype, v_mode,
                           v_mode == KVO_PER_ROW ? v_scales[ri] : 0.0f, vs, v_out + oi);
      }
}

/*
 * Exact softmax attention in fp64 over a dense cache.
 *   q     bf16 [B, Tq, Hq, D]
 *   K, V  fp32 [B, Hkv, Lmax, D]
 *   query head h reads KV head h / (Hq / Hkv)
 *   query j of sequence b sits at pos = lens[b] - Tq + j and sees t <= pos, t < lens[b]
 *   z_t = scale * sum_d q_d K_td; o = sum_t softmax(z)_t V_t; lse = log sum_t exp(z_t)
 *   sink (if given, [Hq] fp32): o *= 1 / (1 + exp(sink[h] - lse))
 *   no visible token: o = 0 and lse = -inf
 * out fp64 [B, Tq, Hq, D]; lse_out fp64 [B, Tq, Hq] (may be NULL); m_out fp64
 * [B, Tq, Hq], the largest logit of each row (may be NULL; -inf with no
 * visible token), so that lse - m = ln of the row's normalizer.
 */
/* Logit of query row qd against key row k: z = scale * q . k, then, with a
 * soft cap c > 0, z -> c * tanh(z / c) ([P] "CUDA kernels": the paged decode
 * kernel takes a softcap; the cap applies to the scaled attention logits). */
static double kvo_logit(const double* qd, const float* k, int D, float scale, float softcap) {
  double z = 0.0;
  for (int d = 0; d < D; ++d) z += qd[d] * (double)k[d];
  z *= (double)scale;
  if (softcap > 0.0f) z = (double)softcap * tanh(z / (double)softcap);
  return z;
}

/* fp64 softmax attention over the dequantized cache, with GQA (query head h
 * reads KV head h / (Hq / Hkv)), causal speculative drafts (query j of
 * sequence b sits at position lens[b] - Tq + j and sees tokens at or before it),
 * an optional sliding window (window > 0: only tokens pos - window + 1 .. pos;
 * [P] "CUDA kernels": sliding-window decode), an optional logit soft cap and an
 * optional per-head sink (o *= 1 / (1 + exp(sink[h] - lse)), [P] ApplyHeadSink).
 * A query with no visible token outputs zeros. */
void kvo_attend_ex2(const uint16_t* q, const float* K, const float* V, int B, int Tq, int Hq, int Hkv,
                    int D, int Lmax, const int32_t* lens, float scale, const float* sink,
                    float softcap, int window, double* out, double* lse_out, double* m_out) {
  int G = Hq / Hkv;
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int j = 0; j < Tq; ++j)
      for (int h = 0; h < Hq; ++h) {
        int hk = h / G;
        size_t qi = (((size_t)b * Tq + j) * Hq + h) * (size_t)D;
        double* o = out + qi;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        int pos = lens[b] - Tq + j;
        int hi = pos + 1 < lens[b] ? pos + 1 : lens[b]; /* tokens [lo, hi) are visible */
        int lo = window > 0 ? pos - window + 1 : 0;
        if (lo < 0) lo = 0;
        if (hi <= lo) {
          if (lse_out) lse_out[((size_t)b * Tq + j) * Hq + h] = -INFINITY;
          if (m_out) m_out[((size_t)b * Tq + j) * Hq + h] = -INFINITY;
          continue;
        }
        const float* Kb = K + ((size_t)b * Hkv + hk) * Lmax * (size_t)D;
        const float* Vb = V + ((size_t)b * Hkv + hk) * Lmax * (size_t)D;
        double qd[512];
        for (int d = 0; d < D; ++d) qd[d] = (double)kvo_bf16_to_float(q[qi + d]);
        double m = -INFINITY;
        /* pass 1: max logit */
        for (int t = lo; t < hi; ++t) {
          double z = kvo_logit(qd, Kb + (size_t)t * D, D, scale, softcap);
          if (z > m) m = z;
        }
        /* pass 2: normalizer and weighted sum of V */
        double l = 0.0;
        for (int t = lo; t < hi; ++t) {
          double p = exp(kvo_logit(qd, Kb + (size_t)t * D, D, scale, softcap) - m);
          l += p;
          for (int d = 0; d < D; ++d) o[d] += p * (double)Vb[(size_t)t * D + d];
        }
        for (int d = 0; d < D; ++d) o[d] /= l;
        double lse = m + log(l);
        if (sink) {
          double f = 1.0 / (1.0 + exp((double)sink[h] - lse));
          for (int d = 0; d < D; ++d) o[d] *= f;
        }
        if (lse_out) lse_out[((size_t)b * Tq + j) * Hq + h] = lse;
        if (m_out) m_out[((size_t)b * Tq + j) * Hq + h] = m;
      }
}

/* The same without the largest logit of each row. */
void kvo_attend_ex(const uint16_t* q, const float* K, const float* V, int B, int Tq, int Hq, int Hkv,
                   int D, int Lmax, const int32_t* lens, float scale, const float* sink,
                   float softcap, int window, double* out, double* lse_out) {
  kvo_attend_ex2(q, K, V, B, Tq, Hq, Hkv, D, Lmax, lens, scale, sink, softcap, window, out, lse_out,
                 NULL);
}

/* The same without soft cap or window. */
void kvo_attend(const uint16_t* q, const float* K, const float* V, int B, int Tq, int Hq, int Hkv,
                int D, int Lmax, const int32_t* lens, float scale, const float* sink, double* out,
                double* lse_out) {
  kvo_attend_ex(q, K, V, B, Tq, Hq, Hkv, D, Lmax, lens, scale, sink, 0.0f, 0, out, lse_out);
}

/* Bytes of cache one token occupies across `layers` layers: K and V rows of
 * every KV head at `bits` bits per element, plus one fp32 scale per row when
 * scales are per row (static per-tensor / per-channel tables are per layer,
 * not per token).  bits = 16 is the unquantized bf16 cache. */
double kvo_cache_bytes_per_token(int bits, int per_row_scales, int layers, int Hkv, int D) {
  double row = (double)D * bits / 8.0 + (per_row_scales ? 4.0 : 0.0);
  return 2.0 * layers * Hkv * row;
}

/* Threads the OpenMP loops above use (for reporting the CPU baseline). */
#ifdef _OPENMP
#include <omp.h>
#endif
int kvo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Run the OpenMP loops above on n threads from now on (timing the baseline on
 * one core and on all of them). */
void kvo_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
