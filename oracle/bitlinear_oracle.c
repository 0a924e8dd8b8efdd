/*
 * CPU oracle for the BitNet b1.58 BitLinear forward.  TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, scalar C11.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product path never does.  It shares
 * no source with the HIP library (no headers, no tables, no helpers).
 *
 * Sources (cited by page and section; the pages are the method's only definition):
 *   [AT]  aratech.ae, "BitNet b1.58: Microsoft's 1-bit LLM that runs a 100B model on
 *         one CPU" (Arabic), section "The solution: BitNet b1.58 - an architecture
 *         designed for ternary weights", sub-sections "Ternary weights {-1, 0, +1}"
 *         (absmean scale, clamp(round(W x scale))) and "BitLinear: the building block"
 *         (per-token absmax int8 activations, largest magnitude -> 127).
 *   [BH]  bhfrc.com news 56965 (Traditional Chinese, BitNet b1.58 on Windows),
 *         section 1.1 (a ternary weight times an activation is add / subtract / skip)
 *         and section 4.1 (2-bit code table 00 -> 0, 01 -> +1, 10 -> -1, 11 -> padding).
 *
 * Numeric conventions (the readings these functions follow):
 *   - The ternarise decision is taken in fp32, as the kernel takes it:
 *     t = fl32(W * s_w) with s_w = fl32(1 / gamma); q = clamp(rint(t), -1, 1) with
 *     round-half-to-even.  gamma is the exact mean: orc_abs_sum_fixed forms the exact sum
 *     of |W|, and the caller divides by the count and rounds once to fp32.
 *   - Activation quantisation per row: a = max |x| (exact), s = fl32(127 / a),
 *     xq = clamp(rint(fl32(x * s)), -127, 127); a row of zeros gives xq = 0.
 *   - Contraction is exact integer arithmetic (int64, checked to fit int32).
 *   - Rescale y = acc * gamma * a / 127 is evaluated in fp64.
 *
 * Packed layout (a choice; the pages give only the code table):
 *   Rows are padded to N_pad = roundup(N, 16), columns to K_pad = roundup(K, 256).
 *   The matrix is a sequence of 1024-byte tiles, tile (nb, c) at byte offset
 *   (nb * (K_pad / 256) + c) * 1024, covering rows 16*nb .. 16*nb+15 and columns
 *   256*c .. 256*c+255.  Inside a tile, row r (0..15) and column offset kk (0..255):
 *       g = kk / 64, i = (kk % 64) / 16, f = (kk % 16) / 4, b = kk % 4
 *       32-bit little-endian word at byte offset 16 * (16 * g + r) + 4 * i,
 *       code in bits [8 * b + 2 * f, 8 * b + 2 * f + 1].
 *   Entries outside N x K hold the padding code 3 (binary 11).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_RANGE -1

int64_t orc_n_pad(int64_t n) { return (n + 15) / 16 * 16; }
int64_t orc_k_pad(int64_t k) { return (k + 255) / 256 * 256; }
int64_t orc_packed_bytes(int64_t n, int64_t k) { return orc_n_pad(n) * orc_k_pad(k) / 4; }

/* [AT] "Ternary weights {-1, 0, +1}": gamma is the mean magnitude taken over the whole
 * weight tensor.  This forms the sum of |w| exactly.  Every finite fp32 is an integer
 * multiple of 2^-149, so the sum is an integer in those units; it is kept in a plain
 * fixed-point accumulator of ORC_SUM_LIMBS 32-bit limbs, least significant first.  A
 * weight with exponent field e and 23-bit fraction f is sig * 2^(e - 150) with
 * sig = f + 2^23 (e >= 1), or f * 2^-149 (e = 0, subnormal): in units of 2^-149 that is
 * sig shifted left by max(e, 1) - 1 bits.  Each weight is added on its own, in index
 * order.  352 bits hold 2^40 weights of the largest fp32 (2^40 * 2^128 * 2^149 < 2^318).
 * Returns ORC_ERR_RANGE for a non-finite weight or more than 2^40 of them.  The division
 * by the count and the rounding to fp32 are done on the exact integer by the caller. */
#define ORC_SUM_LIMBS 11
int orc_sum_limbs(void) { return ORC_SUM_LIMBS; }

int orc_abs_sum_fixed(const float* w, int64_t count, uint32_t* limbs) {
  for (int i = 0; i < ORC_SUM_LIMBS; ++i) limbs[i] = 0;
  if (count < 0 || count > ((int64_t)1 << 40)) return ORC_ERR_RANGE;
  for (int64_t i = 0; i < count; ++i) {
    uint32_t bits;
    memcpy(&bits, &w[i], 4);
    bits &= 0x7FFFFFFFu; /* |w| */
    const uint32_t e = bits >> 23, f = bits & 0x7FFFFFu;
    if (e == 255u) return ORC_ERR_RANGE;
    const uint64_t sig = e ? (uint64_t)f | (1u << 23) : (uint64_t)f;
    const uint32_t shift = e ? e - 1u : 0u; /* 0 .. 253 */
    int li = (int)(shift / 32u);
    uint64_t add = sig << (shift % 32u); /* at most 55 bits */
    while (add != 0 && li < ORC_SUM_LIMBS) {
      const uint64_t s = (uint64_t)limbs[li] + (add & 0xFFFFFFFFu);
      limbs[li] = (uint32_t)s;
      add = (add >> 32) + (s >> 32); /* carry into the next limb */
      ++li;
    }
  }
  return ORC_OK;
}

/* [AT] "Ternary weights": scale_w is the reciprocal of the mean magnitude; each
 * weight is multiplied by it, rounded, and clamped to [-1, 1].  gamma == 0 (an
 * all-zero tensor) yields all-zero codes without dividing. */
void orc_ternarise(const float* w, int64_t count, float gamma, int8_t* q) {
  if (gamma == 0.0f) {
    for (int64_t i = 0; i < count; ++i) q[i] = 0;
    return;
  }
  const float s_w = 1.0f / gamma; /* may be +inf when gamma < 2^-128 */
  for (int64_t i = 0; i < count; ++i) {
    if (w[i] == 0.0f) { /* a zero weight is code 0 at any scale (avoids 0 * inf) */
      q[i] = 0;
      continue;
    }
    const float t = w[i] * s_w;
    float r = rintf(t); /* current rounding mode: round-half-to-even */
    if (r > 1.0f) r = 1.0f;
    if (r < -1.0f) r = -1.0f;
    q[i] = (int8_t)r;
  }
}

/* Byte offset of the word and the bit position that hold code (n, k). */
static void orc_code_position(int64_t n, int64_t k, int64_t k_pad, int64_t* byte_off, int* bit) {
  const int64_t nb = n / 16, r = n % 16;
  const int64_t c = k / 256, kk = k % 256;
  const int64_t g = kk / 64, i = (kk % 64) / 16, f = (kk % 16) / 4, b = kk % 4;
  const int64_t tile = nb * (k_pad / 256) + c;
  *byte_off = tile * 1024 + 16 * (16 * g + r) + 4 * i;
  *bit = (int)(8 * b + 2 * f);
}

/* [BH] section 4.1 code table: 0 -> 00, +1 -> 01, -1 -> 10, padding -> 11.
 * q is [N][K] row-major with values in {-1, 0, 1}. */
int orc_pack(const int8_t* q, int64_t n_rows, int64_t k_cols, uint8_t* packed) {
  const int64_t np = orc_n_pad(n_rows), kp = orc_k_pad(k_cols);
  for (int64_t n = 0; n < np; ++n) {
    for (int64_t k = 0; k < kp; ++k) {
      uint32_t code = 3u;
      if (n < n_rows && k < k_cols) {
        const int8_t v = q[n * k_cols + k];
        if (v == 0) code = 0u;
        else if (v == 1) code = 1u;
        else if (v == -1) code = 2u;
        else return ORC_ERR_RANGE;
      }
      int64_t off;
      int bit;
      orc_code_position(n, k, kp, &off, &bit);
      uint32_t word;
      memcpy(&word, packed + off, 4); /* host is little-endian (x86-64) */
      word &= ~(3u << bit);
      word |= code << bit;
      memcpy(packed + off, &word, 4);
    }
  }
  return ORC_OK;
}

/* Inverse of orc_pack over the full padded grid: codes[N_pad][K_pad] in {0,1,2,3}. */
void orc_unpack_codes(const uint8_t* packed, int64_t n_rows, int64_t k_cols, uint8_t* codes) {
  const int64_t np = orc_n_pad(n_rows), kp = orc_k_pad(k_cols);
  for (int64_t n = 0; n < np; ++n) {
    for (int64_t k = 0; k < kp; ++k) {
      int64_t off;
      int bit;
      orc_code_position(n, k, kp, &off, &bit);
      uint32_t word;
      memcpy(&word, packed + off, 4);
      codes[n * kp + k] = (uint8_t)((word >> bit) & 3u);
    }
  }
}

/* Codes -> ternary values of the N x K matrix; returns ORC_ERR_RANGE if a code
 * inside the matrix is the padding code. */
int orc_unpack(const uint8_t* packed, int64_t n_rows, int64_t k_cols, int8_t* q) {
  const int64_t kp = orc_k_pad(k_cols);
  for (int64_t n = 0; n < n_rows; ++n) {
    for (int64_t k = 0; k < k_cols; ++k) {
      int64_t off;
      int bit;
      orc_code_position(n, k, kp, &off, &bit);
      uint32_t word;
      memcpy(&word, packed + off, 4);
      const uint32_t code = (word >> bit) & 3u;
      if (code == 3u) return ORC_ERR_RANGE;
      q[n * k_cols + k] = code == 0u ? 0 : (code == 1u ? 1 : -1);
    }
  }
  return ORC_OK;
}

/* bf16 -> fp32 widening is exact: the bf16 bits are the top half of the fp32. */
void orc_bf16_to_f32(const uint16_t* in, int64_t count, float* out) {
  for (int64_t i = 0; i < count; ++i) {
    const uint32_t bits = (uint32_t)in[i] << 16;
    memcpy(&out[i], &bits, 4);
  }
}

/* [AT] "BitLinear": per token (row), the largest magnitude maps to 127.
 * xq is [M][K_pad] with zeros in the padding columns; absmax[m] = max_k |x[m][k]|. */
void orc_quant_acts(const float* x, int64_t m_rows, int64_t k_cols, int8_t* xq, float* absmax) {
  const int64_t kp = orc_k_pad(k_cols);
  for (int64_t m = 0; m < m_rows; ++m) {
    const float* row = x + m * k_cols;
    float a = 0.0f;
    for (int64_t k = 0; k < k_cols; ++k) {
      const float v = fabsf(row[k]);
      if (v > a) a = v;
    }
    absmax[m] = a;
    int8_t* out = xq + m * kp;
    for (int64_t k = 0; k < kp; ++k) out[k] = 0;
    if (a == 0.0f) continue;
    const float s = 127.0f / a;
    for (int64_t k = 0; k < k_cols; ++k) {
      float r = rintf(row[k] * s);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      out[k] = (int8_t)r;
    }
  }
}

/* [AT] "BitLinear: the building block": a sub-layer normalisation (a simplified
 * LayerNorm) sits just before the activation quantiser.  Reading: RMS normalisation,
 * no centring and no bias, with a per-feature gain g (NULL: all ones) and eps >= 0,
 *     n[k] = x[k] * g[k] / sqrt(sum_k x[k]^2 / K + eps),
 * then the per-token absmax quantiser on n.  The factor 1/sqrt(...) is one positive
 * number per row, and absmax quantisation maps a row and any positive multiple of it to
 * the same codes (the factor divides out of n[k] * 127 / max|n|).  So the codes are
 * taken on h[k] = fl32(x[k] * g[k]) with exactly the arithmetic of orc_quant_acts, and
 * the factor goes into the scale:
 *     scale[m] = max_k |h[k]| / sqrt(sum_k x[k]^2 / K + eps)     (= max_k |n[k]|)
 * in fp64 (each x^2 is exact in fp64; the sum is in index order).  h_absmax[m] is
 * max_k |h[k]|; a row whose h is all zero gives zero codes and scale 0. */
void orc_subln_quant_acts(const float* x, int64_t m_rows, int64_t k_cols, const float* gain, double eps,
                          int8_t* xq, float* h_absmax, double* scale) {
  const int64_t kp = orc_k_pad(k_cols);
  float* h = (float*)malloc((size_t)(k_cols > 0 ? k_cols : 1) * sizeof(float));
  for (int64_t m = 0; m < m_rows; ++m) {
    const float* row = x + m * k_cols;
    double ss = 0.0;
    for (int64_t k = 0; k < k_cols; ++k) {
      ss += (double)row[k] * (double)row[k];
      h[k] = gain ? row[k] * gain[k] : row[k];
    }
    orc_quant_acts(h, 1, k_cols, xq + m * kp, &h_absmax[m]);
    scale[m] = h_absmax[m] == 0.0f ? 0.0 : (double)h_absmax[m] / sqrt(ss / (double)k_cols + eps);
  }
  free(h);
}

/* [BH] section 1.1: each term is +x, -x or nothing; the sum is exact in integers.
 * q is [N][K] (ternary), xq is [M][ldx]; acc is [M][N].  Returns ORC_ERR_RANGE if
 * a sum does not fit int32. */
int orc_matmul(const int8_t* q, const int8_t* xq, int64_t m_rows, int64_t n_rows,
               int64_t k_cols, int64_t ldx, int32_t* acc) {
  for (int64_t m = 0; m < m_rows; ++m) {
    for (int64_t n = 0; n < n_rows; ++n) {
      int64_t s = 0;
      for (int64_t k = 0; k < k_cols; ++k) s += (int64_t)xq[m * ldx + k] * (int64_t)q[n * k_cols + k];
      if (s > INT32_MAX || s < INT32_MIN) return ORC_ERR_RANGE;
      acc[m * n_rows + n] = (int32_t)s;
    }
  }
  return ORC_OK;
}

/* Undo both scales: weights were divided by gamma, activations multiplied by 127/a. */
void orc_rescale(const int32_t* acc, int64_t m_rows, int64_t n_rows, float gamma,
                 const float* absmax, double* y) {
  for (int64_t m = 0; m < m_rows; ++m)
    for (int64_t n = 0; n < n_rows; ++n)
      y[m * n_rows + n] = (double)acc[m * n_rows + n] * (double)gamma * (double)absmax[m] / 127.0;
}

/* [AT] "BitLinear: the building block": the feed-forward layers use the squared ReLU
 * activation.  Reading for a gate / up pair of BitLinear projections of one input:
 * h = relu(y_gate)^2 * y_up, elementwise, in fp64 on the fp64 outputs of orc_rescale. */
void orc_gated_relu2(const double* y_gate, const double* y_up, int64_t count, double* h) {
  for (int64_t i = 0; i < count; ++i) {
    const double r = y_gate[i] > 0.0 ? y_gate[i] : 0.0;
    h[i] = r * r * y_up[i];
  }
}

/* ---- 1-bit sign-binary variant (contrast point) -------------------------------------
 * lpnh.cn news 2861808, section 2.1: binary weights sign(W) with a scaling factor that
 * compensates the lost magnitude.  Readings: q = +1 for W >= 0 (also -0.0), -1 for
 * W < 0 (a 1-bit code has no zero); the scale beta is the same exact mean |W| as gamma.
 *
 * Packed layout of the binary variant (a choice): N_pad = roundup(N, 16), KB_pad =
 * roundup(K, 512); 1024-byte tiles, tile (nb, c) at (nb * (KB_pad / 512) + c) * 1024,
 * rows 16 nb .. 16 nb + 15, columns 512 c .. 512 c + 511.  Inside a tile, row r and column
 * offset kk: s = kk / 256, g = (kk % 256) / 64, i = (kk % 64) / 16, e = kk % 16; the
 * 32-bit little-endian word at byte 16 * (16 g + r) + 4 * (2 s + i / 2) holds the bit at
 * position 8 * (e % 4) + 4 * (i % 2) + e / 4; bit 1 = +1, bit 0 = -1.  Bits outside N x K
 * are 0. */
int64_t orc_kb_pad(int64_t k) { return (k + 511) / 512 * 512; }
int64_t orc_packed_bytes_binary(int64_t n, int64_t k) { return orc_n_pad(n) * orc_kb_pad(k) / 8; }

void orc_binarise(const float* w, int64_t count, int8_t* q) {
  for (int64_t i = 0; i < count; ++i) q[i] = w[i] < 0.0f ? -1 : 1;
}

static void orc_bin_position(int64_t n, int64_t k, int64_t kbp, int64_t* off, int* bit) {
  const int64_t nb = n / 16, r = n % 16, c = k / 512, kk = k % 512;
  const int64_t s = kk / 256, g = (kk % 256) / 64, i = (kk % 64) / 16, e = kk % 16;
  *off = (nb * (kbp / 512) + c) * 1024 + 16 * (16 * g + r) + 4 * (2 * s + i / 2);
  *bit = (int)(8 * (e % 4) + 4 * (i % 2) + e / 4);
}

int orc_pack_binary(const int8_t* q, int64_t n_rows, int64_t k_cols, uint8_t* packed) {
  const int64_t kbp = orc_kb_pad(k_cols);
  memset(packed, 0, (size_t)orc_packed_bytes_binary(n_rows, k_cols));
  for (int64_t n = 0; n < n_rows; ++n) {
    for (int64_t k = 0; k < k_cols; ++k) {
      const int8_t v = q[n * k_cols + k];
      if (v != 1 && v != -1) return ORC_ERR_RANGE;
      if (v == 1) {
        int64_t off;
        int bit;
        orc_bin_position(n, k, kbp, &off, &bit);
        uint32_t word;
        memcpy(&word, packed + off, 4);
        word |= 1u << bit;
        memcpy(packed + off, &word, 4);
      }
    }
  }
  return ORC_OK;
}

void orc_unpack_binary(const uint8_t* packed, int64_t n_rows, int64_t k_cols, int8_t* q) {
  const int64_t kbp = orc_kb_pad(k_cols);
  for (int64_t n = 0; n < n_rows; ++n) {
    for (int64_t k = 0; k < k_cols; ++k) {
      int64_t off;
      int bit;
      orc_bin_position(n, k, kbp, &off, &bit);
      uint32_t word;
      memcpy(&word, packed + off, 4);
      q[n * k_cols + k] = ((word >> bit) & 1u) ? 1 : -1;
    }
  }
}
