/*
 * qmv_oracle.c -- plain, slow CPU oracle for the quantized decode matvec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no code, header or table with
 * the HIP path: it has its own fp16 decoder, its own block decoders and its own
 * copy of the IQ4_XS codebook.
 *
 * What it computes (Castagna Veloce page, "Kernels for the MI50" and "Fused
 * operations"; zhuai.tech GLM-5.3 page, "A single decode row is not a large
 * matrix multiplication"): y[t][n] = sum_k W[n][k] x[t][k] for 1..16 decode or
 * verify tokens, with W stored in GGUF block formats (Q8_0, q4_K, IQ4_XS) and
 * the activations quantized once to Q8 blocks of 32 that every weight type
 * reuses.  The pages name the formats but print no layout, no quantization rule
 * and no worked example; the readings taken here are:
 *
 *   - block layouts: the GGUF ones (Q8_0 34 B, q4_K 144 B, IQ4_XS 136 B);
 *   - activation block of 32: amax = max|x|, d = amax / 127 (fp32, correctly
 *     rounded), q = round-half-away-from-zero(x / d) (fp32 division) clamped to
 *     [-127, 127], s = sum of q; an all-zero block has d = 0 and q = 0;
 *   - q4_K weight  = d * sc_j * q - dmin * m_j   (the min is subtracted);
 *   - IQ4_XS weight = d * (ls_j - 32) * CB[idx]  (raw 6-bit scale minus 32);
 *   - q5_K (176 B): the q4_K header (d, dmin, the same 12 bytes of 6-bit
 *     scale/min pairs), then 32 bytes qh, then the 128 nibble bytes in the
 *     q4_K order; weight 64c + i of chunk c takes bit 2c of qh[i] as its
 *     fifth bit (value 16), weight 64c + 32 + i bit 2c + 1;
 *     q5_K weight = d * sc_j * q - dmin * m_j with q in 0..31;
 *   - q6_K (210 B): 128 B ql, 64 B qh, 16 int8 scales, fp16 d; weight
 *     128h + 32j + l (half h, quarter j, l < 32) stores the 6-bit value
 *     q = (nibble of ql[64h + 32(j & 1) + l], low for j < 2, high otherwise)
 *         + 16 * (bits 2j..2j+1 of qh[32h + l]),
 *     and weight i of the super-block is d * scales[i / 16] * (q - 32).
 *     Its integer partial per 32-block is P = sum_i scales[i/16] (q_i - 32) qx_i;
 *   - Q8G128 (130 B): fp16 d, int8 q[128]: weight = d * q for a group of 128
 *     (the int8 LM-head format the zhuai.tech page names, read as Q8_0 with
 *     128-weight groups); its 32-blocks dot like Q8_0 and share the group's d.
 *
 * Per 32-weight block b the integer partials are
 *   Q8_0  : P = sum_i qw_i qx_i
 *   q4_K  : A = sc_j * sum_i q_i qx_i,  B = m_j * s_b
 *   IQ4_XS: P = (ls_j - 32) * sum_i CB[idx_i] qx_i
 * and the fp64 terms tau are d_w dx P (Q8_0, IQ4_XS) or d dx A and -dmin dx B
 * (q4_K); y is their sum and mag the sum of their absolute values.
 * Floating point here is IEEE fp64 (terms) and fp32 (activation quantization);
 * build without fast-math and without FP contraction.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { FMT_Q8_0 = 0, FMT_Q4_K = 1, FMT_IQ4_XS = 2, FMT_Q5_K = 3, FMT_Q6_K = 4, FMT_Q8G128 = 5 };

/* K-quants with a per-sub-block min (q4_K, q5_K): two terms per block. */
static int has_min(int fmt) { return fmt == FMT_Q4_K || fmt == FMT_Q5_K; }

/* The 16-entry non-linear int8 codebook of IQ4_XS (shared with IQ4_NL). */
static const int IQ4_CODEBOOK[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                     1,    13,   25,  38,  53,  69,  89,  113};

/* IEEE binary16 -> double, written out from the format definition. */
static double half_to_double(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int64_t oracle_row_bytes(int fmt, int64_t k) {
  switch (fmt) {
    case FMT_Q8_0: return k % 32 ? -1 : (k / 32) * 34;
    case FMT_Q4_K: return k % 256 ? -1 : (k / 256) * 144;
    case FMT_IQ4_XS: return k % 256 ? -1 : (k / 256) * 136;
    case FMT_Q5_K: return k % 256 ? -1 : (k / 256) * 176;
    case FMT_Q6_K: return k % 256 ? -1 : (k / 256) * 210;
    case FMT_Q8G128: return k % 128 ? -1 : (k / 128) * 130;
    default: return -1;
  }
}

/* ------------------------------------------------------------ block decoders */
typedef struct { double d; int q[32]; } q8_0_block;
typedef struct { double d, dmin; int sc[8], m[8], q[256]; } q4_k_block;
typedef struct { double d; int ls[8], idx[256]; } iq4_xs_block;
typedef struct { double d; int sc[16], q[256]; } q6_k_block;  /* q: stored 0..63 */
typedef struct { double d; int q[128]; } q8g128_block;

static void decode_q8g128(const uint8_t* b, q8g128_block* o) {
  o->d = half_to_double(rd16(b));
  for (int i = 0; i < 128; ++i) o->q[i] = (int8_t)b[2 + i];
}

static void decode_q8_0(const uint8_t* b, q8_0_block* o) {
  o->d = half_to_double(rd16(b));
  for (int i = 0; i < 32; ++i) o->q[i] = (int8_t)b[2 + i];
}

/* The 16-byte header shared by q4_K and q5_K: fp16 d, fp16 dmin and the 8
 * packed 6-bit (scale, min) pairs. */
static void decode_kmin_header(const uint8_t* b, q4_k_block* o) {
  o->d = half_to_double(rd16(b));
  o->dmin = half_to_double(rd16(b + 2));
  const uint8_t* S = b + 4;
  for (int j = 0; j < 4; ++j) {
    o->sc[j] = S[j] & 63;
    o->m[j] = S[j + 4] & 63;
  }
  for (int j = 4; j < 8; ++j) {
    o->sc[j] = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
    o->m[j] = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
  }
}

static void decode_q4_k(const uint8_t* b, q4_k_block* o) {
  decode_kmin_header(b, o);
  const uint8_t* Q = b + 16;
  for (int c = 0; c < 4; ++c)
    for (int i = 0; i < 32; ++i) {
      o->q[64 * c + i] = Q[32 * c + i] & 15;
      o->q[64 * c + 32 + i] = Q[32 * c + i] >> 4;
    }
}

/* q5_K: the q4_K nibbles plus a fifth bit per weight from the qh bytes. */
static void decode_q5_k(const uint8_t* b, q4_k_block* o) {
  decode_kmin_header(b, o);
  const uint8_t* H = b + 16;
  const uint8_t* Q = b + 48;
  for (int c = 0; c < 4; ++c)
    for (int i = 0; i < 32; ++i) {
      int lo = Q[32 * c + i] & 15, hi = Q[32 * c + i] >> 4;
      o->q[64 * c + i] = lo + 16 * ((H[i] >> (2 * c)) & 1);
      o->q[64 * c + 32 + i] = hi + 16 * ((H[i] >> (2 * c + 1)) & 1);
    }
}

static void decode_q6_k(const uint8_t* b, q6_k_block* o) {
  const uint8_t* L = b;
  const uint8_t* H = b + 128;
  for (int i = 0; i < 16; ++i) o->sc[i] = (int8_t)b[192 + i];
  o->d = half_to_double(rd16(b + 208));
  for (int h = 0; h < 2; ++h)
    for (int j = 0; j < 4; ++j)
      for (int l = 0; l < 32; ++l) {
        int nib = (L[64 * h + 32 * (j & 1) + l] >> (4 * (j >> 1))) & 15;
        int two = (H[32 * h + l] >> (2 * j)) & 3;
        o->q[128 * h + 32 * j + l] = nib + 16 * two;
      }
}

static void decode_iq4_xs(const uint8_t* b, iq4_xs_block* o) {
  o->d = half_to_double(rd16(b));
  int sh = rd16(b + 2);
  for (int j = 0; j < 8; ++j)
    o->ls[j] = ((b[4 + j / 2] >> (4 * (j % 2))) & 15) | (((sh >> (2 * j)) & 3) << 4);
  const uint8_t* Q = b + 8;
  for (int j = 0; j < 8; ++j)
    for (int i = 0; i < 16; ++i) {
      o->idx[32 * j + i] = Q[16 * j + i] & 15;
      o->idx[32 * j + 16 + i] = Q[16 * j + i] >> 4;
    }
}

/* Fields of every block of n_rows rows.  Q8_0: d[N][K/32], q[N][K].
 * q6_K: d [N][K/256], sc [N][K/256][16] (int8 scales), q [N][K] (0..63).
 * q4_K: d, dmin [N][K/256], sc, m [N][K/256][8], q[N][K] (0..15).
 * IQ4_XS: d [N][K/256], sc = raw ls [N][K/256][8], q = idx [N][K]. */
int oracle_unpack(int fmt, const uint8_t* w, int64_t n_rows, int64_t k, double* d, double* dmin,
                  int32_t* sc, int32_t* m, int32_t* q) {
  int64_t rb = oracle_row_bytes(fmt, k);
  if (rb < 0) return -1;
  for (int64_t n = 0; n < n_rows; ++n) {
    const uint8_t* row = w + n * rb;
    if (fmt == FMT_Q8_0) {
      for (int64_t b = 0; b < k / 32; ++b) {
        q8_0_block blk;
        decode_q8_0(row + b * 34, &blk);
        d[n * (k / 32) + b] = blk.d;
        for (int i = 0; i < 32; ++i) q[n * k + 32 * b + i] = blk.q[i];
      }
    } else if (fmt == FMT_Q8G128) {
      for (int64_t g = 0; g < k / 128; ++g) {
        q8g128_block blk;
        decode_q8g128(row + g * 130, &blk);
        d[n * (k / 128) + g] = blk.d;
        for (int i = 0; i < 128; ++i) q[n * k + 128 * g + i] = blk.q[i];
      }
    } else if (has_min(fmt)) {
      for (int64_t b = 0; b < k / 256; ++b) {
        q4_k_block blk;
        if (fmt == FMT_Q4_K)
          decode_q4_k(row + b * 144, &blk);
        else
          decode_q5_k(row + b * 176, &blk);
        int64_t sb = n * (k / 256) + b;
        d[sb] = blk.d;
        dmin[sb] = blk.dmin;
        for (int j = 0; j < 8; ++j) { sc[sb * 8 + j] = blk.sc[j]; m[sb * 8 + j] = blk.m[j]; }
        for (int i = 0; i < 256; ++i) q[n * k + 256 * b + i] = blk.q[i];
      }
    } else if (fmt == FMT_Q6_K) {
      for (int64_t b = 0; b < k / 256; ++b) {
        q6_k_block blk;
        decode_q6_k(row + b * 210, &blk);
        int64_t sb = n * (k / 256) + b;
        d[sb] = blk.d;
        for (int j = 0; j < 16; ++j) sc[sb * 16 + j] = blk.sc[j];
        for (int i = 0; i < 256; ++i) q[n * k + 256 * b + i] = blk.q[i];
      }
    } else {
      for (int64_t b = 0; b < k / 256; ++b) {
        iq4_xs_block blk;
        decode_iq4_xs(row + b * 136, &blk);
        int64_t sb = n * (k / 256) + b;
        d[sb] = blk.d;
        for (int j = 0; j < 8; ++j) sc[sb * 8 + j] = blk.ls[j];
        for (int i = 0; i < 256; ++i) q[n * k + 256 * b + i] = blk.idx[i];
      }
    }
  }
  return 0;
}

/* Dequantized weights in fp64, out[N][K]. */
int oracle_dequant(int fmt, const uint8_t* w, int64_t n_rows, int64_t k, double* out) {
  int64_t rb = oracle_row_bytes(fmt, k);
  if (rb < 0) return -1;
  for (int64_t n = 0; n < n_rows; ++n) {
    const uint8_t* row = w + n * rb;
    double* o = out + n * k;
    if (fmt == FMT_Q8_0) {
      for (int64_t b = 0; b < k / 32; ++b) {
        q8_0_block blk;
        decode_q8_0(row + b * 34, &blk);
        for (int i = 0; i < 32; ++i) o[32 * b + i] = blk.d * blk.q[i];
      }
    } else if (fmt == FMT_Q8G128) {
      for (int64_t g = 0; g < k / 128; ++g) {
        q8g128_block blk;
        decode_q8g128(row + g * 130, &blk);
        for (int i = 0; i < 128; ++i) o[128 * g + i] = blk.d * blk.q[i];
      }
    } else if (has_min(fmt)) {
      for (int64_t b = 0; b < k / 256; ++b) {
        q4_k_block blk;
        if (fmt == FMT_Q4_K)
          decode_q4_k(row + b * 144, &blk);
        else
          decode_q5_k(row + b * 176, &blk);
        for (int i = 0; i < 256; ++i)
          o[256 * b + i] = blk.d * blk.sc[i / 32] * blk.q[i] - blk.dmin * blk.m[i / 32];
      }
    } else if (fmt == FMT_Q6_K) {
      for (int64_t b = 0; b < k / 256; ++b) {
        q6_k_block blk;
        decode_q6_k(row + b * 210, &blk);
        for (int i = 0; i < 256; ++i) o[256 * b + i] = blk.d * blk.sc[i / 16] * (blk.q[i] - 32);
      }
    } else {
      for (int64_t b = 0; b < k / 256; ++b) {
        iq4_xs_block blk;
        decode_iq4_xs(row + b * 136, &blk);
        for (int i = 0; i < 256; ++i)
          o[256 * b + i] = blk.d * (blk.ls[i / 32] - 32) * IQ4_CODEBOOK[blk.idx[i]];
      }
    }
  }
  return 0;
}

/* ------------------------------------------------- activation quantization */
/* x fp32 [n_tok][ldx] -> qs int8 [n_tok][k], d fp32 [n_tok][k/32],
 * s int32 [n_tok][k/32]. */
int oracle_quantize_act(const float* x, int64_t ldx, int64_t n_tok, int64_t k, int8_t* qs,
                        float* d, int32_t* s) {
  if (k % 32 || ldx < k) return -1;
  int64_t nb = k / 32;
  for (int64_t t = 0; t < n_tok; ++t)
    for (int64_t b = 0; b < nb; ++b) {
      const float* xb = x + t * ldx + 32 * b;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        float a = fabsf(xb[i]);
        if (a > amax) amax = a;
      }
      float db = amax / 127.0f;
      int32_t sum = 0;
      for (int i = 0; i < 32; ++i) {
        int qi = 0;
        if (amax != 0.0f) {
          float v = xb[i] / db;
          qi = (int)roundf(v); /* C roundf: halfway cases away from zero */
          if (qi > 127) qi = 127;
          if (qi < -127) qi = -127;
        }
        qs[t * k + 32 * b + i] = (int8_t)qi;
        sum += qi;
      }
      d[t * nb + b] = db;
      s[t * nb + b] = sum;
    }
  return 0;
}

/* --------------------------------------------------- per-block integer dots */
/* Integer partials of one row against one token, for every 32-block b of K.
 * out[b*nc + 0] = P (or A for q4_K, q5_K), out[b*nc + 1] = B (those two only). */
static void row_block_dots(int fmt, const uint8_t* row, int64_t k, const int8_t* qx,
                           const int32_t* sx, int32_t* out) {
  if (fmt == FMT_Q8_0) {
    for (int64_t b = 0; b < k / 32; ++b) {
      q8_0_block blk;
      decode_q8_0(row + b * 34, &blk);
      int32_t p = 0;
      for (int i = 0; i < 32; ++i) p += blk.q[i] * qx[32 * b + i];
      out[b] = p;
    }
  } else if (fmt == FMT_Q8G128) {
    for (int64_t g = 0; g < k / 128; ++g) {
      q8g128_block blk;
      decode_q8g128(row + g * 130, &blk);
      for (int j = 0; j < 4; ++j) {
        int32_t p = 0;
        for (int i = 0; i < 32; ++i) p += blk.q[32 * j + i] * qx[128 * g + 32 * j + i];
        out[4 * g + j] = p;
      }
    }
  } else if (has_min(fmt)) {
    for (int64_t sb = 0; sb < k / 256; ++sb) {
      q4_k_block blk;
      if (fmt == FMT_Q4_K)
        decode_q4_k(row + sb * 144, &blk);
      else
        decode_q5_k(row + sb * 176, &blk);
      for (int j = 0; j < 8; ++j) {
        int64_t b = sb * 8 + j;
        int32_t a = 0;
        for (int i = 0; i < 32; ++i) a += blk.q[32 * j + i] * qx[32 * b + i];
        out[2 * b] = blk.sc[j] * a;
        out[2 * b + 1] = blk.m[j] * sx[b];
      }
    }
  } else if (fmt == FMT_Q6_K) {
    for (int64_t sb = 0; sb < k / 256; ++sb) {
      q6_k_block blk;
      decode_q6_k(row + sb * 210, &blk);
      for (int j = 0; j < 8; ++j) {
        int64_t b = sb * 8 + j;
        int32_t p = 0;
        for (int i = 0; i < 32; ++i) {
          int w = 32 * j + i;
          p += blk.sc[w / 16] * (blk.q[w] - 32) * qx[32 * b + i];
        }
        out[b] = p;
      }
    }
  } else {
    for (int64_t sb = 0; sb < k / 256; ++sb) {
      iq4_xs_block blk;
      decode_iq4_xs(row + sb * 136, &blk);
      for (int j = 0; j < 8; ++j) {
        int64_t b = sb * 8 + j;
        int32_t p = 0;
        for (int i = 0; i < 32; ++i) p += IQ4_CODEBOOK[blk.idx[32 * j + i]] * qx[32 * b + i];
        out[b] = (blk.ls[j] - 32) * p;
      }
    }
  }
}

/* out int32 [n_tok][n_rows][k/32][nc], nc = 2 for q4_K and q5_K (A, B), else 1. */
int oracle_block_dots(int fmt, const uint8_t* w, int64_t n_rows, int64_t k, const int8_t* qs,
                      const int32_t* s, int64_t n_tok, int32_t* out) {
  int64_t rb = oracle_row_bytes(fmt, k);
  if (rb < 0) return -1;
  int64_t nb = k / 32, nc = has_min(fmt) ? 2 : 1;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < n_rows; ++n)
    for (int64_t t = 0; t < n_tok; ++t)
      row_block_dots(fmt, w + n * rb, k, qs + t * k, s + t * nb, out + ((t * n_rows + n) * nb) * nc);
  return 0;
}

/* Weight scales needed by the fp64 terms of one row, per 32-block. */
static void row_block_scales(int fmt, const uint8_t* row, int64_t k, double* dw, double* dm) {
  if (fmt == FMT_Q8_0) {
    for (int64_t b = 0; b < k / 32; ++b) dw[b] = half_to_double(rd16(row + b * 34));
  } else if (fmt == FMT_Q8G128) {
    for (int64_t b = 0; b < k / 32; ++b) dw[b] = half_to_double(rd16(row + (b / 4) * 130));
  } else {
    int64_t bb = oracle_row_bytes(fmt, 256);
    int64_t d_at = fmt == FMT_Q6_K ? 208 : 0;  /* q6_K keeps d at the end */
    for (int64_t sb = 0; sb < k / 256; ++sb)
      for (int j = 0; j < 8; ++j) {
        dw[sb * 8 + j] = half_to_double(rd16(row + sb * bb + d_at));
        if (has_min(fmt)) dm[sb * 8 + j] = half_to_double(rd16(row + sb * bb + 2));
      }
  }
}

/* y and mag of one row against one token: the sum of the per-block terms and
 * the sum of their absolute values, in fp64. */
static void row_terms(int fmt, const uint8_t* row, int64_t k, const int8_t* qx, const float* dx,
                      const int32_t* sx, int32_t* ibuf, double* dw, double* dm, double* y,
                      double* mag) {
  row_block_dots(fmt, row, k, qx, sx, ibuf);
  row_block_scales(fmt, row, k, dw, dm);
  double acc = 0.0, am = 0.0;
  for (int64_t b = 0; b < k / 32; ++b) {
    if (has_min(fmt)) {
      double tp = dw[b] * (double)dx[b] * (double)ibuf[2 * b];
      double tm = -dm[b] * (double)dx[b] * (double)ibuf[2 * b + 1];
      acc += tp + tm;
      am += fabs(tp) + fabs(tm);
    } else {
      double tau = dw[b] * (double)dx[b] * (double)ibuf[b];
      acc += tau;
      am += fabs(tau);
    }
  }
  *y = acc;
  *mag = am;
}

/* y, mag fp64 [n_tok][n_rows]. */
int oracle_matvec(int fmt, const uint8_t* w, int64_t n_rows, int64_t k, const int8_t* qs,
                  const float* d, const int32_t* s, int64_t n_tok, double* y, double* mag) {
  int64_t rb = oracle_row_bytes(fmt, k);
  if (rb < 0) return -1;
  int64_t nb = k / 32;
#pragma omp parallel
  {
    int32_t* ibuf = (int32_t*)malloc(sizeof(int32_t) * 2 * nb);
    double* dw = (double*)malloc(sizeof(double) * nb);
    double* dm = (double*)malloc(sizeof(double) * nb);
#pragma omp for schedule(static)
    for (int64_t n = 0; n < n_rows; ++n)
      for (int64_t t = 0; t < n_tok; ++t)
        row_terms(fmt, w + n * rb, k, qs + t * k, d + t * nb, s + t * nb, ibuf, dw, dm,
                  &y[t * n_rows + n], &mag[t * n_rows + n]);
    free(ibuf);
    free(dw);
    free(dm);
  }
  return 0;
}

/* Matvec plus a residual (Castagna Veloce page, "Fused operations": matvec +
 * residual add): y[t][n] = sum of the terms of (t, n) + res[t][n], the
 * residual being one more term of the sum (mag gains |res[t][n]|). */
int oracle_matvec_residual(int fmt, const uint8_t* w, int64_t n_rows, int64_t k, const int8_t* qs,
                           const float* d, const int32_t* s, int64_t n_tok, const float* res,
                           int64_t ldr, double* y, double* mag) {
  if (oracle_matvec(fmt, w, n_rows, k, qs, d, s, n_tok, y, mag) != 0) return -1;
  for (int64_t t = 0; t < n_tok; ++t)
    for (int64_t n = 0; n < n_rows; ++n) {
      const double rv = (double)res[t * ldr + n];
      y[t * n_rows + n] += rv;
      mag[t * n_rows + n] += fabs(rv);
    }
  return 0;
}

/* Expert-routed matvec (Castagna Veloce page, "Kernels for the MI50": MoE
 * decode for up to 64 tokens, one pass per expert over its routed tokens).
 * w = [n_experts][n_rows][row bytes].  Slot (t, s) uses expert ids[t][s] and
 * activation row t (x_per_slot = 0) or t*top_k + s (x_per_slot = 1).
 * rw == NULL: y, mag [n_tok][top_k][n_rows], one output per slot.
 * rw != NULL: y[t][n] = sum_s rw[t][s] y_slot, mag = sum_s |rw| mag_slot.
 * A slot whose id is outside [0, n_experts) contributes nothing. */
int oracle_moe_matvec(int fmt, const uint8_t* w, int64_t n_experts, int64_t n_rows, int64_t k,
                      const int8_t* qs, const float* d, const int32_t* s, int x_per_slot,
                      const int32_t* ids, const float* rw, int64_t n_tok, int64_t top_k,
                      double* y, double* mag) {
  int64_t rb = oracle_row_bytes(fmt, k);
  if (rb < 0) return -1;
  int64_t nb = k / 32;
#pragma omp parallel
  {
    int32_t* ibuf = (int32_t*)malloc(sizeof(int32_t) * 2 * nb);
    double* dw = (double*)malloc(sizeof(double) * nb);
    double* dm = (double*)malloc(sizeof(double) * nb);
#pragma omp for schedule(static)
    for (int64_t n = 0; n < n_rows; ++n)
      for (int64_t t = 0; t < n_tok; ++t) {
        double ysum = 0.0, msum = 0.0;
        for (int64_t sl = 0; sl < top_k; ++sl) {
          int32_t e = ids[t * top_k + sl];
          double ys = 0.0, ms = 0.0;
          if (e >= 0 && e < n_experts) {
            int64_t xr = x_per_slot ? t * top_k + sl : t;
            row_terms(fmt, w + (e * n_rows + n) * rb, k, qs + xr * k, d + xr * nb, s + xr * nb,
                      ibuf, dw, dm, &ys, &ms);
          }
          if (rw) {
            ysum += (double)rw[t * top_k + sl] * ys;
            msum += fabs((double)rw[t * top_k + sl]) * ms;
          } else {
            y[(t * top_k + sl) * n_rows + n] = ys;
            mag[(t * top_k + sl) * n_rows + n] = ms;
          }
        }
        if (rw) {
          y[t * n_rows + n] = ysum;
          mag[t * n_rows + n] = msum;
        }
      }
    free(ibuf);
    free(dw);
    free(dm);
  }
  return 0;
}

/*
 * SwiGLU of a gate+up output (Castagna Veloce page, "Fused operations": the
 * gate/up + SwiGLU fusion of the verify batches).  Row r of gu holds the gate
 * half in columns 0..n_ff-1 and the up half in n_ff..2n_ff-1 (one gate+up
 * tensor per expert, gate rows first); h = silu(g) * u with
 * silu(g) = g / (1 + exp(-g)), in fp64 from the fp32 inputs.  The pages give
 * no formula; this is the usual SwiGLU.  The h rows are quantized to Q8
 * activations with oracle_quantize_act by the caller.
 */
int oracle_swiglu(const float* gu, int64_t ldg, int64_t rows, int64_t n_ff, double* h) {
  if (n_ff < 1 || ldg < 2 * n_ff || rows < 0) return 1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < n_ff; ++i) {
      const double g = gu[r * ldg + i];
      const double u = gu[r * ldg + n_ff + i];
      const double e = exp(-g);  /* +inf for very negative g: silu -> -0 */
      h[r * n_ff + i] = g / (1.0 + e) * u;
    }
  return 0;
}

/*
 * Router and top-k (Castagna Veloce page, "Fused operations": router matvec,
 * gating, top-k and weight normalization in one kernel).  The pages give no
 * formula; the readings: router weights fp32 [E][K]; logits l = W x in fp64;
 * the top_k experts by logit, a larger logit first and on equal logits the
 * lower expert index first; weights = softmax over the selected logits (the
 * same as a softmax over all E renormalized over the selected ones).
 * ids int32 [T][top_k], w double [T][top_k], logits double [T][E].
 */
int oracle_router_topk(const float* x, int64_t ldx, int64_t n_tok, int64_t k, const float* wr,
                       int64_t n_experts, int64_t top_k, int32_t* ids, double* w, double* logits) {
  if (n_tok < 0 || k < 1 || ldx < k || n_experts < 1 || top_k < 1 || top_k > n_experts) return 1;
  for (int64_t t = 0; t < n_tok; ++t) {
    double* l = logits + t * n_experts;
    for (int64_t e = 0; e < n_experts; ++e) {
      double acc = 0.0;
      for (int64_t i = 0; i < k; ++i) acc += (double)wr[e * k + i] * (double)x[t * ldx + i];
      l[e] = acc;
    }
    /* selection: top_k passes, each taking the best expert not yet taken */
    for (int64_t j = 0; j < top_k; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < n_experts; ++e) {
        int taken = 0;
        for (int64_t q = 0; q < j; ++q)
          if (ids[t * top_k + q] == (int32_t)e) taken = 1;
        if (taken) continue;
        if (best < 0 || l[e] > l[best]) best = e;  /* strict: ties keep the lower index */
      }
      ids[t * top_k + j] = (int32_t)best;
    }
    double m = l[ids[t * top_k]], sum = 0.0;
    for (int64_t j = 0; j < top_k; ++j) sum += exp(l[ids[t * top_k + j]] - m);
    for (int64_t j = 0; j < top_k; ++j) w[t * top_k + j] = exp(l[ids[t * top_k + j]] - m) / sum;
  }
  return 0;
}

/* The selection and weights of oracle_router_topk, from given logits (fp32,
 * as a kernel computes them): the reference for checking a kernel's choice
 * against its own logits. */
int oracle_topk_from_logits(const float* logits, int64_t n_tok, int64_t n_experts, int64_t top_k,
                            int32_t* ids, double* w) {
  if (n_tok < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts) return 1;
  for (int64_t t = 0; t < n_tok; ++t) {
    const float* l = logits + t * n_experts;
    for (int64_t j = 0; j < top_k; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < n_experts; ++e) {
        int taken = 0;
        for (int64_t q = 0; q < j; ++q)
          if (ids[t * top_k + q] == (int32_t)e) taken = 1;
        if (taken) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      ids[t * top_k + j] = (int32_t)best;
    }
    const double m = l[ids[t * top_k]];
    double sum = 0.0;
    for (int64_t j = 0; j < top_k; ++j) sum += exp((double)l[ids[t * top_k + j]] - m);
    for (int64_t j = 0; j < top_k; ++j) w[t * top_k + j] = exp((double)l[ids[t * top_k + j]] - m) / sum;
  }
  return 0;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
