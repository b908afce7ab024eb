// qmv_quant.hip -- activation Q8 quantizer and the integer block-dot test
// kernel, for gfx950.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

typedef float f32x4 __attribute__((ext_vector_type(4), aligned(4)));

// ------------------------------------------------------ activation quantizer
// Q8 activation blocks (Castagna Veloce page, "Fused operations": activations
// quantized once and reused by every weight type).  Eight lanes per block of
// 32 values, four values per lane from one 16-byte load: the block's max |x|
// and the sum of its quants are 8-lane DPP reductions inside a row, so no
// lane exchange leaves the DPP network.  Divisions are IEEE fp32 (the library
// is built without fast-math) and roundf rounds halfway cases away from zero.
// Lanes past the last block redo the last block and store nothing, which keeps
// every lane of a reduction group active.
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ x, int64_t ldx,
                                                  int n_tok, int k, int8_t* __restrict__ qs,
                                                  float* __restrict__ d, int32_t* __restrict__ s) {
  const int nb = k / 32;
  const int64_t total = (int64_t)n_tok * nb;
  int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const bool valid = blk < total;
  if (!valid) blk = total - 1;
  const int j = threadIdx.x & 7;
  const int64_t t = blk / nb, b = blk % nb;
  const f32x4 v = *reinterpret_cast<const f32x4*>(x + t * ldx + 32 * b + 4 * j);
  const float vv[4] = {v.x, v.y, v.z, v.w};
  float amax = fmaxf(fmaxf(fabsf(vv[0]), fabsf(vv[1])), fmaxf(fabsf(vv[2]), fabsf(vv[3])));
  amax = max8(amax);
  const float db = amax / 127.0f;
  int q[4] = {0, 0, 0, 0};
  if (amax != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = static_cast<int>(roundf(vv[i] / db));
      q[i] = r > 127 ? 127 : (r < -127 ? -127 : r);
    }
  }
  const int sum = sum8(q[0] + q[1] + q[2] + q[3]);
  const uint32_t packed = (uint32_t)(q[0] & 255) | ((uint32_t)(q[1] & 255) << 8) |
                          ((uint32_t)(q[2] & 255) << 16) | ((uint32_t)(q[3] & 255) << 24);
  if (valid) {
    *reinterpret_cast<uint32_t*>(qs + t * k + 32 * b + 4 * j) = packed;
    if (j == 0) {
      d[t * nb + b] = db;
      s[t * nb + b] = sum;
    }
  }
}

hipError_t launch_quantize(const float* x, int64_t ldx, int n_tok, int k, int8_t* qs, float* d,
                           int32_t* s, hipStream_t st) {
  const int64_t blocks = (int64_t)n_tok * (k / 32);
  const int64_t grid = (blocks + 31) / 32;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)grid), dim3(256), 0, st, x, ldx, n_tok, k, qs, d, s);
  return hipGetLastError();
}

// ------------------------------------------------------------- block dots
// One thread per (token, row, 32-block), through the same load, decode and
// integer dot routines as the matvec kernels.
template <int F>
__global__ __launch_bounds__(256) void k_block_dots(const uint8_t* __restrict__ w, int64_t row_bytes,
                                                    int n_rows, int units, ActView xv, int n_tok,
                                                    int32_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)n_tok * n_rows * units) return;
  const int b = (int)(gid % units);
  const int row = (int)((gid / units) % n_rows);
  const int t = (int)(gid / ((int64_t)units * n_rows));
  const Act x{xv.qs, xv.d, xv.s, xv.k, xv.nb};
  const uint8_t* wr = w + (int64_t)row * row_bytes;
  if constexpr (F == FQ4_K) {
    // 32-block b = sub-block jj of super-block sb lives in the low (jj even)
    // or high (jj odd) nibbles of units 2*(jj/2) and 2*(jj/2)+1
    const int sb = b >> 3, jj = b & 7;
    const int u0 = 8 * sb + 2 * (jj >> 1);
    int A = 0, B = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Raw<F> raw;
      Dec<F> dec;
      XFrag<F> xf;
      load_unit(wr, u0 + h, raw);
      decode_unit(raw, u0 + h, dec);
      load_xfrag<F>(x, t, u0 + h, xf);
      int lo, hi;
      unit_int(dec, xf, lo, hi);
      A += (jj & 1) ? dec.sc1 * hi : dec.sc0 * lo;
      if (h == 0) B = (jj & 1) ? dec.m1 * xf.s1 : dec.m0 * xf.s0;
    }
    out[2 * gid] = A;
    out[2 * gid + 1] = B;
  } else {
    Raw<F> raw;
    Dec<F> dec;
    XFrag<F> xf;
    load_unit(wr, b, raw);
    decode_unit(raw, b, dec);
    load_xfrag<F>(x, t, b, xf);
    int lo, hi;
    unit_int(dec, xf, lo, hi);
    int p = lo + hi;
    if constexpr (F == FIQ4_XS) p *= dec.ls;
    out[gid] = p;
  }
}

hipError_t launch_block_dots(int fmt, const uint8_t* w, int64_t row_bytes, int n_rows, int units,
                             ActView x, int n_tok, int32_t* out, hipStream_t st) {
  const int64_t n = (int64_t)n_tok * n_rows * units;
  const unsigned grid = (unsigned)((n + 255) / 256);
  switch (fmt) {
    case FQ8_0:
      hipLaunchKernelGGL(k_block_dots<FQ8_0>, dim3(grid), dim3(256), 0, st, w, row_bytes, n_rows,
                         units, x, n_tok, out);
      break;
    case FQ4_K:
      hipLaunchKernelGGL(k_block_dots<FQ4_K>, dim3(grid), dim3(256), 0, st, w, row_bytes, n_rows,
                         units, x, n_tok, out);
      break;
    case FIQ4_XS:
      hipLaunchKernelGGL(k_block_dots<FIQ4_XS>, dim3(grid), dim3(256), 0, st, w, row_bytes, n_rows,
                         units, x, n_tok, out);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qmv
