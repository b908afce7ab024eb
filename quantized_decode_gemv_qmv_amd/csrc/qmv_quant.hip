// qmv_quant.hip -- activation Q8 quantizer and the integer block-dot test
// kernel, for gfx950.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

// ------------------------------------------------------ activation quantizer
// Q8 activation blocks (Castagna Veloce page, "Fused operations": activations
// quantized once and reused by every weight type).  Eight lanes per block of
// 32 values, four values per lane from one 16-byte load, through q8_block8.
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
  float db;
  int sum;
  const uint32_t packed = q8_block8(vv, db, sum);
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

// --------------------------------------------------------- SwiGLU + Q8
// The step between a gate+up and a down projection (Castagna Veloce page,
// "Fused operations": gate/up + SwiGLU kernels for the verify batches, and
// Q8 activations made once): h = silu(g) * u over the gate and up halves of
// each row of gu, with silu(g) = g / (1 + exp(-g)) in fp32 (accurate expf
// and IEEE division), then the Q8 activation blocks of h exactly as
// k_quantize makes them.  Eight lanes per block of 32, four values per lane.
// h_out (optional) receives the fp32 h the blocks were made from.
__global__ __launch_bounds__(256) void k_swiglu_quantize(const float* __restrict__ gu, int64_t ldg,
                                                         int rows, int n_ff, int8_t* __restrict__ qs,
                                                         float* __restrict__ d, int32_t* __restrict__ s,
                                                         float* __restrict__ h_out) {
  const int nb = n_ff / 32;
  const int64_t total = (int64_t)rows * nb;
  int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const bool valid = blk < total;
  if (!valid) blk = total - 1;
  const int j = threadIdx.x & 7;
  const int64_t r = blk / nb, b = blk % nb;
  const float* row = gu + r * ldg + 32 * b + 4 * j;
  const f32x4 g = *reinterpret_cast<const f32x4*>(row);
  const f32x4 u = *reinterpret_cast<const f32x4*>(row + n_ff);
  const float gg[4] = {g.x, g.y, g.z, g.w}, uu[4] = {u.x, u.y, u.z, u.w};
  float hv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) hv[i] = gg[i] / (1.0f + expf(-gg[i])) * uu[i];
  float db;
  int sum;
  const uint32_t packed = q8_block8(hv, db, sum);
  if (valid) {
    const int64_t o = r * n_ff + 32 * b + 4 * j;
    *reinterpret_cast<uint32_t*>(qs + o) = packed;
    if (h_out != nullptr) *reinterpret_cast<f32x4*>(h_out + o) = f32x4{hv[0], hv[1], hv[2], hv[3]};
    if (j == 0) {
      d[r * nb + b] = db;
      s[r * nb + b] = sum;
    }
  }
}

hipError_t launch_swiglu_quantize(const float* gu, int64_t ldg, int rows, int n_ff, int8_t* qs, float* d,
                                  int32_t* s, float* h_out, hipStream_t st) {
  const int64_t blocks = (int64_t)rows * (n_ff / 32);
  const int64_t grid = (blocks + 31) / 32;
  hipLaunchKernelGGL(k_swiglu_quantize, dim3((unsigned)grid), dim3(256), 0, st, gu, ldg, rows, n_ff, qs, d, s,
                     h_out);
  return hipGetLastError();
}

// ------------------------------------------------------------- block dots
// One thread per (token, row, 32-block), through the same weight decode,
// activation fetch and paired integer dot (own_first, own_pass, own_second)
// as the matvec kernels: thread b holds unit b, whose own block is 32-block b,
// and the threads of a pair (b even, b + 1) sit side by side in one wave
// (K / 32 is a multiple of 8 for the 256-weight formats, so no pair or q6_K
// quad is split by a row or by the grid end).
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
  Raw<F> raw;
  DecO<F> dec;
  XO xo;
  load_unit(wr, b, raw);
  decode_own(raw, b, b & 1, true, dec);
  load_xo<F>(x, t, b, xo);
  const int dot = own_second(dec, xo.s, own_pass<F>(own_first(dec, xo.f)));
  if constexpr (kmin<F>()) {
    // sub-block b: scale times the integer dot, and min times the block sum
    out[2 * gid] = dec.isc * dot;
    out[2 * gid + 1] = dec.im * x.s[(int64_t)t * x.nb + b];
  } else if constexpr (F == FQ6_K) {
    out[gid] = dot;  // the 16-weight scales are applied inside the paired dot
  } else {
    out[gid] = dec.isc * dot;  // Q8_0, Q8G128: isc = 1; IQ4_XS: the signed sub-block scale
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
    case FQ5_K:
      hipLaunchKernelGGL(k_block_dots<FQ5_K>, dim3(grid), dim3(256), 0, st, w, row_bytes, n_rows,
                         units, x, n_tok, out);
      break;
    case FQ6_K:
      hipLaunchKernelGGL(k_block_dots<FQ6_K>, dim3(grid), dim3(256), 0, st, w, row_bytes, n_rows,
                         units, x, n_tok, out);
      break;
    case FQ8G128:
      hipLaunchKernelGGL(k_block_dots<FQ8G128>, dim3(grid), dim3(256), 0, st, w, row_bytes, n_rows,
                         units, x, n_tok, out);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qmv
