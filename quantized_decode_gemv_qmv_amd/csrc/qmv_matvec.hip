// qmv_matvec.hip -- activation Q8 quantizer, dense small-batch matvec (with
// its split-K form) and the integer block-dot test kernel, for gfx950.
//
// Matvec mapping.  A 256-thread workgroup is four waves; a wave is split into
// 64/LPR lane groups and each group owns R consecutive rows.  The LPR lanes of
// a group walk the row's 32-weight units with stride LPR, so for every unit
// index the group reads a contiguous span of the row (16 bytes per lane for
// q4_K / IQ4_XS quants, 34 bytes per lane for Q8_0 blocks) and every weight
// byte is fetched from HBM exactly once.  The activation fragment of a unit is
// loaded once per token and shared by the group's R rows; each decoded weight
// unit is shared by all tokens (one weight read serves the whole verify
// batch: zhuai.tech GLM-5.3 page, "MTP saves full-model execution rounds").
// The weight loads of the next unit are issued before the current unit is
// computed, so every wave keeps two units per row in flight.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

// ------------------------------------------------------ activation quantizer
// One 32-lane half wave per block of 32 values: amax and the block sum are
// half-wave reductions; the divisions are IEEE fp32 (no fast-math), and
// roundf rounds halfway cases away from zero.
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ x, int64_t ldx,
                                                  int n_tok, int k, int8_t* __restrict__ qs,
                                                  float* __restrict__ d, int32_t* __restrict__ s) {
  const int nb = k / 32;
  const int64_t blk = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (blk >= (int64_t)n_tok * nb) return;  // whole half-waves leave together
  const int i = threadIdx.x & 31;
  const int64_t t = blk / nb, b = blk % nb;
  const float v = x[t * ldx + 32 * b + i];
  float amax = fabsf(v);
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
  const float db = amax / 127.0f;
  int q = 0;
  if (amax != 0.0f) {
    q = static_cast<int>(roundf(v / db));
    q = q > 127 ? 127 : (q < -127 ? -127 : q);
  }
  int sum = q;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 32);
  qs[t * k + 32 * b + i] = static_cast<int8_t>(q);
  if (i == 0) {
    d[t * nb + b] = db;
    s[t * nb + b] = sum;
  }
}

hipError_t launch_quantize(const float* x, int64_t ldx, int n_tok, int k, int8_t* qs, float* d,
                           int32_t* s, hipStream_t st) {
  const int64_t blocks = (int64_t)n_tok * (k / 32);
  const int64_t grid = (blocks + 7) / 8;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)grid), dim3(256), 0, st, x, ldx, n_tok, k, qs, d, s);
  return hipGetLastError();
}

// ------------------------------------------------------------------- matvec
template <int F, int TM, int LPR, int R, bool SPLIT>
__global__ __launch_bounds__(256) void k_matvec(const uint8_t* __restrict__ w, int64_t row_bytes,
                                                int n_rows, int units, ActView xv, int n_tok,
                                                float* __restrict__ y, int64_t ldy, int ups,
                                                float* __restrict__ part, int* __restrict__ cnt) {
  constexpr int GPW = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane / LPR, gl = lane % LPR;
  const int row0 = (blockIdx.x * 4 * GPW + wave * GPW + g) * R;
  const Act x{xv.qs, xv.d, xv.s, xv.k, xv.nb};

  const uint8_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = w + (int64_t)min(row0 + r, n_rows - 1) * row_bytes;

  float acc[R][TM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[r][t] = 0.f;

  int ub = 0, ue = units;
  if constexpr (SPLIT) {
    ub = blockIdx.y * ups;
    ue = min(units, ub + ups);
  }

  int u = ub + gl;
  Raw<F> cur[R];
  if (u < ue) {
#pragma unroll
    for (int r = 0; r < R; ++r) load_unit(wr[r], u, cur[r]);
  }
  for (; u < ue; u += LPR) {
    Raw<F> nxt[R];
    const int un = u + LPR;
    if (un < ue) {
#pragma unroll
      for (int r = 0; r < R; ++r) load_unit(wr[r], un, nxt[r]);
    }
    Dec<F> dec[R];
#pragma unroll
    for (int r = 0; r < R; ++r) decode_unit(cur[r], u, dec[r]);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < n_tok) {
        XFrag<F> xf;
        load_xfrag<F>(x, t, u, xf);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][t] += unit_value(dec[r], xf);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) cur[r] = nxt[r];
  }

#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t)
      if (t < n_tok) acc[r][t] = group_sum<LPR>(acc[r][t]);

  // every lane of the group now holds all R*TM sums; spread the stores
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int v = r * TM + t;
      const int row = row0 + r;
      if (t < n_tok && (v % LPR) == gl && row < n_rows) {
        if constexpr (SPLIT)
          __hip_atomic_store(&part[((int64_t)blockIdx.y * n_tok + t) * n_rows + row], acc[r][t],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          y[(int64_t)t * ldy + row] = acc[r][t];
      }
    }

  if constexpr (SPLIT) {
    // The last workgroup of a row tile to finish sums the slices in slice
    // order (deterministic) and re-arms the tile's counter for the next call.
    __shared__ int s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = atomicAdd(&cnt[blockIdx.x], 1);
      s_last = (prev == (int)gridDim.y - 1);
    }
    __syncthreads();
    if (s_last) {
      __threadfence();
      constexpr int RWG = 4 * GPW * R;
      const int r0 = blockIdx.x * RWG;
      for (int i = threadIdx.x; i < n_tok * RWG; i += 256) {
        const int t = i / RWG, row = r0 + i % RWG;
        if (row < n_rows) {
          float sum = 0.f;
          for (int sl = 0; sl < (int)gridDim.y; ++sl)
            sum += __hip_atomic_load(&part[((int64_t)sl * n_tok + t) * n_rows + row],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          y[(int64_t)t * ldy + row] = sum;
        }
      }
      if (threadIdx.x == 0) atomicExch(&cnt[blockIdx.x], 0);
    }
  }
}

// Variant table: (lanes per row group, rows per group).
const Variant kVariants[] = {
    {64, 1, "lpr64_r1"}, {64, 2, "lpr64_r2"}, {32, 1, "lpr32_r1"},
    {32, 2, "lpr32_r2"}, {16, 1, "lpr16_r1"}, {16, 2, "lpr16_r2"},
};
const int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

template <int F, int TM, int LPR, int R>
static hipError_t run_mv(const MatvecLaunch& a, hipStream_t st) {
  constexpr int RWG = 4 * (64 / LPR) * R;
  const unsigned tiles = (unsigned)((a.n_rows + RWG - 1) / RWG);
  if (a.slices > 1) {
    const int ups = (a.units + a.slices - 1) / a.slices;
    hipLaunchKernelGGL((k_matvec<F, TM, LPR, R, true>), dim3(tiles, (unsigned)a.slices), dim3(256),
                       0, st, a.w, a.row_bytes, a.n_rows, a.units, a.x, a.n_tok, a.y, a.ldy, ups,
                       a.part, a.cnt);
  } else {
    hipLaunchKernelGGL((k_matvec<F, TM, LPR, R, false>), dim3(tiles), dim3(256), 0, st, a.w,
                       a.row_bytes, a.n_rows, a.units, a.x, a.n_tok, a.y, a.ldy, 0,
                       (float*)nullptr, (int*)nullptr);
  }
  return hipGetLastError();
}

template <int F, int TM>
static hipError_t run_mv_variant(const MatvecLaunch& a, hipStream_t st) {
  switch (a.variant) {
    case 0: return run_mv<F, TM, 64, 1>(a, st);
    case 1: return run_mv<F, TM, 64, 2>(a, st);
    case 2: return run_mv<F, TM, 32, 1>(a, st);
    case 3: return run_mv<F, TM, 32, 2>(a, st);
    case 4: return run_mv<F, TM, 16, 1>(a, st);
    case 5: return run_mv<F, TM, 16, 2>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int F>
static hipError_t run_mv_tokens(const MatvecLaunch& a, hipStream_t st) {
  if (a.n_tok <= 1) return run_mv_variant<F, 1>(a, st);
  if (a.n_tok <= 2) return run_mv_variant<F, 2>(a, st);
  if (a.n_tok <= 4) return run_mv_variant<F, 4>(a, st);
  if (a.n_tok <= 8) return run_mv_variant<F, 8>(a, st);
  return run_mv_variant<F, 16>(a, st);
}

hipError_t launch_matvec(const MatvecLaunch& a, hipStream_t st) {
  switch (a.fmt) {
    case FQ8_0: return run_mv_tokens<FQ8_0>(a, st);
    case FQ4_K: return run_mv_tokens<FQ4_K>(a, st);
    case FIQ4_XS: return run_mv_tokens<FIQ4_XS>(a, st);
    default: return hipErrorInvalidValue;
  }
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
