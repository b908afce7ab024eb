// qmv_mxf.hip -- flat matrix-core matvec for verify batches (several tokens)
// on gfx950.
//
// The matrix-core tile of qmv_mfma.hip -- 16 weight rows, int8 products of
// v_mfma_i32_16x16x64_i8 whose zero-masked activation rows keep every
// 32-block's integer dot apart, each lane applying the scales of the blocks
// whose bytes it loaded -- scheduled the way the single-token flat kernel is:
// one pass over the rows, no persistent loop and no load ring, so that every
// weight byte of the launch is requested as early as the hardware allows
// (zhuai.tech GLM-5.3 page, "MTP saves full-model execution rounds": the
// tokens of a verify batch share one read of the weights; "A single decode
// row is not a large matrix multiplication": weight traffic decides).
//
// Workgroup (x, y) takes the RT = WPB / KS row tiles x * RT .. of K slice y
// (units y * ups .. + ups; one slice unless SPLIT).  Its activations for that
// slice are staged once in LDS, block-major as in qmv_mfma.hip.  The KS waves
// of a tile split the slice's super-blocks, SBW consecutive ones each, and
// every wave issues all of its weight loads at once, right behind the
// workgroup's activation staging loads: vector-memory loads return in issue
// order, so the LDS copy is stored and its barrier passed while the weights
// are still in flight, and the super-blocks are then computed in arrival
// order.  The KS partial sums of a tile meet in LDS (in wave order) once
// every wave is done with the activations, whose LDS they reuse.
//
// SPLIT (rows too long for one workgroup's LDS): slice y's sums go to the
// caller's workspace and the last workgroup of column x to finish adds the
// slices in slice order, with the arrival protocol of qmv_mfma.hip.
//
// DOTS (the block-dot test hook): each product's exact integer times the
// block's integer weight scale goes to a.dots, and nothing else is stored.
#include "qmv_internal.h"
#include "qmv_mfma.h"

namespace qmv {

// Token rows of the LDS activation copy: the products' rows, except q4_K
// up to four tokens (four of its eight).
constexpr int mxf_staged_rows(int f, int tm) {
  return f == FQ4_K ? (tm <= 4 ? 4 : (tm + 7) / 8 * 8) : (tm + 3) / 4 * 4;
}

template <int F, int TM, int WPB, int SBW, bool SPLIT, bool DOTS>
__global__ __launch_bounds__(64 * WPB) void k_mxf(StreamArgs a) {
  constexpr int TG = mx_tg<F>();
  constexpr int NG = (TM + TG - 1) / TG;  // token groups
  constexpr int TMP = NG * TG;            // token rows of the products
  constexpr int NT = 64 * WPB;
  constexpr bool Q4K = F == FQ4_K;
  constexpr bool P2 = Q4K;  // two blocks per product (q4_K), else four
  // staged token rows: a q4_K product has eight, but up to four tokens only
  // four are staged and the other four activation rows read the zero bytes
  constexpr int TMS = mxf_staged_rows(F, TM);
  constexpr int BS = TMS * 32 + 16;
  // staged 16-byte quant pieces and scale entries per thread whose loads go
  // out ahead of the weights (larger slices load the rest afterwards)
  constexpr int SQ = WPB >= 16 ? 4 : 8;
  constexpr int SD = WPB >= 16 ? 2 : 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t s_mem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, s = lane >> 4;
  const int KS = a.mx_ks;   // waves per row tile
  const int RT = WPB / KS;  // row tiles per workgroup
  const int tl = wave / KS, kp = wave - tl * KS;
  const int tiles = (a.n_rows + 15) >> 4;
  const int tile = (int)blockIdx.x * RT + tl;
  const bool have = tl < RT && tile < tiles;
  const int ub = SPLIT ? (int)blockIdx.y * a.ups : 0;
  const int units = SPLIT ? min(a.ups, a.units - ub) : a.units;
  const int nsb = (units + 7) >> 3;
  const int kc = 8 * nsb;  // staged blocks
  const int sb0 = kp * SBW;
  const int nmine = have ? max(0, min(SBW, nsb - sb0)) : 0;
  const int T = a.n_tok;
  const uint8_t* const wsl = a.w + (SPLIT ? (int64_t)(ub / Fmt<F>::UPB) * Fmt<F>::BB : 0);

  uint8_t* xl = s_mem;
  const int zoff = kc * BS;  // 16 zero bytes
  float* dl = reinterpret_cast<float*>(s_mem + zoff + 16);
  float* sl = dl + kc * TMS;
  const float* gd = reinterpret_cast<const float*>(a.xq + a.off_d);
  const int32_t* gs = reinterpret_cast<const int32_t*>(a.xq + a.off_s);

  // ---- staging loads: the slice's quants of every token row (rows past the
  // call's tokens repeat its last token and are never stored) and the scales
  const int nq = 2 * units, total = TMS * nq;
  const FastDiv dq(nq);
  auto piece = [&](int idx) -> const uint8_t* {
    const int t = dq.div(idx), pc = idx - t * nq;
    return a.xq + (uint32_t)(min(t, T - 1) * a.k + 32 * ub + 16 * pc);
  };
  u32x4 sv[SQ];
#pragma unroll
  for (int i = 0; i < SQ; ++i) sv[i] = ld16(piece(min((int)threadIdx.x + i * NT, total - 1)));
  // scale entries (t, b), read in token-major order (consecutive lanes on
  // consecutive blocks of one token: coalesced) and stored block-major
  const int ns = kc * TMS;
  const FastDiv dk(kc);
  auto sidx = [&](int idx) {
    const int t = dk.div(idx), b = idx - t * kc;
    return min(t, T - 1) * a.nb + ub + min(b, units - 1);
  };
  float dv[SD];
  int iv[SD];
#pragma unroll
  for (int i = 0; i < SD; ++i) {
    const int gi = sidx(min((int)threadIdx.x + i * NT, ns - 1));
    dv[i] = gd[gi];
    iv[i] = Q4K ? gs[gi] : 0;
  }
  // The activations are read by every workgroup from a few kilobytes, which
  // sit on a few memory channels: requested behind the weights of the
  // workgroups already running they queue behind that flood.  So the staging
  // loads complete before this workgroup requests a weight byte.
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_sched_barrier(0);

  // ---- every weight load of the wave (clamped past the end: unconditional)
  // waves without a tile of their own re-read the workgroup's first tile
  // (cache hits), so that their loads stay unconditional
  const int tcl = have ? tile : min((int)blockIdx.x * RT, tiles - 1);
  const uint8_t* const wbase = wsl + (int64_t)tcl * 16 * a.row_bytes;
  const uint32_t woff = (uint32_t)(min(n, a.n_rows - 1 - tcl * 16) * (int)a.row_bytes);
  MxRaw<F> wv[SBW];
#pragma unroll
  for (int j = 0; j < SBW; ++j) mx_load(wbase, woff, 8 * min(sb0 + j, nsb - 1), s, units, wv[j]);
  __builtin_amdgcn_sched_barrier(0);

  // ---- the LDS copy, while the weights are on their way
  auto put = [&](int idx, const u32x4& v) {
    const int t = dq.div(idx), pc = idx - t * nq;
    *reinterpret_cast<u32x4a*>(xl + (pc >> 1) * BS + t * 32 + 16 * (pc & 1)) = v;
  };
#pragma unroll
  for (int i = 0; i < SQ; ++i) {
    const int idx = (int)threadIdx.x + i * NT;
    if (idx < total) put(idx, sv[i]);
  }
  for (int idx = (int)threadIdx.x + SQ * NT; idx < total; idx += NT) put(idx, ld16(piece(idx)));
  auto put_s = [&](int idx, float d, int sx) {
    const int t = dk.div(idx), b = idx - t * kc;
    const bool ok = b < units;  // staged blocks past the slice carry zero scales
    dl[b * TMS + t] = ok ? d : 0.f;
    if constexpr (Q4K) sl[b * TMS + t] = ok ? d * static_cast<float>(sx) : 0.f;
  };
#pragma unroll
  for (int i = 0; i < SD; ++i) {
    const int idx = (int)threadIdx.x + i * NT;
    if (idx < ns) put_s(idx, dv[i], iv[i]);
  }
  for (int idx = (int)threadIdx.x + SD * NT; idx < ns; idx += NT) {
    const int gi = sidx(idx);
    put_s(idx, gd[gi], Q4K ? gs[gi] : 0);
  }
  if (threadIdx.x < 4) reinterpret_cast<uint32_t*>(s_mem + zoff)[threadIdx.x] = 0u;
  __syncthreads();

  // ---- lane coordinates of the products (as in qmv_mfma.hip): A row m is
  // block jA of the product and token tA of the group, with data only in the
  // lanes s that hold block jA's weights (vA); the lane's results D[4s + r][n]
  // are tokens oTok + r of the group and blocks of its own loads
  const int m = lane & 15;
  const int jA = P2 ? (m >> 3) : (m >> 2);
  const int tA = P2 ? (m & 7) : (m & 3);
  // (activation rows past the staged ones take the zero bytes; the lanes of
  // their outputs read the scales of the first tokens, and are never stored)
  const bool vA = (P2 ? (jA == (s >> 1)) : (jA == s)) && tA < TMS;
  constexpr int aMu = P2 ? BS : 16;
  constexpr int oMu = P2 ? TMS * 4 : 0;
  const int aLane = (P2 ? 2 * jA : jA) * BS + tA * 32 + (P2 ? 16 * (s & 1) : 0);
  const int oTok = P2 ? 4 * (s & 1) : 0;
  const int oLane = (P2 ? 2 * (s >> 1) : s) * TMS * 4 + (oTok < TMS ? oTok : 0) * 4;

  float acc[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[g][r] = 0.f;
  u32x4 A[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};

#pragma unroll
  for (int j = 0; j < SBW; ++j) {
    if (j >= nmine) break;  // uniform over the wave
    const int sb = sb0 + j;
    const int u0 = 8 * sb;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      __builtin_amdgcn_sched_barrier(0);  // super-blocks and spans one after the other
      MxDec dec;
      mx_decode(wv[j], p, s, u0, units, dec);
      const int bl = u0 + 4 * p;  // first block of the span
      const int ab = vA ? bl * BS + aLane : zoff;
      const int ob = bl * TMS * 4 + oLane;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g > 0) __builtin_amdgcn_sched_barrier(0);
        if (vA) {
          A[0] = ld16(xl + ab + g * TG * 32);
          A[1] = ld16(xl + ab + g * TG * 32 + aMu);
        }
        if constexpr (DOTS) {
          const int row = tile * 16 + n;
#pragma unroll
          for (int mu = 0; mu < (P2 ? 2 : 1); ++mu) {
            i32x4 d;
            if constexpr (P2) {
              d = mfma64(A[mu], dec.b[mu], i32x4{0, 0, 0, 0});
            } else {
              d = mfma64(A[0], dec.b[0], i32x4{0, 0, 0, 0});
              d = mfma64(A[1], dec.b[1], d);
            }
            const int lb = bl + (P2 ? 2 * (s >> 1) + mu : s);  // unit inside the slice
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = P2 ? g * TG + 4 * (s & 1) + r : g * TG + r;
              if (t < T && row < a.n_rows && lb < units) {
                const int64_t o = ((int64_t)t * a.n_rows + row) * a.units + ub + lb;
                if constexpr (Q4K) {
                  a.dots[2 * o] = dec.isc[mu] * d[r];
                  a.dots[2 * o + 1] = dec.im[mu] * gs[t * a.nb + ub + lb];
                } else {
                  a.dots[o] = dec.isc[0] * d[r];
                }
              }
            }
          }
        } else if constexpr (P2) {
#pragma unroll
          for (int mu = 0; mu < 2; ++mu) {
            const i32x4 d = mfma64(A[mu], dec.b[mu], i32x4{0, 0, 0, 0});
            const int o = ob + mu * oMu + g * TG * 4;
            const f32x4 fx = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(dl) + o);
            const f32x4 fs = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(sl) + o);
            const float fxa[4] = {fx.x, fx.y, fx.z, fx.w}, fsa[4] = {fs.x, fs.y, fs.z, fs.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              acc[g][r] = fmaf(static_cast<float>(d[r]), dec.dw[mu] * fxa[r], acc[g][r]);
              acc[g][r] = fmaf(-dec.wm[mu], fsa[r], acc[g][r]);
            }
          }
        } else {
          i32x4 d = mfma64(A[0], dec.b[0], i32x4{0, 0, 0, 0});
          d = mfma64(A[1], dec.b[1], d);
          const f32x4 fx = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(dl) + ob + g * TG * 4);
          const float fxa[4] = {fx.x, fx.y, fx.z, fx.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[g][r] = fmaf(static_cast<float>(d[r]), dec.dw[0] * fxa[r], acc[g][r]);
        }
      }
    }
  }
  if constexpr (DOTS) return;  // the integers are out; nothing to sum

  // ---- sums: lanes holding the other blocks of the same row and tokens
  // (two blocks per product: lane ^ 32; else lanes ^ 16, ^ 32), then the KS
  // waves of a tile through LDS, in wave order
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = acc[g][r];
      if constexpr (!P2) v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[g][r] = v;
    }
  __syncthreads();  // every wave is done with the activations: their LDS takes the partials
  float* red = reinterpret_cast<float*>(s_mem);  // [WPB][TMP][16]
  if (tl < RT) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = P2 ? g * 8 + 4 * s + r : g * 4 + r;
        const bool mine = P2 ? s < 2 : s == (g & 3);
        if (mine) red[(wave * TMP + t) * 16 + n] = acc[g][r];
      }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < RT * TMP * 16; q += NT) {
    const int tt = q / (TMP * 16), rest = q - tt * (TMP * 16);
    const int t = rest >> 4;
    float sum = 0.f;
    for (int w = 0; w < KS; ++w) sum += red[((tt * KS + w) * TMP) * 16 + rest];
    const int row = ((int)blockIdx.x * RT + tt) * 16 + (rest & 15);
    if (row < a.n_rows && t < T) {
      if constexpr (SPLIT)
        __hip_atomic_store(&a.part[((int64_t)blockIdx.y * T + t) * a.n_rows + row], sum, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else
        a.y[(int64_t)t * a.ldy + row] = sum;
    }
  }

  if constexpr (SPLIT) {
    // The last workgroup of column x to finish adds the slices in slice
    // order.  The partials are device-scope atomic accesses (written through
    // and reloaded by the L2), so each lane waits for its stores to be
    // acknowledged before the barrier and the counter update; no device-scope
    // fence (which would write back and invalidate the XCD's whole L2).
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt, lgkmcnt all zero
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(&a.cnt[blockIdx.x], 1) == (int)gridDim.y - 1;
    __syncthreads();
    if (s_last) {
      const int rw = RT * 16;
      const int r0 = (int)blockIdx.x * rw;
      for (int q = threadIdx.x; q < T * rw; q += NT) {
        const int t = q / rw, row = r0 + (q - t * rw);
        if (row < a.n_rows) {
          float sum = 0.f;
          for (int sl2 = 0; sl2 < (int)gridDim.y; ++sl2)
            sum += __hip_atomic_load(&a.part[((int64_t)sl2 * T + t) * a.n_rows + row], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          a.y[(int64_t)t * a.ldy + row] = sum;
        }
      }
      if (threadIdx.x == 0) atomicExch(&a.cnt[blockIdx.x], 0);
    }
  }
}

#if QMV_MX_FMT == 0  // host planner: defined once, in the Q8_0 unit
// LDS budget of one workgroup's activation slice.
constexpr int64_t kMxfLdsBudget = 144 * 1024;

int mxf_plan(int fmt, int n_tok, int wpb, int sbw, int units, int n_rows, int cus, int64_t lds_per_cu,
             bool can_split, int forced_slices, MxfPlan* p) {
  const int tg = fmt == FQ4_K ? 8 : 4;
  const int tm = n_tok <= 4 ? 4 : n_tok <= 8 ? 8 : 16;
  const int tmp = (tm + tg - 1) / tg * tg;
  const int per_unit = mx_per_unit(fmt, mxf_staged_rows(fmt, tm));
  const int64_t red = (int64_t)wpb * tmp * 16 * 4;
  const int64_t tiles = (n_rows + 15) / 16;
  // slices: the fewest whose LDS copy fits the budget (or the forced count),
  // each a whole number of super-blocks that the workgroup's waves can hold
  int best_s = 0;
  for (int sl = 1; sl <= kMaxSlices; ++sl) {
    if (forced_slices > 0 && sl != forced_slices) continue;
    if (sl > 1 && !can_split) break;
    const int ups = ((units + sl - 1) / sl + 7) / 8 * 8;
    const int real = (units + ups - 1) / ups;
    if (real != sl) continue;  // that many slices of whole super-blocks do not exist
    const int nsb = ups / 8;
    const int ks = (nsb + sbw - 1) / sbw;
    if (ks > wpb) continue;  // the waves cannot hold the slice
    const int64_t lds = (int64_t)ups * per_unit + 16 + 64;
    if (lds > kMxfLdsBudget || lds > lds_per_cu) continue;
    best_s = sl;
    p->slices = sl;
    p->ups = ups;
    p->ks = ks;
    p->rt = wpb / ks;
    p->lds = (size_t)(lds > red + 64 ? lds : red + 64);
    p->grid_x = (int)((tiles + p->rt - 1) / p->rt);
    break;
  }
  (void)cus;
  return best_s;
}
#endif

template <int F, int TM, int WPB, int SBW>
static hipError_t run_mxf(const MatvecLaunch& a, const MxfPlan& p, hipStream_t st) {
  StreamArgs sa{};
  sa.w = a.w;
  sa.row_bytes = a.row_bytes;
  sa.n_rows = a.n_rows;
  sa.units = a.units;
  sa.xq = a.xq;
  sa.act_bytes = (int)a.act_bytes;
  sa.off_d = (int)a.off_d;
  sa.off_s = (int)a.off_s;
  sa.k = a.x.k;
  sa.nb = a.x.nb;
  sa.n_tok = a.n_tok;
  sa.y = a.y;
  sa.ldy = a.ldy;
  sa.mx_ks = p.ks;
  sa.ups = p.ups;
  sa.part = a.part;
  sa.cnt = a.cnt;
  sa.dots = a.dots;
  const dim3 grid((unsigned)p.grid_x, (unsigned)p.slices);
  if (a.dots != nullptr) {
    if (p.slices > 1)
      hipLaunchKernelGGL((k_mxf<F, TM, WPB, SBW, true, true>), grid, dim3(64 * WPB), p.lds, st, sa);
    else
      hipLaunchKernelGGL((k_mxf<F, TM, WPB, SBW, false, true>), grid, dim3(64 * WPB), p.lds, st, sa);
  } else if (p.slices > 1) {
    if (a.part == nullptr || a.cnt == nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_mxf<F, TM, WPB, SBW, true, false>), grid, dim3(64 * WPB), p.lds, st, sa);
  } else {
    hipLaunchKernelGGL((k_mxf<F, TM, WPB, SBW, false, false>), grid, dim3(64 * WPB), p.lds, st, sa);
  }
  return hipGetLastError();
}

template <int F, int TM>
static hipError_t run_mxf_shape(const MatvecLaunch& a, const MxfPlan& p, int wpb, int sbw, hipStream_t st) {
  if (wpb == 16 && sbw == 2) return run_mxf<F, TM, 16, 2>(a, p, st);
  if (wpb == 16 && sbw == 4) return run_mxf<F, TM, 16, 4>(a, p, st);
  if (wpb == 8 && sbw == 4) return run_mxf<F, TM, 8, 4>(a, p, st);
  if (wpb == 8 && sbw == 8) return run_mxf<F, TM, 8, 8>(a, p, st);
  return hipErrorInvalidValue;
}

#ifndef QMV_MX_FMT
#error "compile qmv_mxf.hip with -DQMV_MX_FMT=<format id>"
#endif
template <>
hipError_t launch_mxf_fmt<QMV_MX_FMT>(const MatvecLaunch& a, const MxfPlan& p, hipStream_t st) {
  const Variant& v = kVariants[a.variant];
  if (a.n_tok <= 4) return run_mxf_shape<QMV_MX_FMT, 4>(a, p, v.wpb, v.nu, st);
  if (a.n_tok <= 8) return run_mxf_shape<QMV_MX_FMT, 8>(a, p, v.wpb, v.nu, st);
  return run_mxf_shape<QMV_MX_FMT, 16>(a, p, v.wpb, v.nu, st);
}

#if QMV_MX_FMT == 0
hipError_t launch_mxf(const MatvecLaunch& a, const MxfPlan& p, hipStream_t st) {
  switch (a.fmt) {
    case FQ8_0: return launch_mxf_fmt<FQ8_0>(a, p, st);
    case FQ4_K: return launch_mxf_fmt<FQ4_K>(a, p, st);
    case FIQ4_XS: return launch_mxf_fmt<FIQ4_XS>(a, p, st);
    case FQ8G128: return launch_mxf_fmt<FQ8G128>(a, p, st);
    default: return hipErrorInvalidValue;
  }
}
#endif

}  // namespace qmv
