// qmv_matvec.hip -- dense small-batch matvec kernels for gfx950.
//
// The kernels compute y[t][n] = sum_k W[n][k] x[t][k] from the block weights
// and the Q8 activation buffer; each decoded weight unit serves every token of
// the batch (one weight read for the whole verify batch: zhuai.tech GLM-5.3
// page, "MTP saves full-model execution rounds").  All of them apply units in
// the own-block form of qmv_device.h.
//
// k_flat (one or a few tokens): one wave per row group, the whole grid at
// once, every weight load of the wave issued up front.
//
// k_mt (several tokens): lane groups with LDS-staged activations, chunked so
// that any K fits.
//
// k_stream: persistent waves over (row group, chunk) jobs with the activation
// buffer copied once per workgroup into LDS.  Lane l of a wave takes units
// c*64*NU + l + 64*i (i < NU) of each of the group's rows, so each weight load
// of the wave is one contiguous, fully used span, and the next job's loads
// stay in flight while the current one is computed; every load is
// unconditional (positions past the end re-read a valid unit and carry zero
// scales), so the load counter never has to drain early.  Teams of KS waves
// share a row group and split its chunks (split-K inside one workgroup,
// reduced through LDS: no workspace, no cross-workgroup synchronisation) --
// used for few rows and long K (Castagna Veloce page, "Kernels for the MI50":
// Q8_0 matvec with a split-K variant).
//
// k_matvec (lane groups of LPR lanes per row, activations read from global
// memory) remains for A/B comparison and for the cross-workgroup split-K path
// that runs when the caller passes a workspace and forces slices.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

// -------------------------------------------------------- lane-group kernel
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

  // ub and ue are even (slices are multiples of eight units), so both lanes
  // of every pair run the same iterations
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
    DecO<F> dec[R];
#pragma unroll
    for (int r = 0; r < R; ++r) decode_own(cur[r], u, gl & 1, true, dec[r]);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < n_tok) {
        XO xo;
        load_xo<F>(x, t, u, xo);
        int dv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) dv[r] = own_pass<F>(own_first(dec[r], xo.f));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][t] = own_apply(dec[r], own_second(dec[r], xo.s, dv[r]), xo.p, acc[r][t]);
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
    // Partials are stored and loaded with device-scope atomic accesses (the
    // gfx950 L2 writes them through and reloads them), so waiting for this
    // lane's stores before the barrier and the counter update is enough; a
    // device-scope fence would write back and invalidate the XCD's L2 once
    // per workgroup.
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt, lgkmcnt all zero
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = atomicAdd(&cnt[blockIdx.x], 1);
      s_last = (prev == (int)gridDim.y - 1);
    }
    __syncthreads();
    if (s_last) {
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

// ------------------------------------------------------- streaming kernel
template <int F, int TM, int R, int NU, int WPB, int KS, bool SEG>
__global__ __launch_bounds__(64 * WPB) void k_stream(StreamArgs a) {
  static_assert(KS == 1 || KS == WPB, "a team is one wave or the whole workgroup");
  static_assert(R * TM <= 64, "one output per lane");
  constexpr int CH = 64 * NU;
  constexpr int TPB = WPB / KS;  // teams per workgroup
  constexpr int NT = 64 * WPB;
  extern __shared__ __attribute__((aligned(16))) uint8_t s_mem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int team = blockIdx.x * TPB + wave / KS;
  const int n_teams = gridDim.x * TPB;
  const int kw = wave % KS;
  const int n_groups = (a.n_rows + R - 1) / R;
  const int nch = (a.units + CH - 1) / CH;
  const int mpw = (nch + KS - 1) / KS;  // chunks of one group per wave
  const int my_groups = team < n_groups ? (n_groups - 1 - team) / n_teams + 1 : 0;
  const int jobs = my_groups * mpw;
  const int units = a.units;

  // job j of this wave -> (row group, chunk)
  auto job = [&](int j, int& g, int& c) {
    const int i = j / mpw;
    g = team + i * n_teams;
    c = kw + KS * (j - i * mpw);
  };
  auto load_job = [&](int j, RawS<F> (&buf)[R][NU]) {
    int g, c;
    job(j, g, c);
    const RowSeg sg = row_seg<SEG>(a, g * R);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint8_t* wr = seg_wrow(sg, a.row_bytes, g * R + r);
#pragma unroll
      for (int q = 0; q < NU; ++q) load_unit_s(wr, min(c * CH + lane + 64 * q, units - 1), lane, buf[r][q]);
    }
  };

  // Stage the activation buffer (qs | d | s, the library layout) in LDS.
  // Vector-memory loads retire in issue order, so the first SBS pieces of
  // each thread (cache-resident) are loaded ahead of the first job's weights
  // with clamped indices: the LDS copy and its barrier then complete while
  // the weights are in flight instead of after them.
  constexpr int SBS = 6;
  const int n16 = a.act_bytes >> 4;
  u32x4 sv[SBS];
#pragma unroll
  for (int i = 0; i < SBS; ++i) sv[i] = ld16(a.xq + 16 * (int64_t)min((int)threadIdx.x + i * NT, n16 - 1));
  __builtin_amdgcn_sched_barrier(0);
  RawS<F> cur[R][NU];
  if (jobs > 0) load_job(0, cur);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < SBS; ++i) {
    const int idx = threadIdx.x + i * NT;
    if (idx < n16) reinterpret_cast<u32x4a*>(s_mem)[idx] = sv[i];
  }
  for (int idx = threadIdx.x + SBS * NT; idx < n16; idx += NT)  // large buffers
    reinterpret_cast<u32x4a*>(s_mem)[idx] = ld16(a.xq + 16 * (int64_t)idx);
  __syncthreads();
  const Act x{reinterpret_cast<const int8_t*>(s_mem),
              reinterpret_cast<const float*>(s_mem + a.off_d),
              reinterpret_cast<const int32_t*>(s_mem + a.off_s), a.k, a.nb};
  float* red = reinterpret_cast<float*>(s_mem + a.act_bytes);  // [KS][R*TM]

  float acc[R][TM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[r][t] = 0.f;

  for (int j = 0; j < jobs; ++j) {
    RawS<F> nxt[R][NU];
    load_job(min(j + 1, jobs - 1), nxt);
    int g, c;
    job(j, g, c);
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      const int uraw = c * CH + lane + 64 * q;
      const bool ok = uraw < units;
      const int u = ok ? uraw : units - 1;
      DecO<F> dec[R];
#pragma unroll
      for (int r = 0; r < R; ++r) decode_own(cur[r][q], u, lane & 1, ok, dec[r]);
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        XO xo;
        load_xo<F>(x, t < a.n_tok ? t : a.n_tok - 1, u, xo);
        int dv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) dv[r] = own_pass<F>(own_first(dec[r], xo.f));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][t] = own_apply(dec[r], own_second(dec[r], xo.s, dv[r]), xo.p, acc[r][t]);
      }
    }
    if (j % mpw == mpw - 1) {  // last chunk of the group: reduce and store
      float outv = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          const float sv = wave_sum(acc[r][t]);
          outv = lane == r * TM + t ? sv : outv;
          acc[r][t] = 0.f;
        }
      const int r = lane / TM, t = lane % TM;
      const int row = g * R + r;
      const RowSeg sg = row_seg<SEG>(a, g * R);
      if constexpr (KS == 1) {
        if (lane < R * TM && t < a.n_tok) seg_store(sg, t, row, outv);
      } else {
        if (lane < R * TM) red[kw * R * TM + lane] = outv;
        __syncthreads();
        if (threadIdx.x < R * TM) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < KS; ++w) sum += red[w * R * TM + threadIdx.x];
          const int rr = threadIdx.x / TM, tt = threadIdx.x % TM;
          const int row2 = g * R + rr;
          if (tt < a.n_tok) seg_store(sg, tt, row2, sum);
        }
        __syncthreads();
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int q = 0; q < NU; ++q) cur[r][q] = nxt[r][q];
  }
}

// ------------------------------------------------------------ flat kernel
// One wave per group of R rows, launched for every group at once (no
// persistent loop): the wave issues all the weight loads of its first chunk
// of 64*NU units (one chunk covers the row in the configurations it is
// chosen for) and, with XL false, the activation fragments of the chunk right
// behind them, so both latencies overlap; then it decodes, reduces with DPP
// and stores.  XL true stages the activation buffer in LDS per workgroup
// instead (for token counts whose fragments would not fit in registers).
//
// QX (with XL, one or two tokens): the workgroup makes the Q8 activation
// blocks itself from fp32 x, straight into the LDS copy, with the same block
// routine as the quantizer kernel (so the blocks are identical).  Its x loads
// go out before the weight loads and the quantization runs while the weights
// are on their way; workgroup 0 also writes the blocks to a.xq_out.
template <int F, int TM, int R, int NU, int WPB, bool XL, int OCC, bool SEG, int QXP = 0, bool SPLIT = false>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(1, OCC))) void k_flat(StreamArgs a) {
  static_assert(R * TM <= 64, "one output per lane");
  constexpr bool QX = QXP > 0;  // QXP: x passes held in registers ahead of the weight loads
  static_assert(!QX || (XL && !SEG), "quantizing into the LDS copy");
  // SPLIT: K split over workgroups -- workgroup column y covers units
  // y * ups .. +ups (one chunk) of its rows, stages only that slice of the
  // activations, and writes fp32 partials that the column's last workgroup
  // sums in slice order (the arrival protocol of k_matvec)
  static_assert(!SPLIT || (XL && !SEG && !QX), "a split launch stages a slice of one matrix's activations");
  constexpr int QP = QX ? QXP : 1;
  constexpr int CH = 64 * NU;
  constexpr int NT = 64 * WPB;
  constexpr int TX = XL ? 1 : TM;  // prefetched fragments per unit
  extern __shared__ __attribute__((aligned(16))) uint8_t s_mem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar row bases
  const int row0 = (blockIdx.x * WPB + wave) * R;
  // SPLIT: unit indices below are relative to the slice's first unit ub
  const int ub = SPLIT ? (int)blockIdx.y * a.ups : 0;
  const int units = SPLIT ? min(a.ups, a.units - ub) : a.units;
  const int nch = (units + CH - 1) / CH;
  const RowSeg sg = row_seg<SEG>(a, row0);
  const uint8_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    wr[r] = seg_wrow(sg, a.row_bytes, row0 + r) + (SPLIT ? (int64_t)(ub / Fmt<F>::UPB) * Fmt<F>::BB : 0);

  const Act gx{reinterpret_cast<const int8_t*>(a.xq), reinterpret_cast<const float*>(a.xq + a.off_d),
               reinterpret_cast<const int32_t*>(a.xq + a.off_s), a.k, a.nb};
  // the LDS copy: the whole buffer, or (SPLIT) the slice's quants [T][ups * 32]
  // then its d [T][ups] and s [T][ups]
  const int sk = SPLIT ? a.ups * 32 : a.k, snb = SPLIT ? a.ups : a.nb;
  const int soff_d = SPLIT ? a.n_tok * sk : a.off_d;
  const int soff_s = SPLIT ? soff_d + a.n_tok * snb * 4 : a.off_s;
  const Act lx{reinterpret_cast<const int8_t*>(s_mem), reinterpret_cast<const float*>(s_mem + soff_d),
               reinterpret_cast<const int32_t*>(s_mem + soff_s), sk, snb};
  XO xf[NU][TX];
  // Load order.  Vector-memory loads complete in issue order, so the small,
  // cache-resident activation loads go first -- the fragments themselves, or
  // the first batch of the LDS copy -- and the weight units follow in the
  // order they are computed: unit q can then be decoded while units q+1.. are
  // still on their way from HBM, and the LDS copy is written (and its
  // barrier passed) while all the weights are.  Scheduling barriers keep the
  // compiler from interleaving the phases.  The first batch is loaded
  // unconditionally with clamped indices: a branch around a load makes the
  // compiler wait for its value where the branches join.
  const int n16 = a.act_bytes >> 4;  // LDS copy: 16-byte pieces
  u32x4 stg[4];
  // QX: block p * (NT / 8) + threadIdx.x / 8 of the n_tok * nb blocks, four
  // values per lane (clamped to the last block: the loads stay unconditional)
  const int q_blocks = a.n_tok * a.nb;
  const int q_passes = (q_blocks + NT / 8 - 1) / (NT / 8);
  f32x4 xv[QX ? QP : 1];
  auto x_piece = [&](int p) -> const float* {
    const int blk = min(p * (NT / 8) + ((int)threadIdx.x >> 3), q_blocks - 1);
    const int t = blk / a.nb, b = blk - t * a.nb;
    return a.x + (int64_t)t * a.ldx + 32 * b + 4 * ((int)threadIdx.x & 7);
  };
  // SPLIT staging: pq 16-byte quant pieces per token and one (d, s) pair per
  // unit and token; the first batch (four pieces, one pair per thread) is
  // loaded here, ahead of the weights, with clamped indices
  const int pq = 2 * units, nq = a.n_tok * pq, ns = a.n_tok * units;
  const float* gd = reinterpret_cast<const float*>(a.xq + a.off_d);
  const int32_t* gs = reinterpret_cast<const int32_t*>(a.xq + a.off_s);
  auto sq_src = [&](int idx) -> const uint8_t* {
    const int t = idx / pq, p = idx - t * pq;
    return a.xq + (int64_t)t * a.k + 32 * ub + 16 * p;
  };
  auto sq_dst = [&](int idx) -> u32x4a* {
    const int t = idx / pq, p = idx - t * pq;
    return reinterpret_cast<u32x4a*>(s_mem + t * sk + 16 * p);
  };
  auto ss_src = [&](int idx) -> int {
    const int t = idx / units;
    return t * a.nb + ub + (idx - t * units);
  };
  auto ss_dst = [&](int idx) -> int {
    const int t = idx / units;
    return t * snb + (idx - t * units);
  };
  float sdv = 0.f;
  int32_t ssv = 0;
  if constexpr (QX) {
#pragma unroll
    for (int p = 0; p < QP; ++p) xv[p] = *reinterpret_cast<const f32x4*>(x_piece(min(p, q_passes - 1)));
  } else if constexpr (SPLIT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) stg[i] = ld16(sq_src(min((int)threadIdx.x + i * NT, nq - 1)));
    const int si = ss_src(min((int)threadIdx.x, ns - 1));
    sdv = gd[si];
    ssv = gs[si];
  } else if constexpr (XL) {
#pragma unroll
    for (int i = 0; i < 4; ++i) stg[i] = ld16(a.xq + 16 * (int64_t)min((int)threadIdx.x + i * NT, n16 - 1));
  } else {
#pragma unroll
    for (int q = 0; q < NU; ++q)
#pragma unroll
      for (int t = 0; t < TM; ++t)
        load_xo<F>(gx, t < a.n_tok ? t : a.n_tok - 1, min(lane + 64 * q, units - 1), xf[q][t]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // Unit order: each unit's loads, and later its decode and dot products,
  // are kept apart from the next unit's, so a unit is consumed as soon as its
  // own loads have arrived rather than when the compiler's interleaving
  // first needs a later one.  At one token (q4_K 14336 x 4096 7.78 -> 7.60
  // us, Q8_0 4096 x 4096 5.15 -> 4.96, the Q8_0 head 133.0 -> 126.0) and for
  // q4_K, IQ4_XS and q6_K at two (q4_K 8.37 -> 8.05 on two of three GPUs,
  // 8.68 -> 8.83 on the third; q6_K 14.2 -> 13.9).  Elsewhere it was slower:
  // q6_K at four tokens 15.7 -> 16.7 us, Q8_0 rows of 14336 weights at two
  // 13.41 -> 13.67, the quantizing launch (two tokens 11.6 -> 12.1).
  constexpr bool in_order = !QX && (TM == 1 || (TM == 2 && (F == FQ4_K || F == FIQ4_XS || F == FQ6_K)));
  RawS<F> cur[R][NU];
#pragma unroll
  for (int q = 0; q < NU; ++q) {
#pragma unroll
    for (int r = 0; r < R; ++r) load_unit_s(wr[r], min(lane + 64 * q, units - 1), lane, cur[r][q]);
    if constexpr (in_order) __builtin_amdgcn_sched_barrier(0);
  }
  // batched launches: the residual of the lane's output, loaded right behind
  // the weights and unconditionally (a branch around a load would wait for
  // every load before it): with no residual the same valid address of the
  // output is read and its value ignored
  float rv = 0.f;
  if constexpr (SEG) {
    const int o_r = lane < R * TM ? lane / TM : 0, o_t = min(lane % TM, a.n_tok - 1);
    const int o_lr = min(row0 - sg.first + o_r, sg.rows - 1);
    const float* rp = sg.res != nullptr ? sg.res + (int64_t)o_t * sg.ldr + o_lr : sg.y + (int64_t)o_t * sg.ldy + o_lr;
    rv = *rp;
  }
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (QX) {
    auto put = [&](int p, const f32x4& v) {
      const int blk = p * (NT / 8) + ((int)threadIdx.x >> 3);
      const float vv[4] = {v.x, v.y, v.z, v.w};
      float db;
      int sum;
      const uint32_t packed = q8_block8(vv, db, sum);
      if (blk < q_blocks) {
        const int t = blk / a.nb, b = blk - t * a.nb, j = (int)threadIdx.x & 7;
        const int qo = t * a.k + 32 * b + 4 * j;
        *reinterpret_cast<uint32_t*>(s_mem + qo) = packed;
        if (j == 0) {
          reinterpret_cast<float*>(s_mem + a.off_d)[blk] = db;
          reinterpret_cast<int32_t*>(s_mem + a.off_s)[blk] = sum;
        }
        if (a.xq_out != nullptr && blockIdx.x == 0) {
          *reinterpret_cast<uint32_t*>(a.xq_out + qo) = packed;
          if (j == 0) {
            reinterpret_cast<float*>(a.xq_out + a.off_d)[blk] = db;
            reinterpret_cast<int32_t*>(a.xq_out + a.off_s)[blk] = sum;
          }
        }
      }
    };
#pragma unroll
    for (int p = 0; p < QP; ++p)
      if (p < q_passes) put(p, xv[p]);
    for (int p = QP; p < q_passes; ++p) put(p, *reinterpret_cast<const f32x4*>(x_piece(p)));  // long rows
    __syncthreads();
  } else if constexpr (SPLIT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = threadIdx.x + i * NT;
      if (idx < nq) *sq_dst(idx) = stg[i];
    }
    for (int idx = threadIdx.x + 4 * NT; idx < nq; idx += NT) *sq_dst(idx) = ld16(sq_src(idx));
    float* ld = reinterpret_cast<float*>(s_mem + soff_d);
    int32_t* ls = reinterpret_cast<int32_t*>(s_mem + soff_s);
    if ((int)threadIdx.x < ns) {
      ld[ss_dst(threadIdx.x)] = sdv;
      ls[ss_dst(threadIdx.x)] = ssv;
    }
    for (int idx = threadIdx.x + NT; idx < ns; idx += NT) {
      ld[ss_dst(idx)] = gd[ss_src(idx)];
      ls[ss_dst(idx)] = gs[ss_src(idx)];
    }
    __syncthreads();
  } else if constexpr (XL) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = threadIdx.x + i * NT;
      if (i * NT < n16 && idx < n16) reinterpret_cast<u32x4a*>(s_mem)[idx] = stg[i];
    }
    for (int idx = threadIdx.x + 4 * NT; idx < n16; idx += NT)  // large buffers
      reinterpret_cast<u32x4a*>(s_mem)[idx] = ld16(a.xq + 16 * (int64_t)idx);
    __syncthreads();
  }

  float acc[R][TM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[r][t] = 0.f;

  for (int c = 0; c < nch; ++c) {
    if (c > 0) {  // rows longer than one chunk: plain (unpipelined) loads
#pragma unroll
      for (int q = 0; q < NU; ++q)
#pragma unroll
        for (int r = 0; r < R; ++r)
          load_unit_s(wr[r], min(c * CH + lane + 64 * q, units - 1), lane, cur[r][q]);
    }
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      if (in_order && q > 0) __builtin_amdgcn_sched_barrier(0);
      const int uraw = c * CH + lane + 64 * q;
      const bool ok = uraw < units;
      const int u = ok ? uraw : units - 1;
      // the decode takes the unclamped index: it uses it only for the unit's
      // place in its super-block, which for a valid unit is the same, and
      // here is the lane's own (c * CH and 64 q are multiples of 64), so the
      // header field offsets are fixed per lane; a clamped unit's scales are
      // zero whatever it decodes
      DecO<F> dec[R];
#pragma unroll
      for (int r = 0; r < R; ++r) decode_own(cur[r][q], uraw, lane & 1, ok, dec[r]);
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int tt = t < a.n_tok ? t : a.n_tok - 1;
        XO f;
        if constexpr (XL)
          load_xo<F>(lx, tt, u, f);
        else if (c == 0)
          f = xf[q][t];
        else
          load_xo<F>(gx, tt, u, f);
        int dv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) dv[r] = own_pass<F>(own_first(dec[r], f.f));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][t] = own_apply(dec[r], own_second(dec[r], f.s, dv[r]), f.p, acc[r][t]);
      }
    }
  }

  float outv = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const float sv = wave_sum(acc[r][t]);
      outv = lane == r * TM + t ? sv : outv;
    }
  const int r = lane / TM, t = lane % TM;
  const int lr = row0 + r - sg.first;
  if constexpr (SPLIT) {
    if (lane < R * TM && t < a.n_tok && lr < sg.rows)
      __hip_atomic_store(&a.part[((int64_t)blockIdx.y * a.n_tok + t) * a.n_rows + lr], outv, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    // The column's last workgroup sums the slices in slice order.  The
    // partials are device-scope atomic accesses (written through and
    // reloaded by the L2), so each lane only waits for its stores to be
    // acknowledged before the barrier and the counter update; a device-scope
    // fence would write back and invalidate the XCD's L2.
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt, lgkmcnt all zero
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(&a.cnt[blockIdx.x], 1) == (int)gridDim.y - 1;
    __syncthreads();
    if (s_last) {
      constexpr int RW = WPB * R;
      const int r0 = (int)blockIdx.x * RW;
      for (int q = threadIdx.x; q < a.n_tok * RW; q += NT) {
        const int tq = q / RW, row = r0 + (q - tq * RW);
        if (row < a.n_rows) {
          float sum = 0.f;
          for (int sl = 0; sl < (int)gridDim.y; ++sl)
            sum += __hip_atomic_load(&a.part[((int64_t)sl * a.n_tok + tq) * a.n_rows + row], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          a.y[(int64_t)tq * a.ldy + row] = sum;
        }
      }
      if (threadIdx.x == 0) atomicExch(&a.cnt[blockIdx.x], 0);
    }
  } else if (lane < R * TM && t < a.n_tok && lr < sg.rows) {
    sg.y[(int64_t)t * sg.ldy + lr] = SEG && sg.res != nullptr ? outv + rv : outv;
  }
}

// ------------------------------------------------------ multi-token kernel
// For verify batches (several tokens).  A lane group of 16 lanes owns R rows
// and walks them one unit per lane per iteration (each weight load of a group
// is one contiguous 256-byte span); a wave holds four such groups.  A team of
// KS waves shares the same rows and splits the iterations (partial sums meet
// in LDS at the end), which multiplies the waves in flight when rows are few
// or tokens many.  The activations are staged in LDS chunk by chunk (kc units
// of every token at a time, all waves of the workgroup in step), and the next
// iteration's weight loads are issued before the current one is computed,
// across chunk boundaries too.  Each decoded unit is applied to every token
// and each activation run to the R rows, in the own-block form: eight v_dot4,
// one DPP move (q4_K) and one fp32 scale step per (row, token, unit); units
// past the row end carry zero scales instead of a per-token select.  The LDS
// chunk holds, per unit, the first and the second activation run of every
// token and the (d, d*s) pair of its 32-block, token-minor with an odd token
// stride: a lane finds all its tokens at fixed offsets from one address, and
// the 16 lanes of a group, which read 16 consecutive units, cover every LDS
// bank once (the four groups of a wave read the same addresses).
template <int TM>
constexpr int mt_stride() { return TM % 2 == 0 ? TM + 1 : TM; }

template <int F, int TM, int R, int NU, int WPB, int KS, bool SEG>
__global__ __launch_bounds__(64 * WPB) void k_mt(StreamArgs a) {
  constexpr int LPR = 16, GPW = 4;
  constexpr int STEP = LPR * NU;  // units a lane group covers per iteration
  static_assert(R * TM <= 64 && WPB % KS == 0, "layout");
  constexpr int TEAMS = WPB / KS;
  constexpr int NT = 64 * WPB;
  constexpr int NV = R * TM;
  constexpr int US = mt_stride<TM>();  // token slots per unit
  extern __shared__ __attribute__((aligned(16))) uint8_t s_mem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int team = wave / KS, kw = wave % KS;
  const int g = lane / LPR, gl = lane % LPR, h = lane & 1;
  const int row0 = ((blockIdx.x * TEAMS + team) * GPW + g) * R;
  const int units = a.units, kc = a.kc, T = a.n_tok;
  const int ipc = kc / STEP;
  const int nchunk = (units + kc - 1) / kc;
  // a workgroup's rows (at most 64, a power of two) lie in one matrix
  const RowSeg sg = row_seg<SEG>(a, (int)blockIdx.x * TEAMS * GPW * R);
  const uint8_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = seg_wrow(sg, a.row_bytes, row0 + r);

  // LDS chunk: first runs [kc][US] x 16 B | second runs [kc][US] x 16 B |
  // (d, d*s) [kc][US] x 8 B; then the team partials
  u32x4a* ld_f = reinterpret_cast<u32x4a*>(s_mem);
  u32x4a* ld_s = ld_f + kc * US;
  float2* ld_p = reinterpret_cast<float2*>(ld_s + kc * US);
  float* red = reinterpret_cast<float*>(s_mem + kc * US * 40);
  const float* gd = reinterpret_cast<const float*>(a.xq + a.off_d);
  const int32_t* gs = reinterpret_cast<const int32_t*>(a.xq + a.off_s);

  auto load_it = [&](int c, int cit, RawS<F> (&buf)[R][NU]) {
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      const int u = min(c * kc + cit * STEP + gl + LPR * q, units - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) load_unit_s(wr[r], u, lane, buf[r][q]);
    }
  };
  auto stage = [&](int c) {
    const int c0 = c * kc, cu = min(kc, units - c0);
    const int nq = 2 * cu;  // 16-byte pieces of one token's quants in the chunk
    const FastDiv dq(nq), du(cu);
    for (int base = 0; base < T * nq; base += 4 * NT) {
      u32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = base + threadIdx.x + i * NT;
        const int t = dq.div(idx), pc = idx - t * nq;
        if (idx < T * nq) v[i] = ld16(a.xq + (int64_t)t * a.k + 32 * c0 + 16 * pc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = base + threadIdx.x + i * NT;
        const int t = dq.div(idx), pc = idx - t * nq;
        int un, run;
        own_piece_slot<F>(pc >> 1, pc & 1, un, run);
        if (idx < T * nq) (run ? ld_s : ld_f)[un * US + t] = v[i];
      }
    }
    for (int idx = threadIdx.x; idx < T * cu; idx += NT) {
      const int t = du.div(idx), pc = idx - t * cu;
      const float d = gd[(int64_t)t * a.nb + c0 + pc];
      const int sx = gs[(int64_t)t * a.nb + c0 + pc];
      ld_p[pc * US + t] = make_float2(d, d * static_cast<float>(sx));
    }
  };

  float acc[R][TM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[r][t] = 0.f;

  RawS<F> cur[R][NU];
  load_it(0, kw, cur);
  for (int c = 0; c < nchunk; ++c) {
    __syncthreads();  // every wave is done with the previous chunk
    stage(c);
    __syncthreads();
    for (int cit = kw; cit < ipc; cit += KS) {
      int nc = c, ncit = cit + KS;
      if (ncit >= ipc) {
        nc = c + 1 < nchunk ? c + 1 : c;
        ncit = c + 1 < nchunk ? kw : cit;
      }
      RawS<F> nxt[R][NU];
      load_it(nc, ncit, nxt);
#pragma unroll
      for (int q = 0; q < NU; ++q) {
        const int ul = cit * STEP + gl + LPR * q;  // unit inside the chunk
        const int uraw = c * kc + ul;
        const bool ok = uraw < units;
        const int u = ok ? uraw : units - 1;
        const int li = ok ? ul : 0;  // a staged slot, for units past the end
        DecO<F> dec[R];
#pragma unroll
        for (int r = 0; r < R; ++r) decode_own(cur[r][q], u, h, ok, dec[r]);
        const u32x4a* pf = ld_f + li * US;
        const u32x4a* ps = ld_s + li * US;
        const float2* pp = ld_p + li * US;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          // token slots past the call's token count (t >= T) hold stale LDS
          // bytes: they only feed acc[.][t], which is never stored
          const u32x4 xf = pf[t];
          const u32x4 xs = ps[t];
          const float2 p = pp[t];
          int dv[R];
#pragma unroll
          for (int r = 0; r < R; ++r) dv[r] = own_first(dec[r], xf);
#pragma unroll
          for (int r = 0; r < R; ++r) dv[r] = own_pass<F>(dv[r]);
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r][t] = own_apply(dec[r], own_second(dec[r], xs, dv[r]), p, acc[r][t]);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < NU; ++q) cur[r][q] = nxt[r][q];
    }
  }

  if constexpr (KS == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const float v = lane_group_sum<LPR>(acc[r][t]);
        if (((r * TM + t) % LPR) == gl && t < T) seg_store(sg, t, row0 + r, v);
      }
  } else {
    float* mine = red + ((team * KS + kw) * GPW + g) * NV;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const float v = lane_group_sum<LPR>(acc[r][t]);
        if (((r * TM + t) % LPR) == gl) mine[r * TM + t] = v;
      }
    __syncthreads();
    for (int i = threadIdx.x; i < TEAMS * GPW * NV; i += NT) {
      const int tm = i / (GPW * NV), rest = i - tm * (GPW * NV);
      const int gg = rest / NV, v = rest - gg * NV;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < KS; ++w) sum += red[((tm * KS + w) * GPW + gg) * NV + v];
      const int r = v / TM, t = v % TM;
      const int row = ((blockIdx.x * TEAMS + tm) * GPW + gg) * R + r;
      if (t < T) seg_store(sg, t, row, sum);
    }
  }
}

template <int F, int TM, int LPR, int R>
static hipError_t run_mv(const MatvecLaunch& a, hipStream_t st) {
  constexpr int RWG = 4 * (64 / LPR) * R;
  const unsigned tiles = (unsigned)((a.n_rows + RWG - 1) / RWG);
  if (a.slices > 1) {
    // units per slice, a multiple of eight so that every slice starts on a
    // super-block (lane pairs and header quads stay inside one slice)
    const int ups = ((a.units + a.slices - 1) / a.slices + 7) & ~7;
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

// ------------------------------------------------------- long-row kernel
// Few rows, long K (a few hundred rows of tens of thousands of weights): a
// workgroup of WPB waves takes one group of R rows and its waves split K,
// wave w taking chunks w, w + WPB, .. of 64 * NU units (one chunk each in the
// shapes it is chosen for).  Each wave loads the activation fragments of its
// own chunk straight from global memory, ahead of its weight loads (vector
// loads return in issue order, and the fragments are cache-resident after
// the first workgroups), so no workgroup copies the whole activation buffer
// into LDS: on 256 x 65536 Q8_0 rows that per-workgroup copy, 82 KB for each
// of 256 workgroups, moved more bytes than the weights.  The waves' sums meet
// in LDS and are added in wave order.  One matrix per launch (no segments,
// no residual).
template <int F, int TM, int R, int NU, int WPB>
__global__ __launch_bounds__(64 * WPB) void k_long(StreamArgs a) {
  static_assert(R * TM <= 64 && TM <= 4, "one output per lane, fragments in registers");
  constexpr int CH = 64 * NU;
  __shared__ float red[WPB * R * TM];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = (int)blockIdx.x * R;
  const int units = a.units;
  const int nch = (units + CH - 1) / CH;
  const int mine = wave < nch ? (nch - 1 - wave) / WPB + 1 : 0;  // chunks of this wave
  const Act gx{reinterpret_cast<const int8_t*>(a.xq), reinterpret_cast<const float*>(a.xq + a.off_d),
               reinterpret_cast<const int32_t*>(a.xq + a.off_s), a.k, a.nb};
  const uint8_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = a.w + (int64_t)min(row0 + r, a.n_rows - 1) * a.row_bytes;

  float acc[R][TM];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[r][t] = 0.f;

  for (int i = 0; i < mine; ++i) {
    const int c = wave + WPB * i;
    XO xf[NU][TM];
#pragma unroll
    for (int q = 0; q < NU; ++q)
#pragma unroll
      for (int t = 0; t < TM; ++t)
        load_xo<F>(gx, t < a.n_tok ? t : a.n_tok - 1, min(c * CH + lane + 64 * q, units - 1), xf[q][t]);
    __builtin_amdgcn_sched_barrier(0);
    // With two units per lane, each unit's loads and then its dot products
    // stay in unit order, so a unit is consumed as soon as its own loads have
    // arrived (Q8_0 256 x 65536 at one token: 6.08 -> 5.84 us); with four,
    // the compiler's interleaving is faster (6.10 against 6.36 us).
    constexpr bool in_order = NU <= 2;
    RawS<F> cur[R][NU];
#pragma unroll
    for (int q = 0; q < NU; ++q) {
#pragma unroll
      for (int r = 0; r < R; ++r) load_unit_s(wr[r], min(c * CH + lane + 64 * q, units - 1), lane, cur[r][q]);
      if (in_order || q == NU - 1) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      if (in_order && q > 0) __builtin_amdgcn_sched_barrier(0);
      const int uraw = c * CH + lane + 64 * q;
      const bool ok = uraw < units;
      const int u = ok ? uraw : units - 1;
      DecO<F> dec[R];
#pragma unroll
      for (int r = 0; r < R; ++r) decode_own(cur[r][q], u, lane & 1, ok, dec[r]);
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        int dv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) dv[r] = own_pass<F>(own_first(dec[r], xf[q][t].f));
#pragma unroll
        for (int r = 0; r < R; ++r)
          acc[r][t] = own_apply(dec[r], own_second(dec[r], xf[q][t].s, dv[r]), xf[q][t].p, acc[r][t]);
      }
    }
  }

  float outv = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const float sv = wave_sum(acc[r][t]);
      outv = lane == r * TM + t ? sv : outv;
    }
  if (lane < R * TM) red[wave * R * TM + lane] = outv;
  __syncthreads();
  if (threadIdx.x < R * TM) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WPB; ++w) sum += red[w * R * TM + threadIdx.x];
    const int r = threadIdx.x / TM, t = threadIdx.x % TM;
    if (t < a.n_tok && row0 + r < a.n_rows) a.y[(int64_t)t * a.ldy + row0 + r] = sum;
  }
}

static StreamArgs stream_args(const MatvecLaunch& a) {
  StreamArgs sa;
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
  sa.kc = 0;
  sa.res = a.res;
  sa.ldr = a.ldr;
  sa.seg = a.seg;
  sa.x = nullptr;
  sa.ldx = 0;
  sa.xq_out = nullptr;
  sa.ups = 0;
  sa.part = nullptr;
  sa.cnt = nullptr;
  sa.dots = nullptr;
  return sa;
}

template <int F, int TM, int R, int NU, int WPB, int KS, bool SEG>
static hipError_t run_stream_seg(const MatvecLaunch& a, hipStream_t st) {
  auto kern = k_stream<F, TM, R, NU, WPB, KS, SEG>;
  const size_t lds = (size_t)a.act_bytes + (size_t)KS * R * TM * 4;
  // resident workgroups per CU allowed by registers and waves, measured once
  static const int occ = [&] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 64 * WPB, 0) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  int bpc = blocks_per_cu() > 0 ? blocks_per_cu() : occ;
  const int by_lds = (int)((size_t)a.lds_per_cu / (lds > 0 ? lds : 1));
  if (bpc > by_lds) bpc = by_lds;
  if (bpc < 1) bpc = 1;
  constexpr int TPB = WPB / KS;
  const int64_t groups = (a.n_rows + R - 1) / R;
  const int64_t need = (groups + TPB - 1) / TPB;
  const int64_t cap = (int64_t)a.cus * bpc;
  const unsigned grid = (unsigned)(need < cap ? need : cap);
  StreamArgs sa = stream_args(a);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, st, sa);
  return hipGetLastError();
}

// Every launcher instantiates its kernel twice: for one matrix and for a
// batched launch with a segment table.
template <int F, int TM, int R, int NU, int WPB, int KS>
static hipError_t run_stream(const MatvecLaunch& a, hipStream_t st) {
  return a.seg.n > 0 ? run_stream_seg<F, TM, R, NU, WPB, KS, true>(a, st)
                     : run_stream_seg<F, TM, R, NU, WPB, KS, false>(a, st);
}

template <int F, int TM, int R, int NU, int WPB, bool XL, int OCC = 8>
static hipError_t run_flat(const MatvecLaunch& a, hipStream_t st) {
  if constexpr (!XL && TM > 4) {
    // fragments of more than four tokens do not fit in registers: stage them
    return run_flat<F, TM, R, NU, WPB, true, OCC>(a, st);
  } else {
    const size_t lds = XL ? (size_t)a.act_bytes : 0;
    const int64_t groups = (a.n_rows + R - 1) / R;
    const unsigned grid = (unsigned)((groups + WPB - 1) / WPB);
    StreamArgs sa = stream_args(a);
    if (a.qx) {
      // quantize-in-kernel launches: LDS-staged variants at one or two tokens
      if constexpr (XL && TM <= 2) {
        sa.x = a.xf;
        sa.ldx = a.ldx;
        sa.xq_out = const_cast<uint8_t*>(a.xq);
        const int passes = (int)((a.n_tok * (a.units) + 8 * WPB - 1) / (8 * WPB));  // 8 blocks per wave
        if (passes <= 1)
          hipLaunchKernelGGL((k_flat<F, TM, R, NU, WPB, XL, OCC, false, 1>), dim3(grid), dim3(64 * WPB), lds, st,
                             sa);
        else if (passes <= 2)
          hipLaunchKernelGGL((k_flat<F, TM, R, NU, WPB, XL, OCC, false, 2>), dim3(grid), dim3(64 * WPB), lds, st,
                             sa);
        else if (passes <= 4)
          hipLaunchKernelGGL((k_flat<F, TM, R, NU, WPB, XL, OCC, false, 4>), dim3(grid), dim3(64 * WPB), lds, st,
                             sa);
        else
          hipLaunchKernelGGL((k_flat<F, TM, R, NU, WPB, XL, OCC, false, 8>), dim3(grid), dim3(64 * WPB), lds, st,
                             sa);
      } else {
        return hipErrorInvalidValue;  // the entry point only sends XL variants at <= 2 tokens
      }
    } else if (a.seg.n > 0) {
      hipLaunchKernelGGL((k_flat<F, TM, R, NU, WPB, XL, OCC, true>), dim3(grid), dim3(64 * WPB), lds, st, sa);
    } else if (a.fslices > 1) {
      if constexpr (XL) {
        // K split over workgroups: a.fslices slices of a.fups units
        sa.ups = a.fups;
        sa.part = a.part;
        sa.cnt = a.cnt;
        const size_t lds_s = (size_t)a.n_tok * a.fups * 40;
        hipLaunchKernelGGL((k_flat<F, TM, R, NU, WPB, XL, OCC, false, 0, true>), dim3(grid, (unsigned)a.fslices),
                           dim3(64 * WPB), lds_s, st, sa);
      } else {
        return hipErrorInvalidValue;  // only LDS-staged variants split
      }
    } else {
      hipLaunchKernelGGL((k_flat<F, TM, R, NU, WPB, XL, OCC, false>), dim3(grid), dim3(64 * WPB), lds, st, sa);
    }
    return hipGetLastError();
  }
}

// Units per LDS chunk of the multi-token kernel: as many as fit the budget,
// a multiple of the units one iteration covers (and of 8, one super-block),
// balanced over the chunks the row needs.
static int multi_chunk_units(int units, int n_tok, int step, int64_t lds_budget) {
  const int per_unit = n_tok * 40;  // 32 quant bytes + scale + sum per token
  const int lcm = step % 8 == 0 ? step : step * 8;
  int kmax = (int)(lds_budget / per_unit) / lcm * lcm;
  if (kmax < lcm) return 0;  // does not fit
  const int need = (units + lcm - 1) / lcm * lcm;
  if (kmax >= need) return need;
  const int chunks = (units + kmax - 1) / kmax;
  const int per = (units + chunks - 1) / chunks;
  return (per + lcm - 1) / lcm * lcm;
}

template <int F, int TM, int R, int NU, int WPB, int KS>
static hipError_t run_mt(const MatvecLaunch& a, hipStream_t st) {
  StreamArgs sa = stream_args(a);
  constexpr int RWG = (WPB / KS) * 4 * R;  // rows per workgroup
  const int64_t red_bytes = KS > 1 ? (int64_t)WPB * 4 * R * TM * 4 : 0;
  constexpr int US = mt_stride<TM>();
  sa.kc = multi_chunk_units(a.units, US, 16 * NU, kMultiLdsBudget - red_bytes);
  if (sa.kc <= 0) return hipErrorInvalidValue;
  const size_t lds = (size_t)US * sa.kc * 40 + red_bytes;
  const unsigned grid = (unsigned)((a.n_rows + RWG - 1) / RWG);
  if (a.seg.n > 0)
    hipLaunchKernelGGL((k_mt<F, TM, R, NU, WPB, KS, true>), dim3(grid), dim3(64 * WPB), lds, st, sa);
  else
    hipLaunchKernelGGL((k_mt<F, TM, R, NU, WPB, KS, false>), dim3(grid), dim3(64 * WPB), lds, st, sa);
  return hipGetLastError();
}

// The long-row kernel takes one matrix and fragments of at most four tokens
// held in registers (R * NU * TM <= 8: more spills); a batched launch, or
// more tokens, runs the multi-token kernel mt_r2_w8_k4 instead (segments,
// and LDS staging chunked to fit any K).
template <int F, int TM, int R, int NU, int WPB>
static hipError_t run_long(const MatvecLaunch& a, hipStream_t st) {
  if constexpr (TM > 4 || R * NU * TM > 8) {
    return run_mt<F, TM, 2, 1, 8, 4>(a, st);
  } else {
    if (a.seg.n > 0) return run_mt<F, TM, 2, 1, 8, 4>(a, st);
    const unsigned grid = (unsigned)((a.n_rows + R - 1) / R);
    StreamArgs sa = stream_args(a);
    hipLaunchKernelGGL((k_long<F, TM, R, NU, WPB>), dim3(grid), dim3(64 * WPB), 0, st, sa);
    return hipGetLastError();
  }
}

template <int F, int TM>
static hipError_t run_mv_variant(const MatvecLaunch& a, hipStream_t st) {
  switch (a.variant) {
    case 0: return run_mv<F, TM, 64, 2>(a, st);
    case 1: return run_mv<F, TM, 32, 2>(a, st);
    case 2: return run_stream<F, TM, 1, 2, 4, 1>(a, st);
    case 3: return run_stream<F, TM, 2, 2, 4, 1>(a, st);
    case 4: return run_stream<F, TM, 1, 3, 4, 1>(a, st);
    case 5: return run_stream<F, TM, 1, 2, 16, 1>(a, st);
    case 6: return run_stream<F, TM, 4, 1, 8, 1>(a, st);
    case 7: return run_stream<F, TM, 1, 2, 16, 16>(a, st);
    case 8: return run_flat<F, TM, 1, 2, 4, false>(a, st);
    case 9: return run_flat<F, TM, 2, 2, 4, false>(a, st);
    case 10: return run_flat<F, TM, 1, 3, 4, false>(a, st);
    case 11: return run_flat<F, TM, 1, 4, 4, false>(a, st);
    case 12: return run_flat<F, TM, 1, 7, 4, false, 4>(a, st);
    case 13: return run_flat<F, TM, 1, 2, 4, true>(a, st);
    case 14: return run_flat<F, TM, 1, 2, 16, true>(a, st);
    case 15: return run_flat<F, TM, 1, 3, 16, true>(a, st);
    case 16: return run_flat<F, TM, 1, 7, 8, true>(a, st);
    case 17: return run_flat<F, TM, 2, 2, 16, true>(a, st);
    case 49: return run_flat<F, TM, 2, 2, 4, true>(a, st);
    case 50: return run_flat<F, TM, 4, 2, 4, false>(a, st);
    case 51: return run_flat<F, TM, 4, 2, 4, true>(a, st);
    case 52: return run_flat<F, TM, 2, 2, 8, true>(a, st);
    case 53: return run_flat<F, TM, 2, 2, 2, false>(a, st);
    case 18: return run_mt<F, TM, 2, 1, 8, 2>(a, st);
    case 19: return run_mt<F, TM, 2, 1, 8, 4>(a, st);
    case 20: return run_mt<F, TM, 4, 1, 8, 2>(a, st);
    case 21: return run_mt<F, TM, 4, 1, 4, 1>(a, st);
    case 22: return run_mt<F, TM, 2, 1, 4, 1>(a, st);
    case 23: return run_mt<F, TM, 1, 1, 8, 4>(a, st);
    case 24: return run_mt<F, TM, 2, 1, 16, 8>(a, st);
    case 25: return run_mt<F, TM, 1, 1, 16, 8>(a, st);
    case 26: return run_mt<F, TM, 2, 2, 8, 2>(a, st);
    case 27: return run_mt<F, TM, 2, 2, 8, 1>(a, st);
    case 28: return run_mt<F, TM, 2, 2, 16, 4>(a, st);
    case 29: return run_mt<F, TM, 1, 2, 8, 2>(a, st);
    case 30: return run_mt<F, TM, 2, 4, 8, 2>(a, st);
    case 31: return run_mt<F, TM, 2, 2, 4, 1>(a, st);
    case 32: return run_mt<F, TM, 1, 2, 16, 4>(a, st);
    case 33: return run_mt<F, TM, 1, 4, 16, 4>(a, st);
    // 34..43: the matrix-core kernels (launch_mx, launch_mxf)
    case 44: return run_long<F, TM, 1, 2, 16>(a, st);
    case 45: return run_long<F, TM, 1, 4, 8>(a, st);
    case 46: return run_long<F, TM, 1, 8, 4>(a, st);
    case 47: return run_long<F, TM, 1, 2, 4>(a, st);
    case 48: return run_long<F, TM, 2, 2, 16>(a, st);
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

// This translation unit is compiled once per weight format (QMV_MATVEC_FMT),
// so that the formats' kernels build in parallel; each copy defines the
// vector-kernel entry of its format.
#ifndef QMV_MATVEC_FMT
#error "compile qmv_matvec.hip with -DQMV_MATVEC_FMT=<format id>"
#endif
template <>
hipError_t launch_vector<QMV_MATVEC_FMT>(const MatvecLaunch& a, hipStream_t st) {
  return run_mv_tokens<QMV_MATVEC_FMT>(a, st);
}

}  // namespace qmv
