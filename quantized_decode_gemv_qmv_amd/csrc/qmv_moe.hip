// qmv_moe.hip -- expert-grouped routed matvec for MoE decode (1..64 tokens).
//
// Castagna Veloce page, "Kernels for the MI50": i-quant MoE decode kernels for
// batches of up to 64 tokens, and expert-grouped quantized MoE where each
// active expert runs once over all the tokens routed to it.
//
// k_moe is persistent: a grid of a few workgroups per compute unit, each of
// which
//   1. sorts the slots by expert in LDS once (counting sort of the ids: at
//      most 1024 slots and 1024 experts), giving the U active experts in id
//      order and each one's slot list;
//   2. walks work items = (active expert, chunk of rows) with stride
//      gridDim.x.  For an item it copies the activation rows of the expert's
//      slots into LDS (up to `ts` slots at a time), then its waves walk the
//      chunk's row tiles: a lane group of LPR lanes owns one row of a tile,
//      loads all of the row (NU units per lane, block headers shared by lane
//      quads), decodes it into registers once and applies it, in the
//      own-block form of qmv_device.h, to every staged slot.  Each wave
//      issues the weight loads of its next tile before computing the
//      current one.  Activation reads come from LDS, so the in-order
//      vector-memory counter holds weights only and the prefetch is never
//      drained by a slot's fragments.
// Each active expert's weights are read from HBM once per call (once per
// group of `ts` slots when more tokens than that pick one expert).  The chunk
// size is set on the device from U so that there are about two items per
// workgroup.
//
// Route-weighted combine (y[t] = sum_s w[t][s] * y_slot): k_moe writes each
// slot's output row to the workspace, and k_moe_combine sums them in slot
// order -- deterministic, and the kernel boundary orders the two without any
// device-wide fence.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

constexpr int kMaxSlots = 64 * 16;
constexpr int kMaxExperts = 1024;

template <int F, int LPR, int NU, int WPB, bool WHOLE>
__global__ __launch_bounds__(64 * WPB) void k_moe(MoeLaunch a) {
  constexpr int GPW = 64 / LPR;
  constexpr int RWG = WPB * GPW;  // rows per tile (one per lane group)
  constexpr int NT = 64 * WPB;
  // staged slot rows; during the sort the same bytes hold the ids
  extern __shared__ __attribute__((aligned(16))) uint8_t s_act[];
  int* s_id = reinterpret_cast<int*>(s_act);  // ids, -1 for dropped slots
  __shared__ int s_cnt[kMaxExperts];   // slots per expert, then running offsets
  __shared__ int s_slot[kMaxSlots];    // slots grouped by expert
  __shared__ int s_exp[kMaxExperts];   // active experts in id order
  __shared__ int s_beg[kMaxExperts + 1];  // their first entry in s_slot
  __shared__ int s_U, s_drop;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_slots = a.n_tok * a.top_k;
  const int E = a.n_experts;

  // ---- 1. counting sort of the slots by expert
  for (int e = tid; e < E; e += NT) s_cnt[e] = 0;
  if (tid == 0) s_drop = 0;
  __syncthreads();
  for (int i = tid; i < n_slots; i += NT) {
    const int e = a.ids[i];
    const bool ok = e >= 0 && e < E;
    s_id[i] = ok ? e : -1;
    if (ok)
      atomicAdd(&s_cnt[e], 1);
    else
      atomicAdd(&s_drop, 1);
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of the counts and compaction of the active experts:
    // lane l covers experts [l*per, (l+1)*per)
    const int per = (E + 63) / 64;
    const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
    int sum = 0, act = 0;
    for (int e = e0; e < e1; ++e) {
      sum += s_cnt[e];
      act += s_cnt[e] > 0;
    }
    int isum = sum, iact = act;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int vs = __shfl_up(isum, o, 64), va = __shfl_up(iact, o, 64);
      if (lane >= o) {
        isum += vs;
        iact += va;
      }
    }
    int off = isum - sum, rank = iact - act;
    for (int e = e0; e < e1; ++e) {
      const int c = s_cnt[e];
      if (c > 0) {
        s_exp[rank] = e;
        s_beg[rank] = off;
        ++rank;
      }
      s_cnt[e] = off;
      off += c;
    }
    if (lane == 63) {
      s_U = iact;
      s_beg[iact] = isum;
    }
  }
  __syncthreads();
  for (int i = tid; i < n_slots; i += NT) {
    const int e = s_id[i];
    if (e >= 0) s_slot[atomicAdd(&s_cnt[e], 1)] = i;  // order inside an expert is free
  }
  __syncthreads();
  const int U = s_U;

  // what no item writes: the dropped-slot count, and with one output per
  // slot the zero rows of dropped slots
  if (blockIdx.x == 0 && tid == 0) a.err[0] = s_drop;
  if (s_drop > 0 && a.rw == nullptr) {
    for (int i = 0; i < n_slots; ++i)
      if (s_id[i] < 0)
        for (int r = blockIdx.x * NT + tid; r < a.n_rows; r += gridDim.x * NT)
          a.y[(int64_t)i * a.n_rows + r] = 0.f;
  }
  __syncthreads();  // the ids are dead: their bytes take staged rows next

  // ---- 2. work items: (active expert, chunk of rows)
  const int tiles = (a.n_rows + RWG - 1) / RWG;
  // tiles per chunk: about two items per workgroup
  const int tpc = max(1, (int)(((int64_t)U * tiles + 2 * gridDim.x - 1) / (2 * gridDim.x)));
  const int chunks = (tiles + tpc - 1) / tpc;
  const int nitems = U * chunks;
  const int g = lane / LPR, gl = lane % LPR;
  const int units = a.units, K = a.x.k, nb = a.x.nb;
  // LDS rows: WHOLE -- every activation row of the call, indexed by the
  // slot's activation row; else the rows of up to ts slots of one expert
  const int ts = a.ts;
  const Act x{reinterpret_cast<const int8_t*>(s_act), reinterpret_cast<const float*>(s_act + ts * K),
              reinterpret_cast<const int32_t*>(s_act + ts * K + 4 * ts * nb), K, nb};
  const int8_t* gqs = a.x.qs;
  const float* gd = a.x.d;
  const int32_t* gs = a.x.s;
  auto x_row = [&](int i) { return a.x_per_slot ? i : i / a.top_k; };
  // copy ng rows into LDS: row j of the copy is activation row src(j)
  auto stage = [&](int ng, auto src) {
    const int pr = K / 16;  // 16-byte pieces per row
    for (int idx = tid; idx < ng * pr; idx += NT) {
      const int j = idx / pr, p = idx - j * pr;
      reinterpret_cast<u32x4a*>(s_act)[idx] = ld16(gqs + (int64_t)src(j) * K + 16 * p);
    }
    float* ld_d = reinterpret_cast<float*>(s_act + ts * K);
    int32_t* ld_s = reinterpret_cast<int32_t*>(s_act + ts * K + 4 * ts * nb);
    for (int idx = tid; idx < ng * nb; idx += NT) {
      const int j = idx / nb, p = idx - j * nb;
      ld_d[idx] = gd[(int64_t)src(j) * nb + p];
      ld_s[idx] = gs[(int64_t)src(j) * nb + p];
    }
  };

  // The workgroup's work as one sequence of steps (item, slot group, tile);
  // the weights of the next step are always in flight during the current.
  struct Pos {
    int item, g0, t;
  };
  auto item_t0 = [&](int item) { return (item % chunks) * tpc; };
  auto advance = [&](Pos p) {
    const int rank = p.item / chunks;
    const int t1 = min(item_t0(p.item) + tpc, tiles);
    const int n_e = s_beg[rank + 1] - s_beg[rank];
    if (p.t + 1 < t1) return Pos{p.item, p.g0, p.t + 1};
    if (!WHOLE && p.g0 + ts < n_e) return Pos{p.item, p.g0 + ts, item_t0(p.item)};
    const int ni = p.item + (int)gridDim.x;
    return Pos{ni, 0, ni < nitems ? item_t0(ni) : 0};
  };
  auto load_tile = [&](Pos p, RawS<F> (&raw)[NU]) {
    const int item = min(p.item, nitems - 1);
    const int e = s_exp[item / chunks];
    const int row = min(p.t * RWG + wave * GPW + g, a.n_rows - 1);
    const uint8_t* wr = a.w + ((int64_t)e * a.n_rows + row) * a.row_bytes;
#pragma unroll
    for (int q = 0; q < NU; ++q) load_unit_s(wr, min(gl + LPR * q, units - 1), lane, raw[q]);
  };

  if ((int)blockIdx.x >= nitems) return;  // uniform across the workgroup
  Pos pos{(int)blockIdx.x, 0, item_t0(blockIdx.x)};
  RawS<F> cur[NU];
  load_tile(pos, cur);
  if constexpr (WHOLE) {
    stage(a.x_rows, [](int j) { return j; });
    __syncthreads();
  }
  int staged_item = -1, staged_g0 = -1;
  while (pos.item < nitems) {
    const Pos nx = advance(pos);
    RawS<F> nxt[NU];
    load_tile(nx, nxt);  // unconditional (clamped past the end): no early drain
    const int rank = pos.item / chunks;
    const int b0 = s_beg[rank], n_e = s_beg[rank + 1] - b0;
    const int ng = WHOLE ? n_e : min(ts, n_e - pos.g0);
    if constexpr (!WHOLE) {
      if (pos.item != staged_item || pos.g0 != staged_g0) {
        __syncthreads();  // the previous group's rows are no longer read
        stage(ng, [&](int j) { return x_row(s_slot[b0 + pos.g0 + j]); });
        __syncthreads();
        staged_item = pos.item;
        staged_g0 = pos.g0;
      }
    }
    const int row = pos.t * RWG + wave * GPW + g;
    DecO<F> dec[NU];
#pragma unroll
    for (int q = 0; q < NU; ++q)
      decode_own(cur[q], min(gl + LPR * q, units - 1), gl & 1, gl + LPR * q < units, dec[q]);
    for (int j = 0; j < ng; ++j) {
      const int i = s_slot[b0 + pos.g0 + j];
      const int lr = WHOLE ? x_row(i) : j;  // LDS row of the slot's activations
      XO xo[NU];
#pragma unroll
      for (int q = 0; q < NU; ++q) load_xo<F>(x, lr, min(gl + LPR * q, units - 1), xo[q]);
      int dv[NU];
#pragma unroll
      for (int q = 0; q < NU; ++q) dv[q] = own_pass<F>(own_first(dec[q], xo[q].f));
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < NU; ++q) acc = own_apply(dec[q], own_second(dec[q], xo[q].s, dv[q]), xo[q].p, acc);
      acc = lane_group_sum<LPR>(acc);
      if (gl == 0 && row < a.n_rows) {
        float* out = a.rw == nullptr ? a.y : a.part;
        out[(int64_t)i * a.n_rows + row] = acc;
      }
    }
#pragma unroll
    for (int q = 0; q < NU; ++q) cur[q] = nxt[q];
    pos = nx;
  }
}

// y[t][n] = sum over valid slots s, in slot order, of rw[t][s] * part[t*top_k+s][n].
__global__ __launch_bounds__(256) void k_moe_combine(MoeLaunch a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.n_tok * a.n_rows) return;
  const int t = (int)(idx / a.n_rows), n = (int)(idx % a.n_rows);
  float sum = 0.f;
  for (int s = 0; s < a.top_k; ++s) {
    const int sl = t * a.top_k + s;
    const int e = a.ids[sl];
    if (e >= 0 && e < a.n_experts) sum += a.rw[sl] * a.part[(int64_t)sl * a.n_rows + n];
  }
  a.y[idx] = sum;
}

// Lanes per row and units per lane for a row of `units` units.
static int moe_lpr(int units) { return units <= 64 ? 16 : 64; }
static int moe_nu(int units) {
  const int lpr = moe_lpr(units);
  const int nu = (units + lpr - 1) / lpr;
  return nu <= 1 ? 1 : nu <= 2 ? 2 : nu <= 3 ? 3 : nu <= 4 ? 4 : 8;
}

// LDS bytes for staged slot rows per workgroup, and the largest activation
// buffer copied whole.
constexpr int64_t kMoeStageBytes = 40 * 1024;
constexpr int64_t kMoeWholeBytes = 40 * 1024;

template <int F, int LPR, int NU, bool WHOLE>
static hipError_t run_moe(const MoeLaunch& a0, hipStream_t st) {
  constexpr int WPB = 8;
  MoeLaunch a = a0;
  auto kern = k_moe<F, LPR, NU, WPB, WHOLE>;
  const int64_t row_stage = (int64_t)a.x.k + 8 * a.x.nb;  // qs + d + s of one row
  const int64_t slots = (int64_t)a.n_tok * a.top_k;
  int64_t ts;
  if (WHOLE) {
    ts = a.x_rows;
  } else {
    // an expert is picked at most once per token by a top-k routing, so
    // n_tok staged rows hold all of an expert's slots (more go in further
    // groups)
    ts = kMoeStageBytes / row_stage;
    if (ts > a.n_tok) ts = a.n_tok;
    if (ts < 1) ts = 1;
  }
  a.ts = (int)ts;
  size_t lds = (size_t)(ts * row_stage);
  if (lds < (size_t)kMaxSlots * 4) lds = (size_t)kMaxSlots * 4;  // the ids during the sort
  // resident workgroups per compute unit: the register limit, measured once
  // per instantiation (thread-safe static), then the LDS limit for this call
  struct Occ {
    int regs;
    size_t static_lds;
  };
  static const Occ occ0 = [&] {
    Occ o{1, 0};
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 64 * WPB, 0) == hipSuccess && n > 0) o.regs = n;
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern)) == hipSuccess)
      o.static_lds = fa.sharedSizeBytes;
    return o;
  }();
  int occ = occ0.regs;
  const int by_lds = (int)((size_t)a.lds_per_cu / (occ0.static_lds + lds));
  if (occ > by_lds) occ = by_lds;
  if (occ < 1) occ = 1;
  constexpr int RWG = WPB * (64 / LPR);
  const int64_t tiles = (a.n_rows + RWG - 1) / RWG;
  const int64_t max_items = (slots < a.n_experts ? slots : a.n_experts) * tiles;
  const int64_t cap = (int64_t)a.cus * occ;
  const unsigned grid = (unsigned)(max_items < cap ? max_items : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.rw == nullptr) return e;
  const int64_t outs = (int64_t)a.n_tok * a.n_rows;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Small calls copy every activation row into LDS once; larger ones stage
// each expert's rows per work item.
template <int F, int LPR, int NU>
static hipError_t run_moe_pick(const MoeLaunch& a, hipStream_t st) {
  const int64_t whole = (int64_t)a.x_rows * (a.x.k + 8 * a.x.nb);
  return whole <= kMoeWholeBytes ? run_moe<F, LPR, NU, true>(a, st) : run_moe<F, LPR, NU, false>(a, st);
}

template <int F>
static hipError_t run_moe_fmt(const MoeLaunch& a, hipStream_t st) {
  const int lpr = moe_lpr(a.units), nu = moe_nu(a.units);
  if (lpr == 16) {
    switch (nu) {
      case 1: return run_moe_pick<F, 16, 1>(a, st);
      case 2: return run_moe_pick<F, 16, 2>(a, st);
      case 3: return run_moe_pick<F, 16, 3>(a, st);
      default: return run_moe_pick<F, 16, 4>(a, st);
    }
  }
  switch (nu) {
    case 2: return run_moe_pick<F, 64, 2>(a, st);
    case 3: return run_moe_pick<F, 64, 3>(a, st);
    case 4: return run_moe_pick<F, 64, 4>(a, st);
    default: return run_moe_pick<F, 64, 8>(a, st);
  }
}

hipError_t launch_moe(const MoeLaunch& a, hipStream_t st) {
  switch (a.fmt) {
    case FQ8_0: return run_moe_fmt<FQ8_0>(a, st);
    case FQ4_K: return run_moe_fmt<FQ4_K>(a, st);
    case FIQ4_XS: return run_moe_fmt<FIQ4_XS>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmv
