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
#include "qmv_mfma.h"

namespace qmv {

constexpr int kMaxSlots = 64 * 16;
constexpr int kMaxExperts = 1024;

// Routing in LDS, built by every workgroup of a MoE kernel from the ids (a
// counting sort of the slots by expert): s_exp[0..U) the active experts in id
// order, s_slot[s_beg[r]..s_beg[r+1]) the slots routed to the r-th of them.
// Dropped slots (ids outside [0, E)) are counted; workgroup 0 reports the
// count in the workspace and, with one output row per slot, the other
// workgroups zero those rows.  s_id needs kMaxSlots ints of scratch.
template <int NT>
__device__ void moe_route(const MoeLaunch& a, int* s_id, int* s_cnt, int* s_slot, int* s_exp, int* s_beg,
                          int* s_U, int* s_drop) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_slots = a.n_tok * a.top_k;
  const int E = a.n_experts;
  for (int e = tid; e < E; e += NT) s_cnt[e] = 0;
  if (tid == 0) *s_drop = 0;
  __syncthreads();
  for (int i = tid; i < n_slots; i += NT) {
    const int e = a.ids[i];
    const bool ok = e >= 0 && e < E;
    s_id[i] = ok ? e : -1;
    if (ok)
      atomicAdd(&s_cnt[e], 1);
    else
      atomicAdd(s_drop, 1);
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
      *s_U = iact;
      s_beg[iact] = isum;
    }
  }
  __syncthreads();
  for (int i = tid; i < n_slots; i += NT) {
    const int e = s_id[i];
    if (e >= 0) s_slot[atomicAdd(&s_cnt[e], 1)] = i;  // order inside an expert is free
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) a.err[0] = *s_drop;
  if (*s_drop > 0 && a.rw == nullptr && a.dots == nullptr) {
    for (int i = 0; i < n_slots; ++i)
      if (s_id[i] < 0)
        for (int r = blockIdx.x * NT + tid; r < a.n_rows; r += gridDim.x * NT)
          a.y[(int64_t)i * a.n_rows + r] = 0.f;
  }
  __syncthreads();  // s_id is dead from here on
}

template <int F, int LPR, int NU, int WPB, bool WHOLE>
__global__ __launch_bounds__(64 * WPB) void k_moe(MoeLaunch a) {
  constexpr int GPW = 64 / LPR;
  constexpr int RWG = WPB * GPW;  // rows per tile (one per lane group)
  constexpr int NT = 64 * WPB;
  // staged slot rows; during the sort the same bytes hold the ids
  extern __shared__ __attribute__((aligned(16))) uint8_t s_act[];
  __shared__ int s_cnt[kMaxExperts];      // slots per expert, then running offsets
  __shared__ int s_slot[kMaxSlots];       // slots grouped by expert
  __shared__ int s_exp[kMaxExperts];      // active experts in id order
  __shared__ int s_beg[kMaxExperts + 1];  // their first entry in s_slot
  __shared__ int s_U, s_drop;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  moe_route<NT>(a, reinterpret_cast<int*>(s_act), s_cnt, s_slot, s_exp, s_beg, &s_U, &s_drop);
  const int U = s_U;

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

// Expert-grouped matrix-core kernel, for calls where experts receive several
// slots (the 16-64 token batches).  The dense matrix-core kernel's tile -- 16
// weight rows, one v_mfma_i32_16x16x64_i8 per token group and 64-wide slice
// of K, the per-32-block dots kept apart by zero-masked activation rows (see
// qmv_mfma.hip) -- with the activation rows of an expert's slots as its
// tokens.  Work items are (active expert, chunk of row tiles), walked with
// stride gridDim.x after the routing sort; per item the workgroup stages up
// to TMP of the expert's slot rows (block-major, the whole K) in LDS, and its
// waves walk the chunk's tiles, each tile over the whole K with the next
// super-block's weights in flight.  More slots than TMP go in further groups,
// each reading the expert's rows again.
//
// DOTS (the block-dot test hook): the same routing, staging, loads, decode
// and MFMAs, but each MFMA result -- the exact integer dot of one (slot, row,
// 32-block) -- times the block's integer weight scale goes to a.dots, and no
// output is written.
template <int F, int TM, int WPB, bool DOTS = false>
__global__ __launch_bounds__(64 * WPB) void k_moe_mx(MoeLaunch a) {
  constexpr int TG = mx_tg<F>();
  constexpr int NG = (TM + TG - 1) / TG;  // token groups
  constexpr int TMP = NG * TG;            // staged slot rows
  constexpr int NT = 64 * WPB;
  constexpr bool Q4K = F == FQ4_K;
  constexpr bool P2 = Q4K;  // two blocks per MFMA (q4_K), else four
  constexpr int BS = TMP * 32 + 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t s_act[];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_slot[kMaxSlots];
  __shared__ int s_exp[kMaxExperts];
  __shared__ int s_beg[kMaxExperts + 1];
  __shared__ int s_U, s_drop;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  moe_route<NT>(a, reinterpret_cast<int*>(s_act), s_cnt, s_slot, s_exp, s_beg, &s_U, &s_drop);
  const int U = s_U;

  const int n = lane & 15, s = lane >> 4;
  const int units = a.units, nb = a.x.nb, K = a.x.k;
  const int nsb = (units + 7) >> 3;
  const int kb = 8 * nsb;  // staged blocks
  uint8_t* xl = s_act;
  const int zoff = kb * BS;
  float* dl = reinterpret_cast<float*>(s_act + zoff + 16);
  float* sl = dl + kb * TMP;
  if (tid < 4) reinterpret_cast<uint32_t*>(s_act + zoff)[tid] = 0u;

  // lane coordinates, as in the dense kernel
  const int m = lane & 15;
  const int jA = P2 ? (m >> 3) : (m >> 2);
  const int tA = P2 ? (m & 7) : (m & 3);
  const bool vA = P2 ? (jA == (s >> 1)) : (jA == s);
  constexpr int aMu = P2 ? BS : 16;
  constexpr int oMu = P2 ? TMP * 4 : 0;
  const int aLane = (P2 ? 2 * jA : jA) * BS + tA * 32 + (P2 ? 16 * (s & 1) : 0);
  const int oTok = P2 ? 4 * (s & 1) : 0;
  const int oLane = (P2 ? 2 * (s >> 1) : s) * TMP * 4 + oTok * 4;

  const int tiles = (a.n_rows + 15) >> 4;
  const int tpc = max(1, (int)(((int64_t)U * tiles + 2 * gridDim.x - 1) / (2 * gridDim.x)));
  const int chunks = (tiles + tpc - 1) / tpc;
  const int nitems = U * chunks;
  auto x_row = [&](int i) { return a.x_per_slot ? i : i / a.top_k; };
  float* out = a.rw == nullptr ? a.y : a.part;

  float acc[NG][4];
  u32x4 A[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int rank = item / chunks;
    const int e = s_exp[rank];
    const int b0 = s_beg[rank], n_e = s_beg[rank + 1] - b0;
    const int t0 = (item - rank * chunks) * tpc, t1 = min(t0 + tpc, tiles);
    const uint8_t* we = a.w + (int64_t)e * a.n_rows * a.row_bytes;
    for (int g0 = 0; g0 < n_e; g0 += TMP) {
      const int ng = min(TMP, n_e - g0);
      const int ngr = (ng + TG - 1) / TG;  // token groups with a slot
      __syncthreads();  // the previous group's rows are no longer read
      {
        // stage the group's slot rows: quants block-major, scales zero past
        // ng; loads go out four per thread before their stores
        const int pr = K >> 4;  // 16-byte pieces per row
        const FastDiv dp(pr);
        for (int base = 0; base < TMP * pr; base += 4 * NT) {
          u32x4 v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int idx = min(base + tid + q * NT, TMP * pr - 1);
            const int j = dp.div(idx), pc = idx - j * pr;
            const int xr = x_row(s_slot[b0 + g0 + min(j, ng - 1)]);
            v[q] = ld16(a.x.qs + (int64_t)xr * K + 16 * pc);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int idx = base + tid + q * NT;
            const int j = dp.div(idx), pc = idx - j * pr;
            if (idx < TMP * pr) *reinterpret_cast<u32x4a*>(xl + (pc >> 1) * BS + j * 32 + 16 * (pc & 1)) = v[q];
          }
        }
        // scales: entry (slot row j, block b) read row-major (consecutive
        // lanes on consecutive blocks of one row: coalesced), stored
        // block-major
        const FastDiv dkb(kb);
        for (int base = 0; base < kb * TMP; base += 4 * NT) {
          float dv[4];
          int iv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int idx = base + tid + q * NT;
            const int j = dkb.div(idx), b = idx - j * kb;
            const int xr = x_row(s_slot[b0 + g0 + min(j, ng - 1)]);
            const int64_t gi = (int64_t)xr * nb + min(b, nb - 1);
            dv[q] = a.x.d[gi];
            iv[q] = a.x.s[gi];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int idx = base + tid + q * NT;
            const int j = dkb.div(idx), b = idx - j * kb;
            const bool ok = j < ng && b < nb;
            if (idx < kb * TMP) {
              dl[b * TMP + j] = ok ? dv[q] : 0.f;
              if constexpr (Q4K) sl[b * TMP + j] = ok ? dv[q] * static_cast<float>(iv[q]) : 0.f;
            }
          }
        }
      }
      __syncthreads();
      // the wave's tiles of the chunk, each over all of K, next load in flight
      int lt = t0 + wave, lsb = 0;  // next (tile, super-block) to load
      auto load_next = [&](MxRaw<F>& r) {
        const int t = min(lt, t1 - 1);
        const uint8_t* base = we + (int64_t)t * 16 * a.row_bytes;
        const uint32_t off = (uint32_t)(min(n, a.n_rows - 1 - t * 16) * (int)a.row_bytes);
        mx_load(base, off, 8 * lsb, s, units, r);
        if (++lsb >= nsb) {
          lsb = 0;
          lt += WPB;
        }
      };
      if (t0 + wave >= t1) continue;
      MxRaw<F> cur;
      load_next(cur);
      for (int t = t0 + wave; t < t1; t += WPB) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[g][r] = 0.f;
        for (int sb = 0; sb < nsb; ++sb) {
          MxRaw<F> nxt;
          load_next(nxt);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (p > 0) __builtin_amdgcn_sched_barrier(0);
            MxDec dec;
            mx_decode(cur, p, s, 8 * sb, units, dec);
            const int bl = 8 * sb + 4 * p;
            const int ab = vA ? bl * BS + aLane : zoff;
            const int ob = bl * TMP * 4 + oLane;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              if (g >= ngr) break;
              if (g > 0) __builtin_amdgcn_sched_barrier(0);
              if (vA) {
                A[0] = ld16(xl + ab + g * TG * 32);
                A[1] = ld16(xl + ab + g * TG * 32 + aMu);
              }
              if constexpr (DOTS) {
                // lane (n, s): row t * 16 + n; result r is block bl + (q4_K:
                // 2 (s >> 1) + mu; else s) of the group's slot row (q4_K:
                // 8g + 4 (s & 1) + r; else 4g + r), as in the scale steps below
                const int row = t * 16 + n;
#pragma unroll
                for (int mu = 0; mu < (P2 ? 2 : 1); ++mu) {
                  i32x4 dv;
                  if constexpr (P2) {
                    dv = mfma64(A[mu], dec.b[mu], i32x4{0, 0, 0, 0});
                  } else {
                    dv = mfma64(A[0], dec.b[0], i32x4{0, 0, 0, 0});
                    dv = mfma64(A[1], dec.b[1], dv);
                  }
                  const int blk = bl + (P2 ? 2 * (s >> 1) + mu : s);
#pragma unroll
                  for (int r = 0; r < 4; ++r) {
                    const int j = P2 ? g * TG + 4 * (s & 1) + r : g * TG + r;
                    if (j < ng && row < a.n_rows && blk < units) {
                      const int slot = s_slot[b0 + g0 + j];
                      const int64_t o = ((int64_t)slot * a.n_rows + row) * units + blk;
                      if constexpr (Q4K) {
                        a.dots[2 * o] = dec.isc[mu] * dv[r];
                        a.dots[2 * o + 1] = dec.im[mu] * a.x.s[(int64_t)x_row(slot) * nb + blk];
                      } else {
                        a.dots[o] = dec.isc[0] * dv[r];
                      }
                    }
                  }
                }
              } else if constexpr (P2) {
#pragma unroll
                for (int mu = 0; mu < 2; ++mu) {
                  const i32x4 dv = mfma64(A[mu], dec.b[mu], i32x4{0, 0, 0, 0});
                  const int o = ob + mu * oMu + g * TG * 4;
                  const f32x4 fx = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(dl) + o);
                  const f32x4 fs = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(sl) + o);
                  const float fxa[4] = {fx.x, fx.y, fx.z, fx.w}, fsa[4] = {fs.x, fs.y, fs.z, fs.w};
#pragma unroll
                  for (int r = 0; r < 4; ++r) {
                    acc[g][r] = fmaf(static_cast<float>(dv[r]), dec.dw[mu] * fxa[r], acc[g][r]);
                    acc[g][r] = fmaf(-dec.wm[mu], fsa[r], acc[g][r]);
                  }
                }
              } else {
                i32x4 dv = mfma64(A[0], dec.b[0], i32x4{0, 0, 0, 0});
                dv = mfma64(A[1], dec.b[1], dv);
                const f32x4 fx = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(dl) + ob + g * TG * 4);
                const float fxa[4] = {fx.x, fx.y, fx.z, fx.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  acc[g][r] = fmaf(static_cast<float>(dv[r]), dec.dw[0] * fxa[r], acc[g][r]);
              }
            }
          }
          cur = nxt;
        }
        if constexpr (DOTS) continue;  // the integers are out; nothing to sum
        // lanes holding the other blocks of the same row and slots, then the
        // slot outputs (see the dense kernel for the lane layout)
        const int row = t * 16 + n;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (g >= ngr) break;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = acc[g][r];
            if constexpr (!P2) v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            const int j = P2 ? g * 8 + 4 * s + r : g * 4 + r;
            const bool mine = P2 ? s < 2 : s == (g & 3);
            if (mine && j < ng && row < a.n_rows) out[(int64_t)s_slot[b0 + g0 + j] * a.n_rows + row] = v;
          }
        }
      }
    }
  }
}

// Slots whose expert id is out of range (dropped), counted by one whole wave:
// 64 ids per step under a ballot, so that the ids are loaded together rather
// than one round trip per slot.
__device__ __forceinline__ int count_dropped(const MoeLaunch& a, int n_slots) {
  const int lane = threadIdx.x & 63;
  int drop = 0;
  for (int i0 = 0; i0 < n_slots; i0 += 64) {
    const int i = i0 + lane;
    const int id = i < n_slots ? a.ids[i] : 0;
    drop += __popcll(__ballot(i < n_slots && (id < 0 || id >= a.n_experts)));
  }
  return drop;
}

// y[t][n] = sum over valid slots s, in slot order, of rw[t][s] * part[t*top_k+s][n].
// Every slot's id, route weight and output are loaded before any is used (a
// slot's output row exists whether or not its id is valid), so the loads
// are in flight together instead of one id-then-output round trip per slot;
// the valid slots are then summed in slot order.
constexpr int kCombineMaxTopK = 16;
__global__ __launch_bounds__(256) void k_moe_combine(MoeLaunch a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.n_tok * a.n_rows) return;
  const int t = (int)(idx / a.n_rows), n = (int)(idx % a.n_rows);
  int e[kCombineMaxTopK];
  float wv[kCombineMaxTopK], pv[kCombineMaxTopK];
#pragma unroll
  for (int s = 0; s < kCombineMaxTopK; ++s) {
    if (s < a.top_k) {  // uniform over the grid
      const int sl = t * a.top_k + s;
      e[s] = a.ids[sl];
      wv[s] = a.rw[sl];
      pv[s] = a.part[(int64_t)sl * a.n_rows + n];
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < kCombineMaxTopK; ++s)
    if (s < a.top_k && e[s] >= 0 && e[s] < a.n_experts) sum += wv[s] * pv[s];
  a.y[idx] = sum;
}

// Few-slot routed matvec (decode): with about one slot per routed expert
// there is no weight reuse to group for, and k_moe's routing sort and
// per-item staging only delay the weight stream.  k_moe_flat streams each
// routed expert's rows as the dense flat kernel does: workgroup (x, y) takes
// rows x * WPB * R .. of the expert of slot y, each lane issuing every weight
// load of its R rows (NU units per row) at once, behind its activation
// fragments (cache-resident).  Each expert is read once per call (the
// grouping the pages ask for, Castagna Veloce page, "Kernels for the MI50"):
// the workgroups of the first slot routed to an expert also serve every
// later slot with the same expert, one slot after the other from the same
// weight registers, and those later slots' workgroups exit at once.  A
// wave finds them with one ballot per 64 ids.  Outputs per slot, written as
// k_moe writes them (to y, or to the workspace for the combine); a dropped
// slot's row is zero.

//
// LPR = 16 (rows of fewer than 64 units with one activation row per slot,
// the down projection's 48): a wave
// takes four rows, one per 16-lane group, NU units per lane, so that every
// lane carries units (with one unit per lane a 48-unit row left 16 lanes
// idle); R is 1 and each group's sum is a 16-lane DPP reduction.
template <int F, int NU, int R, int WPB, int LPR = 64>
__global__ __launch_bounds__(64 * WPB) void k_moe_flat(MoeLaunch a) {
  static_assert(LPR == 64 || LPR == 16, "64-lane rows or 16-lane row groups");
  constexpr int RPW = LPR == 64 ? R : 4 * R;  // rows per wave
  constexpr int RS = LPR == 64 ? 1 : 4;       // row step between a lane's rows
  const int lane = threadIdx.x & 63;
  const int lu = LPR == 64 ? lane : (lane & 15);  // lane index inside its row group
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = blockIdx.y;
  const int n_slots = a.n_tok * a.top_k;
  const int e = a.ids[slot];
  const bool valid = e >= 0 && e < a.n_experts;
  const int units = a.units;
  const int row0 = (blockIdx.x * WPB + wave) * RPW + (LPR == 64 ? 0 : (lane >> 4));
  const int xr = a.x_per_slot ? slot : slot / a.top_k;
  const Act gx{a.x.qs, a.x.d, a.x.s, a.x.k, a.x.nb};
  // slots i with the same expert in chunk c (64 ids per chunk), one flag
  // per lane, the same mask in every lane and every wave
  auto same_in = [&](int c) -> uint64_t {
    const int i = c * 64 + lane;
    const int id = i < n_slots ? a.ids[i] : -1;
    return __ballot(valid && id == e);
  };
  // an earlier slot with the same expert makes this workgroup redundant
  // (uniform over the workgroup): that slot's workgroups compute this one
  for (int c = 0; c * 64 < slot; ++c) {
    const uint64_t lo = slot - c * 64 >= 64 ? ~0ull : ((1ull << (slot - c * 64)) - 1);
    if (same_in(c) & lo) return;
  }
  XO xf[NU];
#pragma unroll
  for (int q = 0; q < NU; ++q) load_xo<F>(gx, xr, min(lu + LPR * q, units - 1), xf[q]);
  __builtin_amdgcn_sched_barrier(0);
  const uint8_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    wr[r] = a.w + ((int64_t)(valid ? e : 0) * a.n_rows + min(row0 + RS * r, a.n_rows - 1)) * a.row_bytes;
  RawS<F> cur[R][NU];
#pragma unroll
  for (int q = 0; q < NU; ++q)
#pragma unroll
    for (int r = 0; r < R; ++r) load_unit_s(wr[r], min(lu + LPR * q, units - 1), lane, cur[r][q]);
  __builtin_amdgcn_sched_barrier(0);
  float* out = a.rw == nullptr ? a.y : a.part;
  // one slot: the rows' sums against activation fragments f, stored at slot s
  auto apply = [&](const XO (&f)[NU], int s) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      const int uraw = lu + LPR * q;
      const bool ok = uraw < units;
      const int u = ok ? uraw : units - 1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        DecO<F> dec;
        decode_own(cur[r][q], u, lane & 1, ok, dec);
        const int dv = own_pass<F>(own_first(dec, f[q].f));
        acc[r] = own_apply(dec, own_second(dec, f[q].s, dv), f[q].p, acc[r]);
      }
    }
    if constexpr (LPR == 16) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float sv = lane_group_sum<16>(acc[r]);
        if (lu == 0 && row0 + 4 * r < a.n_rows) out[(int64_t)s * a.n_rows + row0 + 4 * r] = valid ? sv : 0.f;
      }
    } else {
      float outv = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float sv = wave_sum(acc[r]);
        outv = lane == r ? sv : outv;
      }
      if (lane < R && row0 + lane < a.n_rows) out[(int64_t)s * a.n_rows + row0 + lane] = valid ? outv : 0.f;
    }
  };
  apply(xf, slot);
  if (valid) {
    // the later slots with the same expert, in slot order
    for (int c = slot / 64; c * 64 < n_slots; ++c) {
      const int sh = slot - c * 64;  // 0..63 in the slot's own chunk, < 0 after it
      uint64_t m = same_in(c) & (sh < 0 ? ~0ull : ~((2ull << sh) - 1));
      while (m != 0) {  // uniform: the ballot is the same in every lane
        const int s2 = c * 64 + __builtin_ctzll(m);
        m &= m - 1;
        // decode the raw weights again for this slot rather than keep every
        // decoded unit alive across the slots (that doubled the registers of
        // the first slot's pass and halved the waves in flight)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int q = 0; q < NU; ++q) {
            uint32_t* rw = reinterpret_cast<uint32_t*>(&cur[r][q]);
#pragma unroll
            for (int i = 0; i < (int)(sizeof(RawS<F>) / 4); ++i) asm volatile("" : "+v"(rw[i]));
          }
        const int xr2 = a.x_per_slot ? s2 : s2 / a.top_k;
        XO f2[NU];
#pragma unroll
        for (int q = 0; q < NU; ++q) load_xo<F>(gx, xr2, min(lu + LPR * q, units - 1), f2[q]);
        apply(f2, s2);
      }
    }
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) {  // wave 0, all lanes (slot 0 never exits early)
    const int drop = count_dropped(a, n_slots);
    if (threadIdx.x == 0) a.err[0] = drop;
  }
}

// The MoE FFN's gate+up projection with SwiGLU and the Q8 blocks of its
// output folded in (Castagna Veloce page, "Fused operations": gate/up +
// SwiGLU; Q8 activations made once): the few-slot flat kernel, each of its
// workgroups taking 32 gate rows 32x .. 32x + 31 of the expert (waves 0-7,
// four rows each) and the 32 matching up rows n_ff + 32x .. (waves 8-15), so
// that one workgroup holds both halves of one 32-value block of
// h = silu(g) * u.  Per slot the 64 wave sums meet in LDS and eight lanes
// make the block with the quantizer's routine -- the same fp32 operations as
// k_swiglu_quantize on the gate+up output, so the blocks are bit-identical
// to the two-launch path.  The gate+up sums themselves go to a.y if it is
// set.  Expert reads are shared between the slots of one expert as in
// k_moe_flat.
template <int F, int NU>
__global__ __launch_bounds__(1024) void k_moe_gate_up_swiglu(MoeLaunch a) {
  constexpr int R = 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = blockIdx.y;
  const int n_slots = a.n_tok * a.top_k;
  const int e = a.ids[slot];
  const bool valid = e >= 0 && e < a.n_experts;
  const int units = a.units;
  const int n_ff = a.n_ff;
  const int n_rows = 2 * n_ff;  // gate rows, then up rows
  const int b = blockIdx.x;     // the 32-value block of h
  const int row0 = (wave < 8 ? 0 : n_ff) + 32 * b + 4 * (wave & 7);
  const Act gx{a.x.qs, a.x.d, a.x.s, a.x.k, a.x.nb};
  __shared__ float s_gu[64];
  auto same_in = [&](int c) -> uint64_t {
    const int i = c * 64 + lane;
    const int id = i < n_slots ? a.ids[i] : -1;
    return __ballot(valid && id == e);
  };
  for (int c = 0; c * 64 < slot; ++c) {
    const uint64_t lo = slot - c * 64 >= 64 ? ~0ull : ((1ull << (slot - c * 64)) - 1);
    if (same_in(c) & lo) return;  // an earlier slot's workgroups compute this one
  }
  const int xr0 = slot / a.top_k;  // one activation row per token
  XO xf[NU];
#pragma unroll
  for (int q = 0; q < NU; ++q) load_xo<F>(gx, xr0, min(lane + 64 * q, units - 1), xf[q]);
  __builtin_amdgcn_sched_barrier(0);
  const uint8_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = a.w + ((int64_t)(valid ? e : 0) * n_rows + row0 + r) * a.row_bytes;
  RawS<F> cur[R][NU];
#pragma unroll
  for (int q = 0; q < NU; ++q)
#pragma unroll
    for (int r = 0; r < R; ++r) load_unit_s(wr[r], min(lane + 64 * q, units - 1), lane, cur[r][q]);
  __builtin_amdgcn_sched_barrier(0);
  const int nb = n_ff / 32;
  int8_t* h_qs = reinterpret_cast<int8_t*>(a.hq);
  float* h_d = reinterpret_cast<float*>(a.hq + a.h_off_d);
  int32_t* h_s = reinterpret_cast<int32_t*>(a.hq + a.h_off_s);
  auto apply = [&](const XO (&f)[NU], int s) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      const int uraw = lane + 64 * q;
      const bool ok = uraw < units;
      const int u = ok ? uraw : units - 1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        DecO<F> dec;
        decode_own(cur[r][q], u, lane & 1, ok, dec);
        const int dv = own_pass<F>(own_first(dec, f[q].f));
        acc[r] = own_apply(dec, own_second(dec, f[q].s, dv), f[q].p, acc[r]);
      }
    }
    float outv = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sv = wave_sum(acc[r]);
      outv = lane == r ? sv : outv;
    }
    outv = valid ? outv : 0.f;
    if (lane < R) {
      s_gu[(wave < 8 ? 0 : 32) + 4 * (wave & 7) + lane] = outv;
      if (a.y != nullptr) a.y[(int64_t)s * n_rows + row0 + lane] = outv;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane j of each group of 8: values 4j .. 4j + 3 of the block, as
      // k_swiglu_quantize holds them; lanes 0-7 store the block
      const int j = lane & 7;
      float hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = s_gu[4 * j + i], u = s_gu[32 + 4 * j + i];
        hv[i] = g / (1.0f + expf(-g)) * u;
      }
      float db;
      int sum;
      const uint32_t packed = q8_block8(hv, db, sum);
      if (lane < 8) {
        const int64_t o = (int64_t)s * n_ff + 32 * b + 4 * j;
        *reinterpret_cast<uint32_t*>(h_qs + o) = packed;
        if (j == 0) {
          h_d[(int64_t)s * nb + b] = db;
          h_s[(int64_t)s * nb + b] = sum;
        }
      }
    }
    __syncthreads();  // s_gu is reused by the next slot
  };
  apply(xf, slot);
  if (valid) {
    for (int c = slot / 64; c * 64 < n_slots; ++c) {
      const int sh = slot - c * 64;
      uint64_t m = same_in(c) & (sh < 0 ? ~0ull : ~((2ull << sh) - 1));
      while (m != 0) {  // uniform over the workgroup
        const int s2 = c * 64 + __builtin_ctzll(m);
        m &= m - 1;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int q = 0; q < NU; ++q) {
            uint32_t* rw = reinterpret_cast<uint32_t*>(&cur[r][q]);
#pragma unroll
            for (int i = 0; i < (int)(sizeof(RawS<F>) / 4); ++i) asm volatile("" : "+v"(rw[i]));
          }
        XO f2[NU];
#pragma unroll
        for (int q = 0; q < NU; ++q) load_xo<F>(gx, s2 / a.top_k, min(lane + 64 * q, units - 1), f2[q]);
        apply(f2, s2);
      }
    }
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) {  // wave 0, all lanes (slot 0 never exits early)
    const int drop = count_dropped(a, n_slots);
    if (threadIdx.x == 0) a.err[0] = drop;
  }
}

template <int F>
static hipError_t run_gate_up_swiglu(const MoeLaunch& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.n_ff / 32), (unsigned)(a.n_tok * a.top_k));
  if (a.units <= 64)
    hipLaunchKernelGGL((k_moe_gate_up_swiglu<F, 1>), grid, dim3(1024), 0, st, a);
  else
    hipLaunchKernelGGL((k_moe_gate_up_swiglu<F, 2>), grid, dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_moe_gate_up_swiglu(const MoeLaunch& a, hipStream_t st) {
  if (a.units > 128 || a.n_ff % 32 || a.n_rows != 2 * a.n_ff || a.x_per_slot || a.rw != nullptr)
    return hipErrorInvalidValue;
  switch (a.fmt) {
    case FQ8_0: return run_gate_up_swiglu<FQ8_0>(a, st);
    case FQ4_K: return run_gate_up_swiglu<FQ4_K>(a, st);
    case FIQ4_XS: return run_gate_up_swiglu<FIQ4_XS>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// The few-slot flat kernel with the route-weighted combine folded in:
// workgroup (x, t) takes rows x * WPB * R .. of token t for all of its
// top_k <= TK slots, issuing every slot's weight loads at once, and sums the
// slots' outputs (each reduced over the wave exactly as k_moe_flat reduces
// it) times their route weights in slot order -- the same fp32 operations
// in the same order as k_moe_combine, with no per-slot outputs and no second
// launch.  Slots past top_k re-load the last slot and are not added.
template <int F, int NU, int R, int WPB, int TK>
__global__ __launch_bounds__(64 * WPB) void k_moe_flat_comb(MoeLaunch a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.y;
  const int units = a.units;
  const int row0 = (blockIdx.x * WPB + wave) * R;
  const Act gx{a.x.qs, a.x.d, a.x.s, a.x.k, a.x.nb};
  int ev[TK];
  float wv[TK];
#pragma unroll
  for (int s = 0; s < TK; ++s) {
    const int sl = t * a.top_k + min(s, a.top_k - 1);
    ev[s] = a.ids[sl];
    wv[s] = a.rw[sl];
  }
  // With one unit per lane every slot's activation fragments fit beside the
  // weights: issued first (cache-resident), so no slot waits for a second
  // round trip.  Wider rows load each slot's fragments when it is used.
  constexpr bool kPre = NU == 1;
  XO xp[kPre ? TK : 1][NU];
  if constexpr (kPre) {
#pragma unroll
    for (int s = 0; s < TK; ++s) {
      const int xr = a.x_per_slot ? t * a.top_k + min(s, a.top_k - 1) : t;
#pragma unroll
      for (int q = 0; q < NU; ++q) load_xo<F>(gx, xr, min(lane + 64 * q, units - 1), xp[s][q]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  RawS<F> cur[TK][R][NU];
#pragma unroll
  for (int s = 0; s < TK; ++s) {
    const int e = ev[s] >= 0 && ev[s] < a.n_experts ? ev[s] : 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint8_t* wr = a.w + ((int64_t)e * a.n_rows + min(row0 + r, a.n_rows - 1)) * a.row_bytes;
#pragma unroll
      for (int q = 0; q < NU; ++q) load_unit_s(wr, min(lane + 64 * q, units - 1), lane, cur[s][r][q]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float sum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) sum[r] = 0.f;
#pragma unroll
  for (int s = 0; s < TK; ++s) {
    __builtin_amdgcn_sched_barrier(0);  // slots one after the other
    const bool use = s < a.top_k && ev[s] >= 0 && ev[s] < a.n_experts;
    XO xs[NU];
    if constexpr (kPre) {
#pragma unroll
      for (int q = 0; q < NU; ++q) xs[q] = xp[s][q];
    } else {
      const int xr = a.x_per_slot ? t * a.top_k + min(s, a.top_k - 1) : t;
#pragma unroll
      for (int q = 0; q < NU; ++q) load_xo<F>(gx, xr, min(lane + 64 * q, units - 1), xs[q]);
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      const int uraw = lane + 64 * q;
      const bool ok = uraw < units;
      const int u = ok ? uraw : units - 1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        DecO<F> dec;
        decode_own(cur[s][r][q], u, lane & 1, ok, dec);
        const int dv = own_pass<F>(own_first(dec, xs[q].f));
        acc[r] = own_apply(dec, own_second(dec, xs[q].s, dv), xs[q].p, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sv = wave_sum(acc[r]);
      if (use) sum[r] += wv[s] * sv;
    }
  }
  float outv = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) outv = lane == r ? sum[r] : outv;
  if (lane < R && row0 + lane < a.n_rows) a.y[(int64_t)t * a.n_rows + row0 + lane] = outv;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) {  // wave 0, all lanes
    const int drop = count_dropped(a, a.n_tok * a.top_k);
    if (threadIdx.x == 0) a.err[0] = drop;
  }
}

// One token, route-weighted, rows of at most 64 units (the down projection,
// 48 units per row): workgroup (x, t) takes rows 4Rx .. 4Rx + 4R - 1 for
// every slot of token t, wave s for slot s (top_k <= 8), each 16-lane group
// holding R rows with NU units per lane, so that all 64 lanes of a wave carry
// units (one row per wave left 16 of its lanes idle on 48-unit rows) and a
// workgroup runs eight waves of a few loads each rather than one wave of
// every slot's loads.  Every workgroup reads the activation rows of all its
// slots, so R = 2 halves those reads against one row per group (IQ4_XS
// 4096 x 1536: 8.63 -> 8.40 us; four rows per group, 9.10 us, leave too few
// waves).  A lane issues its activation fragments (the slot's own
// row when x is per slot) and then its weight loads; the 16-lane sums of the
// slots meet in LDS and the route-weighted sum is taken over the valid slots
// in slot order, as k_moe_combine takes it.
template <int F, int NU, int R>
__global__ __launch_bounds__(512) void k_moe_comb16(MoeLaunch a) {
  constexpr int RPW = 4 * R;  // rows per workgroup: four 16-lane groups of R rows
  __shared__ float s_part[8][RPW];
  __shared__ float s_w[8];
  __shared__ int s_ok[8];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // the slot
  const int t = blockIdx.y;
  const int units = a.units;
  const int j = lane & 15, rr = lane >> 4;
  const int s = min(wave, a.top_k - 1);
  const int sl = t * a.top_k + s;
  const int e = a.ids[sl];
  const float rw = a.rw[sl];  // loaded beside the id: the final sum reads only LDS
  const bool valid = wave < a.top_k && e >= 0 && e < a.n_experts;
  const int xr = a.x_per_slot ? sl : t;
  const Act gx{a.x.qs, a.x.d, a.x.s, a.x.k, a.x.nb};
  XO xf[NU];
#pragma unroll
  for (int q = 0; q < NU; ++q) load_xo<F>(gx, xr, min(j + 16 * q, units - 1), xf[q]);
  __builtin_amdgcn_sched_barrier(0);
  // row r of group rr is RPW * x + 4 r + rr: the four groups of a wave read
  // four consecutive rows
  const uint8_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    wr[r] = a.w + ((int64_t)(valid ? e : 0) * a.n_rows + min((int)blockIdx.x * RPW + 4 * r + rr, a.n_rows - 1)) *
                      a.row_bytes;
  RawS<F> cur[R][NU];
#pragma unroll
  for (int q = 0; q < NU; ++q)
#pragma unroll
    for (int r = 0; r < R; ++r) load_unit_s(wr[r], min(j + 16 * q, units - 1), lane, cur[r][q]);
  __builtin_amdgcn_sched_barrier(0);
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
  for (int q = 0; q < NU; ++q) {
    const int uraw = j + 16 * q;
    const bool ok = uraw < units;
    const int u = ok ? uraw : units - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      DecO<F> dec;
      decode_own(cur[r][q], u, lane & 1, ok, dec);
      const int dv = own_pass<F>(own_first(dec, xf[q].f));
      acc[r] = own_apply(dec, own_second(dec, xf[q].s, dv), xf[q].p, acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = lane_group_sum<16>(acc[r]);
    if (j == 0) s_part[wave][4 * r + rr] = valid ? v : 0.f;
  }
  if (lane == 0) {
    s_w[wave] = rw;
    s_ok[wave] = valid;
  }
  __syncthreads();
  if (threadIdx.x < RPW) {
    const int r2 = (int)blockIdx.x * RPW + threadIdx.x;
    float sum = 0.f;
    for (int s2 = 0; s2 < a.top_k; ++s2)
      if (s_ok[s2]) sum += s_w[s2] * s_part[s2][threadIdx.x];
    if (r2 < a.n_rows) a.y[(int64_t)t * a.n_rows + r2] = sum;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) {  // wave 0, all lanes
    const int drop = count_dropped(a, a.n_tok * a.top_k);
    if (threadIdx.x == 0) a.err[0] = drop;
  }
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

// Matrix-core launch: TM staged slot rows per group (TMP after rounding to
// token groups), 8-wave workgroups, a persistent grid sized by occupancy.
template <int F, int TM, bool DOTS = false>
static hipError_t run_moe_mx(const MoeLaunch& a0, hipStream_t st) {
  constexpr int WPB = 8;
  constexpr int TG = mx_tg<F>();
  constexpr int TMP = ((TM + TG - 1) / TG) * TG;
  MoeLaunch a = a0;
  auto kern = k_moe_mx<F, TM, WPB, DOTS>;
  const int64_t kb = 8 * (int64_t)((a.units + 7) / 8);
  size_t lds = (size_t)(kb * (TMP * 32 + 16) + 16 + kb * TMP * 4 * (F == FQ4_K ? 2 : 1));
  if (lds < (size_t)kMaxSlots * 4) lds = (size_t)kMaxSlots * 4;  // the ids during the sort
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
  if (occ0.static_lds + lds > (size_t)a.lds_per_cu) return hipErrorInvalidValue;
  int occ = occ0.regs;
  const int by_lds = (int)((size_t)a.lds_per_cu / (occ0.static_lds + lds));
  if (occ > by_lds) occ = by_lds;
  if (occ < 1) occ = 1;
  const int64_t slots = (int64_t)a.n_tok * a.top_k;
  const int64_t tiles = (a.n_rows + 15) / 16;
  const int64_t max_items = (slots < a.n_experts ? slots : a.n_experts) * tiles;
  const int64_t cap = (int64_t)a.cus * occ;
  const unsigned grid = (unsigned)(max_items < cap ? max_items : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.rw == nullptr || DOTS) return e;
  const int64_t outs = (int64_t)a.n_tok * a.n_rows;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_moe_mx_dots(const MoeLaunch& a, int tm, hipStream_t st) {
  if (a.dots == nullptr || (tm != 4 && tm != 8)) return hipErrorInvalidValue;
  switch (a.fmt) {
    case FQ8_0: return tm == 4 ? run_moe_mx<FQ8_0, 4, true>(a, st) : run_moe_mx<FQ8_0, 8, true>(a, st);
    case FQ4_K: return tm == 4 ? run_moe_mx<FQ4_K, 4, true>(a, st) : run_moe_mx<FQ4_K, 8, true>(a, st);
    case FIQ4_XS: return tm == 4 ? run_moe_mx<FIQ4_XS, 4, true>(a, st) : run_moe_mx<FIQ4_XS, 8, true>(a, st);
    default: return hipErrorInvalidValue;
  }
}

static int g_moe_row16 = 0;  // tuning: 0 16-lane row groups on short rows, 1 never
void set_moe_row16(int v) { g_moe_row16 = v; }

template <int F, int R>
static hipError_t run_comb16_r(const MoeLaunch& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.n_rows + 4 * R - 1) / (4 * R)), (unsigned)a.n_tok);
  switch ((a.units + 15) / 16) {
    case 1: hipLaunchKernelGGL((k_moe_comb16<F, 1, R>), grid, dim3(512), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_moe_comb16<F, 2, R>), grid, dim3(512), 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_moe_comb16<F, 3, R>), grid, dim3(512), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_moe_comb16<F, 4, R>), grid, dim3(512), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int F>
static hipError_t run_comb16(const MoeLaunch& a, hipStream_t st) {
  return run_comb16_r<F, 2>(a, st);
}

template <int F, int NU, int R>
static hipError_t run_moe_flat(const MoeLaunch& a, hipStream_t st) {
  constexpr int WPB = 4;
  if (a.rw != nullptr && a.top_k <= 8 && a.n_tok == 1 && a.units <= 64 && g_moe_row16 == 0)
    return run_comb16<F>(a, st);
  if constexpr (NU <= 2) {
    if (a.rw != nullptr && a.top_k <= 8 && a.n_tok == 1) {
      // one token, route-weighted, top_k <= 8: the combine folded into the
      // kernel, one row per wave, every slot's weights in flight (measured
      // 4096 x 1536 down: one token 11.1 -> 10.7 us, 10.2 us with every
      // slot's activation fragments issued up front, and no better with two
      // rows per wave (167 VGPRs, 10.2-10.4 us); at six tokens the
      // per-slot grid and the combine kernel were faster, 39.5 against 43.1)
      const unsigned gx = (unsigned)((a.n_rows + WPB - 1) / WPB);
      hipLaunchKernelGGL((k_moe_flat_comb<F, NU, 1, WPB, 8>), dim3(gx, (unsigned)a.n_tok), dim3(64 * WPB), 0, st, a);
      return hipGetLastError();
    }
  }
  const int64_t slots = (int64_t)a.n_tok * a.top_k;
  const unsigned gx = (unsigned)((a.n_rows + R * WPB - 1) / (R * WPB));
  hipLaunchKernelGGL((k_moe_flat<F, NU, R, WPB>), dim3(gx, (unsigned)slots), dim3(64 * WPB), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.rw == nullptr) return e;
  const int64_t outs = (int64_t)a.n_tok * a.n_rows;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// One row chunk per lane: NU = units / 64 rounded up (at most 8: k <= 16384);
// four rows per wave for rows of one unit per lane, and of two from six
// tokens (measured: 4096 x 1536 at six tokens 42.0 -> 39.4 us; 3072 x 4096
// at one token 12.1 against 12.4 us with four rows, at 16 tokens 144.5 ->
// 138.9 us).
// The per-slot grid with 16-lane row groups: rows of fewer than 64 units
// (the down projection's inputs, one activation row per slot).  Every wave
// reads its slot's activation row, so R = 2 rows per group halve those reads
// against one (48-unit rows, 128 experts, at 2 / 4 / 6 / 8 tokens: 17.35 /
// 27.64 / 38.03 / 48.17 -> 16.22 / 25.39 / 34.72 / 43.73 us, bit-identical).
template <int F, int NU16, int R = 1>
static hipError_t run_moe_flat16(const MoeLaunch& a, hipStream_t st) {
  constexpr int WPB = 4;
  const int64_t slots = (int64_t)a.n_tok * a.top_k;
  const unsigned gx = (unsigned)((a.n_rows + 4 * R * WPB - 1) / (4 * R * WPB));
  hipLaunchKernelGGL((k_moe_flat<F, NU16, R, WPB, 16>), dim3(gx, (unsigned)slots), dim3(64 * WPB), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.rw == nullptr) return e;
  const int64_t outs = (int64_t)a.n_tok * a.n_rows;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int F>
static hipError_t run_moe_flat_fmt(const MoeLaunch& a, hipStream_t st) {
  const int nu = (a.units + 63) / 64;
  // 16-lane row groups for the per-slot inputs of a down projection; a
  // gate+up (one activation row per token) keeps the 64-lane rows that the
  // one-launch FFN kernel reduces the same way, so that its sums are
  // bit-identical to this path's
  if (a.units < 64 && a.x_per_slot && g_moe_row16 == 0 && !(a.rw != nullptr && a.top_k <= 8 && a.n_tok == 1)) {
    switch ((a.units + 15) / 16) {
      case 1: return run_moe_flat16<F, 1>(a, st);
      case 2: return run_moe_flat16<F, 2>(a, st);
      case 3: return run_moe_flat16<F, 3, 2>(a, st);
      default: return run_moe_flat16<F, 4>(a, st);
    }
  }
  // rows of up to 128 blocks: four rows per wave (the 128-expert gate+up,
  // 3072 x 4096 per expert, at 1 / 2 / 4 tokens: 13.99 / 24.19 / 44.39 us with
  // two rows per wave, whose grid of 12288 waves at one token does not fit
  // the device at once, against 13.49 / 23.22 / 40.25 with four)
  switch (nu) {
    case 1: return run_moe_flat<F, 1, 4>(a, st);
    case 2: return run_moe_flat<F, 2, 4>(a, st);
    case 3: return run_moe_flat<F, 3, 1>(a, st);
    case 4: return run_moe_flat<F, 4, 1>(a, st);
    default: return run_moe_flat<F, 8, 1>(a, st);
  }
}

static int g_moe_kernel = 0;  // tuning: 0 automatic, 1 vector-ALU, 2 matrix-core, 3 few-slot flat kernel
void set_moe_kernel(int v) { g_moe_kernel = v; }
int moe_kernel() { return g_moe_kernel; }

// The few-slot flat kernel while grouping slots by expert saves less than
// its routing costs (measured on 128 experts, top-8: one activation row per
// token, 3072 x 4096 rows, up to 20 tokens -- 16.1 -> 12.3 us at one token,
// at 20 / 32 tokens 153.5-158.3 / 232.1 us against 168.6-168.9 / 207.0 for
// the matrix-core kernel, at 24 within 5% either way on two boxes; one row
// per slot, 4096 x 1536, up to 8 tokens -- 13.6 -> 11.6 us at one); then the
// vector-ALU grouped kernel, and the matrix-core kernel when experts receive
// several slots: from 21 tokens with one activation row per token, and with
// one per slot from 21 too, and from 9 for q4_K and for IQ4_XS rows of fewer
// than 48 blocks.  Down projections at 9..20 tokens, us: IQ4_XS 4096 x 1536
// (128 experts) at 12 / 16 / 20 tokens 63.0 / 75.6 / 86.5 with the vector
// kernel against 70.7 / 80.6 / 88.7, Q8_0 2048 x 768 34.0 against 39.8 at 16;
// but q4_K 4096 x 1536 83.9 against 120.7 at 16 with the matrix-core kernel,
// q4_K and IQ4_XS 2048 x 768 23.9 / 24.7 against 32.6 / 32.8 (the boundary
// between 24 and 48 blocks per row is not measured); at 24 / 32 tokens IQ4_XS
// 4096 x 1536 94.8 / 107.2 against 96.5 / 117.1.  4 (8 from 17 tokens) slot
// rows per group.
// Q8_0 experts, whose decode is a byte copy, never gain from the matrix
// cores up to 64 tokens: gate+up on the few-slot kernel (3072 x 4096 at 24 /
// 32 / 48 / 64 tokens 231 / 273 / 339 / 400 us against 387 / 417 / 455 / 495),
// down on the vector kernel from 9 (146 / 167 / 181 / 191 against 181 / 200 /
// 227 / 237).
template <int F>
static bool moe_slots_on_matrix_cores(const MoeLaunch& a) {
  if (F == FQ8_0) return a.n_tok > 64;
  if (a.n_tok >= 21) return true;
  if (!a.x_per_slot || a.n_tok <= 8) return false;
  return F == FQ4_K || (F == FIQ4_XS && a.units < 48);
}
template <int F>
static hipError_t run_moe_any(const MoeLaunch& a, hipStream_t st) {
  // per-slot inputs: the few-slot kernel up to 8 tokens, and up to 12 on
  // IQ4_XS rows of 48 blocks, whose two-row 16-lane groups beat the grouped
  // vector kernel there (4096 x 1536 down at 9 / 12 / 14 / 16 tokens: 48.4 /
  // 60.0 / 68.7 / 75.9 against 52.7 / 63.7 / 68.7 / 75.1 us)
  const int few_slot_max = a.x_per_slot ? (F == FIQ4_XS && a.units == 48 ? 12 : 8) : F == FQ8_0 ? 64 : 20;
  if (g_moe_kernel == 3 || (g_moe_kernel == 0 && a.n_tok <= few_slot_max))
    return run_moe_flat_fmt<F>(a, st);
  const bool mx = g_moe_kernel == 2 || (g_moe_kernel == 0 && moe_slots_on_matrix_cores<F>(a));
  if (mx) {
    const hipError_t e = a.n_tok <= 16 ? run_moe_mx<F, 4>(a, st) : run_moe_mx<F, 8>(a, st);
    if (e != hipErrorInvalidValue) return e;  // else the staged rows do not fit: vector kernel
  }
  return run_moe_fmt<F>(a, st);
}

hipError_t launch_moe(const MoeLaunch& a, hipStream_t st) {
  switch (a.fmt) {
    case FQ8_0: return run_moe_any<FQ8_0>(a, st);
    case FQ4_K: return run_moe_any<FQ4_K>(a, st);
    case FIQ4_XS: return run_moe_any<FIQ4_XS>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmv
