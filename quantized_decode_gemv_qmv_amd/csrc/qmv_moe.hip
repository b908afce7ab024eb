// qmv_moe.hip -- expert-grouped routed matvec for MoE decode (1..64 tokens).
//
// Castagna Veloce page, "Kernels for the MI50": i-quant MoE decode kernels for
// batches of up to 64 tokens, and expert-grouped quantized MoE where each
// active expert runs once over all the tokens routed to it.
//
// k_moe grid: x = row tiles of the expert matrices, y = rank a of an active
// expert (upper bound min(n_experts, n_tok * top_k)).  Each workgroup rebuilds
// the routing it needs in LDS from the ids (at most 1024 slots), so routing
// costs no launch of its own:
//   1. a bitmap of the experts that appear in ids; its population count is
//      the number of active experts U, and the a-th set bit is this
//      workgroup's expert e (workgroups with a >= U leave);
//   2. the slots routed to e, compacted in slot order with wave ballots.
// A lane group of LPR lanes owns one row of W[e]: it issues all the loads of
// the row at once (NU units per lane, block headers shared by lane quads),
// decodes them into registers once and applies them, in the own-block form of
// qmv_device.h, to every slot routed to e, so each active expert's weights
// are read from HBM once per call.  The
// next slot's activation fragments are fetched while the current slot is
// computed.
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

template <int F, int LPR, int NU>
__global__ __launch_bounds__(256) void k_moe(MoeLaunch a) {
  constexpr int GPW = 64 / LPR;
  constexpr int RWG = 4 * GPW;  // rows per workgroup
  __shared__ uint32_t s_bits[kMaxExperts / 32];
  __shared__ int s_list[kMaxSlots];
  __shared__ int s_wcnt[4];
  __shared__ int s_e, s_U;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_slots = a.n_tok * a.top_k;
  const int nwords = (a.n_experts + 31) / 32;
  const int r0 = blockIdx.x * RWG;

  if (tid < nwords) s_bits[tid] = 0u;
  __syncthreads();
  int my_id[kMaxSlots / 256];
  int dropped = 0;
#pragma unroll
  for (int j = 0; j < kMaxSlots / 256; ++j) {
    const int i = tid + 256 * j;
    my_id[j] = i < n_slots ? a.ids[i] : -1;
    const int e = my_id[j];
    if (i < n_slots) {
      if (e >= 0 && e < a.n_experts)
        atomicOr(&s_bits[e >> 5], 1u << (e & 31));
      else
        ++dropped;
    }
  }
  __syncthreads();

  if (wave == 0) {
    const uint32_t bits = lane < nwords ? s_bits[lane] : 0u;
    const int pc = __popc(bits);
    int incl = pc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int total = __shfl(incl, 63, 64);
    const int rank = blockIdx.y;
    const int excl = incl - pc;
    if (rank >= excl && rank < incl) {
      uint32_t b = bits;
      for (int q = 0; q < rank - excl; ++q) b &= b - 1u;
      s_e = lane * 32 + (__ffs(b) - 1);
    }
    if (lane == 0) s_U = total;
  }
  __syncthreads();
  const int U = s_U;

  // Workgroups of active-expert rank 0 also write what no expert writes: the
  // dropped-slot count (workgroup (0, 0)) and, with one output per slot, the
  // zero rows of dropped slots.
  if (blockIdx.y == 0) {
    if (blockIdx.x == 0) {
      int dsum = dropped;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dsum += __shfl_xor(dsum, o, 64);
      if (lane == 0) s_wcnt[wave] = dsum;
      __syncthreads();
      if (tid == 0) a.err[0] = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
      __syncthreads();
    }
    if (a.rw == nullptr) {
      for (int idx = tid; idx < n_slots * RWG; idx += 256) {
        const int i = idx / RWG, row = r0 + idx % RWG;
        const int e = a.ids[i];
        if (row < a.n_rows && (e < 0 || e >= a.n_experts)) a.y[(int64_t)i * a.n_rows + row] = 0.f;
      }
    }
  }
  if ((int)blockIdx.y >= U) return;  // uniform across the workgroup
  const int e = s_e;

  // slots routed to e, in slot order
  int n_e = 0;
  for (int j = 0; j < kMaxSlots / 256; ++j) {
    if (256 * j >= n_slots) break;  // uniform
    const bool f = (tid + 256 * j < n_slots) && my_id[j] == e;
    const uint64_t m = __ballot(f);
    if (lane == 0) s_wcnt[wave] = __popcll(m);
    __syncthreads();
    int off = n_e;
    for (int w = 0; w < wave; ++w) off += s_wcnt[w];
    if (f) s_list[off + __popcll(m & ((1ull << lane) - 1ull))] = tid + 256 * j;
    n_e += s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
    __syncthreads();
  }

  // this lane group's row of W[e]: every load issued at once, decoded once
  const int g = lane / LPR, gl = lane % LPR;
  const int row = r0 + wave * GPW + g;
  const uint8_t* wr = a.w + ((int64_t)e * a.n_rows + min(row, a.n_rows - 1)) * a.row_bytes;
  const Act x{a.x.qs, a.x.d, a.x.s, a.x.k, a.x.nb};
  const int units = a.units;
  DecO<F> dec[NU];
  {
    RawS<F> raw[NU];
#pragma unroll
    for (int q = 0; q < NU; ++q) load_unit_s(wr, min(gl + LPR * q, units - 1), lane, raw[q]);
#pragma unroll
    for (int q = 0; q < NU; ++q)
      decode_own(raw[q], min(gl + LPR * q, units - 1), gl & 1, gl + LPR * q < units, dec[q]);
  }

  auto slot_row = [&](int j) {
    const int i = s_list[j];
    return a.x_per_slot ? i : i / a.top_k;
  };
  XO xf[NU];
  if (n_e > 0) {
    const int xr = slot_row(0);
#pragma unroll
    for (int q = 0; q < NU; ++q) load_xo<F>(x, xr, min(gl + LPR * q, units - 1), xf[q]);
  }
  for (int j = 0; j < n_e; ++j) {
    const int i = s_list[j];
    XO nx[NU];
    const int xr_next = slot_row(min(j + 1, n_e - 1));
#pragma unroll
    for (int q = 0; q < NU; ++q) load_xo<F>(x, xr_next, min(gl + LPR * q, units - 1), nx[q]);
    float acc = 0.f;
    int dv[NU];
#pragma unroll
    for (int q = 0; q < NU; ++q) dv[q] = own_pass<F>(own_first(dec[q], xf[q].f));
#pragma unroll
    for (int q = 0; q < NU; ++q) acc = own_apply(dec[q], own_second(dec[q], xf[q].s, dv[q]), xf[q].p, acc);
    acc = lane_group_sum<LPR>(acc);
    if (gl == 0 && row < a.n_rows) {
      float* out = a.rw == nullptr ? a.y : a.part;
      out[(int64_t)i * a.n_rows + row] = acc;
    }
#pragma unroll
    for (int q = 0; q < NU; ++q) xf[q] = nx[q];
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

int moe_rows_per_wg(int, int units) { return 4 * (64 / moe_lpr(units)); }

template <int F, int LPR, int NU>
static hipError_t run_moe(const MoeLaunch& a, hipStream_t st) {
  constexpr int RWG = 4 * (64 / LPR);
  const unsigned tiles = (unsigned)((a.n_rows + RWG - 1) / RWG);
  const int slots = a.n_tok * a.top_k;
  const unsigned ranks = (unsigned)(slots < a.n_experts ? slots : a.n_experts);
  hipLaunchKernelGGL((k_moe<F, LPR, NU>), dim3(tiles, ranks), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.rw == nullptr) return e;
  const int64_t outs = (int64_t)a.n_tok * a.n_rows;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int F>
static hipError_t run_moe_fmt(const MoeLaunch& a, hipStream_t st) {
  const int lpr = moe_lpr(a.units), nu = moe_nu(a.units);
  if (lpr == 16) {
    switch (nu) {
      case 1: return run_moe<F, 16, 1>(a, st);
      case 2: return run_moe<F, 16, 2>(a, st);
      case 3: return run_moe<F, 16, 3>(a, st);
      default: return run_moe<F, 16, 4>(a, st);
    }
  }
  switch (nu) {
    case 2: return run_moe<F, 64, 2>(a, st);
    case 3: return run_moe<F, 64, 3>(a, st);
    case 4: return run_moe<F, 64, 4>(a, st);
    default: return run_moe<F, 64, 8>(a, st);
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
