// qmv_moe.hip -- expert-grouped routed matvec for MoE decode (1..64 tokens).
//
// Castagna Veloce page, "Kernels for the MI50": i-quant MoE decode kernels for
// batches of up to 64 tokens, and expert-grouped quantized MoE where each
// active expert runs once over all the tokens routed to it.
//
// Grid: x = row tiles of the expert matrices, y = rank a of an active expert
// (upper bound min(n_experts, n_tok * top_k)).  Each workgroup rebuilds the
// routing metadata it needs in LDS from the ids (at most 1024 slots), so the
// whole call is one launch:
//   1. a bitmap of the experts that appear in ids; its population count is
//      the number of active experts U, and the a-th set bit is this
//      workgroup's expert e (workgroups with a >= U leave);
//   2. the slots routed to e, compacted in slot order with wave ballots.
// Each lane group then decodes its row's units of W[e] into registers once and
// reuses them for every slot routed to e, so each active expert's weights are
// read from HBM exactly once per call.
// Route-weighted combine (y[t] = sum_s w[t][s] * y_slot): per-slot outputs go
// to the workspace and the last workgroup to finish a row tile sums them in
// slot order -- deterministic, no float atomics, no second launch.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

constexpr int kMaxSlots = 64 * 16;
constexpr int kMaxExperts = 1024;

template <int F, int LPR, int UPL>
__global__ __launch_bounds__(256) void k_moe(MoeLaunch a) {
  constexpr int GPW = 64 / LPR;
  constexpr int RWG = 4 * GPW;  // rows per workgroup
  __shared__ uint32_t s_bits[kMaxExperts / 32];
  __shared__ int s_list[kMaxSlots];
  __shared__ int s_wcnt[4];
  __shared__ int s_e, s_U, s_last;

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

  // Workgroups of active-expert rank 0 also own the outputs nobody else
  // writes: dropped slots (per-slot mode) or, with no active expert at all,
  // the whole combined output.
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
    } else if (U == 0) {
      for (int idx = tid; idx < a.n_tok * RWG; idx += 256) {
        const int t = idx / RWG, row = r0 + idx % RWG;
        if (row < a.n_rows) a.y[(int64_t)t * a.n_rows + row] = 0.f;
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

  // this lane group's row of W[e], decoded once into registers
  const int g = lane / LPR, gl = lane % LPR;
  const int row = r0 + wave * GPW + g;
  const uint8_t* wr =
      a.w + ((int64_t)e * a.n_rows + min(row, a.n_rows - 1)) * a.row_bytes;
  const Act x{a.x.qs, a.x.d, a.x.s, a.x.k, a.x.nb};
  Dec<F> dec[UPL];
  {
    Raw<F> raw[UPL];
#pragma unroll
    for (int ui = 0; ui < UPL; ++ui) {
      const int u = gl + LPR * ui;
      if (u < a.units) load_unit(wr, u, raw[ui]);
    }
#pragma unroll
    for (int ui = 0; ui < UPL; ++ui) {
      const int u = gl + LPR * ui;
      if (u < a.units) decode_unit(raw[ui], u, dec[ui]);
    }
  }

  for (int j = 0; j < n_e; ++j) {
    const int i = s_list[j];
    const int xr = a.x_per_slot ? i : i / a.top_k;
    float acc = 0.f;
#pragma unroll
    for (int ui = 0; ui < UPL; ++ui) {
      const int u = gl + LPR * ui;
      if (u < a.units) {
        XFrag<F> xf;
        load_xfrag<F>(x, xr, u, xf);
        acc += unit_value(dec[ui], xf);
      }
    }
    acc = group_sum<LPR>(acc);
    if (gl == 0 && row < a.n_rows) {
      if (a.rw == nullptr)
        a.y[(int64_t)i * a.n_rows + row] = acc;
      else
        __hip_atomic_store(&a.part[(int64_t)i * a.n_rows + row], acc, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  if (a.rw != nullptr) {
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&a.cnt[blockIdx.x], 1);
      s_last = (prev == U - 1);
    }
    __syncthreads();
    if (s_last) {
      __threadfence();
      for (int idx = tid; idx < a.n_tok * RWG; idx += 256) {
        const int t = idx / RWG, rr = r0 + idx % RWG;
        if (rr >= a.n_rows) continue;
        float sum = 0.f;
        for (int s = 0; s < a.top_k; ++s) {
          const int sl = t * a.top_k + s;
          const int es = a.ids[sl];
          if (es >= 0 && es < a.n_experts)
            sum += a.rw[sl] * __hip_atomic_load(&a.part[(int64_t)sl * a.n_rows + rr],
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        a.y[(int64_t)t * a.n_rows + rr] = sum;
      }
      if (tid == 0) atomicExch(&a.cnt[blockIdx.x], 0);
    }
  }
}

static int moe_lpr(int units) { return units <= 128 ? 16 : (units <= 256 ? 32 : 64); }

int moe_rows_per_wg(int, int units) { return 4 * (64 / moe_lpr(units)); }

template <int F, int LPR, int UPL>
static hipError_t run_moe(const MoeLaunch& a, hipStream_t st) {
  constexpr int RWG = 4 * (64 / LPR);
  const unsigned tiles = (unsigned)((a.n_rows + RWG - 1) / RWG);
  const int slots = a.n_tok * a.top_k;
  const unsigned ranks = (unsigned)(slots < a.n_experts ? slots : a.n_experts);
  hipLaunchKernelGGL((k_moe<F, LPR, UPL>), dim3(tiles, ranks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int F, int LPR>
static hipError_t run_moe_upl(const MoeLaunch& a, hipStream_t st) {
  const int upl = (a.units + LPR - 1) / LPR;
  if (upl <= 1) return run_moe<F, LPR, 1>(a, st);
  if (upl <= 2) return run_moe<F, LPR, 2>(a, st);
  if (upl <= 4) return run_moe<F, LPR, 4>(a, st);
  if (upl <= 8) return run_moe<F, LPR, 8>(a, st);
  return hipErrorInvalidValue;
}

template <int F>
static hipError_t run_moe_fmt(const MoeLaunch& a, hipStream_t st) {
  switch (moe_lpr(a.units)) {
    case 16: return run_moe_upl<F, 16>(a, st);
    case 32: return run_moe_upl<F, 32>(a, st);
    default: return run_moe_upl<F, 64>(a, st);
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
