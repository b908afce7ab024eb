// qmv_router.hip -- MoE router and top-k, for gfx950 (Castagna Veloce page,
// "Fused operations": router matvec, gating, top-k and weight normalization
// for decode at one to a few tokens).
//
// Two launches.  k_router_logits computes l = W x for a tile of EG experts by
// TG tokens per workgroup (TG: n_tok rounded up to a power of two, at most
// 4): its eight waves split K into interleaved 256-column chunks (one 16-byte
// load per lane, per expert row and per token, two chunks in flight), every
// lane accumulates the EG x TG products of its columns in registers, a
// butterfly across the wave leaves each lane with one product's wave sum, and
// the eight wave sums meet in LDS.  The router weights are read once per token
// group, spread over n_experts / EG workgroups.  Optionally the workgroups
// of the first expert group also write the Q8 activation blocks of their
// tokens: the eight lanes holding a 32-column block run the quantizer's
// block routine on the x values they loaded (the same values and steps as
// k_quantize, so the same bytes).
// k_router_select takes one workgroup per token: each expert's rank is the
// number of experts with a larger logit, or an equal one and a lower index
// (one 64-bit key compare per expert); ranks below top_k are the picks in
// order, and their weights are a softmax over the chosen logits.  Logits are fp32 sums; exp is the accurate expf.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

constexpr int kRouterMaxExperts = 1024;
constexpr int kRouterMaxTopK = 16;
constexpr int kRouterWaves = 8;

// One butterfly step over the first 2H values of v: lanes whose bit H is set
// keep the upper half, the others the lower half, each adding its partner's
// copy of the half it keeps.  After the steps H = P/2 .. 1, lane l holds the
// sum of value l % P over its aligned group of P lanes.
template <int H>
__device__ __forceinline__ void fold(float* v, int lane) {
  const bool hi = (lane & H) != 0;
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const float send = hi ? v[j] : v[j + H];
    const float keep = hi ? v[j + H] : v[j];
    v[j] = keep + __shfl_xor(send, H, 64);
  }
}

template <int P>
__device__ __forceinline__ float fold_all(float* v, int lane) {
  if constexpr (P >= 64) fold<32>(v, lane);
  if constexpr (P >= 32) fold<16>(v, lane);
  if constexpr (P >= 16) fold<8>(v, lane);
  if constexpr (P >= 8) fold<4>(v, lane);
  if constexpr (P >= 4) fold<2>(v, lane);
  if constexpr (P >= 2) fold<1>(v, lane);
  float r = v[0];
#pragma unroll
  for (int o = P; o < 64; o <<= 1) r += __shfl_xor(r, o, 64);  // the other lane groups
  return r;
}

// EG experts x one chunk of 256 columns (one 16-byte load per lane and row),
// TG tokens; rows and tokens past the ends are clamped (their products are
// discarded at the store).
template <int EG, int TG>
struct RouterChunk {
  f32x4 w[EG];
  f32x4 x[TG];
  __device__ __forceinline__ void load(const float* __restrict__ x_, int64_t ldx, int n_tok, int t0, int k,
                                       const float* __restrict__ wr, int n_experts, int e0, int c) {
#pragma unroll
    for (int e = 0; e < EG; ++e)
      w[e] = *reinterpret_cast<const f32x4*>(wr + (int64_t)min(e0 + e, n_experts - 1) * k + c);
#pragma unroll
    for (int t = 0; t < TG; ++t)
      x[t] = *reinterpret_cast<const f32x4*>(x_ + (int64_t)min(t0 + t, n_tok - 1) * ldx + c);
  }
  __device__ __forceinline__ void fma(float* acc) const {
#pragma unroll
    for (int e = 0; e < EG; ++e)
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        float a = acc[e * TG + t];
        a = fmaf(w[e].x, x[t].x, a);
        a = fmaf(w[e].y, x[t].y, a);
        a = fmaf(w[e].z, x[t].z, a);
        a = fmaf(w[e].w, x[t].w, a);
        acc[e * TG + t] = a;
      }
  }
};

template <int EG, int TG>
__global__ __launch_bounds__(64 * kRouterWaves) void k_router_logits(const float* __restrict__ x, int64_t ldx,
                                                                     int n_tok, int k,
                                                                     const float* __restrict__ wr,
                                                                     int n_experts, float* __restrict__ logits,
                                                                     int8_t* __restrict__ xq_qs,
                                                                     float* __restrict__ xq_d,
                                                                     int32_t* __restrict__ xq_s) {
  constexpr int P = EG * TG;
  static_assert(P <= 64 && (P & (P - 1)) == 0, "products per lane: a power of two up to 64");
  __shared__ float red[kRouterWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * EG, t0 = blockIdx.y * TG;
  float acc[P];
#pragma unroll
  for (int i = 0; i < P; ++i) acc[i] = 0.f;

  constexpr int kStep = 4 * 64 * kRouterWaves;  // columns per round of the workgroup
  // Q8 blocks of x: workgroups of the first expert group, uniform per
  // workgroup.  The eight lanes 8i..8i+7 hold the 32 columns of one block
  // (k % 32 == 0), so a block is either wholly inside the loop or wholly out.
  const bool qx = xq_qs != nullptr && blockIdx.x == 0;
  const int nb = k / 32;
  auto put = [&](const RouterChunk<EG, TG>& ch, int col) {
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      if (t0 + t < n_tok) {  // uniform
        const float vv[4] = {ch.x[t].x, ch.x[t].y, ch.x[t].z, ch.x[t].w};
        float db;
        int sum;
        const uint32_t packed = q8_block8(vv, db, sum);
        *reinterpret_cast<uint32_t*>(xq_qs + (int64_t)(t0 + t) * k + col) = packed;
        if ((lane & 7) == 0) {
          xq_d[(int64_t)(t0 + t) * nb + col / 32] = db;
          xq_s[(int64_t)(t0 + t) * nb + col / 32] = sum;
        }
      }
    }
  };
  int c = 4 * (lane + 64 * wave);
  for (; c + kStep < k; c += 2 * kStep) {  // two chunks in flight
    RouterChunk<EG, TG> a, b;
    a.load(x, ldx, n_tok, t0, k, wr, n_experts, e0, c);
    b.load(x, ldx, n_tok, t0, k, wr, n_experts, e0, c + kStep);
    if (qx) {
      put(a, c);
      put(b, c + kStep);
    }
    a.fma(acc);
    b.fma(acc);
  }
  if (c < k) {
    RouterChunk<EG, TG> a;
    a.load(x, ldx, n_tok, t0, k, wr, n_experts, e0, c);
    if (qx) put(a, c);
    a.fma(acc);
  }
  const float r = fold_all<P>(acc, lane);
  red[wave][lane] = r;
  __syncthreads();
  if (wave == 0 && lane < P) {
    float s = red[0][lane];
#pragma unroll
    for (int w = 1; w < kRouterWaves; ++w) s += red[w][lane];
    const int e = e0 + lane / TG, t = t0 + lane % TG;
    if (e < n_experts && t < n_tok) logits[(int64_t)t * n_experts + e] = s;
  }
}

// Expert e's place in the order: the number of experts whose logit is larger,
// or equal with a lower index.  Each expert gets a 64-bit key that orders that
// way (the logit's bits made monotone, -0 taken as +0, above the complement of
// the index), so a rank is one unsigned compare per expert.  Ranks below
// top_k are the picks, in order.
__device__ __forceinline__ uint64_t router_key(float v, int e) {
  uint32_t u = __float_as_uint(v + 0.f);  // -0 -> +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__global__ __launch_bounds__(256) void k_router_select(const float* __restrict__ logits, int n_experts, int top_k,
                                                       int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ uint64_t s_key[kRouterMaxExperts + 3];
  __shared__ float s_val[kRouterMaxExperts];
  __shared__ float s_pv[kRouterMaxTopK];  // chosen logits, in pick order
  __shared__ int s_pi[kRouterMaxTopK];    // chosen experts
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* l = logits + (int64_t)t * n_experts;
  const int n4 = (n_experts + 3) & ~3;
  for (int e = tid; e < n4; e += 256) {
    const float v = e < n_experts ? l[e] : 0.f;
    s_val[e] = v;
    s_key[e] = e < n_experts ? router_key(v, e) : 0;  // 0: below every expert
  }
  if (tid < kRouterMaxTopK) {  // defined picks even for non-finite logits
    s_pv[tid] = 0.f;
    s_pi[tid] = -1;
  }
  __syncthreads();
  for (int e = tid; e < n_experts; e += 256) {
    const uint64_t me = s_key[e];
    // four partial counts, sixteen keys per step: the LDS reads of a step
    // are in flight together
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
#pragma unroll 4
    for (int j = 0; j < n4; j += 4) {
      r0 += s_key[j] > me ? 1 : 0;
      r1 += s_key[j + 1] > me ? 1 : 0;
      r2 += s_key[j + 2] > me ? 1 : 0;
      r3 += s_key[j + 3] > me ? 1 : 0;
    }
    const int rank = (r0 + r1) + (r2 + r3);
    if (rank < top_k) {
      s_pv[rank] = s_val[e];
      s_pi[rank] = e;
    }
  }
  __syncthreads();
  if (tid < top_k) {  // every lane forms the same sum, in pick order
    const float m = s_pv[0];
    float sum = 0.f;
    for (int j = 0; j < top_k; ++j) sum += expf(s_pv[j] - m);
    ids[(int64_t)t * top_k + tid] = s_pi[tid];
    w[(int64_t)t * top_k + tid] = expf(s_pv[tid] - m) / sum;
  }
}

template <int EG, int TG>
static void launch_logits(const float* x, int64_t ldx, int n_tok, int k, const float* wr, int n_experts,
                          float* logits, int8_t* xq_qs, float* xq_d, int32_t* xq_s, hipStream_t st) {
  const dim3 grid((unsigned)((n_experts + EG - 1) / EG), (unsigned)((n_tok + TG - 1) / TG));
  hipLaunchKernelGGL((k_router_logits<EG, TG>), grid, dim3(64 * kRouterWaves), 0, st, x, ldx, n_tok, k, wr,
                     n_experts, logits, xq_qs, xq_d, xq_s);
}

hipError_t launch_router_topk(const float* x, int64_t ldx, int n_tok, int k, const float* wr, int n_experts,
                              int top_k, int32_t* ids, float* w, float* logits, int8_t* xq_qs, float* xq_d,
                              int32_t* xq_s, hipStream_t st) {
  // token groups of up to 4 (each workgroup then reads 4 x rows, 4 expert rows)
  if (n_tok == 1) launch_logits<1, 1>(x, ldx, n_tok, k, wr, n_experts, logits, xq_qs, xq_d, xq_s, st);
  else if (n_tok == 2) launch_logits<2, 2>(x, ldx, n_tok, k, wr, n_experts, logits, xq_qs, xq_d, xq_s, st);
  else launch_logits<4, 4>(x, ldx, n_tok, k, wr, n_experts, logits, xq_qs, xq_d, xq_s, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_router_select, dim3((unsigned)n_tok), dim3(256), 0, st, logits, n_experts, top_k, ids, w);
  return hipGetLastError();
}

}  // namespace qmv
