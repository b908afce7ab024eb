// qmv_router.hip -- MoE router and top-k in one kernel, for gfx950
// (Castagna Veloce page, "Fused operations": router matvec, gating, top-k and
// weight normalization in one kernel, for decode at one to a few tokens).
//
// One workgroup per token.  The token's activations are copied into LDS; the
// four waves take the experts round-robin, each expert's logit a 64-lane dot
// over K (one 16-byte load of the router row per lane and step, a DPP
// reduction).  Wave 0 then selects the top_k experts -- a larger logit first,
// on equal logits the lower expert index -- with one 64-lane argmax per
// pick, and normalizes their weights with a softmax over the chosen logits.
// Logits are fp32 sums; exp is the accurate expf.
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

constexpr int kRouterMaxExperts = 1024;
constexpr int kRouterMaxTopK = 16;

// (value, index) of the better of two candidates: larger value, then lower
// index; an index of -1 is no candidate.
__device__ __forceinline__ bool router_better(float va, int ia, float vb, int ib) {
  if (ia < 0) return false;
  if (ib < 0) return true;
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ x, int64_t ldx, int k,
                                                     const float* __restrict__ wr, int n_experts, int top_k,
                                                     int32_t* __restrict__ ids, float* __restrict__ w,
                                                     float* __restrict__ logits_out) {
  extern __shared__ __attribute__((aligned(16))) float s_x[];  // [k]
  __shared__ float s_l[kRouterMaxExperts];
  __shared__ float s_pv[kRouterMaxTopK];  // chosen logits, in pick order
  __shared__ int s_pi[kRouterMaxTopK];    // chosen experts
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < k / 4; i += 256)
    reinterpret_cast<f32x4*>(s_x)[i] = *reinterpret_cast<const f32x4*>(x + t * ldx + 4 * i);
  __syncthreads();

  for (int e = wave; e < n_experts; e += 4) {
    const float* row = wr + (int64_t)e * k;
    float acc = 0.f;
    for (int i = lane; i < k / 4; i += 64) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(row + 4 * i);
      const f32x4 b = reinterpret_cast<const f32x4*>(s_x)[i];
      acc = fmaf(a.x, b.x, acc);
      acc = fmaf(a.y, b.y, acc);
      acc = fmaf(a.z, b.z, acc);
      acc = fmaf(a.w, b.w, acc);
    }
    const float l = wave_sum(acc);
    if (lane == 0) {
      s_l[e] = l;
      if (logits_out != nullptr) logits_out[(int64_t)t * n_experts + e] = l;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // top_k picks; lane l owns experts l, l + 64, ...
  uint32_t taken = 0;  // bit q: expert l + 64 q is taken
  for (int j = 0; j < top_k; ++j) {
    float bv = 0.f;
    int bi = -1;
    for (int q = 0, e = lane; e < n_experts; ++q, e += 64) {
      const float v = s_l[e];
      if (!((taken >> q) & 1u) && router_better(v, e, bv, bi)) {
        bv = v;
        bi = e;
      }
    }
    // 64-lane argmax (butterfly: every lane ends with the winner)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (router_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi >= 0 && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      s_pv[j] = bv;
      s_pi[j] = bi;
    }
  }
  if (lane == 0) {  // the wave's own LDS writes are visible to it in order
    const float m = s_pv[0];
    float sum = 0.f;
    for (int j = 0; j < top_k; ++j) sum += expf(s_pv[j] - m);
    for (int j = 0; j < top_k; ++j) {
      ids[t * top_k + j] = s_pi[j];
      w[t * top_k + j] = expf(s_pv[j] - m) / sum;
    }
  }
}

hipError_t launch_router_topk(const float* x, int64_t ldx, int n_tok, int k, const float* wr, int n_experts,
                              int top_k, int32_t* ids, float* w, float* logits, hipStream_t st) {
  hipLaunchKernelGGL(k_router_topk, dim3((unsigned)n_tok), dim3(256), (size_t)k * 4, st, x, ldx, k, wr,
                     n_experts, top_k, ids, w, logits);
  return hipGetLastError();
}

}  // namespace qmv
