// qmv_measure.hip -- the plain streaming read behind qmv_stream_read: the
// practical ceiling against which the matvec kernels' weight streams are
// judged (the zhuai.tech GLM-5.3 page, "A faster kernel can still leave the
// full chain slower", measures decode kernels by weight bytes over kernel
// time in its bandwidth breakdown).
#include "qmv_device.h"
#include "qmv_internal.h"

namespace qmv {

// Each 256-lane workgroup reads kReadLoads * 4 KiB: every lane issues its
// kReadLoads 16-byte loads before using any (lanes of a wave on adjacent
// 16-byte pieces), then folds them into one dword.  The loads are
// non-temporal: of the shapes measured on MI355X (two to sixteen loads per
// lane, one pass or grid-stride, plain or non-temporal) this one is the
// fastest or within 3% of it from 17.8 MB to 827 MB; on 827 MB it reads at
// 6.85 TB/s against 6.23 TB/s with plain loads.  The dword is stored only when it equals `key`
// (the caller passes a value that does not occur in practice), so the loads
// cannot be dropped and the kernel writes nothing in the common case.
constexpr int kReadLoads = 4;

__global__ __launch_bounds__(256) void k_stream_read(const uint8_t* __restrict__ p, int64_t n16,
                                                     uint32_t key, uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * (256 * kReadLoads) + threadIdx.x;
  u32x4 v[kReadLoads];
#pragma unroll
  for (int i = 0; i < kReadLoads; ++i) {
    const int64_t idx = base + 256 * i;
    v[i] = idx < n16 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + idx)
                     : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kReadLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (acc == key) sink[0] = acc;
}

hipError_t launch_stream_read(const uint8_t* p, int64_t bytes, uint32_t key, uint32_t* sink, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  const int64_t grid = (n16 + 256 * kReadLoads - 1) / (256 * kReadLoads);
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, st, p, n16, key, sink);
  return hipGetLastError();
}

}  // namespace qmv
