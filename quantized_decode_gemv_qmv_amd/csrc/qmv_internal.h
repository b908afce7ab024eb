// qmv_internal.h -- host-side interface between the C ABI layer and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

// Pointers into a Q8 activation buffer (structure of arrays).
struct ActView {
  const int8_t* qs;
  const float* d;
  const int32_t* s;
  int k;
  int nb;  // k / 32
};

// A dense matvec kernel configuration: lanes per row group and rows per group.
struct Variant {
  int lpr;
  int rows;
  const char* name;
};

extern const Variant kVariants[];
extern const int kNumVariants;

struct MatvecLaunch {
  int fmt;
  const uint8_t* w;
  int64_t row_bytes;
  int n_rows;
  int units;  // k / 32
  ActView x;
  int n_tok;
  float* y;
  int64_t ldy;
  int variant;  // index into kVariants
  // split-K (slices > 1): partial sums [slices][n_tok][n_rows] and one
  // arrival counter per row tile, both in the caller's workspace
  int slices;
  float* part;
  int* cnt;
};

// Rows covered by one 256-thread workgroup of a variant.
inline int rows_per_wg(const Variant& v) { return 4 * (64 / v.lpr) * v.rows; }

hipError_t launch_quantize(const float* x, int64_t ldx, int n_tok, int k, int8_t* qs, float* d,
                           int32_t* s, hipStream_t st);
hipError_t launch_matvec(const MatvecLaunch& a, hipStream_t st);
hipError_t launch_block_dots(int fmt, const uint8_t* w, int64_t row_bytes, int n_rows, int units,
                             ActView x, int n_tok, int32_t* out, hipStream_t st);

struct MoeLaunch {
  int fmt;
  const uint8_t* w;
  int64_t row_bytes;
  int n_experts;
  int n_rows;
  int units;
  ActView x;
  int x_per_slot;
  const int32_t* ids;
  const float* rw;
  int n_tok;
  int top_k;
  float* y;
  // workspace
  int* err;     // dropped-slot count of the call
  int* cnt;     // one arrival counter per row tile (route-weighted combine)
  float* part;  // [n_tok * top_k][n_rows] per-slot outputs (combine only)
};

hipError_t launch_moe(const MoeLaunch& a, hipStream_t st);
int moe_rows_per_wg(int fmt, int units);

}  // namespace qmv
