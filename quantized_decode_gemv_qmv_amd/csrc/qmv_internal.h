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

// A dense matvec kernel configuration.
//   kind 0: lane-group kernel (k_matvec) -- a wave is split into 64/lpr groups
//           of lpr lanes; each group owns `rows` rows and walks units with
//           stride lpr; activations are read from global memory;
//   kind 1: streaming kernel (k_stream) -- workgroups of wpb waves, teams of
//           ks waves (1 or wpb) per group of `rows` rows, `nu` units per lane
//           per chunk, activations staged in LDS;
//   kind 2: flat kernel (k_flat) -- one wave per group of `rows` rows for the
//           whole grid at once, `nu` units per lane; activations prefetched
//           from global memory (xl 0, up to 4 tokens) or staged in LDS (xl 1);
//   kind 3: multi-token kernel (k_mt) -- lane groups of 16 lanes own `rows`
//           rows, one unit per lane per iteration, wpb waves per workgroup in
//           teams of ks waves that split K, activations staged in LDS chunk
//           by chunk;
//   kind 4: matrix-core kernel (k_mx) -- a wave owns 16 rows, wpb waves per
//           workgroup in teams of ks waves that split K, int8 MFMA per
//           32-block, activations staged in LDS chunk by chunk.
struct Variant {
  int kind;
  int lpr;
  int rows;
  int nu;
  int wpb;
  int ks;
  int xl;
  const char* name;
};

extern const Variant kVariants[];
extern const int kNumVariants;

// Kernel arguments of k_stream.
struct StreamArgs {
  const uint8_t* w;
  int64_t row_bytes;
  int n_rows;
  int units;
  const uint8_t* xq;  // activation buffer, copied whole into LDS
  int act_bytes;
  int off_d, off_s;   // byte offsets of d and s inside it
  int k, nb;
  int n_tok;
  float* y;
  int64_t ldy;
  int kc;  // k_mt: units per LDS chunk
};

// LDS bytes k_mt stages per chunk at most (two workgroups per compute unit).
constexpr int64_t kMultiLdsBudget = 80 * 1024;

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
  const uint8_t* xq;  // the activation buffer and its layout
  int64_t act_bytes, off_d, off_s;
  int cus;            // compute units of the device
  int64_t lds_per_cu; // LDS bytes per compute unit
  // split-K (slices > 1): partial sums [slices][n_tok][n_rows] and one
  // arrival counter per row tile, both in the caller's workspace
  int slices;
  float* part;
  int* cnt;
};

// Rows covered by one 256-thread workgroup of a variant.
inline int rows_per_wg(const Variant& v) { return 4 * (64 / v.lpr) * v.rows; }
// Rows covered by one wave.
inline int rows_per_wave(const Variant& v) { return (64 / v.lpr) * v.rows; }

// LDS bytes k_stream needs for an activation buffer of act_bytes bytes and
// a token capacity tm (the staged buffer plus the split-K reduction area).
size_t stream_lds_bytes(const Variant& v, int64_t act_bytes, int tm);
// Tuning: cap on k_stream workgroups per compute unit (0 = occupancy).
void set_blocks_per_cu(int v);

hipError_t launch_quantize(const float* x, int64_t ldx, int n_tok, int k, int8_t* qs, float* d,
                           int32_t* s, hipStream_t st);
hipError_t launch_swiglu_quantize(const float* gu, int64_t ldg, int rows, int n_ff, int8_t* qs, float* d,
                                  int32_t* s, float* h_out, hipStream_t st);
hipError_t launch_router_topk(const float* x, int64_t ldx, int n_tok, int k, const float* wr, int n_experts,
                              int top_k, int32_t* ids, float* w, float* logits, hipStream_t st);
hipError_t launch_matvec(const MatvecLaunch& a, hipStream_t st);
hipError_t launch_mx(const MatvecLaunch& a, hipStream_t st);
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
  int cus;  // compute units of the device (persistent grid size)
  int64_t lds_per_cu;
  int ts;      // slot rows staged in LDS at a time (set at launch)
  int x_rows;  // rows of the activation buffer
  // workspace
  int* err;     // dropped-slot count of the call
  float* part;  // [n_tok * top_k][n_rows] per-slot outputs (combine only)
};

hipError_t launch_moe(const MoeLaunch& a, hipStream_t st);
// Tuning: MoE kernel (0 automatic, 1 vector-ALU, 2 matrix-core).
void set_moe_kernel(int v);

}  // namespace qmv
