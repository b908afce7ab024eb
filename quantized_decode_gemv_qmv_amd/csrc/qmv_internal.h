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
//           32-block, activations staged in LDS chunk by chunk;
//   kind 5: flat matrix-core kernel (k_mxf) -- the same tile in one pass
//           over the rows: wpb waves per workgroup, each holding `nu`
//           super-blocks of one row tile's K slice, all loaded at once
//           (waves per tile and K slices planned per launch);
//   kind 6: long-row kernel (k_long) -- one workgroup of wpb waves per group
//           of `rows` rows, its waves splitting K in chunks of `nu` units per
//           lane, activation fragments loaded from global memory.
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
// The matrix-core kinds (integer MFMA tiles).
inline bool is_mx(const Variant& v) { return v.kind == 4 || v.kind == 5; }
extern const int kNumVariants;

// The matrix a launch row belongs to: its weights, output and residual, its
// first launch row and its row count.
struct RowSeg {
  const uint8_t* w;
  float* y;
  const float* res;  // NULL, or fp32 [n_tok][ldr] added to the outputs
  int64_t ldy, ldr;
  int first, rows;
};

// Matrices of one batched launch (sibling matvecs sharing an activation
// buffer): stacked along the launch's rows, matrix i taking launch rows
// s[i].first .. s[i].first + s[i].rows - 1.  Every first row is a multiple of
// kSegAlign, which every kernel's per-wave (and per-workgroup reduction) row
// span divides, so a wave never straddles two matrices; launch rows between
// one matrix's end and the next one's start only re-read valid rows and
// store nothing.
constexpr int kMaxBatch = 8;
constexpr int kSegAlign = 64;
struct Segs {
  int n;  // 0: a single matrix, described by the w / y / res fields around
  RowSeg s[kMaxBatch];
};

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
  const float* res;  // NULL, or fp32 [n_tok][ldr] added to the outputs
  int64_t ldr;
  Segs seg;
  // flat kernel quantizing its own activations: fp32 x [n_tok][ldx], and the
  // Q8 buffer that workgroup 0 also writes out (the layout of xq)
  const float* x;
  int64_t ldx;
  uint8_t* xq_out;
  // k_mx split over workgroups along K (gridDim.y slices of ups units):
  // partial sums [slices][n_tok][n_rows] and one arrival counter per
  // workgroup column, in the caller's workspace
  int ups;
  float* part;
  int* cnt;
  // k_mxf: waves per row tile
  int mx_ks;
  // integer mode of k_mx (the block-dot test hook): the exact integer of
  // every (token, row, 32-block) goes to dots, int32 [n_tok][n_rows][units][c]
  // (c = 2 for q4_K: sc * sum q qx, m * s; else 1), and no output is stored
  int32_t* dots;
};

#ifdef __HIPCC__
// Segment of launch row `row`, a wave-uniform value.  SEG false (a launch of
// one matrix, never with a residual) compiles to the single-matrix fields
// and a constant null residual; kernels take SEG as a
// template flag so that single-matrix launches carry no table code.  With
// SEG, the index is counted from the first rows and the one entry is then
// read from the kernel arguments.
template <bool SEG>
__device__ inline RowSeg row_seg(const StreamArgs& a, int row) {
  if constexpr (!SEG) return RowSeg{a.w, a.y, nullptr, a.ldy, 0, 0, a.n_rows};  // no residual either
  int i = 0;
#pragma unroll
  for (int j = 1; j < kMaxBatch; ++j) i += (j < a.seg.n && row >= a.seg.s[j].first) ? 1 : 0;
  return a.seg.s[i];
}
// Weight row of launch row `row` inside its segment (clamped to the last row).
__device__ inline const uint8_t* seg_wrow(const RowSeg& s, int64_t row_bytes, int row) {
  return s.w + (int64_t)min(row - s.first, s.rows - 1) * row_bytes;
}
// Output (t, launch row `row`) = v plus the residual, if the row is one of
// the segment's rows.
__device__ inline void seg_store(const RowSeg& s, int t, int row, float v) {
  const int lr = row - s.first;
  if (lr < s.rows) {
    if (s.res != nullptr) v += s.res[(int64_t)t * s.ldr + lr];
    s.y[(int64_t)t * s.ldy + lr] = v;
  }
}
#endif

// K slices of a cross-workgroup split at most (the split-K workspace holds
// the partial sums of this many).
constexpr int kMaxSlices = 32;

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
  const float* res;  // NULL, or fp32 [n_tok][ldr] added to y
  int64_t ldr;
  Segs seg;         // batched launch (seg.n > 0): the matrices; n_rows the launch rows
  // quantize-in-kernel launch (qx): fp32 x [n_tok][ldx] and the Q8 buffer
  // written beside it (xq then points at that buffer too)
  bool qx;
  const float* xf;
  int64_t ldx;
  int variant;  // index into kVariants
  const uint8_t* xq;  // the activation buffer and its layout
  int64_t act_bytes, off_d, off_s;
  int cus;            // compute units of the device
  int64_t lds_per_cu; // LDS bytes per compute unit
  // flat kernel split over workgroups (fslices > 1): slices of fups units
  int fslices, fups;
  // split-K (slices > 1): partial sums [slices][n_tok][n_rows] and one
  // arrival counter per row tile, both in the caller's workspace
  int slices;
  float* part;
  int* cnt;
  // integer mode (launch_mx only): the exact block integers to dots instead
  // of any output; dots_slices 0 unsplit, -1 the automatic split, n >= 2 n
  // K slices over workgroups (no workspace: nothing is reduced)
  int32_t* dots;
  int dots_slices;
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
int blocks_per_cu();
// Tuning: K slices of the matrix-core kernel's cross-workgroup split
// (-1 automatic, 0 never, n >= 2 that many, when a workspace is given).
void set_mx_slices(int v);
int mx_slices();
// Cross-workgroup K split of k_mx for format fmt, n_tok tokens and a
// variant of wpb waves in teams of ks: the slice count (>= 2, units per
// slice in *ups) or 0 for no split.
// forced: -1 automatic, 0 never, n >= 2 that many slices (the mx_slices
// tuning switch supplies it for qmv_matvec).
int mx_split_plan(int fmt, int n_tok, int wpb, int ks, int units, int n_rows, int cus, int64_t lds_per_cu,
                  int forced, int* ups);

hipError_t launch_quantize(const float* x, int64_t ldx, int n_tok, int k, int8_t* qs, float* d,
                           int32_t* s, hipStream_t st);
hipError_t launch_swiglu_quantize(const float* gu, int64_t ldg, int rows, int n_ff, int8_t* qs, float* d,
                                  int32_t* s, float* h_out, hipStream_t st);
hipError_t launch_router_topk(const float* x, int64_t ldx, int n_tok, int k, const float* wr, int n_experts,
                              int top_k, int32_t* ids, float* w, float* logits, int8_t* xq_qs, float* xq_d,
                              int32_t* xq_s, hipStream_t st);
hipError_t launch_matvec(const MatvecLaunch& a, hipStream_t st);
// The vector-ALU kernels of format F (one translation unit per format).
template <int F>
hipError_t launch_vector(const MatvecLaunch& a, hipStream_t st);
hipError_t launch_mx(const MatvecLaunch& a, hipStream_t st);

// Launch plan of the flat matrix-core kernel k_mxf: K slices over workgroups
// (1: none) of ups units each, ks waves per row tile, rt row tiles per
// workgroup, the grid's x size and the dynamic LDS bytes.
struct MxfPlan {
  int slices, ups, ks, rt, grid_x;
  size_t lds;
};
// The plan for a variant of wpb waves holding sbw super-blocks each: the
// fewest K slices whose activations fit one workgroup's LDS (several only if
// can_split; forced_slices > 0 demands that count).  Returns the slice count,
// 0 if no plan fits.
int mxf_plan(int fmt, int n_tok, int wpb, int sbw, int units, int n_rows, int cus, int64_t lds_per_cu,
             bool can_split, int forced_slices, MxfPlan* p);
hipError_t launch_mxf(const MatvecLaunch& a, const MxfPlan& p, hipStream_t st);
template <int F>
hipError_t launch_mxf_fmt(const MatvecLaunch& a, const MxfPlan& p, hipStream_t st);
// The matrix-core kernels of format F (one translation unit per format).
template <int F>
hipError_t launch_mx_fmt(const MatvecLaunch& a, hipStream_t st);
hipError_t launch_stream_read(const uint8_t* p, int64_t bytes, uint32_t key, uint32_t* sink, hipStream_t st);
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
  // the gate+up launch with SwiGLU + Q8 folded in: gate rows 0 .. n_ff-1
  // and up rows n_ff .. 2 n_ff-1; hq the Q8 buffer it writes, h_off_d and
  // h_off_s the byte offsets of its d and s (y: NULL, or the gate+up sums)
  int n_ff;
  uint8_t* hq;
  int64_t h_off_d, h_off_s;
  // integer mode of the matrix-core MoE kernel (the block-dot test hook):
  // the exact integers of every (slot, row, 32-block) of the slot's expert
  // go to dots, int32 [n_tok * top_k][n_rows][units][c], and nothing else
  // is written
  int32_t* dots;
};

hipError_t launch_moe(const MoeLaunch& a, hipStream_t st);
// The fused MoE gate+up + SwiGLU + Q8 kernel (one activation row per token,
// rows of at most 4096 weights; hipErrorInvalidValue otherwise).
hipError_t launch_moe_gate_up_swiglu(const MoeLaunch& a, hipStream_t st);
// The matrix-core MoE kernel with tm (4 or 8) staged slot rows per group, in
// integer mode (a.dots set).
hipError_t launch_moe_mx_dots(const MoeLaunch& a, int tm, hipStream_t st);
// Tuning: MoE kernel (0 automatic, 1 vector-ALU, 2 matrix-core).
void set_moe_kernel(int v);
// Tuning: the few-slot MoE kernels' 16-lane row groups on short rows (0, the
// default) or one row per wave throughout (1).
void set_moe_row16(int v);
int moe_kernel();

}  // namespace qmv
