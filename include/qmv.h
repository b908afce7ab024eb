/*
 * qmv.h -- C ABI of the MI355X (gfx950) quantized decode matvec library.
 *
 * The library computes the decode hot path of llama.cpp-derived engines:
 * small-batch matrix-vector products over block-quantized GGUF weights
 * (Q8_0, q4_K, IQ4_XS) for 1..16 decode or speculative-verify tokens, and the
 * expert-grouped MoE variant for up to 64 tokens (Castagna Veloce page,
 * "Kernels for the MI50": i-quant MoE decode kernels for batches of up to 64
 * tokens, and small-batch matvecs for K-quants, iq4_xs and Q8_0 with a split-K
 * variant for 1 to 16 tokens).  Activations are quantized once to Q8 blocks
 * and the same buffer is reused by every weight type and matrix (same page,
 * "Fused operations": Q8 activations reused across weight types).  Weights are
 * consumed in their compressed block form, never expanded (zhuai.tech GLM-5.3
 * page, "Keep quantized weights compressed in memory").
 *
 * Conventions for every entry point
 *   - W is n_rows x k (n_rows outputs, k the reduction length), rows stored
 *     back to back in the GGUF block layout of its type, no padding:
 *       Q8_0   : 34 B per 32 weights   (fp16 d, int8 q[32]),  w = d * q
 *       q4_K   : 144 B per 256 weights (fp16 d, fp16 dmin, 12 B of packed
 *                6-bit scale/min pairs, 128 B of nibbles),
 *                w = d * sc_j * q - dmin * m_j for sub-block j of 32
 *       IQ4_XS : 136 B per 256 weights (fp16 d, u16 scales_h, u8
 *                scales_l[4], 128 B of 4-bit codebook indices),
 *                w = d * (ls_j - 32) * CB[idx]
 *       q5_K   : 176 B per 256 weights (the q4_K header, 32 B qh, 128 B of
 *                nibbles in the q4_K order; the fifth bit of weight 64c + i
 *                is bit 2c of qh[i], of weight 64c + 32 + i bit 2c + 1),
 *                w = d * sc_j * q - dmin * m_j with q in 0..31
 *                (another K-quant of the small-batch matvecs: Castagna
 *                Veloce page, "Kernels for the MI50"; qmv_matvec,
 *                qmv_matvec_batch and qmv_block_dots take it,
 *                qmv_moe_matvec does not)
 *       q6_K   : 210 B per 256 weights (128 B ql, 64 B qh, int8 scales[16],
 *                fp16 d); weight 128h + 32j + l (half h, quarter j, l < 32)
 *                stores q = nibble of ql[64h + 32(j & 1) + l] (low for j < 2)
 *                + 16 * bits 2j..2j+1 of qh[32h + l], and
 *                w = d * scales[(128h + 32j + l) / 16] * (q - 32)
 *                (same page and entry points as q5_K; blocks are 210 B, so
 *                rows need not be 4-byte aligned: only the base pointer is)
 *       Q8G128 : 130 B per 128 weights (fp16 d, int8 q[128]), w = d * q: the
 *                int8 LM-head format named on the zhuai.tech GLM-5.3 page
 *                ("LM Head uses Q8G128", read as Q8_0 with groups of 128);
 *                k a multiple of 128; same entry points as q5_K
 *   - All pointers except those documented as host pointers are DEVICE
 *     pointers on the current HIP device.  The caller owns every buffer; the
 *     library allocates nothing and keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream).  Every call only enqueues work on that stream and returns; it
 *     never synchronizes.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns an error status and touches no memory.  A failed
 *     launch returns QMV_ERR_HIP.  Device faults surface at the caller's next
 *     synchronization.  No C++ exception crosses this interface.
 *   - Calls on one stream are ordered; calls that share a workspace must not
 *     run concurrently on different streams.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMV_ABI_VERSION 1

typedef enum {
  QMV_Q8_0 = 0,
  QMV_Q4_K = 1,
  QMV_IQ4_XS = 2,
  QMV_Q5_K = 3,
  QMV_Q6_K = 4,
  QMV_Q8G128 = 5
} qmv_type;

typedef enum {
  QMV_OK = 0,
  QMV_ERR_INVALID_ARG = 1, /* null pointer, bad size or stride, bad type  */
  QMV_ERR_UNSUPPORTED = 2, /* valid but outside the supported token range */
  QMV_ERR_MISALIGNED = 3,  /* a pointer breaks its documented alignment   */
  QMV_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required  */
  QMV_ERR_HIP = 5          /* the HIP runtime reported an error           */
} qmv_status;

/* Limits of the decode path. */
#define QMV_MAX_TOKENS 16       /* qmv_matvec: verify batches of 1..16     */
#define QMV_MAX_MOE_TOKENS 64   /* qmv_moe_matvec: batches of 1..64 tokens */
#define QMV_MAX_TOP_K 16
#define QMV_MAX_EXPERTS 1024
#define QMV_MAX_MOE_ROWS 65536  /* qmv_moe_matvec rows per expert           */
#define QMV_MAX_MOE_K 16384     /* qmv_moe_matvec reduction length         */
#define QMV_MAX_ACT_ROWS 65536  /* qmv_quantize_act rows per call          */

int qmv_abi_version(void);
/* The hipError_t code (as an int; 0 if none) of the last HIP runtime error
 * that an entry point called on this thread reported as QMV_ERR_HIP, and
 * its name (hipGetErrorName; static storage, never NULL). */
int qmv_last_hip_error(void);
const char* qmv_last_hip_error_name(void);
const char* qmv_status_string(qmv_status status);

/* Host-only size helpers: return 0 for invalid arguments. */
size_t qmv_row_bytes(qmv_type type, int64_t k);

/*
 * Q8 activation buffer for n_tok rows of length k (k % 32 == 0), structure of
 * arrays, each array 256-byte aligned relative to the buffer start:
 *   offset 0                 : qs int8  [n_tok][k]      quantized values
 *   qmv_act_offset_d(...)    : d  fp32  [n_tok][k/32]   block scales
 *   qmv_act_offset_s(...)    : s  int32 [n_tok][k/32]   block sums of qs
 * qmv_act_bytes() is the total size.  The buffer must be 256-byte aligned.
 */
size_t qmv_act_bytes(int64_t n_tok, int64_t k);
size_t qmv_act_offset_d(int64_t n_tok, int64_t k);
size_t qmv_act_offset_s(int64_t n_tok, int64_t k);

/*
 * qmv_quantize_act -- quantize activations to Q8 blocks of 32.
 * Castagna Veloce page, "Fused operations" (Q8 activations made once and
 * reused across weight types).  Per block of 32 values of a row:
 *   amax = max |x|,  d = amax / 127 (fp32, correctly rounded),
 *   q = x / d (fp32, correctly rounded) rounded half away from zero,
 *       clamped to [-127, 127],   s = sum of q;
 *   an all-zero block gives d = 0, q = 0, s = 0.
 * x   : fp32 [n_tok][ldx] (device), 16-byte aligned, ldx >= k, ldx % 4 == 0
 *       (else QMV_ERR_MISALIGNED: rows are read with 16-byte loads), finite
 *       values.
 * xq  : activation buffer of qmv_act_bytes(n_tok, k) bytes (device, 256-byte
 *       aligned); fully overwritten.
 * 1 <= n_tok <= QMV_MAX_ACT_ROWS, k > 0, k % 32 == 0.
 */
qmv_status qmv_quantize_act(const float* x, int64_t ldx, int64_t n_tok, int64_t k, void* xq,
                            void* stream);

/*
 * qmv_swiglu_quantize -- the step between a MoE gate+up and down projection:
 * SwiGLU of each row, quantized to Q8 blocks for the down projection.
 * Castagna Veloce page, "Fused operations" (gate/up + SwiGLU kernels for the
 * verify batches; Q8 activations made once).  For row r:
 *   g = gu[r][0 .. n_ff-1], u = gu[r][n_ff .. 2 n_ff - 1]  (gate rows first
 *   in a gate+up tensor, as qmv_moe_matvec produces them per slot),
 *   h = g / (1 + exp(-g)) * u  in fp32,
 * then the Q8 blocks of h exactly as qmv_quantize_act makes them.
 * gu    : fp32 [rows][ldg] (device), 16-byte aligned, ldg >= 2 n_ff,
 *         ldg % 4 == 0 (else QMV_ERR_MISALIGNED: 16-byte loads), finite.
 * xq    : activation buffer of qmv_act_bytes(rows, n_ff) bytes (device,
 *         256-byte aligned); fully overwritten.
 * h_out : NULL, or fp32 [rows][n_ff] (device, 16-byte aligned) that receives
 *         the h values the blocks were made from.
 * 1 <= rows <= QMV_MAX_ACT_ROWS, n_ff > 0, n_ff % 32 == 0.
 * Asynchronous on `stream`; allocates nothing.
 */
qmv_status qmv_swiglu_quantize(const float* gu, int64_t ldg, int64_t rows, int64_t n_ff, void* xq,
                               float* h_out, void* stream);

/*
 * qmv_router_topk -- MoE router and top-k: the routing ids and weights that
 * qmv_moe_matvec takes.  Castagna Veloce page, "Fused operations" (router
 * matvec, gating, top-k and weight normalization fused for decode).  For
 * token t:
 *   l[e] = sum_i wr[e][i] x[t][i]            (fp32 sums),
 *   ids[t][0..top_k-1] = the top_k experts by l, a larger logit first and on
 *                        equal logits the lower expert index first,
 *   weights[t][j] = exp(l[ids[t][j]] - l[ids[t][0]]) / sum over the chosen
 *                   (a softmax over the chosen logits).
 * x       : fp32 [n_tok][ldx] (device), 16-byte aligned, ldx >= k, ldx % 4 == 0.
 * wr      : fp32 router weights [n_experts][k] (device), 16-byte aligned.
 * ids     : int32 [n_tok][top_k] (device); weights: fp32 [n_tok][top_k].
 * logits  : fp32 [n_tok][n_experts] (device), receives l (the selection
 *           reads it back: two launches on `stream`).
 * xq      : NULL, or an activation buffer of qmv_act_bytes(n_tok, k) bytes
 *           (device, 256-byte aligned) that receives Q8(x) exactly as
 *           qmv_quantize_act makes it (the router reads all of x anyway; the
 *           routed gate+up projection takes this buffer, which saves the
 *           quantizer's launch).  Requires k % 32 == 0.
 * 1 <= n_tok <= QMV_MAX_MOE_TOKENS, k % 4 == 0, k <= 2^24,
 * 1 <= top_k <= min(n_experts, QMV_MAX_TOP_K), n_experts <= QMV_MAX_EXPERTS.
 * Asynchronous on `stream`; allocates nothing.
 */
qmv_status qmv_router_topk(const float* x, int64_t ldx, int64_t n_tok, int64_t k, const float* wr,
                           int64_t n_experts, int64_t top_k, int32_t* ids, float* weights, float* logits,
                           void* xq, void* stream);

/*
 * qmv_matvec -- y[t][n] = sum_k W[n][k] * xq[t][k] for t < n_tok.
 * Castagna Veloce page, "Kernels for the MI50" (small-batch matvecs for 1 to
 * 16 tokens, Q8_0 with a split-K variant); zhuai.tech GLM-5.3 page, "A single
 * decode row is not a large matrix multiplication".
 * Per 32-weight block the weights and activations meet in an exact integer
 * dot product; the fp16 weight scales and fp32 activation scales are applied
 * to that integer in fp32 and accumulated in fp32 (any order).
 * w    : n_rows x k weights of `type` (device, 16-byte aligned).
 * xq   : activation buffer made by qmv_quantize_act for (n_tok, k) (device).
 * y    : fp32 [n_tok][ldy] (device, 4-byte aligned), ldy >= n_rows; columns
 *        0..n_rows-1 of each row are overwritten, the rest are untouched.
 * ws   : optional workspace (device, 256-byte aligned) enabling the split-K
 *        paths for few-row long-K shapes (K split over the workgroups of
 *        one launch); NULL runs the single-pass kernel.  A split call sums
 *        in another order than the single-pass kernel, so its fp32 result
 *        may differ from that one's in rounding (both within the stated
 *        tolerance); it is the same on every call with the same arguments.
 *        It must hold qmv_matvec_workspace_bytes(type, n_rows, k, n_tok)
 *        bytes, be zero-filled once when allocated, and is left in that state
 *        by every completed call (its counters reset themselves).  One
 *        workspace may serve calls of different shapes, each needing no more
 *        than its size, as long as those calls do not overlap in time.
 * 1 <= n_tok <= QMV_MAX_TOKENS (else QMV_ERR_UNSUPPORTED); n_rows >= 1;
 * k a positive multiple of 32 (Q8_0), 128 (Q8G128) or 256 (the others).
 */
size_t qmv_matvec_workspace_bytes(qmv_type type, int64_t n_rows, int64_t k, int64_t n_tok);
qmv_status qmv_matvec(qmv_type type, const void* w, int64_t n_rows, int64_t k, const void* xq,
                      int64_t n_tok, float* y, int64_t ldy, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * qmv_matvec_x -- the decode step of one matrix from fp32 activations:
 *   xq = Q8(x) exactly as qmv_quantize_act makes it, then
 *   y[t][n] = sum_k W[n][k] * xq[t][k]  exactly as qmv_matvec computes it.
 * Castagna Veloce page, "Fused operations" (Q8 activations; fused kernels for
 * the verify batches) and zhuai.tech GLM-5.3 page, "A faster kernel can
 * still leave the full chain slower" (fewer launches and handoffs).  Where
 * that measured faster (Q8_0 rows of up to 4096 weights at one or two
 * tokens, q4_K ones at one token) the matvec workgroups quantize x
 * themselves, in the one launch, and one of them writes xq; otherwise the
 * call runs the quantizer and then the matvec (two launches, same results).
 * x    : fp32 [n_tok][ldx] (device), 16-byte aligned, ldx >= k, ldx % 4 == 0,
 *        finite values.
 * xq   : activation buffer of qmv_act_bytes(n_tok, k) bytes (device, 256-byte
 *        aligned); receives Q8(x) for reuse by later calls (another matrix
 *        over the same activations).
 * w, n_rows, k, n_tok, y, ldy, ws, ws_bytes: as for qmv_matvec (the
 *        workspace, optional, serves the two-launch path's matvec; every
 *        argument, the workspace's included, is validated before anything
 *        is enqueued).
 * Asynchronous on `stream`; allocates nothing.
 */
qmv_status qmv_matvec_x(qmv_type type, const void* w, int64_t n_rows, int64_t k, const float* x,
                        int64_t ldx, int64_t n_tok, float* y, int64_t ldy, void* xq, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * qmv_matvec_batch -- sibling matvecs over one activation buffer in one
 * launch, each optionally plus a residual:
 *   y_i[t][n] = sum_k W_i[n][k] * xq[t][k]  (+ residual_i[t][n])
 * for every item i and t < n_tok.  Castagna Veloce page, "Fused operations"
 * (batched sibling matvecs and Q8 activations reused across weight types;
 * matvec + residual add kernels for the verify batches).  Every item has the
 * same weight type and reduction length k; each item's arithmetic is that of
 * qmv_matvec, and the residual is added to the fp32 sum once, at the end.
 * items  : HOST array of n_items descriptors, read during the call only:
 *   w        n_rows x k weights of `type` (device, 16-byte aligned);
 *   n_rows   >= 1;
 *   y        fp32 [n_tok][ldy] (device, 4-byte aligned), ldy >= n_rows;
 *            columns 0..n_rows-1 of each row are overwritten;
 *   residual NULL, or fp32 [n_tok][ldr] (device, 4-byte aligned),
 *            ldr >= n_rows; it may be the item's own y with ldr == ldy
 *            (accumulate in place), otherwise it must not overlap any
 *            item's y.
 * The y extents of different items must not overlap.
 * xq     : activation buffer made by qmv_quantize_act for (n_tok, k).
 * 1 <= n_items <= QMV_MAX_BATCH and 1 <= n_tok <= QMV_MAX_TOKENS (else
 * QMV_ERR_UNSUPPORTED); k as for qmv_matvec; overlapping outputs or a bad
 * descriptor give QMV_ERR_INVALID_ARG.  No workspace, no split-K across
 * workgroups.  Asynchronous on `stream`; allocates nothing.
 */
#define QMV_MAX_BATCH 8
typedef struct {
  const void* w;
  int64_t n_rows;
  float* y;
  int64_t ldy;
  const float* residual;
  int64_t ldr;
} qmv_matvec_item;
qmv_status qmv_matvec_batch(qmv_type type, const qmv_matvec_item* items, int64_t n_items, int64_t k,
                            const void* xq, int64_t n_tok, void* stream);

/*
 * qmv_moe_matvec -- expert-grouped routed matvec.
 * Castagna Veloce page, "Kernels for the MI50" (i-quant MoE decode kernels
 * for batches of up to 64 tokens; expert-grouped quantized MoE: each active
 * expert's weights are read once for all the tokens routed to it).
 * w        : n_experts matrices of n_rows x k, back to back (device,
 *            16-byte aligned).
 * xq       : activation buffer with n_tok rows (x_per_slot = 0, e.g. the
 *            gate/up input shared by a token's slots) or n_tok*top_k rows,
 *            row t*top_k + s for slot s of token t (x_per_slot = 1, e.g. the
 *            down-projection input of each slot).
 * ids      : int32 [n_tok][top_k] expert of each slot (device).  An id
 *            outside [0, n_experts) drops that slot: it contributes zero.
 * route_w  : NULL, or fp32 [n_tok][top_k] routing weights (device).
 * y        : route_w == NULL -> fp32 [n_tok][top_k][n_rows], one output row
 *            per slot (dropped slots get zeros);
 *            route_w != NULL -> fp32 [n_tok][n_rows],
 *            y[t] = sum over valid slots s of route_w[t][s] * (W[ids[t][s]] x),
 *            summed in slot order.
 * ws       : workspace of qmv_moe_workspace_bytes(...) bytes (device,
 *            256-byte aligned, zero-filled once when allocated; completed
 *            calls leave its counters at zero; calls of different shapes may
 *            share it if they do not overlap in time).  After a call, the
 *            int32 at offset 0 holds the number of dropped slots of that call.
 * 1 <= n_tok <= QMV_MAX_MOE_TOKENS, 1 <= top_k <= QMV_MAX_TOP_K,
 * 1 <= n_experts <= QMV_MAX_EXPERTS, n_rows <= QMV_MAX_MOE_ROWS and
 * k <= QMV_MAX_MOE_K (else QMV_ERR_UNSUPPORTED); k as for qmv_matvec; type
 * Q8_0, q4_K or IQ4_XS (q5_K, q6_K, Q8G128: QMV_ERR_UNSUPPORTED).
 */
size_t qmv_moe_workspace_bytes(qmv_type type, int64_t n_experts, int64_t n_rows, int64_t k,
                               int64_t n_tok, int64_t top_k);
qmv_status qmv_moe_matvec(qmv_type type, const void* w, int64_t n_experts, int64_t n_rows,
                          int64_t k, const void* xq, int x_per_slot, const int32_t* ids,
                          const float* route_w, int64_t n_tok, int64_t top_k, float* y,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * qmv_moe_gate_up_swiglu -- the MoE FFN's routed gate+up projection with
 * SwiGLU and the Q8 blocks of its output: the down projection's input from
 * one call.  Castagna Veloce page, "Fused operations" (gate/up + SwiGLU; Q8
 * activations made once).  Either path's result is bit-identical to
 *   qmv_moe_matvec(type, w, n_experts, 2 n_ff, k, xq, 0, ids, NULL, ...)
 *   -> gu [n_tok][top_k][2 n_ff], then
 *   qmv_swiglu_quantize(gu, 2 n_ff, n_tok * top_k, n_ff, hq, NULL, ...).
 * w    : n_experts gate+up matrices of 2 n_ff rows (gate rows 0 .. n_ff - 1,
 *        up rows n_ff .. 2 n_ff - 1) by k, back to back (device, 16-byte
 *        aligned); xq: one activation row per token (qmv_quantize_act).
 * hq   : activation buffer of qmv_act_bytes(n_tok * top_k, n_ff) bytes
 *        (device, 256-byte aligned); row t * top_k + s receives Q8(h) of
 *        slot s of token t, h = silu(gate) * up; dropped slots give zeros.
 * gu   : NULL, or fp32 [n_tok][top_k][2 n_ff] (device, 16-byte aligned)
 *        that receives the gate+up outputs.
 * ws   : the workspace of the routed gate+up call
 *        (qmv_moe_workspace_bytes(type, n_experts, 2 n_ff, k, n_tok, top_k)).
 * By default two launches: the routed matvec and qmv_swiglu_quantize (gu,
 * or without it the workspace's per-slot area, carries the gate+up
 * outputs), which measured faster than one.  qmv_set_tuning("ffn_fuse", 1)
 * selects one launch up to 16 tokens on rows of at most 4096 weights (with
 * the automatic or few-slot MoE kernel, see "moe_kernel"): a
 * few-slot kernel whose workgroup holds 32 gate rows and the matching 32 up
 * rows and makes that block of h from them in LDS.
 * n_ff % 32 == 0; other limits and errors as for qmv_moe_matvec.
 */
qmv_status qmv_moe_gate_up_swiglu(qmv_type type, const void* w, int64_t n_experts, int64_t n_ff, int64_t k,
                                  const void* xq, const int32_t* ids, int64_t n_tok, int64_t top_k, void* hq,
                                  float* gu, void* ws, size_t ws_bytes, void* stream);

/*
 * qmv_moe_matvec_noalloc -- qmv_moe_matvec for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc): the same validation, kernels and results, with
 * the workspace taken from a device-resident array inside the library
 * instead of a caller buffer.  It allocates nothing and calls no allocating
 * routine.
 *   - The array holds QMV_MOE_NOALLOC_WS_BYTES bytes; a call whose
 *     qmv_moe_workspace_bytes(...) exceeds that returns QMV_ERR_WORKSPACE
 *     (e.g. 128 experts, top-8, 4096 rows: fits up to 64 tokens).
 *   - Each GPU the library runs on holds its own copy until the process
 *     ends; its address is looked up on the first call on that GPU.
 *   - Every call on a GPU shares that GPU's copy and leaves it holding the
 *     call's per-slot outputs: calls that overlap in time on one GPU (on
 *     different streams) race and must not be issued.
 *   - The dropped-slot count is not reported (it stays in the array).
 * All other arguments as for qmv_moe_matvec.
 */
#define QMV_MOE_NOALLOC_WS_BYTES ((size_t)17 << 20)
qmv_status qmv_moe_matvec_noalloc(qmv_type type, const void* w, int64_t n_experts, int64_t n_rows,
                                  int64_t k, const void* xq, int x_per_slot, const int32_t* ids,
                                  const float* route_w, int64_t n_tok, int64_t top_k, float* y,
                                  void* stream);

/*
 * qmv_block_dots -- test hook: the exact integer partial of every 32-weight
 * block, computed by the same device decode and dot routines as qmv_matvec.
 * out : int32 [n_tok][n_rows][k/32][c] (device), c = 2 for q4_K and q5_K
 *       (A = sc_j * sum q*qx, B = m_j * s_b) and c = 1 otherwise
 *       (q6_K: sum over the block of scales[i/16] * (q_i - 32) * qx_i)
 *       (Q8_0: sum qw*qx; IQ4_XS: (ls_j - 32) * sum CB[idx]*qx).
 * 1 <= n_tok <= QMV_MAX_TOKENS.
 */
qmv_status qmv_block_dots(qmv_type type, const void* w, int64_t n_rows, int64_t k,
                          const void* xq, int64_t n_tok, int32_t* out, void* stream);

/*
 * qmv_block_dots_mx -- test hook: the same exact block integers as
 * qmv_block_dots, computed by the matrix-core kernel of qmv_matvec (its
 * activation staging, weight loads and decode, and the int8 matrix-core
 * products whose zero-masked activation rows keep every 32-block apart),
 * which writes each product's integer times the block's integer weight
 * scale (and, for q4_K, m_j * s_b) instead of applying the fp32 scales.
 * Castagna Veloce page, "Philosophy" (exact changes verified bit-identical
 * against a CPU reference).
 * variant : -1, the matrix-core variant qmv_matvec runs for this shape with
 *           a workspace (else mx_w16_k4_r2 up to 8 tokens, mx_w8_k1_r4
 *           beyond); or the index of a matrix-core variant (qmv_variant_name
 *           "mx_...").
 * slices  : 0 one pass over K; -1 the K split over workgroups qmv_matvec
 *           would make with a workspace (none if it would not split);
 *           2..32 that many K slices (QMV_ERR_UNSUPPORTED if they do not fit).
 * out     : int32 [n_tok][n_rows][k/32][c] as for qmv_block_dots (device).
 * Types Q8_0, q4_K, IQ4_XS and Q8G128 (others: QMV_ERR_UNSUPPORTED);
 * 1 <= n_tok <= QMV_MAX_TOKENS.  No workspace; nothing else is written.
 */
qmv_status qmv_block_dots_mx(qmv_type type, const void* w, int64_t n_rows, int64_t k, const void* xq,
                             int64_t n_tok, int64_t variant, int slices, int32_t* out, void* stream);

/*
 * qmv_moe_block_dots -- test hook: the exact block integers of every routed
 * slot, computed by the matrix-core expert-grouped kernel of qmv_moe_matvec
 * (its routing sort, slot-row staging, weight loads, decode and int8
 * matrix-core products) in place of its fp32 outputs.  Castagna Veloce page,
 * "Kernels for the MI50" (expert-grouped MoE) and "Philosophy".
 * Arguments as for qmv_moe_matvec (no route weights); slot_rows is the number
 * of slot rows staged per group: 4 or 8, or 0 for the automatic choice (4 up
 * to 16 tokens, 8 beyond).
 * out : int32 [n_tok * top_k][n_rows][k/32][c] (device), c = 2 for q4_K
 *       else 1: for slot t * top_k + s the integers of W[ids[t][s]] against
 *       that slot's activation row; the entries of dropped slots are not
 *       written.  QMV_ERR_UNSUPPORTED if the staged rows do not fit in LDS.
 */
qmv_status qmv_moe_block_dots(qmv_type type, const void* w, int64_t n_experts, int64_t n_rows, int64_t k,
                              const void* xq, int x_per_slot, const int32_t* ids, int64_t n_tok, int64_t top_k,
                              int64_t slot_rows, int32_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * qmv_stream_read -- measurement hook: reads the `bytes` bytes at p (device)
 * once with non-temporal 16-byte loads (256-lane workgroups, four loads per
 * lane in flight, lanes on adjacent pieces: the fastest plain read measured
 * on MI355X), and computes nothing from them: the practical ceiling of a
 * kernel streaming the same bytes.  Decode kernels are measured by weight
 * bytes over kernel time (zhuai.tech GLM-5.3 page, "A faster kernel can
 * still leave the full chain slower", its bandwidth breakdown); this gives
 * the same figure for a kernel with no decode at all.
 * sink : one uint32 (device); written only if the fold of the bytes hits a
 *        fixed 32-bit value, so in practice never.
 * bytes a positive multiple of 16 (else QMV_ERR_INVALID_ARG); p 16-byte and
 * sink 4-byte aligned (else QMV_ERR_MISALIGNED).
 */
qmv_status qmv_stream_read(const void* p, int64_t bytes, uint32_t* sink, void* stream);

/*
 * qmv_set_tuning -- process-wide A/B switches (Castagna Veloce page, "New
 * features": each optimization can be switched off for A/B tests).  Keys:
 *   "splitk"  : -1 automatic (default), 0 never, n >= 1 force n K-slices
 *               whenever a workspace is given;
 *   "variant" : -1 automatic (default), else an index into the kernel
 *               variant table of qmv_matvec (see qmv_variant_name); a
 *               variant whose LDS staging does not fit the device runs the
 *               lane-group kernel instead (qmv_pick_variant reports which);
 *   "mx_slices": -1 automatic (default), 0 never, 2..32 force that many
 *               K slices for the matrix-core kernel's split over
 *               workgroups (it needs a workspace; automatic splits only
 *               rows too long for one LDS chunk on too few row tiles to
 *               fill the device);
 *   "flat_split": 0 (default) or 1: let the LDS-staged flat kernel split K
 *               over workgroups (with a workspace) where its workgroups would
 *               not fill the device or a row needs several chunks;
 *   "bpc"     : 0 automatic (default), else a cap on resident workgroups
 *               per compute unit for the persistent streaming kernel;
 *   "moe_kernel": 0 automatic (default), 1 the vector-ALU expert-grouped
 *               kernel, 2 the matrix-core one (which falls back to the
 *               vector-ALU kernel when its staged rows do not fit in LDS),
 *               3 the few-slot flat kernel (each slot's expert rows
 *               streamed without grouping slots by expert);
 *   "moe_row16": 0 (default) the few-slot MoE kernels hold short rows in
 *               16-lane groups (one activation row per slot and rows of
 *               fewer than 64 blocks; one route-weighted token with
 *               top_k <= 8 and rows of at most 64), 1 one row or more per
 *               wave throughout;
 *   "ffn_fuse": -1 automatic (default: two launches), 0 two launches, 1
 *               one launch where it applies, for qmv_moe_gate_up_swiglu.
 * The environment variables QMV_SPLITK, QMV_VARIANT and QMV_MOE_KERNEL set
 * the same switches when the library loads.  Returns QMV_ERR_INVALID_ARG for an unknown key or
 * value.
 */
qmv_status qmv_set_tuning(const char* key, int64_t value);
/* Name of kernel variant `index`, or NULL past the end of the table. */
const char* qmv_variant_name(int64_t index);
/* The variant qmv_matvec would run for these arguments without a workspace
 * (-1 if invalid). */
int64_t qmv_pick_variant(qmv_type type, int64_t n_rows, int64_t k, int64_t n_tok);
/* What qmv_matvec would run with (with_workspace != 0) or without a
 * workspace of qmv_matvec_workspace_bytes bytes: *variant the kernel variant,
 * *slices the K slices split over workgroups (1: no split).  Host only. */
qmv_status qmv_matvec_plan(qmv_type type, int64_t n_rows, int64_t k, int64_t n_tok, int with_workspace,
                           int64_t* variant, int* slices);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
