// qmv_mfma.hip -- matrix-core matvec for verify batches (several tokens) on
// gfx950.
//
// With a few tokens the vector-ALU kernels spend most of their issue slots on
// the int8 dot products (eight v_dot4 per row, token and 32-block).  Here the
// dots run on the matrix cores instead: one v_mfma_i32_16x16x64_i8 multiplies
// 16 weight rows by a 64-wide slice of K for 16 "activation rows".  Its
// result must stay per 32-block, because every 32-block carries its own
// weight and activation scale (Castagna Veloce page, "Kernels for the MI50":
// block-quantized dots; the tolerance and exact integer partials are per
// block).  So each activation row m of the MFMA stands for one (block, token)
// pair and holds that token's activations only in the K slots that carry the
// block's weights, zeros elsewhere: D[m][n] is then exactly the integer dot of
// block(m) of row n with token(m).
//
// Operand layout (measured on gfx950: lane l supplies A row l%16 and B column
// l%16 for its 16 K slots of group s = l/16; it receives D[4s + r][l%16],
// r = 0..3).  B = weights: lane (n, s) holds 16 decoded int8 weights of row n.
// A = activations, staged in LDS.  The slot-to-weight assignment only has to
// agree between A and B, so each format keeps the bytes of one 16-byte load:
//
//   q4_K (2 blocks per MFMA, m = 8j + t, 8 tokens per group): lane s holds
//     16 weights of one sub-block, weights 16(s%2)..+15, and the two lanes
//     s = 2j, 2j+1 together hold block j of the MFMA.  Lane s loads bytes
//     16(s%2)..+15 of nibble pair 2p + s/2 of span p (sub-blocks 4p + 2(s/2)
//     and its neighbour); the low-nibble MFMA then holds sub-blocks 4p and
//     4p+2, the high-nibble one 4p+1 and 4p+3.
//   IQ4_XS, Q8_0 (4 blocks per MFMA, m = 4j + t, 4 tokens per group): lane s
//     loads 32-block 4p+s of span p (IQ4_XS: its 16 index bytes; Q8_0: its
//     32 quants); the first MFMA takes its weights 0..15 (low nibbles / first
//     16 quants), the second 16..31, and both accumulate into one result.
// Activation rows therefore carry data in half (q4_K) or a quarter (IQ4_XS,
// Q8_0) of the lanes; the other lanes' A registers are zeroed once and never
// loaded (the LDS reads run under an execution mask).
//
// A lane's outputs are always one row, one block and four tokens, and the
// block is one whose bytes the lane loaded itself, so its weight scale comes
// from its own registers; the four activation scales are one 16-byte LDS
// read from a block-major copy.  Each result then costs a conversion and one
// or two FMAs per value.
//
// Schedule (as in the vector-ALU multi-token kernel): a wave owns 16 rows;
// teams of KS waves split a row's super-blocks; the activations are staged in
// LDS in chunks that all waves of the workgroup walk in step; the next
// super-block's weight loads are issued before the current one is computed.
//
// With few rows and a long row (fewer row tiles than compute units can hold
// workgroups, activations that need several chunks), and a caller workspace,
// K is split over workgroups instead (SPLIT): workgroup column y covers the
// units y * ups .. +ups of its row tiles, staged once as one chunk, and
// writes fp32 partial sums; the last workgroup of a column to finish sums
// the slices in slice order (the same result on every call) and re-arms the
// column's counter.  Nothing waits on another workgroup.
#include "qmv_internal.h"
#include "qmv_mfma.h"

namespace qmv {

// Work of one wave: its team's row tiles tile0 + i * gridDim.x * TEAMS
// (rounds i), and in each tile the super-blocks sb = kw, kw + KS, .. of the
// row.  A chunk holds ipc super-blocks, a multiple of KS, so the wave's
// super-blocks fall into the chunks in order.  Items q = i * n_it + j are
// loaded PF items ahead of the one computed.
//
// DOTS (the block-dot test hook): the same staging, loads, decode and MFMAs,
// but each MFMA result -- the exact integer dot of one (token, row, 32-block)
// -- times the block's integer weight scale goes to a.dots instead of into
// the fp32 sums, and nothing else is stored.
template <int F, int TM, int WPB, int KS, int PF, bool CH, bool SEG, bool SPLIT = false, bool DOTS = false>
__global__ __launch_bounds__(64 * WPB) void k_mx(StreamArgs a) {
  static_assert(!SPLIT || (!CH && !SEG), "a split launch stages one chunk of one matrix");
  static_assert(!DOTS || !SEG, "the integer mode runs one matrix");
  constexpr int TG = mx_tg<F>();
  constexpr int NG = (TM + TG - 1) / TG;  // token groups
  constexpr int TMP = NG * TG;            // staged token rows
  constexpr int TEAMS = WPB / KS;
  constexpr int NT = 64 * WPB;
  constexpr bool Q4K = F == FQ4_K;
  constexpr bool P2 = Q4K;  // two blocks per MFMA (q4_K), else four
  constexpr int SB = 4;            // staged 16-byte pieces per thread kept in flight
  // LDS, block-major: block b of the chunk holds its 32 quant bytes of every
  // token at b * BS + t * 32 (BS skewed by 16 bytes), its activation scales
  // d at dl[b * TMP + t] and (q4_K) d * s at sl[b * TMP + t]
  constexpr int BS = TMP * 32 + 16;
  static_assert(WPB % KS == 0, "teams");
  extern __shared__ __attribute__((aligned(16))) uint8_t s_mem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int team = wave / KS, kw = wave % KS;
  const int n = lane & 15, s = lane >> 4;
  // SPLIT: this workgroup's K slice starts at unit ub; `units` counts the
  // slice's units and every unit index below is relative to it
  const int ub = SPLIT ? (int)blockIdx.y * a.ups : 0;
  const int units = SPLIT ? min(a.ups, a.units - ub) : a.units;
  const int kc = a.kc, T = a.n_tok;
  const uint8_t* const wsl = a.w + (SPLIT ? (int64_t)(ub / Fmt<F>::UPB) * Fmt<F>::BB : 0);
  const int nsb = (units + 7) >> 3;  // super-blocks of a row
  const int ipc = kc >> 3;           // super-blocks per chunk
  const int nchunk = CH ? (nsb + ipc - 1) / ipc : 1;  // CH: several chunks, one round
  const int tiles = (a.n_rows + 15) >> 4;
  const int tstride = gridDim.x * TEAMS;
  const int tile0 = (int)blockIdx.x * TEAMS + team;
  // rounds of the workgroup (barriers) and of this team (its tiles)
  const int rounds_wg = (tiles - (int)blockIdx.x * TEAMS + tstride - 1) / tstride;
  const int rounds_tm = tile0 < tiles ? (tiles - tile0 + tstride - 1) / tstride : 0;
  const int n_it = nsb > kw ? (nsb - kw + KS - 1) / KS : 0;  // super-blocks per tile

  uint8_t* xl = s_mem;
  const int zoff = kc * BS;  // 16 zero bytes
  float* dl = reinterpret_cast<float*>(s_mem + zoff + 16);
  float* sl = dl + kc * TMP;
  float* red = sl + (Q4K ? kc * TMP : 0);
  if (threadIdx.x < 4) reinterpret_cast<uint32_t*>(s_mem + zoff)[threadIdx.x] = 0u;
  const float* gd = reinterpret_cast<const float*>(a.xq + a.off_d);
  const int32_t* gs = reinterpret_cast<const int32_t*>(a.xq + a.off_s);

  // Lane coordinates.  A row m = lane & 15 stands for block jA of the MFMA
  // and token tA of the group; its slots in K group s carry data only where
  // lane group s holds block jA's weights (vA).  The lane's results
  // D[4s + r][n] are for tokens oTok + r of the group and, for MFMA mu, block
  // oBlk + mu * dB of the span.  aLane / oLane: the lane's LDS byte offsets
  // of its A slots and of its activation scales for the span's first block,
  // token group 0 and mu = 0; aMu / oMu: the step for mu = 1.
  const int m = lane & 15;
  const int jA = P2 ? (m >> 3) : (m >> 2);
  const int tA = P2 ? (m & 7) : (m & 3);
  const bool vA = P2 ? (jA == (s >> 1)) : (jA == s);
  constexpr int aMu = P2 ? BS : 16;
  constexpr int oMu = P2 ? TMP * 4 : 0;
  const int aLane = (P2 ? 2 * jA : jA) * BS + tA * 32 + (P2 ? 16 * (s & 1) : 0);
  const int oTok = P2 ? 4 * (s & 1) : 0;
  const int oLane = (P2 ? 2 * (s >> 1) : s) * TMP * 4 + oTok * 4;

  // Staging of chunk c: quants and scales.  stage_issue loads the first SB
  // pieces of each thread (the caller may queue weight loads behind them);
  // stage_store stores them and moves the rest.
  u32x4 sv[SB];
  auto piece = [&](int c, int idx, const FastDiv& dq) -> const uint8_t* {
    const int t = dq.div(idx), pc = idx - t * (int)dq.d;
    return a.xq + (uint32_t)(min(t, T - 1) * a.k + 32 * (ub + c * kc) + 16 * pc);
  };
  auto stage_issue = [&](int c) {
    const int nq = 2 * min(kc, units - c * kc), total = TMP * nq;
    const FastDiv dq(nq);
#pragma unroll
    for (int i = 0; i < SB; ++i) sv[i] = ld16(piece(c, min((int)threadIdx.x + i * NT, total - 1), dq));
  };
  auto stage_store = [&](int c) {
    const int c0 = c * kc, cu = min(kc, units - c0);
    const int nq = 2 * cu, total = TMP * nq;
    const FastDiv dq(nq);
    auto put = [&](int idx, const u32x4& v) {
      const int t = dq.div(idx), pc = idx - t * nq;
      *reinterpret_cast<u32x4a*>(xl + (pc >> 1) * BS + t * 32 + 16 * (pc & 1)) = v;
    };
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int idx = (int)threadIdx.x + i * NT;
      if (idx < total) put(idx, sv[i]);
    }
    for (int base = SB * NT; base < total; base += SB * NT) {
      u32x4 v[SB];
#pragma unroll
      for (int i = 0; i < SB; ++i) v[i] = ld16(piece(c, min(base + (int)threadIdx.x + i * NT, total - 1), dq));
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int idx = base + (int)threadIdx.x + i * NT;
        if (idx < total) put(idx, v[i]);
      }
    }
    // scales: entry (t, b) read in token-major order (consecutive lanes on
    // consecutive blocks of one token: coalesced), stored block-major
    const FastDiv dk(kc);
    for (int base = 0; base < kc * TMP; base += 4 * NT) {
      float dv[4];
      int iv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = base + (int)threadIdx.x + i * NT;
        const int t = dk.div(idx), b = idx - t * kc;
        const int gi = min(t, T - 1) * a.nb + ub + c0 + min(b, cu - 1);
        dv[i] = gd[gi];
        iv[i] = gs[gi];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = base + (int)threadIdx.x + i * NT;
        const int t = dk.div(idx), b = idx - t * kc;
        const bool ok = b < cu;
        if (idx < kc * TMP) {
          dl[b * TMP + t] = ok ? dv[i] : 0.f;
          if constexpr (Q4K) sl[b * TMP + t] = ok ? dv[i] * static_cast<float>(iv[i]) : 0.f;
        }
      }
    }
  };

  // the wave's items (round i, super-block j of the tile), loaded PF ahead;
  // items past the end re-load the last one
  int hi = 0, hj = 0;  // next item to load
  // batched launches: the loaded tile's matrix rows, i.e. the base of the
  // tile's first row (clamped into its matrix) and the lane's offset from
  // it, kept until the tile changes
  int ltile = -1;
  const uint8_t* lbase = a.w;
  uint32_t loff = 0;
  auto load_next = [&](MxRaw<F>& r) {
    const int tile = min(tile0 + min(hi, max(rounds_tm - 1, 0)) * tstride, tiles - 1);
    const uint8_t* base;
    uint32_t off;
    if constexpr (SEG) {
      if (tile != ltile) {
        ltile = tile;
        const RowSeg sg = row_seg<SEG>(a, tile * 16);
        const int tb = min(tile * 16 - sg.first, sg.rows - 1);
        lbase = sg.w + (int64_t)tb * a.row_bytes;
        loff = (uint32_t)(min(n, sg.rows - 1 - tb) * (int)a.row_bytes);
      }
      base = lbase;
      off = loff;
    } else {
      base = wsl + (int64_t)tile * 16 * a.row_bytes;
      off = (uint32_t)(min(n, a.n_rows - 1 - tile * 16) * (int)a.row_bytes);
    }
    mx_load(base, off, 8 * min(kw + hj * KS, nsb - 1), s, units, r);
    if (++hj >= n_it) {
      hj = 0;
      ++hi;
    }
  };

  float acc[NG][4];
  // A operands: zero in the lanes that carry no data, which never load them
  u32x4 A[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  u32x4 Ag[NG][2];
#pragma unroll
  for (int g = 0; g < NG; ++g) Ag[g][0] = Ag[g][1] = u32x4{0u, 0u, 0u, 0u};

  // One super-block of one row tile: the two spans' MFMAs and scale steps.
  auto compute = [&](const MxRaw<F>& cur, int sb, int c, int tile) {
    const int u0 = 8 * sb;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (p > 0) __builtin_amdgcn_sched_barrier(0);  // spans one after the other
      MxDec dec;
      mx_decode(cur, p, s, u0, units, dec);
      const int bl = 8 * (sb - c * ipc) + 4 * p;  // chunk-local first block of the span
      const int ab = (vA ? bl * BS + aLane : zoff);
      const int ob = bl * TMP * 4 + oLane;
      if constexpr (!DOTS) {
        // every token group's A operands, then all the group products, then
        // the scale steps: the matrix cores work through the later groups'
        // products while the vector ALU converts and scales the earlier ones
        if (vA) {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            Ag[g][0] = ld16(xl + ab + g * TG * 32);
            Ag[g][1] = ld16(xl + ab + g * TG * 32 + aMu);
          }
        }
        i32x4 dg[NG][2];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if constexpr (P2) {
            dg[g][0] = mfma64(Ag[g][0], dec.b[0], i32x4{0, 0, 0, 0});
            dg[g][1] = mfma64(Ag[g][1], dec.b[1], i32x4{0, 0, 0, 0});
          } else {
            dg[g][0] = mfma64(Ag[g][1], dec.b[1], mfma64(Ag[g][0], dec.b[0], i32x4{0, 0, 0, 0}));
          }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
#pragma unroll
          for (int mu = 0; mu < (P2 ? 2 : 1); ++mu) {
            const i32x4 dv = dg[g][mu];
            const int o = ob + mu * oMu + g * TG * 4;
            const f32x4 fx = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(dl) + o);
            const float fxa[4] = {fx.x, fx.y, fx.z, fx.w};
            if constexpr (Q4K) {
              const f32x4 fs = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(sl) + o);
              const float fsa[4] = {fs.x, fs.y, fs.z, fs.w};
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                acc[g][r] = fmaf(static_cast<float>(dv[r]), dec.dw[mu] * fxa[r], acc[g][r]);
                acc[g][r] = fmaf(-dec.wm[mu], fsa[r], acc[g][r]);
              }
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[g][r] = fmaf(static_cast<float>(dv[r]), dec.dw[mu] * fxa[r], acc[g][r]);
            }
          }
        }
        continue;
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g > 0) __builtin_amdgcn_sched_barrier(0);
        if (vA) {
          A[0] = ld16(xl + ab + g * TG * 32);
          A[1] = ld16(xl + ab + g * TG * 32 + aMu);
        }
        if constexpr (DOTS) {
          // lane (n, s): row tile * 16 + n; result r is block bl + (q4_K:
          // 2 (s >> 1) + mu; else s) of token (q4_K: 8g + 4 (s & 1) + r;
          // else 4g + r), as the scale steps below read them
          const int row = tile * 16 + n;
#pragma unroll
          for (int mu = 0; mu < (P2 ? 2 : 1); ++mu) {
            i32x4 dv;
            if constexpr (P2) {
              dv = mfma64(A[mu], dec.b[mu], i32x4{0, 0, 0, 0});
            } else {
              dv = mfma64(A[0], dec.b[0], i32x4{0, 0, 0, 0});
              dv = mfma64(A[1], dec.b[1], dv);
            }
            const int lb = u0 + 4 * p + (P2 ? 2 * (s >> 1) + mu : s);  // unit inside the slice
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = P2 ? g * TG + 4 * (s & 1) + r : g * TG + r;
              if (t < T && row < a.n_rows && lb < units) {
                const int64_t o = ((int64_t)t * a.n_rows + row) * a.units + ub + lb;
                if constexpr (Q4K) {
                  a.dots[2 * o] = dec.isc[mu] * dv[r];
                  a.dots[2 * o + 1] = dec.im[mu] * gs[t * a.nb + ub + lb];
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
            const float fxa[4] = {fx.x, fx.y, fx.z, fx.w};
            if constexpr (Q4K) {
              const f32x4 fs = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(sl) + o);
              const float fsa[4] = {fs.x, fs.y, fs.z, fs.w};
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                acc[g][r] = fmaf(static_cast<float>(dv[r]), dec.dw[mu] * fxa[r], acc[g][r]);
                acc[g][r] = fmaf(-dec.wm[mu], fsa[r], acc[g][r]);
              }
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[g][r] = fmaf(static_cast<float>(dv[r]), dec.dw[mu] * fxa[r], acc[g][r]);
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
  };

  // Ring of PF loaded super-blocks: item q of the wave sits in slot q % PF
  // (relative to the rotation at chunk and round ends); each slot is reloaded
  // with the item PF ahead right after it has been computed.
  MxRaw<F> ring[PF];
  stage_issue(0);
#pragma unroll
  for (int k = 0; k < PF; ++k) load_next(ring[k]);
  stage_store(0);
  __syncthreads();

  for (int i = 0; i < rounds_wg; ++i) {
    const int tile = tile0 + i * tstride;
    const bool have = i < rounds_tm;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[g][r] = 0.f;
    for (int c = 0; c < nchunk; ++c) {
      if (CH && (c > 0 || i > 0)) {  // several chunks: restage
        __syncthreads();  // every wave is done with the previous chunk
        stage_issue(c);
        stage_store(c);
        __syncthreads();
      }
      const int sb0 = c * ipc + kw;
      const int sb_end = min((c + 1) * ipc, nsb);
      const int njc = have && sb0 < sb_end ? (sb_end - sb0 + KS - 1) / KS : 0;
      for (int j0 = 0; j0 < njc; j0 += PF) {
#pragma unroll
        for (int kk = 0; kk < PF; ++kk) {
          if (j0 + kk < njc) {
            compute(ring[kk], sb0 + (j0 + kk) * KS, c, tile);
            load_next(ring[kk]);
          }
        }
      }
      // the wave's next item sits in slot njc % PF: rotate it to slot 0
      for (int x = njc % PF; x > 0; --x) {
        const MxRaw<F> t0 = ring[0];
#pragma unroll
        for (int k = 0; k + 1 < PF; ++k) ring[k] = ring[k + 1];
        ring[PF - 1] = t0;
      }
    }

    if constexpr (DOTS) continue;  // the integers are out; nothing to sum
    // Sum over the lanes that hold the other blocks of the same row and
    // tokens (two blocks per MFMA: lane ^ 32; Q8_0: lanes ^ 16, ^ 32).  Then
    // with two blocks per MFMA lanes s = 0, 1 hold tokens 8g + 4s + r; Q8_0:
    // every lane holds tokens 4g + r and lane group s stores group g = s.
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[g][r];
        if constexpr (!P2) v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        acc[g][r] = v;
      }
    if constexpr (KS == 1) {
      const int row = tile * 16 + n;
      if (have) {
        const RowSeg sg = row_seg<SEG>(a, tile * 16);
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = P2 ? g * 8 + 4 * s + r : g * 4 + r;
            const bool mine = P2 ? s < 2 : s == (g & 3);
            if (mine && t < T) {
              if constexpr (SPLIT) {
                if (row < a.n_rows)
                  __hip_atomic_store(&a.part[((int64_t)blockIdx.y * T + t) * a.n_rows + row], acc[g][r],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              } else {
                seg_store(sg, t, row, acc[g][r]);
              }
            }
          }
      }
    } else {
      // team partials through LDS: red[team][kw][TMP][16], summed in wave order
      float* mine_red = red + ((team * KS + kw) * TMP) * 16;
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = P2 ? g * 8 + 4 * s + r : g * 4 + r;
          const bool mine = P2 ? s < 2 : s == (g & 3);
          if (mine) mine_red[t * 16 + n] = acc[g][r];
        }
      __syncthreads();
      for (int q = threadIdx.x; q < TEAMS * TMP * 16; q += NT) {
        const int tm = q / (TMP * 16), rest = q - tm * (TMP * 16);
        const int t = rest >> 4, nn = rest & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < KS; ++w) sum += red[((tm * KS + w) * TMP) * 16 + rest];
        const int tl = (int)blockIdx.x * TEAMS + tm + i * tstride;  // that team's tile
        const int row = tl * 16 + nn;
        if constexpr (SPLIT) {
          if (row < a.n_rows && t < T)
            __hip_atomic_store(&a.part[((int64_t)blockIdx.y * T + t) * a.n_rows + row], sum,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (tl < tiles && t < T) {
          seg_store(row_seg<SEG>(a, tl * 16), t, row, sum);
        }
      }
      __syncthreads();  // the partials area is reused by the next round
    }
  }

  if constexpr (SPLIT && !DOTS) {
    // The last workgroup of this column (its TEAMS row tiles) to finish sums
    // the slices' partials in slice order.  The partials are stored and
    // loaded with device-scope atomic accesses, which the gfx950 L2 writes
    // through and reloads (the sc1 bit), so they meet at the device's
    // coherence point without a device-scope fence: each lane waits for its
    // stores to be acknowledged before the barrier that precedes the
    // counter update, and the sums are loaded only after the counter's
    // value was seen.  (A device-scope fence here would write back and
    // invalidate this XCD's whole L2 once per workgroup: measured 10x
    // slower overall.)
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt, lgkmcnt all zero
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(&a.cnt[blockIdx.x], 1) == (int)gridDim.y - 1;
    __syncthreads();
    if (s_last) {
      constexpr int RW = TEAMS * 16;
      const int r0 = (int)blockIdx.x * RW;
      for (int q = threadIdx.x; q < T * RW; q += NT) {
        const int t = q / RW, row = r0 + (q - t * RW);
        if (row < a.n_rows) {
          float sum = 0.f;
          for (int sl = 0; sl < (int)gridDim.y; ++sl)
            sum += __hip_atomic_load(&a.part[((int64_t)sl * T + t) * a.n_rows + row], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          a.y[(int64_t)t * a.ldy + row] = sum;
        }
      }
      if (threadIdx.x == 0) atomicExch(&a.cnt[blockIdx.x], 0);
    }
  }
}

// Units (32-blocks) per LDS chunk: a multiple of `step` (whole super-blocks,
// an equal share for every wave of a team), as many as the budget allows,
// balanced over the chunks a row needs.
static int mx_chunk_units(int units, int per_unit, int step, int64_t budget) {
  int kmax = (int)(budget / per_unit) / step * step;
  if (kmax < step) return 0;
  const int need = (units + step - 1) / step * step;
  if (kmax >= need) return need;
  const int chunks = (units + kmax - 1) / kmax;
  const int per = (units + chunks - 1) / chunks;
  return (per + step - 1) / step * step;
}

// LDS budget of one k_mx workgroup: the whole activation buffer when it fits
// in 144 KB (then one workgroup per compute unit stages it once and walks
// its row tiles), else chunks.
constexpr int64_t kMxLdsBudget = 144 * 1024;

// Fixed LDS bytes of a k_mx workgroup (mx_per_unit: qmv_mfma.h).
static int64_t mx_fixed(int wpb, int ks, int tmp) { return 16 + (ks > 1 ? (int64_t)wpb * tmp * 16 * 4 : 0); }

#if QMV_MX_FMT == 0  // host helpers: defined once, in the Q8_0 unit
int mx_split_plan(int fmt, int n_tok, int wpb, int ks, int units, int n_rows, int cus, int64_t lds_per_cu,
                  int forced, int* ups_out) {
  const int tg = fmt == FQ4_K ? 8 : 4;
  const int tm = n_tok <= 4 ? 4 : n_tok <= 8 ? 8 : 16;
  const int tmp = (tm + tg - 1) / tg * tg;
  const int per_unit = mx_per_unit(fmt, tmp);
  const int64_t fixed = mx_fixed(wpb, ks, tmp);
  const int step = 8 * ks;
  if (forced == 0) return 0;
  // a slice is whole wave shares and fits one chunk in the LDS of 2 (8-wave)
  // or 1 (16-wave) workgroups per compute unit, 64 bytes left for the
  // arrival flag
  const int64_t wgs = wpb <= 8 ? 2 : 1;
  const int64_t budget = (kMxLdsBudget < lds_per_cu / wgs ? kMxLdsBudget : lds_per_cu / wgs) - 64 - fixed;
  const int ups_max = (int)(budget / per_unit) / step * step;
  if (ups_max < step) return 0;
  int want = forced;
  if (forced < 0) {
    // automatic: rows that need several chunks unsplit, on fewer row-tile
    // workgroups than compute units, split into as many slices as give
    // every compute unit a workgroup -- if one chunk per slice fits in
    // that many (measured on 4096 x 14336, q4_K and IQ4_XS at 5..16
    // tokens: more, thinner slices cost more than the restaging they save)
    if (mx_chunk_units(units, per_unit, step, kMxLdsBudget - fixed) >= units) return 0;
    const int64_t cols = ((int64_t)(n_rows + 15) / 16 + wpb / ks - 1) / (wpb / ks);
    const int64_t fill = (cus + cols - 1) / cols;
    const int64_t s_lds = (units + ups_max - 1) / ups_max;
    if (fill < 2 || s_lds > fill) return 0;
    want = (int)(fill < kMaxSlices ? fill : kMaxSlices);
  }
  int ups = ((units + want - 1) / want + step - 1) / step * step;
  if (ups > ups_max) ups = ups_max;  // a forced count too small to fit: more slices
  const int slices = (units + ups - 1) / ups;
  if (slices < 2 || slices > kMaxSlices) return 0;
  *ups_out = ups;
  return slices;
}
#endif

template <int F, int TM, int WPB, int KS, int PF>
static hipError_t run_mx(const MatvecLaunch& a, hipStream_t st) {
  constexpr int TG = mx_tg<F>();
  constexpr int TMP = ((TM + TG - 1) / TG) * TG;
  constexpr int TEAMS = WPB / KS;
  StreamArgs sa{};
  sa.w = a.w;
  sa.row_bytes = a.row_bytes;
  sa.n_rows = a.n_rows;
  sa.units = a.units;
  sa.xq = a.xq;
  sa.act_bytes = (int)a.act_bytes;
  sa.off_d = (int)a.off_d;
  sa.off_s = (int)a.off_s;
  sa.k = a.x.k;
  sa.nb = a.x.nb;
  sa.n_tok = a.n_tok;
  sa.y = a.y;
  sa.ldy = a.ldy;
  sa.res = a.res;
  sa.ldr = a.ldr;
  sa.seg = a.seg;
  const int64_t fixed = mx_fixed(WPB, KS, TMP);
  const int per_unit = mx_per_unit(F, TMP);
  sa.kc = mx_chunk_units(a.units, per_unit, 8 * KS, kMxLdsBudget - fixed);
  if (sa.kc <= 0) return hipErrorInvalidValue;
  const size_t lds = (size_t)sa.kc * per_unit + fixed;
  const int64_t tiles = (a.n_rows + 15) / 16;
  const int64_t need = (tiles + TEAMS - 1) / TEAMS;
  if (a.dots != nullptr) {
    // integer mode (test hook): the same launch shapes, no workspace
    sa.dots = a.dots;
    int ups = 0;
    const int slices = a.dots_slices == 0 ? 0
                       : mx_split_plan(F, a.n_tok, WPB, KS, a.units, a.n_rows, a.cus, a.lds_per_cu, a.dots_slices,
                                       &ups);
    if (slices >= 2) {
      sa.kc = ups;
      sa.ups = ups;
      hipLaunchKernelGGL((k_mx<F, TM, WPB, KS, PF, false, false, true, true>), dim3((unsigned)need, (unsigned)slices),
                         dim3(64 * WPB), (size_t)ups * per_unit + fixed, st, sa);
    } else if (a.dots_slices >= 2) {
      return hipErrorInvalidValue;  // the forced slice count does not fit
    } else if (sa.kc >= a.units) {
      const int64_t per_cu = (int64_t)a.lds_per_cu / (int64_t)lds;
      const int64_t cap = (int64_t)a.cus * (per_cu < 1 ? 1 : per_cu);
      hipLaunchKernelGGL((k_mx<F, TM, WPB, KS, PF, false, false, false, true>), dim3((unsigned)(need < cap ? need : cap)),
                         dim3(64 * WPB), lds, st, sa);
    } else {
      hipLaunchKernelGGL((k_mx<F, TM, WPB, KS, PF, true, false, false, true>), dim3((unsigned)need), dim3(64 * WPB),
                         lds, st, sa);
    }
    return hipGetLastError();
  }
  if (a.part != nullptr && a.cnt != nullptr && a.seg.n == 0) {
    int ups = 0;
    const int slices =
        mx_split_plan(F, a.n_tok, WPB, KS, a.units, a.n_rows, a.cus, a.lds_per_cu, mx_slices(), &ups);
    if (slices >= 2) {
      sa.kc = ups;
      sa.ups = ups;
      sa.part = a.part;
      sa.cnt = a.cnt;
      const size_t lds_s = (size_t)ups * per_unit + fixed;
      hipLaunchKernelGGL((k_mx<F, TM, WPB, KS, PF, false, false, true>), dim3((unsigned)need, (unsigned)slices),
                         dim3(64 * WPB), lds_s, st, sa);
      return hipGetLastError();
    }
  }
  if (sa.kc >= a.units) {
    // one K chunk: persistent, as many workgroups as fit at once
    const int64_t per_cu = (int64_t)a.lds_per_cu / (int64_t)lds;
    const int64_t cap = (int64_t)a.cus * (per_cu < 1 ? 1 : per_cu);
    const int64_t grid = need < cap ? need : cap;
    if (a.seg.n > 0)
      hipLaunchKernelGGL((k_mx<F, TM, WPB, KS, PF, false, true>), dim3((unsigned)grid), dim3(64 * WPB), lds, st, sa);
    else
      hipLaunchKernelGGL((k_mx<F, TM, WPB, KS, PF, false, false>), dim3((unsigned)grid), dim3(64 * WPB), lds, st, sa);
  } else {
    // several chunks: one row tile per team, the chunks walked once
    if (a.seg.n > 0)
      hipLaunchKernelGGL((k_mx<F, TM, WPB, KS, PF, true, true>), dim3((unsigned)need), dim3(64 * WPB), lds, st, sa);
    else
      hipLaunchKernelGGL((k_mx<F, TM, WPB, KS, PF, true, false>), dim3((unsigned)need), dim3(64 * WPB), lds, st, sa);
  }
  return hipGetLastError();
}

// variant fields: wpb = waves per workgroup, ks = waves splitting K, nu =
// super-blocks in the load ring
template <int F, int TM>
static hipError_t run_mx_shape(const MatvecLaunch& a, const Variant& v, hipStream_t st) {
  if (v.wpb == 16 && v.nu == 2) {
    switch (v.ks) {
      case 4: return run_mx<F, TM, 16, 4, 2>(a, st);
      case 8: return run_mx<F, TM, 16, 8, 2>(a, st);
      case 16: return run_mx<F, TM, 16, 16, 2>(a, st);
    }
  } else if (v.wpb == 8 && v.nu == 4) {
    switch (v.ks) {
      case 1: return run_mx<F, TM, 8, 1, 4>(a, st);
      case 4: return run_mx<F, TM, 8, 4, 4>(a, st);
      case 8: return run_mx<F, TM, 8, 8, 4>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

template <int F>
static hipError_t run_mx_tokens(const MatvecLaunch& a, const Variant& v, hipStream_t st) {
  if (a.n_tok <= 4) return run_mx_shape<F, 4>(a, v, st);
  if (a.n_tok <= 8) return run_mx_shape<F, 8>(a, v, st);
  return run_mx_shape<F, 16>(a, v, st);
}

// This translation unit is compiled once per weight format with a
// matrix-core decode (QMV_MX_FMT), so that their kernels build in parallel;
// each copy defines the matrix-core entry of its format, and the Q8_0 copy
// also the dispatcher and the split plan.
#ifndef QMV_MX_FMT
#error "compile qmv_mfma.hip with -DQMV_MX_FMT=<format id>"
#endif
template <>
hipError_t launch_mx_fmt<QMV_MX_FMT>(const MatvecLaunch& a, hipStream_t st) {
  return run_mx_tokens<QMV_MX_FMT>(a, kVariants[a.variant], st);
}

#if QMV_MX_FMT == 0
hipError_t launch_mx(const MatvecLaunch& a, hipStream_t st) {
  switch (a.fmt) {
    case FQ8_0: return launch_mx_fmt<FQ8_0>(a, st);
    case FQ4_K: return launch_mx_fmt<FQ4_K>(a, st);
    case FIQ4_XS: return launch_mx_fmt<FIQ4_XS>(a, st);
    case FQ8G128: return launch_mx_fmt<FQ8G128>(a, st);
    default: return hipErrorInvalidValue;
  }
}
#endif

}  // namespace qmv
