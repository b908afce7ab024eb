// qmv_mfma.h -- gfx950 matrix-core building blocks shared by the dense
// (qmv_mfma.hip) and the expert-grouped (qmv_moe.hip) kernels: per-lane weight
// loads of one super-block (8 consecutive 32-blocks), their decode into
// v_mfma_i32_16x16x64_i8 B operands, and the MFMA itself.  The operand layout
// and the zero-masked activation rows that keep every 32-block's integer dot
// separate are described in qmv_mfma.hip.
#pragma once

#include "qmv_device.h"

namespace qmv {

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int F> constexpr int mx_tg() { return F == FQ4_K ? 8 : 4; }  // tokens per group

// Raw bytes of one lane for one super-block (8 consecutive 32-blocks).
template <int F> struct MxRaw;
template <> struct MxRaw<FQ4_K> {
  u32x4 q[2];  // span p = 0, 1: bytes 64p + 16s .. +15 of the nibble area
  u32x4 hdr;   // d | dmin, 12 bytes of packed 6-bit scales and mins
};
template <> struct MxRaw<FIQ4_XS> {
  u32x4 q[2];  // span p: the 16 index bytes of sub-block 4p + s
  u32x2 hdr;   // d | scales_h, scales_l[0..3]
};
template <> struct MxRaw<FQ8_0> {
  Raw<FQ8_0> b[2];  // span p: 32-block 8i + 4p + s
};
template <> struct MxRaw<FQ8G128> {
  Raw<FQ8G128> b[2];  // span p: 32-block 8i + 4p + s (a quarter of group 2i + p)
};

// Loads of one lane for the super-block starting at unit u0: `base` is the
// wave-uniform address of the tile's first row, `off` the lane's row offset
// (32 bits, so that the address is a scalar base plus a vector offset).
__device__ __forceinline__ void mx_load(const uint8_t* base, uint32_t off, int u0, int s, int, MxRaw<FQ4_K>& r) {
  const uint32_t blk = off + 144u * ((uint32_t)u0 >> 3);
  r.hdr = ld_w16(base + blk);
  r.q[0] = ld_w16(base + (blk + 16 + 16 * (uint32_t)s));
  r.q[1] = ld_w16(base + (blk + 80 + 16 * (uint32_t)s));
}
__device__ __forceinline__ void mx_load(const uint8_t* base, uint32_t off, int u0, int s, int, MxRaw<FIQ4_XS>& r) {
  const uint32_t blk = off + 136u * ((uint32_t)u0 >> 3);
  r.hdr = ld_w8(base + blk);
  r.q[0] = ld_w16(base + (blk + 8 + 16 * (uint32_t)s));
  r.q[1] = ld_w16(base + (blk + 72 + 16 * (uint32_t)s));
}
// Q8_0 rows need not be a whole number of super-blocks: units past the row
// end re-read the last unit (their scale is zeroed at decode).
__device__ __forceinline__ void mx_load(const uint8_t* base, uint32_t off, int u0, int s, int units, MxRaw<FQ8_0>& r) {
  load_unit(base + off, min(u0 + s, units - 1), r.b[0]);
  load_unit(base + off, min(u0 + 4 + s, units - 1), r.b[1]);
}

// Q8G128: a super-block is two 128-weight groups; span p is group 2i + p and
// lane group s its quarter s.  Rows need not be a whole number of
// super-blocks: units past the row end re-read the last unit (their scale is
// zeroed at decode).
__device__ __forceinline__ void mx_load(const uint8_t* base, uint32_t off, int u0, int s, int units, MxRaw<FQ8G128>& r) {
  load_unit(base + off, min(u0 + s, units - 1), r.b[0]);
  load_unit(base + off, min(u0 + 4 + s, units - 1), r.b[1]);
}

// Decoded weights of one span for one lane: B operands of the two MFMA
// halves and the scales of the lane's output blocks.
struct MxDec {
  u32x4 b[2];
  float dw[2];  // weight scale of the output block of half h (IQ4_XS, Q8_0: both the same)
  float wm[2];  // q4_K: dmin * m of that block
  // the integer scales behind dw and wm (q4_K: the 6-bit sc and m; IQ4_XS:
  // ls - 32; Q8_0, Q8G128: 1), for the block-dot test hook
  int isc[2], im[2];
};

// q4_K: 6-bit (scale, min) of sub-block c (0..7) from the 12 packed bytes.
__device__ __forceinline__ void q4k_scale_min(const u32x4& hdr, int c, uint32_t& sc, uint32_t& m) {
  const uint32_t jj = 8u * (uint32_t)(c & 3);
  const uint32_t hb = 2u * (uint32_t)(c >> 2);
  const uint32_t s03 = hdr.y, s47 = hdr.z, s811 = hdr.w;
  const uint32_t lo_sc = c < 4 ? s03 : s811;
  const uint32_t lo_m = c < 4 ? s47 : s811;
  sc = bfe(lo_sc, jj, 4) | (bfe(s03, jj + 4 + hb, 2) << 4);
  m = bfe(lo_m, jj + 2 * hb, 4) | (bfe(s47, jj + 4 + hb, 2) << 4);
}

// p = span (0, 1), s = lane group, u0 = first unit of the super-block.
__device__ __forceinline__ void mx_decode(const MxRaw<FQ4_K>& r, int p, int s, int, int, MxDec& o) {
  const u32x4 q = r.q[p];
  o.b[0] = u32x4{q.x & 0x0F0F0F0Fu, q.y & 0x0F0F0F0Fu, q.z & 0x0F0F0F0Fu, q.w & 0x0F0F0F0Fu};
  o.b[1] = u32x4{(q.x >> 4) & 0x0F0F0F0Fu, (q.y >> 4) & 0x0F0F0F0Fu, (q.z >> 4) & 0x0F0F0F0Fu,
                 (q.w >> 4) & 0x0F0F0F0Fu};
  const float d = half_bits_to_float(r.hdr.x), dmin = half_bits_to_float(r.hdr.x >> 16);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t sc, m;
    q4k_scale_min(r.hdr, 4 * p + 2 * (s >> 1) + h, sc, m);
    o.dw[h] = d * static_cast<float>(sc);
    o.wm[h] = dmin * static_cast<float>(m);
    o.isc[h] = static_cast<int>(sc);
    o.im[h] = static_cast<int>(m);
  }
}
__device__ __forceinline__ void mx_decode(const MxRaw<FIQ4_XS>& r, int p, int s, int, int, MxDec& o) {
  const u32x4 q = r.q[p];
  uint32_t lo[4], hi[4];
  iq4_lookup2(q.x, lo[0], hi[0]);
  iq4_lookup2(q.y, lo[1], hi[1]);
  iq4_lookup2(q.z, lo[2], hi[2]);
  iq4_lookup2(q.w, lo[3], hi[3]);
  o.b[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  o.b[1] = u32x4{hi[0], hi[1], hi[2], hi[3]};
  const int c = 4 * p + s;
  const uint32_t lo4 = (r.hdr.y >> (4 * c)) & 15u;
  const uint32_t hi2 = (r.hdr.x >> (16 + 2 * c)) & 3u;
  const int ls = static_cast<int>(lo4 | (hi2 << 4)) - 32;
  o.dw[0] = o.dw[1] = half_bits_to_float(r.hdr.x) * static_cast<float>(ls);
  o.wm[0] = o.wm[1] = 0.f;
  o.isc[0] = o.isc[1] = ls;
  o.im[0] = o.im[1] = 0;
}
__device__ __forceinline__ void mx_decode(const MxRaw<FQ8_0>& r, int p, int s, int u0, int units, MxDec& o) {
  Dec<FQ8_0> d;
  decode_unit(r.b[p], 0, d);
  o.b[0] = u32x4{d.q[0], d.q[1], d.q[2], d.q[3]};
  o.b[1] = u32x4{d.q[4], d.q[5], d.q[6], d.q[7]};
  const bool ok = u0 + 4 * p + s < units;
  o.dw[0] = o.dw[1] = ok ? d.d : 0.f;
  o.wm[0] = o.wm[1] = 0.f;
  o.isc[0] = o.isc[1] = 1;
  o.im[0] = o.im[1] = 0;
}

__device__ __forceinline__ void mx_decode(const MxRaw<FQ8G128>& r, int p, int s, int u0, int units, MxDec& o) {
  const bool ok = u0 + 4 * p + s < units;
  DecO<FQ8G128> d;
  decode_own(r.b[p], 0, 0, ok, d);
  o.b[0] = u32x4{d.q[0], d.q[1], d.q[2], d.q[3]};
  o.b[1] = u32x4{d.q[4], d.q[5], d.q[6], d.q[7]};
  o.dw[0] = o.dw[1] = d.sc;
  o.wm[0] = o.wm[1] = 0.f;
  o.isc[0] = o.isc[1] = 1;
  o.im[0] = o.im[1] = 0;
}

// LDS bytes per staged unit (32-block) of the matrix-core kernels'
// block-major activation copy for tmp token rows: 32 quant bytes per token
// plus a 16-byte skew, and the fp32 scales d (and for q4_K d * s) per token.
inline int mx_per_unit(int fmt, int tmp) { return (tmp * 32 + 16) + tmp * 4 * (fmt == FQ4_K ? 2 : 1); }

__device__ __forceinline__ i32x4 mfma64(const u32x4& a, const u32x4& b, i32x4 c) {
  const i32x4 av = __builtin_bit_cast(i32x4, a);
  const i32x4 bv = __builtin_bit_cast(i32x4, b);
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
}

}  // namespace qmv
