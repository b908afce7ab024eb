// qmv_device.h -- gfx950 device routines shared by the qmv kernels: block
// field decoders, per-unit weight loads, integer dot products and lane
// reductions.
//
// Work unit.  Every kernel walks a weight row in "units" of 16 quant bytes
// (32 weights for Q8_0 and IQ4_XS, which is one 32-block; q4_K units hold the
// same 16 positions of two sub-blocks):
//   Q8_0   : block b                     weights 0..31 of block b
//   IQ4_XS : sub-block c of sb           low nibbles -> weights 0..15,
//                                        high nibbles -> weights 16..31
//   q4_K   : 16 quant bytes c of sb (bytes 16c..16c+15 of the nibble area):
//            low nibbles are weights 16h..16h+15 (h = c & 1) of sub-block
//            j = 2 (c >> 1), high nibbles the same positions of sub-block j+1.
//   q5_K   : as q4_K, plus the 16 qh bytes 16h..16h+15 that carry the fifth
//            bit of those positions (bit j for sub-block j, j + 1 for j + 1).
//   Q8G128 : 32-block u = quarter u & 3 of group u >> 2 (130 B: fp16 d,
//            int8 q[128]); the group's scale is shared by its four units
//   q6_K   : 32-block u (half f = (u & 7) >> 2, quarter j = u & 3) and its
//            partner u ^ 2 take the low and high nibbles of the same 32 ql
//            bytes; the unit holds positions 16h..16h+15, h = (u >> 1) & 1,
//            of both: 16 ql bytes and the 16 qh bytes of those positions.
// So one 16-byte quant load per lane feeds one unit, and the eight lanes of a
// super-block read its 128 quant bytes as one contiguous 128-byte span.
// (GGUF block layouts; the pages name the formats only -- Castagna Veloce
// page, "Kernels for the MI50"; zhuai.tech GLM-5.3 page, "A single decode row
// is not a large matrix multiplication".)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

enum : int { FQ8_0 = 0, FQ4_K = 1, FIQ4_XS = 2, FQ5_K = 3, FQ6_K = 4, FQ8G128 = 5 };

// K-quants with a per-sub-block min (q4_K, q5_K): paired own-block form, two
// integer partials per block.
template <int F> constexpr bool kmin() { return F == FQ4_K || F == FQ5_K; }
// Formats whose unit pairs lanes u and u ^ 1 (the K-quants with a min) or
// u and u ^ 2 (q6_K); the others hold a whole 32-block per lane.
template <int F> constexpr int pair_xor() { return kmin<F>() ? 1 : (F == FQ6_K ? 2 : 0); }

template <int F> struct Fmt;
template <> struct Fmt<FQ8_0> { static constexpr int QK = 32, BB = 34, UPB = 1; };
template <> struct Fmt<FQ4_K> { static constexpr int QK = 256, BB = 144, UPB = 8; };
template <> struct Fmt<FIQ4_XS> { static constexpr int QK = 256, BB = 136, UPB = 8; };
template <> struct Fmt<FQ5_K> { static constexpr int QK = 256, BB = 176, UPB = 8; };
template <> struct Fmt<FQ6_K> { static constexpr int QK = 256, BB = 210, UPB = 8; };
template <> struct Fmt<FQ8G128> { static constexpr int QK = 128, BB = 130, UPB = 4; };

// 16- and 8-byte vectors that only promise 4-byte alignment: gfx950 global
// loads of several dwords need dword alignment only.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x4 __attribute__((ext_vector_type(4), aligned(4)));

// Weight loads.  Plain cached loads: a Q8_0 block is read by three
// instructions (two 16-byte halves and the scale) that share cache lines,
// and non-temporal loads made the later ones miss (measured: the Q8_0 output
// head ran at 3.9 TB/s with them and 5.8 TB/s without).
__device__ __forceinline__ u32x4 ld_w16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld_w8(const uint8_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ uint32_t ld_w2(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}
// 16-byte vector with its natural alignment: activation fragments are
// 16-byte aligned in global memory and in LDS (ds_read_b128).
typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4a*>(p);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h16 & 0xFFFFu)));
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// DPP lane moves inside a 16-lane row (gfx9 encodings): swap neighbours,
// swap pairs, mirror each 8-lane half, mirror the row.
enum : int { DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140 };

// Every control used here reads a lane inside the same row, so no lane is
// ever out of bounds; bound_ctrl lets the move skip initialising its target.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// ------------------------------------------------------------ raw unit loads
template <int F> struct Raw;

// Q8_0 blocks are 34 bytes, so a block starts at an address that is 0 or 2
// mod 4.  At 0 mod 4 the block is read as 16 + 16 + 2 bytes and the quants
// are realigned by two bytes; at 2 mod 4 the quants themselves are dword
// aligned and the scale is a separate 2-byte load.  Neither form reads a byte
// outside the block.
template <> struct Raw<FQ8_0> {
  u32x4 a, b;
  uint32_t h;
  uint32_t odd;
};
template <> struct Raw<FQ4_K> {
  u32x4 q;    // 16 quant bytes of the unit
  u32x4 hdr;  // d | dmin, S[0..3], S[4..7], S[8..11]
};
template <> struct Raw<FIQ4_XS> {
  u32x4 q;    // 16 quant bytes of the unit (= one sub-block)
  u32x2 hdr;  // d | scales_h, scales_l[0..3]
};
template <> struct Raw<FQ5_K> {
  u32x4 q;    // 16 nibble bytes of the unit
  u32x4 hdr;  // the q4_K header
  u32x4 qh;   // the 16 qh bytes of the unit's positions
};
template <> struct Raw<FQ8G128> {
  u32x4 a, b;    // the unit's 32 quants, from the dword at or below them
  uint32_t h;    // its last two quants (used when the quants start 2 mod 4)
  uint32_t odd;  // 1: the quants are dword aligned
  uint32_t d;    // fp16 bits of the group scale
};
template <> struct Raw<FQ6_K> {
  u32x4 ql, qh;        // the 16 ql and 16 qh bytes of the unit's positions
  int sc_own, sc_par;  // int8 scales of those positions in the own and partner block
  uint32_t d;          // fp16 bits of the super-block scale
};

// Unit loads take the row base and 32-bit byte offsets inside the row, so a
// row base held in scalar registers needs no per-lane 64-bit address math.
__device__ __forceinline__ void load_unit(const uint8_t* row, int u, Raw<FQ8_0>& r) {
  const uint32_t off = 34u * (uint32_t)u;
  // the block's alignment mod 4 decides which of its two halves is dword
  // aligned: the quants (address 2 mod 4) or the scale (0 mod 4)
  const uint32_t odd = (((uint32_t)reinterpret_cast<uintptr_t>(row) + off) >> 1) & 1u;
  const uint32_t qoff = odd ? off + 2 : off;
  const uint32_t hoff = odd ? off : off + 32;
  r.a = ld_w16(row + qoff);
  r.b = ld_w16(row + (qoff + 16));
  r.h = ld_w2(row + hoff);
  r.odd = odd;
}
__device__ __forceinline__ void load_unit(const uint8_t* row, int u, Raw<FQ4_K>& r) {
  const uint32_t blk = 144u * ((uint32_t)u >> 3);
  const uint32_t qoff = blk + 16 + 16 * ((uint32_t)u & 7);
  r.q = ld_w16(row + qoff);
  r.hdr = ld_w16(row + blk);
}
// Q8G128 groups are 130 bytes, so a unit's 32 quants start 0 or 2 mod 4.  At
// 2 mod 4 they are read as the 32 bytes from two bytes below them (the last
// two bytes of the previous unit, or the group's scale) plus a 2-byte load of
// their last two, and realigned; no byte outside the group is read.
__device__ __forceinline__ void load_unit(const uint8_t* row, int u, Raw<FQ8G128>& r) {
  const uint32_t goff = 130u * ((uint32_t)u >> 2);
  const uint32_t q0 = goff + 2 + 32 * ((uint32_t)u & 3);
  const uint32_t mis = ((uint32_t)reinterpret_cast<uintptr_t>(row) + q0) & 2u;
  r.a = ld_w16(row + (q0 - mis));
  r.b = ld_w16(row + (q0 - mis + 16));
  r.h = ld_w2(row + q0 + 30);
  r.odd = mis ? 0u : 1u;
  r.d = ld_w2(row + goff);
}
// 16 bytes at byte offset off of a row whose base is 16-byte aligned, where
// row + off may be 2 mod 4 (q6_K blocks are 210 bytes): five dwords from the
// aligned address at or below it, realigned.  A q6_K ql or qh piece ends at
// least 18 bytes before its block's end, and a piece at 2 mod 4 starts at
// least 2 bytes after the row base, so both extra bytes read stay in the row.
__device__ __forceinline__ u32x4 ld16_a2(const uint8_t* row, uint32_t off) {
  const uint8_t* p = row + off;
  const uint32_t sh = (uint32_t)reinterpret_cast<uintptr_t>(p) & 3u;  // 0 or 2
  const uint8_t* a = p - sh;
  const u32x4 v = ld_w16(a);
  const uint32_t e = *reinterpret_cast<const uint32_t*>(a + 16);
  return u32x4{__builtin_amdgcn_alignbyte(v.y, v.x, sh), __builtin_amdgcn_alignbyte(v.z, v.y, sh),
               __builtin_amdgcn_alignbyte(v.w, v.z, sh), __builtin_amdgcn_alignbyte(e, v.w, sh)};
}
// q6_K super-block: ql (128 B) | qh (64 B) | int8 scales[16] | fp16 d.
__device__ __forceinline__ void load_unit(const uint8_t* row, int u, Raw<FQ6_K>& r) {
  const uint32_t blk = 210u * ((uint32_t)u >> 3);
  const uint32_t c = (uint32_t)u & 7, f = c >> 2, j = c & 3, h = (c >> 1) & 1;
  r.ql = ld16_a2(row, blk + 64 * f + 32 * (j & 1) + 16 * h);
  r.qh = ld16_a2(row, blk + 128 + 32 * f + 16 * h);
  const uint32_t s_own = 8 * f + 2 * j + h;  // the partner's is s_own ^ 4
  r.sc_own = *reinterpret_cast<const int8_t*>(row + blk + 192 + s_own);
  r.sc_par = *reinterpret_cast<const int8_t*>(row + blk + 192 + (s_own ^ 4));
  r.d = ld_w2(row + blk + 208);
}
// q5_K super-block: header (16 B) | qh (32 B) | nibbles (128 B); every piece
// is 16-byte aligned (176 = 11 x 16).
__device__ __forceinline__ void load_unit(const uint8_t* row, int u, Raw<FQ5_K>& r) {
  const uint32_t blk = 176u * ((uint32_t)u >> 3);
  const uint32_t qoff = blk + 48 + 16 * ((uint32_t)u & 7);
  r.q = ld_w16(row + qoff);
  r.qh = ld_w16(row + blk + 16 + 16 * ((uint32_t)u & 1));
  r.hdr = ld_w16(row + blk);
}
__device__ __forceinline__ void load_unit(const uint8_t* row, int u, Raw<FIQ4_XS>& r) {
  const uint32_t blk = 136u * ((uint32_t)u >> 3);
  const uint32_t qoff = blk + 8 + 16 * ((uint32_t)u & 7);
  r.q = ld_w16(row + qoff);
  r.hdr = ld_w8(row + blk);
}

// Shared-header unit loads, for kernels whose lanes are all active and whose
// aligned lane quads always read units of one super-block (lane l takes
// units base + l + 64 i, K is a multiple of 256, and lanes past the end clamp
// together).  Each lane loads one dword of its super-block's header -- dword
// (l mod 4) of the 16 q4_K header bytes, dword (l mod 2) of the 8 IQ4_XS ones
// -- and the quad rebuilds the whole header with DPP broadcasts, so a wave
// moves a quarter of the header bytes through the L1 that per-lane 16-byte
// header loads would.
template <int F> struct RawS { Raw<F> r; };  // Q8_0: no header to share
template <> struct RawS<FQ4_K> {
  u32x4 q;
  uint32_t h;
};
template <> struct RawS<FIQ4_XS> {
  u32x4 q;
  uint32_t h;
};
template <> struct RawS<FQ5_K> {
  u32x4 q;
  uint32_t h;
  u32x4 qh;
};

__device__ __forceinline__ void load_unit_s(const uint8_t* row, int u, int lane, RawS<FQ8_0>& r) {
  load_unit(row, u, r.r);
}
__device__ __forceinline__ void load_unit_s(const uint8_t* row, int u, int lane, RawS<FQ6_K>& r) {
  load_unit(row, u, r.r);
}
__device__ __forceinline__ void load_unit_s(const uint8_t* row, int u, int lane, RawS<FQ8G128>& r) {
  load_unit(row, u, r.r);
}
__device__ __forceinline__ void load_unit_s(const uint8_t* row, int u, int lane, RawS<FQ4_K>& r) {
  const uint32_t blk = 144u * ((uint32_t)u >> 3);
  const uint32_t qoff = blk + 16 + 16 * ((uint32_t)u & 7);
  const uint32_t hoff = blk + 4 * ((uint32_t)lane & 3);
  r.q = ld_w16(row + qoff);
  r.h = *reinterpret_cast<const uint32_t*>(row + hoff);
}
__device__ __forceinline__ void load_unit_s(const uint8_t* row, int u, int lane, RawS<FQ5_K>& r) {
  const uint32_t blk = 176u * ((uint32_t)u >> 3);
  const uint32_t qoff = blk + 48 + 16 * ((uint32_t)u & 7);
  const uint32_t hoff = blk + 4 * ((uint32_t)lane & 3);
  r.q = ld_w16(row + qoff);
  r.qh = ld_w16(row + blk + 16 + 16 * ((uint32_t)u & 1));
  r.h = *reinterpret_cast<const uint32_t*>(row + hoff);
}
__device__ __forceinline__ void load_unit_s(const uint8_t* row, int u, int lane, RawS<FIQ4_XS>& r) {
  const uint32_t blk = 136u * ((uint32_t)u >> 3);
  const uint32_t qoff = blk + 8 + 16 * ((uint32_t)u & 7);
  const uint32_t hoff = blk + 4 * ((uint32_t)lane & 1);
  r.q = ld_w16(row + qoff);
  r.h = *reinterpret_cast<const uint32_t*>(row + hoff);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}

// quad_perm controls: broadcast lane k of each quad (k * 0x55), and the
// pairs [0,0,2,2] / [1,1,3,3]
__device__ __forceinline__ Raw<FQ4_K> expand(const RawS<FQ4_K>& s) {
  Raw<FQ4_K> r;
  r.q = s.q;
  r.hdr = u32x4{dpp_u<0x00>(s.h), dpp_u<0x55>(s.h), dpp_u<0xAA>(s.h), dpp_u<0xFF>(s.h)};
  return r;
}
__device__ __forceinline__ Raw<FQ5_K> expand(const RawS<FQ5_K>& s) {
  Raw<FQ5_K> r;
  r.q = s.q;
  r.qh = s.qh;
  r.hdr = u32x4{dpp_u<0x00>(s.h), dpp_u<0x55>(s.h), dpp_u<0xAA>(s.h), dpp_u<0xFF>(s.h)};
  return r;
}
__device__ __forceinline__ Raw<FIQ4_XS> expand(const RawS<FIQ4_XS>& s) {
  Raw<FIQ4_XS> r;
  r.q = s.q;
  r.hdr = u32x2{dpp_u<0xA0>(s.h), dpp_u<0xF5>(s.h)};
  return r;
}
__device__ __forceinline__ Raw<FQ8_0> expand(const RawS<FQ8_0>& s) { return s.r; }
__device__ __forceinline__ Raw<FQ6_K> expand(const RawS<FQ6_K>& s) { return s.r; }
__device__ __forceinline__ Raw<FQ8G128> expand(const RawS<FQ8G128>& s) { return s.r; }

// --------------------------------------------------------------- decoding
template <int F> struct Dec;

template <> struct Dec<FQ8_0> {
  uint32_t q[8];
  float d;
};
template <> struct Dec<FIQ4_XS> {
  uint32_t q[8];
  float d;
  int ls;     // effective sub-block scale, raw 6-bit value minus 32
  float dls;  // d * ls, exact in fp32 (11-bit times 6-bit significand)
};
__device__ __forceinline__ void decode_unit(const Raw<FQ8_0>& r, int, Dec<FQ8_0>& o) {
  const uint32_t w[9] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w, r.h};
  const uint32_t sh = r.odd ? 0u : 2u;
#pragma unroll
  for (int j = 0; j < 8; ++j) o.q[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], sh);
  o.d = half_bits_to_float(r.odd ? r.h : r.a.x);
}

// IQ4_XS non-linear codebook, index -> int8 value, packed four per dword.
constexpr uint32_t pk4(int a, int b, int c, int d) {
  return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
         ((uint32_t)(uint8_t)d << 24);
}
constexpr int8_t IQ4_CB[16] = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113};

// Codebook lookup of 4-bit indices (one per byte, 0..15) -> int8 values, four
// at a time with two byte permutes and an xor.
//
// v_perm_b32 maps a selector byte s to byte s of its 8-byte table for s < 8,
// and to a constant for s = 8..15: the sign of table byte 2 (s - 8) + 1
// replicated over the byte (s = 8..11), 0x00 (s = 12) or 0xFF (s = 13..15).
// An index i is looked up as s = i in table A and as s = i ^ 8 in table B.
// Exactly one of the two selectors is below 8, so the other permute returns
// one of those constants, which depends only on i and on the sign bits of the
// other table; each table entry is the codebook value xor the constant that
// the other table returns for the same index, so A ^ B is the value.  The
// tables depend on each other only through those sign bits, along chains of
// at most four entries, so four rounds of the assignment below reach its fixed
// point; the static_assert checks all sixteen indices against the codebook.
struct Iq4Tabs {
  uint8_t a[8], b[8];
};
constexpr uint8_t perm_byte(const uint8_t (&t)[8], int s) {
  return s < 8 ? t[s] : s >= 13 ? 0xFF : s == 12 ? 0x00 : (t[2 * (s - 8) + 1] & 0x80) ? 0xFF : 0x00;
}
constexpr Iq4Tabs iq4_tabs() {
  Iq4Tabs t{};
  for (int round = 0; round < 4; ++round)
    for (int k = 0; k < 8; ++k) {
      t.a[k] = static_cast<uint8_t>(IQ4_CB[k]) ^ perm_byte(t.b, k ^ 8);
      t.b[k] = static_cast<uint8_t>(IQ4_CB[k + 8]) ^ perm_byte(t.a, k + 8);
    }
  return t;
}
constexpr Iq4Tabs IQ4_T = iq4_tabs();
constexpr bool iq4_tabs_ok() {
  for (int i = 0; i < 16; ++i)
    if ((perm_byte(IQ4_T.a, i) ^ perm_byte(IQ4_T.b, i ^ 8)) != static_cast<uint8_t>(IQ4_CB[i])) return false;
  return true;
}
static_assert(iq4_tabs_ok(), "two-table IQ4_XS codebook lookup");
constexpr uint32_t tab_dw(const uint8_t (&t)[8], int h) {
  return pk4((int8_t)t[4 * h], (int8_t)t[4 * h + 1], (int8_t)t[4 * h + 2], (int8_t)t[4 * h + 3]);
}
constexpr uint32_t IQ4_A0 = tab_dw(IQ4_T.a, 0), IQ4_A1 = tab_dw(IQ4_T.a, 1);
constexpr uint32_t IQ4_B0 = tab_dw(IQ4_T.b, 0), IQ4_B1 = tab_dw(IQ4_T.b, 1);

// Four indices (s: one per byte, 0..15) -> their four codebook values.
__device__ __forceinline__ uint32_t iq4_lookup(uint32_t s) {
  return __builtin_amdgcn_perm(IQ4_A1, IQ4_A0, s) ^ __builtin_amdgcn_perm(IQ4_B1, IQ4_B0, s ^ 0x08080808u);
}

// Both nibbles of four index bytes -> the codebook values of the low nibbles
// (lo) and of the high nibbles (hi).
__device__ __forceinline__ void iq4_lookup2(uint32_t v, uint32_t& lo, uint32_t& hi) {
  lo = iq4_lookup(v & 0x0F0F0F0Fu);
  hi = iq4_lookup((v >> 4) & 0x0F0F0F0Fu);
}

__device__ __forceinline__ void decode_unit(const Raw<FIQ4_XS>& r, int u, Dec<FIQ4_XS>& o) {
  const uint32_t c = (uint32_t)u & 7;
  const uint32_t lo4 = __builtin_amdgcn_ubfe(r.hdr.y, 4 * c, 4);       // scales_l nibble
  const uint32_t hi2 = __builtin_amdgcn_ubfe(r.hdr.x, 16 + 2 * c, 2);  // scales_h bits
  o.ls = static_cast<int>(lo4 | (hi2 << 4)) - 32;
  o.d = half_bits_to_float(r.hdr.x);
  o.dls = o.d * static_cast<float>(o.ls);
  const uint32_t v[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    iq4_lookup2(v[i], o.q[i], o.q[4 + i]);
  }
}

// ----------------------------------------------------- activation fragments
// View of a Q8 activation buffer (structure of arrays, see qmv.h).
struct Act {
  const int8_t* qs;   // [rows][k]
  const float* d;     // [rows][k/32]
  const int32_t* s;   // [rows][k/32]
  int k, nb;
};

// ------------------------------------------------- own-block (paired) form
// How every kernel applies a unit to a token.  Unit u always meets the 32
// activations of 32-block u as its "own" block: for Q8_0 and IQ4_XS the unit
// is that block; for q4_K unit u = 8s + c holds half h = c & 1 of sub-blocks
// 2(c >> 1) and 2(c >> 1) + 1, and global sub-block u is one of those two
// (the low nibbles when h = 0, the high nibbles when h = 1).  So a unit needs
// one weight scale, and one activation scale per token.
//
// The eight weight dwords are split into a "first" and a "second" run of
// four.  For q4_K the first run holds the nibbles of the partner sub-block
// u ^ 1 (lane pairs hold units 2p, 2p+1, which share both sub-blocks) and the
// second the nibbles of the own one.  A token's integer dot is then: the
// first run against its activations, handed to the pair neighbour over DPP,
// which adds its second run on top -- so each lane ends with the complete
// 32-weight dot of its own sub-block, and a token costs eight v_dot4, one
// move and one fp32 scale step per unit.  Kernels that use the pair exchange
// keep both lanes of every pair active and on units 2p, 2p+1 of one row.
template <int F> struct DecO {
  uint32_t q[8];  // q[0..3] first run, q[4..7] second run
  float sc;       // Q8_0, q6_K: d; IQ4_XS: d * (ls - 32); q4_K, q5_K: d * sc of sub-block u
  float wm;       // q4_K, q5_K: dmin * m of sub-block u (0 otherwise)
  int isc, im;    // the integer scale (and q4_K / q5_K min) of the unit; q6_K: the
                  // int8 scale of the own run's 16 positions
  int iscp;       // q6_K: the int8 scale of the first run's 16 positions
};

// Decode unit u (clamped index) for lane parity h; invalid units get zero
// scales so that whatever they meet adds exactly nothing.  The fp32 scales are
// exact products (an 11-bit half significand times a 6-bit integer).
__device__ __forceinline__ void decode_own(const Raw<FQ8_0>& r, int u, int, bool ok, DecO<FQ8_0>& o) {
  Dec<FQ8_0> d;
  decode_unit(r, u, d);
#pragma unroll
  for (int i = 0; i < 8; ++i) o.q[i] = d.q[i];
  o.sc = ok ? d.d : 0.f;
  o.wm = 0.f;
  o.isc = 1;
  o.im = 0;
}
__device__ __forceinline__ void decode_own(const Raw<FIQ4_XS>& r, int u, int, bool ok, DecO<FIQ4_XS>& o) {
  Dec<FIQ4_XS> d;
  decode_unit(r, u, d);
#pragma unroll
  for (int i = 0; i < 8; ++i) o.q[i] = d.q[i];
  o.sc = ok ? d.dls : 0.f;
  o.wm = 0.f;
  o.isc = d.ls;
  o.im = 0;
}
__device__ __forceinline__ uint32_t bfe(uint32_t v, uint32_t off, uint32_t w) {
  return __builtin_amdgcn_ubfe(v, off, w);
}
// q4_K: the 6-bit (scale, min) of sub-block c of the super-block, one formula
// for both packings (no branch): the low 4 bits of the scale come from S[c]
// (c < 4) or S[c+4], of the min from S[c+4] or the high nibble of S[c+4]; the
// top 2 bits sit at bits 4-5 (c < 4) or 6-7 of S[c&3] and S[(c&3)+4].
template <int F>
__device__ __forceinline__ void decode_kmin_scales(const u32x4& hdr, int u, bool ok, DecO<F>& o) {
  const int c = u & 7;  // own sub-block inside the super-block
  const uint32_t jj = 8u * (uint32_t)(c & 3);
  const uint32_t hb = 2u * (uint32_t)(c >> 2);
  const uint32_t s03 = hdr.y, s47 = hdr.z, s811 = hdr.w;
  const uint32_t lo_sc = c < 4 ? s03 : s811;
  const uint32_t lo_m = c < 4 ? s47 : s811;
  const uint32_t sc = bfe(lo_sc, jj, 4) | (bfe(s03, jj + 4 + hb, 2) << 4);
  const uint32_t m = bfe(lo_m, jj + 2 * hb, 4) | (bfe(s47, jj + 4 + hb, 2) << 4);
  const float ws = half_bits_to_float(hdr.x) * static_cast<float>(sc);
  const float wm = half_bits_to_float(hdr.x >> 16) * static_cast<float>(m);
  o.sc = ok ? ws : 0.f;
  o.wm = ok ? wm : 0.f;
  o.isc = static_cast<int>(sc);
  o.im = static_cast<int>(m);
}
// q5_K: the q4_K scales and nibbles, each weight's fifth bit from its qh byte
// (bit j of the byte for sub-block j of the super-block).  As for q4_K, h = 0
// makes the low nibbles (sub-block j0) the own run, h = 1 the high ones.
__device__ __forceinline__ void decode_own(const Raw<FQ5_K>& r, int u, int h, bool ok, DecO<FQ5_K>& o) {
  decode_kmin_scales(r.hdr, u, ok, o);
  const uint32_t j0 = 2u * (((uint32_t)u & 7) >> 1);  // low-nibble sub-block of the unit
  const uint32_t sh_own = 4u * (uint32_t)h, sh_par = 4u - sh_own;
  const uint32_t b_own = j0 + (uint32_t)h, b_par = j0 + 1u - (uint32_t)h;
  const uint32_t v[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
  const uint32_t hv[4] = {r.qh.x, r.qh.y, r.qh.z, r.qh.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.q[i] = ((v[i] >> sh_par) & 0x0F0F0F0Fu) | (((hv[i] >> b_par) & 0x01010101u) << 4);
    o.q[4 + i] = ((v[i] >> sh_own) & 0x0F0F0F0Fu) | (((hv[i] >> b_own) & 0x01010101u) << 4);
  }
}
__device__ __forceinline__ void decode_own(const Raw<FQ4_K>& r, int u, int h, bool ok, DecO<FQ4_K>& o) {
  decode_kmin_scales(r.hdr, u, ok, o);
  // h = 0: own = low nibbles, partner = high; h = 1 the other way round
  const uint32_t sh_own = 4u * (uint32_t)h, sh_par = 4u - sh_own;
  const uint32_t v[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.q[i] = (v[i] >> sh_par) & 0x0F0F0F0Fu;
    o.q[4 + i] = (v[i] >> sh_own) & 0x0F0F0F0Fu;
  }
}
__device__ __forceinline__ void decode_own(const Raw<FQ8G128>& r, int, int, bool ok, DecO<FQ8G128>& o) {
  const uint32_t w[9] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w, r.h};
  const uint32_t sh = r.odd ? 0u : 2u;
#pragma unroll
  for (int j = 0; j < 8; ++j) o.q[j] = __builtin_amdgcn_alignbyte(w[j + 1], w[j], sh);
  o.sc = ok ? half_bits_to_float(r.d) : 0.f;
  o.wm = 0.f;
  o.isc = 1;
  o.im = 0;
}
// q6_K: the stored 6-bit values of both runs (nibble plus two qh bits, the
// quarter's bits 2j..2j+1), minus 32 byte by byte as (v + 96) ^ 128 (no
// carry leaves a byte: v + 96 <= 159), so each byte is the signed value
// q - 32 in -32..31.  The int8 scales multiply the two runs' dots.
__device__ __forceinline__ uint32_t q6_byte_values(uint32_t ql, uint32_t qh, uint32_t nsh, uint32_t hsh) {
  const uint32_t v = ((ql >> nsh) & 0x0F0F0F0Fu) | (((qh >> hsh) & 0x03030303u) << 4);
  return (v + 0x60606060u) ^ 0x80808080u;
}
__device__ __forceinline__ void decode_own(const Raw<FQ6_K>& r, int u, int, bool ok, DecO<FQ6_K>& o) {
  const uint32_t j = (uint32_t)u & 3, jp = j ^ 2;
  const uint32_t ql[4] = {r.ql.x, r.ql.y, r.ql.z, r.ql.w};
  const uint32_t qh[4] = {r.qh.x, r.qh.y, r.qh.z, r.qh.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.q[i] = q6_byte_values(ql[i], qh[i], 4 * (jp >> 1), 2 * jp);
    o.q[4 + i] = q6_byte_values(ql[i], qh[i], 4 * (j >> 1), 2 * j);
  }
  o.sc = ok ? half_bits_to_float(r.d) : 0.f;
  o.wm = 0.f;
  o.isc = r.sc_own;
  o.iscp = r.sc_par;
  o.im = 0;
}
template <int F>
__device__ __forceinline__ void decode_own(const RawS<F>& s, int u, int h, bool ok, DecO<F>& o) {
  decode_own(expand(s), u, h, ok, o);
}

// The activation runs of unit u for one token and the (d, d*s) pair of its
// own 32-block, from a Q8 activation buffer in the library layout (global
// memory or an LDS copy of it).
struct XO {
  u32x4 f, s;
  float2 p;
};
template <int F>
__device__ __forceinline__ void load_xo(const Act& x, int row, int u, XO& o) {
  const int8_t* base = x.qs + (int64_t)row * x.k;
  const int64_t i = (int64_t)row * x.nb + u;
  if constexpr (kmin<F>()) {
    const int h = u & 1;
    o.f = ld16(base + 32 * (u ^ 1) + 16 * h);
    o.s = ld16(base + 32 * u + 16 * h);
    const float d = x.d[i];
    o.p = make_float2(d, d * static_cast<float>(x.s[i]));
  } else if constexpr (F == FQ6_K) {
    const int h = (u >> 1) & 1;
    o.f = ld16(base + 32 * (u ^ 2) + 16 * h);
    o.s = ld16(base + 32 * u + 16 * h);
    o.p = make_float2(x.d[i], 0.f);
  } else {
    o.f = ld16(base + 32 * u);
    o.s = ld16(base + 32 * u + 16);
    o.p = make_float2(x.d[i], 0.f);
  }
}

// Exact integer dot of the own 32-block against one token's activation runs
// (xf meets q[0..3], xs meets q[4..7]), in two steps so that a caller can
// interleave rows: own_first gives the first run's dot, which the caller
// hands through own_pass (the DPP move between pair lanes for q4_K) to
// own_second.
template <int F>
__device__ __forceinline__ int own_first(const DecO<F>& w, const u32x4& xf) {
  int a = 0;
  a = dot4(w.q[0], xf.x, a);
  a = dot4(w.q[1], xf.y, a);
  a = dot4(w.q[2], xf.z, a);
  a = dot4(w.q[3], xf.w, a);
  if constexpr (F == FQ6_K) a *= w.iscp;  // the partner's half, scaled for it
  return a;
}
template <int F>
__device__ __forceinline__ int own_pass(int a) {
  if constexpr (pair_xor<F>() == 1) return dpp_i<DPP_XOR1>(a);  // partner's part of the own block
  if constexpr (pair_xor<F>() == 2) return dpp_i<DPP_XOR2>(a);
  return a;
}
template <int F>
__device__ __forceinline__ int own_second(const DecO<F>& w, const u32x4& xs, int a) {
  if constexpr (F == FQ6_K) {
    int b = 0;
    b = dot4(w.q[4], xs.x, b);
    b = dot4(w.q[5], xs.y, b);
    b = dot4(w.q[6], xs.z, b);
    b = dot4(w.q[7], xs.w, b);
    return a + b * w.isc;
  }
  a = dot4(w.q[4], xs.x, a);
  a = dot4(w.q[5], xs.y, a);
  a = dot4(w.q[6], xs.z, a);
  return dot4(w.q[7], xs.w, a);
}

// acc += d_x * (w.sc * A - w.wm * s_x), with p = (d_x, d_x * s_x).
template <int F>
__device__ __forceinline__ float own_apply(const DecO<F>& w, int dotv, float2 p, float acc) {
  acc = fmaf(static_cast<float>(dotv), p.x * w.sc, acc);
  if constexpr (kmin<F>()) acc = fmaf(-w.wm, p.y, acc);
  return acc;
}

// Where the activation runs of unit u (32-block u) come from, as 16-byte
// pieces (block b, half hb) of a token's quants: Q8_0 / IQ4_XS take (u, 0)
// then (u, 1); q4_K and q5_K take (u ^ 1, u & 1) then (u, u & 1); q6_K takes
// (u ^ 2, h) then (u, h) with h = (u >> 1) & 1.  Inverted for staging: piece
// (b, hb) is the second run of unit b if hb matches the format's rule, else
// the first run of unit b ^ 1 (q4_K, q5_K), b ^ 2 (q6_K) or b (others).
template <int F>
__device__ __forceinline__ void own_piece_slot(int b, int hb, int& unit, int& run) {
  if constexpr (kmin<F>()) {
    const bool second = hb == (b & 1);
    unit = second ? b : (b ^ 1);
    run = second ? 1 : 0;
  } else if constexpr (F == FQ6_K) {  // unit b holds positions ((b >> 1) & 1) of b and b ^ 2
    const bool second = hb == ((b >> 1) & 1);
    unit = second ? b : (b ^ 2);
    run = second ? 1 : 0;
  } else {
    unit = b;
    run = hb;
  }
}

// Division of small non-negative ints by a divisor fixed for a loop:
// q = umulhi(n, ceil(2^32 / d)), exact whenever n * d < 2^32 (here n and d
// stay below 2^16).  Saves the long integer division sequence per element.
struct FastDiv {
  uint32_t d, m;
  __device__ explicit FastDiv(int dv) : d((uint32_t)dv), m(dv > 1 ? 0xFFFFFFFFu / (uint32_t)dv + 1u : 0u) {}
  __device__ int div(int n) const { return d == 1u ? n : (int)__umulhi((uint32_t)n, m); }
};

// ------------------------------------------------------------- reductions
// Sum over the LPR consecutive lanes of a lane group (LPR a power of two).
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over each aligned group of 8 lanes; every lane of the group gets it.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<DPP_XOR1>(v);
  v += dpp_f<DPP_XOR2>(v);
  return v + dpp_f<DPP_HALF_MIRROR>(v);
}
__device__ __forceinline__ int sum8(int v) {
  v += dpp_i<DPP_XOR1>(v);
  v += dpp_i<DPP_XOR2>(v);
  return v + dpp_i<DPP_HALF_MIRROR>(v);
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f<DPP_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_XOR2>(v));
  return fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
}

// Sum over the LPR consecutive lanes of a lane group (LPR 8, 16, 32 or 64,
// every lane active); every lane of the group gets the result.
template <int LPR>
__device__ __forceinline__ float lane_group_sum(float v) {
  v = sum8(v);
  if constexpr (LPR >= 16) v += dpp_f<DPP_MIRROR>(v);  // 16-lane row sums
  if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (LPR == 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Sum over all 64 lanes of a wave (every lane active): row sums with DPP,
// then the four row sums through scalar registers.  Wave-uniform result.
__device__ __forceinline__ float wave_sum(float v) {
  v = sum8(v);
  v += dpp_f<DPP_MIRROR>(v);
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// ----------------------------------------------------- activation quantizer
// One Q8 activation block of 32 values held by an aligned group of 8 lanes,
// four values per lane (Castagna Veloce page, "Fused operations"): amax and
// the quant sum are 8-lane DPP reductions; d = amax / 127 and x / d are IEEE
// fp32 divisions (the library is built without fast-math) and roundf rounds
// halfway cases away from zero.  Returns the lane's four quants packed into a
// dword; every lane of the group gets d and the sum.
__device__ __forceinline__ uint32_t q8_block8(const float (&vv)[4], float& db, int& sum) {
  float amax = fmaxf(fmaxf(fabsf(vv[0]), fabsf(vv[1])), fmaxf(fabsf(vv[2]), fabsf(vv[3])));
  amax = max8(amax);
  db = amax / 127.0f;
  int q[4] = {0, 0, 0, 0};
  if (amax != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = static_cast<int>(roundf(vv[i] / db));
      q[i] = r > 127 ? 127 : (r < -127 ? -127 : r);
    }
  }
  sum = sum8(q[0] + q[1] + q[2] + q[3]);
  return (uint32_t)(q[0] & 255) | ((uint32_t)(q[1] & 255) << 8) | ((uint32_t)(q[2] & 255) << 16) |
         ((uint32_t)(q[3] & 255) << 24);
}

}  // namespace qmv
