"""Seeded synthetic inputs for the quantized decode matvec path.

This module only draws random fields and packs them into the GGUF block byte
layouts; it holds none of the method's arithmetic (no activation quantization,
no dequantization, no dot products).  Both the CPU oracle and the HIP path
consume exactly the bytes and float arrays made here.

Random numbers
--------------
Counter-based SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), with the output function of Vigna's
public-domain splitmix64 ("Stafford mix 13"):

    draw i of stream k  =  mix(key_k + (i + 1) * GAMMA)
    key_k               =  mix(seed XOR fnv1a64(stream name))

Every value is a pure function of (seed, stream name, index), so any row range
of any tensor can be generated on its own and gives the same bytes as a full
generation.

Derived draws
  * uniform integer in [a, b] (ranges < 2**32): one 32-bit half of a draw each,
    low half first, mapped by multiply-shift a + ((u32 * (b - a + 1)) >> 32);
  * 4-bit fields: sixteen nibbles per draw, nibble j = bits 4j..4j+3;
  * uniform double in [0, 1): (u >> 11) * 2**-53;
  * N(0, 1): Box-Muller, z = sqrt(-2 ln(1 - U1)) cos(2 pi U2) in fp64 from draws
    2i and 2i+1, rounded to fp32;
  * fp16 scale: fp64 uniform in [lo, hi] rounded to nearest-even binary16.

Block byte layouts (GGUF block formats; the pages name them but print no
layout, so this is the plain GGUF reading)
  Q8_0   34 B / 32 weights : fp16 d | int8 q[32]
  q4_K  144 B / 256 weights: fp16 d | fp16 dmin | 12 B packed 6-bit (scale, min)
                             x 8 | 128 B nibbles (64-weight chunk c uses bytes
                             32c..32c+31: low nibble -> weight 64c+i, high
                             nibble -> weight 64c+32+i)
  IQ4_XS 136 B / 256 weights: fp16 d | u16 scales_h | u8 scales_l[4] | 128 B
                             nibbles (sub-block j uses bytes 16j..16j+15: low
                             nibble -> weight 32j+i, high -> weight 32j+16+i)
  q5_K  176 B / 256 weights: the q4_K header (16 B) | 32 B qh | 128 B nibbles
                             in the q4_K order; the fifth bit (value 16) of
                             weight 64c+i is bit 2c of qh[i], of weight
                             64c+32+i bit 2c+1 of qh[i]
  Q8G128 130 B / 128 weights: fp16 d | int8 q[128] (int8 groups of 128 with
                             one scale: the LM-head format the zhuai.tech page
                             names; this layout is the Q8_0 one with 128-weight
                             groups)
  q6_K  210 B / 256 weights: 128 B ql | 64 B qh | int8 scales[16] | fp16 d;
                             weight 128h + 32j + l (half h, quarter j, l < 32)
                             is the nibble of ql[64h + 32(j & 1) + l] (low for
                             j < 2, high otherwise) plus 16 x bits 2j..2j+1 of
                             qh[32h + l], minus 32, times scales[8h + 2j + l/16]
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Q8_0", "Q4_K", "IQ4_XS", "FMT_NAMES", "BLOCK_WEIGHTS", "BLOCK_BYTES",
    "row_bytes", "Stream", "stream", "draw_u64", "uniform01", "randint",
    "nibbles", "normal_f32", "scale_f16",
    "pack_q8_0", "pack_q4_k", "pack_iq4_xs", "pack_q5_k", "pack_q6_k", "pack_q8g128", "Q5_K", "Q6_K", "Q8G128",
    "WeightFields", "make_weights", "make_x", "make_routing",
    "CONFIGS", "config",
]

# format ids, shared by convention with the C interfaces
Q8_0, Q4_K, IQ4_XS, Q5_K, Q6_K, Q8G128 = 0, 1, 2, 3, 4, 5
FMT_NAMES = {Q8_0: "q8_0", Q4_K: "q4_K", IQ4_XS: "iq4_xs", Q5_K: "q5_K", Q6_K: "q6_K", Q8G128: "q8g128"}
BLOCK_WEIGHTS = {Q8_0: 32, Q4_K: 256, IQ4_XS: 256, Q5_K: 256, Q6_K: 256, Q8G128: 128}
BLOCK_BYTES = {Q8_0: 34, Q4_K: 144, IQ4_XS: 136, Q5_K: 176, Q6_K: 210, Q8G128: 130}


def row_bytes(fmt: int, k: int) -> int:
    qk = BLOCK_WEIGHTS[fmt]
    if k % qk:
        raise ValueError(f"K={k} is not a multiple of the {FMT_NAMES[fmt]} block ({qk})")
    return (k // qk) * BLOCK_BYTES[fmt]


# --------------------------------------------------------------------------- RNG
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix_inplace(z: np.ndarray) -> np.ndarray:
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def _mix_scalar(v: int) -> int:
    return int(_mix_inplace(np.array([v], dtype=np.uint64))[0])


def _fnv1a64(s: str) -> int:
    h = 0xCBF29CE484222325
    for b in s.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


@dataclass(frozen=True)
class Stream:
    name: str
    seed: int = 0
    key: int = field(init=False)

    def __post_init__(self):
        object.__setattr__(self, "key", _mix_scalar((self.seed ^ _fnv1a64(self.name)) & 0xFFFFFFFFFFFFFFFF))


def stream(name: str, seed: int = 0) -> Stream:
    return Stream(name, seed)


def draw_u64(st: Stream, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of a stream as uint64."""
    out = np.empty(count, dtype=np.uint64)
    key = np.uint64(st.key)
    for c0 in range(0, count, _CHUNK):
        c1 = min(count, c0 + _CHUNK)
        z = np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64)
        z *= _GAMMA
        z += key
        out[c0:c1] = _mix_inplace(z)
    return out


def uniform01(st: Stream, start: int, count: int) -> np.ndarray:
    u = draw_u64(st, start, count)
    return (u >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def randint(st: Stream, start: int, count: int, lo: int, hi: int) -> np.ndarray:
    """Uniform integers in [lo, hi] for elements start..start+count-1 (int64)."""
    n_range = hi - lo + 1
    assert 0 < n_range < (1 << 32)
    d0, d1 = start // 2, (start + count + 1) // 2
    u = draw_u64(st, d0, d1 - d0)
    halves = np.empty(2 * u.size, dtype=np.uint64)
    halves[0::2] = u & np.uint64(0xFFFFFFFF)
    halves[1::2] = u >> np.uint64(32)
    off = start - 2 * d0
    h = halves[off:off + count]
    return lo + ((h * np.uint64(n_range)) >> np.uint64(32)).astype(np.int64)


def nibbles(st: Stream, start: int, count: int) -> np.ndarray:
    """Uniform 4-bit values for elements start..start+count-1 (uint8)."""
    d0, d1 = start // 16, (start + count + 15) // 16
    u = draw_u64(st, d0, d1 - d0)
    shifts = (np.arange(16, dtype=np.uint64) * np.uint64(4))[None, :]
    v = ((u[:, None] >> shifts) & np.uint64(15)).astype(np.uint8).reshape(-1)
    off = start - 16 * d0
    return v[off:off + count]


def normal_f32(st: Stream, start: int, count: int) -> np.ndarray:
    u = uniform01(st, 2 * start, 2 * count)
    u1, u2 = u[0::2], u[1::2]
    z = np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * math.pi * u2)
    return z.astype(np.float32)


def scale_f16(st: Stream, start: int, count: int, lo: float = 1e-3, hi: float = 1e-2) -> np.ndarray:
    u = uniform01(st, start, count)
    return (lo + (hi - lo) * u).astype(np.float16)


# ----------------------------------------------------------------------- packing
def pack_q8_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """d fp16 [N][K/32], q int8 [N][K] -> bytes [N][K/32*34]."""
    n, k = q.shape
    nb = k // 32
    out = np.empty((n, nb, 34), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(d, dtype=np.float16).view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:34] = q.astype(np.int8).view(np.uint8).reshape(n, nb, 32)
    return out.reshape(n, nb * 34)


def q4_k_header(d, dmin, sc, m) -> np.ndarray:
    """First 16 bytes of each q4_K super-block: fp16 d, fp16 dmin, 12 bytes of
    packed 6-bit (scale, min) pairs.  d, dmin [N][S]; sc, m [N][S][8]."""
    n, ns = np.shape(d)
    sc = np.asarray(sc).astype(np.uint8)
    m = np.asarray(m).astype(np.uint8)
    out = np.zeros((n, ns, 16), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(d, dtype=np.float16).view(np.uint8).reshape(n, ns, 2)
    out[:, :, 2:4] = np.ascontiguousarray(dmin, dtype=np.float16).view(np.uint8).reshape(n, ns, 2)
    s = np.zeros((n, ns, 12), dtype=np.uint8)
    s[:, :, 0:4] = sc[:, :, 0:4] & 63
    s[:, :, 4:8] = m[:, :, 0:4] & 63
    s[:, :, 8:12] = (sc[:, :, 4:8] & 15) | ((m[:, :, 4:8] & 15) << 4)
    s[:, :, 0:4] |= (sc[:, :, 4:8] >> 4) << 6
    s[:, :, 4:8] |= (m[:, :, 4:8] >> 4) << 6
    out[:, :, 4:16] = s
    return out


def pack_q4_k(d, dmin, sc, m, q) -> np.ndarray:
    """d, dmin fp16 [N][S]; sc, m uint8 [N][S][8] in 0..63; q uint8 [N][K] in 0..15."""
    n, k = q.shape
    ns = k // 256
    out = np.zeros((n, ns, 144), dtype=np.uint8)
    out[:, :, 0:16] = q4_k_header(d, dmin, sc, m)
    qq = q.astype(np.uint8).reshape(n, ns, 4, 2, 32)  # chunk c, half h, i
    out[:, :, 16:144] = (qq[:, :, :, 0, :] | (qq[:, :, :, 1, :] << 4)).reshape(n, ns, 128)
    return out.reshape(n, ns * 144)


def pack_q5_k(d, dmin, sc, m, q) -> np.ndarray:
    """d, dmin fp16 [N][S]; sc, m uint8 [N][S][8] in 0..63; q uint8 [N][K] in 0..31."""
    n, k = q.shape
    ns = k // 256
    out = np.zeros((n, ns, 176), dtype=np.uint8)
    out[:, :, 0:16] = q4_k_header(d, dmin, sc, m)
    qq = q.astype(np.uint8).reshape(n, ns, 4, 2, 32)  # chunk c, half h, i
    hi = (qq >> 4) & 1
    qh = np.zeros((n, ns, 32), dtype=np.uint8)
    for c in range(4):
        qh |= hi[:, :, c, 0, :] << (2 * c)
        qh |= hi[:, :, c, 1, :] << (2 * c + 1)
    out[:, :, 16:48] = qh
    lo = qq & 15
    out[:, :, 48:176] = (lo[:, :, :, 0, :] | (lo[:, :, :, 1, :] << 4)).reshape(n, ns, 128)
    return out.reshape(n, ns * 176)


def pack_q8g128(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """d fp16 [N][K/128], q int8 [N][K] -> bytes [N][K/128*130]."""
    n, k = q.shape
    ng = k // 128
    out = np.empty((n, ng, 130), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(d, dtype=np.float16).view(np.uint8).reshape(n, ng, 2)
    out[:, :, 2:130] = q.astype(np.int8).view(np.uint8).reshape(n, ng, 128)
    return out.reshape(n, ng * 130)


def pack_q6_k(d, sc, q) -> np.ndarray:
    """d fp16 [N][S]; sc int8 [N][S][16] (one scale per 16 weights); q uint8
    [N][K] in 0..63 (the stored 6-bit value; the weight is sc * (q - 32))."""
    n, k = q.shape
    ns = k // 256
    out = np.zeros((n, ns, 210), dtype=np.uint8)
    qq = q.astype(np.uint8).reshape(n, ns, 2, 4, 32)  # half h, quarter j, l
    lo, hi2 = qq & 15, qq >> 4
    ql = np.zeros((n, ns, 2, 2, 32), dtype=np.uint8)  # half, ql run (j & 1), l
    for j in range(4):
        ql[:, :, :, j & 1, :] |= lo[:, :, :, j, :] << (4 * (j >> 1))
    out[:, :, 0:128] = ql.reshape(n, ns, 128)
    qh = np.zeros((n, ns, 2, 32), dtype=np.uint8)
    for j in range(4):
        qh |= hi2[:, :, :, j, :] << (2 * j)
    out[:, :, 128:192] = qh.reshape(n, ns, 64)
    out[:, :, 192:208] = np.asarray(sc).astype(np.int8).view(np.uint8).reshape(n, ns, 16)
    out[:, :, 208:210] = np.ascontiguousarray(d, dtype=np.float16).view(np.uint8).reshape(n, ns, 2)
    return out.reshape(n, ns * 210)


def iq4_xs_header(d, ls) -> np.ndarray:
    """First 8 bytes of each IQ4_XS super-block: fp16 d, u16 scales_h (two
    high bits per sub-block), scales_l[4] (low nibbles).  ls [N][S][8] raw."""
    n, ns = np.shape(d)
    ls = np.asarray(ls).astype(np.uint16)
    out = np.zeros((n, ns, 8), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(d, dtype=np.float16).view(np.uint8).reshape(n, ns, 2)
    sh = np.zeros((n, ns), dtype=np.uint16)
    for j in range(8):
        sh |= ((ls[:, :, j] >> 4) & 3) << (2 * j)
    out[:, :, 2] = (sh & 0xFF).astype(np.uint8)
    out[:, :, 3] = (sh >> 8).astype(np.uint8)
    lo = (ls & 15).astype(np.uint8)
    out[:, :, 4:8] = lo[:, :, 0::2] | (lo[:, :, 1::2] << 4)
    return out


def pack_iq4_xs(d, ls, idx) -> np.ndarray:
    """d fp16 [N][S]; ls uint8 [N][S][8] raw 6-bit scales; idx uint8 [N][K] in 0..15."""
    n, k = idx.shape
    ns = k // 256
    out = np.zeros((n, ns, 136), dtype=np.uint8)
    out[:, :, 0:8] = iq4_xs_header(d, ls)
    qq = idx.astype(np.uint8).reshape(n, ns, 8, 2, 16)  # sub-block j, half h, i
    out[:, :, 8:136] = (qq[:, :, :, 0, :] | (qq[:, :, :, 1, :] << 4)).reshape(n, ns, 128)
    return out.reshape(n, ns * 136)


# ------------------------------------------------------------------ weights / x
@dataclass
class WeightFields:
    """Drawn fields of a row range (kept for the format tests), plus packed bytes."""
    fmt: int
    rows: tuple
    k: int
    data: np.ndarray                    # uint8 [rows][row_bytes]
    d: np.ndarray | None = None         # fp16 scales
    dmin: np.ndarray | None = None      # fp16 (q4_K)
    sc: np.ndarray | None = None        # 6-bit scales (q4_K, q5_K) / raw ls (IQ4_XS) / int8 (q6_K)
    m: np.ndarray | None = None         # 6-bit mins (q4_K, q5_K)
    q: np.ndarray | None = None         # int8 (Q8_0) / nibbles (q4_K, IQ4_XS) / 5-bit (q5_K) / 6-bit (q6_K)


def make_weights(fmt: int, n_rows: int, k: int, name: str, seed: int = 0,
                 rows: tuple | None = None, keep_fields: bool = False,
                 q8_range=(-127, 127), scale_range=(1e-3, 1e-2)) -> WeightFields:
    """Weights of an n_rows x k matrix (rows r0..r1-1 only if `rows` is given).

    Q8_0  : d ~ fp16 U[1e-3,1e-2], q ~ U{-127..127}
    Q8G128: as Q8_0, one d per 128 weights
    q4_K  : d, dmin ~ fp16 U[1e-3,1e-2], scale and min ~ U{0..63}, q ~ U{0..15}
    IQ4_XS: d ~ fp16 U[1e-3,1e-2], raw 6-bit scale ~ U{0..63}, index ~ U{0..15}
    q5_K  : as q4_K with q ~ U{0..31}
    q6_K  : d ~ fp16 U[1e-3,1e-2], int8 scale per 16 weights ~ U{-127..127},
            stored 6-bit q ~ U{0..63}
    """
    r0, r1 = rows if rows is not None else (0, n_rows)
    assert 0 <= r0 <= r1 <= n_rows
    n = r1 - r0
    row_bytes(fmt, k)  # validates k
    lo, hi = scale_range
    if fmt in (Q8_0, Q8G128):
        nb = k // BLOCK_WEIGHTS[fmt]
        d = scale_f16(stream(name + "/d", seed), r0 * nb, n * nb, lo, hi).reshape(n, nb)
        q = randint(stream(name + "/q", seed), r0 * k, n * k, *q8_range).astype(np.int8).reshape(n, k)
        data = (pack_q8_0 if fmt == Q8_0 else pack_q8g128)(d, q)
        wf = WeightFields(fmt, (r0, r1), k, data)
        if keep_fields:
            wf.d, wf.q = d, q
        return wf
    ns = k // 256
    d = scale_f16(stream(name + "/d", seed), r0 * ns, n * ns, lo, hi).reshape(n, ns)
    if fmt == Q6_K:
        q = randint(stream(name + "/q", seed), r0 * k, n * k, 0, 63).astype(np.uint8).reshape(n, k)
        sc = randint(stream(name + "/sc", seed), r0 * ns * 16, n * ns * 16, -127, 127).astype(np.int8).reshape(n, ns, 16)
        data = pack_q6_k(d, sc, q)
        wf = WeightFields(fmt, (r0, r1), k, data)
        if keep_fields:
            wf.d, wf.sc, wf.q = d, sc, q
        return wf
    if fmt == Q5_K:
        q = randint(stream(name + "/q", seed), r0 * k, n * k, 0, 31).astype(np.uint8).reshape(n, k)
    else:
        q = nibbles(stream(name + "/q", seed), r0 * k, n * k).reshape(n, k)
    if fmt in (Q4_K, Q5_K):
        dmin = scale_f16(stream(name + "/dmin", seed), r0 * ns, n * ns, lo, hi).reshape(n, ns)
        sc = randint(stream(name + "/sc", seed), r0 * ns * 8, n * ns * 8, 0, 63).astype(np.uint8).reshape(n, ns, 8)
        m = randint(stream(name + "/m", seed), r0 * ns * 8, n * ns * 8, 0, 63).astype(np.uint8).reshape(n, ns, 8)
        data = (pack_q4_k if fmt == Q4_K else pack_q5_k)(d, dmin, sc, m, q)
        wf = WeightFields(fmt, (r0, r1), k, data)
        if keep_fields:
            wf.d, wf.dmin, wf.sc, wf.m, wf.q = d, dmin, sc, m, q
        return wf
    if fmt == IQ4_XS:
        ls = randint(stream(name + "/ls", seed), r0 * ns * 8, n * ns * 8, 0, 63).astype(np.uint8).reshape(n, ns, 8)
        data = pack_iq4_xs(d, ls, q)
        wf = WeightFields(fmt, (r0, r1), k, data)
        if keep_fields:
            wf.d, wf.sc, wf.q = d, ls, q
        return wf
    raise ValueError(f"unknown format {fmt}")


def make_x(n_tok: int, k: int, name: str, seed: int = 0) -> np.ndarray:
    """fp32 activations [n_tok][k] ~ N(0,1); token t is the same for every n_tok."""
    return normal_f32(stream(name, seed), 0, n_tok * k).reshape(n_tok, k)


def make_routing(n_tok: int, n_experts: int, top_k: int, name: str, seed: int = 0):
    """Per-token top-k expert ids (distinct, uniform: partial Fisher-Yates) and
    route weights (softmax over top_k N(0,1) draws, fp64 then fp32)."""
    u = uniform01(stream(name + "/ids", seed), 0, n_tok * top_k).reshape(n_tok, top_k)
    ids = np.empty((n_tok, top_k), dtype=np.int32)
    for t in range(n_tok):
        perm = list(range(n_experts))
        for s in range(top_k):
            j = s + int(u[t, s] * (n_experts - s))
            perm[s], perm[j] = perm[j], perm[s]
            ids[t, s] = perm[s]
    g = normal_f32(stream(name + "/rw", seed), 0, n_tok * top_k).reshape(n_tok, top_k).astype(np.float64)
    g = np.exp(g - g.max(axis=1, keepdims=True))
    rw = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, rw


# ----------------------------------------------------------------- workloads
CONFIGS = {
    # dense single-token Q8_0 matvec
    "q8_0_4096x4096": dict(fmt=Q8_0, n=4096, k=4096, tokens=(1,)),
    # q4_K FFN-up shaped matvec, decode/verify batches
    "q4_k_14336x4096": dict(fmt=Q4_K, n=14336, k=4096, tokens=(1, 2, 4, 8, 16)),
    # IQ4_XS down projection
    "iq4_xs_4096x14336": dict(fmt=IQ4_XS, n=4096, k=14336, tokens=(1, 2, 4, 8, 16)),
    # MoE: 128 experts, gate+up 2x1536 rows over K=4096, down 4096 rows over K=1536
    "moe_iq4_xs_e128": dict(fmt=IQ4_XS, n_experts=128, top_k=8, gate_up=(3072, 4096),
                            down=(4096, 1536), tokens=(1, 6, 16, 64)),
    # few-row long-K Q8_0 (split-K path)
    "q8_0_splitk_256x65536": dict(fmt=Q8_0, n=256, k=65536, tokens=(1,)),
    # Q8_0 output head
    "q8_0_head_152064x5120": dict(fmt=Q8_0, n=152064, k=5120, tokens=(1, 2, 4, 8, 16)),
    # q5_K at the q4_K FFN-up shape (a further K-quant of the same small-batch
    # matvecs; no workload of its own)
    "q5_k_14336x4096": dict(fmt=Q5_K, n=14336, k=4096, tokens=(1, 2, 4, 8, 16)),
    "q6_k_14336x4096": dict(fmt=Q6_K, n=14336, k=4096, tokens=(1, 2, 4, 8, 16)),
    # the output head in the int8 group-of-128 format
    "q8g128_head_152064x5120": dict(fmt=Q8G128, n=152064, k=5120, tokens=(1, 2, 4, 8, 16)),
}


def config(name: str) -> dict:
    return dict(CONFIGS[name], name=name)
