"""Torch implementation of the seeded generator, for inputs too large to draw
in numpy in reasonable time (the 152064 x 5120 output head is 827 MB).

It computes the same counter-based SplitMix64 values as ``synth`` (module
docstring there), with int64 tensors standing in for uint64: products wrap
modulo 2**64 and right shifts are masked to act as logical shifts, so every
byte equals the numpy generator's.  The quantized fields (the bulk of the
bytes) are drawn here, on any torch device; the per-block fp16 scales and
6-bit fields come from the numpy functions (they are small, and numpy rounds
fp64 to fp16 in one step).  Holds no arithmetic of the matvec method.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (BLOCK_BYTES, BLOCK_WEIGHTS, IQ4_XS, Q4_K, Q5_K, Q6_K, Q8_0, Q8G128, _GAMMA, _M1, _M2, Stream,
               iq4_xs_header, pack_q6_k, q4_k_header, randint, row_bytes, scale_f16, stream)

__all__ = ["draw_u64", "randint_t", "nibbles_t", "make_weights_t"]

_MASK64 = (1 << 64) - 1


def _s64(v: int) -> int:
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


_G, _C1, _C2 = _s64(int(_GAMMA)), _s64(int(_M1)), _s64(int(_M2))


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = z ^ _lsr(z, 30)
    z = z * _C1
    z = z ^ _lsr(z, 27)
    z = z * _C2
    return z ^ _lsr(z, 31)


def draw_u64(st: Stream, start: int, count: int, device) -> torch.Tensor:
    """Draws start..start+count-1 as int64 tensors holding the uint64 bits."""
    z = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    return _mix(z * _G + _s64(st.key))


def randint_t(st: Stream, start: int, count: int, lo: int, hi: int, device) -> torch.Tensor:
    n_range = hi - lo + 1
    assert 0 < n_range < (1 << 32)
    d0, d1 = start // 2, (start + count + 1) // 2
    u = draw_u64(st, d0, d1 - d0, device)
    halves = torch.stack([u & 0xFFFFFFFF, _lsr(u, 32)], dim=1).reshape(-1)
    off = start - 2 * d0
    h = halves[off:off + count]
    return lo + ((h * n_range) >> 32)


def nibbles_t(st: Stream, start: int, count: int, device) -> torch.Tensor:
    d0, d1 = start // 16, (start + count + 15) // 16
    u = draw_u64(st, d0, d1 - d0, device)
    shifts = torch.arange(16, dtype=torch.int64, device=device) * 4
    v = ((u[:, None] >> shifts[None, :]) & 15).to(torch.uint8).reshape(-1)
    off = start - 16 * d0
    return v[off:off + count]


def make_weights_t(fmt: int, n_rows: int, k: int, name: str, seed: int = 0, device="cuda",
                   chunk_elems: int = 1 << 25, q8_range=(-127, 127),
                   scale_range=(1e-3, 1e-2)) -> torch.Tensor:
    """uint8 [n_rows][row_bytes] on `device`, byte-identical to
    ``synth.make_weights(fmt, n_rows, k, name, seed).data``."""
    rb = row_bytes(fmt, k)
    out = torch.empty((n_rows, rb), dtype=torch.uint8, device=device)
    rows_per = max(1, chunk_elems // k)
    lo, hi = scale_range
    for r0 in range(0, n_rows, rows_per):
        r1 = min(n_rows, r0 + rows_per)
        n = r1 - r0
        if fmt in (Q8_0, Q8G128):
            qk, bb = BLOCK_WEIGHTS[fmt], BLOCK_BYTES[fmt]
            nb = k // qk
            d = scale_f16(stream(name + "/d", seed), r0 * nb, n * nb, lo, hi)
            q = randint_t(stream(name + "/q", seed), r0 * k, n * k, *q8_range, device)
            blk = out[r0:r1].view(n, nb, bb)
            blk[:, :, 0:2] = torch.from_numpy(d.view(np.uint8).reshape(n, nb, 2)).to(device)
            blk[:, :, 2:bb] = q.to(torch.int8).view(torch.uint8).reshape(n, nb, qk)
            continue
        ns = k // 256
        d = scale_f16(stream(name + "/d", seed), r0 * ns, n * ns, lo, hi).reshape(n, ns)
        if fmt == Q6_K:  # packed on the host (the quants are drawn there too)
            q6 = randint_t(stream(name + "/q", seed), r0 * k, n * k, 0, 63, "cpu").to(torch.uint8)
            sc = randint(stream(name + "/sc", seed), r0 * ns * 16, n * ns * 16, -127, 127).reshape(n, ns, 16)
            out[r0:r1] = torch.from_numpy(pack_q6_k(d, sc, q6.numpy().reshape(n, k))).to(device)
            continue
        if fmt == Q5_K:
            q = randint_t(stream(name + "/q", seed), r0 * k, n * k, 0, 31, device).to(torch.uint8)
        else:
            q = nibbles_t(stream(name + "/q", seed), r0 * k, n * k, device)
        if fmt in (Q4_K, Q5_K):
            dmin = scale_f16(stream(name + "/dmin", seed), r0 * ns, n * ns, lo, hi).reshape(n, ns)
            sc = randint(stream(name + "/sc", seed), r0 * ns * 8, n * ns * 8, 0, 63).reshape(n, ns, 8)
            m = randint(stream(name + "/m", seed), r0 * ns * 8, n * ns * 8, 0, 63).reshape(n, ns, 8)
            hdr, hb = q4_k_header(d, dmin, sc, m), 16
            qq = q.reshape(n, ns, 4, 2, 32)   # chunk c, half h, i
            if fmt == Q5_K:  # fifth bits -> qh (bit 2c: low half of chunk c, 2c+1: high half)
                fifth = (qq >> 4) & 1
                qh = torch.zeros((n, ns, 32), dtype=torch.uint8, device=device)
                for c in range(4):
                    qh |= fifth[:, :, c, 0, :] << (2 * c)
                    qh |= fifth[:, :, c, 1, :] << (2 * c + 1)
                qq = qq & 15
                hb = 48
        elif fmt == IQ4_XS:
            ls = randint(stream(name + "/ls", seed), r0 * ns * 8, n * ns * 8, 0, 63).reshape(n, ns, 8)
            hdr, hb = iq4_xs_header(d, ls), 8
            qq = q.reshape(n, ns, 8, 2, 16)   # sub-block j, half h, i
        else:
            raise ValueError(f"unknown format {fmt}")
        blk = out[r0:r1].view(n, ns, rb // ns)
        if fmt == Q5_K:
            blk[:, :, 0:16] = torch.from_numpy(hdr).to(device)
            blk[:, :, 16:48] = qh
        else:
            blk[:, :, 0:hb] = torch.from_numpy(hdr).to(device)
        blk[:, :, hb:] = (qq.select(-2, 0) | (qq.select(-2, 1) << 4)).reshape(n, ns, 128)
    return out
