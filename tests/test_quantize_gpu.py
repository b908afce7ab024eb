"""qmv_quantize_act against the oracle's quantizer: (qs, d, s) bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from golden_io import act_cases
from gpu_util import gpu, need_gpu, say, to_dev, x_host

pytestmark = gpu


def _compare(qmv, x: np.ndarray, what: str, ldx_pad: int = 0):
    t, k = x.shape
    say(f"quantize {what} T={t} K={k} pad={ldx_pad}")
    if ldx_pad:
        xp = np.full((t, k + ldx_pad), np.float32(1e30), np.float32)
        xp[:, :k] = x
        xd = to_dev(xp)[:, :k]
    else:
        xd = to_dev(x)
    xq = qmv.quantize_act(xd)
    qs, d, s = qmv.act_fields(xq, t, k)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(qs.cpu().numpy(), rq), what
    assert np.array_equal(d.cpu().numpy().view(np.uint32), rd.view(np.uint32)), what
    assert np.array_equal(s.cpu().numpy(), rs), what


@pytest.mark.parametrize("k", [4096, 14336, 1536, 65536, 5120])
@pytest.mark.parametrize("t", [1, 2, 16, 64])
def test_config_shapes(k, t):
    qmv = need_gpu()
    _compare(qmv, x_host(t, k, f"qz/{k}"), "normal")


def test_slot_rows_and_stride():
    qmv = need_gpu()
    _compare(qmv, x_host(512, 1536, "qz/slots"), "moe down slots")
    _compare(qmv, x_host(5, 4096, "qz/stride"), "row stride", ldx_pad=96)


def test_hand_cases_and_ties():
    qmv = need_gpu()
    cases = act_cases()
    x = np.stack([c["x"] for c in cases]).reshape(1, -1).astype(np.float32)
    _compare(qmv, x, "hand cases")
    # exact ties at many scales: amax = 127 * 2^e, values (m + 0.5) * 2^e
    rows = []
    for e in range(-12, 6):
        blk = np.zeros(32, np.float32)
        blk[0] = 127 * 2.0 ** e
        blk[1:] = (np.arange(-15, 16)[:31] + 0.5) * 2.0 ** e
        rows.append(blk)
    _compare(qmv, np.concatenate(rows)[None], "ties")


def test_wide_dynamic_range():
    qmv = need_gpu()
    x = x_host(8, 4096, "qz/range").astype(np.float64)
    x *= np.exp2(np.repeat(np.arange(-40, 88, 1)[: 4096 // 32], 32))[None, :] / 8
    x = x.astype(np.float32)
    assert np.isfinite(x).all()
    _compare(qmv, x, "dynamic range")
    z = np.zeros((2, 1024), np.float32)
    z[1, 5] = -0.0
    _compare(qmv, z, "zeros")


def test_overwrites_buffer():
    qmv = need_gpu()
    x = x_host(3, 256, "qz/ow")
    xq = torch.full((qmv.act_bytes(3, 256),), 0xAB, dtype=torch.uint8, device="cuda")
    qmv.quantize_act(to_dev(x), out=xq)
    qs, d, s = qmv.act_fields(xq, 3, 256)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(qs.cpu().numpy(), rq) and np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(d.cpu().numpy(), rd)
