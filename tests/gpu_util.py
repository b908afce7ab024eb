"""Helpers of the GPU parity tests: seeded inputs on the device, oracle
references on the host, and the comparison rules.

Rules (all parity tests):
  * activation quantization (qs, d, s) and per-block integer partials:
    bit-exact;
  * fp32 outputs: |y - y*| <= 1e-4 * sum|terms| for every output, where y*
    and sum|terms| come from the oracle in fp64; an output whose terms are all
    zero must be exactly zero.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.device import make_weights_t

REL_TOL = 1e-4

gpu = pytest.mark.gpu


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_decode_gemv_qmv_amd as qmv
    qmv.lib()  # fails loudly when the HIP library is missing
    return qmv


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def weights(fmt: int, n: int, k: int, name: str, seed: int = 0) -> torch.Tensor:
    """Device weights [n][row_bytes] from the torch generator (byte-identical
    to the numpy generator)."""
    return make_weights_t(fmt, n, k, name, seed, device="cuda")


def x_host(t: int, k: int, name: str) -> np.ndarray:
    return synth.make_x(t, k, name)


def quantize(qmv, x: np.ndarray) -> torch.Tensor:
    return qmv.quantize_act(to_dev(x))


def assert_y(y_gpu: np.ndarray, y_ref: np.ndarray, mag: np.ndarray, what: str = "") -> None:
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    err = np.abs(y_gpu - y_ref)
    tol = REL_TOL * mag
    bad = ~(err <= tol)
    zero = mag == 0
    bad |= zero & (y_gpu != 0)
    if bad.any():
        i = np.argwhere(bad)[0]
        i = tuple(int(v) for v in i)
        raise AssertionError(f"{what}: {int(bad.sum())} outputs off, first at {i}: gpu {y_gpu[i]!r} "
                             f"oracle {y_ref[i]!r} tol {tol[i]!r}")


def sample_rows(n: int, count: int, seed_name: str, edge: int = 32) -> np.ndarray:
    """Row indices: the first and last `edge` rows plus `count` seeded draws."""
    if n <= 2 * edge + count:
        return np.arange(n)
    r = synth.randint(synth.stream(seed_name), 0, count, 0, n - 1)
    return np.unique(np.concatenate([np.arange(edge), np.arange(n - edge, n), r]))


def host_rows(w_dev: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    return w_dev.index_select(0, idx).cpu().numpy()
