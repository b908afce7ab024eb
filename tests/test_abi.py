"""The C-ABI library: it loads, exports every function include/qmv.h declares,
answers the host-only size queries, and rejects invalid calls before any work
is enqueued (every call here returns from host validation: no device is
touched, so these run without a GPU)."""
import ctypes
import subprocess

import pytest

import quantized_decode_gemv_qmv_amd as q

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE = 0, 1, 2, 3, 4
FAKE = 0x10000000  # 256-byte aligned, never dereferenced by host validation


@pytest.fixture(scope="module")
def L():
    return q.lib()


def test_exports_every_declared_symbol(L):
    declared = q.symbols()
    assert len(declared) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", q.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for s in declared:
        assert hasattr(L, s)


def test_abi_version_and_status_strings(L):
    assert L.qmv_abi_version() == 1
    for st in range(6):
        assert L.qmv_status_string(st).decode().startswith("QMV_")
    assert b"unknown" in L.qmv_status_string(99)


@pytest.mark.parametrize("fmt,k,expect", [(0, 4096, 4352), (1, 4096, 2304), (2, 14336, 7616),
                                          (0, 65536, 69632), (0, 5120, 5440), (2, 1536, 816),
                                          (3, 4096, 2816), (3, 288, 0), (4, 4096, 3360), (4, 256, 210),
                                          (5, 5120, 5200), (5, 128, 130), (5, 96, 0),
                                          (0, 48, 0), (1, 288, 0), (2, 0, 0), (6, 256, 0)])
def test_row_bytes(fmt, k, expect):
    assert q.row_bytes(fmt, k) == expect


def test_act_layout():
    for t, k in ((1, 32), (3, 4096), (16, 14336), (512, 1536)):
        od, os_ = q.act_offsets(t, k)
        total = q.act_bytes(t, k)
        assert od % 256 == 0 and os_ % 256 == 0 and od >= t * k
        assert os_ >= od + 4 * t * (k // 32) and total >= os_ + 4 * t * (k // 32)
    assert q.act_bytes(0, 32) == 0 and q.act_bytes(1, 33) == 0


def test_workspace_sizes():
    assert q.matvec_workspace_bytes(0, 256, 65536, 1) > 256 * 4
    assert q.matvec_workspace_bytes(0, 152064, 5120, 1) == 0  # many rows: never split
    assert q.matvec_workspace_bytes(0, 256, 65536, 17) == 0
    assert q.moe_workspace_bytes(2, 128, 3072, 4096, 64, 8) >= 64 * 8 * 3072 * 4
    assert q.moe_workspace_bytes(2, 128, 3072, 4096, 65, 8) == 0
    assert q.moe_workspace_bytes(3, 128, 3072, 4096, 4, 8) == 0  # q5_K: no MoE kernel
    assert q.moe_workspace_bytes(4, 128, 3072, 4096, 4, 8) == 0  # q6_K neither
    assert q.moe_workspace_bytes(5, 128, 3072, 4096, 4, 8) == 0  # nor Q8G128


def _mv(L, fmt=0, w=FAKE, n=4, k=32, xq=FAKE, t=1, y=FAKE, ldy=4, ws=None, wsb=0):
    return L.qmv_matvec(fmt, w, n, k, xq, t, y, ldy, ws, wsb, None)


def test_matvec_validation(L):
    assert _mv(L, w=None) == INVALID
    assert _mv(L, xq=None) == INVALID
    assert _mv(L, y=None) == INVALID
    assert _mv(L, fmt=7) == INVALID
    assert _mv(L, n=0) == INVALID
    assert _mv(L, k=48) == INVALID
    assert _mv(L, fmt=1, k=32) == INVALID
    assert _mv(L, fmt=5, k=32) == INVALID  # Q8G128 rows hold whole 128-groups
    assert _mv(L, fmt=6) == INVALID
    assert _mv(L, ldy=3) == INVALID
    assert _mv(L, t=0) == INVALID
    assert _mv(L, t=17) == UNSUPPORTED
    assert _mv(L, w=FAKE + 8) == MISALIGNED
    assert _mv(L, xq=FAKE + 16) == MISALIGNED
    assert _mv(L, y=FAKE + 2) == MISALIGNED
    need = q.matvec_workspace_bytes(0, 4, 32, 1)
    assert _mv(L, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert _mv(L, ws=FAKE + 64, wsb=need) == MISALIGNED


def test_quantize_validation(L):
    f = L.qmv_quantize_act
    assert f(None, 32, 1, 32, FAKE, None) == INVALID
    assert f(FAKE, 32, 1, 32, None, None) == INVALID
    assert f(FAKE, 32, 0, 32, FAKE, None) == INVALID
    assert f(FAKE, 32, 1, 48, FAKE, None) == INVALID
    assert f(FAKE, 31, 1, 32, FAKE, None) == INVALID
    assert f(FAKE, 32, 65537, 32, FAKE, None) == UNSUPPORTED
    assert f(FAKE + 2, 32, 1, 32, FAKE, None) == MISALIGNED
    assert f(FAKE + 4, 32, 1, 32, FAKE, None) == MISALIGNED  # rows are read 16 bytes at a time
    assert f(FAKE, 33, 2, 32, FAKE, None) == MISALIGNED      # an odd row stride breaks that too
    assert f(FAKE, 34, 2, 32, FAKE, None) == MISALIGNED
    assert f(FAKE, 32, 1, 32, FAKE + 4, None) == MISALIGNED


def test_swiglu_quantize_validation(L):
    f = L.qmv_swiglu_quantize
    assert f(None, 64, 1, 32, FAKE, None, None) == INVALID
    assert f(FAKE, 64, 1, 32, None, None, None) == INVALID
    assert f(FAKE, 64, 0, 32, FAKE, None, None) == INVALID
    assert f(FAKE, 96, 1, 48, FAKE, None, None) == INVALID
    assert f(FAKE, 63, 1, 32, FAKE, None, None) == INVALID
    assert f(FAKE, 64, 65537, 32, FAKE, None, None) == UNSUPPORTED
    assert f(FAKE + 2, 64, 1, 32, FAKE, None, None) == MISALIGNED
    assert f(FAKE + 8, 64, 1, 32, FAKE, None, None) == MISALIGNED
    assert f(FAKE, 65, 2, 32, FAKE, None, None) == MISALIGNED
    assert f(FAKE, 66, 2, 32, FAKE, None, None) == MISALIGNED
    assert f(FAKE, 64, 1, 32, FAKE + 4, None, None) == MISALIGNED
    assert f(FAKE, 64, 1, 32, FAKE, FAKE + 4, None) == MISALIGNED


def test_router_topk_validation(L):
    f = L.qmv_router_topk

    def call(**kw):
        a = dict(x=FAKE, ldx=64, t=2, k=64, wr=FAKE, e=8, top_k=2, ids=FAKE, w=FAKE, logits=FAKE, xq=None)
        a.update(kw)
        return f(a["x"], a["ldx"], a["t"], a["k"], a["wr"], a["e"], a["top_k"], a["ids"], a["w"],
                 a["logits"], a["xq"], None)

    assert call(x=None) == INVALID
    assert call(ids=None) == INVALID
    assert call(logits=None) == INVALID
    assert call(k=62, ldx=64) == INVALID
    assert call(ldx=63) == INVALID
    assert call(top_k=9) == INVALID
    assert call(top_k=0) == INVALID
    assert call(t=65) == UNSUPPORTED
    assert call(k=(1 << 24) + 4, ldx=(1 << 24) + 4) == UNSUPPORTED
    assert call(e=2000, top_k=2) == UNSUPPORTED
    assert call(e=64, top_k=17) == UNSUPPORTED
    assert call(x=FAKE + 4) == MISALIGNED
    assert call(wr=FAKE + 8) == MISALIGNED
    assert call(xq=FAKE, k=48, ldx=48) == INVALID  # Q8 blocks need k % 32 == 0
    assert call(xq=FAKE + 64) == MISALIGNED
    assert call(logits=FAKE + 2) == MISALIGNED


def test_moe_validation(L):
    f = L.qmv_moe_matvec
    ws = q.moe_workspace_bytes(2, 8, 16, 256, 2, 2)

    def call(**kw):
        a = dict(fmt=2, w=FAKE, e=8, n=16, k=256, xq=FAKE, per_slot=0, ids=FAKE, rw=None, t=2,
                 top_k=2, y=FAKE, ws=FAKE, wsb=ws)
        a.update(kw)
        return f(a["fmt"], a["w"], a["e"], a["n"], a["k"], a["xq"], a["per_slot"], a["ids"], a["rw"],
                 a["t"], a["top_k"], a["y"], a["ws"], a["wsb"], None)

    assert call(ids=None) == INVALID
    assert call(ws=None) == INVALID
    assert call(per_slot=2) == INVALID
    assert call(top_k=0) == INVALID
    assert call(t=65) == UNSUPPORTED
    assert call(top_k=17) == UNSUPPORTED
    assert call(e=1025) == UNSUPPORTED
    assert call(k=32768) == UNSUPPORTED
    assert call(ids=FAKE + 2) == MISALIGNED
    assert call(rw=FAKE + 1) == MISALIGNED
    assert call(wsb=ws - 1) == WORKSPACE
    assert call(fmt=3) == UNSUPPORTED  # q5_K experts are not supported
    assert call(fmt=4) == UNSUPPORTED  # nor q6_K ones
    assert call(fmt=5) == UNSUPPORTED  # nor Q8G128 ones


def test_block_dots_validation(L):
    f = L.qmv_block_dots
    assert f(0, None, 4, 32, FAKE, 1, FAKE, None) == INVALID
    assert f(0, FAKE, 4, 32, FAKE, 17, FAKE, None) == UNSUPPORTED
    assert f(0, FAKE, 4, 32, FAKE, 1, FAKE + 1, None) == MISALIGNED


def test_block_dots_mx_validation(L):
    f = L.qmv_block_dots_mx
    mx = [i for i, n in enumerate(q.variants()) if n.startswith("mx_")]
    vec = [i for i, n in enumerate(q.variants()) if not n.startswith("mx_")]
    assert f(1, None, 4, 256, FAKE, 1, -1, 0, FAKE, None) == INVALID
    assert f(1, FAKE, 4, 256, FAKE, 1, vec[0], 0, FAKE, None) == INVALID  # not a matrix-core variant
    assert f(1, FAKE, 4, 256, FAKE, 1, len(q.variants()), 0, FAKE, None) == INVALID
    assert f(1, FAKE, 4, 256, FAKE, 1, mx[0], 1, FAKE, None) == INVALID   # one slice is no split
    assert f(1, FAKE, 4, 256, FAKE, 1, mx[0], 33, FAKE, None) == INVALID
    assert f(3, FAKE, 4, 256, FAKE, 1, -1, 0, FAKE, None) == UNSUPPORTED  # q5_K: no matrix-core decode
    assert f(4, FAKE, 4, 256, FAKE, 1, -1, 0, FAKE, None) == UNSUPPORTED  # nor q6_K
    assert f(1, FAKE, 4, 256, FAKE, 17, -1, 0, FAKE, None) == UNSUPPORTED
    assert f(1, FAKE, 4, 256, FAKE, 1, -1, 32, FAKE, None) == UNSUPPORTED  # 32 slices of one super-block
    assert f(1, FAKE, 4, 256, FAKE + 16, 1, -1, 0, FAKE, None) == MISALIGNED
    assert f(1, FAKE, 4, 256, FAKE, 1, -1, 0, FAKE + 2, None) == MISALIGNED


def test_moe_block_dots_validation(L):
    f = L.qmv_moe_block_dots
    ws = q.moe_workspace_bytes(2, 8, 16, 256, 4, 2)

    def call(fmt=2, w=FAKE, e=8, n=16, k=256, xq=FAKE, ps=0, ids=FAKE, t=4, top_k=2, sr=0, out=FAKE,
             wsp=FAKE, wsb=ws):
        return f(fmt, w, e, n, k, xq, ps, ids, t, top_k, sr, out, wsp, wsb, None)

    assert call(out=None) == INVALID
    assert call(wsp=None) == INVALID
    assert call(sr=5) == INVALID
    assert call(ps=2) == INVALID
    assert call(t=65) == UNSUPPORTED
    assert call(fmt=3) == UNSUPPORTED
    assert call(out=FAKE + 2) == MISALIGNED
    assert call(wsb=ws - 1) == WORKSPACE


def test_matvec_plan():
    # few rows, long K, a workspace: the matrix-core kernel split over workgroups
    v, s = q.matvec_plan(2, 4096, 14336, 16, True)
    assert q.variant_name(v).startswith("mx_") and s >= 1
    v0, s0 = q.matvec_plan(2, 4096, 14336, 16, False)
    assert s0 == 1 and v0 == q.pick_variant(2, 4096, 14336, 16)
    # many rows: never a workspace
    assert q.matvec_plan(0, 152064, 5120, 16, True)[1] == 1
    with pytest.raises(q.QmvError):
        q.matvec_plan(1, 4096, 300, 1, True)


# The kernel and K split qmv_matvec runs for the workload shapes, as the
# variant rules in the library choose them from the sweeps (host-only: the
# library describes an MI355X when no device is present).  (type, rows, K,
# tokens, with workspace) -> (variant, slices)
PLANS = [
    ((1, 14336, 4096, 1, False), ("fl_w4_r2_u2_l", 1)),
    ((1, 14336, 4096, 2, False), ("fl_w4_r2_u2_l", 1)),
    ((1, 14336, 4096, 16, False), ("mx_w8_k4_r4", 1)),
    ((1, 14336, 4096, 8, True), ("mf_w8_b4", 1)),          # flat matrix-core kernel, one pass
    ((1, 14336, 4096, 3, False), ("fl_w4_r2_u2_l", 1)),
    ((1, 14336, 4096, 4, True), ("fl_w4_r2_u2_l", 1)),
    ((1, 14336, 4096, 5, True), ("mf_w8_b4", 1)),
    ((0, 4096, 4096, 4, True), ("fl_w8_r2_u2_l", 1)),
    ((2, 4096, 14336, 1, True), ("fl_w8_r1_u7_l", 1)),
    ((2, 4096, 14336, 16, True), ("mx_w16_k4_r2", 4)),   # split over workgroups with a workspace
    ((2, 4096, 14336, 16, False), ("mx_w8_k8_r4", 1)),
    ((1, 4096, 14336, 16, True), ("mx_w16_k4_r2", 4)),
    ((2, 4096, 4096, 3, False), ("fl_w4_r1_u2_l", 1)),   # rows of 4096 weights, 16 rows per compute unit
    ((1, 4096, 4096, 6, False), ("fl_w8_r2_u2_l", 1)),
    ((2, 8192, 4096, 4, False), ("fl_w8_r2_u2_l", 1)),
    ((2, 8192, 4096, 16, True), ("mf_w8_b4", 1)),
    ((2, 14336, 4096, 6, True), ("mf_w8_b4", 1)),
    ((2, 14336, 4096, 16, True), ("mx_w16_k4_r2", 1)),
    ((1, 8192, 14336, 16, True), ("mx_w8_k1_r4", 4)),    # the sixteen-wave kernel does not split here
    ((2, 8192, 14336, 10, False), ("mx_w8_k4_r4", 1)),
    ((2, 8192, 14336, 4, False), ("mx_w8_k4_r4", 1)),
    ((1, 8192, 14336, 6, False), ("mx_w16_k4_r2", 1)),
    ((1, 28672, 4096, 6, False), ("mx_w8_k1_r4", 1)),
    ((2, 28672, 4096, 4, False), ("fl_w8_r2_u2_l", 1)),
    ((0, 4096, 4096, 1, True), ("fl_w4_r1_u2_l", 1)),
    ((0, 256, 65536, 1, True), ("lk_w16_r1_u2", 1)),     # K split inside one workgroup
    ((0, 256, 65536, 2, True), ("lk_w8_r1_u4", 1)),
    ((1, 256, 65536, 1, True), ("lk_w8_r1_u4", 1)),
    ((1, 256, 32768, 1, True), ("lk_w16_r1_u2", 1)),
    ((0, 256, 65536, 4, True), ("lk_w16_r1_u2", 1)),
    ((1, 512, 16384, 2, False), ("lk_w4_r1_u2", 1)),
    ((2, 1024, 8192, 1, True), ("lk_w4_r1_u2", 1)),
    ((2, 1024, 8192, 4, True), ("fl_w4_r1_u4_g", 1)),
    ((0, 152064, 5120, 16, False), ("mx_w8_k1_r4", 1)),
    ((0, 152064, 5120, 8, False), ("mt_r2_w4_k1", 1)),
    ((5, 152064, 5120, 4, False), ("fl_w16_r1_u3_l", 1)),
    ((5, 152064, 5120, 5, False), ("mt_r2_w4_k1", 1)),
    ((5, 152064, 5120, 2, False), ("st_w4_r1_u3", 1)),
    ((5, 152064, 5120, 16, False), ("mx_w8_k1_r4", 1)),
    ((4, 14336, 4096, 16, False), ("fl_w8_r2_u2_l", 1)),  # q6_K: vector kernels only
    ((4, 14336, 4096, 9, False), ("fl_w4_r2_u2_g", 1)),
    ((4, 14336, 4096, 3, False), ("fl_w4_r2_u2_l", 1)),
    ((3, 14336, 4096, 4, False), ("fl_w4_r2_u2_l", 1)),   # q5_K
    ((3, 14336, 4096, 5, False), ("mt_r2_w8_k2", 1)),
    ((3, 14336, 4096, 2, False), ("fl_w4_r2_u2_l", 1)),
    ((3, 4096, 4096, 16, False), ("mt_r1_w8_k4", 1)),
    ((3, 8192, 4096, 12, False), ("mt_r2_w8_k2", 1)),
    ((3, 14336, 4096, 12, False), ("mt_r4_w8_k2", 1)),
    ((3, 4096, 14336, 6, False), ("fl_w16_r1_u2_l", 1)),
    ((4, 4096, 14336, 16, False), ("mt_r1_w8_k4", 1)),
    ((4, 4096, 14336, 1, False), ("fl_w4_r2_u2_l", 1)),
    ((4, 4096, 4096, 3, False), ("fl_w4_r1_u2_l", 1)),
    ((0, 4096, 4096, 6, False), ("fl_w8_r2_u2_l", 1)),
    ((0, 4096, 4096, 8, False), ("fl_w16_r1_u2_l", 1)),
    ((0, 14336, 4096, 4, False), ("fl_w8_r2_u2_l", 1)),
    ((0, 8192, 4096, 6, False), ("fl_w8_r2_u2_l", 1)),
    ((0, 8192, 4096, 16, True), ("mf_w8_b4", 1)),
    ((0, 14336, 4096, 6, False), ("mt_r2_w4_k1", 1)),
    ((0, 4096, 14336, 3, False), ("fl_w16_r1_u2_l", 1)),
    ((0, 4096, 14336, 1, False), ("fl_w8_r1_u7_l", 1)),
]


@pytest.mark.parametrize("args,expect", PLANS, ids=[f"{a[0]}-{a[1]}x{a[2]}-T{a[3]}{'-ws' if a[4] else ''}"
                                                     for a, _ in PLANS])
def test_plans_of_the_workload_shapes(args, expect):
    v, s = q.matvec_plan(*args)
    assert (q.variant_name(v), s) == expect


def test_stream_read_validation(L):
    f = L.qmv_stream_read
    assert f(None, 4096, FAKE, None) == INVALID
    assert f(FAKE, 4096, None, None) == INVALID
    assert f(FAKE, 0, FAKE, None) == INVALID
    assert f(FAKE, 8, FAKE, None) == INVALID
    assert f(FAKE, 4104, FAKE, None) == INVALID  # not a multiple of 16
    assert f(FAKE + 8, 4096, FAKE, None) == MISALIGNED
    assert f(FAKE, 4096, FAKE + 2, None) == MISALIGNED


def test_tuning_switches(L):
    assert L.qmv_set_tuning(b"bogus", 0) == INVALID
    assert L.qmv_set_tuning(None, 0) == INVALID
    assert L.qmv_set_tuning(b"variant", len(q.variants())) == INVALID
    assert L.qmv_set_tuning(b"splitk", -2) == INVALID
    assert L.qmv_set_tuning(b"variant", -1) == OK
    assert L.qmv_set_tuning(b"splitk", -1) == OK
    assert L.qmv_set_tuning(b"moe_kernel", 4) == INVALID
    assert L.qmv_set_tuning(b"moe_kernel", 0) == OK
    assert L.qmv_set_tuning(b"moe_row16", 2) == INVALID
    assert L.qmv_set_tuning(b"moe_row16", 0) == OK
    for bad in (-2, 1, 33):
        assert L.qmv_set_tuning(b"mx_slices", bad) == INVALID
    assert L.qmv_set_tuning(b"mx_slices", -1) == OK
    assert L.qmv_set_tuning(b"flat_split", 2) == INVALID
    assert L.qmv_set_tuning(b"flat_split", 0) == OK
    assert q.variant_name(-1) is None and q.variant_name(len(q.variants())) is None
    assert q.pick_variant(1, 14336, 4096, 1) >= 0
    assert q.pick_variant(1, 14336, 4096, 17) == -1
    # q5_K has no matrix-core decode: never a matrix-core variant, even forced
    for t in range(1, 17):
        assert not q.variant_name(q.pick_variant(3, 14336, 4096, t)).startswith("mx_")
        assert not q.variant_name(q.pick_variant(4, 14336, 4096, t)).startswith("mx_")
    mx = [i for i, n in enumerate(q.variants()) if n.startswith("mx_")]
    try:
        q.set_tuning("variant", mx[0])
        assert not q.variant_name(q.pick_variant(3, 14336, 4096, 8)).startswith("mx_")
        assert q.variant_name(q.pick_variant(1, 14336, 4096, 8)).startswith("mx_")
    finally:
        q.set_tuning("variant", -1)


def test_matvec_x_validation(L):
    f = L.qmv_matvec_x

    def call(**kw):
        a = dict(fmt=1, w=FAKE, n=4, k=256, x=FAKE, ldx=256, t=1, y=FAKE, ldy=4, xq=FAKE, ws=None, wsb=0)
        a.update(kw)
        return f(a["fmt"], a["w"], a["n"], a["k"], a["x"], a["ldx"], a["t"], a["y"], a["ldy"], a["xq"], a["ws"],
                 a["wsb"], None)

    assert call(x=None) == INVALID
    assert call(xq=None) == INVALID
    assert call(y=None) == INVALID
    assert call(fmt=9) == INVALID
    assert call(k=96) == INVALID
    assert call(ldx=252) == INVALID
    assert call(ldx=258) == INVALID  # rows of x must keep 16-byte alignment
    assert call(ldy=3) == INVALID
    assert call(t=0) == INVALID
    assert call(t=17) == UNSUPPORTED
    assert call(x=FAKE + 4) == MISALIGNED
    assert call(xq=FAKE + 128) == MISALIGNED
    need = q.matvec_workspace_bytes(1, 4, 256, 1)
    assert need > 0
    assert call(ws=FAKE, wsb=need - 1) == WORKSPACE  # checked before the quantizer is enqueued
    assert call(ws=FAKE + 64, wsb=need) == MISALIGNED
    assert call(w=FAKE + 8) == MISALIGNED


def test_matvec_batch_validation(L):
    f = L.qmv_matvec_batch
    Item = q._Item

    def call(items, fmt=0, k=32, xq=FAKE, t=2):
        arr = (Item * max(1, len(items)))(*items)
        return f(fmt, arr, len(items), k, xq, t, None)

    def it(w=FAKE, n=4, y=FAKE, ldy=4, res=None, ldr=0):
        return Item(w, n, y, ldy, res, ldr)

    base = [it(y=FAKE), it(y=FAKE + 4096)]
    assert f(0, None, 1, 32, FAKE, 1, None) == INVALID
    assert call([]) == INVALID
    assert call(base, fmt=5) == INVALID
    assert call(base, xq=None) == INVALID
    assert call(base, t=0) == INVALID
    assert call(base, t=17) == UNSUPPORTED
    assert call([it(y=FAKE + 4096 * i) for i in range(9)]) == UNSUPPORTED
    assert call([it(w=None)]) == INVALID
    assert call([it(n=0)]) == INVALID
    assert call([it(ldy=3)]) == INVALID
    assert call([it(y=None)]) == INVALID
    assert call([it(res=FAKE + 8192, ldr=3)]) == INVALID
    assert call(base, k=48) == INVALID
    assert call(base, fmt=1, k=32) == INVALID
    assert call([it(w=FAKE + 8)]) == MISALIGNED
    assert call([it(y=FAKE + 2)]) == MISALIGNED
    assert call([it(res=FAKE + 8194, ldr=4)]) == MISALIGNED
    assert call(base, xq=FAKE + 16) == MISALIGNED
    # outputs: [T=2][ldy=4] of 4 columns span 32 bytes
    assert call([it(y=FAKE), it(y=FAKE + 28)]) == INVALID      # overlapping outputs
    assert call([it(y=FAKE, ldy=8), it(y=FAKE + 16)]) == INVALID  # interleaved rows overlap the extent
    assert call([it(y=FAKE, res=FAKE + 16, ldr=4)]) == INVALID  # residual overlapping its own output
    assert call([it(y=FAKE, res=FAKE + 4096, ldr=4), it(y=FAKE + 4096)]) == INVALID  # another item's output
    assert call([it(y=FAKE, res=FAKE, ldr=8, ldy=4)]) == INVALID  # in place needs the same stride



def test_moe_noalloc_validation(L):
    """The no-allocation MoE entry point validates as qmv_moe_matvec does and
    rejects calls whose workspace would exceed its device-resident array."""
    f = L.qmv_moe_matvec_noalloc

    def call(fmt=2, w=FAKE, e=128, n=4096, k=1536, xq=FAKE, ps=1, ids=FAKE, rw=FAKE, t=64, top_k=8, y=FAKE):
        return f(fmt, w, e, n, k, xq, ps, ids, rw, t, top_k, y, None)

    assert call(w=None) == INVALID
    assert call(y=None) == INVALID
    assert call(ps=2) == INVALID
    assert call(t=65) == UNSUPPORTED
    assert call(fmt=3) == UNSUPPORTED
    assert call(y=FAKE + 2) == MISALIGNED
    # 64 tokens x top-16 x 8192 rows of per-slot outputs: 32 MiB > the 17 MiB array
    assert q.moe_workspace_bytes(2, 128, 8192, 1536, 64, 16) > (17 << 20)
    assert call(n=8192, top_k=16) == WORKSPACE
