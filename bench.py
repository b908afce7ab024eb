#!/usr/bin/env python3
"""Benchmark of the quantized decode matvec on one MI355X.

One step is one pass of the hot path over one batch of tokens: quantize the
fp32 activations to Q8 blocks (qmv_quantize_act) and run the block-quantized
matvec (qmv_matvec, with the split-K workspace where the shape takes one;
qmv_matvec_batch for sibling matrices), so that the roofline's kernel is the
matvec the step runs.  The same step through qmv_matvec_x (the quantization
fused into the matvec where that is faster) is reported beside it.  The
default workload is the q4_K 14336 x 4096 matvec at one token; --workload /
--tokens select the others.  Inputs are synthetic
(seeded generator) and resident in HBM before timing starts.

The weights are read from a ring of copies of at least 1 GiB, one copy per
step, so every step streams its weights from HBM rather than from the 256 MB
Infinity Cache.  Steps are captured in HIP graphs and replayed; exactly
--steps steps are timed between two device synchronisations.

Output: one JSON line.  `value` is weight bytes per step / time per step
(GB/s).  `roofline` is the matvec kernel against the 8 TB/s HBM peak: its
average duration comes from HIP events around back-to-back replays of the
kernel alone over the same ring (the same figure rocprofv3's kernel trace
reports), `traffic` from the rocprofv3 counter summary under profiles/ when
it was taken from the current kernel sources.  `cpu_baseline` is the CPU
oracle (test infrastructure) timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "weight GB/s & % HBM roofline, q4_K/IQ4_XS matvec at 1–16 tokens"

# name: (format, rows, K, token counts of the workload[, sibling matrices])
WORKLOADS = {
    "q4_k_14336x4096": (1, 14336, 4096, (1, 2, 4, 8, 16)),
    "q5_k_14336x4096": (3, 14336, 4096, (1, 2, 4, 8, 16)),
    "q6_k_14336x4096": (4, 14336, 4096, (1, 2, 4, 8, 16)),
    "q8g128_head_152064x5120": (5, 152064, 5120, (1, 2, 4, 8, 16)),
    # gate and up projections as two separate tensors sharing one activation
    # buffer, one qmv_matvec_batch launch
    "q4_k_siblings_2x14336x4096": (1, 14336, 4096, (1, 2, 4, 8, 16), 2),
    "iq4_xs_4096x14336": (2, 4096, 14336, (1, 2, 4, 8, 16)),
    "q8_0_4096x4096": (0, 4096, 4096, (1,)),
    "q8_0_splitk_256x65536": (0, 256, 65536, (1,)),
    "q8_0_head_152064x5120": (0, 152064, 5120, (1, 2, 4, 8, 16)),
}
FMT_NAME = {0: "Q8_0", 1: "q4_K", 2: "IQ4_XS", 3: "q5_K", 4: "q6_K", 5: "Q8G128"}
# bytes of one row of 32 / 128 / 256 weights per format, and each workload's
# weight bytes per matrix (the algorithmic bytes of one launch)
BLOCK = {0: (32, 34), 1: (256, 144), 2: (256, 136), 3: (256, 176), 4: (256, 210), 5: (128, 130)}
WEIGHT_BYTES = {wl: v[1] * (v[2] // BLOCK[v[0]][0]) * BLOCK[v[0]][1] for wl, v in WORKLOADS.items()}
# MoE decode: 128 IQ4_XS experts, gate+up 3072 x 4096 and down 4096 x 1536 per
# expert, top-8 routing
MOE = dict(name="moe_iq4_xs_e128", ffn_name="moe_ffn_iq4_xs_e128", experts=128, top_k=8,
           gate_up=(3072, 4096), down=(4096, 1536), tokens=(1, 6, 16, 64))
# The device code of the dense kernels: a recorded traffic figure is used
# only while these files are unchanged and the planned variant is the one it
# was taken from (host-side dispatch changes are caught by the latter).
KERNEL_SOURCES = ("qmv_device.h", "qmv_internal.h", "qmv_matvec.hip", "qmv_mfma.h", "qmv_mfma.hip", "qmv_mxf.hip",
                  "qmv_quant.hip")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantized_decode_gemv_qmv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, tokens: int, src_hash: str, variant: str):
    """HBM bytes per launch from profiles/traffic_<workload>_t<T>.txt, if that
    summary was taken from the current kernel sources and the same variant."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_t{tokens}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"^kernel_sources_sha256_16:\s*(\S+)", text, re.M)
    m_bytes = re.search(r"^traffic_bytes_per_launch:\s*([0-9.]+)", text, re.M)
    m_var = re.search(r"^matvec_variant:\s*(\S+)", text, re.M)
    if not m_hash or not m_bytes or not m_var or m_hash.group(1) != src_hash or m_var.group(1) != variant:
        return None
    return float(m_bytes.group(1))


class Ring:
    """Device-resident inputs of one workload: weight ring, activations,
    buffers."""

    def __init__(self, torch, qmv, fmt, n, k, t, name, mats=1):
        from synth import make_x
        from synth.device import make_weights_t

        self.fmt, self.n, self.k, self.t, self.mats = fmt, n, k, t, mats
        # mats == 1: one matrix per copy; else `mats` sibling matrices
        # (separate tensors) per copy, run as one batched launch
        w0 = [make_weights_t(fmt, n, k, f"{name}/W" if mats == 1 else f"{name}/W{j}", device="cuda")
              for j in range(mats)]
        self.weight_bytes = sum(w.numel() for w in w0)
        self.copies = max(2, math.ceil((1 << 30) / self.weight_bytes))
        self.w = [w0] + [[w.clone() for w in w0] for _ in range(self.copies - 1)]
        xs = make_x(8 * t, k, f"{name}/x").reshape(8, t, k)
        self.x = [torch.from_numpy(xs[i]).cuda() for i in range(8)]
        self.xq = torch.empty(qmv.act_bytes(t, k), dtype=torch.uint8, device="cuda")
        qmv.quantize_act(self.x[0], out=self.xq)  # the matvec alone is timed on real activations too
        self.y = [torch.empty((t, n), dtype=torch.float32, device="cuda") for _ in range(mats)]
        wsb = qmv.matvec_workspace_bytes(fmt, n, k, t) if mats == 1 else 0
        self.ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda") if wsb else None

    def step(self, qmv, i):
        qmv.quantize_act(self.x[i % 8], out=self.xq)
        self.matvec_only(qmv, i)

    def matvec_only(self, qmv, i):
        w = self.w[i % self.copies]
        if self.mats == 1:
            qmv.matvec(self.fmt, w[0], self.n, self.k, self.xq, self.t, y=self.y[0], ws=self.ws)
        else:
            qmv.matvec_batch(self.fmt, [(w[j], self.n, self.y[j], None) for j in range(self.mats)],
                             self.k, self.xq, self.t)

    def fused(self, qmv, i):
        """One matrix from fp32 activations: qmv_matvec_x (the matvec
        workgroups quantize x themselves at one or two tokens)."""
        qmv.matvec_x(self.fmt, self.w[i % self.copies][0], self.n, self.k, self.x[i % 8], xq=self.xq,
                     y=self.y[0], ws=self.ws)

    def separate(self, qmv, i):
        """The sibling matrices as separate qmv_matvec launches (comparison)."""
        w = self.w[i % self.copies]
        for j in range(self.mats):
            qmv.matvec(self.fmt, w[j], self.n, self.k, self.xq, self.t, y=self.y[j])


class MoeRing:
    """Device-resident inputs of the MoE decode workload: two copies of the
    expert tensors (alternating), 16 routings, activations and buffers."""

    def __init__(self, torch, qmv, t):
        import numpy as np

        from synth import make_routing, make_x
        from synth.device import make_weights_t

        e, self.top_k = MOE["experts"], MOE["top_k"]
        self.t = t
        (ng, kg), (nd, kd) = MOE["gate_up"], MOE["down"]
        self.shape = (e, ng, kg, nd, kd)
        name = MOE["name"]
        gu = make_weights_t(2, e * ng, kg, f"{name}/gate_up", device="cuda")
        dn = make_weights_t(2, e * nd, kd, f"{name}/down", device="cuda")
        self.gu = [gu, gu.clone()]
        self.dn = [dn, dn.clone()]
        self.bytes_per_expert = (gu.numel() + dn.numel()) // e
        self.routes = []
        for r in range(16):
            ids, rw = make_routing(t, e, self.top_k, f"{name}/route{r}")
            self.routes.append((torch.from_numpy(ids).cuda(), torch.from_numpy(rw).cuda(),
                                len(set(ids.reshape(-1).tolist()))))
        xs = make_x(8 * t, kg, f"{name}/x").reshape(8, t, kg)
        hs = make_x(8 * t * self.top_k, kd, f"{name}/h").reshape(8, t * self.top_k, kd)
        self.x = [torch.from_numpy(xs[i]).cuda() for i in range(8)]
        self.h = [torch.from_numpy(hs[i]).cuda() for i in range(8)]
        self.xq = torch.empty(qmv.act_bytes(t, kg), dtype=torch.uint8, device="cuda")
        self.hq = torch.empty(qmv.act_bytes(t * self.top_k, kd), dtype=torch.uint8, device="cuda")
        qmv.quantize_act(self.x[0], out=self.xq)  # projections timed alone read real activations
        qmv.quantize_act(self.h[0], out=self.hq)
        self.y_gu = torch.empty((t, self.top_k, ng), dtype=torch.float32, device="cuda")
        self.y_dn = torch.empty((t, nd), dtype=torch.float32, device="cuda")
        self.ws_gu = torch.zeros(qmv.moe_workspace_bytes(2, e, ng, kg, t, self.top_k),
                                 dtype=torch.uint8, device="cuda")
        self.ws_dn = torch.zeros(qmv.moe_workspace_bytes(2, e, nd, kd, t, self.top_k),
                                 dtype=torch.uint8, device="cuda")
        # router fp32 [E][K] with N(0, 1/K) entries, so that the logits of an
        # N(0,1) token are about N(0,1) as in the routing of this workload
        self.wr_host = make_x(e, kg, f"{name}/router") * np.float32(1.0 / math.sqrt(kg))
        self.wr = torch.from_numpy(self.wr_host).cuda()
        self.r_ids = torch.empty((t, self.top_k), dtype=torch.int32, device="cuda")
        self.r_w = torch.empty((t, self.top_k), dtype=torch.float32, device="cuda")
        self.r_logits = torch.empty((t, e), dtype=torch.float32, device="cuda")
        self.router_u = None

    def avg_bytes(self, steps):
        """Weight bytes a step reads, averaged over the routings it cycles."""
        return sum(self.routes[i % 16][2] for i in range(steps)) * self.bytes_per_expert / steps

    def gate_up(self, qmv, i):
        e, ng, kg, _, _ = self.shape
        ids = self.routes[i % 16][0]
        qmv.moe_matvec(2, self.gu[i % 2], e, ng, kg, self.xq, False, ids, None, self.ws_gu, y=self.y_gu)

    def down(self, qmv, i):
        e, _, _, nd, kd = self.shape
        ids, rw, _ = self.routes[i % 16]
        qmv.moe_matvec(2, self.dn[i % 2], e, nd, kd, self.hq, True, ids, rw, self.ws_dn, y=self.y_dn)

    def step(self, qmv, i):
        qmv.quantize_act(self.x[i % 8], out=self.xq)
        self.gate_up(qmv, i)
        qmv.quantize_act(self.h[i % 8], out=self.hq)
        self.down(qmv, i)

    def router(self, qmv, i):
        qmv.router_topk(self.x[i % 8], self.wr, self.top_k, ids=self.r_ids, weights=self.r_w,
                        logits=self.r_logits)

    def ffn_step(self, qmv, i):
        """The MoE FFN: router and top-k (writing the Q8 blocks of x as well),
        then the routed gate+up with SwiGLU and the Q8 blocks of its output
        (qmv_moe_gate_up_swiglu, two launches unless one is asked for), then
        the down projection combined with the router's weights."""
        e, ng, kg, nd, kd = self.shape
        # the router also writes the Q8 blocks of x that the gate+up projection takes
        qmv.router_topk(self.x[i % 8], self.wr, self.top_k, ids=self.r_ids, weights=self.r_w,
                        logits=self.r_logits, xq=self.xq)
        qmv.moe_gate_up_swiglu(2, self.gu[i % 2], e, kd, kg, self.xq, self.r_ids, self.ws_gu, hq=self.hq)
        qmv.moe_matvec(2, self.dn[i % 2], e, nd, kd, self.hq, True, self.r_ids, self.r_w, self.ws_dn,
                       y=self.y_dn)

    def ffn_bytes(self, qmv, steps):
        """Weight bytes an FFN step reads (routed experts + the fp32 router),
        averaged over the steps; the router's picks per input are read back
        once, outside any timed region."""
        if self.router_u is None:
            self.router_u = []
            for i in range(8):
                self.router(qmv, i)
                self.router_u.append(len(set(self.r_ids.cpu().reshape(-1).tolist())))
        u = sum(self.router_u[i % 8] for i in range(steps)) / steps
        return u * self.bytes_per_expert + self.wr.numel() * 4, u


def capture(torch, fn, count, start=0):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(count):
                fn(start + i)
    torch.cuda.current_stream().wait_stream(s)
    return g


def run_steps(torch, graphs, steps):
    """Replays graphs covering exactly `steps` steps."""
    g_full, per, g_tail = graphs
    for _ in range(steps // per):
        g_full.replay()
    if g_tail is not None:
        g_tail.replay()


def _replay_samples(torch, g, per, reps):
    """Per-call time (us) of each of `reps` replays of graph g (`per` calls):
    HIP events on the current stream around every replay."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for r in range(reps):
        g.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    return [ev[r].elapsed_time(ev[r + 1]) * 1e3 / per for r in range(reps)]


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


# Untimed work before each measurement.  On MI355X a kernel's time keeps
# falling for about 0.1 s of continuous work after the GPU was idle (IQ4_XS
# 4096 x 14336 at one token: 9.3 us at once, 8.6 us from 0.1 s on); the
# figures are taken at that steady state.
WARM_SECONDS = 0.15


def warm(torch, g, seconds=WARM_SECONDS):
    """Replay graph g until `seconds` of wall time have passed."""
    t0 = time.perf_counter()
    while True:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def timed_replays(torch, fn, per, reps=21):
    """Median per-call time (us) of fn(i) over `reps` back-to-back replays of
    a graph of `per` calls, after WARM_SECONDS of untimed replays (each replay
    timed with HIP events; the graphs are replayed on the stream the events
    are recorded on)."""
    g = capture(torch, fn, per)
    warm(torch, g)
    return median(_replay_samples(torch, g, per, reps))


def kernel_us(torch, qmv, ring, reps=21):
    """Median matvec duration: per-launch average of each of `reps` replays
    of a graph of back-to-back launches of the kernel alone cycling the
    weight ring, then the median over the replays."""
    return timed_replays(torch, lambda i: ring.matvec_only(qmv, i), max(ring.copies, 32), reps)


def moe_cpu_baseline(ring, min_seconds=10.0, ffn=False):
    """The CPU oracle on the MoE step for this token count: quantize x and h,
    gate+up and down routed matvecs over all rows (routing 0); with ffn, h is
    SwiGLU of the gate+up output."""
    import numpy as np

    import oracle
    import synth

    e, ng, kg, nd, kd = ring.shape
    x = synth.make_x(ring.t, kg, f"{MOE['name']}/x")
    if ffn:  # routed by the router on the first input
        ids, rw, _ = oracle.router_topk(x, ring.wr_host, ring.top_k)
        rw = rw.astype(np.float32)
    else:
        ids, rw = synth.make_routing(ring.t, e, ring.top_k, f"{MOE['name']}/route0")
    used = sorted(set(ids.reshape(-1).tolist()))
    remap = {ex: i for i, ex in enumerate(used)}
    # only the routed experts' weights are generated; ids are renumbered onto them
    gu = np.concatenate([synth.make_weights(2, e * ng, kg, f"{MOE['name']}/gate_up",
                                            rows=(ex * ng, (ex + 1) * ng)).data for ex in used])
    dn = np.concatenate([synth.make_weights(2, e * nd, kd, f"{MOE['name']}/down",
                                            rows=(ex * nd, (ex + 1) * nd)).data for ex in used])
    ids2 = np.vectorize(remap.get)(ids).astype(np.int32)
    h = synth.make_x(ring.t * ring.top_k, kd, f"{MOE['name']}/h")
    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    reps, t0 = 0, time.perf_counter()
    while True:
        if ffn:
            oracle.router_topk(x, ring.wr_host, ring.top_k)
        qs, d, s = oracle.quantize_act(x)
        y_gu, _ = oracle.moe_matvec(2, gu, len(used), ng, kg, qs, d, s, ids2, None, False)
        if ffn:
            h = oracle.swiglu(y_gu.reshape(ring.t * ring.top_k, ng).astype(np.float32), kd).astype(np.float32)
        qs, d, s = oracle.quantize_act(h)
        oracle.moe_matvec(2, dn, len(used), nd, kd, qs, d, s, ids2, rw, True)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    nbytes = len(used) * ring.bytes_per_expert + (ring.wr_host.nbytes if ffn else 0)
    return {"value": round(nbytes * reps / el / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"MoE{' FFN' if ffn else ''} step at {ring.t} token(s) "
                      f"({'router on the first input' if ffn else 'routing 0'}, {len(used)} experts), {reps} repetitions "
                      f"in {el:.1f} s"}


def bench_moe(args, torch, qmv, ffn=False):
    t = args.tokens
    log(f"bench: MoE{' FFN' if ffn else ''} T={t}: generating inputs")
    ring = MoeRing(torch, qmv, t)
    if args.profile_launches > 0:
        # plain launches for a profiler: the routed gate+up and down matvecs
        qmv.quantize_act(ring.x[0], out=ring.xq)
        qmv.quantize_act(ring.h[0], out=ring.hq)
        for i in range(2 * args.profile_launches):
            ring.gate_up(qmv, i)
            ring.down(qmv, i)
        torch.cuda.synchronize()
        log(f"bench: {args.profile_launches} profiled MoE steps after as many warmup steps")
        return 0
    per = 64
    step = (lambda i: ring.ffn_step(qmv, i)) if ffn else (lambda i: ring.step(qmv, i))
    g_full = capture(torch, step, per)
    tail = args.steps % per
    g_tail = capture(torch, step, tail) if tail else None
    warm_tail = args.warmup % per
    run_steps(torch, (g_full, per, capture(torch, step, warm_tail) if warm_tail else None), args.warmup)
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} MoE steps")
    t0 = time.perf_counter()
    run_steps(torch, (g_full, per, g_tail), args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    if ffn:
        step_bytes, avg_u = ring.ffn_bytes(qmv, args.steps)
    else:
        step_bytes = ring.avg_bytes(args.steps)
        avg_u = step_bytes / ring.bytes_per_expert
    step_u = avg_u
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    gu_us = timed_replays(torch, lambda i: ring.gate_up(qmv, i), per)
    dn_us = timed_replays(torch, lambda i: ring.down(qmv, i), per)
    router_us = timed_replays(torch, lambda i: ring.router(qmv, i), per) if ffn else None
    if ffn:  # the kernel figures below use the synthetic routings of the plain MoE step
        avg_u = ring.avg_bytes(args.steps) / ring.bytes_per_expert
    gu_bytes = avg_u * ring.gu[0].numel() / ring.shape[0]
    dn_bytes = avg_u * ring.dn[0].numel() / ring.shape[0]
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    cpu = None if args.no_cpu else moe_cpu_baseline(ring, ffn=ffn)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"MoE{' FFN' if ffn else ''} IQ4_XS 128 experts top-8, gate+up 3072x4096 + "
                               f"down 4096x1536, {t} token(s)", "tokens": t,
                   "avg_distinct_experts": round(step_u, 2),
                   "weight_bytes_per_step": round(step_bytes),
                   "step": ("router + top-k (fp32 router 128x4096) + quantize x + gate_up routed matvec + SwiGLU "
                            "and Q8 of its output + down routed matvec weighted by the router" if ffn else
                            "quantize x + gate_up routed matvec + quantize h + down routed matvec")},
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gate_up routed matvec", "kernel_us": round(gu_us, 3),
                     "algorithmic_bytes_per_launch": round(gu_bytes)},
        "down_kernel": {"kernel_us": round(dn_us, 3), "weight_GBps": round(dn_bytes / (dn_us * 1e-6) / 1e9, 1),
                        "algorithmic_bytes_per_launch": round(dn_bytes)},
        **({"router_us": round(router_us, 3)} if ffn else {}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def gpu_clocks():
    """The current shader and memory clock levels of the AMD GPUs the kernel
    driver lists in sysfs (read, never set; no program is started)."""
    import glob

    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            if open(os.path.join(dev, "vendor")).read().strip() != "0x1002":
                continue
            cur = {}
            for f in ("pp_dpm_sclk", "pp_dpm_mclk"):
                path = os.path.join(dev, f)
                if os.path.exists(path):
                    lines = [l.strip() for l in open(path).read().splitlines() if l.strip().endswith("*")]
                    cur[f[7:]] = lines[0] if lines else None
            if cur:
                out[os.path.basename(os.path.dirname(dev))] = cur
        except OSError:
            continue
    return out or None


def device_info(torch, clocks):
    """The GPU and its runtime; the clocks read before the GPU was touched."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "hip": torch.version.hip, "torch": torch.__version__, "clocks": clocks}


def cpu_baseline(fmt, n, k, t, name, min_seconds=10.0, max_seconds=30.0):
    """The CPU oracle (quantize + matvec, the same workload) on this host,
    repeated until at least min_seconds of work; then the quantization alone
    and the matvec on one thread, each for a few seconds."""
    import oracle
    import synth

    rows = min(n, max(1, (64 << 20) // (k // (32, 256, 256, 256, 256, 128)[fmt] * (34, 144, 136, 176, 210, 130)[fmt])))
    w = synth.make_weights(fmt, n, k, f"{name}/W", rows=(0, rows)).data
    x = synth.make_x(t, k, f"{name}/x")
    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    reps, t0 = 0, time.perf_counter()
    while True:
        qs, d, s = oracle.quantize_act(x)
        oracle.matvec(fmt, w, k, qs, d, s)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el >= max_seconds:
            break
    value = w.nbytes * reps / el / 1e9
    qreps, t0 = 0, time.perf_counter()
    while qreps < 3 or time.perf_counter() - t0 < 1.0:
        oracle.quantize_act(x)
        qreps += 1
    quant_s = (time.perf_counter() - t0) / qreps
    rows1 = max(1, rows // 8)
    oracle.set_threads(1)
    reps1, t0 = 0, time.perf_counter()
    while reps1 < 1 or time.perf_counter() - t0 < 3.0:
        oracle.matvec(fmt, w[:rows1], k, qs, d, s)
        reps1 += 1
    el1 = time.perf_counter() - t0
    oracle.set_threads(cores)
    return {"value": round(value, 3), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{FMT_NAME[fmt]} {rows}x{k} matvec (rows 0..{rows - 1} of {n}) at {t} "
                      f"token(s) incl. activation quantization, {reps} repetitions in {el:.1f} s",
            "quantize_us_per_call": round(quant_s * 1e6, 1),
            "matvec_s_per_call": round(el / reps - quant_s, 4),
            "value_1_thread": round(w[:rows1].nbytes * reps1 / el1 / 1e9, 3),
            "sample_1_thread": f"rows 0..{rows1 - 1}, matvec only, {reps1} repetitions in {el1:.1f} s"}


def trace_summary(path: str) -> int:
    """Per-kernel summary of a rocprofv3 kernel trace (the *_kernel_trace.csv
    of --kernel-trace): calls, median, average, min and max duration in us."""
    import csv

    durs = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("KernelName") or "?"
            d = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            durs.setdefault(name, []).append(d)
    print(f"{'calls':>7} {'median_us':>10} {'avg_us':>9} {'min_us':>8} {'max_us':>8}  kernel")
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        print(f"{len(v):7d} {median(v):10.3f} {sum(v) / len(v):9.3f} {min(v):8.3f} {max(v):8.3f}  {name[:150]}")
    return 0


def counter_summary(path: str) -> int:
    """Per-kernel mean per dispatch of every counter in a rocprofv3 --pmc
    counter_collection.csv (one row per dispatch and counter)."""
    import csv

    vals, names = {}, []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            k = row.get("Kernel_Name", "?")
            c = row.get("Counter_Name", "?")
            vals.setdefault(k, {}).setdefault(c, []).append(float(row["Counter_Value"]))
            if c not in names:
                names.append(c)
    for k, cs in vals.items():
        n = max(len(v) for v in cs.values())
        print(f"{k[:150]}  ({n} dispatches)")
        for c in names:
            if c in cs:
                v = cs[c]
                print(f"    {c:40s} mean {sum(v) / len(v):16.1f}  median {median(v):16.1f}")
    return 0


def _counter_rows(path: str):
    """(kernel name, counter value) of every dispatch in a rocprofv3 --pmc
    counter_collection.csv."""
    import csv

    with open(path, newline="") as f:
        return [(row.get("Kernel_Name", "?"), float(row["Counter_Value"])) for row in csv.DictReader(f)]


def traffic_summary(fetch_csv: str, write_csv: str, workload: str, tokens: int, variant: str) -> int:
    """The HBM traffic file of one workload (profiles/traffic_<workload>_t<T>.txt)
    from a FETCH_SIZE and a WRITE_SIZE run of --profile-launches: each counter
    (KiB per dispatch) is scaled by what it reads for the runtime's copy of the
    weight tensor in the same run (the ring's clones: exactly the weight bytes
    read and written), and the matvec's median per dispatch is reported
    against its algorithmic bytes."""
    fmt, n, k, *_ = WORKLOADS[workload]
    wb = WEIGHT_BYTES[workload]
    out = {}
    for what, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path)
        copy = [v for name, v in rows if "copyBuffer" in name]
        mv = {}
        for name, v in rows:
            if name.startswith("void qmv::k_") and "quantize" not in name and "stream_read" not in name:
                mv.setdefault(name, []).append(v)
        if not copy or not mv:
            print(f"{path}: no copy or matvec dispatches", file=sys.stderr)
            return 1
        kname, vals = max(mv.items(), key=lambda kv: len(kv[1]))
        scale = wb / (median(copy) * 1024.0)
        out[what] = (kname, median(copy), len(copy), scale, median(vals), len(vals))
    kname = out["FETCH_SIZE"][0]
    c_f, n_f, s_f, v_f, m_f = out["FETCH_SIZE"][1:]
    c_w, n_w, s_w, v_w, m_w = out["WRITE_SIZE"][1:]
    rd, wr = v_f * 1024.0 * s_f, v_w * 1024.0 * s_w
    # the profile mode runs as many warmup launches as profiled ones
    prof = f"--workload {workload} --tokens {tokens} --profile-launches {m_f // 2}"
    print(f"# HBM traffic of the {FMT_NAME[fmt]} {n}x{k} matvec at {tokens} token(s)")
    print(f"# kernel: {kname}")
    print("#")
    print("# Commands (each counter in a run of its own, one MI355X):")
    print("#   cd /tmp && export TMPDIR=/tmp")
    print(f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o run -- python3 <repo>/bench.py {prof}")
    print(f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o run -- python3 <repo>/bench.py {prof}")
    print(f"#   python3 <repo>/bench.py --traffic-summary <fetch csv> <write csv> --workload {workload} --tokens {tokens}")
    print("#")
    print(f"# Normalisation: the same runs clone the {wb:,}-byte weight tensor (__amd_rocclr_copyBuffer),")
    print("# reading and writing exactly that many bytes.")
    print(f"#   copy FETCH_SIZE median {c_f:.1f} KiB over {n_f} dispatches -> read scale {s_f:.4f}")
    print(f"#   copy WRITE_SIZE median {c_w:.1f} KiB over {n_w} dispatches -> write scale {s_w:.4f}")
    print("#")
    print("# Matvec, per dispatch (median over the run's dispatches):")
    print(f"#   FETCH_SIZE {v_f:.1f} KiB over {m_f} dispatches -> {rd:.0f} bytes read")
    print(f"#   WRITE_SIZE {v_w:.1f} KiB over {m_w} dispatches -> {wr:.0f} bytes written "
          f"(y: {tokens} x {n} x 4 B = {tokens * n * 4})")
    print(f"#   algorithmic weight bytes per launch: {wb} -> read / algorithmic = {rd / wb:.4f}")
    print("#")
    print(f"traffic_bytes_per_launch: {rd + wr:.0f}")
    print(f"kernel_sources_sha256_16: {kernel_source_hash()}")
    print(f"matvec_variant: {variant}")
    return 0


# The metric's token sweep (q4_K and IQ4_XS at 1..16 tokens) and the other
# workload configurations, reported beside the headline by the default run.
SWEEP = (("q4_k_14336x4096", (1, 2, 4, 8, 16)), ("iq4_xs_4096x14336", (1, 2, 4, 8, 16)))
OTHER = (("q8_0_4096x4096", (1,)), ("q8_0_splitk_256x65536", (1,)), ("q8_0_head_152064x5120", (1, 16)))


def sweep_rows(torch, qmv, workload, tokens, reps=21):
    """Matvec kernel time (median over replays) of one workload at each token
    count, against the plain read of the same bytes; and the whole step
    (quantize + matvec)."""
    fmt, n, k, _, *rest = WORKLOADS[workload]
    rows, read_us = [], None
    for t in tokens:
        log(f"bench: {workload} T={t}")
        r = Ring(torch, qmv, fmt, n, k, t, workload)
        if read_us is None:
            sink = torch.zeros(1, dtype=torch.int32, device="cuda")
            read_us = timed_replays(torch, lambda i: qmv.stream_read(r.w[i % r.copies][0].view(-1), sink),
                                    max(r.copies, 32), reps)
        us = kernel_us(torch, qmv, r, reps)
        step_us = timed_replays(torch, lambda i: r.step(qmv, i), max(r.copies, 32), reps)
        vi, slices = qmv.matvec_plan(fmt, n, k, t, r.ws is not None)
        gbs = r.weight_bytes / (us * 1e-6) / 1e9
        rows.append({"workload": workload, "tokens": t, "kernel_us": round(us, 3), "weight_GBps": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "matvecs_per_s": round(1e6 / us, 1),
                     "read_ceiling_us": round(read_us, 3), "frac_of_read_ceiling": round(read_us / us, 4),
                     "step_us": round(step_us, 3),
                     "step_GBps": round(r.weight_bytes / (step_us * 1e-6) / 1e9, 1),
                     "int8_TOPS": round(2.0 * n * k * t / (us * 1e-6) / 1e12, 2),
                     "variant": qmv.variant_name(vi), "k_slices_over_workgroups": slices})
        del r
        torch.cuda.empty_cache()
    return rows


def moe_rows(torch, qmv, tokens, reps=5):
    """The MoE decode step (quantize x, routed gate+up, quantize h, routed
    and route-weighted down) at each token count: median step time; and the
    FFN step (router + top-k, gate+up with SwiGLU and Q8 of its output, down
    with the router's weights)."""
    rows = []
    for t in tokens:
        log(f"bench: MoE step T={t}")
        ring = MoeRing(torch, qmv, t)
        per = 16
        us = timed_replays(torch, lambda i: ring.step(qmv, i), per, reps)
        gu_us = timed_replays(torch, lambda i: ring.gate_up(qmv, i), per, reps)
        dn_us = timed_replays(torch, lambda i: ring.down(qmv, i), per, reps)
        # the FFN step: router + top-k, gate+up with SwiGLU and Q8, down with the router's weights
        ffn_us = timed_replays(torch, lambda i: ring.ffn_step(qmv, i), per, reps)
        fb, fu = ring.ffn_bytes(qmv, per)
        u = ring.avg_bytes(per) / ring.bytes_per_expert
        b = ring.avg_bytes(per)
        rows.append({"workload": "MoE IQ4_XS 128 experts top-8, gate+up 3072x4096 + down 4096x1536", "tokens": t,
                     "avg_distinct_experts": round(u, 2), "weight_bytes_per_step": round(b),
                     "step_us": round(us, 3), "step_GBps": round(b / (us * 1e-6) / 1e9, 1),
                     "hbm_frac_step": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "gate_up_us": round(gu_us, 3), "down_us": round(dn_us, 3),
                     "ffn_step_us": round(ffn_us, 3), "ffn_distinct_experts": round(fu, 2),
                     "ffn_step_GBps": round(fb / (ffn_us * 1e-6) / 1e9, 1)})
        del ring
        torch.cuda.empty_cache()
    return rows


READ_SWEEP_MB = (1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024)


def read_sweep(torch, qmv, reps=15):
    """The plain read's time (qmv_stream_read, median over replays) at sizes
    from 1 MiB to 1 GiB, each call on its own slice of a 2 GiB buffer (so
    that no call finds its bytes in the 256 MB Infinity Cache), and the fit
    t = t0 + bytes / BW over the sizes from 16 MiB: the fixed cost of one
    launch streaming from HBM and the rate it approaches.  A launch that
    reads B bytes can reach at most B / (t0 + B / BW) -- the ceiling the
    matvec kernels are held to."""
    pool = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows = []
    for mb in READ_SWEEP_MB:
        size = mb << 20
        copies = (2 << 30) // size
        per = max(copies, 32)
        us = timed_replays(torch, lambda i: qmv.stream_read(pool[(i % copies) * size:(i % copies + 1) * size], sink),
                           per, reps)
        rows.append({"MiB": mb, "bytes": size, "us": round(us, 3), "GBps": round(size / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(size / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
        log(f"bench: read {mb} MiB {us:.2f} us")
    pts = [(r["bytes"], r["us"]) for r in rows if r["MiB"] >= 16]
    n = len(pts)
    mx = sum(b for b, _ in pts) / n
    my = sum(u for _, u in pts) / n
    slope = sum((b - mx) * (u - my) for b, u in pts) / sum((b - mx) ** 2 for b, _ in pts)
    t0 = my - slope * mx
    bw = 1e-3 / slope  # bytes per us -> GB/s
    ceil = {wl: round(WEIGHT_BYTES[wl] / (t0 + WEIGHT_BYTES[wl] / (bw * 1e3)) / 1e3 / HBM_PEAK_GBS, 4)
            for wl in ("q4_k_14336x4096", "iq4_xs_4096x14336", "q8_0_4096x4096", "q8_0_splitk_256x65536")}
    return {"rows": rows, "fit": {"t0_us": round(t0, 3), "asymptotic_GBps": round(bw, 1),
                                  "sizes": "16 MiB .. 1 GiB"},
            "ceiling_frac_of_peak": ceil}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5000)
    ap.add_argument("--warmup", type=int, default=20000,
                    help="untimed steps before the timed ones (the default is about 0.2 s of the one-token "
                         "q4_K step: the GPU's clocks settle in about 0.1 s of continuous work)")
    ap.add_argument("--workload", default="q4_k_14336x4096",
                    choices=sorted(WORKLOADS) + [MOE["name"], MOE["ffn_name"]])
    ap.add_argument("--tokens", type=int, default=1)
    ap.add_argument("--all-tokens", action="store_true",
                    help="also time the matvec at every token count of the workload")
    ap.add_argument("--quick", action="store_true",
                    help="the headline only: no token sweep, no other configurations")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print per-kernel median/avg/min/max of a rocprofv3 kernel trace and exit")
    ap.add_argument("--counter-summary", metavar="CSV",
                    help="print per-kernel mean counter values of a rocprofv3 --pmc counter_collection.csv and exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic file of --workload/--tokens from a FETCH_SIZE and a WRITE_SIZE "
                         "counter run of --profile-launches and exit")
    ap.add_argument("--profile-launches", type=int, default=0, metavar="N",
                    help="for a profiler: run N plain launches of the workload's matvec alone (cycling the "
                         "weight ring, after N warmup launches) and exit")
    ap.add_argument("--profile-read", action="store_true",
                    help="with --profile-launches: launch the plain read of the weight bytes (qmv_stream_read) "
                         "instead of the matvec")
    ap.add_argument("--read-sweep", action="store_true",
                    help="time the plain read (qmv_stream_read) from 1 MiB to 1 GiB, fit its fixed cost and "
                         "rate, print one JSON line and exit")
    ap.add_argument("--variant", default=None,
                    help="force a matvec kernel variant by name (qmv_set_tuning 'variant')")
    args = ap.parse_args()

    if args.trace_summary is not None:
        return trace_summary(args.trace_summary)
    if args.counter_summary is not None:
        return counter_summary(args.counter_summary)
    if args.traffic_summary is not None:
        # the variant qmv_matvec plans for the workload (host-side: no GPU needed)
        import quantized_decode_gemv_qmv_amd as qmv

        fmt, n, k, *_ = WORKLOADS[args.workload]
        vi, _ = qmv.matvec_plan(fmt, n, k, args.tokens, qmv.matvec_workspace_bytes(fmt, n, k, args.tokens) > 0)
        return traffic_summary(*args.traffic_summary, args.workload, args.tokens, qmv.variant_name(vi))
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: --gpus {args.gpus} is not supported (the matvec is "
              "measured on one GPU's share of the weights; multi-GPU sharding is not built)",
              file=sys.stderr)
        return 2

    clocks = gpu_clocks()  # read before anything touches the GPU

    import torch

    import quantized_decode_gemv_qmv_amd as qmv

    qmv.lib()  # fails loudly without the HIP library
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.read_sweep:
        print(json.dumps({"read_sweep": read_sweep(torch, qmv), "device": device_info(torch, clocks)}), flush=True)
        return 0
    if args.workload in (MOE["name"], MOE["ffn_name"]):
        if not 1 <= args.tokens <= 64:
            print("--tokens must be 1..64 for the MoE workload", file=sys.stderr)
            return 2
        return bench_moe(args, torch, qmv, ffn=args.workload == MOE["ffn_name"])
    fmt, n, k, token_list, *rest = WORKLOADS[args.workload]
    mats = rest[0] if rest else 1
    t = args.tokens
    if not 1 <= t <= 16:
        print("--tokens must be 1..16", file=sys.stderr)
        return 2

    if args.variant is not None:
        if args.variant not in qmv.variants():
            print(f"unknown variant {args.variant}", file=sys.stderr)
            return 2
        qmv.set_tuning("variant", qmv.variants().index(args.variant))
    log(f"bench: {args.workload} T={t}: generating inputs")
    ring = Ring(torch, qmv, fmt, n, k, t, args.workload, mats)
    if args.profile_launches > 0:
        # plain launches (no graph) so that a profiler sees each dispatch
        qmv.quantize_act(ring.x[0], out=ring.xq)
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        for i in range(2 * args.profile_launches):
            if args.profile_read:
                for w in ring.w[i % ring.copies]:
                    qmv.stream_read(w.view(-1), sink)
            else:
                ring.matvec_only(qmv, i)
        torch.cuda.synchronize()
        log(f"bench: {args.profile_launches} profiled launches after as many warmup launches, variant "
            f"{qmv.variant_name(qmv.matvec_plan(fmt, n, k, t, ring.ws is not None)[0]) if mats == 1 else '-'}")
        return 0
    per = max(ring.copies, 64)
    g_full = capture(torch, lambda i: ring.step(qmv, i), per)
    tail = args.steps % per
    g_tail = capture(torch, lambda i: ring.step(qmv, i), tail) if tail else None
    graphs = (g_full, per, g_tail)

    log(f"bench: warmup {args.warmup} steps")
    run_steps(torch, (g_full, per, capture(torch, lambda i: ring.step(qmv, i), args.warmup % per)
                      if args.warmup % per else None), args.warmup)
    torch.cuda.synchronize()

    # exactly --steps steps between two device synchronizations; HIP events
    # on the same stream give their GPU time, the host clock the wall time
    log(f"bench: timing {args.steps} steps")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    run_steps(torch, graphs, args.steps)
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    wall_ms_per_step = elapsed * 1e3 / args.steps
    value = ring.weight_bytes / (ms_per_step * 1e-3) / 1e9

    kus = kernel_us(torch, qmv, ring)
    achieved = ring.weight_bytes / (kus * 1e-6) / 1e9
    # the same step through qmv_matvec_x (fp32 activations in, quantization
    # fused into the matvec where that is faster)
    fused_us = timed_replays(torch, lambda i: ring.fused(qmv, i), max(ring.copies, 32)) if mats == 1 else None
    # the plain read of the same weight bytes (qmv_stream_read over the same
    # ring): the practical ceiling of one launch streaming them
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    read_us = timed_replays(torch, lambda i: [qmv.stream_read(w.view(-1), sink) for w in ring.w[i % ring.copies]],
                            max(ring.copies, 32))
    src_hash = kernel_source_hash()
    # a batch of equal matrices runs the variant of their stacked rows (each
    # matrix padded to a multiple of 64 rows)
    if mats > 1:
        variant, slices = qmv.variant_name(qmv.pick_variant(fmt, mats * ((n + 63) // 64 * 64), k, t)), 1
    else:
        vi, slices = qmv.matvec_plan(fmt, n, k, t, ring.ws is not None)
        variant = qmv.variant_name(vi)
    traffic = recorded_traffic(args.workload, t, src_hash, variant)

    by_tokens = []
    if args.all_tokens:
        for tt in token_list:
            r2 = ring if tt == t else Ring(torch, qmv, fmt, n, k, tt, args.workload, mats)
            us = kernel_us(torch, qmv, r2)
            rec = {"tokens": tt, "kernel_us": round(us, 3),
                   "weight_GBps": round(r2.weight_bytes / (us * 1e-6) / 1e9, 1),
                   "hbm_frac": round(r2.weight_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "matvecs_per_s": round(1e6 / us, 1),
                   "variant": qmv.variant_name(qmv.matvec_plan(fmt, n, k, tt, r2.ws is not None)[0]
                                               if mats == 1 else qmv.pick_variant(fmt, mats * n, k, tt))}
            if mats > 1:
                rec["separate_launches_us"] = round(timed_replays(torch, lambda i: r2.separate(qmv, i),
                                                                  max(r2.copies, 32)), 3)
            by_tokens.append(rec)
            log(f"bench: T={tt} kernel {us:.2f} us")
            if r2 is not ring:
                del r2
                torch.cuda.empty_cache()

    sweep, others, moe = [], [], []
    default_run = args.workload == "q4_k_14336x4096" and t == 1 and not args.quick and not args.all_tokens
    if default_run:
        del ring, g_full, g_tail, graphs
        torch.cuda.empty_cache()
        for wl, toks in SWEEP:
            sweep += sweep_rows(torch, qmv, wl, toks)
        for wl, toks in OTHER:
            others += sweep_rows(torch, qmv, wl, toks, reps=11)
        moe = moe_rows(torch, qmv, (1, 6, 16, 64))

    cpu = None
    if not args.no_cpu:
        log("bench: CPU oracle baseline")
        cpu = cpu_baseline(fmt, n, k, t, args.workload)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": (f"{FMT_NAME[fmt]} matvec {n}x{k}, {t} token(s)" if mats == 1 else
                                f"{mats} sibling {FMT_NAME[fmt]} matvecs {n}x{k} in one launch, {t} token(s)"),
                   "format": FMT_NAME[fmt], "n_rows": n, "k": k, "tokens": t, "matrices": mats,
                   "weight_bytes": ring.weight_bytes if not default_run else WEIGHT_BYTES[args.workload],
                   "step": "qmv_quantize_act + " + ("qmv_matvec" if mats == 1 else "qmv_matvec_batch"),
                   "matvec_variant": variant, "k_slices_over_workgroups": slices},
        "ms_per_step_wall": round(wall_ms_per_step, 6),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "matvecs_per_s": round(1e3 / ms_per_step, 1),
        **({"matvec_x_step_us": round(fused_us, 3),
            "matvec_x_step_GBps": round(WEIGHT_BYTES.get(args.workload, 0) / (fused_us * 1e-6) / 1e9, 1)}
           if fused_us and args.workload in WEIGHT_BYTES else {}),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_us": round(kus, 3), "kernel_us_stat": "median over replays",
                     "algorithmic_bytes_per_launch": WEIGHT_BYTES.get(args.workload, 0) * mats,
                     "kernel_sources_sha256_16": src_hash},
        "read_ceiling": {"kernel_us": round(read_us, 3),
                         "GBps": round(WEIGHT_BYTES.get(args.workload, 0) * mats / (read_us * 1e-6) / 1e9, 1),
                         "frac_of_peak": round(WEIGHT_BYTES.get(args.workload, 0) * mats / (read_us * 1e-6) / 1e9
                                               / HBM_PEAK_GBS, 4),
                         "matvec_frac_of_ceiling": round(read_us / kus, 4),
                         "launches": mats},
        "device": device_info(torch, clocks),
        "cpu_baseline": cpu,
    }
    if by_tokens:
        out["by_tokens"] = by_tokens
    if sweep:
        out["by_tokens"] = sweep
        out["other_configs"] = others
        out["moe_steps"] = moe
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
