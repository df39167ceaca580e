"""Benchmark of the Mamba-3 scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

One step = one pass of the hot path over one batch: m3_state_zero + one
mamba3_prefill of the 1.5B-scale SISO layer (batch 8, 32 heads, headdim 64,
state 128, 4096 tokens, chunk 64, bf16 I/O, fp32 state), inputs resident in
HBM before the timed region.  `value` is prefill throughput in Mtokens/s
(tokens = batch x seqlen, all heads).  The default 200 warm-up steps (~60 ms)
let the GPU reach its steady clocks, which takes ~100 steps from idle; with
only a few warm-up steps the timed region measures the clock ramp.  The same JSON line carries:
  roofline      -- the prefill kernel's algorithmic HBM bytes per launch over
                   its average duration (HIP events on the launch stream),
                   against the MI355X HBM peak of 8 TB/s; `traffic` comes from
                   committed rocprofv3 FETCH_SIZE / WRITE_SIZE counters when
                   they were taken on the current kernel source, else null;
  cpu_baseline  -- the fp64 oracle timed on the host on a bounded sample, one
                   thread (the value) and over all host cores (`all_cores`);
                   the decode entries carry the oracle's ms per step;
  extra         -- decode step (256 x 32 heads, MIMO R=4 N=64 and SISO N=128;
                   1000 steps captured in a HIP graph, plus a run with a
                   512 MiB cache flush between steps), MIMO / 16K-token
                   prefill throughput, the headline shape under the other two
                   discretisation rules and with fp32 I/O, and the gated entry points (pre-gate
                   grouped RMSNorm fused into the store of y) on the headline
                   prefill and both decode shapes, BC normalisation, the MIMO
                   rank down-projection, and the backward pass (all gradients)
                   on the SISO and MIMO prefill shapes.
Prints exactly one JSON line (rank 0).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "state_space_sequence_prefill_amd", "csrc")
# sources whose code the fused prefill launch runs (kernel, device helpers)
HEADLINE = "siso_1p5b_t4096"
METRIC = "Mamba-3 scan prefill Mtokens/s + decode \u00b5s/step; % of MFMA / HBM peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_bytes(w):
    """Algorithmic HBM bytes of one prefill launch: every input read once, y
    written once, the state (h, pending pair) read once and written once."""
    io = 2 if w.io_dtype == "bf16" else 4
    th = w.batch * w.seqlen * w.heads          # token-heads
    per_th = w.rank * (w.headdim + 2 * w.dstate) * io + 8 + (w.dstate // 2) * 4 + w.rank * w.headdim * io
    chains = w.batch * w.heads
    state = chains * (w.headdim * w.dstate * 4 + w.rank * (w.dstate + w.headdim) * io)
    return th * per_th + 2 * state


def prefill_flops(w):
    """Chunked-form FLOPs (full tiles): per token-head 4 R N P + 2 Q R^2 (N + P)."""
    th = w.batch * w.seqlen * w.heads
    return th * (4 * w.rank * w.dstate * w.headdim + 2 * w.chunk * w.rank ** 2 * (w.dstate + w.headdim))


def backward_bytes(w):
    """Algorithmic HBM bytes of one backward pass: every prefill input and dy
    read once, every gradient written once (fp32), the entry state read and
    its gradient written once.  The workspace round trips of the unit
    summaries are the design's own traffic and are reported beside it."""
    io = 2 if w.io_dtype == "bf16" else 4
    th = w.batch * w.seqlen * w.heads
    nh = w.dstate // 2
    reads = w.rank * (2 * w.headdim + 2 * w.dstate) * io + 8 + nh * 4
    writes = w.rank * (w.headdim + 2 * w.dstate) * 4 + 8 + nh * 4
    chains = w.batch * w.heads
    state = chains * (w.headdim * w.dstate * 4 + w.rank * (w.dstate + w.headdim) * io)
    return th * (reads + writes) + state + chains * (w.headdim * w.dstate + w.rank * (w.dstate + w.headdim)) * 4


def backward_workspace_traffic(w):
    """Bytes the backward moves through its workspace: the unit summaries U and
    V are written (local), read and overwritten by E and G (scan), and read
    (grad): eight passes over (units x P x N) fp32 per chain."""
    qu = 64 // w.rank
    units = (w.seqlen + qu - 1) // qu
    return 8 * w.batch * w.heads * units * w.headdim * w.dstate * 4


def gate_bytes(w, tokens):
    """Extra bytes of the output epilogue: the gate input z (one I/O element
    per output) and the fp32 channel weights."""
    e = 2 if w.io_dtype == "bf16" else 4
    return w.batch * tokens * w.heads * w.rank * w.headdim * e + w.heads * w.headdim * 4


def down_bytes_delta(w, tokens):
    """Change in bytes when the R rank outputs are folded into P channels
    before the epilogue: y and z lose the rank axis, the fp32 projection
    weights (heads, R, P) are read once."""
    e = 2 if w.io_dtype == "bf16" else 4
    rows = w.batch * tokens * w.heads * w.headdim
    return -2 * (w.rank - 1) * rows * e + w.heads * w.rank * w.headdim * 4


def decode_bytes(w):
    """Algorithmic bytes of one decode step: h read + written, pending pair
    read + written, one token of x, B, C, dt, lam, theta read, y written."""
    io = 2 if w.io_dtype == "bf16" else 4
    ch = w.batch * w.heads
    h = ch * w.headdim * w.dstate * 4
    pend = ch * w.rank * (w.dstate + w.headdim) * io
    tok = ch * (w.rank * (w.headdim + 2 * w.dstate) * io + 8 + (w.dstate // 2) * 4)
    y = ch * w.rank * w.headdim * io
    return 2 * h + 2 * pend + tok + y


# sources whose code each profiled workload runs (kernels, device helpers)
SRCS = {
    "prefill": ("m3_prefill_pc.hpp", "m3_prefill_pc.hip", "m3_mfma.hpp", "m3_device.hpp"),
    "segments": ("m3_prefill_pc.hpp", "m3_prefill_pc.hip", "m3_prefill.hip", "m3_mfma.hpp", "m3_device.hpp"),
    "decode": ("m3_decode.hip", "m3_decode_mimo.hip", "m3_device.hpp"),
}
# kernels whose dispatches make up one step of each kind
KERNELS = {
    "prefill": ("prefill_pc_kernel", "prefill_kernel<"),
    "segments": ("prefill_pc_kernel", "prefill_kernel<", "segment_scan_kernel"),
    "decode": ("decode_kernel", "decode_mimo_kernel"),
}


def workload_kind(name):
    if name.startswith("decode"):
        return "decode"
    return "segments" if name == "long_siso_t16384" else "prefill"


def source_sha(kind="prefill"):
    h = hashlib.sha256()
    for name in SRCS[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload_name):
    return os.path.join(PROFILES, f"traffic_{workload_name}.json")


def committed_traffic(workload_name):
    """Per-step HBM bytes measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters (scaled by the copy-kernel calibration), if they were recorded
    for the current kernel sources (profiles/traffic_<workload>.json)."""
    p = traffic_path(workload_name)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != source_sha(workload_kind(workload_name)):
        return None
    return rec.get("bytes_per_step")


RAMP_MIN_LAUNCHES = 200
RAMP_MIN_MS = 100.0
# each extra prefill workload: a shorter declared ramp of its own before its
# warm-up, since the decode steps timed before it leave the clocks elsewhere
EXTRA_RAMP_LAUNCHES = 40
EXTRA_RAMP_MS = 20.0


class Prefill:
    def __init__(self, w, seed, long_memory=False, disc="exp_trapezoid", gated=False, down=False, bcnorm=False):
        import torch
        import state_space_sequence_prefill_amd as m3
        from state_space_sequence_prefill_amd import synthetic as syn
        self.m3, self.torch, self.w = m3, torch, w
        self.d = m3.make_dims(w.batch, w.heads, w.headdim, w.dstate, w.rank, w.chunk, w.io_dtype, disc)
        self.inp = syn.draw_torch(w, seed, long_memory=long_memory)
        self.state = m3.State.empty(self.d)
        yshape = (w.batch, w.seqlen, w.heads, w.headdim) if down else (w.batch, w.seqlen, w.heads, w.rank, w.headdim)
        self.y = torch.empty(yshape, dtype=self.inp["x"].dtype, device="cuda")
        nws = m3.mamba3_prefill_workspace_bytes(self.d, w.seqlen)
        self.ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
        self.nlaunch = 1 if not nws else 3
        self.gate = syn.draw_gate_torch(w, seed + 1, folded=down) if gated or down else None
        self.bcnorm = None
        if bcnorm:
            g = torch.Generator(device="cuda")
            g.manual_seed(seed + 2)
            self.bcnorm = tuple(torch.rand((w.heads, w.dstate), generator=g, device="cuda") + 0.5
                                for _ in range(2)) + (1e-6,)

    def step(self, ev=None):
        i = self.inp
        self.m3.m3_state_zero(self.d, self.state)
        if ev is not None:
            ev[0].record()
        if self.bcnorm is not None:
            gate = None if self.gate is None else (self.gate[0], self.gate[1], 1e-5)
            self.m3.mamba3_prefill_ex(self.d, self.w.seqlen, i["x"], i["B"], i["C"], i["dt"], i["lam"], i["theta"],
                                      i["A"], i["D"], self.state, self.y, bcnorm=self.bcnorm, gate=gate,
                                      workspace=self.ws)
        elif self.gate is None:
            self.m3.mamba3_prefill(self.d, self.w.seqlen, i["x"], i["B"], i["C"], i["dt"], i["lam"], i["theta"],
                                   i["A"], i["D"], self.state, self.y, self.ws)
        else:
            z, gw = self.gate[:2]
            dw = self.gate[2] if len(self.gate) > 2 else None
            self.m3.mamba3_prefill_gated(self.d, self.w.seqlen, i["x"], i["B"], i["C"], i["dt"], i["lam"],
                                         i["theta"], i["A"], i["D"], z, gw, 1e-5, self.state, self.y, self.ws,
                                         down=dw)
        if ev is not None:
            ev[1].record()

    def ramp(self, min_launches, min_ms):
        """Untimed steps until at least min_launches launches and min_ms of
        wall time have passed (the GPU's clocks settle meanwhile)."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 0
        while n < min_launches or (time.perf_counter() - t0) * 1e3 < min_ms:
            for _ in range(20):
                self.step()
            n += 20
            torch.cuda.synchronize()
        return {"launches": n, "ms": round((time.perf_counter() - t0) * 1e3, 1)}

    def time_extra(self, steps):
        """An extra workload: its own declared ramp, then 2 warm-up and
        `steps` timed steps."""
        self.ramp(EXTRA_RAMP_LAUNCHES, EXTRA_RAMP_MS)
        return self.time(steps, 2)

    def time(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            self.step(evs[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
        return wall / steps * 1e3, kern_ms


def time_backward(w, seed, steps, warmup):
    """Time mamba3_prefill_backward (all four launches) on one workload."""
    import torch
    import state_space_sequence_prefill_amd as m3
    from state_space_sequence_prefill_amd import synthetic as syn
    d = m3.make_dims(w.batch, w.heads, w.headdim, w.dstate, w.rank, w.chunk, w.io_dtype)
    inp = syn.draw_torch(w, seed)
    T = w.seqlen
    state = m3.State.empty(d)
    m3.m3_state_zero(d, state)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    dy = torch.randn((w.batch, T, w.heads, w.rank, w.headdim), generator=g, device="cuda").to(inp["x"].dtype)
    grads = {k: torch.empty(v, dtype=torch.float32, device="cuda") for k, v in m3.grad_shapes(d, T).items()}
    ws = torch.empty(m3.mamba3_prefill_backward_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")

    def run():
        m3.mamba3_prefill_backward(d, T, inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"],
                                   inp["A"], inp["D"], state, dy, grads, workspace=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nb = backward_bytes(w)
    wt = backward_workspace_traffic(w)
    out = {"ms_per_step": round(ms, 4), "Mtokens_per_s": round(w.batch * T / ms / 1e3, 3),
           "algorithmic_bytes": nb, "hbm_frac": round(nb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
           "workspace_bytes": ws.numel(), "workspace_traffic_bytes": wt,
           "hbm_frac_with_workspace": round((nb + wt) / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    del grads, ws
    torch.cuda.empty_cache()
    return out


def time_decode(w, seed, steps=1000, flush_steps=20, gated=False, down=False, bcnorm=False):
    import torch
    import state_space_sequence_prefill_amd as m3
    from state_space_sequence_prefill_amd import synthetic as syn
    d = m3.make_dims(w.batch, w.heads, w.headdim, w.dstate, w.rank, w.chunk, w.io_dtype)
    nset = 16
    toks = syn.draw_torch(w, seed, seqlen=nset)
    sets = [{k: (v[:, j].contiguous() if v.dim() >= 3 else v) for k, v in toks.items()} for j in range(nset)]
    st = m3.State.empty(d)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    st.h.copy_(torch.randn(st.h.shape, generator=g, device="cuda"))
    st.B_prev.copy_(torch.randn(st.B_prev.shape, generator=g, device="cuda").to(st.B_prev.dtype))
    st.x_prev.copy_(torch.randn(st.x_prev.shape, generator=g, device="cuda").to(st.x_prev.dtype))
    y = torch.empty((w.batch, w.heads, w.headdim) if down else (w.batch, w.heads, w.rank, w.headdim),
                    dtype=toks["x"].dtype, device="cuda")
    dw = None
    if down:
        z, gw, dw = syn.draw_gate_torch(w, seed + 2, folded=True)
        z = z[:, 0].contiguous()
        gated = True
    elif gated:
        z, gw = syn.draw_gate_torch(w, seed + 2)
        z = z[:, 0].contiguous()

    nb = None
    if bcnorm:
        gg = torch.Generator(device="cuda")
        gg.manual_seed(seed + 3)
        nb = tuple(torch.rand((w.heads, w.dstate), generator=gg, device="cuda") + 0.5 for _ in range(2)) + (1e-6,)

    def one(j):
        s = sets[j % nset]
        if bcnorm:
            m3.mamba3_decode_step_ex(d, s["x"], s["B"], s["C"], s["dt"], s["lam"], s["theta"], s["A"], s["D"], st, y,
                                     bcnorm=nb, gate=(z, gw, 1e-5) if gated else None)
        elif gated:
            m3.mamba3_decode_step_gated(d, s["x"], s["B"], s["C"], s["dt"], s["lam"], s["theta"], s["A"], s["D"],
                                        z, gw, 1e-5, st, y, down=dw)
        else:
            m3.mamba3_decode_step(d, s["x"], s["B"], s["C"], s["dt"], s["lam"], s["theta"], s["A"], s["D"], st,
                                  y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for j in range(8):
            one(j)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    per_graph = 100
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(per_graph):
            one(j)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us_graph = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
    # cache-flushed: a 512 MiB write between steps evicts the state from the
    # 256 MB Infinity Cache, so the step streams the state from HBM
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    tot = 0.0
    for j in range(flush_steps):
        flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        one(j)
        b.record()
        torch.cuda.synchronize()
        tot += a.elapsed_time(b)
    us_flush = tot * 1e3 / flush_steps
    nb = decode_bytes(w) + (gate_bytes(w, 1) if gated else 0) + (down_bytes_delta(w, 1) if down else 0)
    nb += 2 * w.heads * w.dstate * 4 if bcnorm else 0
    return {
        "workload": w.name + ("_bcnorm" if bcnorm else "") + ("_down_gated" if down else "_gated" if gated else ""), "batch": w.batch, "heads": w.heads, "headdim": w.headdim, "dstate": w.dstate,
        "rank": w.rank, "us_per_step_graph": round(us_graph, 2), "steps_graph": reps * per_graph,
        "us_per_step_flushed": round(us_flush, 2), "bytes_per_step": nb,
        "hbm_GBs_graph": round(nb / us_graph / 1e3, 1), "hbm_frac_graph": round(nb / us_graph / 1e3 / HBM_PEAK_GBS, 4),
        "hbm_GBs_flushed": round(nb / us_flush / 1e3, 1),
        "hbm_frac_flushed": round(nb / us_flush / 1e3 / HBM_PEAK_GBS, 4),
    }


def cpu_baseline(w, min_seconds=10.0):
    """The fp64 oracle, unchanged, on the host, single-threaded numpy: whole
    batch rows of the workload (all heads, all tokens), one at a time, until
    at least `min_seconds` of CPU time have been spent (at most all rows)."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import contextlib
    import oracle
    from state_space_sequence_prefill_amd import synthetic as syn
    ws = w.with_(batch=1)
    ctx = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    rows, spent = 0, 0.0
    with ctx:
        while rows < w.batch and spent < min_seconds:
            ex = syn.as_exact(syn.draw(ws, 1001 + rows), w.io_dtype)
            t0 = time.perf_counter()
            oracle.prefill(ex["x"], ex["B"], ex["C"], ex["dt"], ex["lam"], ex["theta"], ex["A"], ex["D"])
            spent += time.perf_counter() - t0
            rows += 1
    toks = rows * ws.seqlen
    return {"value": round(toks / spent / 1e6, 8), "unit": "Mtokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of {w.batch} batch rows ({w.heads} heads x {w.seqlen} tokens each), "
                      f"numpy fp64 sequential, one thread, {spent:.1f} s",
            "seconds": round(spent, 2), "cpu": _cpu_model(), "host_cpus": os.cpu_count()}


def _oracle_task(args):
    """One batch row of the workload, a slice of its heads, through the
    oracle (run in a worker process; single-threaded numpy)."""
    name, row, h0, h1 = args
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        pass
    import oracle
    from state_space_sequence_prefill_amd import synthetic as syn
    w = syn.WORKLOADS[name]
    ex = syn.as_exact(syn.draw(w.with_(batch=1), 1001 + row), w.io_dtype)
    sl = {k: (v[:, :, h0:h1] if v.ndim >= 3 else v[h0:h1]) for k, v in ex.items()}
    t0 = time.perf_counter()
    oracle.prefill(sl["x"], sl["B"], sl["C"], sl["dt"], sl["lam"], sl["theta"], sl["A"], sl["D"])
    return time.perf_counter() - t0


def cpu_baseline_all_cores(w, max_workers=16):
    """The same oracle over every batch row, each split into two head halves,
    one task per worker process on the host's cores (at most `max_workers`,
    the host share of one GPU); wall time of the parallel region."""
    import multiprocessing as mp
    workers = max(1, min(max_workers, os.cpu_count() or 1))
    tasks = [(w.name, r, h0, h0 + w.heads // 2) for r in range(w.batch) for h0 in (0, w.heads // 2)]
    ctx = mp.get_context("spawn")  # children never touch the GPU
    try:
        with ctx.Pool(workers) as pool:
            pool.map_async(_cpu_model_noop, range(workers)).get(timeout=300)  # workers up before the clock
            t0 = time.perf_counter()
            per_task = pool.map_async(_oracle_task, tasks).get(timeout=600)
            wall = time.perf_counter() - t0
    except Exception as e:  # a worker that cannot start must not hang the bench
        return {"error": f"{type(e).__name__}: {e}"}
    toks = w.batch * w.seqlen
    return {"value": round(toks / wall / 1e6, 8), "unit": "Mtokens/s", "cores": workers, "kind": "oracle",
            "sample": f"all {w.batch} batch rows, each as two halves of the {w.heads} heads, {len(tasks)} tasks over "
                      f"{workers} processes (numpy fp64, one thread each), {wall:.1f} s wall, "
                      f"{sum(per_task):.1f} s summed task time"}


def _cpu_model_noop(_):
    return 0


def cpu_decode_ms(w, steps=3):
    """The oracle's decode step on one decode workload (all batch x heads at
    once, numpy fp64, one thread): milliseconds per step over `steps` steps."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import contextlib
    import oracle
    from state_space_sequence_prefill_amd import synthetic as syn
    ex = syn.as_exact(syn.draw(w, 2001, seqlen=steps), w.io_dtype)
    state = None
    ctx = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    with ctx:
        t0 = time.perf_counter()
        for t in range(steps):
            _, state = oracle.decode_step(ex["x"][:, t], ex["B"][:, t], ex["C"][:, t], ex["dt"][:, t],
                                          ex["lam"][:, t], ex["theta"][:, t], ex["A"], ex["D"], state)
        el = time.perf_counter() - t0
    return round(el / steps * 1e3, 2)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def profile_prefill(steps, name):
    """A few untimed prefill steps of one workload (for rocprofv3)."""
    import torch
    from state_space_sequence_prefill_amd import synthetic as syn
    pf = Prefill(syn.WORKLOADS[name], seed=1001)
    for _ in range(steps):
        pf.step()
    torch.cuda.synchronize()
    log(f"bench: {steps} prefill steps of {name} done")


def profile_decode(steps, name):
    """A few untimed decode steps of one workload, each after a 512 MiB write
    that evicts the state from the Infinity Cache (for rocprofv3: the decode
    kernel then streams its state from HBM)."""
    import torch
    import state_space_sequence_prefill_amd as m3
    from state_space_sequence_prefill_amd import synthetic as syn
    w = syn.WORKLOADS[name]
    d = m3.make_dims(w.batch, w.heads, w.headdim, w.dstate, w.rank, w.chunk, w.io_dtype)
    tok = syn.draw_torch(w, 7, seqlen=1)
    tok = {k: (v[:, 0].contiguous() if v.dim() >= 3 else v) for k, v in tok.items()}
    st = m3.State.empty(d)
    st.h.normal_()
    st.B_prev.zero_()
    st.x_prev.zero_()
    y = torch.empty((w.batch, w.heads, w.rank, w.headdim), dtype=tok["x"].dtype, device="cuda")
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    for _ in range(steps):
        flush.zero_()
        m3.mamba3_decode_step(d, tok["x"], tok["B"], tok["C"], tok["dt"], tok["lam"], tok["theta"], tok["A"],
                              tok["D"], st, y)
    torch.cuda.synchronize()
    log(f"bench: {steps} flushed decode steps of {name} done")


def profile_copy(steps):
    """Copies of a known size through the library's copy kernel (m3_state_load
    of a 256 x 32 x 64 x 128 state: the fp32 h of 256 MiB and the bf16 pending
    pair of 3 MiB, read and written in one launch): the calibration for
    rocprofv3's FETCH_SIZE / WRITE_SIZE."""
    import torch
    import state_space_sequence_prefill_amd as m3
    d = m3.make_dims(256, 32, 64, 128, 1, 64, "bf16")
    dst = m3.State.empty(d)
    src = m3.State.empty(d)
    src.h.fill_(1.0)
    src.B_prev.zero_()
    src.x_prev.zero_()
    for _ in range(steps):
        m3.m3_state_load(d, dst, src.h, src.B_prev, src.x_prev)
    torch.cuda.synchronize()
    log(f"bench: {steps} state copies of {dst.h.numel() * 4 + dst.B_prev.numel() * 2 + dst.x_prev.numel() * 2} bytes done")


def measured_copy_gbs(steps=20):
    """Achieved HBM bandwidth of a plain copy on this GPU: the library's copy
    kernel moving a 256 MiB fp32 state (m3_state_load; read + written bytes
    over the average launch time, HIP events), beside the 8 TB/s spec."""
    import torch
    import state_space_sequence_prefill_amd as m3
    d = m3.make_dims(256, 32, 64, 128, 1, 64, "bf16")
    dst = m3.State.empty(d)
    src = m3.State.empty(d)
    src.h.fill_(1.0)
    src.B_prev.zero_()
    src.x_prev.zero_()
    for _ in range(5):
        m3.m3_state_load(d, dst, src.h, src.B_prev, src.x_prev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        m3.m3_state_load(d, dst, src.h, src.B_prev, src.x_prev)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    moved = 2 * (dst.h.numel() * 4 + dst.B_prev.numel() * dst.B_prev.element_size()
                 + dst.x_prev.numel() * dst.x_prev.element_size())
    del dst, src
    torch.cuda.empty_cache()
    return round(moved / (ms / 1e3) / 1e9, 1)


PROBE_LIB = os.path.join(ROOT, "state_space_sequence_prefill_amd", "libm3probe.so")


def probe_bandwidth(mib=1024, steps=10, blocks=(256, 512, 1024, 2048, 4096)):
    """Streaming ceilings of this GPU from the probe kernels (libm3probe.so,
    built beside the scan library): read-only, write-only and copy over a
    `mib` MiB buffer (twice the 256 MB Infinity Cache), each at several
    workgroup counts; GB/s of bytes moved over the average launch time (HIP
    events), best workgroup count reported."""
    import ctypes
    import torch
    L = ctypes.CDLL(PROBE_LIB)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.m3probe_read.argtypes = [vp, sz, vp, ctypes.c_int, vp]
    L.m3probe_write.argtypes = [vp, sz, ctypes.c_int, vp]
    L.m3probe_copy.argtypes = [vp, vp, sz, ctypes.c_int, vp]
    nbytes = mib * 1024 * 1024
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    out = torch.empty(max(blocks), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    runs = {
        "read": (lambda nb: L.m3probe_read(a.data_ptr(), nbytes, out.data_ptr(), nb, st), nbytes),
        "write": (lambda nb: L.m3probe_write(b.data_ptr(), nbytes, nb, st), nbytes),
        "copy": (lambda nb: L.m3probe_copy(b.data_ptr(), a.data_ptr(), nbytes, nb, st), 2 * nbytes),
    }
    res = {}
    for name, (fn, moved) in runs.items():
        best = (0.0, 0)
        for nb in blocks:
            for _ in range(3):
                assert fn(nb) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn(nb)
            e1.record()
            torch.cuda.synchronize()
            gbs = moved / (e0.elapsed_time(e1) / steps / 1e3) / 1e9
            best = max(best, (round(gbs, 1), nb))
        res[f"{name}_GBs"] = best[0]
        res[f"{name}_workgroups"] = best[1]
    res["buffer_MiB"] = mib
    del a, b, out
    torch.cuda.empty_cache()
    return res


def _counter_per_dispatch(run_dir, counter, kernel_substr, largest=False):
    """Mean (or, with largest, the maximum) value per dispatch of a counter
    from a rocprofv3 counter_collection.csv under run_dir."""
    import csv
    import glob
    tot = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    key = (f, r["Dispatch_Id"])
                    tot[key] = tot.get(key, 0.0) + float(r["Counter_Value"])
    if not tot:
        raise SystemExit(f"no {counter} rows for {kernel_substr} under {run_dir}")
    vals = list(tot.values())
    return max(vals) if largest else sum(vals) / len(vals)


def _counter_by_dispatch(run_dir, counter, kernel_substrs):
    """{(file, dispatch id): (kernel name, summed value)} of a counter from
    the rocprofv3 counter_collection.csv files under run_dir, for the
    dispatches whose kernel name contains one of kernel_substrs."""
    import csv
    import glob
    tot = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and any(k in r["Kernel_Name"] for k in kernel_substrs):
                    key = (f, r["Dispatch_Id"])
                    name, v = tot.get(key, (r["Kernel_Name"], 0.0))
                    tot[key] = (name, v + float(r["Counter_Value"]))
    if not tot:
        raise SystemExit(f"no {counter} rows for {kernel_substrs} under {run_dir}")
    return tot


def record_traffic(base, name, steps):
    """Write profiles/traffic_<workload>.json from four rocprofv3 counter
    runs under `base`: <workload>_fetch, <workload>_write (FETCH_SIZE /
    WRITE_SIZE over `steps` profiled steps of the workload) and copy_fetch,
    copy_write (the same counters for the 259 MiB state copy).  Counters are KiB
    per dispatch; each is scaled by known copy bytes / the copy's reading.
    Per step: the sum over every dispatch of the step's kernels / steps."""
    copy_bytes = 256 * 32 * (64 * 128 * 4 + 128 * 2 + 64 * 2)  # h, B_prev, x_prev of the calibration copy
    cf = _counter_per_dispatch(os.path.join(base, "copy_fetch"), "FETCH_SIZE", "copy_kernel", largest=True) * 1024
    cw = _counter_per_dispatch(os.path.join(base, "copy_write"), "WRITE_SIZE", "copy_kernel", largest=True) * 1024
    kind = workload_kind(name)
    fetch = _counter_by_dispatch(os.path.join(base, f"{name}_fetch"), "FETCH_SIZE", KERNELS[kind])
    write = _counter_by_dispatch(os.path.join(base, f"{name}_write"), "WRITE_SIZE", KERNELS[kind])
    kf, kw = copy_bytes / cf, copy_bytes / cw
    per_kernel = {}
    for recs, field, k in ((fetch, "fetch_bytes", kf), (write, "write_bytes", kw)):
        for kname, v in recs.values():
            short = next(x for x in KERNELS[kind] if x in kname).rstrip("<")
            e = per_kernel.setdefault(short, {"dispatches": 0, "fetch_bytes": 0.0, "write_bytes": 0.0})
            e[field] += v * 1024 * k
            if field == "fetch_bytes":
                e["dispatches"] += 1
    for e in per_kernel.values():
        e["fetch_bytes_per_dispatch"] = round(e.pop("fetch_bytes") / e["dispatches"])
        e["write_bytes_per_dispatch"] = round(e.pop("write_bytes") / e["dispatches"])
        e["dispatches_per_step"] = e.pop("dispatches") / steps
    total = sum(e["dispatches_per_step"] * (e["fetch_bytes_per_dispatch"] + e["write_bytes_per_dispatch"])
                for e in per_kernel.values())
    from state_space_sequence_prefill_amd import synthetic as syn
    w = syn.WORKLOADS[name]
    alg = decode_bytes(w) if kind == "decode" else prefill_bytes(w)
    rec = {"workload": name, "kernels": per_kernel, "kernel_source_sha": source_sha(kind),
           "copy_fetch_scale": kf, "copy_write_scale": kw, "profiled_steps": steps,
           "bytes_per_step": round(total), "algorithmic_bytes_per_step": alg, "ratio": round(total / alg, 4)}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_path(name), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def summarize_counters(run_dir, name):
    """SQ / GRBM counters of one rocprofv3 --pmc run over profiled steps of a
    prefill workload: per dispatch of the main kernel, plus the derived MFMA
    utilisation (busy cycles of the matrix units over the kernel's cycles x
    1024 SIMDs), the bf16 MFMA FLOPs, the share of a CU's cycles its LDS
    stalls on bank conflicts and the share of a SIMD's cycles spent issuing
    VALU instructions (4 cycles per wave64 instruction)."""
    import csv
    import glob
    kind = workload_kind(name)
    acc = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if not any(k in r["Kernel_Name"] for k in KERNELS[kind]):
                    continue
                key = (f, r["Dispatch_Id"])
                d = acc.setdefault(key, {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not acc:
        raise SystemExit(f"no counter rows under {run_dir}")
    names = sorted({c for d in acc.values() for c in d})
    mean = {c: sum(d.get(c, 0.0) for d in acc.values()) / len(acc) for c in names}
    out = {"workload": name, "dispatches": len(acc), "per_dispatch": {c: round(v, 1) for c, v in mean.items()}}
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "GRBM_GUI_ACTIVE" in mean:
        # GRBM_GUI_ACTIVE comes summed over the 8 XCDs (each counts the
        # kernel's cycles); the matrix units' busy cycles over all 1024 SIMDs
        cycles = mean["GRBM_GUI_ACTIVE"] / 8
        out["gpu_cycles"] = round(cycles)
        out["mfma_busy_frac"] = round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * 1024), 4)
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in mean:
        out["mfma_bf16_flops"] = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    if "gpu_cycles" in out:
        cyc = out["gpu_cycles"]
        if "SQ_LDS_BANK_CONFLICT" in mean:  # cycles the LDS of a CU stalls on bank conflicts, over the kernel's
            out["lds_bank_conflict_frac_per_cu"] = round(mean["SQ_LDS_BANK_CONFLICT"] / (256 * cyc), 4)
        if "SQ_INSTS_VALU" in mean:  # wave64 VALU issue (4 cycles each) per SIMD, over the kernel's cycles
            out["valu_issue_frac_per_simd"] = round(4 * mean["SQ_INSTS_VALU"] / (1024 * cyc), 4)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--profile-prefill", type=int, default=0, metavar="K",
                    help="only run K untimed prefill steps of --workload (for rocprofv3)")
    ap.add_argument("--profile-decode", type=int, default=0, metavar="K",
                    help="only run K untimed cache-flushed decode steps of --workload (for rocprofv3)")
    ap.add_argument("--profile-copy", type=int, default=0, metavar="K",
                    help="only run K 256 MiB copies (counter calibration)")
    ap.add_argument("--probe-bandwidth", action="store_true",
                    help="only print the streaming read / write / copy ceilings (probe kernels)")
    ap.add_argument("--workload", default=None, help="workload of the profile and record modes")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write profiles/traffic_<workload>.json from rocprofv3 counter runs under DIR (no GPU)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print the SQ/GRBM counters of a rocprofv3 --pmc run under DIR (no GPU)")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic, args.workload or HEADLINE, args.profile_prefill or args.profile_decode)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload or HEADLINE)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every (batch, head) chain of the scan is independent, so "
              "N GPUs would run the same kernel on batch/N with no communication; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from state_space_sequence_prefill_amd import synthetic as syn
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.profile_prefill or args.profile_decode or args.profile_copy or args.probe_bandwidth:
        if args.profile_prefill:
            profile_prefill(args.profile_prefill, args.workload or HEADLINE)
        if args.profile_decode:
            profile_decode(args.profile_decode, args.workload or "decode_siso_n128")
        if args.profile_copy:
            profile_copy(args.profile_copy)
        if args.probe_bandwidth:
            print(json.dumps(probe_bandwidth()))
        return

    w = syn.WORKLOADS[HEADLINE]
    pf = Prefill(w, seed=1001)
    # Declared clock ramp (untimed, before the warm-up and the timed steps):
    # from idle the GPU's clocks take ~100 prefill launches to settle, so
    # whatever --warmup asks for, the headline first runs prefill steps until
    # both RAMP_MIN_LAUNCHES launches and RAMP_MIN_MS of wall time have passed.
    ramp = pf.ramp(RAMP_MIN_LAUNCHES, RAMP_MIN_MS)
    log(f"bench: clock ramp {ramp['launches']} launches / {ramp['ms']} ms; prefill {w.name} "
        f"warmup={args.warmup} steps={args.steps}")
    ms_step, kern_ms = pf.time(args.steps, args.warmup)
    tokens = w.batch * w.seqlen
    value = tokens / (ms_step / 1e3) / 1e6
    nbytes = prefill_bytes(w)
    achieved = nbytes / (kern_ms / 1e3) / 1e9
    flops = prefill_flops(w)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Mtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "clock_ramp": ramp,
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "headdim": w.headdim,
                   "dstate": w.dstate, "rank": w.rank, "seqlen": w.seqlen, "chunk": w.chunk,
                   "io_dtype": w.io_dtype, "state_dtype": "f32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(w.name),
                     "kernel": "prefill_pc_kernel (fused pass)", "algorithmic_bytes_per_launch": nbytes,
                     "kernel_ms": round(kern_ms, 4),
                     "mfma_frac_at_measured_time": round(flops / (kern_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    del pf
    torch.cuda.empty_cache()
    log("bench: copy bandwidth")
    cg = measured_copy_gbs()
    line["roofline"]["measured_copy_GBs"] = cg
    line["roofline"]["frac_of_measured_copy"] = round(achieved / cg, 4)
    if os.path.exists(PROBE_LIB):
        log("bench: streaming probes")
        pb = probe_bandwidth()
        line["roofline"]["measured_stream"] = pb
        line["roofline"]["frac_of_measured_read"] = round(achieved / pb["read_GBs"], 4)

    if not args.no_extra:
        extra = {}
        for name in ("decode_mimo_r4_n64", "decode_siso_n128"):
            log(f"bench: decode {name}")
            extra[name] = time_decode(syn.WORKLOADS[name], seed=7)
            extra[name]["traffic_flushed"] = committed_traffic(name)
            torch.cuda.empty_cache()
        for name in ("mimo_r4_t4096", "long_siso_t16384"):
            wx = syn.WORKLOADS[name]
            log(f"bench: prefill {name}")
            p = Prefill(wx, seed=1002)
            ms, kms = p.time_extra(max(3, args.steps // 2))
            nb = prefill_bytes(wx)
            extra[name] = {"ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
                           "Mtokens_per_s": round(wx.batch * wx.seqlen / ms / 1e3, 3),
                           "launches": p.nlaunch, "algorithmic_bytes": nb,
                           "hbm_frac": round(nb / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                           "traffic": committed_traffic(name)}
            del p
            torch.cuda.empty_cache()
        # the other discretisation rules on the headline shape (same kernel;
        # the pages compare Mamba-2's exponential Euler with Mamba-3's rule)
        for disc in ("exp_euler", "decayed_trapezoid"):
            log(f"bench: prefill {w.name} disc={disc}")
            p = Prefill(w, seed=1003, disc=disc)
            ms, kms = p.time_extra(max(3, args.steps // 2))
            extra[f"{w.name}_{disc}"] = {"ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
                                         "Mtokens_per_s": round(w.batch * w.seqlen / ms / 1e3, 3),
                                         "hbm_frac": round(nbytes / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
            del p
            torch.cuda.empty_cache()
        # fp32 I/O on the headline shape (x, B, C, y in fp32; 32-token tiles)
        wf = w.with_(io_dtype="f32")
        log(f"bench: prefill {w.name} fp32 I/O")
        p = Prefill(wf, seed=1005)
        ms, kms = p.time_extra(max(3, args.steps // 2))
        nbf = prefill_bytes(wf)
        extra[f"{w.name}_f32io"] = {"ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
                                    "Mtokens_per_s": round(w.batch * w.seqlen / ms / 1e3, 3),
                                    "algorithmic_bytes": nbf,
                                    "hbm_frac": round(nbf / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        del p
        torch.cuda.empty_cache()
        # the output epilogue (pre-gate grouped RMSNorm) fused into the store
        # of y: the headline shape and both decode shapes
        log(f"bench: gated prefill {w.name}")
        p = Prefill(w, seed=1004, gated=True)
        ms, kms = p.time_extra(max(3, args.steps // 2))
        nbg = nbytes + gate_bytes(w, w.seqlen)
        extra[f"{w.name}_gated"] = {"ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
                                    "Mtokens_per_s": round(w.batch * w.seqlen / ms / 1e3, 3),
                                    "algorithmic_bytes": nbg,
                                    "hbm_frac": round(nbg / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        del p
        torch.cuda.empty_cache()
        for name in ("decode_mimo_r4_n64", "decode_siso_n128"):
            log(f"bench: gated decode {name}")
            extra[f"{name}_gated"] = time_decode(syn.WORKLOADS[name], seed=7, flush_steps=5, gated=True)
            torch.cuda.empty_cache()
        # MIMO with the rank down-projection folded into the store (y and z
        # lose the rank axis), then the epilogue: prefill and decode
        wm = syn.WORKLOADS["mimo_r4_t4096"]
        log(f"bench: down-projected gated prefill {wm.name}")
        p = Prefill(wm, seed=1005, down=True)
        ms, kms = p.time_extra(max(3, args.steps // 2))
        nbd = prefill_bytes(wm) + gate_bytes(wm, wm.seqlen) + down_bytes_delta(wm, wm.seqlen)
        extra[f"{wm.name}_down_gated"] = {"ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
                                          "Mtokens_per_s": round(wm.batch * wm.seqlen / ms / 1e3, 3),
                                          "algorithmic_bytes": nbd,
                                          "hbm_frac": round(nbd / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        del p
        torch.cuda.empty_cache()
        log("bench: down-projected gated decode decode_mimo_r4_n64")
        extra["decode_mimo_r4_n64_down_gated"] = time_decode(syn.WORKLOADS["decode_mimo_r4_n64"], seed=7,
                                                             flush_steps=5, down=True)
        torch.cuda.empty_cache()
        # BC normalisation in the prefill prep (plain and gated y) and in the
        # decode step (gated y); the weights add 2 H N fp32 to the bytes
        for gated in (False, True):
            tag = f"{w.name}_bcnorm" + ("_gated" if gated else "")
            log(f"bench: prefill {tag}")
            p = Prefill(w, seed=1006, gated=gated, bcnorm=True)
            ms, kms = p.time_extra(max(3, args.steps // 2))
            nbb = nbytes + (gate_bytes(w, w.seqlen) if gated else 0) + 2 * w.heads * w.dstate * 4
            extra[tag] = {"ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
                          "Mtokens_per_s": round(w.batch * w.seqlen / ms / 1e3, 3), "algorithmic_bytes": nbb,
                          "hbm_frac": round(nbb / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
            del p
            torch.cuda.empty_cache()
        for name in ("decode_mimo_r4_n64", "decode_siso_n128"):
            log(f"bench: bcnorm gated decode {name}")
            extra[f"{name}_bcnorm_gated"] = time_decode(syn.WORKLOADS[name], seed=7, flush_steps=5, gated=True,
                                                        bcnorm=True)
            torch.cuda.empty_cache()
        # the backward pass (gradients of every input) on both prefill shapes
        for name in (HEADLINE, "mimo_r4_t4096"):
            log(f"bench: backward {name}")
            extra[f"{name}_backward"] = time_backward(syn.WORKLOADS[name], seed=1007, steps=5, warmup=3)
        line["extra"] = extra

    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(w)
        log("bench: cpu baseline (oracle, all host cores)")
        line["cpu_baseline"]["all_cores"] = cpu_baseline_all_cores(w)
        if "extra" in line:
            for name in ("decode_mimo_r4_n64", "decode_siso_n128"):
                log(f"bench: cpu decode (oracle) {name}")
                line["extra"][name]["cpu_oracle_ms_per_step"] = cpu_decode_ms(syn.WORKLOADS[name])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
