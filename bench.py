"""Benchmark of the Mamba-3 scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

One step = one pass of the hot path over one batch: m3_state_zero + one
mamba3_prefill of the 1.5B-scale SISO layer (batch 8, 32 heads, headdim 64,
state 128, 4096 tokens, chunk 64, bf16 I/O, fp32 state), inputs resident in
HBM before the timed region.  `value` is prefill throughput in Mtokens/s
(tokens = batch x seqlen, all heads).  The same JSON line carries:
  roofline      -- the prefill kernel's algorithmic HBM bytes per launch over
                   its average duration (HIP events on the launch stream),
                   against the MI355X HBM peak of 8 TB/s; `traffic` comes from
                   committed rocprofv3 FETCH_SIZE / WRITE_SIZE counters when
                   they were taken on the current kernel source, else null;
  cpu_baseline  -- the fp64 oracle timed on the host on a bounded sample;
  extra         -- decode step (256 x 32 heads, MIMO R=4 N=64 and SISO N=128;
                   1000 steps captured in a HIP graph, plus a run with a
                   512 MiB cache flush between steps), and MIMO / 16K-token
                   prefill throughput.
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
PREFILL_SRC = os.path.join(ROOT, "state_space_sequence_prefill_amd", "csrc", "m3_prefill.hip")


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


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(workload_name):
    """Per-launch HBM bytes measured with rocprofv3 counters, if recorded for
    the current kernel source (profiles/<kernel>_<workload>_traffic.json)."""
    p = os.path.join(PROFILES, f"prefill_{workload_name}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != source_sha(PREFILL_SRC):
        return None
    return rec.get("bytes_per_launch")


class Prefill:
    def __init__(self, w, seed, long_memory=False):
        import torch
        import state_space_sequence_prefill_amd as m3
        from state_space_sequence_prefill_amd import synthetic as syn
        self.m3, self.torch, self.w = m3, torch, w
        self.d = m3.make_dims(w.batch, w.heads, w.headdim, w.dstate, w.rank, w.chunk, w.io_dtype)
        self.inp = syn.draw_torch(w, seed, long_memory=long_memory)
        self.state = m3.State.empty(self.d)
        self.y = torch.empty((w.batch, w.seqlen, w.heads, w.rank, w.headdim), dtype=self.inp["x"].dtype,
                             device="cuda")
        nws = m3.mamba3_prefill_workspace_bytes(self.d, w.seqlen)
        self.ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
        self.nlaunch = 1 if not nws else 3

    def step(self, ev=None):
        i = self.inp
        self.m3.m3_state_zero(self.d, self.state)
        if ev is not None:
            ev[0].record()
        self.m3.mamba3_prefill(self.d, self.w.seqlen, i["x"], i["B"], i["C"], i["dt"], i["lam"], i["theta"],
                               i["A"], i["D"], self.state, self.y, self.ws)
        if ev is not None:
            ev[1].record()

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


def time_decode(w, seed, steps=1000, flush_steps=20):
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
    y = torch.empty((w.batch, w.heads, w.rank, w.headdim), dtype=toks["x"].dtype, device="cuda")

    def one(j):
        s = sets[j % nset]
        m3.mamba3_decode_step(d, s["x"], s["B"], s["C"], s["dt"], s["lam"], s["theta"], s["A"], s["D"], st, y)

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
    nb = decode_bytes(w)
    return {
        "workload": w.name, "batch": w.batch, "heads": w.heads, "headdim": w.headdim, "dstate": w.dstate,
        "rank": w.rank, "us_per_step_graph": round(us_graph, 2), "steps_graph": reps * per_graph,
        "us_per_step_flushed": round(us_flush, 2), "bytes_per_step": nb,
        "hbm_GBs_graph": round(nb / us_graph / 1e3, 1), "hbm_frac_graph": round(nb / us_graph / 1e3 / HBM_PEAK_GBS, 4),
        "hbm_GBs_flushed": round(nb / us_flush / 1e3, 1),
        "hbm_frac_flushed": round(nb / us_flush / 1e3 / HBM_PEAK_GBS, 4),
    }


def cpu_baseline(w):
    """The fp64 oracle, unchanged, on the host: batch row 0 of the workload
    (all heads, all tokens), single-threaded numpy."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle
    from state_space_sequence_prefill_amd import synthetic as syn
    ws = w.with_(batch=1)
    ex = syn.as_exact(syn.draw(ws, 1001), w.io_dtype)
    import contextlib
    ctx = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    with ctx:
        t0 = time.perf_counter()
        oracle.prefill(ex["x"], ex["B"], ex["C"], ex["dt"], ex["lam"], ex["theta"], ex["A"], ex["D"])
        dt = time.perf_counter() - t0
    toks = ws.batch * ws.seqlen
    return {"value": round(toks / dt / 1e6, 8), "unit": "Mtokens/s", "cores": 1, "kind": "oracle",
            "sample": f"batch row 0 of {w.batch} ({w.heads} heads x {w.seqlen} tokens), numpy fp64, "
                      f"{dt:.1f} s", "seconds": round(dt, 2), "cpu": _cpu_model(), "host_cpus": os.cpu_count()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every (batch, head) chain of the scan is independent, so "
              "N GPUs run the same kernel on batch/N (see the sharding notes in DESIGN.md); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from state_space_sequence_prefill_amd import synthetic as syn
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    w = syn.WORKLOADS["siso_1p5b_t4096"]
    log(f"bench: prefill {w.name} warmup={args.warmup} steps={args.steps}")
    pf = Prefill(w, seed=1001)
    ms_step, kern_ms = pf.time(args.steps, args.warmup)
    tokens = w.batch * w.seqlen
    value = tokens / (ms_step / 1e3) / 1e6
    nbytes = prefill_bytes(w)
    achieved = nbytes / (kern_ms / 1e3) / 1e9
    flops = prefill_flops(w)
    line = {
        "metric": "Mamba-3 scan prefill Mtokens/s + decode us/step; % of MFMA / HBM peak",
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
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "headdim": w.headdim,
                   "dstate": w.dstate, "rank": w.rank, "seqlen": w.seqlen, "chunk": w.chunk,
                   "io_dtype": w.io_dtype, "state_dtype": "f32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(w.name),
                     "kernel": "prefill_kernel (fused pass)", "algorithmic_bytes_per_launch": nbytes,
                     "kernel_ms": round(kern_ms, 4),
                     "mfma_frac_at_measured_time": round(flops / (kern_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    del pf
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra = {}
        for name in ("decode_mimo_r4_n64", "decode_siso_n128"):
            log(f"bench: decode {name}")
            extra[name] = time_decode(syn.WORKLOADS[name], seed=7)
            torch.cuda.empty_cache()
        for name in ("mimo_r4_t4096", "long_siso_t16384"):
            wx = syn.WORKLOADS[name]
            log(f"bench: prefill {name}")
            p = Prefill(wx, seed=1002)
            ms, kms = p.time(max(3, args.steps // 2), 2)
            nb = prefill_bytes(wx)
            extra[name] = {"ms_per_step": round(ms, 4), "Mtokens_per_s": round(wx.batch * wx.seqlen / ms / 1e3, 3),
                           "launches": p.nlaunch, "algorithmic_bytes": nb,
                           "hbm_frac": round(nb / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
            del p
            torch.cuda.empty_cache()
        line["extra"] = extra

    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
