"""HIP graph capture of the library's calls (the way the decode and prefill
benchmarks replay them): every replay must give exactly what the same calls
give when launched one by one.  Each graph is replayed several times, with
the program's own eager work (state reloads, buffers overwritten with NaN)
and synchronisations between the replays, and every replay is compared with
the eager result bit for bit (same kernels, same inputs, deterministic)."""

import pytest

from state_space_sequence_prefill_amd import synthetic as syn

from m3_testlib import state_to_gpu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import state_space_sequence_prefill_amd as m3  # noqa: E402

REPLAYS = 3


def _capture(fn, warm=2):
    """fn() launched `warm` times on a side stream (first-call set-up stays
    out of the graph), then captured once."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warm):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _state_copy(s):
    return s.h.clone(), s.B_prev.clone(), s.x_prev.clone()


def _same(a, b, what):
    assert torch.equal(a, b), what


@pytest.mark.parametrize("name,R,N", [("decode_siso_n128", 1, 128), ("decode_mimo_r4_n64", 4, 64)])
def test_decode_steps_graph_replays(name, R, N):
    """Five decode steps captured in one graph, against the same five steps
    launched eagerly from the same state."""
    w = syn.WORKLOADS[name].with_(batch=4, heads=6)
    d = m3.make_dims(w.batch, w.heads, w.headdim, w.dstate, w.rank, w.chunk, w.io_dtype)
    K = 5
    tok = syn.draw_torch(w, 4100, seqlen=K)
    steps = [{k: (v[:, t].contiguous() if k in ("x", "B", "C", "dt", "lam", "theta") else v) for k, v in tok.items()}
             for t in range(K)]
    h0, bp0, xp0 = state_to_gpu(syn.draw_state(w, 4101), w.io_dtype)
    io = tok["x"].dtype
    s = m3.State.empty(d)
    ys = [torch.empty((w.batch, w.heads, w.rank, w.headdim), dtype=io, device="cuda") for _ in range(K)]

    def run():
        for t in range(K):
            a = steps[t]
            m3.mamba3_decode_step(d, a["x"], a["B"], a["C"], a["dt"], a["lam"], a["theta"], a["A"], a["D"], s, ys[t])

    m3.m3_state_load(d, s, h0, bp0, xp0)
    run()
    torch.cuda.synchronize()
    ref_y = [y.clone() for y in ys]
    ref_s = _state_copy(s)
    print(f"[graph decode {name}] batch {w.batch} heads {w.heads} R {R} N {N}, {K} steps", flush=True)
    m3.m3_state_load(d, s, h0, bp0, xp0)
    g = _capture(run)
    for r in range(REPLAYS):
        for y in ys:
            y.fill_(float("nan"))
        m3.m3_state_load(d, s, h0, bp0, xp0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t in range(K):
            _same(ys[t], ref_y[t], f"replay {r} y step {t}")
        for a, b, nm in zip(_state_copy(s), ref_s, ("h", "B_prev", "x_prev")):
            _same(a, b, f"replay {r} {nm}")


@pytest.mark.parametrize("name,seqlen", [("siso_1p5b_t4096", 200), ("mimo_r4_t4096", 77), ("long_siso_t16384", 1500)])
def test_prefill_step_graph_replays(name, seqlen):
    """One benchmark step (state reset + prefill; the long shape takes the
    three-launch segmented path with its workspace) captured in a graph."""
    w = syn.WORKLOADS[name].with_(batch=2, seqlen=seqlen)
    if name == "long_siso_t16384":
        w = w.with_(batch=1, heads=4)
    d = m3.make_dims(w.batch, w.heads, w.headdim, w.dstate, w.rank, w.chunk, w.io_dtype)
    inp = syn.draw_torch(w, 4200)
    s = m3.State.empty(d)
    y = torch.empty((w.batch, w.seqlen, w.heads, w.rank, w.headdim), dtype=inp["x"].dtype, device="cuda")
    nws = m3.mamba3_prefill_workspace_bytes(d, w.seqlen)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None

    def run():
        m3.m3_state_zero(d, s)
        m3.mamba3_prefill(d, w.seqlen, inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["theta"], inp["A"],
                          inp["D"], s, y, ws)

    run()
    torch.cuda.synchronize()
    ref_y, ref_s = y.clone(), _state_copy(s)
    print(f"[graph prefill {name}] batch {w.batch} heads {w.heads} T {w.seqlen} workspace {nws} B", flush=True)
    g = _capture(run)
    for r in range(REPLAYS):
        y.fill_(float("nan"))
        s.h.fill_(float("nan"))
        if ws is not None:
            ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(y, ref_y, f"replay {r} y")
        for a, b, nm in zip(_state_copy(s), ref_s, ("h", "B_prev", "x_prev")):
            _same(a, b, f"replay {r} {nm}")
