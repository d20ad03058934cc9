"""Benchmark: batch-1 8B-shape decode-step weight stream on one MI355X.

One step = embedding row of the previous token, 36 layers x 4 ternary levels
(q|k|v 6144x4096, o 4096x4096, gate|up 24576x4096, down 4096x12288) in
decoder order, the int8 output projection (151,936 x 4,096) and the greedy
argmax.  Steps are captured into HIP graphs (by default four consecutive
steps per graph, each step's token feeding the next step's embedding row on
the device) and replayed; inputs are resident in HBM before the timed region
starts.

Order of work (the release-gate policy of the page "The Neutrino Engine",
sections "One changed token fails the release" and "The engine also runs
weights we did not train": identity is checked before any timing, and timing
is done in interleaved rounds):
  1. build the seeded synthetic workload and upload it;
  2. parity: sampled rows of every level, the full logits' argmax and the
     embedding row against the CPU oracle; abort on any failure;
  3. the timed schedule (by default the stream schedule, which computes the
     step over its fixed per-level inputs with no waits between levels) in
     one HIP graph: untimed replays for --prewarm seconds, --warmup untimed
     steps, exactly --steps timed steps (HIP events on the replay stream;
     graphs of --steps-per-graph chained steps), then --rounds more rounds
     of --steps for the median and p10 / p90; the same step with one step
     per graph and without a graph;
  4. the levels schedule (one kernel per level, in decoder order, as a
     chained step needs), a null graph with as many empty kernels, and the
     chained step, to split dependency and launch overhead from DRAM time;
  5. configurations 1-3 as units of their own, the packing against the
     pages' slab, the small-batch passes and decode attention;
  6. the oracle on a bounded sample of the same workload, each sample round
     right after a GPU timing round of the step, and on one thread.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_BPS = 8.0e12
METRIC = "achieved weight GB/s (% of HBM peak) + µs per batch-1 8B-shape decode step"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--schedule", choices=["stream", "levels"], default="stream",
                   help="timed schedule: stream (the step over its fixed level inputs, no dependency waits) or "
                        "levels (one kernel per level, in decoder order); the other is timed alongside")
    p.add_argument("--layers", type=int, default=36)
    p.add_argument("--no-compare", action="store_true", help="skip the levels-schedule and null-graph timings")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-small-batch", action="store_true", help="skip the small-batch (B = 1, 4, 8, 16) timings")
    p.add_argument("--attention-only", action="store_true",
                   help="only the decode-attention leg (one 8B-shape layer at 4,096 and 32,768 cached positions; "
                        "parity, then timing); prints its JSON object")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle's timed sample")
    p.add_argument("--prewarm", type=float, default=0.3,
                   help="seconds of untimed graph replays before the counted warm-up (steady clocks)")
    p.add_argument("--rounds", type=int, default=15, help="extra timing rounds of --steps steps (median, p10, p90)")
    p.add_argument("--steps-per-graph", type=int, default=4,
                   help="consecutive decode steps captured in one graph for the timed replays (each step's token "
                        "feeds the next step's embedding row on the device)")
    p.add_argument("--no-units", action="store_true", help="skip configurations 1-3 as standalone units")
    p.add_argument("--counters", action="store_true",
                   help="counter-collection run: 3 eager steps of the timed schedule plus a 1 GiB device copy "
                        "(the known-size reference for FETCH_SIZE / WRITE_SIZE); prints nothing else")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Sources of each schedule's step kernel: the HBM traffic counted for a
# kernel stays valid while these files are unchanged.
KERNEL_SOURCES = {
    "stream": ("step_stream.hip", "step_stream.h", "operands.h", "device_common.h", "pwg_internal.h"),
}


def kernel_source_sha(schedule: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "packed_weight_gemv_amd", "csrc")
    for name in sorted(KERNEL_SOURCES.get(schedule, os.listdir(csrc))):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def time_graph(graph, stream, steps, warmup):
    import torch
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per replay


def prewarm(graph, stream, seconds):
    """Replays `graph` untimed for about `seconds` so that clocks and caches
    are in their steady state before the counted warm-up and timed replays
    (the number of those is fixed by the command line; this is not)."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            graph.replay()
        n += 16
        stream.synchronize()
    return n


def time_rounds(graph, stream, steps, rounds):
    """ms per replay over `rounds` rounds of `steps` replays each (HIP events
    on the replay stream, one pair per round)."""
    import torch
    out = []
    with torch.cuda.stream(stream):
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                graph.replay()
            e1.record(stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) / steps)
    return out


def time_steps(graph_s, graph_1, s, stream, steps, warmup, rounds=1):
    """ms per step over exactly `steps` steps: steps // s replays of the
    s-step graph and steps % s replays of the one-step graph, after `warmup`
    untimed steps done the same way; `rounds` timed rounds (HIP events on the
    replay stream, one pair per round)."""
    import torch

    def run(n):
        for _ in range(n // s):
            graph_s.replay()
        for _ in range(n % s):
            graph_1.replay()
    with torch.cuda.stream(stream):
        run(warmup)
        stream.synchronize()
        out = []
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(steps)
            e1.record(stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) / steps)
    return out


def spread(ms_list):
    """Median and 10th / 90th percentiles (us) of per-round ms values."""
    import numpy as np
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return {"median_us": float(np.median(a)), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90)), "rounds": int(a.size)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


class HipGraph:
    """The work `fn` enqueues on `stream`, captured into a HIP graph and
    replayed with hipGraphLaunch on that stream (the HIP runtime's own graph
    API: torch's replay wrapper adds about 2 us of GPU time per replay)."""

    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes as C
            h = C.CDLL("libamdhip64.so")
            vp = C.c_void_p
            for name, args in [("hipStreamBeginCapture", [vp, C.c_int]), ("hipStreamEndCapture", [vp, C.POINTER(vp)]),
                               ("hipGraphInstantiate", [C.POINTER(vp), vp, vp, vp, C.c_size_t]),
                               ("hipGraphLaunch", [vp, vp]), ("hipGraphDestroy", [vp]), ("hipGraphExecDestroy", [vp])]:
                getattr(h, name).argtypes = args
                getattr(h, name).restype = C.c_int
            cls._hip = h
        return cls._hip

    def __init__(self, fn, stream):
        import ctypes as C
        h = self.hip()
        self.exe = None
        self.stream = C.c_void_p(stream.cuda_stream)
        graph = C.c_void_p()
        rc = h.hipStreamBeginCapture(self.stream, 1)  # thread-local capture mode
        if rc != 0:
            raise RuntimeError(f"hipStreamBeginCapture: {rc}")
        try:
            fn()
        finally:
            rc = h.hipStreamEndCapture(self.stream, C.byref(graph))
        if rc != 0:
            raise RuntimeError(f"hipStreamEndCapture: {rc}")
        exe = C.c_void_p()
        rc = h.hipGraphInstantiate(C.byref(exe), graph, None, None, 0)
        h.hipGraphDestroy(graph)
        if rc != 0:
            raise RuntimeError(f"hipGraphInstantiate: {rc}")
        self.exe = exe

    def replay(self):
        rc = self.hip().hipGraphLaunch(self.exe, self.stream)
        if rc != 0:
            raise RuntimeError(f"hipGraphLaunch: {rc}")

    def __del__(self):
        if self.exe is not None and self._hip is not None:
            self._hip.hipGraphExecDestroy(self.exe)


def capture(fn, stream):
    import torch
    with torch.cuda.stream(stream):   # torch ops in fn go to the captured stream too
        fn()                          # one eager run before capture
        stream.synchronize()
        g = HipGraph(fn, stream)
    stream.synchronize()
    return g


def time_direct(fn, stream, steps, warmup):
    """The same work launched without a graph (ms per call)."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / steps


def parity(wl, ref, token_in):
    """Sampled level rows, full logits argmax, embedding row."""
    import numpy as np

    from tests.parity import gemv_report, token_ok
    worst = {"rel_l2": 0.0, "max_rel_to_magnitude": 0.0}
    n_rows = 0
    for smp, lv in zip(wl.samples, wl.desc.levels):
        y = lv[3][torch_index(smp.rows)].cpu().numpy()
        r = gemv_report(y, ref.ternary_gemv(smp.w, smp.scale, smp.x), ref.ternary_gemv_magnitude(smp.w, smp.scale, smp.x))
        if not (r["ok"] and r["finite"]):
            raise SystemExit(f"parity failed at layer {smp.layer} level {smp.level}: {r}")
        worst["rel_l2"] = max(worst["rel_l2"], r["rel_l2"])
        worst["max_rel_to_magnitude"] = max(worst["max_rel_to_magnitude"], r["max_rel_to_magnitude"])
        n_rows += len(smp.rows)
    lr = ref.int8_logits(wl.out_table.q, wl.out_table.scale, wl.h)
    token = int(wl.desc.token_out.cpu()[0])
    if not token_ok(token, lr):
        raise SystemExit(f"parity failed: token {token} vs oracle {int(np.argmax(lr))}")
    er, es, _ = ref.embed_gather(wl.emb_table.q, wl.emb_table.scale, [token_in])
    if not np.array_equal(wl.desc.emb_row_out.cpu().numpy(), er[0]) or float(wl.desc.emb_scale_out.cpu()[0]) != es[0]:
        raise SystemExit("parity failed: embedding row")
    _, gap = ref.greedy_token(lr)
    return {"levels_checked": len(wl.samples), "rows_checked": n_rows, "token": token, "oracle_top2_gap": gap,
            "worst_level_rel_l2": worst["rel_l2"], "worst_rel_to_magnitude": worst["max_rel_to_magnitude"]}


def torch_index(rows):
    import torch
    return torch.from_numpy(rows).to("cuda:0")


def cpu_baseline(target_s: float, step_bytes: int, gpu_round=None):
    """The oracle, as it stands (float64 numpy), on a bounded sample of the
    same seeded workload, in rounds interleaved with GPU timing rounds of the
    step: round r times the GPU step (`gpu_round()`, ms per step), then the
    oracle's four levels of layer r, until about target_s seconds of oracle
    time; then the full output projection and argmax.  The per-layer mean is
    scaled to the step's 36 layers.  All host threads (BLAS threads as the
    library sets them), and one layer again on one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import synth
    from oracle import reference as ref

    def one_layer(layer):
        mats = synth.layer(synth.W_STEP, layer)
        xs = synth.layer_inputs(synth.W_STEP, layer)
        return [(synth.stacked(mats, members), xs[name]) for name, members, _ in synth.LEVELS]

    def run_layer(levels):
        t0 = time.perf_counter()
        for m, x in levels:
            ref.ternary_gemv(m.w, m.scale, x)
        return time.perf_counter() - t0

    layer_s, gpu_ms = [], []
    for layer in range(synth.N_LAYERS):
        if layer_s and sum(layer_s) + float(np.mean(layer_s)) > target_s:
            break
        levels = one_layer(layer)          # generation is not timed
        if gpu_round is not None:
            gpu_ms.append(gpu_round())
        layer_s.append(run_layer(levels))
        del levels
    out_t, _, _, h = synth.vocab_workload(n_ids=1, workload=synth.W_STEP)
    t0 = time.perf_counter()
    lg = ref.int8_logits(out_t.q, out_t.scale, h)
    ref.greedy_token(lg)
    vocab_s = time.perf_counter() - t0
    del out_t, lg
    step_s = float(np.mean(layer_s)) * synth.N_LAYERS + vocab_s
    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    levels = one_layer(0)
    with threadpool_limits(limits=1):
        one_s = run_layer(levels)
    del levels
    # one thread: the layer time scaled by the step's bytes over the layer's
    layer_bytes = sum(r * k // 4 + 4 * r for r, k in ((6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)))
    one_step_s = one_s * step_bytes / layer_bytes
    out = {
        "value": step_bytes / step_s / 1e9, "unit": "GB/s",
        "us_per_step": step_s * 1e6, "cores": int(threads), "kind": "oracle", "cpu_model": cpu_model(),
        "sample": (f"{len(layer_s)} of 36 layers (all 4 levels each, float64 numpy), each timed right after a GPU "
                   f"timing round of the step, plus the full 151936x4096 output projection and argmax; the "
                   f"per-layer mean is scaled to 36 layers"),
        "sample_seconds": float(sum(layer_s) + vocab_s),
        "one_core": {"value": step_bytes / one_step_s / 1e9, "unit": "GB/s", "cores": 1,
                     "us_per_step": one_step_s * 1e6,
                     "sample": "layer 0 (4 levels) on one BLAS thread, scaled to the step by algorithmic bytes",
                     "sample_seconds": one_s},
    }
    if gpu_ms:
        out["interleaved_gpu_rounds"] = spread(gpu_ms)
    return out


def packing_report(wl):
    """Bytes per weight of the packed ternary lane against the pages' per-layer
    slab (72,351,744 bytes for the 8B shape's 192,937,984 weights)."""
    lv = wl.desc.levels[:4]
    weights = sum(r * k for (_, _, _, _, r, k) in lv)
    packed = sum(r * k // 4 for (_, _, _, _, r, k) in lv)
    scales = sum(4 * r for (_, _, _, _, r, k) in lv)
    slab = 72351744
    return {"format": "T2 (2 bits per weight, row scales float32 apart)", "weights_per_layer": weights,
            "packed_bytes_per_layer": packed, "scale_bytes_per_layer": scales,
            "bytes_per_weight": packed / weights, "pages_slab_bytes_per_layer": slab,
            "pages_slab_bytes_per_weight": slab / weights, "ratio_to_pages_slab": packed / slab}


def standalone_units(wl, stream, reps=20):
    """Configurations 1-3 as units of their own, each after a parity check:
    the 1024 x 1024 ternary GEMV (per call, resident, and rotated over 1,100
    copies so that the copies exceed the last-level cache); one 8B-shape
    layer's four levels through the per-call GEMV, rotated over the step's 36
    layers; the int8 output projection + argmax over the 151,936 x 4,096
    table, and the gather of 64 embedding rows."""
    import numpy as np
    import torch

    import packed_weight_gemv_amd as pwg
    import synth
    from oracle import reference as ref
    from tests.parity import assert_gemv, token_ok
    dev = "cuda:0"
    out = {}
    # configuration 1
    w, s_, x = synth.single_gemv()
    blob = torch.from_numpy(pwg.pack_weights(w)).to(dev)
    sd, xd = torch.from_numpy(s_).to(dev), torch.from_numpy(x).to(dev)
    yd = torch.empty(1024, dtype=torch.float32, device=dev)
    pwg.ternary_gemv(blob, sd, 1024, 1024, xd, y=yd, stream=stream)
    stream.synchronize()
    assert_gemv(yd.cpu().numpy(), ref.ternary_gemv(w, s_, x), ref.ternary_gemv_magnitude(w, s_, x), "config 1")
    unit_bytes = 1024 * 1024 // 4 + 4 * 1024
    copies = 1100
    wr = blob.repeat(copies).view(copies, -1)
    sr, xr = sd.repeat(copies).view(copies, -1), xd.repeat(copies).view(copies, -1)
    yr = torch.empty((copies, 1024), dtype=torch.float32, device=dev)
    g_res = capture(lambda: [pwg.ternary_gemv(blob, sd, 1024, 1024, xd, y=yd, stream=stream) for _ in range(copies)],
                    stream)
    prewarm(g_res, stream, 0.05)
    us_res = time_graph(g_res, stream, 5, 1) * 1e3 / copies
    del g_res
    g_rot = capture(lambda: [pwg.ternary_gemv(wr[i], sr[i], 1024, 1024, xr[i], y=yr[i], stream=stream)
                             for i in range(copies)], stream)
    prewarm(g_rot, stream, 0.05)
    us_rot = time_graph(g_rot, stream, 5, 1) * 1e3 / copies
    del g_rot
    us_call = time_direct(lambda: pwg.ternary_gemv(blob, sd, 1024, 1024, xd, y=yd, stream=stream), stream, 2000, 200) * 1e3
    out["config1_1024x1024_gemv"] = {
        "us_per_call_launched": us_call, "us_per_call_in_graph_resident": us_res,
        "us_per_call_in_graph_rotated_1100_copies": us_rot, "bytes_per_call": unit_bytes,
        "rotated_GBps": unit_bytes / (us_rot * 1e-6) / 1e9, "floor_us": unit_bytes / PEAK_HBM_BPS * 1e6,
        "note": "latency-bound: each call is one kernel launch; graph node boundaries included"}
    log(f"config 1: {us_call:.2f} us per launched call, {us_res:.2f} us per call in a graph (resident), "
        f"{us_rot:.2f} us rotated over {copies} copies ({unit_bytes / (us_rot * 1e-6) / 1e9:.0f} GB/s)")
    del wr, sr, xr, yr
    # configuration 2: the per-call GEMV over every level of every layer (one graph)
    rows_w = wl.weights[pwg.LAYOUT_ROWS][0]
    lv = wl.desc.levels
    n_layers = len(lv) // 4
    calls = [(w_, sc, x_, y_, r, k) for w_, (_, sc, x_, y_, r, k) in zip(rows_w, lv)]
    g2 = capture(lambda: [pwg.ternary_gemv(w_, sc, r, k, x_, y=y_, stream=stream) for w_, sc, x_, y_, r, k in calls],
                 stream)
    prewarm(g2, stream, 0.1)
    ms2 = time_graph(g2, stream, reps, 2)
    del g2
    smp = wl.samples[4]
    yv = lv[4][3][torch.from_numpy(smp.rows).to(dev)].cpu().numpy()
    assert_gemv(yv, ref.ternary_gemv(smp.w, smp.scale, smp.x), ref.ternary_gemv_magnitude(smp.w, smp.scale, smp.x),
                "config 2 sample")
    layer_bytes = sum(r * k // 4 + 4 * r for (_, _, _, _, r, k) in lv[:4])
    us_layer = ms2 * 1e3 / n_layers
    out["config2_8b_layer_per_call_gemvs"] = {
        "us_per_layer": us_layer, "bytes_per_layer": layer_bytes, "GBps": layer_bytes / (us_layer * 1e-6) / 1e9,
        "floor_us": layer_bytes / PEAK_HBM_BPS * 1e6, "layers_rotated": n_layers,
        "note": "four pwg_ternary_gemv calls per layer on row-major T2, one graph over all layers"}
    log(f"config 2: {us_layer:.1f} us per layer through per-call GEMVs ({layer_bytes / (us_layer * 1e-6) / 1e9:.0f} GB/s)")
    # configuration 3: int8 projection + argmax, and 64 embedding rows
    table = wl.weights[pwg.LAYOUT_ROWS][1]
    vocab, hidden = table.shape
    ws = torch.zeros(pwg.argmax_workspace_bytes(vocab, 1), dtype=torch.uint8, device=dev)
    tok = torch.empty(1, dtype=torch.int32, device=dev)
    g3 = capture(lambda: pwg.int8_gemv_argmax(table, wl.desc.out_scale, wl.desc.h, workspace=ws, token_out=tok,
                                              stream=stream), stream)
    prewarm(g3, stream, 0.1)
    ms3 = time_graph(g3, stream, reps, 2)
    del g3
    lr = ref.int8_logits(wl.out_table.q, wl.out_table.scale, wl.h)
    if not token_ok(int(tok.cpu()[0]), lr):
        raise SystemExit("config 3 parity failed: token")
    vbytes = vocab * hidden + 4 * vocab
    ids = torch.from_numpy(synth.rng_for(synth.W_VOCAB, 2).integers(0, vocab, size=64).astype(np.int32)).to(dev)
    ro = torch.empty((64, hidden), dtype=torch.int8, device=dev)
    so = torch.empty(64, dtype=torch.float32, device=dev)
    do = torch.empty((64, hidden), dtype=torch.float32, device=dev)
    gfn = lambda: pwg.embed_gather(wl.desc.emb_table, wl.desc.emb_scale, ids, rows_out=ro, scales_out=so,  # noqa: E731
                                   deq_out=do, stream=stream)
    g4 = capture(gfn, stream)
    prewarm(g4, stream, 0.05)
    ms4 = time_graph(g4, stream, 200, 10)
    del g4
    n_in_graph = 50
    g5 = capture(lambda: [gfn() for _ in range(n_in_graph)], stream)
    prewarm(g5, stream, 0.05)
    ms5 = time_graph(g5, stream, 20, 2) / n_in_graph
    del g5
    er, _, _ = ref.embed_gather(wl.emb_table.q, wl.emb_table.scale, ids.cpu().numpy())
    if not np.array_equal(ro.cpu().numpy(), er):
        raise SystemExit("config 3 parity failed: gathered rows")
    out["config3_int8_projection_argmax"] = {
        "us_per_call": ms3 * 1e3, "bytes_per_call": vbytes, "GBps": vbytes / (ms3 * 1e-3) / 1e9,
        "floor_us": vbytes / PEAK_HBM_BPS * 1e6, "kernel": "VALU int8 x five int8 limbs of h, row-major table"}
    out["config3_gather_64_rows"] = {"us_per_call_in_graph": ms5 * 1e3, "us_per_call_one_per_graph": ms4 * 1e3,
                                     "bytes_per_call": 64 * (hidden + 4),
                                     "note": "int8 rows, scales and float32 dequantised rows of 64 ids; "
                                             f"in a graph of {n_in_graph} calls, and one call per graph replay "
                                             "(the replay's launch included)"}
    log(f"config 3: int8 projection + argmax {ms3 * 1e3:.1f} us ({vbytes / (ms3 * 1e-3) / 1e9:.0f} GB/s), "
        f"gather of 64 rows {ms5 * 1e3:.2f} us in a graph of {n_in_graph} ({ms4 * 1e3:.2f} us one per replay)")
    return out


def base3_lane(wl, stream, reps=10):
    """The step's ternary lane in the base-3 format (five weights per byte),
    measured against its own bytes/bandwidth floor and against tiled T2 on
    the same shapes: every 4,096-column row of the 36 layers stacked into one
    1,253,376 x 4,096 matrix and every down row into one 147,456 x 12,288
    matrix (one activation vector per width class; the same bytes per weight
    as the step's 144 levels), one per-call GEMV each, then the int8 output
    projection + argmax; one graph.  Random valid codes generated on the
    device (the instruction stream does not depend on the values); sampled
    rows are checked against the oracle before timing."""
    import numpy as np
    import torch

    import packed_weight_gemv_amd as pwg
    from oracle import base3_format as b3
    from oracle import reference as ref
    from tests.parity import assert_gemv
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    n_layers = len(wl.desc.levels) // 4
    shapes = [(n_layers * (4096 + 1024 + 1024 + 4096 + 12288 + 12288), 4096), (n_layers * 4096, 12288)]
    mats = []
    # every tensor is made and used on `stream` (generation, arrangement,
    # frees), so no work on another stream can race with it
    with torch.cuda.stream(stream):
        for rows, cols in shapes:
            raw = torch.randint(0, 243, (pwg.b3_packed_size(rows, cols),), dtype=torch.uint8, device=dev, generator=g)
            t2 = torch.randint(0, 256, (rows * cols // 4,), dtype=torch.uint8, device=dev, generator=g) & 0x55  # codes 00 / 01
            s_ = torch.empty(rows, dtype=torch.float32, device=dev).uniform_(0.01, 0.1, generator=g)
            x_ = torch.randn(cols, dtype=torch.float32, device=dev, generator=g)
            mats.append({"rows": rows, "cols": cols, "b3": pwg.tile_b3(raw, rows, cols, stream=stream),
                         "t2": pwg.tile_rows(t2, rows, cols // 4, stream=stream), "s": s_, "x": x_,
                         "y": torch.empty(rows, dtype=torch.float32, device=dev)})
            stream.synchronize()
            # parity on sampled rows: the oracle decodes the stored bytes of those rows
            pick = np.sort(np.random.default_rng(rows).choice(rows, 256, replace=False))
            B = pwg.b3_packed_size(1, cols)
            rb = raw.view(rows, B)[torch.from_numpy(pick).to(dev)].cpu().numpy()
            w = b3.decode(rb.reshape(-1), len(pick), cols)
            m = mats[-1]
            pwg.ternary_gemv_b3(m["b3"], m["s"], rows, cols, m["x"], y=m["y"], stream=stream)
            stream.synchronize()
            sv, xv = m["s"].cpu().numpy()[pick], m["x"].cpu().numpy()
            assert_gemv(m["y"].cpu().numpy()[pick], ref.ternary_gemv(w, sv, xv), ref.ternary_gemv_magnitude(w, sv, xv),
                        f"base-3 {rows}x{cols} sample")
            del raw, t2
    table = wl.weights[pwg.LAYOUT_ROWS][1]  # the row-major int8 table (pwg_int8_gemv_argmax's input)
    ws = torch.zeros(pwg.argmax_workspace_bytes(wl.desc.vocab, 1), dtype=torch.uint8, device=dev)
    tok = torch.empty(1, dtype=torch.int32, device=dev)

    def lane(kind):
        def fn():
            for m in mats:
                if kind == "b3":
                    pwg.ternary_gemv_b3(m["b3"], m["s"], m["rows"], m["cols"], m["x"], y=m["y"], stream=stream)
                else:
                    pwg.ternary_gemv_tiled(m["t2"], m["s"], m["rows"], m["cols"], m["x"], y=m["y"], stream=stream)
            pwg.int8_gemv_argmax(table, wl.desc.out_scale, wl.desc.h, workspace=ws, token_out=tok, stream=stream)
        return fn
    out = {}
    vocab_bytes = wl.desc.vocab * wl.desc.hidden + 4 * wl.desc.vocab
    for kind in ("b3", "t2"):
        gr = capture(lane(kind), stream)
        prewarm(gr, stream, 0.1)
        rounds = time_rounds(gr, stream, reps, 5)
        del gr
        us = float(np.median(rounds)) * 1e3
        if kind == "b3":
            wbytes = sum(pwg.b3_tiled_size(m["rows"], m["cols"]) for m in mats)
            stored = sum(pwg.b3_packed_size(m["rows"], m["cols"]) for m in mats)
        else:
            wbytes = stored = sum(m["rows"] * m["cols"] // 4 for m in mats)
        total = wbytes + sum(4 * m["rows"] for m in mats) + vocab_bytes
        total_stored = stored + sum(4 * m["rows"] for m in mats) + vocab_bytes
        out[kind] = {"us": us, "spread": spread(rounds), "bytes_streamed": total, "GBps": total / (us * 1e-6) / 1e9,
                     "floor_us": total / PEAK_HBM_BPS * 1e6, "floor_us_stored_bytes": total_stored / PEAK_HBM_BPS * 1e6,
                     "frac_of_floor": total / PEAK_HBM_BPS * 1e6 / us}
    out["kernels"] = "pwg_ternary_gemv_b3 / pwg_ternary_gemv_tiled per width class, then pwg_int8_gemv_argmax"
    out["note"] = ("the step's ternary lane stacked per width class (one activation vector each); base-3 bytes as "
                   "arranged for the device (30-weight groups in 48-byte windows) and as stored (0.2 B/weight)")
    log(f"base-3 lane: {out['b3']['us']:.1f} us ({out['b3']['GBps']:.0f} GB/s, floor {out['b3']['floor_us']:.1f} us "
        f"as arranged, {out['b3']['floor_us_stored_bytes']:.1f} us stored); T2 on the same shapes: "
        f"{out['t2']['us']:.1f} us ({out['t2']['GBps']:.0f} GB/s, floor {out['t2']['floor_us']:.1f} us)")
    del mats
    return out


def pass_desc(wl, n_layers, batch, seed):
    """A pass over the first n_layers layers' levels and the output table on
    the tiled weights: the stream schedule for one vector, the batched pass
    for 4, 8, 16; seeded inputs of shape (batch, cols) per level."""
    import torch

    import packed_weight_gemv_amd as pwg
    import synth
    tw, tq = wl.weights[pwg.LAYOUT_TILED]
    vocab, hidden = wl.out_table.q.shape
    dev = "cuda:0"
    n = 4 * n_layers
    levels = []
    for i, (w, (_, sc, _, _, r, k)) in enumerate(zip(tw[:n], wl.desc.levels[:n])):
        x = torch.from_numpy(synth.batch_inputs(batch, k, seed + i)).to(dev)
        y = torch.empty((batch, r), dtype=torch.float32, device=dev)
        levels.append((w, sc, x[0] if batch == 1 else x, y[0] if batch == 1 else y, r, k))
    h = torch.from_numpy(synth.batch_inputs(batch, hidden, seed + 9999)).to(dev)
    ids = torch.from_numpy(synth.rng_for(seed, 7).integers(0, vocab, batch).astype("int32")).to(dev)
    d = pwg.StepDesc(levels=levels, out_table=tq, out_scale=wl.desc.out_scale, h=h[0] if batch == 1 else h,
                     emb_table=wl.desc.emb_table, emb_scale=wl.desc.emb_scale, token_in=ids,
                     token_out=torch.empty(batch, dtype=torch.int32, device=dev),
                     emb_row_out=torch.empty((batch, hidden), dtype=torch.int8, device=dev),
                     emb_scale_out=torch.empty(batch, dtype=torch.float32, device=dev),
                     schedule=pwg.SCHEDULE_STREAM, weight_layout=pwg.LAYOUT_TILED, vocab=vocab, hidden=hidden,
                     batch=batch)
    d.workspace = torch.zeros(pwg.step_workspace_bytes(d), dtype=torch.uint8, device=dev)
    d._c = None
    pwg.step_plan(d)
    return d


def decode_attention(stream, contexts=(4096, 32768), reps=200):
    """One layer of grouped-query decode attention at the 8B shape (32 query
    heads over 8 key/value heads of 128, bfloat16 cache) per context length:
    parity of the timed call against the oracle, then HIP-event time per call
    and the rate over the cache bytes read (keys and values)."""
    import math

    import numpy as np
    import torch

    import packed_weight_gemv_amd as pwg
    import synth
    from oracle import attention as at
    out = {}
    n_heads, n_kv, hd = 32, 8, synth.HEAD_DIM
    for ctx in contexts:
        q, k, v = synth.kv_cache(0, ctx)
        dev = torch.device("cuda:0")
        qd = torch.from_numpy(q).to(dev)
        kd, vd = torch.from_numpy(k.view(np.int16)).to(dev), torch.from_numpy(v.view(np.int16)).to(dev)
        ws = torch.zeros(pwg.attention_workspace_bytes(n_heads, n_kv, hd, ctx), dtype=torch.uint8, device=dev)
        o = torch.empty(n_heads * hd, dtype=torch.float32, device=dev)
        scale = 1 / math.sqrt(hd)
        fn = lambda: pwg.gqa_decode_attention(kd, vd, qd, n_heads, n_kv, hd, scale, out=o, workspace=ws,  # noqa: E731
                                              stream=stream)
        with torch.cuda.stream(stream):
            fn()
        stream.synchronize()
        ref = at.gqa_decode(q, k, v, n_heads, n_kv, hd, scale)
        got = o.cpu().numpy().astype(np.float64)
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        if not rel <= 1e-5:
            raise SystemExit(f"decode attention parity failed at {ctx} positions: rel L2 {rel}")
        ms = time_direct(fn, stream, reps, 20)
        nbytes = 2 * ctx * n_kv * hd * 2
        out[str(ctx)] = {"us_per_layer": ms * 1e3, "cache_bytes": nbytes, "GB_per_s": nbytes / (ms * 1e-3) / 1e9,
                         "frac_of_8TBps": nbytes / (ms * 1e-3) / PEAK_HBM_BPS, "rel_l2_vs_oracle": rel}
        log(f"decode attention, {ctx} positions: {ms * 1e3:.2f} us per layer, "
            f"{nbytes / (ms * 1e-3) / 1e9:.0f} GB/s (rel L2 {rel:.1e})")
        del kd, vd, ws
    return out


def small_batch(wl, stream, reps=50):
    """One 8B-shape layer's four levels and the int8 output projection with
    argmax, applied to B activation vectors per pass (the weights stream once
    per pass whatever B is); one HIP graph per B.  The pass is one call of
    the decode step on the tiled weights: the stream schedule for B = 1, the
    batched pass for B = 4, 8, 16.  Also timed: the same products as five
    separate calls (B = 1: the per-call kernels on row-major weights; B > 1: the
    per-call matrix-core kernels on tiled weights), and the batched pass over
    all 36 layers.  Reports weight bytes per second and effective integer
    operations per second (2 per weight per vector)."""
    import torch

    import packed_weight_gemv_amd as pwg
    import synth
    rows_w, table = wl.weights[pwg.LAYOUT_ROWS]   # the batch-1 per-call kernels take row-major weights
    levels = [(w, sc, r, k) for w, (_, sc, _, _, r, k) in zip(rows_w[:4], wl.desc.levels[:4])]
    tiled = wl.weights[pwg.LAYOUT_TILED]
    tlevels = [(w, sc, r, k) for w, (_, sc, _, _, r, k) in zip(tiled[0][:4], wl.desc.levels[:4])]
    tscale = wl.desc.out_scale
    vocab, hidden = table.shape
    t2_weights = sum(r * k for _, _, r, k in levels)
    bytes_ = sum(w.numel() * w.element_size() + sc.numel() * 4 for w, sc, _, _ in levels) + table.numel() + tscale.numel() * 4
    n_all = len(wl.desc.levels) // 4
    all_weights = sum(r * k for (_, _, _, _, r, k) in wl.desc.levels) + vocab * hidden
    all_bytes = wl.algorithmic_bytes()["total"]
    out = []
    for batch in (1, 4, 8, 16):
        d = pass_desc(wl, 1, batch, 20)
        g = capture(lambda: pwg.decode_step_weights(d, stream=stream), stream)
        us = time_graph(g, stream, reps, 5) * 1e3
        pwg.step_status(d)
        del g

        xs = [torch.from_numpy(synth.batch_inputs(batch, k, 20 + i)).to("cuda:0") for i, (_, _, _, k) in enumerate(levels)]
        ys = [torch.empty((batch, r), dtype=torch.float32, device="cuda:0") for _, _, r, _ in levels]
        h = torch.from_numpy(synth.batch_inputs(batch, hidden, 30)).to("cuda:0")
        ws = torch.zeros(pwg.argmax_workspace_bytes(vocab, batch), dtype=torch.uint8, device="cuda:0")
        tok = torch.empty(batch, dtype=torch.int32, device="cuda:0")
        tws = [torch.zeros(max(1, pwg.batch_workspace_bytes(k, batch)), dtype=torch.uint8, device="cuda:0")
               for _, _, _, k in levels]

        def calls():
            if batch > 1:
                for (w, sc, r, k), x, y, wsl in zip(tlevels, xs, ys, tws):
                    pwg.ternary_gemv_tiled(w, sc, r, k, x, y=y, workspace=wsl, stream=stream)
                pwg.int8_gemv_argmax_tiled(tiled[1], tscale, vocab, hidden, h, workspace=ws, token_out=tok,
                                           stream=stream)
                return
            for (w, sc, r, k), x, y in zip(levels, xs, ys):
                pwg.ternary_gemv(w, sc, r, k, x[0], y=y[0], stream=stream)
            pwg.int8_gemv_argmax(table, tscale, h[0], workspace=ws, token_out=tok, stream=stream)
        g = capture(calls, stream)
        us_calls = time_graph(g, stream, reps, 5) * 1e3
        del g

        ops = 2.0 * (t2_weights + vocab * hidden) * batch
        row = {"batch": batch,
               "pass": "stream schedule (one kernel pair)" if batch == 1 else "batched pass (one kernel pair)",
               "us_per_pass": us, "weight_GBps": bytes_ / us / 1e3,
               "pct_of_hbm_peak": 100.0 * bytes_ / (us * 1e-6) / PEAK_HBM_BPS,
               "effective_Tops": ops / us / 1e6,
               "us_per_pass_separate_calls": us_calls,
               "separate_calls": "matrix cores, row-major weights" if batch == 1 else "matrix cores, tiled weights"}
        log(f"small batch B={batch}: {us:.1f} us per pass, {bytes_ / us / 1e3:.0f} GB/s, {ops / us / 1e6:.1f} Top/s"
            f" (separate calls {us_calls:.1f} us)")
        if batch > 1:
            d36 = pass_desc(wl, n_all, batch, 40)
            g = capture(lambda: pwg.decode_step_weights(d36, stream=stream), stream)
            us36 = time_graph(g, stream, 20, 3) * 1e3
            pwg.step_status(d36)
            del g, d36
            row["all_layers_us_per_pass"] = us36
            row["all_layers_weight_GBps"] = all_bytes / us36 / 1e3
            row["all_layers_effective_Tops"] = 2.0 * all_weights * batch / us36 / 1e6
            log(f"  all {n_all} layers B={batch}: {us36:.1f} us per pass, {all_bytes / us36 / 1e3:.0f} GB/s")
        out.append(row)
    return {"config": ("one 8B-shape layer (q|k|v 6144x4096, o 4096x4096, gate|up 24576x4096, down 4096x12288 "
                       "ternary) + int8 output projection 151936x4096 with per-vector argmax, B fp32 N(0,1) "
                       "vectors per pass, one HIP graph per B; also every layer of the step at B > 1"),
            "weight_bytes_per_pass": bytes_, "all_layers_weight_bytes_per_pass": all_bytes, "results": out}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is not built "
                                   "(see the design notes for how the path would shard)", "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np  # noqa: F401
    import torch

    import packed_weight_gemv_amd as pwg
    from oracle import reference as ref
    from packed_weight_gemv_amd.workload import build_step, make_chained

    assert torch.cuda.is_available(), "bench needs a GPU"
    if args.attention_only:
        print(json.dumps({"decode_attention": decode_attention(torch.cuda.Stream())}), flush=True)
        return
    schedule = {"levels": pwg.SCHEDULE_LEVELS, "stream": pwg.SCHEDULE_STREAM}[args.schedule]
    t0 = time.time()
    # both weight arrangements when other schedules or the small-batch
    # kernels (row-major) run next to a tiled stream step
    both = not (args.no_compare and args.no_small_batch)
    wl = build_step(n_layers=args.layers, schedule=schedule, with_logits=False, both_layouts=both)
    log(f"workload built in {time.time() - t0:.1f}s: {len(wl.desc.levels)} levels")
    bytes_ = wl.algorithmic_bytes()
    step_bytes = bytes_["total"]

    stream = torch.cuda.Stream()
    if args.counters:
        wl.set_schedule(schedule)
        pwg.step_plan(wl.desc, stream=stream)
        with torch.cuda.stream(stream):
            for _ in range(3):
                pwg.decode_step_weights(wl.desc, stream=stream)
            src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")   # 1 GiB
            dst = torch.empty_like(src)
            dst.copy_(src)
            del src, dst
            # the per-call kernels on the same kinds of work, for the VALU / MFMA
            # busy counters: the row-major ternary GEMV (matrix cores) on a
            # 393,216 x 4,096 matrix (402 MB, more than the last-level cache;
            # arbitrary bytes: the instruction stream does not depend on the
            # values) and the VALU int8 projection on the output table
            rows_big, cols_big = 393216, 4096
            wbig = torch.randint(0, 256, (pwg.packed_size(rows_big, cols_big),), dtype=torch.uint8,
                                 device="cuda:0")
            sbig = torch.full((rows_big,), 0.05, dtype=torch.float32, device="cuda:0")
            xbig = torch.randn(cols_big, dtype=torch.float32, device="cuda:0")
            ybig = torch.empty(rows_big, dtype=torch.float32, device="cuda:0")
            table = wl.weights[pwg.LAYOUT_ROWS][1] if pwg.LAYOUT_ROWS in wl.weights else None
            for _ in range(3):
                pwg.ternary_gemv(wbig, sbig, rows_big, cols_big, xbig, y=ybig, stream=stream)
                if table is not None:
                    pwg.int8_gemv_argmax(table, wl.desc.out_scale, wl.desc.h, stream=stream)
            # the same matrix shape tiled (T2) and in the base-3 device arrangement
            wt2 = pwg.tile_rows(wbig, rows_big, cols_big // 4, stream=stream)
            del wbig
            wb3 = pwg.tile_b3(torch.randint(0, 243, (pwg.b3_packed_size(rows_big, cols_big),), dtype=torch.uint8,
                                            device="cuda:0"), rows_big, cols_big, stream=stream)
            for _ in range(3):
                pwg.ternary_gemv_tiled(wt2, sbig, rows_big, cols_big, xbig, y=ybig, stream=stream)
                pwg.ternary_gemv_b3(wb3, sbig, rows_big, cols_big, xbig, y=ybig, stream=stream)
            del wt2, wb3
            # small batch (16 vectors) on the per-call matrix-core kernels: the
            # gate|up level (24576 x 4096) and the output table, tiled
            if pwg.LAYOUT_TILED in wl.weights:
                B = 16
                wt = wl.weights[pwg.LAYOUT_TILED][0][2]
                _, sc, _, _, r, k = wl.desc.levels[2]
                xb = torch.randn(B, k, device="cuda:0")
                yb = torch.empty(B, r, device="cuda:0")
                tws = torch.empty(pwg.batch_workspace_bytes(k, B), dtype=torch.uint8, device="cuda:0")
                hb = torch.randn(B, wl.desc.hidden, device="cuda:0")
                iws = torch.empty(pwg.argmax_workspace_bytes(wl.desc.vocab, B), dtype=torch.uint8, device="cuda:0")
                for _ in range(3):
                    pwg.ternary_gemv_tiled(wt, sc, r, k, xb, y=yb, workspace=tws, stream=stream)
                    pwg.int8_gemv_argmax_tiled(wl.weights[pwg.LAYOUT_TILED][1], wl.desc.out_scale, wl.desc.vocab,
                                               wl.desc.hidden, hb, workspace=iws, stream=stream)
        torch.cuda.synchronize()
        pwg.step_status(wl.desc, stream=stream)
        # the batched pass over every layer and the output table, 4 and 16 vectors
        if pwg.LAYOUT_TILED in wl.weights:
            for B in (4, 16):
                d = pass_desc(wl, len(wl.desc.levels) // 4, B, 40)
                with torch.cuda.stream(stream):
                    for _ in range(3):
                        pwg.decode_step_weights(d, stream=stream)
                torch.cuda.synchronize()
                pwg.step_status(d, stream=stream)
                del d
        log("counter run done: 3 steps, one 1 GiB device-to-device copy, 3 row-major ternary GEMVs "
            "(393216x4096), 3 row-major int8 projections, 3 tiled and 3 base-3 ternary GEMVs of the same shape, "
            "3 x 2 tiled small-batch calls (16 vectors) and 3 "
            "batched passes over every layer at 4 and at 16 vectors")
        return

    def run(desc_schedule):
        wl.set_schedule(desc_schedule)
        pwg.step_plan(wl.desc, stream=stream)
        return lambda: pwg.decode_step_weights(wl.desc, stream=stream)

    # 2. parity of the schedule that is timed (two steps: the second gathers
    #    the row of the first step's token, as every timed step does)
    step_fn = run(schedule)
    with torch.cuda.stream(stream):
        step_fn()
        stream.synchronize()
        token1 = int(wl.desc.token_out.cpu()[0])
        step_fn()
        stream.synchronize()
    pwg.step_status(wl.desc, stream=stream)
    par = parity(wl, ref, token1)
    log(f"parity ok: {par}")

    # 3. timed graph replays.  A graph holds S = --steps-per-graph consecutive
    #    steps (each step's token feeds the next step's embedding row on the
    #    device, so the S steps are a decode loop; one graph launch per S
    #    steps).  A time-based pre-warm (clocks settle whatever --warmup
    #    says), --warmup untimed steps, then exactly --steps timed steps
    #    (steps // S replays of the S-step graph, steps % S of the one-step
    #    graph); then repeated rounds of --steps steps for the spread.  The
    #    one-step graph (a graph launch per step) and launches without a
    #    graph are timed too.
    S = max(1, args.steps_per_graph)
    graph = capture(step_fn, stream)
    graph_s = capture(lambda: [step_fn() for _ in range(S)], stream) if S > 1 else graph
    n_pre = prewarm(graph_s, stream, args.prewarm)
    ms = time_steps(graph_s, graph, S, stream, args.steps, args.warmup)[0]
    rounds = time_steps(graph_s, graph, S, stream, args.steps, 0, args.rounds)
    pwg.step_status(wl.desc, stream=stream)
    log(f"{args.schedule}: {ms * 1e3:.1f} us/step, {S} steps per graph (after {n_pre} pre-warm replays); over "
        f"{args.rounds} more rounds of {args.steps}: {spread(rounds)}")
    prewarm(graph, stream, 0.1)
    ms1 = time_graph(graph, stream, args.steps, args.warmup)
    pwg.step_status(wl.desc, stream=stream)
    log(f"{args.schedule}, one step per graph: {ms1 * 1e3:.1f} us/step")
    ms_direct = time_direct(step_fn, stream, args.steps, args.warmup)
    pwg.step_status(wl.desc, stream=stream)
    log(f"{args.schedule} without a graph: {ms_direct * 1e3:.1f} us/step")
    del graph_s
    kernels_per_step = {pwg.SCHEDULE_STREAM: 2}.get(schedule, len(wl.desc.levels) + 3)

    extra = {}
    if not args.no_compare:
        names = {pwg.SCHEDULE_LEVELS: "levels", pwg.SCHEDULE_STREAM: "stream", pwg.SCHEDULE_PERSISTENT: "persistent"}
        for other in (pwg.SCHEDULE_LEVELS, pwg.SCHEDULE_STREAM, pwg.SCHEDULE_PERSISTENT):
            if other == schedule:
                continue
            other_fn = run(other)
            with torch.cuda.stream(stream):   # parity of the compared schedule's token
                other_fn()
                stream.synchronize()
            pwg.step_status(wl.desc, stream=stream)
            g2 = capture(other_fn, stream)
            ms_other = time_graph(g2, stream, args.steps, args.warmup)
            pwg.step_status(wl.desc, stream=stream)
            extra[f"{names[other]}_schedule_us"] = ms_other * 1e3
            del g2
            log(f"{names[other]}: {ms_other * 1e3:.1f} us/step")
        # null twin graph: as many empty kernels as the levels schedule launches
        one = torch.zeros(1, device="cuda:0")
        n_null = len(wl.desc.levels) + 3
        gnull = capture(lambda: [one.add_(0) for _ in range(n_null)], stream)
        ms_null = time_graph(gnull, stream, args.steps, args.warmup)
        extra["null_graph_us"] = ms_null * 1e3
        extra["null_graph_kernels"] = n_null
        # chained step: every level's input formed from earlier outputs
        # (RMSNorm, one-position attention, SwiGLU, residual sums) on the
        # ordered schedules, the dependency chain the stream step leaves out
        for sched_c in (pwg.SCHEDULE_LEVELS, pwg.SCHEDULE_PERSISTENT):
            cs = make_chained(wl, schedule=sched_c)
            pwg.step_plan(cs.desc, stream=stream)
            chain_fn = lambda: pwg.decode_step_weights(cs.desc, stream=stream)  # noqa: E731
            with torch.cuda.stream(stream):
                chain_fn()
                stream.synchronize()
            pwg.step_status(cs.desc, stream=stream)
            tok = int(cs.desc.token_out.cpu()[0])
            if not (0 <= tok < wl.desc.vocab and bool(torch.isfinite(cs.desc.h).all())):
                raise SystemExit(f"chained step produced token {tok} / non-finite hidden state")
            g3 = capture(chain_fn, stream)
            ms_chain = time_graph(g3, stream, args.steps, args.warmup)
            pwg.step_status(cs.desc, stream=stream)
            del g3
            extra[f"chained_{names[sched_c]}_us"] = ms_chain * 1e3
            log(f"chained step, {names[sched_c]} schedule: {ms_chain * 1e3:.1f} us/step")
            del cs
        run(schedule)  # restore the timed schedule's plan

    achieved_bps = step_bytes / (ms * 1e-3)
    floor_us = step_bytes / PEAK_HBM_BPS * 1e6
    result = {
        "metric": METRIC,
        "value": achieved_bps / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_step": ms * 1e3,
        "pct_of_hbm_peak": 100.0 * achieved_bps / PEAK_HBM_BPS,
        "floor_us": floor_us,
        "step_over_floor": ms * 1e3 / floor_us,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f32: ternary FP4 x six e4m3 pieces of x (block-scaled MFMA, exact products, f32 sums); "
                  "int8 x six int8 digits of h (MFMA, exact i32 sums per section); f32 row scales"),
        "data": "synthetic seeded (ternary iid p=1/3, int8 U[-127,127], activations N(0,1))",
        "config": {
            "workload": (f"8B-shape batch-1 decode step: embedding row + {args.layers} layers x (q|k|v 6144x4096, "
                         "o 4096x4096, gate|up 24576x4096, down 4096x12288) ternary T2 + int8 output projection "
                         f"151936x4096 + greedy argmax; HIP graphs of {S} chained steps"),
            "schedule": args.schedule,
            "kernels_per_step": kernels_per_step,
            "algorithmic_bytes_per_step": bytes_,
        },
        "parity": par,
        "timing": {"steps_per_graph": S, "prewarm_replays": n_pre, "prewarm_s": args.prewarm,
                   "warmup_steps": args.warmup, "timed_steps": args.steps, "spread_over_rounds": spread(rounds)},
        "packing": packing_report(wl),
    }
    result.update(extra)

    result["us_per_step_one_step_per_graph"] = ms1 * 1e3
    result["us_per_step_without_graph"] = ms_direct * 1e3
    result["graph_launch_us_per_replay"] = (ms1 - ms) * 1e3 * S / max(1, S - 1) if S > 1 else None

    # roofline of the dominant kernel: the step kernel moves every
    # algorithmic byte of the step; its time is the per-step time of the
    # S-step graph (HIP events on the replay stream), i.e. the step kernel
    # and its input-conversion kernel (about 7 us) back to back
    if schedule == pwg.SCHEDULE_STREAM:
        traffic = None
        tfile = os.path.join(ROOT, "profiles", "step_kernel_traffic.json")
        if os.path.exists(tfile):
            t = json.load(open(tfile))
            if (t.get("kernel_source_sha") == kernel_source_sha(args.schedule) and t.get("layers") == args.layers
                    and t.get("schedule") == args.schedule):
                traffic = t.get("hbm_bytes_per_launch")
        kname = "stream_step_kernel<8> (whole step; timed with its input-conversion kernel)"
        kernel_bps = step_bytes / (ms * 1e-3)
        result["roofline"] = {"bound": "hbm", "achieved": kernel_bps / 1e9, "peak": PEAK_HBM_BPS / 1e9,
                              "unit": "GB/s", "frac": kernel_bps / PEAK_HBM_BPS, "traffic": traffic,
                              "kernel": kname, "per_launch_bytes": step_bytes, "avg_launch_us": ms * 1e3}
    result["kernel_source_sha"] = kernel_source_sha(args.schedule)

    if not args.no_units and pwg.LAYOUT_ROWS in wl.weights:
        result["units"] = standalone_units(wl, stream)
    if not args.no_small_batch:
        result["small_batch"] = small_batch(wl, stream)
    if not args.no_units and pwg.LAYOUT_ROWS in wl.weights:
        result["base3_lane"] = base3_lane(wl, stream)
    if not args.no_compare:
        result["decode_attention"] = decode_attention(stream)

    # 5. oracle CPU baseline (bounded sample), in rounds interleaved with GPU
    #    rounds of the timed step
    if not args.no_cpu_baseline:
        t0 = time.time()
        run(schedule)
        g_cpu = capture(step_fn, stream)
        prewarm(g_cpu, stream, 0.05)
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, step_bytes,
                                              gpu_round=lambda: time_rounds(g_cpu, stream, args.steps, 1)[0])
        del g_cpu
        log(f"cpu baseline in {time.time() - t0:.1f}s: {result['cpu_baseline']['us_per_step'] / 1e6:.1f} s per step "
            f"on {result['cpu_baseline']['cores']} threads, {result['cpu_baseline']['one_core']['us_per_step'] / 1e6:.1f}"
            f" s on one ({result['cpu_baseline']['cpu_model']})")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
