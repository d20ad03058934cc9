"""Level trace of the persistent decode step: where each dependent level's
time goes (page "The Neutrino Engine", section "A 104 microsecond floor
inside a 694 microsecond step" and Fig. 1).

    python -m packed_weight_gemv_amd.trace_step [--chained] [--steps N] [--out FILE]

Builds the seeded 36-layer 8B-shape step (given level inputs, or the chained
step whose inputs are formed from earlier outputs), runs untraced steps to
warm up, then one traced step, and prints, per level kind, the median over
workgroups and layers of each phase (microseconds of the GPU's 100 MHz
real-time counter):

    wait      the control wave waits for the previous level's barrier
    copy      the level's sources are copied into LDS (device-coherent loads)
    form      element-wise formation and conversion to matrix-core operands
    products  the workgroup's tiles on the matrix cores
    publish   sums, scales, stores of the rows (and what they form for the
              next level), arrival once the stores are complete
    period    from the last arrival at the previous level to the last arrival
              at this one: the level's share of the step

Tracing adds one store per event, so the traced step runs longer than the
untraced ones; the untraced time per step is printed for comparison.
"""
from __future__ import annotations

import argparse
import time

import numpy as np
import torch

import packed_weight_gemv_amd as pwg
from packed_weight_gemv_amd.workload import LEVEL_NAMES, build_step, make_chained

TICK_US = 0.01  # 100 MHz


def phases(t: np.ndarray) -> dict:
    """Per-level, per-workgroup phase durations (microseconds) of a trace
    [levels + 1][grid][events]."""
    ev = {n: i for i, n in enumerate(pwg.TRACE_EVENT_NAMES)}
    e = lambda name: t[:, :, ev[name]].astype(np.int64)  # noqa: E731
    out = {
        "wait": e("passed") - e("wait"),
        "copy": e("start") - e("passed"),
        "form": e("converted") - e("start"),
        "products": e("products") - e("converted"),
        "publish": e("arrived") - e("products"),
    }
    return {k: v * TICK_US for k, v in out.items()}


def summarize(t: np.ndarray, level_names: list[str]) -> list[tuple]:
    nl = t.shape[0] - 1
    ph = phases(t)
    arrived = t[:nl, :, pwg.TRACE_EVENT_NAMES.index("arrived")].astype(np.int64).max(axis=1)
    period = np.diff(arrived) * TICK_US
    rows = []
    for kind in dict.fromkeys(level_names):
        idx = [i for i in range(1, nl) if level_names[i] == kind]
        row = [kind, len(idx)]
        for k in ("wait", "copy", "form", "products", "publish"):
            row.append(float(np.median(ph[k][idx])))
        row.append(float(np.median(period[[i - 1 for i in idx]])))
        rows.append(tuple(row))
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--chained", action="store_true", help="inputs formed from earlier outputs")
    ap.add_argument("--steps", type=int, default=20, help="untraced steps timed before the traced one")
    ap.add_argument("--out", help="also write the table (markdown) here")
    args = ap.parse_args(argv)
    stream = torch.cuda.Stream()
    wl = build_step(schedule=pwg.SCHEDULE_PERSISTENT)
    chain = make_chained(wl, schedule=pwg.SCHEDULE_PERSISTENT) if args.chained else None
    desc = chain.desc if chain is not None else wl.desc
    pwg.step_plan(desc, stream=stream)
    with torch.cuda.stream(stream):
        for _ in range(3):
            pwg.decode_step_weights(desc, stream=stream)
        stream.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            pwg.decode_step_weights(desc, stream=stream)
        stream.synchronize()
        us_untraced = (time.perf_counter() - t0) / args.steps * 1e6
    pwg.step_status(desc, stream=stream)
    nl = len(desc.levels)
    trace = torch.zeros(pwg.step_trace_bytes(desc) // 8, dtype=torch.int64, device="cuda:0")
    pwg.step_set_trace(desc, trace, stream=stream)
    with torch.cuda.stream(stream):
        pwg.decode_step_weights(desc, stream=stream)
        stream.synchronize()
    pwg.step_status(desc, stream=stream)
    pwg.step_set_trace(desc, None, stream=stream)
    t = trace.cpu().numpy().reshape(nl + 1, -1, pwg.TRACE_EVENTS)
    names = [LEVEL_NAMES[i % len(LEVEL_NAMES)] for i in range(nl)]
    ev = pwg.TRACE_EVENT_NAMES
    step_us = (t[nl, :, ev.index("products")].max() - t[0, :, ev.index("wait")].min()) * TICK_US
    proj = phases(t)
    lines = [f"persistent step, {'chained' if args.chained else 'given'} level inputs, {nl} levels, "
             f"{t.shape[1]} workgroups",
             f"untraced: {us_untraced:.1f} us per step (launches without a graph); traced step: {step_us:.1f} us",
             "",
             "| level | n | wait | copy | form | products | publish | period |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for r in summarize(t, names):
        lines.append(f"| {r[0]} | {r[1]} | " + " | ".join(f"{v:.2f}" for v in r[2:]) + " |")
    lines.append(f"| output projection | 1 | {np.median(proj['wait'][nl]):.2f} | {np.median(proj['copy'][nl]):.2f} | "
                 f"{np.median(proj['form'][nl]):.2f} | {np.median(proj['products'][nl]):.2f} | | |")
    lines.append("")
    lines.append("Medians over workgroups and layers, microseconds; the first level (no barrier before it) is left out.")
    text = "\n".join(lines)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
