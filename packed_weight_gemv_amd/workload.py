"""Device-resident synthetic decode-step workloads.

Generates the seeded logical weights (synth), packs each level with the
library's packer, uploads packed weights, scales and level inputs to the GPU
and fills a StepDesc.  Logical weights are dropped after packing, except for
a sample of rows per level kept on the host so that a caller can check
sampled outputs at full size.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import synth

from . import (LAYOUT_ROWS, LAYOUT_TILED, SCHEDULE_LEVELS, StepDesc, layout_for_schedule, pack_weights,
               step_workspace_bytes, tile_rows)

LEVEL_NAMES = [name for name, _, _ in synth.LEVELS]


@dataclass
class LevelSample:
    layer: int
    level: str
    rows: np.ndarray       # sampled row indices
    w: np.ndarray          # int8 (n, cols) logical rows
    scale: np.ndarray      # float32 (n,)
    x: np.ndarray          # float32 (cols,)


@dataclass
class StepWorkload:
    desc: StepDesc
    level_shapes: list                      # [(layer, level, rows, cols)]
    samples: list = field(default_factory=list)
    out_table: object = None                # synth.Int8Table (host)
    emb_table: object = None
    h: np.ndarray = None
    token0: int = 0
    packed_bytes: int = 0
    scale_bytes: int = 0
    # device weights per arrangement: {layout: ([w per level], out_table)}
    weights: dict = field(default_factory=dict)

    def set_schedule(self, schedule: int):
        """Points the description at the weight arrangement `schedule` takes
        (both arrangements must have been built) and resizes the workspace."""
        layout = layout_for_schedule(schedule)
        ws, out = self.weights[layout]
        d = self.desc
        d.levels = [(w,) + tuple(lv[1:]) for w, lv in zip(ws, d.levels)]
        d.out_table = out
        d.schedule = schedule
        d.weight_layout = layout
        d._c = None
        need = step_workspace_bytes(d)
        if d.workspace.numel() < need:
            d.workspace = torch.zeros(need, dtype=torch.uint8, device=d.workspace.device)
            d._c = None

    def algorithmic_bytes(self) -> dict:
        vocab, hidden = self.out_table.q.shape
        out = vocab * hidden + vocab * 4
        emb = hidden + 4
        total = self.packed_bytes + self.scale_bytes + out + emb
        return {"ternary_weights": self.packed_bytes, "ternary_scales": self.scale_bytes,
                "output_table": out, "embedding_row": emb, "total": total}


def _level_arrays(workload: int, layer: int, shapes: dict):
    mats = synth.layer(workload, layer, shapes)
    xs = synth.layer_inputs(workload, layer, hidden=shapes["q"][1], inter=shapes["down"][1])
    out = []
    for name, members, _ in synth.LEVELS:
        m = synth.stacked(mats, members)
        out.append((name, m.w, m.scale, xs[name]))
    return out


def build_step(n_layers: int = synth.N_LAYERS, shapes: dict | None = None, vocab: int = synth.VOCAB,
               hidden: int = synth.HIDDEN, workload: int = synth.W_STEP, schedule: int = SCHEDULE_LEVELS,
               with_logits: bool = False, sample_rows: int = 64, device: str = "cuda:0",
               token0: int | None = None, threads: int | None = None, both_layouts: bool = False) -> StepWorkload:
    """Seeded decode-step workload on the device.  The weights are uploaded in
    the arrangement `schedule` takes (tiles for the stream schedule, arranged
    on the device by the library), or in both when `both_layouts`."""
    shapes = shapes or synth.LAYER_SHAPES
    dev = torch.device(device)
    layout = layout_for_schedule(schedule)
    layouts = (LAYOUT_ROWS, LAYOUT_TILED) if both_layouts else (layout,)
    w_by_layout = {lay: [] for lay in layouts}

    def arrange(rows_t, rows, row_bytes):
        out = {}
        if LAYOUT_TILED in layouts:
            out[LAYOUT_TILED] = tile_rows(rows_t, rows, row_bytes)
        if LAYOUT_ROWS in layouts:
            out[LAYOUT_ROWS] = rows_t
        return out

    def one_layer(layer):
        levels = _level_arrays(workload, layer, shapes)
        packed = []
        for name, w, s, x in levels:
            blob = pack_weights(w)
            idx = np.unique(np.concatenate([[0, w.shape[0] - 1],
                                            np.random.default_rng([workload, layer, 77]).integers(0, w.shape[0], sample_rows)]))
            packed.append((name, blob, s, x, w.shape, LevelSample(layer, name, idx, w[idx].copy(), s[idx].copy(), x)))
        return packed

    levels = []
    samples = []
    shapes_out = []
    packed_bytes = scale_bytes = 0
    ex_threads = threads or min(8, synth.n_workers())
    # generate/pack in parallel batches of layers, upload in order
    for start in range(0, n_layers, ex_threads):
        batch = synth.parallel_map(one_layer, list(range(start, min(n_layers, start + ex_threads))))
        for layer_off, packed in enumerate(batch):
            layer = start + layer_off
            for name, blob, s, x, (r, k), smp in packed:
                for lay, t in arrange(torch.from_numpy(blob).to(dev), r, k // 4).items():
                    w_by_layout[lay].append(t)
                wd = w_by_layout[layout][-1]
                sd = torch.from_numpy(s).to(dev)
                xd = torch.from_numpy(x).to(dev)
                yd = torch.empty(r, dtype=torch.float32, device=dev)
                levels.append((wd, sd, xd, yd, r, k))
                samples.append(smp)
                shapes_out.append((layer, name, r, k))
                packed_bytes += blob.nbytes
                scale_bytes += s.nbytes
        del batch

    out_t, emb_t, ids, h = synth.vocab_workload(rows=vocab, cols=hidden, n_ids=1, workload=workload)
    if token0 is None:
        token0 = int(ids[0])
    token = torch.tensor([token0], dtype=torch.int32, device=dev)
    out_by_layout = arrange(torch.from_numpy(out_t.q).to(dev), vocab, hidden)
    torch.cuda.synchronize(dev)
    desc = StepDesc(
        levels=levels,
        out_table=out_by_layout[layout], out_scale=torch.from_numpy(out_t.scale).to(dev),
        h=torch.from_numpy(h).to(dev),
        emb_table=torch.from_numpy(emb_t.q).to(dev), emb_scale=torch.from_numpy(emb_t.scale).to(dev),
        token_in=token, token_out=token,
        emb_row_out=torch.empty(hidden, dtype=torch.int8, device=dev),
        emb_scale_out=torch.empty(4, dtype=torch.float32, device=dev),
        emb_deq_out=torch.empty(hidden, dtype=torch.float32, device=dev),
        logits_out=torch.empty(vocab, dtype=torch.float32, device=dev) if with_logits else None,
        schedule=schedule, weight_layout=layout, vocab=vocab, hidden=hidden)
    desc.workspace = torch.zeros(1, dtype=torch.uint8, device=dev)   # sized below
    need = step_workspace_bytes(desc)
    desc.workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    desc._c = None
    return StepWorkload(desc=desc, level_shapes=shapes_out, samples=samples, out_table=out_t, emb_table=emb_t,
                        h=h, token0=token0, packed_bytes=packed_bytes, scale_bytes=scale_bytes,
                        weights={lay: (w_by_layout[lay], out_by_layout[lay]) for lay in layouts})
