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

from . import (INPUT_ATTN1, INPUT_EMBED_RMSNORM, INPUT_RMSNORM, INPUT_SWIGLU, LAYOUT_ROWS, LAYOUT_TILED,
               SCHEDULE_LEVELS, InputOp, StepDesc, layout_for_schedule, pack_weights, step_workspace_bytes,
               tile_rows)

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


@dataclass
class ChainStep:
    """A chained decode step over a StepWorkload's weights: every level's
    input is formed from earlier outputs (pre-norm decoder layer, attention
    at the first position).  Buffers are per level and per layer so every
    intermediate can be read back."""
    desc: StepDesc
    x: list                 # formed input of each level (device)
    y: list                 # output of each level (device)
    h: list                 # per layer (h entering the layer, h after attention) (device)
    h_final: object         # residual stream after the last layer (device)
    gains: list             # per layer (attention gain, feed-forward gain) (host float32)
    g_final: np.ndarray
    head_dim: int
    group: int
    eps: float


def make_chained(wl: StepWorkload, schedule: int = SCHEDULE_LEVELS, head_dim: int = synth.HEAD_DIM,
                 eps: float = 1e-6, workload: int = synth.W_STEP) -> ChainStep:
    """Chained step on the weights of `wl` (levels qkv, o, gate_up, down per
    layer) in the arrangement `schedule` takes (tiled copies are made on the
    device when `wl` holds only the row-major blobs).  The query rows are o's
    input width; the key and value rows split the rest of qkv equally."""
    d0 = wl.desc
    dev = d0.out_scale.device
    layout = layout_for_schedule(schedule)
    if layout not in wl.weights:
        rws, rout = wl.weights[LAYOUT_ROWS]
        tws = [tile_rows(w, lv[4], lv[5] // 4) for w, lv in zip(rws, d0.levels)]
        wl.weights[layout] = (tws, tile_rows(rout, rout.shape[0], rout.shape[1]))
        torch.cuda.synchronize(dev)
    ws_rows, out_rows = wl.weights[layout]
    hidden = d0.hidden
    n_layers = len(d0.levels) // 4
    f32 = dict(dtype=torch.float32, device=dev)
    levels, xs, ys, hs, gains = [], [], [], [], []
    prev_mid = prev_down = None
    for layer in range(n_layers):
        lv = [d0.levels[4 * layer + j] for j in range(4)]
        qkv_rows, q_rows, inter = lv[0][4], lv[1][5], lv[3][5]
        kv_rows = (qkv_rows - q_rows) // 2
        ga = synth.norm_gain(workload, layer, synth.GAIN_ATTN, hidden)
        gm = synth.norm_gain(workload, layer, synth.GAIN_MLP, hidden)
        gains.append((ga, gm))
        x = [torch.empty(lv[j][5], **f32) for j in range(4)]
        y = [torch.empty(lv[j][4], **f32) for j in range(4)]
        h_l, h_mid = torch.empty(hidden, **f32), torch.empty(hidden, **f32)
        g_attn, g_mlp = torch.from_numpy(ga).to(dev), torch.from_numpy(gm).to(dev)
        if layer == 0:
            op0 = InputOp(INPUT_EMBED_RMSNORM, gamma=g_attn, resid_out=h_l, eps=eps)
        else:
            op0 = InputOp(INPUT_RMSNORM, src=prev_down, resid=prev_mid, gamma=g_attn, resid_out=h_l, eps=eps)
        ops = [op0,
               InputOp(INPUT_ATTN1, src=y[0][q_rows + kv_rows:], head_dim=head_dim, group=q_rows // kv_rows),
               InputOp(INPUT_RMSNORM, src=y[1], resid=h_l, gamma=g_mlp, resid_out=h_mid, eps=eps),
               InputOp(INPUT_SWIGLU, src=y[2])]
        assert y[2].numel() == 2 * inter
        for j in range(4):
            levels.append((ws_rows[4 * layer + j], lv[j][1], x[j], y[j], lv[j][4], lv[j][5], ops[j]))
        xs.extend(x)
        ys.extend(y)
        hs.append((h_l, h_mid))
        prev_mid, prev_down = h_mid, y[3]
    gf = synth.norm_gain(workload, -1, synth.GAIN_FINAL, hidden)
    h_final = torch.empty(hidden, **f32)
    h_out = torch.empty(hidden, **f32)
    desc = StepDesc(
        levels=levels, out_table=out_rows, out_scale=d0.out_scale, h=h_out, emb_table=d0.emb_table,
        emb_scale=d0.emb_scale, token_in=torch.tensor([wl.token0], dtype=torch.int32, device=dev),
        token_out=None, emb_row_out=torch.empty(hidden, dtype=torch.int8, device=dev),
        emb_scale_out=torch.empty(4, **f32), emb_deq_out=torch.empty(hidden, **f32),
        logits_out=torch.empty(d0.vocab, **f32) if d0.logits_out is not None else None,
        schedule=schedule, weight_layout=layout, vocab=d0.vocab, hidden=hidden,
        h_in=InputOp(INPUT_RMSNORM, src=prev_down, resid=prev_mid, gamma=torch.from_numpy(gf).to(dev),
                     resid_out=h_final, eps=eps))
    desc.token_out = desc.token_in
    desc.workspace = torch.zeros(1, dtype=torch.uint8, device=dev)
    desc.workspace = torch.zeros(max(step_workspace_bytes(desc), 16), dtype=torch.uint8, device=dev)
    desc._c = None
    return ChainStep(desc=desc, x=xs, y=ys, h=hs, h_final=h_final, gains=gains, g_final=gf,
                     head_dim=head_dim, group=levels[4][6].group if n_layers else 1, eps=eps)
