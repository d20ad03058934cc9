"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/pwg.h declares, packs T2 bit-exactly as the oracle's
independent encoder does, and rejects bad arguments with the documented codes
before anything reaches the GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import packed_format as pf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pwg = pytest.importorskip("packed_weight_gemv_amd")

ERR_ARG, ERR_ALIGN, ERR_SIZE, ERR_VALUE, ERR_UNSUPPORTED = -1, -2, -3, -4, -6


def header_functions():
    text = open(os.path.join(ROOT, "include", "pwg.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pwg_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    declared = header_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(pwg.lib, name), name
    assert sorted(pwg.EXPORTED) == declared


def test_version_and_error_string():
    assert pwg.version() == 7
    assert isinstance(pwg.last_error(), str)


def test_packed_size():
    assert pwg.packed_size(4096, 4096) == 4096 * 4096 // 4
    assert pwg.packed_size(1, 64) == 16
    for bad in ((0, 64), (1, 0), (1, 100), (-1, 64)):
        assert pwg.packed_size(*bad) == 0


@pytest.mark.parametrize("shape", [(1, 64), (3, 128), (37, 1024), (5, 4160), (2048, 4096)])
def test_pack_matches_oracle_encoder_bit_for_bit(shape):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    w = rng.integers(-1, 2, size=shape, dtype=np.int8)
    blob = pwg.pack_weights(w)
    assert blob.size == pf.packed_nbytes(*shape)
    assert np.array_equal(blob, pf.encode(w))
    assert np.array_equal(pf.decode(blob, *shape), w)
    assert np.array_equal(pwg.unpack_weights(blob, *shape), w)


def test_pack_large_multithreaded_matches_oracle():
    rng = np.random.default_rng(5)
    w = rng.integers(-1, 2, size=(1536, 4096), dtype=np.int8)   # above the threading threshold
    assert np.array_equal(pwg.pack_weights(w), pf.encode(w))


def test_pack_hand_fixture(golden_dir):
    import json
    case = json.load(open(os.path.join(golden_dir, "t2_bytes.json")))["cases"][0]
    w = np.zeros((case["rows"], case["cols"]), np.int8)
    for k, v in case["nonzero"].items():
        w[0, int(k)] = v
    assert pwg.pack_weights(w).tobytes() == bytes.fromhex(case["bytes_hex"])


def test_pack_rejects_values_outside_ternary_and_names_the_first():
    w = np.zeros((4, 128), np.int8)
    w[2, 77] = 2
    w[3, 5] = -2
    with pytest.raises(pwg.PwgError) as e:
        pwg.pack_weights(w)
    assert e.value.code == ERR_VALUE
    assert "row 2" in str(e.value) and "col 77" in str(e.value)


def test_pack_argument_errors():
    w = np.zeros((2, 64), np.int8)
    out = np.zeros(32, np.uint8)
    n = C.c_size_t(0)
    assert pwg._pack(None, 2, 64, out.ctypes.data, 32, C.byref(n)) == ERR_ARG
    assert pwg._pack(w.ctypes.data, 2, 64, None, 32, C.byref(n)) == ERR_ARG
    assert pwg._pack(w.ctypes.data, 2, 60, out.ctypes.data, 32, C.byref(n)) == ERR_ARG
    assert pwg._pack(w.ctypes.data, 0, 64, out.ctypes.data, 32, C.byref(n)) == ERR_ARG
    assert pwg._pack(w.ctypes.data, 2, 64, out.ctypes.data, 31, C.byref(n)) == ERR_SIZE
    assert pwg._pack(w.ctypes.data, 2, 64, out.ctypes.data, 32, C.byref(n)) == 0 and n.value == 32


def test_unpack_rejects_invalid_code():
    blob = np.zeros(16, np.uint8)
    blob[9] = 0b10 << 4   # word 2, byte 1, high nibble, low pair: weight 32 + 10
    with pytest.raises(pwg.PwgError) as e:
        pwg.unpack_weights(blob, 1, 64)
    assert e.value.code == ERR_VALUE and "col 42" in str(e.value)


# Fake, never-dereferenced device addresses: validation must reject the call
# before any HIP work is enqueued.
A = 1 << 20          # 16-byte aligned
MIS = A + 4          # misaligned


def test_ternary_gemv_argument_errors():
    f = pwg._tgemv
    assert f(None, A, 8, 64, A, 1, A, None) == ERR_ARG
    assert f(A, A, 0, 64, A, 1, A, None) == ERR_ARG
    assert f(A, A, 8, 96, A, 1, A, None) == ERR_ARG
    assert f(A, A, 8, 16448, A, 1, A, None) == ERR_ARG          # above the column limit
    assert f(A, A, 8, 64, A, 3, A, None) == ERR_ARG             # batch not in {1,4,8,16}
    assert f(A, A, 8, 64, MIS, 1, A, None) == ERR_ALIGN
    assert f(A, A, 8, 64, A, 1, None, None) == ERR_ARG
    assert f(A, A, 8, 64, A, 2, A, None) == ERR_ARG and "batch" in pwg.last_error()


def test_batch_tiled_argument_errors():
    """The batched matrix-core entry points validate before launching."""
    bw = pwg.batch_workspace_bytes
    assert bw(4096, 16) >= 16 * 4096 * 4 and bw(4096, 4) >= 4 * 4096 * 4
    assert bw(4096, 1) == 16 and bw(1024, 1) == 16 and bw(4160, 1) == 0      # batch 1: no scratch, cols % 256
    assert bw(4096, 2) == 0 and bw(1024, 4) == 0 and bw(3072, 4) == 0 and bw(32768, 4) == 0
    f = pwg._tgemv_tiled
    ws = bw(4096, 8)
    assert f(None, A, 64, 4096, A, 8, A, A, ws, None) == ERR_ARG
    assert f(A, A, 64, 4096, A, 8, A, None, ws, None) == ERR_ARG
    assert f(MIS, A, 64, 4096, A, 8, A, A, ws, None) == ERR_ALIGN
    assert f(A, A, 64, 4096, A, 8, A, A, ws - 1, None) == ERR_SIZE
    assert f(A, A, 64, 4096, A, 2, A, A, ws, None) == ERR_ARG and "batch" in pwg.last_error()
    assert f(A, A, 64, 1024, A, 8, A, A, ws, None) == ERR_UNSUPPORTED
    assert f(A, A, 0, 4096, A, 8, A, A, ws, None) == ERR_ARG
    assert f(A, A, 64, 4160, A, 1, A, A, 16, None) == ERR_UNSUPPORTED and "256" in pwg.last_error()
    g = pwg._i8argmax_tiled
    iw = pwg.argmax_workspace_bytes(1000, 4)
    assert g(A, A, 1000, 4096, A, 1, A, iw, A, None, None) == ERR_ARG
    assert g(A, A, 1000, 768, A, 4, A, iw, A, None, None) == ERR_UNSUPPORTED
    assert g(A, A, 1000, 4096, A, 4, A, iw - 8, A, None, None) == ERR_SIZE
    assert g(A, A, 1000, 4096, A, 4, A, iw, None, None, None) == ERR_ARG
    assert g(A, A, 1000, 4096, A, 4, A, iw, A, MIS, None) == ERR_ALIGN


def test_int8_argmax_argument_errors():
    f = pwg._i8argmax
    ws = pwg.argmax_workspace_bytes(1000, 1)
    # batch > 1: every vector's partial keys plus the operand area of the
    # matrix-core kernel, sized for the widest table (8,192 columns, one
    # byte per value and B-operand column, four columns per vector)
    assert ws >= 8 and pwg.argmax_workspace_bytes(1000, 4) >= 4 * ws + 4 * 8192 * 4
    assert pwg.argmax_workspace_bytes(1000, 16) >= 16 * ws + 16 * 8192 * 4
    assert pwg.argmax_workspace_bytes(0, 1) == 0 and pwg.argmax_workspace_bytes(10, 3) == 0
    assert f(A, A, 1000, 4096, A, 1, A, ws - 8, A, None, None) == ERR_SIZE
    assert f(A, A, 1000, 4096, A, 1, None, ws, A, None, None) == ERR_ARG
    assert f(A, A, 1000, 4096, A, 1, A, ws, A, MIS, None) == ERR_ALIGN
    assert f(A, A, 1000, 12288, A, 1, A, ws, A, None, None) == ERR_UNSUPPORTED
    assert f(A, A, 1000, 4096, A, 5, A, ws, A, None, None) == ERR_ARG


def test_embed_gather_argument_errors():
    f = pwg._gather
    assert f(A, A, 100, 4096, A, 0, A, A, None, None) == 0           # n == 0 is a no-op
    assert f(A, A, 100, 4096, A, -1, A, A, None, None) == ERR_ARG
    assert f(None, A, 100, 4096, A, 4, A, A, None, None) == ERR_ARG
    assert f(A, A, 100, 4096, A, 4, A, A, MIS, None) == ERR_ALIGN


def test_step_argument_errors():
    assert pwg._step(None, None) == ERR_ARG
    d = pwg._StepDesc()
    d.n_levels = 0
    d.schedule = 7
    assert pwg._step(C.byref(d), None) == ERR_ARG and "schedule" in pwg.last_error()
    d.schedule = pwg.SCHEDULE_LEVELS
    d.vocab, d.hidden = 1000, 4096
    for name in ("out_table", "out_scale", "h", "emb_table", "emb_scale", "token_in", "token_out",
                 "emb_row_out", "emb_scale_out", "workspace"):
        setattr(d, name, A)
    d.workspace_bytes = 0
    assert pwg._step(C.byref(d), None) == ERR_SIZE
    d.workspace_bytes = pwg._step_ws(C.byref(d))
    d.h = MIS
    assert pwg._step(C.byref(d), None) == ERR_ALIGN
    d.h = A
    lv = (pwg.Level * 1)(pwg.Level(A, A, A, A, 8, 100))
    d.n_levels, d.levels = 1, C.cast(lv, C.POINTER(pwg.Level))
    assert pwg._step(C.byref(d), None) == ERR_ARG and "level 0" in pwg.last_error()


def test_step_trace_host_errors():
    """The level trace belongs to the persistent schedule: another schedule is
    refused, and without a device no trace buffer size is reported."""
    d = pwg._StepDesc()
    d.vocab, d.hidden = 1000, 4096
    for name in ("out_table", "out_scale", "h", "emb_table", "emb_scale", "token_in", "token_out",
                 "emb_row_out", "emb_scale_out", "workspace"):
        setattr(d, name, A)
    lv = (pwg.Level * 1)(pwg.Level(A, A, A, A, 64, 4096))
    d.n_levels, d.levels = 1, C.cast(lv, C.POINTER(pwg.Level))
    d.schedule, d.weight_layout = pwg.SCHEDULE_STREAM, pwg.LAYOUT_TILED
    assert pwg._step_trace_bytes(C.byref(d)) == 0
    assert pwg._step_set_trace(C.byref(d), None, 0, None) == ERR_UNSUPPORTED
    d.schedule = pwg.SCHEDULE_PERSISTENT
    assert pwg._step_trace_bytes(C.byref(d)) == 0   # no device here


def test_step_layout_errors():
    """Each schedule takes one weight arrangement; the stream and persistent
    schedules also need widths that are multiples of 256 and at most 12288."""
    d = pwg._StepDesc()
    d.vocab, d.hidden = 1000, 4096
    for name in ("out_table", "out_scale", "h", "emb_table", "emb_scale", "token_in", "token_out",
                 "emb_row_out", "emb_scale_out", "workspace"):
        setattr(d, name, A)
    lv = (pwg.Level * 1)(pwg.Level(A, A, A, A, 64, 4096))
    d.n_levels, d.levels = 1, C.cast(lv, C.POINTER(pwg.Level))
    d.weight_layout = 5
    assert pwg._step(C.byref(d), None) == ERR_ARG and "layout" in pwg.last_error()
    d.schedule, d.weight_layout = pwg.SCHEDULE_STREAM, pwg.LAYOUT_ROWS
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED
    d.schedule, d.weight_layout = pwg.SCHEDULE_PERSISTENT, pwg.LAYOUT_ROWS
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED
    d.weight_layout = pwg.LAYOUT_TILED
    d.workspace_bytes = pwg._step_ws(C.byref(d))
    assert d.workspace_bytes > 0
    lv[0] = pwg.Level(A, A, A, A, 64, 4160)            # not a multiple of 256
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED and "256" in pwg.last_error()
    lv[0] = pwg.Level(A, A, A, A, 64, 4096)
    d.batch = 4                                        # the persistent step is batch 1 only
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED
    d.batch = 0
    d.schedule, d.weight_layout = pwg.SCHEDULE_STREAM, pwg.LAYOUT_TILED
    d.workspace_bytes = pwg._step_ws(C.byref(d))
    assert d.workspace_bytes > 0
    lv[0] = pwg.Level(A, A, A, A, 64, 4160)            # not a multiple of 256
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED and "256" in pwg.last_error()
    lv[0] = pwg.Level(A, A, A, A, 64, 16384)           # wider than the LDS operand buffers
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED
    lv[0] = pwg.Level(A, A, A, A, 64, 4096)
    d.hidden = 4160
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED


def test_batched_step_errors():
    """A batched pass (batch 4, 8, 16) takes the stream schedule, tiled
    weights, level widths that are multiples of 2048 and a hidden width that
    is a multiple of 1024; every call here fails validation before anything
    is enqueued."""
    P = lambda k: (1 << 36) + k * (1 << 24)  # noqa: E731  (distinct buffers)
    d = pwg._StepDesc()
    d.vocab, d.hidden = 1000, 4096
    for i, name in enumerate(("out_table", "out_scale", "h", "emb_table", "emb_scale", "token_in", "token_out",
                              "emb_row_out", "emb_scale_out", "workspace")):
        setattr(d, name, P(i))
    lv = (pwg.Level * 2)(pwg.Level(P(20), P(21), P(22), P(23), 64, 4096),
                         pwg.Level(P(24), P(25), P(26), P(27), 100, 12288))
    d.n_levels, d.levels = 2, C.cast(lv, C.POINTER(pwg.Level))
    d.schedule, d.weight_layout = pwg.SCHEDULE_STREAM, pwg.LAYOUT_TILED
    sizes = {}
    for b in (4, 8, 16):
        d.batch = b
        sizes[b] = pwg._step_ws(C.byref(d))
    assert 0 < sizes[4] < sizes[8] < sizes[16]
    d.batch = 16
    d.workspace_bytes = sizes[16] - 1
    assert pwg._step(C.byref(d), None) == ERR_SIZE
    assert pwg._step_plan(C.byref(d), None) == ERR_SIZE
    d.workspace_bytes = sizes[16]
    for bad in (2, 3, 5, 32, -1):
        d.batch = bad
        assert pwg._step_ws(C.byref(d)) == 0
        assert pwg._step(C.byref(d), None) == ERR_ARG and "batch" in pwg.last_error()
    d.batch = 8
    d.schedule, d.weight_layout = pwg.SCHEDULE_LEVELS, pwg.LAYOUT_ROWS
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED
    d.schedule, d.weight_layout = pwg.SCHEDULE_STREAM, pwg.LAYOUT_TILED
    lv[1].cols = 1024                                  # not a multiple of 2048
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED and "2048" in pwg.last_error()
    lv[1].cols = 12288
    d.hidden = 1536                                    # not a multiple of 1024
    assert pwg._step(C.byref(d), None) == ERR_UNSUPPORTED and "1024" in pwg.last_error()
    d.hidden = 4096
    d.h = MIS
    assert pwg._step(C.byref(d), None) == ERR_ALIGN


def distinct_desc(batch=0):
    """A stream-schedule description whose buffers are all distinct (16 MiB
    apart, 16-byte aligned): it passes validation, and the launch then stops
    at the missing plan."""
    P = lambda k: (1 << 36) + k * (1 << 24)  # noqa: E731
    d = pwg._StepDesc()
    d.vocab, d.hidden, d.batch = 1000, 4096, batch
    for i, name in enumerate(("out_table", "out_scale", "h", "emb_table", "emb_scale", "token_in", "token_out",
                              "emb_row_out", "emb_scale_out", "workspace")):
        setattr(d, name, P(i))
    lv = (pwg.Level * 2)(pwg.Level(P(20), P(21), P(22), P(23), 64, 4096), pwg.Level(P(24), P(25), P(26), P(27), 64, 4096))
    d.n_levels, d.levels = 2, C.cast(lv, C.POINTER(pwg.Level))
    d.schedule, d.weight_layout = pwg.SCHEDULE_STREAM, pwg.LAYOUT_TILED
    d.workspace_bytes = pwg._step_ws(C.byref(d))
    assert d.workspace_bytes > 0
    return d, lv, P


@pytest.mark.parametrize("batch", [0, 4])
def test_unordered_schedules_reject_aliased_inputs(batch):
    """The stream schedule and the batched pass run levels in no fixed order,
    so an input (a level's x, or h) that shares memory with anything the step
    writes (a level's y, the logits, the embedding outputs) would be read
    before or after the write at random: PWG_ERR_UNSUPPORTED, for equal and
    for partly overlapping ranges, with the ranges scaled by the batch."""
    d, lv, P = distinct_desc(batch)
    assert pwg._step(C.byref(d), None) == ERR_ARG and "plan" in pwg.last_error()
    nb = max(batch, 1)

    def refused(what):
        rc = pwg._step(C.byref(d), None)
        assert rc == ERR_UNSUPPORTED and "overlaps" in pwg.last_error(), (what, rc, pwg.last_error())

    lv[1].x = lv[0].y                                   # level 1 reads level 0's output
    refused("x1 = y0")
    lv[1].x = P(23) + 64 * 4 * nb - 16                  # starts in y0's last 16 bytes
    refused("x1 inside y0")
    lv[1].x = P(23) + 64 * 4 * nb                       # right after y0: no overlap
    assert pwg._step(C.byref(d), None) == ERR_ARG
    lv[1].x = P(26)
    lv[0].x = lv[0].y                                   # a level reading its own output
    refused("x0 = y0")
    lv[0].x = P(22)
    d.h = lv[1].y                                       # h is a level output
    refused("h = y1")
    d.h = P(2)
    d.logits_out = P(30)
    lv[0].x = P(30) + 400                               # inside the logits
    refused("x0 in logits")
    lv[0].x = P(22)
    d.emb_deq_out = P(31)
    d.h = P(31)                                         # h is the dequantised embedding row
    refused("h = emb_deq_out")
    d.h = P(2)
    lv[0].x = d.emb_row_out                             # x0 is the gathered int8 row
    refused("x0 = emb_row_out")
    lv[0].x = P(22)
    assert pwg._step(C.byref(d), None) == ERR_ARG and "plan" in pwg.last_error()


def test_levels_schedule_takes_chained_pointers():
    """The levels schedule runs levels in decoder order: a level may read the
    previous level's output (validation passes; on this host the launch then
    fails only for want of a device)."""
    d, lv, P = distinct_desc()
    d.schedule, d.weight_layout = pwg.SCHEDULE_LEVELS, pwg.LAYOUT_ROWS
    d.workspace_bytes = pwg._step_ws(C.byref(d))
    lv[1].x = lv[0].y
    rc = pwg._step(C.byref(d), None)
    assert rc not in (ERR_UNSUPPORTED, ERR_ARG, ERR_ALIGN, ERR_SIZE), (rc, pwg.last_error())


def test_stream_launch_needs_a_plan_for_this_description():
    """The stream kernels take every pointer and shape from the device plan
    that pwg_step_plan writes into the workspace: a launch on a workspace that
    holds no plan is refused before anything is enqueued (a launch after a
    changed description is covered on the GPU, where a plan can be made)."""
    for batch in (0, 8):
        d, lv, P = distinct_desc(batch)
        rc = pwg._step(C.byref(d), None)
        assert rc == ERR_ARG and "no plan" in pwg.last_error()


def test_tiled_size():
    assert pwg.tiled_size(16, 64) == 1024
    assert pwg.tiled_size(17, 64) == 2048            # rows padded to 16
    assert pwg.tiled_size(4096, 1024) == 4096 * 1024
    assert pwg.tiled_size(151936, 4096) == 151936 * 4096
    for bad in ((0, 64), (16, 0), (16, 32), (16, 100), (-1, 64)):
        assert pwg.tiled_size(*bad) == 0
    assert pwg.tiled_size(33, 3072) == 48 * 3072


def test_tile_rows_argument_errors():
    f = pwg._tile_rows
    need = pwg.tiled_size(17, 128)
    assert f(None, 17, 128, A, need, None) == ERR_ARG
    assert f(A, 17, 128, None, need, None) == ERR_ARG
    assert f(A, 0, 128, A + (1 << 16), need, None) == ERR_ARG
    assert f(A, 17, 96, A + (1 << 16), need, None) == ERR_ARG
    assert f(MIS, 17, 128, A + (1 << 16), need, None) == ERR_ALIGN
    assert f(A, 17, 128, A + (1 << 16), need - 16, None) == ERR_SIZE
    assert f(A, 17, 128, A + 1024, need, None) == ERR_ARG and "overlap" in pwg.last_error()


def test_chained_input_errors():
    """Level inputs formed from earlier outputs (pwg_input): unknown ops,
    missing sources, overlapping buffers (among the input's and with the
    level's own output), bad head grouping, a negative eps,
    over-long inputs and the schedules that cannot order levels are refused
    before anything is enqueued (every call here fails validation)."""
    P = [A + 256 * k for k in range(8)]
    d = pwg._StepDesc()
    d.vocab, d.hidden = 1000, 4096
    for name in ("out_table", "out_scale", "h", "emb_table", "emb_scale", "token_in", "token_out",
                 "emb_row_out", "emb_scale_out", "workspace"):
        setattr(d, name, A)
    d.schedule, d.weight_layout = pwg.SCHEDULE_LEVELS, pwg.LAYOUT_ROWS
    d.workspace_bytes = 1 << 30
    lv = (pwg.Level * 1)(pwg.Level(P[0], P[1], P[2], P[3], 64, 4096))
    d.n_levels, d.levels = 1, C.cast(lv, C.POINTER(pwg.Level))

    def check(inp, code, text, level=True):
        if level:
            lv[0].input = inp
        else:
            d.h_in = inp
        try:
            assert pwg._step(C.byref(d), None) == code
            assert text in pwg.last_error()
            assert pwg._step_plan(C.byref(d), None) == code
        finally:
            lv[0].input = pwg._Input()
            d.h_in = pwg._Input()

    I = pwg._Input
    check(I(9), ERR_ARG, "unknown input op")
    check(I(-1), ERR_ARG, "unknown input op", level=False)
    check(I(pwg.INPUT_RMSNORM, 0, 0, 1e-6, None, P[4], None, None), ERR_ARG, "gamma")
    check(I(pwg.INPUT_RMSNORM, 0, 0, 1e-6, None, None, P[5], None), ERR_ARG, "resid")
    check(I(pwg.INPUT_RMSNORM, 0, 0, -1.0, None, P[4], P[5], None), ERR_ARG, "eps")
    check(I(pwg.INPUT_RMSNORM, 0, 0, float("nan"), None, P[4], P[5], None), ERR_ARG, "eps")
    check(I(pwg.INPUT_RMSNORM, 0, 0, 1e-6, None, P[4], P[5], P[2]), ERR_ARG, "overlap")   # resid_out == x
    check(I(pwg.INPUT_EMBED_RMSNORM, 0, 0, 1e-6, None, None, P[5], P[5]), ERR_ARG, "overlap")
    check(I(pwg.INPUT_SWIGLU, 0, 0, 0.0, None, None, None, None), ERR_ARG, "src")
    check(I(pwg.INPUT_ATTN1, 0, 4, 0.0, P[6], None, None, None), ERR_ARG, "heads")
    check(I(pwg.INPUT_ATTN1, 128, 3, 0.0, P[6], None, None, None), ERR_ARG, "heads")    # 384 does not divide 4096
    check(I(pwg.INPUT_ATTN1, 128, 4, 0.0, P[2], None, None, None), ERR_ARG, "overlap")  # src == x
    # the level's own output lies apart from everything its input reads or writes
    Y = A + (2 << 20)
    lv[0] = pwg.Level(P[0], P[1], A + (1 << 20), Y, 64, 4096)
    check(I(pwg.INPUT_SWIGLU, 0, 0, 0.0, Y - 4 * 4096, None, None, None), ERR_ARG, "y overlaps its input's src")
    check(I(pwg.INPUT_RMSNORM, 0, 0, 1e-6, None, P[4], P[5], Y + 128), ERR_ARG, "y overlaps its input's resid_out")
    check(I(pwg.INPUT_ATTN1, 128, 4, 0.0, Y - 4 * 1024 + 16, None, None, None), ERR_ARG, "y overlaps its input's src")
    # ordered schedules only, batch 1 only
    d.schedule, d.weight_layout = pwg.SCHEDULE_STREAM, pwg.LAYOUT_TILED
    d.workspace_bytes = 1 << 40
    check(I(pwg.INPUT_SWIGLU, 0, 0, 0.0, P[6], None, None, None), ERR_UNSUPPORTED, "ordered schedule")
    check(I(pwg.INPUT_RMSNORM, 0, 0, 1e-6, None, P[4], P[5], None), ERR_UNSUPPORTED, "ordered schedule", level=False)
    d.schedule, d.weight_layout = pwg.SCHEDULE_LEVELS, pwg.LAYOUT_ROWS
    lv[0] = pwg.Level(P[0], P[1], P[2], P[3], 64, 16384)
    check(I(pwg.INPUT_SWIGLU, 0, 0, 0.0, P[6], None, None, None), ERR_UNSUPPORTED, "at most 12288")


def test_attention_errors():
    """Unsupported head sizes and groups, empty caches, bad scales, null or
    misaligned pointers and short workspaces are refused before anything is
    enqueued (every call here fails validation)."""
    P = [A + 256 * k for k in range(5)]
    assert pwg.attention_workspace_bytes(32, 8, 128, 4096) > 0
    assert pwg.attention_workspace_bytes(32, 8, 96, 4096) == 0
    assert pwg.attention_workspace_bytes(64, 8, 128, 4096) == 0   # group 8
    assert pwg.attention_workspace_bytes(32, 8, 128, 0) == 0
    ws = pwg.attention_workspace_bytes(32, 8, 128, 100)

    def call(*, k=P[0], v=P[1], q=P[2], heads=32, kv=8, hd=128, ctx=100, scale=0.1, out=P[3], w=P[4], wb=ws):
        return pwg._attn(k, v, q, heads, kv, hd, ctx, scale, out, w, wb, None)

    assert call(hd=96) == ERR_UNSUPPORTED
    assert call(heads=64) == ERR_UNSUPPORTED
    assert call(heads=30) == ERR_ARG
    assert call(ctx=0) == ERR_ARG
    assert call(scale=float("inf")) == ERR_ARG
    assert call(k=None) == ERR_ARG
    assert call(q=MIS) == ERR_ALIGN
    assert call(wb=ws - 1) == ERR_SIZE


def test_verify_accept_errors():
    """Draft counts outside [0, 15] and null or misaligned pointers are
    refused before anything is enqueued."""
    P = [A + 256 * k for k in range(4)]
    assert pwg._verify(P[0], P[1], 16, P[2], P[3], None) == ERR_ARG
    assert pwg._verify(P[0], P[1], -1, P[2], P[3], None) == ERR_ARG
    assert pwg._verify(None, P[1], 3, P[2], P[3], None) == ERR_ARG
    assert pwg._verify(P[0], MIS, 3, P[2], P[3], None) == ERR_ALIGN


# ---------------------------------------------------------------- base-3 format
def test_b3_sizes():
    from oracle import base3_format as b3
    assert pwg.b3_packed_size(4096, 4096) == 4096 * 820
    assert pwg.b3_packed_size(1, 1) == 1 and pwg.b3_packed_size(2, 12288) == 2 * 2458
    for bad in ((0, 5), (1, 0), (-1, 5), (1, 16385)):
        assert pwg.b3_packed_size(*bad) == 0
        assert pwg.b3_tiled_size(*bad) == 0
    for rows, cols in ((1, 1), (16, 240), (17, 60), (4096, 4096), (4096, 12288), (33, 1001)):
        assert pwg.b3_tiled_size(rows, cols) == b3.tiled_nbytes(rows, cols)


@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (37, 1001), (5, 4100), (2048, 4096), (3, 12288)])
def test_b3_pack_matches_oracle_encoder_bit_for_bit(shape):
    from oracle import base3_format as b3
    rng = np.random.default_rng(shape[0] * 11 + shape[1])
    w = rng.integers(-1, 2, size=shape, dtype=np.int8)
    blob = pwg.pack_weights_b3(w)
    assert blob.size == b3.packed_nbytes(*shape)
    assert np.array_equal(blob, b3.encode(w))
    assert np.array_equal(pwg.unpack_weights_b3(blob, *shape), w)


def test_b3_pack_hand_fixture(golden_dir):
    import json
    for case in json.load(open(os.path.join(golden_dir, "b3_bytes.json")))["cases"]:
        w = np.array(case["weights"], np.int8)
        assert pwg.pack_weights_b3(w).tobytes() == bytes.fromhex(case["bytes_hex"]), case["derivation"]


def test_b3_pack_and_unpack_errors():
    w = np.zeros((4, 11), np.int8)
    w[2, 7] = 2
    with pytest.raises(pwg.PwgError) as e:
        pwg.pack_weights_b3(w)
    assert e.value.code == ERR_VALUE and "row 2" in str(e.value) and "col 7" in str(e.value)
    out = np.zeros(16, np.uint8)
    n = C.c_size_t(0)
    ok = np.zeros((2, 11), np.int8)
    assert pwg._pack_b3(None, 2, 11, out.ctypes.data, 16, C.byref(n)) == ERR_ARG
    assert pwg._pack_b3(ok.ctypes.data, 2, 0, out.ctypes.data, 16, C.byref(n)) == ERR_ARG
    assert pwg._pack_b3(ok.ctypes.data, 2, 11, out.ctypes.data, 5, C.byref(n)) == ERR_SIZE
    assert pwg._pack_b3(ok.ctypes.data, 2, 11, out.ctypes.data, 6, C.byref(n)) == 0 and n.value == 6
    blob = pwg.pack_weights_b3(np.zeros((3, 12), np.int8))
    blob[7] = 243
    with pytest.raises(pwg.PwgError) as e:
        pwg.unpack_weights_b3(blob, 3, 12)
    assert e.value.code == ERR_VALUE and "row 2" in str(e.value) and "byte 1" in str(e.value)


def test_b3_tile_and_gemv_argument_errors():
    t = pwg._tile_b3
    need = pwg.b3_tiled_size(17, 60)
    assert t(None, 17, 60, A, need, None) == ERR_ARG
    assert t(A, 0, 60, A + (1 << 16), need, None) == ERR_ARG
    assert t(A, 17, 16385, A + (1 << 16), need, None) == ERR_ARG
    assert t(A + 3, 17, 60, MIS + (1 << 16), need, None) == ERR_ALIGN   # dst alignment; src needs none
    assert t(A, 17, 60, A + (1 << 16), need - 1, None) == ERR_SIZE
    assert t(A, 17, 60, A + 16, need, None) == ERR_ARG and "overlap" in pwg.last_error()
    g = pwg._tgemv_b3
    assert g(None, A, 8, 60, A, 1, A, None) == ERR_ARG
    assert g(A, A, 0, 60, A, 1, A, None) == ERR_ARG
    assert g(A, A, 8, 0, A, 1, A, None) == ERR_ARG
    assert g(A, A, 8, 16385, A, 1, A, None) == ERR_ARG
    assert g(A, A, 8, 60, A, 3, A, None) == ERR_ARG and "batch" in pwg.last_error()
    assert g(A, A, 8, 60, MIS, 1, A, None) == ERR_ALIGN
    assert g(A, A, 8, 60, A, 1, None, None) == ERR_ARG


# ---------------------------------------------------------------- packed-blob header
def test_blob_header_matches_the_oracle_and_verifies_every_layout():
    from oracle import base3_format as b3
    from oracle import blob_header as bh
    rng = np.random.default_rng(17)
    w = rng.integers(-1, 2, size=(37, 512)).astype(np.int8)
    payloads = {pwg.BLOB_T2: pf.encode(w), pwg.BLOB_T2_TILED: pf.tile16x64(pf.encode(w).reshape(37, 128)),
                pwg.BLOB_B3: b3.encode(w), pwg.BLOB_B3_TILED: b3.tile(b3.encode(w), 37, 512)}
    for layout, p in payloads.items():
        head = pwg.blob_header(layout, w)
        assert head == bh.make(layout, w)                      # byte for byte, every field
        assert pwg.blob_payload_bytes(layout, 37, 512) == p.size
        pwg.blob_verify(head, p)
        bad = p.copy()
        bad[p.size // 2] ^= 0x01                               # one code changed
        with pytest.raises(pwg.PwgError) as e:
            pwg.blob_verify(head, bad)
        assert e.value.code == ERR_VALUE
        with pytest.raises(pwg.PwgError) as e:
            pwg.blob_verify(head, p[:-1], check_only=True)
        assert e.value.code == ERR_SIZE
    # the header names the matrix, not the packing: every layout carries one checksum
    assert len({bh.parse(pwg.blob_header(l, w))["logical_fnv1a"] for l in payloads}) == 1


def test_blob_header_rejects_malformed_headers():
    w = np.zeros((2, 64), np.int8)
    head = bytearray(pwg.blob_header(pwg.BLOB_T2, w))
    p = np.zeros(32, np.uint8)
    for off, what in ((0, "magic"), (4, "version"), (20, "cols"), (40, "checksum"), (50, "reserved")):
        h = bytearray(head)
        h[off] ^= 0x10
        with pytest.raises(pwg.PwgError) as e:
            pwg.blob_verify(bytes(h), p, check_only=True)
        assert e.value.code == ERR_VALUE, what
    with pytest.raises(pwg.PwgError) as e:
        pwg.blob_header(pwg.BLOB_T2, np.zeros((2, 60), np.int8))   # T2 needs cols % 64 == 0
    assert e.value.code == ERR_ARG
    with pytest.raises(pwg.PwgError) as e:
        pwg.blob_header(pwg.BLOB_B3, np.full((1, 3), 2, np.int8))
    assert e.value.code == ERR_VALUE
    assert pwg.blob_payload_bytes(9, 1, 64) == 0 and pwg.blob_payload_bytes(pwg.BLOB_T2_TILED, 1, 64) == 0
