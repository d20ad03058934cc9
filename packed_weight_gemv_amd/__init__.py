"""Python binding of libpwg (packed ternary weight-streaming decode on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libpwg.so.  PyTorch supplies device memory and streams.  The names
match the C ABI in include/pwg.h without the ``pwg_`` prefix.

The library must be built first (``python packed_weight_gemv_amd/build.py``
or ``__graft_entry__.build()``); importing this package raises if it is
missing, and there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "PwgError", "lib", "packed_size", "pack_weights", "unpack_weights", "ternary_gemv",
    "argmax_workspace_bytes", "int8_gemv_argmax", "int8_gemv_argmax_noalloc", "embed_gather", "Level", "StepDesc",
    "step_workspace_bytes", "step_plan", "decode_step_weights", "step_status", "last_error", "version",
    "tiled_size", "tile_rows", "SCHEDULE_LEVELS", "SCHEDULE_PERSISTENT", "SCHEDULE_STREAM",
    "LAYOUT_ROWS", "LAYOUT_TILED", "layout_for_schedule", "LIB_PATH", "InputOp", "INPUT_GIVEN",
    "INPUT_RMSNORM", "INPUT_EMBED_RMSNORM", "INPUT_ATTN1", "INPUT_SWIGLU", "attention_workspace_bytes",
    "gqa_decode_attention", "verify_accept",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpwg.so")

PWG_OK = 0
ERR_NAMES = {-1: "PWG_ERR_ARG", -2: "PWG_ERR_ALIGN", -3: "PWG_ERR_SIZE", -4: "PWG_ERR_VALUE",
             -5: "PWG_ERR_HIP", -6: "PWG_ERR_UNSUPPORTED"}
SCHEDULE_LEVELS = 0
SCHEDULE_PERSISTENT = 1
SCHEDULE_STREAM = 2
LAYOUT_ROWS = 0
LAYOUT_TILED = 1
# how a level's input is formed in a chained step (pwg.h, pwg_input)
INPUT_GIVEN, INPUT_RMSNORM, INPUT_EMBED_RMSNORM, INPUT_ATTN1, INPUT_SWIGLU = 0, 1, 2, 3, 4


def layout_for_schedule(schedule: int) -> int:
    """Weight arrangement a schedule takes (the stream schedule runs on tiles)."""
    return LAYOUT_ROWS if schedule == SCHEDULE_LEVELS else LAYOUT_TILED


class PwgError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERR_NAMES.get(code, code)}: {message}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libpwg.so is not built ({LIB_PATH}); run `python packed_weight_gemv_amd/build.py`")

# PyTorch ships its own HIP runtime (same soname as the system one).  Loading
# torch first makes libpwg bind to that runtime instead of pulling in a
# second copy, so tensors, streams and kernels share one runtime.
try:
    import torch  # noqa: F401
except ImportError:  # host-only use (packer, argument checks)
    pass

lib = C.CDLL(LIB_PATH)

_i64, _i32, _sz, _vp = C.c_int64, C.c_int32, C.c_size_t, C.c_void_p


class _Input(C.Structure):
    _fields_ = [("op", _i32), ("head_dim", _i32), ("group", _i32), ("eps", C.c_float),
                ("src", _vp), ("resid", _vp), ("gamma", _vp), ("resid_out", _vp)]


class Level(C.Structure):
    _fields_ = [("w_packed", _vp), ("row_scale", _vp), ("x", _vp), ("y", _vp), ("rows", _i64), ("cols", _i64),
                ("input", _Input)]


class _StepDesc(C.Structure):
    _fields_ = [
        ("n_levels", _i32), ("schedule", _i32), ("weight_layout", _i32), ("batch", _i32),
        ("levels", C.POINTER(Level)),
        ("out_table", _vp), ("out_scale", _vp), ("h", _vp), ("vocab", _i64), ("hidden", _i64),
        ("emb_table", _vp), ("emb_scale", _vp), ("token_in", _vp), ("token_out", _vp),
        ("emb_row_out", _vp), ("emb_scale_out", _vp), ("emb_deq_out", _vp), ("logits_out", _vp),
        ("workspace", _vp), ("workspace_bytes", _sz), ("h_in", _Input),
    ]


class BlobHeader(C.Structure):
    _fields_ = [("magic", C.c_uint32), ("version", C.c_uint16), ("layout", C.c_uint16), ("rows", _i64),
                ("cols", _i64), ("payload_bytes", C.c_uint64), ("logical_fnv1a", C.c_uint64),
                ("header_fnv1a", C.c_uint64), ("reserved", C.c_uint64 * 2)]


def _sig(name, restype, *argtypes):
    f = getattr(lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_packed_size = _sig("pwg_packed_size", _sz, _i64, _i64)
_pack = _sig("pwg_pack_weights", C.c_int, _vp, _i64, _i64, _vp, _sz, C.POINTER(_sz))
_unpack = _sig("pwg_unpack_weights", C.c_int, _vp, _i64, _i64, _vp)
_attn_ws = _sig("pwg_attention_workspace_bytes", _sz, _i32, _i32, _i32, _i64)
_attn = _sig("pwg_gqa_decode_attention", C.c_int, _vp, _vp, _vp, _i32, _i32, _i32, _i64, C.c_float, _vp, _vp, _sz,
             _vp)
_verify = _sig("pwg_verify_accept", C.c_int, _vp, _vp, _i32, _vp, _vp, _vp)
_tgemv = _sig("pwg_ternary_gemv", C.c_int, _vp, _vp, _i64, _i64, _vp, _i32, _vp, _vp)
_argmax_ws = _sig("pwg_argmax_workspace_bytes", _sz, _i64, _i32)
_i8argmax = _sig("pwg_int8_gemv_argmax", C.c_int, _vp, _vp, _i64, _i64, _vp, _i32, _vp, _sz, _vp, _vp, _vp)
_i8argmax_na = _sig("pwg_int8_gemv_argmax_noalloc", C.c_int, _vp, _vp, _i64, _i64, _vp, _i32, _vp, _vp, _vp)
_gather = _sig("pwg_embed_gather", C.c_int, _vp, _vp, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _vp)
_batch_ws = _sig("pwg_batch_workspace_bytes", _sz, _i64, _i32)
_tgemv_tiled = _sig("pwg_ternary_gemv_tiled", C.c_int, _vp, _vp, _i64, _i64, _vp, _i32, _vp, _vp, _sz, _vp)
_i8argmax_tiled = _sig("pwg_int8_gemv_argmax_tiled", C.c_int, _vp, _vp, _i64, _i64, _vp, _i32, _vp, _sz, _vp, _vp, _vp)
_tiled_size = _sig("pwg_tiled_size", _sz, _i64, _i64)
_tile_rows = _sig("pwg_tile_rows", C.c_int, _vp, _i64, _i64, _vp, _sz, _vp)
_b3_packed_size = _sig("pwg_b3_packed_size", _sz, _i64, _i64)
_pack_b3 = _sig("pwg_pack_weights_b3", C.c_int, _vp, _i64, _i64, _vp, _sz, C.POINTER(_sz))
_unpack_b3 = _sig("pwg_unpack_weights_b3", C.c_int, _vp, _i64, _i64, _vp)
_b3_tiled_size = _sig("pwg_b3_tiled_size", _sz, _i64, _i64)
_tile_b3 = _sig("pwg_tile_b3", C.c_int, _vp, _i64, _i64, _vp, _sz, _vp)
_tgemv_b3 = _sig("pwg_ternary_gemv_b3", C.c_int, _vp, _vp, _i64, _i64, _vp, _i32, _vp, _vp)
_blob_payload = _sig("pwg_blob_payload_bytes", _sz, _i32, _i64, _i64)
_blob_init = _sig("pwg_blob_header_init", C.c_int, _i32, _vp, _i64, _i64, C.POINTER(BlobHeader))
_blob_check = _sig("pwg_blob_header_check", C.c_int, C.POINTER(BlobHeader), _sz)
_blob_verify = _sig("pwg_blob_verify", C.c_int, C.POINTER(BlobHeader), _vp, _sz)
_step_ws = _sig("pwg_step_workspace_bytes", _sz, C.POINTER(_StepDesc))
_step_plan = _sig("pwg_step_plan", C.c_int, C.POINTER(_StepDesc), _vp)
_step = _sig("pwg_decode_step_weights", C.c_int, C.POINTER(_StepDesc), _vp)
_step_status = _sig("pwg_step_status", C.c_int, C.POINTER(_StepDesc), _vp)
_step_trace_bytes = _sig("pwg_step_trace_bytes", _sz, C.POINTER(_StepDesc))
_step_set_trace = _sig("pwg_step_set_trace", C.c_int, C.POINTER(_StepDesc), _vp, _sz, _vp)
_last_error = _sig("pwg_last_error", C.c_char_p)
_version = _sig("pwg_version", C.c_int)

EXPORTED = ["pwg_packed_size", "pwg_pack_weights", "pwg_unpack_weights", "pwg_ternary_gemv",
            "pwg_argmax_workspace_bytes", "pwg_int8_gemv_argmax", "pwg_embed_gather",
            "pwg_tiled_size", "pwg_tile_rows", "pwg_batch_workspace_bytes", "pwg_ternary_gemv_tiled",
            "pwg_int8_gemv_argmax_tiled",
            "pwg_step_workspace_bytes", "pwg_step_plan", "pwg_decode_step_weights",
            "pwg_step_status", "pwg_last_error", "pwg_version", "pwg_attention_workspace_bytes",
            "pwg_gqa_decode_attention", "pwg_verify_accept", "pwg_int8_gemv_argmax_noalloc",
            "pwg_b3_packed_size", "pwg_pack_weights_b3", "pwg_unpack_weights_b3", "pwg_b3_tiled_size",
            "pwg_tile_b3", "pwg_ternary_gemv_b3", "pwg_blob_payload_bytes", "pwg_blob_header_init",
            "pwg_blob_header_check", "pwg_blob_verify", "pwg_step_trace_bytes", "pwg_step_set_trace"]


def last_error() -> str:
    return _last_error().decode()


def version() -> int:
    return _version()


def _check(rc: int):
    if rc != PWG_OK:
        raise PwgError(rc, last_error())


def _ptr(t) -> int | None:
    """Device or host address of a torch tensor (None stays None)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- host packer
def packed_size(rows: int, cols: int) -> int:
    return _packed_size(rows, cols)


def pack_weights(w: np.ndarray) -> np.ndarray:
    """Pack an int8 (rows, cols) ternary matrix into a uint8 T2 blob (host)."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    if w.ndim != 2:
        raise ValueError("w must be 2-D")
    rows, cols = w.shape
    n = _packed_size(rows, cols)
    out = np.empty(max(n, 1), dtype=np.uint8)
    written = _sz(0)
    _check(_pack(w.ctypes.data, rows, cols, out.ctypes.data, out.nbytes if n else 0, C.byref(written)))
    return out[:written.value]


def unpack_weights(blob: np.ndarray, rows: int, cols: int) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.int8)
    if blob.size < _packed_size(rows, cols):
        raise ValueError("blob too small")
    _check(_unpack(blob.ctypes.data, rows, cols, out.ctypes.data))
    return out


def b3_packed_size(rows: int, cols: int) -> int:
    return _b3_packed_size(rows, cols)


def pack_weights_b3(w: np.ndarray) -> np.ndarray:
    """Pack an int8 (rows, cols) ternary matrix into a uint8 base-3 blob
    (five weights per byte; host)."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    if w.ndim != 2:
        raise ValueError("w must be 2-D")
    rows, cols = w.shape
    n = _b3_packed_size(rows, cols)
    out = np.empty(max(n, 1), dtype=np.uint8)
    written = _sz(0)
    _check(_pack_b3(w.ctypes.data, rows, cols, out.ctypes.data, out.nbytes if n else 0, C.byref(written)))
    return out[:written.value]


def unpack_weights_b3(blob: np.ndarray, rows: int, cols: int) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.int8)
    if blob.size < _b3_packed_size(rows, cols):
        raise ValueError("blob too small")
    _check(_unpack_b3(blob.ctypes.data, rows, cols, out.ctypes.data))
    return out


# ---------------------------------------------------------------- packed-blob header
BLOB_T2, BLOB_T2_TILED, BLOB_B3, BLOB_B3_TILED = 1, 2, 3, 4


def blob_payload_bytes(layout: int, rows: int, cols: int) -> int:
    return _blob_payload(layout, rows, cols)


def blob_header(layout: int, w: np.ndarray) -> bytes:
    """The 64-byte header of the logical matrix w (int8) in `layout`."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    h = BlobHeader()
    _check(_blob_init(layout, w.ctypes.data, w.shape[0], w.shape[1], C.byref(h)))
    return bytes(h)


def blob_verify(header: bytes, payload: np.ndarray, check_only: bool = False):
    """Checks a header (and, unless check_only, the payload's logical values
    against it); raises PwgError."""
    h = BlobHeader.from_buffer_copy(header)
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    if check_only:
        _check(_blob_check(C.byref(h), payload.nbytes))
    else:
        _check(_blob_verify(C.byref(h), payload.ctypes.data, payload.nbytes))


# ---------------------------------------------------------------- GPU entry points
def ternary_gemv(w_packed, row_scale, rows: int, cols: int, x, y=None, stream=None):
    """y = row_scale * (W @ x) for x of shape (cols,) or (batch, cols)."""
    import torch
    batch = 1 if x.dim() == 1 else x.shape[0]
    if y is None:
        y = torch.empty((rows,) if x.dim() == 1 else (batch, rows), dtype=torch.float32, device=x.device)
    _check(_tgemv(_ptr(w_packed), _ptr(row_scale), rows, cols, _ptr(x), batch, _ptr(y), _stream(stream)))
    return y


def argmax_workspace_bytes(rows: int, batch: int = 1) -> int:
    return _argmax_ws(rows, batch)


def int8_gemv_argmax(table, row_scale, h, workspace=None, token_out=None, logits_out=None, stream=None):
    """Greedy token(s) of logits = row_scale * (table @ h); h is (cols,) or (batch, cols)."""
    import torch
    rows, cols = table.shape
    batch = 1 if h.dim() == 1 else h.shape[0]
    if workspace is None:
        workspace = torch.empty(max(1, _argmax_ws(rows, batch)), dtype=torch.uint8, device=h.device)
    if token_out is None:
        token_out = torch.empty(batch, dtype=torch.int32, device=h.device)
    _check(_i8argmax(_ptr(table), _ptr(row_scale), rows, cols, _ptr(h), batch, _ptr(workspace),
                     workspace.numel() * workspace.element_size(), _ptr(token_out), _ptr(logits_out),
                     _stream(stream)))
    return token_out


def int8_gemv_argmax_noalloc(table, row_scale, h, token_out=None, logits_out=None, stream=None):
    """int8_gemv_argmax with the library's fixed scratch array instead of a
    workspace (nothing is allocated by the call; token_out must be given to
    keep the binding allocation-free too)."""
    import torch
    rows, cols = table.shape
    batch = 1 if h.dim() == 1 else h.shape[0]
    if token_out is None:
        token_out = torch.empty(batch, dtype=torch.int32, device=h.device)
    _check(_i8argmax_na(_ptr(table), _ptr(row_scale), rows, cols, _ptr(h), batch, _ptr(token_out), _ptr(logits_out),
                        _stream(stream)))
    return token_out


def embed_gather(table, row_scale, ids, rows_out=None, scales_out=None, deq_out=None, dequant=True, stream=None):
    """Rows table[ids], their scales and (optionally) float32 dequantised rows."""
    import torch
    rows, cols = table.shape
    n = ids.numel()
    dev = ids.device
    if rows_out is None:
        rows_out = torch.empty((n, cols), dtype=torch.int8, device=dev)
    if scales_out is None:
        scales_out = torch.empty(max(n, 1), dtype=torch.float32, device=dev)
    if dequant and deq_out is None:
        deq_out = torch.empty((n, cols), dtype=torch.float32, device=dev)
    _check(_gather(_ptr(table), _ptr(row_scale), rows, cols, _ptr(ids), n, _ptr(rows_out), _ptr(scales_out),
                   _ptr(deq_out) if dequant else None, _stream(stream)))
    return rows_out, scales_out[:n], (deq_out if dequant else None)


# ---------------------------------------------------------------- decode attention
def attention_workspace_bytes(n_heads: int, n_kv: int, head_dim: int, ctx: int) -> int:
    return _attn_ws(n_heads, n_kv, head_dim, ctx)


def gqa_decode_attention(k_cache, v_cache, q, n_heads: int, n_kv: int, head_dim: int, scale: float, out=None,
                         workspace=None, stream=None):
    """One layer's grouped-query decode attention; k_cache, v_cache: int16 or
    uint16 tensors of bfloat16 bits [ctx, n_kv, head_dim] on the device."""
    import torch
    ctx = k_cache.shape[0]
    if out is None:
        out = torch.empty(n_heads * head_dim, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(16, attention_workspace_bytes(n_heads, n_kv, head_dim, ctx)), dtype=torch.uint8,
                                device=q.device)
    _check(_attn(_ptr(k_cache), _ptr(v_cache), _ptr(q), n_heads, n_kv, head_dim, ctx, scale, _ptr(out),
                 _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


# ---------------------------------------------------------------- verify pass
def verify_accept(tokens_in, targets, n_drafts: int, accepted=None, next_token=None, stream=None):
    """Accepted-draft count and next token after a batched verify pass
    (device int32 tensors); returns (accepted, next_token) device tensors."""
    import torch
    dev = tokens_in.device
    if accepted is None:
        accepted = torch.empty(4, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(4, dtype=torch.int32, device=dev)
    _check(_verify(_ptr(tokens_in), _ptr(targets), n_drafts, _ptr(accepted), _ptr(next_token), _stream(stream)))
    return accepted, next_token


# ---------------------------------------------------------------- tiled arrangement
def batch_workspace_bytes(cols: int, batch: int) -> int:
    return _batch_ws(cols, batch)


def ternary_gemv_tiled(w_tiled, row_scale, rows: int, cols: int, x, y=None, workspace=None, stream=None):
    """y = row_scale * (W @ x.T).T for x of shape (batch, cols), batch 1, 4, 8
    or 16 (x of shape (cols,) for one vector), W in the tiled arrangement
    (tile_rows of the T2 blob)."""
    import torch
    batch = 1 if x.dim() == 1 else x.shape[0]
    if x.dim() == 1 and y is None:
        y = torch.empty(rows, dtype=torch.float32, device=x.device)
    if y is None:
        y = torch.empty((batch, rows), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(1, _batch_ws(cols, batch)), dtype=torch.uint8, device=x.device)
    _check(_tgemv_tiled(_ptr(w_tiled), _ptr(row_scale), rows, cols, _ptr(x), batch, _ptr(y), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


def int8_gemv_argmax_tiled(table_tiled, row_scale, rows: int, cols: int, h, workspace=None, token_out=None,
                           logits_out=None, stream=None):
    """Greedy tokens of logits = row_scale * (Q @ h.T) for h (batch, cols),
    batch 4, 8 or 16, Q in the tiled arrangement (tile_rows of the table)."""
    import torch
    batch = h.shape[0]
    if workspace is None:
        workspace = torch.empty(max(1, _argmax_ws(rows, batch)), dtype=torch.uint8, device=h.device)
    if token_out is None:
        token_out = torch.empty(batch, dtype=torch.int32, device=h.device)
    _check(_i8argmax_tiled(_ptr(table_tiled), _ptr(row_scale), rows, cols, _ptr(h), batch, _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _ptr(token_out), _ptr(logits_out),
                           _stream(stream)))
    return token_out


def tiled_size(rows: int, row_bytes: int) -> int:
    return _tiled_size(rows, row_bytes)


def tile_rows(src, rows: int, row_bytes: int, dst=None, stream=None):
    """16-row x 64-byte tile arrangement of a row-major device byte matrix
    (a T2 blob: row_bytes = cols // 4; an int8 table: row_bytes = cols)."""
    import torch
    need = _tiled_size(rows, row_bytes)
    if dst is None:
        dst = torch.empty(max(need, 16), dtype=torch.uint8, device=src.device)
    _check(_tile_rows(_ptr(src), rows, row_bytes, _ptr(dst), dst.numel() * dst.element_size(), _stream(stream)))
    return dst


def b3_tiled_size(rows: int, cols: int) -> int:
    return _b3_tiled_size(rows, cols)


def tile_b3(src, rows: int, cols: int, dst=None, stream=None):
    """Device arrangement of a base-3 blob on the device (768-byte windows of
    30-weight groups)."""
    import torch
    need = _b3_tiled_size(rows, cols)
    if dst is None:
        dst = torch.empty(max(need, 16), dtype=torch.uint8, device=src.device)
    _check(_tile_b3(_ptr(src), rows, cols, _ptr(dst), dst.numel() * dst.element_size(), _stream(stream)))
    return dst


def ternary_gemv_b3(w_b3_tiled, row_scale, rows: int, cols: int, x, y=None, stream=None):
    """y = row_scale * (W @ x) on base-3 weights as tile_b3 arranges them; x
    of shape (cols,) or (batch, cols)."""
    import torch
    batch = 1 if x.dim() == 1 else x.shape[0]
    if y is None:
        y = torch.empty((rows,) if x.dim() == 1 else (batch, rows), dtype=torch.float32, device=x.device)
    _check(_tgemv_b3(_ptr(w_b3_tiled), _ptr(row_scale), rows, cols, _ptr(x), batch, _ptr(y), _stream(stream)))
    return y


# ---------------------------------------------------------------- decode step
@dataclass
class InputOp:
    """How a level's input (or h) is formed in a chained step; keeps its
    tensors alive.  op: INPUT_*; see pwg.h for each op's formula."""
    op: int
    src: object = None
    resid: object = None
    gamma: object = None
    resid_out: object = None
    eps: float = 1e-6
    head_dim: int = 0
    group: int = 0

    def c(self):
        return _Input(self.op, self.head_dim, self.group, self.eps, _ptr(self.src), _ptr(self.resid),
                      _ptr(self.gamma), _ptr(self.resid_out))


@dataclass
class StepDesc:
    """Python-side description of a decode step; keeps every tensor alive."""
    levels: list            # [(w_packed, row_scale, x, y, rows, cols[, InputOp])]
    out_table: object
    out_scale: object
    h: object
    emb_table: object
    emb_scale: object
    token_in: object
    token_out: object
    emb_row_out: object
    emb_scale_out: object
    emb_deq_out: object = None
    logits_out: object = None
    workspace: object = None
    schedule: int = SCHEDULE_LEVELS
    weight_layout: int = LAYOUT_ROWS
    vocab: int | None = None        # rows of the output table (when it is stored tiled)
    hidden: int | None = None
    batch: int = 1                  # 4, 8, 16: batched pass (stream schedule); buffers hold batch rows
    h_in: object = None             # InputOp forming h (chained step), or None: h as given
    _c: object = field(default=None, repr=False)
    _levels_c: object = field(default=None, repr=False)

    def c(self):
        if self._c is None:
            arr = (Level * max(1, len(self.levels)))()
            for i, lv in enumerate(self.levels):
                w, s, x, y, r, k = lv[:6]
                arr[i] = Level(_ptr(w), _ptr(s), _ptr(x), _ptr(y), r, k, lv[6].c() if len(lv) > 6 else _Input())
            self._levels_c = arr
            vocab = self.vocab if self.vocab is not None else self.out_table.shape[0]
            hidden = self.hidden if self.hidden is not None else self.out_table.shape[1]
            ws = self.workspace
            self._c = _StepDesc(
                len(self.levels), self.schedule, self.weight_layout, self.batch, C.cast(arr, C.POINTER(Level)),
                _ptr(self.out_table), _ptr(self.out_scale), _ptr(self.h), vocab, hidden,
                _ptr(self.emb_table), _ptr(self.emb_scale), _ptr(self.token_in), _ptr(self.token_out),
                _ptr(self.emb_row_out), _ptr(self.emb_scale_out), _ptr(self.emb_deq_out), _ptr(self.logits_out),
                _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                self.h_in.c() if self.h_in is not None else _Input())
        return self._c


def step_workspace_bytes(desc: StepDesc) -> int:
    return _step_ws(C.byref(desc.c()))


def step_plan(desc: StepDesc, stream=None):
    _check(_step_plan(C.byref(desc.c()), _stream(stream)))


def decode_step_weights(desc: StepDesc, stream=None):
    _check(_step(C.byref(desc.c()), _stream(stream)))


TRACE_EVENTS = 8
TRACE_EVENT_NAMES = ("wait", "passed", "sources", "start", "converted", "products", "arrived", "unused")


def step_trace_bytes(desc: StepDesc) -> int:
    return _step_trace_bytes(C.byref(desc.c()))


def step_set_trace(desc: StepDesc, trace=None, stream=None):
    """Records the persistent schedule's level trace into `trace` (a device
    uint8/int64 tensor of step_trace_bytes(desc) bytes) on later steps; None
    turns it off.  Synchronous; after step_plan."""
    ptr, nbytes = (None, 0) if trace is None else (trace.data_ptr(), trace.numel() * trace.element_size())
    _check(_step_set_trace(C.byref(desc.c()), ptr, nbytes, _stream(stream)))


def step_status(desc: StepDesc, stream=None):
    """Raises if a stream step or batched pass recorded a timeout of one of
    its bounded waits (synchronous)."""
    _check(_step_status(C.byref(desc.c()), _stream(stream)))
