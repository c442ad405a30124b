"""Python binding of libtpslice.so: argument marshalling only.

Every function here passes raw device pointers (`tensor.data_ptr()`) and HIP streams
(`torch.cuda.Stream.cuda_stream`) to the C ABI declared in include/tpslice.h; all arithmetic runs in
the library's HIP kernels. PyTorch provides device memory and streams: the worker and copy streams a
plan runs on are torch streams, by default from a per-device set this module creates once and keeps
for the life of the process (the library creates and destroys no stream). Importing this module
fails loudly if the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpslice.so")

OK, ERR_INVALID, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(6)
STATIC_SCRATCH_BYTES = 64 << 20  # TPSLICE_STATIC_SCRATCH_BYTES
ACT_GELU, ACT_SWIGLU = 1, 2
F_SERIALIZE, F_COPY_BLIT, F_PIPELINE, F_HANDOFF_ROWS, F_CALLER_WORKER = 0x1, 0x2, 0x4, 0x8, 0x40
F_TILE_SHIFT = 8
# block tile ids (flags bits 8..11); "large" / "small" name the 256 x 256 / 128 x 128 tiles
TILES = {"auto": 0, "256x256": 1, "128x128": 2, "256x320": 3, "128x320": 4, "128x256": 5,
         "128x128w8": 6, "256x256w4": 7, "256x160w4": 8, "256x320w4": 9, "256x224w4": 10, "large": 1,
         "small": 2}
OP_MLP_FWD, OP_ATTNPROJ_FWD, OP_MLP_BWD, OP_ATTNPROJ_BWD, OP_ATTN_CORE_BWD = range(5)
EXPORTS = ("tpslice_plan", "tpslice_plan_destroy", "tpslice_plan_info", "tpslice_plan_piece",
           "tpslice_workspace_size", "tpslice_mlp_fwd", "tpslice_attnproj_fwd", "tpslice_mlp_bwd",
           "tpslice_attnproj_bwd", "tpslice_trace_enable", "tpslice_trace_read",
           "tpslice_handoff_copy", "tpslice_handoff_wait", "tpslice_attn_core_fwd", "tpslice_attn_core_bwd",
           "tpslice_mlp_fwd_static", "tpslice_strand_schedule",
           "tpslice_error_string", "tpslice_last_error")
TRACE_GEMM, TRACE_COPY, TRACE_COLSUM, TRACE_SPLIT_SUM = range(4)
STEPS = ("mlp_up", "mlp_down", "qkv", "out", "mlp_dh", "mlp_dx", "mlp_dw1", "mlp_dw2", "attn_dx", "attn_dc",
         "attn_dwqkv", "attn_dwo", "bias_grad", "handoff")


class TpsliceError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"tpslice error {code}: {msg}")
        self.code = code


class Desc(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64), ("ffn", ctypes.c_int64),
                ("tp_size", ctypes.c_int32), ("n_row_slices", ctypes.c_int32),
                ("n_col_slices", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("act", ctypes.c_int32),
                ("n_streams", ctypes.c_int32), ("n_copy_streams", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("handoff_gbps", ctypes.c_float), ("dh_group", ctypes.c_int32),
                ("up_group", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64), ("ffn_shard", ctypes.c_int64),
                ("n1", ctypes.c_int64), ("qkv_width", ctypes.c_int64), ("ctx_width", ctypes.c_int64),
                ("rows_per_slice", ctypes.c_int64), ("handoff_cols", ctypes.c_int64),
                ("n_row_slices", ctypes.c_int32), ("n_col_slices", ctypes.c_int32),
                ("n_streams", ctypes.c_int32), ("n_copy_streams", ctypes.c_int32),
                ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("k_splits", ctypes.c_int32 * 8),
                ("predicted_forward_us", ctypes.c_double), ("dh_group_slices", ctypes.c_int32),
                ("up_group_slices", ctypes.c_int32), ("k_split_rows", ctypes.c_int32 * 8)]

    SPLIT_NAMES = ("up", "qkv", "dh", "dw1", "dw2", "dc", "dwo", "dwqkv")

    def splits(self):
        return dict(zip(self.SPLIT_NAMES, list(self.k_splits)))

    def split_rows(self):
        return dict(zip(self.SPLIT_NAMES, list(self.k_split_rows)))


class TraceRec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("step", ctypes.c_int32), ("slice", ctypes.c_int32),
                ("piece", ctypes.c_int32), ("stream", ctypes.c_int32), ("call", ctypes.c_int32),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double), ("start_ms", ctypes.c_float),
                ("end_ms", ctypes.c_float), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("waves_m", ctypes.c_int32), ("waves_n", ctypes.c_int32), ("blocks_per_cu", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("epilogue", ctypes.c_int32), ("blocks", ctypes.c_int32),
                ("threads", ctypes.c_int32)]


class StreamsC(ctypes.Structure):
    _fields_ = [("caller", ctypes.c_void_p), ("workers", ctypes.POINTER(ctypes.c_void_p)),
                ("n_workers", ctypes.c_int32), ("copiers", ctypes.POINTER(ctypes.c_void_p)),
                ("n_copiers", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m comm_overlap_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int
    lib.tpslice_plan.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(vp)]
    lib.tpslice_plan_destroy.argtypes = [vp]
    lib.tpslice_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.tpslice_plan_piece.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_int64)]
    lib.tpslice_workspace_size.argtypes = [vp, i32, ctypes.POINTER(sz)]
    ss = ctypes.POINTER(StreamsC)
    lib.tpslice_mlp_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ss]
    lib.tpslice_attnproj_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ss]
    lib.tpslice_mlp_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, ss]
    lib.tpslice_attnproj_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, ss]
    lib.tpslice_trace_enable.argtypes = [vp, i32]
    lib.tpslice_trace_read.argtypes = [vp, ctypes.POINTER(TraceRec), i32, ctypes.POINTER(i32)]
    lib.tpslice_handoff_copy.argtypes = [vp, vp, vp, ss]
    lib.tpslice_handoff_wait.argtypes = [vp, vp]
    lib.tpslice_attn_core_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ss]
    lib.tpslice_attn_core_bwd.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp, sz, ss]
    lib.tpslice_mlp_fwd_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ss]
    lib.tpslice_strand_schedule.argtypes = [ctypes.POINTER(ctypes.c_double), i32, i32, ctypes.POINTER(i32),
                                            ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]
    for name in EXPORTS[:17]:
        getattr(lib, name).restype = st
    lib.tpslice_error_string.argtypes = [st]
    lib.tpslice_error_string.restype = ctypes.c_char_p
    lib.tpslice_last_error.argtypes = []
    lib.tpslice_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(code: int):
    if code != OK:
        raise TpsliceError(code, lib.tpslice_last_error().decode() or lib.tpslice_error_string(code).decode())


def _ptr(t: Optional[torch.Tensor], dtype=torch.bfloat16, name: str = "tensor"):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> Optional[ctypes.c_void_p]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Streams:
    """Worker and copy streams for a plan's calls (torch streams, default priority). The caller owns
    them; the library only queues work on them. A plan takes the first n_streams (or n_streams - 1
    when worker 0 is the caller's stream) workers and the first n_copy_streams copiers; the caller's
    stream must not be one of them."""

    def __init__(self, workers=(), copiers=()):
        self.workers = list(workers)
        self.copiers = list(copiers)

    @classmethod
    def new(cls, n_workers: int, n_copiers: int, device=None):
        return cls([torch.cuda.Stream(device=device) for _ in range(n_workers)],
                   [torch.cuda.Stream(device=device) for _ in range(n_copiers)])


# One set per device, created on first use and kept for the life of the process.
_POOL = {}


def default_streams(n_workers: int, n_copiers: int, caller=None, device=None) -> Streams:
    """The process-wide stream set of `device` (current by default), grown to at least the given
    counts of streams that differ from `caller`."""
    dev = torch.cuda.current_device() if device is None else torch.device(device).index
    pool = _POOL.setdefault(dev, Streams())
    skip = None if caller is None else caller.cuda_stream

    def pick(lst, n):
        out = [s for s in lst if s.cuda_stream != skip]
        while len(out) < n:
            s = torch.cuda.Stream(device=dev)
            lst.append(s)
            if s.cuda_stream != skip and all(s.cuda_stream != o.cuda_stream for o in out):
                out.append(s)
        return out[:max(n, 0)]

    w = pick(pool.workers, n_workers)
    used = {s.cuda_stream for s in w}
    c = [s for s in pick(pool.copiers, n_copiers + len(used)) if s.cuda_stream not in used][:n_copiers]
    return Streams(w, c)


# Plans dropped without close() are destroyed at the next plan's construction (or by collect()),
# not inside the garbage collector.
_DROPPED = []


def collect():
    """Destroy plans that were dropped without close() (blocks until their queued work is done)."""
    while _DROPPED:
        lib.tpslice_plan_destroy(_DROPPED.pop())


def _shape(t: Optional[torch.Tensor], shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


@dataclass
class Config:
    tokens: int
    hidden: int
    ffn: int
    tp_size: int = 1
    n_row_slices: int = 1       # 0: chosen by the plan (slice-count model)
    n_col_slices: int = 1       # 0: chosen by the plan
    n_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 0
    act: str = "gelu"
    n_streams: int = 0
    n_copy_streams: int = 0
    serialize: bool = False
    copy_blit: bool = False
    pipeline: bool = False
    caller_worker: bool = False  # worker stream 0 is the caller's stream
    handoff_rows: bool = False  # c > 1: one contiguous copy per row slice instead of per piece
    tile: str = "auto"  # a key of TILES
    handoff_gbps: float = 0.0  # hand-off rate the automatic slice counts assume (0: local DMA copy)
    dh_group: int = 0  # row slices per dH product of the MLP backward (0: automatic)
    up_group: int = 0  # row slices per up-projection of the MLP forward (0: automatic)

    def desc(self) -> Desc:
        return Desc(self.tokens, self.hidden, self.ffn, self.tp_size, self.n_row_slices, self.n_col_slices,
                    self.n_heads, self.n_kv_heads, self.head_dim,
                    {"gelu": ACT_GELU, "swiglu": ACT_SWIGLU}.get(self.act, 0), self.n_streams,
                    self.n_copy_streams,
                    (F_SERIALIZE if self.serialize else 0) | (F_COPY_BLIT if self.copy_blit else 0)
                    | (F_PIPELINE if self.pipeline else 0) | (F_CALLER_WORKER if self.caller_worker else 0)
                    | (F_HANDOFF_ROWS if self.handoff_rows else 0)
                    | (TILES[self.tile] << F_TILE_SHIFT), float(self.handoff_gbps), int(self.dh_group),
                    int(self.up_group))


class Plan:
    """A validated plan (host memory; streams and events are made on first use)."""

    def __init__(self, cfg: Config, streams: Optional[Streams] = None):
        collect()
        self.cfg = cfg
        self.streams = streams  # None: the process-wide set of the device in use at each call
        h = ctypes.c_void_p()
        d = cfg.desc()
        _check(lib.tpslice_plan(ctypes.byref(d), ctypes.byref(h)))
        self._h = h
        info = PlanInfo()
        _check(lib.tpslice_plan_info(self._h, ctypes.byref(info)))
        self.info = info
        self._ws = {}

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(lib.tpslice_plan_destroy(self._h))
            self._h = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _DROPPED is not None:  # (None while the interpreter shuts down)
            _DROPPED.append(h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _call_streams(self, stream=None, hand_off=True):
        """The C stream set of one call: `stream` (default: torch's current stream) as the caller,
        the plan's worker and copy streams after it."""
        caller = torch.cuda.current_stream() if stream is None else stream
        i = self.info
        serial = self.cfg.serialize
        n_w = 0 if serial else i.n_streams - (1 if (self.cfg.caller_worker or i.n_streams == 1) else 0)
        n_c = 0 if serial or not hand_off else i.n_copy_streams
        s = self.streams if self.streams is not None else default_streams(n_w, n_c, caller)
        w = (ctypes.c_void_p * max(1, len(s.workers)))(*[x.cuda_stream for x in s.workers])
        c = (ctypes.c_void_p * max(1, len(s.copiers)))(*[x.cuda_stream for x in s.copiers])
        self._keep = (w, c)  # alive until the next call; the library reads them during the call only
        return ctypes.byref(StreamsC(caller.cuda_stream, w, len(s.workers), c, len(s.copiers)))

    def trace(self, enable=True, products=True, copies=True):
        """Enable tracing (products and/or hand-off copies) or disable it (enable=False)."""
        mask = (int(products) | (int(copies) << 1)) if enable else 0
        _check(lib.tpslice_trace_enable(self._h, mask))

    def trace_read(self):
        """Records accumulated since the last read (then a new window starts): dicts with kind,
        step, slice, piece, stream, call, flops, bytes, start_ms, end_ms (ms from the first traced
        call's start on the caller stream), and for GEMM launches the kernel's identity (template
        parameters and grid, as a kernel profiler names the dispatch) and grid_x (work-items)."""
        n = ctypes.c_int32()
        _check(lib.tpslice_trace_read(self._h, None, 0, ctypes.byref(n)))
        recs = (TraceRec * max(1, n.value))()
        _check(lib.tpslice_trace_read(self._h, recs, n.value, ctypes.byref(n)))
        out = []
        for r in recs[:n.value]:
            kernel = None
            if r.kind == TRACE_GEMM:
                kernel = (f"gemm_kernel<Tile<{r.tile_m}, {r.tile_n}, {r.waves_m}, {r.waves_n}, {r.blocks_per_cu}>, "
                          f"{r.layout}, {r.epilogue}> grid {r.blocks} x {r.threads}")
            out.append(dict(kind=("gemm", "copy", "colsum", "split_sum")[r.kind], step=STEPS[r.step],
                            slice=r.slice, piece=r.piece, stream=r.stream, call=r.call, flops=r.flops,
                            bytes=r.bytes, start_ms=r.start_ms, end_ms=r.end_ms, kernel=kernel,
                            grid_x=r.blocks * r.threads))
        return out

    def handoff_copy(self, src, dst, stream=None):
        """Only the hand-off copies of a [tokens][hidden] bf16 tensor (no products)."""
        i = self.info
        _shape(src, (i.tokens, i.hidden), "src"); _shape(dst, (i.tokens, i.hidden), "dst")
        _check(lib.tpslice_handoff_copy(self._h, _ptr(src, name="src"), _ptr(dst, name="dst"),
                                        self._call_streams(stream)))

    def handoff_wait(self, stream=None):
        """Make `stream` (default: current) wait for every hand-off copy queued so far."""
        _check(lib.tpslice_handoff_wait(self._h, _stream(stream)))

    def piece(self, index: int):
        out = (ctypes.c_int64 * 4)()
        _check(lib.tpslice_plan_piece(self._h, index, out))
        return tuple(out)

    def workspace_size(self, op: int) -> int:
        n = ctypes.c_size_t()
        _check(lib.tpslice_workspace_size(self._h, op, ctypes.byref(n)))
        return n.value

    def workspace(self, op: int, device="cuda") -> Optional[torch.Tensor]:
        """A cached device workspace for `op` (torch allocations are 256-byte aligned)."""
        n = self.workspace_size(op)
        if n == 0:
            return None
        ws = self._ws.get(op)
        if ws is None or ws.numel() < n:
            ws = torch.empty(n, dtype=torch.uint8, device=device)
            self._ws[op] = ws
        return ws

    @staticmethod
    def _ws_args(ws: Optional[torch.Tensor]):
        if ws is None:
            return None, 0
        return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()

    # ------------------------------------------------------------------------------- entry points
    def mlp_fwd(self, X, W1, b1, W2, Z, U_save=None, Z_handoff=None, workspace=None, stream=None):
        i = self.info
        _shape(X, (i.tokens, i.hidden), "X"); _shape(W1, (i.n1, i.hidden), "W1")
        _shape(b1, (i.n1,), "b1"); _shape(W2, (i.hidden, i.ffn_shard), "W2")
        _shape(Z, (i.tokens, i.hidden), "Z"); _shape(U_save, (i.tokens, i.n1), "U_save")
        _shape(Z_handoff, (i.tokens, i.hidden), "Z_handoff")
        ws = workspace if workspace is not None else self.workspace(OP_MLP_FWD)
        wp, wn = self._ws_args(ws)
        _check(lib.tpslice_mlp_fwd(self._h, _ptr(X, name="X"), _ptr(W1, name="W1"), _ptr(b1, name="b1"),
                                   _ptr(W2, name="W2"), _ptr(Z, name="Z"), _ptr(U_save, name="U_save"),
                                   _ptr(Z_handoff, name="Z_handoff"), wp, wn,
                                   self._call_streams(stream, Z_handoff is not None)))

    def mlp_fwd_static(self, X, W1, b1, W2, Z, U_save=None, Z_handoff=None, stream=None):
        """mlp_fwd with the library's own fixed device scratch as workspace (no allocation)."""
        i = self.info
        _shape(X, (i.tokens, i.hidden), "X"); _shape(W1, (i.n1, i.hidden), "W1")
        _shape(b1, (i.n1,), "b1"); _shape(W2, (i.hidden, i.ffn_shard), "W2")
        _shape(Z, (i.tokens, i.hidden), "Z"); _shape(U_save, (i.tokens, i.n1), "U_save")
        _shape(Z_handoff, (i.tokens, i.hidden), "Z_handoff")
        _check(lib.tpslice_mlp_fwd_static(self._h, _ptr(X, name="X"), _ptr(W1, name="W1"), _ptr(b1, name="b1"),
                                          _ptr(W2, name="W2"), _ptr(Z, name="Z"), _ptr(U_save, name="U_save"),
                                          _ptr(Z_handoff, name="Z_handoff"),
                                          self._call_streams(stream, Z_handoff is not None)))

    def attnproj_fwd(self, X, Wqkv, bqkv, QKV, C, Wo, Z, Z_handoff=None, workspace=None, stream=None):
        i = self.info
        _shape(X, (i.tokens, i.hidden), "X"); _shape(Wqkv, (i.qkv_width, i.hidden), "Wqkv")
        _shape(bqkv, (i.qkv_width,), "bqkv"); _shape(QKV, (i.tokens, i.qkv_width), "QKV")
        _shape(C, (i.tokens, i.ctx_width), "C"); _shape(Wo, (i.hidden, i.ctx_width), "Wo")
        _shape(Z, (i.tokens, i.hidden), "Z"); _shape(Z_handoff, (i.tokens, i.hidden), "Z_handoff")
        ws = workspace if workspace is not None else self.workspace(OP_ATTNPROJ_FWD)
        wp, wn = self._ws_args(ws)
        _check(lib.tpslice_attnproj_fwd(self._h, _ptr(X, name="X"), _ptr(Wqkv, name="Wqkv"),
                                        _ptr(bqkv, name="bqkv"), _ptr(QKV, name="QKV"), _ptr(C, name="C"),
                                        _ptr(Wo, name="Wo"), _ptr(Z, name="Z"),
                                        _ptr(Z_handoff, name="Z_handoff"), wp, wn,
                                        self._call_streams(stream, Z_handoff is not None)))

    def mlp_bwd(self, X, W1, W2, U_saved, dY, dX, dW1, dW2, db1=None, dX_handoff=None, accumulate=False,
                workspace=None, stream=None):
        i = self.info
        _shape(X, (i.tokens, i.hidden), "X"); _shape(W1, (i.n1, i.hidden), "W1")
        _shape(W2, (i.hidden, i.ffn_shard), "W2"); _shape(U_saved, (i.tokens, i.n1), "U_saved")
        _shape(dY, (i.tokens, i.hidden), "dY"); _shape(dX, (i.tokens, i.hidden), "dX")
        _shape(dW1, (i.n1, i.hidden), "dW1"); _shape(dW2, (i.hidden, i.ffn_shard), "dW2")
        _shape(db1, (i.n1,), "db1"); _shape(dX_handoff, (i.tokens, i.hidden), "dX_handoff")
        ws = workspace if workspace is not None else self.workspace(OP_MLP_BWD)
        wp, wn = self._ws_args(ws)
        f32 = torch.float32
        _check(lib.tpslice_mlp_bwd(self._h, _ptr(X, name="X"), _ptr(W1, name="W1"), _ptr(W2, name="W2"),
                                   _ptr(U_saved, name="U_saved"), _ptr(dY, name="dY"), _ptr(dX, name="dX"),
                                   _ptr(dX_handoff, name="dX_handoff"), _ptr(dW1, f32, "dW1"),
                                   _ptr(db1, f32, "db1"), _ptr(dW2, f32, "dW2"), int(bool(accumulate)),
                                   wp, wn, self._call_streams(stream, dX_handoff is not None)))

    def attn_core_fwd(self, QKV, C, seq_len, lse=None, stream=None):
        """Causal attention of every sequence (seq_len consecutive token rows) and query head:
        QKV [tokens][(q + 2 kv) head_dim] -> C [tokens][q head_dim], bf16; lse [tokens][q] fp32 (each
        row's log-sum-exp, for the backward pass) when given."""
        i = self.info
        _shape(QKV, (i.tokens, i.qkv_width), "QKV")
        _shape(C, (i.tokens, i.ctx_width), "C")
        _shape(lse, (i.tokens, i.q_heads), "lse")
        _check(lib.tpslice_attn_core_fwd(self._h, _ptr(QKV, name="QKV"), _ptr(C, name="C"),
                                         _ptr(lse, torch.float32, "lse"), int(seq_len),
                                         self._call_streams(stream, False)))

    def attn_core_bwd(self, QKV, C, lse, dC, dQKV, seq_len, workspace=None, stream=None):
        """Gradient of the attention core: dQKV [tokens][(q + 2 kv) head_dim] bf16 from the forward's
        QKV, C and lse and the gradient dC of C."""
        i = self.info
        _shape(QKV, (i.tokens, i.qkv_width), "QKV"); _shape(C, (i.tokens, i.ctx_width), "C")
        _shape(lse, (i.tokens, i.q_heads), "lse"); _shape(dC, (i.tokens, i.ctx_width), "dC")
        _shape(dQKV, (i.tokens, i.qkv_width), "dQKV")
        ws = workspace if workspace is not None else self.workspace(OP_ATTN_CORE_BWD)
        wp, wn = self._ws_args(ws)
        _check(lib.tpslice_attn_core_bwd(self._h, _ptr(QKV, name="QKV"), _ptr(C, name="C"),
                                         _ptr(lse, torch.float32, "lse"), _ptr(dC, name="dC"),
                                         _ptr(dQKV, name="dQKV"), int(seq_len), wp, wn,
                                         self._call_streams(stream, False)))

    def attnproj_bwd(self, X, Wqkv, dQKV, C, Wo, dY, dX, dC, dWqkv, dWo, dbqkv=None, dX_handoff=None,
                     accumulate=False, workspace=None, stream=None):
        i = self.info
        _shape(X, (i.tokens, i.hidden), "X"); _shape(Wqkv, (i.qkv_width, i.hidden), "Wqkv")
        _shape(dQKV, (i.tokens, i.qkv_width), "dQKV"); _shape(C, (i.tokens, i.ctx_width), "C")
        _shape(Wo, (i.hidden, i.ctx_width), "Wo"); _shape(dY, (i.tokens, i.hidden), "dY")
        _shape(dX, (i.tokens, i.hidden), "dX"); _shape(dC, (i.tokens, i.ctx_width), "dC")
        _shape(dWqkv, (i.qkv_width, i.hidden), "dWqkv"); _shape(dWo, (i.hidden, i.ctx_width), "dWo")
        _shape(dbqkv, (i.qkv_width,), "dbqkv"); _shape(dX_handoff, (i.tokens, i.hidden), "dX_handoff")
        ws = workspace if workspace is not None else self.workspace(OP_ATTNPROJ_BWD)
        wp, wn = self._ws_args(ws)
        f32 = torch.float32
        _check(lib.tpslice_attnproj_bwd(self._h, _ptr(X, name="X"), _ptr(Wqkv, name="Wqkv"),
                                        _ptr(dQKV, name="dQKV"), _ptr(C, name="C"), _ptr(Wo, name="Wo"),
                                        _ptr(dY, name="dY"), _ptr(dX, name="dX"),
                                        _ptr(dX_handoff, name="dX_handoff"), _ptr(dC, name="dC"),
                                        _ptr(dWqkv, f32, "dWqkv"), _ptr(dbqkv, f32, "dbqkv"),
                                        _ptr(dWo, f32, "dWo"), int(bool(accumulate)), wp, wn,
                                        self._call_streams(stream, dX_handoff is not None)))


def plan_for(workload, streams: Optional[Streams] = None, **overrides) -> Plan:
    """A plan for a synthetic workload description (comm_overlap_amd.synth.Workload)."""
    kw = dict(tokens=workload.tokens, hidden=workload.hidden, ffn=workload.ffn, tp_size=workload.tp,
              n_row_slices=workload.row_slices, n_col_slices=workload.col_slices, n_heads=workload.heads,
              n_kv_heads=workload.kv_heads, head_dim=workload.head_dim, act=workload.act)
    kw.update(overrides)
    return Plan(Config(**kw), streams)


def strand_schedule(P):
    """The pairing of least total time of two strands' segments (tpslice_strand_schedule).
    P: (nf + 1) x (nb + 1) nested sequence of measured times as the C function takes them.
    Returns (steps, makespan): steps a list of (forward, backward) 1-based segment numbers, 0 for
    none, in execution order."""
    nf, nb = len(P) - 1, len(P[0]) - 1
    flat = (ctypes.c_double * ((nf + 1) * (nb + 1)))(*[float(v) for row in P for v in row])
    steps = (ctypes.c_int32 * max(2, 2 * (nf + nb)))()
    n = ctypes.c_int32()
    t = ctypes.c_double()
    _check(lib.tpslice_strand_schedule(flat, nf, nb, steps, ctypes.byref(n), ctypes.byref(t)))
    return [(steps[2 * k], steps[2 * k + 1]) for k in range(n.value)], t.value
