"""ctypes binding for libbbd_gemv.so: argument marshalling only.

Every step of the GEMV runs in the library's HIP kernels. This module turns torch tensors
into device pointers, leading dimensions and a stream handle, calls the C ABI declared in
include/gemv.h and raises GemvError on any status other than GEMV_OK. There is no fallback:
if the library is missing, importing the package fails.
"""
from __future__ import annotations

import ctypes
import enum
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libbbd_gemv.so")

MAX_M = 16
MAX_SEGMENTS = 4


class Status(enum.IntEnum):
    OK = 0
    INVALID_ARG = 1
    MISALIGNED = 2
    WORKSPACE = 3
    DEVICE = 4
    CAPTURE = 5
    TIMEOUT = 6


class GemvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = Status(status) if status in Status._value2member_map_ else status
        hip = _lib.gemv_last_hip_error() if status in (Status.DEVICE, Status.CAPTURE) else 0
        self.hip_error = hip
        msg = _lib.gemv_status_string(int(status)).decode()
        super().__init__(f"{where}: {msg} (status {int(status)}, hipError {hip})")


class PlanOpts(ctypes.Structure):
    _fields_ = [("splits", ctypes.c_int), ("rows_per_wave", ctypes.c_int),
                ("waves_per_block", ctypes.c_int), ("unroll", ctypes.c_int),
                ("waves_per_cu", ctypes.c_int), ("mfma", ctypes.c_int),
                ("weights", ctypes.c_int), ("prologue", ctypes.c_int),
                ("int4_fp16", ctypes.c_int)]


class DeviceDesc(ctypes.Structure):
    _fields_ = [("compute_units", ctypes.c_int), ("hbm_bytes_per_s", ctypes.c_double),
                ("latency_s", ctypes.c_double)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("splits", ctypes.c_int), ("rows_per_wave", ctypes.c_int),
                ("waves_per_block", ctypes.c_int), ("unroll", ctypes.c_int),
                ("grid_x", ctypes.c_int), ("grid_y", ctypes.c_int),
                ("block_threads", ctypes.c_int), ("slice", ctypes.c_int64),
                ("depth_bound", ctypes.c_int), ("bytes_in_flight_per_cu", ctypes.c_double),
                ("bytes_in_flight_needed", ctypes.c_double), ("waves_per_cu", ctypes.c_int),
                ("lds_bytes", ctypes.c_int), ("mfma", ctypes.c_int),
                ("mfma_splits", ctypes.c_int), ("mfma_slice", ctypes.c_int64),
                ("mfma_grid_x", ctypes.c_int), ("mfma_depth_bound", ctypes.c_int),
                ("weights", ctypes.c_int), ("prologue", ctypes.c_int),
                ("int4_fp16", ctypes.c_int), ("mfma_rows", ctypes.c_int),
                ("mfma_unaligned_depth", ctypes.c_int)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class Segment(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("n", ctypes.c_int64), ("ldw", ctypes.c_int64),
                ("Y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


class ChainLink(ctypes.Structure):
    _fields_ = [("segs", ctypes.POINTER(Segment)), ("nseg", ctypes.c_int),
                ("X", ctypes.c_void_p), ("k", ctypes.c_int64)]


class ChainOpts(ctypes.Structure):
    _fields_ = [("waves_per_cu", ctypes.c_int), ("spin_limit", ctypes.c_uint)]


# Exported symbols and their C signatures (kept in the order of include/gemv.h).
_I64, _P, _INT, _SZ = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "gemv_bytes_in_flight": (ctypes.c_double, [ctypes.c_double, ctypes.c_double]),
    "gemv_plan": (_INT, [ctypes.POINTER(_P), _I64, _I64, _INT, _INT, ctypes.POINTER(PlanOpts)]),
    "gemv_plan_for": (_INT, [ctypes.POINTER(_P), _I64, _I64, _INT, ctypes.POINTER(DeviceDesc),
                             ctypes.POINTER(PlanOpts)]),
    "gemv_workspace_size": (_SZ, [_P]),
    "gemv_plan_query": (_INT, [_P, ctypes.POINTER(PlanInfo)]),
    "gemv_plan_destroy": (None, [_P]),
    "gemv_run": (_INT, [_P, _P, _I64, _P, _I64, _P, _I64, _P, _SZ, _P]),
    "gemv_run_static": (_INT, [_P, _P, _I64, _P, _I64, _P, _I64, _P]),
    "gemv_fused_run": (_INT, [_P, ctypes.POINTER(Segment), _INT, _P, _I64, _P, _SZ, _P]),
    "gemv_int4_run": (_INT, [_P, _P, _I64, _P, _I64, _P, _P, _P]),
    "gemv_rmsnorm_run": (_INT, [_P, ctypes.POINTER(Segment), _INT, _P, _P, ctypes.c_float, _P]),
    "gemv_graph_begin": (_INT, [_P]),
    "gemv_graph_end": (_INT, [_P, ctypes.POINTER(_P)]),
    "gemv_graph_launch": (_INT, [_P, _P]),
    "gemv_graph_destroy": (None, [_P]),
    "gemv_chain_create": (_INT, [ctypes.POINTER(_P), ctypes.POINTER(ChainLink), _INT, _INT,
                                 ctypes.POINTER(ChainOpts)]),
    "gemv_chain_run": (_INT, [_P, _P]),
    "gemv_chain_check": (_INT, [_P]),
    "gemv_chain_destroy": (None, [_P]),
    "gemv_read_stream": (_INT, [_P, _I64, _I64, _INT, _INT, _P, _P]),
    "gemv_status_string": (ctypes.c_char_p, [_INT]),
    "gemv_last_hip_error": (_INT, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python bandwidth_bound_decode_amd/build.py` "
                          "(the GEMV has no fallback path)")
    so = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(so, name)
        fn.restype = res
        fn.argtypes = args
    return so


_lib = _load()


def lib():
    return _lib


def _check(status: int, where: str):
    if status != Status.OK:
        raise GemvError(status, where)


def bytes_in_flight(bytes_per_s: float, latency_s: float) -> float:
    return float(_lib.gemv_bytes_in_flight(bytes_per_s, latency_s))


WEIGHTS = {"bf16": 0, "int4": 1}
PROLOGUES = {None: 0, "rmsnorm": 1}


def _opts(splits, rows_per_wave, waves_per_block, unroll, waves_per_cu=0, mfma=0,
          weights="bf16", prologue=None, int4_fp16=0):
    return PlanOpts(int(splits), int(rows_per_wave), int(waves_per_block), int(unroll),
                    int(waves_per_cu), int(mfma), WEIGHTS[weights], PROLOGUES[prologue],
                    int(int4_fp16))


class Plan:
    """An immutable launch plan for Y[M][N] = X[M][K] . W[N][K]^T.

    With `desc` (compute_units, hbm_bytes_per_s, latency_s) the plan is made on the host
    only, without touching a GPU; otherwise for the given CUDA/HIP device (default: current).
    """

    def __init__(self, n: int, k: int, m: int = 1, device=None, *, splits: int = 0,
                 rows_per_wave: int = 0, waves_per_block: int = 0, unroll: int = 0,
                 waves_per_cu: int = 0, mfma: int = 0, weights: str = "bf16",
                 prologue: str | None = None, int4_fp16: int = 0,
                 desc: tuple | None = None):
        self._h = ctypes.c_void_p()
        opts = _opts(splits, rows_per_wave, waves_per_block, unroll, waves_per_cu, mfma,
                     weights, prologue, int4_fp16)
        if desc is not None:
            d = DeviceDesc(int(desc[0]), float(desc[1]), float(desc[2]))
            st = _lib.gemv_plan_for(ctypes.byref(self._h), n, k, m, ctypes.byref(d),
                                    ctypes.byref(opts))
        else:
            if device is None:
                device = torch.cuda.current_device()
            idx = torch.device(device).index if not isinstance(device, int) else device
            st = _lib.gemv_plan(ctypes.byref(self._h), n, k, m, int(idx or 0),
                                ctypes.byref(opts))
        _check(st, "gemv_plan")
        self.n, self.k, self.m = int(n), int(k), int(m)

    @property
    def handle(self):
        return self._h

    @property
    def workspace_size(self) -> int:
        return int(_lib.gemv_workspace_size(self._h))

    @property
    def info(self) -> dict:
        out = PlanInfo()
        _check(_lib.gemv_plan_query(self._h, ctypes.byref(out)), "gemv_plan_query")
        return out.as_dict()

    def alloc_workspace(self, device=None) -> torch.Tensor | None:
        """A zero-filled device buffer big enough for this plan (None if it needs none)."""
        size = self.workspace_size
        if size == 0:
            return None
        return torch.zeros(size, dtype=torch.uint8, device=device or "cuda")

    def close(self):
        if self._h:
            _lib.gemv_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _row_stride(t: torch.Tensor, what: str) -> int:
    """Row stride in elements of a 1-D (one row) or 2-D tensor whose rows are contiguous.
    A strided view (buf[::2], M[:, j]) would be read by the kernels as if it were dense,
    so it is refused."""
    if t.dim() not in (1, 2):
        raise ValueError(f"{what} must be 1-D or 2-D")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{what} rows must be contiguous (stride {t.stride(-1)} along the row)")
    if t.dim() == 1:
        return t.shape[0]
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _vector(t: torch.Tensor, what: str):
    """A single-row operand handed over as one pointer: [k] or [1, k], contiguous."""
    if t.dim() == 2 and t.shape[0] != 1:
        raise ValueError(f"{what} must be [k] or [1, k], got {tuple(t.shape)}")
    _row_stride(t, what)


def _on_gpu(what: str, *tensors: torch.Tensor):
    """Every tensor argument is handed to the kernels as a device pointer: refuse host
    tensors (and tensors on different devices) before anything is launched."""
    dev = None
    for t in tensors:
        if not t.is_cuda:
            raise ValueError(f"{what}: every tensor must be on the GPU (got {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{what}: tensors on different devices ({dev}, {t.device})")


def _need(t: torch.Tensor, rows: int, cols: int, what: str):
    """t must hold at least `rows` rows of at least `cols` elements ([cols] when rows == 1)."""
    r, c = (1, t.shape[0]) if t.dim() == 1 else (t.shape[0], t.shape[1])
    if r < rows or c < cols:
        raise ValueError(f"{what} is {tuple(t.shape)}, the plan needs [{rows}, {cols}]")


def _ws(workspace):
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def run(plan: Plan, W: torch.Tensor, X: torch.Tensor, Y: torch.Tensor,
        workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X . W^T on the GPU (Y overwritten). W bf16 [n, >=k], X bf16 [m, k] or [k],
    Y fp32 [m, n] or [n]. Returns Y."""
    if W.dtype != torch.bfloat16 or X.dtype != torch.bfloat16 or Y.dtype != torch.float32:
        raise TypeError("W and X must be bfloat16 and Y float32")
    _on_gpu("gemv_run", W, X, Y, *([workspace] if workspace is not None else []))
    if W.dim() != 2 or W.shape[0] != plan.n:
        raise ValueError(f"W is {tuple(W.shape)}, the plan has {plan.n} rows")
    _need(W, plan.n, plan.k, "W")
    _need(X, plan.m, plan.k, "X")
    _need(Y, plan.m, plan.n, "Y")
    ws_ptr, ws_bytes = _ws(workspace)
    st = _lib.gemv_run(plan.handle, W.data_ptr(), _row_stride(W, "W"), X.data_ptr(),
                       _row_stride(X, "X"), Y.data_ptr(), _row_stride(Y, "Y"), ws_ptr,
                       ws_bytes, _stream_handle(stream))
    _check(st, "gemv_run")
    return Y


def run_static(plan: Plan, W: torch.Tensor, X: torch.Tensor, Y: torch.Tensor,
               stream=None) -> torch.Tensor:
    """run() without a workspace: split partial sums go to the library's static per-GPU
    scratch (gemv_run_static). Calls that overlap on one GPU race. Returns Y."""
    if W.dtype != torch.bfloat16 or X.dtype != torch.bfloat16 or Y.dtype != torch.float32:
        raise TypeError("W and X must be bfloat16 and Y float32")
    _on_gpu("gemv_run_static", W, X, Y)
    if W.dim() != 2 or W.shape[0] != plan.n:
        raise ValueError(f"W is {tuple(W.shape)}, the plan has {plan.n} rows")
    _need(W, plan.n, plan.k, "W")
    _need(X, plan.m, plan.k, "X")
    _need(Y, plan.m, plan.n, "Y")
    st = _lib.gemv_run_static(plan.handle, W.data_ptr(), _row_stride(W, "W"), X.data_ptr(),
                              _row_stride(X, "X"), Y.data_ptr(), _row_stride(Y, "Y"),
                              _stream_handle(stream))
    _check(st, "gemv_run_static")
    return Y


def run_int4(plan: Plan, Wq: torch.Tensor, S: torch.Tensor, X: torch.Tensor, Y: torch.Tensor,
             stream=None) -> torch.Tensor:
    """Y = X . W^T for INT4 weights (plan made with weights="int4"): Wq uint8 [n, ldq]
    packed nibbles, S bf16 [n, lds] group scales, X bf16 [k] or [1, k], Y fp32 [n] or
    [1, n]. Returns Y."""
    if Wq.dtype != torch.uint8 or S.dtype != torch.bfloat16 or X.dtype != torch.bfloat16 or \
            Y.dtype != torch.float32:
        raise TypeError("Wq must be uint8, S and X bfloat16, Y float32")
    _on_gpu("gemv_int4_run", Wq, S, X, Y)
    _need(Wq, plan.n, (plan.k + 1) // 2, "Wq")
    _need(S, plan.n, (plan.k + 127) // 128, "S")
    _need(X, 1, plan.k, "X")
    _need(Y, 1, plan.n, "Y")
    _vector(X, "X")
    _vector(Y, "Y")
    st = _lib.gemv_int4_run(plan.handle, Wq.data_ptr(), _row_stride(Wq, "Wq"), S.data_ptr(),
                            _row_stride(S, "S"), X.data_ptr(), Y.data_ptr(),
                            _stream_handle(stream))
    _check(st, "gemv_int4_run")
    return Y


def rmsnorm_run(plan: Plan, segments, H: torch.Tensor, gamma: torch.Tensor, eps: float,
                stream=None):
    """Y_i = rms_inv * W_i . (gamma * H) for every (W_i, Y_i) in `segments`, with
    rms_inv = 1/sqrt(mean(H^2) + eps), in one launch (plan made with prologue="rmsnorm").
    H and gamma bf16 [k] (or [1, k]); W_i bf16 [n_i, >= k] sharing one row stride; Y_i fp32
    [n_i] (or [1, n_i])."""
    segs = list(segments)
    arr = (Segment * max(len(segs), 1))()
    for i, (w, y) in enumerate(segs):
        if w.dtype != torch.bfloat16 or y.dtype != torch.float32:
            raise TypeError("segment W must be bfloat16 and Y float32")
        _vector(y, "segment Y")
        arr[i] = Segment(w.data_ptr(), w.shape[0], _row_stride(w, "W"), y.data_ptr(),
                         w.shape[0])
    _vector(H, "H")
    _vector(gamma, "gamma")
    if H.dtype != torch.bfloat16 or gamma.dtype != torch.bfloat16:
        raise TypeError("H and gamma must be bfloat16")
    _on_gpu("gemv_rmsnorm_run", H, gamma, *[t for pair in segs for t in pair])
    _need(H, 1, plan.k, "H")
    _need(gamma, 1, plan.k, "gamma")
    for w, y in segs:
        _need(w, w.shape[0], plan.k, "segment W")
        _need(y, 1, w.shape[0], "segment Y")
    st = _lib.gemv_rmsnorm_run(plan.handle, arr, len(segs), H.data_ptr(), gamma.data_ptr(),
                               float(eps), _stream_handle(stream))
    _check(st, "gemv_rmsnorm_run")


def fused_run(plan: Plan, segments, X: torch.Tensor, workspace: torch.Tensor | None = None,
              stream=None):
    """One launch over several (W_i, Y_i) pairs that share X (fused QKV / gate_up)."""
    segs = list(segments)
    arr = (Segment * max(len(segs), 1))()
    for i, (w, y) in enumerate(segs):
        if w.dtype != torch.bfloat16 or y.dtype != torch.float32:
            raise TypeError("segment W must be bfloat16 and Y float32")
        arr[i] = Segment(w.data_ptr(), w.shape[0], _row_stride(w, "W"), y.data_ptr(),
                         _row_stride(y, "Y"))
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    _on_gpu("gemv_fused_run", X, *[t for pair in segs for t in pair],
            *([workspace] if workspace is not None else []))
    _need(X, plan.m, plan.k, "X")
    for w, y in segs:
        _need(w, w.shape[0], plan.k, "segment W")
        _need(y, plan.m, w.shape[0], "segment Y")
    ws_ptr, ws_bytes = _ws(workspace)
    st = _lib.gemv_fused_run(plan.handle, arr, len(segs), X.data_ptr(), _row_stride(X, "X"),
                             ws_ptr, ws_bytes, _stream_handle(stream))
    _check(st, "gemv_fused_run")


def read_stream(buf: torch.Tensor, rows: int, row_bytes: int, unroll: int, waves_per_cu: int,
                sink: torch.Tensor, stream=None):
    """The pure-read streaming kernel (gemv_read_stream): `rows` rows of `row_bytes` bytes
    from the device buffer `buf`, for measuring the read ceiling and bytes in flight."""
    _on_gpu("gemv_read_stream", buf, sink)
    if buf.numel() * buf.element_size() < rows * row_bytes or sink.numel() * sink.element_size() < 4:
        raise ValueError("buffer smaller than rows * row_bytes, or sink under 4 bytes")
    _check(_lib.gemv_read_stream(buf.data_ptr(), rows, row_bytes, unroll, waves_per_cu,
                                 sink.data_ptr(), _stream_handle(stream)), "gemv_read_stream")


class Graph:
    """Capture gemv_run / gemv_fused_run calls issued on `stream` into one replayable graph.

        with Graph(stream) as g:      # begin capture
            run(...); fused_run(...)  # recorded, not executed
        g.launch()                    # replay
    """

    def __init__(self, stream):
        self.stream = stream
        self._h = ctypes.c_void_p()

    def begin(self):
        _check(_lib.gemv_graph_begin(_stream_handle(self.stream)), "gemv_graph_begin")

    def end(self):
        _check(_lib.gemv_graph_end(_stream_handle(self.stream), ctypes.byref(self._h)),
               "gemv_graph_end")

    def __enter__(self):
        self.begin()
        return self

    def __exit__(self, exc_type, exc, tb):
        if exc_type is None:
            self.end()
        else:
            try:
                self.end()
            finally:
                self.destroy()

    def launch(self, stream=None):
        _check(_lib.gemv_graph_launch(self._h, _stream_handle(stream or self.stream)),
               "gemv_graph_launch")

    def destroy(self):
        if self._h:
            _lib.gemv_graph_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


class Chain:
    """Dependent batch-1 GEMVs run by one persistent launch (gemv_chain_* in gemv.h).

    `links` is a list of (segments, X) with segments a list of (W, Y) pairs sharing X: link i
    computes every Y_j = W_j . X, after link i-1 has completed. The tensors must outlive the
    chain.
    """

    def __init__(self, links, device=None, *, waves_per_cu: int = 0, spin_limit: int = 0):
        self._h = ctypes.c_void_p()
        self._keep = []
        arr = (ChainLink * len(links))()
        for i, (segments, x) in enumerate(links):
            segs = (Segment * len(segments))()
            for j, (w, y) in enumerate(segments):
                if w.dtype != torch.bfloat16 or y.dtype != torch.float32:
                    raise TypeError("chain weights must be bfloat16 and outputs float32")
                _vector(y, "chain Y")
                segs[j] = Segment(w.data_ptr(), w.shape[0], _row_stride(w, "W"), y.data_ptr(),
                                  w.shape[0])
            if x.dtype != torch.bfloat16:
                raise TypeError("chain inputs must be bfloat16")
            _vector(x, "chain X")
            _on_gpu("gemv_chain_create", x, *[t for pair in segments for t in pair])
            for w, y in segments:
                _need(w, w.shape[0], x.shape[-1], "chain W")
                _need(y, 1, w.shape[0], "chain Y")
            self._keep.append(segs)
            arr[i] = ChainLink(segs, len(segments), x.data_ptr(), x.shape[-1])
        if device is None:
            device = torch.cuda.current_device()
        idx = torch.device(device).index if not isinstance(device, int) else device
        opts = ChainOpts(int(waves_per_cu), int(spin_limit))
        _check(_lib.gemv_chain_create(ctypes.byref(self._h), arr, len(links), int(idx or 0),
                                      ctypes.byref(opts)), "gemv_chain_create")
        self._keep = None
        self.nlinks = len(links)

    def run(self, stream=None):
        _check(_lib.gemv_chain_run(self._h, _stream_handle(stream)), "gemv_chain_run")

    def check(self):
        """Synchronise; raise GemvError(TIMEOUT) if a dependency wait of a run gave up."""
        _check(_lib.gemv_chain_check(self._h), "gemv_chain_check")

    def destroy(self):
        if self._h:
            _lib.gemv_chain_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
