"""MI355X-native decode GEMV: y = W.x with bf16 (or INT4) W, bf16 x, fp32 accumulation.

The compute runs in hand-written gfx950 HIP kernels inside lib/libbbd_gemv.so (C ABI in
include/gemv.h); this package is the thin ctypes binding over it.
"""
from ._binding import (LIB_PATH, MAX_M, MAX_SEGMENTS, SIGNATURES, Chain, GemvError, Graph,
                       Plan, Status, bytes_in_flight, fused_run, lib, read_stream, rmsnorm_run,
                       run, run_int4, run_static)

__all__ = ["LIB_PATH", "MAX_M", "MAX_SEGMENTS", "SIGNATURES", "Chain", "GemvError", "Graph",
           "Plan", "Status", "bytes_in_flight", "fused_run", "lib", "read_stream",
           "rmsnorm_run", "run", "run_int4", "run_static"]
