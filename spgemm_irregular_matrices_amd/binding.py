"""Thin ctypes binding of the C ABI in ``include/spgemm.h``.

Argument marshalling only: every step of the product runs in the HIP
library. PyTorch supplies device buffers and the stream. There is no CPU
fallback: if the library is not built, or no GPU is visible, calls raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

from . import build as _build

LIB_PATH = _build.LIB

SPGEMM_OK = 0
STATUS = {
    0: "SPGEMM_OK", -1: "SPGEMM_ERR_INVALID_ARG", -2: "SPGEMM_ERR_DIM_MISMATCH",
    -3: "SPGEMM_ERR_INDEX_RANGE", -4: "SPGEMM_ERR_OVERFLOW", -5: "SPGEMM_ERR_OUT_OF_MEMORY",
    -6: "SPGEMM_ERR_PLAN_MISMATCH", -7: "SPGEMM_ERR_HIP", -8: "SPGEMM_ERR_NOT_READY",
    -9: "SPGEMM_ERR_CAPACITY", -10: "SPGEMM_ERR_SCRATCH_LIMIT", -11: "SPGEMM_ERR_INTERNAL",
}
CAPACITY = -9
SCRATCH_LIMIT = -10
NOALLOC_SCRATCH_BYTES = 64 << 20
PHASES = ["validate", "inter_prod_size", "binning", "csr_to_csc", "outer_prod", "histo",
          "multisplit", "heavy_accum", "light_accum", "prefix_sum", "direct_dense", "direct_rank"]
MAX_LEVELS = 8
EXPORTS = ["spgemm_options_default", "spgemm_plan_create", "spgemm_plan_destroy",
           "spgemm_symbolic", "spgemm_numeric", "spgemm_multiply", "spgemm_plan_stats",
           "spgemm_plan_debug", "spgemm_status_string", "spgemm_multiply_noalloc"]


class SpgemmError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({status_string(code)})")


class CSRStruct(ctypes.Structure):
    _fields_ = [("nrows", ctypes.c_int64), ("ncols", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("rowptr", ctypes.c_void_p), ("col", ctypes.c_void_p), ("val", ctypes.c_void_p)]


class Options(ctypes.Structure):
    _fields_ = [("lds_budget_bytes", ctypes.c_int64), ("tau_override", ctypes.c_int64),
                ("chunk_width_override", ctypes.c_int64), ("nchunks_cap", ctypes.c_int32),
                ("validate_inputs", ctypes.c_int32), ("debug_dump", ctypes.c_int32),
                ("timing", ctypes.c_int32), ("max_batch_products", ctypes.c_int64),
                ("symbolic_mode", ctypes.c_int32), ("numeric_mode", ctypes.c_int32),
                ("workspace_limit_bytes", ctypes.c_int64)]


NPH = len(PHASES)


class Stats(ctypes.Structure):
    _fields_ = [("nrows", ctypes.c_int64), ("ncols_c", ctypes.c_int64), ("nnz_c", ctypes.c_int64),
                ("sum_products", ctypes.c_int64), ("max_products", ctypes.c_int64),
                ("heavy_rows", ctypes.c_int64), ("heavy_products", ctypes.c_int64),
                ("tau", ctypes.c_int64), ("final_chunk_width", ctypes.c_int64),
                ("nlevels", ctypes.c_int32), ("nbatches", ctypes.c_int32),
                ("vchunks", ctypes.c_int32 * MAX_LEVELS),
                ("level_in_elems", ctypes.c_int64 * MAX_LEVELS),
                ("level_heavy_chunks", ctypes.c_int64 * MAX_LEVELS),
                ("level_final_chunks", ctypes.c_int64 * MAX_LEVELS),
                ("chat_bytes", ctypes.c_int64),
                ("phase_ms", (ctypes.c_double * NPH) * 2),
                ("phase_launches", (ctypes.c_int64 * NPH) * 2),
                ("phase_bytes", (ctypes.c_double * NPH) * 2),
                ("lds_bytes", ctypes.c_int64), ("light_rows", ctypes.c_int64),
                ("light_products", ctypes.c_int64), ("numeric_path", ctypes.c_int32),
                ("reserved_stats", ctypes.c_int32), ("u_p95", ctypes.c_int64),
                ("u_cv", ctypes.c_double), ("f_u_le", ctypes.c_double * 3),
                ("gamma", ctypes.c_double)]


class DebugMatrix(ctypes.Structure):
    _fields_ = [("nrows", ctypes.c_int64), ("nnz", ctypes.c_int64), ("rowptr", ctypes.c_void_p),
                ("col", ctypes.c_void_p), ("val", ctypes.c_void_p), ("row_key", ctypes.c_void_p),
                ("chunk_width", ctypes.c_int64)]


_lib = None


def load():
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime (same soname as ROCm's): load it
        # first, so that the library binds to it rather than bringing a
        # second runtime into the process beside torch's
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                              "(run __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.spgemm_options_default.argtypes = [ctypes.POINTER(Options)]
        lib.spgemm_options_default.restype = None
        lib.spgemm_plan_create.argtypes = [ctypes.POINTER(P), ctypes.POINTER(Options)]
        lib.spgemm_plan_create.restype = ctypes.c_int
        lib.spgemm_plan_destroy.argtypes = [P]
        lib.spgemm_plan_destroy.restype = None
        lib.spgemm_symbolic.argtypes = [P, ctypes.POINTER(CSRStruct), ctypes.POINTER(CSRStruct),
                                        P, ctypes.POINTER(ctypes.c_int64), P]
        lib.spgemm_symbolic.restype = ctypes.c_int
        lib.spgemm_numeric.argtypes = [P, ctypes.POINTER(CSRStruct), ctypes.POINTER(CSRStruct),
                                       P, P, P, P]
        lib.spgemm_numeric.restype = ctypes.c_int
        lib.spgemm_multiply.argtypes = [P, ctypes.POINTER(CSRStruct), ctypes.POINTER(CSRStruct),
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.POINTER(ctypes.c_int64),
                                        ctypes.c_void_p]
        lib.spgemm_multiply.restype = ctypes.c_int
        lib.spgemm_plan_stats.argtypes = [P, ctypes.POINTER(Stats)]
        lib.spgemm_plan_stats.restype = ctypes.c_int
        lib.spgemm_plan_debug.argtypes = [P, ctypes.c_int, ctypes.POINTER(DebugMatrix)]
        lib.spgemm_plan_debug.restype = ctypes.c_int
        lib.spgemm_multiply_noalloc.argtypes = [ctypes.POINTER(Options), ctypes.POINTER(CSRStruct),
                                                ctypes.POINTER(CSRStruct), ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p]
        lib.spgemm_multiply_noalloc.restype = ctypes.c_int
        lib.spgemm_status_string.argtypes = [ctypes.c_int]
        lib.spgemm_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(code: int) -> str:
    try:
        return load().spgemm_status_string(code).decode()
    except ImportError:
        return "library not loaded"


def _check(rc: int, what: str):
    if rc != SPGEMM_OK:
        raise SpgemmError(rc, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr() if t.numel() > 0 else None


@dataclasses.dataclass
class DeviceCSR:
    """A CSR matrix in device memory (torch tensors on cuda)."""

    nrows: int
    ncols: int
    rowptr: "object"
    col: "object"
    val: "object"

    @property
    def nnz(self) -> int:
        return int(self.col.numel())

    @staticmethod
    def from_host(M, device="cuda") -> "DeviceCSR":
        import torch
        return DeviceCSR(M.nrows, M.ncols, torch.from_numpy(np.ascontiguousarray(M.rowptr)).to(device),
                         torch.from_numpy(np.ascontiguousarray(M.col)).to(device),
                         torch.from_numpy(np.ascontiguousarray(M.val)).to(device))

    def struct(self) -> CSRStruct:
        return CSRStruct(self.nrows, self.ncols, self.nnz, self.rowptr.data_ptr(),
                         _ptr(self.col), _ptr(self.val))


def _stream_handle(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def make_options(tau_override=0, chunk_width_override=0, nchunks_cap=0, lds_budget_bytes=0,
                 validate_inputs=True, debug_dump=False, timing=False, max_batch_products=0,
                 symbolic_mode=0, numeric_mode=0, workspace_limit_bytes=0) -> Options:
    """An spgemm_options record: the library's defaults with these fields set."""
    o = Options()
    load().spgemm_options_default(ctypes.byref(o))
    o.tau_override = tau_override
    o.chunk_width_override = chunk_width_override
    o.nchunks_cap = nchunks_cap
    o.lds_budget_bytes = lds_budget_bytes
    o.validate_inputs = 1 if validate_inputs else 0
    o.debug_dump = 1 if debug_dump else 0
    o.timing = 1 if timing else 0
    o.max_batch_products = max_batch_products
    o.symbolic_mode = symbolic_mode
    o.numeric_mode = numeric_mode
    o.workspace_limit_bytes = workspace_limit_bytes
    return o


class Plan:
    """An spgemm plan: owns device workspace and the symbolic structure."""

    def __init__(self, tau_override=0, chunk_width_override=0, nchunks_cap=0, lds_budget_bytes=0,
                 validate_inputs=True, debug_dump=False, timing=False, max_batch_products=0,
                 symbolic_mode=0, numeric_mode=0, workspace_limit_bytes=0):
        lib = load()
        o = make_options(tau_override=tau_override, chunk_width_override=chunk_width_override,
                         nchunks_cap=nchunks_cap, lds_budget_bytes=lds_budget_bytes,
                         validate_inputs=validate_inputs, debug_dump=debug_dump, timing=timing,
                         max_batch_products=max_batch_products, symbolic_mode=symbolic_mode,
                         numeric_mode=numeric_mode, workspace_limit_bytes=workspace_limit_bytes)
        h = ctypes.c_void_p()
        _check(lib.spgemm_plan_create(ctypes.byref(h), ctypes.byref(o)), "spgemm_plan_create")
        self._h = h
        self._lib = lib

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.spgemm_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def symbolic(self, A: DeviceCSR, B: DeviceCSR, C_rowptr=None, stream=None):
        """Returns (C_rowptr int64 tensor, C_nnz)."""
        import torch
        if C_rowptr is None:
            C_rowptr = torch.empty(A.nrows + 1, dtype=torch.int64, device=A.rowptr.device)
        nnz = ctypes.c_int64(0)
        sa, sb = A.struct(), B.struct()
        _check(self._lib.spgemm_symbolic(self._h, ctypes.byref(sa), ctypes.byref(sb),
                                         C_rowptr.data_ptr(), ctypes.byref(nnz),
                                         _stream_handle(stream)), "spgemm_symbolic")
        return C_rowptr, int(nnz.value)

    def numeric(self, A: DeviceCSR, B: DeviceCSR, C_rowptr, C_col, C_val, stream=None):
        sa, sb = A.struct(), B.struct()
        _check(self._lib.spgemm_numeric(self._h, ctypes.byref(sa), ctypes.byref(sb),
                                        C_rowptr.data_ptr(), _ptr(C_col), _ptr(C_val),
                                        _stream_handle(stream)), "spgemm_numeric")

    def multiply(self, A: DeviceCSR, B: DeviceCSR, stream=None) -> DeviceCSR:
        import torch
        rp, nnz = self.symbolic(A, B, stream=stream)
        dev = A.rowptr.device
        col = torch.empty(nnz, dtype=torch.int32, device=dev)
        val = torch.empty(nnz, dtype=torch.float64, device=dev)
        self.numeric(A, B, rp, col, val, stream=stream)
        return DeviceCSR(A.nrows, B.ncols, rp, col, val)

    def multiply_once(self, A: DeviceCSR, B: DeviceCSR, capacity: int, stream=None):
        """Both phases in one library call with `capacity` entries of room for
        C. Returns (DeviceCSR, True) if C fit, else (DeviceCSR with a valid
        rowptr and empty col/val of the right size, False): then call numeric()."""
        import torch
        dev = A.rowptr.device
        rp = torch.empty(A.nrows + 1, dtype=torch.int64, device=dev)
        col = torch.empty(max(capacity, 0), dtype=torch.int32, device=dev)
        val = torch.empty(max(capacity, 0), dtype=torch.float64, device=dev)
        nnz = ctypes.c_int64(0)
        sa, sb = A.struct(), B.struct()
        rc = self._lib.spgemm_multiply(self._h, ctypes.byref(sa), ctypes.byref(sb),
                                       rp.data_ptr(), _ptr(col), _ptr(val), capacity,
                                       ctypes.byref(nnz), _stream_handle(stream))
        n = int(nnz.value)
        if rc == CAPACITY:
            return DeviceCSR(A.nrows, B.ncols, rp, torch.empty(n, dtype=torch.int32, device=dev),
                             torch.empty(n, dtype=torch.float64, device=dev)), False
        _check(rc, "spgemm_multiply")
        return DeviceCSR(A.nrows, B.ncols, rp, col[:n], val[:n]), True

    def stats(self) -> dict:
        s = Stats()
        _check(self._lib.spgemm_plan_stats(self._h, ctypes.byref(s)), "spgemm_plan_stats")
        L = int(s.nlevels)
        d = {k: getattr(s, k) for k in ("nrows", "ncols_c", "nnz_c", "sum_products",
                                         "max_products", "heavy_rows", "heavy_products", "tau",
                                         "final_chunk_width", "nlevels", "nbatches", "chat_bytes",
                                         "lds_bytes", "light_rows", "light_products",
                                         "numeric_path", "u_p95", "u_cv", "gamma")}
        d["f_u_le"] = [float(s.f_u_le[i]) for i in range(3)]
        d["vchunks"] = [int(s.vchunks[i]) for i in range(L)]
        d["level_in_elems"] = [int(s.level_in_elems[i]) for i in range(L)]
        d["level_heavy_chunks"] = [int(s.level_heavy_chunks[i]) for i in range(L)]
        d["level_final_chunks"] = [int(s.level_final_chunks[i]) for i in range(L)]
        for pi, pn in enumerate(("symbolic", "numeric")):
            d[pn] = {PHASES[i]: {"ms": s.phase_ms[pi][i], "launches": int(s.phase_launches[pi][i]),
                                 "bytes": s.phase_bytes[pi][i]} for i in range(NPH)}
        return d

    def debug(self, which: int):
        """Host copies of C-hat (which=-1) or a multisplit level's output."""
        import torch
        m = DebugMatrix()
        _check(self._lib.spgemm_plan_debug(self._h, which, ctypes.byref(m)), "spgemm_plan_debug")
        torch.cuda.synchronize()
        n, nnz = int(m.nrows), int(m.nnz)

        def grab(ptr, count, dtype):
            t = torch.empty(max(count, 0), dtype=dtype, device="cuda")
            if count > 0 and ptr:
                _hip_copy(t, ptr, count * t.element_size())
            return t.cpu().numpy()

        return {
            "rowptr": grab(m.rowptr, n + 1, torch.int64),
            "col": grab(m.col, nnz, torch.int32),
            "val": grab(m.val, nnz, torch.float64) if m.val else None,
            "row_key": grab(m.row_key, n, torch.int64),
            "chunk_width": int(m.chunk_width),
        }


def multiply_noalloc(A: DeviceCSR, B: DeviceCSR, C_rowptr, C_col, C_val, stream=None,
                     **options) -> int:
    """spgemm_multiply_noalloc into caller-allocated C buffers (capacity = C_col's
    length); returns nnz(C). Raises SpgemmError (CAPACITY too, with C_rowptr valid)."""
    lib = load()
    o = make_options(**options)
    nnz = ctypes.c_int64(0)
    sa, sb = A.struct(), B.struct()
    rc = lib.spgemm_multiply_noalloc(ctypes.byref(o), ctypes.byref(sa), ctypes.byref(sb),
                                     C_rowptr.data_ptr(), _ptr(C_col), _ptr(C_val),
                                     int(C_col.numel()), ctypes.byref(nnz),
                                     _stream_handle(stream))
    _check(rc, "spgemm_multiply_noalloc")
    return int(nnz.value)


def _hip_copy(dst_tensor, src_ptr: int, nbytes: int):
    """Device-to-device copy from a raw library pointer into a torch tensor."""
    import torch
    import torch  # noqa: F401  (its HIP runtime is the one already loaded)
    hip = ctypes.CDLL("libamdhip64.so.7")  # by soname: the runtime already in the process
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    rc = hip.hipMemcpy(dst_tensor.data_ptr(), src_ptr, nbytes, 3)  # hipMemcpyDeviceToDevice
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed ({rc})")
    torch.cuda.synchronize()


def spgemm(A: DeviceCSR, B: DeviceCSR, **plan_kwargs) -> DeviceCSR:
    """One-shot C = A*B on the GPU."""
    with Plan(**plan_kwargs) as p:
        return p.multiply(A, B)
