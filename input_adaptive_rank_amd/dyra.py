"""ctypes binding of libdyra.so (argument marshalling only).

Every step of the DyRA forward runs in the library's HIP kernels; PyTorch
only supplies device memory and the current HIP stream.  The entry points
mirror include/dyra.h one to one:

  prepare_sizes, prepare           offline fit on the host (float64)
  plan_size, plan_pack             pack factors into the device plan layout
  workspace_size, forward          the layer forward on the GPU
  solver_status                    per-segment solver status words
  dense_ref                        dense X W comparator on the same GEMM core

If libdyra.so is missing the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

from .synth import DT_BF16, DT_F32, KIND_BLAST, KIND_BLAST_DIAG, KIND_LOWRANK, KIND_MONARCH  # noqa: F401

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdyra.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dyra.h")

SOLVER_AUTO, SOLVER_CHOL, SOLVER_NS = 0, 1, 2
SOLVERS = {"auto": SOLVER_AUTO, "chol": SOLVER_CHOL, "ns": SOLVER_NS}
SOLVE_OK, SOLVE_NOT_SPD, SOLVE_NOCONV, SOLVE_ZERO, SOLVE_FALLBACK = 0, 1, 2, 3, 4

ERRORS = {0: "DYRA_OK", -1: "DYRA_EINVAL", -2: "DYRA_ESHAPE", -3: "DYRA_EWORKSPACE",
          -4: "DYRA_EHIP", -5: "DYRA_ENOCONV", -6: "DYRA_EDTYPE"}


class DyraError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {ERRORS.get(code, code)}")


class Spec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("k", ctypes.c_int32), ("mblk", ctypes.c_int32),
                ("nb", ctypes.c_int32), ("rb", ctypes.c_int32), ("r", ctypes.c_int32),
                ("c1", ctypes.c_int64), ("c2", ctypes.c_int64)]


_FACTORS = ("U", "V", "B1", "B2", "Ub", "S", "Vb", "P", "R0", "Wres", "res_sv")


class WsOffsets(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in ("A", "Wp", "Lt", "G", "M", "Ginv", "Mp", "Rt", "status", "total",
                                                "wa", "lt_pitch", "prec")]


class Sizes(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in _FACTORS]


class HostFactors(ctypes.Structure):
    _fields_ = [(f, ctypes.POINTER(ctypes.c_double)) for f in _FACTORS]


_lib = None


def lib():
    """Loads libdyra.so (built by input_adaptive_rank_amd.build)."""
    global _lib
    if _lib is None:
        # One HIP runtime per process: PyTorch ships its own libamdhip64
        # (same soname as the system one that libdyra.so is linked against).
        # Loading torch first lets the dynamic loader satisfy libdyra.so's
        # dependency with torch's copy; loading libdyra.so first would map a
        # second runtime beside torch's, and that one finds no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m input_adaptive_rank_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        SP = ctypes.POINTER(Spec)
        sig = {
            "dyra_prepare_sizes": [SP, ctypes.POINTER(Sizes)],
            "dyra_prepare": [SP, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(HostFactors), I32],
            "dyra_prepare_input_aware": [SP, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                         I64, I32, ctypes.POINTER(HostFactors), I32],
            "dyra_plan_size": [SP, I32, ctypes.POINTER(SZ)],
            "dyra_plan_pack": [SP, ctypes.POINTER(HostFactors), I32, P],
            "dyra_workspace_size": [SP, I64, I64, I32, ctypes.POINTER(SZ)],
            "dyra_forward": [SP, P, P, P, P, I64, I64, I32, ctypes.c_float, I32, P, SZ, P],
            "dyra_forward_events": [SP, P, P, P, P, I64, I64, I32, ctypes.c_float, I32, P, SZ, P,
                                    ctypes.POINTER(ctypes.c_void_p), I32],
            "dyra_solver_status": [SP, P, I64, I64, I32, ctypes.POINTER(I32), P],
            "dyra_dense_ref": [P, P, P, P, I64, I64, I64, I32, P],
            "dyra_workspace_offsets": [SP, I64, I64, I32, ctypes.POINTER(WsOffsets)],
            "dyra_workspace_size_als": [SP, I64, I64, I32, I32, ctypes.POINTER(SZ)],
            "dyra_forward_als": [SP, P, P, P, P, I64, I64, I32, ctypes.c_float, I32, I32, P, SZ, P],
            "dyra_forward_noalloc": [SP, P, P, P, P, I64, I64, I32, ctypes.c_float, I32, P, P],
            "dyra_workspace_size_varlen": [SP, I64, ctypes.POINTER(I64), I32, ctypes.POINTER(SZ)],
            "dyra_forward_varlen": [SP, P, P, P, P, I64, ctypes.POINTER(I64), P, I32, ctypes.c_float, I32, P, P,
                                    SZ, P],
            "dyra_workspace_size_varlen_als": [SP, I64, ctypes.POINTER(I64), I32, I32, ctypes.POINTER(SZ)],
            "dyra_forward_varlen_als": [SP, P, P, P, P, I64, ctypes.POINTER(I64), P, I32, ctypes.c_float, I32, I32,
                                        P, P, SZ, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.dyra_status_string.argtypes = [ctypes.c_int]
        L.dyra_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_symbols():
    """Names of the functions include/dyra.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(dyra_\w+)\s*\(", text, re.M)))


def _check(fn, code):
    if code != 0:
        raise DyraError(fn, code)


def make_spec(kind, c1, c2, r, k=0, mblk=0, nb=0, rb=0) -> Spec:
    return Spec(kind=kind, k=k, mblk=mblk, nb=nb, rb=rb, r=r, c1=c1, c2=c2)


def spec_of(w) -> Spec:
    """Spec of a synth.Workload."""
    return make_spec(w.kind, w.c1, w.c2, w.r, k=w.k, mblk=w.mblk, nb=w.nb, rb=w.rb)


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def prepare_sizes(spec: Spec) -> dict:
    s = Sizes()
    _check("dyra_prepare_sizes", lib().dyra_prepare_sizes(ctypes.byref(spec), ctypes.byref(s)))
    return {f: getattr(s, f) for f in _FACTORS}


def _factor_shapes(spec: Spec) -> dict:
    m, nb, rb = spec.mblk, spec.nb, spec.rb
    return {"U": (spec.c1, spec.k), "V": (spec.k, spec.c2), "B1": (m, m, m), "B2": (m, m, m),
            "Ub": (nb, spec.c1 // max(nb, 1), rb),
            "S": (nb, nb, rb) if spec.kind == KIND_BLAST_DIAG else (nb, nb, rb, rb),
            "Vb": (nb, spec.c2 // max(nb, 1), rb),
            "P": (spec.c1, spec.r), "R0": (spec.r, spec.c2), "Wres": (spec.c1, spec.c2), "res_sv": (spec.r,)}


def _host_factors(spec: Spec, arrays: dict) -> HostFactors:
    hf = HostFactors()
    for f in _FACTORS:
        a = arrays.get(f)
        if a is not None:
            setattr(hf, f, _dptr(a))
    return hf


def prepare(W: np.ndarray, spec: Spec, nthreads: int = 0) -> dict:
    """Offline fit on the host.  Returns float64 arrays keyed like dyra_host_factors."""
    W = np.ascontiguousarray(W, dtype=np.float64)
    if W.shape != (spec.c1, spec.c2):
        raise ValueError(f"W must be {spec.c1} x {spec.c2}")
    sizes = prepare_sizes(spec)
    shapes = _factor_shapes(spec)
    out = {f: np.zeros(shapes[f]) for f in _FACTORS if sizes[f] > 0}
    hf = _host_factors(spec, out)
    _check("dyra_prepare", lib().dyra_prepare(ctypes.byref(spec), _dptr(W), ctypes.byref(hf), nthreads))
    return out


INPUT_AWARE_DIAG, INPUT_AWARE_CHOL = 1, 2
INPUT_AWARE = {"diag": INPUT_AWARE_DIAG, "chol": INPUT_AWARE_CHOL}


def prepare_input_aware(W: np.ndarray, spec: Spec, X_cal: np.ndarray, mode: int, nthreads: int = 0) -> dict:
    """Offline fit with an input-aware static start from calibration rows
    X_cal (n_cal x c1).  Returns float64 arrays keyed like dyra_host_factors."""
    W = np.ascontiguousarray(W, dtype=np.float64)
    X_cal = np.ascontiguousarray(X_cal, dtype=np.float64)
    if W.shape != (spec.c1, spec.c2):
        raise ValueError(f"W must be {spec.c1} x {spec.c2}")
    if X_cal.ndim != 2 or X_cal.shape[1] != spec.c1:
        raise ValueError(f"X_cal must be n_cal x {spec.c1}")
    sizes = prepare_sizes(spec)
    shapes = _factor_shapes(spec)
    out = {f: np.zeros(shapes[f]) for f in _FACTORS if sizes[f] > 0}
    hf = _host_factors(spec, out)
    _check("dyra_prepare_input_aware",
           lib().dyra_prepare_input_aware(ctypes.byref(spec), _dptr(W), _dptr(X_cal), X_cal.shape[0], mode,
                                          ctypes.byref(hf), nthreads))
    return out


def plan_size(spec: Spec, dtype: int) -> int:
    n = ctypes.c_size_t()
    _check("dyra_plan_size", lib().dyra_plan_size(ctypes.byref(spec), dtype, ctypes.byref(n)))
    return n.value


def plan_pack(spec: Spec, factors: dict, dtype: int) -> np.ndarray:
    """Host bytes of the device plan (copy them to the GPU once)."""
    arrays = {f: np.ascontiguousarray(v, dtype=np.float64) for f, v in factors.items() if v is not None}
    buf = np.zeros(plan_size(spec, dtype), dtype=np.uint8)
    hf = _host_factors(spec, arrays)
    _check("dyra_plan_pack", lib().dyra_plan_pack(ctypes.byref(spec), ctypes.byref(hf), dtype,
                                                  buf.ctypes.data_as(ctypes.c_void_p)))
    return buf


def workspace_size(spec: Spec, B: int, s: int, dtype: int) -> int:
    n = ctypes.c_size_t()
    _check("dyra_workspace_size", lib().dyra_workspace_size(ctypes.byref(spec), B, s, dtype, ctypes.byref(n)))
    return n.value


def workspace_offsets(spec: Spec, B: int, s: int, dtype: int) -> dict:
    o = WsOffsets()
    _check("dyra_workspace_offsets", lib().dyra_workspace_offsets(ctypes.byref(spec), B, s, dtype, ctypes.byref(o)))
    return {f: getattr(o, f) for f, _ in WsOffsets._fields_}


# ---------------------------------------------------------------------------
# device calls (torch tensors as plain device buffers)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def torch_dtype(dtype: int):
    torch = _torch()
    return torch.bfloat16 if dtype == DT_BF16 else torch.float32


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect_shape(t, name, shape, dtype):
    """Raises ValueError unless tensor t has exactly this shape and dtype.
    The library receives bare pointers, so a wrong size would read or write
    past a buffer on the device: every size is checked here first."""
    if t is None or not hasattr(t, "shape"):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _expect_bytes(t, name, nbytes):
    """A raw byte buffer (plan, workspace): 1-D uint8 of at least nbytes."""
    torch = _torch()
    if t is None or not hasattr(t, "shape"):
        raise ValueError(f"{name} must be a tensor")
    if t.dtype != torch.uint8 or t.dim() != 1:
        raise ValueError(f"{name} must be a 1-D uint8 tensor")
    if t.numel() < nbytes:
        raise ValueError(f"{name} holds {t.numel()} bytes, needs {nbytes}")


def _expect_device(tensors, device):
    """Every (name, tensor) is contiguous and on the GPU `device`."""
    for name, t in tensors:
        if t is None:
            continue
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_forward_tensors(spec: Spec, plan, X, bias, Y, B: int, s: int, dtype: int, workspace, ws_bytes):
    """Shapes and dtypes of every argument first, then contiguity and device.
    ws_bytes: a function of nothing giving the workspace bytes needed."""
    if not (isinstance(B, int) and isinstance(s, int)) or B <= 0 or s <= 0:
        raise ValueError("B and s must be positive integers")
    ws_bytes = ws_bytes()
    td = torch_dtype(dtype)
    n = B * s
    _expect_shape(X, "X", (n, spec.c1), td)
    _expect_shape(Y, "Y", (n, spec.c2), td)
    if bias is not None:
        _expect_shape(bias, "bias", (spec.c2,), td)
    _expect_bytes(plan, "plan", plan_size(spec, dtype))
    if workspace is not None or ws_bytes:
        _expect_bytes(workspace, "workspace", ws_bytes)
    _expect_device([("X", X), ("Y", Y), ("bias", bias), ("plan", plan), ("workspace", workspace)], X.device)
    if Y.data_ptr() < X.data_ptr() + X.numel() * X.element_size() and \
            X.data_ptr() < Y.data_ptr() + Y.numel() * Y.element_size():
        raise ValueError("Y must not overlap X")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def forward(spec: Spec, plan, X, bias, Y, B: int, s: int, dtype: int, eps: float = 1e-6,
            solver: int = SOLVER_AUTO, workspace=None, stream=None):
    """Launches the DyRA forward (asynchronous on `stream`)."""
    _check_forward_tensors(spec, plan, X, bias, Y, B, s, dtype, workspace,
                           lambda: workspace_size(spec, B, s, dtype))
    rc = lib().dyra_forward(ctypes.byref(spec), _dev(plan, "plan"), _dev(X, "X"), _dev(bias, "bias"),
                            _dev(Y, "Y"), B, s, dtype, eps, solver, _dev(workspace, "workspace"),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dyra_forward", rc)


def workspace_size_als(spec: Spec, B: int, s: int, dtype: int, half_steps: int) -> int:
    n = ctypes.c_size_t()
    _check("dyra_workspace_size_als",
           lib().dyra_workspace_size_als(ctypes.byref(spec), B, s, dtype, half_steps, ctypes.byref(n)))
    return n.value


def forward_als(spec: Spec, plan, X, bias, Y, B: int, s: int, dtype: int, eps: float, solver: int,
                half_steps: int, workspace, stream=None):
    """The forward with 2 t = half_steps ALS half-steps (asynchronous)."""
    _check_forward_tensors(spec, plan, X, bias, Y, B, s, dtype, workspace,
                           lambda: workspace_size_als(spec, B, s, dtype, half_steps))
    rc = lib().dyra_forward_als(ctypes.byref(spec), _dev(plan, "plan"), _dev(X, "X"), _dev(bias, "bias"),
                                _dev(Y, "Y"), B, s, dtype, eps, solver, half_steps, _dev(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dyra_forward_als", rc)


def _offsets(offsets) -> np.ndarray:
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    if off.ndim != 1 or off.size < 2:
        raise ValueError("offsets must be a 1-D array of B + 1 row offsets")
    return off


def workspace_size_varlen(spec: Spec, offsets, dtype: int, half_steps: int = 2) -> int:
    off = _offsets(offsets)
    nb = ctypes.c_size_t()
    _check("dyra_workspace_size_varlen_als",
           lib().dyra_workspace_size_varlen_als(ctypes.byref(spec), off.size - 1,
                                                off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), dtype,
                                                half_steps, ctypes.byref(nb)))
    return nb.value


def forward_varlen(spec: Spec, plan, X, bias, Y, offsets, dtype: int, eps: float = 1e-6, solver: int = SOLVER_AUTO,
                   workspace=None, offsets_dev=None, status=None, stream=None, half_steps: int = 2):
    """The forward over ragged segments: segment b is rows offsets[b] ..
    offsets[b + 1] - 1 of X (asynchronous), with 2 t = half_steps ALS
    half-steps.  offsets_dev: a device int32 copy of the offsets (made here
    when not given); status: optional device int32 [B] for the per-segment
    solver status words."""
    torch = _torch()
    off = _offsets(offsets)
    B, n = off.size - 1, int(off[-1])
    if np.any(np.diff(off) < 1) or off[0] != 0:
        raise ValueError("offsets must start at 0 and grow by at least one row per segment")
    _check_forward_tensors(spec, plan, X, bias, Y, 1, n, dtype, workspace,
                           lambda: workspace_size_varlen(spec, off, dtype, half_steps))
    if offsets_dev is None:
        offsets_dev = torch.from_numpy(off.astype(np.int32)).to(X.device)
    _expect_shape(offsets_dev, "offsets_dev", (B + 1,), torch.int32)
    _expect_device([("offsets_dev", offsets_dev)], X.device)
    if status is not None:
        _expect_shape(status, "status", (B,), torch.int32)
        _expect_device([("status", status)], X.device)
    rc = lib().dyra_forward_varlen_als(ctypes.byref(spec), _dev(plan, "plan"), _dev(X, "X"), _dev(bias, "bias"),
                                       _dev(Y, "Y"), B, off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                       _dev(offsets_dev, "offsets_dev"), dtype, eps, solver, half_steps,
                                       _dev(status, "status"), _dev(workspace, "workspace"),
                                       workspace.numel() * workspace.element_size(), _stream(stream))
    _check("dyra_forward_varlen_als", rc)


NOALLOC_MAX_WORKSPACE = 64 << 20   # DYRA_NOALLOC_MAX_WORKSPACE


def forward_noalloc(spec: Spec, plan, X, bias, Y, B: int, s: int, dtype: int, eps: float = 1e-6,
                    solver: int = SOLVER_AUTO, status=None, stream=None):
    """The forward on the library's static device workspace (no allocation,
    asynchronous).  status: optional device int32 tensor [B] that receives
    the per-segment solver status words.  Calls overlapping in time on one
    GPU share that workspace and race."""
    torch = _torch()
    _check_forward_tensors(spec, plan, X, bias, Y, B, s, dtype, None, lambda: 0)
    if status is not None:
        _expect_shape(status, "status", (B,), torch.int32)
        _expect_device([("status", status)], X.device)
    rc = lib().dyra_forward_noalloc(ctypes.byref(spec), _dev(plan, "plan"), _dev(X, "X"), _dev(bias, "bias"),
                                    _dev(Y, "Y"), B, s, dtype, eps, solver, _dev(status, "status"),
                                    _stream(stream))
    _check("dyra_forward_noalloc", rc)


def forward_events(spec: Spec, plan, X, bias, Y, B: int, s: int, dtype: int, eps: float, solver: int,
                   workspace, events, stream=None):
    """dyra_forward recording stage-boundary events (torch.cuda.Event objects
    that have been recorded once, so their HIP handles exist)."""
    _check_forward_tensors(spec, plan, X, bias, Y, B, s, dtype, workspace,
                           lambda: workspace_size(spec, B, s, dtype))
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    rc = lib().dyra_forward_events(ctypes.byref(spec), _dev(plan, "plan"), _dev(X, "X"), _dev(bias, "bias"),
                                   _dev(Y, "Y"), B, s, dtype, eps, solver, _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream), arr,
                                   len(events))
    _check("dyra_forward_events", rc)


def solver_status(spec: Spec, workspace, B: int, s: int, dtype: int, stream=None) -> np.ndarray:
    out = np.zeros(B, dtype=np.int32)
    rc = lib().dyra_solver_status(ctypes.byref(spec), _dev(workspace, "workspace"), B, s, dtype,
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _stream(stream))
    _check("dyra_solver_status", rc)
    return out


def dense_ref(X, Wt, bias, Y, dtype: int, stream=None):
    """Y = X W + bias with Wt = W^T (asynchronous)."""
    td = torch_dtype(dtype)
    if X is None or X.dim() != 2 or Wt is None or Wt.dim() != 2:
        raise ValueError("X and Wt must be 2-D GPU tensors")
    n, c1 = X.shape
    c2 = Wt.shape[0]
    _expect_shape(X, "X", (n, c1), td)
    _expect_shape(Wt, "Wt", (c2, c1), td)
    _expect_shape(Y, "Y", (n, c2), td)
    if bias is not None:
        _expect_shape(bias, "bias", (c2,), td)
    _expect_device([("X", X), ("Wt", Wt), ("Y", Y), ("bias", bias)], X.device)
    rc = lib().dyra_dense_ref(_dev(X, "X"), _dev(Wt, "Wt"), _dev(bias, "bias"), _dev(Y, "Y"), n, c1, c2,
                              dtype, _stream(stream))
    _check("dyra_dense_ref", rc)


def to_device(a: np.ndarray, dtype: int, device="cuda"):
    """Uploads host values (already storage-representable) as a dtype tensor."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device, dtype=torch_dtype(dtype))


class DyraLayer:
    """A prepared DyRA layer resident on one GPU: device plan + workspace."""

    def __init__(self, spec: Spec, factors: dict, dtype: int, bias: np.ndarray | None = None,
                 device="cuda", eps: float = 1e-6, solver: int = SOLVER_AUTO, half_steps: int = 2):
        torch = _torch()
        self.spec, self.dtype, self.eps, self.solver = spec, dtype, eps, solver
        self.half_steps = half_steps   # 2 t ALS half-steps (2: t = 1)
        self.device = torch.device(device)
        host = plan_pack(spec, factors, dtype)
        self.plan = torch.from_numpy(host).to(self.device)
        self.device = self.plan.device          # "cuda" -> "cuda:<index>"
        self.bias = None if bias is None else to_device(bias, dtype, self.device)
        self._ws = None
        self._ws_key = None

    def workspace(self, B: int, s: int):
        torch = _torch()
        key = (B, s)
        if self._ws_key != key:
            n = (workspace_size(self.spec, B, s, self.dtype) if self.half_steps == 2 else
                 workspace_size_als(self.spec, B, s, self.dtype, self.half_steps))
            if self._ws is None or self._ws.numel() < n:
                self._ws = torch.empty(n, dtype=torch.uint8, device=self.device)
            self._ws_key = key
        return self._ws

    def forward(self, X, B: int, s: int, out=None, stream=None):
        torch = _torch()
        if X.dtype != torch_dtype(self.dtype):
            raise ValueError("X dtype does not match the plan dtype")
        if X.device != self.device:
            raise ValueError(f"X is on {X.device}, the layer on {self.device}")
        Y = out if out is not None else torch.empty((B * s, self.spec.c2), dtype=X.dtype, device=X.device)
        ws = self.workspace(B, s)
        if self.half_steps == 2:
            forward(self.spec, self.plan, X, self.bias, Y, B, s, self.dtype, self.eps, self.solver, ws, stream)
        else:
            forward_als(self.spec, self.plan, X, self.bias, Y, B, s, self.dtype, self.eps, self.solver,
                        self.half_steps, ws, stream)
        return Y

    def forward_varlen(self, X, offsets, out=None, stream=None):
        """Ragged segments (the layer's ALS iterations): returns (Y, status)
        with status a device int32 array of the per-segment solver status
        words."""
        torch = _torch()
        off = _offsets(offsets)
        if X.dtype != torch_dtype(self.dtype) or X.device != self.device:
            raise ValueError("X dtype / device does not match the layer")
        Y = out if out is not None else torch.empty((int(off[-1]), self.spec.c2), dtype=X.dtype, device=X.device)
        n = workspace_size_varlen(self.spec, off, self.dtype, self.half_steps)
        ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        st = torch.empty(off.size - 1, dtype=torch.int32, device=self.device)
        forward_varlen(self.spec, self.plan, X, self.bias, Y, off, self.dtype, self.eps, self.solver, ws,
                       status=st, stream=stream, half_steps=self.half_steps)
        return Y, st

    def forward_events(self, X, B: int, s: int, out, events, stream=None):
        ws = self.workspace(B, s)
        forward_events(self.spec, self.plan, X, self.bias, out, B, s, self.dtype, self.eps, self.solver, ws,
                       events, stream)
        return out

    def status(self, B: int, s: int, stream=None) -> np.ndarray:
        return solver_status(self.spec, self.workspace(B, s), B, s, self.dtype, stream)
