"""Thin ctypes binding of libqlora_nf4.so (argument marshalling only).

Every function here has the name of the C entry point it calls. torch is
used for device memory, shapes and the current HIP stream; all arithmetic
happens in the library's HIP kernels. If the library has not been built the
first call raises (there is no fallback path).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# QLORA_NF4_LIB selects another build of the same library (the sanitizer run)
LIB_PATH = os.environ.get("QLORA_NF4_LIB") or os.path.join(HERE, "libqlora_nf4.so")

QLORA_OK = 0
QLORA_ERR_ARG = -1
QLORA_ERR_SHAPE = -2
QLORA_ERR_ALIGN = -3
QLORA_ERR_WORKSPACE = -4
QLORA_ERR_HIP = -5
QLORA_F32 = 0
QLORA_BF16 = 1
QLORA_BLOCK = 64
QLORA_DQ_BLOCK = 256
QLORA_MAX_RANK = 256
# 4-bit data types (qlora_qtype)
QTYPES = {"nf4": 0, "int4": 1, "fp4_e2m1": 2, "fp4_e3m0": 3}

# every symbol declared in include/qlora_nf4.h
EXPORTS = (
    "qlora_status_str", "qlora_last_error", "qlora_nf4_codebook", "qlora_codebook", "qlora_quant_sizes",
    "qlora_quantize", "qlora_dequantize", "qlora_linear_workspace", "qlora_linear_fwd",
    "qlora_linear_bwd", "qlora_set_timing", "qlora_int8_quantize", "qlora_int8_dequantize",
    "qlora_merge_adapters", "qlora_linear_workspace_dropout", "qlora_linear_fwd_dropout",
    "qlora_linear_bwd_dropout", "qlora_lora_dropout", "qlora_clip_grad_norm", "qlora_adam_step",
    "qlora_linear_fwd_noalloc", "qlora_check_conversions", "qlora_probe_mfma", "qlora_probe_read",
    "qlora_quantize_batch", "qlora_quant_batch_workspace",
)
QLORA_NOALLOC_SCRATCH_BYTES = (2 << 20) + (64 << 10)
QLORA_QUANT_BATCH_MAX = 16
QLORA_CLIP_WORKSPACE_BYTES = 8192


class AdamParams(ctypes.Structure):
    """Mirror of the C struct qlora_adam_params."""

    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64)]
INT8_BLOCKS = (64, 128, 256, 512, 1024, 2048, 4096)
QLORA_TIMING_FWD_GEMM = 0
QLORA_TIMING_DX_GEMM = 1
QLORA_TIMING_GEMV = 2
QLORA_TIMING_QUANT = 3
QLORA_TIMING_DEQUANT = 4
QLORA_TIMING_MID_GEMM = 5


class QNF4(ctypes.Structure):
    """Mirror of the C struct qlora_nf4 (host struct of device pointers)."""

    _fields_ = [
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("absmax8", ctypes.c_void_p),
        ("scale2", ctypes.c_void_p),
        ("mean", ctypes.c_void_p),
        ("qtype", ctypes.c_int32),
        ("no_dq", ctypes.c_int32),
        ("absmax32", ctypes.c_void_p),
    ]


class QLoRAError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _load()
        msg = lib.qlora_status_str(status).decode()
        extra = lib.qlora_last_error().decode() if status == QLORA_ERR_HIP else ""
        super().__init__(f"{where}: {msg}" + (f" ({extra})" if extra else ""))
        self.status = status


_LIB = None


def _load():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python {os.path.join(HERE, 'build.py')}`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    lib.qlora_status_str.argtypes = [ctypes.c_int]
    lib.qlora_status_str.restype = ctypes.c_char_p
    lib.qlora_last_error.argtypes = []
    lib.qlora_last_error.restype = ctypes.c_char_p
    lib.qlora_nf4_codebook.argtypes = [P(ctypes.c_float)]
    lib.qlora_nf4_codebook.restype = ctypes.c_int
    lib.qlora_codebook.argtypes = [ctypes.c_int, P(ctypes.c_float)]
    lib.qlora_codebook.restype = ctypes.c_int
    lib.qlora_quant_sizes.argtypes = [i64, i64, P(sz), P(sz), P(sz), P(sz)]
    lib.qlora_quant_sizes.restype = ctypes.c_int
    lib.qlora_quantize.argtypes = [vp, ctypes.c_int, P(QNF4), vp, sz, vp]
    lib.qlora_quantize.restype = ctypes.c_int
    lib.qlora_dequantize.argtypes = [P(QNF4), vp, vp]
    lib.qlora_dequantize.restype = ctypes.c_int
    lib.qlora_linear_workspace.argtypes = [i64, i64, i64, ctypes.c_int, P(sz)]
    lib.qlora_linear_workspace.restype = ctypes.c_int
    lib.qlora_linear_fwd.argtypes = [P(QNF4), vp, i64, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.qlora_linear_fwd.restype = ctypes.c_int
    lib.qlora_linear_bwd.argtypes = [P(QNF4), vp, vp, i64, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp, vp, vp,
                                     ctypes.c_int, vp, sz, vp]
    lib.qlora_linear_bwd.restype = ctypes.c_int
    lib.qlora_linear_fwd_noalloc.argtypes = [P(QNF4), vp, i64, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp, vp]
    lib.qlora_linear_fwd_noalloc.restype = ctypes.c_int
    lib.qlora_set_timing.argtypes = [ctypes.c_int, vp, vp, ctypes.c_int, P(ctypes.c_int)]
    lib.qlora_set_timing.restype = ctypes.c_int
    lib.qlora_quantize_batch.argtypes = [ctypes.c_int, P(vp), ctypes.c_int, P(P(QNF4)), vp, sz, vp]
    lib.qlora_quantize_batch.restype = ctypes.c_int
    lib.qlora_quant_batch_workspace.argtypes = [ctypes.c_int, P(i64), P(i64), P(sz)]
    lib.qlora_quant_batch_workspace.restype = ctypes.c_int
    u64 = ctypes.c_uint64
    lib.qlora_clip_grad_norm.argtypes = [vp, i64, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.qlora_clip_grad_norm.restype = ctypes.c_int
    lib.qlora_adam_step.argtypes = [vp, vp, vp, vp, i64, ctypes.c_void_p, vp, vp, vp]
    lib.qlora_adam_step.restype = ctypes.c_int
    lib.qlora_linear_workspace_dropout.argtypes = [i64, i64, i64, ctypes.c_int, P(sz)]
    lib.qlora_linear_workspace_dropout.restype = ctypes.c_int
    lib.qlora_linear_fwd_dropout.argtypes = [P(QNF4), vp, i64, vp, vp, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                             u64, vp, vp, vp, sz, vp]
    lib.qlora_linear_fwd_dropout.restype = ctypes.c_int
    lib.qlora_linear_bwd_dropout.argtypes = [P(QNF4), vp, vp, i64, vp, vp, ctypes.c_int, ctypes.c_float,
                                             ctypes.c_float, u64, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    lib.qlora_linear_bwd_dropout.restype = ctypes.c_int
    lib.qlora_lora_dropout.argtypes = [vp, i64, ctypes.c_float, u64, vp, vp]
    lib.qlora_lora_dropout.restype = ctypes.c_int
    lib.qlora_merge_adapters.argtypes = [P(QNF4), vp, vp, ctypes.c_int, ctypes.c_float, vp, vp]
    lib.qlora_merge_adapters.restype = ctypes.c_int
    lib.qlora_int8_quantize.argtypes = [vp, ctypes.c_int, i64, ctypes.c_int, vp, vp, vp]
    lib.qlora_int8_quantize.restype = ctypes.c_int
    lib.qlora_int8_dequantize.argtypes = [vp, vp, i64, ctypes.c_int, vp, ctypes.c_int, vp]
    lib.qlora_check_conversions.argtypes = [ctypes.c_uint32, i64, vp, vp, vp, vp]
    lib.qlora_check_conversions.restype = ctypes.c_int
    lib.qlora_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.qlora_probe_mfma.restype = ctypes.c_int
    lib.qlora_probe_read.argtypes = [vp, sz, ctypes.c_uint32, vp, vp]
    lib.qlora_probe_read.restype = ctypes.c_int
    lib.qlora_int8_dequantize.restype = ctypes.c_int
    _LIB = lib
    return lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def _check(status: int, where: str):
    if status != QLORA_OK:
        raise QLoRAError(status, where)


def _stream(stream=None):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run a wrapper with torch's current stream set to its ``stream``
    argument (when one is given), so that the workspace and the outputs it
    allocates belong to the stream the library's kernels run on. The caching
    allocator then hands a freed workspace only to later work on that same
    stream, which the stream orders after the kernels still using it."""
    import functools
    import inspect

    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        import torch

        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)

    return wrapper


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, shape, name):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---- host-only queries ------------------------------------------------------------

def qlora_nf4_codebook() -> np.ndarray:
    out = (ctypes.c_float * 16)()
    _check(_load().qlora_nf4_codebook(out), "qlora_nf4_codebook")
    return np.frombuffer(bytes(out), dtype=np.float32).copy()


def qlora_codebook(qtype: str | int = "nf4") -> np.ndarray:
    """The 16 ascending fp32 values of a 4-bit data type (name or qlora_qtype)."""
    out = (ctypes.c_float * 16)()
    _check(_load().qlora_codebook(_qtype(qtype), out), "qlora_codebook")
    return np.frombuffer(bytes(out), dtype=np.float32).copy()


def _qtype(qtype: str | int) -> int:
    if isinstance(qtype, str):
        if qtype not in QTYPES:
            raise ValueError(f"unknown 4-bit data type {qtype!r}")
        return QTYPES[qtype]
    return int(qtype)


def qlora_quant_sizes(rows: int, cols: int) -> dict:
    a, b, c, d = (ctypes.c_size_t() for _ in range(4))
    _check(_load().qlora_quant_sizes(rows, cols, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                     ctypes.byref(d)), "qlora_quant_sizes")
    return {"codes": a.value, "absmax8": b.value, "scale2": c.value, "workspace": d.value}


def qlora_quant_batch_workspace(shapes) -> int:
    """Scratch bytes of qlora_quantize_batch for a list of (rows, cols)."""
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(a) for a, _ in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(b) for _, b in shapes])
    out = ctypes.c_size_t()
    _check(_load().qlora_quant_batch_workspace(n, rows, cols, ctypes.byref(out)), "qlora_quant_batch_workspace")
    return out.value


def qlora_linear_workspace(M: int, K: int, N: int, r: int) -> int:
    out = ctypes.c_size_t()
    _check(_load().qlora_linear_workspace(M, K, N, r, ctypes.byref(out)), "qlora_linear_workspace")
    return out.value


def qlora_linear_workspace_dropout(M: int, K: int, N: int, r: int) -> int:
    out = ctypes.c_size_t()
    _check(_load().qlora_linear_workspace_dropout(M, K, N, r, ctypes.byref(out)), "qlora_linear_workspace_dropout")
    return out.value


def _need_mem(t, dtype, shape, name):
    """A device tensor, or a pinned host tensor (the kernels reach it over the host link)."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@_on_stream
def qlora_clip_grad_norm(g, max_norm: float, coef=None, norm=None, workspace=None, stream=None):
    """coef = min(1, max_norm / (||g|| + 1e-6)) and the norm (float64), as 1-element device tensors."""
    import torch

    n = g.numel()
    _need_mem(g, torch.float32, tuple(g.shape), "g")
    dev = g.device if g.is_cuda else torch.device("cuda")
    coef = coef if coef is not None else torch.empty(1, dtype=torch.float32, device=dev)
    norm = norm if norm is not None else torch.empty(1, dtype=torch.float64, device=dev)
    ws = _workspace(QLORA_CLIP_WORKSPACE_BYTES, dev, workspace)
    _check(_load().qlora_clip_grad_norm(_ptr(g), n, float(max_norm), _ptr(coef), _ptr(norm), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)), "qlora_clip_grad_norm")
    return coef, norm


@_on_stream
def qlora_adam_step(theta, g, m, v, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                    eps: float = 1e-8, weight_decay: float = 0.0, coef=None, theta_bf16=None, stream=None):
    """One Adam step in place on flat fp32 theta, m, v (each a device tensor or
    pinned host memory) for gradient g, clipped by ``coef`` (1-element tensor)."""
    import torch

    n = theta.numel()
    for t, name in ((theta, "theta"), (g, "g"), (m, "m"), (v, "v")):
        _need_mem(t, torch.float32, (n,), name)
    if theta_bf16 is not None:
        _need_mem(theta_bf16, torch.bfloat16, (n,), "theta_bf16")
    hp = AdamParams(lr, beta1, beta2, eps, weight_decay, step)
    _check(_load().qlora_adam_step(_ptr(theta), _ptr(g), _ptr(m), _ptr(v), n, ctypes.byref(hp), _ptr(coef),
                                   _ptr(theta_bf16), _stream(stream)), "qlora_adam_step")


@_on_stream
def qlora_lora_dropout(X, p: float, seed: int, out=None, stream=None):
    """The dropped adapter input Xd of a bf16 device tensor (same shape)."""
    import torch

    _need(X, torch.bfloat16, tuple(X.shape), "X")
    y = out if out is not None else torch.empty_like(X)
    _need(y, torch.bfloat16, tuple(X.shape), "out")
    _check(_load().qlora_lora_dropout(_ptr(X), X.numel(), float(p), int(seed), _ptr(y), _stream(stream)),
           "qlora_lora_dropout")
    return y


@_on_stream
def qlora_check_conversions(first: int, count: int, bf16=True, e4m3=True, table=False, stream=None):
    """The device conversions on the fp32 bit patterns first .. first + count - 1.

    Returns (bf16 bits as a device int16 tensor or None, E4M3 codes as a
    device uint8 tensor or None, the 256 decoded E4M3 codes as a device
    float32 tensor or None)."""
    import torch

    bf = torch.empty(count, dtype=torch.int16, device="cuda") if bf16 else None
    e8 = torch.empty(count, dtype=torch.uint8, device="cuda") if e4m3 else None
    tb = torch.empty(256, dtype=torch.float32, device="cuda") if table else None
    _check(_load().qlora_check_conversions(int(first) & 0xFFFFFFFF, int(count), _ptr(bf), _ptr(e8), _ptr(tb),
                                           _stream(stream)), "qlora_check_conversions")
    return bf, e8, tb


QLORA_PROBE_READ_GRANULE = 65536


@_on_stream
def qlora_probe_mfma(workgroups: int, iters: int, sink, clocks, stream=None):
    """Enqueue the register-only MFMA loop (measurement aid); sink: device
    float32[workgroups * 512], clocks: device int64[2]."""
    _check(_load().qlora_probe_mfma(int(workgroups), int(iters), _ptr(sink), _ptr(clocks), _stream(stream)),
           "qlora_probe_mfma")


@_on_stream
def qlora_probe_read(src, never: int, sink, stream=None):
    """Enqueue one streaming read of the device tensor src (measurement aid)."""
    _check(_load().qlora_probe_read(_ptr(src), src.numel() * src.element_size(), int(never) & 0xFFFFFFFF,
                                    _ptr(sink), _stream(stream)), "qlora_probe_read")


class KernelTimer:
    """Event brackets around every launch of one kernel class (qlora_set_timing).

    Use as a context manager around the calls to measure; ``durations_ms()``
    then gives the per-launch times from the HIP events on the library's
    stream. Events are created through torch (plumbing only).
    """

    def __init__(self, kernel: int, capacity: int = 4096):
        import torch

        self.kernel = kernel
        self.events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(capacity)]
        # torch creates the underlying HIP event on its first record()
        for a, b in self.events:
            a.record()
            b.record()
        torch.cuda.synchronize()
        if any(not a.cuda_event or not b.cuda_event for a, b in self.events):
            raise RuntimeError("KernelTimer: event creation failed")
        self._start = (ctypes.c_void_p * capacity)(*[e[0].cuda_event for e in self.events])
        self._stop = (ctypes.c_void_p * capacity)(*[e[1].cuda_event for e in self.events])
        self._count = ctypes.c_int(0)
        self.capacity = capacity

    def __enter__(self):
        self._count.value = 0
        _check(_load().qlora_set_timing(self.kernel, self._start, self._stop, self.capacity,
                                        ctypes.byref(self._count)), "qlora_set_timing")
        return self

    def __exit__(self, *exc):
        _load().qlora_set_timing(self.kernel, None, None, 0, None)
        return False

    @property
    def count(self) -> int:
        return self._count.value

    def durations_ms(self) -> list:
        import torch

        torch.cuda.synchronize()
        return [self.events[i][0].elapsed_time(self.events[i][1]) for i in range(self.count)]


def qlora_status_str(status: int) -> str:
    return _load().qlora_status_str(status).decode()


# ---- quantised tensor ----------------------------------------------------------------

@dataclass
class NF4Tensor:
    """A quantised weight [rows][cols]: the device buffers of qlora_nf4."""

    rows: int
    cols: int
    codes: "torch.Tensor"     # uint8 [ceil(rows*cols/2)]
    absmax8: "torch.Tensor"   # uint8 [nb]
    scale2: "torch.Tensor"    # float32 [ng]
    mean: "torch.Tensor"      # float32 [1]
    qtype: int = 0            # qlora_qtype of the codes (QTYPES)
    absmax32: "torch.Tensor | None" = None  # float32 [nb] when stored without double quantisation

    @property
    def double_quant(self) -> bool:
        return self.absmax32 is None

    def struct(self) -> QNF4:
        if self.absmax32 is None:
            return QNF4(self.rows, self.cols, self.codes.data_ptr(), self.absmax8.data_ptr(),
                        self.scale2.data_ptr(), self.mean.data_ptr(), self.qtype, 0, None)
        return QNF4(self.rows, self.cols, self.codes.data_ptr(), None, None, None, self.qtype, 1,
                    self.absmax32.data_ptr())

    @staticmethod
    def empty(rows: int, cols: int, device="cuda", qtype: str | int = "nf4", double_quant: bool = True) -> "NF4Tensor":
        import torch

        s = qlora_quant_sizes(rows, cols)
        codes = torch.empty(max(s["codes"], 1), dtype=torch.uint8, device=device)
        if not double_quant:
            return NF4Tensor(rows, cols, codes, None, None, None, _qtype(qtype),
                             torch.empty(max(s["absmax8"], 1), dtype=torch.float32, device=device))
        return NF4Tensor(rows, cols, codes,
                         torch.empty(max(s["absmax8"], 1), dtype=torch.uint8, device=device),
                         torch.empty(max(s["scale2"] // 4, 1), dtype=torch.float32, device=device),
                         torch.empty(1, dtype=torch.float32, device=device), _qtype(qtype))


def _workspace(nbytes: int, device, ws=None):
    import torch

    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


@_on_stream
def qlora_quantize(W, out: NF4Tensor | None = None, workspace=None, stream=None, qtype: str | int = "nf4",
                   double_quant: bool = True) -> NF4Tensor:
    """NF4 + DQ quantisation of a [rows][cols] fp32 or bf16 device tensor (or another
    4-bit data type: ``qtype``; without double quantisation: ``double_quant=False``;
    an ``out`` tensor keeps its own settings)."""
    import torch

    if W.dim() != 2:
        raise ValueError("W must be 2-D [rows][cols]")
    rows, cols = W.shape
    if W.dtype == torch.float32:
        dt = QLORA_F32
    elif W.dtype == torch.bfloat16:
        dt = QLORA_BF16
    else:
        raise TypeError("W must be float32 or bfloat16")
    _need(W, W.dtype, (rows, cols), "W")
    q = out if out is not None else NF4Tensor.empty(rows, cols, W.device, qtype, double_quant)
    sizes = qlora_quant_sizes(rows, cols)
    ws = _workspace(sizes["workspace"], W.device, workspace)
    st = q.struct()
    _check(_load().qlora_quantize(_ptr(W), dt, ctypes.byref(st), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "qlora_quantize")
    return q


@_on_stream
def qlora_quantize_batch(Ws, outs=None, workspace=None, stream=None, qtype: str | int = "nf4",
                         double_quant: bool = True) -> list:
    """qlora_quantize of several [rows][cols] device tensors (all fp32 or all
    bf16) in one pass; returns their NF4Tensors (``outs`` keep their own
    settings)."""
    import torch

    Ws = list(Ws)
    n = len(Ws)
    if not 1 <= n <= QLORA_QUANT_BATCH_MAX:
        raise ValueError(f"1 to {QLORA_QUANT_BATCH_MAX} tensors per call")
    dt = {torch.float32: QLORA_F32, torch.bfloat16: QLORA_BF16}.get(Ws[0].dtype)
    if dt is None or any(W.dtype != Ws[0].dtype for W in Ws):
        raise TypeError("all tensors float32 or all bfloat16")
    for W in Ws:
        if W.dim() != 2:
            raise ValueError("each W must be 2-D [rows][cols]")
        if W.device != Ws[0].device:
            raise ValueError("all tensors of a batch on one device")
        _need(W, W.dtype, tuple(W.shape), "W")
    qs = list(outs) if outs is not None else [NF4Tensor.empty(W.shape[0], W.shape[1], W.device, qtype, double_quant)
                                              for W in Ws]
    if len(qs) != n:
        raise ValueError("one output per tensor")
    if any(q.codes.device != Ws[0].device for q in qs):
        raise ValueError("outputs on the inputs' device")
    ws = _workspace(qlora_quant_batch_workspace([tuple(W.shape) for W in Ws]), Ws[0].device, workspace)
    structs = [q.struct() for q in qs]
    sp = (ctypes.POINTER(QNF4) * n)(*[ctypes.pointer(st) for st in structs])
    wp = (ctypes.c_void_p * n)(*[W.data_ptr() for W in Ws])
    _check(_load().qlora_quantize_batch(n, wp, dt, sp, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qlora_quantize_batch")
    return qs


@_on_stream
def qlora_dequantize(q: NF4Tensor, out=None, stream=None):
    """doubleDequant to a bf16 [rows][cols] device tensor."""
    import torch

    y = out if out is not None else torch.empty((q.rows, q.cols), dtype=torch.bfloat16, device=q.codes.device)
    _need(y, torch.bfloat16, (q.rows, q.cols), "out")
    st = q.struct()
    _check(_load().qlora_dequantize(ctypes.byref(st), _ptr(y), _stream(stream)), "qlora_dequantize")
    return y


@_on_stream
def qlora_merge_adapters(q: NF4Tensor, L1, L2, scale: float, out=None, stream=None):
    """bf16 [N][K] = dequant(Wt) + s (L1 L2)^T, rounded once to bf16."""
    import torch

    K, r = L1.shape
    _need(L1, torch.bfloat16, (q.cols, r), "L1")
    _need(L2, torch.bfloat16, (r, q.rows), "L2")
    y = out if out is not None else torch.empty((q.rows, q.cols), dtype=torch.bfloat16, device=q.codes.device)
    _need(y, torch.bfloat16, (q.rows, q.cols), "out")
    st = q.struct()
    _check(_load().qlora_merge_adapters(ctypes.byref(st), _ptr(L1), _ptr(L2), r, float(scale), _ptr(y),
                                        _stream(stream)), "qlora_merge_adapters")
    return y


@_on_stream
def qlora_int8_quantize(X, block: int = 64, codes=None, absmax=None, stream=None):
    """Blockwise Int8 absmax codes of a contiguous fp32 or bf16 device tensor
    (flattened); returns (codes int8 [numel], absmax float32 [ceil(numel/block)])."""
    import torch

    if X.dtype == torch.float32:
        dt = QLORA_F32
    elif X.dtype == torch.bfloat16:
        dt = QLORA_BF16
    else:
        raise TypeError("X must be float32 or bfloat16")
    numel = X.numel()
    _need(X, X.dtype, tuple(X.shape), "X")
    nb = -(-numel // block) if block > 0 else 0
    codes = codes if codes is not None else torch.empty(numel, dtype=torch.int8, device=X.device)
    absmax = absmax if absmax is not None else torch.empty(nb, dtype=torch.float32, device=X.device)
    _need(codes, torch.int8, (numel,), "codes")
    _need(absmax, torch.float32, (nb,), "absmax")
    _check(_load().qlora_int8_quantize(_ptr(X), dt, numel, block, _ptr(codes), _ptr(absmax), _stream(stream)),
           "qlora_int8_quantize")
    return codes, absmax


@_on_stream
def qlora_int8_dequantize(codes, absmax, block: int = 64, dtype=None, out=None, stream=None):
    """x' = code * RN32(absmax / 127) as a flat float32 (default) or bfloat16 device tensor."""
    import torch

    dtype = torch.float32 if dtype is None else dtype
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("dtype must be float32 or bfloat16")
    numel = codes.numel()
    _need(codes, torch.int8, (numel,), "codes")
    _need(absmax, torch.float32, (-(-numel // block) if block > 0 else 0,), "absmax")
    y = out if out is not None else torch.empty(numel, dtype=dtype, device=codes.device)
    _need(y, dtype, (numel,), "out")
    dt = QLORA_F32 if dtype == torch.float32 else QLORA_BF16
    _check(_load().qlora_int8_dequantize(_ptr(codes), _ptr(absmax), numel, block, _ptr(y), dt, _stream(stream)),
           "qlora_int8_dequantize")
    return y


@_on_stream
def qlora_linear_fwd(q: NF4Tensor, X, L1, L2, scale: float, want_T: bool = False, Y=None, T_out=None,
                     workspace=None, stream=None, dropout=None):
    """Y = X dequant(Wt)^T + s (X L1) L2; returns (Y, T) with T = bf16(X L1) or None.
    ``dropout=(p, seed)`` applies LoRA dropout to the adapter branch's input."""
    import torch

    M, K = X.shape
    N = q.rows
    r = L1.shape[1]
    if K != q.cols:
        raise ValueError("X columns must equal the weight's in_features")
    _need(X, torch.bfloat16, (M, K), "X")
    _need(L1, torch.bfloat16, (K, r), "L1")
    _need(L2, torch.bfloat16, (r, N), "L2")
    Y = Y if Y is not None else torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, (M, N), "Y")
    if want_T and T_out is None:
        T_out = torch.empty((M, r), dtype=torch.bfloat16, device=X.device)
    if T_out is not None:
        _need(T_out, torch.bfloat16, (M, r), "T_out")
    st = q.struct()
    if dropout is None:
        ws = _workspace(qlora_linear_workspace(M, K, N, r), X.device, workspace)
        _check(_load().qlora_linear_fwd(ctypes.byref(st), _ptr(X), M, _ptr(L1), _ptr(L2), r, float(scale), _ptr(Y),
                                        _ptr(T_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
               "qlora_linear_fwd")
    else:
        p, seed = dropout
        ws = _workspace(qlora_linear_workspace_dropout(M, K, N, r), X.device, workspace)
        _check(_load().qlora_linear_fwd_dropout(ctypes.byref(st), _ptr(X), M, _ptr(L1), _ptr(L2), r, float(scale),
                                                float(p), int(seed), _ptr(Y), _ptr(T_out), _ptr(ws),
                                                ws.numel() * ws.element_size(), _stream(stream)),
               "qlora_linear_fwd_dropout")
    return Y, T_out


def qlora_linear_fwd_noalloc(q: NF4Tensor, X, L1, L2, scale: float, Y, T_out=None, stream=None):
    """Y = X dequant(Wt)^T + s (X L1) L2 for M <= 16 into the caller's Y (and
    T_out), with the library's own scratch: nothing is allocated here or in
    the library."""
    import torch

    M, K = X.shape
    N = q.rows
    r = L1.shape[1]
    if K != q.cols:
        raise ValueError("X columns must equal the weight's in_features")
    _need(X, torch.bfloat16, (M, K), "X")
    _need(L1, torch.bfloat16, (K, r), "L1")
    _need(L2, torch.bfloat16, (r, N), "L2")
    _need(Y, torch.bfloat16, (M, N), "Y")
    if T_out is not None:
        _need(T_out, torch.bfloat16, (M, r), "T_out")
    st = q.struct()
    _check(_load().qlora_linear_fwd_noalloc(ctypes.byref(st), _ptr(X), M, _ptr(L1), _ptr(L2), r, float(scale),
                                            _ptr(Y), _ptr(T_out), _stream(stream)), "qlora_linear_fwd_noalloc")
    return Y, T_out


@_on_stream
def qlora_linear_bwd(q: NF4Tensor, X, dY, L1, L2, scale: float, T=None, need_dX: bool = True,
                     grad_dtype=None, dX=None, dL1=None, dL2=None, workspace=None, stream=None, dropout=None):
    """Returns (dX or None, dL1, dL2) of the QLoRA linear for upstream gradient dY
    (``dropout=(p, seed)``: the same LoRA dropout as the forward)."""
    import torch

    grad_dtype = torch.float32 if grad_dtype is None else grad_dtype
    if grad_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("grad_dtype must be float32 or bfloat16")
    M, K = X.shape
    N = q.rows
    r = L1.shape[1]
    _need(X, torch.bfloat16, (M, K), "X")
    _need(dY, torch.bfloat16, (M, N), "dY")
    _need(L1, torch.bfloat16, (K, r), "L1")
    _need(L2, torch.bfloat16, (r, N), "L2")
    if T is not None:
        _need(T, torch.bfloat16, (M, r), "T")
    if need_dX:
        dX = dX if dX is not None else torch.empty((M, K), dtype=torch.bfloat16, device=X.device)
        _need(dX, torch.bfloat16, (M, K), "dX")
    else:
        dX = None
    dL1 = dL1 if dL1 is not None else torch.empty((K, r), dtype=grad_dtype, device=X.device)
    dL2 = dL2 if dL2 is not None else torch.empty((r, N), dtype=grad_dtype, device=X.device)
    _need(dL1, grad_dtype, (K, r), "dL1")
    _need(dL2, grad_dtype, (r, N), "dL2")
    st = q.struct()
    gd = QLORA_F32 if grad_dtype == torch.float32 else QLORA_BF16
    if dropout is None:
        ws = _workspace(qlora_linear_workspace(M, K, N, r), X.device, workspace)
        _check(_load().qlora_linear_bwd(ctypes.byref(st), _ptr(X), _ptr(dY), M, _ptr(L1), _ptr(L2), r,
                                        float(scale), _ptr(T), _ptr(dX), _ptr(dL1), _ptr(dL2), gd, _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)), "qlora_linear_bwd")
    else:
        p, seed = dropout
        ws = _workspace(qlora_linear_workspace_dropout(M, K, N, r), X.device, workspace)
        _check(_load().qlora_linear_bwd_dropout(ctypes.byref(st), _ptr(X), _ptr(dY), M, _ptr(L1), _ptr(L2), r,
                                                float(scale), float(p), int(seed), _ptr(T), _ptr(dX), _ptr(dL1),
                                                _ptr(dL2), gd, _ptr(ws), ws.numel() * ws.element_size(),
                                                _stream(stream)), "qlora_linear_bwd_dropout")
    return dX, dL1, dL2


# ---- helpers for moving numpy data (bf16 as uint16 bits) ------------------------------

def to_device_bf16(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bit patterns (host) -> bf16 device tensor, same bytes."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_host_bits(t) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
