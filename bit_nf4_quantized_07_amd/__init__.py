"""Python binding of libqlora.so, the gfx950 QLoRA NF4 linear-layer library.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in include/qlora.h.  PyTorch supplies device memory
and the current stream.  There is no CPU fallback: if the library is missing
or no GPU is visible, the compute calls raise.

    qw = quantize(W_fp32_cuda)                       # NF4 + double quant
    Y, T = linear_fwd(X, qw, A, B, alpha)            # bf16 tensors on cuda
    dX, dA, dB = linear_bwd(dY, X, qw, A, B, alpha, T)
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_LAUNCH, ERR_ARG = (
    0, -1, -2, -3, -4, -5, -6, -7)
ERR_SCRATCH = -8
NOALLOC_SCRATCH_BYTES = 64 << 20
BWD_ACCUMULATE_DX = 1
BLOCKSIZE = 64
DQ_BLOCKSIZE = 256

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float

KERNEL_FWD_GEMM, KERNEL_DX_GEMM, KERNEL_GEMV, KERNEL_DX_DEQUANT, KERNEL_FWD_DEQUANT = 1, 2, 3, 4, 5
KERNEL_COUNT = 6


class TimingC(ctypes.Structure):
    """struct qlora_timing of include/qlora.h: caller-owned hipEvent_t handles
    (as integers) recorded around the launches of kernel k = KERNEL_*."""
    _fields_ = [("start", ctypes.c_void_p * KERNEL_COUNT),
                ("stop", ctypes.c_void_p * KERNEL_COUNT)]


class LoraLinearC(ctypes.Structure):
    """struct qlora_lora_linear of include/qlora.h."""
    _fields_ = [("packed", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("mean", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("r", ctypes.c_int), ("alpha", ctypes.c_float)]


# name -> (restype, argtypes), mirroring include/qlora.h
SIGNATURES = {
    "nf4_quantize": (_I, [_P, _I64, _I64, _I, _P, _P, _P]),
    "double_quant": (_I, [_P, _I64, _I, _P, _P, _P, _P]),
    "nf4_dequant": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _I, _P, _P]),
    "qlora_linear_fwd": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _F, _P, _P,
                              _P, ctypes.c_size_t, _P]),
    "qlora_linear_bwd": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _F, _P,
                              _P, _P, _P, _I, _P, ctypes.c_size_t, _P]),
    "qlora_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I, _I]),
    "qlora_merge": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _I, _P, _P, _I, _F, _P, _P]),
    "qlora_linear_fwd_bf16": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _I, _F, _P, _P, _P,
                                   ctypes.c_size_t, _P]),
    "qlora_linear_bwd_bf16": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _I, _F, _P, _P, _P,
                                   _P, _I, _P, ctypes.c_size_t, _P]),
    "codebook_quantize": (_I, [_P, _I64, _I64, _I, _P, _P, _P, _P]),
    "codebook_dequant": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _I, _P, _P, _P]),
    "lora_dropout": (_I, [_P, _I64, _I64, ctypes.c_double, ctypes.c_uint64, _P, _P, _P]),
    "qlora_linear_fwd_dropout": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _F,
                                      _P, _P, _P, ctypes.c_size_t, _P]),
    "qlora_linear_bwd_dropout": (_I, [_P, _P, _P, ctypes.c_double, _I64, _I64, _I64, _P, _P, _P,
                                      _P, _P, _P, _I, _F, _P, _P, _P, _P, _I, _P,
                                      ctypes.c_size_t, _P]),
    "qlora_mlp_fwd": (_I, [_P, _I64, _I64, _I64, ctypes.POINTER(LoraLinearC),
                           ctypes.POINTER(LoraLinearC), _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                           _P]),
    "qlora_mlp_bwd": (_I, [_P, _P, _I64, _I64, _I64, ctypes.POINTER(LoraLinearC),
                           ctypes.POINTER(LoraLinearC), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                           _P, _I, _P, ctypes.c_size_t, _P]),
    "silu_mul_fwd": (_I, [_P, _P, _I64, _P, _P]),
    "silu_mul_bwd": (_I, [_P, _P, _P, _I64, _P, _P, _P]),
    "nf4_codebook": (_I, [_P]),
    "dq_codebook": (_I, [_P, ctypes.POINTER(_I)]),
    "qlora_strerror": (ctypes.c_char_p, [_I]),
    "qlora_version": (_I, []),
    "double_quant_table": (_I, [_P, _I64, _I, _P, _I, _P, _P, _P, _P]),
    "absmax_dequant": (_I, [_P, _P, _P, _I64, _I, _P, _I, _P, _P]),
    "dequant_tables": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _I, _P, _P, _I, _P, _P]),
    "dq_float8_codebook": (_I, [_P, ctypes.POINTER(_I)]),
    "qlora_linear_bwd_noalloc": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _F,
                                      _P, _P, _P, _P, _I, _P]),
    "qlora_linear_fwd_timed": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _F, _P,
                                    _P, _P, ctypes.c_size_t, _P, ctypes.POINTER(TimingC)]),
    "qlora_linear_bwd_timed": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I, _F,
                                    _P, _P, _P, _P, _I, _P, ctypes.c_size_t, _P,
                                    ctypes.POINTER(TimingC)]),
}

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libqlora.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m bit_nf4_quantized_07_amd.build`")
    try:  # make sure torch's HIP runtime is the one in the process
        import torch  # noqa: F401
    except Exception:
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


class QLoRAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load_library().qlora_strerror(status).decode()
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


def _check(fn: str, status: int):
    if status != OK:
        raise QLoRAError(fn, status)


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device=None) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


class _Checker:
    """Validation of every tensor a call hands to the library (inputs and
    outputs): the kernels size their buffer ranges from the call's sizes, not
    from the tensors, so a tensor of the wrong dtype, shape or layout would be
    read or written out of bounds.  Dtypes, shapes and contiguity are checked
    as tensors are named; `device()` then checks that all of them live on one
    HIP device and returns it.  Everything raises ValueError before any
    launch."""

    def __init__(self):
        self.seen = []

    def __call__(self, name, t, dtype, shape):
        torch = _torch()
        if t is None:
            raise ValueError(f"{name}: missing")
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name}: not a tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: not contiguous")
        self.seen.append((name, t))
        return t

    def opt(self, name, t, dtype, shape):
        return None if t is None else self(name, t, dtype, shape)

    def mat(self, name, t, dtype):
        """A 2-D tensor of any shape; returns its shape."""
        torch = _torch()
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name}: a 2-D tensor")
        self(name, t, dtype, tuple(t.shape))
        return tuple(t.shape)

    def weight(self, qw):
        """The stored NF4 weight of a QuantizedWeight."""
        torch = _torch()
        nb = qw.N * qw.K // BLOCKSIZE
        self("packed", qw.packed, torch.uint8, (qw.N * qw.K // 2,))
        self("codes", qw.codes, torch.uint8, (nb,))
        self("scales", qw.scales, torch.float32, ((nb + DQ_BLOCKSIZE - 1) // DQ_BLOCKSIZE,))
        self("mean", qw.mean, torch.float32, (1,))

    def base(self, qw, K):
        """The base weight of a linear (a QuantizedWeight or a bf16 [N, K]
        tensor); returns N."""
        torch = _torch()
        if isinstance(qw, QuantizedWeight):
            if qw.K != K:
                raise ValueError(f"weight has K={qw.K}, activations K={K}")
            self.weight(qw)
            return qw.N
        if not isinstance(qw, torch.Tensor) or qw.dim() != 2:
            raise ValueError("base weight: a QuantizedWeight or a bf16 [N, K] tensor")
        self("W", qw, torch.bfloat16, (qw.shape[0], K))
        return qw.shape[0]

    def adapters(self, A, B, N, K):
        """bf16 A [r, K] and B [N, r]; returns r."""
        torch = _torch()
        if not isinstance(A, torch.Tensor) or A.dim() != 2:
            raise ValueError("A: a bf16 [r, K] tensor")
        r = A.shape[0]
        self("A", A, torch.bfloat16, (r, K))
        self("B", B, torch.bfloat16, (N, r))
        return r

    def mask(self, mask, M, K):
        torch = _torch()
        nw = (M * K + 31) // 32
        if not isinstance(mask, torch.Tensor) or mask.dim() != 1 or mask.numel() < nw:
            raise ValueError(f"mask: a 1-D int32 tensor of at least {nw} words")
        self("mask", mask, torch.int32, tuple(mask.shape))

    def device(self):
        dev = None
        for name, t in self.seen:
            if not t.is_cuda:
                raise ValueError(f"{name}: not on a CUDA (HIP) device")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name}: on {t.device}, expected {dev}")
        return dev


class QuantizedWeight(NamedTuple):
    """NF4 base weight [N, K] with double-quantised block constants."""
    packed: "object"   # uint8 [N*K/2]
    codes: "object"    # uint8 [N*K/64]
    scales: "object"   # fp32  [ceil(N*K/64/256)]
    mean: "object"     # fp32  [1]
    N: int
    K: int

    def nbytes(self) -> int:
        return (self.packed.numel() + self.codes.numel() + 4 * self.scales.numel()
                + 4 * self.mean.numel())


def nf4_quantize(W):
    """W fp32 [N, K] (cuda) -> (packed uint8 [N*K/2], absmax fp32 [N*K/64])."""
    torch = _torch()
    chk = _Checker()
    N, K = chk.mat("W", W, torch.float32)
    dev = chk.device()
    packed = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
    absmax = torch.empty(max(N * K // BLOCKSIZE, 1), dtype=torch.float32, device=dev)
    _check("nf4_quantize", load_library().nf4_quantize(
        _ptr(W), N, K, BLOCKSIZE, _ptr(packed), _ptr(absmax), _stream(dev)))
    return packed, absmax


def double_quant(absmax):
    """absmax fp32 [nb] -> (codes uint8 [nb], scales fp32 [ceil(nb/256)], mean fp32 [1])."""
    torch = _torch()
    chk = _Checker()
    if not isinstance(absmax, torch.Tensor) or absmax.dim() != 1:
        raise ValueError("absmax: a 1-D fp32 tensor")
    chk("absmax", absmax, torch.float32, tuple(absmax.shape))
    dev = chk.device()
    nb = absmax.numel()
    codes = torch.empty(nb, dtype=torch.uint8, device=dev)
    scales = torch.empty((nb + DQ_BLOCKSIZE - 1) // DQ_BLOCKSIZE, dtype=torch.float32, device=dev)
    mean = torch.empty(4, dtype=torch.float32, device=dev)[:1]
    _check("double_quant", load_library().double_quant(
        _ptr(absmax), nb, DQ_BLOCKSIZE, _ptr(codes), _ptr(scales), _ptr(mean), _stream(dev)))
    return codes, scales, mean


def quantize(W) -> QuantizedWeight:
    """NF4 quantisation followed by double quantisation of the constants."""
    packed, absmax = nf4_quantize(W)
    codes, scales, mean = double_quant(absmax)
    return QuantizedWeight(packed, codes, scales, mean, W.shape[0], W.shape[1])


def nf4_dequant(qw: QuantizedWeight):
    """-> bf16 [N, K] dequantised weight."""
    torch = _torch()
    chk = _Checker()
    chk.weight(qw)
    dev = chk.device()
    out = torch.empty(qw.N, qw.K, dtype=torch.bfloat16, device=dev)
    _check("nf4_dequant", load_library().nf4_dequant(
        _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean), qw.N, qw.K,
        BLOCKSIZE, DQ_BLOCKSIZE, _ptr(out), _stream(dev)))
    return out


def merge(qw: QuantizedWeight, A, B, alpha: float, out=None):
    """-> bf16 [N, K]: bf16(w_hat + (alpha / r) B A), the adapter folded into
    the dequantised base (qlora_merge)."""
    torch = _torch()
    chk = _Checker()
    chk.weight(qw)
    r = chk.adapters(A, B, qw.N, qw.K)
    chk.opt("out", out, torch.bfloat16, (qw.N, qw.K))
    dev = chk.device()
    if out is None:
        out = torch.empty(qw.N, qw.K, dtype=torch.bfloat16, device=dev)
    _check("qlora_merge", load_library().qlora_merge(
        _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean), qw.N, qw.K,
        BLOCKSIZE, DQ_BLOCKSIZE, _ptr(A), _ptr(B), r, float(alpha), _ptr(out), _stream(dev)))
    return out


def workspace_bytes(M: int, K: int, N: int, r: int, backward: bool) -> int:
    return int(load_library().qlora_workspace_bytes(M, K, N, r, 1 if backward else 0))


class Workspace:
    """A reusable device workspace that grows on demand.

    Every buffer it hands out is marked as used by the stream of the call
    (`record_stream`), so that when it grows, the caching allocator does not
    hand the old memory to anyone before the work queued on that stream is
    done.  Calls that share one Workspace must still be ordered (one stream,
    or events): the library writes scratch data into it."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, stream=None):
        torch = _torch()
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        if stream is not None:
            self.buf.record_stream(stream)
        return self.buf, self.buf.numel()


# One default workspace per (device, stream): calls on different streams
# never share scratch memory.
_default_ws = {}


def default_workspace(device, stream) -> Workspace:
    """The workspace calls on `stream` (a torch stream) of `device` use when
    the caller passes none: one per (device, stream)."""
    torch = _torch()
    key = (str(torch.device(device)), int(stream.cuda_stream))
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def _ws(device, nbytes, workspace=None):
    stream = _torch().cuda.current_stream(device)
    ws = workspace if workspace is not None else default_workspace(device, stream)
    return ws.get(nbytes, stream)


def linear_fwd(X, qw, A, B, alpha: float, save_T: bool = True,
               out=None, T_out=None, workspace=None, timing: Optional[TimingC] = None):
    """Y = X W_hat^T + (alpha/r) (X A^T) B^T.  Returns (Y, T or None).

    `qw` is a QuantizedWeight (NF4, qlora_linear_fwd) or a bf16 tensor [N, K]
    (unquantised base, qlora_linear_fwd_bf16).  `timing` (NF4 base only): a
    TimingC whose events the library records around its dominant launch."""
    torch = _torch()
    chk = _Checker()
    M, K = chk.mat("X", X, torch.bfloat16)
    N = chk.base(qw, K)
    r = chk.adapters(A, B, N, K)
    chk.opt("out", out, torch.bfloat16, (M, N))
    chk.opt("T_out", T_out, torch.bfloat16, (M, r))
    dev = chk.device()
    Y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    T = T_out if T_out is not None else (
        torch.empty(M, r, dtype=torch.bfloat16, device=dev) if save_T else None)
    nb = workspace_bytes(M, K, N, r, False)
    ws, wsb = _ws(dev, nb, workspace)
    lib = load_library()
    if isinstance(qw, QuantizedWeight):
        args = (_ptr(X), M, K, N, _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales),
                _ptr(qw.mean), _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(T), _ptr(ws), wsb,
                _stream(dev))
        if timing is None:
            _check("qlora_linear_fwd", lib.qlora_linear_fwd(*args))
        else:
            _check("qlora_linear_fwd_timed", lib.qlora_linear_fwd_timed(*args, ctypes.byref(timing)))
    else:
        if timing is not None:
            raise ValueError("timing is supported on the NF4 base only")
        _check("qlora_linear_fwd_bf16", lib.qlora_linear_fwd_bf16(
            _ptr(X), M, K, N, _ptr(qw), _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(T),
            _ptr(ws), wsb, _stream(dev)))
    return Y, T


def _bwd_outputs(chk, M, K, N, r, need_dX, accumulate_into, dX_out, dA_out, dB_out):
    """Checks the caller's output tensors; returns them with the flags and a
    function that allocates the missing ones on the call's device."""
    torch = _torch()
    flags = 0
    if accumulate_into is not None:
        dX = chk("dX", accumulate_into, torch.bfloat16, (M, K))
        flags |= BWD_ACCUMULATE_DX
    else:
        dX = chk.opt("dX", dX_out, torch.bfloat16, (M, K))
    chk.opt("dA", dA_out, torch.float32, (r, K))
    chk.opt("dB", dB_out, torch.float32, (N, r))

    def alloc(dev):
        x = dX if dX is not None else (
            torch.empty(M, K, dtype=torch.bfloat16, device=dev) if need_dX else None)
        a = dA_out if dA_out is not None else torch.empty(r, K, dtype=torch.float32, device=dev)
        b = dB_out if dB_out is not None else torch.empty(N, r, dtype=torch.float32, device=dev)
        return x, a, b
    return flags, alloc


def linear_bwd(dY, X, qw, A, B, alpha: float, T=None, need_dX: bool = True,
               accumulate_into=None, dX_out=None, dA_out=None, dB_out=None, workspace=None,
               timing: Optional[TimingC] = None):
    """Returns (dX bf16 [M,K] or None, dA fp32 [r,K], dB fp32 [N,r]).  `qw` as in
    linear_fwd (QuantizedWeight or a bf16 [N, K] tensor)."""
    torch = _torch()
    chk = _Checker()
    M, K = chk.mat("X", X, torch.bfloat16)
    N = chk.base(qw, K)
    r = chk.adapters(A, B, N, K)
    chk("dY", dY, torch.bfloat16, (M, N))
    chk.opt("T", T, torch.bfloat16, (M, r))
    flags, alloc = _bwd_outputs(chk, M, K, N, r, need_dX, accumulate_into, dX_out, dA_out, dB_out)
    dev = chk.device()
    dX, dA, dB = alloc(dev)
    nb = workspace_bytes(M, K, N, r, True)
    ws, wsb = _ws(dev, nb, workspace)
    lib = load_library()
    if isinstance(qw, QuantizedWeight):
        args = (_ptr(dY), _ptr(X), M, K, N, _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales),
                _ptr(qw.mean), _ptr(A), _ptr(B), r, float(alpha), _ptr(T), _ptr(dX), _ptr(dA),
                _ptr(dB), flags, _ptr(ws), wsb, _stream(dev))
        if timing is None:
            _check("qlora_linear_bwd", lib.qlora_linear_bwd(*args))
        else:
            _check("qlora_linear_bwd_timed", lib.qlora_linear_bwd_timed(*args, ctypes.byref(timing)))
    else:
        if timing is not None:
            raise ValueError("timing is supported on the NF4 base only")
        _check("qlora_linear_bwd_bf16", lib.qlora_linear_bwd_bf16(
            _ptr(dY), _ptr(X), M, K, N, _ptr(qw), _ptr(A), _ptr(B), r, float(alpha), _ptr(T),
            _ptr(dX), _ptr(dA), _ptr(dB), flags, _ptr(ws), wsb, _stream(dev)))
    return dX, dA, dB


def _levels(levels):
    vals = [float(v) for v in levels]
    if len(vals) != 16:
        raise ValueError("a 4-bit codebook has 16 levels")
    return (ctypes.c_float * 16)(*vals)


def codebook_quantize(W, levels):
    """Blockwise quantisation of W fp32 [N, K] onto a 16-level codebook (host
    sequence, ascending) -> (packed uint8 [N*K/2], absmax fp32 [N*K/64])."""
    torch = _torch()
    chk = _Checker()
    N, K = chk.mat("W", W, torch.float32)
    dev = chk.device()
    packed = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
    absmax = torch.empty(max(N * K // BLOCKSIZE, 1), dtype=torch.float32, device=dev)
    lv = _levels(levels)
    _check("codebook_quantize", load_library().codebook_quantize(
        _ptr(W), N, K, BLOCKSIZE, ctypes.cast(lv, _P), _ptr(packed), _ptr(absmax), _stream(dev)))
    return packed, absmax


def quantize_with_codebook(W, levels) -> QuantizedWeight:
    """codebook_quantize followed by double quantisation of the constants."""
    packed, absmax = codebook_quantize(W, levels)
    codes, scales, mean = double_quant(absmax)
    return QuantizedWeight(packed, codes, scales, mean, W.shape[0], W.shape[1])


def codebook_dequant(qw: QuantizedWeight, levels):
    """-> bf16 [N, K] dequantised with the given 16-level codebook."""
    torch = _torch()
    chk = _Checker()
    chk.weight(qw)
    dev = chk.device()
    out = torch.empty(qw.N, qw.K, dtype=torch.bfloat16, device=dev)
    lv = _levels(levels)
    _check("codebook_dequant", load_library().codebook_dequant(
        _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean), qw.N, qw.K,
        BLOCKSIZE, DQ_BLOCKSIZE, ctypes.cast(lv, _P), _ptr(out), _stream(dev)))
    return out


def dropout(X, p: float, seed: int, Xd_out=None, mask_out=None):
    """LoRA dropout of the adapter input: -> (Xd bf16 [M, K], mask int32
    [M*K/32], bit i % 32 of word i // 32 = element i kept)."""
    torch = _torch()
    chk = _Checker()
    M, K = chk.mat("X", X, torch.bfloat16)
    chk.opt("Xd", Xd_out, torch.bfloat16, (M, K))
    if mask_out is not None:
        chk.mask(mask_out, M, K)
    dev = chk.device()
    nw = (M * K + 31) // 32
    Xd = Xd_out if Xd_out is not None else torch.empty_like(X)
    mask = mask_out if mask_out is not None else torch.empty(max(nw, 4), dtype=torch.int32,
                                                             device=dev)
    _check("lora_dropout", load_library().lora_dropout(
        _ptr(X), M, K, float(p), int(seed) & (2**64 - 1), _ptr(Xd), _ptr(mask), _stream(dev)))
    return Xd, mask[:nw]


def linear_fwd_dropout(X, Xd, qw: QuantizedWeight, A, B, alpha: float, save_T: bool = True,
                       out=None, T_out=None, workspace=None):
    """Y = X W_hat^T + (alpha/r) (Xd A^T) B^T with Xd the dropped adapter
    input.  Returns (Y, T = Xd A^T or None)."""
    torch = _torch()
    chk = _Checker()
    M, K = chk.mat("X", X, torch.bfloat16)
    chk("Xd", Xd, torch.bfloat16, (M, K))
    if not isinstance(qw, QuantizedWeight):
        raise ValueError("the dropout path takes an NF4 QuantizedWeight")
    N = chk.base(qw, K)
    r = chk.adapters(A, B, N, K)
    chk.opt("out", out, torch.bfloat16, (M, N))
    chk.opt("T_out", T_out, torch.bfloat16, (M, r))
    dev = chk.device()
    Y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    T = T_out if T_out is not None else (
        torch.empty(M, r, dtype=torch.bfloat16, device=dev) if save_T else None)
    nb = workspace_bytes(M, K, N, r, False)
    ws, wsb = _ws(dev, nb, workspace)
    _check("qlora_linear_fwd_dropout", load_library().qlora_linear_fwd_dropout(
        _ptr(X), _ptr(Xd), M, K, N, _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales),
        _ptr(qw.mean), _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(T), _ptr(ws), wsb,
        _stream(dev)))
    return Y, T


def linear_bwd_dropout(dY, Xd, mask, p: float, qw: QuantizedWeight, A, B, alpha: float, T=None,
                       need_dX: bool = True, accumulate_into=None, dX_out=None, dA_out=None,
                       dB_out=None, workspace=None):
    """Backward of linear_fwd_dropout (mask and p from `dropout`).  Returns
    (dX bf16 or None, dA fp32 [r, K], dB fp32 [N, r])."""
    torch = _torch()
    chk = _Checker()
    M, K = chk.mat("Xd", Xd, torch.bfloat16)
    if not isinstance(qw, QuantizedWeight):
        raise ValueError("the dropout path takes an NF4 QuantizedWeight")
    N = chk.base(qw, K)
    r = chk.adapters(A, B, N, K)
    chk("dY", dY, torch.bfloat16, (M, N))
    chk.mask(mask, M, K)
    chk.opt("T", T, torch.bfloat16, (M, r))
    flags, alloc = _bwd_outputs(chk, M, K, N, r, need_dX, accumulate_into, dX_out, dA_out, dB_out)
    dev = chk.device()
    dX, dA, dB = alloc(dev)
    nb = workspace_bytes(M, K, N, r, True)
    ws, wsb = _ws(dev, nb, workspace)
    _check("qlora_linear_bwd_dropout", load_library().qlora_linear_bwd_dropout(
        _ptr(dY), _ptr(Xd), _ptr(mask), float(p), M, K, N, _ptr(qw.packed), _ptr(qw.codes),
        _ptr(qw.scales), _ptr(qw.mean), _ptr(A), _ptr(B), r, float(alpha), _ptr(T), _ptr(dX),
        _ptr(dA), _ptr(dB), flags, _ptr(ws), wsb, _stream(dev)))
    return dX, dA, dB


def _lora_linear(chk, lin, K) -> LoraLinearC:
    qw, A, B, alpha = lin
    if not isinstance(qw, QuantizedWeight):
        raise ValueError("MLP projections take NF4 QuantizedWeights")
    N = chk.base(qw, K)
    chk.adapters(A, B, N, K)
    return LoraLinearC(_ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean),
                       _ptr(A), _ptr(B), A.shape[0], float(alpha))


def mlp_fwd(X, gate, up, out=None, workspace=None):
    """Gate/up projections of a SiLU-gated MLP and the gating in one call.
    gate, up: (QuantizedWeight [I, K], A, B, alpha).  Returns
    (G, U, H, Tg, Tu), bf16; `out` may hold preallocated tensors of the same
    names (a dict)."""
    torch = _torch()
    chk = _Checker()
    M, K = chk.mat("X", X, torch.bfloat16)
    I = gate[0].N
    if up[0].N != I:
        raise ValueError("gate and up weights differ in shape")
    lg, lu = _lora_linear(chk, gate, K), _lora_linear(chk, up, K)
    rg, ru = gate[1].shape[0], up[1].shape[0]
    out = out or {}
    cols = dict(G=I, U=I, H=I, Tg=rg, Tu=ru)
    for name, c in cols.items():
        chk.opt(name, out.get(name), torch.bfloat16, (M, c))
    dev = chk.device()
    t = {n: out[n] if out.get(n) is not None else
         torch.empty(M, c, dtype=torch.bfloat16, device=dev) for n, c in cols.items()}
    nb = max(workspace_bytes(M, K, I, rg, False), workspace_bytes(M, K, I, ru, False))
    ws, wsb = _ws(dev, nb, workspace)
    _check("qlora_mlp_fwd", load_library().qlora_mlp_fwd(
        _ptr(X), M, K, I, ctypes.byref(lg), ctypes.byref(lu), _ptr(t["G"]), _ptr(t["U"]),
        _ptr(t["H"]), _ptr(t["Tg"]), _ptr(t["Tu"]), _ptr(ws), wsb, _stream(dev)))
    return t["G"], t["U"], t["H"], t["Tg"], t["Tu"]


def mlp_bwd(dH, X, gate, up, G, U, Tg, Tu, accumulate_into=None, workspace=None):
    """Backward of mlp_fwd from dH.  Returns (dX, (dAg, dBg), (dAu, dBu), dG, dU)."""
    torch = _torch()
    chk = _Checker()
    M, K = chk.mat("X", X, torch.bfloat16)
    I = gate[0].N
    if up[0].N != I:
        raise ValueError("gate and up weights differ in shape")
    lg, lu = _lora_linear(chk, gate, K), _lora_linear(chk, up, K)
    rg, ru = gate[1].shape[0], up[1].shape[0]
    for name, tt, c in (("dH", dH, I), ("G", G, I), ("U", U, I), ("Tg", Tg, rg), ("Tu", Tu, ru)):
        chk(name, tt, torch.bfloat16, (M, c))
    chk.opt("dX", accumulate_into, torch.bfloat16, (M, K))
    dev = chk.device()
    dG, dU = torch.empty_like(G), torch.empty_like(U)
    flags = 0
    if accumulate_into is not None:
        dX = accumulate_into
        flags |= BWD_ACCUMULATE_DX
    else:
        dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    f32 = lambda *s: torch.empty(*s, dtype=torch.float32, device=dev)
    dAg, dBg, dAu, dBu = f32(rg, K), f32(I, rg), f32(ru, K), f32(I, ru)
    nb = max(workspace_bytes(M, K, I, rg, True), workspace_bytes(M, K, I, ru, True))
    ws, wsb = _ws(dev, nb, workspace)
    _check("qlora_mlp_bwd", load_library().qlora_mlp_bwd(
        _ptr(dH), _ptr(X), M, K, I, ctypes.byref(lg), ctypes.byref(lu), _ptr(G), _ptr(U),
        _ptr(Tg), _ptr(Tu), _ptr(dG), _ptr(dU), _ptr(dX), _ptr(dAg), _ptr(dBg), _ptr(dAu),
        _ptr(dBu), flags, _ptr(ws), wsb, _stream(dev)))
    return dX, (dAg, dBg), (dAu, dBu), dG, dU


def silu_mul_fwd(G, Up, out=None):
    torch = _torch()
    chk = _Checker()
    shape = tuple(G.shape)
    chk("G", G, torch.bfloat16, shape)
    chk("Up", Up, torch.bfloat16, shape)
    chk.opt("out", out, torch.bfloat16, shape)
    dev = chk.device()
    H = out if out is not None else torch.empty_like(G)
    _check("silu_mul_fwd", load_library().silu_mul_fwd(
        _ptr(G), _ptr(Up), G.numel(), _ptr(H), _stream(dev)))
    return H


def silu_mul_bwd(dH, G, Up):
    torch = _torch()
    chk = _Checker()
    shape = tuple(G.shape)
    chk("G", G, torch.bfloat16, shape)
    chk("dH", dH, torch.bfloat16, shape)
    chk("Up", Up, torch.bfloat16, shape)
    dev = chk.device()
    dG, dU = torch.empty_like(G), torch.empty_like(Up)
    _check("silu_mul_bwd", load_library().silu_mul_bwd(
        _ptr(dH), _ptr(G), _ptr(Up), G.numel(), _ptr(dG), _ptr(dU), _stream(dev)))
    return dG, dU


def codebook():
    """The 16 NF4 levels the kernels embed (host copy)."""
    buf = (ctypes.c_float * 16)()
    _check("nf4_codebook", load_library().nf4_codebook(ctypes.cast(buf, _P)))
    return list(buf)


def dq_float8_levels():
    """The 253 levels of the 8-bit-float second-level table (host copy)."""
    buf = (ctypes.c_float * 256)()
    n = _I(0)
    _check("dq_float8_codebook", load_library().dq_float8_codebook(ctypes.cast(buf, _P),
                                                                   ctypes.byref(n)))
    return list(buf)[: n.value]


def _levels8(levels):
    vals = [float(v) for v in levels]
    if not 2 <= len(vals) <= 256:
        raise ValueError("a second-level table has 2 to 256 levels")
    return (ctypes.c_float * len(vals))(*vals), len(vals)


def double_quant_table(absmax, levels):
    """double_quant with the given second-level table (host sequence,
    ascending) -> (codes uint8 [nb], scales fp32, mean fp32 [1])."""
    torch = _torch()
    chk = _Checker()
    if not isinstance(absmax, torch.Tensor) or absmax.dim() != 1:
        raise ValueError("absmax: a 1-D fp32 tensor")
    chk("absmax", absmax, torch.float32, tuple(absmax.shape))
    dev = chk.device()
    nb = absmax.numel()
    codes = torch.empty(nb, dtype=torch.uint8, device=dev)
    scales = torch.empty((nb + DQ_BLOCKSIZE - 1) // DQ_BLOCKSIZE, dtype=torch.float32, device=dev)
    mean = torch.empty(4, dtype=torch.float32, device=dev)[:1]
    lv, n = _levels8(levels)
    _check("double_quant_table", load_library().double_quant_table(
        _ptr(absmax), nb, DQ_BLOCKSIZE, ctypes.cast(lv, _P), n, _ptr(codes), _ptr(scales),
        _ptr(mean), _stream(dev)))
    return codes, scales, mean


def absmax_dequant(codes, scales, mean, levels):
    """-> fp32 [nb]: the decoded block constants fp32(fp32(levels[c] * s) + mean)."""
    torch = _torch()
    chk = _Checker()
    if not isinstance(codes, torch.Tensor) or codes.dim() != 1:
        raise ValueError("codes: a 1-D uint8 tensor")
    nb = codes.numel()
    chk("codes", codes, torch.uint8, (nb,))
    chk("scales", scales, torch.float32, ((nb + DQ_BLOCKSIZE - 1) // DQ_BLOCKSIZE,))
    chk("mean", mean, torch.float32, (1,))
    dev = chk.device()
    out = torch.empty(nb, dtype=torch.float32, device=dev)
    lv, n = _levels8(levels)
    _check("absmax_dequant", load_library().absmax_dequant(
        _ptr(codes), _ptr(scales), _ptr(mean), nb, DQ_BLOCKSIZE, ctypes.cast(lv, _P), n,
        _ptr(out), _stream(dev)))
    return out


def dequant_tables(qw: QuantizedWeight, levels8, levels4=None):
    """-> bf16 [N, K]: the weight dequantised with the given second-level table
    (and 4-bit codebook; None = NF4)."""
    torch = _torch()
    chk = _Checker()
    chk.weight(qw)
    dev = chk.device()
    out = torch.empty(qw.N, qw.K, dtype=torch.bfloat16, device=dev)
    lv8, n8 = _levels8(levels8)
    lv4 = None if levels4 is None else ctypes.cast(_levels(levels4), _P)
    _check("dequant_tables", load_library().dequant_tables(
        _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean), qw.N, qw.K, BLOCKSIZE,
        DQ_BLOCKSIZE, lv4, ctypes.cast(lv8, _P), n8, _ptr(out), _stream(dev)))
    return out


def dq_levels():
    buf = (ctypes.c_float * 256)()
    n = _I(0)
    _check("dq_codebook", load_library().dq_codebook(ctypes.cast(buf, _P), ctypes.byref(n)))
    return list(buf)[: n.value]
