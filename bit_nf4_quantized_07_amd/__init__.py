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
BWD_ACCUMULATE_DX = 1
BLOCKSIZE = 64
DQ_BLOCKSIZE = 256

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float

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
    "qlora_set_kernel_timer": (_I, [_I, _P, _P]),
}

KERNEL_FWD_GEMM, KERNEL_DX_GEMM, KERNEL_GEMV, KERNEL_DX_DEQUANT = 1, 2, 3, 4

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


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA (HIP) tensors")


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
    _need_cuda(W)
    N, K = W.shape
    packed = torch.empty(N * K // 2, dtype=torch.uint8, device=W.device)
    absmax = torch.empty(max(N * K // BLOCKSIZE, 1), dtype=torch.float32, device=W.device)
    _check("nf4_quantize", load_library().nf4_quantize(
        _ptr(W), N, K, BLOCKSIZE, _ptr(packed), _ptr(absmax), _stream(W.device)))
    return packed, absmax


def double_quant(absmax):
    """absmax fp32 [nb] -> (codes uint8 [nb], scales fp32 [ceil(nb/256)], mean fp32 [1])."""
    torch = _torch()
    _need_cuda(absmax)
    nb = absmax.numel()
    codes = torch.empty(nb, dtype=torch.uint8, device=absmax.device)
    scales = torch.empty((nb + DQ_BLOCKSIZE - 1) // DQ_BLOCKSIZE, dtype=torch.float32,
                         device=absmax.device)
    mean = torch.empty(4, dtype=torch.float32, device=absmax.device)[:1]
    _check("double_quant", load_library().double_quant(
        _ptr(absmax), nb, DQ_BLOCKSIZE, _ptr(codes), _ptr(scales), _ptr(mean),
        _stream(absmax.device)))
    return codes, scales, mean


def quantize(W) -> QuantizedWeight:
    """NF4 quantisation followed by double quantisation of the constants."""
    packed, absmax = nf4_quantize(W)
    codes, scales, mean = double_quant(absmax)
    return QuantizedWeight(packed, codes, scales, mean, W.shape[0], W.shape[1])


def nf4_dequant(qw: QuantizedWeight):
    """-> bf16 [N, K] dequantised weight."""
    torch = _torch()
    out = torch.empty(qw.N, qw.K, dtype=torch.bfloat16, device=qw.packed.device)
    _check("nf4_dequant", load_library().nf4_dequant(
        _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean), qw.N, qw.K,
        BLOCKSIZE, DQ_BLOCKSIZE, _ptr(out), _stream(out.device)))
    return out


def merge(qw: QuantizedWeight, A, B, alpha: float, out=None):
    """-> bf16 [N, K]: bf16(w_hat + (alpha / r) B A), the adapter folded into
    the dequantised base (qlora_merge)."""
    torch = _torch()
    _need_cuda(A, B)
    r = A.shape[0]
    if out is None:
        out = torch.empty(qw.N, qw.K, dtype=torch.bfloat16, device=qw.packed.device)
    _check("qlora_merge", load_library().qlora_merge(
        _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean), qw.N, qw.K,
        BLOCKSIZE, DQ_BLOCKSIZE, _ptr(A), _ptr(B), r, float(alpha), _ptr(out),
        _stream(out.device)))
    return out


def workspace_bytes(M: int, K: int, N: int, r: int, backward: bool) -> int:
    return int(load_library().qlora_workspace_bytes(M, K, N, r, 1 if backward else 0))


class Workspace:
    """A reusable device workspace that grows on demand."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        torch = _torch()
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf, self.buf.numel()


_default_ws = {}


def _ws(device, nbytes):
    key = str(device)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key].get(nbytes)


def _weight_rows(w) -> int:
    return w.N if isinstance(w, QuantizedWeight) else w.shape[0]


def linear_fwd(X, qw, A, B, alpha: float, save_T: bool = True,
               out=None, T_out=None, workspace=None):
    """Y = X W_hat^T + (alpha/r) (X A^T) B^T.  Returns (Y, T or None).

    `qw` is a QuantizedWeight (NF4, qlora_linear_fwd) or a bf16 tensor [N, K]
    (unquantised base, qlora_linear_fwd_bf16)."""
    torch = _torch()
    M, K = X.shape
    r = A.shape[0]
    N = _weight_rows(qw)
    _need_cuda(X, A, B)
    Y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=X.device)
    T = T_out if T_out is not None else (
        torch.empty(M, r, dtype=torch.bfloat16, device=X.device) if save_T else None)
    nb = workspace_bytes(M, K, N, r, False)
    ws, wsb = (workspace.get(nb) if workspace is not None else _ws(X.device, nb))
    lib = load_library()
    if isinstance(qw, QuantizedWeight):
        _check("qlora_linear_fwd", lib.qlora_linear_fwd(
            _ptr(X), M, K, N, _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean),
            _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(T), _ptr(ws), wsb, _stream(X.device)))
    else:
        _need_cuda(qw)
        _check("qlora_linear_fwd_bf16", lib.qlora_linear_fwd_bf16(
            _ptr(X), M, K, N, _ptr(qw), _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(T),
            _ptr(ws), wsb, _stream(X.device)))
    return Y, T


def linear_bwd(dY, X, qw, A, B, alpha: float, T=None, need_dX: bool = True,
               accumulate_into=None, dX_out=None, dA_out=None, dB_out=None, workspace=None):
    """Returns (dX bf16 [M,K] or None, dA fp32 [r,K], dB fp32 [N,r]).  `qw` as in
    linear_fwd (QuantizedWeight or a bf16 [N, K] tensor)."""
    torch = _torch()
    M, K = X.shape
    r = A.shape[0]
    N = _weight_rows(qw)
    _need_cuda(dY, X, A, B, T)
    flags = 0
    if accumulate_into is not None:
        dX = accumulate_into
        flags |= BWD_ACCUMULATE_DX
    elif dX_out is not None:
        dX = dX_out
    else:
        dX = torch.empty(M, K, dtype=torch.bfloat16, device=X.device) if need_dX else None
    dA = dA_out if dA_out is not None else torch.empty(r, K, dtype=torch.float32, device=X.device)
    dB = dB_out if dB_out is not None else torch.empty(N, r, dtype=torch.float32,
                                                       device=X.device)
    nb = workspace_bytes(M, K, N, r, True)
    ws, wsb = (workspace.get(nb) if workspace is not None else _ws(X.device, nb))
    lib = load_library()
    if isinstance(qw, QuantizedWeight):
        _check("qlora_linear_bwd", lib.qlora_linear_bwd(
            _ptr(dY), _ptr(X), M, K, N, _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales),
            _ptr(qw.mean), _ptr(A), _ptr(B), r, float(alpha), _ptr(T), _ptr(dX), _ptr(dA),
            _ptr(dB), flags, _ptr(ws), wsb, _stream(X.device)))
    else:
        _need_cuda(qw)
        _check("qlora_linear_bwd_bf16", lib.qlora_linear_bwd_bf16(
            _ptr(dY), _ptr(X), M, K, N, _ptr(qw), _ptr(A), _ptr(B), r, float(alpha), _ptr(T),
            _ptr(dX), _ptr(dA), _ptr(dB), flags, _ptr(ws), wsb, _stream(X.device)))
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
    _need_cuda(W)
    N, K = W.shape
    packed = torch.empty(N * K // 2, dtype=torch.uint8, device=W.device)
    absmax = torch.empty(max(N * K // BLOCKSIZE, 1), dtype=torch.float32, device=W.device)
    lv = _levels(levels)
    _check("codebook_quantize", load_library().codebook_quantize(
        _ptr(W), N, K, BLOCKSIZE, ctypes.cast(lv, _P), _ptr(packed), _ptr(absmax),
        _stream(W.device)))
    return packed, absmax


def quantize_with_codebook(W, levels) -> QuantizedWeight:
    """codebook_quantize followed by double quantisation of the constants."""
    packed, absmax = codebook_quantize(W, levels)
    codes, scales, mean = double_quant(absmax)
    return QuantizedWeight(packed, codes, scales, mean, W.shape[0], W.shape[1])


def codebook_dequant(qw: QuantizedWeight, levels):
    """-> bf16 [N, K] dequantised with the given 16-level codebook."""
    torch = _torch()
    out = torch.empty(qw.N, qw.K, dtype=torch.bfloat16, device=qw.packed.device)
    lv = _levels(levels)
    _check("codebook_dequant", load_library().codebook_dequant(
        _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean), qw.N, qw.K,
        BLOCKSIZE, DQ_BLOCKSIZE, ctypes.cast(lv, _P), _ptr(out), _stream(out.device)))
    return out


def dropout(X, p: float, seed: int, Xd_out=None, mask_out=None):
    """LoRA dropout of the adapter input: -> (Xd bf16 [M, K], mask int32
    [M*K/32], bit i % 32 of word i // 32 = element i kept)."""
    torch = _torch()
    _need_cuda(X, Xd_out, mask_out)
    M, K = X.shape
    Xd = Xd_out if Xd_out is not None else torch.empty_like(X)
    mask = mask_out if mask_out is not None else torch.empty(
        max((M * K + 31) // 32, 4), dtype=torch.int32, device=X.device)
    _check("lora_dropout", load_library().lora_dropout(
        _ptr(X), M, K, float(p), int(seed) & (2**64 - 1), _ptr(Xd), _ptr(mask), _stream(X.device)))
    return Xd, mask[:(M * K + 31) // 32]


def linear_fwd_dropout(X, Xd, qw: QuantizedWeight, A, B, alpha: float, save_T: bool = True,
                       out=None, T_out=None, workspace=None):
    """Y = X W_hat^T + (alpha/r) (Xd A^T) B^T with Xd the dropped adapter
    input.  Returns (Y, T = Xd A^T or None)."""
    torch = _torch()
    M, K = X.shape
    r = A.shape[0]
    _need_cuda(X, Xd, A, B)
    Y = out if out is not None else torch.empty(M, qw.N, dtype=torch.bfloat16, device=X.device)
    T = T_out if T_out is not None else (
        torch.empty(M, r, dtype=torch.bfloat16, device=X.device) if save_T else None)
    nb = workspace_bytes(M, K, qw.N, r, False)
    ws, wsb = (workspace.get(nb) if workspace is not None else _ws(X.device, nb))
    _check("qlora_linear_fwd_dropout", load_library().qlora_linear_fwd_dropout(
        _ptr(X), _ptr(Xd), M, K, qw.N, _ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales),
        _ptr(qw.mean), _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(T), _ptr(ws), wsb,
        _stream(X.device)))
    return Y, T


def linear_bwd_dropout(dY, Xd, mask, p: float, qw: QuantizedWeight, A, B, alpha: float, T=None,
                       need_dX: bool = True, accumulate_into=None, dX_out=None, dA_out=None,
                       dB_out=None, workspace=None):
    """Backward of linear_fwd_dropout (mask and p from `dropout`).  Returns
    (dX bf16 or None, dA fp32 [r, K], dB fp32 [N, r])."""
    torch = _torch()
    M, K = Xd.shape
    r = A.shape[0]
    _need_cuda(dY, Xd, mask, A, B, T)
    flags = 0
    if accumulate_into is not None:
        dX = accumulate_into
        flags |= BWD_ACCUMULATE_DX
    elif dX_out is not None:
        dX = dX_out
    else:
        dX = torch.empty(M, K, dtype=torch.bfloat16, device=Xd.device) if need_dX else None
    dA = dA_out if dA_out is not None else torch.empty(r, K, dtype=torch.float32, device=Xd.device)
    dB = dB_out if dB_out is not None else torch.empty(qw.N, r, dtype=torch.float32,
                                                       device=Xd.device)
    nb = workspace_bytes(M, K, qw.N, r, True)
    ws, wsb = (workspace.get(nb) if workspace is not None else _ws(Xd.device, nb))
    _check("qlora_linear_bwd_dropout", load_library().qlora_linear_bwd_dropout(
        _ptr(dY), _ptr(Xd), _ptr(mask), float(p), M, K, qw.N, _ptr(qw.packed), _ptr(qw.codes),
        _ptr(qw.scales), _ptr(qw.mean), _ptr(A), _ptr(B), r, float(alpha), _ptr(T), _ptr(dX),
        _ptr(dA), _ptr(dB), flags, _ptr(ws), wsb, _stream(Xd.device)))
    return dX, dA, dB


def _lora_linear(qw: QuantizedWeight, A, B, alpha: float) -> LoraLinearC:
    _need_cuda(A, B)
    return LoraLinearC(_ptr(qw.packed), _ptr(qw.codes), _ptr(qw.scales), _ptr(qw.mean),
                       _ptr(A), _ptr(B), A.shape[0], float(alpha))


def mlp_fwd(X, gate, up, out=None, workspace=None):
    """Gate/up projections of a SiLU-gated MLP and the gating in one call.
    gate, up: (QuantizedWeight [I, K], A, B, alpha).  Returns
    (G, U, H, Tg, Tu), bf16; `out` may hold preallocated tensors of the same
    names (a dict)."""
    torch = _torch()
    _need_cuda(X)
    M, K = X.shape
    qg, qu = gate[0], up[0]
    I = qg.N
    out = out or {}
    mk = lambda n, c: out[n] if n in out else torch.empty(M, c, dtype=torch.bfloat16,
                                                            device=X.device)
    G, U, H = mk("G", I), mk("U", I), mk("H", I)
    Tg, Tu = mk("Tg", gate[1].shape[0]), mk("Tu", up[1].shape[0])
    nb = max(workspace_bytes(M, K, I, gate[1].shape[0], False),
             workspace_bytes(M, K, I, up[1].shape[0], False))
    ws, wsb = (workspace.get(nb) if workspace is not None else _ws(X.device, nb))
    lg, lu = _lora_linear(*gate), _lora_linear(*up)
    _check("qlora_mlp_fwd", load_library().qlora_mlp_fwd(
        _ptr(X), M, K, I, ctypes.byref(lg), ctypes.byref(lu), _ptr(G), _ptr(U), _ptr(H), _ptr(Tg),
        _ptr(Tu), _ptr(ws), wsb, _stream(X.device)))
    return G, U, H, Tg, Tu


def mlp_bwd(dH, X, gate, up, G, U, Tg, Tu, accumulate_into=None, workspace=None):
    """Backward of mlp_fwd from dH.  Returns (dX, (dAg, dBg), (dAu, dBu), dG, dU)."""
    torch = _torch()
    _need_cuda(dH, X, G, U, Tg, Tu)
    M, K = X.shape
    qg, qu = gate[0], up[0]
    I = qg.N
    dG, dU = torch.empty_like(G), torch.empty_like(U)
    flags = 0
    if accumulate_into is not None:
        dX = accumulate_into
        flags |= BWD_ACCUMULATE_DX
    else:
        dX = torch.empty(M, K, dtype=torch.bfloat16, device=X.device)
    f32 = lambda *s: torch.empty(*s, dtype=torch.float32, device=X.device)
    rg, ru = gate[1].shape[0], up[1].shape[0]
    dAg, dBg, dAu, dBu = f32(rg, K), f32(I, rg), f32(ru, K), f32(I, ru)
    nb = max(workspace_bytes(M, K, I, rg, True), workspace_bytes(M, K, I, ru, True))
    ws, wsb = (workspace.get(nb) if workspace is not None else _ws(X.device, nb))
    lg, lu = _lora_linear(*gate), _lora_linear(*up)
    _check("qlora_mlp_bwd", load_library().qlora_mlp_bwd(
        _ptr(dH), _ptr(X), M, K, I, ctypes.byref(lg), ctypes.byref(lu), _ptr(G), _ptr(U),
        _ptr(Tg), _ptr(Tu), _ptr(dG), _ptr(dU), _ptr(dX), _ptr(dAg), _ptr(dBg), _ptr(dAu),
        _ptr(dBu), flags, _ptr(ws), wsb, _stream(X.device)))
    return dX, (dAg, dBg), (dAu, dBu), dG, dU


def silu_mul_fwd(G, Up, out=None):
    torch = _torch()
    _need_cuda(G, Up)
    H = out if out is not None else torch.empty_like(G)
    _check("silu_mul_fwd", load_library().silu_mul_fwd(
        _ptr(G), _ptr(Up), G.numel(), _ptr(H), _stream(G.device)))
    return H


def silu_mul_bwd(dH, G, Up):
    torch = _torch()
    _need_cuda(dH, G, Up)
    dG, dU = torch.empty_like(G), torch.empty_like(Up)
    _check("silu_mul_bwd", load_library().silu_mul_bwd(
        _ptr(dH), _ptr(G), _ptr(Up), G.numel(), _ptr(dG), _ptr(dU), _stream(G.device)))
    return dG, dU


def codebook():
    """The 16 NF4 levels the kernels embed (host copy)."""
    buf = (ctypes.c_float * 16)()
    _check("nf4_codebook", load_library().nf4_codebook(ctypes.cast(buf, _P)))
    return list(buf)


def dq_levels():
    buf = (ctypes.c_float * 256)()
    n = _I(0)
    _check("dq_codebook", load_library().dq_codebook(ctypes.cast(buf, _P), ctypes.byref(n)))
    return list(buf)[: n.value]
