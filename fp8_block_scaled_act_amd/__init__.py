"""Python binding of libfp8bs (FP8 e4m3 quantize-and-multiply path for MI355X).

Argument marshalling only: every step runs in the HIP kernels of
``libfp8bs.so`` (C ABI in ``include/fp8bs.h``). PyTorch provides device memory
and the current stream. There is no CPU fallback: if the library is missing
or cannot be loaded, every call raises.

Entry points (same names as the C ABI):
    fp8_act_quant_block(x)           -> (q, s)   x bf16 [M, K]; s fp32 [M, K/128]
    fp8_amax_quant_tensor(x)         -> (q, s)   any shape; s fp32 [1]
    fp8_gemm_blockscaled(a, sa, w, sw) -> c      c bf16 [M, N] = A . W^T
    fp8_weight_quant_block(w)        -> (q, s)   w bf16 [N, K]; s fp32 [N/128, K/128]
    fp8_act_quant_block_ue8m0, fp8_weight_quant_block_ue8m0, fp8_gemm_blockscaled_ue8m0:
                                     the same with power-of-two scales
    fp8_act_quant_block_f32(x)       -> (q, s)   x fp32 [M, K]
    fp8_gemm_tensorscaled(a, sa, w, sw) -> c     one scale per tensor (sa, sw [1])
``q`` tensors are ``torch.float8_e4m3fn`` (the OCP e4m3 "fn" bytes). Each
function also accepts preallocated outputs (``out=``) so that a caller can
time or graph-capture calls without allocations.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH",
    "lib",
    "Fp8bsError",
    "fp8_act_quant_block",
    "fp8_amax_quant_tensor",
    "fp8_amax_quant_tensor_workspace_bytes",
    "fp8_amax_quant_tensor_noalloc",
    "fp8_amax_tensor",
    "fp8_static_quant_tensor",
    "fp8_gemm_blockscaled",
    "fp8_gemm_blockscaled_workspace_bytes",
    "fp8_weight_quant_block",
    "fp8_act_quant_block_ue8m0",
    "fp8_weight_quant_block_ue8m0",
    "fp8_gemm_blockscaled_ue8m0",
    "fp8_act_quant_block_f32",
    "fp8_gemm_tensorscaled",
    "fp8_act_quant_gemm_blockscaled_workspace_bytes",
    "fp8_act_quant_gemm_blockscaled",
    "fp8_act_quant_block_tensor_workspace_bytes",
    "fp8_act_quant_block_tensor",
    "debug_encode_e4m3",
    "debug_mfma_block",
    "EXPORTED_SYMBOLS",
]

# the library built in this package directory (fp8_block_scaled_act_amd.build)
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8bs.so")

EXPORTED_SYMBOLS = (
    "fp8bs_status_string",
    "fp8_act_quant_block",
    "fp8_amax_quant_tensor_workspace_bytes",
    "fp8_amax_quant_tensor",
    "fp8_amax_quant_tensor_noalloc",
    "fp8_amax_tensor",
    "fp8_static_quant_tensor",
    "fp8_gemm_blockscaled_workspace_bytes",
    "fp8_gemm_blockscaled",
    "fp8_weight_quant_block",
    "fp8_act_quant_block_ue8m0",
    "fp8_weight_quant_block_ue8m0",
    "fp8_gemm_blockscaled_ue8m0",
    "fp8_act_quant_block_f32",
    "fp8_gemm_tensorscaled",
    "fp8_act_quant_gemm_blockscaled_workspace_bytes",
    "fp8_act_quant_gemm_blockscaled",
    "fp8_act_quant_block_tensor_workspace_bytes",
    "fp8_act_quant_block_tensor",
    "fp8bs_debug_encode_e4m3",
    "fp8bs_debug_mfma_block",
)

E4M3 = torch.float8_e4m3fn


class Fp8bsError(RuntimeError):
    """A non-zero status from libfp8bs."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfp8bs.so (once). Raises if it is missing: no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m fp8_block_scaled_act_amd.build`"
        )
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz, fp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    L.fp8bs_status_string.argtypes = [ctypes.c_int]
    L.fp8bs_status_string.restype = ctypes.c_char_p
    L.fp8_act_quant_block.argtypes = [vp, i64, i64, vp, fp, vp]
    L.fp8_act_quant_block.restype = ctypes.c_int
    L.fp8_amax_quant_tensor_workspace_bytes.argtypes = [i64]
    L.fp8_amax_quant_tensor_workspace_bytes.restype = sz
    L.fp8_amax_quant_tensor.argtypes = [vp, i64, vp, fp, vp, sz, vp]
    L.fp8_amax_quant_tensor.restype = ctypes.c_int
    L.fp8_amax_quant_tensor_noalloc.argtypes = [vp, i64, vp, fp, vp]
    L.fp8_amax_quant_tensor_noalloc.restype = ctypes.c_int
    L.fp8_amax_tensor.argtypes = [vp, i64, fp, fp, vp, sz, vp]
    L.fp8_amax_tensor.restype = ctypes.c_int
    L.fp8_static_quant_tensor.argtypes = [vp, i64, fp, vp, vp]
    L.fp8_static_quant_tensor.restype = ctypes.c_int
    L.fp8_gemm_blockscaled_workspace_bytes.argtypes = [i64, i64, i64]
    L.fp8_gemm_blockscaled_workspace_bytes.restype = sz
    L.fp8_gemm_blockscaled.argtypes = [vp, fp, vp, fp, vp, i64, i64, i64, vp, sz, vp]
    L.fp8_gemm_blockscaled.restype = ctypes.c_int
    L.fp8_weight_quant_block.argtypes = [vp, i64, i64, vp, fp, vp]
    L.fp8_weight_quant_block.restype = ctypes.c_int
    L.fp8_act_quant_block_ue8m0.argtypes = [vp, i64, i64, vp, fp, vp]
    L.fp8_act_quant_block_ue8m0.restype = ctypes.c_int
    L.fp8_weight_quant_block_ue8m0.argtypes = [vp, i64, i64, vp, fp, vp]
    L.fp8_weight_quant_block_ue8m0.restype = ctypes.c_int
    L.fp8_gemm_blockscaled_ue8m0.argtypes = [vp, fp, vp, fp, vp, i64, i64, i64, vp, sz, vp]
    L.fp8_gemm_blockscaled_ue8m0.restype = ctypes.c_int
    L.fp8_act_quant_block_f32.argtypes = [fp, i64, i64, vp, fp, vp]
    L.fp8_act_quant_block_f32.restype = ctypes.c_int
    L.fp8_gemm_tensorscaled.argtypes = [vp, fp, vp, fp, vp, i64, i64, i64, vp, sz, vp]
    L.fp8_gemm_tensorscaled.restype = ctypes.c_int
    L.fp8_act_quant_gemm_blockscaled_workspace_bytes.argtypes = [i64, i64, i64]
    L.fp8_act_quant_gemm_blockscaled_workspace_bytes.restype = sz
    L.fp8_act_quant_gemm_blockscaled.argtypes = [vp, vp, fp, vp, i64, i64, i64, vp, sz, vp]
    L.fp8_act_quant_gemm_blockscaled.restype = ctypes.c_int
    L.fp8_act_quant_block_tensor_workspace_bytes.argtypes = [i64, i64]
    L.fp8_act_quant_block_tensor_workspace_bytes.restype = sz
    L.fp8_act_quant_block_tensor.argtypes = [vp, i64, i64, vp, fp, vp, fp, vp, sz, vp]
    L.fp8_act_quant_block_tensor.restype = ctypes.c_int
    L.fp8bs_debug_encode_e4m3.argtypes = [fp, vp, i64, vp]
    L.fp8bs_debug_encode_e4m3.restype = ctypes.c_int
    L.fp8bs_debug_mfma_block.argtypes = [vp, vp, fp, i64, vp]
    L.fp8bs_debug_mfma_block.restype = ctypes.c_int
    _lib = L
    return L


def _check(fn: str, rc: int):
    if rc != 0:
        raise Fp8bsError(fn, rc, lib().fp8bs_status_string(rc).decode())


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (strided views are not supported)")


def _out(t, name: str, dtypes, shape, device):
    """A caller-supplied output: a contiguous tensor of one of ``dtypes``, of
    exactly ``shape``, on ``device`` (the kernels write all of it)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


_CODES = (E4M3, torch.uint8)
_F32 = (torch.float32,)
_BF16 = (torch.bfloat16,)


def _workspace(ws, need: int, device):
    """The workspace to pass: the caller's (a contiguous tensor on
    ``device``; its size in bytes is what the library is told) or a new one
    of ``need`` bytes; None when no workspace is needed and none was given."""
    if ws is None:
        return torch.empty((need,), dtype=torch.uint8, device=device) if need > 0 else None
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws


def _nbytes(ws) -> int:
    return ws.numel() * ws.element_size() if ws is not None else 0


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _act_quant(fn: str, x: torch.Tensor, out, dtype=torch.bfloat16):
    _need(x, "x", dtype)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    sshape = (M, K // 128 if K % 128 == 0 else 1)
    if out is None:
        q = torch.empty((M, K), dtype=E4M3, device=x.device)
        s = torch.empty(sshape, dtype=torch.float32, device=x.device)
    else:
        q, s = out
        _out(q, "q", _CODES, (M, K), x.device)
        _out(s, "scale", _F32, sshape, x.device)
    with torch.cuda.device(x.device):
        rc = getattr(lib(), fn)(_ptr(x), M, K, _ptr(q), _ptr(s), ctypes.c_void_p(_stream(x.device)))
    _check(fn, rc)
    return q, s


def fp8_act_quant_block(x: torch.Tensor, out=None):
    """1x128 block quantization of bf16 ``x`` [M, K] (K % 128 == 0)."""
    return _act_quant("fp8_act_quant_block", x, out)


def fp8_act_quant_block_ue8m0(x: torch.Tensor, out=None):
    """1x128 block quantization with power-of-two scales."""
    return _act_quant("fp8_act_quant_block_ue8m0", x, out)


def fp8_act_quant_block_f32(x: torch.Tensor, out=None):
    """1x128 block quantization of float32 ``x`` [M, K]."""
    return _act_quant("fp8_act_quant_block_f32", x, out, dtype=torch.float32)


def fp8_amax_quant_tensor_workspace_bytes(numel: int) -> int:
    return int(lib().fp8_amax_quant_tensor_workspace_bytes(int(numel)))


def fp8_amax_quant_tensor(x: torch.Tensor, out=None, workspace=None):
    """Per-tensor quantization of bf16 ``x`` (any shape) with an exact amax."""
    _need(x, "x", torch.bfloat16)
    numel = x.numel()
    if out is None:
        q = torch.empty(x.shape, dtype=E4M3, device=x.device)
        s = torch.empty((1,), dtype=torch.float32, device=x.device)
    else:
        q, s = out
        _out(q, "q", _CODES, x.shape, x.device)
        _out(s, "scale", _F32, (1,), x.device)
    wsb = fp8_amax_quant_tensor_workspace_bytes(numel) if numel > 0 else 0
    workspace = _workspace(workspace, wsb, x.device)
    with torch.cuda.device(x.device):
        rc = lib().fp8_amax_quant_tensor(
            _ptr(x), numel, _ptr(q), _ptr(s), _ptr(workspace), _nbytes(workspace),
            ctypes.c_void_p(_stream(x.device)))
    _check("fp8_amax_quant_tensor", rc)
    return q, s


def fp8_amax_tensor(x: torch.Tensor, out=None, workspace=None):
    """The amax stage alone: (amax, scale), one fp32 each, of bf16 ``x``."""
    _need(x, "x", torch.bfloat16)
    if out is None:
        amax = torch.empty((1,), dtype=torch.float32, device=x.device)
        s = torch.empty((1,), dtype=torch.float32, device=x.device)
    else:
        amax, s = out
        _out(amax, "amax", _F32, (1,), x.device)
        _out(s, "scale", _F32, (1,), x.device)
    numel = x.numel()
    wsb = fp8_amax_quant_tensor_workspace_bytes(numel) if numel > 0 else 0
    workspace = _workspace(workspace, wsb, x.device)
    with torch.cuda.device(x.device):
        rc = lib().fp8_amax_tensor(_ptr(x), numel, _ptr(amax), _ptr(s), _ptr(workspace), _nbytes(workspace),
                                   ctypes.c_void_p(_stream(x.device)))
    _check("fp8_amax_tensor", rc)
    return amax, s


def fp8_static_quant_tensor(x: torch.Tensor, scale: torch.Tensor, out=None):
    """Quantization of bf16 ``x`` (any shape) with a given scale: ``scale`` is
    a float32 tensor of one element on x's device (read by the kernel).
    Returns the e4m3 codes."""
    _need(x, "x", torch.bfloat16)
    _need(scale, "scale", torch.float32, x.device)
    if scale.numel() != 1:
        raise ValueError(f"scale must hold one element, got {scale.numel()}")
    if out is None:
        q = torch.empty(x.shape, dtype=E4M3, device=x.device)
    else:
        q = _out(out, "q", _CODES, x.shape, x.device)
    with torch.cuda.device(x.device):
        rc = lib().fp8_static_quant_tensor(_ptr(x), x.numel(), _ptr(scale), _ptr(q),
                                           ctypes.c_void_p(_stream(x.device)))
    _check("fp8_static_quant_tensor", rc)
    return q


def fp8_amax_quant_tensor_noalloc(x: torch.Tensor, out=None):
    """fp8_amax_quant_tensor with its scratch in the library's own device
    array: the C call allocates nothing (pass ``out`` to allocate nothing
    here either). Calls that overlap on one GPU race."""
    _need(x, "x", torch.bfloat16)
    if out is None:
        q = torch.empty(x.shape, dtype=E4M3, device=x.device)
        s = torch.empty((1,), dtype=torch.float32, device=x.device)
    else:
        q, s = out
        _out(q, "q", _CODES, x.shape, x.device)
        _out(s, "scale", _F32, (1,), x.device)
    with torch.cuda.device(x.device):
        rc = lib().fp8_amax_quant_tensor_noalloc(_ptr(x), x.numel(), _ptr(q), _ptr(s),
                                                 ctypes.c_void_p(_stream(x.device)))
    _check("fp8_amax_quant_tensor_noalloc", rc)
    return q, s


def fp8_act_quant_block_tensor_workspace_bytes(M: int, K: int) -> int:
    return int(lib().fp8_act_quant_block_tensor_workspace_bytes(M, K))


def fp8_act_quant_block_tensor(x: torch.Tensor, out=None, workspace=None):
    """Block and per-tensor quantization of the same bf16 ``x`` [M, K]:
    returns (q_block, block_scale, q_tensor, tensor_scale), bit for bit those
    of fp8_act_quant_block and fp8_amax_quant_tensor."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    sshape = (M, K // 128 if K % 128 == 0 else 1)
    if out is None:
        qb = torch.empty((M, K), dtype=E4M3, device=x.device)
        sb = torch.empty(sshape, dtype=torch.float32, device=x.device)
        qt = torch.empty((M, K), dtype=E4M3, device=x.device)
        st = torch.empty((1,), dtype=torch.float32, device=x.device)
    else:
        qb, sb, qt, st = out
        _out(qb, "q_block", _CODES, (M, K), x.device)
        _out(sb, "block_scale", _F32, sshape, x.device)
        _out(qt, "q_tensor", _CODES, (M, K), x.device)
        _out(st, "tensor_scale", _F32, (1,), x.device)
    wsb = fp8_act_quant_block_tensor_workspace_bytes(M, K)
    workspace = _workspace(workspace, wsb, x.device)
    fn = "fp8_act_quant_block_tensor"
    with torch.cuda.device(x.device):
        rc = getattr(lib(), fn)(_ptr(x), M, K, _ptr(qb), _ptr(sb), _ptr(qt), _ptr(st), _ptr(workspace),
                                _nbytes(workspace), ctypes.c_void_p(_stream(x.device)))
    _check(fn, rc)
    return qb, sb, qt, st


def fp8_gemm_blockscaled_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().fp8_gemm_blockscaled_workspace_bytes(int(M), int(N), int(K)))


def _as_u8(t):
    return t.view(torch.uint8) if t.dtype == E4M3 else t


def _gemm(fn, a, a_scale, w, w_scale, out, workspace, per_tensor=False):
    for t, n in ((a, "a"), (w, "w")):
        if t.dtype not in (E4M3, torch.uint8):
            raise TypeError(f"{n} must be float8_e4m3fn (or its uint8 bytes)")
    a, w = _as_u8(a), _as_u8(w)
    _need(a, "a", torch.uint8)
    _need(w, "w", torch.uint8, a.device)
    _need(a_scale, "a_scale", torch.float32, a.device)
    _need(w_scale, "w_scale", torch.float32, a.device)
    if a.dim() != 2 or w.dim() != 2 or a.shape[1] != w.shape[1]:
        raise ValueError("a must be [M, K] and w [N, K]")
    M, K = a.shape
    N = w.shape[0]
    if per_tensor:
        if a_scale.numel() != 1 or w_scale.numel() != 1:
            raise ValueError("a_scale and w_scale must hold one value each")
    elif a_scale.shape != (M, K // 128) or w_scale.shape != (N // 128, K // 128):
        raise ValueError("a_scale must be [M, K/128] and w_scale [N/128, K/128]")
    if out is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    else:
        c = _out(out, "out", _BF16, (M, N), a.device)
    wsb = fp8_gemm_blockscaled_workspace_bytes(M, N, K)
    workspace = _workspace(workspace, wsb, a.device)
    with torch.cuda.device(a.device):
        rc = getattr(lib(), fn)(
            _ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(c), M, N, K, _ptr(workspace),
            _nbytes(workspace), ctypes.c_void_p(_stream(a.device)))
    _check(fn, rc)
    return c


def fp8_gemm_blockscaled(a, a_scale, w, w_scale, out=None, workspace=None):
    """C = A . W^T (bf16 [M, N]) from e4m3 A [M, K] with 1x128 scales and e4m3
    W [N, K] with 128x128 scales."""
    return _gemm("fp8_gemm_blockscaled", a, a_scale, w, w_scale, out, workspace)


def fp8_gemm_blockscaled_ue8m0(a, a_scale, w, w_scale, out=None, workspace=None):
    """As fp8_gemm_blockscaled, for power-of-two scales (applied by the matrix cores)."""
    return _gemm("fp8_gemm_blockscaled_ue8m0", a, a_scale, w, w_scale, out, workspace)


def fp8_gemm_tensorscaled(a, a_scale, w, w_scale, out=None, workspace=None):
    """C = a_scale * w_scale * (A . W^T) (bf16 [M, N]); one fp32 scale per
    operand, as a one-element device tensor (fp8_amax_quant_tensor's output)."""
    return _gemm("fp8_gemm_tensorscaled", a, a_scale, w, w_scale, out, workspace, per_tensor=True)


def fp8_act_quant_gemm_blockscaled_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().fp8_act_quant_gemm_blockscaled_workspace_bytes(M, N, K))


def fp8_act_quant_gemm_blockscaled(x, w, w_scale, out=None, workspace=None):
    """C = A_q . W^T (bf16 [M, N]) where (A_q, a_scale) is the 1x128 block
    quantization of the bf16 activations x [M, K]; one kernel for decode
    batches (M <= 8), else act-quant and GEMM through the workspace."""
    _need(x, "x", torch.bfloat16)
    if w.dtype not in (E4M3, torch.uint8):
        raise TypeError("w must be float8_e4m3fn (or its uint8 bytes)")
    w = _as_u8(w)
    _need(w, "w", torch.uint8, x.device)
    _need(w_scale, "w_scale", torch.float32, x.device)
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [M, K] and w [N, K]")
    M, K = x.shape
    N = w.shape[0]
    if w_scale.shape != (N // 128, K // 128):
        raise ValueError("w_scale must be [N/128, K/128]")
    if out is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        c = _out(out, "out", _BF16, (M, N), x.device)
    wsb = fp8_act_quant_gemm_blockscaled_workspace_bytes(M, N, K)
    workspace = _workspace(workspace, wsb, x.device)
    fn = "fp8_act_quant_gemm_blockscaled"
    with torch.cuda.device(x.device):
        rc = getattr(lib(), fn)(
            _ptr(x), _ptr(w), _ptr(w_scale), _ptr(c), M, N, K, _ptr(workspace),
            _nbytes(workspace), ctypes.c_void_p(_stream(x.device)))
    _check(fn, rc)
    return c


def _weight_quant(fn, w: torch.Tensor, out):
    _need(w, "w", torch.bfloat16)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    N, K = w.shape
    sshape = (max(N // 128, 1), max(K // 128, 1))
    if out is None:
        q = torch.empty((N, K), dtype=E4M3, device=w.device)
        s = torch.empty(sshape, dtype=torch.float32, device=w.device)
    else:
        q, s = out
        _out(q, "q", _CODES, (N, K), w.device)
        _out(s, "scale", _F32, sshape, w.device)
    with torch.cuda.device(w.device):
        rc = getattr(lib(), fn)(_ptr(w), N, K, _ptr(q), _ptr(s), ctypes.c_void_p(_stream(w.device)))
    _check(fn, rc)
    return q, s


def fp8_weight_quant_block(w: torch.Tensor, out=None):
    """128x128 block quantization of a bf16 weight [N, K]."""
    return _weight_quant("fp8_weight_quant_block", w, out)


def fp8_weight_quant_block_ue8m0(w: torch.Tensor, out=None):
    """128x128 block quantization with power-of-two scales."""
    return _weight_quant("fp8_weight_quant_block_ue8m0", w, out)


def debug_encode_e4m3(v: torch.Tensor, out=None):
    """Test hook: the library's fp32 -> e4m3 rounding, elementwise."""
    _need(v, "v", torch.float32)
    o = torch.empty(v.shape, dtype=torch.uint8, device=v.device) if out is None else \
        _out(out, "out", (torch.uint8,), v.shape, v.device)
    with torch.cuda.device(v.device):
        rc = lib().fp8bs_debug_encode_e4m3(_ptr(v), _ptr(o), v.numel(), ctypes.c_void_p(_stream(v.device)))
    _check("fp8bs_debug_encode_e4m3", rc)
    return o


def debug_mfma_block(a: torch.Tensor, w: torch.Tensor, out=None):
    """Test hook: the matrix cores' fp32 dot products of one K block.
    a, w: uint8 [tiles, 16, 128] codes; returns d float32 [tiles, 16, 16]
    with d[t, n, m] = sum_k w[t, n, k] * a[t, m, k]."""
    a, w = _as_u8(a), _as_u8(w)
    _need(a, "a", torch.uint8)
    _need(w, "w", torch.uint8, a.device)
    if a.dim() != 3 or tuple(a.shape[1:]) != (16, 128) or a.shape != w.shape:
        raise ValueError("a and w must both be [tiles, 16, 128]")
    tiles = a.shape[0]
    d = torch.empty((tiles, 16, 16), dtype=torch.float32, device=a.device) if out is None else \
        _out(out, "out", _F32, (tiles, 16, 16), a.device)
    with torch.cuda.device(a.device):
        rc = lib().fp8bs_debug_mfma_block(_ptr(a), _ptr(w), _ptr(d), tiles, ctypes.c_void_p(_stream(a.device)))
    _check("fp8bs_debug_mfma_block", rc)
    return d
