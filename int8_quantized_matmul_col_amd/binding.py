"""Python binding of libint8mm.so (argument marshalling only).

Every function here has the name of the C entry point it calls
(include/int8mm.h) and does nothing but check dtypes/devices, allocate the
output tensors with torch, and pass raw device pointers plus torch's current
HIP stream across the C ABI.  All arithmetic runs in the library's HIP
kernels; there is no fallback of any kind: if the library is missing the
call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libint8mm.so")

INT8MM_OK = 0
INT8MM_EINVAL = -1
INT8MM_ESHAPE = -2
INT8MM_EWORKSPACE = -3
INT8MM_EHIP = -4
INT8MM_ESCRATCH = -5
INT8MM_MAX_K = 133144
INT8MM_DECODE_MAX_M = 16
INT8MM_MAX_COUNT_THRESHOLDS = 64

# Default outlier threshold (the value of the pages' 8-bit loading config).
DEFAULT_THRESHOLD = 6.0

# Exported symbols and their C signatures: (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "int8_weight_ld": (ctypes.c_int64, [_I64]),
    "int8_weight_bytes": (ctypes.c_int64, [_I64, _I64]),
    "int8_prepare_weight": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "int8_pack_weight": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "int8_matmul_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "int8_matmul": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _P,
                                   ctypes.c_size_t, _P]),
    "int8_linear": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I64, _P, ctypes.c_float, _P, _P,
                                   ctypes.c_size_t, _P]),
    "int8_matmul_profiled": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _P,
                                            ctypes.c_size_t, _P, _P, _P]),
    "int8_column_absmax": (ctypes.c_int, [_P, _I64, _I64, _P, _P, ctypes.c_size_t, _P]),
    "int8_outlier_counts": (ctypes.c_int, [_P, _I64, _P, ctypes.c_int, _P, _P]),
    "int8_matmul_stages": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I64, ctypes.c_float,
                                          _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                          _P, ctypes.c_size_t, _P]),
    "int8_matmul_noalloc": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _P]),
    "int8_matmul_noalloc_max_workspace": (ctypes.c_size_t, []),
    "int8mm_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "int8mm_last_hip_error": (ctypes.c_char_p, []),
}

_lib: Optional[ctypes.CDLL] = None


class Int8mmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        msg = lib.int8mm_strerror(status).decode()
        if status == INT8MM_EHIP:
            msg += ": " + lib.int8mm_last_hip_error().decode()
        super().__init__(f"{fn} failed with status {status} ({msg})")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libint8mm.so (once).  torch is imported first so that the HIP
    runtime it carries is the one the library binds to."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads the HIP runtime)
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m int8_quantized_matmul_col_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != INT8MM_OK:
        raise Int8mmError(fn, status)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _require(t, dtype, name: str, device=None) -> None:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_out(t, shape, dtype, name: str, device=None) -> None:
    """A caller-supplied output buffer must have exactly the shape the
    kernels write (they write every element of it, and nothing beyond)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    _require(t, dtype, name, device)


def int8_weight_ld(K: int) -> int:
    """Row stride of the prepared weight and of the [.][ldk] stage buffers."""
    return int(load().int8_weight_ld(int(K)))


def int8_weight_bytes(N: int, K: int) -> int:
    """Bytes of a prepared weight (panel-tiled, rows padded to 256)."""
    return int(load().int8_weight_bytes(int(N), int(K)))


PANEL = 256  # rows per panel of the tiled layout


def padded_rows(R: int) -> int:
    return (int(R) + PANEL - 1) // PANEL * PANEL


def untile(buf, rows: int):
    """Row-major view of a panel-tiled [Rp][L] buffer (any dtype), first
    `rows` rows.  Byte b of row r sits at
    ((r/256)*(row_bytes/64) + b/64)*16384 + (r%256)*64 + b%64."""
    import torch
    Rp, L = buf.shape
    row_bytes = L * buf.element_size()
    b = buf.contiguous().view(torch.uint8).reshape(Rp // PANEL, row_bytes // 64, PANEL, 64)
    b = b.permute(0, 2, 1, 3).reshape(Rp, row_bytes)
    return b.view(buf.dtype)[:rows]


def unpack_weight(Wq, N: int, K: int):
    """Row-major int8 [N][K] copy of a prepared weight."""
    return untile(Wq, N)[:, :K]


def int8_matmul_workspace_size(M: int, K: int, N: int) -> int:
    return int(load().int8_matmul_workspace_size(int(M), int(K), int(N)))


def int8_prepare_weight(W, out: Optional[Tuple] = None):
    """W: float16 [N][K] on the GPU -> (Wq, w_scale float32 [N]); Wq is the
    panel-tiled int8 weight, stored as an int8 tensor [Np][ldk]
    (Np = N rounded up to 256; see unpack_weight for a row-major copy)."""
    import torch
    lib = load()
    _require(W, torch.float16, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N][K]")
    N, K = W.shape
    ldk = int8_weight_ld(K)
    if out is None:
        Wq = torch.empty((padded_rows(N), ldk), dtype=torch.int8, device=W.device)
        ws = torch.empty((N,), dtype=torch.float32, device=W.device)
    else:
        Wq, ws = out
        _check_out(Wq, (padded_rows(N), ldk), torch.int8, "out[0] (Wq)", W.device)
        _check_out(ws, (N,), torch.float32, "out[1] (w_scale)", W.device)
    st = lib.int8_prepare_weight(_ptr(W), N, K, _ptr(Wq), _ptr(ws), _stream(W.device))
    _check("int8_prepare_weight", st)
    return Wq, ws


def int8_pack_weight(codes, out=None):
    """codes: int8 [N][K] row-major (an absmax/127 per-channel quantization,
    values in [-127, 127]) -> the prepared weight Wq int8 [Np][ldk]
    (panel-tiled), for use with the caller's own per-channel scales."""
    import torch
    lib = load()
    _require(codes, torch.int8, "codes")
    if codes.dim() != 2:
        raise ValueError("codes must be 2-D [N][K]")
    N, K = codes.shape
    Wq = out if out is not None else torch.empty((padded_rows(N), int8_weight_ld(K)),
                                                 dtype=torch.int8, device=codes.device)
    if out is not None:
        _check_out(Wq, (padded_rows(N), int8_weight_ld(K)), torch.int8, "out", codes.device)
    st = lib.int8_pack_weight(_ptr(codes), N, K, _ptr(Wq), _stream(codes.device))
    _check("int8_pack_weight", st)
    return Wq


def workspace_for(M: int, K: int, N: int, device):
    import torch
    nbytes = int8_matmul_workspace_size(M, K, N)
    if nbytes == 0:
        raise Int8mmError("int8_matmul_workspace_size", INT8MM_ESHAPE)
    return torch.empty((nbytes,), dtype=torch.uint8, device=device)


def int8_matmul(X, Wq, w_scale, threshold: float = DEFAULT_THRESHOLD, out=None, workspace=None,
                K: Optional[int] = None):
    """Y = decomposed int8 matmul of X (float16 [M][K]) with the prepared
    weight (Wq int8 [N][ldk], w_scale float32 [N]).  Returns float16 [M][N]."""
    import torch
    lib = load()
    _require(X, torch.float16, "X")
    dev = X.device
    _require(Wq, torch.int8, "Wq", dev)
    _require(w_scale, torch.float32, "w_scale", dev)
    M, Kx = X.shape
    K = Kx if K is None else K
    N = w_scale.numel()
    if Kx != K or Wq.numel() != int8_weight_bytes(N, K):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, Wq {tuple(Wq.shape)}, "
                         f"w_scale {tuple(w_scale.shape)}")
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    if out is not None:
        _check_out(Y, (M, N), torch.float16, "out", dev)
    ws = workspace if workspace is not None else workspace_for(M, K, N, dev)
    st = lib.int8_matmul(_ptr(X), M, K, _ptr(Wq), _ptr(w_scale), N, float(threshold), _ptr(Y),
                         _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check("int8_matmul", st)
    return Y


def int8_matmul_noalloc(X, Wq, w_scale, threshold: float = DEFAULT_THRESHOLD, out=None):
    """int8_matmul through the library's static workspace (no workspace
    argument, nothing allocated by the call; `out` preallocated when the
    caller cannot allocate).  Shapes whose workspace exceeds
    int8_matmul_noalloc_max_workspace() raise (INT8MM_ESCRATCH)."""
    import torch
    lib = load()
    _require(X, torch.float16, "X")
    dev = X.device
    _require(Wq, torch.int8, "Wq", dev)
    _require(w_scale, torch.float32, "w_scale", dev)
    M, K = X.shape
    N = w_scale.numel()
    if Wq.numel() != int8_weight_bytes(N, K):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, Wq {tuple(Wq.shape)}, "
                         f"w_scale {tuple(w_scale.shape)}")
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    if out is not None:
        _check_out(Y, (M, N), torch.float16, "out", dev)
    st = lib.int8_matmul_noalloc(_ptr(X), M, K, _ptr(Wq), _ptr(w_scale), N, float(threshold),
                                 _ptr(Y), _stream(dev))
    _check("int8_matmul_noalloc", st)
    return Y


def int8_matmul_noalloc_max_workspace() -> int:
    return int(load().int8_matmul_noalloc_max_workspace())


def int8_linear(X, Wq, w_scale, bias=None, threshold: float = DEFAULT_THRESHOLD, out=None,
                workspace=None):
    """Y = int8_matmul(X) + bias: the forward of an 8-bit linear layer.
    X float16 [M][K], the prepared weight (Wq, w_scale), bias float16 [N] or
    None.  Returns float16 [M][N]."""
    import torch
    lib = load()
    _require(X, torch.float16, "X")
    dev = X.device
    _require(Wq, torch.int8, "Wq", dev)
    _require(w_scale, torch.float32, "w_scale", dev)
    M, K = X.shape
    N = w_scale.numel()
    if Wq.numel() != int8_weight_bytes(N, K):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, Wq {tuple(Wq.shape)}, "
                         f"w_scale {tuple(w_scale.shape)}")
    if bias is not None:
        _require(bias, torch.float16, "bias", dev)
        if bias.numel() != N:
            raise ValueError(f"bias has {bias.numel()} entries, expected {N}")
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
    if out is not None:
        _check_out(Y, (M, N), torch.float16, "out", dev)
    ws = workspace if workspace is not None else workspace_for(M, K, N, dev)
    st = lib.int8_linear(_ptr(X), M, K, _ptr(Wq), _ptr(w_scale), N, _ptr(bias), float(threshold),
                         _ptr(Y), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check("int8_linear", st)
    return Y


def int8_column_absmax(X, out=None, workspace=None):
    """colmax[k] = max_m |X[m][k]| (float16 [K], exact) of X float16 [M][K]:
    what the outlier test compares with the threshold."""
    import torch
    lib = load()
    _require(X, torch.float16, "X")
    if X.dim() != 2:
        raise ValueError("X must be 2-D [M][K]")
    dev = X.device
    M, K = X.shape
    cm = out if out is not None else torch.empty((K,), dtype=torch.float16, device=dev)
    if out is not None:
        _check_out(cm, (K,), torch.float16, "out", dev)
    ws = workspace if workspace is not None else workspace_for(M, K, 0, dev)
    st = lib.int8_column_absmax(_ptr(X), M, K, _ptr(cm), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(dev))
    _check("int8_column_absmax", st)
    return cm


def int8_outlier_counts(colmax, thresholds, out=None):
    """counts[i] = number of columns with colmax[k] > thresholds[i] (int32
    [len(thresholds)] on colmax's device): |O| at each threshold, counted on
    the GPU with the outlier test's own comparison.  colmax float16 [K] (from
    int8_column_absmax); at most INT8MM_MAX_COUNT_THRESHOLDS thresholds, each
    >= 0 (+inf allowed)."""
    import torch
    lib = load()
    _require(colmax, torch.float16, "colmax")
    if colmax.dim() != 1:
        raise ValueError("colmax must be 1-D [K]")
    ts = [float(t) for t in thresholds]
    n = len(ts)
    dev = colmax.device
    counts = out if out is not None else torch.empty((n,), dtype=torch.int32, device=dev)
    if out is not None:
        _check_out(counts, (n,), torch.int32, "out", dev)
    arr = (ctypes.c_float * max(n, 1))(*ts)
    st = lib.int8_outlier_counts(_ptr(colmax), colmax.numel(), arr, n, _ptr(counts), _stream(dev))
    _check("int8_outlier_counts", st)
    return counts


def int8_matmul_profiled(X, Wq, w_scale, threshold: float, out, workspace, ev_start: int,
                         ev_stop: int):
    """int8_matmul with raw hipEvent_t handles recorded around the matmul
    kernel (for timing that kernel alone).  All tensors preallocated."""
    import torch
    lib = load()
    M, K = X.shape
    N = w_scale.numel()
    _check_out(out, (M, N), torch.float16, "out", X.device)
    st = lib.int8_matmul_profiled(_ptr(X), M, K, _ptr(Wq), _ptr(w_scale), N, float(threshold),
                                  _ptr(out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream(X.device), ev_start, ev_stop)
    _check("int8_matmul_profiled", st)
    return out


def int8_matmul_stages(X, Wq, w_scale, threshold: float = DEFAULT_THRESHOLD,
                       want_c: bool = True, workspace=None) -> Dict[str, object]:
    """Runs the same kernels as int8_matmul and returns every intermediate:
    mask, n_outliers, outlier_idx, Xq [M][ldk], x_scale, X_O [M][ldk],
    W_O [N][ldk] (row-major views of the library's tiled buffers) and C
    (want_c) or Y."""
    import torch
    lib = load()
    _require(X, torch.float16, "X")
    dev = X.device
    _require(Wq, torch.int8, "Wq", dev)
    _require(w_scale, torch.float32, "w_scale", dev)
    M, K = X.shape
    N = w_scale.numel()
    ldk = int8_weight_ld(K)
    if Wq.numel() != int8_weight_bytes(N, K):
        raise ValueError("shape mismatch")
    Mp, Np = padded_rows(M), padded_rows(N)
    o = dict(
        mask=torch.zeros((K,), dtype=torch.uint8, device=dev),
        n_outliers=torch.full((1,), -1, dtype=torch.int32, device=dev),
        outlier_idx=torch.full((K,), -1, dtype=torch.int32, device=dev),
        Xq=torch.zeros((Mp, ldk), dtype=torch.int8, device=dev),
        x_scale=torch.zeros((M,), dtype=torch.float32, device=dev),
        X_O=torch.zeros((Mp, ldk), dtype=torch.float16, device=dev),
        W_O=torch.zeros((Np, ldk), dtype=torch.float16, device=dev),
    )
    C = torch.zeros((M, N), dtype=torch.int32, device=dev) if want_c else None
    Y = None if want_c else torch.empty((M, N), dtype=torch.float16, device=dev)
    ws = workspace if workspace is not None else workspace_for(M, K, N, dev)
    st = lib.int8_matmul_stages(
        _ptr(X), M, K, _ptr(Wq), _ptr(w_scale), N, float(threshold),
        _ptr(o["mask"]), _ptr(o["n_outliers"]), _ptr(o["outlier_idx"]), _ptr(o["Xq"]),
        _ptr(o["x_scale"]), _ptr(o["X_O"]), _ptr(o["W_O"]), _ptr(C), _ptr(Y),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check("int8_matmul_stages", st)
    o["Xq"] = untile(o["Xq"], M)
    o["X_O"] = untile(o["X_O"], M)
    o["W_O"] = untile(o["W_O"], N)
    if want_c:
        o["C"] = C
    else:
        o["Y"] = Y
    return o
