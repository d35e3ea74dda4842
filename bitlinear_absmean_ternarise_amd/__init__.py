"""Python binding of libbitlinear.so (MI355X / gfx950 BitNet b1.58 BitLinear).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  If the
built library is missing, importing this package raises: there is no CPU
fallback.

Entry points mirror include/bitlinear.h:
    packed_bytes, pack_workspace_bytes, pack_weights, pack_binary, quant_act,
    rmsnorm_quant_act, forward, forward_grouped, flip_update, flip_stats,
    adamw_step, pack_transposed, backward_input, backward_input_grouped, pack_weights_grouped, strerror,
    forward_grouped_noalloc, quant_forward_grouped,
    packed_bytes_b1, pack_binary_b1, forward_b1, forward_b1_grouped, quant_forward_b1_grouped,
    forward_grouped_dot4,
    layout_version
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libbitlinear.so")

BL_OK = 0
STATUS = {0: "BL_OK", -1: "BL_ERR_NULL", -2: "BL_ERR_SHAPE", -3: "BL_ERR_ALIGN", -4: "BL_ERR_VALUE",
          -5: "BL_ERR_DEVICE", -6: "BL_ERR_ARCH", -7: "BL_ERR_WORKSPACE",
          -8: "BL_ERR_SCRATCH"}


class BitLinearError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({strerror(status)})")


class ForwardArgs(C.Structure):
    """Mirror of bitlinear_forward_args."""
    _fields_ = [("packed", C.c_void_p), ("gamma", C.c_void_p), ("N", C.c_int64), ("K", C.c_int64),
                ("xq", C.c_void_p), ("x_scale", C.c_void_p), ("M", C.c_int64), ("y", C.c_void_p),
                ("acc", C.c_void_p)]


MAX_GROUP = 8


class QuantForwardArgs(C.Structure):
    """Mirror of bitlinear_quant_forward_args."""
    _fields_ = [("packed", C.c_void_p), ("gamma", C.c_void_p), ("N", C.c_int64), ("K", C.c_int64),
                ("x", C.c_void_p), ("M", C.c_int64), ("xq", C.c_void_p), ("x_scale", C.c_void_p),
                ("y", C.c_void_p), ("acc", C.c_void_p)]


class PackArgs(C.Structure):
    """Mirror of bitlinear_pack_args."""
    _fields_ = [("W", C.c_void_p), ("N", C.c_int64), ("K", C.c_int64), ("eps", C.c_float),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t), ("packed", C.c_void_p),
                ("gamma", C.c_void_p), ("packed_t", C.c_void_p)]


MAX_PACK_GROUP = 64


class BackwardArgs(C.Structure):
    """Mirror of bitlinear_backward_args."""
    _fields_ = [("packed_t", C.c_void_p), ("gamma", C.c_void_p), ("N", C.c_int64), ("dy", C.c_void_p)]


MAX_BACKWARD_GROUP = 4


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python bitlinear_absmean_ternarise_amd/build.py` "
                          "(there is no CPU fallback)")
    L = C.CDLL(LIB_PATH)
    i64, p, sz = C.c_int64, C.c_void_p, C.c_size_t
    L.bitlinear_packed_bytes.argtypes = [i64, i64, C.POINTER(sz)]
    L.bitlinear_pack_workspace_bytes.argtypes = [i64, i64, C.POINTER(sz)]
    L.bitlinear_pack_weights.argtypes = [p, i64, i64, C.c_float, p, sz, p, p, p]
    L.bitlinear_quant_act.argtypes = [p, i64, i64, C.c_float, p, p, p]
    L.bitlinear_pack_binary.argtypes = [p, i64, i64, p, sz, p, p, p, p]
    L.bitlinear_flip_stats.argtypes = [p, p, i64, C.c_int32, p, p, p]
    d = C.c_double
    L.bitlinear_adamw_step.argtypes = [p, p, p, p, i64, C.c_int32, d, d, d, d, d, p, p, p]
    L.bitlinear_rmsnorm_quant_act.argtypes = [p, p, i64, i64, C.c_float, C.c_float, p, p, p]
    L.bitlinear_forward.argtypes = [p, p, i64, i64, p, p, i64, p, p, p]
    L.bitlinear_pack_transposed.argtypes = [p, i64, i64, p, p]
    L.bitlinear_pack_weights_grouped.argtypes = [C.POINTER(PackArgs), C.c_int, p]
    L.bitlinear_backward_input.argtypes = [p, p, i64, i64, p, i64, p, C.c_int, p]
    L.bitlinear_flip_update.argtypes = [p, p, i64, C.c_int32, p, p, p]
    L.bitlinear_backward_input_grouped.argtypes = [C.POINTER(BackwardArgs), C.c_int, i64, i64, p, C.c_int, p]
    L.bitlinear_forward_grouped.argtypes = [C.POINTER(ForwardArgs), C.c_int, p]
    L.bitlinear_forward_workspace_bytes.argtypes = [C.POINTER(ForwardArgs), C.c_int, C.POINTER(sz)]
    L.bitlinear_forward_grouped_ws.argtypes = [C.POINTER(ForwardArgs), C.c_int, p, sz, p]
    L.bitlinear_forward_grouped_noalloc.argtypes = [C.POINTER(ForwardArgs), C.c_int, p]
    L.bitlinear_quant_forward_grouped.argtypes = [C.POINTER(QuantForwardArgs), C.c_int, C.c_float, p, sz, p]
    L.bitlinear_quant_forward_workspace_bytes.argtypes = [C.POINTER(QuantForwardArgs), C.c_int, C.POINTER(sz)]
    L.bitlinear_packed_bytes_b1.argtypes = [i64, i64, C.POINTER(sz)]
    L.bitlinear_pack_binary_b1.argtypes = [p, i64, i64, p, sz, p, p, p, p]
    L.bitlinear_forward_b1.argtypes = [p, p, i64, i64, p, p, i64, p, p, p]
    L.bitlinear_forward_b1_grouped.argtypes = [C.POINTER(ForwardArgs), C.c_int, p]
    L.bitlinear_forward_grouped_dot4.argtypes = [C.POINTER(ForwardArgs), C.c_int, p]
    L.bitlinear_quant_forward_b1_grouped.argtypes = [C.POINTER(QuantForwardArgs), C.c_int, C.c_float, p]
    L.bitlinear_strerror.argtypes = [C.c_int]
    L.bitlinear_strerror.restype = C.c_char_p
    L.bitlinear_layout_version.argtypes = []
    for f in ("bitlinear_packed_bytes", "bitlinear_pack_workspace_bytes", "bitlinear_pack_weights",
              "bitlinear_quant_act", "bitlinear_rmsnorm_quant_act", "bitlinear_forward", "bitlinear_pack_binary",
              "bitlinear_flip_stats", "bitlinear_adamw_step", "bitlinear_forward_grouped",
              "bitlinear_pack_transposed", "bitlinear_backward_input", "bitlinear_pack_weights_grouped", "bitlinear_flip_update",
              "bitlinear_forward_workspace_bytes", "bitlinear_forward_grouped_ws", "bitlinear_layout_version",
              "bitlinear_backward_input_grouped", "bitlinear_forward_grouped_noalloc",
              "bitlinear_quant_forward_grouped", "bitlinear_quant_forward_workspace_bytes",
              "bitlinear_packed_bytes_b1", "bitlinear_pack_binary_b1", "bitlinear_forward_b1",
              "bitlinear_forward_b1_grouped", "bitlinear_forward_grouped_dot4",
              "bitlinear_quant_forward_b1_grouped"):
        getattr(L, f).restype = C.c_int
    return L


lib = _load()


def strerror(status: int) -> str:
    return lib.bitlinear_strerror(int(status)).decode()


def layout_version() -> int:
    return int(lib.bitlinear_layout_version())


def _check(rc: int, what: str):
    if rc != BL_OK:
        raise BitLinearError(rc, what)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def packed_bytes(N: int, K: int) -> int:
    out = C.c_size_t()
    _check(lib.bitlinear_packed_bytes(N, K, C.byref(out)), "packed_bytes")
    return out.value


def pack_workspace_bytes(N: int, K: int) -> int:
    out = C.c_size_t()
    _check(lib.bitlinear_pack_workspace_bytes(N, K, C.byref(out)), "pack_workspace_bytes")
    return out.value


def pack_weights(W: torch.Tensor, eps: float = 1e-5, packed: torch.Tensor | None = None,
                 gamma: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """W fp32 [N][K] -> (packed uint8 [packed_bytes], gamma fp32 [1])."""
    _need(W, "W", torch.float32, 2)
    N, K = W.shape
    dev = W.device
    if packed is None:
        packed = torch.empty(packed_bytes(N, K), dtype=torch.uint8, device=dev)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(pack_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    _check(lib.bitlinear_pack_weights(_ptr(W), N, K, C.c_float(eps), _ptr(workspace), workspace.numel(),
                                      _ptr(packed), _ptr(gamma), _stream(W)), "pack_weights")
    return packed, gamma


def pack_binary(W: torch.Tensor, packed: torch.Tensor | None = None, beta: torch.Tensor | None = None,
                alpha: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Binary BitNet weights: W fp32 [N][K] -> (packed uint8, beta fp32 [1],
    alpha fp32 [1]); forward() takes (packed, beta) like (packed, gamma)."""
    _need(W, "W", torch.float32, 2)
    N, K = W.shape
    dev = W.device
    if packed is None:
        packed = torch.empty(packed_bytes(N, K), dtype=torch.uint8, device=dev)
    if beta is None:
        beta = torch.empty(1, dtype=torch.float32, device=dev)
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(pack_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    _check(lib.bitlinear_pack_binary(_ptr(W), N, K, _ptr(workspace), workspace.numel(), _ptr(packed), _ptr(beta),
                                     _ptr(alpha), _stream(W)), "pack_binary")
    return packed, beta, alpha


def packed_bytes_b1(N: int, K: int) -> int:
    """Bytes of layout b1 (one bit per binary code; K % 64 == 0)."""
    out = C.c_size_t()
    _check(lib.bitlinear_packed_bytes_b1(N, K, C.byref(out)), "packed_bytes_b1")
    return out.value


def pack_binary_b1(W: torch.Tensor, packed: torch.Tensor | None = None, beta: torch.Tensor | None = None,
                   alpha: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Binary BitNet weights in layout b1: W fp32 [N][K] -> (packed uint8
    [packed_bytes_b1], beta fp32 [1], alpha fp32 [1]); forward_b1() reads them."""
    _need(W, "W", torch.float32, 2)
    N, K = W.shape
    dev = W.device
    if packed is None:
        packed = torch.empty(packed_bytes_b1(N, K), dtype=torch.uint8, device=dev)
    if beta is None:
        beta = torch.empty(1, dtype=torch.float32, device=dev)
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(pack_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    _check(lib.bitlinear_pack_binary_b1(_ptr(W), N, K, _ptr(workspace), workspace.numel(), _ptr(packed),
                                        _ptr(beta), _ptr(alpha), _stream(W)), "pack_binary_b1")
    return packed, beta, alpha


def forward_b1(packed: torch.Tensor, beta: torch.Tensor, N: int, K: int, xq: torch.Tensor,
               x_scale: torch.Tensor, y: torch.Tensor | None = None, acc: torch.Tensor | bool | None = None):
    """forward() over layout b1: y bf16 [M][N] = rescale(xq @ codes^T) with
    beta; acc=True (or an int32 [M][N] tensor) also returns the int32 sums."""
    _need(xq, "xq", torch.int8, 2)
    _need(x_scale, "x_scale", torch.float32, 1)
    _need(packed, "packed", torch.uint8, 1)
    _need(beta, "beta", torch.float32, 1)
    M = xq.shape[0]
    if xq.shape[1] != K or x_scale.shape[0] != M or packed.numel() != packed_bytes_b1(N, K):
        raise ValueError("inconsistent shapes")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    acc_t = None
    if acc is True:
        acc_t = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    elif isinstance(acc, torch.Tensor):
        _need(acc, "acc", torch.int32, 2)
        acc_t = acc
    _check(lib.bitlinear_forward_b1(_ptr(packed), _ptr(beta), N, K, _ptr(xq), _ptr(x_scale), M, _ptr(y),
                                    _ptr(acc_t), _stream(xq)), "forward_b1")
    return (y, acc_t) if acc_t is not None else y


def forward_b1_grouped(entries):
    """Several forward_b1 calls in one launch.  `entries`: dicts with keys
    packed (layout b1), gamma (beta), N, K, xq, x_scale, y and optionally acc.
    Returns the list of y."""
    if not 1 <= len(entries) <= MAX_GROUP:
        raise ValueError(f"1..{MAX_GROUP} entries")
    arr, stream = _forward_arr(entries, b1=True)
    _check(lib.bitlinear_forward_b1_grouped(arr, len(entries), stream), "forward_b1_grouped")
    return [e["y"] for e in entries]


def quant_act(x: torch.Tensor, eps: float = 1e-5, xq: torch.Tensor | None = None,
              x_scale: torch.Tensor | None = None):
    """x bf16 [M][K] -> (xq int8 [M][K], x_scale fp32 [M])."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib.bitlinear_quant_act(_ptr(x), M, K, C.c_float(eps), _ptr(xq), _ptr(x_scale), _stream(x)),
           "quant_act")
    return xq, x_scale


def rmsnorm_quant_act(x: torch.Tensor, gain: torch.Tensor | None = None, eps_norm: float = 1e-6,
                      eps: float = 1e-5, xq: torch.Tensor | None = None, x_scale: torch.Tensor | None = None):
    """x bf16 [M][K] -> RMSNorm (optional fp32 gain [K]) fused with the
    activation quant -> (xq int8 [M][K], x_scale fp32 [M])."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if gain is not None:
        _need(gain, "gain", torch.float32, 1)
        if gain.numel() != K:
            raise ValueError("gain must have K entries")
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib.bitlinear_rmsnorm_quant_act(_ptr(x), _ptr(gain), M, K, C.c_float(eps_norm), C.c_float(eps), _ptr(xq),
                                           _ptr(x_scale), _stream(x)), "rmsnorm_quant_act")
    return xq, x_scale


def forward(packed: torch.Tensor, gamma: torch.Tensor, N: int, K: int, xq: torch.Tensor,
            x_scale: torch.Tensor, y: torch.Tensor | None = None, acc: torch.Tensor | bool | None = None,
            workspace="auto"):
    """y bf16 [M][N] = rescale(xq @ codes^T).  acc=True (or an int32 [M][N]
    tensor) also returns the exact int32 accumulators.  `workspace` as for
    forward_grouped ("auto", None, or a uint8 device tensor)."""
    _need(xq, "xq", torch.int8, 2)
    _need(x_scale, "x_scale", torch.float32, 1)
    _need(packed, "packed", torch.uint8, 1)
    _need(gamma, "gamma", torch.float32, 1)
    M = xq.shape[0]
    if xq.shape[1] != K or x_scale.shape[0] != M or packed.numel() != packed_bytes(N, K):
        raise ValueError("inconsistent shapes")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    acc_t = None
    if acc is True:
        acc_t = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    elif isinstance(acc, torch.Tensor):
        _need(acc, "acc", torch.int32, 2)
        acc_t = acc
    if workspace is not None and M > 0:
        forward_grouped([dict(packed=packed, gamma=gamma, N=N, K=K, xq=xq, x_scale=x_scale, y=y, acc=acc_t)],
                        workspace=workspace)
    else:
        _check(lib.bitlinear_forward(_ptr(packed), _ptr(gamma), N, K, _ptr(xq), _ptr(x_scale), M, _ptr(y),
                                     _ptr(acc_t), _stream(xq)), "forward")
    return (y, acc_t) if acc_t is not None else y


def pack_weights_grouped(Ws, eps: float = 1e-5, outs=None, workspaces=None, transposed=None):
    """Several fp32 [N][K] weights packed in one call; returns a list of
    (packed, gamma) equal to pack_weights() of each.  `outs` (a list of
    (packed, gamma)) and `workspaces` may be given to reuse buffers.
    `transposed`: True (allocate) or a list of uint8 buffers to also receive
    each tensor's codes in layout t1 (returned as a third element)."""
    if not 1 <= len(Ws) <= MAX_PACK_GROUP:
        raise ValueError(f"1..{MAX_PACK_GROUP} tensors")
    arr = (PackArgs * len(Ws))()
    res = []
    for i, W in enumerate(Ws):
        _need(W, "W", torch.float32, 2)
        N, K = W.shape
        if outs is None:
            pk = torch.empty(packed_bytes(N, K), dtype=torch.uint8, device=W.device)
            g = torch.empty(1, dtype=torch.float32, device=W.device)
        else:
            pk, g = outs[i]
        ws = workspaces[i] if workspaces is not None else torch.empty(pack_workspace_bytes(N, K), dtype=torch.uint8,
                                                                      device=W.device)
        _need(pk, "packed", torch.uint8, 1)
        _need(g, "gamma", torch.float32, 1)
        if pk.numel() != packed_bytes(N, K) or ws.numel() < pack_workspace_bytes(N, K):
            raise ValueError("buffer sizes")
        pt = None
        if transposed is True:
            pt = torch.empty(packed_bytes(K, N), dtype=torch.uint8, device=W.device)
        elif transposed is not None:
            pt = transposed[i]
        if pt is not None:
            _need(pt, "packed_t", torch.uint8, 1)
            if pt.numel() != packed_bytes(K, N):
                raise ValueError("packed_t has the wrong size")
        arr[i] = PackArgs(W.data_ptr(), N, K, float(eps), ws.data_ptr(), ws.numel(), pk.data_ptr(), g.data_ptr(),
                          None if pt is None else pt.data_ptr())
        res.append((pk, g, pt, ws))
    _check(lib.bitlinear_pack_weights_grouped(arr, len(Ws), _stream(Ws[0])), "pack_weights_grouped")
    if transposed is None:
        return [(pk, g) for pk, g, _, _ in res]
    return [(pk, g, pt) for pk, g, pt, _ in res]


def pack_transposed(packed: torch.Tensor, N: int, K: int, packed_t: torch.Tensor | None = None):
    """Layout v1 codes of an N x K weight -> the same codes in layout t1 (for
    backward_input)."""
    _need(packed, "packed", torch.uint8, 1)
    if packed.numel() != packed_bytes(N, K):
        raise ValueError("inconsistent shapes")
    if packed_t is None:
        packed_t = torch.empty(packed_bytes(K, N), dtype=torch.uint8, device=packed.device)
    _need(packed_t, "packed_t", torch.uint8, 1)
    if packed_t.numel() != packed_bytes(K, N):
        raise ValueError("packed_t has the wrong size")
    _check(lib.bitlinear_pack_transposed(_ptr(packed), N, K, _ptr(packed_t), _stream(packed)), "pack_transposed")
    return packed_t


def backward_input(packed_t: torch.Tensor, gamma: torch.Tensor, N: int, K: int, dy: torch.Tensor,
                   dx: torch.Tensor | None = None, accumulate: bool = False):
    """STE gradient to the input: dx bf16 [M][K] = gamma * dy @ codes
    (+ dx when accumulate)."""
    _need(packed_t, "packed_t", torch.uint8, 1)
    _need(gamma, "gamma", torch.float32, 1)
    _need(dy, "dy", torch.bfloat16, 2)
    M = dy.shape[0]
    if dy.shape[1] != N or packed_t.numel() != packed_bytes(K, N):
        raise ValueError("inconsistent shapes")
    if dx is None:
        if accumulate:
            raise ValueError("accumulate needs dx")
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device)
    _need(dx, "dx", torch.bfloat16, 2)
    if tuple(dx.shape) != (M, K):
        raise ValueError("dx has the wrong shape")
    _check(lib.bitlinear_backward_input(_ptr(packed_t), _ptr(gamma), N, K, _ptr(dy), M, _ptr(dx),
                                        1 if accumulate else 0, _stream(dy)), "backward_input")
    return dx


def backward_input_grouped(entries, K: int, dx: torch.Tensor | None = None, accumulate: bool = False):
    """Input gradient of several layers that read one input: `entries` is a
    list of (packed_t, gamma, N, dy) as for backward_input, all with the same
    M rows; dx bf16 [M][K] receives the sum of their gradients (added to dx
    when accumulate), rounded as per-entry backward_input calls round it."""
    if not 1 <= len(entries) <= MAX_BACKWARD_GROUP:
        raise ValueError(f"1..{MAX_BACKWARD_GROUP} entries")
    arr = (BackwardArgs * len(entries))()
    M = entries[0][3].shape[0] if entries[0][3].dim() == 2 else -1
    for i, (packed_t, gamma, N, dy) in enumerate(entries):
        _need(packed_t, "packed_t", torch.uint8, 1)
        _need(gamma, "gamma", torch.float32, 1)
        _need(dy, "dy", torch.bfloat16, 2)
        if tuple(dy.shape) != (M, N) or packed_t.numel() != packed_bytes(K, N):
            raise ValueError(f"entry {i}: inconsistent shapes")
        arr[i] = BackwardArgs(packed_t.data_ptr(), gamma.data_ptr(), int(N), dy.data_ptr())
    dy0 = entries[0][3]
    if dx is None:
        if accumulate:
            raise ValueError("accumulate needs dx")
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dy0.device)
    _need(dx, "dx", torch.bfloat16, 2)
    if tuple(dx.shape) != (M, K):
        raise ValueError("dx has the wrong shape")
    _check(lib.bitlinear_backward_input_grouped(arr, len(entries), int(K), M, _ptr(dx), 1 if accumulate else 0,
                                                _stream(dy0)), "backward_input_grouped")
    return dx


def _forward_arr(entries, b1: bool = False):
    arr = (ForwardArgs * len(entries))()
    stream = None
    for i, e in enumerate(entries):
        xq, xs, y = e["xq"], e["x_scale"], e["y"]
        _need(xq, "xq", torch.int8, 2)
        _need(xs, "x_scale", torch.float32, 1)
        _need(e["packed"], "packed", torch.uint8, 1)
        _need(e["gamma"], "gamma", torch.float32, 1)
        _need(y, "y", torch.bfloat16, 2)
        acc = e.get("acc")
        if acc is not None:
            _need(acc, "acc", torch.int32, 2)
        M, N, K = xq.shape[0], int(e["N"]), int(e["K"])
        if xq.shape[1] != K or xs.shape[0] != M or tuple(y.shape) != (M, N) or \
                e["packed"].numel() != (packed_bytes_b1(N, K) if b1 else packed_bytes(N, K)):
            raise ValueError(f"entry {i}: inconsistent shapes")
        arr[i] = ForwardArgs(e["packed"].data_ptr(), e["gamma"].data_ptr(), N, K, xq.data_ptr(), xs.data_ptr(),
                             M, y.data_ptr(), acc.data_ptr() if acc is not None else None)
        stream = stream or _stream(xq)
    return arr, stream


def _quant_forward_arr(entries, b1: bool = False):
    """QuantForwardArgs for quant_forward_grouped / quant_forward_b1_grouped,
    allocating xq / x_scale where absent (shared by entries with the same x)."""
    if not 1 <= len(entries) <= MAX_GROUP:
        raise ValueError(f"1..{MAX_GROUP} entries")
    arr = (QuantForwardArgs * len(entries))()
    stream = None
    shared = {}
    out = []
    for i, e in enumerate(entries):
        x, y = e["x"], e["y"]
        _need(x, "x", torch.bfloat16, 2)
        _need(e["packed"], "packed", torch.uint8, 1)
        _need(e["gamma"], "gamma", torch.float32, 1)
        _need(y, "y", torch.bfloat16, 2)
        M, N, K = x.shape[0], int(e["N"]), int(e["K"])
        xq, xs = e.get("xq"), e.get("x_scale")
        if xq is None and xs is None and x.data_ptr() in shared:
            xq, xs = shared[x.data_ptr()]
        if xq is None:
            xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        if xs is None:
            xs = torch.empty(M, dtype=torch.float32, device=x.device)
        shared.setdefault(x.data_ptr(), (xq, xs))
        _need(xq, "xq", torch.int8, 2)
        _need(xs, "x_scale", torch.float32, 1)
        acc = e.get("acc")
        if acc is not None:
            _need(acc, "acc", torch.int32, 2)
        if x.shape[1] != K or tuple(xq.shape) != (M, K) or xs.shape[0] != M or tuple(y.shape) != (M, N) or \
                e["packed"].numel() != (packed_bytes_b1(N, K) if b1 else packed_bytes(N, K)):
            raise ValueError(f"entry {i}: inconsistent shapes")
        arr[i] = QuantForwardArgs(e["packed"].data_ptr(), e["gamma"].data_ptr(), N, K, x.data_ptr(), M,
                                  xq.data_ptr(), xs.data_ptr(), y.data_ptr(),
                                  acc.data_ptr() if acc is not None else None)
        stream = stream or _stream(x)
        out.append((y, xq, xs))
    return arr, stream, out


def quant_forward_grouped(entries, eps: float = 1e-5, workspace="auto"):
    """Activation quant and forward in one call (bitlinear_quant_forward_grouped).
    `entries`: dicts with keys packed, gamma, N, K, x (bf16 [M][K]), y (bf16
    [M][N]), and optionally xq (int8 [M][K]), x_scale (fp32 [M]) and acc
    (int32 [M][N]); xq / x_scale are allocated when absent.  Entries that pass
    the same x tensor and no xq / x_scale of their own share one pair.
    `workspace` as for forward_grouped ("auto", None or a uint8 device tensor):
    used when the call falls back to separate launches for 14..64 tokens.
    Returns the list of (y, xq, x_scale)."""
    arr, stream, out = _quant_forward_arr(entries)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a tensor')
        need = C.c_size_t(0)
        _check(lib.bitlinear_quant_forward_workspace_bytes(arr, len(entries), C.byref(need)),
               "quant_forward_workspace_bytes")
        workspace = torch.empty(need.value, dtype=torch.uint8, device=entries[0]["x"].device) if need.value else None
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
    _check(lib.bitlinear_quant_forward_grouped(arr, len(entries), C.c_float(eps), _ptr(workspace),
                                               0 if workspace is None else workspace.numel(), stream),
           "quant_forward_grouped")
    return out


def quant_forward_b1_grouped(entries, eps: float = 1e-5):
    """quant_forward_grouped over binary weights in layout b1 (each entry's
    packed / gamma from pack_binary_b1): the activation quant and the b1
    forward in one call.  Returns the list of (y, xq, x_scale)."""
    arr, stream, out = _quant_forward_arr(entries, b1=True)
    _check(lib.bitlinear_quant_forward_b1_grouped(arr, len(entries), C.c_float(eps), stream), "quant_forward_b1_grouped")
    return out


def forward_grouped_noalloc(entries):
    """forward_grouped whose split-K scratch is the library's fixed scratch
    (bitlinear_forward_grouped_noalloc): nothing is allocated, by the
    library or here.  Calls that overlap on one GPU race on that scratch."""
    if not 1 <= len(entries) <= MAX_GROUP:
        raise ValueError(f"1..{MAX_GROUP} entries")
    arr, stream = _forward_arr(entries)
    _check(lib.bitlinear_forward_grouped_noalloc(arr, len(entries), stream), "forward_grouped_noalloc")
    return [e["y"] for e in entries]


def forward_grouped_dot4(entries):
    """forward_grouped with the contraction on the vector ALUs (v_dot4_i32_i8)
    for 1..4 tokens: the same results bit for bit.  Returns the list of y."""
    if not 1 <= len(entries) <= MAX_GROUP:
        raise ValueError(f"1..{MAX_GROUP} entries")
    arr, stream = _forward_arr(entries)
    _check(lib.bitlinear_forward_grouped_dot4(arr, len(entries), stream), "forward_grouped_dot4")
    return [e["y"] for e in entries]


def forward_grouped(entries, workspace="auto"):
    """Several independent forwards in one call.  `entries` is a list of dicts
    with keys packed, gamma, N, K, xq, x_scale, y and optionally acc (tensors
    as for forward(); y and acc must be given).  Returns the list of y.
    `workspace`: "auto" allocates the scratch that the split-K path for
    14..64 tokens needs (none otherwise); None never uses it; a uint8 device
    tensor is used as the scratch (it must be large enough)."""
    if not 1 <= len(entries) <= MAX_GROUP:
        raise ValueError(f"1..{MAX_GROUP} entries")
    arr, stream = _forward_arr(entries)
    if workspace is None:
        _check(lib.bitlinear_forward_grouped(arr, len(entries), stream), "forward_grouped")
        return [e["y"] for e in entries]
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a tensor')
        need = forward_workspace_bytes(entries, _arr=arr)
        workspace = torch.empty(need, dtype=torch.uint8, device=entries[0]["xq"].device) if need else None
    if workspace is None:
        _check(lib.bitlinear_forward_grouped(arr, len(entries), stream), "forward_grouped")
    else:
        _need(workspace, "workspace", torch.uint8, 1)
        _check(lib.bitlinear_forward_grouped_ws(arr, len(entries), _ptr(workspace), workspace.numel(), stream),
               "forward_grouped_ws")
    return [e["y"] for e in entries]


def forward_workspace_bytes(entries, _arr=None) -> int:
    """Bytes of scratch the split-K path needs for these forward_grouped
    entries (0: the call takes no workspace)."""
    if _arr is None:
        _arr = (ForwardArgs * len(entries))()
        for i, e in enumerate(entries):
            acc = e.get("acc")
            _arr[i] = ForwardArgs(e["packed"].data_ptr(), e["gamma"].data_ptr(), int(e["N"]), int(e["K"]),
                                  e["xq"].data_ptr(), e["x_scale"].data_ptr(), e["xq"].shape[0], e["y"].data_ptr(),
                                  acc.data_ptr() if acc is not None else None)
    out = C.c_size_t(0)
    _check(lib.bitlinear_forward_workspace_bytes(_arr, len(entries), C.byref(out)), "forward_workspace_bytes")
    return int(out.value)


def adamw_step(W: torch.Tensor, grad: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, t: int,
               lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
               flip_count: torch.Tensor | None = None, last_flip: torch.Tensor | None = None):
    """One AdamW step (fp32 tensors updated in place); with the int16
    counters the sign-flip tracker is updated in the same pass."""
    for t_, nm in ((W, "W"), (grad, "grad"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        _need(t_, nm, torch.float32)
    n = W.numel()
    if not (grad.numel() == exp_avg.numel() == exp_avg_sq.numel() == n):
        raise ValueError("inconsistent sizes")
    if flip_count is not None:
        _need(flip_count, "flip_count", torch.int16)
        _need(last_flip, "last_flip", torch.int16)
        if not (flip_count.numel() == last_flip.numel() == n):
            raise ValueError("inconsistent sizes")
    _check(lib.bitlinear_adamw_step(_ptr(W), _ptr(grad), _ptr(exp_avg), _ptr(exp_avg_sq), n, int(t), float(lr),
                                    float(beta1), float(beta2), float(eps), float(weight_decay), _ptr(flip_count),
                                    _ptr(last_flip), _stream(W)), "adamw_step")
    return W


def flip_stats(flip_count: torch.Tensor, last_flip: torch.Tensor, T: int,
               sign_age: torch.Tensor | None = None, flip_rate: torch.Tensor | None = None):
    """(sign_age, flip_rate) fp32 [n] after T steps from the two int16 counters."""
    _need(flip_count, "flip_count", torch.int16)
    _need(last_flip, "last_flip", torch.int16)
    n = flip_count.numel()
    if last_flip.numel() != n:
        raise ValueError("inconsistent sizes")
    if sign_age is None:
        sign_age = torch.empty(n, dtype=torch.float32, device=flip_count.device)
    if flip_rate is None:
        flip_rate = torch.empty(n, dtype=torch.float32, device=flip_count.device)
    _check(lib.bitlinear_flip_stats(_ptr(flip_count), _ptr(last_flip), n, int(T), _ptr(sign_age), _ptr(flip_rate),
                                    _stream(flip_count)), "flip_stats")
    return sign_age, flip_rate


def flip_update(w_prev: torch.Tensor, w_curr: torch.Tensor, step: int, flip_count: torch.Tensor,
                last_flip: torch.Tensor):
    """Update flip_count / last_flip (int16, in place) from two fp32 snapshots."""
    _need(w_prev, "w_prev", torch.float32)
    _need(w_curr, "w_curr", torch.float32)
    _need(flip_count, "flip_count", torch.int16)
    _need(last_flip, "last_flip", torch.int16)
    n = w_prev.numel()
    if not (w_curr.numel() == flip_count.numel() == last_flip.numel() == n):
        raise ValueError("inconsistent sizes")
    _check(lib.bitlinear_flip_update(_ptr(w_prev), _ptr(w_curr), n, int(step), _ptr(flip_count),
                                     _ptr(last_flip), _stream(w_prev)), "flip_update")
    return flip_count, last_flip
