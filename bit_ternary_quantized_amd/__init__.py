"""Python binding of the gfx950 BitLinear library (libbitnet_amd.so).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  Each function has the name of the C entry point it wraps
(include/bitnet.h has the full contract); torch supplies device memory and
the current stream.  Outputs not passed in are allocated here with torch.

There is no fallback: if the library is missing or a call fails, an error
is raised.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitnet_amd.so")

BITNET_OK = 0
BITNET_F32, BITNET_BF16 = 0, 1
BITNET_LAYOUT_ROWS, BITNET_LAYOUT_DECODE = 0, 1
(BITNET_OP_WEIGHT_QUANT, BITNET_OP_LINEAR_BWD_STE, BITNET_OP_LINEAR_FWD, BITNET_OP_CODE_COUNTS,
 BITNET_OP_WEIGHT_QUANT_ROWS) = 0, 1, 2, 3, 4
GEMV_MAX_M = 16  # linear_fwd runs the packed GEMV up to this many tokens

EXPORTS = (
    "bitnet_weight_quant", "bitnet_act_quant", "bitnet_linear_fwd", "bitnet_linear_bwd_ste",
    "bitnet_pack_ternary", "bitnet_rmsnorm_bwd", "bitnet_linear_bwd_ste_gated", "bitnet_weight_clamp",
    "bitnet_code_counts", "bitnet_weight_quant_rows", "bitnet_linear_fwd_channel",
    "bitnet_linear_bwd_ste_channel", "bitnet_linear_fwd_decode", "bitnet_quant_operands",
    "bitnet_decode_layout_bytes", "bitnet_pack_decode",
    "bitnet_workspace_bytes", "bitnet_status_str", "bitnet_version",
)


class BitnetError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libbitnet_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} not found: build it with `python bit_ternary_quantized_amd/build.py`")
    lib = ctypes.CDLL(path)
    i64, p, c_int, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sigs = {
        "bitnet_weight_quant": (c_int, [p, c_int, i64, i64, p, p, p, sz, p]),
        "bitnet_act_quant": (c_int, [p, c_int, i64, i64, ctypes.c_float, p, p, p]),
        "bitnet_linear_fwd": (c_int, [p, p, p, p, i64, i64, i64, p, p, p]),
        "bitnet_linear_bwd_ste": (c_int, [p, c_int, p, p, p, p, i64, i64, i64, p, c_int, p, p, sz, p]),
        "bitnet_pack_ternary": (c_int, [p, i64, i64, p, p]),
        "bitnet_rmsnorm_bwd": (c_int, [p, c_int, p, c_int, i64, i64, ctypes.c_float, p, c_int, p]),
        "bitnet_linear_bwd_ste_gated": (c_int, [p, c_int, p, p, p, p, p, c_int, ctypes.c_float, ctypes.c_float,
                                                i64, i64, i64, p, c_int, p, p, sz, p]),
        "bitnet_weight_clamp": (c_int, [p, c_int, i64, i64, ctypes.c_float, ctypes.c_float, p]),
        "bitnet_code_counts": (c_int, [p, i64, i64, p, p, sz, p]),
        "bitnet_weight_quant_rows": (c_int, [p, c_int, i64, i64, p, p, p, sz, p]),
        "bitnet_linear_fwd_channel": (c_int, [p, p, p, p, i64, i64, i64, p, p, p]),
        "bitnet_linear_bwd_ste_channel": (c_int, [p, c_int, p, p, p, p, i64, i64, i64, p, c_int, p, p, sz, p]),
        "bitnet_linear_fwd_decode": (c_int, [p, c_int, p, c_int, p, i64, i64, i64, ctypes.c_float, p, p, p, p]),
        "bitnet_decode_layout_bytes": (i64, [i64, i64]),
        "bitnet_pack_decode": (c_int, [p, i64, i64, p, p]),
        "bitnet_quant_operands": (c_int, [p, c_int, i64, i64, ctypes.c_float, p, p, p, c_int, i64, p, p, p, sz, p]),
        "bitnet_workspace_bytes": (sz, [c_int, i64, i64, i64]),
        "bitnet_status_str": (ctypes.c_char_p, [c_int]),
        "bitnet_version": (c_int, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != BITNET_OK:
        raise BitnetError(fn, status, bitnet_status_str(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return BITNET_F32
    if t.dtype == torch.bfloat16:
        return BITNET_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def bitnet_status_str(status: int) -> str:
    return load_library().bitnet_status_str(int(status)).decode()


def bitnet_version() -> int:
    return int(load_library().bitnet_version())


def bitnet_workspace_bytes(op: int, M: int, N: int, K: int) -> int:
    return int(load_library().bitnet_workspace_bytes(int(op), int(M), int(N), int(K)))


def bitnet_weight_quant(W: torch.Tensor, W_packed=None, gamma=None, workspace=None, stream=None):
    """Absmean ternary codes, 2-bit packed -> (W_packed uint8 [N,K/4], gamma f32 [1])."""
    lib = load_library()
    _need(W, "W")
    N, K = W.shape
    dev = W.device
    if W_packed is None:
        W_packed = torch.empty(N, K // 4, dtype=torch.uint8, device=dev)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=dev)
    need = bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT, 0, N, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check("bitnet_weight_quant", lib.bitnet_weight_quant(
        _ptr(W), _dtype_code(W), N, K, _ptr(W_packed), _ptr(gamma), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return W_packed, gamma


def bitnet_act_quant(X: torch.Tensor, eps: float = 1e-5, Xq=None, scale_x=None, stream=None):
    """RMSNorm + per-token absmax int8 -> (Xq int8 [M,K], scale_x f32 [M])."""
    lib = load_library()
    _need(X, "X")
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty(M, K, dtype=torch.int8, device=X.device)
    if scale_x is None:
        scale_x = torch.empty(M, dtype=torch.float32, device=X.device)
    _check("bitnet_act_quant", lib.bitnet_act_quant(
        _ptr(X), _dtype_code(X), M, K, ctypes.c_float(eps), _ptr(Xq), _ptr(scale_x), _stream(stream)))
    return Xq, scale_x


def bitnet_quant_operands(X, W, eps: float = 1e-5, Xq=None, scale_x=None, W_packed=None, gamma=None,
                          workspace=None, stream=None):
    """act_quant(X) and weight_quant(W) with one launch fewer -> (Xq, scale_x, W_packed, gamma)."""
    lib = load_library()
    _need(X, "X")
    _need(W, "W")
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("X and W must share K")
    dev = X.device
    if Xq is None:
        Xq = torch.empty(M, K, dtype=torch.int8, device=dev)
    if scale_x is None:
        scale_x = torch.empty(M, dtype=torch.float32, device=dev)
    if W_packed is None:
        W_packed = torch.empty(N, K // 4, dtype=torch.uint8, device=dev)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=dev)
    ws_bytes = lib.bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT, 0, N, K)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    _check("bitnet_quant_operands", lib.bitnet_quant_operands(
        _ptr(X), _dtype_code(X), M, K, ctypes.c_float(eps), _ptr(Xq), _ptr(scale_x), _ptr(W), _dtype_code(W), N,
        _ptr(W_packed), _ptr(gamma), _ptr(workspace), workspace.numel(), _stream(stream)))
    return Xq, scale_x, W_packed, gamma


def bitnet_linear_fwd(Xq, scale_x, W_packed, gamma, Y=None, acc=None, want_acc=False, stream=None):
    """y = (Xq . codes^T) * gamma / scale_x -> (Y f32 [M,N], acc int32 [M,N] or None)."""
    lib = load_library()
    for t, n in ((Xq, "Xq"), (scale_x, "scale_x"), (W_packed, "W_packed"), (gamma, "gamma")):
        _need(t, n)
    M, K = Xq.shape
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must be [N, K/4]")
    if Y is None:
        Y = torch.empty(M, N, dtype=torch.float32, device=Xq.device)
    if acc is None and want_acc:
        acc = torch.empty(M, N, dtype=torch.int32, device=Xq.device)
    _check("bitnet_linear_fwd", lib.bitnet_linear_fwd(
        _ptr(Xq), _ptr(scale_x), _ptr(W_packed), _ptr(gamma), M, N, K, _ptr(Y), _ptr(acc),
        _stream(stream)))
    return Y, acc


def bitnet_linear_bwd_ste(grad_y, Xq, scale_x, W_packed, gamma, want_grad_x=True, want_grad_W=True,
                          gx_dtype=torch.float32, grad_x=None, grad_W=None, workspace=None,
                          stream=None):
    """STE backward -> (grad_x [M,K] f32/bf16 or None, grad_W f32 [N,K] or None)."""
    lib = load_library()
    for t, n in ((grad_y, "grad_y"), (Xq, "Xq"), (scale_x, "scale_x"), (W_packed, "W_packed"),
                 (gamma, "gamma")):
        _need(t, n)
    M, K = Xq.shape
    N = W_packed.shape[0]
    dev = Xq.device
    if grad_x is None and want_grad_x:
        grad_x = torch.empty(M, K, dtype=gx_dtype, device=dev)
    if grad_W is None and want_grad_W:
        grad_W = torch.empty(N, K, dtype=torch.float32, device=dev)
    need = bitnet_workspace_bytes(BITNET_OP_LINEAR_BWD_STE, M, N, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    gx_code = _dtype_code(grad_x) if grad_x is not None else BITNET_F32
    _check("bitnet_linear_bwd_ste", lib.bitnet_linear_bwd_ste(
        _ptr(grad_y), _dtype_code(grad_y), _ptr(Xq), _ptr(scale_x), _ptr(W_packed), _ptr(gamma),
        M, N, K, _ptr(grad_x), gx_code, _ptr(grad_W), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return grad_x, grad_W


def bitnet_rmsnorm_bwd(X, grad_n, eps: float = 1e-5, out_dtype=torch.float32, grad_X=None, stream=None):
    """Backward of the unit-gain RMSNorm: grad w.r.t. its input X given grad_n
    (w.r.t. its output) -> grad_X [M,K] f32/bf16."""
    lib = load_library()
    _need(X, "X")
    _need(grad_n, "grad_n")
    M, K = X.shape
    if tuple(grad_n.shape) != (M, K):
        raise ValueError("grad_n must have X's shape")
    if grad_X is None:
        grad_X = torch.empty(M, K, dtype=out_dtype, device=X.device)
    _check("bitnet_rmsnorm_bwd", lib.bitnet_rmsnorm_bwd(
        _ptr(X), _dtype_code(X), _ptr(grad_n), _dtype_code(grad_n), M, K, ctypes.c_float(eps),
        _ptr(grad_X), _dtype_code(grad_X), _stream(stream)))
    return grad_X


def bitnet_linear_bwd_ste_gated(grad_y, Xq, scale_x, W_packed, gamma, W, w_lo=-1.0, w_hi=1.0,
                                want_grad_x=True, want_grad_W=True, gx_dtype=torch.float32, grad_x=None,
                                grad_W=None, workspace=None, stream=None):
    """STE backward with grad_W zeroed where the master weight W lies outside
    [w_lo, w_hi] -> (grad_x or None, grad_W or None)."""
    lib = load_library()
    for t, n in ((grad_y, "grad_y"), (Xq, "Xq"), (scale_x, "scale_x"), (W_packed, "W_packed"),
                 (gamma, "gamma"), (W, "W")):
        _need(t, n)
    M, K = Xq.shape
    N = W_packed.shape[0]
    if tuple(W.shape) != (N, K):
        raise ValueError("W must be [N, K]")
    dev = Xq.device
    if grad_x is None and want_grad_x:
        grad_x = torch.empty(M, K, dtype=gx_dtype, device=dev)
    if grad_W is None and want_grad_W:
        grad_W = torch.empty(N, K, dtype=torch.float32, device=dev)
    need = bitnet_workspace_bytes(BITNET_OP_LINEAR_BWD_STE, M, N, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    gx_code = _dtype_code(grad_x) if grad_x is not None else BITNET_F32
    _check("bitnet_linear_bwd_ste_gated", lib.bitnet_linear_bwd_ste_gated(
        _ptr(grad_y), _dtype_code(grad_y), _ptr(Xq), _ptr(scale_x), _ptr(W_packed), _ptr(gamma),
        _ptr(W), _dtype_code(W), ctypes.c_float(w_lo), ctypes.c_float(w_hi), M, N, K, _ptr(grad_x), gx_code,
        _ptr(grad_W), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return grad_x, grad_W


def bitnet_weight_clamp(W, lo=-1.0, hi=1.0, stream=None):
    """Clamp the master weights in place to [lo, hi]; returns W."""
    lib = load_library()
    _need(W, "W")
    N, K = W.shape
    _check("bitnet_weight_clamp", lib.bitnet_weight_clamp(
        _ptr(W), _dtype_code(W), N, K, ctypes.c_float(lo), ctypes.c_float(hi), _stream(stream)))
    return W


def bitnet_weight_quant_rows(W: torch.Tensor, W_packed=None, gamma=None, workspace=None, stream=None):
    """Per-output-channel absmean codes -> (W_packed uint8 [N,K/4], gamma f32 [N])."""
    lib = load_library()
    _need(W, "W")
    N, K = W.shape
    dev = W.device
    if W_packed is None:
        W_packed = torch.empty(N, K // 4, dtype=torch.uint8, device=dev)
    if gamma is None:
        gamma = torch.empty(N, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT_ROWS, 0, N, K), dtype=torch.uint8,
                                device=dev)
    _check("bitnet_weight_quant_rows", lib.bitnet_weight_quant_rows(
        _ptr(W), _dtype_code(W), N, K, _ptr(W_packed), _ptr(gamma), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return W_packed, gamma


def bitnet_linear_fwd_channel(Xq, scale_x, W_packed, s, Y=None, acc=None, want_acc=False, stream=None):
    """y = (Xq . codes^T) * s[n] / scale_x[m] -> (Y f32 [M,N], acc int32 or None)."""
    lib = load_library()
    for t, n in ((Xq, "Xq"), (scale_x, "scale_x"), (W_packed, "W_packed"), (s, "s")):
        _need(t, n)
    M, K = Xq.shape
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K or s.numel() != N:
        raise ValueError("W_packed must be [N, K/4] and s [N]")
    if Y is None:
        Y = torch.empty(M, N, dtype=torch.float32, device=Xq.device)
    if acc is None and want_acc:
        acc = torch.empty(M, N, dtype=torch.int32, device=Xq.device)
    _check("bitnet_linear_fwd_channel", lib.bitnet_linear_fwd_channel(
        _ptr(Xq), _ptr(scale_x), _ptr(W_packed), _ptr(s), M, N, K, _ptr(Y), _ptr(acc), _stream(stream)))
    return Y, acc


def bitnet_linear_fwd_decode(X, W_packed, gamma, eps: float = 1e-5, Y=None, Xq=None, scale_x=None,
                             want_q=False, stream=None, N=None):
    """Decode forward in one launch: act_quant(X) then the packed GEMV, M <= 16,
    K <= 4096 -> (Y f32 [M,N], Xq int8 or None, scale_x f32 or None).

    W_packed is [N, K/4] packed rows, or (with N given) the 1-D output of
    bitnet_pack_decode for those rows."""
    lib = load_library()
    for t, n in ((X, "X"), (W_packed, "W_packed"), (gamma, "gamma")):
        _need(t, n)
    M, K = X.shape
    if N is None:
        layout = BITNET_LAYOUT_ROWS
        N = W_packed.shape[0]
        if W_packed.dim() != 2 or W_packed.shape[1] * 4 != K:
            raise ValueError("W_packed must be [N, K/4]")
    else:
        layout = BITNET_LAYOUT_DECODE
        need = bitnet_decode_layout_bytes(N, K)
        if W_packed.dim() != 1 or W_packed.dtype != torch.uint8 or W_packed.numel() != need:
            raise ValueError(f"a decode-layout W_packed is 1-D uint8 of {need} bytes")
    if Y is None:
        Y = torch.empty(M, N, dtype=torch.float32, device=X.device)
    if want_q and Xq is None:
        Xq = torch.empty(M, K, dtype=torch.int8, device=X.device)
    if want_q and scale_x is None:
        scale_x = torch.empty(M, dtype=torch.float32, device=X.device)
    _check("bitnet_linear_fwd_decode", lib.bitnet_linear_fwd_decode(
        _ptr(X), _dtype_code(X), _ptr(W_packed), layout, _ptr(gamma), M, N, K, ctypes.c_float(eps),
        _ptr(Y), _ptr(Xq), _ptr(scale_x), _stream(stream)))
    return Y, Xq, scale_x


def bitnet_decode_layout_bytes(N: int, K: int) -> int:
    """Bytes of the decode layout of [N, K/4] packed rows (ValueError if unsupported)."""
    n = load_library().bitnet_decode_layout_bytes(N, K)
    if n < 0:
        raise ValueError(f"no decode layout for N={N}, K={K} (K must be 4096)")
    return n


def bitnet_pack_decode(W_packed, W_decode=None, stream=None):
    """Packed rows [N, K/4] -> the same bytes in the decode layout (1-D uint8)."""
    lib = load_library()
    _need(W_packed, "W_packed")
    N, KB = W_packed.shape
    K = 4 * KB
    need = bitnet_decode_layout_bytes(N, K)
    if W_decode is None:
        W_decode = torch.empty(need, dtype=torch.uint8, device=W_packed.device)
    elif W_decode.numel() != need:
        raise ValueError(f"W_decode must hold {need} bytes")
    _check("bitnet_pack_decode", lib.bitnet_pack_decode(_ptr(W_packed), N, K, _ptr(W_decode), _stream(stream)))
    return W_decode


def bitnet_linear_bwd_ste_channel(grad_y, Xq, scale_x, W_packed, s, want_grad_x=True, want_grad_W=True,
                                  gx_dtype=torch.float32, grad_x=None, grad_W=None, workspace=None, stream=None):
    """STE backward at W_deq = s[n] * code -> (grad_x or None, grad_W or None)."""
    lib = load_library()
    for t, n in ((grad_y, "grad_y"), (Xq, "Xq"), (scale_x, "scale_x"), (W_packed, "W_packed"), (s, "s")):
        _need(t, n)
    M, K = Xq.shape
    N = W_packed.shape[0]
    if s.numel() != N:
        raise ValueError("s must be [N]")
    dev = Xq.device
    if grad_x is None and want_grad_x:
        grad_x = torch.empty(M, K, dtype=gx_dtype, device=dev)
    if grad_W is None and want_grad_W:
        grad_W = torch.empty(N, K, dtype=torch.float32, device=dev)
    need = bitnet_workspace_bytes(BITNET_OP_LINEAR_BWD_STE, M, N, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    gx_code = _dtype_code(grad_x) if grad_x is not None else BITNET_F32
    _check("bitnet_linear_bwd_ste_channel", lib.bitnet_linear_bwd_ste_channel(
        _ptr(grad_y), _dtype_code(grad_y), _ptr(Xq), _ptr(scale_x), _ptr(W_packed), _ptr(s), M, N, K,
        _ptr(grad_x), gx_code, _ptr(grad_W), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return grad_x, grad_W


def bitnet_code_counts(W_packed, K: int, counts=None, workspace=None, stream=None):
    """Counts of the packed codes -> int64 device tensor [zeros, +1, -1, unused 11]."""
    lib = load_library()
    _need(W_packed, "W_packed")
    N = W_packed.shape[0]
    if W_packed.shape[1] * 4 != K:
        raise ValueError("W_packed must be [N, K/4]")
    if counts is None:
        counts = torch.empty(4, dtype=torch.int64, device=W_packed.device)
    if workspace is None:
        workspace = torch.empty(bitnet_workspace_bytes(BITNET_OP_CODE_COUNTS, 0, N, K), dtype=torch.uint8,
                                device=W_packed.device)
    _check("bitnet_code_counts", lib.bitnet_code_counts(
        _ptr(W_packed), N, K, _ptr(counts), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return counts


def bitnet_pack_ternary(codes: torch.Tensor, W_packed=None, stream=None):
    """int8 codes [N,K] -> packed uint8 [N,K/4]."""
    lib = load_library()
    _need(codes, "codes")
    N, K = codes.shape
    if W_packed is None:
        W_packed = torch.empty(N, K // 4, dtype=torch.uint8, device=codes.device)
    _check("bitnet_pack_ternary", lib.bitnet_pack_ternary(
        _ptr(codes), N, K, _ptr(W_packed), _stream(stream)))
    return W_packed


def bitlinear_forward(X, W, eps: float = 1e-5, want_acc=False, stream=None):
    """The whole forward of one layer on the device: act quant, weight quant, linear.

    Returns a dict with Xq, scale_x, W_packed, gamma, Y (and acc when asked).
    """
    Xq, scale_x = bitnet_act_quant(X, eps, stream=stream)
    W_packed, gamma = bitnet_weight_quant(W, stream=stream)
    Y, acc = bitnet_linear_fwd(Xq, scale_x, W_packed, gamma, want_acc=want_acc, stream=stream)
    return {"Xq": Xq, "scale_x": scale_x, "W_packed": W_packed, "gamma": gamma, "Y": Y, "acc": acc}
