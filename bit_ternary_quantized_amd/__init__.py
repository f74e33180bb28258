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
 BITNET_OP_WEIGHT_QUANT_ROWS, BITNET_OP_WEIGHT_QUANT_COUNTED) = 0, 1, 2, 3, 4, 5
GEMV_MAX_M = 16  # linear_fwd runs the packed GEMV up to this many tokens
BITNET_E_SCRATCH = -7
NOALLOC_MAX_N = 1 << 18  # rows bitnet_weight_quant_noalloc's fixed scratch holds

EXPORTS = (
    "bitnet_weight_quant", "bitnet_act_quant", "bitnet_linear_fwd", "bitnet_linear_bwd_ste",
    "bitnet_pack_ternary", "bitnet_rmsnorm_bwd", "bitnet_linear_bwd_ste_gated", "bitnet_weight_clamp",
    "bitnet_code_counts", "bitnet_weight_quant_rows", "bitnet_linear_fwd_channel",
    "bitnet_linear_bwd_ste_channel", "bitnet_linear_fwd_decode", "bitnet_quant_operands",
    "bitnet_decode_layout_bytes", "bitnet_pack_decode",
    "bitnet_workspace_bytes", "bitnet_status_str", "bitnet_version",
    "bitnet_weight_quant_noalloc", "bitnet_channel_scale_grad", "bitnet_weight_quant_counted",
    "bitnet_set_gate_polls",
    # calibration kernels (include/bitnet_calib.h): measured ceilings
    "bitnet_calib_stream_read", "bitnet_calib_mfma", "bitnet_calib_mfma_ops",
)
BITNET_CALIB_MFMA_I8, BITNET_CALIB_MFMA_BF16, BITNET_CALIB_MFMA_I8_TERNARY, BITNET_CALIB_MFMA_BF16_TERNARY = 0, 1, 2, 3


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
        "bitnet_set_gate_polls": (c_int, [c_int]),
        "bitnet_weight_quant_noalloc": (c_int, [p, c_int, i64, i64, p, p, p]),
        "bitnet_channel_scale_grad": (c_int, [p, p, i64, i64, p, p]),
        "bitnet_weight_quant_counted": (c_int, [p, c_int, i64, i64, p, p, p, p, sz, p]),
        "bitnet_calib_stream_read": (c_int, [p, i64, c_int, p, p]),
        "bitnet_calib_mfma": (c_int, [c_int, c_int, c_int, p, p, p]),
        "bitnet_calib_mfma_ops": (ctypes.c_double, [c_int, c_int, c_int]),
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


F32, BF16, I8, U8, I32, I64 = (torch.float32,), (torch.bfloat16,), (torch.int8,), (torch.uint8,), (torch.int32,), \
    (torch.int64,)
FLOAT = (torch.float32, torch.bfloat16)


def _req(t, name: str, dtypes, numel: int = 0, dim=None, device=None):
    """Check a tensor before its pointer reaches the library: present, of one
    of `dtypes`, contiguous, `dim`-dimensional when given and holding at least
    `numel` elements.  A tensor the kernels would read or write out of bounds
    is a ValueError here, never a launch.  Where the tensors live is checked
    by _on_gpu once every tensor of the call has passed this."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {numel}")
    return t


def _on_gpu(**tensors):
    """Every tensor handed to one call is a device tensor, all on one device
    (None entries are absent optional outputs)."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the call's other tensors on {dev}")


def _opt(t, name: str, dtypes, numel: int, device):
    """_req for an optional output (None passes)."""
    return None if t is None else _req(t, name, dtypes, numel, device=device)


def _ws(t, name: str, need: int, device):
    """A workspace: a contiguous device tensor of at least `need` bytes."""
    if t is None:
        if need == 0:
            return None
        raise ValueError(f"{name}: {need} bytes required")
    _req(t, name, None, 0, device=device)
    if t.numel() * t.element_size() < need:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {need}")
    return t


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def bitnet_status_str(status: int) -> str:
    return load_library().bitnet_status_str(int(status)).decode()


def bitnet_version() -> int:
    return int(load_library().bitnet_version())


def bitnet_set_gate_polls(reads: int) -> int:
    """Reads of the published weight-quant threshold before a pack workgroup
    evaluates it itself (tests set 0 to run that path) -> the previous value."""
    r = int(load_library().bitnet_set_gate_polls(int(reads)))
    if r < 0:
        _check("bitnet_set_gate_polls", r)
    return r


def bitnet_workspace_bytes(op: int, M: int, N: int, K: int) -> int:
    return int(load_library().bitnet_workspace_bytes(int(op), int(M), int(N), int(K)))


def _alloc(t, shape, dtype, device):
    return torch.empty(*shape, dtype=dtype, device=device) if t is None else t


def _mk(t, name, what="[rows, cols]"):
    """Rows and columns of a 2-D input tensor."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor {what}")
    return int(t.shape[0]), int(t.shape[1])


def bitnet_weight_quant(W: torch.Tensor, W_packed=None, gamma=None, workspace=None, stream=None):
    """Absmean ternary codes, 2-bit packed -> (W_packed uint8 [N,K/4], gamma f32 [1])."""
    lib = load_library()
    N, K = _mk(W, "W", "[N, K]")
    _req(W, "W", FLOAT)
    dev = W.device
    need = bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT, 0, N, K)
    W_packed = _req(_alloc(W_packed, (N, K // 4), torch.uint8, dev), "W_packed", U8, N * (K // 4), device=dev)
    gamma = _req(_alloc(gamma, (1,), torch.float32, dev), "gamma", F32, 1, device=dev)
    workspace = _ws(_alloc(workspace, (need,), torch.uint8, dev), "workspace", need, dev)
    _on_gpu(W=W, W_packed=W_packed, gamma=gamma, workspace=workspace)
    _check("bitnet_weight_quant", lib.bitnet_weight_quant(
        _ptr(W), _dtype_code(W), N, K, _ptr(W_packed), _ptr(gamma), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))
    return W_packed, gamma


def bitnet_weight_quant_counted(W: torch.Tensor, W_packed=None, gamma=None, counts=None, workspace=None,
                                stream=None):
    """bitnet_weight_quant plus the code counts of its result, counted as the
    codes are written -> (W_packed, gamma, counts int64 [zeros, +1, -1, unused 11])."""
    lib = load_library()
    N, K = _mk(W, "W", "[N, K]")
    _req(W, "W", FLOAT)
    dev = W.device
    need = bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT_COUNTED, 0, N, K)
    W_packed = _req(_alloc(W_packed, (N, K // 4), torch.uint8, dev), "W_packed", U8, N * (K // 4), device=dev)
    gamma = _req(_alloc(gamma, (1,), torch.float32, dev), "gamma", F32, 1, device=dev)
    counts = _req(_alloc(counts, (4,), torch.int64, dev), "counts", I64, 4, device=dev)
    workspace = _ws(_alloc(workspace, (need,), torch.uint8, dev), "workspace", need, dev)
    _on_gpu(W=W, W_packed=W_packed, gamma=gamma, counts=counts, workspace=workspace)
    _check("bitnet_weight_quant_counted", lib.bitnet_weight_quant_counted(
        _ptr(W), _dtype_code(W), N, K, _ptr(W_packed), _ptr(gamma), _ptr(counts), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))
    return W_packed, gamma, counts


def bitnet_weight_quant_noalloc(W: torch.Tensor, W_packed, gamma, stream=None):
    """bitnet_weight_quant without a workspace (the library's fixed device
    scratch; N <= NOALLOC_MAX_N) into caller-provided W_packed and gamma."""
    lib = load_library()
    N, K = _mk(W, "W", "[N, K]")
    _req(W, "W", FLOAT)
    _req(W_packed, "W_packed", U8, N * (K // 4))
    _req(gamma, "gamma", F32, 1)
    _on_gpu(W=W, W_packed=W_packed, gamma=gamma)
    _check("bitnet_weight_quant_noalloc", lib.bitnet_weight_quant_noalloc(
        _ptr(W), _dtype_code(W), N, K, _ptr(W_packed), _ptr(gamma), _stream(stream)))
    return W_packed, gamma


def bitnet_act_quant(X: torch.Tensor, eps: float = 1e-5, Xq=None, scale_x=None, stream=None):
    """RMSNorm + per-token absmax int8 -> (Xq int8 [M,K], scale_x f32 [M])."""
    lib = load_library()
    M, K = _mk(X, "X", "[M, K]")
    _req(X, "X", FLOAT)
    dev = X.device
    Xq = _req(_alloc(Xq, (M, K), torch.int8, dev), "Xq", I8, M * K, device=dev)
    scale_x = _req(_alloc(scale_x, (M,), torch.float32, dev), "scale_x", F32, M, device=dev)
    _on_gpu(X=X, Xq=Xq, scale_x=scale_x)
    _check("bitnet_act_quant", lib.bitnet_act_quant(
        _ptr(X), _dtype_code(X), M, K, ctypes.c_float(eps), _ptr(Xq), _ptr(scale_x), _stream(stream)))
    return Xq, scale_x


def bitnet_quant_operands(X, W, eps: float = 1e-5, Xq=None, scale_x=None, W_packed=None, gamma=None,
                          workspace=None, stream=None):
    """act_quant(X) and weight_quant(W) with one launch fewer -> (Xq, scale_x, W_packed, gamma)."""
    lib = load_library()
    M, K = _mk(X, "X", "[M, K]")
    N, Kw = _mk(W, "W", "[N, K]")
    if Kw != K:
        raise ValueError("X and W must share K")
    _req(X, "X", FLOAT)
    dev = X.device
    _req(W, "W", FLOAT, device=dev)
    need = bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT, 0, N, K)
    Xq = _req(_alloc(Xq, (M, K), torch.int8, dev), "Xq", I8, M * K, device=dev)
    scale_x = _req(_alloc(scale_x, (M,), torch.float32, dev), "scale_x", F32, M, device=dev)
    W_packed = _req(_alloc(W_packed, (N, K // 4), torch.uint8, dev), "W_packed", U8, N * (K // 4), device=dev)
    gamma = _req(_alloc(gamma, (1,), torch.float32, dev), "gamma", F32, 1, device=dev)
    workspace = _ws(_alloc(workspace, (max(need, 16),), torch.uint8, dev), "workspace", need, dev)
    _on_gpu(X=X, W=W, Xq=Xq, scale_x=scale_x, W_packed=W_packed, gamma=gamma, workspace=workspace)
    _check("bitnet_quant_operands", lib.bitnet_quant_operands(
        _ptr(X), _dtype_code(X), M, K, ctypes.c_float(eps), _ptr(Xq), _ptr(scale_x), _ptr(W), _dtype_code(W), N,
        _ptr(W_packed), _ptr(gamma), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return Xq, scale_x, W_packed, gamma


def _linear_operands(Xq, scale_x, W_packed, scale, scale_name, scale_numel):
    """Shapes and checks shared by the forward and backward calls:
    Xq int8 [M,K], scale_x f32 [M], W_packed uint8 [N,K/4], a scale."""
    M, K = _mk(Xq, "Xq", "[M, K]")
    N, KB = _mk(W_packed, "W_packed", "[N, K/4]")
    if KB * 4 != K:
        raise ValueError(f"W_packed must be [N, K/4] = [{N}, {K // 4}], got [{N}, {KB}]")
    _req(Xq, "Xq", I8)
    dev = Xq.device
    _req(W_packed, "W_packed", U8, device=dev)
    _req(scale_x, "scale_x", F32, M, device=dev)
    _req(scale, scale_name, F32, scale_numel(N), device=dev)
    return M, N, K, dev


def bitnet_linear_fwd(Xq, scale_x, W_packed, gamma, Y=None, acc=None, want_acc=False, stream=None):
    """y = (Xq . codes^T) * gamma / scale_x -> (Y f32 [M,N], acc int32 [M,N] or None)."""
    lib = load_library()
    M, N, K, dev = _linear_operands(Xq, scale_x, W_packed, gamma, "gamma", lambda n: 1)
    Y = _req(_alloc(Y, (M, N), torch.float32, dev), "Y", F32, M * N, device=dev)
    if acc is None and want_acc:
        acc = torch.empty(M, N, dtype=torch.int32, device=dev)
    acc = _opt(acc, "acc", I32, M * N, dev)
    _on_gpu(Xq=Xq, scale_x=scale_x, W_packed=W_packed, gamma=gamma, Y=Y, acc=acc)
    _check("bitnet_linear_fwd", lib.bitnet_linear_fwd(
        _ptr(Xq), _ptr(scale_x), _ptr(W_packed), _ptr(gamma), M, N, K, _ptr(Y), _ptr(acc),
        _stream(stream)))
    return Y, acc


def _bwd_outputs(grad_y, M, N, K, dev, want_grad_x, want_grad_W, gx_dtype, grad_x, grad_W, workspace):
    gy_rows, gy_cols = _mk(grad_y, "grad_y", "[M, N]")
    if (gy_rows, gy_cols) != (M, N):
        raise ValueError(f"grad_y must be [M, N] = [{M}, {N}], got [{gy_rows}, {gy_cols}]")
    _req(grad_y, "grad_y", BF16, device=dev)
    if grad_x is None and want_grad_x:
        grad_x = torch.empty(M, K, dtype=gx_dtype, device=dev)
    if grad_W is None and want_grad_W:
        grad_W = torch.empty(N, K, dtype=torch.float32, device=dev)
    grad_x = _opt(grad_x, "grad_x", FLOAT, M * K, dev)
    grad_W = _opt(grad_W, "grad_W", F32, N * K, dev)
    if grad_x is None and grad_W is None:
        raise ValueError("at least one of grad_x, grad_W must be computed")
    need = bitnet_workspace_bytes(BITNET_OP_LINEAR_BWD_STE, M, N, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    workspace = _ws(workspace, "workspace", need, dev)
    return grad_x, grad_W, workspace


def bitnet_linear_bwd_ste(grad_y, Xq, scale_x, W_packed, gamma, want_grad_x=True, want_grad_W=True,
                          gx_dtype=torch.float32, grad_x=None, grad_W=None, workspace=None,
                          stream=None):
    """STE backward -> (grad_x [M,K] f32/bf16 or None, grad_W f32 [N,K] or None)."""
    lib = load_library()
    M, N, K, dev = _linear_operands(Xq, scale_x, W_packed, gamma, "gamma", lambda n: 1)
    grad_x, grad_W, workspace = _bwd_outputs(grad_y, M, N, K, dev, want_grad_x, want_grad_W, gx_dtype, grad_x,
                                             grad_W, workspace)
    gx_code = _dtype_code(grad_x) if grad_x is not None else BITNET_F32
    _on_gpu(grad_y=grad_y, Xq=Xq, scale_x=scale_x, W_packed=W_packed, gamma=gamma, grad_x=grad_x, grad_W=grad_W,
            workspace=workspace)
    _check("bitnet_linear_bwd_ste", lib.bitnet_linear_bwd_ste(
        _ptr(grad_y), BITNET_BF16, _ptr(Xq), _ptr(scale_x), _ptr(W_packed), _ptr(gamma),
        M, N, K, _ptr(grad_x), gx_code, _ptr(grad_W), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return grad_x, grad_W


def bitnet_rmsnorm_bwd(X, grad_n, eps: float = 1e-5, out_dtype=torch.float32, grad_X=None, stream=None):
    """Backward of the unit-gain RMSNorm: grad w.r.t. its input X given grad_n
    (w.r.t. its output) -> grad_X [M,K] f32/bf16."""
    lib = load_library()
    M, K = _mk(X, "X", "[M, K]")
    if _mk(grad_n, "grad_n", "[M, K]") != (M, K):
        raise ValueError("grad_n must have X's shape")
    _req(X, "X", FLOAT)
    dev = X.device
    _req(grad_n, "grad_n", FLOAT, device=dev)
    grad_X = _req(_alloc(grad_X, (M, K), out_dtype, dev), "grad_X", FLOAT, M * K, device=dev)
    _on_gpu(X=X, grad_n=grad_n, grad_X=grad_X)
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
    M, N, K, dev = _linear_operands(Xq, scale_x, W_packed, gamma, "gamma", lambda n: 1)
    if _mk(W, "W", "[N, K]") != (N, K):
        raise ValueError("W must be [N, K]")
    _req(W, "W", FLOAT, device=dev)
    grad_x, grad_W, workspace = _bwd_outputs(grad_y, M, N, K, dev, want_grad_x, want_grad_W, gx_dtype, grad_x,
                                             grad_W, workspace)
    gx_code = _dtype_code(grad_x) if grad_x is not None else BITNET_F32
    _on_gpu(grad_y=grad_y, Xq=Xq, scale_x=scale_x, W_packed=W_packed, gamma=gamma, W=W, grad_x=grad_x, grad_W=grad_W,
            workspace=workspace)
    _check("bitnet_linear_bwd_ste_gated", lib.bitnet_linear_bwd_ste_gated(
        _ptr(grad_y), BITNET_BF16, _ptr(Xq), _ptr(scale_x), _ptr(W_packed), _ptr(gamma),
        _ptr(W), _dtype_code(W), ctypes.c_float(w_lo), ctypes.c_float(w_hi), M, N, K, _ptr(grad_x), gx_code,
        _ptr(grad_W), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return grad_x, grad_W


def bitnet_weight_clamp(W, lo=-1.0, hi=1.0, stream=None):
    """Clamp the master weights in place to [lo, hi]; returns W."""
    lib = load_library()
    N, K = _mk(W, "W", "[N, K]")
    _req(W, "W", FLOAT)
    _on_gpu(W=W)
    _check("bitnet_weight_clamp", lib.bitnet_weight_clamp(
        _ptr(W), _dtype_code(W), N, K, ctypes.c_float(lo), ctypes.c_float(hi), _stream(stream)))
    return W


def bitnet_weight_quant_rows(W: torch.Tensor, W_packed=None, gamma=None, workspace=None, stream=None):
    """Per-output-channel absmean codes -> (W_packed uint8 [N,K/4], gamma f32 [N])."""
    lib = load_library()
    N, K = _mk(W, "W", "[N, K]")
    _req(W, "W", FLOAT)
    dev = W.device
    need = bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT_ROWS, 0, N, K)
    W_packed = _req(_alloc(W_packed, (N, K // 4), torch.uint8, dev), "W_packed", U8, N * (K // 4), device=dev)
    gamma = _req(_alloc(gamma, (N,), torch.float32, dev), "gamma", F32, N, device=dev)
    workspace = _ws(_alloc(workspace, (need,), torch.uint8, dev), "workspace", need, dev)
    _on_gpu(W=W, W_packed=W_packed, gamma=gamma, workspace=workspace)
    _check("bitnet_weight_quant_rows", lib.bitnet_weight_quant_rows(
        _ptr(W), _dtype_code(W), N, K, _ptr(W_packed), _ptr(gamma), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))
    return W_packed, gamma


def bitnet_linear_fwd_channel(Xq, scale_x, W_packed, s, Y=None, acc=None, want_acc=False, stream=None):
    """y = (Xq . codes^T) * s[n] / scale_x[m] -> (Y f32 [M,N], acc int32 or None)."""
    lib = load_library()
    M, N, K, dev = _linear_operands(Xq, scale_x, W_packed, s, "s", lambda n: n)
    Y = _req(_alloc(Y, (M, N), torch.float32, dev), "Y", F32, M * N, device=dev)
    if acc is None and want_acc:
        acc = torch.empty(M, N, dtype=torch.int32, device=dev)
    acc = _opt(acc, "acc", I32, M * N, dev)
    _on_gpu(Xq=Xq, scale_x=scale_x, W_packed=W_packed, s=s, Y=Y, acc=acc)
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
    M, K = _mk(X, "X", "[M, K]")
    _req(X, "X", FLOAT)
    dev = X.device
    if N is None:
        layout = BITNET_LAYOUT_ROWS
        if not isinstance(W_packed, torch.Tensor) or W_packed.dim() != 2 or W_packed.shape[1] * 4 != K:
            raise ValueError("W_packed must be [N, K/4]")
        N = int(W_packed.shape[0])
        _req(W_packed, "W_packed", U8, device=dev)
    else:
        layout = BITNET_LAYOUT_DECODE
        need = bitnet_decode_layout_bytes(N, K)
        if not isinstance(W_packed, torch.Tensor) or W_packed.dim() != 1 or W_packed.dtype != torch.uint8 \
                or W_packed.numel() != need:
            raise ValueError(f"a decode-layout W_packed is 1-D uint8 of {need} bytes")
        _req(W_packed, "W_packed", U8, need, device=dev)
    _req(gamma, "gamma", F32, 1, device=dev)
    Y = _req(_alloc(Y, (M, N), torch.float32, dev), "Y", F32, M * N, device=dev)
    if want_q and Xq is None:
        Xq = torch.empty(M, K, dtype=torch.int8, device=dev)
    if want_q and scale_x is None:
        scale_x = torch.empty(M, dtype=torch.float32, device=dev)
    Xq = _opt(Xq, "Xq", I8, M * K, dev)
    scale_x = _opt(scale_x, "scale_x", F32, M, dev)
    _on_gpu(X=X, W_packed=W_packed, gamma=gamma, Y=Y, Xq=Xq, scale_x=scale_x)
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
    N, KB = _mk(W_packed, "W_packed", "[N, K/4]")
    _req(W_packed, "W_packed", U8)
    dev = W_packed.device
    K = 4 * KB
    need = bitnet_decode_layout_bytes(N, K)
    W_decode = _req(_alloc(W_decode, (need,), torch.uint8, dev), "W_decode", U8, need, device=dev)
    _on_gpu(W_packed=W_packed, W_decode=W_decode)
    _check("bitnet_pack_decode", lib.bitnet_pack_decode(_ptr(W_packed), N, K, _ptr(W_decode), _stream(stream)))
    return W_decode


def bitnet_linear_bwd_ste_channel(grad_y, Xq, scale_x, W_packed, s, want_grad_x=True, want_grad_W=True,
                                  gx_dtype=torch.float32, grad_x=None, grad_W=None, workspace=None, stream=None):
    """STE backward at W_deq = s[n] * code -> (grad_x or None, grad_W or None)."""
    lib = load_library()
    M, N, K, dev = _linear_operands(Xq, scale_x, W_packed, s, "s", lambda n: n)
    grad_x, grad_W, workspace = _bwd_outputs(grad_y, M, N, K, dev, want_grad_x, want_grad_W, gx_dtype, grad_x,
                                             grad_W, workspace)
    gx_code = _dtype_code(grad_x) if grad_x is not None else BITNET_F32
    _on_gpu(grad_y=grad_y, Xq=Xq, scale_x=scale_x, W_packed=W_packed, s=s, grad_x=grad_x, grad_W=grad_W,
            workspace=workspace)
    _check("bitnet_linear_bwd_ste_channel", lib.bitnet_linear_bwd_ste_channel(
        _ptr(grad_y), BITNET_BF16, _ptr(Xq), _ptr(scale_x), _ptr(W_packed), _ptr(s), M, N, K,
        _ptr(grad_x), gx_code, _ptr(grad_W), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return grad_x, grad_W


def bitnet_channel_scale_grad(grad_W, W_packed, grad_s=None, stream=None):
    """Gradient of a learned per-output-channel scale from the STE backward's
    grad_W [N,K] and the packed codes -> grad_s f32 [N]."""
    lib = load_library()
    N, K = _mk(grad_W, "grad_W", "[N, K]")
    if _mk(W_packed, "W_packed", "[N, K/4]") != (N, K // 4) or K % 4:
        raise ValueError(f"W_packed must be [N, K/4] = [{N}, {K // 4}]")
    _req(grad_W, "grad_W", F32)
    dev = grad_W.device
    _req(W_packed, "W_packed", U8)
    grad_s = _req(_alloc(grad_s, (N,), torch.float32, dev), "grad_s", F32, N)
    _on_gpu(grad_W=grad_W, W_packed=W_packed, grad_s=grad_s)
    _check("bitnet_channel_scale_grad", lib.bitnet_channel_scale_grad(
        _ptr(grad_W), _ptr(W_packed), N, K, _ptr(grad_s), _stream(stream)))
    return grad_s


def bitnet_code_counts(W_packed, K: int, counts=None, workspace=None, stream=None):
    """Counts of the packed codes -> int64 device tensor [zeros, +1, -1, unused 11]."""
    lib = load_library()
    N, KB = _mk(W_packed, "W_packed", "[N, K/4]")
    if KB * 4 != K:
        raise ValueError("W_packed must be [N, K/4]")
    _req(W_packed, "W_packed", U8)
    dev = W_packed.device
    need = bitnet_workspace_bytes(BITNET_OP_CODE_COUNTS, 0, N, K)
    counts = _req(_alloc(counts, (4,), torch.int64, dev), "counts", I64, 4, device=dev)
    workspace = _ws(_alloc(workspace, (need,), torch.uint8, dev), "workspace", need, dev)
    _on_gpu(W_packed=W_packed, counts=counts, workspace=workspace)
    _check("bitnet_code_counts", lib.bitnet_code_counts(
        _ptr(W_packed), N, K, _ptr(counts), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return counts


def bitnet_pack_ternary(codes: torch.Tensor, W_packed=None, stream=None):
    """int8 codes [N,K] -> packed uint8 [N,K/4]."""
    lib = load_library()
    N, K = _mk(codes, "codes", "[N, K]")
    _req(codes, "codes", I8)
    dev = codes.device
    W_packed = _req(_alloc(W_packed, (N, K // 4), torch.uint8, dev), "W_packed", U8, N * (K // 4), device=dev)
    _on_gpu(codes=codes, W_packed=W_packed)
    _check("bitnet_pack_ternary", lib.bitnet_pack_ternary(
        _ptr(codes), N, K, _ptr(W_packed), _stream(stream)))
    return W_packed


def bitnet_calib_stream_read(src, nbytes: int = None, workgroups: int = 1024, sink=None, stream=None):
    """One-launch read of the first `nbytes` bytes of `src` (the measured
    streaming ceiling of a bandwidth-bound call of that byte count)."""
    lib = load_library()
    _req(src, "src", None)
    nbytes = _nbytes(src) if nbytes is None else int(nbytes)
    if nbytes > _nbytes(src):
        raise ValueError(f"src holds {_nbytes(src)} bytes, fewer than {nbytes}")
    sink = _req(_alloc(sink, (1,), torch.int32, src.device), "sink", I32, 1)
    _on_gpu(src=src, sink=sink)
    _check("bitnet_calib_stream_read", lib.bitnet_calib_stream_read(
        _ptr(src), nbytes, int(workgroups), _ptr(sink), _stream(stream)))
    return sink


def bitnet_calib_mfma(kind: int, workgroups: int, iters: int, sink=None, clocks=None, device="cuda",
                      stream=None):
    """Back-to-back MFMAs (int8 or bf16) -> (clocks int64 [workgroups, 2]: shader
    cycles and 100 MHz ticks of each workgroup's loop, operation count)."""
    lib = load_library()
    sink = _req(_alloc(sink, (1,), torch.int32, device), "sink", I32, 1)
    clocks = _req(_alloc(clocks, (workgroups, 2), torch.int64, device), "clocks", I64, 2 * workgroups)
    _on_gpu(sink=sink, clocks=clocks)
    _check("bitnet_calib_mfma", lib.bitnet_calib_mfma(int(kind), int(workgroups), int(iters), _ptr(sink),
                                                      _ptr(clocks), _stream(stream)))
    return clocks, float(lib.bitnet_calib_mfma_ops(int(kind), int(workgroups), int(iters)))


def bitlinear_forward(X, W, eps: float = 1e-5, want_acc=False, stream=None):
    """The whole forward of one layer on the device: act quant, weight quant, linear.

    Returns a dict with Xq, scale_x, W_packed, gamma, Y (and acc when asked).
    """
    Xq, scale_x = bitnet_act_quant(X, eps, stream=stream)
    W_packed, gamma = bitnet_weight_quant(W, stream=stream)
    Y, acc = bitnet_linear_fwd(Xq, scale_x, W_packed, gamma, want_acc=want_acc, stream=stream)
    return {"Xq": Xq, "scale_x": scale_x, "W_packed": W_packed, "gamma": gamma, "Y": Y, "acc": acc}
