"""CPU oracle for the BitNet b1.58 BitLinear hot path (test infrastructure).

Only the tests, the entry point's smoke check and the benchmark's CPU
baseline may import this package.  It wraps oracle/oracle.c (plain C, built
by oracle/build.py) with numpy marshalling and shares nothing with the HIP
library.

Arrays: float32 inputs are numpy float32; bfloat16 inputs are passed as
their raw 16-bit patterns in a numpy uint16 array (the C side widens them
exactly).  Outputs that decide integers are int8 / float32; references that
decide nothing are float64.

Pinned against the pages and mathematics in tests/test_oracle_pins.py; the
reduction order (tree_sum) and the RMSNorm / divide-by-gamma readings are
readings of this library's contract; no page prints them.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "oracle_set_threads": (None, [ctypes.c_int]),
        "oracle_get_threads": (ctypes.c_int, []),
        "oracle_tree_sum_f32": (ctypes.c_float, [_p, _i64]),
        "oracle_act_quant": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_float, _p, _p]),
        "oracle_weight_quant": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _p, _p]),
        "oracle_pack": (ctypes.c_int, [_p, _i64, _i64, _p]),
        "oracle_unpack": (ctypes.c_int, [_p, _i64, _i64, _p]),
        "oracle_gemm_i32": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _p]),
        "oracle_gemm_i32_at": (ctypes.c_int, [_p, _p, _i64, _p, _p, _i64, _p]),
        "oracle_dequant": (ctypes.c_int, [_p, _p, ctypes.c_float, _i64, _i64, _p]),
        "oracle_ste_grad_x": (ctypes.c_int, [_p, ctypes.c_int, _p, ctypes.c_float, _i64, _i64, _i64, _p]),
        "oracle_ste_grad_w": (ctypes.c_int, [_p, ctypes.c_int, _p, _p, _i64, _i64, _i64, _p]),
        "oracle_ste_grad_x_at": (ctypes.c_int, [_p, ctypes.c_int, _p, ctypes.c_float, _i64, _i64, _i64,
                                                _p, _p, _i64, _p]),
        "oracle_ste_grad_w_at": (ctypes.c_int, [_p, ctypes.c_int, _p, _p, _i64, _i64, _i64,
                                                _p, _p, _i64, _p]),
        "oracle_rmsnorm_bwd": (ctypes.c_int, [_p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, ctypes.c_float, _p]),
        "oracle_ste_gate": (ctypes.c_int, [_p, _p, ctypes.c_int, _i64, _i64, ctypes.c_float, ctypes.c_float, _p]),
        "oracle_weight_clamp": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_float, ctypes.c_float, _p]),
        "oracle_code_counts": (ctypes.c_int, [_p, _i64, _i64, _p]),
        "oracle_weight_quant_rows": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _p, _p]),
        "oracle_dequant_channel": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _p]),
        "oracle_ste_grad_x_channel": (ctypes.c_int, [_p, ctypes.c_int, _p, _p, _i64, _i64, _i64, _p]),
        "oracle_channel_scale_grad": (ctypes.c_int, [_p, ctypes.c_int, _p, _p, _p, _i64, _i64, _i64, _p]),
        "oracle_channel_scale_grad_at": (ctypes.c_int, [_p, ctypes.c_int, _p, _p, _p, _i64, _i64, _i64, _p, _i64,
                                                        _p]),
        "oracle_codes_row_dot": (ctypes.c_int, [_p, _p, _i64, _i64, _p]),
        "oracle_mul_add_probe": (ctypes.c_float, [ctypes.c_float, ctypes.c_float, ctypes.c_float]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def _float_input(x):
    """Return (contiguous array, dtype flag) for fp32 or bf16-bit inputs."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), BF16
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), F32
    raise TypeError(f"oracle expects float32 or bf16 bits (uint16), got {x.dtype}")


def set_threads(n: int):
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def tree_sum(v) -> np.float32:
    """Canonical pairwise tree sum in binary32 (zero-padded to a power of 2)."""
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    return np.float32(_load().oracle_tree_sum_f32(_ptr(v), v.size))


def act_quant(x, eps: float = 1e-5):
    """RMSNorm (unit gain) then per-token absmax int8 -> (q int8 [M,K], scale_x f32 [M])."""
    x, dt = _float_input(x)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    _check(_load().oracle_act_quant(_ptr(x), dt, M, K, ctypes.c_float(eps), _ptr(q), _ptr(s)), "act_quant")
    return q, s


def weight_quant(w):
    """Absmean ternary quantization -> (codes int8 [N,K] in {-1,0,1}, gamma float32)."""
    w, dt = _float_input(w)
    N, K = w.shape
    c = np.empty((N, K), np.int8)
    g = np.zeros(1, np.float32)
    _check(_load().oracle_weight_quant(_ptr(w), dt, N, K, _ptr(c), _ptr(g)), "weight_quant")
    return c, np.float32(g[0])


def pack(codes):
    """Ternary codes int8 [N,K] -> packed uint8 [N,K/4] (00=0, 01=+1, 10=-1)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = codes.shape
    out = np.empty((N, K // 4), np.uint8)
    _check(_load().oracle_pack(_ptr(codes), N, K, _ptr(out)), "pack")
    return out


def unpack(packed, K: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    out = np.empty((N, K), np.int8)
    _check(_load().oracle_unpack(_ptr(packed), N, K, _ptr(out)), "unpack")
    return out


def gemm_i32(q, codes):
    """acc[m,n] = sum_k q[m,k]*c[n,k] exactly (int64 accumulate, fits int32)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    M, K = q.shape
    N, K2 = codes.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_gemm_i32(_ptr(q), _ptr(codes), M, N, K, _ptr(acc)), "gemm_i32")
    return acc


def gemm_i32_at(q, codes, ms, ns):
    q = np.ascontiguousarray(q, dtype=np.int8)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    K = q.shape[1]
    assert codes.shape[1] == K and ms.shape == ns.shape
    assert ms.size == 0 or (ms.min() >= 0 and ms.max() < q.shape[0] and ns.min() >= 0 and ns.max() < codes.shape[0])
    out = np.empty(ms.size, np.int32)
    _check(_load().oracle_gemm_i32_at(_ptr(q), _ptr(codes), K, _ptr(ms), _ptr(ns), ms.size, _ptr(out)), "gemm_i32_at")
    return out


def dequant(acc, scale_x, gamma):
    """y[m,n] = acc*gamma/scale_x[m] in float64."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    scale_x = np.ascontiguousarray(scale_x, dtype=np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_dequant(_ptr(acc), _ptr(scale_x), ctypes.c_float(gamma), M, N, _ptr(y)), "dequant")
    return y


def linear_fwd(q, scale_x, codes, gamma):
    """Forward from the quantized operands: (acc int32, y float64)."""
    acc = gemm_i32(q, codes)
    return acc, dequant(acc, scale_x, gamma)


def ste_grad_x(gy, codes, gamma):
    gy, dt = _float_input(gy)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    M, N = gy.shape
    K = codes.shape[1]
    assert codes.shape[0] == N
    out = np.empty((M, K), np.float64)
    _check(_load().oracle_ste_grad_x(_ptr(gy), dt, _ptr(codes), ctypes.c_float(gamma), M, N, K, _ptr(out)),
           "ste_grad_x")
    return out


def ste_grad_w(gy, q, scale_x):
    gy, dt = _float_input(gy)
    q = np.ascontiguousarray(q, dtype=np.int8)
    scale_x = np.ascontiguousarray(scale_x, dtype=np.float32)
    M, N = gy.shape
    K = q.shape[1]
    assert q.shape[0] == M and scale_x.shape == (M,)
    out = np.empty((N, K), np.float64)
    _check(_load().oracle_ste_grad_w(_ptr(gy), dt, _ptr(q), _ptr(scale_x), M, N, K, _ptr(out)), "ste_grad_w")
    return out


def ste_grad_x_at(gy, codes, gamma, ms, ks):
    gy, dt = _float_input(gy)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ks = np.ascontiguousarray(ks, dtype=np.int64)
    M, N = gy.shape
    K = codes.shape[1]
    assert codes.shape[0] == N and ms.shape == ks.shape
    assert ms.size == 0 or (ms.min() >= 0 and ms.max() < M and ks.min() >= 0 and ks.max() < K)
    out = np.empty(ms.size, np.float64)
    _check(_load().oracle_ste_grad_x_at(_ptr(gy), dt, _ptr(codes), ctypes.c_float(gamma), M, N, K,
                                        _ptr(ms), _ptr(ks), ms.size, _ptr(out)), "ste_grad_x_at")
    return out


def ste_grad_w_at(gy, q, scale_x, ns, ks):
    gy, dt = _float_input(gy)
    q = np.ascontiguousarray(q, dtype=np.int8)
    scale_x = np.ascontiguousarray(scale_x, dtype=np.float32)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    ks = np.ascontiguousarray(ks, dtype=np.int64)
    M, N = gy.shape
    K = q.shape[1]
    assert q.shape[0] == M and ns.shape == ks.shape
    assert ns.size == 0 or (ns.min() >= 0 and ns.max() < N and ks.min() >= 0 and ks.max() < K)
    out = np.empty(ns.size, np.float64)
    _check(_load().oracle_ste_grad_w_at(_ptr(gy), dt, _ptr(q), _ptr(scale_x), M, N, K,
                                        _ptr(ns), _ptr(ks), ns.size, _ptr(out)), "ste_grad_w_at")
    return out


def rmsnorm_bwd(x, g, eps: float = 1e-5):
    """Gradient w.r.t. the RMSNorm input x given g = dL/d(RMSNorm output)
    (unit gain, eps inside the root), float64."""
    x, xt = _float_input(x)
    g, gt = _float_input(g)
    assert x.shape == g.shape and x.ndim == 2
    M, K = x.shape
    out = np.empty((M, K), np.float64)
    _check(_load().oracle_rmsnorm_bwd(_ptr(x), xt, _ptr(g), gt, M, K, ctypes.c_float(eps), _ptr(out)),
           "rmsnorm_bwd")
    return out


def ste_gate(grad, w, lo: float = -1.0, hi: float = 1.0):
    """grad (float64 [N,K]) where lo <= w <= hi (the master weights), else 0."""
    grad = np.ascontiguousarray(grad, dtype=np.float64)
    w, wt = _float_input(w)
    assert grad.shape == w.shape and w.ndim == 2
    N, K = w.shape
    out = np.empty((N, K), np.float64)
    _check(_load().oracle_ste_gate(_ptr(grad), _ptr(w), wt, N, K, ctypes.c_float(lo), ctypes.c_float(hi),
                                   _ptr(out)), "ste_gate")
    return out


def weight_clamp(w, lo: float = -1.0, hi: float = 1.0):
    """Master weights clamped to [lo, hi], same dtype (bf16 as uint16 bits)."""
    w, wt = _float_input(w)
    assert w.ndim == 2
    N, K = w.shape
    out = np.empty_like(w)
    _check(_load().oracle_weight_clamp(_ptr(w), wt, N, K, ctypes.c_float(lo), ctypes.c_float(hi), _ptr(out)),
           "weight_clamp")
    return out


def code_counts(packed, K: int):
    """Counts of the codes in packed weights [N, K/4]: (zeros, +1, -1, unused 11)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    assert packed.shape[1] * 4 == K
    out = np.zeros(4, np.uint64)
    _check(_load().oracle_code_counts(_ptr(packed), N, K, _ptr(out)), "code_counts")
    return out


def weight_quant_rows(w):
    """Per-output-channel absmean codes -> (int8 codes [N,K], float32 gamma [N])."""
    w, wt = _float_input(w)
    N, K = w.shape
    codes = np.empty((N, K), np.int8)
    gamma = np.empty(N, np.float32)
    _check(_load().oracle_weight_quant_rows(_ptr(w), wt, N, K, _ptr(codes), _ptr(gamma)), "weight_quant_rows")
    return codes, gamma


def linear_fwd_channel(q, scale_x, codes, s):
    """(exact int32 acc, float64 y = acc * s[n] / scale_x[m])."""
    acc = gemm_i32(q, codes)
    scale_x = np.ascontiguousarray(scale_x, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    M, N = acc.shape
    assert scale_x.shape == (M,) and s.shape == (N,)
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_dequant_channel(_ptr(acc), _ptr(scale_x), _ptr(s), M, N, _ptr(y)), "dequant_channel")
    return acc, y


def ste_grad_x_channel(gy, codes, s):
    gy, dt = _float_input(gy)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    M, N = gy.shape
    K = codes.shape[1]
    assert codes.shape[0] == N and s.shape == (N,)
    out = np.empty((M, K), np.float64)
    _check(_load().oracle_ste_grad_x_channel(_ptr(gy), dt, _ptr(codes), _ptr(s), M, N, K, _ptr(out)),
           "ste_grad_x_channel")
    return out


def channel_scale_grad(gy, q, scale_x, codes, ns=None):
    """Gradient of a learned per-output-channel scale s (float64 [N], or at
    the sampled channels ns): sum_m gy[m,n] * acc[m,n] / scale_x[m]."""
    gy, dt = _float_input(gy)
    q = np.ascontiguousarray(q, dtype=np.int8)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scale_x = np.ascontiguousarray(scale_x, dtype=np.float32)
    M, N = gy.shape
    K = q.shape[1]
    assert q.shape == (M, K) and codes.shape == (N, K) and scale_x.shape == (M,)
    if ns is None:
        out = np.empty(N, np.float64)
        _check(_load().oracle_channel_scale_grad(_ptr(gy), dt, _ptr(q), _ptr(scale_x), _ptr(codes), M, N, K,
                                                 _ptr(out)), "channel_scale_grad")
        return out
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ns.size, np.float64)
    _check(_load().oracle_channel_scale_grad_at(_ptr(gy), dt, _ptr(q), _ptr(scale_x), _ptr(codes), M, N, K,
                                                _ptr(ns), ns.size, _ptr(out)), "channel_scale_grad_at")
    return out


def codes_row_dot(G, codes):
    """sum_k codes[n,k] * G[n,k] per row in binary32 (canonical tree; a zero
    total as +0) -> float32 [N]."""
    G = np.ascontiguousarray(G, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = G.shape
    assert codes.shape == (N, K)
    out = np.empty(N, np.float32)
    _check(_load().oracle_codes_row_dot(_ptr(G), _ptr(codes), N, K, _ptr(out)), "codes_row_dot")
    return out


def mul_add_probe(a: float, b: float, c: float) -> np.float32:
    return np.float32(_load().oracle_mul_add_probe(a, b, c))
