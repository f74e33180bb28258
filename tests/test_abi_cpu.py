"""The C-ABI library loads on a host without a GPU, exports every entry point
include/bitnet.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

import bit_ternary_quantized_amd as bt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitnet.h")
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

# Fake, 16-byte-aligned device addresses: every call below fails its host
# checks first, so nothing is ever dereferenced or launched.
P = ctypes.c_void_p(1 << 20)
NULL = None


def declared_functions(paths=None):
    names = set()
    for path in paths or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(bitnet_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_four_calls_and_helpers():
    for n in ("bitnet_weight_quant", "bitnet_act_quant", "bitnet_linear_fwd", "bitnet_linear_bwd_ste"):
        assert n in declared_functions([HEADER])
    names = declared_functions()
    for n in ("bitnet_weight_quant", "bitnet_act_quant", "bitnet_linear_fwd", "bitnet_linear_bwd_ste"):
        assert n in names
    assert set(names) == set(bt.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = bt.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    raw = ctypes.CDLL(bt.LIB_PATH)
    for n in declared_functions():
        getattr(raw, n)  # raises AttributeError when missing


def test_status_strings_and_version():
    assert bt.bitnet_status_str(0) == "ok"
    for s in range(-7, 0):
        assert bt.bitnet_status_str(s) not in ("ok", "unknown status")
    assert bt.bitnet_status_str(-99) == "unknown status"
    assert bt.bitnet_version() >= 10000


def test_workspace_sizes():
    assert bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_FWD, 8, 8, 16) == 0
    wq = bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, 0, 28672, 8192)
    assert wq >= 28672 * 4 + 4 and wq % 256 == 0
    # grad_W of a large, tall layer fills the GPU without splitting its tokens
    # and reads X_deq transposed: K x M bf16
    assert bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, 4096, 28672, 8192) == 8192 * 4096 * 2
    # the token count rounded up to 8 in that copy
    assert bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, 4093, 28672, 8192) == 8192 * 4096 * 2
    # a large, short one (N = 4096) needs no workspace
    assert bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, 8192, 4096, 4096) == 0
    # a small one (N*K = 1376*512) splits 8192 tokens: fp32 partial tiles
    bw = bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, 8192, 1376, 512)
    assert bw >= 2 * 1376 * 512 * 4 and bw % 256 == 0
    assert bt.bitnet_workspace_bytes(7, 1, 1, 4) == 0
    assert bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, -1, 4, 4) == 0


def test_weight_quant_rejects_bad_arguments():
    lib = bt.load_library()
    ws = 1 << 20
    assert lib.bitnet_weight_quant(NULL, 0, 4, 4, P, P, P, ws, NULL) == -1
    assert lib.bitnet_weight_quant(P, 7, 4, 4, P, P, P, ws, NULL) == -3
    assert lib.bitnet_weight_quant(P, 0, 0, 4, P, P, P, ws, NULL) == -2
    assert lib.bitnet_weight_quant(P, 0, 4, 6, P, P, P, ws, NULL) == -2       # K % 4
    assert lib.bitnet_weight_quant(P, 0, 4, 4, ctypes.c_void_p((1 << 20) + 2), P, P, ws, NULL) == -4
    assert lib.bitnet_weight_quant(P, 0, 4, 4, P, P, P, 16, NULL) == -5      # workspace too small
    assert lib.bitnet_weight_quant(P, 0, 4, 4, P, P, NULL, ws, NULL) == -5


def test_act_quant_rejects_bad_arguments():
    lib = bt.load_library()
    e = ctypes.c_float(1e-5)
    assert lib.bitnet_act_quant(NULL, 0, 4, 4, e, P, P, NULL) == -1
    assert lib.bitnet_act_quant(P, 2, 4, 4, e, P, P, NULL) == -3
    assert lib.bitnet_act_quant(P, 0, 0, 4, e, P, P, NULL) == -2
    assert lib.bitnet_act_quant(P, 0, 4, -1, e, P, P, NULL) == -2
    assert lib.bitnet_act_quant(P, 0, 4, 4, ctypes.c_float(-1.0), P, P, NULL) == -1
    assert lib.bitnet_act_quant(ctypes.c_void_p((1 << 20) + 8), 0, 4, 4, e, P, P, NULL) == -4


def test_linear_fwd_rejects_bad_arguments():
    lib = bt.load_library()
    assert lib.bitnet_linear_fwd(P, P, P, P, 4, 4, 16, NULL, NULL, NULL) == -1
    assert lib.bitnet_linear_fwd(P, P, P, P, 4, 4, 8, P, NULL, NULL) == -2     # K % 16
    assert lib.bitnet_linear_fwd(P, P, P, P, 4, 0, 16, P, NULL, NULL) == -2
    assert lib.bitnet_linear_fwd(P, P, P, P, 4, 4, 1 << 24, P, NULL, NULL) == -2
    assert lib.bitnet_linear_fwd(P, P, P, P, 4, 1 << 23, 16, P, NULL, NULL) == -2  # N limit
    assert lib.bitnet_linear_fwd(P, P, P, P, 4, 4, 16, P, ctypes.c_void_p((1 << 20) + 4), NULL) == -4


def test_linear_bwd_rejects_bad_arguments():
    lib = bt.load_library()
    ws = 1 << 30
    assert lib.bitnet_linear_bwd_ste(P, 1, P, P, P, P, 4, 4, 16, NULL, 0, NULL, P, ws, NULL) == -1
    assert lib.bitnet_linear_bwd_ste(P, 0, P, P, P, P, 4, 4, 16, P, 0, P, P, ws, NULL) == -3   # fp32 gy
    assert lib.bitnet_linear_bwd_ste(P, 1, P, P, P, P, 4, 4, 16, P, 5, P, P, ws, NULL) == -3
    assert lib.bitnet_linear_bwd_ste(P, 1, P, P, P, P, 4, 4, 12, P, 0, P, P, ws, NULL) == -2
    assert lib.bitnet_linear_bwd_ste(P, 1, P, P, P, P, 4, 1 << 23, 16, P, 0, P, P, ws, NULL) == -2
    assert lib.bitnet_linear_bwd_ste(P, 1, P, P, P, P, 4, 4, 1 << 24, P, 0, P, P, ws, NULL) == -2
    ws_need = bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, 8192, 1376, 512)
    assert lib.bitnet_linear_bwd_ste(P, 1, P, P, P, P, 8192, 1376, 512, P, 0, P, P, ws_need - 256, NULL) == -5
    assert lib.bitnet_linear_bwd_ste(P, 1, P, P, P, P, 8192, 1376, 512, P, 0, P, NULL, ws_need, NULL) == -5


def test_rmsnorm_bwd_rejects_bad_arguments():
    lib = bt.load_library()
    e = ctypes.c_float(1e-5)
    assert lib.bitnet_rmsnorm_bwd(NULL, 1, P, 0, 4, 8, e, P, 0, NULL) == -1
    assert lib.bitnet_rmsnorm_bwd(P, 1, P, 0, 4, 8, e, NULL, 0, NULL) == -1
    assert lib.bitnet_rmsnorm_bwd(P, 2, P, 0, 4, 8, e, P, 0, NULL) == -3
    assert lib.bitnet_rmsnorm_bwd(P, 1, P, 0, 4, 8, e, P, 9, NULL) == -3
    assert lib.bitnet_rmsnorm_bwd(P, 1, P, 0, 0, 8, e, P, 0, NULL) == -2
    assert lib.bitnet_rmsnorm_bwd(P, 1, P, 0, 4, 12, e, P, 0, NULL) == -2      # K % 8
    assert lib.bitnet_rmsnorm_bwd(P, 1, P, 0, 4, 8, ctypes.c_float(-1.0), P, 0, NULL) == -1
    assert lib.bitnet_rmsnorm_bwd(P, 1, ctypes.c_void_p((1 << 20) + 4), 0, 4, 8, e, P, 0, NULL) == -4


def test_gated_bwd_and_clamp_reject_bad_arguments():
    lib = bt.load_library()
    ws = 1 << 30
    f = ctypes.c_float
    ok = (f(-1.0), f(1.0))
    # W missing, W dtype, NaN bound, W misaligned, then the plain call's checks
    assert lib.bitnet_linear_bwd_ste_gated(P, 1, P, P, P, P, NULL, 0, *ok, 4, 4, 16, P, 0, P, P, ws, NULL) == -1
    assert lib.bitnet_linear_bwd_ste_gated(P, 1, P, P, P, P, P, 4, *ok, 4, 4, 16, P, 0, P, P, ws, NULL) == -3
    assert lib.bitnet_linear_bwd_ste_gated(P, 1, P, P, P, P, P, 0, f(float("nan")), f(1.0), 4, 4, 16, P, 0, P, P,
                                           ws, NULL) == -1
    assert lib.bitnet_linear_bwd_ste_gated(P, 1, P, P, P, P, ctypes.c_void_p((1 << 20) + 4), 0, *ok, 4, 4, 16, P, 0,
                                           P, P, ws, NULL) == -4
    assert lib.bitnet_linear_bwd_ste_gated(P, 1, P, P, P, P, P, 0, *ok, 4, 4, 12, P, 0, P, P, ws, NULL) == -2
    assert lib.bitnet_linear_bwd_ste_gated(P, 0, P, P, P, P, P, 0, *ok, 4, 4, 16, P, 0, P, P, ws, NULL) == -3
    ws_need = bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, 8192, 1376, 512)
    assert lib.bitnet_linear_bwd_ste_gated(P, 1, P, P, P, P, P, 0, *ok, 8192, 1376, 512, P, 0, P, P, ws_need - 256,
                                           NULL) == -5
    assert lib.bitnet_weight_clamp(NULL, 0, 4, 4, *ok, NULL) == -1
    assert lib.bitnet_weight_clamp(P, 3, 4, 4, *ok, NULL) == -3
    assert lib.bitnet_weight_clamp(P, 0, 0, 4, *ok, NULL) == -2
    assert lib.bitnet_weight_clamp(P, 0, 4, 4, f(1.0), f(-1.0), NULL) == -1   # lo > hi
    assert lib.bitnet_weight_clamp(P, 0, 4, 4, f(float("nan")), f(1.0), NULL) == -1
    assert lib.bitnet_weight_clamp(ctypes.c_void_p((1 << 20) + 2), 1, 4, 4, *ok, NULL) == -4


def test_code_counts_reject_bad_arguments():
    lib = bt.load_library()
    ws = bt.bitnet_workspace_bytes(bt.BITNET_OP_CODE_COUNTS, 0, 4, 4)
    assert ws > 0 and ws % 16 == 0
    assert lib.bitnet_code_counts(NULL, 4, 4, P, P, ws, NULL) == -1
    assert lib.bitnet_code_counts(P, 4, 4, NULL, P, ws, NULL) == -1
    assert lib.bitnet_code_counts(P, 4, 6, P, P, ws, NULL) == -2
    assert lib.bitnet_code_counts(P, 0, 4, P, P, ws, NULL) == -2
    assert lib.bitnet_code_counts(ctypes.c_void_p((1 << 20) + 4), 4, 4, P, P, ws, NULL) == -4
    assert lib.bitnet_code_counts(P, 4, 4, ctypes.c_void_p((1 << 20) + 4), P, ws, NULL) == -4
    assert lib.bitnet_code_counts(P, 4, 4, P, P, ws - 16, NULL) == -5
    assert lib.bitnet_code_counts(P, 4, 4, P, NULL, ws, NULL) == -5


def test_channel_calls_reject_bad_arguments():
    lib = bt.load_library()
    ws = bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT_ROWS, 0, 4, 4)
    assert ws >= 2 * 4 * 4 and ws % 256 == 0
    assert lib.bitnet_weight_quant_rows(NULL, 0, 4, 4, P, P, P, ws, NULL) == -1
    assert lib.bitnet_weight_quant_rows(P, 5, 4, 4, P, P, P, ws, NULL) == -3
    assert lib.bitnet_weight_quant_rows(P, 0, 4, 6, P, P, P, ws, NULL) == -2
    assert lib.bitnet_weight_quant_rows(P, 0, 4, 4, P, P, P, 16, NULL) == -5
    assert lib.bitnet_linear_fwd_channel(P, P, P, NULL, 4, 4, 16, P, NULL, NULL) == -1
    assert lib.bitnet_linear_fwd_channel(P, P, P, P, 4, 4, 8, P, NULL, NULL) == -2
    assert lib.bitnet_linear_bwd_ste_channel(P, 1, P, P, P, NULL, 4, 4, 16, P, 0, NULL, NULL, 0, NULL) == -1
    assert lib.bitnet_linear_bwd_ste_channel(P, 0, P, P, P, P, 4, 4, 16, P, 0, NULL, NULL, 0, NULL) == -3


def test_decode_call_rejects_bad_arguments():
    lib = bt.load_library()
    eps = ctypes.c_float(1e-5)
    R, D = bt.BITNET_LAYOUT_ROWS, bt.BITNET_LAYOUT_DECODE

    def f(X, dt, W, gamma, M, N, K, e, Y, Xq, sx, stream, layout=R):
        return lib.bitnet_linear_fwd_decode(X, dt, W, layout, gamma, M, N, K, e, Y, Xq, sx, stream)

    # (X, dtype, W_packed, gamma, M, N, K, eps, Y, Xq, scale_x, stream)
    assert f(NULL, 1, P, P, 1, 16, 64, eps, P, NULL, NULL, NULL) == -1
    assert f(P, 1, P, NULL, 1, 16, 64, eps, P, NULL, NULL, NULL) == -1
    assert f(P, 1, P, P, 1, 16, 64, eps, NULL, NULL, NULL, NULL) == -1
    assert f(P, 2, P, P, 1, 16, 64, eps, P, NULL, NULL, NULL) == -3
    assert f(P, 1, P, P, 1, 16, 64, ctypes.c_float(-1.0), P, NULL, NULL, NULL) == -1
    assert f(P, 1, P, P, 17, 16, 64, eps, P, NULL, NULL, NULL) == -2   # M > 16: two calls instead
    assert f(P, 1, P, P, 0, 16, 64, eps, P, NULL, NULL, NULL) == -2
    assert f(P, 1, P, P, 1, 16, 4112, eps, P, NULL, NULL, NULL) == -2  # K > 4096
    assert f(P, 0, P, P, 9, 16, 4096, eps, P, NULL, NULL, NULL) == -2  # 9 fp32 rows of 4096: 144 blocks
    assert f(P, 1, P, P, 1, 16, 72, eps, P, NULL, NULL, NULL) == -2    # K % 16
    assert f(P, 1, P, P, 1, 0, 64, eps, P, NULL, NULL, NULL) == -2
    odd = ctypes.c_void_p((1 << 20) + 4)
    assert f(odd, 1, P, P, 1, 16, 64, eps, P, NULL, NULL, NULL) == -4
    assert f(P, 1, P, P, 1, 16, 64, eps, P, odd, NULL, NULL) == -4
    assert f(P, 1, P, P, 1, 16, 64, eps, P, NULL, ctypes.c_void_p((1 << 20) + 2), NULL) == -4
    # the decode layout: an unknown layout code, a K it is not defined for
    assert f(P, 1, P, P, 1, 16, 4096, eps, P, NULL, NULL, NULL, layout=2) == -1
    assert f(P, 1, P, P, 1, 16, 2048, eps, P, NULL, NULL, NULL, layout=D) == -2


def test_decode_layout_size_and_pack_argument_checks():
    lib = bt.load_library()
    # ceil(N / 16) row groups of 16 rows, K / 4 bytes a row
    assert lib.bitnet_decode_layout_bytes(16, 4096) == 16 * 1024
    assert lib.bitnet_decode_layout_bytes(17, 4096) == 32 * 1024
    assert lib.bitnet_decode_layout_bytes(11008, 4096) == 11008 * 1024
    assert lib.bitnet_decode_layout_bytes(1, 4096) == 16 * 1024
    assert lib.bitnet_decode_layout_bytes(16, 2048) == -1
    assert lib.bitnet_decode_layout_bytes(0, 4096) == -1
    assert lib.bitnet_decode_layout_bytes(1 << 23, 4096) == -1
    with pytest.raises(ValueError):
        bt.bitnet_decode_layout_bytes(16, 8192)
    assert lib.bitnet_pack_decode(NULL, 16, 4096, P, NULL) == -1
    assert lib.bitnet_pack_decode(P, 16, 4096, NULL, NULL) == -1
    assert lib.bitnet_pack_decode(P, 16, 1024, P, NULL) == -2
    assert lib.bitnet_pack_decode(P, 0, 4096, P, NULL) == -2
    assert lib.bitnet_pack_decode(ctypes.c_void_p((1 << 20) + 8), 16, 4096, P, NULL) == -4


def test_quant_operands_rejects_bad_arguments():
    lib = bt.load_library()
    f = lib.bitnet_quant_operands
    eps = ctypes.c_float(1e-5)
    ws = bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, 0, 8, 16)
    # (X, xdt, M, K, eps, Xq, scale_x, W, wdt, N, W_packed, gamma, ws, ws_bytes, stream)
    assert f(NULL, 1, 4, 16, eps, P, P, P, 0, 8, P, P, P, ws, NULL) == -1
    assert f(P, 1, 4, 16, eps, P, P, NULL, 0, 8, P, P, P, ws, NULL) == -1
    assert f(P, 1, 4, 16, eps, P, P, P, 0, 8, P, NULL, P, ws, NULL) == -1
    assert f(P, 3, 4, 16, eps, P, P, P, 0, 8, P, P, P, ws, NULL) == -3
    assert f(P, 1, 4, 16, eps, P, P, P, 7, 8, P, P, P, ws, NULL) == -3
    assert f(P, 1, 4, 18, eps, P, P, P, 0, 8, P, P, P, ws, NULL) == -2
    assert f(P, 1, 0, 16, eps, P, P, P, 0, 8, P, P, P, ws, NULL) == -2
    assert f(P, 1, 4, 16, ctypes.c_float(-1.0), P, P, P, 0, 8, P, P, P, ws, NULL) == -1
    assert f(P, 1, 4, 16, eps, P, P, ctypes.c_void_p((1 << 20) + 4), 0, 8, P, P, P, ws, NULL) == -4
    assert f(P, 1, 4, 16, eps, P, P, P, 0, 8, P, P, P, ws - 16, NULL) == -5
    assert f(P, 1, 4, 16, eps, P, P, P, 0, 8, P, P, NULL, ws, NULL) == -5


def test_pack_rejects_bad_arguments():
    lib = bt.load_library()
    assert lib.bitnet_pack_ternary(NULL, 4, 4, P, NULL) == -1
    assert lib.bitnet_pack_ternary(P, 4, 5, P, NULL) == -2
    assert lib.bitnet_pack_ternary(P, 4, 4, ctypes.c_void_p((1 << 20) + 1), NULL) == -4


def test_binding_has_no_silent_fallback(tmp_path):
    # a missing library is an error, never a CPU path
    with pytest.raises(ImportError):
        bt._lib_saved = bt._lib
        try:
            bt._lib = None
            bt.load_library(str(tmp_path / "missing.so"))
        finally:
            bt._lib = bt._lib_saved


def _raises(fn, *a, match=None, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_binding_checks_tensors_before_any_call():
    # dtype, shape, contiguity and size are checked before the device; on this
    # host every tensor is a CPU tensor, so a well-formed argument list stops
    # at "must be a device tensor" and nothing reaches the library
    import torch
    M, N, K = 8, 16, 64
    X = torch.zeros(M, K, dtype=torch.bfloat16)
    W = torch.zeros(N, K, dtype=torch.float32)
    Xq = torch.zeros(M, K, dtype=torch.int8)
    sx = torch.ones(M, dtype=torch.float32)
    wp = torch.zeros(N, K // 4, dtype=torch.uint8)
    g = torch.ones(1, dtype=torch.float32)
    gy = torch.zeros(M, N, dtype=torch.bfloat16)
    # the quantizers
    _raises(bt.bitnet_act_quant, X.half(), match="X must be")
    _raises(bt.bitnet_act_quant, X[:, ::2], match="contiguous")
    _raises(bt.bitnet_act_quant, X.reshape(-1), match="2-D")
    _raises(bt.bitnet_act_quant, X, match="device tensor")
    _raises(bt.bitnet_weight_quant, W.double(), match="W must be")
    _raises(bt.bitnet_weight_quant, W, match="device tensor")
    _raises(bt.bitnet_quant_operands, X, W[:, :32], match="share K")
    # forward: every tensor's dtype and size
    _raises(bt.bitnet_linear_fwd, Xq.float(), sx, wp, g, match="Xq must be")
    _raises(bt.bitnet_linear_fwd, Xq, sx[:M - 1], wp, g, match="scale_x holds")
    _raises(bt.bitnet_linear_fwd, Xq, sx.double(), wp, g, match="scale_x must be")
    _raises(bt.bitnet_linear_fwd, Xq, sx, wp[:, :8], g, match="W_packed must be")
    _raises(bt.bitnet_linear_fwd, Xq, sx, wp, g[:0], match="gamma holds")
    _raises(bt.bitnet_linear_fwd, Xq, sx, wp, g, match="device tensor")
    # backward: grad_y's shape and dtype, the outputs' sizes
    _raises(bt.bitnet_linear_bwd_ste, gy.float(), Xq, sx, wp, g, match="grad_y must be torch.bfloat16")
    _raises(bt.bitnet_linear_bwd_ste, gy, Xq, sx, wp, g, grad_W=torch.zeros(N, K - 1), match="grad_W holds")
    _raises(bt.bitnet_linear_bwd_ste, gy, Xq, sx, wp, g, grad_x=torch.zeros(M, K, dtype=torch.int32),
            match="grad_x must be")
    _raises(bt.bitnet_linear_bwd_ste, gy, Xq, sx, wp, g, want_grad_x=False, want_grad_W=False, match="at least one")
    _raises(bt.bitnet_linear_bwd_ste, gy, Xq, sx, wp, g, match="device tensor")
    _raises(bt.bitnet_linear_bwd_ste, gy[:, :N - 1].contiguous(), Xq, sx, wp, g, match="grad_y must be")
    _raises(bt.bitnet_linear_bwd_ste_channel, gy, Xq, sx, wp, g, match="s holds")
    _raises(bt.bitnet_linear_bwd_ste_gated, gy, Xq, sx, wp, g, W[:, :32], match="W must be")
    _raises(bt.bitnet_rmsnorm_bwd, X, X[:4], match="grad_n")
    _raises(bt.bitnet_code_counts, wp, K + 4, match="W_packed must be")
    _raises(bt.bitnet_pack_ternary, Xq.float(), match="codes must be")
    _raises(bt.bitnet_linear_fwd_decode, X, wp.reshape(-1), g, match="W_packed must be")
    _raises(bt.bitnet_linear_fwd_decode, X, wp, g, N=N, match="decode")


def test_binding_rejects_undersized_outputs():
    # an output too small for the kernels' writes, or of the wrong dtype, is
    # rejected on the host; the device check comes after every tensor's size
    # and dtype checks
    import torch
    from bit_ternary_quantized_amd import _on_gpu, _req, _ws
    Y = torch.zeros(3, 4, dtype=torch.float32)
    with pytest.raises(ValueError, match="holds 12 elements"):
        _req(Y, "Y", bt.F32, 13)
    with pytest.raises(ValueError, match="Y must be"):
        _req(Y.half(), "Y", bt.F32, 12)
    assert _req(Y, "Y", bt.F32, 12) is Y
    with pytest.raises(ValueError, match="Y must be a device tensor"):
        _on_gpu(acc=None, Y=Y)
    with pytest.raises(ValueError, match="is required"):
        _req(None, "Y", bt.F32, 12)
    with pytest.raises(ValueError, match="bytes required"):
        _ws(None, "workspace", 256, None)
    assert _ws(None, "workspace", 0, None) is None
    with pytest.raises(ValueError, match="holds 48 bytes, needs 64"):
        _ws(Y, "workspace", 64, None)


def test_calibration_calls_reject_bad_arguments():
    lib = bt.load_library()
    f = lib.bitnet_calib_stream_read
    assert f(NULL, 1024, 64, P, NULL) == -1
    assert f(P, 1024, 64, NULL, NULL) == -1
    assert f(P, 1000, 64, P, NULL) == -2   # not whole 16-byte loads
    assert f(P, 0, 64, P, NULL) == -2
    assert f(P, 1024, 0, P, NULL) == -2
    assert f(ctypes.c_void_p((1 << 20) + 4), 1024, 64, P, NULL) == -4
    g = lib.bitnet_calib_mfma
    assert g(0, 4, 1, NULL, P, NULL) == -1
    assert g(4, 4, 1, P, P, NULL) == -1    # unknown kind
    assert g(-1, 4, 1, P, P, NULL) == -1
    assert g(0, 0, 1, P, P, NULL) == -2
    assert g(1, 4, 0, P, P, NULL) == -2
    assert g(0, 4, 1, P, ctypes.c_void_p((1 << 20) + 4), NULL) == -4
    # 4 waves x 8 MFMAs per iteration; 2*32*32*32 int8 ops, 2*32*32*16 bf16 flops
    assert lib.bitnet_calib_mfma_ops(0, 3, 5) == 3 * 4 * 8 * 5 * 65536
    assert lib.bitnet_calib_mfma_ops(1, 3, 5) == 3 * 4 * 8 * 5 * 32768
    assert lib.bitnet_calib_mfma_ops(2, 3, 5) == 3 * 4 * 8 * 5 * 65536
    assert lib.bitnet_calib_mfma_ops(3, 3, 5) == 3 * 4 * 8 * 5 * 32768
    assert lib.bitnet_calib_mfma_ops(4, 3, 5) == 0.0


def test_noalloc_weight_quant_rejects_bad_arguments():
    lib = bt.load_library()
    f = lib.bitnet_weight_quant_noalloc
    assert f(NULL, 0, 4, 4, P, P, NULL) == -1
    assert f(P, 0, 4, 4, NULL, P, NULL) == -1
    assert f(P, 7, 4, 4, P, P, NULL) == -3
    assert f(P, 0, 4, 6, P, P, NULL) == -2
    assert f(P, 0, 0, 4, P, P, NULL) == -2
    # more rows than the fixed scratch holds: its own status, nothing launched
    assert f(P, 0, (1 << 18) + 1, 4, P, P, NULL) == -7
    assert bt.bitnet_status_str(-7) != "unknown status"
    assert f(ctypes.c_void_p((1 << 20) + 8), 0, 4, 4, P, P, NULL) == -4


def test_weight_quant_counted_rejects_bad_arguments():
    lib = bt.load_library()
    f = lib.bitnet_weight_quant_counted
    ws = bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT_COUNTED, 0, 8, 16)
    assert ws >= bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, 0, 8, 16) + 8
    # one 8-byte pair per 4096 weights
    big = bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT_COUNTED, 0, 4096, 4096)
    assert big >= bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, 0, 4096, 4096) + 8 * 4096
    # (W, dtype, N, K, W_packed, gamma, counts, ws, ws_bytes, stream)
    assert f(NULL, 0, 8, 16, P, P, P, P, ws, NULL) == -1
    assert f(P, 0, 8, 16, P, P, NULL, P, ws, NULL) == -1
    assert f(P, 5, 8, 16, P, P, P, P, ws, NULL) == -3
    assert f(P, 0, 8, 18, P, P, P, P, ws, NULL) == -2
    assert f(P, 0, 0, 16, P, P, P, P, ws, NULL) == -2
    assert f(P, 0, 8, 16, P, P, ctypes.c_void_p((1 << 20) + 4), P, ws, NULL) == -4
    assert f(P, 0, 8, 16, P, P, P, P, ws - 16, NULL) == -5
    assert f(P, 0, 8, 16, P, P, P, NULL, ws, NULL) == -5


def test_channel_scale_grad_rejects_bad_arguments():
    lib = bt.load_library()
    f = lib.bitnet_channel_scale_grad
    assert f(NULL, P, 4, 16, P, NULL) == -1
    assert f(P, NULL, 4, 16, P, NULL) == -1
    assert f(P, P, 4, 16, NULL, NULL) == -1
    assert f(P, P, 4, 8, P, NULL) == -2     # K % 16
    assert f(P, P, 0, 16, P, NULL) == -2
    assert f(P, P, 4, 1 << 24, P, NULL) == -2
    assert f(ctypes.c_void_p((1 << 20) + 4), P, 4, 16, P, NULL) == -4
    assert f(P, P, 4, 16, ctypes.c_void_p((1 << 20) + 2), NULL) == -4


def test_set_gate_polls_bounds_and_previous_value():
    f = bt.load_library().bitnet_set_gate_polls
    assert f(-1) == -1 and f(1025) == -1  # BITNET_E_ARG, nothing changed
    prev = f(7)
    assert prev == 32  # the default
    assert f(0) == 7
    assert f(prev) == 0
    assert bt.bitnet_set_gate_polls(32) == 32
