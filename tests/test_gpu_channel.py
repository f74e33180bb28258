"""Per-output-channel scales against the oracle: per-row codes and gammas
bit-exact, the forward (exact int32, y within 1e-3) on the GEMV and GEMM
paths, and the STE grad_x within 2e-2 (grad_W does not involve the scale and
must equal the per-matrix call's bit for bit)."""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import assert_grad_close, assert_y_close, f32_bits_equal, host, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,dt", [(1, 4, "f32"), (37, 64, "f32"), (257, 1040, "f32"), (1376, 512, "f32"),
                                    (300, 272, "bf16")])
def test_weight_quant_rows(N, K, dt):
    print(f"weight_quant_rows N={N} K={K} {dt}", flush=True)
    w = workloads.normal((N, K), 0.02, seed=N + 3 * K, dtype=dt)
    if N > 3:
        w[1] = 0       # gamma floor, every code 0
        w[2] *= 50     # a row on another scale
    wp, g = bt.bitnet_weight_quant_rows(to_dev(w))
    torch.cuda.synchronize()
    c_ref, g_ref = oracle.weight_quant_rows(host(w))
    assert f32_bits_equal(g.cpu().numpy(), g_ref)
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(c_ref))


def _operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.integers(-127, 128, (M, K), dtype=np.int8))
    codes = torch.from_numpy(rng.integers(-1, 2, (N, K), dtype=np.int8))
    sx = torch.from_numpy(rng.uniform(20, 45, M).astype(np.float32))
    s = torch.from_numpy(rng.uniform(0.005, 0.05, N).astype(np.float32))
    return q, codes, sx, s


# GEMV (M <= 16), GEMM with ragged edges, many tiles per workgroup
# (the last two: 17-64 tokens as GEMV blocks; 200 tokens on 128-row GEMM tiles)
FWD_SHAPES = [(1, 300, 256), (1, 70, 8192), (16, 1000, 512), (300, 513, 1040), (4200, 4100, 64), (40, 300, 1024),
              (200, 1000, 4096)]


@pytest.mark.parametrize("M,N,K", FWD_SHAPES)
def test_linear_fwd_channel(M, N, K):
    print(f"linear_fwd_channel M={M} N={N} K={K}", flush=True)
    q, codes, sx, s = _operands(M, N, K, seed=M + N + K)
    wp = bt.bitnet_pack_ternary(to_dev(codes))
    Y, acc = bt.bitnet_linear_fwd_channel(to_dev(q), to_dev(sx), wp, to_dev(s), want_acc=True)
    torch.cuda.synchronize()
    acc_ref, y_ref = oracle.linear_fwd_channel(q.numpy(), sx.numpy(), codes.numpy(), s.numpy())
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(Y.cpu().numpy(), y_ref)


# 128x128 tiles with N % 8 != 0, 256x256 tiles
BWD_SHAPES = [(300, 257, 272), (4096, 64, 4096)]


@pytest.mark.parametrize("M,N,K", BWD_SHAPES)
def test_linear_bwd_ste_channel(M, N, K):
    print(f"linear_bwd_ste_channel M={M} N={N} K={K}", flush=True)
    q, codes, sx, s = _operands(M, N, K, seed=7 * M + N)
    gy = workloads.normal((M, N), 1e-3, seed=M + 2 * N, dtype="bf16")
    wp = bt.bitnet_pack_ternary(to_dev(codes))
    args = (to_dev(gy), to_dev(q), to_dev(sx), wp)
    gx, gw = bt.bitnet_linear_bwd_ste_channel(*args, to_dev(s))
    _, gw0 = bt.bitnet_linear_bwd_ste(*args, to_dev(torch.tensor([0.01])), want_grad_x=False)
    torch.cuda.synchronize()
    assert_grad_close(gx.cpu().numpy(), oracle.ste_grad_x_channel(host(gy), codes.numpy(), s.numpy()), "grad_x")
    assert torch.equal(gw, gw0)


def test_channel_end_to_end_with_row_gammas():
    # per-row weight quant feeding the per-channel forward and backward
    d = workloads.linear_inputs(96, 200, 320, x_dtype="bf16", w_dtype="f32", seed=23)
    Xq, sx = bt.bitnet_act_quant(to_dev(d["x"]))
    wp, g = bt.bitnet_weight_quant_rows(to_dev(d["w"]))
    Y, acc = bt.bitnet_linear_fwd_channel(Xq, sx, wp, g, want_acc=True)
    gx, _ = bt.bitnet_linear_bwd_ste_channel(to_dev(d["gy"]), Xq, sx, wp, g, want_grad_W=False)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.act_quant(host(d["x"]))
    assert np.array_equal(Xq.cpu().numpy(), q_ref) and f32_bits_equal(sx.cpu().numpy(), s_ref)
    c_ref, g_ref = oracle.weight_quant_rows(host(d["w"]))
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(c_ref)) and f32_bits_equal(g.cpu().numpy(), g_ref)
    acc_ref, y_ref = oracle.linear_fwd_channel(q_ref, s_ref, c_ref, g_ref)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(Y.cpu().numpy(), y_ref)
    assert_grad_close(gx.cpu().numpy(), oracle.ste_grad_x_channel(host(d["gy"]), c_ref, g_ref), "grad_x")
