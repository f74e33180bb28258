"""GPU parity of the BitLinear forward (int8 MFMA GEMM and packed GEMV) and
the STE backward (bf16 MFMA GEMMs) against the CPU oracle.

Forward: int32 accumulators bit-exact, Y within relative 1e-3 of the
float64 reference.  Backward: within 2e-2 (elementwise against |r| + RMS(r)
and as a relative Frobenius error) of the float64 reference.
"""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import assert_grad_close, assert_y_close, host, to_dev

pytestmark = pytest.mark.gpu


def _quantized_operands(M, N, K, seed, p_zero=0.35):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-127, 128, (M, K), generator=g, dtype=torch.int64).to(torch.int8)
    codes = workloads.ternary_codes(N, K, p_zero, seed=seed + 1)
    scale_x = (20.0 + 30.0 * torch.rand(M, generator=g, dtype=torch.float64)).to(torch.float32)
    gamma = torch.tensor([0.0123], dtype=torch.float32)
    return q, codes, scale_x, gamma


FWD_SHAPES = [
    # GEMV path (M <= 16)
    (1, 16, 16), (1, 300, 256), (2, 33, 1040), (5, 257, 4096), (16, 1000, 512),
    (16, 64, 16384), (3, 17, 48),
    # one token with K % 64 == 0 (the row GEMV): one chunk per lane, two, a
    # ragged second chunk, a single chunk for the whole row
    (1, 4099, 64), (1, 33, 8192), (1, 17, 4160), (1, 1000, 4096),
    # 17 to 64 tokens: blocks of 16 through the GEMV (the last block 1 to 16
    # tokens, one token taking the row GEMV)
    (17, 300, 256), (33, 1000, 4096), (64, 257, 1040), (48, 4099, 64), (49, 33, 8192),
    # 65 tokens and more with few tiles (128-row tiles, two workgroups a CU)
    (65, 4100, 1024), (200, 1000, 4096), (129, 257, 2048), (300, 11008, 4096),
    # GEMM path: several tiles plus ragged edges in M, N and K
    (17, 16, 16), (100, 300, 256), (256, 256, 64), (300, 513, 1040),
    (513, 257, 4096), (1000, 40, 48),
    # more 256 x 256 tiles than CUs: workgroups walk several tiles (ragged
    # edges; K a multiple of the step, and not)
    (4200, 4100, 64), (4196, 4132, 48),
]


@pytest.mark.parametrize("M,N,K", FWD_SHAPES)
def test_linear_fwd_exact_acc(M, N, K):
    print(f"linear_fwd M={M} N={N} K={K}", flush=True)
    q, codes, scale_x, gamma = _quantized_operands(M, N, K, seed=M * 31 + N * 7 + K)
    wp = oracle.pack(codes.numpy())
    Y, acc = bt.bitnet_linear_fwd(to_dev(q), to_dev(scale_x), to_dev(torch.from_numpy(wp)),
                                  to_dev(gamma), want_acc=True)
    torch.cuda.synchronize()
    acc_ref, y_ref = oracle.linear_fwd(q.numpy(), scale_x.numpy(), codes.numpy(), float(gamma[0]))
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(Y.cpu().numpy(), y_ref)


def test_linear_fwd_extreme_values():
    # |acc| = 128*K at the int8 extremes: int32 accumulation must not wrap
    M, N, K = 20, 32, 4096
    q = torch.full((M, K), -128, dtype=torch.int8)
    q[::2] = 127
    codes = torch.full((N, K), -1, dtype=torch.int8)
    codes[::3] = 1
    scale_x = torch.full((M,), 3.0)
    gamma = torch.tensor([0.5])
    wp = oracle.pack(codes.numpy())
    for m in (M, 4, 1):  # GEMM, GEMV and one-token row GEMV paths
        Y, acc = bt.bitnet_linear_fwd(to_dev(q[:m]), to_dev(scale_x[:m]), to_dev(torch.from_numpy(wp)),
                                      to_dev(gamma), want_acc=True)
        acc_ref, y_ref = oracle.linear_fwd(q[:m].numpy(), scale_x[:m].numpy(), codes.numpy(), 0.5)
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        assert_y_close(Y.cpu().numpy(), y_ref)


def test_linear_fwd_all_zero_codes_give_zero():
    M, N, K = 40, 48, 256
    q, _, scale_x, gamma = _quantized_operands(M, N, K, seed=5)
    wp = torch.zeros(N, K // 4, dtype=torch.uint8)
    Y, acc = bt.bitnet_linear_fwd(to_dev(q), to_dev(scale_x), to_dev(wp), to_dev(gamma), want_acc=True)
    assert not acc.any().item() and not Y.any().item()


BWD_SHAPES = [(1, 16, 16), (17, 33, 64), (300, 257, 272), (256, 256, 256), (600, 100, 48), (64, 1376, 512)]


@pytest.mark.parametrize("M,N,K", BWD_SHAPES)
@pytest.mark.parametrize("gx_dtype", [torch.float32, torch.bfloat16])
def test_linear_bwd_ste(M, N, K, gx_dtype):
    print(f"linear_bwd M={M} N={N} K={K} {gx_dtype}", flush=True)
    q, codes, scale_x, gamma = _quantized_operands(M, N, K, seed=M + 3 * N + 5 * K)
    gy = workloads.normal((M, N), 1e-3, seed=M + N, dtype="bf16")
    wp = oracle.pack(codes.numpy())
    gx, gw = bt.bitnet_linear_bwd_ste(to_dev(gy), to_dev(q), to_dev(scale_x), to_dev(torch.from_numpy(wp)),
                                      to_dev(gamma), gx_dtype=gx_dtype)
    torch.cuda.synchronize()
    gx_ref = oracle.ste_grad_x(host(gy), codes.numpy(), float(gamma[0]))
    gw_ref = oracle.ste_grad_w(host(gy), q.numpy(), scale_x.numpy())
    assert_grad_close(gx.float().cpu().numpy(), gx_ref, "grad_x")
    assert_grad_close(gw.cpu().numpy(), gw_ref, "grad_W")


# More output tiles than the chip has CUs, so the persistent workgroups take
# a second tile (ragged tile edges on every side): grad_x on the 128 x 128
# tiles (289 of them), grad_x on the 256 x 256 tiles (289), the same with a
# contraction length N % 8 != 0 (one tile a workgroup, element-wise loads),
# and grad_W on the 256 x 256 tiles of a short output (N < 8192: X_deq
# converted in the loop).
LOOP_SHAPES = [(2100, 264, 2096), (4100, 264, 4208), (4100, 261, 4208), (300, 4200, 4208)]


@pytest.mark.parametrize("M,N,K", LOOP_SHAPES)
def test_linear_bwd_more_tiles_than_cus(M, N, K):
    print(f"linear_bwd loop M={M} N={N} K={K}", flush=True)
    q, codes, scale_x, gamma = _quantized_operands(M, N, K, seed=7 * M + N + K)
    gy = workloads.normal((M, N), 1e-3, seed=M + 2 * N, dtype="bf16")
    wp = oracle.pack(codes.numpy())
    gx, gw = bt.bitnet_linear_bwd_ste(to_dev(gy), to_dev(q), to_dev(scale_x), to_dev(torch.from_numpy(wp)),
                                      to_dev(gamma))
    torch.cuda.synchronize()
    gx_ref = oracle.ste_grad_x(host(gy), codes.numpy(), float(gamma[0]))
    gw_ref = oracle.ste_grad_w(host(gy), q.numpy(), scale_x.numpy())
    assert_grad_close(gx.cpu().numpy(), gx_ref, "grad_x")
    assert_grad_close(gw.cpu().numpy(), gw_ref, "grad_W")


# grad_W of these splits its token range over workgroups (fewer than 256
# output tiles, at least 1024 tokens): 4 even splits, 2 with a ragged last
# split and ragged tile edges, 5 with a short last split.  The workspace
# starts as 0xff bytes (its contents on entry must not matter), and grad_W
# is also computed alone.
SPLIT_SHAPES = [(2048, 100, 48), (1100, 257, 272), (3000, 130, 144)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_linear_bwd_token_split(M, N, K):
    print(f"linear_bwd token split M={M} N={N} K={K}", flush=True)
    q, codes, scale_x, gamma = _quantized_operands(M, N, K, seed=M + 7 * N + K)
    gy = workloads.normal((M, N), 1e-3, seed=M + 2 * N, dtype="bf16")
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    nws = bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, M, N, K)
    assert nws > 0
    ws = torch.full((nws,), 255, dtype=torch.uint8, device="cuda")
    args = (to_dev(gy), to_dev(q), to_dev(scale_x), wp, to_dev(gamma))
    gw_ref = oracle.ste_grad_w(host(gy), q.numpy(), scale_x.numpy())
    gx, gw = bt.bitnet_linear_bwd_ste(*args, workspace=ws)
    torch.cuda.synchronize()
    assert_grad_close(gx.cpu().numpy(), oracle.ste_grad_x(host(gy), codes.numpy(), float(gamma[0])), "grad_x")
    assert_grad_close(gw.cpu().numpy(), gw_ref, "grad_W")
    first = gw.cpu().numpy()
    ws.fill_(255)
    _, gw2 = bt.bitnet_linear_bwd_ste(*args, want_grad_x=False, workspace=ws)
    _, gw3 = bt.bitnet_linear_bwd_ste(*args, want_grad_x=False, workspace=ws)
    torch.cuda.synchronize()
    # the split partials are added in split order: identical bits every call
    assert np.array_equal(gw2.cpu().numpy(), first)
    assert np.array_equal(gw3.cpu().numpy(), first)


# grad_W of a tall output (N >= 8192) on the 256 x 256 tiles reads X_deq
# transposed from the workspace (K x M rounded up to 8 tokens, bf16), written
# by a pass before the product: token counts that are not a multiple of 8 (the
# copy's zero padding), ragged tile edges in N and K, a workspace that starts
# as 0xff bytes, repeat calls (identical bits), and the range-gated variant
# whose gate rides in the product's epilogue.
XT_SHAPES = [(300, 8200, 2000), (1029, 8192, 2064), (40, 8448, 1936), (1, 8192, 2048), (7, 8200, 2048)]


@pytest.mark.parametrize("M,N,K", XT_SHAPES)
def test_linear_bwd_grad_w_from_transposed_x(M, N, K):
    print(f"linear_bwd grad_W from X_deq^T M={M} N={N} K={K}", flush=True)
    nws = bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, M, N, K)
    assert nws >= K * ((M + 7) // 8 * 8) * 2  # the transposed copy is in use
    q, codes, scale_x, gamma = _quantized_operands(M, N, K, seed=M + 11 * N + K)
    gy = workloads.normal((M, N), 1e-3, seed=M + 5 * N, dtype="bf16")
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    ws = torch.full((nws,), 255, dtype=torch.uint8, device="cuda")
    args = (to_dev(gy), to_dev(q), to_dev(scale_x), wp, to_dev(gamma))
    _, gw = bt.bitnet_linear_bwd_ste(*args, want_grad_x=False, workspace=ws)
    torch.cuda.synchronize()
    gw_ref = oracle.ste_grad_w(host(gy), q.numpy(), scale_x.numpy())
    first = gw.cpu().numpy()
    assert_grad_close(first, gw_ref, "grad_W")
    ws.fill_(255)
    _, gw2 = bt.bitnet_linear_bwd_ste(*args, want_grad_x=False, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(gw2.cpu().numpy(), first)
    # the gated variant: master weights around the gate bounds
    w = workloads.normal((N, K), 0.5, seed=M + N + 1, dtype="f32")
    _, gwg = bt.bitnet_linear_bwd_ste_gated(*args, to_dev(w), -0.6, 0.6, want_grad_x=False, workspace=ws)
    torch.cuda.synchronize()
    gated_ref = oracle.ste_gate(gw_ref, workloads.host_array(w), -0.6, 0.6)
    got = gwg.cpu().numpy()
    wn = workloads.host_array(w)
    outside = (wn < np.float32(-0.6)) | (wn > np.float32(0.6))
    assert outside.any() and (~outside).any()
    assert (got[outside] == 0).all()
    assert np.array_equal(got[~outside], first[~outside])
    assert_grad_close(got, gated_ref, "gated grad_W")


def test_linear_bwd_single_outputs():
    M, N, K = 70, 90, 128
    q, codes, scale_x, gamma = _quantized_operands(M, N, K, seed=9)
    gy = workloads.normal((M, N), 1e-3, seed=10, dtype="bf16")
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    gx, gw = bt.bitnet_linear_bwd_ste(to_dev(gy), to_dev(q), to_dev(scale_x), wp, to_dev(gamma),
                                      want_grad_W=False)
    assert gw is None
    assert_grad_close(gx.cpu().numpy(), oracle.ste_grad_x(host(gy), codes.numpy(), float(gamma[0])), "grad_x")
    gx, gw = bt.bitnet_linear_bwd_ste(to_dev(gy), to_dev(q), to_dev(scale_x), wp, to_dev(gamma),
                                      want_grad_x=False)
    assert gx is None
    assert_grad_close(gw.cpu().numpy(), oracle.ste_grad_w(host(gy), q.numpy(), scale_x.numpy()), "grad_W")


def test_end_to_end_small_layer():
    # RMSNorm + act quant, weight quant, forward, STE backward: every stage
    # against the oracle on the same seeded inputs
    d = workloads.linear_inputs(96, 200, 320, x_dtype="bf16", w_dtype="f32", seed=21)
    out = bt.bitlinear_forward(to_dev(d["x"]), to_dev(d["w"]), want_acc=True)
    q_ref, s_ref = oracle.act_quant(host(d["x"]))
    c_ref, g_ref = oracle.weight_quant(host(d["w"]))
    assert np.array_equal(out["Xq"].cpu().numpy(), q_ref)
    assert np.array_equal(out["W_packed"].cpu().numpy(), oracle.pack(c_ref))
    acc_ref, y_ref = oracle.linear_fwd(q_ref, s_ref, c_ref, g_ref)
    assert np.array_equal(out["acc"].cpu().numpy(), acc_ref)
    assert_y_close(out["Y"].cpu().numpy(), y_ref)
    gx, gw = bt.bitnet_linear_bwd_ste(to_dev(d["gy"]), out["Xq"], out["scale_x"], out["W_packed"], out["gamma"])
    assert_grad_close(gx.cpu().numpy(), oracle.ste_grad_x(host(d["gy"]), c_ref, g_ref), "grad_x")
    assert_grad_close(gw.cpu().numpy(), oracle.ste_grad_w(host(d["gy"]), q_ref, s_ref), "grad_W")


def test_forward_paths_give_the_same_bits():
    # the same token rows through the GEMM (M = 40), the GEMV (M = 9, 4) and
    # the one-token row GEMV (M = 1): one epilogue formula, so identical bits
    M, N, K = 40, 300, 1024
    q, codes, scale_x, gamma = _quantized_operands(M, N, K, seed=77)
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    qd, sd, gd = to_dev(q), to_dev(scale_x), to_dev(gamma)
    y_all, a_all = bt.bitnet_linear_fwd(qd, sd, wp, gd, want_acc=True)
    for m in (9, 4, 1):
        y, a = bt.bitnet_linear_fwd(qd[:m].contiguous(), sd[:m].contiguous(), wp, gd, want_acc=True)
        torch.cuda.synchronize()
        assert torch.equal(a, a_all[:m])
        assert torch.equal(y.view(torch.int32), y_all[:m].view(torch.int32))
