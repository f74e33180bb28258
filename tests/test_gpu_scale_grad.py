"""Gradient of a learned per-output-channel scale (bitnet_channel_scale_grad)
against the oracle.

The call reduces grad_W against the codes, so on seeded grad_W inputs it must
equal the oracle's binary32 row dot (canonical tree) bit for bit.  Chained
after the per-channel STE backward it must match the oracle's float64
definition grad_s[n] = sum_m gy[m,n] * acc[m,n] / scale_x[m] within the
gradient tolerance 2e-2 (elementwise against |r| + RMS(r), and as a relative
Frobenius error)."""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import assert_grad_close, f32_bits_equal, host, to_dev

pytestmark = pytest.mark.gpu


def _codes(N, K, seed, p_zero=0.35):
    return workloads.ternary_codes(N, K, p_zero, seed)


# one block, several blocks with a ragged last one, long rows, many rows
SHAPES = [(1, 16), (3, 48), (5, 256), (17, 272), (33, 1040), (1376, 512), (64, 4112), (7, 16384), (4099, 64)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_scale_grad_is_the_oracle_row_dot_bit_for_bit(N, K):
    print(f"channel_scale_grad N={N} K={K}", flush=True)
    G = workloads.normal((N, K), 1e-3, seed=N + K, dtype="f32")
    codes = _codes(N, K, seed=3 * N + K)
    gs = bt.bitnet_channel_scale_grad(to_dev(G), bt.bitnet_pack_ternary(to_dev(codes)))
    torch.cuda.synchronize()
    ref = oracle.codes_row_dot(G.numpy(), codes.numpy())
    assert f32_bits_equal(gs.cpu().numpy(), ref)


def test_scale_grad_special_rows():
    N, K = 6, 512
    G = workloads.normal((N, K), 1.0, seed=5, dtype="f32")
    codes = _codes(N, K, seed=6)
    codes[0] = 0                       # no code: +0 whatever G holds
    G[1] = -G[1].abs()
    codes[1] = 0                       # products all -0: still +0
    G[2, :4] = torch.tensor([1e8, 1.0, -1e8, 1.0])
    G[2, 4:] = 0.0
    codes[2] = 1                       # the tree order decides: 0, not 1
    codes[3] = 1                       # the row's tree sum
    codes[4] = -1                      # its exact negation
    G[4] = G[3]
    G[5] = 0.0                         # grad_W of zeros
    gs = bt.bitnet_channel_scale_grad(to_dev(G), bt.bitnet_pack_ternary(to_dev(codes))).cpu().numpy()
    ref = oracle.codes_row_dot(G.numpy(), codes.numpy())
    assert f32_bits_equal(gs, ref)
    assert gs[0] == 0.0 and not np.signbit(gs[0]) and not np.signbit(gs[1]) and gs[2] == 0.0
    assert gs[4] == -gs[3]


@pytest.mark.parametrize("M,N,K", [(300, 257, 272), (4096, 64, 4096), (8192, 1376, 512)])
def test_scale_grad_after_the_channel_backward(M, N, K):
    # the end-to-end chain: act-quantized operands and codes -> the
    # per-channel STE backward's grad_W -> grad_s, against the float64
    # definition (the forward's scale does not enter the gradient)
    print(f"channel backward -> scale grad M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + N + K)
    q = torch.from_numpy(rng.integers(-127, 128, (M, K), dtype=np.int8))
    sx = torch.from_numpy(rng.uniform(20, 45, M).astype(np.float32))
    codes = _codes(N, K, seed=N + 5)
    s = torch.from_numpy(rng.uniform(0.005, 0.05, N).astype(np.float32))
    gy = workloads.normal((M, N), 1e-3, seed=M + 2 * N, dtype="bf16")
    wp = bt.bitnet_pack_ternary(to_dev(codes))
    _, gw = bt.bitnet_linear_bwd_ste_channel(to_dev(gy), to_dev(q), to_dev(sx), wp, to_dev(s), want_grad_x=False)
    gs = bt.bitnet_channel_scale_grad(gw, wp)
    torch.cuda.synchronize()
    ref = oracle.channel_scale_grad(host(gy), q.numpy(), sx.numpy(), codes.numpy())
    assert_grad_close(gs.cpu().numpy(), ref, "grad_s")


def test_scale_grad_full_size_qat_70b_mlp():
    # the 70B-shaped MLP layer with per-row gammas: every stage from the
    # workload's X, W and grad_y; grad_s at sampled channels
    print("scale grad full size qat_70b_mlp", flush=True)
    d = workloads.workload("qat_70b_mlp")
    M, N, K = d["M"], d["N"], d["K"]
    Xq, sx = bt.bitnet_act_quant(to_dev(d["x"]))
    wp, g = bt.bitnet_weight_quant_rows(to_dev(d["w"]))
    _, gw = bt.bitnet_linear_bwd_ste_channel(to_dev(d["gy"]), Xq, sx, wp, g, want_grad_x=False)
    gs = bt.bitnet_channel_scale_grad(gw, wp)
    torch.cuda.synchronize()
    del gw
    q_ref, s_ref = oracle.act_quant(host(d["x"]))
    assert np.array_equal(Xq.cpu().numpy(), q_ref) and f32_bits_equal(sx.cpu().numpy(), s_ref)
    c_ref, g_ref = oracle.weight_quant_rows(host(d["w"]))
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(c_ref)) and f32_bits_equal(g.cpu().numpy(), g_ref)
    ns = np.unique(np.concatenate([np.random.default_rng(7).choice(N, 60, replace=False), [0, N - 1]]))
    ref = oracle.channel_scale_grad(host(d["gy"]), q_ref, s_ref, c_ref, ns=ns)
    assert_grad_close(gs.cpu().numpy()[ns], ref, "grad_s (sampled)")
