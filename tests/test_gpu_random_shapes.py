"""Parity on seeded random shapes: every call against the oracle (or, for the
fused calls, against the two calls they replace) on shapes drawn once from a
fixed seed, so that ragged edges land at places the hand-picked shapes of the
other files do not.  Sizes stay small enough for the oracle to finish in
seconds (at most 3e8 multiply-adds per product).
"""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import assert_grad_close, assert_y_close, f32_bits_equal, host, to_dev

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20251203)


def _dim(lo, hi, mult=1):
    return int(_rng.integers(lo // mult, hi // mult + 1)) * mult


def _product_shapes(count, m_hi, n_hi, k_hi, cap):
    out = []
    while len(out) < count:
        M = _dim(1, m_hi) if _rng.random() < 0.75 else _dim(1, 16)
        N, K = _dim(1, n_hi), _dim(16, k_hi, 16)
        if M * N * K <= cap:
            out.append((M, N, K))
    return out


ACT_SHAPES = [(_dim(1, 300), _dim(4, 20000, 4), str(_rng.choice(["f32", "bf16"]))) for _ in range(12)]
WQ_SHAPES = [(_dim(1, 600), _dim(4, 5000, 4), str(_rng.choice(["f32", "bf16"]))) for _ in range(10)]
# the GEMV (M <= 16), the one-token row GEMV, and the GEMM with ragged tiles
FWD_SHAPES = _product_shapes(14, 700, 700, 4200, 1e8) + [(1, _dim(1, 3000), _dim(64, 8192, 64)) for _ in range(2)]
# backward, including token ranges long enough for grad_W's token split
BWD_SHAPES = _product_shapes(10, 4000, 400, 1200, 3e8)
DEC_SHAPES = [(_dim(1, 16), _dim(1, 3000), _dim(16, 4096, 16)) for _ in range(10)] + \
    [(1, _dim(1, 3000), _dim(64, 4096, 64)) for _ in range(2)]
# large weight matrices (gamma published by one pack workgroup: the five-wave
# reader form when one round of workgroups covers the matrix, the four-wave
# form otherwise), with token counts on both sides of the weight bytes so
# that the two-quantizer call takes each of its two orders
# (K mostly a whole number of row blocks, which the two-quantizer call needs
# for its fused launches; now and then a ragged one)
def _big_k():
    return int(_rng.choice([2048, 4096, 8192])) if _rng.random() < 0.75 else _dim(2048, 8192, 4)


BIG_WQ_SHAPES = [(_dim(1500, 9000), _big_k(), str(_rng.choice(["f32", "bf16"])), _dim(1, 3) / 2)
                 for _ in range(8)]


def _x(M, K, dt, seed):
    return workloads.normal((M, K), 1.0, seed=seed, dtype=dt)


@pytest.mark.parametrize("M,K,dt", ACT_SHAPES)
def test_random_act_quant(M, K, dt):
    print(f"random act_quant M={M} K={K} {dt}", flush=True)
    x = _x(M, K, dt, seed=M + K)
    q, s = bt.bitnet_act_quant(to_dev(x))
    q_ref, s_ref = oracle.act_quant(host(x))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert f32_bits_equal(s.cpu().numpy(), s_ref)


@pytest.mark.parametrize("N,K,dt", WQ_SHAPES)
def test_random_weight_quant(N, K, dt):
    print(f"random weight_quant N={N} K={K} {dt}", flush=True)
    w = workloads.normal((N, K), 0.02, seed=N * 3 + K, dtype=dt)
    wp, g = bt.bitnet_weight_quant(to_dev(w))
    c_ref, g_ref = oracle.weight_quant(host(w))
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(c_ref))
    assert f32_bits_equal(g.cpu().numpy(), np.array([g_ref], np.float32))


def _operands(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-127, 128, (M, K), generator=g, dtype=torch.int64).to(torch.int8)
    codes = workloads.ternary_codes(N, K, 0.35, seed=seed + 1)
    scale_x = (20.0 + 30.0 * torch.rand(M, generator=g, dtype=torch.float64)).to(torch.float32)
    return q, codes, scale_x, torch.tensor([0.0123], dtype=torch.float32)


@pytest.mark.parametrize("M,N,K", FWD_SHAPES)
def test_random_linear_fwd(M, N, K):
    print(f"random linear_fwd M={M} N={N} K={K}", flush=True)
    q, codes, scale_x, gamma = _operands(M, N, K, seed=M * 7 + N * 3 + K)
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    Y, acc = bt.bitnet_linear_fwd(to_dev(q), to_dev(scale_x), wp, to_dev(gamma), want_acc=True)
    acc_ref, y_ref = oracle.linear_fwd(q.numpy(), scale_x.numpy(), codes.numpy(), float(gamma[0]))
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(Y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("M,N,K", BWD_SHAPES)
def test_random_linear_bwd(M, N, K):
    print(f"random linear_bwd M={M} N={N} K={K}", flush=True)
    q, codes, scale_x, gamma = _operands(M, N, K, seed=M + N * 5 + K * 3)
    gy = workloads.normal((M, N), 1e-3, seed=M + N, dtype="bf16")
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    gx, gw = bt.bitnet_linear_bwd_ste(to_dev(gy), to_dev(q), to_dev(scale_x), wp, to_dev(gamma))
    torch.cuda.synchronize()
    assert_grad_close(gx.cpu().numpy(), oracle.ste_grad_x(host(gy), codes.numpy(), float(gamma[0])), "grad_x")
    assert_grad_close(gw.cpu().numpy(), oracle.ste_grad_w(host(gy), q.numpy(), scale_x.numpy()), "grad_W")


@pytest.mark.parametrize("M,N,K", DEC_SHAPES)
def test_random_decode_and_quant_operands(M, N, K):
    print(f"random decode / quant_operands M={M} N={N} K={K}", flush=True)
    x = to_dev(_x(M, K, "bf16", seed=M + N + K))
    codes = workloads.ternary_codes(N, K, 0.35, seed=N + K)
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    gamma = to_dev(torch.tensor([0.0173], dtype=torch.float32))
    y, q, s = bt.bitnet_linear_fwd_decode(x, wp, gamma, want_q=True)
    q2, s2 = bt.bitnet_act_quant(x)
    y2, _ = bt.bitnet_linear_fwd(q2, s2, wp, gamma)
    torch.cuda.synchronize()
    assert torch.equal(q, q2)
    assert f32_bits_equal(s.cpu().numpy(), s2.cpu().numpy())
    assert f32_bits_equal(y.cpu().numpy(), y2.cpu().numpy())
    # both quantizers in one call against the two calls
    w = to_dev(workloads.normal((N, K), 0.02, seed=K, dtype="f32"))
    q3, s3, wp3, g3 = bt.bitnet_quant_operands(x, w)
    wp4, g4 = bt.bitnet_weight_quant(w)
    torch.cuda.synchronize()
    assert torch.equal(q3, q2) and f32_bits_equal(s3.cpu().numpy(), s2.cpu().numpy())
    assert torch.equal(wp3, wp4) and f32_bits_equal(g3.cpu().numpy(), g4.cpu().numpy())


@pytest.mark.parametrize("N,K,dt,tokens_per_row", BIG_WQ_SHAPES)
def test_random_large_weight_quant_counted_and_quant_operands(N, K, dt, tokens_per_row):
    M = max(1, int(N * tokens_per_row))
    print(f"random large weight quant N={N} K={K} {dt}, quant_operands M={M}", flush=True)
    w = workloads.normal((N, K), 0.02, seed=N * 3 + K, dtype=dt)
    x = _x(M, K, "bf16", seed=M + K)
    c_ref, g_ref = oracle.weight_quant(host(w))
    packed_ref = oracle.pack(c_ref)
    wp, g = bt.bitnet_weight_quant(to_dev(w))
    wp2, g2, counts = bt.bitnet_weight_quant_counted(to_dev(w))
    q3, s3, wp3, g3 = bt.bitnet_quant_operands(to_dev(x), to_dev(w))
    torch.cuda.synchronize()
    for p_, g_ in ((wp, g), (wp2, g2), (wp3, g3)):
        assert np.array_equal(p_.cpu().numpy(), packed_ref)
        assert f32_bits_equal(g_.cpu().numpy(), np.array([g_ref], np.float32))
    assert np.array_equal(counts.cpu().numpy(), oracle.code_counts(packed_ref, K).astype(np.int64))
    q_ref, s_ref = oracle.act_quant(host(x))
    assert np.array_equal(q3.cpu().numpy(), q_ref)
    assert f32_bits_equal(s3.cpu().numpy(), s_ref)
