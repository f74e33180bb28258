"""The largest shapes the boundary accepts, on the GPU against the oracle.

- The longest contraction of the forward (K = 2^24 - 16): int8 extremes
  times +-1 codes give |acc| = 128 K, within 2^11 of the int32 limit.  The
  expected accumulators are the closed form (every row of q and of the codes
  constant: acc = q_m * c_n * K), Y the oracle's dequantization of them.
- The widest forward output (N = 2^23 - 1; tile stores use 32-bit offsets):
  accumulators at sampled columns against the oracle, both the GEMV (M <= 16)
  and the GEMM.
- More than 2^31 elements in one operand (65552 x 32768): act_quant,
  weight_quant, the forward and both STE products, each checked against the
  oracle on sampled rows, columns or entries that include the last rows
  (whose element offsets pass 2^31).  Inputs are drawn on the device with a
  seeded torch generator; the oracle sees copies of the sampled parts.
- The STE backward at the widest output (N = 2^23 - 1: grad_x contracts
  over it) and the longest rows (K = 2^24 - 16), at sampled rows and columns.
"""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import DEV, assert_grad_close, assert_y_close, f32_bits_equal, host

pytestmark = pytest.mark.gpu

BIG_M, BIG_K = 65552, 32768  # M * K = 2^31 + 2^19
assert BIG_M * BIG_K > 2 ** 31


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device=DEV).manual_seed(seed)


def _rows(M: int, seed: int, count: int = 24) -> np.ndarray:
    r = np.random.default_rng(seed).choice(M, size=count, replace=False)
    return np.unique(np.concatenate([r, [0, 1, M - 16, M - 2, M - 1]]))


def test_fwd_longest_contraction():
    K = (1 << 24) - 16
    M, N = 20, 24
    print(f"linear_fwd longest K={K} M={M} N={N}", flush=True)
    qv = np.where(np.arange(M) % 2 == 0, 127, -128).astype(np.int8)       # per row
    cv = np.array([1, -1, 0], dtype=np.int8)[np.arange(N) % 3]              # per code row
    q = torch.from_numpy(qv).to(DEV)[:, None].expand(M, K).contiguous()
    # packed rows: 0x55 = four +1 codes, 0xAA = four -1 codes, 0 = zeros
    byte = torch.tensor([0x55, 0xAA, 0x00], dtype=torch.uint8)[torch.arange(N) % 3]
    wp = byte.to(DEV)[:, None].expand(N, K // 4).contiguous()
    scale_x = torch.linspace(20.0, 40.0, M, dtype=torch.float32, device=DEV)
    gamma = torch.tensor([0.0137], dtype=torch.float32, device=DEV)
    Y, acc = bt.bitnet_linear_fwd(q, scale_x, wp, gamma, want_acc=True)
    torch.cuda.synchronize()
    acc_ref = (qv.astype(np.int64)[:, None] * cv.astype(np.int64)[None, :] * K)
    assert np.abs(acc_ref).max() == 128 * K and 128 * K < 2 ** 31
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    y_ref = oracle.dequant(acc_ref.astype(np.int32), scale_x.cpu().numpy(), float(gamma[0]))
    assert_y_close(Y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("M", [1, 16, 40])  # one-token row GEMV, GEMV, GEMM
def test_fwd_widest_output(M):
    N, K = (1 << 23) - 1, 16
    print(f"linear_fwd widest N={N} M={M} K={K}", flush=True)
    codes = workloads.ternary_codes(N, K, 0.35, seed=M)
    q = workloads.int8_uniform(M, K, seed=M + 1)
    scale_x = torch.full((M,), 30.0)
    gamma = torch.tensor([0.02], dtype=torch.float32)
    wp = torch.from_numpy(oracle.pack(codes.numpy())).to(DEV)
    Y, acc = bt.bitnet_linear_fwd(q.to(DEV), scale_x.to(DEV), wp, gamma.to(DEV), want_acc=True)
    rng = np.random.default_rng(M)
    cols = np.unique(np.concatenate([rng.integers(0, N, 3000), np.arange(N - 300, N), np.arange(300)]))
    ci = torch.from_numpy(cols).to(DEV)
    acc_s = acc.index_select(1, ci).cpu().numpy()
    y_s = Y.index_select(1, ci).cpu().numpy()
    torch.cuda.synchronize()
    acc_ref, y_ref = oracle.linear_fwd(q.numpy(), scale_x.numpy(), codes.numpy()[cols], float(gamma[0]))
    assert np.array_equal(acc_s, acc_ref)
    assert_y_close(y_s, y_ref)


@pytest.fixture(scope="module")
def big():
    """X bf16, q, scale_x, W bf16, codes of a layer with M * K > 2^31."""
    print(f"large operands M={BIG_M} K={BIG_K}", flush=True)
    x = torch.randn(BIG_M, BIG_K, generator=_gen(1), device=DEV, dtype=torch.float32).to(torch.bfloat16)
    Xq, scale_x = bt.bitnet_act_quant(x)
    out = {"x": x, "Xq": Xq, "scale_x": scale_x}
    yield out
    out.clear()
    torch.cuda.empty_cache()


def test_act_quant_past_2_31_elements(big):
    rows = _rows(BIG_M, 3)
    ri = torch.from_numpy(rows).to(DEV)
    q_ref, s_ref = oracle.act_quant(host(big["x"].index_select(0, ri)))
    assert np.array_equal(big["Xq"].index_select(0, ri).cpu().numpy(), q_ref)
    assert f32_bits_equal(big["scale_x"].index_select(0, ri).cpu().numpy(), s_ref)


def test_weight_quant_past_2_31_elements():
    # W [65552, 32768]: the codes and gamma of the whole matrix against the oracle
    print(f"weight_quant N={BIG_M} K={BIG_K}", flush=True)
    w = (torch.randn(BIG_M, BIG_K, generator=_gen(2), device=DEV, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    wp, gamma = bt.bitnet_weight_quant(w)
    torch.cuda.synchronize()
    w_host = host(w)
    del w
    codes_ref, g_ref = oracle.weight_quant(w_host)
    del w_host
    assert f32_bits_equal(gamma.cpu().numpy(), np.array([g_ref], np.float32))
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(codes_ref))


def test_linear_past_2_31_elements(big):
    # forward and STE backward with q [65552, 32768] (2^31 + 2^19 bytes)
    N = 48
    print(f"linear fwd/bwd M={BIG_M} N={N} K={BIG_K}", flush=True)
    codes = workloads.ternary_codes(N, BIG_K, 0.35, seed=5)
    wp = torch.from_numpy(oracle.pack(codes.numpy())).to(DEV)
    gamma = torch.tensor([0.0123], dtype=torch.float32, device=DEV)
    # seeded int8 operands and scales of this size (inputs, not act_quant's
    # outputs: every reference below is computed from them)
    Xq = torch.randint(-127, 128, (BIG_M, BIG_K), generator=_gen(9), device=DEV, dtype=torch.int32).to(torch.int8)
    scale_x = torch.linspace(20.0, 40.0, BIG_M, dtype=torch.float32, device=DEV)
    gy = (torch.randn(BIG_M, N, generator=_gen(6), device=DEV, dtype=torch.float32) * 1e-3).to(torch.bfloat16)
    Y, acc = bt.bitnet_linear_fwd(Xq, scale_x, wp, gamma, want_acc=True)
    gx, gw = bt.bitnet_linear_bwd_ste(gy, Xq, scale_x, wp, gamma)
    torch.cuda.synchronize()
    rows = _rows(BIG_M, 7)
    ri = torch.from_numpy(rows).to(DEV)
    q_rows = Xq.index_select(0, ri).cpu().numpy()
    s_rows = scale_x.index_select(0, ri).cpu().numpy()
    acc_ref, y_ref = oracle.linear_fwd(q_rows, s_rows, codes.numpy(), float(gamma[0]))
    assert np.array_equal(acc.index_select(0, ri).cpu().numpy(), acc_ref)
    assert_y_close(Y.index_select(0, ri).cpu().numpy(), y_ref)
    gy_h = host(gy)
    gx_ref = oracle.ste_grad_x(gy_h[rows], codes.numpy(), float(gamma[0]))
    assert_grad_close(gx.index_select(0, ri).cpu().numpy(), gx_ref, "grad_x")
    # grad_W at sampled columns: the whole token range of those q columns
    cols = np.unique(np.concatenate([np.random.default_rng(8).integers(0, BIG_K, 40), [0, BIG_K - 1]]))
    ci = torch.from_numpy(cols).to(DEV)
    q_cols = Xq.index_select(1, ci).cpu().numpy()
    gw_ref = oracle.ste_grad_w(gy_h, q_cols, scale_x.cpu().numpy())
    assert_grad_close(gw.index_select(1, ci).cpu().numpy(), gw_ref, "grad_W")


def test_bwd_widest_output():
    # N = 2^23 - 1: grad_x contracts over 8.4M output features, grad_W has
    # 8.4M rows
    M, N, K = 300, (1 << 23) - 1, 16
    print(f"linear_bwd widest N={N} M={M} K={K}", flush=True)
    codes = workloads.ternary_codes(N, K, 0.35, seed=11)
    q = workloads.int8_uniform(M, K, seed=12)
    scale_x = torch.linspace(20.0, 40.0, M, dtype=torch.float32)
    gamma = 0.0123
    wp = torch.from_numpy(oracle.pack(codes.numpy())).to(DEV)
    gy = (torch.randn(M, N, generator=_gen(13), device=DEV, dtype=torch.float32) * 1e-3).to(torch.bfloat16)
    gx, gw = bt.bitnet_linear_bwd_ste(gy, q.to(DEV), scale_x.to(DEV), wp,
                                      torch.tensor([gamma], dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    rows = _rows(M, 14)
    ri = torch.from_numpy(rows).to(DEV)
    gx_ref = oracle.ste_grad_x(host(gy.index_select(0, ri)), codes.numpy(), gamma)
    assert_grad_close(gx.index_select(0, ri).cpu().numpy(), gx_ref, "grad_x")
    rng = np.random.default_rng(15)
    ns = np.unique(np.concatenate([rng.integers(0, N, 3000), np.arange(N - 300, N), np.arange(300)]))
    ni = torch.from_numpy(ns).to(DEV)
    gw_ref = oracle.ste_grad_w(host(gy.index_select(1, ni)), q.numpy(), scale_x.numpy())
    assert_grad_close(gw.index_select(0, ni).cpu().numpy(), gw_ref, "grad_W")


def test_bwd_longest_rows():
    # K = 2^24 - 16: grad_x rows and grad_W rows of 16.8M entries
    M, N, K = 20, 24, (1 << 24) - 16
    print(f"linear_bwd longest K={K} M={M} N={N}", flush=True)
    q = torch.randint(-127, 128, (M, K), generator=_gen(16), device=DEV, dtype=torch.int32).to(torch.int8)
    codes = torch.randint(-1, 2, (N, K), generator=_gen(17), device=DEV, dtype=torch.int32).to(torch.int8)
    codes_h = codes.cpu().numpy()
    wp = torch.from_numpy(oracle.pack(codes_h)).to(DEV)
    del codes
    scale_x = torch.linspace(20.0, 40.0, M, dtype=torch.float32)
    gamma = 0.0123
    gy = (torch.randn(M, N, generator=_gen(18), device=DEV, dtype=torch.float32) * 1e-3).to(torch.bfloat16)
    gx, gw = bt.bitnet_linear_bwd_ste(gy, q, scale_x.to(DEV), wp,
                                      torch.tensor([gamma], dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    gy_h = host(gy)
    rng = np.random.default_rng(19)
    ks = np.unique(np.concatenate([rng.integers(0, K, 4000), np.arange(K - 300, K), np.arange(300)]))
    ki = torch.from_numpy(ks).to(DEV)
    gx_ref = oracle.ste_grad_x(gy_h, np.ascontiguousarray(codes_h[:, ks]), gamma)
    assert_grad_close(gx.index_select(1, ki).cpu().numpy(), gx_ref, "grad_x")
    gw_ref = oracle.ste_grad_w(gy_h, q.index_select(1, ki).cpu().numpy(), scale_x.numpy())
    assert_grad_close(gw.index_select(1, ki).cpu().numpy(), gw_ref, "grad_W")
