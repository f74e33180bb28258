"""Fused decode forward (bitnet_linear_fwd_decode): the activation quantizer
and the packed GEMV in one launch.

The call promises bit-identical results to bitnet_act_quant followed by
bitnet_linear_fwd, so q, scale_x and Y are compared bit for bit with those
two calls; q and scale_x are also compared bit for bit with the oracle's
act_quant, and Y with the oracle's forward within relative 1e-3.
"""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import assert_y_close, f32_bits_equal, host, to_dev

pytestmark = pytest.mark.gpu


def _case(M, N, K, dtype, seed, special=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g)
    if special == "zero_row":
        x[0] = 0.0
    elif special == "outliers":
        x[:, ::97] *= 40.0
    elif special == "single":
        x.zero_()
        x[:, K // 2] = -2.5
    codes = workloads.ternary_codes(N, K, 0.35, seed=seed + 1)
    gamma = torch.tensor([0.0173], dtype=torch.float32)
    return x.to(dtype), codes, gamma


def _check(x, codes, gamma):
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    xd, gd = to_dev(x), to_dev(gamma)
    y, q, s = bt.bitnet_linear_fwd_decode(xd, wp, gd, want_q=True)
    q2, s2 = bt.bitnet_act_quant(xd)
    y2, _ = bt.bitnet_linear_fwd(q2, s2, wp, gd)
    torch.cuda.synchronize()
    # the two-call path, bit for bit
    assert torch.equal(q, q2)
    assert f32_bits_equal(s.cpu().numpy(), s2.cpu().numpy())
    assert f32_bits_equal(y.cpu().numpy(), y2.cpu().numpy())
    # the oracle
    q_ref, s_ref = oracle.act_quant(host(x))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert f32_bits_equal(s.cpu().numpy(), s_ref)
    _, y_ref = oracle.linear_fwd(q_ref, s_ref, codes.numpy(), float(gamma[0]))
    assert_y_close(y.cpu().numpy(), y_ref)
    return y


# M: one token, a few, 8 / 9, 16; K: one MFMA step, partial 512-element
# blocks (ragged lane chunks), whole 1024-column steps and the 4096 limit
# (fp32: at most 128 row blocks of 256, e.g. 8 rows of 4096); N: one row
# group, ragged groups, more groups than CUs
DECODE_SHAPES = [
    (1, 16, 16), (1, 300, 256), (3, 33, 1040), (8, 100, 528), (8, 257, 4096), (9, 70, 4096),
    (16, 1000, 512), (16, 64, 4096), (5, 4200, 2048), (2, 17, 48), (4, 40, 4096),
    # one token with K % 64 == 0 (the row kernel): a partial last block, N
    # ragged against the 32-row workgroups, the smallest K
    (1, 100, 1088), (1, 4099, 4096), (1, 33, 64),
]


@pytest.mark.parametrize("M,N,K", DECODE_SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_matches_two_calls_and_oracle(M, N, K, dtype):
    print(f"linear_fwd_decode M={M} N={N} K={K} {dtype}", flush=True)
    x, codes, gamma = _case(M, N, K, dtype, seed=M * 131 + N * 7 + K)
    if dtype == torch.float32 and M * -(-K // 256) > 128:
        # beyond the call's documented register budget: rejected, nothing launched
        wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
        with pytest.raises(bt.BitnetError):
            bt.bitnet_linear_fwd_decode(to_dev(x), wp, to_dev(gamma))
        return
    _check(x, codes, gamma)


@pytest.mark.parametrize("special", ["zero_row", "outliers", "single"])
@pytest.mark.parametrize("M", [1, 4])
def test_decode_special_rows(special, M):
    print(f"linear_fwd_decode special {special} M={M}", flush=True)
    x, codes, gamma = _case(M, 96, 1024, torch.bfloat16, seed=7, special=special)
    _check(x, codes, gamma)


@pytest.mark.parametrize("M", [1, 16])
def test_decode_full_size(M):
    # the 7B-class decode layer: K = 4096, N = 11008
    print(f"linear_fwd_decode full size M={M}", flush=True)
    x, codes, gamma = _case(M, 11008, 4096, torch.bfloat16, seed=M)
    _check(x, codes, gamma)


def test_decode_rejects_shapes_beyond_the_register_budget():
    x, codes, gamma = _case(9, 32, 4096, torch.float32, seed=3)
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    with pytest.raises(bt.BitnetError):
        bt.bitnet_linear_fwd_decode(to_dev(x), wp, to_dev(gamma))


def test_decode_without_q_outputs_and_repeat():
    # Xq / scale_x not requested; two calls in a row give the same Y
    x, codes, gamma = _case(6, 200, 768, torch.bfloat16, seed=11)
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    y1, q1, s1 = bt.bitnet_linear_fwd_decode(to_dev(x), wp, to_dev(gamma))
    y2, _, _ = bt.bitnet_linear_fwd_decode(to_dev(x), wp, to_dev(gamma))
    torch.cuda.synchronize()
    assert q1 is None and s1 is None
    assert torch.equal(y1, y2)


def _decode_layout_host(wp: np.ndarray) -> np.ndarray:
    """The decode layout written out with numpy from its definition: the
    16-byte piece of (row group, wave v, lane 16 g + c) is packed bytes
    64 v + 16 g .. + 15 of row 16 * group + c (K = 4096), rows past N zero."""
    N, KB = wp.shape
    G = -(-N // 16)
    pad = np.zeros((G * 16, KB), dtype=np.uint8)
    pad[:N] = wp
    # [group][c][v][g][b] -> [group][v][g][c][b]
    return pad.reshape(G, 16, 16, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("N", [1, 16, 33, 4200, 11008])
def test_pack_decode_matches_the_layout_definition(N):
    print(f"pack_decode N={N}", flush=True)
    codes = workloads.ternary_codes(N, 4096, 0.35, seed=N)
    wp = oracle.pack(codes.numpy())
    wd = bt.bitnet_pack_decode(to_dev(torch.from_numpy(wp)))
    torch.cuda.synchronize()
    assert np.array_equal(wd.cpu().numpy(), _decode_layout_host(wp))


@pytest.mark.parametrize("M,N", [(1, 16), (1, 11008), (3, 33), (8, 4200), (16, 257), (16, 11008)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_layout_gives_the_same_bits(M, N, dtype):
    # the decode layout changes where the weights are read from, nothing else
    print(f"linear_fwd_decode decode layout M={M} N={N} {dtype}", flush=True)
    x, codes, gamma = _case(M, N, 4096, dtype, seed=M * 7 + N)
    wp = to_dev(torch.from_numpy(oracle.pack(codes.numpy())))
    wd = bt.bitnet_pack_decode(wp)
    xd, gd = to_dev(x), to_dev(gamma)
    if dtype == torch.float32 and M > 8:
        # fp32 X: at most 8 rows of 4096 (the call's register budget); the
        # call rejects the shape in either layout and enqueues nothing
        for w_arg, n_arg in ((wp, None), (wd, N)):
            with pytest.raises(bt.BitnetError) as e:
                bt.bitnet_linear_fwd_decode(xd, w_arg, gd, N=n_arg)
            assert e.value.status == -2
        return
    y, q, s = bt.bitnet_linear_fwd_decode(xd, wp, gd, want_q=True)
    y2, q2, s2 = bt.bitnet_linear_fwd_decode(xd, wd, gd, want_q=True, N=N)
    torch.cuda.synchronize()
    assert torch.equal(q, q2)
    assert f32_bits_equal(s.cpu().numpy(), s2.cpu().numpy())
    assert f32_bits_equal(y.cpu().numpy(), y2.cpu().numpy())
    if M == 1 and N == 11008:
        q_ref, s_ref = oracle.act_quant(host(x))
        _, y_ref = oracle.linear_fwd(q_ref, s_ref, codes.numpy(), float(gamma[0]))
        assert_y_close(y2.cpu().numpy(), y_ref)
