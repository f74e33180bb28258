"""Range-gated STE (bitnet_linear_bwd_ste_gated) and the master-weight clamp
(bitnet_weight_clamp) against the oracle.

Gated grad_W: the gate is a decision on the weights (exact on both sides), so
every blocked entry must be exactly 0 and every passed entry within the
gradient tolerance of the ungated oracle value; grad_x must be bit-identical
to the ungated call.  The clamp is bit-exact.
"""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import f32_bits_equal, host, to_dev

pytestmark = pytest.mark.gpu


def _operands(M, N, K, w_dtype, seed):
    d = workloads.linear_inputs(M, N, K, x_dtype="bf16", w_dtype=w_dtype, w_std=0.8, seed=seed)
    w = d["w"]
    w.view(-1)[:4] = torch.tensor([-1.0, 1.0, -0.5, 1.5], dtype=w.dtype)  # the bounds hit exactly
    x, wd, gy = to_dev(d["x"]), to_dev(w), to_dev(d["gy"])
    Xq, sx = bt.bitnet_act_quant(x)
    Wp, gamma = bt.bitnet_weight_quant(wd)
    return d, wd, gy, Xq, sx, Wp, gamma


def _oracle_q(d, Xq, sx):
    """The oracle's q and scale_x of the layer's X, checked equal to the
    library's (the references below are built from the oracle's)."""
    q_ref, s_ref = oracle.act_quant(host(d["x"]))
    assert np.array_equal(Xq.cpu().numpy(), q_ref) and f32_bits_equal(sx.cpu().numpy(), s_ref)
    return q_ref, s_ref


# plain 128x128 tiles, a token split (2048 tokens over 100x48), 256x256 tiles
GATE_SHAPES = [(300, 257, 272), (2048, 100, 48), (64, 1024, 16384)]


@pytest.mark.parametrize("M,N,K", GATE_SHAPES)
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_gated_ste_grad_w(M, N, K, w_dtype):
    print(f"gated STE M={M} N={N} K={K} W={w_dtype}", flush=True)
    d, wd, gy, Xq, sx, Wp, gamma = _operands(M, N, K, w_dtype, seed=M + N + K)
    gx0, _ = bt.bitnet_linear_bwd_ste(gy, Xq, sx, Wp, gamma, want_grad_W=False)
    torch.cuda.synchronize()
    q_ref, s_ref = _oracle_q(d, Xq, sx)
    ref = oracle.ste_grad_w(host(gy), q_ref, s_ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    for lo, hi in ((-1.0, 1.0), (-0.5, 0.25)):
        gx, gw = bt.bitnet_linear_bwd_ste_gated(gy, Xq, sx, Wp, gamma, wd, lo, hi)
        torch.cuda.synchronize()
        assert torch.equal(gx, gx0), "grad_x must not depend on the gate"
        gated = oracle.ste_gate(ref, host(wd), lo, hi)
        g = gw.cpu().numpy()
        wf = wd.float().cpu().numpy()
        out = (wf < lo) | (wf > hi)
        assert out.any() and (~out).any()
        assert not g[out].any(), "blocked entries must be exactly 0"
        # passed entries: the ungated gradient's tolerance
        err = np.abs(g[~out].astype(np.float64) - gated[~out])
        assert (err <= 2e-2 * (np.abs(gated[~out]) + rms)).all()


def test_gated_ste_grad_w_only_and_wide_range():
    # grad_W alone (token split, reduction kernel gates), and a range that
    # blocks nothing equals the plain STE bit for bit
    M, N, K = 2048, 100, 48
    d, wd, gy, Xq, sx, Wp, gamma = _operands(M, N, K, "f32", seed=3)
    _, gw_all = bt.bitnet_linear_bwd_ste_gated(gy, Xq, sx, Wp, gamma, wd, -1e30, 1e30, want_grad_x=False)
    _, gw_plain = bt.bitnet_linear_bwd_ste(gy, Xq, sx, Wp, gamma, want_grad_x=False)
    _, gw_none = bt.bitnet_linear_bwd_ste_gated(gy, Xq, sx, Wp, gamma, wd, 2.0, 1.0, want_grad_x=False)
    torch.cuda.synchronize()
    assert torch.equal(gw_all, gw_plain)
    assert not gw_none.any()


@pytest.mark.parametrize("N,K", [(7, 13), (1, 3), (1376, 512), (33, 1000)])
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_weight_clamp(N, K, w_dtype):
    print(f"weight clamp N={N} K={K} {w_dtype}", flush=True)
    w = workloads.normal((N, K), 1.5, seed=N * K, dtype=w_dtype)
    for lo, hi in ((-1.0, 1.0), (-0.3, 0.7)):
        wd = to_dev(w)
        bt.bitnet_weight_clamp(wd, lo, hi)
        torch.cuda.synchronize()
        want = oracle.weight_clamp(host(w), lo, hi)
        got = host(wd)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
