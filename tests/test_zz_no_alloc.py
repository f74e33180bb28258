"""bitnet_weight_quant_noalloc: the weight quantizer on the library's fixed
device scratch (no workspace, nothing allocated), called through the C ABI
and checked bit for bit against bitnet_weight_quant with a caller workspace
and against the oracle, on calls in a row whose later inputs are smaller (the
scratch keeps the previous call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import f32_bits_equal, host, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(W, Wp, g):
    lib = bt.load_library()
    st = lib.bitnet_weight_quant_noalloc(
        ctypes.c_void_p(W.data_ptr()), bt.BITNET_BF16 if W.dtype == torch.bfloat16 else bt.BITNET_F32,
        W.shape[0], W.shape[1], ctypes.c_void_p(Wp.data_ptr()), ctypes.c_void_p(g.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _case(N, K, dtype, std, seed):
    return workloads.normal((N, K), std, seed, dtype)


# a large layer first, then smaller ones, then a larger one again
SEQUENCE = [(4096, 4096, "bf16", 0.02), (1376, 512, "f32", 0.02), (300, 256, "bf16", 0.05), (33, 64, "f32", 1.0),
            (28672, 1024, "f32", 0.01)]


def test_noalloc_matches_the_workspace_call_on_calls_in_a_row():
    for i, (N, K, dt, std) in enumerate(SEQUENCE):
        print(f"weight_quant_noalloc N={N} K={K} {dt}", flush=True)
        w = _case(N, K, dt, std, seed=10 + i)
        wd = to_dev(w)
        wp = torch.full((N, K // 4), 0xAB, dtype=torch.uint8, device=wd.device)
        g = torch.full((1,), -1.0, dtype=torch.float32, device=wd.device)
        assert _noalloc(wd, wp, g) == 0
        wp_ref, g_ref = bt.bitnet_weight_quant(wd)
        torch.cuda.synchronize()
        assert torch.equal(wp, wp_ref), "packed codes differ from the workspace call"
        assert f32_bits_equal(g.cpu().numpy(), g_ref.cpu().numpy()), "gamma differs from the workspace call"
        c_o, g_o = oracle.weight_quant(host(w))
        assert np.array_equal(wp.cpu().numpy(), oracle.pack(c_o)), "packed codes differ from the oracle"
        assert f32_bits_equal(g.cpu().numpy(), np.array([g_o], np.float32))


def test_noalloc_repeat_is_bit_identical_and_all_zero_weights():
    w = to_dev(_case(512, 1024, "bf16", 0.02, seed=3))
    z = torch.zeros(64, 128, dtype=torch.float32, device=w.device)
    outs = []
    for W in (w, z, w):
        wp = torch.empty(W.shape[0], W.shape[1] // 4, dtype=torch.uint8, device=w.device)
        g = torch.empty(1, dtype=torch.float32, device=w.device)
        assert _noalloc(W, wp, g) == 0
        outs.append((wp, g))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[2][0]) and torch.equal(outs[0][1], outs[2][1])
    # all-zero weights: gamma = 1e-5 and every code 0
    assert float(outs[1][1].cpu()[0]) == np.float32(1e-5) and int(outs[1][0].sum()) == 0


def test_noalloc_at_its_limit_and_beyond():
    N = bt.NOALLOC_MAX_N
    w = to_dev(_case(N, 16, "f32", 0.02, seed=5))
    wp = torch.empty(N, 4, dtype=torch.uint8, device=w.device)
    g = torch.empty(1, dtype=torch.float32, device=w.device)
    assert _noalloc(w, wp, g) == 0
    wp_ref, g_ref = bt.bitnet_weight_quant(w)
    torch.cuda.synchronize()
    assert torch.equal(wp, wp_ref) and torch.equal(g, g_ref)
    # one row more than the scratch holds: rejected before any launch
    w2 = torch.zeros(N + 1, 16, dtype=torch.float32, device=w.device)
    wp2 = torch.empty(N + 1, 4, dtype=torch.uint8, device=w.device)
    assert _noalloc(w2, wp2, g) == bt.BITNET_E_SCRATCH
    with pytest.raises(bt.BitnetError):
        bt.bitnet_weight_quant_noalloc(w2, wp2, g)
