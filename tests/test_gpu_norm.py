"""RMSNorm backward (bitnet_rmsnorm_bwd) against the float64 oracle.

The kernel computes in fp32; the oracle is the exact derivative in float64.
Bound, elementwise: |d - r| <= tol * (|r| + RMS(r)) with tol = 1e-4 for fp32
output and 8e-3 for bf16 output (one bf16 rounding, 2^-9, plus fp32 error).
"""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import host, to_dev

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _check(d, ref, tol, what):
    d = d.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bad = np.abs(d - ref) > tol * (np.abs(ref) + rms)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} beyond {tol}; worst "
                           f"{float((np.abs(d - ref) / (np.abs(ref) + rms)).max()):.3e}")


# rows of 1 / 2 / 4 blocks of 512 stay in registers; longer rows stream twice
SHAPES = [(1, 8), (3, 520), (17, 512), (64, 1024), (33, 2056), (5, 4096), (7, 8232), (32, 256)]


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("x_dt,g_dt,o_dt", [("bf16", "f32", "f32"), ("f32", "f32", "f32"),
                                            ("bf16", "bf16", "bf16"), ("f32", "bf16", "f32")])
def test_rmsnorm_bwd(M, K, x_dt, g_dt, o_dt):
    print(f"rmsnorm_bwd M={M} K={K} x={x_dt} g={g_dt} out={o_dt}", flush=True)
    x = workloads.normal((M, K), 1.0, seed=M * 13 + K, dtype=x_dt)
    g = workloads.normal((M, K), 1e-3, seed=M + 7 * K, dtype=g_dt)
    if M > 2:
        x[1] = 0  # all-zero row: r = 1/sqrt(eps), the gradient is r * g
    dx = bt.bitnet_rmsnorm_bwd(to_dev(x), to_dev(g), 1e-5, out_dtype=TORCH_DT[o_dt])
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_bwd(host(x), host(g), 1e-5)
    _check(dx.float().cpu().numpy(), ref, 1e-4 if o_dt == "f32" else 8e-3, "grad_X")


@pytest.mark.parametrize("name", ["small_llama", "qat_70b_mlp"])
def test_rmsnorm_bwd_full_size(name):
    # the layer's RMSNorm input and an fp32 upstream gradient of its shape
    # (the STE backward's grad_x), every element checked
    print(f"rmsnorm_bwd full size {name}", flush=True)
    d = workloads.workload(name)
    M, K = d["M"], d["K"]
    g = workloads.normal((M, K), 1e-3, seed=5, dtype="f32")
    dx = bt.bitnet_rmsnorm_bwd(to_dev(d["x"]), to_dev(g), 1e-5)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_bwd(host(d["x"]), host(g), 1e-5)
    _check(dx.cpu().numpy(), ref, 1e-4, f"grad_X ({name})")


def test_rmsnorm_bwd_is_deterministic():
    x = to_dev(workloads.normal((300, 4096), 1.0, seed=3, dtype="bf16"))
    g = to_dev(workloads.normal((300, 4096), 1e-3, seed=4, dtype="f32"))
    a = bt.bitnet_rmsnorm_bwd(x, g)
    b = bt.bitnet_rmsnorm_bwd(x, g)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
