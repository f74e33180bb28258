"""Seeded synthetic inputs for the BitLinear hot path.

This module only draws random tensors of the workloads' shapes and
distributions; it holds none of the method's arithmetic, so both the HIP
path and the CPU oracle can take their inputs from it.  Every tensor comes
from its own torch CPU generator (seeds: X = 0, W = 1, grad_y = 2,
auxiliaries = 3, each offset by `seed`), so the same call gives the same bits
on any host running this torch build.  bf16 tensors are drawn in fp32 and
rounded to nearest-even.

Workloads (LLM-layer shapes; tokens M, in-features K, out-features N):
  tiny         M=32,   K=256,  N=256    X fp32 N(0,1), W fp32 N(0,0.02)
  small_llama  M=8192, K=512,  N=1376   X bf16 N(0,1), W fp32 N(0,0.02),
                                        grad_y bf16 N(0,1e-3)
  decode_7b    M=1..16, K=4096, N=11008 int8 activations uniform in
                                        [-127,127]; ternary codes i.i.d. with
                                        P(0)=0.35, P(+1)=P(-1)=0.325;
                                        gamma = 0.02*sqrt(2/pi)
  prefill_7b   M=8192, K=4096, N=4096   X bf16 N(0,1) with 4 (0.1%) outlier
                                        columns x20, W bf16 N(0,0.02)
  qat_70b_mlp  M=4096, K=8192, N=28672  X bf16 N(0,1), W fp32 N(0,0.01),
                                        grad_y bf16 N(0,1e-3)
"""
import math

import torch

SEED_X, SEED_W, SEED_GY, SEED_AUX = 0, 1, 2, 3
SEED_XDEC = 4  # decode's unquantized activations

WORKLOADS = {
    "tiny": dict(M=32, K=256, N=256, x_dtype="f32", w_dtype="f32", w_std=0.02, gy=False),
    "small_llama": dict(M=8192, K=512, N=1376, x_dtype="bf16", w_dtype="f32", w_std=0.02, gy=True, gy_std=1e-3),
    "decode_7b": dict(M=16, K=4096, N=11008, p_zero=0.35),
    "prefill_7b": dict(M=8192, K=4096, N=4096, x_dtype="bf16", w_dtype="bf16", w_std=0.02, gy=False,
                       outlier_frac=0.001, outlier_gain=20.0),
    "qat_70b_mlp": dict(M=4096, K=8192, N=28672, x_dtype="bf16", w_dtype="f32", w_std=0.01, gy=True, gy_std=1e-3),
}

DECODE_MS = (1, 2, 4, 8, 16)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def normal(shape, std: float, seed: int, dtype: str = "f32") -> torch.Tensor:
    t = torch.randn(*shape, generator=_gen(seed), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(_dtype(dtype)).contiguous()


def outlier_columns(K: int, frac: float, seed: int) -> torch.Tensor:
    """round(frac*K) distinct column indices, seeded."""
    n_out = max(1, int(round(frac * K)))
    return torch.randperm(K, generator=_gen(seed))[:n_out].sort().values


def linear_inputs(M: int, N: int, K: int, x_dtype: str = "bf16", w_dtype: str = "f32",
                  w_std: float = 0.02, gy: bool = True, gy_std: float = 1e-3, seed: int = 0,
                  outlier_frac: float = 0.0, outlier_gain: float = 20.0) -> dict:
    """X [M,K], W [N,K] and optionally grad_y [M,N] for one BitLinear layer."""
    x = torch.randn(M, K, generator=_gen(SEED_X + seed), dtype=torch.float32)
    cols = None
    if outlier_frac > 0.0:
        cols = outlier_columns(K, outlier_frac, SEED_AUX + seed)
        x[:, cols] *= outlier_gain
    out = {
        "x": x.to(_dtype(x_dtype)).contiguous(),
        "w": normal((N, K), w_std, SEED_W + seed, w_dtype),
        "M": M, "N": N, "K": K,
    }
    if cols is not None:
        out["outlier_cols"] = cols
    if gy:
        out["gy"] = normal((M, N), gy_std, SEED_GY + seed, "bf16")
    return out


def ternary_codes(N: int, K: int, p_zero: float, seed: int) -> torch.Tensor:
    """int8 [N,K] i.i.d. in {-1,0,+1}: P(0)=p_zero, P(+1)=P(-1)=(1-p_zero)/2."""
    u = torch.rand(N, K, generator=_gen(seed), dtype=torch.float64)
    c = torch.zeros(N, K, dtype=torch.int8)
    p_pos = p_zero + (1.0 - p_zero) / 2.0
    c[(u >= p_zero) & (u < p_pos)] = 1
    c[u >= p_pos] = -1
    return c


def int8_uniform(M: int, K: int, seed: int, lo: int = -127, hi: int = 127) -> torch.Tensor:
    return torch.randint(lo, hi + 1, (M, K), generator=_gen(seed), dtype=torch.int64).to(torch.int8)


def decode_inputs(M: int, K: int = 4096, N: int = 11008, p_zero: float = 0.35, seed: int = 0) -> dict:
    """Pre-quantized decode workload: int8 activations, ternary codes, scales.

    The per-token activation scales are drawn uniform in [25, 45] (the range
    127/max|z| takes for a 4096-wide N(0,1) row); gamma is the mean |w| of
    N(0, 0.02) weights.
    """
    q = int8_uniform(M, K, SEED_X + seed)
    codes = ternary_codes(N, K, p_zero, SEED_W + seed)
    scale_x = (25.0 + 20.0 * torch.rand(M, generator=_gen(SEED_AUX + seed), dtype=torch.float64)).to(torch.float32)
    gamma = torch.tensor([0.02 * math.sqrt(2.0 / math.pi)], dtype=torch.float32)
    # the unquantized layer input of the same tokens (bf16 N(0,1)), for the
    # fused decode call that quantizes it itself
    x = torch.randn(M, K, generator=_gen(SEED_XDEC + seed), dtype=torch.float32).to(torch.bfloat16)
    return {"q": q, "codes": codes, "scale_x": scale_x, "gamma": gamma, "x": x, "M": M, "N": N, "K": K}


def workload(name: str, seed: int = 0, M: int = None) -> dict:
    """Inputs of a named workload (decode_7b takes M in 1..16)."""
    spec = dict(WORKLOADS[name])
    if name == "decode_7b":
        return decode_inputs(M if M is not None else spec["M"], spec["K"], spec["N"], spec["p_zero"], seed)
    M_ = M if M is not None else spec.pop("M")
    spec.pop("M", None)
    return linear_inputs(M_, spec.pop("N"), spec.pop("K"), seed=seed, **spec)


def bf16_bits(t: torch.Tensor):
    """Raw 16-bit patterns of a bf16 tensor as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def host_array(t: torch.Tensor):
    """numpy view for the oracle: fp32 as float32, bf16 as its uint16 bits."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.contiguous().numpy()
