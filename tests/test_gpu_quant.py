"""GPU parity of the quantizers against the CPU oracle: bit-exact int8
activations, scale_x bits, ternary codes (packed bytes) and gamma bits."""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import DEV, f32_bits_equal, host, to_dev

pytestmark = pytest.mark.gpu


def _act_case(M, K, dtype, seed, special=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g)
    if special == "zero_rows":
        x[::3] = 0.0
    elif special == "outliers":
        x[:, ::97] *= 40.0
    elif special == "tiny":
        x *= 1e-3
    elif special == "single":
        x.zero_()
        x[:, K // 2] = -2.5
    return x.to(dtype)


@pytest.mark.parametrize("M,K,dtype,special", [
    (32, 256, torch.float32, None),          # the tiny workload's shape
    (1, 4, torch.float32, None),
    (3, 12, torch.float32, None),            # K not a multiple of the 16-byte vector (bf16)
    (17, 100, torch.bfloat16, None),
    (5, 1000, torch.float32, None),
    (64, 512, torch.bfloat16, "zero_rows"),
    (33, 4096, torch.bfloat16, "outliers"),
    (9, 8192, torch.bfloat16, None),
    (9, 4096, torch.float32, "tiny"),
    (4, 520, torch.float32, "single"),
    (3, 20000, torch.bfloat16, None),        # streamed (row beyond the register cache)
    (2, 12345, torch.float32, None),
])
def test_act_quant_bit_exact(M, K, dtype, special):
    print(f"act_quant M={M} K={K} {dtype} {special}", flush=True)
    x = _act_case(M, K, dtype, seed=M * 1000 + K, special=special)
    q, s = bt.bitnet_act_quant(to_dev(x))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.act_quant(host(x))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert f32_bits_equal(s.cpu().numpy(), s_ref)


def _weight_case(N, K, dtype, seed, special=None):
    if special == "zero":
        return torch.zeros(N, K, dtype=dtype)
    w = workloads.normal((N, K), 0.02, seed=seed, dtype="f32")
    if special == "heavy":
        w[:, :3] *= 50.0
    return w.to(dtype)


@pytest.mark.parametrize("N,K,dtype,special", [
    (256, 256, torch.float32, None),
    (1, 4, torch.float32, None),
    (5, 12, torch.float32, None),
    (37, 100, torch.bfloat16, None),
    (300, 512, torch.float32, None),
    (129, 1028, torch.bfloat16, "heavy"),
    (1376, 512, torch.float32, None),
    (64, 8192, torch.float32, None),
    (7, 64, torch.float32, "zero"),
    (4099, 64, torch.bfloat16, None),        # many rows: second-level tree over > 4096 sums
    # large matrices: gamma evaluated by the pack launch's workgroup 0 and
    # published to the other workgroups (ragged last workgroup)
    (2111, 4096, torch.bfloat16, "heavy"),
    (4099, 1024, torch.float32, None),
])
def test_weight_quant_bit_exact(N, K, dtype, special):
    print(f"weight_quant N={N} K={K} {dtype} {special}", flush=True)
    w = _weight_case(N, K, dtype, seed=N * 7 + K, special=special)
    wp, gamma = bt.bitnet_weight_quant(to_dev(w))
    torch.cuda.synchronize()
    c_ref, g_ref = oracle.weight_quant(host(w))
    assert f32_bits_equal(gamma.cpu().numpy(), np.array([g_ref], np.float32))
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(c_ref))


def test_weight_quant_published_threshold_is_per_call():
    # one workspace for consecutive calls on matrices with different gammas:
    # every call must use its own threshold, never the word a previous call
    # published (the row-sum pass clears it)
    N, K = 2111, 4096
    ws = torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, 0, N, K), dtype=torch.uint8,
                     device="cuda")
    base = _weight_case(N, K, torch.float32, seed=91)
    for scale in (1.0, 3.0, 0.25):
        w = base * scale
        wp, gamma = bt.bitnet_weight_quant(to_dev(w), workspace=ws)
        torch.cuda.synchronize()
        c_ref, g_ref = oracle.weight_quant(host(w))
        assert f32_bits_equal(gamma.cpu().numpy(), np.array([g_ref], np.float32))
        assert np.array_equal(wp.cpu().numpy(), oracle.pack(c_ref))


@pytest.mark.parametrize("N,K,dt", [
    (4096, 4096, torch.bfloat16),  # one round of workgroups: the fifth (reading) wave evaluates
    (2111, 4096, torch.bfloat16),
    (4099, 4096, torch.float32),   # several rounds: the four waves evaluate together
    (8209, 8192, torch.bfloat16),
])
def test_weight_quant_threshold_fallback_gives_the_same_bits(N, K, dt):
    # with no reads of the published threshold every pack workgroup but the
    # first evaluates gamma's threshold itself from the row sums: the codes
    # and gamma must not change (weight quant, the counted call and the
    # two-quantizer call)
    print(f"threshold fallback N={N} K={K} {dt}", flush=True)
    w = _weight_case(N, K, dt, seed=N + K)
    # twice as many token rows as weight rows: more activation bytes than
    # weight bytes, so the two-quantizer call packs beside act_quant
    x = workloads.normal((2 * N, K), 1.0, seed=5, dtype="bf16")
    c_ref, g_ref = oracle.weight_quant(host(w))
    packed_ref = oracle.pack(c_ref)
    prev = bt.bitnet_set_gate_polls(0)
    try:
        wp, gamma = bt.bitnet_weight_quant(to_dev(w))
        wp2, gamma2, counts = bt.bitnet_weight_quant_counted(to_dev(w))
        _, _, wp3, gamma3 = bt.bitnet_quant_operands(to_dev(x), to_dev(w), 1e-5)
        torch.cuda.synchronize()
    finally:
        bt.bitnet_set_gate_polls(prev)
    for p_, g_ in ((wp, gamma), (wp2, gamma2), (wp3, gamma3)):
        assert f32_bits_equal(g_.cpu().numpy(), np.array([g_ref], np.float32))
        assert np.array_equal(p_.cpu().numpy(), packed_ref)
    assert np.array_equal(counts.cpu().numpy(), oracle.code_counts(packed_ref, K).astype(np.int64))


@pytest.mark.parametrize("j", [25, 31, 41, 47, 97, 127])
def test_weight_quant_near_tie_matches_division(j):
    # gamma = j*2^-8 exactly and entries one ulp above gamma/2: the decision
    # must follow the correctly rounded quotient (oracle), not a reciprocal
    from test_oracle_pins import near_tie_matrix
    W, g = near_tie_matrix(j)
    W = np.tile(W, (4, 2))  # 4 x 16: same mean
    wp, gamma = bt.bitnet_weight_quant(to_dev(torch.from_numpy(W)))
    c_ref, g_ref = oracle.weight_quant(W)
    assert g_ref == g
    assert f32_bits_equal(gamma.cpu().numpy(), np.array([g_ref], np.float32))
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(c_ref))


def test_weight_quant_exact_half_ties():
    # every W/gamma is an exact half-integer: round-half-to-even decides
    from test_oracle_pins import exact_half_tie_matrix
    _, W = exact_half_tie_matrix()
    wp, gamma = bt.bitnet_weight_quant(to_dev(torch.from_numpy(W)))
    c_ref, g_ref = oracle.weight_quant(W)
    assert f32_bits_equal(gamma.cpu().numpy(), np.array([g_ref], np.float32))
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(c_ref))


@pytest.mark.parametrize("N,K", [(1, 4), (37, 96), (11008, 4096)])
def test_pack_ternary_matches_oracle(N, K):
    c = workloads.ternary_codes(N, K, 0.35, seed=N + K)
    wp = bt.bitnet_pack_ternary(to_dev(c))
    torch.cuda.synchronize()
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(c.numpy()))


def test_quantizers_are_deterministic():
    x = _act_case(64, 4096, torch.bfloat16, seed=3)
    w = _weight_case(512, 4096, torch.float32, seed=4)
    xd, wd = to_dev(x), to_dev(w)
    q1, s1 = bt.bitnet_act_quant(xd)
    q2, s2 = bt.bitnet_act_quant(xd)
    p1, g1 = bt.bitnet_weight_quant(wd)
    p2, g2 = bt.bitnet_weight_quant(wd)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    assert torch.equal(p1, p2) and torch.equal(g1, g2)


# both quantizers in one call (bitnet_quant_operands): the row-walking
# activation kernel shares its launch with the weight row sums when K is
# 1, 2, 4, 8 or 16 whole blocks (512 bf16 / 256 fp32 elements), else the two
# calls' kernels run in order; either way the outputs must equal the two
# calls' bit for bit
@pytest.mark.parametrize("M,N,K,xdt,wdt", [
    (300, 257, 512, torch.bfloat16, torch.float32),    # one bf16 block
    (1000, 64, 256, torch.float32, torch.bfloat16),    # one fp32 block
    (64, 300, 4096, torch.bfloat16, torch.bfloat16),   # 8 blocks
    (9, 1376, 8192, torch.bfloat16, torch.float32),    # 16 blocks
    (17, 33, 100, torch.bfloat16, torch.float32),      # ragged K: the general activation kernel
    (5000, 8, 1024, torch.float32, torch.float32),     # more rows than the row-walking grid
    # large N: gamma evaluated by the pack launch's workgroup 0 and published
    # to the other workgroups (ragged last workgroup)
    (300, 2111, 4096, torch.bfloat16, torch.bfloat16),
    (64, 2111, 4096, torch.float32, torch.float32),
    # more activation bytes than weight bytes and gamma published: the pack
    # beside act_quant in the second launch
    (8192, 2111, 4096, torch.bfloat16, torch.bfloat16),
    (8200, 2500, 4096, torch.float32, torch.bfloat16),
])
def test_quant_operands_matches_the_two_calls(M, N, K, xdt, wdt):
    print(f"quant_operands M={M} N={N} K={K} {xdt} {wdt}", flush=True)
    x = _act_case(M, K, xdt, seed=M + K)
    w = _weight_case(N, K, wdt, seed=N + K)
    q, s, wp, g = bt.bitnet_quant_operands(to_dev(x), to_dev(w))
    q2, s2 = bt.bitnet_act_quant(to_dev(x))
    wp2, g2 = bt.bitnet_weight_quant(to_dev(w))
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(wp, wp2)
    assert f32_bits_equal(s.cpu().numpy(), s2.cpu().numpy())
    assert f32_bits_equal(g.cpu().numpy(), g2.cpu().numpy())
    q_ref, s_ref = oracle.act_quant(host(x))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert f32_bits_equal(s.cpu().numpy(), s_ref)
    codes_ref, g_ref = oracle.weight_quant(host(w))
    assert np.array_equal(wp.cpu().numpy(), oracle.pack(codes_ref))
    assert f32_bits_equal(g.cpu().numpy(), np.array([g_ref], np.float32))
