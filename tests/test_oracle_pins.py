"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages give (the 2-bit code table), a hand-worked example, a closed form, an
invariant the pages state, a library routine the step reduces to, or brute
force on tiny inputs.  Page titles:
  [NOTES] "BitNet 1.5技术解析：2比特量化在神经网络中的应用与挑战"
  [ENG]   "BitNet 三元权重量化训练工程：直通估计器与梯度裁剪实践"
  [WALL]  "1.58-bit量化技术突破AI算力与内存墙限制"
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32_EPS = 2.0 ** -24  # unit roundoff of binary32


# ------------------------------------------------------------------ tree sum
# The summation order is the library's contract (the pages only say "mean");
# the pins below check the tree against exact arithmetic and hand-worked
# order-sensitive cases.

def test_tree_sum_exact_on_integers():
    for n in [1, 2, 3, 5, 7, 8, 13, 64, 100, 1000, 4097]:
        v = np.arange(n, dtype=np.float32)
        assert oracle.tree_sum(v) == np.float32(n * (n - 1) // 2)


def test_tree_sum_worked_order_cases():
    t = np.float32(2.0 ** -24)
    # n = 4: (1 + t) + (t + t) = 1 + 2^-23.  A left-to-right loop gives 1.
    assert oracle.tree_sum([1.0, t, t, t]) == np.float32(1.0 + 2.0 ** -23)
    # n = 3 is padded with +0: (1 + t) + (t + 0); 1 + t is a tie -> 1, then 1 + t -> 1.
    assert oracle.tree_sum([1.0, t, t]) == np.float32(1.0)
    # order matters: (t + t) + (1 + 0) = 1 + 2^-23.
    assert oracle.tree_sum([t, t, 1.0]) == np.float32(1.0 + 2.0 ** -23)
    # n = 8 puts the small terms in the second half: (1+0+0+0) + ((t+t)+(t+t)) = 1 + 2^-22.
    assert oracle.tree_sum([1.0, 0, 0, 0, t, t, t, t]) == np.float32(1.0 + 2.0 ** -22)


def test_tree_sum_error_bound():
    rng = np.random.default_rng(5)
    for n in [7, 256, 1000, 65536, 100003]:
        v = np.abs(rng.standard_normal(n)).astype(np.float32)
        exact = math.fsum(float(a) for a in v)
        depth = max(1, math.ceil(math.log2(n)))
        assert abs(float(oracle.tree_sum(v)) - exact) <= depth * F32_EPS * exact * 1.0001


def test_tree_sum_split_invariance():
    # Any split into aligned power-of-two blocks combined in index order
    # reproduces the tree; zero padding is exact for non-negative terms.
    rng = np.random.default_rng(6)
    v = np.abs(rng.standard_normal(3000)).astype(np.float32)
    whole = oracle.tree_sum(v)
    for blk in [1, 4, 64, 256, 1024, 2048]:
        parts = [oracle.tree_sum(v[i:i + blk]) if i + blk <= v.size else
                 oracle.tree_sum(np.concatenate([v[i:], np.zeros(blk - (v.size - i), np.float32)]))
                 for i in range(0, v.size, blk)]
        assert oracle.tree_sum(np.array(parts, np.float32)) == whole


# ----------------------------------------------------------- act quant (O2)
# [NOTES 2.2], [NOTES 3.1], [ENG STE section]

def test_act_quant_worked_example():
    # x = [3, -4, 0, 0]: RMSNorm cancels in q, so q = round(127 * x / max|x|)
    # = round([95.25, -127, 0, 0]) = [95, -127, 0, 0].
    q, s = oracle.act_quant(np.array([[3.0, -4.0, 0.0, 0.0]], np.float32))
    assert q.tolist() == [[95, -127, 0, 0]]
    # scale = 127 * sqrt(mean(x^2) + 1e-5) / max|x| = 127 * sqrt(6.25001) / 4
    assert abs(float(s[0]) - 127.0 * math.sqrt(6.25 + 1e-5) / 4.0) <= 4e-7 * float(s[0])


def test_act_quant_zero_row():
    # all-zero token: the 1e-5 floor on the max gives scale 127/1e-5 and q = 0
    q, s = oracle.act_quant(np.zeros((2, 64), np.float32))
    assert not q.any()
    assert s[0] == np.float32(127.0) / np.float32(1e-5)


def _act_inputs():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[3] *= 1e-3          # mean square far below 1e-5: eps placement shows
    x[4] *= 1e3
    x[5, 17] = 40.0       # outlier
    x[6] += 3.0           # non-zero mean (LayerNorm would differ)
    x[7, :] = 0.0
    x[7, 5] = -2.0        # single non-zero entry
    return x


def test_act_quant_invariants():
    x = _act_inputs()
    q, s = oracle.act_quant(x)
    assert q.dtype == np.int8
    assert q.min() >= -128 and q.max() <= 127
    # every row with a non-zero entry reaches |q| = 127 exactly once the
    # per-token absmax is used (P: scale = 127 / max|x| per row)
    assert (np.abs(q.astype(np.int32)).max(axis=1) == 127).all()
    assert (s > 0).all()


def test_act_quant_closed_form():
    x = _act_inputs()
    q, s = oracle.act_quant(x)
    xd = x.astype(np.float64)
    amax = np.abs(xd).max(axis=1, keepdims=True)
    target = 127.0 * xd / amax                      # unit-gain RMSNorm cancels
    assert np.abs(q - target).max() <= 0.5 + 1e-4
    frac = np.abs(target - np.floor(target) - 0.5)
    clear = frac > 1e-4                              # away from a rounding tie
    assert (q[clear] == np.round(target[clear])).all()
    # scale_x = 127 * sqrt(mean(x^2) + eps) / max|x|  (eps inside the root)
    ref = 127.0 * np.sqrt((xd ** 2).mean(axis=1) + 1e-5) / amax[:, 0]
    assert np.abs(s / ref - 1.0).max() <= 2e-6


def test_act_quant_bf16_matches_widened_fp32():
    g = torch.Generator().manual_seed(11)
    xb = torch.randn(16, 256, generator=g).to(torch.bfloat16)
    q1, s1 = oracle.act_quant(workloads.bf16_bits(xb))
    q2, s2 = oracle.act_quant(xb.float().numpy())
    assert (q1 == q2).all() and (s1 == s2).all()


# ---------------------------------------------------------- weight quant (O3)
# [NOTES 2.1], [WALL 2.2], [ENG STE section]

@pytest.mark.parametrize("w,gamma,codes", [
    ([1.0, 7.0, 0.0, 0.0], 2.0, [0, 1, 0, 0]),       # 0.5 is a tie -> 0
    ([3.0, 5.0, 0.0, 0.0], 2.0, [1, 1, 0, 0]),       # 1.5, 2.5 -> 2 -> clamp 1
    ([-2.0, 2.0, 2.0, -2.0], 2.0, [-1, 1, 1, -1]),
    ([-1.0, 0.4, 0.0, 0.6], 0.5, [-1, 1, 0, 1]),     # -2, 0.8, 0, 1.2
])
def test_weight_quant_worked(w, gamma, codes):
    c, g = oracle.weight_quant(np.array([w], np.float32))
    assert g == np.float32(gamma)
    assert c.tolist() == [codes]


def test_weight_quant_two_rows_mean_over_whole_matrix():
    # gamma is the mean over the whole matrix, not per row: mean|W| = 16/8 = 2
    c, g = oracle.weight_quant(np.array([[1, 1, 1, 1], [3, 3, 3, 3]], np.float32))
    assert g == np.float32(2.0)
    assert c.tolist() == [[0, 0, 0, 0], [1, 1, 1, 1]]


def test_weight_quant_all_zero():
    c, g = oracle.weight_quant(np.zeros((3, 8), np.float32))
    assert g == np.float32(1e-5)
    assert not c.any()


def exact_half_tie_matrix(seed: int = 8):
    """Integer matrix A (8x32, |A| <= 6) with sum|A| = 512, and W = A * 2^-6.

    mean|W| = 512 * 2^-6 / 256 = 2^-5 exactly, so every W/gamma = A/2 is an
    exact half-integer and round-half-to-even decides each code.
    """
    rng = np.random.default_rng(seed)
    A = rng.integers(-6, 7, size=(8, 32)).astype(np.int64)
    deficit = 512 - int(np.abs(A).sum())
    i = 0
    while deficit != 0:                       # adjust magnitudes to reach 512
        r, col = divmod(i, 32)
        r %= 8
        step = int(np.sign(deficit))
        if 0 <= abs(A[r, col]) + step <= 6:
            A[r, col] = (abs(A[r, col]) + step) * (1 if A[r, col] >= 0 else -1)
            deficit -= step
        i += 1
    assert np.abs(A).sum() == 512
    return A, (A.astype(np.float64) * 2.0 ** -6).astype(np.float32)


def test_weight_quant_exact_half_ties():
    # |A| <= 1 -> |W/gamma| <= 0.5 -> 0 (0.5 is a tie to even); else sign(A)
    A, W = exact_half_tie_matrix()
    c, g = oracle.weight_quant(W)
    assert g == np.float32(2.0 ** -5)
    expect = np.where(np.abs(A) <= 1, 0, np.sign(A))
    for a, e in zip(A.ravel(), expect.ravel()):  # Python's round is half-to-even
        r = round(Fraction(int(a), 2))
        assert max(-1, min(1, r)) == e
    assert (c == expect).all()


def near_tie_matrix(j: int):
    """1x8 matrix with gamma = j*2^-8 exactly and entries one ulp above gamma/2.

    Entries come in pairs (p, gamma - p) and (1.5 gamma, 1.5 gamma), so every
    partial sum of |W| is an exact multiple of gamma and mean|W| = gamma.
    p = gamma/2 + 1 ulp puts W/gamma just above the 0.5 tie.
    """
    g = np.float32(j * 2.0 ** -8)
    p = np.nextafter(np.float32(g / np.float32(2)), np.float32(np.inf))
    r = np.float32(g - p)
    h = np.float32(1.5) * g
    return np.array([[p, r, h, h, -p, -r, -h, h]], np.float32), g


@pytest.mark.parametrize("j", [25, 31, 41, 47, 97, 127])
def test_weight_quant_near_tie_divides(j):
    # For these gammas fl(p / gamma) > 0.5 while fl(p * fl(1/gamma)) == 0.5:
    # the code must follow the division ([WALL 2.2]: W / gamma), here
    # evaluated by numpy's IEEE float32 division.
    W, g = near_tie_matrix(j)
    c, gq = oracle.weight_quant(W)
    assert gq == g
    ref = np.clip(np.rint(W / g), -1, 1).astype(np.int8)
    assert ref[0, 0] == 1 and np.rint(W[0, 0] * (np.float32(1) / g)) == 0
    assert (c == ref).all()


def test_weight_quant_gamma_is_mean_abs():
    rng = np.random.default_rng(9)
    W = (0.02 * rng.standard_normal((300, 520))).astype(np.float32)
    _, g = oracle.weight_quant(W)
    exact = math.fsum(abs(float(a)) for a in W.ravel()) / W.size
    depth = math.ceil(math.log2(300)) + math.ceil(math.log2(520)) + 1
    assert abs(float(g) - exact) <= depth * F32_EPS * exact


def test_weight_codes_match_library_division():
    # With gamma fixed, the code step is clamp(round(W / gamma), -1, 1)
    # ([WALL 2.2]); torch's CPU float32 division and round (half to even) are
    # an independent evaluation of it.
    rng = np.random.default_rng(10)
    W = (0.02 * rng.standard_normal((257, 384))).astype(np.float32)
    c, g = oracle.weight_quant(W)
    ref = torch.clamp(torch.round(torch.from_numpy(W) / torch.tensor(g)), -1, 1).to(torch.int8).numpy()
    assert (c == ref).all()
    # The notes page multiplies by 1/gamma instead; that reading differs from
    # the division only where W/gamma sits within an ulp of +-0.5.
    ref2 = torch.clamp(torch.round(torch.from_numpy(W) * (1.0 / torch.tensor(g))), -1, 1).to(torch.int8).numpy()
    assert (c != ref2).mean() < 1e-3


def test_weight_quant_invariants_and_zero_ratio():
    # Codes lie in {-1,0,1}.  For Gaussian W, gamma -> sigma*sqrt(2/pi) and a
    # code is 0 when |W| <= gamma/2, so P(0) = erf(1 / (2 sqrt(pi))) = 0.3101.
    w = workloads.normal((1024, 1024), 0.02, seed=12)
    c, g = oracle.weight_quant(w.numpy())
    assert set(np.unique(c).tolist()) <= {-1, 0, 1}
    p0 = math.erf(1.0 / (2.0 * math.sqrt(math.pi)))
    assert abs(p0 - 0.3101) < 1e-4
    n = c.size
    sigma = math.sqrt(p0 * (1 - p0) / n)
    assert abs((c == 0).mean() - p0) < 6 * sigma
    assert abs((c == 1).mean() - (c == -1).mean()) < 6 * math.sqrt(0.5 / n) * 2
    assert abs(float(g) - 0.02 * math.sqrt(2 / math.pi)) < 0.02 * 0.01


# ------------------------------------------------------------ packing (D1)
# [WALL 4.1]

def _read_code_table():
    table, ratio = {}, None
    with open(os.path.join(GOLDEN, "ternary_code_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            a, b = line.split()
            if a == "fp16_ratio":
                ratio = int(b)
            elif b != "reserved":
                table[int(b)] = int(a, 2)
    return table, ratio


def test_pack_code_table_from_page():
    table, ratio = _read_code_table()
    assert table == {0: 0b00, 1: 0b01, -1: 0b10}
    for v, bits in table.items():
        for j in range(4):           # each of the four slots of a byte
            codes = np.zeros((1, 4), np.int8)
            codes[0, j] = v
            assert oracle.pack(codes)[0, 0] == bits << (2 * j)
    # a row of K codes takes K/4 bytes: 1/8 of fp16 storage
    codes = np.zeros((3, 64), np.int8)
    assert oracle.pack(codes).nbytes * ratio == 3 * 64 * 2


def test_pack_layout_example_and_roundtrip():
    # codes [0, +1, -1, 0] -> 00 | 01<<2 | 10<<4 | 00<<6 = 0x24
    assert oracle.pack(np.array([[0, 1, -1, 0]], np.int8))[0, 0] == 0x24
    c = workloads.ternary_codes(37, 96, 0.35, seed=4).numpy()
    p = oracle.pack(c)
    assert p.shape == (37, 24)
    # the reserved pattern 11 never occurs
    for j in range(4):
        assert not (((p >> (2 * j)) & 3) == 3).any()
    assert (oracle.unpack(p, 96) == c).all()


def test_pack_rejects_non_ternary():
    with pytest.raises(RuntimeError):
        oracle.pack(np.array([[0, 2, 0, 0]], np.int8))


# ------------------------------------------------------------- GEMM (O4)
# [NOTES 3.1] (linear on the quantized operands), [NOTES 5.2] (wide
# accumulator), [WALL 3.1] (add / subtract / skip)

def test_gemm_brute_force_triple_loop():
    rng = np.random.default_rng(13)
    q = rng.integers(-128, 128, size=(5, 12)).astype(np.int8)
    c = rng.integers(-1, 2, size=(7, 12)).astype(np.int8)
    acc = oracle.gemm_i32(q, c)
    for m in range(5):
        for n in range(7):
            s = 0
            for k in range(12):
                s += int(q[m, k]) * int(c[n, k])
            assert acc[m, n] == s


def test_gemm_add_subtract_skip_formulation():
    # +1 adds the activation, -1 subtracts it, 0 skips it.
    rng = np.random.default_rng(14)
    q = rng.integers(-127, 128, size=(4, 40)).astype(np.int8)
    c = rng.integers(-1, 2, size=(9, 40)).astype(np.int8)
    acc = oracle.gemm_i32(q, c)
    for m in range(4):
        for n in range(9):
            y = 0
            for k in range(40):
                if c[n, k] == 1:
                    y += int(q[m, k])
                elif c[n, k] == -1:
                    y -= int(q[m, k])
            assert acc[m, n] == y


@pytest.mark.parametrize("K", [4, 8])
def test_gemm_exhaustive_code_patterns(K):
    pats = np.array(np.meshgrid(*[[-1, 0, 1]] * K, indexing="ij")).reshape(K, -1).T.astype(np.int8)
    rng = np.random.default_rng(15)
    q = rng.integers(-128, 128, size=(3, K)).astype(np.int8)
    acc = oracle.gemm_i32(q, pats)
    assert acc.shape == (3, 3 ** K)
    for n in range(0, 3 ** K, 7 if K == 8 else 1):
        for m in range(3):
            assert acc[m, n] == sum(int(q[m, k]) * int(pats[n, k]) for k in range(K))


def test_gemm_special_cases_and_sampled_form():
    rng = np.random.default_rng(16)
    c = rng.integers(-1, 2, size=(11, 64)).astype(np.int8)
    ones = np.ones((2, 64), np.int8)
    assert (oracle.gemm_i32(ones, c) == c.astype(np.int32).sum(axis=1)[None, :]).all()
    q = rng.integers(-128, 128, size=(3, 64)).astype(np.int8)
    assert (oracle.gemm_i32(q, np.ones((1, 64), np.int8))[:, 0] == q.astype(np.int32).sum(axis=1)).all()
    # extremes of the int8 range: |acc| = 128*K
    K = 8192
    qm = np.full((1, K), -128, np.int8)
    cm = np.full((1, K), -1, np.int8)
    assert oracle.gemm_i32(qm, cm)[0, 0] == 128 * K
    full = oracle.gemm_i32(q, c)
    ms = np.array([0, 2, 1, 2])
    ns = np.array([10, 0, 5, 7])
    assert (oracle.gemm_i32_at(q, c, ms, ns) == full[ms, ns]).all()


def test_gemm_int32_overflow_detected():
    K = 1 << 24
    with pytest.raises(RuntimeError):
        oracle.gemm_i32(np.full((1, K), -128, np.int8), np.full((1, K), -1, np.int8))


# ---------------------------------------------------- dequant + STE (O5, O6)
# [NOTES 2.1, 2.2, 3.1], [WALL 3.2]: identity STE through both quantizers.

def _small_layer(M=6, N=5, K=12, seed=17):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    c = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    s = rng.uniform(20, 60, size=M).astype(np.float32)
    g = np.float32(0.0123)
    gy = rng.standard_normal((M, N)).astype(np.float32)
    return q, c, s, g, gy


def test_dequant_equals_linear_on_dequantized_operands():
    q, c, s, g, _ = _small_layer()
    acc, y = oracle.linear_fwd(q, s, c, g)
    xd = torch.from_numpy(q.astype(np.float64) / s.astype(np.float64)[:, None])
    wd = torch.from_numpy(float(g) * c.astype(np.float64))
    ref = torch.nn.functional.linear(xd, wd).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)


def test_ste_grads_equal_autograd_of_plain_linear():
    q, c, s, g, gy = _small_layer(M=9, N=7, K=16)
    xd = torch.tensor(q.astype(np.float64) / s.astype(np.float64)[:, None], requires_grad=True)
    wd = torch.tensor(float(g) * c.astype(np.float64), requires_grad=True)
    torch.nn.functional.linear(xd, wd).backward(torch.from_numpy(gy.astype(np.float64)))
    gx = oracle.ste_grad_x(gy, c, g)
    gw = oracle.ste_grad_w(gy, q, s)
    assert np.allclose(gx, xd.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert np.allclose(gw, wd.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_ste_detach_trick_passes_gradient_unchanged():
    # x + (quantize(x) - x).detach(): the forward value is the quantized one,
    # the gradient w.r.t. x is the gradient w.r.t. the quantized value.
    q, c, s, g, gy = _small_layer(M=4, N=3, K=8, seed=18)
    xn = torch.randn(4, 8, dtype=torch.float64, requires_grad=True)
    w = torch.randn(3, 8, dtype=torch.float64, requires_grad=True)
    xq = xn + (torch.from_numpy(q.astype(np.float64) / s.astype(np.float64)[:, None]) - xn).detach()
    wq = w + (torch.from_numpy(float(g) * c.astype(np.float64)) - w).detach()
    torch.nn.functional.linear(xq, wq).backward(torch.from_numpy(gy.astype(np.float64)))
    assert np.allclose(oracle.ste_grad_x(gy, c, g), xn.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert np.allclose(oracle.ste_grad_w(gy, q, s), w.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_ste_unit_upstream_gradient():
    q, c, s, g, _ = _small_layer(M=5, N=4, K=8, seed=19)
    m, n = 3, 2
    gy = np.zeros((5, 4), np.float32)
    gy[m, n] = 1.0
    gw = oracle.ste_grad_w(gy, q, s)
    expect = np.zeros((4, 8))
    expect[n] = q[m].astype(np.float64) / float(s[m])
    assert np.array_equal(gw, expect)
    gx = oracle.ste_grad_x(gy, c, g)
    ex = np.zeros((5, 8))
    ex[m] = float(g) * c[n].astype(np.float64)
    assert np.array_equal(gx, ex)


def test_ste_sampled_forms_and_bf16_grad():
    rng = np.random.default_rng(20)
    q, c, s, g, _ = _small_layer(M=8, N=6, K=12, seed=20)
    gyb = torch.from_numpy(rng.standard_normal((8, 6)).astype(np.float32)).to(torch.bfloat16)
    bits = workloads.bf16_bits(gyb)
    gx = oracle.ste_grad_x(bits, c, g)
    gw = oracle.ste_grad_w(bits, q, s)
    assert np.array_equal(gx, oracle.ste_grad_x(gyb.float().numpy(), c, g))
    ms, ks = np.array([0, 7, 3]), np.array([11, 0, 5])
    assert np.array_equal(oracle.ste_grad_x_at(bits, c, g, ms, ks), gx[ms, ks])
    ns = np.array([5, 0, 2])
    assert np.array_equal(oracle.ste_grad_w_at(bits, q, s, ns, ks), gw[ns, ks])


# ------------------------------------------------------------ build rule

# ------------------------------------------------------ RMSNorm backward
# [NOTES] 3.1 puts an RMSNorm (unit gain) in front of the quantizer; its
# backward is the exact derivative of the forward reading (eps inside the
# root).  Pinned by finite differences of that forward, by torch autograd of
# the forward written out directly, and by closed forms.

def _rms_forward64(x, eps):
    # eps as the binary32 value the oracle receives
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + float(np.float32(eps)))


def test_rmsnorm_bwd_matches_finite_differences():
    rng = np.random.default_rng(40)
    M, K, eps = 3, 7, 1e-5
    x = rng.standard_normal((M, K)).astype(np.float32)
    g = rng.standard_normal((M, K)).astype(np.float32)
    dx = oracle.rmsnorm_bwd(x, g, eps)
    h = 1e-6
    for m in range(M):
        for k in range(K):
            xp = x.astype(np.float64).copy()
            xm = xp.copy()
            xp[m, k] += h
            xm[m, k] -= h
            num = (np.sum(g * _rms_forward64(xp, eps)) - np.sum(g * _rms_forward64(xm, eps))) / (2 * h)
            assert abs(num - dx[m, k]) <= 1e-6 * (1 + abs(dx[m, k])), (m, k, num, dx[m, k])


def test_rmsnorm_bwd_equals_autograd_of_forward():
    rng = np.random.default_rng(41)
    M, K, eps = 5, 96, 1e-5
    x = rng.standard_normal((M, K)).astype(np.float32)
    g = rng.standard_normal((M, K)).astype(np.float32)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    n = xt * torch.rsqrt(xt.pow(2).mean(dim=1, keepdim=True) + float(np.float32(eps)))
    n.backward(torch.tensor(g, dtype=torch.float64))
    np.testing.assert_allclose(oracle.rmsnorm_bwd(x, g, eps), xt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_rmsnorm_bwd_closed_forms():
    rng = np.random.default_rng(42)
    # K = 1: n = x / sqrt(x^2 + eps), dn/dx = eps / (x^2 + eps)^(3/2)
    eps = 0.25
    x = np.array([[0.5], [-2.0], [0.0]], np.float32)
    g = np.array([[1.0], [3.0], [-2.0]], np.float32)
    want = g.astype(np.float64) * eps / (x.astype(np.float64) ** 2 + eps) ** 1.5
    np.testing.assert_allclose(oracle.rmsnorm_bwd(x, g, eps), want, rtol=1e-6)
    # x . dx = (sum_k g_k n_k) * eps / (mean x^2 + eps): zero when eps = 0
    M, K = 4, 33
    x = rng.standard_normal((M, K)).astype(np.float32)
    g = rng.standard_normal((M, K)).astype(np.float32)
    for eps in (1e-5, 0.5):
        dx = oracle.rmsnorm_bwd(x, g, eps)
        x64 = x.astype(np.float64)
        ms = np.mean(x64 * x64, axis=1)
        dot = np.sum(g * _rms_forward64(x, eps), axis=1)
        e32 = float(np.float32(eps))
        np.testing.assert_allclose(np.sum(x64 * dx, axis=1), dot * e32 / (ms + e32), rtol=1e-9, atol=1e-12)
    # eps = 0: the forward is scale invariant, so dx(a x) = dx(x) / a
    dx1 = oracle.rmsnorm_bwd(x, g, 0.0)
    dx2 = oracle.rmsnorm_bwd((4.0 * x).astype(np.float32), g, 0.0)
    np.testing.assert_allclose(dx2, dx1 / 4.0, rtol=1e-12, atol=1e-14)
    # bf16 inputs widen exactly
    xb = workloads.bf16_bits(torch.tensor(x).to(torch.bfloat16))
    gb = workloads.bf16_bits(torch.tensor(g).to(torch.bfloat16))
    xw = (xb.astype(np.uint32) << 16).view(np.float32)
    gw = (gb.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(oracle.rmsnorm_bwd(xb, gb, 1e-5), oracle.rmsnorm_bwd(xw, gw, 1e-5))


# ------------------------------------------- range-gated STE, weight clamp
def _golden_gate_cases():
    cases = []
    for line in open(os.path.join(GOLDEN, "ste_gate_cases.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fields = [f.split() for f in line.split("|")]
        kind, dt, lo, hi = fields[0]
        vals = [[float.fromhex(v) if "0x" in v else float(v) for v in f] for f in fields[1:]]
        cases.append((kind, dt, float(lo), float(hi), vals))
    return cases


def _as_dtype(vals, dt):
    a = np.array(vals, np.float32)
    if dt == "bf16":
        b = workloads.bf16_bits(torch.tensor(a).to(torch.bfloat16))
        assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), a), "fixture value not bf16"
        return b[None, :]
    return a[None, :]


def test_ste_gate_and_clamp_golden_cases():
    cases = _golden_gate_cases()
    assert len(cases) >= 7
    for kind, dt, lo, hi, vals in cases:
        w = _as_dtype(vals[0], dt)
        if kind == "gate":
            got = oracle.ste_gate(np.array([vals[1]], np.float64), w, lo, hi)
            assert np.array_equal(got, np.array([vals[2]], np.float64)), (dt, lo, hi, got)
        else:
            got = oracle.weight_clamp(w, lo, hi)
            want = _as_dtype(vals[1], dt)
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (dt, lo, hi, got)


def test_ste_gate_equals_autograd_through_clamp():
    # torch's clamp passes its gradient where lo <= w <= hi (inclusive), so
    # the gated STE is the gradient through clamp(W) of the plain STE layer
    rng = np.random.default_rng(50)
    N, K, M = 6, 40, 9
    w = (rng.standard_normal((N, K)) * 0.8).astype(np.float32)
    w[0, :4] = [-1.0, 1.0, -0.5, 0.25]  # bounds hit exactly
    gy = rng.standard_normal((M, N)).astype(np.float32)
    xd = rng.standard_normal((M, K))
    for lo, hi in ((-1.0, 1.0), (-0.5, 0.25)):
        wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
        y = torch.nn.functional.linear(torch.tensor(xd), torch.clamp(wt, lo, hi))
        y.backward(torch.tensor(gy, dtype=torch.float64))
        plain = gy.astype(np.float64).T @ xd  # the STE gradient without the gate
        np.testing.assert_allclose(oracle.ste_gate(plain, w, lo, hi), wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    # an unbounded range is the plain STE, an empty one blocks everything
    g = rng.standard_normal((N, K))
    assert np.array_equal(oracle.ste_gate(g, w, -np.inf, np.inf), g)
    assert not oracle.ste_gate(g, w, 1.0, -1.0).any()


def test_weight_clamp_equals_torch_clamp():
    rng = np.random.default_rng(51)
    w = (rng.standard_normal((7, 64)) * 2).astype(np.float32)
    for lo, hi in ((-1.0, 1.0), (-0.3, 0.7)):
        np.testing.assert_array_equal(oracle.weight_clamp(w, lo, hi), torch.clamp(torch.tensor(w), lo, hi).numpy())
        wb = torch.tensor(w).to(torch.bfloat16)
        want = torch.clamp(wb.float(), lo, hi).to(torch.bfloat16)
        np.testing.assert_array_equal(oracle.weight_clamp(workloads.bf16_bits(wb), lo, hi), workloads.bf16_bits(want))
    c = oracle.weight_clamp(w)
    assert np.array_equal(oracle.weight_clamp(c), c)  # idempotent


# ------------------------------------------------------------ code counts
def test_code_counts_hand_packed_bytes():
    # byte 0b10_01_00_01: columns 0..3 = +1, 0, +1, -1 ([WALL] 4.1 table, the
    # code of column k in bits 2k..2k+1); 0xff: four unused 11 patterns
    packed = np.array([[0b10010001, 0x00], [0xFF, 0b01010101]], np.uint8)
    np.testing.assert_array_equal(oracle.code_counts(packed, 8), [1 + 4, 2 + 4, 1, 4])


def test_code_counts_match_the_codes():
    rng = np.random.default_rng(60)
    w = (rng.standard_normal((37, 64)) * 0.02).astype(np.float32)
    codes, _ = oracle.weight_quant(w)
    cnt = oracle.code_counts(oracle.pack(codes), 64)
    assert int(cnt.sum()) == codes.size and cnt[3] == 0
    assert (int(cnt[0]), int(cnt[1]), int(cnt[2])) == (int((codes == 0).sum()), int((codes == 1).sum()),
                                                       int((codes == -1).sum()))
    # -W swaps the +1 and -1 counts
    c2 = oracle.code_counts(oracle.pack(oracle.weight_quant(-w)[0]), 64)
    assert (c2[0], c2[1], c2[2]) == (cnt[0], cnt[2], cnt[1])


# ------------------------------------------- per-output-channel scales
def test_weight_quant_rows_is_the_matrix_rule_per_row():
    rng = np.random.default_rng(80)
    w = (rng.standard_normal((9, 40)) * 0.02).astype(np.float32)
    w[3] = 0.0                       # an all-zero row: gamma floor, all codes 0
    w[5] *= 100.0                    # rows on different scales get their own gamma
    codes, gamma = oracle.weight_quant_rows(w)
    for n in range(w.shape[0]):
        c1, g1 = oracle.weight_quant(w[n:n + 1])
        assert np.array_equal(codes[n:n + 1], c1) and gamma[n] == np.float32(g1)
    assert gamma[3] == np.float32(1e-5) and not codes[3].any()
    # worked case: rows [1,7,0,0] and [3,5,0,0] both have gamma 2
    c, g = oracle.weight_quant_rows(np.array([[1, 7, 0, 0], [3, 5, 0, 0]], np.float32))
    assert g.tolist() == [2.0, 2.0] and c.tolist() == [[0, 1, 0, 0], [1, 1, 0, 0]]


def test_channel_forward_and_grad_x():
    rng = np.random.default_rng(81)
    M, N, K = 6, 10, 32
    q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    codes = rng.integers(-1, 2, (N, K), dtype=np.int8)
    sx = rng.uniform(20, 40, M).astype(np.float32)
    # one scale for every channel reduces to the per-matrix forward
    acc, y = oracle.linear_fwd_channel(q, sx, codes, np.full(N, 0.0125, np.float32))
    acc0, y0 = oracle.linear_fwd(q, sx, codes, 0.0125)
    assert np.array_equal(acc, acc0)
    np.testing.assert_allclose(y, y0, rtol=1e-15)
    # per-channel scales: autograd of the linear map at W_deq = s_n * c
    s = rng.uniform(0.01, 0.05, N).astype(np.float32)
    gy = rng.standard_normal((M, N)).astype(np.float32)
    xt = torch.tensor(q.astype(np.float64) / sx[:, None], requires_grad=True)
    wdeq = torch.tensor(s.astype(np.float64)[:, None] * codes.astype(np.float64))
    torch.nn.functional.linear(xt, wdeq).backward(torch.tensor(gy, dtype=torch.float64))
    np.testing.assert_allclose(oracle.ste_grad_x_channel(gy, codes, s), xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    _, y = oracle.linear_fwd_channel(q, sx, codes, s)
    np.testing.assert_allclose(y, (xt.detach().numpy() @ wdeq.numpy().T), rtol=1e-12)


# ------------------------------- gradient of a learned per-channel scale
# "BitNet量化感知训练中的梯度传播优化", section on the BitLinear
# implementation, 1: output = (sign(W) . s) x with s in R^{d_out x 1}
# learned by gradient descent.

def test_channel_scale_grad_equals_autograd_of_the_scaled_linear():
    # float64 autograd of y = X_deq . (c * s)^T with s a parameter
    rng = np.random.default_rng(90)
    M, N, K = 7, 9, 24
    q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    codes = rng.integers(-1, 2, (N, K), dtype=np.int8)
    sx = rng.uniform(20, 40, M).astype(np.float32)
    gy = rng.standard_normal((M, N)).astype(np.float32)
    s = torch.tensor(rng.uniform(0.01, 0.05, N), dtype=torch.float64, requires_grad=True)
    xd = torch.tensor(q.astype(np.float64) / sx.astype(np.float64)[:, None])
    c = torch.tensor(codes.astype(np.float64))
    torch.nn.functional.linear(xd, c * s[:, None]).backward(torch.tensor(gy, dtype=torch.float64))
    gs = oracle.channel_scale_grad(gy, q, sx, codes)
    np.testing.assert_allclose(gs, s.grad.numpy(), rtol=1e-12, atol=1e-13)
    # sampled form, and the bf16-bits input path
    ns = np.array([0, 8, 3, 3], np.int64)
    np.testing.assert_array_equal(oracle.channel_scale_grad(gy, q, sx, codes, ns=ns), gs[ns])
    gyb = workloads.bf16_bits(torch.from_numpy(gy).to(torch.bfloat16))
    gyw = torch.from_numpy(gy).to(torch.bfloat16).double().numpy()
    ref = ((q.astype(np.float64) @ codes.astype(np.float64).T) / sx.astype(np.float64)[:, None] * gyw).sum(0)
    np.testing.assert_allclose(oracle.channel_scale_grad(gyb, q, sx, codes), ref, rtol=1e-12, atol=1e-13)


def test_channel_scale_grad_worked_case():
    # q = [[1, 2], [3, -4]], codes = [[1, -1], [0, 1]], scale_x = [2, 4]:
    # acc = q c^T = [[-1, 2], [7, -4]]; acc / scale_x = [[-0.5, 1], [1.75, -1]]
    # gy = [[1, 0.5], [2, -1]]: grad_s = [1*-0.5 + 2*1.75, 0.5*1 + -1*-1] = [3, 1.5]
    q = np.array([[1, 2], [3, -4]], np.int8)
    codes = np.array([[1, -1], [0, 1]], np.int8)
    sx = np.array([2, 4], np.float32)
    gy = np.array([[1, 0.5], [2, -1]], np.float32)
    assert oracle.channel_scale_grad(gy, q, sx, codes).tolist() == [3.0, 1.5]
    # a unit upstream gradient at (m, n) picks acc[m, n] / scale_x[m]
    e = np.zeros((2, 2), np.float32)
    e[1, 0] = 1.0
    assert oracle.channel_scale_grad(e, q, sx, codes).tolist() == [1.75, 0.0]


def test_channel_scale_grad_is_the_code_dot_of_grad_w():
    # exchanging the sums: grad_s[n] = sum_k c[n,k] * grad_W[n,k]
    rng = np.random.default_rng(91)
    M, N, K = 11, 6, 40
    q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    codes = rng.integers(-1, 2, (N, K), dtype=np.int8)
    sx = rng.uniform(20, 40, M).astype(np.float32)
    gy = rng.standard_normal((M, N)).astype(np.float32)
    gw = oracle.ste_grad_w(gy, q, sx)
    np.testing.assert_allclose((codes.astype(np.float64) * gw).sum(1), oracle.channel_scale_grad(gy, q, sx, codes),
                               rtol=1e-11, atol=1e-12)


def test_codes_row_dot_order_and_signs():
    # the canonical tree: (1e8 + 1) + (-1e8 + 1) = 1e8 + -1e8 = 0 in binary32,
    # where a left-to-right sum would give 1
    G = np.array([[1e8, 1.0, -1e8, 1.0]], np.float32)
    one = np.ones((1, 4), np.int8)
    assert oracle.codes_row_dot(G, one)[0] == np.float32(0.0)
    # codes flip signs exactly; zero codes give +0 whatever the signs of G
    c = np.array([[1, -1, -1, 0]], np.int8)
    assert oracle.codes_row_dot(np.array([[2.0, 3.0, -5.0, 7.0]], np.float32), c)[0] == np.float32(4.0)
    z = oracle.codes_row_dot(np.array([[-1.0, -2.0, -3.0, -4.0]], np.float32), np.zeros((1, 4), np.int8))[0]
    assert z == 0.0 and not np.signbit(z)
    # all codes +1: the tree sum of the row; negated codes: the exact negation
    rng = np.random.default_rng(92)
    G = rng.standard_normal((5, 300)).astype(np.float32)
    ones = np.ones((5, 300), np.int8)
    for n in range(5):
        assert oracle.codes_row_dot(G, ones)[n] == oracle.tree_sum(G[n]) + np.float32(0.0)
    cr = rng.integers(-1, 2, (5, 300), dtype=np.int8)
    np.testing.assert_array_equal(oracle.codes_row_dot(G, -cr), -oracle.codes_row_dot(G, cr) + np.float32(0.0))
    # close to the float64 dot product (within the tree's error bound)
    ref = (cr.astype(np.float64) * G.astype(np.float64)).sum(1)
    bound = 300 * 2.0 ** -24 * np.abs(G.astype(np.float64)).sum(1)
    assert (np.abs(oracle.codes_row_dot(G, cr) - ref) <= bound).all()


def test_oracle_does_not_contract_multiply_add():
    # a*b = 1 + 2^-11 + 2^-24 rounds to 1 + 2^-11 (tie to even), so the
    # unfused result is 0 while fma(a, b, c) would be 2^-24.
    a = 1.0 + 2.0 ** -12
    assert oracle.mul_add_probe(a, a, -(1.0 + 2.0 ** -11)) == np.float32(0.0)
