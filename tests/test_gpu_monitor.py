"""Code counts (bitnet_code_counts) against the oracle: exact integers."""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import host, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(1, 4), (3, 20), (37, 64), (257, 1040), (1376, 512)])
def test_code_counts_of_quantized_weights(N, K):
    print(f"code counts N={N} K={K}", flush=True)
    w = workloads.normal((N, K), 0.02, seed=N + K)
    wp, _ = bt.bitnet_weight_quant(to_dev(w))
    c = bt.bitnet_code_counts(wp, K)
    c2 = bt.bitnet_code_counts(wp, K)  # counters cleared on every call
    torch.cuda.synchronize()
    packed_ref = oracle.pack(oracle.weight_quant(host(w))[0])
    assert np.array_equal(wp.cpu().numpy(), packed_ref)
    want = oracle.code_counts(packed_ref, K).astype(np.int64)
    assert np.array_equal(c.cpu().numpy(), want)
    assert np.array_equal(c2.cpu().numpy(), want)
    assert int(want.sum()) == N * K and want[3] == 0


def test_code_counts_raw_bytes_and_edge_cases():
    rng = np.random.default_rng(70)
    raw = rng.integers(0, 256, size=(33, 25), dtype=np.uint8)  # every pattern, 11 included; ragged bytes
    c = bt.bitnet_code_counts(to_dev(torch.from_numpy(raw)), 100)
    zero = bt.bitnet_code_counts(bt.bitnet_weight_quant(torch.zeros(8, 64, device="cuda"))[0], 64)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), oracle.code_counts(raw, 100).astype(np.int64))
    assert zero.cpu().tolist() == [8 * 64, 0, 0, 0]


def test_code_counts_decode_layer():
    d = workloads.workload("decode_7b", M=1)
    wp = bt.bitnet_pack_ternary(to_dev(d["codes"]))
    c = bt.bitnet_code_counts(wp, d["codes"].shape[1])
    torch.cuda.synchronize()
    codes = d["codes"].numpy()
    want = [int((codes == 0).sum()), int((codes == 1).sum()), int((codes == -1).sum()), 0]
    assert c.cpu().tolist() == want


# the weight quantizer that counts the codes as it packs them: the same
# codes and gamma as the oracle, the counts of those codes; small matrices
# (gamma in every pack workgroup) and large ones (gamma published by one)
@pytest.mark.parametrize("N,K,dt", [(1, 4, "f32"), (37, 100, "bf16"), (1376, 512, "f32"), (2111, 4096, "bf16"),
                                    (4099, 1024, "f32"), (8209, 8192, "bf16"), (16411, 8192, "bf16")])
def test_weight_quant_counted(N, K, dt):
    # the last two cases have more pack workgroups (8209, 16411) than the
    # 256-thread final sum takes in one pass (4096): the 1024-thread sum, in
    # one pass and in two (16384 a pass)
    print(f"weight_quant_counted N={N} K={K} {dt}", flush=True)
    w = workloads.normal((N, K), 0.02, seed=3 * N + K, dtype=dt)
    wp, g, c = bt.bitnet_weight_quant_counted(to_dev(w))
    torch.cuda.synchronize()
    codes_ref, g_ref = oracle.weight_quant(host(w))
    packed_ref = oracle.pack(codes_ref)
    assert np.array_equal(wp.cpu().numpy(), packed_ref)
    assert g.cpu().numpy().view(np.uint32)[0] == np.array([g_ref], np.float32).view(np.uint32)[0]
    want = oracle.code_counts(packed_ref, K).astype(np.int64)
    assert np.array_equal(c.cpu().numpy(), want)
    assert int(want.sum()) == N * K and want[3] == 0


def test_weight_quant_counted_reuses_its_workspace():
    # one workspace for a large call, then a small one, then an all-zero one:
    # the count slots are cleared by every call before it adds into them
    big, small = (2111, 4096), (64, 256)
    ws = torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT_COUNTED, 0, *big), dtype=torch.uint8,
                     device="cuda")
    for (N, K), zero in ((big, False), (small, False), (small, True), (big, False)):
        w = torch.zeros(N, K) if zero else workloads.normal((N, K), 0.02, seed=N + 5 * K, dtype="f32")
        wp, g, c = bt.bitnet_weight_quant_counted(to_dev(w), workspace=ws)
        torch.cuda.synchronize()
        packed_ref = oracle.pack(oracle.weight_quant(host(w))[0])
        assert np.array_equal(wp.cpu().numpy(), packed_ref)
        assert np.array_equal(c.cpu().numpy(), oracle.code_counts(packed_ref, K).astype(np.int64))
        if zero:
            assert c.cpu().tolist() == [N * K, 0, 0, 0]
