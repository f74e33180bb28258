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
