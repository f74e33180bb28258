"""Parity at the full workload sizes, through the same calls the benchmark
times (every output preallocated, the backward with its workspace).

The oracle cannot redo a 70B-shaped product in seconds, so it quantizes both
operands in full (every activation row and its scale, the weight codes and
gamma) and computes the products at sampled entries one by one: the int32
accumulators, Y and both STE gradients.  Every reference is built from the
oracle's own q, scale_x, codes and gamma, never from the GPU's buffers.
Integer results must match bit for bit; Y within relative 1e-3; gradients
within 2e-2 (the elementwise form against |r| + RMS of the sampled
references).  The decode GEMV is checked on every output at each token count.
"""
import numpy as np
import pytest
import torch

import bit_ternary_quantized_amd as bt
import oracle
import workloads
from gpu_util import assert_grad_close, assert_y_close, f32_bits_equal, host, sample_pairs, to_dev

pytestmark = pytest.mark.gpu

LAYERS = ["tiny", "small_llama", "prefill_7b", "qat_70b_mlp"]
N_SAMPLES = 1500  # sampled (row, column) pairs per output


@pytest.mark.parametrize("name", LAYERS)
def test_layer_full_size(name):
    print(f"full-size layer {name}", flush=True)
    d = workloads.workload(name)
    M, N, K = d["M"], d["N"], d["K"]
    x, w = to_dev(d["x"]), to_dev(d["w"])
    dev = x.device
    Xq = torch.empty(M, K, dtype=torch.int8, device=dev)
    scale_x = torch.empty(M, dtype=torch.float32, device=dev)
    W_packed = torch.empty(N, K // 4, dtype=torch.uint8, device=dev)
    gamma = torch.empty(1, dtype=torch.float32, device=dev)
    ws_wq = torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, M, N, K), dtype=torch.uint8,
                        device=dev)
    Y = torch.empty(M, N, dtype=torch.float32, device=dev)
    bt.bitnet_act_quant(x, 1e-5, Xq=Xq, scale_x=scale_x)
    bt.bitnet_weight_quant(w, W_packed=W_packed, gamma=gamma, workspace=ws_wq)
    bt.bitnet_linear_fwd(Xq, scale_x, W_packed, gamma, Y=Y)
    torch.cuda.synchronize()

    # weight quant: codes and gamma in full
    c_ref, g_ref = oracle.weight_quant(host(d["w"]))
    assert f32_bits_equal(gamma.cpu().numpy(), np.array([g_ref], np.float32)), "gamma bits"
    assert np.array_equal(W_packed.cpu().numpy(), oracle.pack(c_ref)), "packed codes"
    print(f"  weight quant ok (gamma {g_ref:.6e})", flush=True)

    # act quant: every row, bit-exact
    q_ref, s_ref = oracle.act_quant(host(d["x"]))
    q_gpu = Xq.cpu().numpy()
    bad = np.flatnonzero((q_gpu != q_ref).any(axis=1))
    assert bad.size == 0, f"Xq differs on {bad.size} of {M} rows (first {bad[:8].tolist()})"
    assert f32_bits_equal(scale_x.cpu().numpy(), s_ref), "scale_x bits"
    del q_gpu
    print(f"  act quant ok on all {M} rows", flush=True)

    # forward: exact int32 at sampled (m, n), the reference from the oracle's
    # q and codes; Y from the launch the benchmark times (no accumulator
    # output)
    ms, ns = sample_pairs(M, N, N_SAMPLES, seed=2)
    acc_ref = oracle.gemm_i32_at(q_ref, c_ref, ms, ns)
    y_ref = acc_ref.astype(np.float64) * np.float64(g_ref) / s_ref[ms].astype(np.float64)
    assert_y_close(Y.cpu().numpy()[ms, ns], y_ref, "Y (sampled)")
    _, acc = bt.bitnet_linear_fwd(Xq, scale_x, W_packed, gamma, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy()[ms, ns], acc_ref), "int32 acc (sampled)"
    print(f"  forward ok on {ms.size} samples", flush=True)

    if d.get("gy") is None:
        return
    gy = to_dev(d["gy"])
    grad_x = torch.empty(M, K, dtype=torch.float32, device=dev)
    grad_W = torch.empty(N, K, dtype=torch.float32, device=dev)
    nws = bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, M, N, K)
    ws_bwd = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    bt.bitnet_linear_bwd_ste(gy, Xq, scale_x, W_packed, gamma, grad_x=grad_x, grad_W=grad_W,
                             workspace=ws_bwd)
    torch.cuda.synchronize()
    gyh = host(d["gy"])
    mk, kk = sample_pairs(M, K, N_SAMPLES, seed=3)
    gx_ref = oracle.ste_grad_x_at(gyh, c_ref, g_ref, mk, kk)
    assert_grad_close(grad_x.cpu().numpy()[mk, kk], gx_ref, "grad_x (sampled)")
    nk_, kw = sample_pairs(N, K, N_SAMPLES, seed=4)
    gw_ref = oracle.ste_grad_w_at(gyh, q_ref, s_ref, nk_, kw)
    assert_grad_close(grad_W.cpu().numpy()[nk_, kw], gw_ref, "grad_W (sampled)")
    print(f"  backward ok on {mk.size} + {nk_.size} samples", flush=True)


@pytest.mark.parametrize("M", workloads.DECODE_MS)
def test_decode_full_size(M):
    print(f"full-size decode M={M}", flush=True)
    d = workloads.workload("decode_7b", M=M)
    q, codes, scale_x, gamma = d["q"], d["codes"], d["scale_x"], d["gamma"]
    wp = bt.bitnet_pack_ternary(to_dev(codes))
    Y, acc = bt.bitnet_linear_fwd(to_dev(q), to_dev(scale_x), wp, to_dev(gamma), want_acc=True)
    Y2, _ = bt.bitnet_linear_fwd(to_dev(q), to_dev(scale_x), wp, to_dev(gamma))
    torch.cuda.synchronize()
    acc_ref, y_ref = oracle.linear_fwd(q.numpy(), scale_x.numpy(), codes.numpy(), float(gamma[0]))
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(Y.cpu().numpy(), y_ref)
    assert np.array_equal(Y.cpu().numpy(), Y2.cpu().numpy())
