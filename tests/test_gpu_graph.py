"""A whole BitLinear step captured as one HIP graph with two streams (the
quantizers of X and W in parallel, then the forward, then grad_x and grad_W
in parallel), as bench.py runs it.  Every call is deterministic, so every
replay must reproduce the eager results bit for bit; the outputs are cleared
and other eager work runs between the replays.
"""
import pytest
import torch

import bit_ternary_quantized_amd as bt
import workloads
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _buffers(M, N, K, dev):
    ws = bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, 0, N, K)
    wb = bt.bitnet_workspace_bytes(bt.BITNET_OP_LINEAR_BWD_STE, M, N, K)
    return {
        "Xq": torch.empty(M, K, dtype=torch.int8, device=dev),
        "scale_x": torch.empty(M, dtype=torch.float32, device=dev),
        "W_packed": torch.empty(N, K // 4, dtype=torch.uint8, device=dev),
        "gamma": torch.empty(1, dtype=torch.float32, device=dev),
        "Y": torch.empty(M, N, dtype=torch.float32, device=dev),
        "grad_x": torch.empty(M, K, dtype=torch.float32, device=dev),
        "grad_W": torch.empty(N, K, dtype=torch.float32, device=dev),
        "ws_wq": torch.empty(max(ws, 16), dtype=torch.uint8, device=dev),
        "ws_bwd": torch.empty(max(wb, 16), dtype=torch.uint8, device=dev),
    }


def _calls(x, w, gy, b):
    return {
        "act_quant": lambda: bt.bitnet_act_quant(x, 1e-5, Xq=b["Xq"], scale_x=b["scale_x"]),
        "weight_quant": lambda: bt.bitnet_weight_quant(w, W_packed=b["W_packed"], gamma=b["gamma"],
                                                       workspace=b["ws_wq"]),
        "linear_fwd": lambda: bt.bitnet_linear_fwd(b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], Y=b["Y"]),
        "grad_x": lambda: bt.bitnet_linear_bwd_ste(gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"],
                                                   want_grad_W=False, grad_x=b["grad_x"]),
        "grad_W": lambda: bt.bitnet_linear_bwd_ste(gy, b["Xq"], b["scale_x"], b["W_packed"], b["gamma"],
                                                   want_grad_x=False, grad_W=b["grad_W"], workspace=b["ws_bwd"]),
    }


OUTS = ("Xq", "scale_x", "W_packed", "gamma", "Y", "grad_x", "grad_W")


# plain; token-split grad_W; a tall output whose grad_W reads X_deq^T from the workspace
@pytest.mark.parametrize("M,N,K", [(300, 257, 272), (2048, 100, 48), (300, 8200, 2000)])
def test_two_stream_step_graph_replays_match_eager(M, N, K):
    print(f"two-stream step graph M={M} N={N} K={K}", flush=True)
    d = workloads.linear_inputs(M, N, K, x_dtype="bf16", w_dtype="f32", seed=M + N)
    x, w, gy = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["gy"])
    b = _buffers(M, N, K, x.device)
    c = _calls(x, w, gy, b)
    for n in ("act_quant", "weight_quant", "linear_fwd", "grad_x", "grad_W"):
        c[n]()
    torch.cuda.synchronize()
    ref = {n: b[n].clone() for n in OUTS}

    side = torch.cuda.Stream()

    def fork_join(main_fn, side_fn):
        main = torch.cuda.current_stream()
        e0 = torch.cuda.Event()
        e0.record(main)
        side.wait_event(e0)
        with torch.cuda.stream(side):
            side_fn()
        e1 = torch.cuda.Event()
        e1.record(side)
        main_fn()
        main.wait_event(e1)

    def step():
        fork_join(c["act_quant"], c["weight_quant"])
        c["linear_fwd"]()
        fork_join(c["grad_x"], c["grad_W"])

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    other = to_dev(workloads.normal((64, 128), 1.0, seed=9, dtype="bf16"))
    for rep in range(3):
        for n in OUTS:
            b[n].zero_()
        bt.bitnet_act_quant(other)  # eager library work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(b[n], ref[n]), f"replay {rep}: {n} differs from the eager result"


def test_published_threshold_graph_replays_follow_the_weights():
    # the bench step's calls at a size where one pack workgroup publishes the
    # weight threshold (the two-quantizer call packing beside act_quant, the
    # five-wave weight quant, the counted call), captured once; the weights
    # are rescaled in place between replays, so every replay must publish its
    # own threshold (the row-sum launch clears the word) and match eager calls
    M, N, K = 8192, 4096, 2048
    print(f"published-threshold graph M={M} N={N} K={K}", flush=True)
    dev = "cuda"
    x = to_dev(workloads.normal((M, K), 1.0, seed=3, dtype="bf16"))
    w = to_dev(workloads.normal((N, K), 0.02, seed=4, dtype="bf16"))

    def bufs():
        return {
            "Xq": torch.empty(M, K, dtype=torch.int8, device=dev),
            "scale_x": torch.empty(M, dtype=torch.float32, device=dev),
            "W_packed": torch.empty(N, K // 4, dtype=torch.uint8, device=dev),
            "gamma": torch.empty(1, dtype=torch.float32, device=dev),
            "Y": torch.empty(M, N, dtype=torch.float32, device=dev),
            "W2": torch.empty(N, K // 4, dtype=torch.uint8, device=dev),
            "g2": torch.empty(1, dtype=torch.float32, device=dev),
            "W3": torch.empty(N, K // 4, dtype=torch.uint8, device=dev),
            "g3": torch.empty(1, dtype=torch.float32, device=dev),
            "counts": torch.empty(4, dtype=torch.int64, device=dev),
            "ws": torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, 0, N, K), dtype=torch.uint8,
                              device=dev),
            "ws2": torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT, 0, N, K), dtype=torch.uint8,
                               device=dev),
            "ws3": torch.empty(bt.bitnet_workspace_bytes(bt.BITNET_OP_WEIGHT_QUANT_COUNTED, 0, N, K),
                               dtype=torch.uint8, device=dev),
        }

    def step(b):
        bt.bitnet_quant_operands(x, w, 1e-5, Xq=b["Xq"], scale_x=b["scale_x"], W_packed=b["W_packed"],
                                 gamma=b["gamma"], workspace=b["ws"])
        bt.bitnet_linear_fwd(b["Xq"], b["scale_x"], b["W_packed"], b["gamma"], Y=b["Y"])
        bt.bitnet_weight_quant(w, W_packed=b["W2"], gamma=b["g2"], workspace=b["ws2"])
        bt.bitnet_weight_quant_counted(w, W_packed=b["W3"], gamma=b["g3"], counts=b["counts"], workspace=b["ws3"])

    b, ref = bufs(), bufs()
    outs = ("Xq", "scale_x", "W_packed", "gamma", "Y", "W2", "g2", "W3", "g3", "counts")
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step(b)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(b)
    torch.cuda.synchronize()
    for rep, scale in enumerate((1.0, 3.0, 0.25)):
        w.mul_(scale)
        for n in outs:
            b[n].zero_()
        step(ref)  # eager, on the same weights
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in outs:
            assert torch.equal(b[n], ref[n]), f"replay {rep}: {n} differs from the eager result"
        assert int(b["counts"].sum()) == N * K
