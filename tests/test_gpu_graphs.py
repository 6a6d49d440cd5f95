"""The entry points captured in HIP graphs (as the benchmark times them):
every replay, with the program's own eager work and synchronisations in
between and the outputs cleared before it, must reproduce the eager result
bit for bit (every kernel here is deterministic).  All buffers are allocated
before the capture and stay referenced while the graph lives."""
import numpy as np
import pytest

import bit_bitlinear_amd as hbl
import oracle
import workloads
from parity import to_dev, to_host

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _announce(msg):
    print("[case] " + msg, flush=True)


def _replay_and_compare(run, outputs, eager_between):
    """run() queues the work; outputs are the tensors it writes."""
    import torch
    run()
    torch.cuda.synchronize()
    ref = [to_host(o).copy() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(REPLAYS):
        for o in outputs:
            o.zero_()
        eager_between()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert np.array_equal(to_host(o), r), "replay %d differs from the eager result" % i
    return g


def _eager_noise():
    """Unrelated eager work between replays (a small forward of its own)."""
    import torch
    rng = np.random.default_rng(99)
    X = to_dev(rng.standard_normal((8, 256)).astype(np.float32))
    W = to_dev(workloads.w_latent(rng, 32, 256))
    hbl.hbl_forward_latent(X, W, hbl.Config(act_bits=8))
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["wo_1.3b", "decode_m1", "decode_m16"])
def test_forward_latent_graph_replays(name):
    import torch
    layer = workloads.by_name(name)
    M, K, N = layer.M, layer.K, layer.N
    _announce("graph forward_latent %s" % layer.desc)
    X, W, _ = workloads.make_inputs(layer, 0)
    Xd = to_dev(X)
    Wd = to_dev(W)
    cfg = hbl.Config(act_bits=layer.act_bits, hadamard=layer.hadamard)
    ydt = torch.bfloat16 if layer.y_dtype == "bf16" else torch.float32
    Y = torch.empty((M, N), dtype=ydt, device="cuda:0")
    Wp = torch.empty((N, K // 4), dtype=torch.uint8, device="cuda:0")
    alpha = torch.empty(1, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(max(1, hbl.hbl_forward_workspace_bytes(M, K, N, cfg)), dtype=torch.uint8, device="cuda:0")
    wws = torch.empty(hbl.hbl_weight_workspace_bytes(N, K), dtype=torch.uint8, device="cuda:0")

    def run():
        hbl.hbl_forward_latent(Xd, Wd, cfg, y_dtype=ydt, W_packed=Wp, alpha=alpha, Y=Y, ws=ws, wws=wws)

    g = _replay_and_compare(run, [Y, Wp, alpha], _eager_noise)
    # the packed weights of the replays are the oracle's, bit for bit
    assert np.array_equal(to_host(Wp), oracle.pack_ternary(oracle.ternarize(W, to_host(alpha)[0], 1e-5)))
    del g


def test_backward_graph_replays():
    import torch
    M, K, N = 512, 2048, 768
    _announce("graph backward M=%d K=%d N=%d" % (M, K, N))
    rng = np.random.default_rng(5)
    X = to_dev(workloads.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    dY = to_dev(rng.standard_normal((M, N)).astype(np.float32))
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(workloads.w_latent(rng, N, K)))
    cfg = hbl.Config(act_bits=4)
    dX = torch.empty((M, K), dtype=torch.float32, device="cuda:0")
    dW = torch.empty((N, K), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(hbl.hbl_backward_workspace_bytes(M, K, N, cfg, True), dtype=torch.uint8, device="cuda:0")

    def run():
        hbl.hbl_backward(dY, X, Wp, alpha, cfg, dX=dX, dW=dW, ws=ws)

    del_g = _replay_and_compare(run, [dX, dW], _eager_noise)
    del del_g


def test_heads_and_base3_graph_replays():
    import torch
    _announce("graph heads + base3")
    rng = np.random.default_rng(8)
    M, H, D = 1024, 8, 128
    Xh = to_dev(workloads.f32_to_bf16_bits(workloads.head_states(rng, M, H, D)))
    codes = torch.empty((M, H, D * 3 // 8), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((M, H), dtype=torch.float32, device="cuda:0")
    K, N = 8192, 1024
    Xd = to_dev(rng.standard_normal((1, K)).astype(np.float32))
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(workloads.w_latent(rng, N, K)))
    W3 = torch.empty((N, hbl.hbl_base3_weight_bytes(1, K)), dtype=torch.uint8, device="cuda:0")
    cfg = hbl.Config(act_bits=4)
    Y = torch.empty((1, N), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(hbl.hbl_workspace_bytes(1, K, cfg), dtype=torch.uint8, device="cuda:0")

    def run():
        hbl.hbl_quantize_heads(Xh, H, 3, 1e-5, codes=codes, scales=scales)
        hbl.hbl_pack_base3(Wp, K, W3=W3)
        hbl.hbl_forward_base3(Xd, W3, alpha, N, cfg, Y=Y, ws=ws)

    g = _replay_and_compare(run, [codes, scales, W3, Y], _eager_noise)
    del g


def test_fp4_fp6_graph_replays():
    """The FP6 x FP4 path: weight conversion, FP6 activation codes, the GEMM
    and the forward, all in one graph, against the eager results."""
    import torch
    M, K, N = 1000, 4096, 2048  # ragged M: a partial last tile row
    _announce("graph fp4/fp6 M=%d K=%d N=%d" % (M, K, N))
    rng = np.random.default_rng(9)
    Xd = to_dev(workloads.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(workloads.w_latent(rng, N, K)))
    cfg = hbl.Config(act_bits=4, hadamard=True)
    W4 = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda:0")
    codes6 = torch.empty((M, K * 3 // 4), dtype=torch.uint8, device="cuda:0")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda:0")
    Y1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    Y2 = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(hbl.hbl_forward_fp4_workspace_bytes(M, K, cfg), dtype=torch.uint8, device="cuda:0")

    def run():
        hbl.hbl_pack_fp4(Wp, K, W4=W4)
        hbl.hbl_quantize_activations_fp6(Xd, cfg, codes6=codes6, xscale=xs)
        hbl.hbl_gemm_fp6fp4(codes6, xs, K, W4, alpha, N, Y=Y1)
        hbl.hbl_forward_fp4(Xd, W4, alpha, N, cfg, Y=Y2, ws=ws)

    g = _replay_and_compare(run, [W4, codes6, xs, Y1, Y2], _eager_noise)
    del g


def test_forward_noalloc_graph_replays():
    """The no-allocation forward is meant for graph capture: replays of the
    captured call reproduce hbl_forward's eager result bit for bit."""
    import torch
    layer = workloads.by_name("wo_1.3b")
    M, K, N = layer.M, layer.K, layer.N
    _announce("graph forward_noalloc %s" % layer.desc)
    X, W, _ = workloads.make_inputs(layer, 0)
    Xd = to_dev(X)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    cfg = hbl.Config(act_bits=layer.act_bits, hadamard=layer.hadamard)
    Y_ref = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")

    def run():
        hbl.hbl_forward_noalloc(Xd, Wp, alpha, N, cfg, Y=Y)

    g = _replay_and_compare(run, [Y], _eager_noise)
    assert np.array_equal(to_host(Y), to_host(Y_ref)), "no-alloc forward differs from hbl_forward"
    del g
