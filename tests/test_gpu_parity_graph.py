"""HIP-graph capture of the library's launch sequences.

The entry points launch only kernels on the caller's stream (no allocation,
no memset, no host synchronisation), so a caller may capture them in a HIP
graph. Each case runs eagerly, captures the same calls, then replays the
graph three times with eager work on the same buffers in between, and checks
every replay bit for bit against the eager result."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import assert_exact, log, make_layers, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import bitlinear_amd
    return bitlinear_amd


def _replay_check(torch, calls, outputs, reset):
    """calls(): the launches; outputs: tensors they write; reset(): eager work
    that disturbs the outputs (and restores in-place inputs) before a replay."""
    reset()
    calls()
    torch.cuda.synchronize()
    want = [to_host(o).copy() for o in outputs]
    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        for o in outputs:  # garbage in every output before the replay
            o.view(torch.uint8).fill_(0x5A + rep)
        reset()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outputs, want)):
            assert_exact(to_host(o).view(np.uint8), w.view(np.uint8), f"output {i}, replay {rep}")


def test_graph_quant_gemv(bl):
    import torch
    dev = torch.device("cuda", 0)
    d = 512
    log("graph quant + gemv")
    g = W.rng(W.W_GEMV, 7, W.T_Q)
    p = to_dev(bl.bitlinear_pack(W.ternary(g, d, d)))
    sw = W.weight_scale(g)
    x = to_dev(W.activations(W.rng(W.W_GEMV, 7, W.T_X), 1, d))
    q = torch.empty((1, d), dtype=torch.int8, device=dev)
    s = torch.empty(1, dtype=torch.float32, device=dev)
    qs = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty((1, d), dtype=torch.float32, device=dev)

    def calls():
        bl.bitlinear_quant_act(x, None, 1e-5, q, s, qs)
        bl.bitlinear_gemv(p, sw, d, d, q, s, qs, 1, None, y)

    _replay_check(torch, calls, [q, s, qs, y], lambda: None)


@pytest.mark.parametrize("m,k,norm", [(1, 2560, False), (1, 10240, True), (3, 2048, True)])
def test_graph_forward(bl, m, k, norm):
    """bitlinear_forward in a graph: the one-launch forms (one wave per workgroup,
    512 threads) and the quant launch with prefetch workgroups + GEMV."""
    import torch
    dev = torch.device("cuda", 0)
    n = 1000
    log(f"graph forward m={m} k={k} norm={norm}")
    g = W.rng(W.W_GEMV, 8, k)
    p = to_dev(bl.bitlinear_pack(W.ternary(g, n, k)))
    sw = W.weight_scale(g)
    x = to_dev(W.activations(W.rng(W.W_GEMV, 8, W.T_X), m, k))
    gain = to_dev(W.gains(g, k)) if norm else None
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    s = torch.empty(m, dtype=torch.float32, device=dev)
    qs = torch.empty(m, dtype=torch.int32, device=dev)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)

    def calls():
        bl.bitlinear_forward(x, gain, 1e-5, p, sw, n, q, s, qs, y)

    _replay_check(torch, calls, [q, s, qs, y], lambda: None)


@pytest.mark.parametrize("m", [1, 20])
def test_graph_ffn(bl, m):
    import torch
    dev = torch.device("cuda", 0)
    d, f = 256, 1024
    log(f"graph ffn m={m}")
    gg = [W.rng(W.W_FFN, 3, tid) for tid in (W.T_GATE, W.T_UP, W.T_DOWN)]
    shapes = ((f, d), (f, d), (d, f))
    packs = [to_dev(bl.bitlinear_pack(W.ternary(gx, n, k))) for gx, (n, k) in zip(gg, shapes)]
    sc = [float(W.weight_scale(gx)) for gx in gg]
    x = to_dev(W.activations(W.rng(W.W_FFN, 3, W.T_X), m, d))
    gn = to_dev(np.linspace(0.5, 1.5, d).astype(np.float32))
    gs = to_dev(np.linspace(1.5, 0.5, f).astype(np.float32))
    out = torch.empty((m, d), dtype=torch.float32, device=dev)
    ws = torch.empty(bl.bitnet_ffn_workspace_bytes(m, d, f), dtype=torch.uint8, device=dev)

    def calls():
        bl.bitnet_ffn(x, m, d, f, gn, gs, 1e-5, packs[0], sc[0], packs[1], sc[1], packs[2], sc[2], x, out, ws)

    _replay_check(torch, calls, [out], lambda: None)


@pytest.mark.parametrize("m", [12, 32, 40])
def test_graph_layer_stream_and_head(bl, olib, m):
    """Multi-token layer stream (one launch per step) plus the LM head with the
    fused argmax; x is updated in place, so every run starts from a copy of x0."""
    import torch
    dev = torch.device("cuda", 0)
    n_layers, d, f, vocab = 2, 256, 512, 1000
    log(f"graph stream + head m={m}")
    layers, dw = make_layers(W.W_STREAM, n_layers, d, f, m, olib)
    x0 = to_dev(W.activations(W.rng(W.W_STREAM, 997, W.T_X), m, d))
    x = x0.clone()
    qkv = torch.empty((n_layers, m, 3 * d), dtype=torch.float32, device=dev)
    ws = torch.zeros(bl.bitnet_stream_workspace_bytes(m, d, f), dtype=torch.uint8, device=dev)
    gh = W.rng(W.W_BATCHED, 5, W.T_HEAD)
    head = to_dev(bl.bitlinear_pack(W.ternary(gh, vocab, d)))
    sh = W.weight_scale(gh)
    gfin = to_dev(np.ones(d, np.float32))
    qf = torch.empty((m, d), dtype=torch.int8, device=dev)
    sf = torch.empty(m, dtype=torch.float32, device=dev)
    qsf = torch.empty(m, dtype=torch.int32, device=dev)
    idx = torch.empty(m, dtype=torch.int32, device=dev)
    wsh = torch.empty(bl.bitlinear_gemm_workspace_bytes(m, vocab, d, 1), dtype=torch.uint8, device=dev)

    def calls():
        bl.bitnet_decode_stream(dw["weights"], dw["scales"], dw["gains"], dw["z"], n_layers, m, d, f, 1e-5, x, qkv,
                                ws)
        bl.bitlinear_quant_act(x, gfin, 1e-5, qf, sf, qsf)
        bl.bitlinear_gemm(head, sh, vocab, d, qf, sf, qsf, m, None, None, None, idx, wsh)

    _replay_check(torch, calls, [x, qkv, qf, sf, qsf, idx], lambda: x.copy_(x0))


def test_graph_one_token_stream(bl, olib):
    """One token of a shape with a persistent kernel: the eager call runs the
    persistent kernel, the captured one the launch-per-step path (the library
    does not record the persistent launch, whose waits span the whole grid);
    the replays must equal the eager result bit for bit."""
    import torch
    dev = torch.device("cuda", 0)
    n_layers, d, f, m = 2, 256, 1024, 1
    log("graph one-token stream")
    layers, dw = make_layers(W.W_STREAM, n_layers, d, f, m, olib)
    x0 = to_dev(W.activations(W.rng(W.W_STREAM, 996, W.T_X), m, d))
    x = x0.clone()
    qkv = torch.empty((n_layers, m, 3 * d), dtype=torch.float32, device=dev)
    ws = torch.zeros(bl.bitnet_stream_workspace_bytes(m, d, f), dtype=torch.uint8, device=dev)

    def calls():
        bl.bitnet_decode_stream(dw["weights"], dw["scales"], dw["gains"], dw["z"], n_layers, m, d, f, 1e-5, x, qkv,
                                ws)

    _replay_check(torch, calls, [x, qkv], lambda: x.copy_(x0))


def test_graph_decode_step_two_sequences(bl, olib):
    """The decode step with attention for two sequences (launch per step both
    eagerly and captured): RoPE, the cache append at pos, attention over the
    prefilled caches, o and the FFN; every replay equals the eager call."""
    import torch
    dev = torch.device("cuda", 0)
    n_layers, d, f, m, heads, max_seq, pos = 2, 256, 1024, 2, 4, 64, 9
    hd = d // heads
    log("graph decode step, two sequences")
    layers, dw = make_layers(W.W_STREAM, n_layers, d, f, m, olib)
    g = W.rng(160, 0, 0)
    x0 = to_dev(W.activations(g, m, d))
    x = x0.clone()
    kc = to_dev(g.standard_normal((n_layers, m, heads, max_seq, hd)).astype(np.float32))
    vc = to_dev(g.standard_normal((n_layers, m, heads, max_seq, hd)).astype(np.float32))
    c, s_ = bl.bitnet_rope_table(10000.0, hd, max_seq)
    cd, sd = to_dev(c), to_dev(s_)
    qkv = torch.empty((n_layers, m, 3 * d), dtype=torch.float32, device=dev)
    attn = torch.empty((n_layers, m, d), dtype=torch.float32, device=dev)
    ws = torch.zeros(bl.bitnet_decode_step_workspace_bytes(m, d, f, heads, max_seq), dtype=torch.uint8, device=dev)

    def calls():
        bl.bitnet_decode_step(dw["weights"], dw["scales"], dw["gains"], n_layers, m, d, f, heads, 1e-5, cd, sd, pos,
                              kc, vc, x, qkv, attn, ws)

    kc0, vc0 = kc.clone(), vc.clone()

    def reset():  # the caches back to their state before the step
        x.copy_(x0)
        kc.copy_(kc0)
        vc.copy_(vc0)

    _replay_check(torch, calls, [x, qkv, attn, kc, vc], reset)
