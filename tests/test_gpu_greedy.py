"""GPU parity of the greedy-decoding entry points against the oracle, through the
C ABI: the ternary embedding lookup, the LM head with repetition penalty and
greedy choice, and whole greedy steps (embedding, layer stream, final norm,
penalised head, history append) run several times in a row on the device.

Bar: embeddings and penalised logits bit-identical (the same fp32 operations on
both sides), chosen tokens and histories exact."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_exact, log, make_layers, pack_both, to_dev, to_host, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import bitlinear_amd
    return bitlinear_amd


@pytest.mark.parametrize("vocab,d,m", [(1000, 2560, 37), (50000, 2048, 32), (7, 64, 9), (3, 128, 1)])
def test_embed(bl, olib, vocab, d, m):
    import torch
    log(f"embed vocab={vocab} d={d} m={m}")
    g = W.rng(130, vocab, d)
    t = W.ternary(g, vocab, d)
    s_e = W.weight_scale(g)
    table = pack_both(t, olib)
    tokens = g.integers(0, vocab, m).astype(np.int32)
    tokens[0] = vocab - 1
    if m > 3:
        tokens[1], tokens[2], tokens[3] = -1, vocab, 2 ** 31 - 1  # outside the table: zero rows
    x = torch.full((m, d), float("nan"), dtype=torch.float32, device=torch_dev())
    bl.bitnet_embed(to_dev(table), s_e, to_dev(tokens), x)
    want = oracle.embed(table, s_e, tokens, d, olib)
    assert_exact(to_host(x).view(np.uint32), want.view(np.uint32), "embedding bits")


def _head_case(bl, olib, m, n, k, stride, penalty, seed, ties=False):
    import torch
    log(f"greedy head m={m} n={n} k={k} stride={stride} penalty={penalty}")
    g = W.rng(131, seed, m)
    t = W.ternary(g, n, k)
    if ties:
        # duplicated rows make equal logits; the penalty then decides between them
        t[n - 1] = t[0]
        t[n // 2] = t[1]
    s_h = W.weight_scale(g)
    p = pack_both(t, olib)
    x = W.activations(g, m, k)
    q, s, qs = oracle.quant_act(x, None, 1e-5, olib)
    hist = g.integers(-5, n + 5, (m, max(stride, 1))).astype(np.int32)[:, :stride] if stride else None
    hist_len = None
    if stride:
        hist_len = g.integers(0, stride + 3, m).astype(np.int32)  # some beyond the stride: clamped
        # the current argmax of each row into its history, so the penalty matters
        _, acc = oracle.bitlinear(p, s_h, k, q, s, olib)
        top = np.argmax(acc, axis=1)
        for r in range(m):
            hist[r, 0] = top[r]
            hist_len[r] = max(hist_len[r], 1)
    dev = torch_dev()
    logits = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    nxt = torch.full((m,), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(bl.bitnet_greedy_head_workspace_bytes(m, n), dtype=torch.uint8, device=dev)
    bl.bitnet_greedy_head(to_dev(p), s_h, n, k, to_dev(q), to_dev(s), to_dev(qs), m,
                          to_dev(hist) if stride else None, to_dev(hist_len) if stride else None, penalty, logits,
                          nxt, ws)
    raw, _ = oracle.bitlinear(p, s_h, k, q, s, olib)
    want_idx, want_pen = oracle.penalty_argmax(raw, hist if stride else np.zeros((m, 0), np.int32),
                                               hist_len if stride else np.zeros(m, np.int32), penalty, olib)
    assert_exact(to_host(logits).view(np.uint32), want_pen.view(np.uint32), "penalised logits bits")
    assert_exact(to_host(nxt), want_idx, "next token")
    return want_idx


@pytest.mark.parametrize("m,n,k,stride,penalty", [(1, 50000, 2560, 64, 1.1), (32, 50000, 2048, 48, 1.1),
                                                   (7, 3000, 256, 5, 1.3), (3, 257, 64, 0, 1.1),
                                                   (32, 1000, 128, 200, 1.0), (5, 999, 192, 9, 2.0),
                                                   (1, 999, 192, 0, 1.1), (1, 7, 64, 3, 2.0)])
def test_greedy_head(bl, olib, m, n, k, stride, penalty):
    """m = 1 runs the head as a GEMV, larger m as the MFMA skinny product."""
    _head_case(bl, olib, m, n, k, stride, penalty, seed=m + n)


def test_greedy_head_ties_and_flips(bl, olib):
    """Duplicated weight rows give equal logits; with the first of each pair in
    the history the penalty must move the choice, and with penalty 1 the lower
    index must win."""
    for m in (16, 1):  # 1: the GEMV form of the head
        for penalty in (1.1, 1.0, 2.0):
            _head_case(bl, olib, m, 640, 128, 8, penalty, seed=7, ties=True)


def _step_inputs(bl, olib, d, f, n_layers, vocab, m, seed):
    g = W.rng(132, seed, 0)
    t_emb = W.ternary(g, vocab, d)
    s_emb = W.weight_scale(g)
    t_head = W.ternary(g, vocab, d)
    s_head = W.weight_scale(g)
    g_final = W.gains(g, d)
    layers, dev = make_layers(W.W_STREAM, n_layers, d, f, m, olib)
    return dict(emb=pack_both(t_emb, olib), s_emb=s_emb, head=pack_both(t_head, olib), s_head=s_head,
                g_final=g_final, layers=layers, dev=dev, tokens=g.integers(0, vocab, m).astype(np.int32))


@pytest.mark.parametrize("m,d,f,n_layers,vocab,stride,steps", [(1, 256, 1024, 2, 3000, 8, 4),
                                                                (4, 256, 1024, 2, 3000, 3, 4),
                                                                (12, 256, 1024, 2, 1500, 16, 3),
                                                                (1, 2560, 10240, 2, 50000, 64, 12)])
def test_greedy_step_loop(bl, olib, m, d, f, n_layers, vocab, stride, steps):
    """Several greedy steps on the device with no host round trip in between,
    against the oracle's greedy_step applied as often (the chosen tokens, the
    histories and the final hidden states of every step). A history of 3 slots
    fills up and then stays as it is. The last case runs twelve tokens of two
    3B-shape layers and the 50000-token head: the persistent stream and the
    block form of the LM head with the penalty."""
    import torch
    log(f"greedy step loop m={m} d={d} f={f} layers={n_layers} vocab={vocab} steps={steps}")
    inp = _step_inputs(bl, olib, d, f, n_layers, vocab, m, seed=m)
    dev = torch_dev()
    dw = inp["dev"]
    tokens = to_dev(inp["tokens"])
    hist = torch.zeros((m, stride), dtype=torch.int32, device=dev)
    hist_len = torch.zeros(m, dtype=torch.int32, device=dev)
    x = torch.empty((m, d), dtype=torch.float32, device=dev)
    ws = torch.zeros(bl.bitnet_greedy_step_workspace_bytes(m, d, f, vocab), dtype=torch.uint8, device=dev)
    emb, head, gf = to_dev(inp["emb"]), to_dev(inp["head"]), to_dev(inp["g_final"])
    o_tok = inp["tokens"].copy()
    o_hist = np.zeros((m, stride), np.int32)
    o_len = np.zeros(m, np.int32)
    got_tokens, got_x = [], []
    for _ in range(steps):
        bl.bitnet_greedy_step(emb, inp["s_emb"], dw["weights"], dw["scales"], dw["gains"], dw["z"], n_layers, d, f,
                              1e-5, gf, head, inp["s_head"], tokens, hist, hist_len, 1.1, x, None, ws)
        got_tokens.append(tokens.clone())
        got_x.append(x.clone())
    for i in range(steps):
        o_tok, o_hist, o_len, o_x = oracle.greedy_step(o_tok, inp["emb"], inp["s_emb"], inp["layers"],
                                                       inp["g_final"], 1e-5, inp["head"], inp["s_head"], o_hist,
                                                       o_len, 1.1, olib)
        assert_exact(to_host(got_x[i]).view(np.uint32), o_x.view(np.uint32), f"hidden state bits, step {i}")
        assert_exact(to_host(got_tokens[i]), o_tok, f"tokens, step {i}")
    assert_exact(to_host(hist), o_hist, "histories")
    assert_exact(to_host(hist_len), o_len, "history lengths")


@pytest.mark.parametrize("d,f,vocab", [(2560, 10240, 50000), (192, 384, 999), (64, 128, 1), (64, 128, 7),
                                        (128, 256, 33), (256, 512, 8193), (4096, 8192, 300)])
def test_greedy_step_one_sequence_logits(bl, olib, d, f, vocab):
    """One sequence: the final norm + quant runs inside the head's launch (one
    workgroup per CU on a block of head rows; 999 and 8193 columns leave a
    short last block, 1 to 33 columns give blocks of one row; d from 64, one
    value per thread, to 4096, eight). Three steps with the penalised logits
    requested; tokens, hidden states, histories and every penalised logit
    against the oracle."""
    import torch
    m, n_layers, stride, steps = 1, 2, 16, 3
    log(f"greedy one sequence d={d} f={f} vocab={vocab}")
    inp = _step_inputs(bl, olib, d, f, n_layers, vocab, m, seed=77)
    dev = torch_dev()
    dw = inp["dev"]
    tokens = to_dev(inp["tokens"])
    hist = torch.zeros((m, stride), dtype=torch.int32, device=dev)
    hist_len = torch.zeros(m, dtype=torch.int32, device=dev)
    x = torch.empty((m, d), dtype=torch.float32, device=dev)
    logits = torch.empty((m, vocab), dtype=torch.float32, device=dev)
    ws = torch.zeros(bl.bitnet_greedy_step_workspace_bytes(m, d, f, vocab), dtype=torch.uint8, device=dev)
    emb, head, gf = to_dev(inp["emb"]), to_dev(inp["head"]), to_dev(inp["g_final"])
    o_tok = inp["tokens"].copy()
    o_hist = np.zeros((m, stride), np.int32)
    o_len = np.zeros(m, np.int32)
    for step in range(steps):
        bl.bitnet_greedy_step(emb, inp["s_emb"], dw["weights"], dw["scales"], dw["gains"], dw["z"], n_layers, d, f,
                              1e-5, gf, head, inp["s_head"], tokens, hist, hist_len, 1.1, x, logits, ws)
        o_x = oracle.embed(inp["emb"], inp["s_emb"], o_tok, d, olib)
        o_x, _ = oracle.chain(o_x, inp["layers"], 1e-5, olib)
        _, o_pen, _ = oracle.greedy_head(o_x, inp["g_final"], 1e-5, inp["head"], inp["s_head"], o_hist, o_len, 1.1,
                                         olib)
        o_tok, o_hist, o_len, _ = oracle.greedy_step(o_tok, inp["emb"], inp["s_emb"], inp["layers"], inp["g_final"],
                                                     1e-5, inp["head"], inp["s_head"], o_hist, o_len, 1.1, olib)
        assert_exact(to_host(x).view(np.uint32), o_x.view(np.uint32), f"hidden state bits, step {step}")
        assert_exact(to_host(logits).view(np.uint32), o_pen.view(np.uint32), f"penalised logits, step {step}")
        assert_exact(to_host(tokens), o_tok, f"tokens, step {step}")
    assert_exact(to_host(hist), o_hist, "histories")
    assert_exact(to_host(hist_len), o_len, "history lengths")
