"""Parity over seeded random shapes, through the C ABI: the activation quant,
the GEMV, the fused quant + GEMV, the GEMM in its three call forms (every
output with the argmax; y only; y over a residual), the FFN and the layer
stream, each against the oracle on the same inputs. The shapes are drawn from
one fixed seed (log-uniform token counts, widths in multiples of 64 from 64
up), so every run checks the same cases; together they cross the launch
choices of each entry point (one wave or a workgroup per row, GEMV lanes per
row, skinny / 32 x 256 / 64 x 160 / 128 x 160 / 128 x 320 tiles, ragged row
and column tiles, K tails, the K-split down product of the batched stream)
at sizes the fixed cases of the other files do not name, and the samplers over
row counts and lengths that split the rows' passes over 1 to 64 workgroups
with ragged slices."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_exact, assert_f32, log, make_layers, pack_both, run_stream, stream_ctrl, to_dev, \
    to_host, torch_dev

pytestmark = pytest.mark.gpu

_G = np.random.default_rng(20260)


def _tokens(lo, hi, size):
    return np.exp(_G.uniform(np.log(lo), np.log(hi + 1), size)).astype(int).clip(lo, hi)


def _w64(lo, hi, size):
    return 64 * _G.integers(lo, hi + 1, size)


def _cases(*cols):
    return [tuple(int(v) for v in row) for row in zip(*cols)]


QUANT_SWEEP = _cases(_tokens(1, 300, 12), _w64(1, 256, 12), _G.integers(0, 2, 12))
GEMV_SWEEP = _cases(_G.integers(1, 4000, 12), _w64(1, 160, 12), _G.integers(1, 9, 12))
FWD_SWEEP = _cases(_G.integers(1, 6000, 8), _w64(1, 256, 8), _G.integers(0, 2, 8))
GEMM_SWEEP = _cases(_tokens(1, 300, 18), _G.integers(1, 3000, 18), _w64(1, 64, 18), np.arange(18) % 3)
FFN_SWEEP = _cases(_tokens(1, 300, 8), _w64(1, 16, 8), _w64(2, 48, 8), _G.integers(0, 2, 8))
STREAM_SWEEP = _cases(_G.integers(1, 3, 6), _tokens(1, 40, 6), _w64(1, 8, 6), _w64(2, 24, 6))
# sampling: rows, row length, top-k (k) or nucleus (p in thousandths), temperature in tenths
SAMPLE_SWEEP = _cases(_tokens(1, 300, 12), _tokens(1, 60000, 12), _G.integers(0, 2, 12), _G.integers(1, 1000, 12),
                      _G.integers(3, 25, 12))


@pytest.fixture(scope="module")
def bl():
    import bitlinear_amd
    return bitlinear_amd


@pytest.mark.parametrize("m,k,norm", QUANT_SWEEP)
def test_sweep_quant_act(bl, olib, m, k, norm):
    import torch
    m, k, norm = int(m), int(k), bool(norm)
    log(f"sweep quant m={m} k={k} norm={norm}")
    g = W.rng(140, m, k)
    x = W.activations(g, m, k, outliers=True)
    gain = W.gains(g, k) if norm else None
    dev = torch_dev()
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    s = torch.empty(m, dtype=torch.float32, device=dev)
    qs = torch.empty(m, dtype=torch.int32, device=dev)
    bl.bitlinear_quant_act(to_dev(x), to_dev(gain) if norm else None, 1e-5, q, s, qs)
    oq, os_, oqs = oracle.quant_act(x, gain, 1e-5, olib)
    assert_exact(to_host(q), oq, "q")
    assert_exact(to_host(s).view(np.uint32), os_.view(np.uint32), "s_a bits")
    assert_exact(to_host(qs), oqs, "sum(q)")


@pytest.mark.parametrize("n,k,m", GEMV_SWEEP)
def test_sweep_gemv(bl, olib, n, k, m):
    import torch
    n, k, m = int(n), int(k), int(m)
    log(f"sweep gemv n={n} k={k} m={m}")
    g = W.rng(141, n, k + m)
    p = pack_both(W.ternary(g, n, k), olib)
    sw = W.weight_scale(g)
    q, s, qs = oracle.quant_act(W.activations(g, m, k), None, 1e-5, olib)
    res = W.activations(g, m, n)
    dev = torch_dev()
    acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    y = to_dev(res)  # y over the residual, in place
    bl.bitlinear_gemv(to_dev(p), sw, n, k, to_dev(q), to_dev(s), to_dev(qs), m, y, y, acc)
    oy, oacc = oracle.bitlinear(p, sw, k, q, s, olib)
    assert_exact(to_host(acc), oacc, "acc")
    assert_f32(to_host(y), oracle.residual_add(res, oy, olib), "y + residual")


@pytest.mark.parametrize("n,k,norm", FWD_SWEEP)
def test_sweep_forward_one_token(bl, olib, n, k, norm):
    """bitlinear_forward at one token: the quant inside the GEMV's launch (one
    wave per workgroup up to K = 4096, 512-thread workgroups on blocks of rows
    above)."""
    import torch
    n, k, norm = int(n), int(k), bool(norm)
    log(f"sweep forward n={n} k={k} norm={norm}")
    g = W.rng(142, n, k)
    p = pack_both(W.ternary(g, n, k), olib)
    sw = W.weight_scale(g)
    x = W.activations(g, 1, k, outliers=True)
    gain = W.gains(g, k) if norm else None
    dev = torch_dev()
    q = torch.empty((1, k), dtype=torch.int8, device=dev)
    s = torch.empty(1, dtype=torch.float32, device=dev)
    qs = torch.empty(1, dtype=torch.int32, device=dev)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)
    bl.bitlinear_forward(to_dev(x), to_dev(gain) if norm else None, 1e-5, to_dev(p), sw, n, q, s, qs, y)
    oq, os_, _ = oracle.quant_act(x, gain, 1e-5, olib)
    oy, _ = oracle.bitlinear(p, sw, k, oq, os_, olib)
    assert_exact(to_host(q), oq, "q")
    assert_f32(to_host(y), oy, "y")


@pytest.mark.parametrize("m,n,k,form", GEMM_SWEEP)
def test_sweep_gemm(bl, olib, m, n, k, form):
    """form 0: y, exact accumulators and the row argmax; 1: y only; 2: y over
    a residual."""
    import torch
    m, n, k, form = int(m), int(n), int(k), int(form)
    log(f"sweep gemm m={m} n={n} k={k} form={form}")
    g = W.rng(143, m + n, k + form)
    p = pack_both(W.ternary(g, n, k), olib)
    sw = W.weight_scale(g)
    q, s, qs = oracle.quant_act(W.activations(g, m, k, outliers=True), None, 1e-5, olib)
    dev = torch_dev()
    oy, oacc = oracle.bitlinear(p, sw, k, q, s, olib)
    args = (to_dev(p), sw, n, k, to_dev(q), to_dev(s), to_dev(qs), m)
    if form == 0:
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        acc = torch.empty((m, n), dtype=torch.int32, device=dev)
        am = torch.empty(m, dtype=torch.int32, device=dev)
        ws = torch.empty(max(bl.bitlinear_gemm_workspace_bytes(m, n, k, 1), 8), dtype=torch.uint8, device=dev)
        bl.bitlinear_gemm(*args, None, y, acc, am, ws)
        assert_exact(to_host(acc), oacc, "acc")
        assert_f32(to_host(y), oy, "y")
        assert_exact(to_host(am), oracle.argmax_rows(oacc, olib), "row argmax")
    elif form == 1:
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
        bl.bitlinear_gemm(*args, None, y)
        assert_f32(to_host(y), oy, "y")
    else:
        res = W.activations(g, m, n)
        y = to_dev(res)
        bl.bitlinear_gemm(*args, y, y)
        assert_f32(to_host(y), oracle.residual_add(res, oy, olib), "y + residual")


@pytest.mark.parametrize("m,d,f,acc", FFN_SWEEP)
def test_sweep_ffn(bl, olib, m, d, f, acc):
    import torch
    m, d, f, acc = int(m), int(d), int(f), bool(acc)
    log(f"sweep ffn m={m} d={d} f={f} acc={acc}")
    g = W.rng(144, m, d + f)
    tg, tu, td = W.ternary(g, f, d), W.ternary(g, f, d), W.ternary(g, d, f)
    sg, su, sd = W.weight_scale(g), W.weight_scale(g), W.weight_scale(g)
    x = W.activations(g, m, d)
    gn, gs = W.gains(g, d), W.gains(g, f)
    pg, pu, pd = pack_both(tg, olib), pack_both(tu, olib), pack_both(td, olib)
    dev = torch_dev()
    out = torch.empty((m, d), dtype=torch.float32, device=dev)
    ws = torch.full((bl.bitnet_ffn_workspace_bytes(m, d, f),), 0x5A, dtype=torch.uint8, device=dev)
    bl.bitnet_ffn(to_dev(x), m, d, f, to_dev(gn), to_dev(gs), 1e-5, to_dev(pg), sg, to_dev(pu), su, to_dev(pd), sd,
                  None, out, ws, flags=bl.BITNET_FFN_WRITE_ACC if acc else 0)
    r = oracle.ffn(x, gn, gs, 1e-5, pg, sg, pu, su, pd, sd, olib)
    view = lambda seg: to_host(bl.ffn_workspace_view(ws, m, d, f, seg))
    assert_f32(view("h"), r["h"], "h")
    if acc:
        assert_exact(view("acc_gate"), r["acc_gate"], "acc_gate")
        assert_exact(view("acc_down"), r["acc_down"], "acc_down")
    assert_f32(to_host(out), r["out"], "out")


@pytest.mark.parametrize("n_layers,m,d,f", STREAM_SWEEP)
def test_sweep_stream(bl, olib, n_layers, m, d, f):
    n_layers, m, d, f = int(n_layers), int(m), int(d), int(f)
    log(f"sweep stream layers={n_layers} m={m} d={d} f={f}")
    layers, dev = make_layers(W.W_STREAM, n_layers, d, f, m, olib)
    x0 = W.activations(W.rng(W.W_STREAM, 997, m), m, d)
    x, qkv, ws = run_stream(dev, n_layers, m, d, f, 1e-5, x0)
    assert stream_ctrl(ws)[1] == 0, "stream status word"
    ox, oqkv = oracle.chain(x0, layers, 1e-5, olib)
    for l in range(n_layers):
        assert_f32(qkv[l], oqkv[l], f"qkv layer {l}")
    assert_f32(x, ox, "x after the stream")


@pytest.mark.parametrize("m,n,topp,param,temp10", SAMPLE_SWEEP)
def test_sweep_sample(bl, olib, m, n, topp, param, temp10):
    import torch
    temp = temp10 / 10.0
    g = W.rng(145, m, n)
    logits = (g.standard_normal((m, n)) * g.uniform(0.5, 4.0)).astype(np.float32)
    u = g.random(m)
    log(f"sweep sample m={m} n={n} {'topp' if topp else 'topk'} {param} T={temp}")
    dev = torch_dev()
    tok = torch.full((m,), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(bl.bitnet_sample_workspace_bytes(m, n), dtype=torch.uint8, device=dev)
    ud = torch.from_numpy(np.ascontiguousarray(u, np.float64)).to(dev)
    if topp:
        p = param / 1000.0
        bl.bitnet_sample_topp(to_dev(logits), p, temp, ud, tok, ws)
        want = oracle.sample_topp(logits, p, temp, u, olib)
    else:
        bl.bitnet_sample_topk(to_dev(logits), param, temp, ud, tok, ws)
        want = oracle.sample_topk(logits, param, temp, u, olib)
    assert_exact(to_host(tok), want, "sampled tokens")
