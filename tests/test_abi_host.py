"""C ABI on the CPU: the library loads without a GPU, exports every symbol of
include/bitlinear.h, its host packer and weight_quant match the oracle bit for
bit, and every argument check of the device entry points fires on the host
before any launch (no device memory is touched: the pointers below are never
dereferenced)."""
import os
import re

import numpy as np
import pytest

import bitlinear_amd as bl
import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)) - {"defined"})


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(bl._lib, name), name
    assert sorted(bl.EXPORTS) == names


def test_abi_version_and_strerror():
    assert bl.abi_version() == 1
    for code in range(-7, 1):
        assert bl.strerror(code) and bl.strerror(code) != "unknown status"
    assert bl.strerror(-99) == "unknown status"


# ---- packer / weight_quant vs oracle -----------------------------------------------

@pytest.mark.parametrize("n,k,seed", [(1, 4, 0), (3, 8, 1), (17, 64, 2), (256, 2560, 3), (5, 10244, 4)])
def test_pack_matches_oracle(n, k, seed, olib):
    t = W.ternary(W.rng(90, seed, 0), n, k)
    assert (bl.bitlinear_pack(t) == oracle.pack(t, olib)).all()


def test_pack_adversarial_rows(olib):
    import itertools
    tuples = np.array(list(itertools.product((-1, 0, 1), repeat=4)), np.int8)
    assert (bl.bitlinear_pack(tuples) == oracle.pack(tuples, olib)).all()
    for fill in (-1, 0, 1):
        t = np.full((7, 128), fill, np.int8)
        assert (bl.bitlinear_pack(t) == oracle.pack(t, olib)).all()


def test_pack_rejects_bad_input():
    t = np.zeros((2, 8), np.int8)
    t[1, 5] = 2
    out = np.full((2, 2), 0xEE, np.uint8)
    with pytest.raises(bl.BitlinearError) as e:
        bl.bitlinear_pack(t, out)
    assert e.value.status == bl.BL_ERR_VALUE
    assert (out == 0xEE).all(), "nothing may be written on error"
    with pytest.raises(bl.BitlinearError) as e:
        bl.bitlinear_pack(np.zeros((2, 6), np.int8), np.zeros((2, 1), np.uint8))
    assert e.value.status == bl.BL_ERR_SHAPE
    assert bl._lib.bitlinear_pack(None, 1, 4, 16) == bl.BL_ERR_NULL


@pytest.mark.parametrize("seed,sigma", [(0, 0.02), (1, 1.0), (2, 1e-3)])
def test_weight_quant_matches_oracle(seed, sigma, olib):
    w = W.random_fp32_weights(W.rng(91, seed, 0), 96, 320, sigma)
    t1, s1 = bl.bitlinear_weight_quant(w)
    t2, s2 = oracle.weight_quant(w, olib)
    assert s1 == s2
    assert (t1 == t2).all()


def test_weight_quant_ties_and_zero(olib):
    a = np.float32(0.125)
    w = np.array([[a, -a, 3 * a, -3 * a]], np.float32)
    for arr in (w, np.zeros((4, 8), np.float32)):
        t1, s1 = bl.bitlinear_weight_quant(arr)
        t2, s2 = oracle.weight_quant(arr, olib)
        assert s1 == s2 and (t1 == t2).all()
    bad = np.ones((2, 2), np.float32)
    bad[0, 1] = np.nan
    with pytest.raises(bl.BitlinearError) as e:
        bl.bitlinear_weight_quant(bad)
    assert e.value.status == bl.BL_ERR_VALUE


# ---- argument checks of the device entry points (host only) -------------------------

A = 1 << 20       # a 256-aligned fake address, never dereferenced
U = A + 1         # misaligned
S = None          # null stream


def test_quant_act_checks():
    f = bl._lib.bitlinear_quant_act
    assert f(None, None, 1e-5, 1, 64, A, A, A, S) == bl.BL_ERR_NULL
    assert f(A, None, 1e-5, 1, 64, None, A, A, S) == bl.BL_ERR_NULL
    assert f(A, None, 1e-5, 1, 64, A, None, A, S) == bl.BL_ERR_NULL
    assert f(A, None, 1e-5, 0, 64, A, A, A, S) == bl.BL_ERR_SHAPE
    assert f(A, None, 1e-5, 1, 96, A, A, A, S) == bl.BL_ERR_SHAPE
    assert f(A, None, 1e-5, 1, 0, A, A, A, S) == bl.BL_ERR_SHAPE
    assert f(U, None, 1e-5, 1, 64, A, A, A, S) == bl.BL_ERR_ALIGN
    assert f(A, A + 4, 1e-5, 1, 64, A, A, A, S) == bl.BL_ERR_ALIGN
    assert f(A, None, 1e-5, 1, 64, A + 8, A, A, S) == bl.BL_ERR_ALIGN


def test_gemv_checks():
    f = bl._lib.bitlinear_gemv
    ok = dict(p=A, s=40.0, n=16, k=64, q=A, sa=A, qs=A, m=1, r=None, y=A, acc=None)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["p"], a["s"], a["n"], a["k"], a["q"], a["sa"], a["qs"], a["m"], a["r"], a["y"], a["acc"], S)

    assert call(p=None) == bl.BL_ERR_NULL
    assert call(qs=None) == bl.BL_ERR_NULL
    assert call(y=None) == bl.BL_ERR_NULL
    assert call(m=0) == bl.BL_ERR_SHAPE
    assert call(m=9) == bl.BL_ERR_SHAPE
    assert call(k=100) == bl.BL_ERR_SHAPE
    assert call(k=65536) == bl.BL_ERR_SHAPE
    assert call(n=0) == bl.BL_ERR_SHAPE
    assert call(p=A + 4) == bl.BL_ERR_ALIGN
    assert call(q=A + 8) == bl.BL_ERR_ALIGN
    assert call(y=U) == bl.BL_ERR_ALIGN
    assert call(s=0.0) == bl.BL_ERR_VALUE
    assert call(s=-3.0) == bl.BL_ERR_VALUE
    assert call(s=float("inf")) == bl.BL_ERR_VALUE
    assert call(s=float("nan")) == bl.BL_ERR_VALUE


def test_forward_checks():
    f = bl._lib.bitlinear_forward
    ok = dict(x=A, g=None, p=A, s=40.0, n=16, k=64, m=1, q=A, sa=A, qs=A, y=A)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["x"], a["g"], 1e-5, a["p"], a["s"], a["n"], a["k"], a["m"], a["q"], a["sa"], a["qs"], a["y"], S)

    assert call(x=None) == bl.BL_ERR_NULL
    assert call(p=None) == bl.BL_ERR_NULL
    assert call(q=None) == bl.BL_ERR_NULL
    assert call(sa=None) == bl.BL_ERR_NULL
    assert call(qs=None) == bl.BL_ERR_NULL
    assert call(y=None) == bl.BL_ERR_NULL
    assert call(m=0) == bl.BL_ERR_SHAPE
    assert call(m=9) == bl.BL_ERR_SHAPE
    assert call(k=96) == bl.BL_ERR_SHAPE
    assert call(k=65536) == bl.BL_ERR_SHAPE
    assert call(n=0) == bl.BL_ERR_SHAPE
    assert call(x=A + 4) == bl.BL_ERR_ALIGN
    assert call(g=A + 8) == bl.BL_ERR_ALIGN
    assert call(p=A + 4) == bl.BL_ERR_ALIGN
    assert call(q=A + 8) == bl.BL_ERR_ALIGN
    assert call(sa=U) == bl.BL_ERR_ALIGN
    assert call(y=U) == bl.BL_ERR_ALIGN
    assert call(s=0.0) == bl.BL_ERR_VALUE
    assert call(s=float("nan")) == bl.BL_ERR_VALUE


def test_gemm_checks():
    f = bl._lib.bitlinear_gemm
    ok = dict(p=A, s=40.0, n=16, k=64, q=A, sa=A, qs=A, m=3, r=None, y=A, acc=None, am=None, ws=None, wsb=0)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["p"], a["s"], a["n"], a["k"], a["q"], a["sa"], a["qs"], a["m"], a["r"], a["y"], a["acc"], a["am"],
                 a["ws"], a["wsb"], S)

    assert call(y=None) == bl.BL_ERR_NULL
    assert call(am=A) == bl.BL_ERR_NULL           # argmax without workspace
    assert call(am=A, ws=A, wsb=8) == bl.BL_ERR_WORKSPACE
    assert bl.bitlinear_gemm_workspace_bytes(3, 16, 64, 1) >= 24
    assert bl.bitlinear_gemm_workspace_bytes(3, 16, 64, 0) == 0
    assert call(m=0) == bl.BL_ERR_SHAPE
    assert call(k=32) == bl.BL_ERR_SHAPE
    assert call(am=A, ws=A + 4, wsb=256) == bl.BL_ERR_ALIGN
    assert call(s=0.0) == bl.BL_ERR_VALUE


def test_gemm_noalloc_checks():
    """Every check of bitlinear_gemm_noalloc fires on the host before any device
    call (this container has no GPU: a call that got past them would fail with
    BL_ERR_DEVICE instead)."""
    f = bl._lib.bitlinear_gemm_noalloc
    ok = dict(p=A, s=40.0, n=16, k=64, q=A, sa=A, qs=A, m=3, r=None, y=A, acc=None, am=None)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["p"], a["s"], a["n"], a["k"], a["q"], a["sa"], a["qs"], a["m"], a["r"], a["y"], a["acc"], a["am"],
                 S)

    cap = bl.bitlinear_gemm_noalloc_max_scratch_bytes()
    assert cap == 1 << 20
    assert call(p=None) == bl.BL_ERR_NULL
    assert call(y=None) == bl.BL_ERR_NULL
    assert call(m=0) == bl.BL_ERR_SHAPE
    assert call(k=96) == bl.BL_ERR_SHAPE
    assert call(p=A + 4) == bl.BL_ERR_ALIGN
    assert call(am=U) == bl.BL_ERR_ALIGN
    assert call(s=float("nan")) == bl.BL_ERR_VALUE
    # the LM head of the pages (32 tokens x 50000) fits; beyond the array it is refused
    assert bl.bitlinear_gemm_workspace_bytes(32, 50000, 2048, 1) <= cap
    n_big = 32 * (cap // (32 * 8)) + 64
    assert bl.bitlinear_gemm_workspace_bytes(32, n_big, 2048, 1) > cap
    assert call(m=32, n=n_big, k=2048, am=A) == bl.BL_ERR_WORKSPACE
    assert call(m=cap // 8 + 64, n=16, k=64, am=A) == bl.BL_ERR_WORKSPACE


def test_ffn_checks():
    f = bl._lib.bitnet_ffn
    m, d, f_ = 1, 64, 128
    need = bl.bitnet_ffn_workspace_bytes(m, d, f_)
    ok = dict(x=A, m=m, d=d, f=f_, g=A, gs=A, eps=1e-5, wg=A, sg=1.0, wu=A, su=1.0, wd=A, sd=1.0, r=None, out=A,
              ws=A, wsb=need, flags=0)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["x"], a["m"], a["d"], a["f"], a["g"], a["gs"], a["eps"], a["wg"], a["sg"], a["wu"], a["su"],
                 a["wd"], a["sd"], a["r"], a["out"], a["ws"], a["wsb"], a["flags"], S)

    assert call(g=None) == bl.BL_ERR_NULL
    assert call(ws=None) == bl.BL_ERR_NULL
    assert call(d=96) == bl.BL_ERR_SHAPE
    assert call(f=100) == bl.BL_ERR_SHAPE
    assert call(ws=A + 16) == bl.BL_ERR_ALIGN
    assert call(wd=A + 4) == bl.BL_ERR_ALIGN
    assert call(su=0.0) == bl.BL_ERR_VALUE
    assert call(wsb=need - 1) == bl.BL_ERR_WORKSPACE


def test_ffn_workspace_layout():
    m, d, f = 3, 2560, 10240
    total = bl.bitnet_ffn_workspace_bytes(m, d, f)
    sizes = {"q1": m * d, "s1": 4 * m, "qs1": 4 * m, "h": 4 * m * f, "q2": m * f, "s2": 4 * m, "qs2": 4 * m,
             "acc_gate": 4 * m * f, "acc_up": 4 * m * f, "acc_down": 4 * m * d, "gate": 0, "up": 0}
    spans = []
    for seg in bl.FFN_WS_SEGMENTS:
        off = bl.bitnet_ffn_workspace_offset(m, d, f, seg)
        assert off % 256 == 0
        spans.append((off, off + sizes[seg]))
    spans.sort()
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0, "segments overlap"
    assert spans[-1][1] <= total
    assert bl.bitnet_ffn_workspace_offset(m, d, f, 99) == 2 ** 64 - 1


def test_stream_checks():
    f = bl._lib.bitnet_decode_stream
    m, d, ff = 1, 64, 128
    need = bl.bitnet_stream_workspace_bytes(m, d, ff)
    assert bl.bitnet_layer_bytes(2560, 10240) == 26_214_400
    assert bl.bitnet_layer_bytes(2048, 8192) == 402_653_184 // 24
    assert f(A, A, A, A, 2, m, d, ff, 1e-5, A, None, A, need - 1, S) == bl.BL_ERR_WORKSPACE
    assert f(A, A, A, None, 2, m, d, ff, 1e-5, A, None, A, need, S) == bl.BL_ERR_NULL
    assert f(A, A, A, A, 0, m, d, ff, 1e-5, A, None, A, need, S) == bl.BL_ERR_SHAPE
    assert f(A, A, A, A, 2, m, 80, ff, 1e-5, A, None, A, need, S) == bl.BL_ERR_SHAPE
    assert f(A + 8, A, A, A, 2, m, d, ff, 1e-5, A, None, A, need, S) == bl.BL_ERR_ALIGN


def test_header_states_the_oracle_partial_order():
    """The numerics contract of the header names the same RMSNorm summation
    order as the oracle: the partial count, and ascending butterfly offsets
    from 1 up to half the partial count."""
    text = re.sub(r"\s+", " ", open(HEADER).read())
    m = re.search(r"(\d+) strided partials", text)
    assert m, "the header does not state the partial count"
    header_partials = int(m.group(1))
    src = open(os.path.join(ROOT, "oracle", "bitlinear_oracle.c")).read()
    oracle_partials = int(re.search(r"#define ORACLE_PARTIALS (\d+)", src).group(1))
    assert header_partials == oracle_partials
    m = re.search(r"offsets 1, 2, 4, \.\.\., (\d+) in that ascending order", text)
    assert m, "the header does not state ascending butterfly offsets"
    assert int(m.group(1)) == oracle_partials // 2
    assert "for (int off = 1; off < ORACLE_PARTIALS; off *= 2)" in src


def test_embed_checks():
    f = bl._lib.bitnet_embed
    ok = dict(t=A, s=40.0, v=100, d=64, tok=A, m=2, x=A)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["t"], a["s"], a["v"], a["d"], a["tok"], a["m"], a["x"], S)

    assert call(t=None) == bl.BL_ERR_NULL
    assert call(tok=None) == bl.BL_ERR_NULL
    assert call(x=None) == bl.BL_ERR_NULL
    assert call(d=96) == bl.BL_ERR_SHAPE
    assert call(v=0) == bl.BL_ERR_SHAPE
    assert call(m=0) == bl.BL_ERR_SHAPE
    assert call(t=A + 4) == bl.BL_ERR_ALIGN
    assert call(x=A + 4) == bl.BL_ERR_ALIGN
    assert call(tok=U) == bl.BL_ERR_ALIGN
    assert call(s=0.0) == bl.BL_ERR_VALUE
    assert call(s=float("inf")) == bl.BL_ERR_VALUE


def test_greedy_head_checks():
    f = bl._lib.bitnet_greedy_head
    m, n = 4, 1000
    need = bl.bitnet_greedy_head_workspace_bytes(m, n)
    assert need > 0 and bl.bitnet_greedy_head_workspace_bytes(33, n) == 0
    ok = dict(h=A, s=40.0, n=n, k=64, q=A, sa=A, qs=A, m=m, hist=A, stride=8, hl=A, p=1.1, lg=None, nx=A, ws=A,
              wsb=need)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["h"], a["s"], a["n"], a["k"], a["q"], a["sa"], a["qs"], a["m"], a["hist"], a["stride"], a["hl"],
                 a["p"], a["lg"], a["nx"], a["ws"], a["wsb"], S)

    assert call(h=None) == bl.BL_ERR_NULL
    assert call(nx=None) == bl.BL_ERR_NULL
    assert call(hist=None) == bl.BL_ERR_NULL
    assert call(hl=None) == bl.BL_ERR_NULL
    assert call(m=33) == bl.BL_ERR_SHAPE
    assert call(k=100) == bl.BL_ERR_SHAPE
    assert call(stride=-1) == bl.BL_ERR_SHAPE
    assert call(ws=A + 128) == bl.BL_ERR_ALIGN
    assert call(hist=U) == bl.BL_ERR_ALIGN
    assert call(p=0.0) == bl.BL_ERR_VALUE
    assert call(p=float("nan")) == bl.BL_ERR_VALUE
    assert call(s=-1.0) == bl.BL_ERR_VALUE
    assert call(wsb=need - 1) == bl.BL_ERR_WORKSPACE


def test_greedy_step_checks():
    f = bl._lib.bitnet_greedy_step
    m, d, ff, vocab = 2, 64, 128, 500
    need = bl.bitnet_greedy_step_workspace_bytes(m, d, ff, vocab)
    assert need >= bl.bitnet_stream_workspace_bytes(m, d, ff)
    ok = dict(e=A, se=30.0, v=vocab, w=A, sc=A, g=A, z=A, L=2, d=d, f=ff, eps=1e-5, gf=A, h=A, sh=40.0, tok=A, m=m,
              hist=A, stride=4, hl=A, p=1.1, x=A, lg=None, ws=A, wsb=need)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["e"], a["se"], a["v"], a["w"], a["sc"], a["g"], a["z"], a["L"], a["d"], a["f"], a["eps"], a["gf"],
                 a["h"], a["sh"], a["tok"], a["m"], a["hist"], a["stride"], a["hl"], a["p"], a["x"], a["lg"], a["ws"],
                 a["wsb"], S)

    assert call(e=None) == bl.BL_ERR_NULL
    assert call(tok=None) == bl.BL_ERR_NULL
    assert call(z=None) == bl.BL_ERR_NULL
    assert call(hist=None) == bl.BL_ERR_NULL
    assert call(m=33) == bl.BL_ERR_SHAPE
    assert call(d=100) == bl.BL_ERR_SHAPE
    assert call(L=0) == bl.BL_ERR_SHAPE
    assert call(x=A + 4) == bl.BL_ERR_ALIGN
    assert call(ws=A + 16) == bl.BL_ERR_ALIGN
    assert call(p=-1.0) == bl.BL_ERR_VALUE
    assert call(se=0.0) == bl.BL_ERR_VALUE
    assert call(wsb=need - 1) == bl.BL_ERR_WORKSPACE


def test_sample_checks():
    m, n = 3, 100
    need = bl.bitnet_sample_workspace_bytes(m, n)
    assert need >= m * n * 8
    for name in ("bitnet_sample_topk", "bitnet_sample_topp"):
        f = getattr(bl._lib, name)
        par = 5 if name.endswith("topk") else 0.9

        def call(**kw):
            a = {**dict(l=A, m=m, n=n, p=par, t=1.0, u=A, tok=A, ws=A, wsb=need), **kw}
            return f(a["l"], a["m"], a["n"], a["p"], a["t"], a["u"], a["tok"], a["ws"], a["wsb"], S)

        assert call(l=None) == bl.BL_ERR_NULL
        assert call(u=None) == bl.BL_ERR_NULL
        assert call(tok=None) == bl.BL_ERR_NULL
        assert call(m=0) == bl.BL_ERR_SHAPE
        assert call(n=0) == bl.BL_ERR_SHAPE
        assert call(n=1 << 23, wsb=1 << 40) == bl.BL_ERR_SHAPE  # the total weight would not fit an int64
        assert call(u=A + 4) == bl.BL_ERR_ALIGN
        assert call(ws=A + 8) == bl.BL_ERR_ALIGN
        assert call(t=0.0) == bl.BL_ERR_VALUE
        assert call(p=0) == bl.BL_ERR_VALUE
        assert call(wsb=need - 1) == bl.BL_ERR_WORKSPACE


@pytest.mark.parametrize("base,hd,npos", [(10000.0, 80, 64), (10000.0, 128, 33), (500000.0, 64, 17), (2.5, 2, 5)])
def test_rope_table_matches_oracle(base, hd, npos, olib):
    c, s = bl.bitnet_rope_table(base, hd, npos)
    oc, os_ = oracle.rope_table(base, hd, npos, olib)
    assert (c.view(np.uint32) == oc.view(np.uint32)).all() and (s.view(np.uint32) == os_.view(np.uint32)).all()


def test_rope_table_checks():
    f = bl._lib.bitnet_rope_table
    assert f(10000.0, 8, 4, None, A) == bl.BL_ERR_NULL
    assert f(10000.0, 7, 4, A, A) == bl.BL_ERR_SHAPE
    assert f(10000.0, 8, 0, A, A) == bl.BL_ERR_SHAPE
    assert f(1.0, 8, 4, A, A) == bl.BL_ERR_VALUE


def test_decode_step_checks():
    f = bl._lib.bitnet_decode_step
    m, d, ff, H, S = 1, 256, 512, 4, 64
    need = bl.bitnet_decode_step_workspace_bytes(m, d, ff, H, S)
    assert need > bl.bitnet_stream_workspace_bytes(m, d, ff)
    ok = dict(w=A, sc=A, g=A, L=2, m=m, d=d, f=ff, H=H, eps=1e-5, c=A, s=A, S=S, pos=3, kc=A, vc=A, x=A, qkv=None,
              at=None, ws=A, wsb=need)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["w"], a["sc"], a["g"], a["L"], a["m"], a["d"], a["f"], a["H"], a["eps"], a["c"], a["s"], a["S"],
                 a["pos"], a["kc"], a["vc"], a["x"], a["qkv"], a["at"], a["ws"], a["wsb"], S_)

    S_ = None
    assert call(kc=None) == bl.BL_ERR_NULL
    assert call(c=None) == bl.BL_ERR_NULL
    assert call(pos=S) == bl.BL_ERR_SHAPE
    assert call(pos=-1) == bl.BL_ERR_SHAPE
    assert call(H=3) == bl.BL_ERR_SHAPE       # d % H != 0
    assert call(H=128) == bl.BL_ERR_SHAPE     # hd = 2, not a multiple of 4
    assert call(H=1, d=512, f=512) == bl.BL_ERR_SHAPE  # hd = 512 > 256
    assert call(kc=A + 4) == bl.BL_ERR_ALIGN
    assert call(at=A + 8) == bl.BL_ERR_ALIGN
    assert call(wsb=need - 1) == bl.BL_ERR_WORKSPACE
