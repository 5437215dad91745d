"""HIP path vs the CPU oracle, element by element, through the C ABI.

Sizes span several tiles with ragged tails, up to the full shapes of the
benchmark for single projections."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_exact, assert_f32, log, pack_both, to_dev, to_host, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import bitlinear_amd
    return bitlinear_amd


def quant_gpu(bl, x, gain, eps):
    import torch
    m, k = x.shape
    dev = torch_dev()
    xd = to_dev(x)
    gd = to_dev(gain) if gain is not None else None
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    s = torch.empty(m, dtype=torch.float32, device=dev)
    qs = torch.empty(m, dtype=torch.int32, device=dev)
    bl.bitlinear_quant_act(xd, gd, eps, q, s, qs)
    return to_host(q), to_host(s), to_host(qs)


# ---- activation quant ------------------------------------------------------------------

# few rows: up to 16384 values register-resident in a 512-thread workgroup (4,
# 8, 16, 20 or 32 values per thread), longer rows the three-pass kernel; from
# 256 rows one wave per row (2 .. 32 float4 chunks per lane, ragged tails)
QUANT_CASES = [(1, 64), (1, 2560), (1, 10240), (3, 192), (7, 640), (33, 2560), (5, 16384), (4, 8192), (2, 4160),
               (2, 16448), (300, 2560), (256, 192), (256, 640), (256, 2048), (259, 4096), (257, 8192), (260, 4160),
               (258, 10240)]


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("m,k", QUANT_CASES)
def test_quant_act(bl, olib, m, k, norm):
    log(f"quant_act m={m} k={k} norm={norm}")
    g = W.rng(100, m, k)
    x = W.activations(g, m, k, outliers=True) * np.float32(g.uniform(0.01, 50))
    gain = W.gains(g, k) if norm else None
    q, s, qs = quant_gpu(bl, x, gain, 1e-5)
    oq, os_, oqs = oracle.quant_act(x, gain, 1e-5, olib)
    assert_exact(q, oq, "q")
    assert_exact(s.view(np.uint32), os_.view(np.uint32), "act_scale bits")
    assert_exact(qs, oqs, "act_sum")


def midpoint_row(k, seed, eps=1e-5):
    """A row x of k fp32 values whose RMSNorm scale in fp64, 1 / sqrt(ss / k + eps)
    with ss the fixed-order sum of squares, lies within 2^-47 (relative) of the
    midpoint between two fp32 values, so that any error above about 2^-47 in
    the divide, square root or reciprocal flips the fp32 scale. The last
    element is scanned over 2^23 fp32 values whose squares step ss by about
    2^-46 (relative); the sum follows the same 512-partial butterfly tree."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(k).astype(np.float32)
    x[0] = 1.0  # its normalised value (gain 1) is the scale itself
    f = k - 1
    sq = x.astype(np.float64) ** 2
    parts = np.zeros(512)
    for p_ in range(512):
        acc = 0.0
        for j in range(p_, k, 512):
            if j != f:
                acc += sq[j]
        parts[p_] = acc
    pf = f % 512
    ss_approx = float(np.sum(sq[:-1]))
    x0 = np.float32(np.sqrt(ss_approx) * 2.0 ** -12)
    cand = (np.float64(x0) * (1.0 + np.arange(1 << 23, dtype=np.float64) * 2.0 ** -23)).astype(np.float32)
    # leaf pf of the butterfly tree, then its sibling subtree at each level
    node = parts[pf] + cand.astype(np.float64) ** 2
    lo_idx = pf
    for lev in range(9):
        size = 1 << lev
        sib_start = (lo_idx ^ size) & ~(size - 1)
        sib = parts[sib_start:sib_start + size]
        # the sibling subtree's own sum in the same butterfly order
        t = sib.copy()
        while t.size > 1:
            t = t[0::2] + t[1::2]
        node = node + t[0]
        lo_idx &= ~size
    r64 = 1.0 / np.sqrt(node / k + eps)
    r32 = r64.astype(np.float32)
    b = r32.view(np.uint32)
    lo = 0.5 * (r32.astype(np.float64) + (b - 1).view(np.float32).astype(np.float64))
    hi = 0.5 * (r32.astype(np.float64) + (b + 1).view(np.float32).astype(np.float64))
    dist = np.minimum(r64 - lo, hi - r64) / r64
    j = int(np.argmin(dist))
    assert dist[j] < 2.0 ** -47, dist[j]
    x[f] = cand[j]
    return x


@pytest.mark.parametrize("m,k", [(1, 64), (1, 2560), (3, 10240), (256, 2048), (1, 20480)])
def test_quant_act_rms_scale_near_fp32_midpoint(bl, olib, m, k):
    """Rows whose RMSNorm scale sits next to an fp32 rounding boundary (for
    k = 64, exactly on it: a tie to even): only correctly rounded fp64 divide
    and square root give the oracle's fp32 scale. Every kernel of the quant
    dispatch gets one (one workgroup per row, one wave per row at 256 rows,
    three passes above 16384)."""
    log(f"quant_act midpoint rows m={m} k={k}")
    g = W.rng(100, 7000 + m, k)
    x = W.activations(g, m, k)
    x[m // 2] = midpoint_row(k, 11 + k)
    gain = np.ones(k, np.float32)
    q, s, qs = quant_gpu(bl, x, gain, 1e-5)
    oq, os_, oqs = oracle.quant_act(x, gain, 1e-5, olib)
    assert_exact(q, oq, "q")
    assert_exact(s.view(np.uint32), os_.view(np.uint32), "act_scale bits")
    assert_exact(qs, oqs, "act_sum")


def test_quant_act_special_rows(bl, olib):
    """Ties at +-0.5 of a code, an all-zero row, a constant row, one huge outlier,
    tiny values near the absmax floor."""
    k = 256
    rows = []
    r = np.zeros(k, np.float32)
    r[0] = 127.0
    r[1:128] = np.arange(127, dtype=np.float32) + np.float32(0.5)   # every x.5 tie (s_a = 1)
    r[128:255] = -(np.arange(127, dtype=np.float32) + np.float32(0.5))
    rows.append(r)
    rows.append(np.zeros(k, np.float32))
    rows.append(np.full(k, -3.25, np.float32))
    r = np.full(k, 1e-3, np.float32)
    r[77] = 1e6
    rows.append(r)
    rows.append(np.full(k, 3e-6, np.float32))
    x = np.stack(rows)
    for gain in (None, np.ones(k, np.float32)):
        q, s, qs = quant_gpu(bl, x, gain, 1e-5)
        oq, os_, oqs = oracle.quant_act(x, gain, 1e-5, olib)
        assert_exact(q, oq, "q")
        assert_exact(s.view(np.uint32), os_.view(np.uint32), "act_scale bits")
        assert_exact(qs, oqs, "act_sum")
    assert q.min() > -128


# ---- GEMV ---------------------------------------------------------------------------------

GEMV_CASES = [(16, 64, 1), (40, 192, 1), (2560, 2560, 1), (10240, 2560, 1), (2560, 10240, 1), (7, 640, 1),
              (13, 32768, 1), (100, 2048, 2), (333, 8192, 3), (64, 640, 5), (129, 2560, 8)]


def _gemv_inputs(case_id, n, k, m, olib):
    g = W.rng(101, case_id, 0)
    t = W.ternary(g, n, k)
    sw = W.weight_scale(g)
    x = W.activations(g, m, k)
    res = W.activations(g, m, n)
    p = pack_both(t, olib)
    q, s, qs = oracle.quant_act(x, None, 1e-5, olib)
    return p, sw, q, s, qs, res


@pytest.mark.parametrize("n,k,m", GEMV_CASES)
def test_gemv(bl, olib, n, k, m):
    import torch
    log(f"gemv n={n} k={k} m={m}")
    p, sw, q, s, qs, res = _gemv_inputs(n * 7 + k + m, n, k, m, olib)
    dev = torch_dev()
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    bl.bitlinear_gemv(to_dev(p), sw, n, k, to_dev(q), to_dev(s), to_dev(qs), m, None, y, acc)
    oy, oacc = oracle.bitlinear(p, sw, k, q, s, olib)
    assert_exact(to_host(acc), oacc, "acc")
    assert_f32(to_host(y), oy, "y")
    # residual, in place (y aliases the residual)
    yr = to_dev(res)
    bl.bitlinear_gemv(to_dev(p), sw, n, k, to_dev(q), to_dev(s), to_dev(qs), m, yr, yr, None)
    assert_f32(to_host(yr), oracle.residual_add(res, oy, olib), "y + residual")


# ---- GEMM ------------------------------------------------------------------------------------

# m <= 32 runs the skinny kernels (one or two 32-row tiles per wave, K split
# over up to 16 waves, ragged K tails); larger m the tiled GEMM: 32 x 256 tiles
# up to 64 tokens, above that 128 x 320 tiles, or, while the 128 x 320 tiling
# would give fewer than 512 tiles, 64 x 160 tiles with 128-deep K steps (K a
# multiple of 128: (130, 200, 640), (257, 2560, 1024)) or 128 x 160 tiles with
# 64-deep ones ((200, 700, 320)); (2100, 10000): 544 tiles of 128 x 320, ragged
# in both directions.
GEMM_CASES = [(1, 16, 64), (5, 100, 192), (32, 2048, 2048), (130, 200, 640), (256, 384, 2560), (37, 2560, 10240),
              (300, 129, 128), (32, 8192, 2048), (64, 50000, 2048), (32, 50000, 2048), (17, 16448, 320),
              (9, 33, 4160), (24, 700, 8448), (2100, 10000, 64), (257, 2560, 1024), (200, 700, 320)]


@pytest.mark.parametrize("m,n,k", GEMM_CASES)
def test_gemm(bl, olib, m, n, k):
    import torch
    log(f"gemm m={m} n={n} k={k}")
    g = W.rng(102, m + n, k)
    t = W.ternary(g, n, k)
    sw = W.weight_scale(g)
    x = W.activations(g, m, k, outliers=True)
    p = pack_both(t, olib)
    q, s, qs = oracle.quant_act(x, None, 1e-5, olib)
    dev = torch_dev()
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    am = torch.empty(m, dtype=torch.int32, device=dev)
    ws = torch.empty(max(bl.bitlinear_gemm_workspace_bytes(m, n, k, 1), 8), dtype=torch.uint8, device=dev)
    bl.bitlinear_gemm(to_dev(p), sw, n, k, to_dev(q), to_dev(s), to_dev(qs), m, None, y, acc, am, ws)
    oy, oacc = oracle.bitlinear(p, sw, k, q, s, olib)
    assert_exact(to_host(acc), oacc, "acc")
    assert_f32(to_host(y), oy, "y")
    assert_exact(to_host(am), oracle.argmax_rows(oacc, olib), "row argmax")
    assert_exact(to_host(am), np.argmax(oy, axis=1).astype(np.int32), "argmax of logits")


def test_gemm_prefill_full_size_sampled_rows(bl, olib):
    """The prefill product at the benchmark's size and launch configuration
    (2048 tokens x K = 2560 -> N = 10240, 128 x 320 block tiles, activations with
    1 % outliers x20). The quant of all rows is checked against the oracle. Then
    the call the benchmark times -- y only, no residual, accumulators or argmax,
    so every tile takes the branch-free epilogue -- is checked on sampled rows
    (at least one in every 128-row block tile, plus tile and half edges), every
    column; a second call that also writes the accumulators checks them exactly."""
    import torch
    m, k, n = 2048, 2560, 10240
    log(f"gemm full size m={m} n={n} k={k}")
    g = W.rng(103, m, n)
    t = W.ternary(g, n, k)
    sw = W.weight_scale(g)
    x = W.activations(g, m, k, outliers=True)
    p = pack_both(t, olib)
    dev = torch_dev()
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    s = torch.empty(m, dtype=torch.float32, device=dev)
    qs = torch.empty(m, dtype=torch.int32, device=dev)
    bl.bitlinear_quant_act(to_dev(x), None, 1e-5, q, s, qs)
    oq, os_, oqs = oracle.quant_act(x, None, 1e-5, olib)
    assert_exact(to_host(q), oq, "q")
    assert_exact(to_host(s).view(np.uint32), os_.view(np.uint32), "act_scale bits")
    assert_exact(to_host(qs), oqs, "act_sum")
    pick = W.rng(103, 1, 1)
    rows = set([0, 1, 63, 64, 127, 128, 129, 1023, 1024, 1151, 2046, 2047])
    rows |= {int(tile * 128 + pick.integers(0, 128)) for tile in range(m // 128)}
    rows = sorted(rows)
    oy, oacc = oracle.bitlinear(p, sw, k, oq[rows], os_[rows], olib)
    pd = to_dev(p)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    bl.bitlinear_gemm(pd, sw, n, k, q, s, qs, m, None, y)
    assert_f32(to_host(y)[rows], oy, "y, y-only call (sampled rows)")
    y2 = torch.empty((m, n), dtype=torch.float32, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev)
    bl.bitlinear_gemm(pd, sw, n, k, q, s, qs, m, None, y2, acc, None, None)
    acca = to_host(acc)
    assert_exact(acca[rows], oacc, "acc (sampled rows)")
    assert_f32(to_host(y2)[rows], oy, "y with acc (sampled rows)")
    assert_exact(to_host(y2).view(np.uint32), to_host(y).view(np.uint32), "y-only call == general call, all rows")


# (m, n, k): tiles that all take the branch-free y-only epilogue, and ragged
# shapes where interior tiles take it and edge tiles the general one, for both
# block-tile configurations (m <= 64 and m > 64).
GEMM_Y_ONLY_CASES = [(256, 640, 256), (300, 1000, 320), (129, 330, 2560), (64, 512, 128), (65, 700, 192),
                     (40, 257, 64), (2048, 640, 64), (2100, 10000, 64), (2048, 2560, 640), (257, 2560, 1024),
                     (1000, 2500, 1152)]


@pytest.mark.parametrize("m,n,k", GEMM_Y_ONLY_CASES)
def test_gemm_y_only(bl, olib, m, n, k):
    import torch
    log(f"gemm y-only m={m} n={n} k={k}")
    g = W.rng(106, m + n, k)
    t = W.ternary(g, n, k)
    sw = W.weight_scale(g)
    x = W.activations(g, m, k, outliers=True)
    p = pack_both(t, olib)
    q, s, qs = oracle.quant_act(x, None, 1e-5, olib)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=torch_dev())
    bl.bitlinear_gemm(to_dev(p), sw, n, k, to_dev(q), to_dev(s), to_dev(qs), m, None, y)
    oy, _ = oracle.bitlinear(p, sw, k, q, s, olib)
    assert_f32(to_host(y), oy, "y")


@pytest.mark.parametrize("m", [7, 40])
def test_gemm_argmax_ties_no_logits(bl, olib, m):
    """Duplicated weight rows make ties; the lowest index must win, without y."""
    import torch
    n, k = 300, 128
    g = W.rng(103, 0, 0)
    t = W.ternary(g, n, k)
    t[250] = t[3]
    t[299] = t[3]
    t[17] = t[200]
    x = W.activations(g, m, k)
    x[2] = t[3].astype(np.float32) * np.float32(2.0)   # row 2 maximal at 3, 250, 299
    p = pack_both(t, olib)
    q, s, qs = oracle.quant_act(x, None, 1e-5, olib)
    dev = torch_dev()
    am = torch.empty(m, dtype=torch.int32, device=dev)
    ws = torch.empty(bl.bitlinear_gemm_workspace_bytes(m, n, k, 1), dtype=torch.uint8, device=dev)
    bl.bitlinear_gemm(to_dev(p), 30.0, n, k, to_dev(q), to_dev(s), to_dev(qs), m, None, None, None, am, ws)
    oacc = oracle.matmul_i32(oracle.unpack(p, k, olib), q, olib)
    got = to_host(am)
    assert_exact(got, oracle.argmax_rows(oacc, olib), "row argmax")
    assert got[2] == 3


@pytest.mark.parametrize("m", [40, 20])
def test_gemm_residual_and_stride(bl, olib, m):
    import torch
    n, k = 96, 256
    g = W.rng(104, 0, m)
    t = W.ternary(g, n, k)
    x = W.activations(g, m, k)
    res = W.activations(g, m, n)
    p = pack_both(t, olib)
    q, s, qs = oracle.quant_act(x, None, 1e-5, olib)
    y = to_dev(res)
    bl.bitlinear_gemm(to_dev(p), 25.0, n, k, to_dev(q), to_dev(s), to_dev(qs), m, y, y)
    oy, _ = oracle.bitlinear(p, np.float32(25.0), k, q, s, olib)
    assert_f32(to_host(y), oracle.residual_add(res, oy, olib), "y + residual")


# ---- FFN -----------------------------------------------------------------------------------------

def _ffn_case(bl, olib, m, d, f, seed, with_residual, write_acc=True):
    """One bitnet_ffn call against oracle.ffn, every intermediate of the
    workspace; without write_acc the accumulators are not written (above 64
    tokens the gate/up GEMM's interior tiles then store h with no per-element
    checks) and everything else is compared."""
    import torch
    log(f"ffn m={m} d={d} f={f} write_acc={write_acc}")
    g = W.rng(105, seed, 0)
    tg, tu, td = W.ternary(g, f, d), W.ternary(g, f, d), W.ternary(g, d, f)
    sg, su, sd = W.weight_scale(g), W.weight_scale(g), W.weight_scale(g)
    x = W.activations(g, m, d)
    gn, gs = W.gains(g, d), W.gains(g, f)
    pg, pu, pd = pack_both(tg, olib), pack_both(tu, olib), pack_both(td, olib)
    res = W.activations(g, m, d) if with_residual else None
    dev = torch_dev()
    out = torch.empty((m, d), dtype=torch.float32, device=dev)
    # the workspace's content on entry is unspecified: start from garbage
    ws = torch.full((bl.bitnet_ffn_workspace_bytes(m, d, f),), 0x5A, dtype=torch.uint8, device=dev)
    bl.bitnet_ffn(to_dev(x), m, d, f, to_dev(gn), to_dev(gs), 1e-5, to_dev(pg), sg, to_dev(pu), su, to_dev(pd), sd,
                  to_dev(res) if res is not None else None, out, ws,
                  flags=bl.BITNET_FFN_WRITE_ACC if write_acc else 0)
    r = oracle.ffn(x, gn, gs, 1e-5, pg, sg, pu, su, pd, sd, olib)
    view = lambda seg: to_host(bl.ffn_workspace_view(ws, m, d, f, seg))
    assert_exact(view("q1"), r["q1"], "q1")
    assert_exact(view("s1").view(np.uint32), r["s1"].view(np.uint32), "s1 bits")
    assert_exact(view("qs1"), r["qs1"], "qs1")
    if write_acc:
        assert_exact(view("acc_gate"), r["acc_gate"], "acc_gate")
        assert_exact(view("acc_up"), r["acc_up"], "acc_up")
    assert_f32(view("h"), r["h"], "h")
    assert_exact(view("q2"), r["q2"], "q2")
    assert_exact(view("s2").view(np.uint32), r["s2"].view(np.uint32), "s2 bits")
    assert_exact(view("qs2"), r["qs2"], "qs2")
    if write_acc:
        assert_exact(view("acc_down"), r["acc_down"], "acc_down")
    want = r["out"] if res is None else oracle.residual_add(res, r["out"], olib)
    assert_f32(to_host(out), want, "out")


@pytest.mark.parametrize("m,d,f,res", [(1, 64, 128, False), (1, 192, 640, True), (3, 256, 1024, False),
                                        (1, 2560, 10240, False), (8, 640, 2560, True), (12, 320, 640, False),
                                        (40, 256, 512, True), (1, 256, 1024, True), (1, 2048, 8192, True),
                                        (1, 2560, 10240, True),
                                        # above 32 tokens: the paired gate/up MFMA GEMM, with ragged
                                        # row tiles (32 / 128 rows) and column tiles (128 / 160 columns)
                                        (33, 256, 1024, False), (64, 128, 1088, True), (65, 256, 1024, True),
                                        (130, 320, 1088, False), (300, 256, 640, True), (257, 192, 2624, False)])
def test_ffn(bl, olib, m, d, f, res):
    _ffn_case(bl, olib, m, d, f, m * 1000 + d + f, res)


@pytest.mark.parametrize("m,d,f,res", [(40, 256, 512, True), (64, 256, 1024, False), (65, 256, 1024, True),
                                        (130, 320, 1088, False), (300, 256, 640, True), (257, 192, 2624, False),
                                        (512, 512, 2048, False)])
def test_ffn_without_accumulators(bl, olib, m, d, f, res):
    """Above 64 tokens without BITNET_FFN_WRITE_ACC: interior gate/up tiles take
    the epilogue without per-element checks, edge tiles the general one."""
    _ffn_case(bl, olib, m, d, f, m * 1000 + d + f + 7, res, write_acc=False)


@pytest.mark.parametrize("write_acc", [True, False])
def test_ffn_prefill_full_size_sampled_rows(bl, olib, write_acc):
    """The FFN at 2048 tokens with BitNet-3B shapes (d = 2560, f = 10240): the
    paired gate/up GEMM with relu(gate)^2 * up in its epilogue, the sub-norm +
    quant of h and the down GEMM. Every intermediate of sampled rows (at least
    one in every 128-row block tile, plus tile edges) against the oracle's FFN
    of those rows: q1, s1, sum(q1), the exact gate and up accumulators, h, q2,
    s2, sum(q2), the exact down accumulators and out (rows are independent).
    Without the accumulators (the benchmark's call) everything else again."""
    import torch
    m, d, f = 2048, 2560, 10240
    log(f"ffn full size m={m} d={d} f={f} write_acc={write_acc}")
    g = W.rng(107, 0, 0)
    tg, tu, td = W.ternary(g, f, d), W.ternary(g, f, d), W.ternary(g, d, f)
    sg, su, sd = W.weight_scale(g), W.weight_scale(g), W.weight_scale(g)
    x = W.activations(g, m, d, outliers=True)
    gn, gs = W.gains(g, d), W.gains(g, f)
    pg, pu, pd = pack_both(tg, olib), pack_both(tu, olib), pack_both(td, olib)
    dev = torch_dev()
    out = torch.empty((m, d), dtype=torch.float32, device=dev)
    ws = torch.full((bl.bitnet_ffn_workspace_bytes(m, d, f),), 0x5A, dtype=torch.uint8, device=dev)
    bl.bitnet_ffn(to_dev(x), m, d, f, to_dev(gn), to_dev(gs), 1e-5, to_dev(pg), sg, to_dev(pu), su, to_dev(pd), sd,
                  None, out, ws, flags=bl.BITNET_FFN_WRITE_ACC if write_acc else 0)
    pick = W.rng(107, 1, 1)
    rows = sorted({0, 127, 128, 1023, 2047} | {int(t * 128 + pick.integers(0, 128)) for t in range(m // 128)})
    r = oracle.ffn(x[rows], gn, gs, 1e-5, pg, sg, pu, su, pd, sd, olib)
    view = lambda seg: to_host(bl.ffn_workspace_view(ws, m, d, f, seg))[rows]
    assert_exact(view("q1"), r["q1"], "q1")
    assert_exact(view("s1").view(np.uint32), r["s1"].view(np.uint32), "s1 bits")
    assert_exact(view("qs1"), r["qs1"], "qs1")
    if write_acc:
        assert_exact(view("acc_gate"), r["acc_gate"], "acc_gate")
        assert_exact(view("acc_up"), r["acc_up"], "acc_up")
    assert_f32(view("h"), r["h"], "h")
    assert_exact(view("q2"), r["q2"], "q2")
    assert_exact(view("s2").view(np.uint32), r["s2"].view(np.uint32), "s2 bits")
    assert_exact(view("qs2"), r["qs2"], "qs2")
    if write_acc:
        assert_exact(view("acc_down"), r["acc_down"], "acc_down")
    assert_f32(to_host(out)[rows], r["out"], "out")


# ---- layer stream ------------------------------------------------------------------------------------

@pytest.mark.parametrize("n_layers,m,d,f", [(2, 1, 128, 512), (3, 2, 256, 640), (3, 1, 256, 1024),
                                            (2, 1, 2560, 10240), (2, 1, 2048, 8192), (2, 12, 192, 384),
                                            (2, 9, 320, 1088), (2, 25, 512, 1536), (2, 32, 2048, 8192),
                                            (3, 32, 256, 1024), (3, 9, 256, 1024), (2, 16, 2560, 10240),
                                            (2, 33, 256, 512), (1, 16, 256, 8448)])
def test_decode_stream(bl, olib, n_layers, m, d, f):
    """The layer stream against oracle.chain. At 9..32 tokens the down
    product of every layer but the last splits K over 2 or 4 workgroups where
    d and f allow it (f = 1536, 8192, 1024: 4 parts; 2560 x 10240: 2; f = 384
    and 1088: none), and the next layer's norm + quant finishes it."""
    from gpu_helpers import make_layers, run_stream, stream_ctrl
    log(f"stream layers={n_layers} m={m} d={d} f={f}")
    layers, dev = make_layers(W.W_STREAM, n_layers, d, f, m, olib)
    x0 = W.activations(W.rng(W.W_STREAM, 999, W.T_X), m, d)
    x, qkv, ws = run_stream(dev, n_layers, m, d, f, 1e-5, x0)
    assert stream_ctrl(ws)[1] == 0, "stream status word"
    ox, oqkv = oracle.chain(x0, layers, 1e-5, olib)
    for l in range(n_layers):
        assert_f32(qkv[l], oqkv[l], f"qkv layer {l}")
    assert_f32(x, ox, "x after the stream")


def test_decode_stream_absmax_not_at_largest_product(bl, olib):
    """Layer 0's input and attention gains from tests/crafted.py: the element
    with the largest exact |x g| is not the one with the largest rounded |y|.
    The persistent kernel first takes the absmax from the largest product and
    must notice the larger |y| and quantize again; q/k/v and x must match the
    oracle bit for bit."""
    from crafted import absmax_flip
    from gpu_helpers import make_layers, run_stream, stream_ctrl
    n_layers, d, f = 2, 256, 1024
    log("stream with the absmax away from the largest product")
    layers, dev = make_layers(W.W_STREAM, n_layers, d, f, 1, olib)
    x, g = absmax_flip(d)
    layers[0]["g_attn"] = g
    dev["gains"][0, :d] = to_dev(g)
    x0 = x[None, :]
    gx, gqkv, ws = run_stream(dev, n_layers, 1, d, f, 1e-5, x0)
    assert stream_ctrl(ws)[1] == 0, "stream status word"
    ox, oqkv = oracle.chain(x0, layers, 1e-5, olib)
    for l in range(n_layers):
        assert_f32(gqkv[l], oqkv[l], f"qkv layer {l}")
    assert_f32(gx, ox, "x after the stream")


@pytest.mark.parametrize("d,f", [(256, 1024), (2560, 10240)])
def test_decode_stream_all_zero_vectors(bl, olib, d, f):
    """x = 0 and z = 0: every vector the persistent kernel hands over (x, x
    after o, h) is +-0 in every word, which is the encoding's "not written"
    value once negated. Three layers, two calls (both copies of each vector
    carry zeros); the results must still come out, all zero, like the oracle's."""
    from gpu_helpers import make_layers, run_stream, stream_ctrl
    n_layers = 3
    log(f"stream zeros d={d} f={f}")
    layers, dev = make_layers(W.W_STREAM, n_layers, d, f, 1, olib)
    dev["z"].zero_()
    for lw in layers:
        lw["z"] = np.zeros_like(lw["z"])
    x = np.zeros((1, d), np.float32)
    ws = None
    for call in range(2):
        gx, gqkv, ws = run_stream(dev, n_layers, 1, d, f, 1e-5, x, ws)
        assert stream_ctrl(ws)[1] == 0, "stream status word"
        ox, oqkv = oracle.chain(x, layers, 1e-5, olib)
        for l in range(n_layers):
            assert_f32(gqkv[l], oqkv[l], f"qkv layer {l} call {call}")
        assert_f32(gx, ox, f"x after call {call}")
        assert not np.any(gx), "all-zero stream stays zero"
        x = gx


@pytest.mark.parametrize("d,f", [(256, 1024), (2560, 10240)])
def test_decode_stream_repeated_calls(bl, olib, d, f):
    """Three tokens through one workspace: each call continues the phase counter
    and reads the previous call's output; every result matches the oracle."""
    from gpu_helpers import make_layers, run_stream, stream_ctrl
    n_layers = 3
    log(f"stream repeated d={d} f={f}")
    layers, dev = make_layers(W.W_STREAM, n_layers, d, f, 1, olib)
    x = W.activations(W.rng(W.W_STREAM, 998, W.T_X), 1, d)
    ws = None
    for call in range(3):
        gx, _, ws = run_stream(dev, n_layers, 1, d, f, 1e-5, x, ws)
        epoch, status = stream_ctrl(ws)
        assert status == 0
        x, _ = oracle.chain(x, layers, 1e-5, olib)
        assert_f32(gx, x, f"x after call {call}")
        x = gx
    assert epoch == 3 * 4 * n_layers, "one-token calls of these shapes run the persistent kernel"


def test_decode_stream_long_run_repeatable(bl, olib):
    """400 consecutive tokens through one workspace on the full grid of the
    persistent kernel (2 layers of the 3B shape), run twice from the same input:
    the two runs' sequences of hidden states agree bit for bit (no hand-over
    leaves a trace of timing in the results), the status word stays clear, and
    sampled calls match the oracle on their own input."""
    import torch
    from gpu_helpers import make_layers, new_stream_workspace, stream_ctrl
    n_layers, d, f, calls, checked = 2, 2560, 10240, 400, (0, 199, 399)
    log(f"stream long run layers={n_layers} d={d} f={f} calls={calls}")
    layers, dev = make_layers(W.W_STREAM, n_layers, d, f, 1, olib)
    x0 = W.activations(W.rng(W.W_STREAM, 996, W.T_X), 1, d)
    qkv = torch.empty((n_layers, 1, 3 * d), dtype=torch.float32, device=torch_dev())
    runs = []
    for run in range(2):
        ws = new_stream_workspace(1, d, f)
        x = to_dev(x0)
        seq = torch.empty((calls, d), dtype=torch.float32, device=torch_dev())
        inputs = {}
        for c in range(calls):
            if c in checked:
                inputs[c] = to_host(x)
            bl.bitnet_decode_stream(dev["weights"], dev["scales"], dev["gains"], dev["z"], n_layers, 1, d, f, 1e-5,
                                    x, qkv, ws)
            seq[c] = x[0]
        epoch, status = stream_ctrl(ws)
        assert status == 0, f"stream status word, run {run}"
        assert epoch == calls * 4 * n_layers
        out = to_host(seq)
        for c in checked:
            want, _ = oracle.chain(inputs[c], layers, 1e-5, olib)
            assert_f32(out[c:c + 1], want, f"run {run} call {c}")
        runs.append(out)
    assert_exact(runs[0].view(np.uint32), runs[1].view(np.uint32), "hidden states of the two runs")
