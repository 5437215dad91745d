"""bitlinear_forward (a BitLinear applied to a few tokens in one call) against the
CPU oracle -- quant_act, then the ternary product and dequant -- and, bit for bit,
against the two calls it composes, through the C ABI.

One token with k <= 4096 takes the one-launch kernel (every workgroup quantizes
the row itself: 2 .. 16 float4 chunks per lane, ragged row counts against the 8
rows of a workgroup); longer rows and several tokens take the quant launch with
the L2 prefetch and the GEMV."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_exact, assert_f32, log, pack_both, to_dev, to_host, torch_dev

pytestmark = pytest.mark.gpu

FWD_CASES = [(1, 8, 64), (1, 2560, 2560), (1, 1000, 2048), (1, 7, 4096), (1, 513, 320), (1, 10240, 2560),
             (1, 3, 192), (1, 2560, 8192), (1, 2560, 10240), (3, 2560, 2560), (8, 100, 4096)]


@pytest.fixture(scope="module")
def bl():
    import bitlinear_amd
    return bitlinear_amd


def run_forward(bl, x, gain, p, sw, n):
    import torch
    m, k = x.shape
    dev = torch_dev()
    q = torch.full((m, k), 0x5A, dtype=torch.int8, device=dev)
    s = torch.full((m,), -1.0, dtype=torch.float32, device=dev)
    qs = torch.full((m,), -7, dtype=torch.int32, device=dev)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    bl.bitlinear_forward(to_dev(x), to_dev(gain) if gain is not None else None, 1e-5, to_dev(p), sw, n, q, s, qs, y)
    return to_host(q), to_host(s), to_host(qs), to_host(y)


def check_against_oracle(olib, x, gain, p, sw, k, got):
    q, s, qs, y = got
    oq, os_, oqs = oracle.quant_act(x, gain, 1e-5, olib)
    assert_exact(q, oq, "q")
    assert_exact(s.view(np.uint32), os_.view(np.uint32), "act_scale bits")
    assert_exact(qs, oqs, "act_sum")
    oy, _ = oracle.bitlinear(p, sw, k, oq, os_, olib)
    assert_f32(y, oy, "y")


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("m,n,k", FWD_CASES)
def test_forward(bl, olib, m, n, k, norm):
    import torch
    log(f"forward m={m} n={n} k={k} norm={norm}")
    g = W.rng(106, m * 31 + n, k)
    t = W.ternary(g, n, k)
    sw = W.weight_scale(g)
    x = W.activations(g, m, k, outliers=True)
    gain = W.gains(g, k) if norm else None
    p = pack_both(t, olib)
    got = run_forward(bl, x, gain, p, sw, n)
    check_against_oracle(olib, x, gain, p, sw, k, got)
    # the two calls it composes give the same bits
    dev = torch_dev()
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    s = torch.empty(m, dtype=torch.float32, device=dev)
    qs = torch.empty(m, dtype=torch.int32, device=dev)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    bl.bitlinear_quant_act(to_dev(x), to_dev(gain) if gain is not None else None, 1e-5, q, s, qs)
    bl.bitlinear_gemv(to_dev(p), sw, n, k, q, s, qs, m, None, y)
    assert_exact(got[3].view(np.uint32), to_host(y).view(np.uint32), "y vs quant_act + gemv")


def test_forward_special_rows(bl, olib):
    """One-launch path on rows the quant treats specially: all zeros (absmax floor),
    a constant row, one huge outlier, values at the +-0.5 rounding ties, and a row
    whose RMSNorm scale lies next to an fp32 rounding midpoint."""
    from test_gpu_parity import midpoint_row
    k, n = 2560, 136
    g = W.rng(107, 0, 0)
    t = W.ternary(g, n, k)
    sw = W.weight_scale(g)
    p = pack_both(t, olib)
    rows = [np.zeros(k, np.float32), np.full(k, 0.37, np.float32)]
    spike = W.activations(g, 1, k)[0]
    spike[1234] = np.float32(1e4)
    rows.append(spike)
    ties = np.full(k, 1.0, np.float32)
    ties[::3] = np.float32(127.0 / 254.0)  # y * s_a lands on +-0.5 multiples
    ties[1::7] = np.float32(-63.5 / 127.0)
    rows.append(ties)
    rows.append(midpoint_row(k, 11 + k))
    for i, row in enumerate(rows):
        for gain in (None, np.ones(k, np.float32)):
            log(f"forward special row {i} norm={gain is not None}")
            x = row.reshape(1, k)
            check_against_oracle(olib, x, gain, p, sw, k, run_forward(bl, x, gain, p, sw, n))
