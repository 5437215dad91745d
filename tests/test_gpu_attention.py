"""GPU parity of the decode step with attention (bitnet_decode_step) against the
oracle, through the C ABI.

The device computes attention in fp32 (scores, expf, sums), the oracle in fp64
from the definition, so the attention outputs are compared within a bound
derived from fp32 rounding (below). Everything else is integer or follows the
same fp32 operation order: the oracle continues each layer from the device's
attention output (oracle.layer_attn(..., attn_in=...)), so q/k/v, the rotated
caches and the hidden state after every step must match bit for bit.

Bound on one attention output element of a head with scores s_j over
positions 0 .. pos (u = 2^-24): each fp32 score is within
e_s = (hd + 4) u max_j sum_i |q_i k_ji| / sqrt(hd) of the exact one; each
weight e^(s_j - max) is then within a relative 2 e_s + 4 u (expf adds a few
ulps); the chunked sums add (pos + 1 + 4 * chunks) u relative to
sum_j e_j |v_j|, chunks being the number of chunks merged (256 positions
each, or up to min(256 / heads, 32) shorter ones in the persistent kernel;
the bound takes the larger count). With V = max |v| over the head's
positions the output is off
by at most V (2 (2 e_s + 4 u) + (pos + 5 + 4 chunks) u); the test allows
twice that."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_exact, log, make_layers, stream_ctrl, to_dev, to_host, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import bitlinear_amd
    return bitlinear_amd


def _attn_bound(q_rot, kc, vc, pos, hd):
    """Per-element bound [m][H][hd] from the oracle's q_rot [m][H][hd] and caches."""
    u = 2.0 ** -24
    m, heads = q_rot.shape[:2]
    # chunks merged: 256-position chunks, or (the persistent kernel, when a head
    # has fewer of those than workgroups) up to min(256 / heads, 32) shorter ones
    n256 = (pos + 1 + 255) // 256
    chunks = max(n256, min(256 // heads, 32))
    bound = np.empty((m, heads, hd))
    for r in range(m):
        for h in range(heads):
            k = kc[r, h, :pos + 1].astype(np.float64)
            v = vc[r, h, :pos + 1].astype(np.float64)
            sabs = (np.abs(k) @ np.abs(q_rot[r, h].astype(np.float64))).max() / np.sqrt(hd)
            e_s = (hd + 4) * u * sabs
            vmax = np.abs(v).max()
            bound[r, h, :] = 2 * vmax * (2 * (2 * e_s + 4 * u) + (pos + 5 + 4 * chunks) * u) + 1e-30
    return bound


def _run_steps(bl, olib, n_layers, m, d, f, heads, max_seq, positions, seed, prefill=0):
    """Decode steps at the given positions (caches optionally prefilled with
    random entries below prefill), checking every step."""
    import torch
    dev = torch_dev()
    hd = d // heads
    layers, dw = make_layers(W.W_STREAM, n_layers, d, f, m, olib)
    g = W.rng(150, seed, 0)
    x0 = W.activations(g, m, d)
    c, s = bl.bitnet_rope_table(10000.0, hd, max_seq)
    kc_h = np.zeros((n_layers, m, heads, max_seq, hd), np.float32)
    vc_h = np.zeros_like(kc_h)
    if prefill:
        kc_h[:, :, :, :prefill] = g.standard_normal((n_layers, m, heads, prefill, hd)).astype(np.float32)
        vc_h[:, :, :, :prefill] = g.standard_normal((n_layers, m, heads, prefill, hd)).astype(np.float32)
    kc, vc = to_dev(kc_h), to_dev(vc_h)
    o_kc, o_vc = kc_h.copy(), vc_h.copy()
    x = to_dev(x0)
    xo = x0.copy()
    qkv = torch.empty((n_layers, m, 3 * d), dtype=torch.float32, device=dev)
    attn = torch.empty((n_layers, m, d), dtype=torch.float32, device=dev)
    ws = torch.zeros(bl.bitnet_decode_step_workspace_bytes(m, d, f, heads, max_seq), dtype=torch.uint8, device=dev)
    cd, sd = to_dev(c), to_dev(s)
    worst = 0.0
    for pos in positions:
        log(f"decode step m={m} d={d} heads={heads} pos={pos}")
        bl.bitnet_decode_step(dw["weights"], dw["scales"], dw["gains"], n_layers, m, d, f, heads, 1e-5, cd, sd, pos,
                              kc, vc, x, qkv, attn, ws)
        g_qkv, g_attn = to_host(qkv), to_host(attn)
        for l, lw in enumerate(layers):
            xn, o_qkv, o_attn = oracle.layer_attn(xo, lw, 1e-5, heads, c, s, o_kc[l], o_vc[l], pos,
                                                  attn_in=g_attn[l], lib=olib)
            assert_exact(g_qkv[l].view(np.uint32), o_qkv.view(np.uint32), f"qkv bits, layer {l}, pos {pos}")
            q_rot = oracle.rope_apply(o_qkv[:, :d].reshape(m, heads, hd), c[pos], s[pos], olib)
            bound = _attn_bound(q_rot, o_kc[l], o_vc[l], pos, hd).reshape(m, d)
            err = np.abs(g_attn[l].astype(np.float64) - o_attn.astype(np.float64))
            assert np.all(err <= bound), f"attention beyond bound at layer {l}, pos {pos}: {(err / bound).max()}"
            worst = max(worst, float((err / bound).max()))
            xo = xn
        assert_exact(to_host(kc).view(np.uint32), o_kc.view(np.uint32), f"k cache bits, pos {pos}")
        assert_exact(to_host(vc).view(np.uint32), o_vc.view(np.uint32), f"v cache bits, pos {pos}")
        assert_exact(to_host(x).view(np.uint32), xo.view(np.uint32), f"hidden state bits, pos {pos}")
    assert stream_ctrl(ws)[1] == 0, "stream status word"
    log(f"  largest attention error / bound: {worst:.3g}")


@pytest.mark.parametrize("m", [1, 3, 12, 40])
def test_decode_steps_from_position_0(bl, olib, m):
    """Six consecutive steps from an empty cache; 1, 3, 12 and 40 sequences take
    the GEMV, skinny and GEMM paths of the layer stream."""
    _run_steps(bl, olib, 2, m, 256, 1024, 4, 64, list(range(6)), seed=m)


def test_decode_step_long_context(bl, olib):
    """Positions 700 .. 702 over a prefilled cache: three 256-position chunks
    are combined."""
    _run_steps(bl, olib, 2, 2, 256, 512, 2, 1024, [700, 701, 702], seed=9, prefill=700)


def test_decode_step_bitnet_3b_shapes(bl, olib):
    """BitNet-3B shapes (d = 2560, 32 heads of 80, f = 10240), two layers, one
    sequence at position 300 over a prefilled cache, then position 301 (one
    sequence: the persistent kernel, two 256-position chunks)."""
    _run_steps(bl, olib, 2, 1, 2560, 10240, 32, 512, [300, 301], seed=10, prefill=300)


def test_decode_step_persistent_long_context(bl, olib):
    """One sequence (the persistent kernel) at positions 700 .. 702 over a
    prefilled cache: three chunks merged inside one head's workgroup; then
    position 1023 (the cache's last slot, four chunks) and position 0 again
    (one position)."""
    _run_steps(bl, olib, 2, 1, 256, 1024, 2, 1024, [700, 701, 702, 1023, 0], seed=11, prefill=700)


@pytest.mark.parametrize("d,f,heads", [(2560, 10240, 32), (256, 1024, 2)])
def test_decode_step_persistent_longest_cache(bl, olib, d, f, heads):
    """One sequence with the persistent kernel's largest cache, 8192 positions,
    at positions 8190 and 8191 over a prefilled cache: the full 32 chunks of 256,
    four per workgroup of a head at the 3B shape (32 heads of 80), one per
    workgroup for 32 of the 128 workgroups of a head of 128 values."""
    _run_steps(bl, olib, 2, 1, d, f, heads, 8192, [8190, 8191], seed=17, prefill=8190)


@pytest.mark.parametrize("m", [1, 3])
def test_decode_step_largest_head(bl, olib, m):
    """Heads of 256 values, the largest accepted (d = 512, 2 heads), at positions
    300 and 301 over a prefilled cache: one sequence in the persistent kernel
    (19 chunks of 16 positions), three through the launch-per-step kernels."""
    _run_steps(bl, olib, 2, m, 512, 1024, 2, 600, [300, 301], seed=18, prefill=300)


def test_decode_step_one_sequence_long_cache_launch_path(bl, olib):
    """One sequence with a cache of 8448 positions, beyond the persistent
    kernel's 8192: the launch-per-step path at m = 1, positions 8200 and 8447
    (33 chunks of 256) over a prefilled cache."""
    _run_steps(bl, olib, 1, 1, 256, 1024, 2, 8448, [8200, 8447], seed=14, prefill=8200)


def test_decode_step_persistent_heads_of_4(bl, olib):
    """One sequence with 64 heads of 4 values (the smallest head), positions 0 .. 2."""
    _run_steps(bl, olib, 2, 1, 256, 1024, 64, 64, [0, 1, 2], seed=12)


def test_decode_step_bitnet_1p3b_shapes(bl, olib):
    """BitNet-1.3B shapes (d = 2048, 16 heads of 128, f = 8192), two layers, one
    sequence at positions 255 and 256 (one chunk, then two)."""
    _run_steps(bl, olib, 2, 1, 2048, 8192, 16, 512, [255, 256], seed=13, prefill=255)


def test_decode_step_persistent_short_chunks(bl, olib):
    """One sequence with 32 heads of 8 values (8 workgroups per head): at
    position 15 the 16 positions form one chunk; at 16 a chunk of 16 cache
    rows and one holding only the new position; at 17 and 47 two and three
    chunks of 16, merged by the head's first workgroup."""
    _run_steps(bl, olib, 2, 1, 256, 1024, 32, 64, [15, 16, 17, 47], seed=15, prefill=15)


def test_decode_step_long_run_repeatable(bl, olib):
    """200 consecutive steps (positions 700 .. 899 over a prefilled cache of
    1024) of two layers of the 3B shape on one sequence, the persistent kernel,
    run twice from the same caches and input: the hidden states of every step
    and the caches at the end agree bit for bit between the two runs (the
    attention hand-overs leave no trace of timing in the results), and the
    status word stays clear. Each step's values against the oracle are the
    business of the tests above."""
    import torch
    n_layers, m, d, f, heads, max_seq, first, steps = 2, 1, 2560, 10240, 32, 1024, 700, 200
    hd = d // heads
    log(f"decode step long run d={d} heads={heads} positions {first}..{first + steps - 1}")
    _, dw = make_layers(W.W_STREAM, n_layers, d, f, m, olib)
    g = W.rng(150, 16, 0)
    x0 = W.activations(g, m, d)
    kc_h = np.zeros((n_layers, m, heads, max_seq, hd), np.float32)
    vc_h = np.zeros_like(kc_h)
    kc_h[:, :, :, :first] = g.standard_normal((n_layers, m, heads, first, hd)).astype(np.float32)
    vc_h[:, :, :, :first] = g.standard_normal((n_layers, m, heads, first, hd)).astype(np.float32)
    c, s = bl.bitnet_rope_table(10000.0, hd, max_seq)
    cd, sd = to_dev(c), to_dev(s)
    dev = torch_dev()
    runs = []
    for run in range(2):
        kc, vc, x = to_dev(kc_h), to_dev(vc_h), to_dev(x0)
        ws = torch.zeros(bl.bitnet_decode_step_workspace_bytes(m, d, f, heads, max_seq), dtype=torch.uint8,
                         device=dev)
        seq = torch.empty((steps, d), dtype=torch.float32, device=dev)
        for i in range(steps):
            bl.bitnet_decode_step(dw["weights"], dw["scales"], dw["gains"], n_layers, m, d, f, heads, 1e-5, cd, sd,
                                  first + i, kc, vc, x, None, None, ws)
            seq[i] = x[0]
        assert stream_ctrl(ws)[1] == 0, f"stream status word, run {run}"
        runs.append((to_host(seq), to_host(kc), to_host(vc)))
    for name, a, b in zip(("hidden states", "k cache", "v cache"), runs[0], runs[1]):
        assert_exact(a.view(np.uint32), b.view(np.uint32), f"{name} of the two runs")
    assert np.all(np.isfinite(runs[0][0]))


def _random_attention_cases(n):
    """Seeded (m, d, heads, max_seq, pos) with hd = d / heads from 4 to 128."""
    g = np.random.default_rng(31337)
    cases = []
    while len(cases) < n:
        heads = int(g.choice([2, 4, 8, 16, 32, 64]))
        hd = int(g.choice([4, 8, 16, 32, 64, 80, 128]))
        d = heads * hd
        if d % 64 or d > 2560 or heads > 256:
            continue
        m = int(g.choice([1, 1, 1, 2, 3]))
        max_seq = int(g.integers(2, 2048))
        pos = int(g.integers(0, max_seq))
        cases.append((m, d, heads, max_seq, pos))
    return cases


@pytest.mark.parametrize("m,d,heads,max_seq,pos", _random_attention_cases(10))
def test_decode_step_random_shapes(bl, olib, m, d, heads, max_seq, pos):
    """One decode step at a random position over a prefilled cache, for seeded
    head counts, head sizes (4 .. 128), sequence counts and cache lengths: the
    persistent kernel's chunking (one chunk, shorter chunks over a head's
    workgroups, 256-position chunks) at one sequence, the launch-per-step path
    at several."""
    _run_steps(bl, olib, 1, m, d, 4 * d, heads, max_seq, [pos], seed=200 + pos, prefill=pos)
