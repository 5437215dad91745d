"""GPU parity of top-k and nucleus sampling against the oracle, through the C
ABI: for every row the sampled token must be the oracle's, exactly (both sides
take every decision on identical fp64 values and exact integer sums). Logits:
N(0, s^2) rows, integer-valued rows full of ties, rows with a huge spread (most
weights 0), constant rows; draws u: random, 0, 1/2 and the largest double below
1; a pair of equal logits where u = 1/2 is exactly a boundary."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_exact, log, to_dev, to_host, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import bitlinear_amd
    return bitlinear_amd


def _rows(g, m, n):
    kinds = []
    rows = []
    for r in range(m):
        kind = r % 4
        if kind == 0:
            rows.append(g.standard_normal(n) * g.uniform(0.5, 4.0))
        elif kind == 1:
            rows.append(g.integers(-4, 5, n).astype(np.float64))
        elif kind == 2:
            rows.append(g.standard_normal(n) * 60.0)
        else:
            rows.append(np.full(n, g.uniform(-3, 3)))
        kinds.append(kind)
    return np.stack(rows).astype(np.float32)


def _draws(g, m):
    u = g.random(m)
    special = [0.0, 0.5, 1.0 - 2.0 ** -53]
    for i, v in enumerate(special[:m]):
        u[i] = v
    return u


def _run(bl, logits, u, mode, param, temp):
    import torch
    m, n = logits.shape
    dev = torch_dev()
    tok = torch.full((m,), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(bl.bitnet_sample_workspace_bytes(m, n), dtype=torch.uint8, device=dev)
    ud = torch.from_numpy(np.ascontiguousarray(u, np.float64)).to(dev)
    if mode == "topk":
        bl.bitnet_sample_topk(to_dev(logits), param, temp, ud, tok, ws)
    else:
        bl.bitnet_sample_topp(to_dev(logits), param, temp, ud, tok, ws)
    return to_host(tok)


@pytest.mark.parametrize("n", [50000, 1000, 7, 1])
@pytest.mark.parametrize("mode,param,temp", [("topk", 1, 1.0), ("topk", 5, 0.7), ("topk", 40, 1.0),
                                             ("topk", 1000, 1.5), ("topk", 60000, 1.0), ("topp", 0.1, 1.0),
                                             ("topp", 0.5, 0.8), ("topp", 0.9, 1.0), ("topp", 0.999, 2.0),
                                             ("topp", 1.0, 1.0), ("topp", 1.5, 0.5)])
def test_sample_matches_oracle(bl, olib, n, mode, param, temp):
    m = 24
    log(f"sample {mode} {param} T={temp} n={n}")
    g = W.rng(140, n, int(param * 1000) + int(temp * 10))
    logits = _rows(g, m, n)
    u = _draws(g, m)
    got = _run(bl, logits, u, mode, param, temp)
    want = (oracle.sample_topk(logits, param, temp, u, olib) if mode == "topk"
            else oracle.sample_topp(logits, param, temp, u, olib))
    assert_exact(got, want, f"{mode} tokens")


def test_sample_exact_boundary(bl, olib):
    """Equal logits at indices 1 and 2 (weights 2^40 each) with top-2: u just
    below 1/2 takes index 1, u = 1/2 takes index 2."""
    logits = np.tile(np.array([[0.25, 2.0, 2.0, -1.0]], np.float32), (3, 1))
    u = np.array([0.5 - 2.0 ** -53, 0.5, 0.0])
    assert _run(bl, logits, u, "topk", 2, 1.0).tolist() == [1, 2, 1]
    assert (oracle.sample_topk(logits, 2, 1.0, u, olib) == [1, 2, 1]).all()


def test_sample_vocab_rows_many_draws(bl, olib):
    """32 rows of 50000 logits from the ternary LM head's scale of values, 4
    draws per row (the rows repeated), both samplers."""
    g = W.rng(141, 0, 0)
    base = (g.standard_normal((32, 50000)) * 3.0).astype(np.float32)
    logits = np.repeat(base, 4, axis=0)
    u = g.random(logits.shape[0])
    for mode, param in (("topk", 50), ("topp", 0.9)):
        got = _run(bl, logits, u, mode, param, 0.8)
        want = (oracle.sample_topk(logits, param, 0.8, u, olib) if mode == "topk"
                else oracle.sample_topp(logits, param, 0.8, u, olib))
        assert_exact(got, want, f"{mode} tokens, vocabulary rows")
