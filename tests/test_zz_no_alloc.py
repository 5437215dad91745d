"""bitlinear_gemm_noalloc (argmax keys in the library's static device array)
against bitlinear_gemm with a caller workspace, through the C ABI: the same
outputs bit for bit on consecutive calls, the second one smaller, on both the
m <= 32 (per-tile keys) and the m > 32 (per-row atomic keys) paths; and an
argmax larger than the array refused with BL_ERR_WORKSPACE, nothing written."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import assert_exact, log, pack_both, to_dev, to_host, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import bitlinear_amd
    return bitlinear_amd


def _inputs(olib, m, n, k, seed):
    g = W.rng(120, seed, m)
    t = W.ternary(g, n, k)
    sw = W.weight_scale(g)
    x = W.activations(g, m, k)
    p = pack_both(t, olib)
    q, s, qs = oracle.quant_act(x, None, 1e-5, olib)
    return p, sw, q, s, qs


def _both(bl, olib, m, n, k, seed, with_argmax=True):
    import torch
    log(f"noalloc gemm m={m} n={n} k={k} argmax={with_argmax}")
    p, sw, q, s, qs = _inputs(olib, m, n, k, seed)
    dev = torch_dev()
    pd, qd, sd, qsd = to_dev(p), to_dev(q), to_dev(s), to_dev(qs)
    y0 = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    acc0 = torch.empty((m, n), dtype=torch.int32, device=dev)
    am0 = torch.full((m,), -1, dtype=torch.int32, device=dev) if with_argmax else None
    ws = torch.empty(max(bl.bitlinear_gemm_workspace_bytes(m, n, k, 1), 8), dtype=torch.uint8, device=dev)
    bl.bitlinear_gemm(pd, sw, n, k, qd, sd, qsd, m, None, y0, acc0, am0, ws if with_argmax else None)
    y1 = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
    acc1 = torch.empty((m, n), dtype=torch.int32, device=dev)
    am1 = torch.full((m,), -1, dtype=torch.int32, device=dev) if with_argmax else None
    bl.bitlinear_gemm_noalloc(pd, sw, n, k, qd, sd, qsd, m, None, y1, acc1, am1)
    assert_exact(to_host(y1).view(np.uint32), to_host(y0).view(np.uint32), "y bits, noalloc vs workspace")
    assert_exact(to_host(acc1), to_host(acc0), "acc, noalloc vs workspace")
    if with_argmax:
        got = to_host(am1)
        assert_exact(got, to_host(am0), "argmax, noalloc vs workspace")
        oacc = oracle.matmul_i32(oracle.unpack(p, k, olib), q, olib)
        assert_exact(got, oracle.argmax_rows(oacc, olib), "argmax vs oracle")


def test_noalloc_skinny_path_two_calls(bl, olib):
    # the LM head shape of the pages' 1.3B model, then a smaller call
    _both(bl, olib, 32, 50000, 2048, 0)
    _both(bl, olib, 7, 3000, 256, 1)


def test_noalloc_gemm_path_two_calls(bl, olib):
    _both(bl, olib, 40, 300, 128, 2)
    _both(bl, olib, 36, 130, 64, 3)


def test_noalloc_without_argmax(bl, olib):
    _both(bl, olib, 64, 640, 256, 4, with_argmax=False)


def test_noalloc_refuses_an_argmax_larger_than_the_array(bl, olib):
    import torch
    cap = bl.bitlinear_gemm_noalloc_max_scratch_bytes()
    m, k = 32, 64
    n = 32 * (cap // (32 * 8)) + 64
    assert bl.bitlinear_gemm_workspace_bytes(m, n, k, 1) > cap
    dev = torch_dev()
    p = torch.zeros((n, k // 4), dtype=torch.uint8, device=dev)
    q = torch.zeros((m, k), dtype=torch.int8, device=dev)
    s = torch.ones(m, dtype=torch.float32, device=dev)
    qs = torch.zeros(m, dtype=torch.int32, device=dev)
    am = torch.full((m,), -7, dtype=torch.int32, device=dev)
    with pytest.raises(bl.BitlinearError) as e:
        bl.bitlinear_gemm_noalloc(p, 30.0, n, k, q, s, qs, m, None, None, None, am)
    assert e.value.status == bl.BL_ERR_WORKSPACE
    assert (to_host(am) == -7).all()
