"""The hand-found inputs of tests/crafted.py have the property their GPU tests
rely on, checked against the oracle (CPU only)."""
import numpy as np

import oracle
from crafted import absmax_flip


def _rmsnorm_factor(x, eps):
    """r = fl32(1 / sqrt(S / n + eps)) with S the fixed-order fp64 sum of squares:
    512 strided partials (ascending k), then an xor butterfly with offsets 1 .. 256."""
    part = np.zeros(512)
    for k, v in enumerate(x.astype(np.float64)):
        part[k % 512] += v * v
    off = 1
    while off < 512:
        part = part + part[np.arange(512) ^ off]
        off *= 2
    return np.float32(1.0 / np.sqrt(part[0] / len(x) + eps))


def test_absmax_flip_input(olib):
    """Element 0 holds the largest exact |x g|, yet the absmax comes from element
    1, whose product rounds to the larger |y|: the oracle's scale is 127 / |y_1|,
    which differs from 127 / |y_0|. A kernel that took the absmax from the largest
    product alone would quantize with the other scale."""
    x, g = absmax_flip()
    prod = np.abs(x.astype(np.float64) * g.astype(np.float64))
    assert int(np.argmax(prod)) == 0 and np.all(prod[2:] < prod[1]) and prod[1] < prod[0]
    r = _rmsnorm_factor(x, 1e-5)
    y0 = np.float32(np.float32(x[0] * r) * g[0])
    y1 = np.float32(np.float32(x[1] * r) * g[1])
    assert abs(y1) > abs(y0)
    _, s, _ = oracle.quant_act(x[None, :], g, 1e-5, olib)
    assert s[0] == np.float32(127.0) / np.float32(abs(y1))
    assert s[0] != np.float32(127.0) / np.float32(abs(y0))
