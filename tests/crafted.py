"""Hand-found inputs for rare branches of the kernels (CPU-side data only).

absmax_flip(): a 256-value input x and RMSNorm gains g in which the element with
the largest exact |x g| (element 0) is not the one with the largest rounded
|y| = |fl32(fl32(x r) g)| (element 1; r the fixed-order RMSNorm factor): the
activation quant's absmax comes from element 1. The other 254 values are the
seeded activations and gains of workloads.py; the four values below were found
by a CPU search over fp32 neighbours (b g_b just below a g_a)."""
import numpy as np

import workloads as W

# element 0: a, g_a; element 1: b, g_b (fp32 bit patterns)
ABSMAX_FLIP = {"x0": 0x407D5FDB, "g0": 0x3F8BBCFA, "x1": 0x408F8D0F, "g1": 0x3F76A506}


def _f32(bits):
    return np.array([bits], np.uint32).view(np.float32)[0]


def absmax_flip(d=256):
    x = W.activations(W.rng(W.W_STREAM, 997, W.T_X), 1, d)[0].copy()
    g = W.gains(W.rng(W.W_STREAM, 0, W.T_G_ATTN), d).copy()
    x[0], g[0] = _f32(ABSMAX_FLIP["x0"]), _f32(ABSMAX_FLIP["g0"])
    x[1], g[1] = _f32(ABSMAX_FLIP["x1"]), _f32(ABSMAX_FLIP["g1"])
    return x, g
