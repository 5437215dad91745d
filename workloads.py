"""Seeded synthetic inputs and the model shapes of the BitNet pages.

This module is shared by the oracle side and the HIP side, so it holds none of
the method's arithmetic: no packing, no quantization, no norms. It only draws
random numbers and states shapes.

Shapes come from "BitNet Model - Complete Inference Pipeline" (Hesper API,
Models.BitNet), section "Model Configurations" (BitNet-3B and BitNet-1.3B), and
from "Transformer Block" (Hesper API, Layers.TransformerBlock), section
"Memory Layout" (q, k, v, o are dim x dim; gate and up dim -> ffn; down
ffn -> dim).

Recipe (one numpy PCG64 stream per tensor, seeded by
SeedSequence([2026, workload, layer, tensor])):
  * ternary weights: u uniform on {0..9}; t = -1 if u < 3, +1 if u >= 7, else 0,
    i.e. P(-1) = P(+1) = 0.3 and P(0) = 0.4;
  * per-tensor weight scale s_w uniform on (20, 60), fp32;
  * activations N(0, 1) fp32; with outliers, each element is multiplied by 20
    with probability 0.01;
  * RMSNorm gains: 1.0 for benchmarks, uniform on (0.5, 1.5) for parity cases;
  * attention stand-ins (input of the o projection) N(0, 1).
"""
import numpy as np

SEED_ROOT = 2026

# Model shapes from the pages.
BITNET_3B = dict(name="BitNet-3B", dim=2560, ffn=10240, layers=32, heads=32, vocab=50000)
BITNET_1P3B = dict(name="BitNet-1.3B", dim=2048, ffn=8192, layers=24, heads=16, vocab=50000)

# Workload ids used in seeds.
W_GEMV, W_FFN, W_STREAM, W_PREFILL, W_BATCHED = 0, 1, 2, 3, 4

# Tensor ids within a layer.
T_Q, T_K, T_V, T_O, T_GATE, T_UP, T_DOWN = range(7)
T_X, T_Z, T_G_ATTN, T_G_ATTN_SUB, T_G_FFN, T_G_FFN_SUB, T_HEAD, T_G_FINAL = range(7, 15)
T_EMB, T_TOKENS = 15, 16
LINEAR_NAMES = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")
SCALE_NAMES = ("sq", "sk", "sv", "so", "sg", "su", "sd")


def rng(workload, layer, tensor):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, workload, layer, tensor])))


def ternary(g, n, k):
    """int8 [n][k] with P(-1) = P(+1) = 0.3, P(0) = 0.4."""
    u = g.integers(0, 10, size=(n, k), dtype=np.uint8)
    return (u >= 7).astype(np.int8) - (u < 3).astype(np.int8)


def weight_scale(g):
    return np.float32(g.uniform(20.0, 60.0))


def activations(g, m, k, outliers=False):
    x = g.standard_normal((m, k), dtype=np.float32)
    if outliers:
        mask = g.random((m, k)) < 0.01
        x[mask] *= np.float32(20.0)
    return x


def gains(g, k, ones=False):
    if ones:
        return np.ones(k, np.float32)
    return g.uniform(0.5, 1.5, size=k).astype(np.float32)


def linear_shapes(dim, ffn):
    """(n_out, k_in) of the seven BitLinears of one layer, in T_Q..T_DOWN order."""
    return [(dim, dim)] * 4 + [(ffn, dim), (ffn, dim), (dim, ffn)]


def layer_inputs(workload, layer, dim, ffn, m, bench_gains=False):
    """Ternary weights (unpacked int8), scales, gains and the stand-in z for one layer."""
    out = {}
    for tid, (n, k) in enumerate(linear_shapes(dim, ffn)):
        g = rng(workload, layer, tid)
        out[LINEAR_NAMES[tid]] = ternary(g, n, k)
        out[SCALE_NAMES[tid]] = weight_scale(g)
    out["z"] = activations(rng(workload, layer, T_Z), m, dim)
    for tid, key, k in ((T_G_ATTN, "g_attn", dim), (T_G_ATTN_SUB, "g_attn_sub", dim),
                        (T_G_FFN, "g_ffn", dim), (T_G_FFN_SUB, "g_ffn_sub", ffn)):
        out[key] = gains(rng(workload, layer, tid), k, ones=bench_gains)
    return out


def random_fp32_weights(g, n, k, sigma=0.02):
    """fp32 weights for weight_quant cases (N(0, sigma^2))."""
    return (g.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)).astype(np.float32)
