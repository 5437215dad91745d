"""CPU oracle of the BitNet b1.58 BitLinear path (numpy front end over liboracle.so).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this package. It shares no code with the HIP path.

The arithmetic lives in ``bitlinear_oracle.c``; this module marshals numpy
arrays and composes the primitives in the order the pages give:

* ``ffn`` follows "Transformer Block" (Hesper API, Layers.TransformerBlock),
  sections "Feed-Forward Network (FFN)" and "Forward Pass" steps 4-8, with the
  ffnSubNorm that "Layer Structure" lists between the gating and ffnDown.
* ``chain`` is the per-layer stream of seven BitLinears of the same page
  ("Memory Layout": q, k, v, o, gate, up, down), each behind an RMSNorm as in
  "Add Support for BitNet Architecture Inference" (candle PR 2664).  Attention
  itself is left out: q/k/v are computed and returned, and the o projection
  reads a seeded stand-in vector passed in by the caller.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i8p = ctypes.POINTER(ctypes.c_int8)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64 = ctypes.c_int64


class OracleError(RuntimeError):
    pass


def load(path=None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        from . import build as _b
        _b.build(out=p, quiet=True)
    lib = ctypes.CDLL(p)
    lib.ref_weight_quant.argtypes = [_f32p, _i64, _i64, _i8p, _f32p]
    lib.ref_pack.argtypes = [_i8p, _i64, _i64, _u8p]
    lib.ref_unpack.argtypes = [_u8p, _i64, _i64, _i8p]
    lib.ref_sumsq.argtypes = [_f32p, _i64]
    lib.ref_sumsq.restype = ctypes.c_double
    lib.ref_rmsnorm.argtypes = [_f32p, _f32p, ctypes.c_float, _i64, _i64, _f32p]
    lib.ref_activation_quant.argtypes = [_f32p, _i64, _i64, _i8p, _f32p, _i32p]
    lib.ref_matmul_i32.argtypes = [_i8p, _i8p, _i64, _i64, _i64, _i32p]
    lib.ref_dequant.argtypes = [_i32p, _f32p, ctypes.c_float, _i64, _i64, _f32p]
    lib.ref_bitlinear.argtypes = [_u8p, ctypes.c_float, _i64, _i64, _i8p, _f32p, _i64, _f32p, _i32p]
    lib.ref_relu2_mul.argtypes = [_f32p, _f32p, _i64, _f32p]
    lib.ref_relu2_mul.restype = None
    lib.ref_residual_add.argtypes = [_f32p, _f32p, _i64]
    lib.ref_residual_add.restype = None
    lib.ref_argmax_rows.argtypes = [_i32p, _i64, _i64, _i32p]
    lib.ref_embed.argtypes = [_u8p, ctypes.c_float, _i64, _i64, _i32p, _i64, _f32p]
    lib.ref_penalty_argmax.argtypes = [_f32p, _i64, _i64, _i32p, _i64, _i32p, ctypes.c_float, _i32p]
    lib.ref_exp_neg.argtypes = [ctypes.c_double]
    lib.ref_exp_neg.restype = ctypes.c_double
    lib.ref_sample.argtypes = [_f32p, _i64, _i64, ctypes.c_int, _i64, ctypes.c_float, ctypes.c_float,
                               ctypes.POINTER(ctypes.c_double), _i32p]
    lib.ref_rope_table.argtypes = [ctypes.c_double, _i64, _i64, _f32p, _f32p]
    lib.ref_rope_apply.argtypes = [_f32p, _f32p, _f32p, _i64]
    lib.ref_rope_apply.restype = None
    lib.ref_attention.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _i64, _f32p]
    lib.ref_set_threads.argtypes = [ctypes.c_int]
    lib.ref_set_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def set_threads(n, lib=None):
    """Threads of the oracle's row-parallel loops (n <= 0: unchanged); returns the setting."""
    lib = lib or load()
    return int(lib.ref_set_threads(int(n)))


def _ptr(a, ty):
    return a.ctypes.data_as(ty)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


# --- primitives ---------------------------------------------------------------

def weight_quant(w, lib=None):
    """fp32 W[n][k] -> (t int8[n][k], s_w fp32): absmean ternary quantization."""
    lib = lib or load()
    w = _c(w, np.float32)
    n, k = w.shape
    t = np.empty((n, k), np.int8)
    s = np.zeros(1, np.float32)
    _check(lib.ref_weight_quant(_ptr(w, _f32p), n, k, _ptr(t, _i8p), _ptr(s, _f32p)), "weight_quant")
    return t, np.float32(s[0])


def pack(t, lib=None):
    """int8 t[n][k] in {-1,0,1} -> uint8 packed[n][k/4] (TQ2_0, 4 codes/byte)."""
    lib = lib or load()
    t = _c(t, np.int8)
    n, k = t.shape
    out = np.empty((n, k // 4), np.uint8)
    _check(lib.ref_pack(_ptr(t, _i8p), n, k, _ptr(out, _u8p)), "pack")
    return out


def unpack(packed, k, lib=None):
    lib = lib or load()
    packed = _c(packed, np.uint8)
    n = packed.shape[0]
    t = np.empty((n, k), np.int8)
    _check(lib.ref_unpack(_ptr(packed, _u8p), n, k, _ptr(t, _i8p)), "unpack")
    return t


def sumsq(x, lib=None):
    """The RMSNorm sum of squares of one vector, in the fixed fp64 order."""
    lib = lib or load()
    x = _c(x, np.float32)
    return float(lib.ref_sumsq(_ptr(x, _f32p), x.size))


def rmsnorm(x, g, eps, lib=None):
    lib = lib or load()
    x = _c(x, np.float32)
    m, k = x.shape
    g = _c(g, np.float32)
    y = np.empty_like(x)
    _check(lib.ref_rmsnorm(_ptr(x, _f32p), _ptr(g, _f32p), ctypes.c_float(eps), m, k, _ptr(y, _f32p)), "rmsnorm")
    return y


def activation_quant(y, lib=None):
    """fp32 y[m][k] -> (q int8[m][k], s_a fp32[m], qsum int32[m])."""
    lib = lib or load()
    y = _c(y, np.float32)
    m, k = y.shape
    q = np.empty((m, k), np.int8)
    s = np.empty(m, np.float32)
    qs = np.empty(m, np.int32)
    _check(lib.ref_activation_quant(_ptr(y, _f32p), m, k, _ptr(q, _i8p), _ptr(s, _f32p), _ptr(qs, _i32p)),
           "activation_quant")
    return q, s, qs


def quant_act(x, gain=None, eps=1e-5, lib=None):
    """[RMSNorm(gain, eps) +] activation_quant. gain None means no norm."""
    x = _c(np.atleast_2d(x), np.float32)
    y = x if gain is None else rmsnorm(x, gain, eps, lib)
    return activation_quant(y, lib)


def matmul_i32(t, q, lib=None):
    """acc[m][n] = sum_k t[n][k] q[m][k] (exact int32)."""
    lib = lib or load()
    t = _c(t, np.int8)
    q = _c(np.atleast_2d(q), np.int8)
    n, k = t.shape
    m = q.shape[0]
    acc = np.empty((m, n), np.int32)
    _check(lib.ref_matmul_i32(_ptr(t, _i8p), _ptr(q, _i8p), m, n, k, _ptr(acc, _i32p)), "matmul_i32")
    return acc


def dequant(acc, s_a, s_w, lib=None):
    lib = lib or load()
    acc = _c(acc, np.int32)
    m, n = acc.shape
    s_a = _c(s_a, np.float32)
    y = np.empty((m, n), np.float32)
    _check(lib.ref_dequant(_ptr(acc, _i32p), _ptr(s_a, _f32p), ctypes.c_float(s_w), m, n, _ptr(y, _f32p)),
           "dequant")
    return y


def bitlinear(packed, s_w, k, q, s_a, lib=None):
    """One BitLinear on quantized activations -> (y fp32[m][n], acc int32[m][n])."""
    lib = lib or load()
    packed = _c(packed, np.uint8)
    q = _c(np.atleast_2d(q), np.int8)
    s_a = _c(s_a, np.float32)
    n = packed.shape[0]
    m = q.shape[0]
    y = np.empty((m, n), np.float32)
    acc = np.empty((m, n), np.int32)
    _check(lib.ref_bitlinear(_ptr(packed, _u8p), ctypes.c_float(s_w), n, k, _ptr(q, _i8p), _ptr(s_a, _f32p), m,
                             _ptr(y, _f32p), _ptr(acc, _i32p)), "bitlinear")
    return y, acc


def relu2_mul(gate, up, lib=None):
    lib = lib or load()
    gate = _c(gate, np.float32)
    up = _c(up, np.float32)
    h = np.empty_like(gate)
    lib.ref_relu2_mul(_ptr(gate, _f32p), _ptr(up, _f32p), gate.size, _ptr(h, _f32p))
    return h


def residual_add(x, d, lib=None):
    """Returns fl32(x + d) as a new array."""
    lib = lib or load()
    out = _c(x, np.float32).copy()
    d = _c(d, np.float32)
    lib.ref_residual_add(_ptr(out, _f32p), _ptr(d, _f32p), out.size)
    return out


def argmax_rows(acc, lib=None):
    lib = lib or load()
    acc = _c(acc, np.int32)
    m, n = acc.shape
    idx = np.empty(m, np.int32)
    _check(lib.ref_argmax_rows(_ptr(acc, _i32p), m, n, _ptr(idx, _i32p)), "argmax_rows")
    return idx


def embed(table, s_e, tokens, d, lib=None):
    """Ternary embedding lookup: x[r] = t[tokens[r]] / s_e (zero row for an id
    outside the table). table: packed [vocab][d/4]."""
    lib = lib or load()
    table = _c(table, np.uint8)
    tokens = _c(np.atleast_1d(tokens), np.int32)
    vocab = table.shape[0]
    x = np.empty((tokens.size, d), np.float32)
    _check(lib.ref_embed(_ptr(table, _u8p), ctypes.c_float(s_e), vocab, d, _ptr(tokens, _i32p), tokens.size,
                         _ptr(x, _f32p)), "embed")
    return x


def penalty_argmax(logits, hist, hist_len, penalty, lib=None):
    """Repetition penalty over each row's history, then the lowest-index argmax.
    Returns (idx int32[m], penalised logits). hist: int32 [m][stride]."""
    lib = lib or load()
    out = _c(np.atleast_2d(logits), np.float32).copy()
    m, n = out.shape
    hist = _c(np.atleast_2d(hist), np.int32)
    hist_len = _c(np.atleast_1d(hist_len), np.int32)
    idx = np.empty(m, np.int32)
    _check(lib.ref_penalty_argmax(_ptr(out, _f32p), m, n, _ptr(hist, _i32p), hist.shape[1], _ptr(hist_len, _i32p),
                                  ctypes.c_float(penalty), _ptr(idx, _i32p)), "penalty_argmax")
    return idx, out


def exp_neg(x, lib=None):
    """The sampler's exponential of x in [-32, 0] (0 below -32)."""
    lib = lib or load()
    return float(lib.ref_exp_neg(float(x)))


def _sample(logits, mode, k, p, temperature, u, lib):
    lib = lib or load()
    logits = _c(np.atleast_2d(logits), np.float32)
    m, n = logits.shape
    u = _c(np.atleast_1d(u), np.float64)
    assert u.size == m
    idx = np.empty(m, np.int32)
    _check(lib.ref_sample(_ptr(logits, _f32p), m, n, mode, int(k), ctypes.c_float(p), ctypes.c_float(temperature),
                          u.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), _ptr(idx, _i32p)), "sample")
    return idx


def sample_topk(logits, k, temperature, u, lib=None):
    """Top-k sampling of each row with its uniform draw u[r] in [0, 1)."""
    return _sample(logits, 0, k, 1.0, temperature, u, lib)


def sample_topp(logits, p, temperature, u, lib=None):
    """Nucleus (top-p) sampling of each row with its uniform draw u[r] in [0, 1)."""
    return _sample(logits, 1, 1, p, temperature, u, lib)


def rope_table(base, hd, max_pos, lib=None):
    """(cos, sin) fp32 [max_pos][hd/2] of the rotary embedding."""
    lib = lib or load()
    c = np.empty((max_pos, hd // 2), np.float32)
    s = np.empty((max_pos, hd // 2), np.float32)
    _check(lib.ref_rope_table(float(base), hd, max_pos, _ptr(c, _f32p), _ptr(s, _f32p)), "rope_table")
    return c, s


def rope_apply(x, c_row, s_row, lib=None):
    """Rotate every head vector of x[..., hd] (fp32, last axis) with one table row."""
    lib = lib or load()
    out = _c(x, np.float32).copy()
    hd = out.shape[-1]
    c_row = _c(c_row, np.float32)
    s_row = _c(s_row, np.float32)
    flat = out.reshape(-1, hd)
    for v in flat:
        lib.ref_rope_apply(_ptr(v, _f32p), _ptr(c_row, _f32p), _ptr(s_row, _f32p), hd)
    return flat.reshape(out.shape)


def attention(q, k_cache, v_cache, pos, lib=None):
    """q [m][H][hd]; caches [m][H][max_seq][hd] -> out [m][H*hd] (fp64 inside)."""
    lib = lib or load()
    q = _c(q, np.float32)
    k_cache = _c(k_cache, np.float32)
    v_cache = _c(v_cache, np.float32)
    m, heads, hd = q.shape
    max_seq = k_cache.shape[2]
    out = np.empty((m, heads * hd), np.float32)
    _check(lib.ref_attention(_ptr(q, _f32p), _ptr(k_cache, _f32p), _ptr(v_cache, _f32p), m, heads, hd, max_seq, pos,
                             _ptr(out, _f32p)), "attention")
    return out


# --- compositions -------------------------------------------------------------

def ffn(x, norm_gain, sub_norm_gain, eps, w_gate, s_gate, w_up, s_up, w_down, s_down, lib=None):
    """BitNet FFN sub-layer without the residual add. Returns every intermediate.

    x[m][d] fp32; w_gate/w_up packed [f][d/4]; w_down packed [d][f/4].
    """
    x = _c(np.atleast_2d(x), np.float32)
    d = x.shape[1]
    f = w_gate.shape[0]
    q1, s1, qs1 = quant_act(x, norm_gain, eps, lib)
    gate, acc_gate = bitlinear(w_gate, s_gate, d, q1, s1, lib)
    up, acc_up = bitlinear(w_up, s_up, d, q1, s1, lib)
    h = relu2_mul(gate, up, lib)
    q2, s2, qs2 = quant_act(h, sub_norm_gain, eps, lib)
    out, acc_down = bitlinear(w_down, s_down, f, q2, s2, lib)
    return dict(q1=q1, s1=s1, qs1=qs1, acc_gate=acc_gate, acc_up=acc_up, gate=gate, up=up, h=h,
                q2=q2, s2=s2, qs2=qs2, acc_down=acc_down, out=out)


def layer(x, lw, eps, lib=None):
    """One decoder layer of the BitLinear stream (attention math excluded).

    lw: dict with packed weights wq, wk, wv, wo ([d][d/4]), wg, wu ([f][d/4]),
    wd ([d][f/4]), their scales sq..sd, gains g_attn, g_attn_sub, g_ffn,
    g_ffn_sub ([d], [d], [d], [f]) and z ([m][d]), the stand-in for the
    attention output that feeds the o projection.
    Returns (x_next, qkv[m][3d]).
    """
    x = _c(np.atleast_2d(x), np.float32)
    d = x.shape[1]
    a, sa, _ = quant_act(x, lw["g_attn"], eps, lib)
    yq, _ = bitlinear(lw["wq"], lw["sq"], d, a, sa, lib)
    yk, _ = bitlinear(lw["wk"], lw["sk"], d, a, sa, lib)
    yv, _ = bitlinear(lw["wv"], lw["sv"], d, a, sa, lib)
    o_in, so, _ = quant_act(lw["z"], lw["g_attn_sub"], eps, lib)
    yo, _ = bitlinear(lw["wo"], lw["so"], d, o_in, so, lib)
    x = residual_add(x, yo, lib)
    f = ffn(x, lw["g_ffn"], lw["g_ffn_sub"], eps, lw["wg"], lw["sg"], lw["wu"], lw["su"], lw["wd"], lw["sd"], lib)
    x = residual_add(x, f["out"], lib)
    return x, np.concatenate([yq, yk, yv], axis=1)


def chain(x, layers, eps, lib=None):
    """Run ``layer`` over a list of layer weight dicts. Returns (x, [qkv per layer])."""
    qkvs = []
    for lw in layers:
        x, qkv = layer(x, lw, eps, lib)
        qkvs.append(qkv)
    return x, qkvs


def lm_head_argmax(x, g_final, eps, w_head, s_head, lib=None):
    """Final RMSNorm + activation quant, ternary LM head, per-row greedy argmax.
    Returns (idx int32[m], acc int32[m][vocab])."""
    x = _c(np.atleast_2d(x), np.float32)
    d = x.shape[1]
    q, s, _ = quant_act(x, g_final, eps, lib)
    t = unpack(w_head, d, lib)
    acc = matmul_i32(t, q, lib)
    return argmax_rows(acc, lib), acc


def greedy_head(x, g_final, eps, w_head, s_head, hist, hist_len, penalty, lib=None):
    """Final RMSNorm + activation quant, ternary LM head, repetition penalty over
    each row's history and the greedy choice ("BitNet Model - Complete
    Inference Pipeline": "Architecture" -- final RMSNorm, LM head, sampling;
    "GPU Argmax" -- gpuArgmaxWithPenalty). Returns (idx, penalised logits,
    raw logits)."""
    x = _c(np.atleast_2d(x), np.float32)
    d = x.shape[1]
    q, s, _ = quant_act(x, g_final, eps, lib)
    logits, _ = bitlinear(w_head, s_head, d, q, s, lib)
    idx, pen = penalty_argmax(logits, hist, hist_len, penalty, lib)
    return idx, pen, logits


def greedy_step(tokens, table, s_e, layers, g_final, eps, w_head, s_head, hist, hist_len, penalty, lib=None):
    """One greedy decoding step ("Text Generation / Greedy Decoding"): embed the
    current tokens, run the layer stream, choose the next tokens with the
    penalised greedy head, and append them to the histories (a full history
    is left as it is). Returns (next tokens, new hist, new hist_len, x)."""
    d = table.shape[1] * 4
    x = embed(table, s_e, tokens, d, lib)
    x, _ = chain(x, layers, eps, lib)
    idx, _, _ = greedy_head(x, g_final, eps, w_head, s_head, hist, hist_len, penalty, lib)
    hist = np.array(hist, np.int32, copy=True)
    hist_len = np.array(hist_len, np.int32, copy=True)
    for r in range(idx.size):
        if hist_len[r] < hist.shape[1]:
            hist[r, hist_len[r]] = idx[r]
            hist_len[r] += 1
    return idx, hist, hist_len, x


def layer_attn(x, lw, eps, heads, cos_t, sin_t, k_cache, v_cache, pos, attn_in=None, lib=None):
    """One decoder layer with attention ("Transformer Block", "Forward Pass with
    KV Cache"): a = quant(rmsnorm(x, g_attn)); q, k, v = BitLinear(a); q and k
    rotated for position pos; k, v written to the caches (in place, [m][H][S][hd]);
    attn = attention over positions 0 .. pos; x += BitLinear_o(quant(rmsnorm(attn,
    g_attn_sub))); x += ffn(x). attn_in, if given, replaces the computed
    attention output downstream (to continue from another implementation's
    floating-point attention). Returns (x_next, qkv [m][3d], attn [m][d])."""
    x = _c(np.atleast_2d(x), np.float32)
    m, d = x.shape
    hd = d // heads
    a, sa, _ = quant_act(x, lw["g_attn"], eps, lib)
    yq, _ = bitlinear(lw["wq"], lw["sq"], d, a, sa, lib)
    yk, _ = bitlinear(lw["wk"], lw["sk"], d, a, sa, lib)
    yv, _ = bitlinear(lw["wv"], lw["sv"], d, a, sa, lib)
    q_rot = rope_apply(yq.reshape(m, heads, hd), cos_t[pos], sin_t[pos], lib)
    k_rot = rope_apply(yk.reshape(m, heads, hd), cos_t[pos], sin_t[pos], lib)
    k_cache[:, :, pos, :] = k_rot
    v_cache[:, :, pos, :] = yv.reshape(m, heads, hd)
    attn = attention(q_rot, k_cache, v_cache, pos, lib)
    use = attn if attn_in is None else _c(attn_in, np.float32)
    o_in, so, _ = quant_act(use, lw["g_attn_sub"], eps, lib)
    yo, _ = bitlinear(lw["wo"], lw["so"], d, o_in, so, lib)
    x = residual_add(x, yo, lib)
    f = ffn(x, lw["g_ffn"], lw["g_ffn_sub"], eps, lw["wg"], lw["sg"], lw["wu"], lw["su"], lw["wd"], lw["sd"], lib)
    x = residual_add(x, f["out"], lib)
    return x, np.concatenate([yq, yk, yv], axis=1), attn
