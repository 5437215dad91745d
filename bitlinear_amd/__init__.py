"""Python binding of libbitlinear.so (the BitNet b1.58 BitLinear path on MI355X).

Thin marshalling layer: every function has the name of its C entry point
(include/bitlinear.h), checks dtype / device / contiguity of its arguments, and
passes raw pointers and sizes to the library. All arithmetic runs in the HIP
kernels. torch is used only for device memory and streams; host-side calls
(bitlinear_pack, bitlinear_weight_quant) take numpy arrays.

Importing this module loads the built library and raises ImportError if it is
missing: there is no fallback path.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

BL_OK = 0
BL_ERR_NULL = -1
BL_ERR_SHAPE = -2
BL_ERR_ALIGN = -3
BL_ERR_VALUE = -4
BL_ERR_WORKSPACE = -5
BL_ERR_LAUNCH = -6
BL_ERR_DEVICE = -7

BITNET_FFN_WRITE_ACC = 1
FFN_WS_SEGMENTS = ("q1", "s1", "qs1", "h", "q2", "s2", "qs2", "acc_gate", "acc_up", "acc_down", "gate", "up")

# Every symbol the header declares (checked by the CPU tests).
EXPORTS = (
    "bitlinear_abi_version", "bitlinear_strerror", "bitlinear_pack", "bitlinear_weight_quant",
    "bitlinear_quant_act", "bitlinear_gemv", "bitlinear_forward", "bitlinear_gemm_workspace_bytes", "bitlinear_gemm",
    "bitnet_ffn_workspace_bytes", "bitnet_ffn_workspace_offset", "bitnet_ffn", "bitnet_layer_bytes",
    "bitnet_stream_workspace_bytes", "bitnet_decode_stream",
    "bitlinear_probe_read", "bitlinear_probe_mfma_ops", "bitlinear_probe_mfma_i8", "bitlinear_probe_mfma_i8_dense",
    "bitlinear_gemm_noalloc", "bitlinear_gemm_noalloc_max_scratch_bytes",
    "bitnet_embed", "bitnet_greedy_head_workspace_bytes", "bitnet_greedy_head", "bitnet_greedy_step_workspace_bytes",
    "bitnet_greedy_step", "bitnet_sample_workspace_bytes", "bitnet_sample_topk", "bitnet_sample_topp",
    "bitnet_decode_step_workspace_bytes", "bitnet_decode_step", "bitnet_rope_table",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")

# torch ships its own HIP runtime, and the library is linked against it. torch
# must be loaded first so that the library binds to that same runtime instance
# (a second runtime would not know torch's streams or allocations).
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped():
    try:
        with open(f"/proc/{os.getpid()}/maps") as fh:
            return sorted({line.split()[-1] for line in fh if "libamdhip64" in line})
    except OSError:
        return []


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError(f"two HIP runtimes are loaded ({_hip_runtimes_mapped()}); import torch before any other "
                      "HIP library")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "bitlinear_abi_version": ([], _I),
    "bitlinear_strerror": ([_I], ctypes.c_char_p),
    "bitlinear_pack": ([_P, _I64, _I64, _P], _I),
    "bitlinear_weight_quant": ([_P, _I64, _I64, _P, _P], _I),
    "bitlinear_quant_act": ([_P, _P, _F, _I64, _I64, _P, _P, _P, _P], _I),
    "bitlinear_gemv": ([_P, _F, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _P], _I),
    "bitlinear_forward": ([_P, _P, _F, _P, _F, _I64, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "bitlinear_gemm_workspace_bytes": ([_I64, _I64, _I64, _I], _SZ),
    "bitlinear_gemm": ([_P, _F, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "bitnet_ffn_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "bitnet_ffn_workspace_offset": ([_I64, _I64, _I64, _I], _SZ),
    "bitnet_ffn": ([_P, _I64, _I64, _I64, _P, _P, _F, _P, _F, _P, _F, _P, _F, _P, _P, _P, _SZ, _I, _P], _I),
    "bitnet_layer_bytes": ([_I64, _I64], _SZ),
    "bitnet_stream_workspace_bytes": ([_I64, _I64, _I64], _SZ),
    "bitnet_decode_stream": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _P, _P, _P, _SZ, _P], _I),
    "bitlinear_gemm_noalloc": ([_P, _F, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _P, _P], _I),
    "bitlinear_gemm_noalloc_max_scratch_bytes": ([], _SZ),
    "bitnet_embed": ([_P, _F, _I64, _I64, _P, _I64, _P, _P], _I),
    "bitnet_greedy_head_workspace_bytes": ([_I64, _I64], _SZ),
    "bitnet_greedy_head": ([_P, _F, _I64, _I64, _P, _P, _P, _I64, _P, _I64, _P, _F, _P, _P, _P, _SZ, _P], _I),
    "bitnet_greedy_step_workspace_bytes": ([_I64, _I64, _I64, _I64], _SZ),
    "bitnet_greedy_step": ([_P, _F, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _F, _P, _P, _F, _P, _I64, _P, _I64, _P,
                            _F, _P, _P, _P, _SZ, _P], _I),
    "bitnet_sample_workspace_bytes": ([_I64, _I64], _SZ),
    "bitnet_sample_topk": ([_P, _I64, _I64, _I64, _F, _P, _P, _P, _SZ, _P], _I),
    "bitnet_sample_topp": ([_P, _I64, _I64, _F, _F, _P, _P, _P, _SZ, _P], _I),
    "bitnet_decode_step_workspace_bytes": ([_I64, _I64, _I64, _I64, _I64], _SZ),
    "bitnet_decode_step": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P,
                            _SZ, _P], _I),
    "bitnet_rope_table": ([ctypes.c_double, _I64, _I64, _P, _P], _I),
    "bitlinear_probe_read": ([_P, _SZ, _P, _P], _I),
    "bitlinear_probe_mfma_ops": ([_I64], _I64),
    "bitlinear_probe_mfma_i8": ([_I64, _P, _P], _I),
    "bitlinear_probe_mfma_i8_dense": ([_I64, _P, _P], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class BitlinearError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {_lib.bitlinear_strerror(status).decode()} (status {status})")


def _check(status, what):
    if status != BL_OK:
        raise BitlinearError(status, what)


def _dev(t, dtype=None, name="tensor", optional=False):
    """Device pointer of a contiguous torch tensor (or None)."""
    if t is None:
        if optional:
            return None
        raise BitlinearError(BL_ERR_NULL, f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _host(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a C-contiguous numpy array of {np.dtype(dtype)}")
    return a.ctypes.data


# The current stream's raw handle straight from torch's C layer (0.1 us), not
# through a Stream object (about 3 us a call), when this torch build has it.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    if stream is not None:
        return stream
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def abi_version():
    return _lib.bitlinear_abi_version()


def strerror(status):
    return _lib.bitlinear_strerror(status).decode()


# ---- host ------------------------------------------------------------------------

def bitlinear_pack(t, packed=None):
    """numpy int8 t[n][k] -> numpy uint8 packed[n][k/4] (TQ2_0)."""
    n, k = t.shape
    if packed is None:
        packed = np.empty((n, max(k // 4, 0)), np.uint8)
    _check(_lib.bitlinear_pack(_host(t, np.int8, "t"), n, k, _host(packed, np.uint8, "packed")), "bitlinear_pack")
    return packed


def bitlinear_weight_quant(w):
    """numpy fp32 W[n][k] -> (int8 t[n][k], float s_w)."""
    n, k = w.shape
    t = np.empty((n, k), np.int8)
    s = np.zeros(1, np.float32)
    _check(_lib.bitlinear_weight_quant(_host(w, np.float32, "w"), n, k, t.ctypes.data, s.ctypes.data),
           "bitlinear_weight_quant")
    return t, np.float32(s[0])


# ---- device ------------------------------------------------------------------------

def bitlinear_quant_act(x, gain, eps, q, act_scale, act_sum, stream=None):
    """[RMSNorm +] activation quant of x[m][k] (fp32, GPU) into q, act_scale, act_sum."""
    m, k = x.shape
    _check(_lib.bitlinear_quant_act(_dev(x, torch.float32, "x"), _dev(gain, torch.float32, "gain", True), eps, m, k,
                                    _dev(q, torch.int8, "q"), _dev(act_scale, torch.float32, "act_scale"),
                                    _dev(act_sum, torch.int32, "act_sum", True), _stream(stream)),
           "bitlinear_quant_act")


def bitlinear_gemv(packed, w_scale, n, k, q, act_scale, act_sum, m, residual, y, acc_out=None, stream=None):
    _check(_lib.bitlinear_gemv(_dev(packed, torch.uint8, "packed"), float(w_scale), n, k, _dev(q, torch.int8, "q"),
                               _dev(act_scale, torch.float32, "act_scale"), _dev(act_sum, torch.int32, "act_sum"), m,
                               _dev(residual, torch.float32, "residual", True), _dev(y, torch.float32, "y"),
                               _dev(acc_out, torch.int32, "acc_out", True), _stream(stream)), "bitlinear_gemv")


def bitlinear_forward(x, gain, eps, packed, w_scale, n, q, act_scale, act_sum, y, stream=None):
    """[RMSNorm +] quant + GEMV of x[m][k] (fp32, GPU) into y[m][n]; q, act_scale, act_sum receive the quant."""
    m, k = x.shape
    _check(_lib.bitlinear_forward(_dev(x, torch.float32, "x"), _dev(gain, torch.float32, "gain", True), eps,
                                  _dev(packed, torch.uint8, "packed"), float(w_scale), n, k, m,
                                  _dev(q, torch.int8, "q"), _dev(act_scale, torch.float32, "act_scale"),
                                  _dev(act_sum, torch.int32, "act_sum"), _dev(y, torch.float32, "y"),
                                  _stream(stream)), "bitlinear_forward")


def bitlinear_gemm_workspace_bytes(m, n, k, with_argmax):
    return _lib.bitlinear_gemm_workspace_bytes(m, n, k, int(bool(with_argmax)))


def bitlinear_gemm(packed, w_scale, n, k, q, act_scale, act_sum, m, residual, y, acc_out=None, row_argmax=None,
                   workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.bitlinear_gemm(_dev(packed, torch.uint8, "packed"), float(w_scale), n, k, _dev(q, torch.int8, "q"),
                               _dev(act_scale, torch.float32, "act_scale"), _dev(act_sum, torch.int32, "act_sum"), m,
                               _dev(residual, torch.float32, "residual", True),
                               _dev(y, torch.float32, "y", True), _dev(acc_out, torch.int32, "acc_out", True),
                               _dev(row_argmax, torch.int32, "row_argmax", True),
                               _dev(workspace, None, "workspace", True), ws_bytes, _stream(stream)), "bitlinear_gemm")


def bitlinear_gemm_noalloc(packed, w_scale, n, k, q, act_scale, act_sum, m, residual, y, acc_out=None,
                           row_argmax=None, stream=None):
    """bitlinear_gemm with the argmax keys in the library's static device array (no workspace)."""
    _check(_lib.bitlinear_gemm_noalloc(_dev(packed, torch.uint8, "packed"), float(w_scale), n, k,
                                       _dev(q, torch.int8, "q"), _dev(act_scale, torch.float32, "act_scale"),
                                       _dev(act_sum, torch.int32, "act_sum"), m,
                                       _dev(residual, torch.float32, "residual", True),
                                       _dev(y, torch.float32, "y", True), _dev(acc_out, torch.int32, "acc_out", True),
                                       _dev(row_argmax, torch.int32, "row_argmax", True), _stream(stream)),
           "bitlinear_gemm_noalloc")


def bitlinear_gemm_noalloc_max_scratch_bytes():
    return _lib.bitlinear_gemm_noalloc_max_scratch_bytes()


def bitnet_ffn_workspace_bytes(m, d, f):
    return _lib.bitnet_ffn_workspace_bytes(m, d, f)


def bitnet_ffn_workspace_offset(m, d, f, segment):
    if isinstance(segment, str):
        segment = FFN_WS_SEGMENTS.index(segment)
    return _lib.bitnet_ffn_workspace_offset(m, d, f, segment)


def bitnet_ffn(x, m, d, f, norm_gain, sub_norm_gain, eps, w_gate, s_gate, w_up, s_up, w_down, s_down, residual, out,
               workspace, flags=0, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.bitnet_ffn(_dev(x, torch.float32, "x"), m, d, f, _dev(norm_gain, torch.float32, "norm_gain"),
                           _dev(sub_norm_gain, torch.float32, "sub_norm_gain"), eps,
                           _dev(w_gate, torch.uint8, "w_gate"), float(s_gate), _dev(w_up, torch.uint8, "w_up"),
                           float(s_up), _dev(w_down, torch.uint8, "w_down"), float(s_down),
                           _dev(residual, torch.float32, "residual", True), _dev(out, torch.float32, "out"),
                           _dev(workspace, None, "workspace"), ws_bytes, int(flags), _stream(stream)), "bitnet_ffn")


def bitnet_layer_bytes(d, f):
    return _lib.bitnet_layer_bytes(d, f)


def bitnet_stream_workspace_bytes(m, d, f):
    return _lib.bitnet_stream_workspace_bytes(m, d, f)


def bitnet_decode_stream(weights, scales, gains, z, n_layers, m, d, f, eps, x, qkv, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.bitnet_decode_stream(_dev(weights, torch.uint8, "weights"), _dev(scales, torch.float32, "scales"),
                                     _dev(gains, torch.float32, "gains"), _dev(z, torch.float32, "z"), n_layers, m,
                                     d, f, eps, _dev(x, torch.float32, "x"), _dev(qkv, torch.float32, "qkv", True),
                                     _dev(workspace, None, "workspace"), ws_bytes, _stream(stream)),
           "bitnet_decode_stream")


def ffn_workspace_view(workspace, m, d, f, segment):
    """A typed view of one FFN workspace segment (for inspecting intermediates)."""
    shapes = {"q1": ((m, d), torch.int8), "s1": ((m,), torch.float32), "qs1": ((m,), torch.int32),
              "h": ((m, f), torch.float32), "q2": ((m, f), torch.int8), "s2": ((m,), torch.float32),
              "qs2": ((m,), torch.int32), "acc_gate": ((m, f), torch.int32), "acc_up": ((m, f), torch.int32),
              "acc_down": ((m, d), torch.int32), "gate": ((m, f), torch.float32), "up": ((m, f), torch.float32)}
    if segment in ("gate", "up"):
        raise ValueError(f"workspace segment {segment!r} is reserved and empty")
    shape, dtype = shapes[segment]
    off = bitnet_ffn_workspace_offset(m, d, f, segment)
    nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    return workspace[off:off + nbytes].view(dtype).view(shape)


# ---- decode step with attention ---------------------------------------------------------

def bitnet_rope_table(base, head_dim, max_pos):
    """Host: (cos, sin) numpy fp32 [max_pos][head_dim/2] of the rotary embedding."""
    c = np.empty((max_pos, head_dim // 2), np.float32)
    s = np.empty((max_pos, head_dim // 2), np.float32)
    _check(_lib.bitnet_rope_table(float(base), head_dim, max_pos, c.ctypes.data, s.ctypes.data), "bitnet_rope_table")
    return c, s


def bitnet_decode_step_workspace_bytes(m, d, f, n_heads, max_seq):
    return _lib.bitnet_decode_step_workspace_bytes(m, d, f, n_heads, max_seq)


def bitnet_decode_step(weights, scales, gains, n_layers, m, d, f, n_heads, eps, rope_cos, rope_sin, pos, k_cache,
                       v_cache, x, qkv, attn, workspace, stream=None):
    max_seq = rope_cos.shape[0]
    _check(_lib.bitnet_decode_step(_dev(weights, torch.uint8, "weights"), _dev(scales, torch.float32, "scales"),
                                   _dev(gains, torch.float32, "gains"), n_layers, m, d, f, n_heads, eps,
                                   _dev(rope_cos, torch.float32, "rope_cos"), _dev(rope_sin, torch.float32, "rope_sin"),
                                   max_seq, pos, _dev(k_cache, torch.float32, "k_cache"),
                                   _dev(v_cache, torch.float32, "v_cache"), _dev(x, torch.float32, "x"),
                                   _dev(qkv, torch.float32, "qkv", True), _dev(attn, torch.float32, "attn", True),
                                   _dev(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "bitnet_decode_step")


# ---- greedy decoding ------------------------------------------------------------------

def bitnet_embed(table, s_emb, tokens, x, stream=None):
    """x[r] = ternary embedding row tokens[r] / s_emb (table packed [vocab][d/4])."""
    vocab = table.shape[0]
    m, d = x.shape
    _check(_lib.bitnet_embed(_dev(table, torch.uint8, "table"), float(s_emb), vocab, d,
                             _dev(tokens, torch.int32, "tokens"), m, _dev(x, torch.float32, "x"), _stream(stream)),
           "bitnet_embed")


def bitnet_greedy_head_workspace_bytes(m, n):
    return _lib.bitnet_greedy_head_workspace_bytes(m, n)


def _hist_args(hist, hist_len):
    if hist is None:
        return None, 0, None
    return _dev(hist, torch.int32, "hist"), hist.shape[1], _dev(hist_len, torch.int32, "hist_len")


def bitnet_greedy_head(head, s_head, n, k, q, act_scale, act_sum, m, hist, hist_len, penalty, logits, next_token,
                       workspace, stream=None):
    h, stride, hl = _hist_args(hist, hist_len)
    _check(_lib.bitnet_greedy_head(_dev(head, torch.uint8, "head"), float(s_head), n, k, _dev(q, torch.int8, "q"),
                                   _dev(act_scale, torch.float32, "act_scale"), _dev(act_sum, torch.int32, "act_sum"),
                                   m, h, stride, hl, float(penalty), _dev(logits, torch.float32, "logits", True),
                                   _dev(next_token, torch.int32, "next_token"), _dev(workspace, None, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "bitnet_greedy_head")


def bitnet_greedy_step_workspace_bytes(m, d, f, vocab):
    return _lib.bitnet_greedy_step_workspace_bytes(m, d, f, vocab)


def bitnet_greedy_step(embed_table, s_emb, weights, scales, gains, z, n_layers, d, f, eps, g_final, head, s_head,
                       tokens, hist, hist_len, penalty, x, logits, workspace, stream=None):
    vocab = embed_table.shape[0]
    m = tokens.numel()
    h, stride, hl = _hist_args(hist, hist_len)
    _check(_lib.bitnet_greedy_step(_dev(embed_table, torch.uint8, "embed_table"), float(s_emb), vocab,
                                   _dev(weights, torch.uint8, "weights"), _dev(scales, torch.float32, "scales"),
                                   _dev(gains, torch.float32, "gains"), _dev(z, torch.float32, "z"), n_layers, d, f,
                                   eps, _dev(g_final, torch.float32, "g_final"), _dev(head, torch.uint8, "head"),
                                   float(s_head), _dev(tokens, torch.int32, "tokens"), m, h, stride, hl,
                                   float(penalty), _dev(x, torch.float32, "x"),
                                   _dev(logits, torch.float32, "logits", True), _dev(workspace, None, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "bitnet_greedy_step")


# ---- top-k / nucleus sampling ----------------------------------------------------------

def bitnet_sample_workspace_bytes(m, n):
    return _lib.bitnet_sample_workspace_bytes(m, n)


def bitnet_sample_topk(logits, k, temperature, u, token, workspace, stream=None):
    """Top-k sampling of each row of logits[m][n] with its uniform u[r] (fp64) in [0, 1)."""
    m, n = logits.shape
    _check(_lib.bitnet_sample_topk(_dev(logits, torch.float32, "logits"), m, n, int(k), float(temperature),
                                   _dev(u, torch.float64, "u"), _dev(token, torch.int32, "token"),
                                   _dev(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "bitnet_sample_topk")


def bitnet_sample_topp(logits, p, temperature, u, token, workspace, stream=None):
    """Nucleus (top-p) sampling of each row of logits[m][n] with its uniform u[r] (fp64) in [0, 1)."""
    m, n = logits.shape
    _check(_lib.bitnet_sample_topp(_dev(logits, torch.float32, "logits"), m, n, float(p), float(temperature),
                                   _dev(u, torch.float64, "u"), _dev(token, torch.int32, "token"),
                                   _dev(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "bitnet_sample_topp")


# ---- roofline probes (measurement tools) -----------------------------------------------

def bitlinear_probe_read(buf, sink, stream=None):
    """Read every byte of the GPU tensor buf once (the HBM read-stream probe)."""
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.bitlinear_probe_read(_dev(buf, None, "buf"), nbytes, _dev(sink, torch.int32, "sink"),
                                     _stream(stream)), "bitlinear_probe_read")
    return nbytes


def bitlinear_probe_mfma_i8(iters, sink, stream=None):
    """int8 MFMA-only probe; returns the int8 operations of the call."""
    _check(_lib.bitlinear_probe_mfma_i8(int(iters), _dev(sink, torch.int32, "sink"), _stream(stream)),
           "bitlinear_probe_mfma_i8")
    return _lib.bitlinear_probe_mfma_ops(int(iters))


def bitlinear_probe_mfma_i8_dense(iters, sink, stream=None):
    """int8 MFMA-only probe on random-looking, changing operands; returns the int8 operations of the call."""
    _check(_lib.bitlinear_probe_mfma_i8_dense(int(iters), _dev(sink, torch.int32, "sink"), _stream(stream)),
           "bitlinear_probe_mfma_i8_dense")
    return _lib.bitlinear_probe_mfma_ops(int(iters))
