/*
 * bitlinear.h -- C ABI of the BitNet b1.58 BitLinear hot path on MI355X (gfx950).
 *
 * A BitLinear multiplies ternary weights t in {-1, 0, +1} by 8-bit activations:
 *   - weights are stored 2-bit packed, four per byte (the TQ2_0 size of 0.25 byte
 *     per weight: "BitNet Model - Complete Inference Pipeline", Hesper API,
 *     section "Memory Footprint (BitNet-3B with TQ2_0)"), with one fp32 scale
 *     s_w = 1/mean|W| per tensor (the weight_quant of "Add Support for BitNet
 *     Architecture Inference", candle PR 2664);
 *   - activations are quantized per token: an optional RMSNorm (the same PR puts
 *     one in front of every BitLinear), then absmax scaling to 127, rounding and
 *     clamping to int8 (its activation_quant);
 *   - the product is accumulated exactly in int32 and rescaled once in fp32 by
 *     1/(s_a * s_w).
 * The FFN entry point follows "Transformer Block" (Hesper API,
 * Layers.TransformerBlock), sections "Feed-Forward Network (FFN)" and
 * "Forward Pass" steps 4-8, with the ffnSubNorm of "Layer Structure".
 *
 * Layouts (row-major, no padding):
 *   W       : t[n][k], n = output features, k = input features (k contiguous).
 *   packed  : uint8 [n][k/4]; byte i of row r holds weights k = 4i..4i+3 as
 *             2-bit codes c = t + 1 in {0, 1, 2}, least significant field first
 *             (field j at bits 2j..2j+1). Code 3 never appears.
 *   x, y    : fp32 [m][k] / [m][n], one row per token.
 *   q       : int8 [m][k]; act_scale fp32 [m] (= 127/absmax of the normed row);
 *   act_sum : int32 [m], the sum of the row's q (the kernels use it: they
 *             multiply codes c = t + 1 and subtract act_sum).
 *
 * Numerics (identical on every entry point):
 *   RMSNorm  ss = fp64 sum of x^2 in one fixed order: 512 strided partials
 *            (partial l sums x[i]^2 for i = l, l + 512, l + 1024, ... in
 *            ascending i), then an xor-butterfly over the 512 partials with
 *            offsets 1, 2, 4, ..., 256 in that ascending order (at each offset
 *            every partial l becomes p[l] + p[l ^ offset]); ss = p[0].
 *            Then, each step rounded in fp64: w = 1 / sqrt(ss / k + eps),
 *            r = fl32(w); y = fl32(fl32(x * r) * g).
 *   quant    s_a = fl32(127 / max(absmax(y), 1e-5)); q = clamp(rne(fl32(y*s_a)),
 *            -128, 127) with round-half-to-even.
 *   dequant  p = fl32(s_a * s_w); inv = fl32(1 / p); y = fl32((float)acc * inv);
 *            with a residual: y = fl32(residual + fl32((float)acc * inv)).
 *   FFN      g = max(gate, 0); h = fl32(fl32(g * g) * up).
 *   Every fp32 / fp64 operation above rounds on its own (no fused multiply-add),
 *   and division and square root are correctly rounded.
 *
 * Conventions:
 *   - Every pointer marked "device" is caller-owned device memory (for example
 *     a torch tensor's data pointer). The library never allocates, frees or
 *     retains memory, never synchronises, and never reads device memory on the
 *     host. Host pointers are read/written only during the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Device
 *     calls are asynchronous on it and may be captured into a HIP graph; the
 *     pointers must then stay valid for the life of the graph.
 *   - Status codes: 0 = BL_OK, negative = error. All argument checks happen on
 *     the host before any launch; on an error nothing is launched or written.
 *     A kernel launch failure returns BL_ERR_LAUNCH; faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   - Device calls need k % 64 == 0 (packed rows are whole 16-byte chunks),
 *     16-byte aligned packed/q pointers and 4-byte aligned fp32/int32 pointers.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BL_OK 0
#define BL_ERR_NULL (-1)      /* a required pointer is NULL */
#define BL_ERR_SHAPE (-2)     /* a size is <= 0, not a multiple of what the call needs, or too large */
#define BL_ERR_ALIGN (-3)     /* a pointer is not aligned as stated above */
#define BL_ERR_VALUE (-4)     /* a value is out of range (a weight outside {-1,0,1}, a non-finite input) */
#define BL_ERR_WORKSPACE (-5) /* the workspace is smaller than the matching *_workspace_bytes() */
#define BL_ERR_LAUNCH (-6)    /* a kernel launch failed (hipGetLastError after the launch) */
#define BL_ERR_DEVICE (-7)    /* no usable gfx950 device, or a HIP runtime call failed */

/* ABI version of this header (bumped on any incompatible change). */
int bitlinear_abi_version(void);

/* Static text for a status code (never NULL). */
const char *bitlinear_strerror(int status);

/* ---------------------------------------------------------------- host --- */

/* Ternary packer (TQ2_0, layout above). Host memory only.
 *   t      : host int8 [n][k], every value in {-1, 0, 1}.
 *   packed : host uint8 [n][k/4], written in full on success.
 * Errors: BL_ERR_NULL; BL_ERR_SHAPE if n <= 0, k <= 0 or k % 4 != 0;
 *         BL_ERR_VALUE if any t is outside {-1, 0, 1} (nothing is written). */
int bitlinear_pack(const int8_t *t, int64_t n, int64_t k, uint8_t *packed);

/* weight_quant of the b1.58 method on the host: s_w = fl32(1 / max(mean|W|, 1e-5))
 * with mean|W| an fp64 sum in row-major order over n*k, then
 * t = clamp(rne(fl32(W * s_w)), -1, 1).
 *   w : host fp32 [n][k]; t : host int8 [n][k]; w_scale : host fp32 [1].
 * Errors: BL_ERR_NULL; BL_ERR_SHAPE (n, k <= 0); BL_ERR_VALUE (non-finite W). */
int bitlinear_weight_quant(const float *w, int64_t n, int64_t k, int8_t *t, float *w_scale);

/* -------------------------------------------------------------- device --- */

/* [RMSNorm(gain, eps) +] per-token absmax activation quant.
 *   x         : device fp32 [m][k].
 *   gain      : device fp32 [k], or NULL for no RMSNorm (q quantizes x itself).
 *   eps       : RMSNorm epsilon (ignored when gain is NULL), widened to fp64.
 *   q         : device int8 [m][k]; act_scale : device fp32 [m];
 *   act_sum   : device int32 [m] or NULL.
 * Launch forms (results are identical): from 256 tokens on, one wave per token
 * with the row in registers (k <= 4096 with a gain, k <= 8192 without); else
 * one 512-thread workgroup per token, the row in registers up to k = 16384 and
 * read three times (sum of squares, absmax, codes) above that.
 * Errors: NULL, SHAPE (m, k <= 0, k % 64 != 0), ALIGN, LAUNCH. Non-finite x is
 * out of contract (results unspecified). */
int bitlinear_quant_act(const float *x, const float *gain, float eps, int64_t m, int64_t k,
                        int8_t *q, float *act_scale, int32_t *act_sum, void *stream);

/* Decode GEMV, m in [1, 8]: y[m][n] = [residual +] dequant(P . q). At decode
 * the time goes into the layers' BitLinear weights ("BitNet Model - Complete
 * Inference Pipeline", Hesper API, section "Performance (BitNet-3B on A100)";
 * the per-layer weights of "Transformer Block", section "Memory Layout"), so
 * this product is a stream of the packed weights.
 *   packed    : device uint8 [n][k/4], 16-byte aligned.
 *   w_scale   : the tensor's s_w (> 0).
 *   q, act_scale, act_sum : from bitlinear_quant_act (act_sum is required).
 *   residual  : device fp32 [m][n] or NULL; may alias y.
 *   y         : device fp32 [m][n].
 *   acc_out   : device int32 [m][n] (the exact accumulators) or NULL.
 * Streams the packed weights with 16-byte loads; codes are unpacked in
 * registers and multiplied with 4-way int8 dot products, reduced across lanes.
 * Errors: NULL, SHAPE (m outside [1, 8], n <= 0, k % 64 != 0, k > 32768),
 * ALIGN, VALUE (w_scale not > 0), LAUNCH. */
int bitlinear_gemv(const uint8_t *packed, float w_scale, int64_t n, int64_t k,
                   const int8_t *q, const float *act_scale, const int32_t *act_sum, int64_t m,
                   const float *residual, float *y, int32_t *acc_out, void *stream);

/* Decode BitLinear in one call, m in [1, 8]: y[m][n] = dequant(P . quant([RMSNorm](x))),
 * the composition of bitlinear_quant_act and bitlinear_gemv (no residual), with the same
 * results bit for bit. A BitLinear applied to a token: the layer of the pages'
 * "BitLinear" ("Add Support for BitNet Architecture Inference", candle PR 2664: an
 * RMSNorm before the BitLinear, activation_quant, ternary matmul, one rescale; and
 * "Transformer Block", Hesper API, section "Forward Pass").
 *   x, gain, eps : as bitlinear_quant_act (x [m][k], gain [k] or NULL).
 *   packed, w_scale, n, k : as bitlinear_gemv.
 *   q, act_scale, act_sum : device int8 [m][k], fp32 [m], int32 [m], caller-allocated; they
 *               receive the quantized activations exactly as bitlinear_quant_act writes them.
 *   y         : device fp32 [m][n].
 * For m == 1 and k <= 16384 this is one launch: every workgroup quantizes x itself (the
 * same operations in the same order as the quant kernel; one wave per workgroup up to
 * k = 4096, 512 threads above) and then runs its weight rows, so the quant adds no launch
 * and no round trip through memory. Otherwise the quant launch also pulls P into the
 * memory-side cache for the GEMV launch that follows it.
 * Errors: NULL, SHAPE (m outside [1, 8], n <= 0, k % 64 != 0, k > 32768), ALIGN (x, gain,
 * packed, q 16-byte; act_scale, act_sum, y 4-byte), VALUE (w_scale not > 0), LAUNCH. */
int bitlinear_forward(const float *x, const float *gain, float eps, const uint8_t *packed, float w_scale,
                      int64_t n, int64_t k, int64_t m, int8_t *q, float *act_scale, int32_t *act_sum,
                      float *y, void *stream);

/* Workspace bytes bitlinear_gemm needs (0 unless a per-row argmax is asked for):
 * 8 bytes per token and 32-column tile for m <= 32, 8 bytes per token above. */
size_t bitlinear_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int with_argmax);

/* GEMM on int8 matrix cores (prefill, batched decode, ternary LM head):
 * y[m][n] = [residual +] dequant(q . P^T), optional fused per-row argmax.
 * The prefill product is the "Tiled matmul" step of "BitNet Model - Complete
 * Inference Pipeline" (section "Performance (BitNet-3B on A100)", "With
 * optimizations"); the LM head projects to the vocabulary ("Architecture"), and
 * row_argmax is the greedy choice of "Text Generation / Greedy Decoding" done
 * on the device as the page's "GPU Argmax" does (argmaxKernel, gpuArgmax: only
 * the index comes back).
 *   packed, w_scale, q, act_scale, act_sum : as bitlinear_gemv; any m >= 1.
 *   residual   : device fp32 [m][n] or NULL (may alias y).
 *   y          : device fp32 [m][n], or NULL when row_argmax is given (logits
 *                are then not written).
 *   acc_out    : device int32 [m][n] or NULL.
 *   row_argmax : device int32 [m] or NULL: per row, the lowest n holding the
 *                largest accumulator (the same as the first argmax of y, since
 *                the rescale is monotone and exact on distinct integers).
 *   workspace  : device memory of bitlinear_gemm_workspace_bytes(m, n, k, 1)
 *                bytes (8-byte aligned) when row_argmax is given, else unused.
 * m <= 32: every token is a row of one v_mfma_i32_32x32x32_i8 A tile, K is
 * split across the waves of a workgroup, and the argmax goes through one key
 * per token and 32-column tile in the workspace plus a reduction kernel.
 * m > 32: block tiles staged in LDS (ternary tiles unpacked in registers from
 * a packed LDS tile) on v_mfma_i32_16x16x64_i8 / 32x32x32_i8, argmax by a
 * 64-bit atomicMax key per row. Results are identical either way.
 * Errors: NULL (y and row_argmax both NULL, ...), SHAPE, ALIGN, VALUE,
 * WORKSPACE, LAUNCH. */
int bitlinear_gemm(const uint8_t *packed, float w_scale, int64_t n, int64_t k,
                   const int8_t *q, const float *act_scale, const int32_t *act_sum, int64_t m,
                   const float *residual, float *y, int32_t *acc_out, int32_t *row_argmax,
                   void *workspace, size_t workspace_bytes, void *stream);

/* bitlinear_gemm for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same computation and results as bitlinear_gemm, but the argmax keys live
 * in a library-owned static device array of
 * bitlinear_gemm_noalloc_max_scratch_bytes() bytes (1 MiB) instead of a
 * workspace argument; each GPU the library runs on holds its own copy of the
 * array until the process ends. The call allocates and frees nothing; on its
 * first use on a GPU it looks up that GPU's copy (hipGetSymbolAddress).
 *   Arguments : as bitlinear_gemm, without workspace / workspace_bytes.
 *   Limit     : with row_argmax, bitlinear_gemm_workspace_bytes(m, n, k, 1)
 *               must not exceed the array (m <= 32: m * ceil(n / 32) * 8 bytes,
 *               e.g. 32 tokens x 50000 columns = 400,128 B; m > 32: 8 bytes per
 *               token); larger requests fail with BL_ERR_WORKSPACE before any
 *               device call. Without row_argmax the array is not used.
 * Every call on one GPU shares that GPU's array, so calls that overlap in time
 * on one GPU (different streams, or concurrent host threads) race on it and
 * must be serialised by the caller. The array keeps the last call's contents;
 * each call writes every key it reads, so nothing needs clearing between calls.
 * Errors: as bitlinear_gemm; BL_ERR_DEVICE if the array cannot be located. */
size_t bitlinear_gemm_noalloc_max_scratch_bytes(void);
int bitlinear_gemm_noalloc(const uint8_t *packed, float w_scale, int64_t n, int64_t k,
                           const int8_t *q, const float *act_scale, const int32_t *act_sum, int64_t m,
                           const float *residual, float *y, int32_t *acc_out, int32_t *row_argmax,
                           void *stream);

/* BitNet FFN sub-layer without the residual of the block (pass `residual` to
 * add one):
 *   q1  = quant(rmsnorm(x, norm_gain))                       [m][d]
 *   gate, up = dequant(W_gate . q1), dequant(W_up . q1)       [m][f]
 *   h   = relu(gate)^2 * up                                   [m][f]
 *   q2  = quant(rmsnorm(h, sub_norm_gain))                    [m][f]
 *   out = [residual +] dequant(W_down . q2)                   [m][d]
 *   x           : device fp32 [m][d].
 *   norm_gain   : device fp32 [d];  sub_norm_gain : device fp32 [f].
 *   w_gate, w_up: device packed [f][d/4];  w_down : device packed [d][f/4].
 *   s_gate, s_up, s_down : weight scales.
 *   residual    : device fp32 [m][d] or NULL (may alias out).
 *   out         : device fp32 [m][d].
 *   workspace   : device, >= bitnet_ffn_workspace_bytes(m, d, f), 256-byte
 *                 aligned; holds every intermediate at the offsets given by
 *                 bitnet_ffn_workspace_offset().
 *   flags       : BITNET_FFN_WRITE_ACC also stores acc_gate, acc_up, acc_down.
 * gate and up always run in one launch that streams both weight matrices and
 * applies relu(gate)^2 * up in its epilogue: a GEMV for m <= 8, a skinny MFMA
 * product for m <= 32, and above that an MFMA GEMM whose B tiles interleave
 * W_gate and W_up rows, so gate and up of a column meet in one wave. At m == 1 (d <= 4096, and
 * 4096 < f <= 16384 for the second half) each norm + quant runs inside the
 * launch of the product it feeds, so the FFN is two launches; the workspace
 * still receives q1, s1, qs1, h, q2, s2, qs2. Up to 32 tokens each norm + quant
 * launch also pulls the next product's weights into the memory-side cache. d and f must be
 * multiples of 64. Errors: NULL, SHAPE, ALIGN, VALUE, WORKSPACE, LAUNCH. */
#define BITNET_FFN_WRITE_ACC 1
enum bitnet_ffn_ws_segment {
    BITNET_FFN_WS_Q1 = 0,    /* int8  [m][d] */
    BITNET_FFN_WS_S1,        /* fp32  [m]    */
    BITNET_FFN_WS_QS1,       /* int32 [m]    */
    BITNET_FFN_WS_H,         /* fp32  [m][f] */
    BITNET_FFN_WS_Q2,        /* int8  [m][f] */
    BITNET_FFN_WS_S2,        /* fp32  [m]    */
    BITNET_FFN_WS_QS2,       /* int32 [m]    */
    BITNET_FFN_WS_ACC_GATE,  /* int32 [m][f] (with BITNET_FFN_WRITE_ACC) */
    BITNET_FFN_WS_ACC_UP,    /* int32 [m][f] (with BITNET_FFN_WRITE_ACC) */
    BITNET_FFN_WS_ACC_DOWN,  /* int32 [m][d] (with BITNET_FFN_WRITE_ACC) */
    BITNET_FFN_WS_GATE,      /* reserved, 0 bytes (gate is never stored on its own) */
    BITNET_FFN_WS_UP,        /* reserved, 0 bytes (up is never stored on its own) */
    BITNET_FFN_WS_COUNT
};
size_t bitnet_ffn_workspace_bytes(int64_t m, int64_t d, int64_t f);
/* Byte offset of a segment inside the FFN workspace; (size_t)-1 for a bad segment. */
size_t bitnet_ffn_workspace_offset(int64_t m, int64_t d, int64_t f, int segment);
int bitnet_ffn(const float *x, int64_t m, int64_t d, int64_t f,
               const float *norm_gain, const float *sub_norm_gain, float eps,
               const uint8_t *w_gate, float s_gate, const uint8_t *w_up, float s_up,
               const uint8_t *w_down, float s_down,
               const float *residual, float *out, void *workspace, size_t workspace_bytes,
               int flags, void *stream);

/* Decoder-layer stream of BitLinears with attention math left out: for each
 * layer l in order ("Transformer Block", "Forward Pass"; "Memory Layout" for
 * the seven projections):
 *   a      = quant(rmsnorm(x, g_attn))
 *   q,k,v  = dequant(W_q . a), dequant(W_k . a), dequant(W_v . a)  -> qkv[l]
 *   o_in   = quant(rmsnorm(z[l], g_attn_sub))   (z: stand-in for attention)
 *   x      = x + dequant(W_o . o_in)
 *   x      = x + ffn(x)                         (as bitnet_ffn)
 * The projections run in that order, each after the one before it.
 *   weights : device, n_layers consecutive layer blobs of bitnet_layer_bytes(d, f)
 *             bytes; inside a blob the packed tensors W_q, W_k, W_v, W_o
 *             ([d][d/4] each), W_gate, W_up ([f][d/4] each), W_down ([d][f/4])
 *             follow each other with no gap.
 *   scales  : device fp32 [n_layers][7] (q, k, v, o, gate, up, down).
 *   gains   : device fp32 [n_layers][3d + f]: g_attn, g_attn_sub, g_ffn ([d]
 *             each), g_ffn_sub ([f]).
 *   z       : device fp32 [n_layers][m][d].
 *   x       : device fp32 [m][d], updated in place.
 *   qkv     : device fp32 [n_layers][m][3d] or NULL (then written to the
 *             workspace and overwritten layer by layer).
 *   workspace: device, >= bitnet_stream_workspace_bytes(m, d, f), 256-aligned,
 *             zero-filled before its first use and then kept between calls:
 *             its first 8 bytes are two uint32 words {phase counter, status}.
 * d and f must be multiples of 64; m >= 1.
 * At m == 1, for the compiled shapes (d, f) = (2560, 10240), (2048, 8192) and
 * (256, 1024) on a device with at least 256 CUs that each fit one of its
 * workgroups, the whole stream runs as one persistent kernel of 256
 * workgroups, all resident at once, that hands each step's output vector to
 * the next step through flag-tagged words in the workspace. It needs the CUs
 * to itself: work running at the same time on other streams can keep a
 * workgroup from becoming resident, and the call then ends by timeout.
 * Every wait in it is bounded (2 s from the start of that wait, so the bound
 * does not grow with n_layers); on a timeout the kernel stops early and
 * sets status = 1 (status = 2: the phase counter is exhausted after about 2^31
 * steps). A nonzero status stays set, and further calls do nothing, until the
 * workspace is zero-filled again; the caller reads it after synchronising.
 * Calls that share a workspace must not overlap. Other shapes, and any call
 * made while the stream is being captured into a graph, run one launch per
 * step (at 9..32 tokens one MFMA launch per projection, q/k/v together and
 * gate/up fused), with the same results.
 * Errors: NULL, SHAPE, ALIGN, WORKSPACE, LAUNCH. */
size_t bitnet_layer_bytes(int64_t d, int64_t f);
size_t bitnet_stream_workspace_bytes(int64_t m, int64_t d, int64_t f);
int bitnet_decode_stream(const uint8_t *weights, const float *scales, const float *gains, const float *z,
                         int64_t n_layers, int64_t m, int64_t d, int64_t f, float eps,
                         float *x, float *qkv, void *workspace, size_t workspace_bytes, void *stream);

/* -------------------------------------------- decode step with attention --- */
/* The decoder layer stream of bitnet_decode_stream with real single-token
 * attention in place of the stand-in z ("BitNet Model - Complete Inference
 * Pipeline": "KV Cache State", forwardSingleToken; "Transformer Block":
 * "Forward Pass with KV Cache", forwardWithCache; Config: numHeads, headDim,
 * ropeBase). m sequences, each with its own cache, at the same position pos.
 * For each layer l:
 *   a      = quant(rmsnorm(x, g_attn));  q, k, v = dequant(W . a)  -> qkv[l]
 *   heads  : head h owns columns h hd .. h hd + hd - 1, hd = d / n_heads;
 *   RoPE   : in every head of q and k the pairs (x[2i], x[2i+1]) turn by the
 *            angle pos * theta_i with the table row pos: (a, b) ->
 *            (fl32(fl32(a c) - fl32(b s)), fl32(fl32(a s) + fl32(b c)));
 *   cache  : the rotated k and v are written at position pos of layer l;
 *   attn   = per head softmax(q . K[0..pos]^T / sqrt(hd)) V[0..pos]   -> attn[l]
 *            (fp32 on the device: scores, expf, sums; not bit-exact, see the
 *            design notes for the bound);
 *   x      = x + dequant(W_o . quant(rmsnorm(attn, g_attn_sub)))
 *   x      = x + ffn(x)
 *   weights, scales, gains, n_layers, m, d, f, eps : as bitnet_decode_stream.
 *   n_heads   : d % n_heads == 0, hd % 4 == 0, hd <= 256.
 *   rope_cos, rope_sin : host-computed tables, device fp32 [max_seq][hd / 2]
 *               (bitnet_rope_table).
 *   k_cache, v_cache : device fp32 [n_layers][m][n_heads][max_seq][hd], 16-byte
 *               aligned; positions 0 .. pos-1 hold earlier steps' entries.
 *   x         : device fp32 [m][d], updated in place.
 *   qkv       : device fp32 [n_layers][m][3d] or NULL (q, k, v before RoPE).
 *   attn      : device fp32 [n_layers][m][d] or NULL (attention outputs).
 *   workspace : bitnet_decode_step_workspace_bytes(m, d, f, n_heads, max_seq)
 *               bytes, 256-aligned, zero-filled before its first use and then
 *               kept between calls (its first 8 bytes are the stream's
 *               {phase counter, status} words).
 * At m == 1, for the persistent kernel's shapes and device (as in
 * bitnet_decode_stream) with n_heads <= 256 and max_seq <= 8192, the whole
 * step is one persistent launch: q, k and v are published like the stream's
 * other vectors, 256 / n_heads workgroups per head split its positions
 * 0 .. pos into chunks (256 positions, or, while that leaves workgroups of
 * the head idle, up to 32 shorter chunks of at least 16), and the head's first
 * workgroup merges the chunks by rescaling (RoPE and the cache append are done
 * by the workgroup holding pos); the o projection waits for the published
 * attention output. Its timeout
 * and status rules are those of bitnet_decode_stream. Otherwise (and while the
 * stream is being captured into a graph) it runs one launch per step: RoPE and
 * append, one workgroup per (sequence, head, 256 positions), a merge launch.
 * Both compute the same fp32 attention arithmetic up to the order of the
 * terms of the scores and of the weighted sums, within the same bound.
 * Errors: NULL, SHAPE (pos outside [0, max_seq), ...), ALIGN, WORKSPACE, LAUNCH. */
size_t bitnet_decode_step_workspace_bytes(int64_t m, int64_t d, int64_t f, int64_t n_heads, int64_t max_seq);
int bitnet_decode_step(const uint8_t *weights, const float *scales, const float *gains, int64_t n_layers,
                       int64_t m, int64_t d, int64_t f, int64_t n_heads, float eps,
                       const float *rope_cos, const float *rope_sin, int64_t max_seq, int64_t pos,
                       float *k_cache, float *v_cache, float *x, float *qkv, float *attn,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Host helper: the rotary-embedding table. theta_i = pow(base, -(2i) / head_dim),
 * angle = pos * theta_i, cos and sin in fp64, each rounded once to fp32.
 *   cos_out, sin_out : host fp32 [max_pos][head_dim / 2].
 * The pages name ropeBase without its value; the usual 10000 is the reading.
 * Errors: NULL, SHAPE (odd or non-positive head_dim, max_pos <= 0), VALUE (base <= 1). */
int bitnet_rope_table(double base, int64_t head_dim, int64_t max_pos, float *cos_out, float *sin_out);

/* ------------------------------------------------------ greedy decoding --- */
/* The device side of greedy text generation around the BitLinear stream
 * ("BitNet Model - Complete Inference Pipeline", Hesper API: "Architecture"
 * -- TQ2_0 embedding, the transformer blocks, final RMSNorm, LM head;
 * "Text Generation / Greedy Decoding"; "GPU Argmax" -- repetitionPenaltyKernel,
 * appendPenaltyToken and gpuArgmaxWithPenalty, whose penalty and argmax run in
 * one submit and return only the token index). */

/* Ternary embedding lookup: x[r][k] = t[tokens[r]][k] / s_emb, with the table
 * packed like any ternary tensor (uint8 [vocab][d/4], layout above) and one
 * fp32 scale. A token id outside [0, vocab) gives a zero row (ids are device
 * data, so they are not checked on the host).
 *   table  : device uint8 [vocab][d/4], 16-byte aligned.
 *   tokens : device int32 [m].  x : device fp32 [m][d], 16-byte aligned.
 * Errors: NULL, SHAPE (d % 64 != 0, d > 32768, vocab or m <= 0), ALIGN,
 * VALUE (s_emb not > 0 or not finite), LAUNCH. */
int bitnet_embed(const uint8_t *table, float s_emb, int64_t vocab, int64_t d, const int32_t *tokens,
                 int64_t m, float *x, void *stream);

/* LM head with repetition penalty and greedy choice, m <= 32 sequences:
 *   logits[r][c] = dequant(P . q[r]) as bitlinear_gemm computes it;
 *   every distinct id v in hist[r][0 .. hist_len[r]) with 0 <= v < n has its
 *   logit l replaced, once, by fl32(l / penalty) if l > 0, else by
 *   fl32(l * penalty) (ids outside [0, n) are ignored, hist_len[r] is clamped
 *   to [0, hist_stride]);
 *   next_token[r] = the lowest c holding the largest penalised logit.
 * It runs as three launches on the stream: the per-sequence penalty bitmaps,
 * the product whose epilogue penalises and forms fp32 argmax keys (no logits
 * need to be written; one sequence: a GEMV, several: the skinny MFMA
 * product), and the per-sequence key reduction.
 *   head, s_head, n, k : the LM head, packed [n][k/4] (n = vocabulary).
 *   q, act_scale, act_sum : the final-norm quant of the hidden states.
 *   hist      : device int32 [m][hist_stride] (NULL when hist_stride == 0);
 *   hist_len  : device int32 [m] (NULL when hist_stride == 0).
 *   penalty   : > 0 and finite; 1 leaves the logits as they are.
 *   logits    : device fp32 [m][n] receiving the penalised logits, or NULL.
 *   next_token: device int32 [m].
 *   workspace : bitnet_greedy_head_workspace_bytes(m, n) bytes, 256-aligned.
 * Errors: NULL, SHAPE (m outside [1, 32], ...), ALIGN, VALUE, WORKSPACE, LAUNCH. */
size_t bitnet_greedy_head_workspace_bytes(int64_t m, int64_t n);
int bitnet_greedy_head(const uint8_t *head, float s_head, int64_t n, int64_t k,
                       const int8_t *q, const float *act_scale, const int32_t *act_sum, int64_t m,
                       const int32_t *hist, int64_t hist_stride, const int32_t *hist_len, float penalty,
                       float *logits, int32_t *next_token, void *workspace, size_t workspace_bytes,
                       void *stream);

/* One greedy decoding step of m <= 32 sequences on the device, with no host
 * synchronisation and no host round trip, in this order on the stream:
 *   x = bitnet_embed(tokens)
 *   x = the layer stream of bitnet_decode_stream over x (stand-in z for attention)
 *   q = quant(rmsnorm(x, g_final))
 *   tokens = bitnet_greedy_head(q, hist, hist_len, penalty)     (in place)
 *   hist[r][hist_len[r]] = tokens[r]; hist_len[r] += 1   (while hist_len < stride)
 * so the next call continues from the chosen tokens; the host reads tokens or
 * hist when it wants them (4 bytes per sequence and step). The embedding
 * launch also builds the penalty bitmaps, and the launch that reduces the
 * head's argmax keys appends the tokens; for one sequence with d <= 4096 the
 * final norm + quant runs inside the head's launch (one workgroup per CU on
 * a block of head rows), so the step is four launches besides the stream's.
 *   embed_table, s_emb, vocab : the embedding ([vocab][d/4]).
 *   weights, scales, gains, z, n_layers, d, f, eps : as bitnet_decode_stream.
 *   g_final   : device fp32 [d];  head, s_head : the LM head ([vocab][d/4]).
 *   tokens    : device int32 [m], the current tokens in, the chosen ones out.
 *   hist, hist_stride, hist_len, penalty : as bitnet_greedy_head (updated).
 *   x         : device fp32 [m][d], receives the final hidden states.
 *   logits    : device fp32 [m][vocab] (penalised) or NULL.
 *   workspace : bitnet_greedy_step_workspace_bytes(m, d, f, vocab) bytes,
 *               256-aligned, zero-filled before its first use and then kept
 *               (it holds the stream's workspace first).
 * Errors: NULL, SHAPE, ALIGN, VALUE, WORKSPACE, LAUNCH. */
size_t bitnet_greedy_step_workspace_bytes(int64_t m, int64_t d, int64_t f, int64_t vocab);
int bitnet_greedy_step(const uint8_t *embed_table, float s_emb, int64_t vocab,
                       const uint8_t *weights, const float *scales, const float *gains, const float *z,
                       int64_t n_layers, int64_t d, int64_t f, float eps,
                       const float *g_final, const uint8_t *head, float s_head,
                       int32_t *tokens, int64_t m, int32_t *hist, int64_t hist_stride, int32_t *hist_len,
                       float penalty, float *x, float *logits, void *workspace, size_t workspace_bytes,
                       void *stream);

/* ------------------------------------------------- top-k / nucleus sampling --- */
/* Sampling of the next token from m rows of n fp32 logits ("BitNet Model -
 * Complete Inference Pipeline", section "Text Generation": Top-k Sampling and
 * Nucleus (Top-p) Sampling; sampleTopK, sampleNucleus). The random numbers are
 * the caller's: u[r] uniform in [0, 1), one per row (device fp64; values
 * outside [0, 1) are clamped into the kept set).
 * Definition (both calls):
 *   - tokens are taken in sorted order: descending logit, the lower index first
 *     among equal logits (-0 and +0 are equal);
 *   - token i weighs w_i = rne(2^40 * E((l_i - l_max) / T)), an exact int64,
 *     with (l_i - l_max) / T one correctly rounded fp64 division and E the
 *     fp64 exponential on [-32, 0] given by: k = rne(x * fl64(1/ln2)),
 *     r = (x - k * H) - k * L (H = 0x1.62e42fee00000p-1, L = 0x1.a39ef35793c76p-33:
 *     ln2 split into a 32-bit head and a tail), e^r = the Taylor series through
 *     r^13 / 13! by Horner's rule, scaled by 2^k; E = 0 below -32. Every fp64
 *     operation rounds on its own;
 *   - top-k keeps the first min(k, n) tokens; top-p keeps the shortest sorted
 *     prefix whose weight reaches max(1, min(Z, ceil(fl64(p * Z)))), Z = the total
 *     weight (the smallest set with probability >= p);
 *   - with M the kept weight and r = min(M - 1, max(0, floor(fl64(u * M)))), the
 *     chosen token is the first kept token whose cumulative weight exceeds r.
 * Three launches on the stream: the row maxima (per slice), the weights and
 * first-level histograms (up to 64 workgroups per row, 256 in all, merged by
 * exact integer atomics), then one 1024-thread workgroup per row for the radix
 * selections over 64-bit (logit, index) keys whose per-digit weight sums are
 * exact integers.
 *   logits    : device fp32 [m][n] (finite), 1 <= n < 2^23 (so the total
 *               weight, at most n 2^40, fits in an int64).
 *   temperature : > 0 and finite.  k >= 1 (k > n keeps all); p > 0 (p >= 1 keeps
 *               every token of nonzero weight).
 *   token     : device int32 [m].
 *   workspace : bitnet_sample_workspace_bytes(m, n) bytes (the weights, slice maxima,
 *               histograms and totals), 256-aligned; no contents carried between calls.
 * Errors: NULL, SHAPE, ALIGN, VALUE, WORKSPACE, LAUNCH. */
size_t bitnet_sample_workspace_bytes(int64_t m, int64_t n);
int bitnet_sample_topk(const float *logits, int64_t m, int64_t n, int64_t k, float temperature, const double *u,
                       int32_t *token, void *workspace, size_t workspace_bytes, void *stream);
int bitnet_sample_topp(const float *logits, int64_t m, int64_t n, float p, float temperature, const double *u,
                       int32_t *token, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------- roofline probes --- */
/* Measurement tools, not part of the method: they give the measured ceilings
 * that throughput is reported against next to the nominal MI355X peaks.
 *
 * bitlinear_probe_read: reads every byte of buf once (16-byte loads, eight in
 * flight per thread, two 1024-thread workgroups per CU) and xors a fold of
 * the data into *sink (device uint32). Bytes read = bytes.
 *   buf : device, 16-byte aligned; bytes : > 0, a multiple of 16.
 * Errors: NULL, SHAPE, ALIGN, DEVICE, LAUNCH. */
int bitlinear_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* bitlinear_probe_mfma_i8: every wave (two per SIMD on every CU) issues
 * iters x 8 independent v_mfma_i32_16x16x64_i8 on register operands and
 * nothing else; *sink (device uint32) is touched only to keep the results
 * alive. The operands are one pair of small values (mostly zero bytes).
 * bitlinear_probe_mfma_i8_dense: the same with each of the 8 chains on its
 * own pair of random-looking operand bytes, so consecutive MFMAs see
 * different, fully toggling operands as a GEMM on real data does (the matrix
 * cores draw more power, and the clock may drop).
 * bitlinear_probe_mfma_ops(iters) is the number of int8 operations (2 per
 * multiply-add) one call of either performs on the current device (0 on error).
 * Errors: NULL, SHAPE (iters <= 0 or > 2^40), ALIGN, DEVICE, LAUNCH. */
int64_t bitlinear_probe_mfma_ops(int64_t iters);
int bitlinear_probe_mfma_i8(int64_t iters, uint32_t *sink, void *stream);
int bitlinear_probe_mfma_i8_dense(int64_t iters, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
