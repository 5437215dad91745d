// api.hip -- the device entry points of the C ABI: argument checks on the host,
// then launches on the caller's stream. No allocation, no synchronisation, no
// host reads of device memory.
#include <algorithm>
#include <mutex>

#include "internal.h"
#include "prefetch.h"

namespace {

using bl::aligned;

constexpr int64_t kMaxGemvM = 8;
constexpr int64_t kMaxSkinnyM = 32;
constexpr int64_t kMaxGemvK = 32768;
constexpr int64_t kMaxDim = (int64_t)1 << 30;

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool dim_ok(int64_t v) { return v > 0 && v <= kMaxDim; }

// k must be a positive multiple of 64 (whole 16-byte packed chunks).
inline bool k_ok(int64_t k) { return dim_ok(k) && (k % 64) == 0; }

struct Layout {
    size_t off[BITNET_FFN_WS_COUNT];
    size_t total;
};

Layout ffn_layout(int64_t m, int64_t d, int64_t f)
{
    // the last two segments (gate, up) are reserved and empty: no path writes
    // gate or up separately any more
    const size_t sz[BITNET_FFN_WS_COUNT] = {
        (size_t)(m * d),     (size_t)m * 4,     (size_t)m * 4, (size_t)(m * f) * 4,
        (size_t)(m * f),     (size_t)m * 4,     (size_t)m * 4, (size_t)(m * f) * 4,
        (size_t)(m * f) * 4, (size_t)(m * d) * 4, 0, 0,
    };
    Layout l{};
    size_t at = 0;
    for (int i = 0; i < BITNET_FFN_WS_COUNT; ++i) {
        l.off[i] = at;
        at = align_up(at + sz[i], 256);
    }
    l.total = at;
    return l;
}

// Stream workspace: control words {epoch, status} and the published vectors of
// the persistent one-token kernel, then a (q, s, qs) for d, o_in for d, the
// FFN workspace, the q/k/v scratch of the launch-per-step path and the K-split
// partial sums of its down product at 9..32 tokens.
struct StreamLayout {
    size_t ctrl, ll, q_a, s_a, qs_a, q_o, s_o, qs_o, ffn, qkv, part, total;
};

constexpr int kMaxKSplit = 4;

// K split of the down product (d rows, K = f) at 9..32 tokens: its d / 32
// tiles alone would occupy a quarter of the CUs at d = 2048, each workgroup
// pulling all 32 x f activation bytes; split so that tiles x parts still fits
// one workgroup per CU and every part is a whole number of 128-input steps.
// (The o product, K = d, gains less from a split than its reducer then costs.)
int batched_ksplit(int64_t d, int64_t f)
{
    const int64_t tiles = (d + 31) / 32;
    if (d > 8192) return 1;  // the reducing quant holds 16 values per thread at most
    for (int ks = kMaxKSplit; ks > 1; ks /= 2)
        if (tiles * ks <= 256 && f % (128 * ks) == 0) return ks;
    return 1;
}

StreamLayout stream_layout(int64_t m, int64_t d, int64_t f)
{
    StreamLayout l{};
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t o = at;
        at = align_up(at + bytes, 256);
        return o;
    };
    l.ctrl = take(256);
    l.ll = take(bl::stream_ll_words((int)d, (int)f) * 8);
    l.q_a = take((size_t)(m * d));
    l.s_a = take((size_t)m * 4);
    l.qs_a = take((size_t)m * 4);
    l.q_o = take((size_t)(m * d));
    l.s_o = take((size_t)m * 4);
    l.qs_o = take((size_t)m * 4);
    l.ffn = take(ffn_layout(m, d, f).total);
    l.qkv = take((size_t)(m * 3 * d) * 4);
    l.part = take((size_t)(kMaxKSplit * m * d) * 4);
    l.total = at;
    return l;
}

template <typename T>
inline T* at(void* base, size_t off)
{
    return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off);
}

// A skinny product of one matrix (or of stacked matrices with per-matrix
// scales from w_scale_ptr, n_per_scale rows each).
bl::SkinnyArgs skinny(const uint8_t* w, const float* w_scale_ptr, float w_scale, int n_per_scale, int n, int k,
                      const int8_t* q, const float* act_scale, const int32_t* act_sum, int m, const float* residual,
                      float* y, int ldy, int32_t* acc = nullptr)
{
    bl::SkinnyArgs a;
    a.w0 = w;
    a.w_scale_ptr = w_scale_ptr;
    a.w_scale0 = w_scale;
    a.n_per_scale = n_per_scale;
    a.n = n;
    a.k = k;
    a.q = q;
    a.act_scale = act_scale;
    a.act_sum = act_sum;
    a.m = m;
    a.residual = residual;
    a.y = y;
    a.ldy = ldy;
    a.acc0 = acc;
    return a;
}

// The product as ks partial sums over K (no epilogue: the next norm + quant
// finishes it with the residual, launch_quant_reduce).
void split_k(bl::SkinnyArgs& a, int32_t* part, int ks)
{
    a.residual = nullptr;
    a.y = nullptr;
    a.part = part;
    a.ksplit = ks;
}

// The fused gate/up of f rows over d inputs: h[m][f] = relu(gate)^2 * up.
bl::SkinnyArgs skinny_gateup(const uint8_t* w_gate, float s_gate, const uint8_t* w_up, float s_up,
                             const float* scale_ptr, int f, int d, const int8_t* q, const float* act_scale,
                             const int32_t* act_sum, int m, float* h, int32_t* acc_gate, int32_t* acc_up)
{
    bl::SkinnyArgs a = skinny(w_gate, scale_ptr, s_gate, f, f, d, q, act_scale, act_sum, m, nullptr, h, f, acc_gate);
    a.w1 = w_up;
    a.w_scale1 = s_up;
    a.acc1 = acc_up;
    return a;
}

// True while s records into a graph (or the query fails). A capture takes the
// launch-per-step path (same results): a replayed graph may run next to other
// work that holds CUs, which the persistent kernel needs to itself.
bool capturing(hipStream_t s)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) return true;
    return st != hipStreamCaptureStatusNone;
}

int ffn_impl(const float* x, int64_t m, int64_t d, int64_t f, const float* g_ffn, const float* g_sub, float eps,
             const uint8_t* w_gate, float s_gate, const uint8_t* w_up, float s_up, const uint8_t* w_down,
             float s_down, const float* scale_ptr /* [gate, up, down] or null */, const float* residual, float* out,
             void* ws, int flags, hipStream_t s)
{
    const Layout L = ffn_layout(m, d, f);
    int8_t* q1 = at<int8_t>(ws, L.off[BITNET_FFN_WS_Q1]);
    float* s1 = at<float>(ws, L.off[BITNET_FFN_WS_S1]);
    int32_t* qs1 = at<int32_t>(ws, L.off[BITNET_FFN_WS_QS1]);
    float* h = at<float>(ws, L.off[BITNET_FFN_WS_H]);
    int8_t* q2 = at<int8_t>(ws, L.off[BITNET_FFN_WS_Q2]);
    float* s2 = at<float>(ws, L.off[BITNET_FFN_WS_S2]);
    int32_t* qs2 = at<int32_t>(ws, L.off[BITNET_FFN_WS_QS2]);
    const bool keep = (flags & BITNET_FFN_WRITE_ACC) != 0;
    int32_t* acc_g = keep ? at<int32_t>(ws, L.off[BITNET_FFN_WS_ACC_GATE]) : nullptr;
    int32_t* acc_u = keep ? at<int32_t>(ws, L.off[BITNET_FFN_WS_ACC_UP]) : nullptr;
    int32_t* acc_d = keep ? at<int32_t>(ws, L.off[BITNET_FFN_WS_ACC_DOWN]) : nullptr;
    const int M = (int)m, D = (int)d, F = (int)f;
    // Up to 32 tokens the products are short, latency-bound weight streams:
    // each norm + quant launch also pulls the next product's weight lines
    // into the memory-side cache (extra workgroups, no effect on results).
    const bool pre = m <= kMaxSkinnyM;
    const bool gemv = m <= kMaxGemvM;
    const uint32_t wb = (uint32_t)((size_t)f * d / 4);
    const uint32_t ch_gu = (uint32_t)(gemv ? bl::gemv_rows_per_block(D) : bl::skinny_rows_per_tile(F, true)) * (D / 4);
    const uint32_t ch_dn = (uint32_t)(gemv ? bl::gemv_rows_per_block(F) : bl::skinny_rows_per_tile(D, false)) * (F / 4);
    const bl::Prefetch pf_gu = {{w_gate, w_up}, {wb, wb}, ch_gu};
    const bl::Prefetch pf_dn = {{w_down, nullptr}, {wb, 0u}, ch_dn};

    int rc;
    if (bl::fwd_fits(M, D)) {
        // one token: the norm + quant of x runs inside the gate/up launch
        rc = bl::launch_fwd_gateup(x, g_ffn, eps, w_gate, s_gate, w_up, s_up, scale_ptr, F, D, h, q1, s1, qs1, acc_g,
                                   acc_u, s);
    } else if ((rc = bl::launch_quant_act(x, g_ffn, eps, M, D, q1, s1, qs1, s, false, pre ? &pf_gu : nullptr))) {
        return rc;
    } else if (m <= kMaxGemvM) {
        rc = bl::launch_gateup(w_gate, s_gate, w_up, s_up, scale_ptr, F, D, q1, s1, qs1, M, h, acc_g, acc_u, s);
    } else if (m <= kMaxSkinnyM) {
        rc = bl::launch_skinny(skinny_gateup(w_gate, s_gate, w_up, s_up, scale_ptr, F, D, q1, s1, qs1, M, h, acc_g,
                                             acc_u),
                               true, s);
    } else {
        // gate and up in one MFMA product with relu(gate)^2 * up in its epilogue
        rc = bl::launch_gemm_gateup(w_gate, s_gate, w_up, s_up, scale_ptr, F, D, q1, s1, qs1, M, h, acc_g, acc_u, s);
    }
    if (rc) return rc;
    const float* sdp = scale_ptr ? scale_ptr + 2 : nullptr;
    if (bl::fwd_block_fits(M, F))  // one token: the sub-norm + quant of h runs inside the down launch
        return bl::launch_fwd_block(h, g_sub, eps, w_down, s_down, sdp, D, F, residual, out, acc_d, q2, s2, qs2, s);
    rc = bl::launch_quant_act(h, g_sub, eps, M, F, q2, s2, qs2, s, false, pre ? &pf_dn : nullptr);
    if (rc) return rc;
    if (m <= kMaxGemvM)
        return bl::launch_gemv(w_down, s_down, sdp, D, F, q2, s2, qs2, M, residual, out, acc_d, s);
    if (m <= kMaxSkinnyM)
        return bl::launch_skinny(skinny(w_down, sdp, s_down, D, D, F, q2, s2, qs2, M, residual, out, D, acc_d), true,
                                 s);
    return bl::launch_gemm(w_down, s_down, sdp, D, F, q2, s2, qs2, M, residual, out, D, acc_d, nullptr, nullptr, s);
}

// ---- library-owned scratch for callers that cannot allocate -------------------
//
// A static device array: each GPU the library runs on holds its own copy until
// the process ends. Host code never passes the array's name to a kernel (on
// the host it names a stand-in, not device memory): the device address of the
// current GPU's copy is looked up once per device with hipGetSymbolAddress and
// only that address is used.
constexpr size_t kStaticScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current GPU's scratch copy (looked up on the first call
// on that GPU, with that GPU current), or an error status.
int static_scratch(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BL_ERR_DEVICE;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&]() { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
    if (slot.err != hipSuccess || slot.ptr == nullptr) return BL_ERR_DEVICE;
    *out = slot.ptr;
    return BL_OK;
}

// Argument checks of bitlinear_gemm, then its launches. ws_given: the call has
// a workspace (the caller's, or the library's static array, passed as
// workspace == NULL); a caller's workspace must be 8-byte aligned.
int gemm_check(const uint8_t* packed, float w_scale, int64_t n, int64_t k, const int8_t* q, const float* act_scale,
               const int32_t* act_sum, int64_t m, const float* residual, const float* y, const int32_t* acc_out,
               const int32_t* row_argmax, const void* workspace, bool ws_given, size_t workspace_bytes);
int gemm_launch(const uint8_t* packed, float w_scale, int64_t n, int64_t k, const int8_t* q, const float* act_scale,
                const int32_t* act_sum, int64_t m, const float* residual, float* y, int32_t* acc_out,
                int32_t* row_argmax, void* workspace, hipStream_t s);

// Greedy-head workspace: the per-sequence penalty bitmaps, then the argmax
// keys (one per sequence and 32-column tile).
struct HeadLayout {
    size_t bits, keys, total;
};

HeadLayout head_layout(int64_t m, int64_t n)
{
    HeadLayout l{};
    l.bits = 0;
    l.keys = align_up((size_t)m * (size_t)bl::penalty_words((int)n) * 4, 256);
    l.total = l.keys + align_up((size_t)m * (size_t)((n + 31) / 32) * 8, 256);
    return l;
}

// Greedy-step workspace: the stream's (zero-filled once, then kept), the final
// norm + quant of x, then the head's.
struct StepLayout {
    size_t stream, q, s, qs, head, total;
};

StepLayout step_layout(int64_t m, int64_t d, int64_t f, int64_t vocab)
{
    StepLayout l{};
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t o = at;
        at = align_up(at + bytes, 256);
        return o;
    };
    l.stream = take(stream_layout(m, d, f).total);
    l.q = take((size_t)(m * d));
    l.s = take((size_t)m * 4);
    l.qs = take((size_t)m * 4);
    l.head = take(head_layout(m, vocab).total);
    l.total = at;
    return l;
}

// The LM head with the repetition penalty and the greedy choice (m <= 32,
// validated): bitmaps (unless bits_ready: the caller built them in the head's
// workspace), the skinny product with penalised fp32 keys, the per-token
// reduction into next -- which, given app_hist, also appends next to the
// histories.
int greedy_head_launch(const uint8_t* head, float s_head, int64_t n, int64_t k, const int8_t* q,
                       const float* act_scale, const int32_t* act_sum, int64_t m, const int32_t* hist,
                       int64_t hist_stride, const int32_t* hist_len, float penalty, float* logits, int32_t* next,
                       void* ws, hipStream_t s, bool bits_ready = false, int32_t* app_hist = nullptr,
                       int32_t* app_len = nullptr)
{
    const HeadLayout L = head_layout(m, n);
    uint32_t* bits = at<uint32_t>(ws, L.bits);
    unsigned long long* keys = at<unsigned long long>(ws, L.keys);
    int rc = bits_ready ? BL_OK : bl::launch_penalty_bits(hist, (int)hist_stride, hist_len, (int)n, (int)m, bits, s);
    if (rc) return rc;
    if (m == 1) {
        // one token: a GEMV streams the head at the GEMV's rate
        int tiles = 0;
        rc = bl::launch_head_gemv(head, s_head, (int)n, (int)k, q, act_scale, act_sum, bits, penalty, logits, keys,
                                  (int)((n + 31) / 32), &tiles, s);
        if (rc) return rc;
        return bl::launch_tile_argmax(keys, tiles, 1, next, s, app_hist, (int)hist_stride, app_len);
    }
    bl::SkinnyArgs a =
        skinny(head, nullptr, s_head, 1, (int)n, (int)k, q, act_scale, act_sum, (int)m, nullptr, logits, (int)n);
    a.tile_keys = keys;
    a.pen_bits = bits;
    a.pen_words = bl::penalty_words((int)n);
    a.penalty = penalty;
    rc = bl::launch_skinny(a, true, s);
    if (rc) return rc;
    return bl::launch_tile_argmax(keys, bl::skinny_tiles((int)n, false), (int)m, next, s, app_hist, (int)hist_stride,
                                  app_len);
}

// The launch-per-step layer stream (any m). Without attn, the o projection of
// layer l reads the stand-in z[l]; with attn, it reads the attention output of
// the layer (RoPE, cache append and attention over positions 0 .. pos after
// the q/k/v product).
struct AttnCtx {
    int heads, max_seq, pos;
    const float *rope_cos, *rope_sin;
    float *k_cache, *v_cache;  // [n_layers][m][heads][max_seq][hd]
    float *q_rot, *part;       // scratch
    float* attn;               // [n_layers][m][d] or null (then attn_scratch, reused)
    float* attn_scratch;       // [m][d]
};

int stream_steps(const uint8_t* weights, const float* scales, const float* gains, const float* z, int64_t n_layers,
                 int64_t m, int64_t d, int64_t f, float eps, float* x, float* qkv, void* workspace,
                 const AttnCtx* attn, hipStream_t s)
{
    const StreamLayout L = stream_layout(m, d, f);
    // the o projection's input of layer l: the stand-in, or the layer's attention output
    auto o_input = [&](int64_t l, float* qkv_l) -> const float* {
        if (!attn) return z + (size_t)l * m * d;
        float* out = attn->attn ? attn->attn + (size_t)l * m * d : attn->attn_scratch;
        const size_t cache_layer = (size_t)m * d * attn->max_seq;  // heads * hd = d per position
        if (bl::launch_attention(qkv_l, (int)(3 * d), (int)m, (int)d, attn->heads, attn->rope_cos, attn->rope_sin,
                                 attn->max_seq, attn->pos, attn->k_cache + (size_t)l * cache_layer,
                                 attn->v_cache + (size_t)l * cache_layer, attn->q_rot, attn->part, out, (int)d, s))
            return nullptr;
        return out;
    };
    int8_t* qa = at<int8_t>(workspace, L.q_a);
    float* sa = at<float>(workspace, L.s_a);
    int32_t* qsa = at<int32_t>(workspace, L.qs_a);
    int8_t* qo = at<int8_t>(workspace, L.q_o);
    float* so = at<float>(workspace, L.s_o);
    int32_t* qso = at<int32_t>(workspace, L.qs_o);
    void* ffn_ws = at<void>(workspace, L.ffn);
    const int M = (int)m, D = (int)d, F = (int)f;
    const size_t blob = bitnet_layer_bytes(d, f);
    const size_t dd = (size_t)(d * d) / 4, fd = (size_t)(f * d) / 4;
    const size_t gstride = (size_t)(3 * d + f);
    if (m > kMaxGemvM && m <= kMaxSkinnyM) {
        // 9..32 tokens: every projection is one skinny MFMA launch over
        // activations quantised straight into its operand order
        const Layout FL = ffn_layout(m, d, f);
        int8_t* q1 = at<int8_t>(ffn_ws, FL.off[BITNET_FFN_WS_Q1]);
        float* s1 = at<float>(ffn_ws, FL.off[BITNET_FFN_WS_S1]);
        int32_t* qs1 = at<int32_t>(ffn_ws, FL.off[BITNET_FFN_WS_QS1]);
        float* h = at<float>(ffn_ws, FL.off[BITNET_FFN_WS_H]);
        int8_t* q2 = at<int8_t>(ffn_ws, FL.off[BITNET_FFN_WS_Q2]);
        float* s2 = at<float>(ffn_ws, FL.off[BITNET_FFN_WS_S2]);
        int32_t* qs2 = at<int32_t>(ffn_ws, FL.off[BITNET_FFN_WS_QS2]);
        int32_t* part = at<int32_t>(workspace, L.part);
        const int ks = batched_ksplit(d, f);
        for (int64_t l = 0; l < n_layers; ++l) {
            const uint8_t* wl = weights + (size_t)l * blob;
            const float* sl = scales + 7 * l;
            const float* gl = gains + l * gstride;
            float* qkv_l = qkv ? qkv + (size_t)l * m * 3 * d : at<float>(workspace, L.qkv);
            const uint8_t* wg = wl + 4 * dd;
            // each norm + quant also pulls the next product's weight lines into the
            // memory-side cache
            const uint32_t rd = (uint32_t)(D / 4), rf = (uint32_t)(F / 4);
            const bl::Prefetch pf_qkv = {{wl, nullptr}, {(uint32_t)(3 * dd), 0u},
                                         (uint32_t)bl::skinny_rows_per_tile(3 * D, false) * rd};
            const bl::Prefetch pf_o = {{wl + 3 * dd, nullptr}, {(uint32_t)dd, 0u},
                                       (uint32_t)bl::skinny_rows_per_tile(D, false) * rd};
            const bl::Prefetch pf_gu = {{wg, wg + fd}, {(uint32_t)fd, (uint32_t)fd},
                                        (uint32_t)bl::skinny_rows_per_tile(F, true) * rd};
            const bl::Prefetch pf_dn = {{wg + 2 * fd, nullptr}, {(uint32_t)fd, 0u},
                                        (uint32_t)bl::skinny_rows_per_tile(D, false) * rf};
            // x after the previous layer's down product: finished by this norm +
            // quant when that product was split (every layer but the last)
            int rc = l > 0 && ks > 1
                         ? bl::launch_quant_reduce(x, gl, eps, M, D, part, ks, qs2, s2, sl - 7 + 6, qa, sa, qsa, s,
                                                   &pf_qkv)
                         : bl::launch_quant_act(x, gl, eps, M, D, qa, sa, qsa, s, true, &pf_qkv);
            if (!rc)
                rc = bl::launch_skinny(skinny(wl, sl, 0.0f, D, 3 * D, D, qa, sa, qsa, M, nullptr, qkv_l, 3 * D), false,
                                       s);
            const float* o_src = rc ? nullptr : o_input(l, qkv_l);
            if (!rc && !o_src) rc = BL_ERR_LAUNCH;
            if (!rc) rc = bl::launch_quant_act(o_src, gl + d, eps, M, D, qo, so, qso, s, true, &pf_o);
            if (!rc)
                rc = bl::launch_skinny(skinny(wl + 3 * dd, sl + 3, 0.0f, D, D, D, qo, so, qso, M, x, x, D), false, s);
            if (!rc) rc = bl::launch_quant_act(x, gl + 2 * d, eps, M, D, q1, s1, qs1, s, true, &pf_gu);
            if (!rc)
                rc = bl::launch_skinny(skinny_gateup(wg, 0.0f, wg + fd, 0.0f, sl + 4, F, D, q1, s1, qs1, M, h, nullptr,
                                                     nullptr),
                                       false, s);
            if (!rc) rc = bl::launch_quant_act(h, gl + 3 * d, eps, M, F, q2, s2, qs2, s, true, &pf_dn);
            if (!rc) {
                // down: partial sums per K part, finished by the next layer's
                // norm + quant; the last layer writes x itself
                bl::SkinnyArgs adn = skinny(wg + 2 * fd, sl + 6, 0.0f, D, D, F, q2, s2, qs2, M, x, x, D);
                if (ks > 1 && l + 1 < n_layers) split_k(adn, part, ks);
                rc = bl::launch_skinny(adn, false, s);
            }
            if (rc) return rc;
        }
        return BL_OK;
    }
    for (int64_t l = 0; l < n_layers; ++l) {
        const uint8_t* wl = weights + (size_t)l * blob;
        const float* sl = scales + 7 * l;
        const float* gl = gains + l * gstride;
        float* qkv_l = qkv ? qkv + (size_t)l * m * 3 * d : at<float>(workspace, L.qkv);
        // m <= 8 here: q/k/v and o are GEMV launches over D inputs
        const uint32_t ch = (uint32_t)bl::gemv_rows_per_block(D) * (uint32_t)(D / 4);
        const bl::Prefetch pf_qkv = {{wl, nullptr}, {(uint32_t)(3 * dd), 0u}, ch};
        const bl::Prefetch pf_o = {{wl + 3 * dd, nullptr}, {(uint32_t)dd, 0u}, ch};
        const bool pre = m <= kMaxGemvM;
        int rc = bl::launch_quant_act(x, gl, eps, M, D, qa, sa, qsa, s, false, pre ? &pf_qkv : nullptr);
        if (rc) return rc;
        if (m <= kMaxGemvM) {
            const uint8_t* qkv_w[3] = {wl, wl + dd, wl + 2 * dd};
            rc = bl::launch_gemv_multi(3, qkv_w, sl, D, D, qa, sa, qsa, M, qkv_l, 3 * D, s);
        } else {
            for (int j = 0; j < 3 && !rc; ++j)  // column block j of qkv[m][3d]
                rc = bl::launch_gemm(wl + j * dd, 0.0f, sl + j, D, D, qa, sa, qsa, M, nullptr, qkv_l + (size_t)j * d,
                                     3 * D, nullptr, nullptr, nullptr, s);
        }
        if (rc) return rc;
        const float* o_src = o_input(l, qkv_l);
        if (!o_src) return BL_ERR_LAUNCH;
        rc = bl::launch_quant_act(o_src, gl + d, eps, M, D, qo, so, qso, s, false, pre ? &pf_o : nullptr);
        if (rc) return rc;
        if (m <= kMaxGemvM)
            rc = bl::launch_gemv(wl + 3 * dd, 0.0f, sl + 3, D, D, qo, so, qso, M, x, x, nullptr, s);
        else
            rc = bl::launch_gemm(wl + 3 * dd, 0.0f, sl + 3, D, D, qo, so, qso, M, x, x, D, nullptr, nullptr, nullptr, s);
        if (rc) return rc;
        rc = ffn_impl(x, m, d, f, gl + 2 * d, gl + 3 * d, eps, wl + 4 * dd, 0.0f, wl + 4 * dd + fd, 0.0f,
                      wl + 4 * dd + 2 * fd, 0.0f, sl + 4, x, x, ffn_ws, 0, s);
        if (rc) return rc;
    }
    return BL_OK;
}

}  // namespace

extern "C" {

int bitlinear_quant_act(const float* x, const float* gain, float eps, int64_t m, int64_t k, int8_t* q,
                        float* act_scale, int32_t* act_sum, void* stream)
{
    if (!x || !q || !act_scale) return BL_ERR_NULL;
    if (!dim_ok(m) || !k_ok(k) || m > 0x7fffffff) return BL_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(q, 16) || (gain && !aligned(gain, 16)) || !aligned(act_scale, 4) ||
        (act_sum && !aligned(act_sum, 4)))
        return BL_ERR_ALIGN;
    return bl::launch_quant_act(x, gain, eps, (int)m, (int)k, q, act_scale, act_sum, as_stream(stream));
}

int bitlinear_gemv(const uint8_t* packed, float w_scale, int64_t n, int64_t k, const int8_t* q,
                   const float* act_scale, const int32_t* act_sum, int64_t m, const float* residual, float* y,
                   int32_t* acc_out, void* stream)
{
    if (!packed || !q || !act_scale || !act_sum || !y) return BL_ERR_NULL;
    if (m < 1 || m > kMaxGemvM || !dim_ok(n) || !k_ok(k) || k > kMaxGemvK) return BL_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(q, 16) || !aligned(act_scale, 4) || !aligned(act_sum, 4) ||
        !aligned(y, 4) || (residual && !aligned(residual, 4)) || (acc_out && !aligned(acc_out, 4)))
        return BL_ERR_ALIGN;
    if (!(w_scale > 0.0f) || !(w_scale < INFINITY)) return BL_ERR_VALUE;
    return bl::launch_gemv(packed, w_scale, nullptr, (int)n, (int)k, q, act_scale, act_sum, (int)m, residual, y,
                           acc_out, as_stream(stream));
}

int bitlinear_forward(const float* x, const float* gain, float eps, const uint8_t* packed, float w_scale, int64_t n,
                      int64_t k, int64_t m, int8_t* q, float* act_scale, int32_t* act_sum, float* y, void* stream)
{
    if (!x || !packed || !q || !act_scale || !act_sum || !y) return BL_ERR_NULL;
    if (m < 1 || m > kMaxGemvM || !dim_ok(n) || !k_ok(k) || k > kMaxGemvK) return BL_ERR_SHAPE;
    if (!aligned(x, 16) || (gain && !aligned(gain, 16)) || !aligned(packed, 16) || !aligned(q, 16) ||
        !aligned(act_scale, 4) || !aligned(act_sum, 4) || !aligned(y, 4))
        return BL_ERR_ALIGN;
    if (!(w_scale > 0.0f) || !(w_scale < INFINITY)) return BL_ERR_VALUE;
    const hipStream_t s = as_stream(stream);
    if (bl::fwd_fits((int)m, (int)k))
        return bl::launch_fwd(x, gain, eps, packed, w_scale, (int)n, (int)k, y, q, act_scale, act_sum, s);
    if (bl::fwd_block_fits((int)m, (int)k))
        return bl::launch_fwd_block(x, gain, eps, packed, w_scale, nullptr, (int)n, (int)k, nullptr, y, nullptr, q,
                                    act_scale, act_sum, s);
    const uint64_t wbytes = std::min<uint64_t>((uint64_t)n * (uint64_t)k / 4, 0xfffffffcull);
    const bl::Prefetch pf = {{packed, nullptr}, {(uint32_t)wbytes, 0u},
                             (uint32_t)bl::gemv_rows_per_block((int)k) * (uint32_t)(k / 4)};
    const int rc = bl::launch_quant_act(x, gain, eps, (int)m, (int)k, q, act_scale, act_sum, s, false, &pf);
    if (rc) return rc;
    return bl::launch_gemv(packed, w_scale, nullptr, (int)n, (int)k, q, act_scale, act_sum, (int)m, nullptr, y,
                           nullptr, s);
}

size_t bitlinear_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int with_argmax)
{
    (void)k;
    if (!with_argmax || m <= 0 || n <= 0) return 0;
    if (m <= kMaxSkinnyM)  // one key per token and 32-column tile
        return align_up((size_t)m * (size_t)((n + 31) / 32) * 8, 256);
    return align_up((size_t)m * 8, 256);
}

int bitlinear_gemm(const uint8_t* packed, float w_scale, int64_t n, int64_t k, const int8_t* q,
                   const float* act_scale, const int32_t* act_sum, int64_t m, const float* residual, float* y,
                   int32_t* acc_out, int32_t* row_argmax, void* workspace, size_t workspace_bytes, void* stream)
{
    if (row_argmax && !workspace) return BL_ERR_NULL;
    const int rc = gemm_check(packed, w_scale, n, k, q, act_scale, act_sum, m, residual, y, acc_out, row_argmax,
                              workspace, workspace != nullptr, workspace_bytes);
    if (rc != BL_OK) return rc;
    return gemm_launch(packed, w_scale, n, k, q, act_scale, act_sum, m, residual, y, acc_out, row_argmax, workspace,
                       as_stream(stream));
}

int bitlinear_gemm_noalloc(const uint8_t* packed, float w_scale, int64_t n, int64_t k, const int8_t* q,
                           const float* act_scale, const int32_t* act_sum, int64_t m, const float* residual,
                           float* y, int32_t* acc_out, int32_t* row_argmax, void* stream)
{
    // every argument check first (an argmax needing more than the static array
    // fails as BL_ERR_WORKSPACE), then the device address of the array
    const int rc = gemm_check(packed, w_scale, n, k, q, act_scale, act_sum, m, residual, y, acc_out, row_argmax,
                              nullptr, true, kStaticScratchBytes);
    if (rc != BL_OK) return rc;
    void* ws = nullptr;
    if (row_argmax) {
        const int src = static_scratch(&ws);
        if (src != BL_OK) return src;
    }
    return gemm_launch(packed, w_scale, n, k, q, act_scale, act_sum, m, residual, y, acc_out, row_argmax, ws,
                       as_stream(stream));
}

size_t bitlinear_gemm_noalloc_max_scratch_bytes(void) { return kStaticScratchBytes; }

}  // extern "C"

namespace {

int gemm_check(const uint8_t* packed, float w_scale, int64_t n, int64_t k, const int8_t* q, const float* act_scale,
               const int32_t* act_sum, int64_t m, const float* residual, const float* y, const int32_t* acc_out,
               const int32_t* row_argmax, const void* workspace, bool ws_given, size_t workspace_bytes)
{
    if (!packed || !q || !act_scale || !act_sum) return BL_ERR_NULL;
    if (!y && !row_argmax) return BL_ERR_NULL;
    if (row_argmax && !ws_given) return BL_ERR_NULL;
    if (!dim_ok(m) || !dim_ok(n) || !k_ok(k) || m > 0x7fffffff || n > 0x7fffffff || m * n > ((int64_t)1 << 40))
        return BL_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(q, 16) || !aligned(act_scale, 4) || !aligned(act_sum, 4) ||
        (y && !aligned(y, 4)) || (residual && !aligned(residual, 4)) || (acc_out && !aligned(acc_out, 4)) ||
        (row_argmax && !aligned(row_argmax, 4)) || (workspace && !aligned(workspace, 8)))
        return BL_ERR_ALIGN;
    if (!(w_scale > 0.0f) || !(w_scale < INFINITY)) return BL_ERR_VALUE;
    if (row_argmax && workspace_bytes < bitlinear_gemm_workspace_bytes(m, n, k, 1)) return BL_ERR_WORKSPACE;
    return BL_OK;
}

int gemm_launch(const uint8_t* packed, float w_scale, int64_t n, int64_t k, const int8_t* q, const float* act_scale,
                const int32_t* act_sum, int64_t m, const float* residual, float* y, int32_t* acc_out,
                int32_t* row_argmax, void* workspace, hipStream_t s)
{
    if (m <= kMaxSkinnyM) {
        bl::SkinnyArgs a = skinny(packed, nullptr, w_scale, 1, (int)n, (int)k, q, act_scale, act_sum, (int)m, residual,
                                  y, (int)n, acc_out);
        unsigned long long* keys = row_argmax ? static_cast<unsigned long long*>(workspace) : nullptr;
        a.tile_keys = keys;
        int rc = bl::launch_skinny(a, true, s);
        if (!rc && keys) rc = bl::launch_tile_argmax(keys, bl::skinny_tiles((int)n, false), (int)m, row_argmax, s);
        return rc;
    }
    return bl::launch_gemm(packed, w_scale, nullptr, (int)n, (int)k, q, act_scale, act_sum, (int)m, residual, y,
                           (int)n, acc_out, row_argmax, static_cast<unsigned long long*>(workspace), s);
}

}  // namespace

extern "C" {

size_t bitnet_ffn_workspace_bytes(int64_t m, int64_t d, int64_t f)
{
    if (m <= 0 || d <= 0 || f <= 0) return 0;
    return ffn_layout(m, d, f).total;
}

size_t bitnet_ffn_workspace_offset(int64_t m, int64_t d, int64_t f, int segment)
{
    if (m <= 0 || d <= 0 || f <= 0 || segment < 0 || segment >= BITNET_FFN_WS_COUNT) return (size_t)-1;
    return ffn_layout(m, d, f).off[segment];
}

int bitnet_ffn(const float* x, int64_t m, int64_t d, int64_t f, const float* norm_gain, const float* sub_norm_gain,
               float eps, const uint8_t* w_gate, float s_gate, const uint8_t* w_up, float s_up,
               const uint8_t* w_down, float s_down, const float* residual, float* out, void* workspace,
               size_t workspace_bytes, int flags, void* stream)
{
    if (!x || !norm_gain || !sub_norm_gain || !w_gate || !w_up || !w_down || !out || !workspace) return BL_ERR_NULL;
    if (!dim_ok(m) || !k_ok(d) || !k_ok(f) || m > 0x7fffffff || f > kMaxGemvK || d > kMaxGemvK)
        return BL_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(norm_gain, 16) || !aligned(sub_norm_gain, 16) || !aligned(w_gate, 16) ||
        !aligned(w_up, 16) || !aligned(w_down, 16) || !aligned(out, 4) || (residual && !aligned(residual, 4)) ||
        !aligned(workspace, 256))
        return BL_ERR_ALIGN;
    if (!(s_gate > 0.0f) || !(s_up > 0.0f) || !(s_down > 0.0f) || !(s_gate < INFINITY) || !(s_up < INFINITY) ||
        !(s_down < INFINITY))
        return BL_ERR_VALUE;
    if (workspace_bytes < bitnet_ffn_workspace_bytes(m, d, f)) return BL_ERR_WORKSPACE;
    return ffn_impl(x, m, d, f, norm_gain, sub_norm_gain, eps, w_gate, s_gate, w_up, s_up, w_down, s_down, nullptr,
                    residual, out, workspace, flags, as_stream(stream));
}

size_t bitnet_layer_bytes(int64_t d, int64_t f)
{
    if (d <= 0 || f <= 0) return 0;
    return (size_t)(d * d) + (size_t)(3 * d * f) / 4;
}

size_t bitnet_stream_workspace_bytes(int64_t m, int64_t d, int64_t f)
{
    if (m <= 0 || d <= 0 || f <= 0) return 0;
    return stream_layout(m, d, f).total;
}

int bitnet_decode_stream(const uint8_t* weights, const float* scales, const float* gains, const float* z,
                         int64_t n_layers, int64_t m, int64_t d, int64_t f, float eps, float* x, float* qkv,
                         void* workspace, size_t workspace_bytes, void* stream)
{
    if (!weights || !scales || !gains || !z || !x || !workspace) return BL_ERR_NULL;
    if (!dim_ok(n_layers) || !dim_ok(m) || !k_ok(d) || !k_ok(f) || d > kMaxGemvK || f > kMaxGemvK ||
        m > 0x7fffffff)
        return BL_ERR_SHAPE;
    if (!aligned(weights, 16) || !aligned(scales, 4) || !aligned(gains, 16) || !aligned(z, 16) || !aligned(x, 16) ||
        (qkv && !aligned(qkv, 16)) || !aligned(workspace, 256))
        return BL_ERR_ALIGN;
    if (workspace_bytes < bitnet_stream_workspace_bytes(m, d, f)) return BL_ERR_WORKSPACE;
    const hipStream_t s = as_stream(stream);
    const StreamLayout L = stream_layout(m, d, f);
    if (bl::stream_persistent_fits((int)m, (int)d, (int)f, nullptr) && !capturing(s)) {
        float* qkv_out = qkv ? qkv : at<float>(workspace, L.qkv);
        return bl::launch_stream_persistent(weights, scales, gains, z, (int)n_layers, (int)d, (int)f, eps, x, qkv_out,
                                            qkv ? 3 * d : 0, at<void>(workspace, L.ll),
                                            at<uint32_t>(workspace, L.ctrl), nullptr, s);
    }
    return stream_steps(weights, scales, gains, z, n_layers, m, d, f, eps, x, qkv, workspace, nullptr, s);
}

// ---- decode step with attention -------------------------------------------------

size_t bitnet_decode_step_workspace_bytes(int64_t m, int64_t d, int64_t f, int64_t n_heads, int64_t max_seq)
{
    if (m <= 0 || d <= 0 || f <= 0 || n_heads <= 0 || max_seq <= 0 || d % n_heads != 0 || max_seq > 0x7fffffff)
        return 0;
    const size_t hd = (size_t)(d / n_heads);
    size_t at = align_up(stream_layout(m, d, f).total, 256);
    at += align_up((size_t)(m * d) * 4, 256);  // rotated q
    at += align_up((size_t)(m * d) * 4, 256);  // attention output scratch
    // chunk partials: fp32 for the launch path, epoch-tagged 8-byte words for the persistent one
    // (which cuts short contexts into up to 32 chunks)
    const size_t chunks = std::max<size_t>((size_t)bl::attn_chunks((int)max_seq), (size_t)bl::kStreamAttnMaxChunks);
    at += align_up((size_t)m * (size_t)n_heads * chunks * (hd + 2) * 8, 256);
    return at;
}

int bitnet_decode_step(const uint8_t* weights, const float* scales, const float* gains, int64_t n_layers, int64_t m,
                       int64_t d, int64_t f, int64_t n_heads, float eps, const float* rope_cos, const float* rope_sin,
                       int64_t max_seq, int64_t pos, float* k_cache, float* v_cache, float* x, float* qkv,
                       float* attn, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!weights || !scales || !gains || !rope_cos || !rope_sin || !k_cache || !v_cache || !x || !workspace)
        return BL_ERR_NULL;
    if (!dim_ok(n_layers) || !dim_ok(m) || !k_ok(d) || !k_ok(f) || d > kMaxGemvK || f > kMaxGemvK ||
        m > 0x7fffffff || n_heads <= 0 || d % n_heads != 0 || (d / n_heads) % 4 != 0 || d / n_heads > 256 ||
        max_seq <= 0 || max_seq > 0x7fffffff || pos < 0 || pos >= max_seq)
        return BL_ERR_SHAPE;
    if (!aligned(weights, 16) || !aligned(scales, 4) || !aligned(gains, 16) || !aligned(rope_cos, 4) ||
        !aligned(rope_sin, 4) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(x, 16) ||
        (qkv && !aligned(qkv, 16)) || (attn && !aligned(attn, 16)) || !aligned(workspace, 256))
        return BL_ERR_ALIGN;
    if (workspace_bytes < bitnet_decode_step_workspace_bytes(m, d, f, n_heads, max_seq)) return BL_ERR_WORKSPACE;
    const hipStream_t s = as_stream(stream);
    const size_t part_off = align_up(stream_layout(m, d, f).total, 256) + 2 * align_up((size_t)(m * d) * 4, 256);
    {
        // one sequence: the whole step as one persistent launch
        const bl::StreamAttn pa = {(int)n_heads, (int)max_seq, (int)pos, rope_cos, rope_sin, k_cache, v_cache, attn,
                                   at<void>(workspace, part_off)};
        if (bl::stream_persistent_fits((int)m, (int)d, (int)f, &pa) && !capturing(s)) {
            const StreamLayout L = stream_layout(m, d, f);
            float* qkv_out = qkv ? qkv : at<float>(workspace, L.qkv);
            return bl::launch_stream_persistent(weights, scales, gains, nullptr, (int)n_layers, (int)d, (int)f, eps, x,
                                                qkv_out, qkv ? 3 * d : 0, at<void>(workspace, L.ll),
                                                at<uint32_t>(workspace, L.ctrl), &pa, s);
        }
    }
    size_t at_off = align_up(stream_layout(m, d, f).total, 256);
    AttnCtx ctx;
    ctx.heads = (int)n_heads;
    ctx.max_seq = (int)max_seq;
    ctx.pos = (int)pos;
    ctx.rope_cos = rope_cos;
    ctx.rope_sin = rope_sin;
    ctx.k_cache = k_cache;
    ctx.v_cache = v_cache;
    ctx.q_rot = at<float>(workspace, at_off);
    at_off += align_up((size_t)(m * d) * 4, 256);
    ctx.attn_scratch = at<float>(workspace, at_off);
    at_off += align_up((size_t)(m * d) * 4, 256);
    ctx.part = at<float>(workspace, at_off);
    ctx.attn = attn;
    return stream_steps(weights, scales, gains, nullptr, n_layers, m, d, f, eps, x, qkv, workspace, &ctx, s);
}

// ---- greedy decoding around the stream ----------------------------------------

int bitnet_embed(const uint8_t* table, float s_emb, int64_t vocab, int64_t d, const int32_t* tokens, int64_t m,
                 float* x, void* stream)
{
    if (!table || !tokens || !x) return BL_ERR_NULL;
    if (!dim_ok(vocab) || !k_ok(d) || !dim_ok(m) || vocab > 0x7fffffff || d > kMaxGemvK || m > 0x7fffffff)
        return BL_ERR_SHAPE;
    if (!aligned(table, 16) || !aligned(tokens, 4) || !aligned(x, 16)) return BL_ERR_ALIGN;
    if (!(s_emb > 0.0f) || !(s_emb < INFINITY)) return BL_ERR_VALUE;
    return bl::launch_embed(table, s_emb, (int)vocab, (int)d, tokens, (int)m, x, as_stream(stream));
}

size_t bitnet_greedy_head_workspace_bytes(int64_t m, int64_t n)
{
    if (m <= 0 || n <= 0 || m > kMaxSkinnyM || n > 0x7fffffff) return 0;
    return head_layout(m, n).total;
}

int bitnet_greedy_head(const uint8_t* head, float s_head, int64_t n, int64_t k, const int8_t* q,
                       const float* act_scale, const int32_t* act_sum, int64_t m, const int32_t* hist,
                       int64_t hist_stride, const int32_t* hist_len, float penalty, float* logits,
                       int32_t* next_token, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!head || !q || !act_scale || !act_sum || !next_token || !workspace) return BL_ERR_NULL;
    if (hist_stride > 0 && (!hist || !hist_len)) return BL_ERR_NULL;
    if (m < 1 || m > kMaxSkinnyM || !dim_ok(n) || n > 0x7fffffff || !k_ok(k) || hist_stride < 0 ||
        hist_stride > 0x7fffffff)
        return BL_ERR_SHAPE;
    if (!aligned(head, 16) || !aligned(q, 16) || !aligned(act_scale, 4) || !aligned(act_sum, 4) ||
        !aligned(next_token, 4) || (logits && !aligned(logits, 4)) || (hist && !aligned(hist, 4)) ||
        (hist_len && !aligned(hist_len, 4)) || !aligned(workspace, 256))
        return BL_ERR_ALIGN;
    if (!(s_head > 0.0f) || !(s_head < INFINITY) || !(penalty > 0.0f) || !(penalty < INFINITY)) return BL_ERR_VALUE;
    if (workspace_bytes < bitnet_greedy_head_workspace_bytes(m, n)) return BL_ERR_WORKSPACE;
    return greedy_head_launch(head, s_head, n, k, q, act_scale, act_sum, m, hist, hist_stride, hist_len, penalty,
                              logits, next_token, workspace, as_stream(stream));
}

size_t bitnet_greedy_step_workspace_bytes(int64_t m, int64_t d, int64_t f, int64_t vocab)
{
    if (m <= 0 || d <= 0 || f <= 0 || vocab <= 0 || m > kMaxSkinnyM || vocab > 0x7fffffff) return 0;
    return step_layout(m, d, f, vocab).total;
}

int bitnet_greedy_step(const uint8_t* embed_table, float s_emb, int64_t vocab, const uint8_t* weights,
                       const float* scales, const float* gains, const float* z, int64_t n_layers, int64_t d,
                       int64_t f, float eps, const float* g_final, const uint8_t* head, float s_head, int32_t* tokens,
                       int64_t m, int32_t* hist, int64_t hist_stride, int32_t* hist_len, float penalty, float* x,
                       float* logits, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!embed_table || !weights || !scales || !gains || !z || !g_final || !head || !tokens || !x || !workspace)
        return BL_ERR_NULL;
    if (hist_stride > 0 && (!hist || !hist_len)) return BL_ERR_NULL;
    if (m < 1 || m > kMaxSkinnyM || !dim_ok(vocab) || vocab > 0x7fffffff || !dim_ok(n_layers) || !k_ok(d) ||
        !k_ok(f) || d > kMaxGemvK || f > kMaxGemvK || hist_stride < 0 || hist_stride > 0x7fffffff)
        return BL_ERR_SHAPE;
    if (!aligned(embed_table, 16) || !aligned(head, 16) || !aligned(g_final, 16) || !aligned(tokens, 4) ||
        !aligned(x, 16) || (logits && !aligned(logits, 4)) || (hist && !aligned(hist, 4)) ||
        (hist_len && !aligned(hist_len, 4)) || !aligned(workspace, 256))
        return BL_ERR_ALIGN;
    if (!(s_emb > 0.0f) || !(s_emb < INFINITY) || !(s_head > 0.0f) || !(s_head < INFINITY) || !(penalty > 0.0f) ||
        !(penalty < INFINITY))
        return BL_ERR_VALUE;
    if (workspace_bytes < bitnet_greedy_step_workspace_bytes(m, d, f, vocab)) return BL_ERR_WORKSPACE;
    const StepLayout L = step_layout(m, d, f, vocab);
    const hipStream_t s = as_stream(stream);
    // 1. embedding of the current tokens; the same launch builds the head's
    // penalty bitmaps (the histories do not change before the head reads them)
    const bl::PenaltyRows pen = {hist, (int)hist_stride, hist_len,
                                 at<uint32_t>(at<void>(workspace, L.head), head_layout(m, vocab).bits)};
    int rc = bl::launch_embed(embed_table, s_emb, (int)vocab, (int)d, tokens, (int)m, x, s, &pen);
    if (rc) return rc;
    // 2. the layer stream over x, in place (its own checks run here)
    rc = bitnet_decode_stream(weights, scales, gains, z, n_layers, m, d, f, eps, x, nullptr,
                              at<void>(workspace, L.stream), stream_layout(m, d, f).total, stream);
    if (rc) return rc;
    // 3. final RMSNorm + quant, 4. penalised LM head + greedy choice into tokens,
    // 5. the chosen tokens join the histories (the next step embeds them): in the
    // launch that reduces the head's keys
    int32_t* app_hist = hist_stride > 0 ? hist : nullptr;
    int32_t* app_len = hist_stride > 0 ? hist_len : nullptr;
    if (m == 1 && bl::fwd_fits(1, (int)d)) {
        // one sequence: the final norm + quant runs inside the head's launch
        const HeadLayout HL = head_layout(m, vocab);
        void* hws = at<void>(workspace, L.head);
        int tiles = 0;
        rc = bl::launch_head_block(x, g_final, eps, head, s_head, (int)vocab, (int)d, at<uint32_t>(hws, HL.bits),
                                   penalty, logits, at<unsigned long long>(hws, HL.keys), (int)((vocab + 31) / 32),
                                   &tiles, s);
        if (rc) return rc;
        return bl::launch_tile_argmax(at<unsigned long long>(hws, HL.keys), tiles, 1, tokens, s, app_hist,
                                      (int)hist_stride, app_len);
    }
    int8_t* qf = at<int8_t>(workspace, L.q);
    float* sf = at<float>(workspace, L.s);
    int32_t* qsf = at<int32_t>(workspace, L.qs);
    rc = bl::launch_quant_act(x, g_final, eps, (int)m, (int)d, qf, sf, qsf, s);
    if (rc) return rc;
    return greedy_head_launch(head, s_head, vocab, d, qf, sf, qsf, m, hist, hist_stride, hist_len, penalty, logits,
                              tokens, at<void>(workspace, L.head), s, true, app_hist, app_len);
}

// ---- top-k and nucleus sampling --------------------------------------------------

size_t bitnet_sample_workspace_bytes(int64_t m, int64_t n)
{
    if (m <= 0 || n <= 0 || m > 0x7fffffff || n >= (int64_t)1 << 23) return 0;
    return bl::sample_workspace_bytes((int)m, (int)n);
}

namespace {

int sample_check(const float* logits, int64_t m, int64_t n, float temperature, const double* u, const int32_t* token,
                 const void* workspace, size_t workspace_bytes)
{
    if (!logits || !u || !token || !workspace) return BL_ERR_NULL;
    // n < 2^23: a total weight of n tokens of at most 2^40 each fits in an int64
    if (!dim_ok(m) || !dim_ok(n) || m > 0x7fffffff || n >= (int64_t)1 << 23) return BL_ERR_SHAPE;
    if (!aligned(logits, 4) || !aligned(u, 8) || !aligned(token, 4) || !aligned(workspace, 256)) return BL_ERR_ALIGN;
    if (!(temperature > 0.0f) || !(temperature < INFINITY)) return BL_ERR_VALUE;
    if (workspace_bytes < bitnet_sample_workspace_bytes(m, n)) return BL_ERR_WORKSPACE;
    return BL_OK;
}

}  // namespace

int bitnet_sample_topk(const float* logits, int64_t m, int64_t n, int64_t k, float temperature, const double* u,
                       int32_t* token, void* workspace, size_t workspace_bytes, void* stream)
{
    const int rc = sample_check(logits, m, n, temperature, u, token, workspace, workspace_bytes);
    if (rc != BL_OK) return rc;
    if (k < 1) return BL_ERR_VALUE;
    const int kk = (int)std::min<int64_t>(k, n);
    return bl::launch_sample(false, logits, (int)m, (int)n, kk, 1.0f, temperature, u, token, workspace, as_stream(stream));
}

int bitnet_sample_topp(const float* logits, int64_t m, int64_t n, float p, float temperature, const double* u,
                       int32_t* token, void* workspace, size_t workspace_bytes, void* stream)
{
    const int rc = sample_check(logits, m, n, temperature, u, token, workspace, workspace_bytes);
    if (rc != BL_OK) return rc;
    if (!(p > 0.0f) || !(p < INFINITY)) return BL_ERR_VALUE;
    return bl::launch_sample(true, logits, (int)m, (int)n, 1, p, temperature, u, token, workspace, as_stream(stream));
}

}  // extern "C"
