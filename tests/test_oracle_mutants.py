"""The pins catch plausible mistakes: each mutant below plants one mistake in a
temporary copy of the oracle (C source or Python composition) and at least one
pin must fail on it. Runs on the CPU only; the real oracle is never modified."""
import importlib.util
import os
import subprocess
import sys

import pytest

import oracle
from oracle_pins import ALL_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C_SRC = os.path.join(ROOT, "oracle", "bitlinear_oracle.c")
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")

# (name, original text, planted text) in bitlinear_oracle.c
C_MUTANTS = [
    ("pack_code_flip", "(unsigned)(t[r * k + 4 * i + j] + 1)", "(unsigned)(1 - t[r * k + 4 * i + j])"),
    ("pack_field_order", "byte |= code << (2 * j);", "byte |= code << (6 - 2 * j);"),
    ("unpack_sign", "(int8_t)((int)code - 1)", "(int8_t)(1 - (int)code)"),
    ("unpack_accepts_code3", "if (code == 3u) return -4;", "if (code == 4u) return -4;"),
    ("aq_round_half_away", "float r = nearbyintf(v);\n            if (r > 127.0f)",
     "float r = roundf(v);\n            if (r > 127.0f)"),
    ("aq_scale_128", "float scale = 127.0f /", "float scale = 128.0f /"),
    ("aq_no_abs", "float a = fabsf(yr[i]);", "float a = yr[i];"),
    ("aq_qsum_positive_only", "sum += qi;", "sum += (qi > 0 ? qi : 0);"),
    ("aq_floor_missing", "float scale = 127.0f / (amax > floor_ ? amax : floor_);",
     "float scale = 127.0f / (amax > 0.0f ? amax : 1.0f);"),
    ("sumsq_drop_last", "for (int64_t i = 0; i < k; i++) {\n        double v",
     "for (int64_t i = 0; i + 1 < k; i++) {\n        double v"),
    ("sumsq_64_partials", "p[i % ORACLE_PARTIALS] += v * v;", "p[i % 64] += v * v;"),
    ("sumsq_descending_butterfly", "for (int off = 1; off < ORACLE_PARTIALS; off *= 2) {",
     "for (int off = ORACLE_PARTIALS / 2; off >= 1; off /= 2) {"),
    ("rms_no_mean", "sqrt(ss / (double)k + (double)eps)", "sqrt(ss + (double)eps)"),
    ("rms_no_eps", "sqrt(ss / (double)k + (double)eps)", "sqrt(ss / (double)k)"),
    ("rms_no_sqrt", "1.0 / sqrt(ss / (double)k + (double)eps)", "1.0 / (ss / (double)k + (double)eps)"),
    ("rms_no_gain", "y[row * k + i] = a * g[i];", "y[row * k + i] = a;"),
    ("wq_absmax", "sum += fabs((double)w[i]);", "sum = fmax(sum, fabs((double)w[i]));"),
    ("wq_no_clamp", "if (r > 1.0f) r = 1.0f;", "if (r > 2.0f) r = 2.0f;"),
    ("wq_round_half_away", "float r = nearbyintf(v);\n        if (r > 1.0f)", "float r = roundf(v);\n        if (r > 1.0f)"),
    ("mm_transposed_out", "acc[row * n + col] = s;", "acc[col * m + row] = s;"),
    ("mm_wrong_k", "s += (int32_t)tr[i] * (int32_t)qr[i];", "s += (int32_t)tr[i] * (int32_t)qr[k - 1 - i];"),
    ("dq_inverted", "float inv = 1.0f / prod;", "float inv = prod;"),
    ("dq_no_sw", "float prod = s_a[row] * s_w;", "float prod = s_a[row];"),
    ("dq_row0_scale", "float prod = s_a[row] * s_w;", "float prod = s_a[0] * s_w;"),
    ("relu_not_squared", "float g2 = g * g;", "float g2 = g;"),
    ("relu_on_up", "h[i] = g2 * up[i];", "h[i] = g2 * (up[i] > 0.0f ? up[i] : 0.0f);"),
    ("relu_missing", "float g = gate[i] > 0.0f ? gate[i] : 0.0f;", "float g = gate[i];"),
    ("argmax_last_tie", "if (a[col] > a[best]) best = col;", "if (a[col] >= a[best]) best = col;"),
    ("residual_sub", "x[i] = x[i] + d[i];", "x[i] = x[i] - d[i];"),
    # floating-point operation order (caught by the exact-rational pins)
    ("dq_recip_product", "float inv = 1.0f / prod;", "float inv = (1.0f / s_a[row]) * (1.0f / s_w);"),
    ("dq_divide", "y[row * n + col] = (float)acc[row * n + col] * inv;",
     "y[row * n + col] = (float)acc[row * n + col] / prod;"),
    ("dq_inv_fp64", "float inv = 1.0f / prod;", "float inv = (float)(1.0 / ((double)s_a[row] * (double)s_w));"),
    ("rms_r_times_g", "float a = xr[i] * r;\n            y[row * k + i] = a * g[i];",
     "y[row * k + i] = xr[i] * (r * g[i]);"),
    ("rms_xr_fp64", "float a = xr[i] * r;", "float a = (float)((double)xr[i] * r64);"),
    ("rms_apply_fp64", "float a = xr[i] * r;\n            y[row * k + i] = a * g[i];",
     "y[row * k + i] = (float)((double)xr[i] * (double)r * (double)g[i]);"),
    ("relu2_order", "float g2 = g * g;\n        h[i] = g2 * up[i];", "h[i] = (g * up[i]) * g;"),
    ("relu2_fp64", "float g2 = g * g;\n        h[i] = g2 * up[i];", "h[i] = (float)((double)g * g * up[i]);"),
    ("aq_scale_fp64_in_product", "float v = yr[i] * scale;",
     "float v = (float)((double)yr[i] * (127.0 / (double)(amax > floor_ ? amax : floor_)));"),
    ("aq_round_exact_product", "float r = nearbyintf(v);\n            if (r > 127.0f)",
     "float r = (float)nearbyint((double)yr[i] * (double)scale);\n            if (r > 127.0f)"),
    ("aq_div_then_mul", "float v = yr[i] * scale;", "float v = yr[i] / (amax > floor_ ? amax : floor_) * 127.0f;"),
    # embedding lookup
    ("emb_no_scale", "x[r * d + k] = (float)t[k] / s_e;", "x[r * d + k] = (float)t[k];"),
    ("emb_times_scale", "x[r * d + k] = (float)t[k] / s_e;", "x[r * d + k] = (float)t[k] * s_e;"),
    ("emb_wrong_row", "rc = ref_unpack(table + tok * (d / 4), 1, d, t);",
     "rc = ref_unpack(table + (tok ^ 1) % vocab * (d / 4), 1, d, t);"),
    ("emb_negative_zero", "for (int64_t k = 0; k < d; k++) x[r * d + k] = 0.0f;",
     "for (int64_t k = 0; k < d; k++) x[r * d + k] = -0.0f;"),
    # repetition penalty and greedy choice
    ("pen_directions_swapped", "l[v] = l[v] > 0.0f ? l[v] / penalty : l[v] * penalty;",
     "l[v] = l[v] > 0.0f ? l[v] * penalty : l[v] / penalty;"),
    ("pen_always_divide", "l[v] = l[v] > 0.0f ? l[v] / penalty : l[v] * penalty;", "l[v] = l[v] / penalty;"),
    ("pen_every_occurrence", "if (v < 0 || v >= n || seen[v]) continue;", "if (v < 0 || v >= n) continue;"),
    ("pen_last_tie", "if (l[c] > l[best]) best = c;\n        idx[r]", "if (l[c] >= l[best]) best = c;\n        idx[r]"),
    ("pen_whole_stride", "int64_t len = hist_len ? hist_len[r] : 0;", "int64_t len = hist_stride;"),
    # top-k / nucleus sampling
    ("smp_sort_ascending", "if (la != lb) return la > lb ? -1 : 1;", "if (la != lb) return la < lb ? -1 : 1;"),
    ("smp_ties_high_first", "return a < b ? -1 : (a > b ? 1 : 0);", "return a > b ? -1 : (a < b ? 1 : 0);"),
    ("smp_temperature_times", "((double)l[i] - (double)lmax) / (double)temperature;",
     "((double)l[i] - (double)lmax) * (double)temperature;"),
    ("smp_nucleus_excludes_crossing", "while (kept < n && cum < target) cum += w[order[kept++]];",
     "while (kept < n && cum + w[order[kept]] < target) cum += w[order[kept++]];\n            if (kept == 0) kept = 1;"),
    ("smp_topk_one_more", "kept = k < n ? k : n;", "kept = k < n ? k + 1 : n;"),
    ("smp_cum_ge", "if (cum > r) {", "if (cum >= r) {"),
    ("smp_exp_no_tail", "const double r = (x - k * ORACLE_LN2_HEAD) - k * ORACLE_LN2_TAIL;",
     "const double r = x - k * ORACLE_LN2_HEAD;"),
    # rotary embedding and attention
    ("rope_sign", "x[2 * i + 1] = as + bc;", "x[2 * i + 1] = bc - as;"),
    ("rope_theta_half", "const double theta = pow(base, -(double)(2 * i) / (double)hd);",
     "const double theta = pow(base, -(double)(i) / (double)hd);"),
    ("attn_no_scale", "sc[j] = dot * scale;", "sc[j] = dot;"),
    ("attn_drops_current", "for (int64_t j = 0; j <= pos; j++) {\n                const double e",
     "for (int64_t j = 0; j < pos; j++) {\n                const double e"),
    ("attn_head0_keys", "const float *K = k_cache + ((r * heads + h) * max_seq) * hd;",
     "const float *K = k_cache + ((r * heads) * max_seq) * hd;"),
    ("smp_exp_short_series", "for (int j = 12; j >= 0; j--) poly = poly * r + inv_fact[j];",
     "for (int j = 12; j >= 0; j--) poly = poly * r + (j > 7 ? 0.0 : inv_fact[j]);"),
]

# Equivalent rewrites, not mutants: they give the same bits on every input, so
# no pin can (or should) tell them apart. s_a = (float)(127.0 / (double)amax) is
# the correctly rounded fp32 quotient (a double-precision quotient rounded to
# single is exact-rounded: 53 >= 2 * 24 + 2), and (double)y * (double)s_a is the
# exact product of two floats, so rounding it to float equals the fp32 product.

# (name, original, planted) in oracle/__init__.py
PY_MUTANTS = [
    ("ffn_no_subnorm", "q2, s2, qs2 = quant_act(h, sub_norm_gain, eps, lib)", "q2, s2, qs2 = quant_act(h, None, eps, lib)"),
    ("ffn_gate_up_swapped", "h = relu2_mul(gate, up, lib)", "h = relu2_mul(up, gate, lib)"),
    ("ffn_up_uses_gate_w", "up, acc_up = bitlinear(w_up, s_up, d, q1, s1, lib)",
     "up, acc_up = bitlinear(w_gate, s_up, d, q1, s1, lib)"),
    ("ffn_no_norm", "q1, s1, qs1 = quant_act(x, norm_gain, eps, lib)", "q1, s1, qs1 = quant_act(x, None, eps, lib)"),
    ("layer_no_residual_o",
     "quant_act(lw[\"z\"], lw[\"g_attn_sub\"], eps, lib)\n    yo, _ = bitlinear(lw[\"wo\"], lw[\"so\"], d, o_in, so, lib)\n"
     "    x = residual_add(x, yo, lib)\n",
     "quant_act(lw[\"z\"], lw[\"g_attn_sub\"], eps, lib)\n    yo, _ = bitlinear(lw[\"wo\"], lw[\"so\"], d, o_in, so, lib)\n"
     "    x = x\n"),
    ("layer_o_reads_x", "o_in, so, _ = quant_act(lw[\"z\"], lw[\"g_attn_sub\"], eps, lib)",
     "o_in, so, _ = quant_act(x, lw[\"g_attn_sub\"], eps, lib)"),
    ("layer_ffn_from_old_x",
     "quant_act(lw[\"z\"], lw[\"g_attn_sub\"], eps, lib)\n    yo, _ = bitlinear(lw[\"wo\"], lw[\"so\"], d, o_in, so, lib)\n"
     "    x = residual_add(x, yo, lib)\n    f = ffn(x, lw[\"g_ffn\"]",
     "quant_act(lw[\"z\"], lw[\"g_attn_sub\"], eps, lib)\n    yo, _ = bitlinear(lw[\"wo\"], lw[\"so\"], d, o_in, so, lib)\n"
     "    x = residual_add(x, yo, lib)\n    f = ffn(x - yo, lw[\"g_ffn\"]"),
    ("attn_layer_no_residual_o",
     "o_in, so, _ = quant_act(use, lw[\"g_attn_sub\"], eps, lib)\n    yo, _ = bitlinear(lw[\"wo\"], lw[\"so\"], d, o_in, so, lib)\n"
     "    x = residual_add(x, yo, lib)\n",
     "o_in, so, _ = quant_act(use, lw[\"g_attn_sub\"], eps, lib)\n    yo, _ = bitlinear(lw[\"wo\"], lw[\"so\"], d, o_in, so, lib)\n"
     "    x = x\n"),
    ("attn_layer_o_reads_x", "o_in, so, _ = quant_act(use, lw[\"g_attn_sub\"], eps, lib)",
     "o_in, so, _ = quant_act(x, lw[\"g_attn_sub\"], eps, lib)"),
    ("layer_q_uses_wk", "    d = x.shape[1]\n    a, sa, _ = quant_act(x, lw[\"g_attn\"], eps, lib)\n"
     "    yq, _ = bitlinear(lw[\"wq\"], lw[\"sq\"], d, a, sa, lib)",
     "    d = x.shape[1]\n    a, sa, _ = quant_act(x, lw[\"g_attn\"], eps, lib)\n"
     "    yq, _ = bitlinear(lw[\"wk\"], lw[\"sq\"], d, a, sa, lib)"),
    ("attn_layer_q_uses_wk", "    hd = d // heads\n    a, sa, _ = quant_act(x, lw[\"g_attn\"], eps, lib)\n"
     "    yq, _ = bitlinear(lw[\"wq\"], lw[\"sq\"], d, a, sa, lib)",
     "    hd = d // heads\n    a, sa, _ = quant_act(x, lw[\"g_attn\"], eps, lib)\n"
     "    yq, _ = bitlinear(lw[\"wk\"], lw[\"sq\"], d, a, sa, lib)"),
    ("attn_layer_k_unrotated", "k_cache[:, :, pos, :] = k_rot", "k_cache[:, :, pos, :] = yk.reshape(m, heads, hd)"),
    ("attn_layer_v_rotated", "v_cache[:, :, pos, :] = yv.reshape(m, heads, hd)", "v_cache[:, :, pos, :] = k_rot"),
]


def _any_pin_fails(o, lib):
    for pin in ALL_PINS:
        try:
            pin(o, lib)
        except Exception:  # AssertionError, or an error the mistake provokes
            return pin.__name__
    return None


@pytest.mark.parametrize("name,old,new", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_mutant_caught(name, old, new, tmp_path):
    src = open(C_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", str(mut),
                    "-o", str(so), "-lm"], check=True)
    lib = oracle.load(str(so))
    caught = _any_pin_fails(oracle, lib)
    assert caught, f"no pin caught mutant {name}"


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_py_mutant_caught(name, old, new, olib):
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    modname = f"oracle_mutant_{name}"
    spec = importlib.util.spec_from_loader(modname, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__dict__["__file__"] = PY_SRC
    exec(compile(src.replace(old, new), f"<{modname}>", "exec"), mod.__dict__)
    sys.modules.pop(modname, None)
    caught = _any_pin_fails(mod, olib)
    assert caught, f"no pin caught mutant {name}"
