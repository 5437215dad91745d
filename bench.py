#!/usr/bin/env python3
"""Benchmark of the BitNet b1.58 BitLinear hot path on one MI355X.

Timed step: one decode token through the full BitNet-3B BitLinear stream --
32 layers x 7 BitLinears (q, k, v, o 2560x2560; gate, up 2560->10240; down
10240->2560), each behind its RMSNorm + activation quant, with the ReLU^2 x up
gating and the residual adds; attention math is left out (the o projection
reads a seeded stand-in). 838,860,800 bytes of packed ternary weights are
streamed per step, so the headline value is the weight-stream rate in GB/s
(with ms/token beside it).

Also reported in the same JSON line:
  prefill  : activation quant of 2048 x 2560 fp32 tokens (1% outliers x20), then
             the int8-MFMA GEMM against 10240 x 2560 ternary weights -> fp32;
             int8 TOPS of the GEMM (2 M N K per call) and of quant + GEMM.
  batched  : BitNet-1.3B stream at 32 tokens (24 layers x 7 BitLinears), then
             the final norm + quant and the ternary LM head 2048 -> 50000 with
             the fused per-row argmax.
  gemv     : one 2560 -> 2560 BitLinear (quant + GEMV, bitlinear_forward) at 1 token.
  ffn      : the BitNet-3B FFN sub-layer at 1 token.
  roofline : the dominant kernel against HBM or MFMA peak.
  cpu_baseline : the CPU oracle on a bounded sample of the same workload.

Inputs are synthetic and seeded (workloads.py): ternary weights with
P(-1) = P(+1) = 0.3, scales U(20, 60), activations N(0, 1), unit gains.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
METRIC = "BitLinear decode weight-stream GB/s + ms/token (3B shapes); prefill int8 TOPS"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ensure_built():
    lib = os.path.join(ROOT, "bitlinear_amd", "libbitlinear.so")
    olib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not (os.path.exists(lib) and os.path.exists(olib)):
        import __graft_entry__
        __graft_entry__.build()


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.s.record()
        return self

    def __exit__(self, *a):
        self.e.record()
        self.e.synchronize()
        self.ms = self.s.elapsed_time(self.e)


def build_stream(bl, workload, n_layers, d, f, m, T):
    """Seeded layers packed with the library's host packer and uploaded as one
    resident blob. Returns host copies for the oracle too."""
    blobs, scales, gains, zs, host_layers = [], [], [], [], []
    for l in range(n_layers):
        raw = W.layer_inputs(workload, l, d, f, m, bench_gains=True)
        lw = {}
        for name, sname in zip(W.LINEAR_NAMES, W.SCALE_NAMES):
            lw[name] = bl.bitlinear_pack(raw[name])
            lw[sname] = raw[sname]
            blobs.append(lw[name].reshape(-1))
        for key in ("g_attn", "g_attn_sub", "g_ffn", "g_ffn_sub", "z"):
            lw[key] = raw[key]
        scales.append(np.array([raw[s] for s in W.SCALE_NAMES], np.float32))
        gains.append(np.concatenate([raw["g_attn"], raw["g_attn_sub"], raw["g_ffn"], raw["g_ffn_sub"]]))
        zs.append(raw["z"])
        host_layers.append(lw)
        del raw
    dev = dict(weights=T(np.concatenate(blobs)), scales=T(np.stack(scales)), gains=T(np.stack(gains)),
               z=T(np.stack(zs)))
    return dev, host_layers


def run_stream_step(bl, dev, n_layers, m, d, f, x, qkv, ws):
    bl.bitnet_decode_stream(dev["weights"], dev["scales"], dev["gains"], dev["z"], n_layers, m, d, f, 1e-5, x, qkv, ws)


# HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE, each scaled by the
# factor the same counter gives for a plain 512 MiB device copy (FETCH_SIZE x 2.0,
# WRITE_SIZE x 1.0); summaries in profiles/. Each entry holds the sha256 of the
# kernel sources it was measured on: once they change the figure no longer
# describes the kernel and is reported as null.
TRAFFIC_BYTES_PER_LAUNCH = {
    "stream_3b": {"bytes": 886819440,
                  "sources": {"bitlinear_amd/csrc/stream.hip":
                              "e645a874de944912ab7870c8f1f190762db1d11eb25b167ab15ab344e98b6faf",
                              "bitlinear_amd/csrc/prefetch.h":
                              "e07403f1545fce716dbaf7fef4eca8d1c39dc6219697959362bb28e7a103b074",
                              "bitlinear_amd/csrc/wave.h":
                              "c69e873099defc85d5684275fbfcce86285892ceef0209e5a6afd9ff57cb9c81"}},
}


def traffic_bytes(key):
    """Counter-derived bytes for `key`, or None if its sources changed since."""
    import hashlib
    e = TRAFFIC_BYTES_PER_LAUNCH.get(key)
    if e is None:
        return None
    for rel, digest in e["sources"].items():
        with open(os.path.join(ROOT, rel), "rb") as fh:
            if hashlib.sha256(fh.read()).hexdigest() != digest:
                return None
    return e["bytes"]


def stream_is_persistent(ws):
    """The persistent one-token path advances the phase counter in the workspace."""
    import torch
    torch.cuda.synchronize()
    return int(ws[:4].view(torch.int32).item()) != 0


def copy_probe():
    import torch
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    with Timer() as tm:
        for _ in range(20):
            dst.copy_(src)
    print(json.dumps({"copy_bytes_each_way": n, "ms_per_copy": tm.ms / 20,
                      "gbs_read_plus_write": 2 * n / (tm.ms / 20 * 1e-3) / 1e9}), flush=True)


def omp_threads():
    v = os.environ.get("OMP_NUM_THREADS")
    return int(v) if v and v.isdigit() else os.cpu_count()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def per_call_stats(torch, fn, iters):
    """fn() run iters times with a HIP event pair around each call on the
    current stream (the one the library launches on). Returns the per-call
    median and the 10th / 90th percentiles in ms."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for s, e in evs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    t = np.array([s.elapsed_time(e) for s, e in evs])
    return {"median_ms": round(float(np.median(t)), 5), "p10_ms": round(float(np.percentile(t, 10)), 5),
            "p90_ms": round(float(np.percentile(t, 90)), 5), "calls": iters}


def probe_peaks(bl, torch, dev0):
    """Measured ceilings: the HBM read-stream probe over 4 GiB and the
    int8-MFMA-only probe (best of a few runs each)."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev0)
    buf = torch.ones(4 << 30, dtype=torch.uint8, device=dev0)
    bl.bitlinear_probe_read(buf, sink)
    best = 0.0
    for _ in range(5):
        with Timer() as t:
            nb = bl.bitlinear_probe_read(buf, sink)
        best = max(best, nb / (t.ms * 1e-3) / 1e9)
    del buf
    iters = 20000
    tops = {}
    for name, fn in (("int8_mfma_tops", bl.bitlinear_probe_mfma_i8),
                     ("int8_mfma_tops_dense", bl.bitlinear_probe_mfma_i8_dense)):
        fn(100, sink)
        best_ops = 0.0
        for _ in range(3):
            with Timer() as t:
                ops = fn(iters, sink)
            best_ops = max(best_ops, ops / (t.ms * 1e-3) / 1e12)
        tops[name] = round(best_ops, 1)
    torch.cuda.synchronize()
    return {"hbm_read_gbs": round(best, 1), **tops,
            "how": "bitlinear_probe_read over 4 GiB (best of 5); bitlinear_probe_mfma_i8, 2 waves per SIMD x "
                   "8 independent v_mfma_i32_16x16x64_i8 chains on one pair of small operands (best of 3); "
                   "bitlinear_probe_mfma_i8_dense, the same with each chain on its own random operand bytes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="only the headline decode stream")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 512 MiB device copy (calibrates rocprof byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only; there is no multi-GPU path (run with --gpus 1)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return
    ensure_built()
    import torch
    import bitlinear_amd as bl
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev0 = torch.device("cuda:0")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev0)

    # ---- headline: BitNet-3B decode stream, 1 token ------------------------------------
    cfg = W.BITNET_3B
    L, d, f, m = cfg["layers"], cfg["dim"], cfg["ffn"], 1
    t0 = time.perf_counter()
    dev, host_layers = build_stream(bl, W.W_STREAM, L, d, f, m, T)
    weight_bytes = L * bl.bitnet_layer_bytes(d, f)
    log(f"3B stream inputs ready in {time.perf_counter() - t0:.1f}s ({weight_bytes} packed weight bytes)")
    x0 = W.activations(W.rng(W.W_STREAM, 999, W.T_X), m, d)
    x = T(x0)
    qkv = torch.empty((L, m, 3 * d), dtype=torch.float32, device=dev0)
    ws = torch.zeros(bl.bitnet_stream_workspace_bytes(m, d, f), dtype=torch.uint8, device=dev0)

    # first step from x0, checked against the oracle below (same inputs)
    run_stream_step(bl, dev, L, m, d, f, x, qkv, ws)
    torch.cuda.synchronize()
    x_first = x.cpu().numpy()
    qkv_first = qkv.cpu().numpy()

    for _ in range(args.warmup):
        run_stream_step(bl, dev, L, m, d, f, x, qkv, ws)
    torch.cuda.synchronize()
    # the timed region: exactly K steps back to back, one event pair around
    # them all (an event recorded between two steps puts a marker on the
    # stream that delays the next launch by about 15 us)
    tw0 = time.perf_counter()
    with Timer() as tm:
        for i in range(args.steps):
            run_stream_step(bl, dev, L, m, d, f, x, qkv, ws)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - tw0) * 1e3
    # the per-step distribution from a second pass of K steps, an event pair
    # around each (outside the timed region)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for i in range(args.steps):
        step_ev[i][0].record()
        run_stream_step(bl, dev, L, m, d, f, x, qkv, ws)
        step_ev[i][1].record()
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in step_ev])
    status = int(ws[4:8].view(torch.int32).item())
    if status != 0:
        raise RuntimeError(f"decode stream status word {status}: the persistent kernel gave up; timing is void")
    ms_per_step = wall_ms / args.steps
    ev_ms_per_step = tm.ms / args.steps
    value = weight_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"decode stream: {ms_per_step:.4f} ms/token wall, {ev_ms_per_step:.4f} ms/token events, {value:.1f} GB/s")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded ternary weights, N(0,1) activations)",
        "config": {"workload": "BitNet-3B decode weight stream: 32 layers x 7 BitLinears, 1 token, "
                               "attention math excluded", "layers": L, "dim": d, "ffn": f, "tokens": m,
                   "weight_bytes_per_step": weight_bytes},
        "ms_per_token": round(ms_per_step, 5),
        "ms_per_step_events": {"mean": round(ev_ms_per_step, 5), "median": round(float(np.median(step_ms)), 5),
                               "p10": round(float(np.percentile(step_ms, 10)), 5),
                               "p90": round(float(np.percentile(step_ms, 90)), 5),
                               "note": "mean: one event pair around the timed steps; median / p10 / p90: a "
                                       "second pass of as many steps with an event pair around each"},
    }

    # roofline of the dominant kernel: at one token the whole stream is one
    # launch of the persistent kernel, so the per-step event time is its duration
    persistent = bl._lib.bitnet_stream_workspace_bytes(m, d, f) > 0 and stream_is_persistent(ws)
    kname = ("stream_kernel<2560, 10240> (one persistent launch per token)" if persistent
             else "bitnet_decode_stream launches of one token")
    achieved = weight_bytes / (ev_ms_per_step * 1e-3) / 1e9
    peaks = probe_peaks(bl, torch, dev0)
    log(f"probes: HBM read {peaks['hbm_read_gbs']} GB/s, int8 MFMA {peaks['int8_mfma_tops']} TOP/s "
        f"({peaks['int8_mfma_tops_dense']} on random operands)")
    result["roofline"] = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                          "traffic": traffic_bytes("stream_3b"),
                          "algorithmic_bytes": weight_bytes,
                          "probe_peak": peaks["hbm_read_gbs"], "frac_of_probe": round(achieved / peaks["hbm_read_gbs"], 4)}
    result["probe_peaks"] = peaks

    # ---- CPU oracle baseline + parity of the first step ----------------------------------
    if not args.no_cpu:
        import oracle
        olib = oracle.load()
        tc0 = time.perf_counter()
        ox, oqkv = oracle.chain(x0, host_layers, 1e-5, olib)
        first_s = time.perf_counter() - tc0
        exact = bool(np.array_equal(ox.view(np.uint32), x_first.view(np.uint32)) and
                     all(np.array_equal(oqkv[l].view(np.uint32), qkv_first[l].view(np.uint32)) for l in range(L)))
        rel = float(np.max(np.abs(ox.astype(np.float64) - x_first) / np.maximum(np.abs(ox), 1e-30)))
        tokens, xo = 1, ox
        while time.perf_counter() - tc0 < 10.0 and tokens < 64:  # about 10 s of CPU work
            xo, _ = oracle.chain(xo, host_layers, 1e-5, olib)
            tokens += 1
        cpu_s = time.perf_counter() - tc0
        result["cpu_baseline"] = {"value": round(tokens * weight_bytes / cpu_s / 1e9, 4), "unit": "GB/s",
                                  "cores": oracle.set_threads(0, olib), "kind": "oracle",
                                  "sample": f"{tokens} consecutive tokens of the same 32-layer stream (all 224 "
                                            f"BitLinears each), {cpu_s:.2f} s",
                                  "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
        result["parity_first_step"] = {"bit_exact": exact, "max_rel_err_x": rel}
        log(f"oracle: {first_s:.2f}s for one token, {tokens} tokens in {cpu_s:.2f}s; first GPU step bit-exact: {exact}")
    if not args.no_extra:
        result["greedy"] = greedy_leg(bl, torch, T, dev0, dev, host_layers if not args.no_cpu else None, L, d, f)
        result["decode_with_attention"] = attention_leg(bl, torch, dev0, dev, L, d, f)
    del host_layers

    if not args.no_extra:
        result.update(extra_measurements(bl, torch, T, dev0, check=not args.no_cpu, peaks=peaks))
    if not args.no_cpu:
        result["cpu_single_core"] = single_core_oracle()
    print(json.dumps(result), flush=True)


def attention_leg(bl, torch, dev0, dev, L, d, f):
    """BitNet-3B decode step with attention (bitnet_decode_step; one sequence,
    so the whole step is one persistent launch): 32 heads of 80, caches of 2048
    positions filled with N(0, 1), at positions 128 and 2047. Bytes per token:
    the 838,860,800 weight bytes plus the K and V rows read,
    2 x 32 layers x 2560 x 4 x (pos + 1)."""
    heads, hd, max_seq, m = W.BITNET_3B["heads"], d // W.BITNET_3B["heads"], 2048, 1
    c, s = bl.bitnet_rope_table(10000.0, hd, max_seq)
    cd, sd = torch.from_numpy(c).to(dev0), torch.from_numpy(s).to(dev0)
    gen = torch.Generator(device=dev0)
    gen.manual_seed(2026)
    kc = torch.randn((L, m, heads, max_seq, hd), generator=gen, device=dev0, dtype=torch.float32)
    vc = torch.randn((L, m, heads, max_seq, hd), generator=gen, device=dev0, dtype=torch.float32)
    x = torch.from_numpy(W.activations(W.rng(W.W_STREAM, 998, W.T_X), m, d)).to(dev0)
    ws = torch.zeros(bl.bitnet_decode_step_workspace_bytes(m, d, f, heads, max_seq), dtype=torch.uint8, device=dev0)
    res = {"workload": "BitNet-3B decode step with attention: 32 layers x (q/k/v, RoPE + KV-cache append, "
                       "attention over 0..pos, o, FFN), 1 sequence, 32 heads of 80, one persistent launch per token"}
    for pos in (128, 2047):
        def step():
            bl.bitnet_decode_step(dev["weights"], dev["scales"], dev["gains"], L, m, d, f, heads, 1e-5, cd, sd, pos,
                                  kc, vc, x, None, None, ws)
        for _ in range(2):
            step()
        iters = 10
        with Timer() as t:
            for _ in range(iters):
                step()
        ms = t.ms / iters
        status = int(ws[4:8].view(torch.int32).item())
        if status != 0:
            raise RuntimeError(f"decode step status word {status}: the persistent kernel gave up; timing is void")
        nbytes = L * bl.bitnet_layer_bytes(d, f) + 2 * L * d * 4 * (pos + 1)
        res[f"pos_{pos}"] = {"ms_per_token": round(ms, 4), "bytes_per_token": nbytes,
                             "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del kc, vc
    log(f"decode with attention: {res}")
    return res


def greedy_leg(bl, torch, T, dev0, dev, host_layers, L, d, f):
    """Greedy decoding of one BitNet-3B sequence on the device: per step the
    ternary embedding of the current token, the 32-layer stream, the final
    norm + quant and the 50000-token LM head with a repetition penalty of 1.1
    over the history and the greedy choice, which is appended to the history
    -- bitnet_greedy_step, one submit per token, no host round trip."""
    vocab, m, cap = W.BITNET_3B["vocab"], 1, 256
    ge, gh = W.rng(W.W_STREAM, 0, W.T_EMB), W.rng(W.W_STREAM, 0, W.T_HEAD)
    emb_h, head_h = bl.bitlinear_pack(W.ternary(ge, vocab, d)), bl.bitlinear_pack(W.ternary(gh, vocab, d))
    s_emb, s_head = float(W.weight_scale(ge)), float(W.weight_scale(gh))
    emb, head = T(emb_h), T(head_h)
    gf = T(np.ones(d, np.float32))
    tok0 = W.rng(W.W_STREAM, 0, W.T_TOKENS).integers(0, vocab, m).astype(np.int32)
    tokens = T(tok0)
    hist = torch.zeros((m, cap), dtype=torch.int32, device=dev0)
    hlen = torch.zeros(m, dtype=torch.int32, device=dev0)
    x = torch.empty((m, d), dtype=torch.float32, device=dev0)
    ws = torch.zeros(bl.bitnet_greedy_step_workspace_bytes(m, d, f, vocab), dtype=torch.uint8, device=dev0)

    def step():
        bl.bitnet_greedy_step(emb, s_emb, dev["weights"], dev["scales"], dev["gains"], dev["z"], L, d, f, 1e-5, gf,
                              head, s_head, tokens, hist, hlen, 1.1, x, None, ws)
    n_check = 2
    for _ in range(n_check):
        step()
    torch.cuda.synchronize()
    first = hist[0, :n_check].cpu().numpy().copy()
    steps = 40
    with Timer() as t:
        for _ in range(steps):
            step()
    ms = t.ms / steps
    stats = per_call_stats(torch, step, 20)
    wbytes = L * bl.bitnet_layer_bytes(d, f) + vocab * d // 4 + d // 4
    res = {"workload": "BitNet-3B greedy decoding, 1 sequence: embedding + 32 layers (attention math excluded) + "
                       "final norm + LM head 2560 -> 50000 with repetition penalty 1.1 + argmax + history append, "
                       "one bitnet_greedy_step per token", "ms_per_token": round(ms, 4),
           "tokens_per_s": round(1e3 / ms, 1), "per_step": stats, "weight_bytes_per_token": wbytes,
           "weight_gbs": round(wbytes / (ms * 1e-3) / 1e9, 1)}
    if host_layers is not None:
        import oracle
        olib = oracle.load()
        o_tok, o_hist, o_len = tok0.copy(), np.zeros((m, cap), np.int32), np.zeros(m, np.int32)
        for _ in range(n_check):
            o_tok, o_hist, o_len, _ = oracle.greedy_step(o_tok, emb_h, s_emb, host_layers, np.ones(d, np.float32),
                                                         1e-5, head_h, s_head, o_hist, o_len, 1.1, olib)
        res["parity_first_steps"] = {"steps": n_check, "tokens_match": bool(np.array_equal(first, o_hist[0, :n_check]))}
    log(f"greedy: {ms:.4f} ms/token ({res.get('parity_first_steps')})")
    return res


def sampling_leg(bl, torch, T, dev0, check):
    """Top-k (k = 50) and nucleus (p = 0.9) sampling at temperature 0.8 of 32
    rows of 50000 logits (N(0, 3^2)), with one uniform draw per row."""
    m, n = 32, W.BITNET_3B["vocab"]
    g = W.rng(W.W_BATCHED, 5, 0)
    lh = (g.standard_normal((m, n)) * 3.0).astype(np.float32)
    uh = g.random(m)
    logits, u = T(lh), T(uh)
    tok = torch.empty(m, dtype=torch.int32, device=dev0)
    ws = torch.empty(bl.bitnet_sample_workspace_bytes(m, n), dtype=torch.uint8, device=dev0)
    res = {"workload": "32 rows x 50000 logits, temperature 0.8, one draw per row"}
    for name, fn, param in (("topk_50", bl.bitnet_sample_topk, 50), ("topp_0.9", bl.bitnet_sample_topp, 0.9)):
        for _ in range(3):
            fn(logits, param, 0.8, u, tok, ws)
        iters = 20
        with Timer() as t:
            for _ in range(iters):
                fn(logits, param, 0.8, u, tok, ws)
        entry = {"us_per_call": round(t.ms / iters * 1e3, 2)}
        if check:
            import oracle
            want = (oracle.sample_topk if name.startswith("topk") else oracle.sample_topp)(lh, param, 0.8, uh)
            entry["matches_oracle"] = bool(np.array_equal(tok.cpu().numpy(), want))
        res[name] = entry
    log(f"sampling: {res}")
    return res


def vendor_int8_gemm(torch, dev0, q, t_rows):
    """Context for the prefill GEMM: the library int8 GEMM of this PyTorch build
    (torch._int_mm, hipBLASLt on ROCm) on the same M x K activations against an
    int8 [N][K] weight matrix (ternary values, one byte each), y = q . W^T in
    int32. Not the same product (no 2-bit weights, no dequant), the same MFMA
    work."""
    M, K = q.shape
    gen = torch.Generator(device=dev0)
    gen.manual_seed(7)
    wt = torch.randint(-1, 2, (t_rows, K), generator=gen, device=dev0, dtype=torch.int8)
    try:
        def call():
            return torch._int_mm(q, wt.t())
        for _ in range(3):
            call()
        iters = 20
        with Timer() as tv:
            for _ in range(iters):
                call()
        ms = tv.ms / iters
        res = {"call": "torch._int_mm(q [M][K] int8, W^T) with W [N][K] int8", "ms": round(ms, 4),
               "tops": round(2.0 * M * t_rows * K / (ms * 1e-3) / 1e12, 1)}
    except Exception as ex:  # an op this build lacks is reported, not fatal
        res = {"call": "torch._int_mm", "error": str(ex)[:200]}
    del wt
    return res


def prefill_ffn_leg(bl, torch, T, dev0, check):
    """The FFN sub-layer at 2048 tokens (d = 2560, f = 10240): quant of x, the
    paired gate/up MFMA GEMM with relu(gate)^2 * up in its epilogue, sub-norm +
    quant of h, down GEMM. 2 M (2 d f + f d) int8 operations per call."""
    M, d, f = 2048, 2560, 10240
    gg = [W.rng(W.W_PREFILL, 1, tid) for tid in (W.T_GATE, W.T_UP, W.T_DOWN)]
    packs = [bl.bitlinear_pack(W.ternary(gx, n, k)) for gx, (n, k) in zip(gg, ((f, d), (f, d), (d, f)))]
    scales = [float(W.weight_scale(gx)) for gx in gg]
    pw = [T(pk) for pk in packs]
    xh = W.activations(W.rng(W.W_PREFILL, 1, W.T_X), M, d, outliers=True)
    x = T(xh)
    gn, gs = T(np.ones(d, np.float32)), T(np.ones(f, np.float32))
    o = torch.empty((M, d), dtype=torch.float32, device=dev0)
    ws = torch.empty(bl.bitnet_ffn_workspace_bytes(M, d, f), dtype=torch.uint8, device=dev0)

    def call():
        bl.bitnet_ffn(x, M, d, f, gn, gs, 1e-5, pw[0], scales[0], pw[1], scales[1], pw[2], scales[2], None, o, ws)
    for _ in range(3):
        call()
    iters = 10
    with Timer() as t:
        for _ in range(iters):
            call()
    ms = t.ms / iters
    stats = per_call_stats(torch, call, iters)
    ops = 2.0 * M * (2 * d * f + f * d)
    tops = ops / (ms * 1e-3) / 1e12
    res = {"workload": "BitNet-3B FFN at 2048 tokens: quant(x) -> paired gate/up MFMA GEMM with relu(gate)^2 x up "
                       "epilogue -> sub-norm + quant(h) -> down GEMM", "ms": round(ms, 4), "tops": round(tops, 1),
           "per_call": stats, "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4), "algorithmic_ops": int(ops)}
    log(f"prefill FFN: {ms:.4f} ms = {tops:.1f} TOPS")
    if check:
        import oracle
        olib = oracle.load()
        pick = W.rng(W.W_PREFILL, 2, 1)
        rows = sorted({0, M - 1} | {int(tt * 128 + pick.integers(0, 128)) for tt in range(M // 128)})
        opk = [oracle.pack(W.ternary(gx, n, k), olib) for gx, (n, k) in
               zip([W.rng(W.W_PREFILL, 1, tid) for tid in (W.T_GATE, W.T_UP, W.T_DOWN)], ((f, d), (f, d), (d, f)))]
        r = oracle.ffn(xh[rows], np.ones(d, np.float32), np.ones(f, np.float32), 1e-5, opk[0], scales[0], opk[1],
                       scales[1], opk[2], scales[2], olib)
        got = o.cpu().numpy()[rows]
        res["parity_sampled_rows"] = {"rows": len(rows),
                                      "bit_exact": bool(np.array_equal(got.view(np.uint32), r["out"].view(np.uint32)))}
        log(f"prefill FFN parity on {len(rows)} rows: {res['parity_sampled_rows']}")
    return res


def single_core_oracle():
    """The oracle on one thread: in full for the one-token workloads (2560 -> 2560
    quant + GEMV, the 3B FFN, one 3B stream token), and on a stated slice scaled
    linearly for prefill (128 of 2048 rows) and the 1.3B 32-token step (one
    token of 32 through 24 layers and the LM head)."""
    import oracle
    olib = oracle.load()
    prev = oracle.set_threads(0, olib)
    oracle.set_threads(1, olib)
    out = {"threads": 1, "cpu_model": cpu_model()}
    try:
        d, f = 2560, 10240
        g = W.rng(W.W_GEMV, 0, W.T_Q)
        p = oracle.pack(W.ternary(g, d, d), olib)
        x = W.activations(W.rng(W.W_GEMV, 0, W.T_X), 1, d)
        t0 = time.perf_counter()
        q, s, _ = oracle.quant_act(x, None, 1e-5, olib)
        oracle.bitlinear(p, np.float32(30.0), d, q, s, olib)
        out["gemv_2560_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
        gg = [W.rng(W.W_FFN, 0, tid) for tid in (W.T_GATE, W.T_UP, W.T_DOWN)]
        pk = [oracle.pack(W.ternary(gx, n, k), olib) for gx, (n, k) in zip(gg, ((f, d), (f, d), (d, f)))]
        xf = W.activations(W.rng(W.W_FFN, 0, W.T_X), 1, d)
        t0 = time.perf_counter()
        oracle.ffn(xf, np.ones(d, np.float32), np.ones(f, np.float32), 1e-5, pk[0], 30.0, pk[1], 30.0, pk[2], 30.0,
                   olib)
        out["ffn_3b_1token_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
        layers = []
        for l in range(32):
            raw = W.layer_inputs(W.W_STREAM, l, d, f, 1, bench_gains=True)
            lw = {k: raw[k] for k in ("g_attn", "g_attn_sub", "g_ffn", "g_ffn_sub", "z")}
            for name, sname in zip(W.LINEAR_NAMES, W.SCALE_NAMES):
                lw[name] = oracle.pack(raw[name], olib)
                lw[sname] = raw[sname]
            layers.append(lw)
        x0 = W.activations(W.rng(W.W_STREAM, 999, W.T_X), 1, d)
        t0 = time.perf_counter()
        oracle.chain(x0, layers, 1e-5, olib)
        out["stream_3b_1token_s"] = round(time.perf_counter() - t0, 3)
        del layers
        M, K, N, rows = 2048, 2560, 10240, 128
        gp = W.rng(W.W_PREFILL, 0, W.T_GATE)
        pp = oracle.pack(W.ternary(gp, N, K), olib)
        xp = W.activations(W.rng(W.W_PREFILL, 0, W.T_X), rows, K, outliers=True)
        t0 = time.perf_counter()
        q, s, _ = oracle.quant_act(xp, None, 1e-5, olib)
        oracle.bitlinear(pp, np.float32(30.0), K, q, s, olib)
        ts = time.perf_counter() - t0
        out["prefill_2048x2560x10240_s"] = {"value": round(ts * M / rows, 2), "extrapolated": True,
                                            "measured": f"{rows} of {M} rows in {ts:.2f} s, scaled by {M // rows}"}
        cfg = W.BITNET_1P3B
        d1, f1, V = cfg["dim"], cfg["ffn"], cfg["vocab"]
        layers = []
        for l in range(cfg["layers"]):
            raw = W.layer_inputs(W.W_BATCHED, l, d1, f1, 1, bench_gains=True)
            lw = {k: raw[k] for k in ("g_attn", "g_attn_sub", "g_ffn", "g_ffn_sub", "z")}
            for name, sname in zip(W.LINEAR_NAMES, W.SCALE_NAMES):
                lw[name] = oracle.pack(raw[name], olib)
                lw[sname] = raw[sname]
            layers.append(lw)
        gh = W.rng(W.W_BATCHED, 0, W.T_HEAD)
        head = oracle.pack(W.ternary(gh, V, d1), olib)
        x1 = W.activations(W.rng(W.W_BATCHED, 999, W.T_X), 1, d1)
        t0 = time.perf_counter()
        xo, _ = oracle.chain(x1, layers, 1e-5, olib)
        oracle.lm_head_argmax(xo, np.ones(d1, np.float32), 1e-5, head, 30.0, olib)
        ts = time.perf_counter() - t0
        out["batched_1p3b_32tokens_s"] = {"value": round(ts * 32, 2), "extrapolated": True,
                                          "measured": f"1 of 32 tokens in {ts:.2f} s, scaled by 32"}
    finally:
        oracle.set_threads(prev, olib)
    log(f"single-core oracle: {out}")
    return out


def graph_ms(torch, calls, outputs):
    """Time `calls` replayed from a HIP graph (the launches only, without the
    per-call Python and ctypes cost). Returns (ms per replay, whether the
    replay's outputs equal those of the eager run just before it)."""
    calls()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    g.replay()
    torch.cuda.synchronize()
    same = all(bool(torch.equal(o.view(torch.uint8), w.view(torch.uint8))) for o, w in zip(outputs, want))
    with Timer() as t:
        g.replay()
    del g
    return t.ms, same


def extra_measurements(bl, torch, T, dev0, check=True, peaks=None):
    out = {}
    # ---- single BitLinear decode GEMV 2560 -> 2560 (quant + GEMV), weights rotated
    # over > 512 MiB of copies so that they stream from HBM, not the 256 MB MALL ----
    d = 2560
    g = W.rng(W.W_GEMV, 0, W.T_Q)
    p0 = bl.bitlinear_pack(W.ternary(g, d, d))
    sw = W.weight_scale(g)
    copies = 320
    pw = T(np.ascontiguousarray(np.broadcast_to(p0, (copies,) + p0.shape)))
    x1 = T(W.activations(W.rng(W.W_GEMV, 0, W.T_X), 1, d))
    q1 = torch.empty((1, d), dtype=torch.int8, device=dev0)
    s1 = torch.empty(1, dtype=torch.float32, device=dev0)
    qs1 = torch.empty(1, dtype=torch.int32, device=dev0)
    y1 = torch.empty((1, d), dtype=torch.float32, device=dev0)
    for i in range(8):
        bl.bitlinear_forward(x1, None, 1e-5, pw[i], sw, d, q1, s1, qs1, y1)
    # one call of bitlinear_forward (one launch: every workgroup quantizes x itself)
    with Timer() as tg:
        for i in range(copies):
            bl.bitlinear_forward(x1, None, 1e-5, pw[i], sw, d, q1, s1, qs1, y1)
    ms = tg.ms / copies

    def fwd_calls():
        for i in range(copies):
            bl.bitlinear_forward(x1, None, 1e-5, pw[i], sw, d, q1, s1, qs1, y1)
    gms, gsame = graph_ms(torch, fwd_calls, [q1, s1, qs1, y1])
    gms /= copies
    # for context: the same as two calls, bitlinear_quant_act then bitlinear_gemv
    with Timer() as t2:
        for i in range(copies):
            bl.bitlinear_quant_act(x1, None, 1e-5, q1, s1, qs1)
            bl.bitlinear_gemv(pw[i], sw, d, d, q1, s1, qs1, 1, None, y1)
    ms2 = t2.ms / copies

    def two_calls():
        for i in range(copies):
            bl.bitlinear_quant_act(x1, None, 1e-5, q1, s1, qs1)
            bl.bitlinear_gemv(pw[i], sw, d, d, q1, s1, qs1, 1, None, y1)
    gms2, _ = graph_ms(torch, two_calls, [q1, s1, qs1, y1])
    gms2 /= copies
    rot = [0]

    def one_fwd():
        i = rot[0] % copies
        rot[0] += 1
        bl.bitlinear_forward(x1, None, 1e-5, pw[i], sw, d, q1, s1, qs1, y1)
    gemv_stats = per_call_stats(torch, one_fwd, copies)
    out["gemv"] = {"workload": "BitLinear 2560 -> 2560 at 1 token (quant + GEMV, 1,638,400 packed B) through "
                               "bitlinear_forward, weights rotated over 320 copies",
                   "per_call": gemv_stats,
                   "us_per_call": round(ms * 1e3, 3), "weight_gbs": round(d * d / 4 / (ms * 1e-3) / 1e9, 1),
                   "frac_hbm": round(d * d / 4 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "us_per_call_graph": round(gms * 1e3, 3),
                   "weight_gbs_graph": round(d * d / 4 / (gms * 1e-3) / 1e9, 1),
                   "graph_matches_eager": gsame,
                   "us_per_call_quant_then_gemv": round(ms2 * 1e3, 3),
                   "us_per_call_quant_then_gemv_graph": round(gms2 * 1e3, 3)}
    del pw
    # For context: the same GEMV kernel streaming a long matrix (2560 -> 163840,
    # 104,857,600 packed bytes) in one launch, where the launch and first-load
    # latency that bound the 1.6 MB call are amortised.
    nl = 64 * d
    gl = torch.Generator(device=dev0)
    gl.manual_seed(11)
    valid = torch.tensor([sum(((v // 3 ** j) % 3) << (2 * j) for j in range(4)) for v in range(81)],
                         dtype=torch.uint8, device=dev0)
    pl = valid[torch.randint(0, 81, (nl * d // 4,), generator=gl, device=dev0)]
    yl = torch.empty((1, nl), dtype=torch.float32, device=dev0)
    bl.bitlinear_quant_act(x1, None, 1e-5, q1, s1, qs1)
    for _ in range(3):
        bl.bitlinear_gemv(pl, sw, nl, d, q1, s1, qs1, 1, None, yl)
    with Timer() as tl:
        for _ in range(10):
            bl.bitlinear_gemv(pl, sw, nl, d, q1, s1, qs1, 1, None, yl)
    lms = tl.ms / 10
    out["gemv"]["long_matrix"] = {"shape": f"1 token, K={d} -> N={nl}", "packed_bytes": nl * d // 4,
                                  "us_per_call": round(lms * 1e3, 2),
                                  "weight_gbs": round(nl * d / 4 / (lms * 1e-3) / 1e9, 1),
                                  "frac_hbm": round(nl * d / 4 / (lms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"gemv over a long matrix: {out['gemv']['long_matrix']}")
    del pl, yl
    # ---- BitNet-3B FFN at one token, weights rotated over 27 copies (531 MB) ----
    f = 10240
    gg = [W.rng(W.W_FFN, 0, tid) for tid in (W.T_GATE, W.T_UP, W.T_DOWN)]
    shapes = ((f, d), (f, d), (d, f))
    packs = [bl.bitlinear_pack(W.ternary(gx, n, k)) for gx, (n, k) in zip(gg, shapes)]
    scales = [float(W.weight_scale(gx)) for gx in gg]
    fcopies = 27
    fw = [T(np.ascontiguousarray(np.broadcast_to(pk, (fcopies,) + pk.shape))) for pk in packs]
    xf = T(W.activations(W.rng(W.W_FFN, 0, W.T_X), 1, d))
    gn = T(np.ones(d, np.float32))
    gs = T(np.ones(f, np.float32))
    of = torch.empty((1, d), dtype=torch.float32, device=dev0)
    wsf = torch.empty(bl.bitnet_ffn_workspace_bytes(1, d, f), dtype=torch.uint8, device=dev0)
    for i in range(3):
        bl.bitnet_ffn(xf, 1, d, f, gn, gs, 1e-5, fw[0][i], scales[0], fw[1][i], scales[1], fw[2][i], scales[2],
                      None, of, wsf)
    with Timer() as tf:
        for i in range(fcopies):
            bl.bitnet_ffn(xf, 1, d, f, gn, gs, 1e-5, fw[0][i], scales[0], fw[1][i], scales[1], fw[2][i],
                          scales[2], None, of, wsf)
    ms = tf.ms / fcopies
    fb = 3 * d * f // 4

    def ffn_calls():
        for i in range(fcopies):
            bl.bitnet_ffn(xf, 1, d, f, gn, gs, 1e-5, fw[0][i], scales[0], fw[1][i], scales[1], fw[2][i],
                          scales[2], None, of, wsf)
    gms, gsame = graph_ms(torch, ffn_calls, [of])
    gms /= fcopies
    rotf = [0]

    def one_ffn():
        i = rotf[0] % fcopies
        rotf[0] += 1
        bl.bitnet_ffn(xf, 1, d, f, gn, gs, 1e-5, fw[0][i], scales[0], fw[1][i], scales[1], fw[2][i], scales[2],
                      None, of, wsf)
    ffn_stats = per_call_stats(torch, one_ffn, 4 * fcopies)
    out["ffn"] = {"workload": "BitNet-3B FFN at 1 token (19,660,800 packed B), weights rotated over 27 copies",
                  "per_call": ffn_stats,
                  "us_per_call": round(ms * 1e3, 3), "weight_gbs": round(fb / (ms * 1e-3) / 1e9, 1),
                  "frac_hbm": round(fb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "us_per_call_graph": round(gms * 1e3, 3), "weight_gbs_graph": round(fb / (gms * 1e-3) / 1e9, 1),
                  "frac_hbm_graph": round(fb / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "graph_matches_eager": gsame}
    log(f"gemv {out['gemv']['us_per_call']} us ({out['gemv']['us_per_call_graph']} us from a graph; two calls "
        f"{out['gemv']['us_per_call_quant_then_gemv']} / {out['gemv']['us_per_call_quant_then_gemv_graph']} us), "
        f"ffn {out['ffn']['us_per_call']} us ({out['ffn']['us_per_call_graph']} us from a graph)")
    del fw
    # ---- prefill GEMM 2048 x 2560 -> 10240 ----
    M, K, N = 2048, 2560, 10240
    g = W.rng(W.W_PREFILL, 0, W.T_GATE)
    t = W.ternary(g, N, K)
    sw = W.weight_scale(g)
    p = T(bl.bitlinear_pack(t))
    del t
    x = T(W.activations(W.rng(W.W_PREFILL, 0, W.T_X), M, K, outliers=True))
    q = torch.empty((M, K), dtype=torch.int8, device=dev0)
    s = torch.empty(M, dtype=torch.float32, device=dev0)
    qs = torch.empty(M, dtype=torch.int32, device=dev0)
    y = torch.empty((M, N), dtype=torch.float32, device=dev0)
    bl.bitlinear_quant_act(x, None, 1e-5, q, s, qs)
    for _ in range(3):
        bl.bitlinear_gemm(p, sw, N, K, q, s, qs, M, None, y)
    iters = 20
    with Timer() as tg:
        for _ in range(iters):
            bl.bitlinear_gemm(p, sw, N, K, q, s, qs, M, None, y)
    with Timer() as tq:
        for _ in range(iters):
            bl.bitlinear_quant_act(x, None, 1e-5, q, s, qs)
            bl.bitlinear_gemm(p, sw, N, K, q, s, qs, M, None, y)
    ops = 2.0 * M * N * K
    gemm_ms = tg.ms / iters
    gemm_stats = per_call_stats(torch, lambda: bl.bitlinear_gemm(p, sw, N, K, q, s, qs, M, None, y), iters)
    tops = ops / (gemm_ms * 1e-3) / 1e12
    out["prefill"] = {"workload": "quant 2048x2560 fp32 (1% outliers x20) + GEMM vs 10240x2560 ternary -> fp32",
                      "gemm_ms": round(gemm_ms, 4), "gemm_tops": round(tops, 1),
                      "gemm_per_call": gemm_stats,
                      "quant_plus_gemm_ms": round(tq.ms / iters, 4),
                      "quant_plus_gemm_tops": round(ops / (tq.ms / iters * 1e-3) / 1e12, 1),
                      "peak_tops": INT8_PEAK_TOPS,
                      "gemm_frac": round(tops / INT8_PEAK_TOPS, 4),
                      "roofline": {"kernel": "gemm_kernel<128x320 tiles> (int8 MFMA 16x16x64)", "bound": "mfma",
                                   "achieved": round(tops, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                                   "frac": round(tops / INT8_PEAK_TOPS, 4), "algorithmic_ops": int(ops),
                                   "traffic": None}}
    if peaks:
        # the measured ceiling with operands like a GEMM's (random bytes, changing every MFMA)
        dense = peaks["int8_mfma_tops_dense"]
        out["prefill"]["roofline"]["probe_peak_dense"] = dense
        out["prefill"]["roofline"]["frac_of_probe_dense"] = round(tops / dense, 4)
    log(f"prefill: GEMM {gemm_ms:.4f} ms = {out['prefill']['gemm_tops']} TOPS")
    out["prefill"]["vendor_int8_gemm"] = vendor_int8_gemm(torch, dev0, q, t_rows=N)
    log(f"prefill: vendor int8 GEMM on the same shape: {out['prefill']['vendor_int8_gemm']}")
    if check:
        # the timed call's y against the oracle: one random row in every
        # 128-row block tile, plus the first and last rows, every column
        import oracle
        olib = oracle.load()
        pick = W.rng(W.W_PREFILL, 1, 1)
        rows = sorted({0, M - 1} | {int(tt * 128 + pick.integers(0, 128)) for tt in range(M // 128)})
        xh = x.cpu().numpy()[rows]
        oq, os_, _ = oracle.quant_act(xh, None, 1e-5, olib)
        oy, _ = oracle.bitlinear(p.cpu().numpy(), sw, K, oq, os_, olib)
        got = y.cpu().numpy()[rows]
        err = np.abs(got.astype(np.float64) - oy) / np.maximum(np.abs(oy.astype(np.float64)), 1e-30)
        out["prefill"]["parity_sampled_rows"] = {"rows": len(rows), "bit_exact": bool(np.array_equal(
            got.view(np.uint32), oy.view(np.uint32))), "max_rel_err": float(err.max())}
        log(f"prefill parity on {len(rows)} rows: {out['prefill']['parity_sampled_rows']}")
    del p, x, q, y

    # ---- top-k / nucleus sampling over the vocabulary ----
    out["sampling"] = sampling_leg(bl, torch, T, dev0, check)

    # ---- prefill FFN, 2048 tokens, BitNet-3B shapes ----
    out["prefill_ffn"] = prefill_ffn_leg(bl, torch, T, dev0, check)

    # ---- batched decode, 1.3B, 32 tokens, + LM head argmax ----
    cfg = W.BITNET_1P3B
    L, d, f, m, V = cfg["layers"], cfg["dim"], cfg["ffn"], 32, cfg["vocab"]
    dev, host_b = build_stream(bl, W.W_BATCHED, L, d, f, m, T)
    gh = W.rng(W.W_BATCHED, 0, W.T_HEAD)
    head = T(bl.bitlinear_pack(W.ternary(gh, V, d)))
    sh = W.weight_scale(gh)
    gfin = T(np.ones(d, np.float32))
    xb = T(W.activations(W.rng(W.W_BATCHED, 999, W.T_X), m, d))
    qkv = torch.empty((L, m, 3 * d), dtype=torch.float32, device=dev0)
    ws = torch.zeros(bl.bitnet_stream_workspace_bytes(m, d, f), dtype=torch.uint8, device=dev0)
    qf = torch.empty((m, d), dtype=torch.int8, device=dev0)
    sf = torch.empty(m, dtype=torch.float32, device=dev0)
    qsf = torch.empty(m, dtype=torch.int32, device=dev0)
    idx = torch.empty(m, dtype=torch.int32, device=dev0)
    wsh = torch.empty(bl.bitlinear_gemm_workspace_bytes(m, V, d, 1), dtype=torch.uint8, device=dev0)

    def batched_step():
        run_stream_step(bl, dev, L, m, d, f, xb, qkv, ws)
        bl.bitlinear_quant_act(xb, gfin, 1e-5, qf, sf, qsf)
        bl.bitlinear_gemm(head, sh, V, d, qf, sf, qsf, m, None, None, None, idx, wsh)

    # parity of the first stream step on sampled tokens: every row goes through
    # the layers on its own (per-token norms, products and stand-in), so the
    # oracle runs the chosen rows alone, bit for bit
    batched_check = None
    if check:
        import oracle
        olib = oracle.load()
        x_in = xb.cpu().numpy().copy()
        run_stream_step(bl, dev, L, m, d, f, xb, qkv, ws)
        x_gpu, qkv_gpu = xb.cpu().numpy(), qkv.cpu().numpy()
        rows = [0, m - 1]
        exact = True
        for r in rows:
            lr = [dict(lw, z=lw["z"][r:r + 1]) for lw in host_b]
            ox, oqkv = oracle.chain(x_in[r:r + 1], lr, 1e-5, olib)
            exact = exact and bool(np.array_equal(ox.view(np.uint32), x_gpu[r:r + 1].view(np.uint32)))
            exact = exact and all(np.array_equal(oqkv[l].view(np.uint32), qkv_gpu[l, r:r + 1].view(np.uint32))
                                  for l in range(L))
        batched_check = {"tokens": rows, "bit_exact": exact}
        xb.copy_(T(x_in))
    del host_b

    for _ in range(2):
        batched_step()
    iters = 10
    with Timer() as tb:
        for _ in range(iters):
            batched_step()
    bytes_b = L * bl.bitnet_layer_bytes(d, f) + V * d // 4
    ms_b = tb.ms / iters
    batched_stats = per_call_stats(torch, batched_step, iters)
    # x is updated in place, so the eager/graph comparison restarts both from one x
    x_start = xb.clone()

    def batched_from_start():
        xb.copy_(x_start)
        batched_step()
    gms, gsame = graph_ms(torch, batched_from_start, [xb, idx])
    out["batched"] = {"workload": "BitNet-1.3B stream, 32 tokens, 24 layers x 7 BitLinears + LM head 2048->50000 "
                                  "with fused argmax", "ms_per_step": round(ms_b, 4),
                      "weight_gbs": round(bytes_b / (ms_b * 1e-3) / 1e9, 1),
                      "us_per_token": round(ms_b * 1e3 / m, 3), "weight_bytes": bytes_b,
                      "frac_hbm": round(bytes_b / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "ms_per_step_graph": round(gms, 4),
                      "weight_gbs_graph": round(bytes_b / (gms * 1e-3) / 1e9, 1),
                      "graph_matches_eager": gsame, "per_step": batched_stats,
                      "parity_first_step": batched_check,
                      "roofline": {"kernel": "the step's launches (skinny MFMA products, quant, LM head argmax)",
                                   "bound": "hbm", "achieved": round(bytes_b / (ms_b * 1e-3) / 1e9, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(bytes_b / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "algorithmic_bytes": bytes_b, "traffic": None}}
    log(f"batched: {ms_b:.4f} ms per 32-token step ({gms:.4f} ms from a graph)")
    del dev, head
    return out


if __name__ == "__main__":
    main()
