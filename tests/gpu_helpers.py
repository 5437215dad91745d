"""Shared helpers of the GPU parity tests: identical seeded inputs for the HIP
path and the oracle, and the comparison rules.

Comparison rules (the parity bar): int8 codes, packed bytes, int32 accumulators
and argmax indices bit-exact; fp32 outputs within 1e-6 relative error (the
implementations follow the same operation order, so they are expected to be
bit-exact and the tests also count non-identical elements)."""
import sys

import numpy as np

import oracle
import workloads as W

F32_RTOL = 1e-6


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dev())


def to_host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_exact(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[0]}: {got.reshape(-1)[bad[0]]} vs " \
                          f"{want.reshape(-1)[bad[0]]}"


def assert_f32(got, want, what, rtol=F32_RTOL):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    tol = rtol * np.maximum(np.abs(want.astype(np.float64)), np.finfo(np.float32).tiny)
    bad = np.flatnonzero(err.reshape(-1) > tol.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} beyond rtol {rtol}; first at {bad[0]}: " \
                          f"{got.reshape(-1)[bad[0]]!r} vs {want.reshape(-1)[bad[0]]!r}"
    differ = int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))
    if differ:
        log(f"  note: {what}: {differ} elements within tolerance but not bit-identical")
    return differ


def pack_both(t, olib):
    """Pack with the library's host packer and with the oracle; they must agree."""
    import bitlinear_amd as bl
    p = bl.bitlinear_pack(t)
    assert_exact(p, oracle.pack(t, olib), "packed bytes")
    return p


def make_layers(workload, n_layers, d, f, m, olib, bench_gains=False):
    """Seeded layer inputs, packed, as (oracle layer dicts, device blob tensors)."""
    import torch
    import bitlinear_amd as bl
    layers = []
    blobs, scales, gains, zs = [], [], [], []
    for l in range(n_layers):
        raw = W.layer_inputs(workload, l, d, f, m, bench_gains=bench_gains)
        lw = {}
        for name, sname in zip(W.LINEAR_NAMES, W.SCALE_NAMES):
            lw[name] = pack_both(raw[name], olib) if l < 2 else bl.bitlinear_pack(raw[name])
            lw[sname] = raw[sname]
            blobs.append(lw[name].reshape(-1))
        for key in ("g_attn", "g_attn_sub", "g_ffn", "g_ffn_sub", "z"):
            lw[key] = raw[key]
        scales.append(np.array([raw[s] for s in W.SCALE_NAMES], np.float32))
        gains.append(np.concatenate([raw["g_attn"], raw["g_attn_sub"], raw["g_ffn"], raw["g_ffn_sub"]]))
        zs.append(raw["z"])
        layers.append(lw)
    dev = dict(weights=to_dev(np.concatenate(blobs)), scales=to_dev(np.stack(scales)),
               gains=to_dev(np.stack(gains)), z=to_dev(np.stack(zs)))
    assert dev["weights"].numel() == n_layers * bl.bitnet_layer_bytes(d, f)
    del torch
    return layers, dev


def new_stream_workspace(m, d, f):
    """A zero-filled stream workspace (the persistent path keeps a phase counter in it)."""
    import torch
    import bitlinear_amd as bl
    return torch.zeros(bl.bitnet_stream_workspace_bytes(m, d, f), dtype=torch.uint8, device=torch_dev())


def stream_ctrl(ws):
    """(phase counter, status) words at the start of a stream workspace."""
    import torch
    torch.cuda.synchronize()
    c = ws[:8].view(torch.int32).cpu().numpy()
    return int(c[0]), int(c[1])


def run_stream(dev, n_layers, m, d, f, eps, x0, ws=None):
    """Run bitnet_decode_stream on the GPU; returns (x, qkv, workspace)."""
    import torch
    import bitlinear_amd as bl
    x = to_dev(x0)
    qkv = torch.empty((n_layers, m, 3 * d), dtype=torch.float32, device=torch_dev())
    if ws is None:
        ws = new_stream_workspace(m, d, f)
    bl.bitnet_decode_stream(dev["weights"], dev["scales"], dev["gains"], dev["z"], n_layers, m, d, f, eps, x, qkv, ws)
    return to_host(x), to_host(qkv), ws
