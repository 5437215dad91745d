"""Pins of the CPU oracle: checks against facts that do not come from the oracle.

Each pin is a function ``pin_x(o, lib)`` of an oracle module ``o`` and its C
library ``lib``; it raises AssertionError when the oracle is wrong. The
mutation test reuses them against copies of the oracle with planted mistakes.

Sources of truth used here (never the oracle itself):
  * hand-worked fixtures under tests/golden/ (each cites its page and section);
  * the pages' packed-size arithmetic ("Memory Footprint" on the Hesper
    BitNet page, "Memory Layout" on the Hesper TransformerBlock page);
  * closed forms: identity / sign-flip / permutation weights, one-hot inputs,
    power-of-two scalings, constant vectors;
  * exact rational arithmetic (fractions, decimal) within a stated error bound;
  * numpy's int64 matmul and argmax on tiny cases (library routines).
"""
import decimal
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _ulp32(v):
    v = abs(np.float32(v))
    return float(np.spacing(v)) if v != 0 else float(np.finfo(np.float32).tiny)


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# --- TQ2_0 codec ----------------------------------------------------------------

def pin_codec_golden(o, lib):
    """Hand-derived bytes for the stated layout (tests/golden/tq2_codec.txt)."""
    for row in _read_fixture("tq2_codec.txt"):
        lhs, rhs = row.split("->")
        t = np.array([int(v) for v in lhs.split()], np.int8).reshape(1, 4)
        byte = int(rhs.strip(), 16)
        p = o.pack(t, lib)
        assert p.shape == (1, 1) and int(p[0, 0]) == byte, (t, p, byte)
        assert (o.unpack(p, 4, lib) == t).all()


def pin_codec_exhaustive(o, lib):
    """All 81 ternary 4-tuples map to 81 distinct bytes with no code-3 field, and
    back; the 175 bytes holding a code-3 field are rejected."""
    import itertools
    tuples = np.array(list(itertools.product((-1, 0, 1), repeat=4)), np.int8)
    p = o.pack(tuples, lib)  # 81 rows of K=4 -> one byte each
    vals = [int(b) for b in p[:, 0]]
    assert len(set(vals)) == 81
    for b in vals:
        assert all(((b >> (2 * j)) & 3) != 3 for j in range(4))
    assert (o.unpack(p, 4, lib) == tuples).all()
    good = set(vals)
    for b in range(256):
        if b in good:
            continue
        try:
            o.unpack(np.array([[b]], np.uint8), 4, lib)
        except o.OracleError:
            continue
        raise AssertionError(f"byte {b:#x} with a code-3 field was accepted")


def pin_codec_value_range(o, lib):
    """Values outside {-1, 0, 1} are rejected; K not a multiple of 4 is rejected."""
    for bad in (2, -2, 127, -128):
        t = np.zeros((1, 4), np.int8)
        t[0, 2] = bad
        try:
            o.pack(t, lib)
        except o.OracleError:
            continue
        raise AssertionError(f"value {bad} accepted")
    try:
        o.pack(np.zeros((1, 6), np.int8), lib)
    except o.OracleError:
        pass
    else:
        raise AssertionError("k % 4 != 0 accepted")


def pin_codec_row_layout(o, lib):
    """Byte i of row n covers weights 4i..4i+3 of that row (a single +1 at (n, k)
    lands in byte k//4 of row n, field k%4, and nowhere else)."""
    n, k = 5, 24
    for (r, c) in ((0, 0), (2, 7), (4, 23), (3, 12)):
        t = np.full((n, k), -1, np.int8)
        t[r, c] = 1
        p = o.pack(t, lib)
        assert p.shape == (n, k // 4)
        expect = np.zeros((n, k // 4), np.uint8)
        expect[r, c // 4] = 2 << (2 * (c % 4))
        assert (p == expect).all(), (r, c)


def pin_packed_sizes(o, lib):
    """The pages' packed-size arithmetic: count * n * k * 0.25 bytes, matching the
    printed MB figure to the printed precision. Every output byte is written (a
    valid code byte is never 0xff) and nothing past the end."""
    for row in _read_fixture("packed_sizes.txt"):
        n, k, count, mb, _src = row.split()
        n, k, count, mb = int(n), int(k), int(count), float(mb)
        exact = count * n * k // 4
        digits = len(repr(mb).split(".")[1]) if repr(mb).split(".")[1] != "0" else 0
        assert abs(exact / 1e6 - mb) < 10.0 ** (-digits), (row, exact)
        t = np.zeros((n, k), np.int8)
        buf = np.full(n * k // 4 + 64, 0xFF, np.uint8)
        view = buf[: n * k // 4].reshape(n, k // 4)
        rc = lib.ref_pack(t.ctypes.data_as(o._i8p), n, k, view.ctypes.data_as(o._u8p))
        assert rc == 0
        assert (buf[n * k // 4:] == 0xFF).all(), "wrote past the end"
        assert (view == 0x55).all(), "zero weights must pack to 0x55 everywhere"


def pin_layer_bytes(o, lib):
    """One BitNet-3B layer is 26,214,400 packed bytes and 32 layers 838,860,800
    ("Memory Layout": ~26 MB per layer, ~832 MB for 32 layers; "Memory
    Footprint": 32 x 26 MB). Pack one of each shape and sum."""
    d, f = 2560, 10240
    shapes = [(d, d)] * 4 + [(f, d), (f, d), (d, f)]
    total = 0
    for n, k in shapes:
        total += o.pack(np.zeros((n, k), np.int8), lib).nbytes
    assert total == 26_214_400
    assert round(total / 1e6) == 26
    assert 32 * total == 838_860_800
    assert abs(32 * round(total / 1e6) - 832) == 0


# --- activation quant -----------------------------------------------------------

def pin_quant_golden(o, lib):
    """Hand-worked absmax/round-half-even cases (tests/golden/quant_cases.txt)."""
    for row in _read_fixture("quant_cases.txt"):
        ys, sa, qs, qsum = [s.strip() for s in row.split("|")]
        y = np.array([float(v) for v in ys.split()], np.float32).reshape(1, -1)
        q, s, qsm = o.activation_quant(y, lib)
        assert float(s[0]) == float(sa), (row, s)
        assert q[0].tolist() == [int(v) for v in qs.split()], (row, q)
        assert int(qsm[0]) == int(qsum), (row, qsm)


def pin_quant_bounds(o, lib):
    """The absmax element maps to +-127, |q| <= 127 and q never hits -128;
    qsum is the integer sum of q (checked with numpy int64)."""
    g = _rng(11)
    for k in (1, 4, 64, 257, 2560):
        x = g.standard_normal((7, k)).astype(np.float32) * np.float32(g.uniform(1e-3, 1e3))
        q, s, qs = o.activation_quant(x, lib)
        for r in range(7):
            j = int(np.argmax(np.abs(x[r])))
            assert abs(int(q[r, j])) == 127 and np.sign(q[r, j]) == np.sign(x[r, j])
            assert np.abs(q[r].astype(np.int64)).max() == 127
        assert q.min() > -128
        assert (qs.astype(np.int64) == q.astype(np.int64).sum(1)).all()


def pin_quant_pow2_scaling(o, lib):
    """Multiplying a token by 2^e leaves q unchanged and divides s_a by 2^e (all
    products are exact in binary floating point)."""
    g = _rng(12)
    x = g.standard_normal((5, 300)).astype(np.float32)
    q0, s0, _ = o.activation_quant(x, lib)
    for e in (-7, -1, 3, 10):
        q1, s1, _ = o.activation_quant(x * np.float32(2.0 ** e), lib)
        assert (q1 == q0).all()
        assert (s1 == s0 * np.float32(2.0 ** -e)).all()


def pin_quant_scale_value(o, lib):
    """s_a is the correctly rounded fp32 of 127/absmax (checked with Fraction)."""
    g = _rng(13)
    x = g.standard_normal((20, 100)).astype(np.float32)
    _, s, _ = o.activation_quant(x, lib)
    for r in range(20):
        amax = Fraction(float(np.abs(x[r]).max()))
        exact = Fraction(127) / amax
        assert abs(Fraction(float(s[r])) - exact) <= Fraction(_ulp32(s[r])) / 2


def pin_quant_error_bound(o, lib):
    """q / s_a reconstructs y within half a quantization step (plus one fp32
    rounding of y*s_a): the defining property of round-to-nearest codes."""
    g = _rng(14)
    x = g.standard_normal((6, 512)).astype(np.float32)
    q, s, _ = o.activation_quant(x, lib)
    for r in range(6):
        err = np.abs(q[r].astype(np.float64) / float(s[r]) - x[r].astype(np.float64))
        bound = (0.5 + 127 * 2.0 ** -23) / float(s[r])
        assert err.max() <= bound


# --- RMSNorm ----------------------------------------------------------------------

def _exact_r(x, eps):
    """1/sqrt(mean(x^2) + eps) with 60 significant digits, from an exact sum."""
    ss = sum(Fraction(float(v)) ** 2 for v in x)
    mean = ss / len(x) + Fraction(float(np.float32(eps)))
    ctx = decimal.Context(prec=60)
    dm = ctx.divide(decimal.Decimal(mean.numerator), decimal.Decimal(mean.denominator))
    return ctx.divide(decimal.Decimal(1), ctx.sqrt(dm))


def pin_sumsq_exact_bound(o, lib):
    """The fixed-order fp64 sum of squares is the exact sum of all K squares
    within the fp64 summation bound K * 2^-53 * sum."""
    g = _rng(21)
    for k in (1, 3, 64, 255, 256, 257, 1000, 2560):
        x = (g.standard_normal(k) * g.uniform(0.01, 100)).astype(np.float32)
        exact = sum(Fraction(float(v)) ** 2 for v in x)
        got = Fraction(o.sumsq(x, lib))
        assert abs(got - exact) <= exact * Fraction(k + 8, 2 ** 53), k


def pin_sumsq_order(o, lib):
    """The sum of squares follows the stated order exactly: 512 strided partials
    (partial l sums x[k]^2 for k = l, l+512, ... ascending), then a pairwise
    xor-butterfly with offsets 1, 2, 4, ..., 256. Hand-worked cases with squares
    2^52 and 1 (fp64 spacing is 2 above 2^53, so a 1 that meets 2^53 alone is
    lost to round-half-even); K = 1024, x = 0 elsewhere:
      A: x[0] = x[512] = 2^26, x[64] = x[128] = 1. Partial 0 = 2^53; the 1s in
         partials 64 and 128 each meet 2^53 alone -> 2^53.
         (64 or 128 partials, or a left-to-right sum, give 2^53 + 2.)
      B: x[0] = x[128] = 2^26, x[512] = x[640] = 1. Partials 0 and 128 are each
         2^52 + 1 (exact) and meet at offset 128 -> 2^53 + 2.
         (128 or 256 partials, or a left-to-right sum, give 2^53.)
      C: x[0] = x[512] = 2^26, x[1] = x[257] = 1. Ascending offsets add partial 1
         to 2^53 first (lost), then partial 257 alone (lost) -> 2^53.
         (Descending offsets pair the two 1s first -> 2^53 + 2.)"""
    big = np.float32(2.0 ** 26)
    xa = np.zeros(1024, np.float32)
    xa[[0, 512]] = big
    xa[[64, 128]] = 1.0
    assert o.sumsq(xa, lib) == 2.0 ** 53
    xb = np.zeros(1024, np.float32)
    xb[[0, 128]] = big
    xb[[512, 640]] = 1.0
    assert o.sumsq(xb, lib) == 2.0 ** 53 + 2.0
    xc = np.zeros(1024, np.float32)
    xc[[0, 512]] = big
    xc[[1, 257]] = 1.0
    assert o.sumsq(xc, lib) == 2.0 ** 53


def pin_rmsnorm_closed_form(o, lib):
    """y = x * r * g with r = 1/sqrt(mean(x^2) + eps): each y is within 1.5 fp32
    ulps of the exact product (one rounding of r, two of the products)."""
    g = _rng(22)
    for k, eps in ((4, 0.0), (64, 1e-5), (300, 1e-5), (2560, 1e-6), (16, 1.0)):
        x = g.standard_normal((1, k)).astype(np.float32)
        gain = g.uniform(0.5, 1.5, k).astype(np.float32)
        y = o.rmsnorm(x, gain, eps, lib)[0]
        r = _exact_r(x[0], eps)
        for i in range(0, k, max(1, k // 37)):
            exact = decimal.Decimal(float(x[0, i])) * r * decimal.Decimal(float(gain[i]))
            err = abs(decimal.Decimal(float(y[i])) - exact)
            assert err <= decimal.Decimal(2.0 * _ulp32(y[i])), (k, eps, i)


def pin_rmsnorm_constant(o, lib):
    """A constant vector c with unit gains and eps = 0 normalises to sign(c),
    so activation_quant gives 127 * sign(c) everywhere."""
    for c in (3.0, -0.125, 1e-3, 77.5):
        for k in (4, 100, 2560):
            x = np.full((1, k), c, np.float32)
            q, s, qs = o.quant_act(x, np.ones(k, np.float32), 0.0, lib)
            assert (q == 127 * int(np.sign(c))).all()
            assert int(qs[0]) == 127 * int(np.sign(c)) * k


def pin_rmsnorm_pow2(o, lib):
    """With eps = 0, scaling x by 2^e leaves the normalised y unchanged exactly."""
    g = _rng(23)
    x = g.standard_normal((3, 640)).astype(np.float32)
    gain = g.uniform(0.5, 1.5, 640).astype(np.float32)
    y0 = o.rmsnorm(x, gain, 0.0, lib)
    for e in (-5, 4, 20):
        y1 = o.rmsnorm(x * np.float32(2.0 ** e), gain, 0.0, lib)
        assert (y1 == y0).all()


def pin_rmsnorm_eps(o, lib):
    """eps enters under the root: with x = 0 except one element a, K = 1 and
    eps = 3 a^2, r = 1/(2|a|) exactly, so y = g/2 * sign(a)."""
    for a in (0.5, -2.0, 8.0):
        x = np.array([[a]], np.float32)
        y = o.rmsnorm(x, np.array([3.0], np.float32), 3.0 * a * a, lib)
        assert float(y[0, 0]) == 1.5 * np.sign(a), y


# --- weight quant -----------------------------------------------------------------

def pin_weight_quant_closed_form(o, lib):
    """absmean scale: W = [a, -a, 3a, -3a, 0, 0, 0, 0] has mean|W| = a, so
    s_w = 1/a and t = [1, -1, 1, -1, 0, 0, 0, 0] (3 clamps to 1). An absmax
    scale would give s_w = 1/(3a) and zeros in the first two places."""
    for a in (0.125, 2.0, 1.0 / 64):
        w = np.array([[a, -a, 3 * a, -3 * a, 0, 0, 0, 0]], np.float32)
        t, s = o.weight_quant(w, lib)
        assert float(s) == 1.0 / a
        assert t[0].tolist() == [1, -1, 1, -1, 0, 0, 0, 0]


def pin_weight_quant_ties(o, lib):
    """W = [a, -a, 3a, -3a] has mean 2a, s_w = 1/(2a): W*s_w = [.5, -.5, 1.5, -1.5]
    rounds half to even to [0, 0, 2, -2] and clamps to [0, 0, 1, -1]."""
    a = 0.125
    w = np.array([[a, -a, 3 * a, -3 * a]], np.float32)
    t, s = o.weight_quant(w, lib)
    assert float(s) == 4.0
    assert t[0].tolist() == [0, 0, 1, -1]


def pin_weight_quant_recovers_ternary(o, lib):
    """W = c * t for a ternary t with half its entries nonzero: mean|W| = c/2,
    s_w = 2/c and t is recovered exactly (W*s_w = 2t clamps to t)."""
    g = _rng(31)
    t0 = np.zeros((16, 64), np.int8)
    idx = g.permutation(16 * 64)[: 16 * 32]
    t0.flat[idx] = g.choice(np.array([-1, 1], np.int8), size=idx.size)
    for c in (0.25, 4.0):
        t, s = o.weight_quant(t0.astype(np.float32) * np.float32(c), lib)
        assert float(s) == 2.0 / c
        assert (t == t0).all()


def pin_weight_quant_mean(o, lib):
    """s_w is 1/mean|W| (numpy's float64 mean, within fp32 rounding)."""
    g = _rng(32)
    w = (g.standard_normal((33, 96)) * 0.02).astype(np.float32)
    _, s = o.weight_quant(w, lib)
    ref = 1.0 / np.mean(np.abs(w.astype(np.float64)))
    assert abs(float(s) - ref) <= 1.0 * _ulp32(s)


# --- matmul / dequant ----------------------------------------------------------------

def pin_matmul_bruteforce(o, lib):
    """Exact int32 products against numpy's int64 matmul on small random shapes
    (non-square, so a transposed operand or output fails)."""
    g = _rng(41)
    for _ in range(40):
        m, n, k = int(g.integers(1, 17)), int(g.integers(1, 17)), 4 * int(g.integers(1, 5))
        t = g.integers(-1, 2, (n, k)).astype(np.int8)
        q = g.integers(-127, 128, (m, k)).astype(np.int8)
        acc = o.matmul_i32(t, q, lib)
        assert acc.shape == (m, n)
        assert (acc.astype(np.int64) == q.astype(np.int64) @ t.astype(np.int64).T).all()


def pin_matmul_k4_exhaustive_rows(o, lib):
    """Every ternary row of K=4 against sampled int8 vectors, through the packed
    path (pack -> bitlinear), against numpy."""
    import itertools
    t = np.array(list(itertools.product((-1, 0, 1), repeat=4)), np.int8)
    g = _rng(42)
    q = g.integers(-127, 128, (64, 4)).astype(np.int8)
    p = o.pack(t, lib)
    s_a = np.ones(64, np.float32)
    _, acc = o.bitlinear(p, np.float32(1.0), 4, q, s_a, lib)
    assert (acc.astype(np.int64) == q.astype(np.int64) @ t.astype(np.int64).T).all()


def pin_matmul_invariants(o, lib):
    """Identity gives q, -I gives -q, a permutation permutes q, zero rows give 0,
    all-(+1) rows give sum(q) and all-(-1) rows give -sum(q)."""
    g = _rng(43)
    k = 64
    q = g.integers(-127, 128, (3, k)).astype(np.int8)
    eye = np.eye(k, dtype=np.int8)
    assert (o.matmul_i32(eye, q, lib) == q).all()
    assert (o.matmul_i32(-eye, q, lib) == -q.astype(np.int32)).all()
    perm = g.permutation(k)
    assert (o.matmul_i32(eye[perm], q, lib) == q[:, perm]).all()
    special = np.stack([np.zeros(k, np.int8), np.ones(k, np.int8), -np.ones(k, np.int8)])
    acc = o.matmul_i32(special, q, lib)
    s = q.astype(np.int64).sum(1)
    assert (acc[:, 0] == 0).all() and (acc[:, 1] == s).all() and (acc[:, 2] == -s).all()


def pin_int32_bound(o, lib):
    """x = +-c everywhere gives q = +-127; with t = sign(q), acc = 127 K exactly
    (1,300,480 at K = 10240) and the fp32 conversion is exact."""
    k = 10240
    g = _rng(44)
    sgn = g.choice(np.array([-1, 1], np.int8), size=k)
    x = (sgn.astype(np.float32) * np.float32(3.5)).reshape(1, k)
    q, s, _ = o.activation_quant(x, lib)
    assert (q[0] == 127 * sgn).all()
    p = o.pack(sgn.reshape(1, k), lib)
    y, acc = o.bitlinear(p, np.float32(1.0), k, q, s, lib)
    assert int(acc[0, 0]) == 1_300_480
    assert float(y[0, 0]) == float(np.float32(1_300_480) * (np.float32(1.0) / s[0]))


def pin_dequant_pow2(o, lib):
    """Power-of-two scales make the dequant exact: s_a = 2^a, s_w = 2^b gives
    y = acc * 2^-(a+b)."""
    g = _rng(45)
    acc = g.integers(-2 ** 20, 2 ** 20, (4, 9)).astype(np.int32)
    for a, b in ((3, 5), (-2, 7), (0, 0)):
        s_a = np.full(4, 2.0 ** a, np.float32)
        y = o.dequant(acc, s_a, np.float32(2.0 ** b), lib)
        assert (y.astype(np.float64) == acc.astype(np.float64) * 2.0 ** -(a + b)).all()


def pin_dequant_per_row(o, lib):
    """Each row uses its own s_a: rows with s_a = 1, 2, 4 differ by exactly 2x."""
    acc = np.tile(np.arange(-5, 6, dtype=np.int32), (3, 1))
    y = o.dequant(acc, np.array([1, 2, 4], np.float32), np.float32(1.0), lib)
    assert (y[0] == 2 * y[1]).all() and (y[1] == 2 * y[2]).all()


def pin_bitlinear_onehot(o, lib):
    """x = v e_j: q = 127 sign(v) e_j, s_a = 127/|v|, so y[n] = t[n][j] v / s_w
    within a few fp32 ulps (the float matmul the quantization approximates)."""
    g = _rng(46)
    n, k = 24, 64
    t = g.integers(-1, 2, (n, k)).astype(np.int8)
    p = o.pack(t, lib)
    s_w = np.float32(37.0)
    for j, v in ((0, 2.5), (17, -0.3), (63, 1000.0)):
        x = np.zeros((1, k), np.float32)
        x[0, j] = v
        q, s, _ = o.activation_quant(x, lib)
        y, _ = o.bitlinear(p, s_w, k, q, s, lib)
        exact = t[:, j].astype(np.float64) * v / float(s_w)
        assert np.all(np.abs(y[0] - exact) <= 4 * np.abs(exact) * 2.0 ** -24), (j, y[0], exact)


def pin_bitlinear_error_bound(o, lib):
    """The whole BitLinear approximates the float product (t/s_w) x: the error
    is at most sum_k |t[n][k]| * (0.5 + eps) / (s_a s_w), the activation
    quantization step, plus fp32 rounding of the dequant."""
    g = _rng(47)
    n, k, m = 40, 256, 3
    t = g.integers(-1, 2, (n, k)).astype(np.int8)
    p = o.pack(t, lib)
    s_w = np.float32(29.5)
    x = g.standard_normal((m, k)).astype(np.float32)
    q, s, _ = o.activation_quant(x, lib)
    y, _ = o.bitlinear(p, s_w, k, q, s, lib)
    exact = x.astype(np.float64) @ t.astype(np.float64).T / float(s_w)
    for r in range(m):
        bound = np.abs(t).sum(1) * (0.5 + 1e-4) / (float(s[r]) * float(s_w)) + 4 * np.abs(y[r]) * 2.0 ** -24
        assert np.all(np.abs(y[r] - exact[r]) <= bound + 1e-12), r


# --- argmax ------------------------------------------------------------------------

def pin_argmax(o, lib):
    """Lowest index wins ties; agrees with numpy's argmax (first occurrence)."""
    acc = np.array([[1, 5, 5, 2], [7, 7, 7, 7], [-3, -1, -2, -1], [0, 0, 0, 9]], np.int32)
    assert o.argmax_rows(acc, lib).tolist() == [1, 0, 1, 3]
    g = _rng(51)
    a = g.integers(-5, 5, (50, 30)).astype(np.int32)
    assert (o.argmax_rows(a, lib) == np.argmax(a, axis=1)).all()


# --- FFN ------------------------------------------------------------------------------

def pin_relu2_mul(o, lib):
    """h = relu(gate)^2 * up, elementwise: the gate is squared after the ReLU, the
    up projection passes through unchanged."""
    gate = np.array([-2.0, 0.0, 3.0, 0.5, 1.0], np.float32)
    up = np.array([5.0, 7.0, 2.0, -4.0, -1.5], np.float32)
    h = o.relu2_mul(gate, up, lib)
    assert h.tolist() == [0.0, 0.0, 18.0, -1.0, -1.5]


def _ffn_onehot_expect(tg, tu, td, sg, su, sd, d, j, sv):
    """Closed form of the FFN for a one-hot input with sign sv at j, unit gains and
    eps = 0 (see pin_ffn_onehot). Returns gate, up, h, out and the bound on
    |out - exact| set by the quantization step of q2."""
    gate = tg[:, j] * sv * np.sqrt(d) / float(sg)
    up = tu[:, j] * sv * np.sqrt(d) / float(su)
    h = np.maximum(gate, 0) ** 2 * up
    if not np.any(h != 0):
        return gate, up, h, np.zeros(td.shape[0]), np.zeros(td.shape[0])
    hn = h / np.sqrt(np.mean(h * h))
    out = td.astype(np.float64) @ hn / float(sd)
    step = np.abs(td).sum(1) * 0.5 / (127.0 / np.abs(hn).max()) / float(sd)
    return gate, up, h, out, step


def pin_ffn_onehot(o, lib):
    """Closed form of the FFN for a one-hot input x = v e_j with unit gains and
    eps = 0: the norm maps x to sqrt(D) sign(v) e_j, so q1 = 127 sign(v) e_j and
    gate[f] = T_g[f][j] sign(v) sqrt(D)/s_g, up[f] = T_u[f][j] sign(v) sqrt(D)/s_u,
    h = relu(gate)^2 up; the sub-norm and down projection then give
    out = (t_d/s_d) * rmsnorm(h) up to the quantization step of q2."""
    g = _rng(61)
    d, f = 16, 32
    tg = g.integers(-1, 2, (f, d)).astype(np.int8)
    tu = g.integers(-1, 2, (f, d)).astype(np.int8)
    td = g.integers(-1, 2, (d, f)).astype(np.int8)
    sg, su, sd = np.float32(2.0), np.float32(8.0), np.float32(2.0)
    ones_d, ones_f = np.ones(d, np.float32), np.ones(f, np.float32)
    for j, v in ((3, 1.75), (10, -0.5)):
        x = np.zeros((1, d), np.float32)
        x[0, j] = v
        r = o.ffn(x, ones_d, ones_f, 0.0, o.pack(tg, lib), sg, o.pack(tu, lib), su, o.pack(td, lib), sd, lib)
        gate, up, h, out, step = _ffn_onehot_expect(tg, tu, td, sg, su, sd, d, j, np.sign(v))
        assert np.allclose(r["gate"][0], gate, rtol=1e-6, atol=0)
        assert np.allclose(r["up"][0], up, rtol=1e-6, atol=0)
        assert np.allclose(r["h"][0], h, rtol=1e-5, atol=1e-7)
        assert np.all(np.abs(r["out"][0] - out) <= step + 1e-5), (r["out"][0], out)


def pin_layer_closed_form(o, lib):
    """One layer in closed form: x = 0, the stand-in z = v e_0 and W_o with a single
    +1 at (j, 0). Then a (the attention-norm quant of x) is 0, so q/k/v are 0;
    the o projection gives y_o = sign(v) sqrt(D)/s_o e_j; the FFN reads
    x' = x + y_o (one-hot) and adds its one-hot closed form:
    x_next = y_o + out(x'). (A tiny eps keeps the norm of x = 0 finite.)"""
    g = _rng(64)
    d, f = 16, 32
    tg = g.integers(-1, 2, (f, d)).astype(np.int8)
    tu = g.integers(-1, 2, (f, d)).astype(np.int8)
    td = g.integers(-1, 2, (d, f)).astype(np.int8)
    for j, v in ((5, 0.75), (12, -3.0)):
        to = np.zeros((d, d), np.int8)
        to[j, 0] = 1
        lw = {"wq": o.pack(g.integers(-1, 2, (d, d)).astype(np.int8), lib), "sq": np.float32(30.0),
              "wk": o.pack(g.integers(-1, 2, (d, d)).astype(np.int8), lib), "sk": np.float32(31.0),
              "wv": o.pack(g.integers(-1, 2, (d, d)).astype(np.int8), lib), "sv": np.float32(32.0),
              "wo": o.pack(to, lib), "so": np.float32(2.0),
              "wg": o.pack(tg, lib), "sg": np.float32(2.0), "wu": o.pack(tu, lib), "su": np.float32(8.0),
              "wd": o.pack(td, lib), "sd": np.float32(2.0),
              "g_attn": np.ones(d, np.float32), "g_attn_sub": np.ones(d, np.float32),
              "g_ffn": np.ones(d, np.float32), "g_ffn_sub": np.ones(f, np.float32)}
        z = np.zeros((1, d), np.float32)
        z[0, 0] = v
        lw["z"] = z
        # eps = 1e-12 keeps r finite for x = 0 and moves the closed form by ~1e-11.
        x_next, qkv = o.layer(np.zeros((1, d), np.float32), lw, 1e-12, lib)
        assert (qkv == 0).all()
        yo = np.zeros(d)
        yo[j] = np.sign(v) * np.sqrt(d) / 2.0
        _, _, _, out, step = _ffn_onehot_expect(tg, tu, td, 2.0, 8.0, 2.0, d, j, np.sign(v))
        assert np.all(np.abs(x_next[0] - (yo + out)) <= step + 1e-5), (x_next[0], yo + out)


def pin_ffn_zero_paths(o, lib):
    """Zero up weights (or a gate that is never positive) give h = 0 and out = 0."""
    g = _rng(62)
    d, f = 16, 32
    x = g.standard_normal((2, d)).astype(np.float32)
    tg = g.integers(-1, 2, (f, d)).astype(np.int8)
    td = g.integers(-1, 2, (d, f)).astype(np.int8)
    gd, gf = np.ones(d, np.float32), np.ones(f, np.float32)
    r = o.ffn(x, gd, gf, 1e-5, o.pack(tg, lib), 10.0, o.pack(np.zeros((f, d), np.int8), lib), 10.0,
              o.pack(td, lib), 10.0, lib)
    assert (r["h"] == 0).all() and (r["out"] == 0).all()
    xpos = np.abs(x)
    r = o.ffn(xpos, gd, gf, 1e-5, o.pack(-np.ones((f, d), np.int8), lib), 10.0, o.pack(tg, lib), 10.0,
              o.pack(td, lib), 10.0, lib)
    assert (r["gate"] < 0).all() and (r["h"] == 0).all() and (r["out"] == 0).all()


def pin_ffn_subnorm_present(o, lib):
    """The sub-norm gain scales h before its quantization: doubling the sub-norm
    gain leaves q2 unchanged and doubles out exactly (s2 halves), while a gain that zeroes
    half of h changes q2 (the norm sits between the gating and the down
    projection)."""
    g = _rng(63)
    d, f = 16, 64
    x = g.standard_normal((1, d)).astype(np.float32)
    w = [o.pack(g.integers(-1, 2, s).astype(np.int8), lib) for s in ((f, d), (f, d), (d, f))]
    gd = np.ones(d, np.float32)
    r1 = o.ffn(x, gd, np.ones(f, np.float32), 0.0, w[0], 3.0, w[1], 3.0, w[2], 3.0, lib)
    r2 = o.ffn(x, gd, np.full(f, 2.0, np.float32), 0.0, w[0], 3.0, w[1], 3.0, w[2], 3.0, lib)
    assert (r1["q2"] == r2["q2"]).all() and (r2["out"] == 2 * r1["out"]).all()
    half = np.ones(f, np.float32)
    half[: f // 2] = 0.0
    r3 = o.ffn(x, gd, half, 0.0, w[0], 3.0, w[1], 3.0, w[2], 3.0, lib)
    hz = r1["h"][0].copy()
    if np.any(hz[: f // 2] != 0):
        assert (r3["q2"][0, : f // 2] == 0).all()
        assert not (r3["q2"] == r1["q2"]).all()


# --- layer chain ------------------------------------------------------------------------

def _layer_weights(o, lib, g, d, f, zero=()):
    lw = {}
    for name, (n, k) in zip(("wq", "wk", "wv", "wo", "wg", "wu", "wd"),
                            [(d, d)] * 4 + [(f, d), (f, d), (d, f)]):
        t = np.zeros((n, k), np.int8) if name in zero else g.integers(-1, 2, (n, k)).astype(np.int8)
        lw[name] = o.pack(t, lib)
        lw["s" + name[1]] = np.float32(g.uniform(20, 60))
    lw["z"] = g.standard_normal((1, d)).astype(np.float32)
    for key, k in (("g_attn", d), ("g_attn_sub", d), ("g_ffn", d), ("g_ffn_sub", f)):
        lw[key] = g.uniform(0.5, 1.5, k).astype(np.float32)
    return lw


def pin_chain_zero_weights(o, lib):
    """With zero o, gate, up and down weights every residual adds +0 and x passes
    through the stream unchanged; q/k/v still read the attention norm of x."""
    g = _rng(71)
    d, f = 16, 32
    x = g.standard_normal((1, d)).astype(np.float32)
    layers = [_layer_weights(o, lib, g, d, f, zero=("wo", "wg", "wu", "wd")) for _ in range(3)]
    x2, qkvs = o.chain(x, layers, 1e-5, lib)
    assert (x2 == x).all()
    for lw, qkv in zip(layers, qkvs):
        a, sa, _ = o.quant_act(x, lw["g_attn"], 1e-5, lib)
        tq = o.unpack(lw["wq"], d, lib)
        q_ref = a.astype(np.int64) @ tq.astype(np.int64).T
        assert (np.round(qkv[0, :d].astype(np.float64) * float(sa[0]) * float(lw["sq"])) == q_ref[0]).all()


def pin_chain_residual(o, lib):
    """The o projection output and the FFN output are each added to x once: with
    only wo nonzero, x_next - x equals the o projection of the stand-in z."""
    g = _rng(72)
    d, f = 16, 32
    x = g.standard_normal((1, d)).astype(np.float32)
    lw = _layer_weights(o, lib, g, d, f, zero=("wg", "wu", "wd"))
    x2, _ = o.layer(x, lw, 1e-5, lib)
    zq, zs, _ = o.quant_act(lw["z"], lw["g_attn_sub"], 1e-5, lib)
    to = o.unpack(lw["wo"], d, lib).astype(np.int64)
    yo = (zq.astype(np.int64) @ to.T)[0] / (float(zs[0]) * float(lw["so"]))
    assert np.allclose(x2[0] - x[0], yo, rtol=1e-5, atol=1e-6)


# --- floating-point operation order, derived with exact rational arithmetic -------------
#
# The pages fix no fp32 operation order, so the oracle states one (the numerics
# contract of the ABI header, the same readings on both sides). The pins below
# derive the bits that order must give with exact rational arithmetic and one
# explicit IEEE rounding per operation (tests/exact_fp.py, no floating-point
# hardware), on inputs where the plausible other orders round differently. Each
# pin also checks that its inputs tell the stated order from those others, so it
# cannot pass by accident on inputs where every order agrees.

def _differs(counts, name, got, want):
    if got != want:
        counts[name] = counts.get(name, 0) + 1


def _require_discrimination(counts, names, what):
    missing = [n for n in names if counts.get(n, 0) == 0]
    assert not missing, f"{what}: the inputs do not tell the stated order from {missing}"


def pin_dequant_order_exact(o, lib):
    """Dequant rounds three times, in this order: p = fl32(s_a * s_w),
    inv = fl32(1 / p), y = fl32(acc * inv). Seeded accumulators over the whole
    int32 range a BitLinear reaches (|acc| <= 127 * 10240) and scales of the
    sizes the path sees; expected bits from exact rationals. Ruled out by the
    same inputs: acc / p, acc * fl32(fl32(1/s_a) * fl32(1/s_w)), and an inverse
    taken from the exact product fl32(1 / (s_a s_w))."""
    from exact_fp import f32, fl32
    g = _rng(81)
    m, n = 48, 12
    counts = {}
    for s_w in (np.float32(23.75), np.float32(g.uniform(20, 60)), np.float32(g.uniform(20, 60))):
        acc = g.integers(-1_300_480, 1_300_481, (m, n)).astype(np.int32)
        s_a = g.uniform(0.5, 400.0, m).astype(np.float32)
        y = o.dequant(acc, s_a, s_w, lib)
        sw = f32(s_w)
        for r in range(m):
            sa = f32(s_a[r])
            p = fl32(sa * sw)
            inv = fl32(1 / p)
            inv_split = fl32(fl32(1 / sa) * fl32(1 / sw))
            inv_exact = fl32(1 / (sa * sw))
            for c in range(n):
                a = Fraction(int(acc[r, c]))
                want = fl32(a * inv)
                assert Fraction(float(y[r, c])) == want, (r, c, float(y[r, c]), float(want))
                _differs(counts, "acc / p", fl32(a / p), want)
                _differs(counts, "(1/s_a)(1/s_w)", fl32(a * inv_split), want)
                _differs(counts, "1/(s_a s_w) exact", fl32(a * inv_exact), want)
    _require_discrimination(counts, ("acc / p", "(1/s_a)(1/s_w)", "1/(s_a s_w) exact"), "dequant")


def pin_rmsnorm_apply_exact(o, lib):
    """RMSNorm: w = fl64(1 / fl64(sqrt(fl64(fl64(ss / K) + eps)))), r = fl32(w),
    y = fl32(fl32(x * r) * g). The inputs have at most 12 significant bits, so
    every x^2 and their sum are exact in fp64 whatever the summation order, and
    ss is the exact sum of squares; every other step is derived with one exact
    IEEE rounding. Ruled out by the same inputs: x * fl32(r * g), one rounding
    of the exact x r g, and x * w taken before r is rounded to fp32."""
    from exact_fp import f32, fl32, fl64, sqrt64
    g = _rng(82)
    counts = {}
    for k, eps in ((64, 1e-5), (640, 1e-6), (1024, 0.0), (96, 0.25)):
        x = (g.integers(-2047, 2048, (3, k)) / 256.0).astype(np.float32)
        gain = g.uniform(0.5, 1.5, k).astype(np.float32)
        y = o.rmsnorm(x, gain, eps, lib)
        eps_q = f32(np.float32(eps))
        for row in range(3):
            ss = sum(f32(v) ** 2 for v in x[row])
            assert fl64(ss) == ss
            w = fl64(1 / sqrt64(fl64(fl64(ss / k) + eps_q)))
            r = fl32(w)
            for i in range(k):
                xi, gi = f32(x[row, i]), f32(gain[i])
                want = fl32(fl32(xi * r) * gi)
                assert Fraction(float(y[row, i])) == want, (k, row, i)
                _differs(counts, "x (r g)", fl32(xi * fl32(r * gi)), want)
                _differs(counts, "x r g rounded once", fl32(xi * r * gi), want)
                _differs(counts, "x w before rounding r", fl32(fl32(xi * w) * gi), want)
    _require_discrimination(counts, ("x (r g)", "x r g rounded once", "x w before rounding r"), "rmsnorm")


def pin_quant_order_exact(o, lib):
    """activation_quant: s_a = fl32(127 / absmax), v = fl32(y * s_a),
    q = rne(v). Rows hold values placed within a few fp32 ulps of a half-integer
    step y s_a = j + 1/2, where the order of roundings decides the code. Expected
    codes from exact rationals. Ruled out by the same rows: fl32(fl32(y / absmax)
    * 127), rounding the exact product y s_a, and a product with the fp64 scale
    127 / absmax (unrounded to fp32)."""
    from exact_fp import f32, fl32, fl64, rne_int
    g = _rng(83)
    counts = {}
    for amax in (np.float32(1.0), np.float32(g.uniform(0.3, 30)), np.float32(g.uniform(0.3, 30)),
                 np.float32(g.uniform(0.3, 30)), np.float32(g.uniform(30, 3000))):
        A = f32(amax)
        s_a = fl32(Fraction(127) / A)
        vals = [float(amax)]
        for _ in range(60):
            j = int(g.integers(0, 126))
            sign = 1 if g.random() < 0.5 else -1
            y0 = np.float32(float(Fraction(2 * j + 1, 2) / s_a)) * np.float32(sign)
            for step in range(-2, 3):
                v = y0
                for _ in range(abs(step)):
                    v = np.nextafter(v, np.float32(np.inf) if step > 0 else np.float32(-np.inf))
                if abs(float(v)) < float(amax):
                    vals.append(float(v))
        row = np.array(vals, np.float32).reshape(1, -1)
        q, s, _ = o.activation_quant(row, lib)
        assert Fraction(float(s[0])) == s_a
        for i, v in enumerate(row[0]):
            y = f32(v)
            want = max(-128, min(127, rne_int(fl32(y * s_a))))
            assert int(q[0, i]) == want, (float(amax), i, float(v), int(q[0, i]), want)
            _differs(counts, "y / absmax * 127", max(-128, min(127, rne_int(fl32(fl32(y / A) * 127)))), want)
            _differs(counts, "exact y s_a", max(-128, min(127, rne_int(y * s_a))), want)
            _differs(counts, "fp64 scale", max(-128, min(127, rne_int(fl32(fl64(y * fl64(Fraction(127) / A)))))),
                     want)
    _require_discrimination(counts, ("y / absmax * 127", "exact y s_a", "fp64 scale"), "activation_quant")


def pin_relu2_order_exact(o, lib):
    """The FFN gating rounds twice, square first: h = fl32(fl32(g g) * up) with
    g = max(gate, 0). Expected bits from exact rationals on seeded gate / up
    values. Ruled out by the same inputs: fl32(fl32(g up) g) and one rounding of
    the exact g^2 up."""
    from exact_fp import f32, fl32
    g = _rng(84)
    gate = (g.standard_normal(600) * 3).astype(np.float32)
    up = (g.standard_normal(600) * 3).astype(np.float32)
    h = o.relu2_mul(gate, up, lib)
    counts = {}
    for i in range(gate.size):
        gg = max(f32(gate[i]), Fraction(0))
        u = f32(up[i])
        want = fl32(fl32(gg * gg) * u)
        assert Fraction(float(h[i])) == want, (i, float(gate[i]), float(up[i]))
        _differs(counts, "(g up) g", fl32(fl32(gg * u) * gg), want)
        _differs(counts, "g^2 up rounded once", fl32(gg * gg * u), want)
    _require_discrimination(counts, ("(g up) g", "g^2 up rounded once"), "relu2_mul")


def pin_residual_exact(o, lib):
    """The residual add is one fp32 addition: x + d rounded once."""
    from exact_fp import f32, fl32
    g = _rng(85)
    x = (g.standard_normal(300) * 10).astype(np.float32)
    d = (g.standard_normal(300) * 1e-3).astype(np.float32)
    out = o.residual_add(x, d, lib)
    for i in range(x.size):
        assert Fraction(float(out[i])) == fl32(f32(x[i]) + f32(d[i])), i


# --- embedding lookup and the penalised greedy choice --------------------------------------

def pin_embed_closed_form(o, lib):
    """The ternary embedding returns row tokens[r] of the table dequantized as
    t / s_e: with s_e = 4 every value is exactly -0.25, 0 or 0.25; with s_e = 37
    the nonzero values are +-fl32(1/37) (exact rationals); an id outside the
    table gives a zero row. The rows are checked against the unpacked table the
    test built (not the oracle's unpack), on a non-square table so a transposed
    or shifted row fails."""
    from exact_fp import f32, fl32
    g = _rng(91)
    vocab, d = 7, 24
    t = g.integers(-1, 2, (vocab, d)).astype(np.int8)
    table = o.pack(t, lib)
    tokens = np.array([2, 0, 6, -1, 7, 3, 2], np.int32)
    x = o.embed(table, np.float32(4.0), tokens, d, lib)
    for r, v in enumerate(tokens):
        want = t[v].astype(np.float32) * np.float32(0.25) if 0 <= v < vocab else np.zeros(d, np.float32)
        assert (x[r] == want).all(), (r, v)
    x = o.embed(table, np.float32(37.0), tokens, d, lib)
    inv = fl32(Fraction(1) / f32(np.float32(37.0)))
    for r, v in enumerate(tokens):
        for k in range(d):
            want = (int(t[v, k]) * inv) if 0 <= v < vocab else Fraction(0)
            assert Fraction(float(x[r, k])) == want, (r, k)
    assert (x[3] == 0).all() and (x[4] == 0).all() and not np.signbit(x[3]).any()


def pin_embed_one_hot_rows(o, lib):
    """Table rows with a single +1 (the rest -1): the lookup of row v has +1/s_e
    exactly at that column and -1/s_e everywhere else."""
    vocab, d = 5, 16
    t = -np.ones((vocab, d), np.int8)
    cols = [0, 15, 7, 8, 3]
    for v, c in enumerate(cols):
        t[v, c] = 1
    x = o.embed(o.pack(t, lib), np.float32(2.0), np.arange(vocab, dtype=np.int32), d, lib)
    for v, c in enumerate(cols):
        want = np.full(d, -0.5, np.float32)
        want[c] = 0.5
        assert (x[v] == want).all(), v


def _penalty_cases():
    for row in _read_fixture("penalty_cases.txt"):
        lg, hist, p, idx, bits, _why = [f.strip() for f in row.split("|")]
        logits = np.array([float(v) for v in lg.split()], np.float32)
        h = [int(v) for v in hist.split()]
        yield logits, h, np.float32(float(p)), int(idx), [int(b, 16) for b in bits.split()]


def pin_penalty_golden(o, lib):
    """Hand-worked penalised greedy choices (tests/golden/penalty_cases.txt): the
    index and the bits of every penalised logit, one row at a time and all
    rows at once (each row with its own history, padded history rows and a
    history length below the stride)."""
    cases = list(_penalty_cases())
    for logits, h, p, idx, bits in cases:
        hist = np.array([h + [0]], np.int32)  # one slot past the length: must be ignored
        got, pen = o.penalty_argmax(logits.reshape(1, -1), hist, np.array([len(h)], np.int32), p, lib)
        assert int(got[0]) == idx, (logits, h, p, int(got[0]), idx)
        assert pen[0].view(np.uint32).tolist() == bits, (logits, h, pen[0])


def pin_penalty_rows_are_independent(o, lib):
    """Several rows at once: row r uses only hist[r][0 .. hist_len[r]); a length
    beyond the stride is clamped to it."""
    g = _rng(92)
    m, n, stride = 5, 40, 6
    logits = g.standard_normal((m, n)).astype(np.float32)
    hist = g.integers(-3, n + 3, (m, stride)).astype(np.int32)
    hist_len = np.array([0, 3, 6, 2, 99], np.int32)
    idx, pen = o.penalty_argmax(logits, hist, hist_len, np.float32(1.3), lib)
    for r in range(m):
        one, pen1 = o.penalty_argmax(logits[r:r + 1], hist[r:r + 1, :min(hist_len[r], stride)],
                                     np.array([min(hist_len[r], stride)], np.int32), np.float32(1.3), lib)
        assert idx[r] == one[0] and (pen[r] == pen1[0]).all(), r
        touched = {int(v) for v in hist[r, :min(hist_len[r], stride)] if 0 <= v < n}
        for c in range(n):
            if c not in touched:
                assert pen[r, c] == logits[r, c]
            elif logits[r, c] > 0:
                assert pen[r, c] < logits[r, c]
            else:
                assert pen[r, c] <= logits[r, c]
        assert idx[r] == int(np.argmax(pen[r]))


# --- top-k and nucleus sampling ----------------------------------------------------------------

def pin_sample_exp_vs_library(o, lib):
    """The sampler's exponential against the C library's (math.exp): within 2
    fp64 ulps on a grid and on random points of [-32, 0], exactly 1 at 0 and
    exactly 2^-k at -k ln2 for small k, 0 below -32, and monotone."""
    import math
    g = _rng(93)
    xs = np.concatenate([np.linspace(-32.0, 0.0, 4001), -g.random(2000) * 32.0, -g.random(500) * 1e-6])
    prev = None
    for x in np.sort(xs):
        got = o.exp_neg(float(x), lib)
        want = math.exp(float(x))
        assert abs(got - want) <= 2 * abs(want) * 2.0 ** -52, (x, got, want)
        if prev is not None:
            assert got >= prev
        prev = got
    assert o.exp_neg(0.0, lib) == 1.0
    assert o.exp_neg(-32.5, lib) == 0.0 and o.exp_neg(-1e9, lib) == 0.0


def _grid_counts(o, lib, logits, sampler, n_u):
    """Tokens drawn for the regular u grid (i + 1/2) / n_u: each token's count
    divided by n_u is within 1 / n_u of its probability, for any monotone map."""
    us = (np.arange(n_u) + 0.5) / n_u
    toks = sampler(np.repeat(logits.reshape(1, -1), n_u, 0), us)
    return toks, np.bincount(toks, minlength=logits.size) / n_u


def pin_sample_topk_distribution(o, lib):
    """Top-k draws over a regular grid of u reproduce the softmax of the k
    largest logits at temperature T (probabilities from numpy's exp in fp64),
    never choose a token outside them, and walk the tokens in descending logit
    order as u grows."""
    g = _rng(94)
    logits = (g.standard_normal(12) * 1.5).astype(np.float32)
    k, t = 6, 0.8
    toks, freq = _grid_counts(o, lib, logits, lambda L, U: o.sample_topk(L, k, t, U, lib), 20000)
    top = np.argsort(-logits.astype(np.float64), kind="stable")[:k]
    w = np.exp((logits[top].astype(np.float64) - logits.max()) / t)
    prob = np.zeros(logits.size)
    prob[top] = w / w.sum()
    assert np.all(np.abs(freq - prob) <= 1.0 / 20000 + 1e-9), (freq, prob)
    ranks = {int(tok): r for r, tok in enumerate(top)}
    seq = [ranks[int(v)] for v in toks]
    assert all(a <= b for a, b in zip(seq, seq[1:])), "tokens must be walked in sorted order"


def pin_sample_topk_special_cases(o, lib):
    """k = 1 is the greedy choice (numpy's first argmax) for any u; a tiny
    temperature leaves only the largest logit; two equal logits split [0, 1) at
    exactly u = 1/2: the weights are 2^40 each, r = floor(u * 2^41), and the
    lower index is taken while r < 2^40."""
    g = _rng(95)
    logits = g.integers(-3, 4, (6, 9)).astype(np.float32)  # many ties
    for u in (0.0, 0.3, 0.999999):
        got = o.sample_topk(logits, 1, 1.0, np.full(6, u), lib)
        assert (got == np.argmax(logits, axis=1)).all()
    distinct = (g.permutation(9) - 4.0).astype(np.float32).reshape(1, -1)
    for u in (0.0, 0.5, 0.9999):
        assert o.sample_topk(distinct, 9, 1e-4, [u], lib)[0] == int(np.argmax(distinct))
    pair = np.array([[0.25, 2.0, 2.0, -1.0]], np.float32)
    assert o.sample_topk(pair, 2, 1.0, [0.5 - 2.0 ** -53], lib)[0] == 1
    assert o.sample_topk(pair, 2, 1.0, [0.5], lib)[0] == 2
    assert o.sample_topk(pair, 2, 1.0, [0.0], lib)[0] == 1


def pin_sample_tie_order(o, lib):
    """Among equal logits the lower index comes first: it is kept first at the
    top-k boundary and sampled for the lower u."""
    l1 = np.array([[1.0, 3.0, 3.0, 2.0]], np.float32)
    assert o.sample_topk(l1, 2, 1.0, [0.25], lib)[0] == 1 and o.sample_topk(l1, 2, 1.0, [0.75], lib)[0] == 2
    l2 = np.array([[3.0, 2.0, 2.0, 1.0]], np.float32)
    reach = {int(o.sample_topk(l2, 2, 1.0, [u], lib)[0]) for u in np.linspace(0.0, 0.999, 200)}
    assert reach == {0, 1}


def pin_sample_nucleus(o, lib):
    """Nucleus sets from logits ln(1/2), ln(1/4), ln(1/8), ln(1/16), ln(1/16):
    the smallest sorted prefix whose probability reaches p, the token that
    crosses p included (p = 0.6 keeps two tokens, where a literal
    "cumulative <= p" would keep one), p >= 1 keeps every token; draws over a
    u grid follow the renormalised probabilities of the kept tokens."""
    probs = np.array([0.5, 0.25, 0.125, 0.0625, 0.0625])
    order = np.array([3, 0, 4, 1, 2])  # scatter them, so index order is not sorted order
    logits = np.empty(5, np.float32)
    logits[order] = np.log(probs).astype(np.float32)
    for p, kept in ((0.3, 1), (0.6, 2), (0.74, 2), (0.8, 3), (0.9, 4), (1.0, 5)):
        toks, freq = _grid_counts(o, lib, logits, lambda L, U: o.sample_topp(L, p, 1.0, U, lib), 4000)
        assert set(np.unique(toks).tolist()) == set(order[:kept].tolist()), (p, np.unique(toks))
        w = np.exp(logits[order[:kept]].astype(np.float64) - logits.max())
        want = np.zeros(5)
        want[order[:kept]] = w / w.sum()
        assert np.all(np.abs(freq - want) <= 1.0 / 4000 + 1e-9), (p, freq, want)


def pin_sample_temperature(o, lib):
    """Temperature divides the logits: T = 2 flattens two tokens with logits
    ln(3) and 0 from probabilities 3/4, 1/4 to sqrt(3) / (1 + sqrt(3)) and
    1 / (1 + sqrt(3))."""
    logits = np.array([np.log(3.0), 0.0], np.float32)
    for t in (1.0, 2.0, 0.5):
        _, freq = _grid_counts(o, lib, logits, lambda L, U: o.sample_topk(L, 2, t, U, lib), 10000)
        w = np.exp((logits.astype(np.float64) - logits.max()) / t)
        assert abs(freq[0] - w[0] / w.sum()) <= 1e-4 + 1e-9, (t, freq)


# --- rotary embedding and single-token attention -----------------------------------------------

def pin_rope_table(o, lib):
    """The table against numpy's fp64 cos / sin rounded once: position 0 is the
    identity (cos 1, sin 0), frequency 0 turns by one radian per position,
    frequency hd/4 by base^(-1/2) radians (1/100 for base 10000), and every
    entry is fl32 of cos / sin of pos * base^(-2i/hd)."""
    hd, npos = 80, 40
    c, s = o.rope_table(10000.0, hd, npos, lib)
    assert (c[0] == 1.0).all() and (s[0] == 0.0).all()
    pos = np.arange(npos, dtype=np.float64)
    assert (c[:, 0] == np.cos(pos).astype(np.float32)).all() and (s[:, 0] == np.sin(pos).astype(np.float32)).all()
    assert (c[:, hd // 4] == np.cos(pos / 100.0).astype(np.float32)).all()
    theta = 10000.0 ** (-(2.0 * np.arange(hd // 2)) / hd)
    ang = pos[:, None] * theta[None, :]
    assert (c == np.cos(ang).astype(np.float32)).all() and (s == np.sin(ang).astype(np.float32)).all()


def pin_rope_rotation(o, lib):
    """The rotation turns pairs (x[2i], x[2i+1]) of a head vector: a one-hot
    vector stays within its pair; the four products and the difference / sum
    round in the stated order (exact rationals); the norm is kept within a few
    ulps; and q(m) . k(n) depends on m - n only (the defining property), within
    fp32 rounding."""
    from exact_fp import f32, fl32
    hd = 16
    c, s = o.rope_table(10000.0, hd, 64, lib)
    for j in range(hd):
        e = np.zeros(hd, np.float32)
        e[j] = 1.0
        r = o.rope_apply(e, c[7], s[7], lib)
        pair = {2 * (j // 2), 2 * (j // 2) + 1}
        assert all(r[i] == 0 for i in range(hd) if i not in pair), j
    g = _rng(96)
    x = g.standard_normal(hd).astype(np.float32)
    r = o.rope_apply(x, c[9], s[9], lib)
    for i in range(hd // 2):
        a, b, ci, si = f32(x[2 * i]), f32(x[2 * i + 1]), f32(c[9, i]), f32(s[9, i])
        assert Fraction(float(r[2 * i])) == fl32(fl32(a * ci) - fl32(b * si))
        assert Fraction(float(r[2 * i + 1])) == fl32(fl32(a * si) + fl32(b * ci))
    assert abs(np.linalg.norm(r.astype(np.float64)) / np.linalg.norm(x.astype(np.float64)) - 1) < 1e-6
    q = g.standard_normal(hd).astype(np.float32)
    k = g.standard_normal(hd).astype(np.float32)
    dots = []
    for mpos, npos in ((10, 3), (20, 13), (40, 33)):
        dots.append(float(o.rope_apply(q, c[mpos], s[mpos], lib).astype(np.float64) @
                          o.rope_apply(k, c[npos], s[npos], lib).astype(np.float64)))
    assert max(dots) - min(dots) < 1e-5 * (np.abs(q).sum() * np.abs(k).sum())


def pin_attention_closed_forms(o, lib):
    """Attention over positions 0 .. pos: at pos 0 the output is v_0 exactly;
    with q = 0 every weight is equal and the output is the mean of v_0 .. v_pos;
    otherwise it equals softmax(q k^T / sqrt(hd)) V from numpy's fp64 exp,
    rounded once to fp32 (within one fp32 ulp of that value); heads and
    sequences use only their own q and cache."""
    g = _rng(97)
    m, heads, hd, smax = 2, 3, 8, 10
    kc = g.standard_normal((m, heads, smax, hd)).astype(np.float32)
    vc = g.standard_normal((m, heads, smax, hd)).astype(np.float32)
    q = g.standard_normal((m, heads, hd)).astype(np.float32)
    out0 = o.attention(q, kc, vc, 0, lib)
    assert (out0.reshape(m, heads, hd) == vc[:, :, 0, :]).all()
    outz = o.attention(np.zeros_like(q), kc, vc, 6, lib).reshape(m, heads, hd)
    assert np.allclose(outz, vc[:, :, :7, :].astype(np.float64).mean(2), rtol=0, atol=1e-6)
    for pos in (3, 9):
        out = o.attention(q, kc, vc, pos, lib).reshape(m, heads, hd)
        for r in range(m):
            for h in range(heads):
                sc = kc[r, h, :pos + 1].astype(np.float64) @ q[r, h].astype(np.float64) / np.sqrt(hd)
                w = np.exp(sc - sc.max())
                want = (w @ vc[r, h, :pos + 1].astype(np.float64)) / w.sum()
                ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
                assert np.all(np.abs(out[r, h] - want) <= ulp), (pos, r, h)


def pin_layer_attention_position0(o, lib):
    """At position 0 the attention output is the value vector itself, so the
    attention layer equals the stand-in layer fed z = v (the o projection then
    reads quant(rmsnorm(v))), and the caches receive the rotated k (position 0:
    unrotated) and v."""
    g = _rng(98)
    d, f, heads, m = 32, 64, 4, 2
    lw = _layer_weights(o, lib, g, d, f)
    x = g.standard_normal((m, d)).astype(np.float32)
    c, s = o.rope_table(10000.0, d // heads, 4, lib)
    kc = np.zeros((m, heads, 4, d // heads), np.float32)
    vc = np.zeros_like(kc)
    xa, qkv, attn = o.layer_attn(x, lw, 1e-5, heads, c, s, kc, vc, 0, lib=lib)
    v = qkv[:, 2 * d:]
    assert (attn == v).all()
    assert (kc[:, :, 0, :].reshape(m, d) == qkv[:, d:2 * d]).all() and (vc[:, :, 0, :].reshape(m, d) == v).all()
    lw2 = dict(lw)
    lw2["z"] = v
    xs, _ = o.layer(x, lw2, 1e-5, lib)
    assert (xa == xs).all()
    # a later position: the cached k is the rotation of the projected k by that
    # position's table row (first pair of every head, exact rationals), v is
    # stored as it is
    from exact_fp import f32, fl32
    _, qkv3, _ = o.layer_attn(x, lw, 1e-5, heads, c, s, kc, vc, 3, lib=lib)
    hd = d // heads
    for r in range(m):
        for h in range(heads):
            a, b = f32(qkv3[r, d + h * hd]), f32(qkv3[r, d + h * hd + 1])
            ci, si = f32(c[3, 0]), f32(s[3, 0])
            assert Fraction(float(kc[r, h, 3, 0])) == fl32(fl32(a * ci) - fl32(b * si))
            assert Fraction(float(kc[r, h, 3, 1])) == fl32(fl32(a * si) + fl32(b * ci))
    assert (vc[:, :, 3, :].reshape(m, d) == qkv3[:, 2 * d:]).all()
    # q, k, v are the three projections of quant(rmsnorm(x, g_attn)), in that
    # order (numpy's int64 product with the unpacked weights, then the scale)
    a, sa, _ = o.quant_act(x, lw["g_attn"], 1e-5, lib)
    for blk, (wn, sn) in enumerate((("wq", "sq"), ("wk", "sk"), ("wv", "sv"))):
        acc = a.astype(np.int64) @ o.unpack(lw[wn], d, lib).astype(np.int64).T
        got = qkv3[:, blk * d:(blk + 1) * d].astype(np.float64) * sa[:, None].astype(np.float64) * float(lw[sn])
        assert (np.round(got) == acc).all(), wn


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
