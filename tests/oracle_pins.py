"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each pin is a function taking an ``oracle.Oracle`` and raising AssertionError
when the oracle disagrees with the pages, with closed forms, with exact
rational arithmetic or with an independent library routine (numpy's binary16
conversions, numpy's float64 matmul). They are collected by
test_oracle_pins.py, and test_planted_mistakes.py runs them against oracle
builds with one deliberate mistake each to show that every mistake is caught.
"""
import bisect
import json
import os
from fractions import Fraction

import numpy as np

import synthetic

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GROUP = 128


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16_bits(v):
    return np.array(v, dtype=np.float64).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- fp16 codec

def pin_f16_decode_exhaustive(o):
    """All 65,536 binary16 patterns decode as numpy's float16 does."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.f16_to_f64(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def _f16_finite_positive():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    return bits, bits.view(np.float16).astype(np.float64)


def pin_f16_encode_rne(o):
    """Rounding to binary16 (ties to even) agrees with numpy on every finite
    value, every midpoint, both neighbours of every midpoint, overflow edges
    and random doubles over the whole range."""
    bits, vals = _f16_finite_positive()
    assert np.array_equal(o.f64_to_f16(vals), bits)
    assert np.array_equal(o.f64_to_f16(-vals), bits | 0x8000)
    mids = (vals[:-1] + vals[1:]) / 2.0          # exact in float64
    probes = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    probes = np.concatenate([probes, -probes])
    edge = np.array([65504.0, 65519.999, 65520.0, 65536.0, 1e300, 2.0 ** -25,
                     3 * 2.0 ** -26, 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25, 1e-300])
    rng = np.random.default_rng(7)
    rnd = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), 200000)) * rng.choice([-1.0, 1.0], 200000)
    for arr in (probes, edge, -edge, rnd):
        want = arr.astype(np.float16).view(np.uint16)
        got = o.f64_to_f16(arr)
        assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]
    assert o.f64_to_f16(np.array([np.nan]))[0] & 0x7C00 == 0x7C00
    assert o.f64_to_f16(np.array([np.nan]))[0] & 0x03FF != 0


# ------------------------------------------------------------------ layout

def pin_layout_worked_word(o):
    """The nibble interleave reproduces the ValueShuffle word of the H100
    runtime page (and is AWQ's interleaved order)."""
    g = _load("valueshuffle_word.json")
    assert [s // 4 for s in g["shift_of_weight"]] == g["awq_order"]
    slots = [int(name[1:]) for name in g["slot_contents"]]
    assert [slots.index(j) for j in range(8)] == g["awq_order"]
    N, K = 1, 128
    q = np.zeros((N, K), np.uint8)
    q[0, :8] = g["worked_example"]["weights"]
    s = np.zeros((N, 1), np.uint16)
    z = np.zeros((N, 1), np.uint8)
    wq, _, _ = o.pack(q, s, z)
    word = int(wq[:4].view("<u4")[0])
    assert word == int(g["worked_example"]["word_hex"], 16), hex(word)


def pin_layout_tile_locality(o):
    """Layout statement: tile (t, g) is 1024 bytes holding rows 16t..16t+15 and
    columns 128g..128g+127; within it, the 16 bytes of lane l hold one row,
    16t + l % 16. Checked by lighting one weight at a time."""
    N, K = 37, 512
    G = K // GROUP
    rng = np.random.default_rng(3)
    for _ in range(60):
        n, k = int(rng.integers(N)), int(rng.integers(K))
        q = np.zeros((N, K), np.uint8)
        q[n, k] = 15
        wq, _, _ = o.pack(q, np.zeros((N, G), np.uint16), np.zeros((N, G), np.uint8))
        nz = np.flatnonzero(wq)
        assert nz.size == 1
        byte = int(nz[0])
        tile = byte // 1024
        assert tile == (n // 16) * G + k // GROUP
        lane = (byte % 1024) // 16
        assert lane % 16 == n % 16
        kb = (byte % 16) // 4
        assert kb == (k % GROUP) // 32
        assert lane // 16 == (k % 32) // 8


def pin_layout_scale_zero_locality(o):
    """Layout statement for scales and zeros: the block of tile (t, g) holds
    the 16 fp16 scales of rows 16t..16t+15 for group g in row order (32
    bytes at ((t G + g) 16) * 2), and their 16 zero nibbles in 8 bytes at
    (t G + g) * 8, the even row of each pair in the low nibble. Checked by
    lighting one scale and one zero at a time, mostly in row tiles t > 0 and
    in the ragged last tile."""
    N, K = 53, 640
    G = K // GROUP
    rng = np.random.default_rng(5)
    picks = [(int(rng.integers(16, N)), int(rng.integers(G))) for _ in range(40)] + [(N - 1, G - 1), (16, 0), (0, 0)]
    for n, g in picks:
        s = np.zeros((N, G), np.uint16)
        s[n, g] = 0x3C00
        z = np.zeros((N, G), np.uint8)
        z[n, g] = 9
        _, sp, zp = o.pack(np.zeros((N, K), np.uint8), s, z)
        t, i = n // 16, n % 16
        nz = np.flatnonzero(sp)
        assert nz.size == 1 and int(nz[0]) == ((t * G + g) * 16 + i) * 2 + 1, (n, g, nz)  # 0x3C00 little-endian
        nz = np.flatnonzero(zp)
        assert nz.size == 1 and int(nz[0]) == (t * G + g) * 8 + i // 2, (n, g, nz)
        assert int(zp[nz[0]]) == (9 << 4 if i % 2 else 9), (n, g, int(zp[nz[0]]))


def pin_layout_roundtrip(o):
    """unpack(pack(q, s, z)) == (q, s, z) bit for bit, on random data, ragged
    N, G not a multiple of 8, and the all-0 / all-15 / walking-nibble cases."""
    rng = np.random.default_rng(11)
    for N, K in [(1, 128), (17, 384), (40, 1152), (16, 896), (3, 2048)]:
        G = K // GROUP
        cases = [
            (rng.integers(0, 16, (N, K), dtype=np.uint8), rng.integers(0, 65536, (N, G), dtype=np.uint16),
             rng.integers(0, 16, (N, G), dtype=np.uint8)),
            (np.zeros((N, K), np.uint8), np.zeros((N, G), np.uint16), np.zeros((N, G), np.uint8)),
            (np.full((N, K), 15, np.uint8), np.full((N, G), 0xFFFF, np.uint16), np.full((N, G), 15, np.uint8)),
        ]
        walk = np.zeros((N, K), np.uint8)
        walk[np.arange(N)[:, None], (np.arange(N)[:, None] * 7 + np.arange(0, K, 9)[None, :]) % K] = \
            (np.arange(N)[:, None] % 15 + 1)
        cases.append((walk, np.arange(N * G, dtype=np.uint16).reshape(N, G),
                      (np.arange(N * G) % 16).astype(np.uint8).reshape(N, G)))
        for q, s, z in cases:
            wq, sp, zp = o.pack(q, s, z)
            q2, s2, z2 = o.unpack(N, K, wq, sp, zp)
            assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(z, z2)


def pin_layout_padding_zero(o):
    """Rows past N are zero in every buffer."""
    N, K = 5, 640
    G = K // GROUP
    q = np.full((N, K), 15, np.uint8)
    wq, sp, zp = o.pack(q, np.full((N, G), 0x3C00, np.uint16), np.full((N, G), 15, np.uint8))
    q16, s16, z16 = o.unpack(16, K, wq, sp, zp)
    assert not q16[N:].any() and not s16[N:].any() and not z16[N:].any()
    assert (q16[:N] == 15).all()
    assert int(np.unpackbits(wq).sum()) == N * K * 4
    # One 16-row tile per group: 16 scales and 8 zero bytes each, rows past
    # N zero, so each group's block holds exactly N nonzero entries.
    assert sp.size == 16 * G * 2 and zp.size == 16 * G // 2
    blocks = sp.view(np.uint16).reshape(G, 16)
    assert (blocks[:, :N] == 0x3C00).all() and not blocks[:, N:].any()
    zb = zp.reshape(G, 8)
    assert (zb[:, :N // 2] == 0xFF).all() and (zb[:, N // 2] == 0x0F).all() and not zb[:, N // 2 + 1:].any()


# ------------------------------------------------------------- arithmetic

def pin_dequant_special_cases(o):
    """s = 1, z = 0 gives w = q; q = z gives 0; the signed symmetric format of
    the pages (two's-complement nibble t, zero point 0) stored as q = t xor 8,
    z = 8 gives w = t * s; 128 consecutive weights share one scale."""
    rng = np.random.default_rng(5)
    N, K = 9, 768
    G = K // GROUP
    q = rng.integers(0, 16, (N, K), dtype=np.uint8)
    w = o.dequant(q, np.full((N, G), 0x3C00, np.uint16), np.zeros((N, G), np.uint8))
    assert np.array_equal(w, q.astype(np.float64))
    zz = rng.integers(0, 16, (N, G), dtype=np.uint8)
    w = o.dequant(np.repeat(zz, GROUP, axis=1), rng.integers(0, 0x7C00, (N, G), dtype=np.uint16), zz)
    assert not w.any()
    nib = rng.integers(0, 16, (N, K), dtype=np.uint8)
    t = np.where(nib >= 8, nib.astype(np.int64) - 16, nib.astype(np.int64))  # sign extension
    s = _f16_bits(np.abs(rng.normal(0, 0.02, (N, G))) + 1e-3)
    w = o.dequant(nib ^ 8, s, np.full((N, G), 8, np.uint8))
    sd = np.repeat(s.view(np.float16).astype(np.float64), GROUP, axis=1)
    assert np.array_equal(w, t * sd)
    pow2 = _f16_bits(2.0 ** (np.arange(G) - 3))[None, :].repeat(N, 0)
    w = o.dequant(np.full((N, K), 9, np.uint8), pow2, np.full((N, G), 8, np.uint8))
    assert np.array_equal(w, np.repeat(2.0 ** (np.arange(G) - 3), GROUP)[None, :].repeat(N, 0))


def _case_inputs(c):
    M, N, K = c["M"], c["N"], c["K"]
    G = K // GROUP
    q = np.full((N, K), c["q"], np.uint8)
    for n, k, v in c.get("q_at", []):
        q[n, k] = v
    z = np.full((N, G), c["z"], np.uint8)
    if "s_groups" in c:
        s = _f16_bits(np.array(c["s_groups"]))[None, :].repeat(N, 0)
    else:
        s = np.full((N, G), _f16_bits(c["s"]), np.uint16)
    if "x_rows" in c:
        x = _f16_bits(np.array(c["x_rows"])[:, None].repeat(K, 1))
    else:
        x = np.full((M, K), _f16_bits(c["x"]), np.uint16)
    for m, k, v in c.get("x_at", []):
        x[m, k] = _f16_bits(v)
    return q, s, z, x


def pin_gemv_tiny_cases(o):
    """Hand-derived closed forms (tests/golden/tiny_gemv_cases.json)."""
    for c in _load("tiny_gemv_cases.json")["cases"]:
        q, s, z, x = _case_inputs(c)
        ref, absref = o.gemv(q, s, z, x)
        assert np.array_equal(ref, np.array(c["y"])), (c["name"], ref)
        assert np.array_equal(absref, np.array(c["absref"])), (c["name"], absref)
        assert np.array_equal(o.f64_to_f16(ref), _f16_bits(np.array(c["y"]))), c["name"]


def _fp16_table():
    bits, vals = _f16_finite_positive()
    return bits, [Fraction(float(v)) for v in vals]


def _rne16_exact(value, table):
    """Nearest binary16 to an exact rational, ties to even mantissa, by search."""
    bits, fr = table
    a = abs(value)
    if a >= Fraction(65520):
        b = 0x7C00
    else:
        i = bisect.bisect_left(fr, a)
        if i < len(fr) and fr[i] == a:
            b = int(bits[i])
        else:
            lo, hi = i - 1, i
            dl, dh = a - fr[lo], fr[hi] - a
            if dl < dh or (dl == dh and int(bits[lo]) % 2 == 0):
                b = int(bits[lo])
            else:
                b = int(bits[hi])
    return b | (0x8000 if value < 0 else 0)


def pin_gemv_exact_rational(o):
    """On small random inputs, the oracle's fp64 sum lies within its
    accumulation bound of the exact rational sum, and its rounding of the
    fp64 sum to fp16 equals exact rounding of the exact sum (away from ties
    that the fp64 sum cannot resolve)."""
    rng = np.random.default_rng(19)
    table = _fp16_table()
    for M, N, K in [(2, 3, 256), (1, 4, 384), (3, 2, 128)]:
        q, s, z = synthetic.weights(N, K, seed=int(rng.integers(1 << 30)))
        x = synthetic.activations(M, K, seed=int(rng.integers(1 << 30)))
        ref, absref = o.gemv(q, s, z, x)
        sf = s.view(np.float16).astype(np.float64)
        xf = x.view(np.float16).astype(np.float64)
        for m in range(M):
            for n in range(N):
                exact = Fraction(0)
                for k in range(K):
                    g = k // GROUP
                    exact += (int(q[n, k]) - int(z[n, g])) * Fraction(float(sf[n, g])) * Fraction(float(xf[m, k]))
                err = abs(Fraction(float(ref[m, n])) - exact)
                assert err <= Fraction(K * 2.0 ** -52) * Fraction(float(absref[m, n])), (m, n)
                want16 = _rne16_exact(exact, table)
                got16 = int(o.f64_to_f16(np.array([ref[m, n]]))[0])
                assert got16 == want16, (m, n, hex(got16), hex(want16))


def pin_gemv_vs_numpy(o):
    """The oracle's matvec equals numpy's float64 matmul of its own dequantized
    W (a library routine) to within fp64 accumulation error; this fixes the
    row/column roles for non-square shapes and M > 1."""
    rng = np.random.default_rng(23)
    for M, N, K in [(1, 48, 896), (3, 17, 1280), (8, 5, 256)]:
        q, s, z = synthetic.weights(N, K, seed=int(rng.integers(1 << 30)))
        x = synthetic.activations(M, K, seed=int(rng.integers(1 << 30)))
        ref, absref = o.gemv(q, s, z, x)
        w = o.dequant(q, s, z)
        want = x.view(np.float16).astype(np.float64) @ w.T
        assert np.all(np.abs(ref - want) <= 4 * K * 2.0 ** -53 * absref + 1e-300)
        assert np.allclose(absref, np.abs(x.view(np.float16).astype(np.float64)) @ np.abs(w.T), rtol=1e-12, atol=0)


def pin_gemv_one_hot(o):
    """x = e_k picks column k: y[n] = w[n][k] exactly."""
    rng = np.random.default_rng(29)
    N, K = 21, 512
    q, s, z = synthetic.weights(N, K, seed=4)
    w = o.dequant(q, s, z)
    for k in rng.integers(0, K, 12):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3C00
        ref, _ = o.gemv(q, s, z, x)
        assert np.array_equal(ref[0], w[:, k])
        sk = s[:, k // GROUP].view(np.float16).astype(np.float64)
        assert np.array_equal(ref[0], (q[:, k].astype(np.float64) - z[:, k // GROUP]) * sk)


def pin_gemv_invariants(o):
    """Scaling x by 2 scales y by 2 exactly; permuting rows of W permutes y;
    swapping activation rows swaps output rows."""
    rng = np.random.default_rng(31)
    M, N, K = 3, 33, 640
    q, s, z = synthetic.weights(N, K, seed=8)
    x = synthetic.activations(M, K, seed=9)
    ref, absref = o.gemv(q, s, z, x)
    x2 = _f16_bits(x.view(np.float16).astype(np.float64) * 2.0)
    ref2, _ = o.gemv(q, s, z, x2)
    assert np.array_equal(ref2, 2.0 * ref)
    p = rng.permutation(N)
    refp, _ = o.gemv(q[p], s[p], z[p], x)
    assert np.array_equal(refp, ref[:, p])
    refm, _ = o.gemv(q, s, z, x[::-1].copy())
    assert np.array_equal(refm, ref[::-1])


def pin_gemv_packed_matches_logical(o):
    """The product computed from packed buffers equals the product from the
    logical tensors bit for bit (full and sampled rows)."""
    for M, N, K in [(1, 40, 896), (5, 19, 1152)]:
        q, s, z = synthetic.weights(N, K, seed=N)
        x = synthetic.activations(M, K, seed=K)
        ref, absref = o.gemv(q, s, z, x)
        wq, sp, zp = o.pack(q, s, z)
        ref2, absref2 = o.gemv_packed(M, N, K, wq, sp, zp, x)
        assert np.array_equal(ref, ref2) and np.array_equal(absref, absref2)
        rows = np.array([0, N - 1, N // 2, 7])
        ref3, _ = o.gemv_packed(M, N, K, wq, sp, zp, x, rows=rows)
        assert np.array_equal(ref3, ref[:, rows])


# ---------------------------------------------------------------- quantizer

def _quant_groups(seed, N=6, K=512):
    """fp16 weights with the workload's spread plus awkward groups: all zero,
    constant positive, constant negative, all positive, one huge outlier."""
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, 0.02, (N, K))
    w[0, 0:128] = 0.0
    w[1, 128:256] = 0.37
    w[2, 256:384] = -1.5
    w[3, 384:512] = np.abs(w[3, 384:512]) + 0.1
    w[4, 5] = 300.0
    return w.astype(np.float16).view(np.uint16)


def pin_quantize_scale_definition(o):
    """s is the fp16 rounding (numpy's own RNE conversion) of absmax / 7
    (symmetric) or of (max(w, 0) - min(w, 0)) / 15 (asymmetric), per row and
    group; symmetric z is 8 everywhere and q - 8 stays in [-8, 7]."""
    w16 = _quant_groups(51)
    wd = w16.view(np.float16).astype(np.float64)
    N, K = wd.shape
    g = wd.reshape(N, K // GROUP, GROUP)
    q, s, z = o.quantize(w16, 0)
    assert np.array_equal(s, (np.abs(g).max(axis=2) / 7.0).astype(np.float16).view(np.uint16))
    assert (z == 8).all() and q.max() <= 15
    q, s, z = o.quantize(w16, 1)
    lo, hi = np.minimum(g.min(axis=2), 0.0), np.maximum(g.max(axis=2), 0.0)
    assert np.array_equal(s, ((hi - lo) / 15.0).astype(np.float16).view(np.uint16))
    assert q.max() <= 15 and z.max() <= 15


def pin_quantize_nearest_code(o):
    """Brute force: given the stored s and z, every weight's code is one of
    the nearest of all 16 codes (round to nearest, then clamp to the code
    range, can do no better); 0 is represented exactly in both modes."""
    w16 = _quant_groups(53)
    wd = w16.view(np.float16).astype(np.float64)
    codes = np.arange(16, dtype=np.float64)
    for mode in (0, 1):
        q, s, z = o.quantize(w16, mode)
        sd = np.repeat(s.view(np.float16).astype(np.float64), GROUP, axis=1)
        zd = np.repeat(z.astype(np.float64), GROUP, axis=1)
        err = np.abs(wd - (q - zd) * sd)
        best = np.abs(wd[..., None] - (codes - zd[..., None]) * sd[..., None]).min(axis=2)
        assert (err <= best * (1 + 1e-12) + 1e-300).all(), mode
        assert not (((q - zd) * sd)[wd == 0.0]).any()  # zero weights dequantize to exactly 0
        inside = (sd > 0)
        assert (err[inside] <= sd[inside] / 2 * (1 + 1e-12) + 1e-300).all() or mode == 1


def pin_quantize_degenerate_groups(o):
    """An all-zero group gets scale 0 and q = z (dequantizes to 0); the
    symmetric grid holds +-absmax at +-7; a group of multiples of a power of
    two up to 7 times it quantizes exactly."""
    w16 = _quant_groups(57)
    for mode in (0, 1):
        q, s, z = o.quantize(w16, mode)
        assert s[0, 0] == 0 and (q[0, :128] == z[0, 0]).all()
    c = 2.0 ** -6
    t = np.tile(np.arange(-7, 8), 9)[:128].astype(np.float64)
    w = np.zeros((1, 128))
    w[0] = t * c
    q, s, z = o.quantize(w.astype(np.float16).view(np.uint16), 0)
    assert s[0, 0] == np.float16(c).view(np.uint16) and np.array_equal(q[0].astype(int) - 8, t.astype(int))
    q, s, z = o.quantize(_quant_groups(57), 0)
    row2 = q[2, 256:384].astype(int) - 8  # constant -1.5: absmax / 7 scale, every code -7
    assert (row2 == -7).all()


# ------------------------------------------------------------------ SwiGLU

def pin_silu_definition(o):
    """silu(v) = v * logistic(v), against scipy's logistic function (an
    independent library routine); silu(0) = 0; the reflection identity
    silu(-v) = silu(v) - v; saturation to v and to 0."""
    from scipy.special import expit
    import oracle
    v = np.concatenate([np.linspace(-30, 30, 6001), [0.0, 1e-300, -1e-300, 1e-8, 700.0, -700.0]])
    got = oracle.silu(v)
    assert np.allclose(got, v * expit(v), rtol=4e-16, atol=0)
    assert oracle.silu(0.0) == 0.0
    assert np.allclose(oracle.silu(-v[:6001]), got[:6001] - v[:6001], rtol=1e-12, atol=1e-12)
    assert oracle.silu(80.0) == 80.0 and abs(oracle.silu(-80.0)) < 1e-30
    assert oracle.silu(-1000.0) == 0.0  # exp overflow handled, no NaN


def pin_silu_lipschitz_constant(o):
    """SILU_LIPSCHITZ bounds |silu'| and is tight: central differences of
    scipy's v * logistic(v) peak at 1.0998 near v = 2.4."""
    from scipy.special import expit
    import oracle
    v = np.linspace(-40, 40, 400001)
    h = 1e-5
    d = ((v + h) * expit(v + h) - (v - h) * expit(v - h)) / (2 * h)
    assert np.abs(d).max() <= oracle.SILU_LIPSCHITZ
    assert np.abs(d).max() > oracle.SILU_LIPSCHITZ - 2e-4
    assert 2.3 < v[np.argmax(d)] < 2.5


def pin_swiglu_composition(o):
    """x = e_k makes g and u single dequantized weights, so the fused
    reference must be silu(w_gate[n][k]) * w_up[n][k] exactly; with an up
    matrix whose column k dequantizes to 1 it must be silu(g) alone (which
    fixes the gate/up roles); rows of gate and up stay paired."""
    from scipy.special import expit
    import oracle
    F, K = 24, 384
    qg, sg, zg = synthetic.weights(F, K, seed=41, tensor_id=1)
    qu, su, zu = synthetic.weights(F, K, seed=41, tensor_id=2)
    wg, wu = o.dequant(qg, sg, zg), o.dequant(qu, su, zu)
    for k in (0, 129, 383):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3C00
        ref, bound = oracle.gemv_swiglu(o, qg, sg, zg, qu, su, zu, x)
        want = wg[:, k] * expit(wg[:, k]) * wu[:, k]
        assert np.allclose(ref[0], want, rtol=1e-15, atol=0) and (bound > 0).all()
    ones_q = np.full((F, K), 1, np.uint8)
    ones_s = np.full((F, K // GROUP), 0x3C00, np.uint16)
    ones_z = np.zeros((F, K // GROUP), np.uint8)
    x = synthetic.activations(2, K, seed=43)
    x[:, :] = 0
    x[:, 7] = 0x3C00  # one-hot: u = 1 for every row, g = w_gate[:, 7]
    ref, _ = oracle.gemv_swiglu(o, qg, sg, zg, ones_q, ones_s, ones_z, x)
    assert np.allclose(ref, wg[:, 7] * expit(wg[:, 7]), rtol=1e-15, atol=0)
    p = np.random.default_rng(44).permutation(F)
    x = synthetic.activations(1, K, seed=45)
    ref, _ = oracle.gemv_swiglu(o, qg, sg, zg, qu, su, zu, x)
    refp, _ = oracle.gemv_swiglu(o, qg[p], sg[p], zg[p], qu[p], su[p], zu[p], x)
    assert np.array_equal(refp, ref[:, p])


def pin_swiglu_bound_admits_rounded_reference(o):
    """The acceptance bound is at least the fp16 rounding of the exact value
    (a correct fp16 answer can always pass) and well below the output scale,
    so an O(1) mistake cannot hide in it. (It inherits the GEMV bound's
    2e-3 * sum|w x|, about 25 x |y| at K = 1024, once from g and once from
    u: about 11% of the mean |y| here.)"""
    import oracle
    F, K = 64, 1024
    qg, sg, zg = synthetic.weights(F, K, seed=47, tensor_id=1)
    qu, su, zu = synthetic.weights(F, K, seed=47, tensor_id=2)
    x = synthetic.activations(3, K, seed=48)
    ref, bound = oracle.gemv_swiglu(o, qg, sg, zg, qu, su, zu, x)
    r16 = o.f16_to_f64(o.f64_to_f16(ref))
    assert (np.abs(r16 - ref) <= bound).all()
    assert np.median(bound / np.abs(ref).mean()) < 0.2



# ------------------------------------------------------- INT8 activations

def _grid_activations(seed, M=3, K=512, exps=(0, -3, 2, -7)):
    """Activations already on an int8 grid: each group holds integers in
    [-127, 127] including one +-127, times a power of two that varies by row
    and group, so that the group's code scale is exactly that power."""
    rng = np.random.default_rng(seed)
    G = K // GROUP
    c = rng.integers(-127, 128, size=(M, G, GROUP))
    where = rng.integers(0, GROUP, size=(M, G))
    sign = rng.choice([-1, 1], size=(M, G))
    for m in range(M):
        for g in range(G):
            c[m, g, where[m, g]] = 127 * sign[m, g]
    e = np.array([[exps[(m + 2 * g) % len(exps)] for g in range(G)] for m in range(M)], dtype=np.float64)
    x = c * np.exp2(e)[..., None]
    return c.reshape(M, K), np.exp2(e), x.reshape(M, K).astype(np.float16).view(np.uint16)


def pin_act_quant_on_grid(o):
    """A group of integers in [-127, 127] holding +-127, times 2^e, has code
    scale exactly 2^e, codes equal to the integers and a code sum equal to
    theirs (every step is exact there)."""
    c, scale, x = _grid_activations(61)
    xq, sx, xsum = o.act_quant_i8(x)
    assert np.array_equal(sx.astype(np.float64), scale)
    assert np.array_equal(xq.astype(np.int64), c)
    M, K = c.shape
    assert np.array_equal(xsum.astype(np.int64), c.reshape(M, K // GROUP, GROUP).sum(axis=2))


def pin_act_quant_ties_to_even(o):
    """With code scale 1, halves round to the even neighbour."""
    x = np.zeros((1, GROUP))
    x[0, 0] = 127.0
    vals = [0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 3.5, -3.5, 126.5, -126.5, 0.25, 0.75]
    want = [0, 0, 2, -2, 2, -2, 4, -4, 126, -126, 0, 1]
    x[0, 1:1 + len(vals)] = vals
    xq, sx, xsum = o.act_quant_i8(x.astype(np.float16).view(np.uint16))
    assert sx[0, 0] == 1.0
    assert xq[0, 1:1 + len(vals)].tolist() == want
    assert xsum[0, 0] == 127 + sum(want)


def pin_act_quant_nearest_code(o):
    """Brute force over all 255 codes: every code is a nearest one for the
    stored scale (to within the fp32 rounding of the decision); the absmax
    element takes code +-127; the scale is absmax / 127 to within one fp32
    rounding; an all-zero group has scale 0, codes 0 and sum 0."""
    x = synthetic.activations(4, 1024, seed=63).view(np.float16).astype(np.float64)
    x[1, 128:256] = 0.0
    x[2, 256:384] = -np.abs(x[2, 256:384])
    x[3, 0:128] *= 2.0 ** -12  # small groups, subnormal fp16 among them
    x16 = x.astype(np.float16).view(np.uint16)
    xd = x16.view(np.float16).astype(np.float64)
    xq, sx, xsum = o.act_quant_i8(x16)
    M, K = xd.shape
    sd = np.repeat(sx.astype(np.float64), GROUP, axis=1)
    codes = np.arange(-127, 128, dtype=np.float64)
    err = np.abs(xd - xq * sd)
    best = np.abs(xd[..., None] - codes * sd[..., None]).min(axis=2)
    assert (err <= best + sd * 2.0 ** -20).all()
    g = xd.reshape(M, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    assert (np.abs(sx.astype(np.float64) * 127.0 - amax) <= amax * 2.0 ** -23).all()
    arg = np.abs(g).argmax(axis=2)
    top = np.take_along_axis(xq.reshape(M, K // GROUP, GROUP).astype(np.int64), arg[..., None], 2)[..., 0]
    nz = amax > 0
    assert (np.abs(top[nz]) == 127).all()
    assert sx[1, 1] == 0 and not xq[1, 128:256].any() and xsum[1, 1] == 0
    assert np.array_equal(xsum.astype(np.int64), xq.reshape(M, K // GROUP, GROUP).astype(np.int64).sum(axis=2))


def pin_act_quant_power_of_two_scaling(o):
    """Doubling the activations doubles every scale bit-exactly and leaves
    the codes unchanged (fp32 scaling by 2 is exact, away from overflow)."""
    x = synthetic.activations(3, 512, seed=65)
    x2 = (x.view(np.float16).astype(np.float64) * 2.0).astype(np.float16).view(np.uint16)
    a = o.act_quant_i8(x)
    b = o.act_quant_i8(x2)
    assert np.array_equal(b[0], a[0]) and np.array_equal(b[2], a[2])
    assert np.array_equal(b[1], a[1] * np.float32(2.0))


def pin_gemv_a8_tiny_case(o):
    """Worked by hand: K = 128, q - z = 3 on k = 0..3, s = 0.5, activations
    (127, -4.4, 2.6, 0.5) with scale 1 give codes (127, -4, 3, 0), so
    y = 0.5 * 1 * 3 * (127 - 4 + 3 + 0) = 189; a second row with every
    activation negated gives -189."""
    q = np.full((1, GROUP), 5, np.uint8)
    q[0, :4] = 8
    z = np.full((1, 1), 5, np.uint8)
    s = np.array([[np.float16(0.5).view(np.uint16)]], np.uint16)
    x = np.zeros((2, GROUP))
    x[0, :4] = [127.0, -4.4, 2.6, 0.5]
    x[1] = -x[0]
    xq, sx, _ = o.act_quant_i8(x.astype(np.float16).view(np.uint16))
    ref, absref = o.gemv_a8(q, s, z, xq, sx)
    assert ref[0, 0] == 189.0 and ref[1, 0] == -189.0 and absref[0, 0] == 189.0


def pin_gemv_a8_matches_fp_path_on_grid(o):
    """When the activations are already on the int8 grid their codes are
    exact, so the integer-sum product equals the fp16-activation product of
    the (separately pinned) main oracle, row by row and group scale by group
    scale."""
    _, _, x = _grid_activations(67, M=3, K=768)
    q, s, z = synthetic.weights(40, 768, seed=68)
    xq, sx, _ = o.act_quant_i8(x)
    ref8, abs8 = o.gemv_a8(q, s, z, xq, sx)
    ref, absref = o.gemv(q, s, z, x)
    assert (abs8 <= absref * (1 + 1e-12)).all()  # |group sums| summed, against |w x| summed
    assert (np.abs(ref8 - ref) <= 1e-12 * absref).all()
    rows = np.array([39, 0, 17])
    r8, _ = o.gemv_a8(q, s, z, xq, sx, rows=rows)
    assert np.array_equal(r8, ref8[:, rows])


def pin_gemv_a8_quantization_error_bound(o):
    """On the workload's activations the integer-sum product differs from the
    exact fp16-activation product by no more than the codes' rounding allows,
    sum_g s * (sx / 2) * sum_k |q - z| (codes never clamp: |x| <= absmax);
    and, the rounding errors being independent, the root-mean-square
    difference is a small fraction of the outputs' (about 0.7% here)."""
    K = 1024
    q, s, z = synthetic.weights(48, K, seed=69)
    x = synthetic.activations(5, K, seed=70)
    xq, sx, _ = o.act_quant_i8(x)
    ref8, _ = o.gemv_a8(q, s, z, xq, sx)
    ref, _ = o.gemv(q, s, z, x)
    G = K // GROUP
    sd = o.f16_to_f64(s)                                                   # [N][G]
    wabs = np.abs(q.astype(np.int64) - np.repeat(z, GROUP, axis=1)).reshape(48, G, GROUP).sum(axis=2)
    allow = (sd * wabs) @ (sx.astype(np.float64).T / 2.0)                  # [N][M]
    assert (np.abs(ref8 - ref) <= allow.T * (1 + 1e-9) + 1e-12).all()
    assert np.sqrt(((ref8 - ref) ** 2).mean()) < 0.02 * np.sqrt((ref ** 2).mean())


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
