"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test names what it pins: a closed form, an exhaustive enumeration, a
library routine on a special case, a hand-derived example (tests/golden/)
or brute force on tiny inputs.  Sources are cited by page title and part:
  [LG] LiquidGEMM, Pith review of arXiv 2509.01229 ("What carries the
       argument"; referee summary; major comment 3 = paper Sec. 4 Eq. 7;
       minor comment 2 = Eq. 10; circularity audit = Eq. 11/12).
  [FQ] FireQ, arXiv 2505.20839, abstract.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as wl


# ----------------------------------------------------------------- P1 ------
def _all_valid_triples():
    m = np.arange(-128, 128).reshape(-1, 1, 1)
    s = np.arange(0, 256).reshape(1, -1, 1)
    q = np.arange(0, 16).reshape(1, 1, -1)
    val = m + q * s
    ok = (val >= -128) & (val <= 127)
    mm, ss, qq = np.broadcast_arrays(m, s, q)
    return mm[ok], ss[ok], qq[ok]


def test_p1_identity_exhaustive():
    """[LG] Eq. 12: (q*s + a) XOR 0x80 with a = 128 + m equals the affine
    dequantisation m + q*s, with no carry out of the UINT8 byte, for every
    (m, s, q) whose value is an INT8."""
    m, s, q = _all_valid_triples()
    n = m.size
    assert n == 176198  # count of valid triples (independent enumeration)
    codes = q.astype(np.uint8).reshape(n, 1)
    su8 = s.astype(np.uint8).reshape(n, 1)
    au8 = (128 + m).astype(np.uint8).reshape(n, 1)
    dec = oracle.lqq_decode(codes, su8, au8, 1, check_carry=True)
    np.testing.assert_array_equal(dec.reshape(-1).astype(np.int64), m + q * s)


def test_p1_carry_is_reported():
    """Outside the INT8 range the byte would carry; the oracle must say so."""
    codes = np.array([[15]], np.uint8)
    with pytest.raises(AssertionError):
        oracle.lqq_decode(codes, np.array([[17]], np.uint8),
                          np.array([[1]], np.uint8), 1, check_carry=True)


def test_p1_swar_lanes_carry_free():
    """Four codes per 32-bit word, multiplied and offset as two 16-bit lanes
    (each holding two code bytes), give the four scalar decodes: the byte
    lanes never carry into each other when every q*s + a <= 255."""
    rng = np.random.default_rng(5)
    m, s, q = _all_valid_triples()
    idx = rng.integers(0, m.size, size=(20000,))
    for i0 in range(0, 20000, 4000):
        sel = idx[i0:i0 + 4000]
        # one (m, s) per word, four codes whose values stay in range
        mm, ss = m[sel], s[sel]
        qmax = np.where(ss > 0, (127 - mm) // np.maximum(ss, 1), 15)
        qmax = np.minimum(qmax, 15)
        qs = rng.integers(0, qmax[:, None] + 1, size=(sel.size, 4))
        word = (qs[:, 0] | (qs[:, 1] << 8) | (qs[:, 2] << 16) | (qs[:, 3] << 24))
        a = 128 + mm
        lo = (word & 0xFFFF) * ss + (a | (a << 8))
        hi = ((word >> 16) & 0xFFFF) * ss + (a | (a << 8))
        res = ((lo & 0xFFFF) | ((hi & 0xFFFF) << 16)) ^ 0x80808080
        got = np.stack([((res >> (8 * j)) & 0xFF) for j in range(4)], 1)
        got = np.where(got > 127, got - 256, got)
        np.testing.assert_array_equal(got, mm[:, None] + qs * ss[:, None])


# ----------------------------------------------------------------- P2 ------
def _exhaustive_groups(lo, hi, g=64):
    """Groups covering every (m, M, Q) with lo <= m <= Q <= M <= hi."""
    rows = []
    per = g - 2
    for m in range(lo, hi + 1):
        for M in range(m, hi + 1):
            vals = np.arange(m, M + 1)
            for c0 in range(0, vals.size, per):
                chunk = vals[c0:c0 + per]
                row = np.full(g, m, np.int64)
                row[1] = M
                row[2:2 + chunk.size] = chunk
                rows.append(row)
    return np.asarray(rows, np.int8)


@pytest.fixture(scope="module")
def groups_127():
    return _exhaustive_groups(-127, 127)


def test_p2_quantizer_bounds_full_range(groups_127):
    """[LG] major comment 3 / minor comment 2: integer scale, nearest
    rounding.  Exhaustive over -127 <= m <= Q <= M <= 127:
      * s is the least integer >= 1 with R/s <= 15;
      * a = 128 + m;
      * every decoded value is an INT8 that never exceeds 127 (no wrap);
      * unsaturated codes are the nearest grid point (ties upward);
      * saturated codes sit below Q by less than one step."""
    Q = groups_127
    codes, s, a, nsat = oracle.lqq_encode(Q, 64)
    s = s[:, 0].astype(np.int64)
    a = a[:, 0].astype(np.int64)
    Qi = Q.astype(np.int64)
    m, M = Qi.min(1), Qi.max(1)
    R = M - m
    assert np.all(R <= 15 * s)
    assert np.all((s == 1) | (R > 15 * (s - 1)))
    np.testing.assert_array_equal(a, 128 + m)
    dec = oracle.lqq_decode(codes, s.astype(np.uint8)[:, None],
                            a.astype(np.uint8)[:, None], 64).astype(np.int64)
    q = codes.astype(np.int64)
    np.testing.assert_array_equal(dec, m[:, None] + q * s[:, None])
    assert dec.max() <= 127 and dec.min() >= -127
    # nearest grid point, ties upward, unless lowered by the saturation
    err = Qi - dec
    cap = (127 - m) // s
    sat = q == cap[:, None]
    near = (2 * np.abs(err) < s[:, None]) | (2 * err == -s[:, None])
    unsat_ok = near | sat
    assert np.all(unsat_ok)
    assert np.all(err[sat] < s[:, None].repeat(64, 1)[sat])
    assert np.all(err[~sat] <= s[:, None].repeat(64, 1)[~sat] // 2)
    assert nsat > 0  # the full +-127 range does need the saturation


def test_p2_protective_range_needs_no_saturation():
    """[LG] circularity audit / Eq. 11: on [-119, 119] the multiply-add stays
    in UINT8 by construction: scale <= 16 (the review's number) and the
    saturation never fires."""
    Q = _exhaustive_groups(-119, 119)
    codes, s, a, nsat = oracle.lqq_encode(Q, 64)
    assert int(s.max()) == 16
    assert nsat == 0
    dec = oracle.lqq_decode(codes, s, a, 64)
    assert np.abs(dec.astype(np.int64) - Q.astype(np.int64)).max() <= 8


def test_golden_lqq_examples(golden_dir):
    """Hand-derived groups from the page's definitions."""
    path = os.path.join(golden_dir, "lqq_examples.txt")
    n_cases = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        vals, s, a, codes, dec, nsat = [f.split() for f in line.split("|")]
        v = np.array([int(t) for t in vals], np.int64)
        # pad to a group of 64 by repeating the first value, which is the
        # group minimum in every example (code 0, never saturated)
        g = np.full(64, v[0], np.int64)
        g[:v.size] = v
        c, ss, aa, ns = oracle.lqq_encode(g.astype(np.int8).reshape(1, 64), 64)
        assert int(ss[0, 0]) == int(s[0]), line
        assert int(aa[0, 0]) == int(a[0]), line
        assert list(c[0, :v.size]) == [int(t) for t in codes], line
        d = oracle.lqq_decode(c, ss, aa, 64)
        assert list(d[0, :v.size]) == [int(t) for t in dec], line
        assert v[0] == v.min(), line
        assert ns == int(nsat[0]), line
        n_cases += 1
    assert n_cases == 7


# ----------------------------------------------------------------- P3 ------
def test_p3_lossless_when_range_fits_4_bits():
    """If every group spans at most 15, s = 1 and the decode returns Q
    exactly, so the W4A8 GEMM is the plain INT8 GEMM (numpy int64 matmul)."""
    rng = np.random.default_rng(11)
    N, K, M, g = 48, 384, 7, 64
    base = rng.integers(-127, 113, size=(N, K // g, 1))
    Q = (base + rng.integers(0, 16, size=(N, K // g, g))).reshape(N, K)
    Q = Q.astype(np.int8)
    codes, s, a, nsat = oracle.lqq_encode(Q, g)
    assert np.all(s == 1) and nsat == 0
    dec = oracle.lqq_decode(codes, s, a, g)
    np.testing.assert_array_equal(dec, Q)
    X = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = oracle.gemm_i32(X, dec)
    np.testing.assert_array_equal(acc, X.astype(np.int64) @ Q.astype(np.int64).T)


# ----------------------------------------------------------------- P4 ------
def test_p4_bruteforce_tiny_gemm_and_epilogue():
    """Tiny shapes: the int32 GEMM of the decoded weights equals an fp64
    matmul exactly (all values < 2^53) and a pure-Python triple loop; the
    fp16 epilogue equals numpy's float64 -> float16 rounding of the fp64
    product acc * sx * sw."""
    for (M, N, K, g, seed) in [(3, 16, 128, 64, 1), (8, 32, 256, 128, 2),
                               (5, 16, 256, 64, 3)]:
        W = wl.gen_weights(N, K, seed)
        X = wl.gen_activations(M, K, seed + 10, seed + 20)
        pk = oracle.w4a8_pack(W, g)
        X8, sx = oracle.quant_sym_rows(X, 127)
        acc, y, yd = oracle.w4a8_gemm(X8, sx, pk, g)
        dec = oracle.lqq_decode(pk["codes"], pk["s_u8"], pk["a_u8"], g)
        ref = X8.astype(np.float64) @ dec.astype(np.float64).T
        np.testing.assert_array_equal(acc.astype(np.float64), ref)
        for (mi, ni) in [(0, 0), (M - 1, N - 1), (M // 2, 3)]:
            s_ = sum(int(X8[mi, k]) * int(dec[ni, k]) for k in range(K))
            assert acc[mi, ni] == s_
        v = acc.astype(np.float64) * sx.astype(np.float64)[:, None] * \
            pk["sw"].astype(np.float64)[None, :]
        np.testing.assert_array_equal(yd, v)
        np.testing.assert_array_equal(y, v.astype(np.float16).view(np.uint16))


def test_gemm_i32_matches_numpy_random():
    """Library routine on random operands (integer matmul, exact)."""
    rng = np.random.default_rng(3)
    X = rng.integers(-127, 128, size=(9, 640)).astype(np.int8)
    W = rng.integers(-128, 128, size=(33, 640)).astype(np.int8)
    np.testing.assert_array_equal(oracle.gemm_i32(X, W),
                                  X.astype(np.int64) @ W.astype(np.int64).T)


# ------------------------------------------------------- fp16 / bf16 -------
def test_round_f16_matches_numpy():
    """numpy converts float64 to float16 with one nearest-even rounding."""
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e6, 2.0 ** -24,
         2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25],
    ])
    # exact ties between neighbouring halves
    h = rng.integers(0, 0x7BFF, 5000).astype(np.uint16).view(np.float16)
    h2 = (h.view(np.uint16) + 1).view(np.float16)
    ties = (h.astype(np.float64) + h2.astype(np.float64)) / 2
    v = np.concatenate([v, ties, -ties])
    np.testing.assert_array_equal(oracle.round_f16(v),
                                  v.astype(np.float16).view(np.uint16))


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_round_bf16_nearest_even():
    """bfloat16 rounding: the result is a bfloat16 value, it is the nearer of
    the two bfloat16 neighbours of v (found by truncating the float32 bit
    pattern), and exact midpoints go to the even pattern."""
    rng = np.random.default_rng(8)
    v = rng.standard_normal(50000) * 10.0 ** rng.integers(-6, 6, 50000)
    out = oracle.round_bf16(v)
    r = _bf16_value(out)
    # neighbours: truncate toward zero at float32 then at bfloat16
    f = np.abs(v).astype(np.float32)
    # float32 rounding may cross a bfloat16 boundary, so take a +-1 window
    t = (f.view(np.uint32) >> 16).astype(np.int64)
    cands = np.stack([t - 1, t, t + 1, t + 2], 1)
    cv = _bf16_value(cands.astype(np.uint16)) * np.sign(v)[:, None]
    dist = np.abs(cv - v[:, None])
    best = dist.min(1)
    assert np.all(np.abs(r - v) == best)
    # midpoints
    b = rng.integers(0x3800, 0x4700, 5000).astype(np.uint16)
    lo, hi = _bf16_value(b), _bf16_value(b + 1)
    mid = (lo + hi) / 2
    got = oracle.round_bf16(mid)
    want = np.where(b % 2 == 0, b, b + 1).astype(np.uint16)
    np.testing.assert_array_equal(got, want)


# ------------------------------------------------------------ e4m3 ---------
def test_e4m3_decode_table():
    """OCP 8-bit float E4M3 ("fn": no infinities) definition points."""
    b = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_decode(b)
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6
    assert v[0x30] == 0.5 and v[0x38] == 1.0 and v[0x40] == 2.0
    assert v[0x44] == 3.0 and v[0x4E] == 7.0 and v[0x77] == 240.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    np.testing.assert_array_equal(v[0x80:0xFF], -pos)


def test_e4m3_encode_nearest_even_saturating():
    b = np.arange(0x7F, dtype=np.uint8)
    vals = oracle.e4m3_decode(b)
    # every finite value round-trips, with sign
    np.testing.assert_array_equal(oracle.e4m3_encode(vals.astype(np.float32)), b)
    np.testing.assert_array_equal(oracle.e4m3_encode(-vals.astype(np.float32)),
                                  b | 0x80)
    # midpoints go to the even code
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2)
    got = oracle.e4m3_encode(mids)
    want = np.where(b[:-1] % 2 == 0, b[:-1], b[:-1] + 1)
    np.testing.assert_array_equal(got, want)
    # brute force nearest on random values, saturation above 448
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-4, 3, 20000))
    x = x.astype(np.float32)
    got = oracle.e4m3_decode(oracle.e4m3_encode(x))
    d = np.abs(np.abs(x.astype(np.float64))[:, None] - vals[None, :])
    assert np.all(np.abs(np.abs(got) - np.abs(x)) == d.min(1))
    big = np.array([448.0, 460.0, 1e4, -1e30], np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(big), [0x7E, 0x7E, 0x7E, 0xFE])
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_quant_rows_e4m3_scale():
    """[FQ] abstract (FP8 activations): the largest magnitude maps to 448."""
    x = wl.gen_activations(6, 512, 1, 2)
    q, s = oracle.quant_rows_e4m3(x)
    np.testing.assert_array_equal(s, (np.abs(x).max(1) / np.float32(448)).astype(np.float32))
    dec = oracle.e4m3_decode(q)
    assert np.all(np.abs(dec).max(1) == 448.0)
    rel = np.abs(dec * s[:, None] - x) / np.maximum(np.abs(x), 1e-3)
    assert np.median(rel) < 0.04


def _e4m3_magnitudes():
    """The 127 finite non-negative OCP e4m3 values, code 0x00 .. 0x7E, from
    the format definition (bias 7; exponent field 0 is subnormal, m/8 *
    2^-6), written here independently of the oracle's decoder."""
    vals = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, np.float64)


def _e4m3_codes_brute(quot):
    """Nearest finite e4m3 code of each float32 quotient by exhaustive search
    over all 127 magnitudes; ties go to the even code; magnitudes above 448
    saturate to 448 (0x7E); the sign bit is copied (zeros keep it)."""
    vals = _e4m3_magnitudes()
    a = np.abs(quot.astype(np.float64)).ravel()
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes (at most two, adjacent), take the even one
    even = cand & (np.arange(0x7F)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    code = code.astype(np.uint8) | np.where(np.signbit(quot.ravel()), 0x80, 0).astype(np.uint8)
    return code.reshape(quot.shape)


def test_quant_rows_e4m3_every_code():
    """Per-token e4m3 codes element by element ([FQ] abstract: FP8
    activations; the reading: scale = max|x| / 448 in float32, codes =
    e4m3 of the float32 quotient x / scale, nearest with ties to even,
    saturating).  The expected codes come from numpy's float32 quotient
    and an exhaustive nearest search over the format's values, on rows
    whose scales are not powers of two.  Each row also holds quotients
    placed exactly on midpoints between neighbouring e4m3 values, where a
    quotient formed another way (in double precision, or as x times the
    reciprocal 448 / max) would round to the other neighbour."""
    rng = np.random.default_rng(31)
    vals = _e4m3_magnitudes()
    mids = (vals[:-1] + vals[1:]) / 2
    rows, cols = 12, 1024
    x = (rng.standard_normal((rows, cols)) * 3.0).astype(np.float32)
    x[:, rng.choice(cols, 10, replace=False)] *= np.float32(20.0)
    x[:, 5] = 0.0
    x[:, 6] = -0.0
    n_ties = 0
    for r in range(rows):
        amax = np.float32(rng.uniform(3.0, 90.0))  # never a power of two
        while float(amax) == 2.0 ** np.round(np.log2(float(amax))):
            amax = np.float32(rng.uniform(3.0, 90.0))
        row = np.clip(x[r], -amax, amax)
        row[0] = amax
        s = np.float32(amax) / np.float32(448.0)
        # midpoint quotients: x = the float32 nearest s * mid, nudged one ulp
        # either way until the float32 quotient x / s is the midpoint itself
        placed = 0
        for i, mdp in enumerate(mids[::3]):
            xv = np.float32(mdp * float(s))
            for cand in (xv, np.nextafter(xv, np.float32(np.inf)),
                         np.nextafter(xv, np.float32(-np.inf))):
                if float(np.float32(cand) / s) == mdp and abs(cand) <= amax:
                    sign = np.float32(-1.0) if i % 2 else np.float32(1.0)
                    row[16 + placed] = sign * cand
                    placed += 1
                    break
        n_ties += placed
        x[r] = row
    q, s = oracle.quant_rows_e4m3(x)
    want_s = (np.abs(x).max(axis=1) / np.float32(448.0)).astype(np.float32)
    np.testing.assert_array_equal(s, want_s)
    quot = (x / want_s[:, None]).astype(np.float32)  # numpy: float32 IEEE division
    want = _e4m3_codes_brute(quot)
    np.testing.assert_array_equal(q, want)
    assert n_ties > 20 * rows  # the midpoint cases are really there
    # the reading's alternatives differ from it on those rows
    recip = (x * (np.float32(448.0) / np.abs(x).max(axis=1))[:, None]).astype(np.float32)
    assert not np.array_equal(_e4m3_codes_brute(recip), want)
    dq = x.astype(np.float64) / want_s[:, None].astype(np.float64)
    dcode = _e4m3_codes_brute(dq)
    assert not np.array_equal(dcode, want)


# ------------------------------------------------------ per-row quant ------
def test_quant_sym_rows_properties():
    rng = np.random.default_rng(12)
    # exact integers times a power of two come back exactly
    k = rng.integers(-127, 128, size=(5, 300)).astype(np.float32)
    k[:, 0] = 127
    q, s = oracle.quant_sym_rows(k * np.float32(2.0 ** -5), 127)
    np.testing.assert_array_equal(s, np.float32(2.0 ** -5))
    np.testing.assert_array_equal(q, k.astype(np.int8))
    # ties round to even: values at (j + 1/2) * scale with scale = 1
    t = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, 126.5, -126.5]], np.float32)
    q, s = oracle.quant_sym_rows(t, 127)
    assert s[0] == 1.0
    assert list(q[0]) == [127, 0, 2, 2, 0, -2, 126, -126]
    # all-zero row -> scale 1 and zero codes; sign symmetry; the max hits qmax
    x = wl.gen_weights(4, 256, 3)
    x[2] = 0
    q, s = oracle.quant_sym_rows(x, 119)
    assert s[2] == 1.0 and np.all(q[2] == 0)
    qn, sn = oracle.quant_sym_rows(-x, 119)
    np.testing.assert_array_equal(qn, -q)
    for r in (0, 1, 3):
        assert np.abs(q[r]).max() == 119
        err = np.abs(x[r].astype(np.float64) - q[r] * np.float64(s[r]))
        assert err.max() <= 0.5 * s[r] * (1 + 1e-6)


def test_int4_sign_magnitude():
    """INT4 per-channel weights of the FP8 variant ([FQ] abstract)."""
    v = np.arange(-7, 8, dtype=np.int8)
    c = oracle.int4_sm_codes(v)
    assert list(c) == [15, 14, 13, 12, 11, 10, 9, 0, 1, 2, 3, 4, 5, 6, 7]
    np.testing.assert_array_equal(oracle.int4_sm_values(c), v)
    pk = oracle.w4fp8_pack(wl.gen_weights(32, 256, 4))
    assert np.abs(pk["q"]).max() == 7


# ------------------------------------------------------------ layout -------
def test_pack_layout_golden(golden_dir):
    path = os.path.join(golden_dir, "pack_layout.txt")
    n = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        N, K, r, k, byte, hi = map(int, line.split())
        codes = np.zeros((N, K), np.uint8)
        codes[r, k] = 0xA
        wq = oracle.pack_nibbles(codes)
        nz = np.nonzero(wq)[0]
        assert list(nz) == [byte], line
        assert wq[byte] == (0xA << (4 * hi)), line
        n += 1
    assert n == 11


def test_param_panels_golden(golden_dir):
    path = os.path.join(golden_dir, "param_panels.txt")
    n_ok = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        N, G, n, j, byte = map(int, line.split())
        p = np.zeros((N, G), np.uint8)
        p[n, j] = 0x5A
        out = oracle.params_to_panels(p)
        assert list(np.nonzero(out)[0]) == [byte], line
        n_ok += 1
    assert n_ok == 9


def test_param_panels_bijective():
    rng = np.random.default_rng(21)
    p = rng.integers(0, 256, size=(192, 5)).astype(np.uint8)
    out = oracle.params_to_panels(p)
    assert sorted(out.tolist()) == sorted(p.reshape(-1).tolist())
    np.testing.assert_array_equal(oracle.params_from_panels(out, 192, 5), p)
    idx = np.arange(192 * 5, dtype=np.int64).reshape(192, 5)
    # positions are a permutation: tag every entry with a distinct id
    ids = oracle.params_to_panels((idx % 251).astype(np.uint8))
    assert ids.size == 960


def test_pack_layout_bijective():
    rng = np.random.default_rng(4)
    N, K = 48, 384
    codes = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    wq = oracle.pack_nibbles(codes)
    np.testing.assert_array_equal(oracle.unpack_nibbles(wq, N, K), codes)
    # every nibble of the output is written exactly once
    seen = []
    for idx in rng.choice(N * K, 300, replace=False):
        one = np.zeros(N * K, np.uint8)
        one[idx] = 1
        wq1 = oracle.pack_nibbles(one.reshape(N, K))
        pos = np.nonzero(wq1)[0]
        assert pos.size == 1 and wq1[pos[0]] in (0x01, 0x10)
        seen.append(2 * int(pos[0]) + (wq1[pos[0]] == 0x10))
    assert len(set(seen)) == 300


# ------------------------------------------------------- FP8 variant -------
def test_p6_fp8_reference_exact_special_case():
    """FP8 e4m3 holds small integers exactly; with unit scales the FP8
    reference equals the integer GEMM (numpy int64 matmul), and on random
    FP8 data the unscaled sum equals an fp64 matmul of the decoded values."""
    rng = np.random.default_rng(13)
    M, N, K = 6, 32, 256
    xi = rng.integers(-16, 17, size=(M, K)).astype(np.float32)
    X8 = oracle.e4m3_encode(xi)
    np.testing.assert_array_equal(oracle.e4m3_decode(X8), xi)
    qi = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    ref, pre = oracle.w4fp8_ref(X8, np.ones(M, np.float32), qi, np.ones(N, np.float32))
    want = xi.astype(np.int64) @ qi.astype(np.int64).T
    np.testing.assert_array_equal(ref, want.astype(np.float64))
    x = wl.gen_activations(M, K, 5, 6)
    X8, sx = oracle.quant_rows_e4m3(x)
    sw = rng.random(N).astype(np.float32)
    ref, pre = oracle.w4fp8_ref(X8, sx, qi, sw)
    np.testing.assert_array_equal(pre, oracle.e4m3_decode(X8) @ qi.astype(np.float64).T)
    np.testing.assert_allclose(ref, pre * sx[:, None].astype(np.float64) *
                               sw[None, :].astype(np.float64), rtol=1e-15)


def test_widening_definition_points():
    """Half and bfloat16 widening at points fixed by the formats'
    definitions: one, the largest finite values, the smallest subnormals,
    signed zero, and a mid-range value."""
    f16 = oracle.widen_f16(np.array([0x3C00, 0x7BFF, 0x0001, 0x0400, 0x8000, 0xC500, 0x3555],
                                    np.uint16))
    want16 = [1.0, 65504.0, 2.0 ** -24, 2.0 ** -14, -0.0, -5.0, 1.0 / 3.0]
    np.testing.assert_allclose(f16[:6], want16[:6], rtol=0, atol=0)
    assert np.signbit(f16[4])
    assert abs(float(f16[6]) - 1.0 / 3.0) < 2.0 ** -12     # 0x3555 = 0.333251953125
    assert float(f16[6]) == 0.333251953125
    bf = oracle.widen_bf16(np.array([0x3F80, 0x7F7F, 0x0001, 0x0080, 0x8000, 0xC0A0, 0x3EAB],
                                    np.uint16))
    wantb = [1.0, float(np.float32(3.3895313892515355e38)), 2.0 ** -133, 2.0 ** -126, -0.0, -5.0]
    np.testing.assert_array_equal(bf[:6], np.array(wantb, np.float32))
    assert np.signbit(bf[4])
    assert float(bf[6]) == 0.333984375                      # 0x3EAB
    # widening is exact: bfloat16 rounding of the widened value returns the bits
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    np.testing.assert_array_equal(oracle.round_bf16(oracle.widen_bf16(bits[finite])),
                                  bits[finite])
    h = bits[(bits & 0x7C00) != 0x7C00]
    np.testing.assert_array_equal(oracle.round_f16(oracle.widen_f16(h).astype(np.float64)), h)


def test_fp8_group_fold_golden(golden_dir):
    """Hand-worked folded per-group FP8 weights (tests/golden/fp8_group_fold.txt)."""
    N, K, g = 16, 128, 64
    W = np.zeros((N, K), np.float32)
    exp_t, exp_s, exp_q = None, [], []
    for line in open(os.path.join(golden_dir, "fp8_group_fold.txt")):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "W":
            W[int(f[1]), int(f[2])] = float(f[3])
        elif f[0] == "T":
            exp_t = float(f[1])
        elif f[0] == "S":
            exp_s.append((int(f[1]), int(f[2]), float(f[3]), float(f[4])))
        elif f[0] == "Q":
            exp_q.append((int(f[1]), int(f[2]), int(f[3]), int(f[4], 16)))
    pk = oracle.w4fp8g_pack(W, g)
    assert pk["t"] == exp_t
    for r, j, sg, fo in exp_s:
        assert pk["sg"][r, j] == np.float32(sg) and pk["f"][r, j] == np.float32(fo), (r, j)
    for r, k, q, w8 in exp_q:
        assert pk["q"][r, k] == q and pk["w8"][r, k] == w8, (r, k, pk["q"][r, k], hex(pk["w8"][r, k]))


def test_fp8_group_fold_exact_case():
    """Power-of-two group scales with small |q| * f: the folded FP8 weights
    are exactly q * s_g / t, so the reference equals an exact float64 matmul
    of the original weights (scaled by sx), independent of e4m3 rounding."""
    rng = np.random.default_rng(21)
    N, K, g = 32, 256, 128
    q = rng.integers(-7, 8, size=(N, K)).astype(np.float64)
    q[:, ::g] = 7                                           # every group reaches 7
    e = rng.integers(-9, -3, size=(N, K // g))
    e[0, 0] = -3                                            # the largest group: 7*2^-3
    W = (q * np.repeat(2.0 ** e, g, axis=1)).astype(np.float32)
    pk = oracle.w4fp8g_pack(W, g)
    np.testing.assert_array_equal(pk["q"], q.astype(np.int8))
    t = pk["t"]
    assert t == 7 * 2.0 ** -3 / 448                          # 2^-9, exact
    w8v = oracle.e4m3_decode(pk["w8"])
    np.testing.assert_array_equal(w8v * t, W.astype(np.float64))
    M = 5
    X8 = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    X8[(X8 & 0x7F) == 0x7F] = 0                              # no NaN codes
    sx = rng.random(M).astype(np.float32)
    ref, pre = oracle.w4fp8g_ref(X8, sx, pk["w8"], t)
    exact = oracle.e4m3_decode(X8) @ W.astype(np.float64).T
    np.testing.assert_array_equal(pre * t, exact)


def test_fp8_group_fold_error_bound():
    """At any size: |w8 t - W| <= s_g / 2 (INT4 rounding) + the e4m3 error of
    |q| f (relative 2^-4 for normals, absolute 2^-10 for subnormals) times t,
    and no folded value exceeds 448."""
    rng = np.random.default_rng(22)
    N, K, g = 64, 512, 64
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    W[3, 64:128] = 0.0
    pk = oracle.w4fp8g_pack(W, g)
    t = pk["t"]
    sg = np.repeat(pk["sg"].astype(np.float64), g, axis=1)
    f = np.repeat(pk["f"].astype(np.float64), g, axis=1)
    qf = np.abs(pk["q"].astype(np.float64)) * f
    assert qf.max() <= 448.0 * (1 + 2.0 ** -22)
    e4_err = np.maximum(qf * 2.0 ** -4, 2.0 ** -10)
    err = np.abs(oracle.e4m3_decode(pk["w8"]) * t - W.astype(np.float64))
    assert np.all(err <= sg / 2 * (1 + 2.0 ** -20) + e4_err * t)
    assert np.all(pk["w8"][3, 64:128] == 0)


def test_generator_deterministic():
    a = wl.gen_weights(64, 128, 7)
    b = wl.gen_weights(64, 128, 7)
    np.testing.assert_array_equal(a, b)
    x = wl.gen_activations(4, 1000, 1, 2)
    ch = wl.outlier_channels(1000, 2)
    assert ch.size == 10 and np.unique(ch).size == 10
    assert abs(float(a.std()) - 0.02) < 0.002


# ------------------------------------------------- W8A8 comparison path ----
def test_w8_layout_golden(golden_dir):
    n = 0
    for line in open(os.path.join(golden_dir, "w8_layout.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        N, K, r, k, byte = map(int, line.split())
        Q = np.zeros((N, K), np.int8)
        Q[r, k] = -77
        out = oracle.pack_w8(Q)
        assert list(np.nonzero(out)[0]) == [byte], line
        assert out[byte] == -77
        n += 1
    assert n == 13


def test_w8_layout_is_a_permutation():
    """Every code lands in exactly one byte and unpacking restores it."""
    rng = np.random.default_rng(12)
    N, K = 48, 384
    Q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    np.testing.assert_array_equal(oracle.unpack_w8(oracle.pack_w8(Q), N, K), Q)
    idx = np.arange(N * K, dtype=np.int64)
    # pack the index itself byte-wise: low byte and high bytes separately
    lo = oracle.pack_w8((idx & 0x7F).astype(np.int8).reshape(N, K)).astype(np.int64)
    mid = oracle.pack_w8(((idx >> 7) & 0x7F).astype(np.int8).reshape(N, K)).astype(np.int64)
    hi = oracle.pack_w8(((idx >> 14) & 0x7F).astype(np.int8).reshape(N, K)).astype(np.int64)
    where = lo | (mid << 7) | (hi << 14)
    assert sorted(where.tolist()) == list(range(N * K))


def test_w8a8_brute_force_tiny():
    """W8A8 on tiny shapes against pure-Python loops: per-channel INT8 codes
    from the definition (scale max/127, round half even, clamp), integer
    sums, and the fp16 epilogue value before rounding."""
    rng = np.random.default_rng(13)
    M, N, K = 3, 16, 128
    W = rng.standard_normal((N, K)).astype(np.float32)
    X = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    sx = (rng.random(M).astype(np.float32) + np.float32(0.5)) / np.float32(100)
    pk = oracle.w8a8_pack(W)
    for n in range(N):
        s = np.float32(np.max(np.abs(W[n]))) / np.float32(127)
        assert pk["sw"][n] == s
        for k in range(0, K, 7):
            v = np.float32(W[n, k]) / s
            q = int(np.clip(np.rint(v), -127, 127))
            assert pk["Q"][n, k] == q
    acc, y, yd = oracle.w8a8_gemm(X, sx, pk)
    for m in range(M):
        for n in range(N):
            tot = sum(int(X[m, k]) * int(pk["Q"][n, k]) for k in range(K))
            assert acc[m, n] == tot
            assert yd[m, n] == float(tot) * float(sx[m]) * float(pk["sw"][n])


def test_w8a8_equals_w4a8_when_groups_lossless():
    """When every LiquidQuant group spans at most 15 INT8 steps, its second
    level is lossless (s = 1), so the W4A8 and W8A8 integer results agree."""
    rng = np.random.default_rng(14)
    M, N, K, g = 5, 32, 256, 64
    base = rng.integers(-100, 90, size=(N, K // g, 1))
    base[:, 0] = 112  # group 0 spans 112..127
    Q = (base + rng.integers(0, 16, size=(N, K // g, g))).reshape(N, K)
    Q[:, 0] = 127  # fixes every channel's scale: W = Q exactly with sw = 1
    Wf = Q.astype(np.float32)
    X = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    sx = np.ones(M, np.float32)
    p8 = oracle.w8a8_pack(Wf)
    np.testing.assert_array_equal(p8["Q"], Q.astype(np.int8))
    Qg = p8["Q"].reshape(N, K // g, g)
    lossless = (Qg.max(axis=2).astype(int) - Qg.min(axis=2).astype(int) <= 15)
    p4 = oracle.w4a8_pack(Wf, g)
    acc4, _, _ = oracle.w4a8_gemm(X, sx, p4, g)
    acc8, _, _ = oracle.w8a8_gemm(X, sx, p8)
    assert lossless.all()
    assert np.all(p4["s_u8"] == 1)
    np.testing.assert_array_equal(acc4, acc8)
    np.testing.assert_array_equal(acc8, X.astype(np.int64) @ Q.astype(np.int64).T)
