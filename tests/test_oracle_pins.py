"""Pins of the CPU oracle to facts fixed outside itself: format definitions,
hand-derived fixtures, closed forms, invariants and brute force computed by a
different route (Python integers, exact rationals, dequantize-then-matmul).

A plausible slip in the oracle (dropped term, wrong sign or index,
transposed operand, wrong rounding) fails at least one of these.
"""
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32(v) -> float:
    """Round a Python float (binary64) to binary32."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _rne_int(fr: Fraction) -> int:
    """Round an exact rational to the nearest integer, ties to even."""
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


# ---------------------------------------------------------------- int8 act quant

def test_int8_ties_fixture():
    lines = [l for l in open(os.path.join(GOLD, "int8_act_ties.txt")) if not l.startswith("#")]
    vals = {l.split(":")[0]: l.split(":")[1].split() for l in lines if ":" in l}
    x = np.array([float(v) for v in vals["x"]], dtype=np.float32)[None, :]
    codes, s = O.quantize_act_int8(x)
    assert s[0] == np.float32(vals["scale"][0])
    assert codes[0].tolist() == [int(c) for c in vals["codes"]]


def test_int8_bruteforce_all_bf16_patterns():
    """Every finite bf16 value, placed in rows of fixed absmax, against exact
    rational arithmetic: scale = f32(amax/127); code = rne(f32(x/scale))."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f32(bits)
    v = v[np.isfinite(v)]
    for amax in (1.0, 3.0, 448.0, 1e-3, 7.25):
        row = v[np.abs(v) <= amax]
        x = np.concatenate([[np.float32(amax)], row]).astype(np.float32)[None, :]
        codes, s = O.quantize_act_int8(x)
        s_ref = _f32(amax / 127.0)               # binary64 divide then round: correctly rounded
        assert float(s[0]) == s_ref
        # f64 quotient rounded to f32 is the correctly rounded f32 quotient (53 >= 2*24+2)
        q32 = np.array([_f32(float(t) / s_ref) for t in x[0]], dtype=np.float64)
        ref = np.array([max(-127, min(127, _rne_int(Fraction(q)))) for q in q32])
        assert np.array_equal(codes[0].astype(np.int64), ref)


def test_int8_quotients_near_half_steps():
    """Rows at non-power-of-two absmax whose float32 values put fl32(x/scale)
    within a few float32 steps of every half-integer k + 1/2: the code is
    decided by the correctly rounded float32 quotient (exact rationals here),
    which a reciprocal multiply or a float64 scale gets wrong at some of
    them."""
    for amax in (3.0, 7.25, 0.3, 1e-3, 5.5, 123.4, 0.07):
        amax32 = np.float32(amax)
        s_ref = _f32(float(amax32) / 127.0)
        xs = []
        for k in range(127):
            c = np.float32(float(Fraction(2 * k + 1, 2) * Fraction(s_ref)))
            for _ in range(3):
                c = np.nextafter(c, np.float32(0))
            for _ in range(7):
                if abs(c) <= amax32:
                    xs += [c, -c]
                c = np.nextafter(c, np.float32(1e30))
        x = np.array([amax32] + xs, dtype=np.float32)[None, :]
        codes, s = O.quantize_act_int8(x)
        assert float(s[0]) == s_ref
        ref = [max(-127, min(127, _rne_int(Fraction(_f32(float(Fraction(float(t)) / Fraction(s_ref)))))))
               for t in x[0]]
        assert codes[0].astype(np.int64).tolist() == ref, amax


def test_int8_invariants_random_rows():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 300)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    x[5] = 0.0
    codes, s = O.quantize_act_int8(x)
    assert s[5] == 0 and not codes[5].any()
    nz = np.arange(64) != 5
    assert np.all(np.abs(codes[nz]).max(axis=1) == 127)          # absmax maps to 127
    assert np.all((np.sign(codes) == np.sign(x)) | (codes == 0))  # sign kept or zero
    assert codes.min() >= -127                                     # -128 never produced
    err = np.abs(x[nz].astype(np.float64) / s[nz, None].astype(np.float64) - codes[nz])
    assert err.max() <= 0.5 + 1e-5


# ---------------------------------------------------------------- fp8 e4m3

def _e4m3_value_exact(code: int) -> Fraction:
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0:
        return s * Fraction(m, 2 ** 9)
    return s * Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def test_e4m3_fixture():
    for line in open(os.path.join(GOLD, "e4m3_codes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v, c = line.split()
        got = int(O.e4m3_encode(np.array([float(v)], dtype=np.float32))[0])
        assert got == int(c, 16), (v, hex(got), c)


def test_e4m3_decode_matches_exact_definition():
    for c in range(256):
        d = O.e4m3_decode(np.array([c], dtype=np.uint8))[0]
        if c & 0x7F == 0x7F:
            assert np.isnan(d)
        else:
            assert Fraction(d) == _e4m3_value_exact(c)


def test_e4m3_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = O.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes)


def test_e4m3_encode_is_nearest_even_bruteforce():
    """Against a scan over all finite codes with exact rationals."""
    finite = [c for c in range(128) if c != 0x7F]
    exact = {c: _e4m3_value_exact(c) for c in finite}
    rng = np.random.default_rng(3)
    # random magnitudes across the whole range, plus every midpoint and its neighbours
    mags = list(np.exp2(rng.uniform(-12, 9.2, 3000)).astype(np.float32))
    srt = sorted(finite, key=lambda c: exact[c])
    for a, b in zip(srt[:-1], srt[1:]):
        mid = np.float32(float((exact[a] + exact[b]) / 2))
        mags += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    v = np.array(mags, dtype=np.float32)
    v = np.concatenate([v, -v])
    got = O.e4m3_encode(v)
    for x, c in zip(v, got):
        a = Fraction(float(abs(x)))
        a = min(a, Fraction(448))
        best = min(finite, key=lambda k: (abs(exact[k] - a), k % 2))
        want = best | (0x80 if np.signbit(x) else 0)
        assert int(c) == want, (float(x), hex(int(c)), hex(want))


def test_e4m3_encode_is_monotone_in_magnitude():
    """The encoder's code (sign bit aside) never decreases as |v| grows, and
    the sign bit is the input's. Over random finite patterns of both signs
    (sorted by magnitude), every power of two and its neighbours, and both
    zeros. The exhaustive GPU check of the encode relies on it: a run of equal
    GPU codes whose two ends the oracle maps to that code is then matched by
    the oracle at every point in between."""
    rng = np.random.default_rng(11)
    mags = rng.integers(0, 0x7F800000, 400_000, dtype=np.uint32)
    p2 = (np.arange(1, 255, dtype=np.uint32) << 23)
    mags = np.unique(np.concatenate([mags, p2, p2 - 1, p2 + 1, np.array([0, 1, 0x7F7FFFFF], np.uint32)]))
    for sign in (0, 1):
        v = (mags | np.uint32(sign << 31)).view(np.float32)
        c = O.e4m3_encode(v)
        assert np.all((c >> 7) == sign)
        assert np.all(np.diff((c & 0x7F).astype(np.int32)) >= 0)
        assert (c[0] & 0x7F) == 0 and (c[-1] & 0x7F) == 0x7E


def test_fp8_act_quant_rows():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((32, 200)).astype(np.float32)
    x[3] = 0
    codes, s = O.quantize_act_fp8(x)
    assert s[3] == 0 and not codes[3].any()
    dec = O.e4m3_decode(codes)
    nz = np.arange(32) != 3
    assert np.all(np.abs(dec[nz]).max(axis=1) == 448.0)           # absmax row hits 448
    assert np.all(s[nz] == (np.abs(x[nz]).max(axis=1) / np.float32(448)).astype(np.float32))
    # relative error of each code within half an E4M3 ulp (2^-4) in the normal range
    xs = x[nz].astype(np.float64) / s[nz, None]
    big = np.abs(xs) >= 2.0 ** -6
    assert np.all(np.abs(dec[nz][big] - xs[big]) <= np.abs(xs[big]) * 2.0 ** -4 + 1e-12)


def _e4m3_nearest_by_midpoints(q32: np.ndarray) -> np.ndarray:
    """E4M3 code of float32 values by the format's definition, written out
    with midpoints: the positive finite codes 0x00..0x7E increase with their
    exact values; |q| (saturated at 448) takes the code whose interval between
    neighbouring midpoints holds it, and on a midpoint itself the even code of
    the two. Midpoints of E4M3 values are exact in binary64, so the
    comparisons are exact. The sign bit is the input's."""
    vals = [_e4m3_value_exact(c) for c in range(127)]
    assert all(a < b for a, b in zip(vals[:-1], vals[1:]))
    mids = np.array([float((vals[i] + vals[i + 1]) / 2) for i in range(126)])
    assert all(Fraction(m) == (vals[i] + vals[i + 1]) / 2 for i, m in enumerate(mids))
    a = np.minimum(np.abs(np.asarray(q32, dtype=np.float64)), 448.0)
    below = np.searchsorted(mids, a, side="left")          # midpoints strictly below |q|
    on_mid = (below < 126) & (mids[np.minimum(below, 125)] == a)
    code = np.where(on_mid & (below % 2 == 1), below + 1, below)
    return (code.astype(np.uint8) | (np.signbit(q32).astype(np.uint8) << 7)).astype(np.uint8)


def test_fp8_bruteforce_all_bf16_patterns():
    """Every finite bf16 value, placed in rows of fixed absmax (powers of two
    and not), against exact arithmetic: scale = f32(amax/448) (a binary64
    divide rounded to binary32 is the correctly rounded binary32 quotient),
    code = E4M3 of f32(x/scale) by midpoints. A reciprocal multiply, a
    float64 scale or quotient, or a wrong tie rule fails here."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f32(bits)
    v = v[np.isfinite(v)]
    for amax in (1.0, 3.0, 7.25, 0.3, 1e-3, 448.0):
        amax32 = np.float32(amax)
        row = v[np.abs(v) <= amax32]
        x = np.concatenate([[amax32], row]).astype(np.float32)[None, :]
        codes, s = O.quantize_act_fp8(x)
        s_ref = _f32(float(amax32) / 448.0)
        assert float(s[0]) == s_ref, amax
        q32 = np.array([_f32(float(t) / s_ref) for t in x[0]], dtype=np.float32)
        ref = _e4m3_nearest_by_midpoints(q32)
        assert np.array_equal(codes[0], ref), (amax, int(np.sum(codes[0] != ref)))
        assert O.e4m3_decode(codes[:, :1])[0, 0] == 448.0       # the absmax itself maps to 448


def test_fp8_quantizer_midpoint_rows():
    """Rows whose quotients sit exactly on E4M3 midpoints and one float32 step
    either side: scale 1 (absmax 448), so x/scale = x."""
    vals = [_e4m3_value_exact(c) for c in range(127)]
    mids = [np.float32(float((a + b) / 2)) for a, b in zip(vals[:-1], vals[1:])]
    row = [np.float32(448.0)]
    for m in mids:
        row += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9)), -m]
    x = np.array(row, dtype=np.float32)[None, :]
    codes, s = O.quantize_act_fp8(x)
    assert s[0] == np.float32(1.0)
    assert np.array_equal(codes[0], _e4m3_nearest_by_midpoints(x[0]))


def test_fp8_quotients_near_midpoints():
    """Rows at non-power-of-two absmax whose values put fl32(x/scale) within
    a few float32 steps of every E4M3 midpoint: the code is decided by the
    correctly rounded float32 quotient (exact rationals here), which a
    reciprocal multiply or a quotient kept in float64 gets wrong at some."""
    vals = [_e4m3_value_exact(c) for c in range(127)]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    for amax in (3.0, 7.25, 0.3, 1e-3, 5.5, 123.4, 0.07):
        amax32 = np.float32(amax)
        s_ref = _f32(float(amax32) / 448.0)
        xs = []
        for m in mids:
            c = np.float32(float(m) * s_ref)
            for _ in range(3):
                c = np.nextafter(c, np.float32(0))
            for _ in range(7):
                if abs(c) <= amax32:
                    xs += [c, -c]
                c = np.nextafter(c, np.float32(1e30))
        x = np.array([amax32] + xs, dtype=np.float32)[None, :]
        codes, s = O.quantize_act_fp8(x)
        assert float(s[0]) == s_ref
        # exact quotient rounded once to binary32 (all quotients here are normal)
        q32 = np.array([float(_round_binary(Fraction(float(t)) / Fraction(s_ref), 24)) for t in x[0]],
                       dtype=np.float32)
        assert np.array_equal(codes[0], _e4m3_nearest_by_midpoints(q32)), amax


def test_int4_values_exact_in_e4m3():
    v = np.arange(-8, 8, dtype=np.float32)
    assert np.array_equal(O.e4m3_decode(O.e4m3_encode(v)), v.astype(np.float64))


# ---------------------------------------------------------------- layouts

def test_gptq_word_fixture():
    for line in open(os.path.join(GOLD, "gptq_words.txt")):
        if line.startswith("#") or not line.strip():
            continue
        parts = line.split()
        w = np.array([[int(parts[0], 16)]], dtype=np.uint32).view(np.int32)
        assert O.unpack_gptq_kn(w)[:, 0].tolist() == [int(p) for p in parts[1:]]
        assert O.unpack_ct_nk(w)[0].tolist() == [int(p) for p in parts[1:]]


def test_gptq_unpack_bruteforce_python_ints():
    rng = np.random.default_rng(5)
    qw = rng.integers(0, 2 ** 32, (6, 5), dtype=np.uint32).view(np.int32)
    q = O.unpack_gptq_kn(qw)
    assert q.shape == (48, 5)
    for k in range(48):
        for n in range(5):
            word = int(qw.view(np.uint32)[k // 8, n])
            assert q[k, n] == (word // 16 ** (k % 8)) % 16


def test_pack_unpack_roundtrip_and_extremes():
    rng = np.random.default_rng(9)
    for q in (rng.integers(0, 16, (7, 64)), np.zeros((3, 8), int), np.full((3, 8), 15)):
        q = q.astype(np.uint8)
        assert np.array_equal(O.unpack_nibble_bytes(O.pack_nibble_bytes(q)), q)
    b = rng.integers(0, 256, (4, 16), dtype=np.uint8)
    assert np.array_equal(O.pack_nibble_bytes(O.unpack_nibble_bytes(b)), b)


def test_int32_words_are_the_byte_stream():
    """8 codes per little-endian int32 == two codes per byte (zentorch page)."""
    rng = np.random.default_rng(1)
    w = rng.integers(0, 2 ** 32, (9, 12), dtype=np.uint32).view(np.int32)
    assert np.array_equal(O.unpack_ct_nk(w), O.unpack_nibble_bytes(w.view(np.uint8)))


def test_xor_0x88_exhaustive():
    """Signed int4 (two's complement nibble) s -> uint4b8 code s + 8, per nibble."""
    for lo in range(-8, 8):
        for hi in range(-8, 8):
            byte = (lo & 0xF) | ((hi & 0xF) << 4)
            word = np.array([byte, 0x00, 0x00, 0x00], dtype=np.uint8)   # other nibbles: 0 -> 8
            out = O.repack_signed_int4_to_uint4b8(word)
            codes = O.unpack_ct_nk(out.reshape(1, 1))[0]
            assert codes[0] == lo + 8 and codes[1] == hi + 8
            assert np.all(codes[2:] == 8)


# ---------------------------------------------------------------- partials / epilogue

def test_partials_bruteforce_python_ints():
    rng = np.random.default_rng(21)
    M, K, N, g = 3, 64, 5, 32
    codes = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(0, 2 ** 32, (K // 8, N), dtype=np.uint32).view(np.int32)
    P = O.group_partials(codes, O.unpack_gptq_kn(qw), g)
    for m in range(M):
        for gg in range(K // g):
            for n in range(N):
                s = 0
                for k in range(gg * g, (gg + 1) * g):
                    word = int(qw.view(np.uint32)[k // 8, n])
                    s += int(codes[m, k]) * (((word >> (4 * (k % 8))) & 15) - 8)
                assert P[m, gg, n] == s


def test_partials_additive_and_group_minus1_is_K():
    rng = np.random.default_rng(22)
    M, K, N = 9, 512, 24
    codes = rng.integers(-127, 128, (M, K)).astype(np.int8)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    P128 = O.group_partials(codes, q, 128)
    Pch = O.group_partials(codes, q, -1)
    PK = O.group_partials(codes, q, K)
    assert Pch.shape == (M, 1, N)
    assert np.array_equal(P128.sum(axis=1), Pch[:, 0])
    assert np.array_equal(Pch, PK)
    assert np.abs(Pch).max() <= 127 * 8 * K


def test_epilogue_vs_dequantize_then_matmul():
    rng = np.random.default_rng(23)
    M, K, N, g = 6, 256, 40, 64
    codes = rng.integers(-127, 128, (M, K)).astype(np.int8)
    s_a = rng.uniform(0.001, 0.1, M).astype(np.float32)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    sc = rng.uniform(0.005, 0.02, (K // g, N)).astype(np.float16)
    bias = rng.standard_normal(N)
    y = O.w4a8_epilogue(O.group_partials(codes, q, g), s_a, sc.astype(np.float32), bias)
    Xh = codes.astype(np.float64) * s_a.astype(np.float64)[:, None]
    Wh = (q.astype(np.float64) - 8.0) * np.repeat(sc.astype(np.float64), g, axis=0)
    ref = Xh @ Wh + bias
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_epilogue_one_hot_and_all_eights():
    rng = np.random.default_rng(24)
    K, N, g = 256, 16, 128
    qw = rng.integers(0, 2 ** 32, (K // 8, N), dtype=np.uint32).view(np.int32)
    sc = rng.uniform(0.005, 0.02, (K // g, N)).astype(np.float16)
    k0, alpha = 170, 3.25
    x = np.zeros((1, K), np.float32)
    x[0, k0] = alpha
    xb = x.view(np.uint32) >> 16                      # exact bf16 bits (alpha is exact)
    out = O.w4a8_reference(xb.astype(np.uint16), "bf16", qw, sc, g)
    q = O.unpack_gptq_kn(qw)
    want = alpha * (q[k0].astype(np.float64) - 8) * sc[k0 // g].astype(np.float64)
    assert np.allclose(out["y"][0], want, rtol=1e-6)
    # all codes 8 => zero weights => y == bias
    qw8 = np.full((K // 8, N), 0x88888888, dtype=np.uint32).view(np.int32)
    xb2 = (rng.standard_normal((4, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bias = (rng.standard_normal(N).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out8 = O.w4a8_reference(xb2, "bf16", qw8, sc, g, bias_bits=bias)
    assert np.array_equal(out8["y"], np.broadcast_to(O.bf16_bits_to_f32(bias).astype(np.float64), (4, N)))


def test_equal_scales_grouped_equals_per_channel():
    rng = np.random.default_rng(25)
    M, K, N = 5, 384, 32
    codes = rng.integers(-127, 128, (M, K)).astype(np.int8)
    s_a = rng.uniform(0.01, 0.1, M).astype(np.float32)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    col = rng.uniform(0.005, 0.02, N).astype(np.float16).astype(np.float32)
    y_g = O.w4a8_epilogue(O.group_partials(codes, q, 128), s_a, np.tile(col, (K // 128, 1)))
    y_c = O.w4a8_epilogue(O.group_partials(codes, q, -1), s_a, col[None, :])
    assert np.allclose(y_g, y_c, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- W4A16

def test_w4a16_factored_identity_and_one_hot():
    rng = np.random.default_rng(31)
    M, K, N, g = 3, 256, 20, 64
    xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wb = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sb = (rng.uniform(0.005, 0.02, (N, K // g)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    zb = ((rng.standard_normal((N, K // g)) * 0.01).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = O.w4a16_reference(xb, wb, sb, zb, g)
    # factored form by loops: y = sum_g s*sum x(q-8) + z*sum x
    x = O.bf16_bits_to_f32(xb).astype(np.float64)
    s = O.bf16_bits_to_f32(sb).astype(np.float64)
    z = O.bf16_bits_to_f32(zb).astype(np.float64)
    ref = np.zeros((M, N))
    for n in range(N):
        row = wb[n]
        codes = [(int(row[j // 2]) >> (4 * (j % 2))) & 15 for j in range(K)]
        for m in range(M):
            tot = 0.0
            for gg in range(K // g):
                ks = range(gg * g, (gg + 1) * g)
                tot += s[n, gg] * sum(x[m, k] * (codes[k] - 8) for k in ks) + z[n, gg] * sum(x[m, k] for k in ks)
            ref[m, n] = tot
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    # one-hot x picks one dequantized weight column
    k0 = 77
    xo = np.zeros((1, K), np.uint16)
    xo[0, k0] = 0x3F80                                      # bf16 1.0
    y1 = O.w4a16_reference(xo, wb, sb, zb, g)[0]
    q = O.unpack_nibble_bytes(wb)[:, k0].astype(np.float64)
    assert np.array_equal(y1, (q - 8) * s[:, k0 // g] + z[:, k0 // g])


def test_quantize_groupwise_reproduces_extremes():
    rng = np.random.default_rng(32)
    w = rng.standard_normal((12, 128)) * 0.05
    q, s, z = O.quantize_groupwise(w, 64)
    deq = O.dequantize_groupwise(q, s, z, 64)
    wf = w.reshape(12, 2, 64)
    lo = (0.0 - 8) * s + z
    hi = (15.0 - 8) * s + z
    assert np.allclose(lo, wf.min(-1), rtol=0, atol=1e-12)
    assert np.allclose(hi, wf.max(-1), rtol=0, atol=1e-12)
    assert np.all(np.abs(deq - w) <= np.repeat(s, 64, axis=1) / 2 + 1e-12)
    assert q.min() == 0 and q.max() == 15
    with pytest.raises(ValueError):
        O.quantize_groupwise(w[:, :100], 64)


# ---------------------------------------------------------------- routed experts

def _tiny_moe(seed=41, E=4, K=256, N=64, T=32, topk=2):
    from int4_weight_quantized_amd import workloads as W
    return W.moe_inputs(E, K, N, 128, T, topk, seed)


def test_routing_structure():
    d = _tiny_moe()
    rt, off = d["row_token"], d["expert_offsets"]
    assert off[0] == 0 and off[-1] == d["T"] * d["topk"] and np.all(np.diff(off) >= 0)
    pairs = set()
    for e in range(d["E"]):
        toks = rt[off[e]:off[e + 1]]
        assert np.all(np.diff(toks) > 0)                    # stable by token, no duplicates
        pairs |= {(int(t), e) for t in toks}
    per_tok = np.bincount([t for t, _ in pairs], minlength=d["T"])
    assert np.all(per_tok == d["topk"])


def test_grouped_bruteforce_and_segments():
    d = _tiny_moe()
    x32 = O.bf16_bits_to_f32(d["x"])
    a8, s_a = O.quantize_act_fp8(x32)
    y = O.grouped_fp8_reference(a8, s_a, d["row_token"], d["expert_offsets"], d["w"], d["scales"], 128)
    off = d["expert_offsets"]
    # brute force: dequantize activations and weights fully, per routed row
    for e in range(d["E"]):
        Wd = np.zeros((d["K"], d["N"]))
        for n in range(d["N"]):
            for k in range(d["K"]):
                word = int(d["w"].view(np.uint32)[e, n, k // 8])
                qv = (word >> (4 * (k % 8))) & 15
                Wd[k, n] = (qv - 8) * float(d["scales"][e, k // 128, n])
        for r in range(off[e], off[e + 1]):
            t = d["row_token"][r]
            xa = O.e4m3_decode(a8[t]) * float(s_a[t])
            assert np.allclose(y[r], xa @ Wd, rtol=1e-12, atol=1e-12)
    # a row subset gives the same numbers
    rows = np.array([5, 0, 63, 17])
    ys = O.grouped_fp8_reference(a8, s_a, d["row_token"], off, d["w"], d["scales"], 128, rows=rows)
    assert np.array_equal(ys, y[rows])


def test_grouped_single_expert_is_dense():
    d = _tiny_moe(seed=42, E=1, T=16, topk=1)
    x32 = O.bf16_bits_to_f32(d["x"])
    a8, s_a = O.quantize_act_fp8(x32)
    y = O.grouped_fp8_reference(a8, s_a, d["row_token"], d["expert_offsets"], d["w"], d["scales"], 128)
    assert np.array_equal(d["row_token"], np.arange(16))
    A = O.e4m3_decode(a8) * s_a.astype(np.float64)[:, None]
    q = O.unpack_ct_nk(d["w"][0]).astype(np.float64) - 8
    Wd = q * np.repeat(d["scales"][0].astype(np.float64), 128, axis=0).T
    assert np.allclose(y, A @ Wd.T, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ weight-only path on GPTQ weights

def test_w4a16_gptq_reduces_to_byte_layout_path():
    """Same codes in the GPTQ words and in the two-per-byte layout, zero offsets
    0 and scales representable in both fp16 and bf16: the weight-only GPTQ
    reference equals the (separately pinned) byte-layout reference."""
    rng = np.random.default_rng(41)
    M, K, N, g = 3, 256, 24, 64
    xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q = rng.integers(0, 16, (K, N))
    words = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        words |= (q[i::8, :].astype(np.uint32) << np.uint32(4 * i))
    s = (rng.integers(1, 128, (K // g, N)) * 2.0 ** -12).astype(np.float32)   # exact in fp16 and bf16
    y = O.w4a16_gptq_reference(xb, "bf16", words.view(np.int32), s.astype(np.float16), g)
    wbytes = O.pack_nibble_bytes(q.T.astype(np.uint8))                        # [N, K/2]
    sb = (s.T.copy().view(np.uint32) >> 16).astype(np.uint16)
    zb = np.zeros_like(sb)
    ref = O.w4a16_reference(xb, wbytes, sb, zb, g)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_w4a16_gptq_one_hot_and_bias():
    rng = np.random.default_rng(42)
    K, N, g = 128, 16, 64
    words = rng.integers(0, 2**32, (K // 8, N), dtype=np.uint32).view(np.int32)
    s = rng.uniform(0.005, 0.02, (K // g, N)).astype(np.float16)
    k = 77
    x = np.zeros((1, K), dtype=np.float32)
    x[0, k] = 3.0
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    y = O.w4a16_gptq_reference(xb, "bf16", words, s, g)[0]
    qk = (words.view(np.uint32)[k // 8] >> np.uint32(4 * (k % 8))) & 15
    assert np.array_equal(y, 3.0 * (qk.astype(np.float64) - 8) * s[k // g].astype(np.float64))
    bias = (np.arange(N, dtype=np.float32) / 8).astype(np.float16).view(np.uint16)
    xh = x.astype(np.float16).view(np.uint16)
    yb = O.w4a16_gptq_reference(xh, "f16", words, s, g, bias_bits=bias)[0]
    assert np.array_equal(yb, y + np.arange(N) / 8)


def test_w4a16_gptq_brute_force_per_channel():
    rng = np.random.default_rng(43)
    M, K, N = 2, 24, 8
    words = rng.integers(0, 2**32, (K // 8, N), dtype=np.uint32)
    s = rng.uniform(0.005, 0.02, (1, N)).astype(np.float16)
    xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = O.w4a16_gptq_reference(xb, "bf16", words.view(np.int32), s, -1)
    x = O.bf16_bits_to_f32(xb).astype(np.float64)
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for kk in range(K):
                code = (int(words[kk // 8, n]) >> (4 * (kk % 8))) & 15
                tot += x[m, kk] * (code - 8) * float(s[0, n])
            assert abs(y[m, n] - tot) <= 1e-12 * max(1.0, abs(tot))


# ------------------------------------------------------------------ groupwise quantizer in float32

def test_quantize_groupwise_f32_properties():
    """The float32 quantizer against what the page fixes: every group's min
    gets code 0 and its max code 15; the dequantized extremes come back to
    within float32 rounding; codes agree with the float64 quantizer except
    where the float64 quotient sits within float32 rounding of a half step."""
    rng = np.random.default_rng(51)
    w = (rng.standard_normal((6, 512)) * rng.uniform(0.01, 3.0, (6, 1))).astype(np.float32)
    w[0, :64] = 0.25                               # constant group: scale from the 1e-9 clamp
    g = 64
    q, s, z = O.quantize_groupwise_f32(w, g)
    assert q.dtype == np.uint8 and s.dtype == np.float32 and z.dtype == np.float32
    wf = w.reshape(6, -1, g)
    qf = q.reshape(6, -1, g)
    imin, imax = wf.argmin(-1), wf.argmax(-1)
    for r in range(6):
        for gg in range(wf.shape[1]):
            assert qf[r, gg, imin[r, gg]] == 0
            if wf[r, gg].max() > wf[r, gg].min():
                assert qf[r, gg, imax[r, gg]] == 15
    assert s[0, 0] == np.float32(np.float32(1e-9) / np.float32(15)) and np.all(q[0, :64] == 0)
    deq = (q.reshape(6, -1, g).astype(np.float64) - 8) * s[..., None] + z[..., None]
    assert np.allclose(deq.min(-1), wf.min(-1), rtol=0, atol=4 * np.abs(wf).max() * 2.0 ** -23)
    assert np.allclose(deq.max(-1), wf.max(-1), rtol=0, atol=4 * np.abs(wf).max() * 2.0 ** -23)
    q64, s64, _ = O.quantize_groupwise(w.astype(np.float64), g)
    quot = (wf.astype(np.float64) - wf.min(-1, keepdims=True)) / s64[..., None]
    near_half = np.abs(quot - np.floor(quot) - 0.5) < 1e-4
    assert np.array_equal(q.reshape(quot.shape)[~near_half], q64.reshape(quot.shape)[~near_half])


def test_quantize_groupwise_f32_worked_example():
    """A group worked by hand: values 0, 1, ..., 15 scaled by 0.5 give
    scale 0.5, zero 4.0 and codes 0..15 (every quotient is an exact integer)."""
    w = (np.arange(64, dtype=np.float32) % 16 * np.float32(0.5)).reshape(1, 64)
    q, s, z = O.quantize_groupwise_f32(w, 64)
    assert s[0, 0] == np.float32(0.5) and z[0, 0] == np.float32(4.0)
    assert np.array_equal(q[0], (np.arange(64) % 16).astype(np.uint8))


def test_unpack_i8_nk_exhaustive():
    """int8 [N, K] weights: every int4 value -8..7 maps to its uint4b8 code
    v + 8, the same code the signed-nibble XOR 0x88 repack gives."""
    v = np.arange(-8, 8, dtype=np.int8).reshape(1, 16)
    q = O.unpack_i8_nk(v)
    assert np.array_equal(q[0], np.arange(16, dtype=np.uint8))
    nib = (v.astype(np.int16) & 0xF).astype(np.uint8)                 # two's-complement nibbles
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)     # two per byte, low first
    assert np.array_equal(O.unpack_nibble_bytes(packed ^ np.uint8(0x88)), q)
    with pytest.raises(AssertionError):
        O.unpack_i8_nk(np.array([[8]], dtype=np.int8))


def test_static_int8_quantizer():
    """Static scale: hand-worked ties and saturation; with the row's own
    dynamic scale it gives the (separately pinned) dynamic codes."""
    x = np.array([[0.25, 0.75, -0.75, 63.25, -63.75, 500.0, -500.0, 0.0]], dtype=np.float32)
    c = O.quantize_act_int8_static(x, 0.5)
    assert c.tolist() == [[0, 2, -2, 126, -128 + 1, 127, -127, 0]]     # 0.5->0, 1.5->2, 126.5->126, -127.5 clamps
    assert not O.quantize_act_int8_static(x, 0.0).any()
    rng = np.random.default_rng(61)
    xr = rng.standard_normal((5, 300)).astype(np.float32)
    codes, s = O.quantize_act_int8(xr)
    for m in range(5):
        assert np.array_equal(O.quantize_act_int8_static(xr[m:m + 1], s[m]), codes[m:m + 1])


# ------------------------------------------------------------------ asymmetric activations

def test_asym_int8_worked_example():
    """Hand-worked (reading of [ct_w4a8] input_symmetric=False on the [cpu_int4]
    min/max grid): row [0, 100.5, 101.5, 255, 37] has min 0, max 255, so the
    step is exactly 1 and the offset 0 + 128 = 128. Code + 128 counts steps
    from the minimum: 0, 100.5 -> 100 and 101.5 -> 102 (ties to even), 255, 37.
    Scaling the row by 2**-3 scales step and offset and keeps the codes."""
    x = np.array([[0, 100.5, 101.5, 255, 37]], dtype=np.float32)
    want = np.array([[-128, -28, -26, 127, -91]], dtype=np.int8)
    for k in (0, -3, 5):
        c, s, z = O.quantize_act_int8_asym(x * np.float32(2.0 ** k))
        assert np.array_equal(c, want) and s[0] == 2.0 ** k and z[0] == 128 * 2.0 ** k
    # shifted by -40: min -40 -> offset -40 + 128, same codes
    c, s, z = O.quantize_act_int8_asym(x - np.float32(40))
    assert np.array_equal(c, want) and s[0] == 1 and z[0] == 88


def test_asym_int8_invariants_and_constant_rows():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 300)) * rng.uniform(0.01, 30, (64, 1)) + rng.uniform(-5, 5, (64, 1)))
    x = x.astype(np.float32)
    c, s, z = O.quantize_act_int8_asym(x)
    lo, hi = x.min(1), x.max(1)
    for m in range(64):
        # the grid spans the row: its minimum sits on code -128, its maximum on 127
        assert c[m, np.argmin(x[m])] == -128 and c[m, np.argmax(x[m])] == 127
        # every value is within half a step (plus fp32 slack) of its grid point
        deq = c[m].astype(np.float64) * s[m] + z[m]
        assert np.all(np.abs(deq - x[m]) <= 0.5 * s[m] * (1 + 1e-5) + 1e-6 * (abs(lo[m]) + abs(hi[m])))
        # codes are monotone in x
        o = np.argsort(x[m], kind="stable")
        assert np.all(np.diff(c[m][o].astype(np.int32)) >= 0)
        # the step is the range over 255 levels
        assert abs(float(s[m]) - (float(hi[m]) - float(lo[m])) / 255) <= 1e-6 * float(s[m])
    # a constant row: no step, every code at -128, offset = the value (exact)
    cc, sc, zc = O.quantize_act_int8_asym(np.full((2, 7), -3.25, dtype=np.float32))
    assert np.all(cc == -128) and np.all(sc == 0) and np.all(zc == np.float32(-3.25))


def test_asym_epilogue_vs_dequantize_then_matmul():
    """y = sum_k (code*s + z) * (q-8) * scale, the definition, against the
    factored s * sum_g scale * P + z * C[n] the reference computes; plus the
    constant-row special case y[n] = value * C[n] and C against a loop."""
    rng = np.random.default_rng(5)
    M, K, N = 5, 256, 24
    for group in (64, -1):
        G = 1 if group == -1 else K // group
        x = rng.standard_normal((M, K)).astype(np.float32) + np.float32(1.5)
        x[3] = np.float32(0.75)                                   # constant row
        xb = (x.view(np.uint32) >> 16).astype(np.uint16)          # bf16 bits (truncated: any bf16 input)
        qw = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32).view(np.int32)
        sc = rng.uniform(0.005, 0.02, (G, N)).astype(np.float16)
        ref = O.w4a8_reference_asym(xb, "bf16", qw, sc, group)
        x32 = O.bf16_bits_to_f32(xb)
        c, s, z = O.quantize_act_int8_asym(x32)
        q = O.unpack_gptq_kn(qw).astype(np.float64)
        g_eff = K if group == -1 else group
        Wd = (q - 8) * np.repeat(sc.astype(np.float64), g_eff, axis=0)
        Xd = c.astype(np.float64) * s.astype(np.float64)[:, None] + z.astype(np.float64)[:, None]
        assert np.allclose(ref["y"], Xd @ Wd, rtol=1e-12, atol=1e-12)
        C = np.zeros(N)
        for n in range(N):
            for k in range(K):
                C[n] += (q[k, n] - 8) * float(sc[k // g_eff, n])
        assert np.allclose(O.weight_offsets(O.unpack_gptq_kn(qw), sc, group), C, rtol=1e-12, atol=1e-12)
        assert np.allclose(ref["y"][3], float(x32[3, 0]) * C, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- bf16 rounding and the prefill dequantization

def _round_binary(fr: Fraction, p: int) -> Fraction:
    """Round an exact rational to p significant bits, nearest even (normal range)."""
    if fr == 0:
        return Fraction(0)
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - (p - 1))
    return sgn * _rne_int(a / ulp) * ulp


def test_f32_to_bf16_rounding():
    """Against exact rational rounding to 8 significant bits and against the
    library's float32 -> bfloat16 cast, on random values, exact ties of both
    parities and their float32 neighbours."""
    import torch
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(4000) * np.exp2(rng.uniform(-30, 30, 4000))).astype(np.float32)
    ties = (rng.integers(1, 1 << 16, 500).astype(np.uint32) << 16) | np.uint32(0x8000)
    t = ties.view(np.float32)
    v = np.concatenate([v, t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(np.inf)), -t])
    v = v[np.isfinite(v)]
    got = O.f32_to_bf16_bits(v)
    for x, g in zip(v[:1500], got[:1500]):
        want = _round_binary(Fraction(float(x)), 8)
        assert Fraction(float(O.bf16_bits_to_f32(np.array([g]))[0])) == want, (float(x), hex(int(g)))
    lib = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, lib)


def test_dequantize_bf16_fixture():
    """Hand-worked values (tests/golden/dequant_bf16.txt), including ties where
    the one-rounding reading and op-by-op bf16 rounding differ."""
    for line in open(os.path.join(GOLD, "dequant_bf16.txt")):
        if line.startswith("#") or not line.strip():
            continue
        q, sc, z, w = line.split()
        sb = O.f32_to_bf16_bits(np.array([[float(sc)]], dtype=np.float32))
        zb = O.f32_to_bf16_bits(np.array([[float(z)]], dtype=np.float32))
        assert O.bf16_bits_to_f32(sb)[0, 0] == float(sc) and O.bf16_bits_to_f32(zb)[0, 0] == float(z)
        got = O.dequantize_bf16(np.full((1, 64), int(q), np.uint8), sb, zb, 64)
        assert np.all(got == int(w, 16)), (line, hex(int(got[0, 0])))


def test_dequantize_bf16_exact_rationals():
    """Random codes, bf16 scales and offsets: the exact value (q - 8)*s + z
    rounded to float32 and then to bf16, with rationals, per element."""
    rng = np.random.default_rng(17)
    N, K, g = 6, 256, 64
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    sb = O.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (N, K // g)).astype(np.float32))
    zb = O.f32_to_bf16_bits((rng.standard_normal((N, K // g)) * 0.01).astype(np.float32))
    got = O.dequantize_bf16(q, sb, zb, g)
    s = O.bf16_bits_to_f32(sb)
    z = O.bf16_bits_to_f32(zb)
    for n in range(N):
        for k in range(K):
            ex = (int(q[n, k]) - 8) * Fraction(float(s[n, k // g])) + Fraction(float(z[n, k // g]))
            want = _round_binary(_round_binary(ex, 24), 8)
            assert Fraction(float(O.bf16_bits_to_f32(got[n:n + 1, k:k + 1])[0, 0])) == want, (n, k)


def test_prefill_reference_reduces_to_exact_w4a16():
    """With zero offsets and power-of-two scales every dequantized weight is
    exact in bf16, so the prefill reference equals the exact W4A16 reference
    (pinned separately); with general scales they differ by at most the bf16
    rounding of each weight."""
    rng = np.random.default_rng(23)
    M, N, K, g = 5, 24, 256, 64
    xb = O.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    wb = O.pack_nibble_bytes(q)
    s_pow2 = O.f32_to_bf16_bits(np.exp2(rng.integers(-9, -5, (N, K // g))).astype(np.float32))
    z0 = np.zeros((N, K // g), np.uint16)
    a = O.w4a16_prefill_reference(xb, wb, s_pow2, z0, g)
    b = O.w4a16_reference(xb, wb, s_pow2, z0, g)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    sb = O.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (N, K // g)).astype(np.float32))
    zb = O.f32_to_bf16_bits((rng.standard_normal((N, K // g)) * 0.01).astype(np.float32))
    a = O.w4a16_prefill_reference(xb, wb, sb, zb, g)
    b = O.w4a16_reference(xb, wb, sb, zb, g)
    x = O.bf16_bits_to_f32(xb).astype(np.float64)
    wexact = O.dequantize_groupwise(q, O.bf16_bits_to_f32(sb), O.bf16_bits_to_f32(zb), g)
    bound = np.abs(x) @ (np.abs(wexact) * 2.0 ** -8).T
    assert np.all(np.abs(a - b) <= bound + 1e-12)
    assert not np.allclose(a, b, rtol=0, atol=1e-9)              # the rounding is really there
