"""Host check of the division scheme the activation quantizer runs on the GPU
(csrc/quant_act.hip): a per-row reciprocal (hardware reciprocal, within 1 ulp,
plus one Newton step) and two fma corrections of the quotient by its
remainder must give the correctly rounded fp32 quotient x / s, which is what
the codes are decided on.

Every fp32 operation is modelled exactly: operands are rationals, each
result is rounded to the nearest fp32 (ties to even) once, as fma and the
other single operations do. The hardware reciprocal is modelled as the
correctly rounded one and its two neighbours (any value within 1 ulp)."""
import numpy as np
from fractions import Fraction as F

ONE = F(1)


def rn32(v: F) -> F:
    """Nearest fp32 to the rational v (ties to even), subnormals included."""
    if v == 0:
        return F(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = F(2) ** (e - 23)
    m = a / ulp
    whole = m.numerator // m.denominator
    rest = m - whole
    if rest > F(1, 2) or (rest == F(1, 2) and whole % 2 == 1):
        whole += 1
    return sign * whole * ulp


def kernel_quotient(x: float, s: float, y0: float) -> F:
    X, S, Y0 = F(x), F(s), F(y0)
    y = rn32(rn32(-S * Y0 + ONE) * Y0 + Y0)    # Newton step on the reciprocal
    q0 = rn32(X * y)
    r0 = rn32(-S * q0 + X)
    q1 = rn32(r0 * y + q0)
    r1 = rn32(-S * q1 + X)
    return rn32(r1 * y + q1)


def reciprocals(s: float):
    y = np.float32(1.0) / np.float32(s)
    return [float(np.nextafter(y, np.float32(0))), float(y), float(np.nextafter(y, np.float32(np.inf)))]


def bf16_round(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float32)
    return (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def test_random_rows_match_exact_rounding():
    rng = np.random.default_rng(7)
    checked = 0
    for it in range(120):
        amax = bf16_round(np.float32(abs(rng.standard_normal()) * 2.0 ** int(rng.integers(-60, 60)) + 1e-30))
        s = float(np.float32(amax) / np.float32(127.0 if it % 2 else 448.0))
        if it % 5 == 0:
            s = float(np.float32(2.0 ** rng.uniform(-90, 90)))
            amax = np.float32(127.25 * s)
        xs = bf16_round(rng.standard_normal(8).astype(np.float32) * np.float32(amax))
        for y0 in reciprocals(s):
            for x in xs:
                assert kernel_quotient(float(x), s, y0) == rn32(F(float(x)) / F(s)), (float(x), s, y0)
                checked += 1
    assert checked > 2000


def test_quotients_near_rounding_boundaries():
    """Quotients a few ulps from int8 half-steps and from E4M3 midpoints,
    where a faithful but not correctly rounded quotient would flip a code."""
    rng = np.random.default_rng(11)
    for it in range(150):
        s = float(np.float32(2.0 ** rng.uniform(-80, 80)))
        if it % 2:
            h = float(rng.integers(-127, 127)) + 0.5
        else:
            h = 2.0 ** int(rng.integers(-9, 8)) * (1 + (2 * int(rng.integers(0, 8)) + 1) / 16)
        x0 = np.float32(h * s)
        xs = [x0]
        up, down = x0, x0
        for _ in range(2):
            up = np.nextafter(up, np.float32(np.inf))
            down = np.nextafter(down, np.float32(-np.inf))
            xs += [up, down]
        for y0 in reciprocals(s):
            for x in xs:
                assert kernel_quotient(float(x), s, y0) == rn32(F(float(x)) / F(s)), (float(x), s, y0)


def hard_cases(n: int, rng):
    """(x, s) whose quotient lies within about 2^-48 (relative) of the
    midpoint between two fp32 values: with S odd (24 bits), K = r / S mod 2^25
    for a small odd r makes K*S - r a multiple of 2^25, so x = (K*S - r) / 2^25
    has 24 bits and x / S = K / 2^25 - r / (2^25 S), next to the midpoint
    K / 2^25 (K odd, 25 bits)."""
    out = []
    while len(out) < n:
        S = int(rng.integers(2 ** 23, 2 ** 24)) | 1
        r = int(rng.choice([-7, -5, -3, -1, 1, 3, 5, 7]))
        K = (r * pow(S, -1, 2 ** 25)) % 2 ** 25
        if not (2 ** 24 <= K < 2 ** 25):
            continue
        X = (K * S - r) // 2 ** 25
        if not (2 ** 23 <= X < 2 ** 24):
            continue
        a = int(rng.integers(-110, 67))                # s = S 2^a in [2^-90, 2^90]
        c = a + int(rng.integers(-10, 8))              # quotient between about 2^-11 and 2^8
        out.append((float(X) * 2.0 ** c, float(S) * 2.0 ** a))
    return out


def test_quotients_next_to_fp32_midpoints():
    """The hardest cases for a division that is only faithful (the same
    corrections on the unrefined hardware reciprocal miss some of them)."""
    rng = np.random.default_rng(5)
    for x, s in hard_cases(300, rng):
        assert np.float32(x) == x and np.float32(s) == s
        for y0 in reciprocals(s):
            assert kernel_quotient(x, s, y0) == rn32(F(x) / F(s)), (x, s, y0)


def test_rn32_against_numpy():
    """The rounding model itself: float32 division in numpy is correctly rounded."""
    rng = np.random.default_rng(3)
    a = rng.standard_normal(300).astype(np.float32) * np.float32(2.0) ** rng.integers(-40, 40, 300).astype(np.float32)
    b = rng.standard_normal(300).astype(np.float32) * np.float32(2.0) ** rng.integers(-40, 40, 300).astype(np.float32)
    for x, y in zip(a, b):
        assert rn32(F(float(x)) / F(float(y))) == F(float(np.float32(x) / np.float32(y)))
