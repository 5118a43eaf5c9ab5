"""Mutation check of the oracle's pins (CPU).

Each case plants one plausible mistake in a copy of oracle/w4_oracle.py (a
text replacement, compiled into a separate module; the real oracle is not
touched) and runs the pin tests of test_oracle_pins.py against that copy:
at least one pin must fail. The pins run in file order and a case stops at
its first failing pin (the pins are tried cheapest first); only an
assertion counts as a catch.

Mutants that cannot be caught because they compute the same thing are not
listed here: clamping int8 codes at -128 (the clamp never binds, |x/s| <=
127(1 + 2^-24)) and a float32 quotient formed in float64 first (a quotient
rounded to 53 and then to 24 bits is the correctly rounded one).
"""
import inspect
import os
import time
import types

import pytest

import test_oracle_pins as P

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "w4_oracle.py")

MUTANTS = {
    # activation quantizers
    "int8_reciprocal": ("q = x32[nz] / scale[nz][:, None]          # fp32 / fp32, correctly rounded",
                        "q = x32[nz] * (F32(1.0) / scale[nz])[:, None]"),
    "int8_round_away": ("codes[nz] = np.clip(np.rint(q), -127, 127).astype(np.int8)",
                        "codes[nz] = np.clip(np.trunc(q + np.copysign(F32(0.5), q)), -127, 127).astype(np.int8)"),
    "int8_div_128": ("scale = (amax / F32(127.0)).astype(F32)\n    codes = np.zeros(x32.shape, dtype=np.int8)",
                     "scale = (amax / F32(128.0)).astype(F32)\n    codes = np.zeros(x32.shape, dtype=np.int8)"),
    "fp8_reciprocal": ("codes[nz] = e4m3_encode(x32[nz] / scale[nz][:, None])",
                       "codes[nz] = e4m3_encode(x32[nz] * (F32(1.0) / scale[nz])[:, None])"),
    "fp8_scale_f64": ("scale = (amax / F32(448.0)).astype(F32)\n    codes = np.zeros(x32.shape, dtype=np.uint8)",
                      "scale = (amax.astype(np.float64) / 448.0)\n    codes = np.zeros(x32.shape, dtype=np.uint8)"),
    "fp8_div_447": ("scale = (amax / F32(448.0)).astype(F32)\n    codes = np.zeros(x32.shape, dtype=np.uint8)",
                    "scale = (amax / F32(447.0)).astype(F32)\n    codes = np.zeros(x32.shape, dtype=np.uint8)"),
    "e4m3_ties_away": ("pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))", "pick_hi = (d_hi <= d_lo)"),
    "e4m3_ties_odd": ("pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))",
                      "pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 1))"),
    "e4m3_bias_8": ("mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))",
                    "mag = np.where(e == 0, m * 2.0 ** -10, (1.0 + m / 8.0) * np.exp2(e - 8.0))"),
    "asym_offset_127": ("offset = (lo + F32(128.0) * scale).astype(F32)", "offset = (lo + F32(127.0) * scale).astype(F32)"),
    "asym_255_levels": ("scale = (d / F32(255.0)).astype(F32)", "scale = (d / F32(256.0)).astype(F32)"),
    # weight layouts
    "nibbles_msb_first": ("shifts = (4 * np.arange(8, dtype=np.uint32))", "shifts = (4 * np.arange(7, -1, -1, dtype=np.uint32))"),
    "bytes_swapped": ("out[:, 0::2] = b & 0x0F\n    out[:, 1::2] = b >> 4", "out[:, 0::2] = b >> 4\n    out[:, 1::2] = b & 0x0F"),
    "xor_0x80": ("u = np.ascontiguousarray(np.asarray(b).view(np.uint8)) ^ np.uint8(0x88)",
                 "u = np.ascontiguousarray(np.asarray(b).view(np.uint8)) ^ np.uint8(0x80)"),
    "i8_zero_7": ("return (v + 8).astype(np.uint8)", "return (v + 7).astype(np.uint8)"),
    # W4A8 partials and epilogue
    "partials_zero_7": ("W = q_kn.astype(np.float64) - 8.0\n    P = np.empty", "W = q_kn.astype(np.float64) - 7.0\n    P = np.empty"),
    "epilogue_scales_transposed": ('y = np.einsum("mgn,gn->mn", P.astype(np.float64), S)',
                                   'y = np.einsum("mgn,gn->mn", P.astype(np.float64), S[::-1])'),
    "epilogue_no_row_scale": ("    y *= np.asarray(a_scale, dtype=np.float64)[:, None]\n", "\n"),
    "offsets_zero_7": ("W = (q_kn.astype(np.int64) - 8).reshape(K // g_eff, g_eff, -1).sum(axis=1)",
                       "W = (q_kn.astype(np.int64) - 7).reshape(K // g_eff, g_eff, -1).sum(axis=1)"),
    # W4A16 and the vocab table
    "w4a16_zero_sign": ("    return (q - 8.0) * s + z\n", "    return (q - 8.0) * s - z\n"),
    "groupwise_min_7": ("zero = wmin + 8.0 * scale", "zero = wmin + 7.0 * scale"),
    "groupwise_div_16": ("scale = np.maximum(wmax - wmin, 1e-9) / 15.0", "scale = np.maximum(wmax - wmin, 1e-9) / 16.0"),
    # grouped FP8
    "grouped_row_not_token": ("t = np.asarray(row_token)[rows[sel]]", "t = rows[sel] % a8.shape[0]"),
    "grouped_zero_7": ("W = unpack_ct_nk(w_enk[e]).astype(np.float64) - 8.0      # [N, K]",
                       "W = unpack_ct_nk(w_enk[e]).astype(np.float64) - 7.0      # [N, K]"),
    # bf16 rounding, the prefill dequantization and reference
    "bf16_truncate": ("up = (low > 0x8000) | ((low == 0x8000) & ((kept & np.uint64(1)) == 1))", "up = low < 0"),
    "bf16_ties_up": ("up = (low > 0x8000) | ((low == 0x8000) & ((kept & np.uint64(1)) == 1))", "up = low >= 0x8000"),
    "dequant_rounds_twice": ("    w32 = (prod + z).astype(F32)\n",
                             "    w32 = bf16_bits_to_f32(f32_to_bf16_bits(bf16_bits_to_f32(f32_to_bf16_bits(prod)) + z))\n"),
    "dequant_zero_dropped": ("    w32 = (prod + z).astype(F32)\n", "    w32 = (prod + 0 * z).astype(F32)\n"),
    "dequant_zero_7": ("    prod = (q.astype(F32) - F32(8.0)) * s\n", "    prod = (q.astype(F32) - F32(7.0)) * s\n"),
    "prefill_exact_weights": (
        "    Wb = bf16_bits_to_f32(dequantize_bf16(unpack_nibble_bytes(w_bytes), scale_bits, zero_bits, group))\n",
        "    Wb = dequantize_groupwise(unpack_nibble_bytes(w_bytes), bf16_bits_to_f32(scale_bits), "
        "bf16_bits_to_f32(zero_bits), group)\n"),
}

_ALL_PINS = [f for name, f in inspect.getmembers(P, inspect.isfunction)
             if name.startswith("test_") and f.__module__ == P.__name__]


def _pins_by_cost():
    """The pins, each run once on the real oracle (they must all pass there),
    cheapest first, so that a mutant meets the quick pins before the brute
    force ones."""
    cost = []
    for f in _ALL_PINS:
        t0 = time.perf_counter()
        f()
        cost.append((time.perf_counter() - t0, f.__code__.co_firstlineno, f))
    return [f for _, _, f in sorted(cost, key=lambda c: c[:2])]


_PINS = []


def _mutant_module(name: str, old: str, new: str) -> types.ModuleType:
    src = open(SRC_PATH).read()
    assert src.count(old) == 1, f"{name}: the text to replace is not in the oracle exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    old, new = MUTANTS[name]
    if not _PINS:
        _PINS.extend(_pins_by_cost())
    monkeypatch.setattr(P, "O", _mutant_module(name, old, new))
    for pin in _PINS:
        try:
            pin()
        except AssertionError:
            return                                   # caught by this pin
    pytest.fail(f"no pin fails on mutant {name}")
