"""Plain CPU oracle of the int4-weight quantized linear layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path. It shares no code,
table or helper with the HIP library.

Every function follows a passage of the source pages, cited by page and
symbol:
  [inc_w4a8]   vLLM docs page vllm.model_executor.layers.quantization.inc.
               schemes.inc_w4a8_linear, class INCXPUW4A8LinearMethod
  [ct_w4a8]    vLLM v0.10.1.1 docs page ...compressed_tensors.schemes.
               compressed_tensors_w4a8_int, class CompressedTensorsW4A8Int
  [w4afp8]     vLLM docs page vllm.model_executor.layers.quantization.w4afp8
  [zentorch]   vLLM docs page vllm.model_executor.kernels.linear.
               mixed_precision.zentorch, class ZentorchWNA16LinearKernel
  [cpu_int4]   vllm-omni page model_executor/layers/quantization/cpu_int4.py

Precision. Floating point is carried in float64, except where a float result
decides an integer code (the activation quantizers): there both the oracle
and the kernels take the decision in float32 (the pages fix no precision;
fp32 is the kernels'), with IEEE correctly rounded division and
round-half-to-even. Integer sums are exact (float64 matmuls of
integer-valued operands whose sums stay far below 2**53 are exact).

Readings where the pages are silent are marked READING and listed in the
design notes: rounding is RNE, the int8 scale is fp32 absmax/127 and codes
are x/scale (fp32 divide), an all-zero row has scale 0 and codes 0, the FP8
format is OCP E4M3FN with saturation, weight codes sit LSB-first in their
words, the zero point is the constant 8.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# --------------------------------------------------------------------------
# 16-bit float formats (definitions): bf16 is the upper half of an IEEE
# binary32; fp16 is IEEE binary16 (numpy's float16).
# --------------------------------------------------------------------------


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits_to_f32(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def half_bits_to_f32(bits, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(bits)
    if dtype == "f16":
        return f16_bits_to_f32(bits)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Per-token symmetric int8 activation quantization.
# [inc_w4a8] docstring and apply_weights: activations are quantized per token
# (row) to symmetric int8 on the fly before the int8 GEMM; the op returns the
# codes and one scale per token. scale = absmax / 127 (symmetric int8 grid).
# READING: codes = clamp(rne(x / scale), -127, 127) in fp32; all-zero row ->
# scale 0, codes 0.
# --------------------------------------------------------------------------


def quantize_act_int8(x32: np.ndarray):
    """x32 float32 [M, K] -> (codes int8 [M, K], scale float32 [M])."""
    x32 = np.asarray(x32, dtype=F32)
    assert np.all(np.isfinite(x32)), "oracle assumes finite activations"
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], F32)
    scale = (amax / F32(127.0)).astype(F32)
    codes = np.zeros(x32.shape, dtype=np.int8)
    nz = scale > 0
    if np.any(nz):
        q = x32[nz] / scale[nz][:, None]          # fp32 / fp32, correctly rounded
        codes[nz] = np.clip(np.rint(q), -127, 127).astype(np.int8)
    return codes, scale


# --------------------------------------------------------------------------
# FP8 E4M3 (OCP "E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
# infinities; S.1111.111 is NaN; largest finite 448; subnormals m * 2**-9.
# [w4afp8] W4AFP8Config.__init__: routed-expert activations are 8-bit float,
# symmetric, per token, dynamic. READING: OCP E4M3FN (absmax/448 implies the
# 448 maximum), scale = absmax / 448 in fp32, code = E4M3 of fp32(x / scale)
# rounded to nearest even with saturation to +-448, sign kept (also for 0).
# --------------------------------------------------------------------------


def quantize_act_int8_static(x32: np.ndarray, s) -> np.ndarray:
    """[ct_w4a8] is_static_input_scheme: one calibrated fp32 scale for every
    row. READING: code = clamp(rne(fl32(x / s)), -127, 127), the symmetric int8
    rule of the dynamic path with the row scale replaced; s = 0 gives zeros."""
    x32 = np.asarray(x32, dtype=np.float32)
    s = np.float32(s)
    if not s > 0:
        return np.zeros(x32.shape, dtype=np.int8)
    return np.clip(np.rint(x32 / s), -127, 127).astype(np.int8)


def quantize_act_int8_asym(x32: np.ndarray):
    """Per-token asymmetric int8: x32 float32 [M, K] -> (codes int8 [M, K],
    scale float32 [M], offset float32 [M]) with x ~ code * scale + offset.

    [ct_w4a8] __init__ carries an input_symmetric flag and [inc_w4a8]
    apply_weights passes the per-token quant op's zero output to the GEMM;
    neither page prints the asymmetric arithmetic. READING: the min/max grid
    of [cpu_int4] quantize_groupwise (scale = (max - min) / (levels - 1),
    codes counted from min, an additive offset in value units) with 256
    levels, in fp32:
        d = fl32(max - min),  scale = fl32(d / 255),
        code = clamp(rne(fl32(fl32(x - min) / scale)), 0, 255) - 128,
        offset = fl32(min + 128 * scale).
    A constant row has scale 0, codes -128 and offset = min (exact). Inputs
    whose fp32 range max - min overflows are outside the reading."""
    x32 = np.asarray(x32, dtype=F32)
    assert np.all(np.isfinite(x32)), "oracle assumes finite activations"
    M, K = x32.shape
    codes = np.full((M, K), -128, dtype=np.int8)
    if K == 0:
        z = np.zeros(M, F32)
        return codes, z, z.copy()
    lo = np.min(x32, axis=1).astype(F32)
    hi = np.max(x32, axis=1).astype(F32)
    d = (hi - lo).astype(F32)
    assert np.all(np.isfinite(d)), "row range overflows fp32"
    scale = (d / F32(255.0)).astype(F32)
    offset = (lo + F32(128.0) * scale).astype(F32)        # 128 * scale is exact
    nz = scale > 0
    if np.any(nz):
        t = (x32[nz] - lo[nz][:, None]).astype(F32)        # fp32, rounded once
        q = (t / scale[nz][:, None]).astype(F32)           # fp32 / fp32, correctly rounded
        codes[nz] = (np.clip(np.rint(q), 0, 255) - 128).astype(np.int8)
    return codes, scale, offset


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


_E4M3_POS = e4m3_decode(np.arange(127, dtype=np.uint8))   # codes 0x00..0x7E, increasing


def e4m3_encode(v32) -> np.ndarray:
    """float32 -> E4M3 code: nearest representable, ties to the even code,
    saturating at 448; the sign bit follows the input's sign bit."""
    v32 = np.asarray(v32, dtype=F32)
    assert np.all(np.isfinite(v32))
    sign = np.signbit(v32).astype(np.uint8) << 7
    a = np.minimum(np.abs(v32.astype(np.float64)), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_E4M3_POS[hi] == a, hi, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_act_fp8(x32: np.ndarray):
    """x32 float32 [T, K] -> (E4M3 codes uint8 [T, K], scale float32 [T])."""
    x32 = np.asarray(x32, dtype=F32)
    assert np.all(np.isfinite(x32))
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], F32)
    scale = (amax / F32(448.0)).astype(F32)
    codes = np.zeros(x32.shape, dtype=np.uint8)
    nz = scale > 0
    if np.any(nz):
        codes[nz] = e4m3_encode(x32[nz] / scale[nz][:, None])
    return codes, scale


# --------------------------------------------------------------------------
# Weight layouts. A 4-bit code q in 0..15 stands for the integer q - 8
# ("uint4b8": unsigned with bias 8; [w4afp8] _repack_signed_int4_to_uint4b8,
# [inc_w4a8] symmetric int4 weights). READING: inside a word the code of the
# lowest K index sits in the lowest nibble ([cpu_int4] byte layout low nibble
# first; [zentorch] notes 8 codes per int32 are the same little-endian byte
# stream as two codes per byte).
# --------------------------------------------------------------------------


def _nibbles_of_words(words: np.ndarray) -> np.ndarray:
    """int32 [..., W] -> uint8 codes [..., 8W], code i of word j at index 8j+i."""
    u = np.asarray(words).view(np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    q = (u[..., None] >> shifts) & np.uint32(0xF)
    return q.reshape(*u.shape[:-1], u.shape[-1] * 8).astype(np.uint8)


def unpack_gptq_kn(qweight: np.ndarray) -> np.ndarray:
    """GPTQ qweight int32 [K/8, N], 8 codes per word along K ([inc_w4a8]:
    the output dim is qweight.shape[1]) -> codes uint8 [K, N]."""
    return _nibbles_of_words(np.ascontiguousarray(np.asarray(qweight).T)).T.copy()


def unpack_ct_nk(w: np.ndarray) -> np.ndarray:
    """compressed-tensors weight_packed int32 [..., N, K/8] packed along the
    input dim ([zentorch] _zentorch_woq_eligible) -> codes uint8 [..., N, K]."""
    return _nibbles_of_words(w)


def unpack_i8_nk(w: np.ndarray) -> np.ndarray:
    """[ct_w4a8] create_weights: weight_packed int8 [N, K], one signed int4
    value per byte -> codes uint8 [N, K] with the zero point 8 (q = v + 8)."""
    v = np.asarray(w, dtype=np.int16)
    assert v.min() >= -8 and v.max() <= 7, "int4 values"
    return (v + 8).astype(np.uint8)


def pack_nibble_bytes(q: np.ndarray) -> np.ndarray:
    """[cpu_int4] pack_nibbles: codes [N, K] -> uint8 [N, K/2], byte j holds
    code 2j in its low nibble and code 2j+1 in its high nibble."""
    q = np.asarray(q).astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibble_bytes(b: np.ndarray) -> np.ndarray:
    """[cpu_int4] unpack_nibbles: uint8 [N, K/2] -> codes uint8 [N, K]."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], b.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = b & 0x0F
    out[:, 1::2] = b >> 4
    return out


def repack_signed_int4_to_uint4b8(b: np.ndarray) -> np.ndarray:
    """[w4afp8] _repack_signed_int4_to_uint4b8: signed int4 codes two per byte
    -> uint4b8 codes eight per int32, by XOR with 0x88 on every byte (adds 8
    mod 16 to each nibble). b: int8/uint8 [..., 4W] -> int32 [..., W]."""
    u = np.ascontiguousarray(np.asarray(b).view(np.uint8)) ^ np.uint8(0x88)
    return u.view(np.int32)


def quantize_groupwise(w: np.ndarray, group: int):
    """[cpu_int4] quantize_groupwise, in float64: per row and group of
    `group` columns, scale = max(max - min, 1e-9) / 15, zero = min + 8*scale,
    q = clamp(round((w - min)/scale), 0, 15); dequantized (q-8)*scale+zero."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if k % group:
        raise ValueError(f"input dim {k} is not a multiple of group size {group}")
    wf = w.reshape(n, k // group, group)
    wmin, wmax = wf.min(axis=-1), wf.max(axis=-1)
    scale = np.maximum(wmax - wmin, 1e-9) / 15.0
    zero = wmin + 8.0 * scale
    q = np.clip(np.rint((wf - wmin[..., None]) / scale[..., None]), 0, 15)
    return q.reshape(n, k).astype(np.uint8), scale, zero


def quantize_groupwise_f32(w32: np.ndarray, group: int):
    """[cpu_int4] quantize_groupwise with its own precision: the page converts
    the weights to float32 (w.float()) and every step is a float32 operation,
    each rounded to nearest even; torch's round_ is half-to-even. Returns codes
    uint8 [N, K], scale and zero float32 [N, K/group]."""
    w = np.asarray(w32, dtype=np.float32)
    n, k = w.shape
    if k % group:
        raise ValueError(f"input dim {k} is not a multiple of group size {group}")
    wf = w.reshape(n, k // group, group)
    wmin, wmax = wf.min(axis=-1), wf.max(axis=-1)
    scale = np.maximum(wmax - wmin, np.float32(1e-9)) / np.float32(15.0)
    zero = wmin + np.float32(8.0) * scale
    q = np.clip(np.rint((wf - wmin[..., None]) / scale[..., None]), np.float32(0), np.float32(15))
    assert scale.dtype == np.float32 and q.dtype == np.float32
    return q.reshape(n, k).astype(np.uint8), scale, zero


def dequantize_groupwise(q, scale, zero, group: int) -> np.ndarray:
    """[cpu_int4] w = (q - 8) * scale + zero, scale/zero per (row, group)."""
    q = np.asarray(q, dtype=np.float64)
    n, k = q.shape
    s = np.repeat(np.asarray(scale, np.float64), group, axis=1)
    z = np.repeat(np.asarray(zero, np.float64), group, axis=1)
    return (q - 8.0) * s + z


def f32_to_bf16_bits(v32) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to the even bf16):
    keep the upper 16 bits, add one unit in their last place when the lower
    16 bits exceed half of it, or equal half of it and the kept part is odd.
    Finite inputs only."""
    u = np.asarray(v32, dtype=F32).view(np.uint32).astype(np.uint64)
    kept = u >> np.uint64(16)
    low = u & np.uint64(0xFFFF)
    up = (low > 0x8000) | ((low == 0x8000) & ((kept & np.uint64(1)) == 1))
    return (kept + up.astype(np.uint64)).astype(np.uint16)


def dequantize_bf16(q, scale_bits, zero_bits, group: int) -> np.ndarray:
    """[cpu_int4] dequantize / _dequantize_halves, the prefill path: the weight
    w = (q - 8) * scale + zero unpacked to a bf16 matrix [N, K] (returned as
    bf16 bit patterns) for the ordinary bf16 GEMM.

    READING: the page hands the bf16 expression to torch.compile, which
    evaluates it in float32 and rounds once, to bf16, when it stores the
    result. So: (q - 8) * scale in float32 (exact: a 4-bit integer times an
    8-bit significand), + zero rounded to float32, then rounded to bf16,
    nearest even. (Evaluated op by op in bf16, each of the two operations
    would round to bf16.)"""
    q = np.asarray(q, dtype=np.uint8)
    n, k = q.shape
    s = np.repeat(bf16_bits_to_f32(scale_bits), group, axis=1)
    z = np.repeat(bf16_bits_to_f32(zero_bits), group, axis=1)
    prod = (q.astype(F32) - F32(8.0)) * s
    w32 = (prod + z).astype(F32)
    assert w32.dtype == F32
    return f32_to_bf16_bits(w32)


def w4a16_prefill_reference(x_bits, w_bytes, scale_bits, zero_bits, group: int) -> np.ndarray:
    """[cpu_int4] _cpu_int4_linear, batches at or above the threshold: the
    bf16 activations times the transposed bf16 weight of dequantize_bf16,
    y [M, N] in float64 (the GEMM itself exact)."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    Wb = bf16_bits_to_f32(dequantize_bf16(unpack_nibble_bytes(w_bytes), scale_bits, zero_bits, group))
    return x @ Wb.astype(np.float64).T


# --------------------------------------------------------------------------
# W4A8 GEMM. [inc_w4a8] apply_weights: int8 codes with per-token scales,
# int4 weights with per-group fp16 scales, bias fused; output in the
# activation dtype. Group -1 means per-channel: a single group spanning the
# input dim ([ct_w4a8] create_weights effective group; [zentorch]
# can_implement). No act-order / g_idx and no zero-point tensor (zero is 8).
# --------------------------------------------------------------------------


def effective_group(group: int, K: int) -> int:
    g = K if group == -1 else group
    if g <= 0 or K % g:
        raise ValueError(f"group {group} does not divide K={K}")
    return g


def group_partials(codes: np.ndarray, q_kn: np.ndarray, group: int) -> np.ndarray:
    """P[m, g, n] = sum_{k in group g} codes[m, k] * (q[k, n] - 8), exact (int64)."""
    M, K = codes.shape
    g_eff = effective_group(group, K)
    G = K // g_eff
    A = codes.astype(np.float64)
    W = q_kn.astype(np.float64) - 8.0
    P = np.empty((M, G, q_kn.shape[1]), dtype=np.int64)
    for g in range(G):
        sl = slice(g * g_eff, (g + 1) * g_eff)
        P[:, g, :] = np.rint(A[:, sl] @ W[sl, :]).astype(np.int64)   # exact integers
    return P


def w4a8_epilogue(P: np.ndarray, a_scale: np.ndarray, scales_gn: np.ndarray,
                  bias: np.ndarray | None = None) -> np.ndarray:
    """y[m, n] = a_scale[m] * sum_g scale[g, n] * P[m, g, n] (+ bias[n]), float64."""
    S = np.asarray(scales_gn, dtype=np.float64)
    y = np.einsum("mgn,gn->mn", P.astype(np.float64), S)
    y *= np.asarray(a_scale, dtype=np.float64)[:, None]
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)[None, :]
    return y


def w4a8_reference(x_bits, x_dtype, qweight, scales_f16, group, bias_bits=None, rows=None):
    """Whole W4A8 forward on the original layouts. Quantization covers every
    row; partials and outputs only `rows` (all rows if None)."""
    x32 = half_bits_to_f32(x_bits, x_dtype)
    codes, a_scale = quantize_act_int8(x32)
    q = unpack_gptq_kn(qweight)
    r = np.arange(codes.shape[0]) if rows is None else np.asarray(rows)
    P = group_partials(codes[r], q, group)
    bias = None if bias_bits is None else half_bits_to_f32(bias_bits, x_dtype)
    y = w4a8_epilogue(P, a_scale[r], np.asarray(scales_f16, dtype=np.float32), bias)
    return dict(codes=codes, a_scale=a_scale, P=P, y=y, rows=r)


def weight_offsets(q_kn: np.ndarray, scales_gn, group: int) -> np.ndarray:
    """C[n] = sum_g scale[g, n] * sum_{k in g} (q[k, n] - 8), float64: what an
    activation offset z contributes to output column n per unit of z, since
    sum_k z * (q[k, n] - 8) * scale[k // g, n] = z * C[n]."""
    K = q_kn.shape[0]
    g_eff = effective_group(group, K)
    S = np.asarray(scales_gn, dtype=np.float64)
    W = (q_kn.astype(np.int64) - 8).reshape(K // g_eff, g_eff, -1).sum(axis=1)   # exact integers
    return (S * W).sum(axis=0)


def w4a8_reference_asym(x_bits, x_dtype, qweight, scales_f16, group, bias_bits=None, rows=None):
    """W4A8 forward with asymmetric per-token activations on the original
    layouts: y = sum_k (code * s + z) * (q - 8) * scale (+ bias)
              = s * sum_g scale * P + z * C[n] (+ bias), float64."""
    x32 = half_bits_to_f32(x_bits, x_dtype)
    codes, a_scale, a_off = quantize_act_int8_asym(x32)
    q = unpack_gptq_kn(qweight)
    r = np.arange(codes.shape[0]) if rows is None else np.asarray(rows)
    P = group_partials(codes[r], q, group)
    S = np.asarray(scales_f16, dtype=np.float32)
    bias = None if bias_bits is None else half_bits_to_f32(bias_bits, x_dtype)
    y = w4a8_epilogue(P, a_scale[r], S, bias)
    y += np.asarray(a_off[r], dtype=np.float64)[:, None] * weight_offsets(q, S, group)[None, :]
    return dict(codes=codes, a_scale=a_scale, a_offset=a_off, P=P, y=y, rows=r)


# --------------------------------------------------------------------------
# Weight-only path on the GPTQ weights ([inc_w4a8] class docstring: the int8
# and the weight-only kernels take bit-identical weights; apply_weights: below
# _MIN_TOKENS_FOR_INT8 tokens the layer runs the weight-only path). The
# activations stay unquantized; the weight of (k, n) is (q - 8) * scale[g, n].
# --------------------------------------------------------------------------


def w4a16_gptq_reference(x_bits, x_dtype, qweight, scales_gn, group, bias_bits=None) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * (q[k, n] - 8) * scale[k // g, n] (+ bias[n]), float64."""
    x = half_bits_to_f32(x_bits, x_dtype).astype(np.float64)
    W = unpack_gptq_kn(qweight).astype(np.float64) - 8.0            # [K, N]
    g = effective_group(group, W.shape[0])
    S = np.repeat(np.asarray(scales_gn, dtype=np.float64), g, axis=0)  # [K, N]
    y = x @ (W * S)
    if bias_bits is not None:
        y += half_bits_to_f32(bias_bits, x_dtype).astype(np.float64)[None, :]
    return y


# --------------------------------------------------------------------------
# W4A16 ([cpu_int4] module docstring and CPUInt4EmbeddingMethod.embedding):
# bf16 activations, weights w = (q - 8) * scale + zero with bf16 scale and
# zero per (output row, group), codes two per byte low nibble first.
# --------------------------------------------------------------------------


def w4a16_reference(x_bits, w_bytes, scale_bits, zero_bits, group: int) -> np.ndarray:
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    q = unpack_nibble_bytes(w_bytes)
    s = bf16_bits_to_f32(scale_bits)
    z = bf16_bits_to_f32(zero_bits)
    W = dequantize_groupwise(q, s, z, group)                     # [N, K] float64
    return x @ W.T


# --------------------------------------------------------------------------
# Routed experts with FP8 activations ([w4afp8] W4AFP8Config: int4 group-128
# expert weights, symmetric, with per-token dynamic FP8 activations). For a
# routed row r of expert e carrying token t:
#   y[r, n] = s_a[t] * sum_g scale[e, g, n] * sum_{k in g} dec(a8[t, k]) * (q[e, n, k] - 8)
# READING: rows are grouped by expert (expert_offsets prefix sums), the
# output is in that row order; no routing weights, no combine.
# --------------------------------------------------------------------------


def grouped_fp8_reference(a8, a_scale, row_token, expert_offsets, w_enk, scales_egn,
                          group: int, rows=None) -> np.ndarray:
    """Returns y float64 for `rows` (default: all routed rows), in that order."""
    E = len(expert_offsets) - 1
    N = w_enk.shape[1]
    K = w_enk.shape[2] * 8
    g_eff = effective_group(group, K)
    G = K // g_eff
    R = int(expert_offsets[-1])
    rows = np.arange(R) if rows is None else np.asarray(rows)
    expert_of_row = np.searchsorted(np.asarray(expert_offsets), rows, side="right") - 1
    y = np.zeros((len(rows), N), dtype=np.float64)
    for e in range(E):
        sel = np.nonzero(expert_of_row == e)[0]
        if sel.size == 0:
            continue
        t = np.asarray(row_token)[rows[sel]]
        A = e4m3_decode(a8[t])                                  # [n_e, K]
        W = unpack_ct_nk(w_enk[e]).astype(np.float64) - 8.0      # [N, K]
        S = np.asarray(scales_egn[e], dtype=np.float64)          # [G, N]
        acc = np.zeros((sel.size, N), dtype=np.float64)
        for g in range(G):
            sl = slice(g * g_eff, (g + 1) * g_eff)
            acc += (A[:, sl] @ W[:, sl].T) * S[g][None, :]       # inner sums exact
        y[sel] = acc * np.asarray(a_scale, np.float64)[t][:, None]
    return y
