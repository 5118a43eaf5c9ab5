"""GPU property tests: hypothesis-drawn small shapes and seeds against the
oracle, canary-padded output buffers (no write outside the output), and
non-finite activations (unspecified values, but the call succeeds).

Shapes stay small so that the oracle finishes each example in milliseconds;
the example counts are fixed and derandomized so a run is reproducible."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle as O
from int4_weight_quantized_amd import ops
from int4_weight_quantized_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
SETTINGS = settings(max_examples=25, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])


def dev_half(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(DEV)


def close(gpu: torch.Tensor, y64: np.ndarray) -> bool:
    g = gpu.float().cpu().numpy().astype(np.float64)
    return bool(np.all(np.abs(g - y64) <= 1e-3 + 1e-2 * np.abs(y64)))


@st.composite
def w4a8_shapes(draw):
    # 192 and 384: groups that do not divide 256 (a 64- or 128-deep part of
    # a 256-K range can fall in either of two groups)
    group = draw(st.sampled_from([-1, 64, 128, 192, 256, 384]))
    kmul = 64 if group == -1 else group
    K = kmul * draw(st.integers(1, 4)) if group != -1 else 8 * draw(st.integers(1, 80))
    N = 8 * draw(st.integers(1, 40))
    M = draw(st.integers(1, 70))
    return M, K, N, group, draw(st.sampled_from(["bf16", "f16"])), draw(st.booleans()), draw(st.integers(0, 2**31 - 1))


@SETTINGS
@given(w4a8_shapes())
def test_w4a8_layer_random_shapes(shape):
    M, K, N, group, dtype, bias, seed = shape
    d = W.w4a8_inputs(M, K, N, group, dtype, seed=seed, with_bias=bias)
    x = dev_half(d["x"], dtype)
    wt = ops.w4_repack(torch.from_numpy(d["qweight"]).to(DEV), ops.W4_LAYOUT_GPTQ_KN, K, N)
    sc = torch.from_numpy(d["scales"]).to(DEV)
    b = dev_half(d["bias"], dtype) if bias else None
    codes, s, _ = ops.w4a8_quantize_act(x)
    y = ops.w4a8_gemm(codes, s, wt, sc, group, N, out_dtype=x.dtype, bias=b)
    ref = O.w4a8_reference(d["x"], dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"])
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert close(y, ref["y"]), (M, K, N, group, dtype, bias, seed)
    P = ops.w4a8_gemm_partials(codes, wt, group, N)
    assert np.array_equal(P.cpu().numpy().astype(np.int64), ref["P"])


@SETTINGS
@given(w4a8_shapes())
def test_w4a8_asym_random_shapes(shape):
    """Asymmetric activations (shifted so rows are one-signed or skewed):
    codes, scales and offsets bit-exact, outputs within tolerance."""
    M, K, N, group, dtype, bias, seed = shape
    d = W.w4a8_inputs(M, K, N, group, dtype, seed=seed, with_bias=bias)
    shift = np.float32((seed % 7) - 3)
    x32 = O.half_bits_to_f32(d["x"], dtype) + shift
    xb = W.to_half_bits(x32, dtype)
    x = dev_half(xb, dtype)
    wt = ops.w4_repack(torch.from_numpy(d["qweight"]).to(DEV), ops.W4_LAYOUT_GPTQ_KN, K, N)
    sc = torch.from_numpy(d["scales"]).to(DEV)
    b = dev_half(d["bias"], dtype) if bias else None
    codes, s, z = ops.w4a8_quantize_act_asym(x)
    woff = ops.w4a8_weight_offsets(wt, sc, group, K, N)
    y = ops.w4a8_gemm_asym(codes, s, z, wt, sc, group, woff, N, out_dtype=x.dtype, bias=b)
    ref = O.w4a8_reference_asym(xb, dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"])
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(s.cpu().numpy(), ref["a_scale"]) and np.array_equal(z.cpu().numpy(), ref["a_offset"])
    assert close(y, ref["y"]), (M, K, N, group, dtype, bias, seed)


@st.composite
def decode_shapes(draw):
    group = draw(st.sampled_from([64, 128, 256, 512]))
    K = group * draw(st.integers(1, 6))
    N = 8 * draw(st.integers(1, 60))
    return draw(st.integers(1, 16)), K, N, group, draw(st.booleans()), draw(st.integers(0, 2**31 - 1))


@SETTINGS
@given(decode_shapes())
def test_w4a16_decode_random_shapes(shape):
    M, K, N, group, zero, seed = shape
    d = W.w4a16_inputs(M, K, N, group, seed=seed)
    wt, stl = ops.w4a16_repack(torch.from_numpy(d["w"]).to(DEV), dev_half(d["scale"], "bf16"),
                               dev_half(d["zero"], "bf16") if zero else None, group)
    y = ops.w4a16_gemm(dev_half(d["x"], "bf16"), wt, stl, group, N)
    zb = d["zero"] if zero else np.zeros_like(d["zero"])
    assert close(y, O.w4a16_reference(d["x"], d["w"], d["scale"], zb, group)), (M, K, N, group, zero, seed)


@SETTINGS
@given(w4a8_shapes())
def test_weight_only_tiled_random_shapes(shape):
    M, K, N, group, dtype, bias, seed = shape
    M = min(M, 16)
    d = W.w4a8_inputs(M, K, N, group, dtype, seed=seed, with_bias=bias)
    wt = ops.w4_repack(torch.from_numpy(d["qweight"]).to(DEV), ops.W4_LAYOUT_GPTQ_KN, K, N)
    sc = torch.from_numpy(d["scales"]).to(DEV)
    b = dev_half(d["bias"], dtype) if bias else None
    y = ops.w4a16_tiled_gemm(dev_half(d["x"], dtype), wt, sc, group, N, bias=b)
    ref = O.w4a16_gptq_reference(d["x"], dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"])
    assert close(y, ref), (M, K, N, group, dtype, bias, seed)


# ------------------------------------------------------------------ canary-padded outputs

PAD = 4096          # bytes of canary on each side (a multiple of 16 keeps the output aligned)


def padded(numel: int, dtype) -> tuple[torch.Tensor, torch.Tensor]:
    """A buffer with PAD canary bytes on both sides of `numel` elements;
    returns (whole uint8 buffer, the output view)."""
    esz = torch.empty((), dtype=dtype).element_size()
    buf = torch.full((2 * PAD + numel * esz,), 0xA5, dtype=torch.uint8, device=DEV)
    return buf, buf[PAD:PAD + numel * esz].view(dtype)


def canaries_intact(buf: torch.Tensor) -> bool:
    return bool((buf[:PAD] == 0xA5).all()) and bool((buf[-PAD:] == 0xA5).all())


@pytest.mark.parametrize("M,K,N,group", [(1, 256, 8, 128), (130, 384, 136, 128), (77, 200, 264, -1), (16, 4096, 1032, 64),
                                         (64, 1024, 264, 128)])
def test_canaries_w4a8_and_weight_only(M, K, N, group):
    d = W.w4a8_inputs(M, K, N, group, "bf16", seed=M + N, with_bias=True)
    x = dev_half(d["x"], "bf16")
    wt = ops.w4_repack(torch.from_numpy(d["qweight"]).to(DEV), ops.W4_LAYOUT_GPTQ_KN, K, N)
    sc = torch.from_numpy(d["scales"]).to(DEV)
    b = dev_half(d["bias"], "bf16")
    cbuf, codes = padded(M * K, torch.int8)
    sbuf, s = padded(M, torch.float32)
    ops.quantize_act_into(x, codes.view(M, K), s)
    ybuf, y = padded(M * N, torch.bfloat16)
    ops.w4a8_gemm(codes.view(M, K), s, wt, sc, group, N, bias=b, out=y.view(M, N))
    lbuf, yl = padded(M * N, torch.bfloat16)
    ops.w4_linear(x, wt, sc, group, N, bias=b, out=yl.view(M, N))          # dispatch (split K when few rows)
    torch.cuda.synchronize()
    assert canaries_intact(cbuf) and canaries_intact(sbuf) and canaries_intact(ybuf) and canaries_intact(lbuf)
    # asymmetric path: codes, scales, offsets, weight offsets and output
    abuf, ac = padded(M * K, torch.int8)
    asbuf, a_s = padded(M, torch.float32)
    azbuf, a_z = padded(M, torch.float32)
    ops.w4a8_quantize_act_asym_into(x, ac.view(M, K), a_s, a_z)
    wobuf, wo = padded(N, torch.float32)
    wo.copy_(ops.w4a8_weight_offsets(wt, sc, group, K, N))
    wo2buf, wo2 = padded(N, torch.float32)
    _check_offsets = ops.lib().w4a8_weight_offsets(ops._ptr(wt), ops._ptr(sc), ops.W4_F16, group, K, N,
                                                  ops._ptr(wo2), ops._stream(None))
    assert _check_offsets == 0
    yabuf, ya = padded(M * N, torch.bfloat16)
    ops.w4a8_gemm_asym(ac.view(M, K), a_s, a_z, wt, sc, group, wo, N, bias=b, out=ya.view(M, N))
    torch.cuda.synchronize()
    assert all(canaries_intact(t) for t in (abuf, asbuf, azbuf, wo2buf, yabuf))
    if M <= 16:
        tbuf, yt = padded(M * N, torch.bfloat16)
        ops.w4a16_tiled_gemm(x, wt, sc, group, N, bias=b, out=yt.view(M, N))
        torch.cuda.synchronize()
        assert canaries_intact(tbuf)


@pytest.mark.parametrize("M,K,N,group", [(1, 4096, 1000, 64), (13, 192, 24, 64), (16, 1536, 72, 512),
                                         (8, 512, 14336, 64), (1, 256, 9000, 128)])
def test_canaries_decode(M, K, N, group):
    d = W.w4a16_inputs(M, K, N, group, seed=M + K)
    wt, stl = ops.w4a16_repack(torch.from_numpy(d["w"]).to(DEV), dev_half(d["scale"], "bf16"),
                               dev_half(d["zero"], "bf16"), group)
    ybuf, y = padded(M * N, torch.bfloat16)
    ops.w4a16_gemm(dev_half(d["x"], "bf16"), wt, stl, group, N, out=y.view(M, N))
    ids = torch.tensor([0, N - 1, 5, -3], dtype=torch.int32, device=DEV)
    ebuf, e = padded(4 * K, torch.bfloat16)
    ops.w4a16_embedding(ids, wt, stl, group, N, K, out=e.view(4, K))
    torch.cuda.synchronize()
    assert canaries_intact(ybuf) and canaries_intact(ebuf)


def test_canaries_grouped():
    d = W.moe_inputs(4, 256, 72, 128, 40, 2, seed=3)
    x = dev_half(d["x"], "bf16")
    a8, s, gs = ops.w4a8_quantize_act(x, "fp8", 128)
    wt = ops.w4_repack(torch.from_numpy(d["w"]).to(DEV), ops.W4_LAYOUT_CT_NK, d["K"], d["N"], batch=d["E"])
    sc = torch.from_numpy(d["scales"]).to(DEV)
    rt = torch.from_numpy(d["row_token"]).to(DEV)
    off = torch.from_numpy(d["expert_offsets"]).to(DEV)
    R = rt.shape[0]
    ybuf, y = padded(R * d["N"], torch.bfloat16)
    ops.w4a8_grouped_gemm(a8, s, gs, rt, off, wt, sc, 128, d["N"], out=y.view(R, d["N"]))
    torch.cuda.synchronize()
    assert canaries_intact(ybuf)


# ------------------------------------------------------------------ non-finite activations

def test_nonfinite_rows_are_accepted():
    """NaN / Inf activations give unspecified values (documented), but the
    calls succeed and the finite rows are still exact."""
    M, K, N, group = 4, 256, 64, 128
    d = W.w4a8_inputs(M, K, N, group, "bf16", seed=9)
    x32 = O.half_bits_to_f32(d["x"], "bf16").copy()
    x32[1, 7] = np.nan
    x32[2, 3] = np.inf
    bits = W.to_half_bits(x32, "bf16")
    x = dev_half(bits, "bf16")
    codes, s, _ = ops.w4a8_quantize_act(x)
    wt = ops.w4_repack(torch.from_numpy(d["qweight"]).to(DEV), ops.W4_LAYOUT_GPTQ_KN, K, N)
    sc = torch.from_numpy(d["scales"]).to(DEV)
    y = ops.w4a8_gemm(codes, s, wt, sc, group, N)
    torch.cuda.synchronize()
    rc, rs = O.quantize_act_int8(x32[[0, 3]])
    assert np.array_equal(codes.cpu().numpy()[[0, 3]], rc) and np.array_equal(s.cpu().numpy()[[0, 3]], rs)
    ref = O.w4a8_reference(bits[[0, 3]], "bf16", d["qweight"], d["scales"], group)["y"]
    assert close(y[[0, 3]], ref)
