"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Bars: activation codes and scales, and the int32 per-group partial sums, are
bit-exact; outputs satisfy |gpu - y| <= 1e-3 + 1e-2 |y| against the oracle's
unrounded float64 result. Full workload sizes run on the GPU exactly as the
benchmark launches them; where the oracle cannot cover every output in
seconds it checks a seeded sample of rows.
"""
import numpy as np
import pytest
import torch

import oracle as O
from int4_weight_quantized_amd import ops
from int4_weight_quantized_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_half(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(gpu: np.ndarray, y64: np.ndarray, ctx: str):
    tol = 1e-3 + 1e-2 * np.abs(y64)
    err = np.abs(gpu - y64)
    bad = err > tol
    assert not bad.any(), (f"{ctx}: {int(bad.sum())} of {bad.size} outside 1e-3+1e-2|y|; "
                           f"worst excess {(err - tol).max():.3e} at {np.unravel_index(np.argmax(err - tol), err.shape)}")


def f32_to_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    return W.to_half_bits(x32, dtype)


# ------------------------------------------------------------------ activation quantization

@pytest.mark.parametrize("name", ["w4a8_tiny", "w4a8_up_proj", "w4a8_down_proj"])
def test_quant_int8_workloads_bit_exact(name):
    d = W.named(name)
    print(f"\n[quant int8] {name} M={d['M']} K={d['K']}", flush=True)
    codes, s, _ = ops.w4a8_quantize_act(dev_half(d["x"], d["x_dtype"]))
    rc, rs = O.quantize_act_int8(O.half_bits_to_f32(d["x"], d["x_dtype"]))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def _edge_rows(K: int, dtype: str, rng) -> np.ndarray:
    x = rng.standard_normal((12, K)).astype(np.float32)
    x[0] = 0.0                                   # all-zero row -> scale 0, codes 0
    x[1] = -0.0
    x[2, :] = 0.0
    x[2, K // 3] = -3.0                           # single nonzero
    x[3] *= 1e4
    x[4] *= 1e-30 if dtype == "bf16" else 1e-3    # tiny (fp32 subnormal scales for bf16)
    x[5, ::2] = -0.0
    x[6] = np.where(np.arange(K) % 2, 127.0, -2.5)   # exact ties when amax = 127
    x[7, :] = 1.0
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K", [8, 24, 200, 4096, 16392])
def test_quant_int8_edges(dtype, K):
    rng = np.random.default_rng(K)
    bits = f32_to_bits(_edge_rows(K, dtype, rng), dtype)
    codes, s, _ = ops.w4a8_quantize_act(dev_half(bits, dtype))
    rc, rs = O.quantize_act_int8(O.half_bits_to_f32(bits, dtype))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def _all_bf16_rows():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f32(bits)
    bits = bits[np.isfinite(v)]
    K = (bits.size // 8) * 8
    bits = bits[:K]
    rows = [bits]
    for amax in (1.0, 448.0, 3.5e4, 1e-20):
        v = O.bf16_bits_to_f32(bits)
        keep = np.where(np.abs(v) <= amax, bits, np.uint16(0))
        row = keep.copy()
        row[0] = W.to_half_bits(np.array([amax], np.float32), "bf16")[0]
        rows.append(row)
    return np.stack(rows)


def test_quant_int8_every_bf16_pattern():
    bits = _all_bf16_rows()
    codes, s, _ = ops.w4a8_quantize_act(dev_half(bits, "bf16"))
    rc, rs = O.quantize_act_int8(O.bf16_bits_to_f32(bits))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quant_fp8_every_bf16_pattern_and_group_sums():
    bits = _all_bf16_rows()
    bits = bits[:, : (bits.shape[1] // 128) * 128]
    codes, s, gs = ops.w4a8_quantize_act(dev_half(bits, "bf16"), "fp8", 128)
    rc, rs = O.quantize_act_fp8(O.bf16_bits_to_f32(bits))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    dec = O.e4m3_decode(rc).reshape(rc.shape[0], -1, 128)
    want = dec.sum(-1)
    scale = np.abs(dec).sum(-1)
    assert np.all(np.abs(gs.cpu().numpy() - want) <= 1e-6 * scale + 1e-30)


@pytest.mark.parametrize("sign", [0, 1])
def test_fp8_encode_every_finite_fp32(sign):
    """The quantizer's fp32 -> E4M3 step (clamp to +-448, hardware conversion)
    on every finite fp32 of one sign, 2^31 - 2^23 inputs: the GPU codes are
    cut into runs of equal code, and the oracle's encoder must give that code
    at both ends of every run; with its code monotone in |v| (a CPU pin) it
    then agrees at every input."""
    first, n = sign << 31, 0x7F800000
    print(f"\n[fp8 encode] sign={sign} patterns=0x{first:08x}..+0x{n:08x}", flush=True)
    codes = ops.w4_fp8_encode_range(first, n, device=DEV)
    starts = (torch.nonzero(codes[1:] != codes[:-1]).flatten() + 1).cpu().numpy()
    starts = np.concatenate([[0], starts]).astype(np.int64)
    ends = np.append(starts[1:] - 1, n - 1)
    run_codes = codes[torch.from_numpy(starts).to(DEV)].cpu().numpy()
    del codes
    assert len(starts) == 127                      # one run per code 0x00..0x7E of the sign
    for a, b, c in zip(starts, ends, run_codes):
        v = (np.array([a, b], dtype=np.uint64) + first).astype(np.uint32).view(np.float32)
        got = O.e4m3_encode(v)
        assert got[0] == c and got[1] == c, (hex(first + int(a)), hex(first + int(b)), hex(int(c)), got)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K", [128, 384, 16512])
def test_quant_fp8_edges(dtype, K):
    rng = np.random.default_rng(K + 1)
    bits = f32_to_bits(_edge_rows(K, dtype, rng), dtype)
    codes, s, gs = ops.w4a8_quantize_act(dev_half(bits, dtype), "fp8", 128)
    rc, rs = O.quantize_act_fp8(O.half_bits_to_f32(bits, dtype))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quant_fp8_moe_activations_bit_exact():
    d = W.named("w4afp8_moe")
    print(f"\n[quant fp8] T={d['T']} K={d['K']}", flush=True)
    codes, s, gs = ops.w4a8_quantize_act(dev_half(d["x"], "bf16"), "fp8", d["group"])
    rc, rs = O.quantize_act_fp8(O.bf16_bits_to_f32(d["x"]))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    dec = O.e4m3_decode(rc).reshape(rc.shape[0], -1, d["group"])
    assert np.all(np.abs(gs.cpu().numpy() - dec.sum(-1)) <= 1e-6 * np.abs(dec).sum(-1) + 1e-30)


# ------------------------------------------------------------------ W4A8 GEMM

def _w4a8_dev(d):
    x = dev_half(d["x"], d["x_dtype"])
    qw = torch.from_numpy(d["qweight"]).to(DEV)
    sc = torch.from_numpy(d["scales"]).to(DEV)
    wt = ops.w4_repack(qw, ops.W4_LAYOUT_GPTQ_KN, d["K"], d["N"])
    return x, wt, sc


EDGE_SHAPES = [  # (M, K, N, group)
    (1, 64, 8, -1), (5, 8, 8, -1), (130, 200, 24, -1), (33, 192, 136, 64),
    (17, 512, 256, 256), (129, 384, 264, 128), (64, 1024, 512, 128), (3, 14336, 16, -1),
    (9, 384, 40, -1), (67, 640, 136, -1), (200, 1408, 264, -1),
    # groups of an odd number of 64-deep chunks: group boundaries fall inside K steps
    (40, 576, 136, 192), (70, 1152, 264, 384), (9, 960, 40, 320), (131, 1920, 136, 640),
]


@pytest.mark.parametrize("M,K,N,group", EDGE_SHAPES)
def test_partials_bit_exact_edges(M, K, N, group):
    d = W.w4a8_inputs(M, K, N, group, "bf16", seed=M * 7 + K + N)
    x, wt, _ = _w4a8_dev(d)
    codes, s, _ = ops.w4a8_quantize_act(x)
    P = ops.w4a8_gemm_partials(codes, wt, group, N)
    ref = O.w4a8_reference(d["x"], "bf16", d["qweight"], d["scales"], group)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(P.cpu().numpy().astype(np.int64), ref["P"])


@pytest.mark.parametrize("name,rows,all_rows", [("w4a8_tiny", None, True), ("w4a8_up_proj", 64, False),
                                                ("w4a8_down_proj", 64, True)])
def test_partials_bit_exact_workloads(name, rows, all_rows):
    """Exact int32 group partials against the oracle on a row sample. With
    all_rows the hook runs on every row, in the block shape the GEMM of that
    size takes (per-channel at M=8192: the 128 x 256 blocks); the up-
    projection's group-128 kernel has one block shape, so its sample runs
    alone."""
    d = W.named(name)
    x, wt, _ = _w4a8_dev(d)
    codes, s, _ = ops.w4a8_quantize_act(x)
    rng = np.random.default_rng(99)
    r = np.arange(d["M"]) if rows is None else np.sort(rng.choice(d["M"], rows, replace=False))
    print(f"\n[partials] {name} rows={len(r)} K={d['K']} N={d['N']}", flush=True)
    rt = torch.from_numpy(r).to(DEV)
    if all_rows:
        P = ops.w4a8_gemm_partials(codes, wt, d["group"], d["N"])[rt]
    else:
        P = ops.w4a8_gemm_partials(codes[rt].contiguous(), wt, d["group"], d["N"])
    rc, rs = O.quantize_act_int8(O.half_bits_to_f32(d["x"][r], d["x_dtype"]))
    Pref = O.group_partials(rc, O.unpack_gptq_kn(d["qweight"]), d["group"])
    assert np.array_equal(P.cpu().numpy().astype(np.int64), Pref)


@pytest.mark.parametrize("M,K,N", [(2051, 200, 3944), (2176, 1024, 4096)])
def test_per_channel_wide_blocks(M, K, N):
    """Per-channel shapes with at least 256 blocks of 128 x 256 (the wide
    kernel): ragged rows, a ragged K step, and a last block whose second
    128-column weight tile lies past N; exact partials and outputs on a row
    sample (first and last rows included)."""
    d = W.w4a8_inputs(M, K, N, -1, "bf16", seed=M + K + N, with_bias=True)
    x, wt, sc = _w4a8_dev(d)
    bias = dev_half(d["bias"], "bf16")
    codes, s, _ = ops.w4a8_quantize_act(x)
    P = ops.w4a8_gemm_partials(codes, wt, -1, N)
    y = ops.w4a8_gemm(codes, s, wt, sc, -1, N, out_dtype=x.dtype, bias=bias)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    r = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 40, replace=False)]))
    ref = O.w4a8_reference(d["x"], "bf16", d["qweight"], d["scales"], -1, bias_bits=d["bias"], rows=r)
    rt = torch.from_numpy(r).to(DEV)
    assert np.array_equal(P[rt].cpu().numpy().astype(np.int64), ref["P"])
    assert_close(to_f64(y[rt]), ref["y"], f"wide per-channel {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N,group", EDGE_SHAPES)
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_w4a8_gemm_edges(M, K, N, group, out_dtype):
    d = W.w4a8_inputs(M, K, N, group, out_dtype, seed=M + K * 3 + N, with_bias=True)
    x, wt, sc = _w4a8_dev(d)
    bias = dev_half(d["bias"], out_dtype)
    codes, s, _ = ops.w4a8_quantize_act(x)
    y = ops.w4a8_gemm(codes, s, wt, sc, group, N, out_dtype=x.dtype, bias=bias)
    ref = O.w4a8_reference(d["x"], out_dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"])
    assert_close(to_f64(y), ref["y"], f"w4a8 {M}x{K}x{N} g{group} {out_dtype}")
    y0 = ops.w4a8_gemm(codes, s, wt, sc, group, N, out_dtype=x.dtype)       # without bias
    ref0 = O.w4a8_epilogue(ref["P"], ref["a_scale"], d["scales"].astype(np.float32))
    assert_close(to_f64(y0), ref0, "no bias")


@pytest.mark.parametrize("name", ["w4a8_tiny", "w4a8_up_proj", "w4a8_down_proj"])
def test_w4a8_linear_workloads(name):
    """The full layer (quantize + GEMM) at the workload's size; oracle on a row sample."""
    d = W.named(name)
    print(f"\n[w4a8 linear] {name} M={d['M']} K={d['K']} N={d['N']} g={d['group']}", flush=True)
    x, wt, sc = _w4a8_dev(d)
    codes, s, _ = ops.w4a8_quantize_act(x)
    y = ops.w4a8_gemm(codes, s, wt, sc, d["group"], d["N"], out_dtype=x.dtype)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.arange(d["M"]) if d["M"] <= 64 else np.sort(rng.choice(d["M"], 48, replace=False))
    ref = O.w4a8_reference(d["x"], d["x_dtype"], d["qweight"], d["scales"], d["group"], rows=rows)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert_close(to_f64(y[torch.from_numpy(rows).to(DEV)]), ref["y"], name)
    assert torch.isfinite(y.float()).all()


def test_repack_layouts_agree():
    """compressed-tensors [N,K/8], signed-int4 bytes and int8 [N,K] give the same tiled weights as GPTQ."""
    K, N = 384, 264
    d = W.w4a8_inputs(8, K, N, 128, "bf16", seed=5)
    qw = d["qweight"]                                          # GPTQ [K/8, N]
    ct = np.ascontiguousarray(qw.T)                            # CT [N, K/8]: same words, transposed
    s4 = (ct.view(np.uint8) ^ np.uint8(0x88)).copy()           # signed int4 bytes [N, K/2]
    t_g = ops.w4_repack(torch.from_numpy(qw).to(DEV), ops.W4_LAYOUT_GPTQ_KN, K, N)
    t_c = ops.w4_repack(torch.from_numpy(ct).to(DEV), ops.W4_LAYOUT_CT_NK, K, N)
    t_s = ops.w4_repack(torch.from_numpy(s4).to(DEV), ops.W4_LAYOUT_S4_NK, K, N)
    i8 = (O.unpack_gptq_kn(qw).T.astype(np.int16) - 8).astype(np.int8)   # int8 [N, K], values -8..7
    assert np.array_equal(O.unpack_i8_nk(i8), O.unpack_gptq_kn(qw).T)
    t_i = ops.w4_repack(torch.from_numpy(np.ascontiguousarray(i8)).to(DEV), ops.W4_LAYOUT_I8_NK, K, N)
    assert torch.equal(t_g, t_c) and torch.equal(t_g, t_s) and torch.equal(t_g, t_i)
    codes = torch.randint(-127, 128, (8, K), dtype=torch.int8, device=DEV)
    P = ops.w4a8_gemm_partials(codes, t_s, 128, N)
    Pref = O.group_partials(codes.cpu().numpy(), O.unpack_gptq_kn(qw), 128)
    assert np.array_equal(P.cpu().numpy().astype(np.int64), Pref)


@pytest.mark.parametrize("N,K", [(1, 2), (3, 30), (16, 64), (37, 1030), (1000, 4096), (5, 8)])
def test_nibble_pack_unpack(N, K):
    """w4_pack_nibbles / w4_unpack_nibbles bit-exact against the oracle's byte
    layout (flat 16-byte chunks plus a byte-wise tail)."""
    rng = np.random.default_rng(N * 31 + K)
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    packed = ops.w4_pack_nibbles(torch.from_numpy(q).to(DEV))
    assert np.array_equal(packed.cpu().numpy(), O.pack_nibble_bytes(q))
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    codes = ops.w4_unpack_nibbles(torch.from_numpy(b).to(DEV))
    assert np.array_equal(codes.cpu().numpy(), O.unpack_nibble_bytes(b))
    assert torch.equal(ops.w4_unpack_nibbles(packed), torch.from_numpy(q).to(DEV))


# ------------------------------------------------------------------ W4A16 decode

def _w4a16_run(d, with_zero=True):
    x = dev_half(d["x"], "bf16")
    w = torch.from_numpy(d["w"]).to(DEV)
    s = dev_half(d["scale"], "bf16")
    z = dev_half(d["zero"], "bf16") if with_zero else None
    wt, st = ops.w4a16_repack(w, s, z, d["group"])
    return ops.w4a16_gemm(x, wt, st, d["group"], d["N"])


@pytest.mark.parametrize("M", [1, 8])
def test_w4a16_decode_workload(M):
    d = W.named("w4a16_decode", M=M)
    print(f"\n[w4a16] M={M} K={d['K']} N={d['N']}", flush=True)
    y = _w4a16_run(d)
    ref = O.w4a16_reference(d["x"], d["w"], d["scale"], d["zero"], d["group"])
    assert_close(to_f64(y), ref, f"w4a16 M={M}")


@pytest.mark.parametrize("M,K,N,group,zero", [
    (16, 64, 8, 64, True), (3, 192, 24, 64, True), (2, 512, 136, 128, True), (1, 256, 40, 256, False),
    (13, 14336, 64, 64, True), (8, 4096, 1000, 64, True), (4, 1536, 72, 512, True), (5, 8192, 4104, 128, True),
    (1, 512, 9000, 64, True), (8, 256, 16392, 128, True), (2, 1024, 7176, 256, False),
    # one row tile per block (M <= 4, K <= 4096): two windows per wave, a
    # partial last window, a wave with no second window, four rows
    (1, 3200, 200, 64, True), (2, 4096, 136, 128, False), (4, 2560, 264, 256, True), (3, 3584, 40, 64, True),
    # two row tiles per block (5 to 8 rows), an odd tile count
    (6, 2048, 264, 128, True), (7, 4096, 40, 256, False), (5, 1536, 1032, 64, True),
    # the one-row-tile kernel's four-wave form over many row tiles (tied-head shapes), a partial last tile
    (3, 2048, 16392, 64, True), (2, 1024, 32776, 128, False), (4, 2048, 8200, 512, True)])
def test_w4a16_edges(M, K, N, group, zero):
    d = W.w4a16_inputs(M, K, N, group, seed=M + K + N)
    y = _w4a16_run(d, with_zero=zero)
    zb = d["zero"] if zero else np.zeros_like(d["zero"])
    ref = O.w4a16_reference(d["x"], d["w"], d["scale"], zb, group)
    assert_close(to_f64(y), ref, f"w4a16 {M}x{K}x{N} g{group}")


# ------------------------------------------------------------------ routed experts (FP8)

def _moe_run(d):
    x = dev_half(d["x"], "bf16")
    a8, s, gs = ops.w4a8_quantize_act(x, "fp8", d["group"])
    w = torch.from_numpy(d["w"]).to(DEV)
    wt = ops.w4_repack(w, ops.W4_LAYOUT_CT_NK, d["K"], d["N"], batch=d["E"])
    sc = torch.from_numpy(d["scales"]).to(DEV)
    rt = torch.from_numpy(d["row_token"]).to(DEV)
    off = torch.from_numpy(d["expert_offsets"]).to(DEV)
    y = ops.w4a8_grouped_gemm(a8, s, gs, rt, off, wt, sc, d["group"], d["N"])
    return a8, s, y


@pytest.mark.parametrize("E,K,N,group,T,topk", [
    (4, 256, 64, 128, 32, 2), (1, 384, 8, 128, 16, 1), (8, 512, 136, 256, 300, 3), (16, 128, 128, 128, 5, 2),
    (2, 1024, 64, 512, 40, 2),       # group 512 (four K steps per group)
    (2, 256, 72, 128, 300, 2)])      # ~300 rows per expert: several row tiles, ragged last tile
def test_grouped_small(E, K, N, group, T, topk):
    d = W.moe_inputs(E, K, N, group, T, topk, seed=E * 100 + T)
    a8, s, y = _moe_run(d)
    rc, rs = O.quantize_act_fp8(O.bf16_bits_to_f32(d["x"]))
    assert np.array_equal(a8.cpu().numpy(), rc) and np.array_equal(s.cpu().numpy(), rs)
    ref = O.grouped_fp8_reference(rc, rs, d["row_token"], d["expert_offsets"], d["w"], d["scales"], group)
    assert_close(to_f64(y), ref, f"grouped E={E} K={K} N={N}")


@pytest.mark.parametrize("counts", [
    (0, 64, 65, 130, 0, 200, 1),     # empty experts between ragged ones
    (63, 64, 128, 129, 192, 193)])   # last row tiles of 63, 64, 128, 1, 64 and 65 rows
def test_grouped_ragged_counts(counts):
    """Expert row counts around the row tile and its halves (the two waves
    of a column half each own 64 rows), empty experts included."""
    counts = np.array(counts)
    d = W.moe_inputs(len(counts), 256, 136, 128, 256, 1, seed=int(counts.sum()))
    rng = np.random.default_rng(12)
    d["row_token"] = rng.integers(0, d["T"], int(counts.sum())).astype(np.int32)
    d["expert_offsets"] = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a8, s, y = _moe_run(d)
    rc, rs = O.quantize_act_fp8(O.bf16_bits_to_f32(d["x"]))
    ref = O.grouped_fp8_reference(rc, rs, d["row_token"], d["expert_offsets"], d["w"], d["scales"], d["group"])
    assert_close(to_f64(y), ref, f"grouped counts={tuple(counts)}")


def test_grouped_moe_workload():
    d = W.named("w4afp8_moe")
    print(f"\n[moe] E={d['E']} T={d['T']} K={d['K']} N={d['N']}", flush=True)
    a8, s, y = _moe_run(d)
    torch.cuda.synchronize()
    rc, rs = O.quantize_act_fp8(O.bf16_bits_to_f32(d["x"]))
    assert np.array_equal(a8.cpu().numpy(), rc)
    off = d["expert_offsets"]
    rng = np.random.default_rng(3)
    rows = []
    for e in range(d["E"]):                                  # every expert: its first and last row, two more
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            rows += [lo, hi - 1] + list(rng.integers(lo, hi, 2))
    last = max(e for e in range(d["E"]) if off[e + 1] > off[e])
    rows += list(range(int(off[last]), int(off[last + 1])))  # every row of the last expert (ragged last tile)
    rows = np.unique(np.array(rows))
    print(f"[moe] checking {rows.size} routed rows of {int(off[-1])}", flush=True)
    ref = O.grouped_fp8_reference(rc, rs, d["row_token"], off, d["w"], d["scales"], d["group"], rows=rows)
    assert_close(to_f64(y[torch.from_numpy(rows).to(DEV)]), ref, "moe sample")
    assert torch.isfinite(y.float()).all()


# ------------------------------------------------------------------ weight-only path on the tiled weights

def _tiled_weights(d):
    wt = ops.w4_repack(torch.from_numpy(d["qweight"]).to(DEV), ops.W4_LAYOUT_GPTQ_KN, d["K"], d["N"])
    sc = torch.from_numpy(np.ascontiguousarray(d["scales"])).to(DEV)
    return wt, sc


@pytest.mark.parametrize("M,K,N,group,dtype,bias", [
    (1, 4096, 14336, 128, "bf16", False), (8, 4096, 14336, 128, "bf16", True), (16, 256, 256, 128, "bf16", False),
    (3, 192, 24, 64, "f16", True), (5, 1024, 264, -1, "bf16", False), (1, 8192, 136, 512, "f16", False),
    (13, 14336, 72, 256, "bf16", True), (2, 200, 40, -1, "f16", False), (16, 4096, 1000, 64, "f16", True),
    (4, 4352, 4104, 128, "bf16", False),
    # groups that do not divide a wave's 256-K range: group boundaries inside it
    (3, 768, 136, 384, "bf16", True), (5, 1152, 264, 192, "f16", False), (1, 1920, 40, 320, "bf16", False),
    (7, 2560, 72, 640, "bf16", True), (16, 4608, 520, 1152, "f16", False), (2, 3072, 264, 768, "bf16", True)])
def test_w4a16_tiled(M, K, N, group, dtype, bias):
    d = W.w4a8_inputs(M, K, N, group, dtype, seed=7 * M + K + N, with_bias=bias)
    print(f"\n[w4a16 tiled] M={M} K={K} N={N} g={group} {dtype} bias={bias}", flush=True)
    wt, sc = _tiled_weights(d)
    x = dev_half(d["x"], dtype)
    b = dev_half(d["bias"], dtype) if bias else None
    y = ops.w4a16_tiled_gemm(x, wt, sc, group, N, bias=b)
    assert y.dtype == x.dtype
    ref = O.w4a16_gptq_reference(d["x"], dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"])
    assert_close(to_f64(y), ref, f"w4a16 tiled {M}x{K}x{N} g{group} {dtype}")


@pytest.mark.parametrize("M,threshold,group,dtype,K", [
    (20, 32, 128, "bf16", 1024), (20, 8, 128, "bf16", 1024), (1, 0, 128, "bf16", 1024), (40, 0, 128, "f16", 1024),
    (40, 0, 64, "bf16", 1024), (300, 0, 128, "bf16", 1024), (33, 0, -1, "f16", 1024),
    # groups 192 and 384 on both sides of the threshold
    (20, 0, 192, "bf16", 1152), (40, 0, 192, "f16", 1152), (9, 0, 384, "f16", 1152), (70, 0, 384, "bf16", 1152)])
def test_w4_linear_dispatch(M, threshold, group, dtype, K):
    """Both sides of the per-call dispatch on the same tiled weights: the
    weight-only path (16 rows per launch) below the threshold, per-token int8
    quantization + W4A8 GEMM from it up (group 128 with few tiles splits K:
    fp32 partial tiles summed by a second kernel)."""
    N = 520
    d = W.w4a8_inputs(M, K, N, group, dtype, seed=M + 101 * threshold, with_bias=True)
    print(f"\n[w4_linear] M={M} threshold={threshold} group={group} {dtype}", flush=True)
    wt, sc = _tiled_weights(d)
    x = dev_half(d["x"], dtype)
    b = dev_half(d["bias"], dtype)
    y = ops.w4_linear(x, wt, sc, group, N, bias=b, min_tokens_int8=threshold)
    assert y.dtype == x.dtype
    t = threshold if threshold > 0 else ops.W4_LINEAR_MIN_TOKENS_INT8
    if M < t:
        ref = O.w4a16_gptq_reference(d["x"], dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"])
    else:
        ref = O.w4a8_reference(d["x"], dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"])["y"]
    assert_close(to_f64(y), ref, f"w4_linear M={M} threshold={threshold}")
    y2 = ops.w4_linear(x, wt, sc, group, N, bias=b, min_tokens_int8=threshold)
    assert torch.equal(y, y2)                                   # reproducible (fixed sum order)


# ------------------------------------------------------------------ vocab table: groupwise quantizer and embedding

def _rne_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("N,K,group,wdt,szdt", [
    (37, 512, 64, "bf16", "f32"), (8, 4096, 128, "f16", "f32"), (16, 1536, 512, "f32", "bf16"), (200, 256, 256, "bf16", "bf16")])
def test_quantize_groupwise(N, K, group, wdt, szdt):
    rng = np.random.default_rng(N * 7 + K)
    w32 = (rng.standard_normal((N, K)) * rng.uniform(0.001, 2.0, (N, 1))).astype(np.float32)
    w32[0, :group] = 1.5                                   # a constant group
    print(f"\n[quantize_groupwise] N={N} K={K} g={group} {wdt} -> {szdt}", flush=True)
    if wdt == "f32":
        wd, wref = torch.from_numpy(w32).to(DEV), w32
    else:
        bits = W.to_half_bits(w32, wdt)
        wd, wref = dev_half(bits, wdt), O.half_bits_to_f32(bits, wdt)
    packed, s, z = ops.w4_quantize_groupwise(wd, group, torch.float32 if szdt == "f32" else torch.bfloat16)
    q, rs, rz = O.quantize_groupwise_f32(wref, group)
    assert np.array_equal(packed.cpu().numpy(), O.pack_nibble_bytes(q))
    if szdt == "f32":
        assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(z.cpu().numpy(), rz)
    else:
        assert np.array_equal(s.view(torch.int16).cpu().numpy().view(np.uint16), _rne_bf16_bits(rs))
        assert np.array_equal(z.view(torch.int16).cpu().numpy().view(np.uint16), _rne_bf16_bits(rz))


@pytest.mark.parametrize("V,K,group,T", [(1000, 2048, 64, 37), (136, 1536, 128, 300), (64, 192, 64, 9)])
def test_embedding_and_tied_head(V, K, group, T):
    """The gather reads the decode head's tiled buffers: rows dequantized as
    (q-8)*scale+zero (to bf16), and the head on the same buffers is the
    W4A16 GEMM; ids outside the table give zero rows."""
    d = W.w4a16_inputs(4, K, V, group, seed=V + K + T)
    print(f"\n[embedding] V={V} K={K} g={group} T={T}", flush=True)
    wt, st = ops.w4a16_repack(torch.from_numpy(d["w"]).to(DEV), dev_half(d["scale"], "bf16"),
                              dev_half(d["zero"], "bf16"), group)
    rng = np.random.default_rng(T)
    ids = rng.integers(0, V, T).astype(np.int32)
    ids[0], ids[-1] = V - 1, 0
    ids[T // 2] = -1
    if T > 2:
        ids[1] = V                                           # outside the table
    emb = ops.w4a16_embedding(torch.from_numpy(ids).to(DEV), wt, st, group, V, K)
    table = O.dequantize_groupwise(O.unpack_nibble_bytes(d["w"]), O.bf16_bits_to_f32(d["scale"]),
                                   O.bf16_bits_to_f32(d["zero"]), group)
    valid = (ids >= 0) & (ids < V)
    ref = np.zeros((T, K))
    ref[valid] = table[ids[valid]]
    got = to_f64(emb)
    assert np.all(got[~valid] == 0.0)
    assert_close(got, ref, f"embedding V={V} K={K}")
    head = ops.w4a16_gemm(dev_half(d["x"], "bf16"), wt, st, group, V)
    assert_close(to_f64(head), O.w4a16_reference(d["x"], d["w"], d["scale"], d["zero"], group), "tied head")


# ------------------------------------------------------------------ static (calibrated) activation scale

@pytest.mark.parametrize("dtype,code", [("bf16", "i8"), ("f16", "i8"), ("bf16", "fp8")])
def test_static_quant_and_gemm(dtype, code):
    M, K, N, group = 40, 1024, 264, 128
    d = W.w4a8_inputs(M, K, N, group, dtype, seed=77, outlier_frac=0.01)
    x32 = O.half_bits_to_f32(d["x"], dtype)
    s_static = np.float32(np.abs(x32).max() / 2 / (127.0 if code == "i8" else 448.0))   # half the range: saturates
    print(f"\n[static quant] {dtype} {code} s={s_static}", flush=True)
    x = dev_half(d["x"], dtype)
    sd = torch.tensor([s_static], dtype=torch.float32, device=DEV)
    codes, scales, gs = ops.w4a8_quantize_act_static(x, sd, code, group_sums_group=128 if code == "fp8" else None)
    assert np.all(scales.cpu().numpy() == s_static)
    if code == "i8":
        rc = O.quantize_act_int8_static(x32, s_static)
        assert np.array_equal(codes.cpu().numpy(), rc)
        assert (np.abs(rc) == 127).sum() > 0                      # some saturated
        wt, sc = _tiled_weights(d)
        y = ops.w4a8_gemm(codes, scales, wt, sc, group, N, out_dtype=x.dtype)
        P = O.group_partials(rc, O.unpack_gptq_kn(d["qweight"]), group)
        ref = O.w4a8_epilogue(P, np.full(M, s_static), np.asarray(d["scales"], dtype=np.float32))
        assert_close(to_f64(y), ref, f"static W4A8 {dtype}")
    else:
        rc = O.e4m3_encode((x32 / s_static).astype(np.float32))
        assert np.array_equal(codes.cpu().numpy(), rc)
        dec = O.e4m3_decode(rc).reshape(M, -1, 128)
        assert np.all(np.abs(gs.cpu().numpy() - dec.sum(-1)) <= 1e-6 * np.abs(dec).sum(-1) + 1e-30)


def test_fp8_static_quotients_near_midpoints():
    """The FP8 conversion at every decision boundary: E4M3 midpoints share 16
    significands across binades (the normal ones (2k+1)/16 above 1, the
    subnormal ones k/8), so a row of signed powers of two divided by a
    calibrated scale s = 1/t, with t one of those significands moved by up to
    four float32 steps, puts quotients within a few steps of every midpoint,
    below the smallest subnormal and past 448. Each code is compared with the
    oracle's encoding of the float32 quotient."""
    sig = [1.0 + (2 * k + 1) / 16.0 for k in range(8)] + [k / 8.0 for k in range(8, 16)]
    e = np.arange(-20, 21)
    row = np.concatenate([np.exp2(e), -np.exp2(e)]).astype(np.float32)
    row = np.concatenate([row, np.zeros((-row.size) % 8, np.float32)])
    xb = O.f32_to_bf16_bits(row[None, :])
    assert np.array_equal(O.bf16_bits_to_f32(xb)[0], row)                     # powers of two: exact in bf16
    x = dev_half(xb, "bf16")
    x32 = O.bf16_bits_to_f32(xb)
    n_checked = 0
    for p in sig:
        for k in range(-4, 5):
            t = np.float32(p) + np.float32(k) * np.spacing(np.float32(p))
            s_static = np.float32(np.float32(1.0) / t)
            sd = torch.tensor([s_static], dtype=torch.float32, device=DEV)
            codes, _, _ = ops.w4a8_quantize_act_static(x, sd, "fp8")
            ref = O.e4m3_encode((x32 / s_static).astype(np.float32))
            got = codes.cpu().numpy()
            assert np.array_equal(got, ref), (p, k, float(s_static), int(np.sum(got != ref)))
            n_checked += row.size
    print(f"\n[fp8 static midpoints] {n_checked} quotients", flush=True)


# ------------------------------------------------------------------ prefill: dequantize once, ordinary GEMM

@pytest.mark.parametrize("N,K,group,zero", [(136, 192, 64, True), (1000, 4096, 128, False), (264, 1536, 512, True)])
def test_w4a16_dequantize(N, K, group, zero):
    """Bit-exact against the oracle's bf16 dequantization (one float32
    evaluation, one rounding to bf16, nearest even)."""
    d = W.w4a16_inputs(4, K, N, group, seed=N + K + group)
    print(f"\n[dequantize] N={N} K={K} g={group} zero={zero}", flush=True)
    z = dev_half(d["zero"], "bf16") if zero else None
    wd = ops.w4a16_dequantize(torch.from_numpy(d["w"]).to(DEV), dev_half(d["scale"], "bf16"), z, group)
    zb = d["zero"] if zero else np.zeros_like(d["zero"])
    ref = O.dequantize_bf16(O.unpack_nibble_bytes(d["w"]), d["scale"], zb, group)
    assert np.array_equal(wd.view(torch.int16).cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("M,N,K", [(1, 8, 64), (37, 264, 192), (256, 256, 64), (300, 520, 1024), (513, 1000, 640),
                                   (1024, 2048, 4096), (64, 14336, 4096),
                                   (4096, 8192, 128), (2100, 8200, 192)])   # these two take 256-column tiles
def test_w4a16_prefill_gemm(M, N, K):
    """The bf16 GEMM alone on random bf16 operands (ragged tiles in M and N,
    K of 1 to 64 steps, both tile widths) against the exact product of the
    same bf16 values (a row sample above 1024 rows)."""
    rng = np.random.default_rng(M * 7 + N + K)
    xb = W.to_half_bits(rng.standard_normal((M, K), dtype=np.float32), "bf16")
    wb = W.to_half_bits((rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.05)), "bf16")
    print(f"\n[prefill gemm] M={M} N={N} K={K}", flush=True)
    y = ops.w4a16_prefill_gemm(dev_half(xb, "bf16"), dev_half(wb, "bf16"))
    rows = np.arange(M) if M <= 1024 else np.unique(np.concatenate(
        [np.random.default_rng(M).choice(M, 64, replace=False), [0, M - 1]]))
    ref = O.bf16_bits_to_f32(xb[rows]).astype(np.float64) @ O.bf16_bits_to_f32(wb).astype(np.float64).T
    assert_close(to_f64(y[torch.from_numpy(rows).to(DEV)]), ref, f"prefill gemm {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,group", [(64, 1000, 4096, 64), (300, 264, 1536, 128), (17, 136, 1024, 512)])
def test_w4a16_prefill_path(M, N, K, group):
    """w4a16_prefill (dequantize to bf16 in the workspace, then the bf16 GEMM)
    against the oracle's prefill reference: the same bf16 weights, exact
    products and sums."""
    d = W.w4a16_inputs(M, K, N, group, seed=M + N)
    print(f"\n[prefill] M={M} N={N} K={K} g={group}", flush=True)
    y = ops.w4a16_prefill(dev_half(d["x"], "bf16"), torch.from_numpy(d["w"]).to(DEV), dev_half(d["scale"], "bf16"),
                          dev_half(d["zero"], "bf16"), group)
    ref = O.w4a16_prefill_reference(d["x"], d["w"], d["scale"], d["zero"], group)
    assert_close(to_f64(y), ref, f"prefill {M}x{N}x{K} g{group}")


def test_w4a16_prefill_workload():
    """The prefill workload at full size (M=4096, K=4096, N=14336, group 64) as
    the benchmark launches it; the oracle on a sample of rows."""
    d = W.named("w4a16_prefill")
    print(f"\n[prefill workload] M={d['M']} N={d['N']} K={d['K']} g={d['group']}", flush=True)
    y = ops.w4a16_prefill(dev_half(d["x"], "bf16"), torch.from_numpy(d["w"]).to(DEV), dev_half(d["scale"], "bf16"),
                          dev_half(d["zero"], "bf16"), d["group"])
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(11).choice(d["M"], 48, replace=False))
    ref = O.w4a16_prefill_reference(d["x"][rows], d["w"], d["scale"], d["zero"], d["group"])
    assert_close(to_f64(y[torch.from_numpy(rows).to(DEV)]), ref, "prefill workload")
    assert torch.isfinite(y.float()).all()


# ------------------------------------------------------------------ asymmetric activations

@pytest.mark.parametrize("name", ["w4a8_tiny", "w4a8_up_proj", "w4a8_down_proj"])
def test_quant_asym_workloads_bit_exact(name):
    d = W.named(name)
    print(f"\n[quant asym] {name} M={d['M']} K={d['K']}", flush=True)
    x = dev_half(d["x"], d["x_dtype"])
    codes, s, z = ops.w4a8_quantize_act_asym(x)
    rc, rs, rz = O.quantize_act_int8_asym(O.half_bits_to_f32(d["x"], d["x_dtype"]))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(z.cpu().numpy(), rz)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K", [8, 72, 4096, 20000])
def test_quant_asym_edges(dtype, K):
    rng = np.random.default_rng(K + (dtype == "f16"))
    M = 37
    x = (rng.standard_normal((M, K)) * rng.uniform(0.01, 50, (M, 1)) + rng.uniform(-20, 20, (M, 1)))
    x[3] = 1.5                                    # constant row
    x[4] = 0.0                                    # all zeros
    x[5, :] = np.abs(x[5, :])                     # one-signed row
    bits = W.to_half_bits(x.astype(np.float32), dtype)
    codes, s, z = ops.w4a8_quantize_act_asym(dev_half(bits, dtype))
    rc, rs, rz = O.quantize_act_int8_asym(O.half_bits_to_f32(bits, dtype))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(z.cpu().numpy(), rz)


ASYM_SHAPES = [(16, 256, 256, 128), (1, 64, 8, -1), (130, 200, 24, -1), (33, 192, 136, 64),
               (129, 384, 264, 128), (64, 1024, 512, 256), (9, 640, 40, -1)]


@pytest.mark.parametrize("M,K,N,group", ASYM_SHAPES)
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_w4a8_asym_gemm(M, K, N, group, out_dtype):
    d = W.w4a8_inputs(M, K, N, group, out_dtype, seed=M + 5 * K + N, with_bias=True)
    x, wt, sc = _w4a8_dev(d)
    # shift the activations so the rows are far from symmetric
    xs = (x.float() + 2.0).to(x.dtype)
    xs_bits = xs.view(torch.int16).cpu().numpy().view(np.uint16)
    codes, s, z = ops.w4a8_quantize_act_asym(xs)
    woff = ops.w4a8_weight_offsets(wt, sc, group, K, N)
    bias = dev_half(d["bias"], out_dtype)
    y = ops.w4a8_gemm_asym(codes, s, z, wt, sc, group, woff, N, out_dtype=xs.dtype, bias=bias)
    ref = O.w4a8_reference_asym(xs_bits, out_dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"])
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    Cref = O.weight_offsets(O.unpack_gptq_kn(d["qweight"]), d["scales"].astype(np.float32), group)
    assert np.allclose(woff.cpu().numpy().astype(np.float64), Cref, rtol=1e-5, atol=1e-5)
    assert_close(to_f64(y), ref["y"], f"w4a8 asym {M}x{K}x{N} g{group} {out_dtype}")


def test_w4a8_asym_per_channel_wide_rows():
    """Asymmetric activations with per-channel weights at a size that takes
    the 128 x 256 blocks (shifted activations, fp16, bias); the oracle on a
    row sample with the first and last rows."""
    M, K, N = 2176, 1024, 4096
    d = W.w4a8_inputs(M, K, N, -1, "f16", seed=31, with_bias=True)
    x, wt, sc = _w4a8_dev(d)
    xs = (x.float() + 1.5).to(x.dtype)
    xs_bits = xs.view(torch.int16).cpu().numpy().view(np.uint16)
    codes, s, z = ops.w4a8_quantize_act_asym(xs)
    woff = ops.w4a8_weight_offsets(wt, sc, -1, K, N)
    bias = dev_half(d["bias"], "f16")
    y = ops.w4a8_gemm_asym(codes, s, z, wt, sc, -1, woff, N, out_dtype=xs.dtype, bias=bias)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(9).choice(M, 30, replace=False)]))
    ref = O.w4a8_reference_asym(xs_bits, "f16", d["qweight"], d["scales"], -1, bias_bits=d["bias"], rows=rows)
    assert np.array_equal(codes.cpu().numpy()[rows], ref["codes"][rows])
    assert_close(to_f64(y[torch.from_numpy(rows).to(DEV)]), ref["y"], "w4a8 asym per-channel wide")


def test_w4a8_asym_up_proj_rows():
    """The up-projection workload with asymmetric activations, at full size;
    the oracle on a row sample."""
    d = W.named("w4a8_up_proj")
    x, wt, sc = _w4a8_dev(d)
    codes, s, z = ops.w4a8_quantize_act_asym(x)
    woff = ops.w4a8_weight_offsets(wt, sc, d["group"], d["K"], d["N"])
    y = ops.w4a8_gemm_asym(codes, s, z, wt, sc, d["group"], woff, d["N"], out_dtype=x.dtype)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(8).choice(d["M"], 32, replace=False))
    ref = O.w4a8_reference_asym(d["x"], d["x_dtype"], d["qweight"], d["scales"], d["group"], rows=rows)
    assert_close(to_f64(y[torch.from_numpy(rows).to(DEV)]), ref["y"], "w4a8 asym up_proj")


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_probe_mfma_runs(kind):
    """The measured-peak loop (measurement support, not a hot-path kernel):
    it runs, reports the op count of its documented shape and writes every
    thread's value."""
    sink = torch.full((1024 * 256,), -7, dtype=torch.int32, device=DEV)
    n_ops = ops.w4_probe_mfma(kind, 3, sink)
    torch.cuda.synchronize()
    k = {0: 64, 1: 128, 2: 32}[kind]
    assert n_ops == 1024 * 4 * 8 * 3 * 2 * 16 * 16 * k
    assert int((sink == -7).sum()) < sink.numel() // 2
