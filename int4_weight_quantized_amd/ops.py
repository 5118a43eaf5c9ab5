"""ctypes binding of libw4.so: one Python function per C entry point, same
names, argument marshalling only (torch tensors -> device pointers, dtype
codes, the current HIP stream). Every step runs in the HIP library; there
is no fallback. A missing library or a failed call raises."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4.so")

W4_BF16, W4_F16, W4_F32, W4_I8, W4_FP8_E4M3 = 1, 2, 3, 4, 5
W4_LAYOUT_GPTQ_KN, W4_LAYOUT_CT_NK, W4_LAYOUT_S4_NK, W4_LAYOUT_I8_NK = 1, 2, 3, 4
W4_LINEAR_MIN_TOKENS_INT8 = 33          # include/w4.h: the library's default dispatch threshold
ERRORS = {0: "OK", -1: "INVALID", -2: "ALIGN", -3: "GROUP", -4: "DTYPE", -5: "UNSUPPORTED", -6: "HIP"}

_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int

_SIGS = {
    "w4a8_quantize_act": [_P, _I, _I64, _I64, _I64, _P, _I, _P, _P, _I64, _P],
    "w4a8_quantize_act_static": [_P, _I, _I64, _I64, _I64, _P, _P, _I, _P, _P, _I64, _P],
    "w4_repack_bytes": [_I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "w4_repack": [_P, _I, _I64, _I64, _I64, _P, _P],
    "w4a8_gemm": [_P, _P, _P, _P, _I, _I64, _P, _P, _I, _I64, _I64, _I64, _P],
    "w4a8_gemm_partials": [_P, _P, _I64, _P, _I64, _I64, _I64, _P],
    "w4a16_repack_bytes": [_I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)],
    "w4a16_repack": [_P, _P, _P, _I, _I64, _I64, _I64, _P, _P, _P],
    "w4a16_gemm": [_P, _P, _P, _I64, _P, _I64, _I64, _I64, _P],
    "w4a8_grouped_gemm": [_P, _I, _P, _P, _P, _P, _I64, _P, _P, _I, _I64, _P, _I, _I64, _I64, _I64, _I64, _P],
    "w4a16_tiled_gemm": [_P, _I, _P, _P, _I, _I64, _P, _P, _I64, _I64, _I64, _P],
    "w4_linear_workspace_bytes": [_I64, _I64, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "w4_linear": [_P, _I, _P, _P, _I, _I64, _P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_size_t, _P],
    "w4_linear_noalloc": [_P, _I, _P, _P, _I, _I64, _P, _P, _I64, _I64, _I64, _I64, _P],
    "w4a16_dequantize": [_P, _P, _P, _I, _I64, _I64, _I64, _P, _P],
    "w4a16_prefill_gemm": [_P, _P, _P, _I64, _I64, _I64, _P],
    "w4a16_prefill_workspace_bytes": [_I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "w4a16_prefill": [_P, _P, _P, _P, _I, _I64, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P],
    "w4_quantize_groupwise": [_P, _I, _I64, _I64, _I64, _P, _P, _P, _I, _P],
    "w4a16_embedding": [_P, _I64, _P, _P, _I64, _I64, _I64, _P, _P],
    "w4a8_quantize_act_asym": [_P, _I, _I64, _I64, _I64, _P, _P, _P, _P],
    "w4a8_weight_offsets": [_P, _P, _I, _I64, _I64, _I64, _P, _P],
    "w4a8_gemm_asym": [_P, _P, _P, _P, _P, _I, _I64, _P, _P, _P, _I, _I64, _I64, _I64, _P],
    "w4_fp8_encode_range": [ctypes.c_uint32, _I64, _P, _P],
    "w4_probe_mfma": [_I, _I64, _P, _I64, ctypes.POINTER(ctypes.c_double), _P],
    "w4_pack_nibbles": [_P, _I64, _I64, _P, _P],
    "w4_unpack_nibbles": [_P, _I64, _I64, _P, _P],
    "w4_last_error": [],
    "w4_version": [],
}


class W4Error(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {ERRORS.get(code, code)} ({code}): {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libw4.so (built in-tree by build.py). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with int4_weight_quantized_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "w4_last_error" else ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise W4Error(fn, rc, lib().w4_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() or None


def _stream(stream=None) -> int | None:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def _half_code(dt) -> int:
    if dt == torch.bfloat16:
        return W4_BF16
    if dt == torch.float16:
        return W4_F16
    raise TypeError(f"unsupported half dtype {dt}")


# ----------------------------------------------------------------- entry points

def w4a8_quantize_act(x: torch.Tensor, code_dtype: str = "i8", group_sums_group: int | None = None,
                      stream=None):
    """x [M, K] bf16/fp16 -> (codes [M, K] int8 or uint8 E4M3 bits, scales fp32 [M],
    group_sums fp32 [M, K/group] or None)."""
    M, K = x.shape
    fp8 = code_dtype == "fp8"
    codes = torch.empty((M, K), dtype=torch.uint8 if fp8 else torch.int8, device=x.device)
    scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    gs = None
    if group_sums_group is not None:
        gs = torch.empty((M, K // group_sums_group), dtype=torch.float32, device=x.device)
    quantize_act_into(x, codes, scales, gs, group_sums_group or 0, fp8, stream)
    return codes, scales, gs


def quantize_act_into(x, codes, scales, group_sums=None, group=0, fp8=False, stream=None):
    M, K = x.shape
    _check("w4a8_quantize_act", lib().w4a8_quantize_act(
        _ptr(x), _half_code(x.dtype), M, K, K, _ptr(codes), W4_FP8_E4M3 if fp8 else W4_I8,
        _ptr(scales), _ptr(group_sums), group, _stream(stream)))


def w4a8_quantize_act_static(x: torch.Tensor, static_scale: torch.Tensor, code_dtype: str = "i8",
                             group_sums_group: int | None = None, stream=None):
    """As w4a8_quantize_act with a calibrated per-tensor scale (device fp32 tensor of one element)."""
    M, K = x.shape
    fp8 = code_dtype == "fp8"
    codes = torch.empty((M, K), dtype=torch.uint8 if fp8 else torch.int8, device=x.device)
    scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    gs = None
    if group_sums_group is not None:
        gs = torch.empty((M, K // group_sums_group), dtype=torch.float32, device=x.device)
    _check("w4a8_quantize_act_static", lib().w4a8_quantize_act_static(
        _ptr(x), _half_code(x.dtype), M, K, K, _ptr(static_scale), _ptr(codes), W4_FP8_E4M3 if fp8 else W4_I8,
        _ptr(scales), _ptr(gs), group_sums_group or 0, _stream(stream)))
    return codes, scales, gs


def w4a8_quantize_act_asym(x: torch.Tensor, stream=None):
    """x [M, K] bf16/fp16 -> (codes int8 [M, K], scales fp32 [M], offsets fp32 [M]),
    x ~ code * scale + offset per row."""
    M, K = x.shape
    codes = torch.empty((M, K), dtype=torch.int8, device=x.device)
    scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    offsets = torch.empty((M,), dtype=torch.float32, device=x.device)
    w4a8_quantize_act_asym_into(x, codes, scales, offsets, stream)
    return codes, scales, offsets


def w4a8_quantize_act_asym_into(x, codes, scales, offsets, stream=None):
    M, K = x.shape
    _check("w4a8_quantize_act_asym", lib().w4a8_quantize_act_asym(
        _ptr(x), _half_code(x.dtype), M, K, K, _ptr(codes), _ptr(scales), _ptr(offsets), _stream(stream)))


def w4a8_weight_offsets(w_tiled, w_scale, group: int, K: int, N: int, stream=None) -> torch.Tensor:
    """fp32 [N]: sum_g w_scale[g, n] * sum_{k in g} (q[k, n] - 8), from the tiled weights."""
    out = torch.empty((N,), dtype=torch.float32, device=w_tiled.device)
    sdt = W4_F16 if w_scale.dtype == torch.float16 else (W4_BF16 if w_scale.dtype == torch.bfloat16 else W4_F32)
    _check("w4a8_weight_offsets", lib().w4a8_weight_offsets(
        _ptr(w_tiled), _ptr(w_scale), sdt, group, K, N, _ptr(out), _stream(stream)))
    return out


def w4a8_gemm_asym(a, a_scale, a_offset, w_tiled, w_scale, group: int, w_offsets, N: int,
                   out_dtype=torch.bfloat16, bias=None, out=None, stream=None):
    M, K = a.shape
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    sdt = W4_F16 if w_scale.dtype == torch.float16 else (W4_BF16 if w_scale.dtype == torch.bfloat16 else W4_F32)
    _check("w4a8_gemm_asym", lib().w4a8_gemm_asym(
        _ptr(a), _ptr(a_scale), _ptr(a_offset), _ptr(w_tiled), _ptr(w_scale), sdt, group, _ptr(w_offsets),
        _ptr(bias), _ptr(out), _half_code(out.dtype), M, N, K, _stream(stream)))
    return out


def w4_repack_bytes(K: int, N: int) -> int:
    n = ctypes.c_size_t(0)
    _check("w4_repack_bytes", lib().w4_repack_bytes(K, N, ctypes.byref(n)))
    return n.value


def w4_repack(src: torch.Tensor, layout: int, K: int, N: int, batch: int = 1, stream=None) -> torch.Tensor:
    """Repack `batch` int4 matrices into the kernel-tiled layout (uint8 buffer)."""
    nbytes = w4_repack_bytes(K, N)
    dst = torch.empty((batch, nbytes), dtype=torch.uint8, device=src.device)
    _check("w4_repack", lib().w4_repack(_ptr(src), layout, K, N, batch, _ptr(dst), _stream(stream)))
    return dst


def w4_fp8_encode_range(first_bits: int, n: int, out=None, device="cuda", stream=None) -> torch.Tensor:
    """E4M3 codes (uint8 [n]) of the fp32 values with bit patterns
    first_bits .. first_bits + n - 1, by the quantizer's own conversion."""
    if out is None:
        out = torch.empty((n,), dtype=torch.uint8, device=device)
    _check("w4_fp8_encode_range", lib().w4_fp8_encode_range(first_bits, n, _ptr(out), _stream(stream)))
    return out


def w4_probe_mfma(kind: int, iters: int, sink: torch.Tensor, stream=None) -> float:
    """Launch the pure-MFMA loop (0 int8, 1 fp8, 2 bf16); returns its op count."""
    ops_ = ctypes.c_double(0.0)
    _check("w4_probe_mfma", lib().w4_probe_mfma(kind, iters, _ptr(sink), sink.numel(), ctypes.byref(ops_),
                                                _stream(stream)))
    return ops_.value


def w4_pack_nibbles(codes: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """codes uint8 [N, K] (0..15) -> uint8 [N, K/2], low nibble first."""
    N, K = codes.shape
    if out is None:
        out = torch.empty((N, K // 2), dtype=torch.uint8, device=codes.device)
    _check("w4_pack_nibbles", lib().w4_pack_nibbles(_ptr(codes), N, K, _ptr(out), _stream(stream)))
    return out


def w4_unpack_nibbles(packed: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """uint8 [N, K/2] -> codes uint8 [N, K]."""
    N, K = packed.shape[0], packed.shape[1] * 2
    if out is None:
        out = torch.empty((N, K), dtype=torch.uint8, device=packed.device)
    _check("w4_unpack_nibbles", lib().w4_unpack_nibbles(_ptr(packed), N, K, _ptr(out), _stream(stream)))
    return out


def w4a8_gemm(a, a_scale, w_tiled, w_scale, group: int, N: int, out_dtype=torch.bfloat16, bias=None,
              out=None, stream=None):
    M, K = a.shape
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    sdt = W4_F16 if w_scale.dtype == torch.float16 else (W4_BF16 if w_scale.dtype == torch.bfloat16 else W4_F32)
    _check("w4a8_gemm", lib().w4a8_gemm(
        _ptr(a), _ptr(a_scale), _ptr(w_tiled), _ptr(w_scale), sdt, group, _ptr(bias), _ptr(out),
        _half_code(out.dtype), M, N, K, _stream(stream)))
    return out


def w4a8_gemm_partials(a, w_tiled, group: int, N: int, stream=None):
    M, K = a.shape
    G = 1 if group == -1 else K // group
    P = torch.empty((M, G, N), dtype=torch.int32, device=a.device)
    _check("w4a8_gemm_partials", lib().w4a8_gemm_partials(
        _ptr(a), _ptr(w_tiled), group, _ptr(P), M, N, K, _stream(stream)))
    return P


def w4a16_repack_bytes(K: int, N: int, group: int):
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("w4a16_repack_bytes", lib().w4a16_repack_bytes(K, N, group, ctypes.byref(wb), ctypes.byref(sb)))
    return wb.value, sb.value


def w4a16_repack(w, scale, zero, group: int, stream=None):
    """Load-time repack of byte-layout weights [N, K/2] with bf16 scale/zero [N, K/group]
    into (w_tiled, sz_tiled) uint8 buffers."""
    N, K = w.shape[0], w.shape[1] * 2
    wb, sb = w4a16_repack_bytes(K, N, group)
    wt = torch.empty((wb,), dtype=torch.uint8, device=w.device)
    st = torch.empty((sb,), dtype=torch.uint8, device=w.device)
    _check("w4a16_repack", lib().w4a16_repack(
        _ptr(w), _ptr(scale), _ptr(zero), _half_code(scale.dtype), group, K, N, _ptr(wt), _ptr(st),
        _stream(stream)))
    return wt, st


def w4a16_gemm(x, w_tiled, sz_tiled, group: int, N: int, out=None, stream=None):
    M, K = x.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check("w4a16_gemm", lib().w4a16_gemm(
        _ptr(x), _ptr(w_tiled), _ptr(sz_tiled), group, _ptr(out), M, N, K, _stream(stream)))
    return out


def w4a8_grouped_gemm(a8, a_scale, a_group_sums, row_token, expert_offsets, w_tiled, w_scale,
                      group: int, N: int, out=None, stream=None):
    T, K = a8.shape
    R = row_token.shape[0]
    E = expert_offsets.shape[0] - 1
    if out is None:
        out = torch.empty((R, N), dtype=torch.bfloat16, device=a8.device)
    _check("w4a8_grouped_gemm", lib().w4a8_grouped_gemm(
        _ptr(a8), W4_FP8_E4M3, _ptr(a_scale), _ptr(a_group_sums), _ptr(row_token), _ptr(expert_offsets),
        E, _ptr(w_tiled), _ptr(w_scale), W4_F16, group, _ptr(out), W4_BF16, T, R, N, K, _stream(stream)))
    return out


def w4a16_tiled_gemm(x, w_tiled, w_scale, group: int, N: int, bias=None, out=None, stream=None):
    """Weight-only path on the w4_repack tiles: x [M <= 16, K] bf16/fp16 -> out [M, N] (x dtype)."""
    M, K = x.shape
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check("w4a16_tiled_gemm", lib().w4a16_tiled_gemm(
        _ptr(x), _half_code(x.dtype), _ptr(w_tiled), _ptr(w_scale), W4_F16 if w_scale.dtype == torch.float16 else W4_BF16,
        group, _ptr(bias), _ptr(out), M, N, K, _stream(stream)))
    return out


def w4_linear_workspace_bytes(M: int, N: int, K: int, group: int, min_tokens_int8: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check("w4_linear_workspace_bytes", lib().w4_linear_workspace_bytes(M, N, K, group, min_tokens_int8,
                                                                        ctypes.byref(n)))
    return n.value


def w4_linear(x, w_tiled, w_scale, group: int, N: int, bias=None, min_tokens_int8: int = 0, out=None,
              workspace=None, stream=None):
    """The layer with its per-call dispatch: int8 path from min_tokens_int8 rows up (<= 0: the library's
    default), weight-only path below. The workspace (uint8, device) is allocated here if not given."""
    M, K = x.shape
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    need = w4_linear_workspace_bytes(M, N, K, group, min_tokens_int8)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    _check("w4_linear", lib().w4_linear(
        _ptr(x), _half_code(x.dtype), _ptr(w_tiled), _ptr(w_scale), W4_F16 if w_scale.dtype == torch.float16 else W4_BF16,
        group, _ptr(bias), _ptr(out), M, N, K, min_tokens_int8, _ptr(workspace) if need else None,
        workspace.numel() if workspace is not None else 0, _stream(stream)))
    return out


W4_LINEAR_NOALLOC_SCRATCH_BYTES = 64 << 20     # include/w4.h


def w4_linear_noalloc(x, w_tiled, w_scale, group: int, N: int, bias=None, min_tokens_int8: int = 0, out=None,
                      stream=None):
    """w4_linear with the library's own device scratch (no workspace argument)."""
    M, K = x.shape
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check("w4_linear_noalloc", lib().w4_linear_noalloc(
        _ptr(x), _half_code(x.dtype), _ptr(w_tiled), _ptr(w_scale), W4_F16, group, _ptr(bias), _ptr(out), M, N, K,
        min_tokens_int8, _stream(stream)))
    return out


def w4a16_dequantize(w, scale, zero, group: int, out=None, stream=None):
    """Row-major int4 bytes [N, K/2] with bf16 scale/zero [N, K/group] -> bf16 weights [N, K]."""
    N, K = w.shape[0], w.shape[1] * 2
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=w.device)
    _check("w4a16_dequantize", lib().w4a16_dequantize(
        _ptr(w), _ptr(scale), _ptr(zero), _half_code(scale.dtype), group, K, N, _ptr(out), _stream(stream)))
    return out


def w4_quantize_groupwise(w, group: int, sz_dtype=torch.float32, stream=None):
    """w [N, K] bf16/fp16/fp32 -> (packed uint8 [N, K/2], scale [N, K/group], zero [N, K/group])."""
    N, K = w.shape
    wdt = {torch.bfloat16: W4_BF16, torch.float16: W4_F16, torch.float32: W4_F32}[w.dtype]
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    scale = torch.empty((N, K // group), dtype=sz_dtype, device=w.device)
    zero = torch.empty_like(scale)
    _check("w4_quantize_groupwise", lib().w4_quantize_groupwise(
        _ptr(w), wdt, N, K, group, _ptr(packed), _ptr(scale), _ptr(zero),
        W4_F32 if sz_dtype == torch.float32 else W4_BF16, _stream(stream)))
    return packed, scale, zero


def w4a16_embedding(ids, w_tiled, sz_tiled, group: int, V: int, K: int, out=None, stream=None):
    """ids int32 [T] -> bf16 [T, K]: rows of the tiled [V, K] table, dequantized."""
    T = ids.numel()
    if out is None:
        out = torch.empty((T, K), dtype=torch.bfloat16, device=ids.device)
    _check("w4a16_embedding", lib().w4a16_embedding(
        _ptr(ids), T, _ptr(w_tiled), _ptr(sz_tiled), group, V, K, _ptr(out), _stream(stream)))
    return out


def w4_version() -> int:
    return lib().w4_version()


def w4a16_prefill_gemm(x, w, out=None, stream=None):
    """bf16 x [M, K] times bf16 w [N, K] transposed -> bf16 [M, N]."""
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check("w4a16_prefill_gemm", lib().w4a16_prefill_gemm(_ptr(x), _ptr(w), _ptr(out), M, N, K, _stream(stream)))
    return out


def w4a16_prefill_workspace_bytes(N: int, K: int) -> int:
    n = ctypes.c_size_t(0)
    _check("w4a16_prefill_workspace_bytes", lib().w4a16_prefill_workspace_bytes(N, K, ctypes.byref(n)))
    return n.value


def w4a16_prefill(x, w, scale, zero, group: int, out=None, workspace=None, stream=None):
    """The W4A16 prefill path: dequantize the byte-layout weights [N, K/2] to bf16 (in the workspace) and
    run the bf16 GEMM. The workspace (uint8, device) is allocated here if not given."""
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    need = w4a16_prefill_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    _check("w4a16_prefill", lib().w4a16_prefill(
        _ptr(x), _ptr(w), _ptr(scale), _ptr(zero), _half_code(scale.dtype), group, _ptr(out), M, N, K,
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out
