"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU (argument
validation runs on the host and enqueues nothing)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(w4\w*)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    from int4_weight_quantized_amd import ops
    if not os.path.exists(ops.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ops.lib()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ("w4a8_quantize_act", "w4a8_gemm", "w4a16_gemm", "w4a16_repack", "w4a8_grouped_gemm", "w4_repack",
                 "w4_repack_bytes", "w4a8_gemm_partials", "w4a16_tiled_gemm", "w4_linear", "w4_linear_workspace_bytes",
                 "w4_quantize_groupwise", "w4a16_embedding", "w4a8_quantize_act_static", "w4a16_dequantize",
                 "w4a8_quantize_act_asym", "w4a8_weight_offsets", "w4a8_gemm_asym",
                 "w4_pack_nibbles", "w4_unpack_nibbles", "w4a16_prefill_gemm", "w4a16_prefill",
                 "w4a16_prefill_workspace_bytes", "w4_linear_noalloc", "w4_fp8_encode_range", "w4_probe_mfma", "w4_last_error",
                 "w4_version"):
        assert must in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert L.w4_version() == 103


def _err(L):
    return L.w4_last_error().decode()


def test_dim_alignment_errors_name_the_sizes(L):
    # both GEMM dims must be multiples of 8; the message names the offender
    rc = L.w4a8_gemm(None, None, None, None, 2, 128, None, None, 1, 16, 256, 200 + 4, None)
    assert rc == -2 and "input K=204" in _err(L)
    rc = L.w4a8_gemm(None, None, None, None, 2, -1, None, None, 1, 16, 260, 256, None)
    assert rc == -2 and "output N=260" in _err(L)


def test_scale_dtype_rule(L):
    # bf16 scales would be misread by an fp16-reading kernel: refused
    rc = L.w4a8_gemm(None, None, None, None, 1, 128, None, None, 1, 16, 256, 256, None)
    assert rc == -4 and "fp16" in _err(L)


def test_group_rules(L):
    assert L.w4a8_gemm(None, None, None, None, 2, 96, None, None, 1, 16, 256, 288, None) == -3
    assert L.w4a8_gemm(None, None, None, None, 2, 128, None, None, 1, 16, 256, 192, None) == -3
    assert L.w4a16_gemm(None, None, None, 48, None, 1, 256, 256, None) == -3
    assert L.w4a16_gemm(None, None, None, 1024, None, 1, 256, 2048, None) == -3
    assert L.w4a8_grouped_gemm(None, 5, None, None, None, None, 4, None, None, 2, 64, None, 1,
                               8, 8, 256, 256, None) == -3


def test_int32_group_limit(L):
    """The int8 kernels sum 16*a*(q-8) over a K-group in int32: per-channel K
    (or a group) above 132096 is refused before anything is launched, with
    the sizes named; 132096 itself passes validation (and then stops at the
    null pointers)."""
    K_bad, K_ok = 132096 + 8, 132096
    rc = L.w4a8_gemm(None, None, None, None, 2, -1, None, None, 1, 16, 256, K_bad, None)
    assert rc == -5 and b"132104" in L.w4_last_error()
    assert L.w4a8_gemm(None, None, None, None, 2, -1, None, None, 1, 16, 256, K_ok, None) == -1
    assert L.w4a8_gemm_partials(None, None, -1, None, 16, 256, K_bad, None) == -5
    assert L.w4a8_gemm(None, None, None, None, 2, 132096 + 64, None, None, 1, 16, 256, 2 * (132096 + 64), None) == -5
    buf = ctypes.create_string_buffer(64)
    ptr = ctypes.c_void_p((ctypes.addressof(buf) + 15) & ~15)      # never dereferenced: validation fails first
    assert L.w4_linear(ptr, 1, ptr, ptr, 2, -1, None, ptr, 16, 256, K_bad, 1, None, 0, None) == -5


def test_output_alignment(L):
    # the GEMM writes 16-byte row segments: a misaligned output is refused
    p = ctypes.c_void_p
    rc = L.w4a8_gemm(p(256), p(256), p(256), p(256), 2, 128, None, p(256 + 2), 1, 16, 256, 256, None)
    assert rc == -2 and "out must be 16-byte aligned" in _err(L)


def test_null_and_negative(L):
    assert L.w4a8_gemm(None, None, None, None, 2, 128, None, None, 1, 16, 256, 256, None) == -1
    assert L.w4a8_quantize_act(None, 1, -1, 256, 256, None, 4, None, None, 0, None) == -1
    assert L.w4a8_gemm(None, None, None, None, 2, 128, None, None, 1, 16, 256, 0, None) == -1


def test_empty_inputs_are_noops(L):
    # M == 0 (or N == 0) enqueues nothing and succeeds even with null buffers
    assert L.w4a8_gemm(None, None, None, None, 2, 128, None, None, 1, 0, 256, 256, None) == 0
    assert L.w4a8_quantize_act(None, 1, 0, 256, 256, None, 4, None, None, 0, None) == 0
    assert L.w4a16_gemm(None, None, None, 64, None, 0, 256, 256, None) == 0


def test_decode_batch_limit(L):
    assert L.w4a16_gemm(None, None, None, 64, None, 17, 256, 256, None) == -5


def test_w4a16_repack_bytes(L):
    wb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.w4a16_repack_bytes(4096, 14336, 64, ctypes.byref(wb), ctypes.byref(sb)) == 0
    assert wb.value == 14336 * 4096 // 2 and sb.value == 14336 * 64 * 4
    assert L.w4a16_repack_bytes(192, 24, 64, ctypes.byref(wb), ctypes.byref(sb)) == 0
    assert wb.value == 2 * 1 * 4096 and sb.value == 2 * 1 * 512      # 16-row tiles x 512-wide windows


def test_repack_bytes(L):
    n = ctypes.c_size_t()
    assert L.w4_repack_bytes(4096, 14336, ctypes.byref(n)) == 0
    assert n.value == 4096 * 14336 // 2
    assert L.w4_repack_bytes(200, 8, ctypes.byref(n)) == 0
    assert n.value == 2 * 1 * 8192               # padded to 128 x 128 tiles


def test_linear_workspace_and_dispatch_checks(L):
    n = ctypes.c_size_t()
    r256 = lambda b: (b + 255) // 256 * 256
    assert L.w4_linear_workspace_bytes(10, 14336, 4096, 128, 0, ctypes.byref(n)) == 0 and n.value == 0   # weight-only
    # 64 rows, group 128: 112 tiles -> K split in 4 (fp32 partial tiles after codes and scales)
    assert L.w4_linear_workspace_bytes(64, 14336, 4096, 128, 0, ctypes.byref(n)) == 0
    assert n.value == 64 * 4096 + r256(64 * 4) + 4 * 64 * 14336 * 4
    # group 64 never splits; 4096 rows fill the chip
    assert L.w4_linear_workspace_bytes(64, 14336, 4096, 64, 0, ctypes.byref(n)) == 0
    assert n.value == 64 * 4096 + r256(64 * 4)
    assert L.w4_linear_workspace_bytes(4096, 14336, 4096, 128, 0, ctypes.byref(n)) == 0
    assert n.value == 4096 * 4096 + r256(4096 * 4)
    assert L.w4_linear_workspace_bytes(100, 200, 256, 128, 0, ctypes.byref(n)) == 0   # K = 2 steps: no split
    assert n.value == r256(100 * 256) + r256(100 * 4)
    assert L.w4_linear_workspace_bytes(64, 14336, 4096, 128, 65, ctypes.byref(n)) == 0 and n.value == 0
    p = ctypes.c_void_p
    # too small a workspace for the int8 path is refused before any launch
    rc = L.w4_linear(p(256), 1, p(256), p(256), 2, 128, None, p(256), 64, 256, 4096, 0, None, 0, None)
    assert rc == -1 and "workspace" in _err(L)
    # the weight-only kernel takes at most 16 rows; fp16 scales only
    assert L.w4a16_tiled_gemm(p(256), 1, p(256), p(256), 2, 128, None, p(256), 17, 256, 4096, None) == -5
    assert L.w4a16_tiled_gemm(p(256), 1, p(256), p(256), 1, 128, None, p(256), 4, 256, 4096, None) == -4
    assert L.w4a16_tiled_gemm(p(256), 1, p(256), p(256), 2, 96, None, p(256), 4, 256, 4096, None) == -3


def test_asym_entry_points_validate(L):
    """Asymmetric activations: argument checks on the host, before any launch."""
    assert L.w4a8_quantize_act_asym(None, 1, 4, 12, 12, None, None, None, None) == -2        # K % 8
    assert L.w4a8_quantize_act_asym(None, 7, 4, 16, 16, None, None, None, None) == -4        # dtype
    assert L.w4a8_quantize_act_asym(None, 1, 4, 16, 16, None, None, None, None) == -1        # null
    assert L.w4a8_quantize_act_asym(None, 1, 0, 16, 16, None, None, None, None) == 0         # empty
    assert L.w4a8_weight_offsets(None, None, 1, 128, 256, 256, None, None) == -4             # bf16 scales
    assert L.w4a8_weight_offsets(None, None, 2, 96, 288, 256, None, None) == -3              # group
    assert L.w4a8_weight_offsets(None, None, 2, 128, 256, 256, None, None) == -1             # null
    assert L.w4a8_gemm_asym(None, None, None, None, None, 2, 128, None, None, None, 1, 16, 256, 256, None) == -1
    assert L.w4a8_gemm_asym(None, None, None, None, None, 1, 128, None, None, None, 1, 16, 256, 256, None) == -4
    assert L.w4a8_gemm_asym(None, None, None, None, None, 2, 96, None, None, None, 1, 16, 256, 288, None) == -3
    assert L.w4a8_gemm_asym(None, None, None, None, None, 2, 128, None, None, None, 1, 0, 256, 256, None) == 0


def test_asym_int32_group_limit(L):
    """Asymmetric codes reach -128, so the asymmetric GEMM's largest K-group
    is 131071 (16 * 128 * 8 * g < 2^31), below the symmetric 132096."""
    K_bad = 131072
    assert L.w4a8_gemm_asym(None, None, None, None, None, 2, -1, None, None, None, 1, 16, 256, K_bad, None) == -5
    assert b"131071" in L.w4_last_error()
    assert L.w4a8_gemm_asym(None, None, None, None, None, 2, -1, None, None, None, 1, 16, 256, K_bad - 8, None) == -1
    # the symmetric GEMM still takes that K
    assert L.w4a8_gemm(None, None, None, None, 2, -1, None, None, 1, 16, 256, K_bad, None) == -1


def test_nibble_entry_points_validate(L):
    p = ctypes.c_void_p
    for fn in (L.w4_pack_nibbles, L.w4_unpack_nibbles):
        assert fn(p(256), 4, 7, p(256), None) == -2                  # K odd
        assert fn(p(256), -1, 8, p(256), None) == -1                 # negative
        assert fn(None, 4, 8, p(256), None) == -1                    # null
        assert fn(p(256 + 8), 4, 8, p(256), None) == -2              # misaligned
        assert fn(None, 0, 8, None, None) == 0 and fn(None, 4, 0, None, None) == 0   # empty
        assert fn(p(256), 1 << 30, 1 << 12, p(256), None) == -5      # too large


def test_fp8_encode_range_validates(L):
    p = ctypes.c_void_p
    assert L.w4_fp8_encode_range(0, -8, p(256), None) == -1          # negative
    assert L.w4_fp8_encode_range(0, 12, p(256), None) == -2          # not a multiple of 8
    assert L.w4_fp8_encode_range(0xFFFFFFF8, 16, p(256), None) == -1 and "2^32" in _err(L)
    assert L.w4_fp8_encode_range(0, 8, None, None) == -1             # null
    assert L.w4_fp8_encode_range(0, 8, p(260), None) == -2           # misaligned
    assert L.w4_fp8_encode_range(0xFFFFFFFF, 0, None, None) == 0     # empty


def test_probe_mfma_validates(L):
    p = ctypes.c_void_p
    ops_ = ctypes.c_double(0.0)
    assert L.w4_probe_mfma(3, 16, p(256), 1 << 20, ctypes.byref(ops_), None) == -1      # kind
    assert L.w4_probe_mfma(0, 0, p(256), 1 << 20, ctypes.byref(ops_), None) == -1       # iters
    assert L.w4_probe_mfma(0, 16, None, 1 << 20, ctypes.byref(ops_), None) == -1        # null sink
    assert L.w4_probe_mfma(0, 16, p(256), 1 << 10, ctypes.byref(ops_), None) == -1      # small sink
    assert L.w4_probe_mfma(0, 16, p(258), 1 << 20, ctypes.byref(ops_), None) == -2      # misaligned
    assert ops_.value == 0.0                    # nothing set on a refused call


def test_noalloc_scratch_limit(L):
    """w4_linear_noalloc refuses, on the host and before any HIP call, a call
    whose workspace exceeds its 64 MiB scratch array; M == 0 is a no-op."""
    p = ctypes.c_void_p
    rc = L.w4_linear_noalloc(p(256), 1, p(256), p(256), 2, 128, None, p(256), 8192, 256, 8192, 0, None)
    assert rc == -5 and "scratch" in _err(L)
    assert L.w4_linear_noalloc(p(256), 1, p(256), p(256), 1, 128, None, p(256), 64, 256, 4096, 0, None) == -4
    assert L.w4_linear_noalloc(None, 1, None, None, 2, 128, None, None, 0, 256, 4096, 0, None) == 0


def test_prefill_entry_points_validate(L):
    p = ctypes.c_void_p
    n = ctypes.c_size_t()
    assert L.w4a16_prefill_workspace_bytes(14336, 4096, ctypes.byref(n)) == 0 and n.value == 14336 * 4096 * 2
    assert L.w4a16_prefill_gemm(p(256), p(256), p(256), 16, 256, 96, None) == -2        # K % 64
    assert L.w4a16_prefill_gemm(p(256), p(256), p(256), 16, 252, 128, None) == -2       # N % 8
    assert L.w4a16_prefill_gemm(p(256 + 8), p(256), p(256), 16, 256, 128, None) == -2   # alignment
    assert L.w4a16_prefill_gemm(None, p(256), p(256), 16, 256, 128, None) == -1
    assert L.w4a16_prefill_gemm(None, None, None, 0, 256, 128, None) == 0               # empty
    # dequantize + GEMM: group rule, dtype, workspace size, all before any launch
    assert L.w4a16_prefill(p(256), p(256), p(256), None, 1, 96, p(256), 16, 256, 384, p(256), 1 << 20, None) == -3
    assert L.w4a16_prefill(p(256), p(256), p(256), None, 2, 64, p(256), 16, 256, 384, p(256), 1 << 20, None) == -4
    rc = L.w4a16_prefill(p(256), p(256), p(256), None, 1, 64, p(256), 16, 256, 384, p(256), 100, None)
    assert rc == -1 and "workspace" in _err(L)
