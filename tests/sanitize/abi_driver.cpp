// Host driver for the sanitizer build of the C ABI: every call below fails
// validation (or is an empty no-op), so nothing reaches a GPU. AddressSanitizer
// and UndefinedBehaviorSanitizer watch the validation code, the error-message
// formatting (including messages longer than its buffer) and the workspace
// arithmetic.
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/w4.h"

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d (%s)\n", what, got, want, w4_last_error());
    ++failures;
  }
}

int main() {
  void* p = reinterpret_cast<void*>(256);
  void* odd = reinterpret_cast<void*>(258);
  size_t n = 0, wb = 0, sb = 0;
  expect(w4_version() >= 100, 1, "version");
  // quantizer
  expect(w4a8_quantize_act(nullptr, W4_BF16, -1, 256, 256, nullptr, W4_I8, nullptr, nullptr, 0, nullptr), W4_ERR_INVALID, "q neg");
  expect(w4a8_quantize_act(p, 9, 4, 256, 256, p, W4_I8, (float*)p, nullptr, 0, nullptr), W4_ERR_DTYPE, "q dtype");
  expect(w4a8_quantize_act(p, W4_BF16, 4, 250, 256, p, W4_I8, (float*)p, nullptr, 0, nullptr), W4_ERR_ALIGN, "q K");
  expect(w4a8_quantize_act(p, W4_BF16, 4, 256, 128, p, W4_I8, (float*)p, nullptr, 0, nullptr), W4_ERR_ALIGN, "q ldx");
  expect(w4a8_quantize_act(p, W4_BF16, 4, 256, 256, p, W4_I8, (float*)p, (float*)p, 128, nullptr), W4_ERR_DTYPE, "q gsum i8");
  expect(w4a8_quantize_act(p, W4_BF16, 4, 256, 256, p, W4_FP8_E4M3, (float*)p, (float*)p, 96, nullptr), W4_ERR_GROUP, "q group");
  expect(w4a8_quantize_act(odd, W4_BF16, 4, 256, 256, p, W4_I8, (float*)p, nullptr, 0, nullptr), W4_ERR_ALIGN, "q align");
  expect(w4a8_quantize_act(nullptr, W4_BF16, 0, 256, 256, nullptr, W4_I8, nullptr, nullptr, 0, nullptr), W4_OK, "q empty");
  expect(w4a8_quantize_act_static(p, W4_BF16, 4, 256, 256, nullptr, p, W4_I8, (float*)p, nullptr, 0, nullptr), W4_ERR_INVALID, "qs null");
  // repack
  expect(w4_repack_bytes(100, 24, &n), W4_ERR_ALIGN, "rb align");
  expect(w4_repack_bytes(256, 24, nullptr), W4_ERR_INVALID, "rb null");
  expect(w4_repack(p, 7, 256, 256, 1, p, nullptr), W4_ERR_INVALID, "r layout");
  expect(w4_repack(p, W4_LAYOUT_I8_NK, 256, 256, 1, odd, nullptr), W4_ERR_ALIGN, "r align");
  expect(w4_repack(p, W4_LAYOUT_GPTQ_KN, 256, 256, 70000, p, nullptr), W4_ERR_INVALID, "r batch");
  // GEMMs
  expect(w4a8_gemm((const int8_t*)p, (const float*)p, p, p, W4_BF16, 128, nullptr, p, W4_BF16, 4, 256, 256, nullptr), W4_ERR_DTYPE, "g sdt");
  expect(w4a8_gemm((const int8_t*)p, (const float*)p, p, p, W4_F16, 96, nullptr, p, W4_BF16, 4, 256, 288, nullptr), W4_ERR_GROUP, "g group");
  expect(w4a8_gemm((const int8_t*)p, (const float*)p, p, p, W4_F16, 128, nullptr, odd, W4_BF16, 4, 256, 256, nullptr), W4_ERR_ALIGN, "g out");
  expect(w4a8_gemm((const int8_t*)p, (const float*)p, p, p, W4_F16, 128, nullptr, p, W4_BF16, 4, 260, 256, nullptr), W4_ERR_ALIGN, "g N");
  expect(w4a8_gemm_partials(nullptr, nullptr, 128, nullptr, 4, 256, 256, nullptr), W4_ERR_INVALID, "gp null");
  expect(w4a16_repack_bytes(4096, 14336, 48, &wb, &sb), W4_ERR_GROUP, "w16 rb group");
  expect(w4a16_repack_bytes(1 << 20, 1 << 14, 64, &wb, &sb), W4_ERR_UNSUPPORTED, "w16 rb big");
  expect(w4a16_gemm(p, p, p, 64, p, 17, 256, 256, nullptr), W4_ERR_UNSUPPORTED, "w16 M");
  expect(w4a16_repack(nullptr, nullptr, nullptr, W4_F16, 64, 256, 256, nullptr, nullptr, nullptr), W4_ERR_DTYPE, "w16r dt");
  expect(w4a8_grouped_gemm(p, W4_FP8_E4M3, (const float*)p, (const float*)p, (const int32_t*)p, (const int32_t*)p, 4, p, p,
                           W4_F16, 128, p, W4_BF16, 1 << 20, 64, 256, 4096, nullptr), W4_ERR_UNSUPPORTED, "grp T*K");
  expect(w4a8_grouped_gemm(p, W4_I8, (const float*)p, (const float*)p, (const int32_t*)p, (const int32_t*)p, 4, p, p,
                           W4_F16, 128, p, W4_BF16, 8, 64, 256, 4096, nullptr), W4_ERR_DTYPE, "grp dt");
  // weight-only, dispatch, vocab table
  expect(w4a16_tiled_gemm(p, W4_BF16, p, p, W4_F16, 128, nullptr, p, 17, 256, 4096, nullptr), W4_ERR_UNSUPPORTED, "t M");
  expect(w4_linear_workspace_bytes(64, 14336, 4096, 128, 0, &n), W4_OK, "lw");
  expect(n == (size_t)64 * 4096 + 256 + (size_t)4 * 64 * 14336 * 4, 1, "lw size");
  expect(w4_linear(p, W4_BF16, p, p, W4_F16, 128, nullptr, p, 64, 14336, 4096, 0, nullptr, 0, nullptr), W4_ERR_INVALID, "l ws");
  expect(w4_linear(p, W4_BF16, p, p, W4_F16, 128, nullptr, odd, 4, 256, 4096, 0, nullptr, 0, nullptr), W4_ERR_ALIGN, "l out");
  expect(w4_quantize_groupwise(p, W4_BF16, 4, 256, 96, (uint8_t*)p, p, p, W4_F32, nullptr), W4_ERR_GROUP, "qg group");
  expect(w4_quantize_groupwise(p, W4_I8, 4, 256, 64, (uint8_t*)p, p, p, W4_F32, nullptr), W4_ERR_DTYPE, "qg dt");
  expect(w4a16_embedding(nullptr, 4, p, p, 64, 100, 256, p, nullptr), W4_ERR_ALIGN, "emb V");
  expect(w4a16_embedding(nullptr, 4, p, p, 64, 128, 256, p, nullptr), W4_ERR_INVALID, "emb null");
  expect(w4_linear_noalloc(p, W4_BF16, p, p, W4_F16, 128, nullptr, p, 32768, 14336, 4096, 0, nullptr),
         W4_ERR_UNSUPPORTED, "na scratch");
  expect(w4_linear_noalloc(p, W4_BF16, p, p, W4_F16, -1, nullptr, p, 64, 256, 132160, 0, nullptr), W4_ERR_UNSUPPORTED,
         "na group");
  expect(w4_linear_noalloc(p, W4_BF16, p, p, W4_F16, 128, nullptr, odd, 4, 256, 4096, 0, nullptr), W4_ERR_ALIGN,
         "na out");
  expect(w4_linear_noalloc(nullptr, W4_BF16, nullptr, nullptr, W4_F16, 128, nullptr, nullptr, 0, 256, 4096, 0, nullptr),
         W4_OK, "na empty");
  // asymmetric int8 path
  expect(w4a8_quantize_act_asym(p, W4_BF16, 4, 252, 256, (int8_t*)p, (float*)p, (float*)p, nullptr), W4_ERR_ALIGN, "qa K");
  expect(w4a8_quantize_act_asym(p, W4_F32, 4, 256, 256, (int8_t*)p, (float*)p, (float*)p, nullptr), W4_ERR_DTYPE, "qa dt");
  expect(w4a8_quantize_act_asym(p, W4_BF16, 4, 256, 256, (int8_t*)odd, (float*)p, (float*)p, nullptr), W4_ERR_ALIGN,
         "qa codes");
  expect(w4a8_quantize_act_asym(p, W4_BF16, 4, 256, 256, (int8_t*)p, (float*)p, nullptr, nullptr), W4_ERR_INVALID,
         "qa null");
  expect(w4a8_quantize_act_asym(nullptr, W4_BF16, 0, 256, 256, nullptr, nullptr, nullptr, nullptr), W4_OK, "qa empty");
  expect(w4a8_weight_offsets(p, p, W4_BF16, 128, 256, 256, (float*)p, nullptr), W4_ERR_DTYPE, "wo dt");
  expect(w4a8_weight_offsets(p, p, W4_F16, 96, 288, 256, (float*)p, nullptr), W4_ERR_GROUP, "wo group");
  expect(w4a8_weight_offsets(p, p, W4_F16, 128, 256, 256, nullptr, nullptr), W4_ERR_INVALID, "wo null");
  expect(w4a8_weight_offsets(nullptr, nullptr, W4_F16, 128, 256, 0, nullptr, nullptr), W4_OK, "wo empty");
  expect(w4a8_gemm_asym((const int8_t*)p, (const float*)p, (const float*)p, p, p, W4_F32, 128, (const float*)p, nullptr,
                        p, W4_BF16, 4, 256, 256, nullptr), W4_ERR_DTYPE, "ga sdt");
  expect(w4a8_gemm_asym((const int8_t*)p, (const float*)p, (const float*)p, p, p, W4_F16, -1, (const float*)p, nullptr,
                        p, W4_BF16, 4, 256, 131136, nullptr), W4_ERR_UNSUPPORTED, "ga group");
  expect(w4a8_gemm_asym((const int8_t*)p, (const float*)p, nullptr, p, p, W4_F16, 128, (const float*)p, nullptr, p,
                        W4_BF16, 4, 256, 256, nullptr), W4_ERR_INVALID, "ga null");
  expect(w4a8_gemm_asym((const int8_t*)p, (const float*)p, (const float*)p, p, p, W4_F16, 128, (const float*)p, nullptr,
                        odd, W4_F16, 4, 256, 256, nullptr), W4_ERR_ALIGN, "ga out");
  // bf16 weight-only: dequantization and prefill
  expect(w4a16_dequantize((const uint8_t*)p, p, p, W4_F16, 128, 256, 256, p, nullptr), W4_ERR_DTYPE, "dq dt");
  expect(w4a16_dequantize((const uint8_t*)p, p, p, W4_BF16, 96, 288, 256, p, nullptr), W4_ERR_GROUP, "dq group");
  expect(w4a16_dequantize((const uint8_t*)odd, p, p, W4_BF16, 128, 256, 256, p, nullptr), W4_ERR_ALIGN, "dq w");
  expect(w4a16_dequantize(nullptr, nullptr, nullptr, W4_BF16, 128, 256, 0, nullptr, nullptr), W4_OK, "dq empty");
  expect(w4a16_prefill_gemm(p, p, p, 16, 256, 96, nullptr), W4_ERR_ALIGN, "pg K");
  expect(w4a16_prefill_gemm(p, p, p, -1, 256, 256, nullptr), W4_ERR_INVALID, "pg M");
  expect(w4a16_prefill_gemm(p, p, odd, 16, 256, 256, nullptr), W4_ERR_ALIGN, "pg out");
  expect(w4a16_prefill_gemm(nullptr, nullptr, nullptr, 0, 256, 256, nullptr), W4_OK, "pg empty");
  expect(w4a16_prefill_workspace_bytes(14336, 4096, &n), W4_OK, "pw");
  expect(n == (size_t)14336 * 4096 * 2, 1, "pw size");
  expect(w4a16_prefill_workspace_bytes(256, 0, &n), W4_ERR_INVALID, "pw K");
  expect(w4a16_prefill_workspace_bytes(256, 256, nullptr), W4_ERR_INVALID, "pw null");
  expect(w4a16_prefill(p, (const uint8_t*)p, p, p, W4_BF16, 128, p, 16, 256, 4096, p, 4096, nullptr), W4_ERR_INVALID,
         "pf ws");
  expect(w4a16_prefill(p, (const uint8_t*)p, p, p, W4_BF16, 128, p, 16, 256, 4096, odd, (size_t)1 << 21, nullptr),
         W4_ERR_ALIGN, "pf ws align");
  expect(w4a16_prefill(p, (const uint8_t*)p, p, p, W4_F16, 64, p, 16, 256, 4096, p, (size_t)1 << 22, nullptr),
         W4_ERR_DTYPE, "pf dt");
  // FP8 encode test hook
  expect(w4_fp8_encode_range(0, -8, (uint8_t*)p, nullptr), W4_ERR_INVALID, "fe n");
  expect(w4_fp8_encode_range(0, 12, (uint8_t*)p, nullptr), W4_ERR_ALIGN, "fe n8");
  expect(w4_fp8_encode_range(0xFFFFFFF8u, 16, (uint8_t*)p, nullptr), W4_ERR_INVALID, "fe range");
  expect(w4_fp8_encode_range(0, 8, nullptr, nullptr), W4_ERR_INVALID, "fe null");
  expect(w4_fp8_encode_range(0, 8, (uint8_t*)p + 4, nullptr), W4_ERR_ALIGN, "fe align");
  expect(w4_fp8_encode_range(0xFFFFFFFFu, 0, nullptr, nullptr), W4_OK, "fe empty");
  // MFMA peak probe
  double ops = 0.0;
  expect(w4_probe_mfma(3, 16, (int32_t*)p, 1 << 20, &ops, nullptr), W4_ERR_INVALID, "pm kind");
  expect(w4_probe_mfma(0, 0, (int32_t*)p, 1 << 20, &ops, nullptr), W4_ERR_INVALID, "pm iters");
  expect(w4_probe_mfma(0, 16, (int32_t*)p, 16, &ops, nullptr), W4_ERR_INVALID, "pm sink");
  expect(w4_probe_mfma(0, 16, (int32_t*)odd, 1 << 20, &ops, nullptr), W4_ERR_ALIGN, "pm align");
  expect(w4_probe_mfma(0, 16, (int32_t*)p, 1 << 20, nullptr, nullptr), W4_ERR_INVALID, "pm ops");
  // nibble packing
  expect(w4_pack_nibbles((const uint8_t*)p, 4, 255, (uint8_t*)p, nullptr), W4_ERR_ALIGN, "pk K");
  expect(w4_pack_nibbles((const uint8_t*)p, -1, 256, (uint8_t*)p, nullptr), W4_ERR_INVALID, "pk N");
  expect(w4_unpack_nibbles((const uint8_t*)odd, 4, 256, (uint8_t*)p, nullptr), W4_ERR_ALIGN, "upk align");
  expect(w4_unpack_nibbles(nullptr, 0, 256, nullptr, nullptr), W4_OK, "upk empty");
  expect(w4_unpack_nibbles((const uint8_t*)p, 4, 256, nullptr, nullptr), W4_ERR_INVALID, "upk null");
  // the longest message paths: every argument named, sizes at their widest
  expect(w4a8_gemm((const int8_t*)p, (const float*)p, p, p, W4_F16, 128, nullptr, p, W4_BF16, 4,
                   (int64_t)1 << 62 | 4, ((int64_t)1 << 62) | 12, nullptr), W4_ERR_UNSUPPORTED, "g huge");
  if (std::strlen(w4_last_error()) >= 512) { std::printf("FAIL message length\n"); ++failures; }
  return failures ? 1 : 0;
}
