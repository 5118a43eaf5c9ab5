// C ABI of libw4.so (declared in include/w4.h): argument validation, error
// reporting and kernel launches. Validation runs entirely on the host and
// touches no HIP API, so a rejected call enqueues nothing.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/w4.h"
#include "w4_device.h"

namespace w4 {
hipError_t launch_quant_act(const void* x, bool bf16, int64_t M, int64_t K, int64_t ldx, void* codes,
                            bool fp8, float* scales, float* gsums, int group, hipStream_t stream,
                            const float* static_scale = nullptr);
size_t tiled_bytes(int64_t K, int64_t N);
hipError_t launch_repack(const void* src, int layout, int64_t K, int64_t N, int64_t batch, void* dst,
                         hipStream_t stream);
hipError_t launch_w4a8_gemm(const int8_t* a, const float* a_scale, const void* w_tiled, const void* w_scale,
                            int64_t group, const void* bias, void* out, bool out_bf16, int32_t* partials,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream,
                            const float* a_off = nullptr, const float* w_off = nullptr);
hipError_t launch_quant_act_asym(const void* x, bool bf16, int64_t M, int64_t K, int64_t ldx, void* codes,
                                 float* scales, float* offsets, hipStream_t stream);
hipError_t launch_fp8_encode_range(uint32_t first, int64_t n, uint8_t* codes, hipStream_t stream);
double probe_mfma_ops(int kind, int64_t iters);
int64_t probe_sink_elems();
hipError_t launch_probe_mfma(int kind, int64_t iters, int32_t* sink, hipStream_t stream);
hipError_t launch_weight_offsets(const void* w_tiled, const void* w_scale, int64_t group, int64_t K, int64_t N,
                                 float* out, hipStream_t stream);
void w4a16_tiled_bytes(int64_t K, int64_t N, size_t* wbytes, size_t* szbytes);
int w4a8_split_count(int64_t M, int64_t N, int64_t K, int64_t group);
hipError_t launch_w4a8_gemm_split(const int8_t* a, const float* a_scale, const void* w_tiled, const void* w_scale,
                                  const void* bias, void* out, bool out_bf16, int64_t M, int64_t N, int64_t K,
                                  int splits, float* ws, hipStream_t stream);
hipError_t launch_w4a16_repack(const uint8_t* w, const void* scale, const void* zero, int64_t group, int64_t K,
                               int64_t N, void* w_tiled, void* sz_tiled, hipStream_t stream);
hipError_t launch_w4a16(const void* x, const void* w_tiled, const void* sz_tiled, int64_t group, void* out,
                        int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_w4a16_tiled(const void* x, bool f16, const void* w_tiled, const void* w_scale, int64_t group,
                              const void* bias, void* out, int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_quantize_groupwise(const void* w, int w_dtype_code, int64_t N, int64_t K, int64_t group,
                                     void* packed, void* scale, void* zero, bool sz_bf16, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* w, const void* scale, const void* zero, int64_t group, int64_t N,
                             int64_t K, void* out, hipStream_t stream);
hipError_t launch_embedding(const int32_t* ids, int64_t T, const void* w_tiled, const void* sz_tiled, int64_t group,
                            int64_t V, int64_t K, void* out, hipStream_t stream);
hipError_t launch_bf16_gemm_nt(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream);
hipError_t launch_nibbles(const uint8_t* src, uint8_t* dst, int64_t N, int64_t K, bool pack, hipStream_t stream);
hipError_t launch_grouped_fp8(const void* a, const float* a_scale, const float* gsum, const int32_t* row_token,
                              const int32_t* offsets, int64_t E, const void* w_tiled, size_t w_bytes_per_expert,
                              const void* w_scale, int64_t group, void* out, int64_t T, int64_t R, int64_t N,
                              int64_t K, hipStream_t stream);
}  // namespace w4

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return W4_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(W4_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;

// Shared checks of the GEMM dimensions: [inc_w4a8] create_weights requires
// both GEMM dims to be multiples of 8 and names the offending sizes.
int check_mnk(const char* fn, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0)
    return fail(W4_ERR_INVALID, "%s: sizes must be M >= 0, N >= 0, K > 0 (got M=%lld N=%lld K=%lld)", fn,
                (long long)M, (long long)N, (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > ((int64_t)1 << 24))
    return fail(W4_ERR_UNSUPPORTED, "%s: sizes too large (M=%lld N=%lld K=%lld)", fn, (long long)M,
                (long long)N, (long long)K);
  if (K % 8 || N % 8) {
    char buf[96] = "";
    if (K % 8) snprintf(buf, sizeof(buf), "input K=%lld", (long long)K);
    if (N % 8)
      snprintf(buf + strlen(buf), sizeof(buf) - strlen(buf), "%soutput N=%lld", (K % 8) ? ", " : "",
               (long long)N);
    return fail(W4_ERR_ALIGN, "%s: in/out sizes must be multiples of 8, got %s (shape K=%lld, N=%lld)", fn, buf,
                (long long)K, (long long)N);
  }
  return W4_OK;
}

}  // namespace

extern "C" {

const char* w4_last_error(void) { return g_err; }

int w4_version(void) { return 103; }

static int quantize_act(const char* fn, const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, void* codes,
                        int code_dtype, float* scales, float* group_sums, int64_t group, const float* static_scale,
                        void* stream) {
  if (M < 0 || K < 0) return fail(W4_ERR_INVALID, "%s: negative size M=%lld K=%lld", fn, (long long)M, (long long)K);
  if (x_dtype != W4_BF16 && x_dtype != W4_F16)
    return fail(W4_ERR_DTYPE, "%s: activations must be bf16 or fp16 (dtype code %d)", fn, x_dtype);
  if (code_dtype != W4_I8 && code_dtype != W4_FP8_E4M3)
    return fail(W4_ERR_DTYPE, "%s: codes must be int8 or fp8 e4m3 (dtype code %d)", fn, code_dtype);
  if (K % 8) return fail(W4_ERR_ALIGN, "%s: K=%lld is not a multiple of 8", fn, (long long)K);
  if (M > kMaxDim || K > ((int64_t)1 << 24))
    return fail(W4_ERR_UNSUPPORTED, "%s: sizes too large (M=%lld K=%lld)", fn, (long long)M, (long long)K);
  if (ldx < K || ldx % 8)
    return fail(W4_ERR_ALIGN, "%s: ldx=%lld must be >= K=%lld and a multiple of 8", fn, (long long)ldx,
                (long long)K);
  if (group_sums) {
    if (code_dtype != W4_FP8_E4M3)
      return fail(W4_ERR_DTYPE, "%s: group sums are produced for fp8 codes only", fn);
    const int64_t gc = group / 8;
    if (group <= 0 || group % 8 || K % group || gc > 64 || (gc & (gc - 1)))
      return fail(W4_ERR_GROUP, "%s: group sums need group in {8,16,...,512} (power of two) dividing K, got %lld "
                  "(K=%lld)", fn, (long long)group, (long long)K);
  }
  if (M == 0) return ok();
  if (!x || !codes || !scales) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(x)) return fail(W4_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(codes) & 7u) != 0) return fail(W4_ERR_ALIGN, "%s: codes must be 8-byte aligned", fn);
  return hip_status(w4::launch_quant_act(x, x_dtype == W4_BF16, M, K, ldx, codes, code_dtype == W4_FP8_E4M3,
                                         scales, group_sums, (int)(group_sums ? group : 8),
                                         static_cast<hipStream_t>(stream), static_scale),
                    fn);
}

int w4a8_quantize_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, void* codes,
                      int code_dtype, float* scales, float* group_sums, int64_t group, void* stream) {
  return quantize_act("w4a8_quantize_act", x, x_dtype, M, K, ldx, codes, code_dtype, scales, group_sums, group,
                      nullptr, stream);
}

int w4a8_quantize_act_static(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             const float* static_scale, void* codes, int code_dtype, float* scales,
                             float* group_sums, int64_t group, void* stream) {
  const char* fn = "w4a8_quantize_act_static";
  if (!static_scale && M > 0) return fail(W4_ERR_INVALID, "%s: null static scale", fn);
  return quantize_act(fn, x, x_dtype, M, K, ldx, codes, code_dtype, scales, group_sums, group, static_scale, stream);
}

int w4_repack_bytes(int64_t K, int64_t N, size_t* bytes) {
  const char* fn = "w4_repack_bytes";
  if (!bytes) return fail(W4_ERR_INVALID, "%s: null output pointer", fn);
  int rc = check_mnk(fn, 0, N, K);
  if (rc) return rc;
  *bytes = w4::tiled_bytes(K, N);
  return ok();
}

int w4_repack(const void* src, int layout, int64_t K, int64_t N, int64_t batch, void* dst, void* stream) {
  const char* fn = "w4_repack";
  int rc = check_mnk(fn, 0, N, K);
  if (rc) return rc;
  if (layout != W4_LAYOUT_GPTQ_KN && layout != W4_LAYOUT_CT_NK && layout != W4_LAYOUT_S4_NK &&
      layout != W4_LAYOUT_I8_NK)
    return fail(W4_ERR_INVALID, "%s: unknown source layout %d", fn, layout);
  if (batch < 0 || batch > 65535) return fail(W4_ERR_INVALID, "%s: batch=%lld out of range", fn, (long long)batch);
  if (batch == 0 || N == 0) return ok();
  if (!src || !dst) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(dst)) return fail(W4_ERR_ALIGN, "%s: dst must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(src) & 3u) != 0) return fail(W4_ERR_ALIGN, "%s: src must be 4-byte aligned", fn);
  return hip_status(w4::launch_repack(src, layout, K, N, batch, dst, static_cast<hipStream_t>(stream)), fn);
}

// The int8 kernels sum 16 * a * (q - 8) over a whole group in int32 (the
// nibble is unpacked as a byte 16 (q - 8)): |sum| <= 16 * 127 * 8 * group,
// below 2^31 for groups of at most 132096 (= K for per-channel weights).
// Asymmetric codes reach -128: |sum| <= 16 * 128 * 8 * group, below 2^31 for
// groups of at most 131071.
constexpr int64_t kMaxInt8Group = 132096;
constexpr int64_t kMaxInt8GroupAsym = 131071;
static int check_int32_range(const char* fn, int64_t group, int64_t K, int64_t max_group = kMaxInt8Group) {
  const int64_t g = group == -1 ? K : group;
  if (g > max_group)
    return fail(W4_ERR_UNSUPPORTED,
                "%s: a K-group of %lld exceeds %lld, the largest whose int32 partial sums cannot overflow", fn,
                (long long)g, (long long)max_group);
  return W4_OK;
}

static int check_gemm(const char* fn, const int8_t* a, const void* w_tiled, int64_t group, int64_t M, int64_t N,
                      int64_t K) {
  int rc = check_mnk(fn, M, N, K);
  if (rc) return rc;
  if (group != -1 && (group <= 0 || group % 64 || K % group))
    return fail(W4_ERR_GROUP, "%s: group size %lld must be -1 (per channel) or a multiple of 64 dividing K=%lld", fn,
                (long long)group, (long long)K);
  rc = check_int32_range(fn, group, K);
  if (rc) return rc;
  if (M == 0 || N == 0) return W4_OK;
  if (!a || !w_tiled) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(w_tiled)) return fail(W4_ERR_ALIGN, "%s: w_tiled must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(a) & 7u) != 0) return fail(W4_ERR_ALIGN, "%s: a must be 8-byte aligned", fn);
  return W4_OK;
}

int w4a8_gemm(const int8_t* a, const float* a_scale, const void* w_tiled, const void* w_scale, int scale_dtype,
              int64_t group, const void* bias, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
              void* stream) {
  const char* fn = "w4a8_gemm";
  if (scale_dtype != W4_F16)
    return fail(W4_ERR_DTYPE, "%s: weight scales must be fp16 (dtype code %d); the int8 kernel reads them as fp16",
                fn, scale_dtype);
  if (out_dtype != W4_BF16 && out_dtype != W4_F16)
    return fail(W4_ERR_DTYPE, "%s: output must be bf16 or fp16 (dtype code %d)", fn, out_dtype);
  int rc = check_gemm(fn, a, w_tiled, group, M, N, K);
  if (rc) return rc;
  if (M == 0 || N == 0) return ok();
  if (!a_scale || !w_scale || !out) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(out)) return fail(W4_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
  return hip_status(w4::launch_w4a8_gemm(a, a_scale, w_tiled, w_scale, group, bias, out, out_dtype == W4_BF16,
                                         nullptr, M, N, K, static_cast<hipStream_t>(stream)),
                    fn);
}

int w4a8_gemm_partials(const int8_t* a, const void* w_tiled, int64_t group, int32_t* partials, int64_t M, int64_t N,
                       int64_t K, void* stream) {
  const char* fn = "w4a8_gemm_partials";
  int rc = check_gemm(fn, a, w_tiled, group, M, N, K);
  if (rc) return rc;
  if (M == 0 || N == 0) return ok();
  if (!partials) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  return hip_status(w4::launch_w4a8_gemm(a, nullptr, w_tiled, nullptr, group, nullptr, nullptr, true, partials, M, N,
                                         K, static_cast<hipStream_t>(stream)),
                    fn);
}

int w4a8_quantize_act_asym(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t* codes,
                           float* scales, float* offsets, void* stream) {
  const char* fn = "w4a8_quantize_act_asym";
  if (M < 0 || K < 0) return fail(W4_ERR_INVALID, "%s: negative size M=%lld K=%lld", fn, (long long)M, (long long)K);
  if (x_dtype != W4_BF16 && x_dtype != W4_F16)
    return fail(W4_ERR_DTYPE, "%s: activations must be bf16 or fp16 (dtype code %d)", fn, x_dtype);
  if (K % 8) return fail(W4_ERR_ALIGN, "%s: K=%lld is not a multiple of 8", fn, (long long)K);
  if (M > kMaxDim || K > ((int64_t)1 << 24))
    return fail(W4_ERR_UNSUPPORTED, "%s: sizes too large (M=%lld K=%lld)", fn, (long long)M, (long long)K);
  if (ldx < K || ldx % 8)
    return fail(W4_ERR_ALIGN, "%s: ldx=%lld must be >= K=%lld and a multiple of 8", fn, (long long)ldx,
                (long long)K);
  if (M == 0) return ok();
  if (!x || !codes || !scales || !offsets) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(x)) return fail(W4_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(codes) & 7u) != 0) return fail(W4_ERR_ALIGN, "%s: codes must be 8-byte aligned", fn);
  return hip_status(w4::launch_quant_act_asym(x, x_dtype == W4_BF16, M, K, ldx, codes, scales, offsets,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

int w4a8_weight_offsets(const void* w_tiled, const void* w_scale, int scale_dtype, int64_t group, int64_t K,
                        int64_t N, float* out, void* stream) {
  const char* fn = "w4a8_weight_offsets";
  if (scale_dtype != W4_F16) return fail(W4_ERR_DTYPE, "%s: weight scales must be fp16 (dtype code %d)", fn, scale_dtype);
  int rc = check_mnk(fn, 0, N, K);
  if (rc) return rc;
  if (group != -1 && (group <= 0 || group % 64 || K % group))
    return fail(W4_ERR_GROUP, "%s: group size %lld must be -1 (per channel) or a multiple of 64 dividing K=%lld", fn,
                (long long)group, (long long)K);
  if (N == 0) return ok();
  if (!w_tiled || !w_scale || !out) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(w_tiled)) return fail(W4_ERR_ALIGN, "%s: w_tiled must be 16-byte aligned", fn);
  return hip_status(w4::launch_weight_offsets(w_tiled, w_scale, group, K, N, out, static_cast<hipStream_t>(stream)),
                    fn);
}

int w4a8_gemm_asym(const int8_t* a, const float* a_scale, const float* a_offset, const void* w_tiled,
                   const void* w_scale, int scale_dtype, int64_t group, const float* w_offsets, const void* bias,
                   void* out, int out_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  const char* fn = "w4a8_gemm_asym";
  if (scale_dtype != W4_F16)
    return fail(W4_ERR_DTYPE, "%s: weight scales must be fp16 (dtype code %d); the int8 kernel reads them as fp16",
                fn, scale_dtype);
  if (out_dtype != W4_BF16 && out_dtype != W4_F16)
    return fail(W4_ERR_DTYPE, "%s: output must be bf16 or fp16 (dtype code %d)", fn, out_dtype);
  int rc = check_mnk(fn, M, N, K);
  if (!rc && (group == -1 || group > 0)) rc = check_int32_range(fn, group, K, kMaxInt8GroupAsym);
  if (!rc) rc = check_gemm(fn, a, w_tiled, group, M, N, K);
  if (rc) return rc;
  if (M == 0 || N == 0) return ok();
  if (!a_scale || !a_offset || !w_scale || !w_offsets || !out)
    return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(out)) return fail(W4_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
  return hip_status(w4::launch_w4a8_gemm(a, a_scale, w_tiled, w_scale, group, bias, out, out_dtype == W4_BF16,
                                         nullptr, M, N, K, static_cast<hipStream_t>(stream), a_offset, w_offsets),
                    fn);
}

static int check_w4a16(const char* fn, int64_t group, int64_t N, int64_t K) {
  int rc = check_mnk(fn, 0, N, K);
  if (rc) return rc;
  if (group != 64 && group != 128 && group != 256 && group != 512)
    return fail(W4_ERR_GROUP, "%s: group size %lld must be 64, 128, 256 or 512", fn, (long long)group);
  if (K % group) return fail(W4_ERR_GROUP, "%s: group size %lld does not divide K=%lld", fn, (long long)group, (long long)K);
  size_t wb, sb;
  w4::w4a16_tiled_bytes(K, N, &wb, &sb);
  if (wb >= ((size_t)1 << 31) || (uint64_t)N * (uint64_t)K >= ((uint64_t)1 << 31))
    return fail(W4_ERR_UNSUPPORTED, "%s: weight matrix too large (N=%lld K=%lld)", fn, (long long)N, (long long)K);
  return W4_OK;
}

int w4a16_repack_bytes(int64_t K, int64_t N, int64_t group, size_t* w_bytes, size_t* sz_bytes) {
  const char* fn = "w4a16_repack_bytes";
  if (!w_bytes || !sz_bytes) return fail(W4_ERR_INVALID, "%s: null output pointer", fn);
  int rc = check_w4a16(fn, group, N, K);
  if (rc) return rc;
  w4::w4a16_tiled_bytes(K, N, w_bytes, sz_bytes);
  return ok();
}

int w4a16_repack(const uint8_t* w, const void* scale, const void* zero, int sz_dtype, int64_t group, int64_t K,
                 int64_t N, void* w_tiled, void* sz_tiled, void* stream) {
  const char* fn = "w4a16_repack";
  if (sz_dtype != W4_BF16) return fail(W4_ERR_DTYPE, "%s: scale and zero must be bf16 (dtype code %d)", fn, sz_dtype);
  int rc = check_w4a16(fn, group, N, K);
  if (rc) return rc;
  if (N == 0) return ok();
  if (!w || !scale || !w_tiled || !sz_tiled) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(w_tiled) || !aligned16(sz_tiled))
    return fail(W4_ERR_ALIGN, "%s: w_tiled and sz_tiled must be 16-byte aligned", fn);
  return hip_status(w4::launch_w4a16_repack(w, scale, zero, group, K, N, w_tiled, sz_tiled,
                                            static_cast<hipStream_t>(stream)), fn);
}

int w4a16_gemm(const void* x, const void* w_tiled, const void* sz_tiled, int64_t group, void* out, int64_t M,
               int64_t N, int64_t K, void* stream) {
  const char* fn = "w4a16_gemm";
  if (M < 0) return fail(W4_ERR_INVALID, "%s: negative M=%lld", fn, (long long)M);
  int rc = check_w4a16(fn, group, N, K);
  if (rc) return rc;
  if (M > 16) return fail(W4_ERR_UNSUPPORTED, "%s: M=%lld > 16 (decode kernel handles up to 16 rows)", fn, (long long)M);
  if (M == 0 || N == 0) return ok();
  if (!x || !w_tiled || !sz_tiled || !out) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(x) || !aligned16(w_tiled) || !aligned16(sz_tiled))
    return fail(W4_ERR_ALIGN, "%s: x, w_tiled and sz_tiled must be 16-byte aligned", fn);
  return hip_status(w4::launch_w4a16(x, w_tiled, sz_tiled, group, out, M, N, K, static_cast<hipStream_t>(stream)), fn);
}

int w4a8_grouped_gemm(const void* a, int a_dtype, const float* a_scale, const float* a_group_sums,
                      const int32_t* row_token, const int32_t* expert_offsets, int64_t E, const void* w_tiled,
                      const void* w_scale, int scale_dtype, int64_t group, void* out, int out_dtype, int64_t T,
                      int64_t R, int64_t N, int64_t K, void* stream) {
  const char* fn = "w4a8_grouped_gemm";
  if (a_dtype != W4_FP8_E4M3) return fail(W4_ERR_DTYPE, "%s: activations must be fp8 e4m3 (dtype code %d)", fn, a_dtype);
  if (scale_dtype != W4_F16) return fail(W4_ERR_DTYPE, "%s: weight scales must be fp16 (dtype code %d)", fn, scale_dtype);
  if (out_dtype != W4_BF16) return fail(W4_ERR_DTYPE, "%s: output must be bf16 (dtype code %d)", fn, out_dtype);
  int rc = check_mnk(fn, R, N, K);
  if (rc) return rc;
  if (E < 0 || E > 65535 || T < 0) return fail(W4_ERR_INVALID, "%s: E=%lld T=%lld out of range", fn, (long long)E, (long long)T);
  const int64_t gt = group / 128;
  if (group <= 0 || group % 128 || K % group || gt > 4 || (gt & (gt - 1)))
    return fail(W4_ERR_GROUP, "%s: group size %lld must be 128, 256 or 512 and divide K=%lld", fn, (long long)group,
                (long long)K);
  if (R == 0 || N == 0 || E == 0) return ok();
  if (T <= 0 || (int64_t)T * K >= ((int64_t)1 << 31))
    return fail(W4_ERR_UNSUPPORTED, "%s: token count T=%lld out of range for K=%lld (T*K must be below 2^31)", fn,
                (long long)T, (long long)K);
  if (!a || !a_scale || !a_group_sums || !row_token || !expert_offsets || !w_tiled || !w_scale || !out)
    return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(a) || !aligned16(w_tiled) || !aligned16(out))
    return fail(W4_ERR_ALIGN, "%s: a, w_tiled and out must be 16-byte aligned", fn);
  return hip_status(w4::launch_grouped_fp8(a, a_scale, a_group_sums, row_token, expert_offsets, E, w_tiled,
                                           w4::tiled_bytes(K, N), w_scale, group, out, T, R, N, K,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

static int check_tiled(const char* fn, const void* x, int x_dtype, const void* w_tiled, const void* w_scale,
                       int scale_dtype, int64_t group, int64_t M, int64_t N, int64_t K) {
  if (x_dtype != W4_BF16 && x_dtype != W4_F16)
    return fail(W4_ERR_DTYPE, "%s: activations must be bf16 or fp16 (dtype code %d)", fn, x_dtype);
  if (scale_dtype != W4_F16)
    return fail(W4_ERR_DTYPE, "%s: weight scales must be fp16 (dtype code %d)", fn, scale_dtype);
  int rc = check_mnk(fn, M, N, K);
  if (rc) return rc;
  if (group != -1 && (group <= 0 || group % 64 || K % group))
    return fail(W4_ERR_GROUP, "%s: group size %lld must be -1 (per channel) or a multiple of 64 dividing K=%lld", fn,
                (long long)group, (long long)K);
  if (M == 0 || N == 0) return W4_OK;
  if (!x || !w_tiled || !w_scale) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(w_tiled)) return fail(W4_ERR_ALIGN, "%s: w_tiled must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(x) & 7u) != 0) return fail(W4_ERR_ALIGN, "%s: x must be 8-byte aligned", fn);
  return W4_OK;
}

int w4a16_tiled_gemm(const void* x, int x_dtype, const void* w_tiled, const void* w_scale, int scale_dtype,
                     int64_t group, const void* bias, void* out, int64_t M, int64_t N, int64_t K, void* stream) {
  const char* fn = "w4a16_tiled_gemm";
  int rc = check_tiled(fn, x, x_dtype, w_tiled, w_scale, scale_dtype, group, M, N, K);
  if (rc) return rc;
  if (M > 16) return fail(W4_ERR_UNSUPPORTED, "%s: M=%lld > 16 (the kernel takes up to 16 rows)", fn, (long long)M);
  if (M == 0 || N == 0) return ok();
  if (!out) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  return hip_status(w4::launch_w4a16_tiled(x, x_dtype == W4_F16, w_tiled, w_scale, group, bias, out, M, N, K,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

static int64_t linear_threshold(int64_t t) { return t > 0 ? t : W4_LINEAR_MIN_TOKENS_INT8; }

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// int8 codes first, then the fp32 row scales, then (K split) the fp32
// partial tiles [splits][M][N]; each part starts on a 256-byte boundary
struct LinearWs {
  size_t codes, scales, partials, total;
  int splits;
};
static LinearWs linear_workspace(int64_t M, int64_t N, int64_t K, int64_t group, int64_t t) {
  LinearWs w{0, 0, 0, 0, 1};
  if (M < linear_threshold(t)) return w;
  w.splits = w4::w4a8_split_count(M, N, K, group);
  w.codes = 0;
  w.scales = round256((size_t)M * (size_t)K);
  w.partials = w.scales + round256((size_t)M * 4);
  w.total = w.partials + (w.splits > 1 ? (size_t)w.splits * (size_t)M * (size_t)N * 4 : 0);
  return w;
}

int w4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group, int64_t min_tokens_int8,
                              size_t* bytes) {
  const char* fn = "w4_linear_workspace_bytes";
  if (!bytes) return fail(W4_ERR_INVALID, "%s: null output pointer", fn);
  if (M < 0 || N < 0 || K <= 0) return fail(W4_ERR_INVALID, "%s: sizes must be M >= 0, N >= 0, K > 0", fn);
  *bytes = linear_workspace(M, N, K, group, min_tokens_int8).total;
  return ok();
}

static int linear_impl(const char* fn, const void* x, int x_dtype, const void* w_tiled, const void* w_scale,
                       int scale_dtype, int64_t group, const void* bias, void* out, int64_t M, int64_t N, int64_t K,
                       int64_t min_tokens_int8, void* workspace, size_t workspace_bytes, void* stream);

int w4_linear(const void* x, int x_dtype, const void* w_tiled, const void* w_scale, int scale_dtype, int64_t group,
              const void* bias, void* out, int64_t M, int64_t N, int64_t K, int64_t min_tokens_int8, void* workspace,
              size_t workspace_bytes, void* stream) {
  return linear_impl("w4_linear", x, x_dtype, w_tiled, w_scale, scale_dtype, group, bias, out, M, N, K,
                     min_tokens_int8, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- w4_linear_noalloc: the workspace of w4_linear in a file-scope device
// array. Its address differs per GPU; it is looked up once per device (with
// that device current) and kept. Host code never passes the array's name to
// a kernel: the name is a host-side stand-in, not a device address.
namespace {
constexpr size_t kNoAllocScratchBytes = W4_LINEAR_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(const char* fn, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W4_ERR_HIP, "%s: hipGetDevice: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(W4_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(W4_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: HIP error %d (%s)", fn, dev, (int)e,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return W4_OK;
}
}  // namespace

extern "C" {

int w4_linear_noalloc(const void* x, int x_dtype, const void* w_tiled, const void* w_scale, int scale_dtype,
                      int64_t group, const void* bias, void* out, int64_t M, int64_t N, int64_t K,
                      int64_t min_tokens_int8, void* stream) {
  const char* fn = "w4_linear_noalloc";
  int rc = check_tiled(fn, x, x_dtype, w_tiled, w_scale, scale_dtype, group, M, N, K);
  if (rc) return rc;
  rc = check_int32_range(fn, group, K);
  if (rc) return rc;
  if (M == 0 || N == 0) return ok();
  const size_t need = linear_workspace(M, N, K, group, min_tokens_int8).total;
  if (need > kNoAllocScratchBytes)
    return fail(W4_ERR_UNSUPPORTED, "%s: M=%lld N=%lld K=%lld needs %zu bytes of scratch, above its %zu-byte maximum",
                fn, (long long)M, (long long)N, (long long)K, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need) {
    rc = scratch_of_current_device(fn, &ws);
    if (rc) return rc;
  }
  return linear_impl(fn, x, x_dtype, w_tiled, w_scale, scale_dtype, group, bias, out, M, N, K, min_tokens_int8, ws,
                     need ? kNoAllocScratchBytes : 0, stream);
}

}  // extern "C"

static int linear_impl(const char* fn, const void* x, int x_dtype, const void* w_tiled, const void* w_scale,
                       int scale_dtype, int64_t group, const void* bias, void* out, int64_t M, int64_t N, int64_t K,
                       int64_t min_tokens_int8, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_tiled(fn, x, x_dtype, w_tiled, w_scale, scale_dtype, group, M, N, K);
  if (rc) return rc;
  rc = check_int32_range(fn, group, K);
  if (rc) return rc;
  if (M == 0 || N == 0) return ok();
  if (!out) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(out) || !aligned16(x)) return fail(W4_ERR_ALIGN, "%s: x and out must be 16-byte aligned", fn);
  const LinearWs lw = linear_workspace(M, N, K, group, min_tokens_int8);
  const size_t need = lw.total;
  if (workspace_bytes < need || (need && !workspace))
    return fail(W4_ERR_INVALID, "%s: workspace of %zu bytes is smaller than the %zu needed for M=%lld K=%lld", fn,
                workspace_bytes, need, (long long)M, (long long)K);
  if (need && !aligned16(workspace)) return fail(W4_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool f16 = x_dtype == W4_F16;
  if (M < linear_threshold(min_tokens_int8)) {
    // weight-only path, 16 rows per launch
    for (int64_t m0 = 0; m0 < M; m0 += 16) {
      const int64_t rows = M - m0 < 16 ? M - m0 : 16;
      rc = hip_status(w4::launch_w4a16_tiled(static_cast<const uint16_t*>(x) + m0 * K, f16, w_tiled, w_scale, group,
                                             bias, static_cast<uint16_t*>(out) + m0 * N, rows, N, K, st),
                      fn);
      if (rc) return rc;
    }
    return ok();
  }
  uint8_t* wsb = static_cast<uint8_t*>(workspace);
  int8_t* codes = reinterpret_cast<int8_t*>(wsb + lw.codes);
  float* scales = reinterpret_cast<float*>(wsb + lw.scales);
  rc = hip_status(w4::launch_quant_act(x, !f16, M, K, K, codes, false, scales, nullptr, 0, st), fn);
  if (rc) return rc;
  if (lw.splits > 1)   // few rows: K split over blocks, fp32 partial tiles summed by a second kernel
    return hip_status(w4::launch_w4a8_gemm_split(codes, scales, w_tiled, w_scale, bias, out, !f16, M, N, K, lw.splits,
                                                 reinterpret_cast<float*>(wsb + lw.partials), st),
                      fn);
  return hip_status(w4::launch_w4a8_gemm(codes, scales, w_tiled, w_scale, group, bias, out, !f16, nullptr, M, N, K, st),
                    fn);
}

extern "C" {

int w4_quantize_groupwise(const void* w, int w_dtype, int64_t N, int64_t K, int64_t group, uint8_t* packed,
                          void* scale, void* zero, int sz_dtype, void* stream) {
  const char* fn = "w4_quantize_groupwise";
  if (w_dtype != W4_BF16 && w_dtype != W4_F16 && w_dtype != W4_F32)
    return fail(W4_ERR_DTYPE, "%s: weights must be bf16, fp16 or fp32 (dtype code %d)", fn, w_dtype);
  if (sz_dtype != W4_F32 && sz_dtype != W4_BF16)
    return fail(W4_ERR_DTYPE, "%s: scale and zero must be fp32 or bf16 (dtype code %d)", fn, sz_dtype);
  // rows are independent: any N; K is split into whole groups
  if (N < 0 || K <= 0 || N > kMaxDim || K > ((int64_t)1 << 24))
    return fail(W4_ERR_INVALID, "%s: sizes out of range (N=%lld K=%lld)", fn, (long long)N, (long long)K);
  if (group != 64 && group != 128 && group != 256 && group != 512)
    return fail(W4_ERR_GROUP, "%s: group size %lld must be 64, 128, 256 or 512", fn, (long long)group);
  if (K % group) return fail(W4_ERR_GROUP, "%s: group size %lld does not divide K=%lld", fn, (long long)group, (long long)K);
  if (N == 0) return ok();
  if (!w || !packed || !scale || !zero) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(w) || (reinterpret_cast<uintptr_t>(packed) & 3u))
    return fail(W4_ERR_ALIGN, "%s: w must be 16-byte and packed 4-byte aligned", fn);
  const int code = w_dtype == W4_BF16 ? 0 : (w_dtype == W4_F16 ? 1 : 2);
  return hip_status(w4::launch_quantize_groupwise(w, code, N, K, group, packed, scale, zero, sz_dtype == W4_BF16,
                                                  static_cast<hipStream_t>(stream)),
                    fn);
}

int w4a16_embedding(const int32_t* ids, int64_t T, const void* w_tiled, const void* sz_tiled, int64_t group,
                    int64_t V, int64_t K, void* out, void* stream) {
  const char* fn = "w4a16_embedding";
  if (T < 0 || V < 0) return fail(W4_ERR_INVALID, "%s: negative size (T=%lld V=%lld)", fn, (long long)T, (long long)V);
  int rc = check_w4a16(fn, group, V, K);
  if (rc) return rc;
  if (T == 0) return ok();
  if (!ids || !w_tiled || !sz_tiled || !out) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(w_tiled) || !aligned16(sz_tiled) || !aligned16(out))
    return fail(W4_ERR_ALIGN, "%s: w_tiled, sz_tiled and out must be 16-byte aligned", fn);
  return hip_status(w4::launch_embedding(ids, T, w_tiled, sz_tiled, group, V, K, out, static_cast<hipStream_t>(stream)),
                    fn);
}

int w4a16_dequantize(const uint8_t* w, const void* scale, const void* zero, int sz_dtype, int64_t group, int64_t K,
                     int64_t N, void* out, void* stream) {
  const char* fn = "w4a16_dequantize";
  if (sz_dtype != W4_BF16) return fail(W4_ERR_DTYPE, "%s: scale and zero must be bf16 (dtype code %d)", fn, sz_dtype);
  int rc = check_w4a16(fn, group, N, K);
  if (rc) return rc;
  if (N == 0) return ok();
  if (!w || !scale || !out) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if ((reinterpret_cast<uintptr_t>(w) & 7u) || !aligned16(out))
    return fail(W4_ERR_ALIGN, "%s: w must be 8-byte and out 16-byte aligned", fn);
  return hip_status(w4::launch_dequantize(w, scale, zero, group, N, K, out, static_cast<hipStream_t>(stream)), fn);
}

static int check_prefill_gemm(const char* fn, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0)
    return fail(W4_ERR_INVALID, "%s: sizes must be M >= 0, N >= 0, K > 0 (got M=%lld N=%lld K=%lld)", fn,
                (long long)M, (long long)N, (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > ((int64_t)1 << 22))
    return fail(W4_ERR_UNSUPPORTED, "%s: sizes too large (M=%lld N=%lld K=%lld)", fn, (long long)M, (long long)N,
                (long long)K);
  if (K % 64 || N % 8)
    return fail(W4_ERR_ALIGN, "%s: K=%lld must be a multiple of 64 and N=%lld of 8", fn, (long long)K, (long long)N);
  return W4_OK;
}

int w4a16_prefill_gemm(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K, void* stream) {
  const char* fn = "w4a16_prefill_gemm";
  int rc = check_prefill_gemm(fn, M, N, K);
  if (rc) return rc;
  if (M == 0 || N == 0) return ok();
  if (!x || !w || !out) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(x) || !aligned16(w) || !aligned16(out))
    return fail(W4_ERR_ALIGN, "%s: x, w and out must be 16-byte aligned", fn);
  return hip_status(w4::launch_bf16_gemm_nt(x, w, out, M, N, K, static_cast<hipStream_t>(stream)), fn);
}

int w4a16_prefill_workspace_bytes(int64_t N, int64_t K, size_t* bytes) {
  const char* fn = "w4a16_prefill_workspace_bytes";
  if (!bytes) return fail(W4_ERR_INVALID, "%s: null output pointer", fn);
  if (N < 0 || K <= 0) return fail(W4_ERR_INVALID, "%s: sizes must be N >= 0, K > 0", fn);
  *bytes = (size_t)N * (size_t)K * 2;
  return ok();
}

int w4a16_prefill(const void* x, const uint8_t* w, const void* scale, const void* zero, int sz_dtype, int64_t group,
                  void* out, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                  void* stream) {
  const char* fn = "w4a16_prefill";
  if (sz_dtype != W4_BF16) return fail(W4_ERR_DTYPE, "%s: scale and zero must be bf16 (dtype code %d)", fn, sz_dtype);
  int rc = check_w4a16(fn, group, N, K);
  if (!rc) rc = check_prefill_gemm(fn, M, N, K);
  if (rc) return rc;
  if (M == 0 || N == 0) return ok();
  if (!x || !w || !scale || !out) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  const size_t need = (size_t)N * (size_t)K * 2;
  if (!workspace || workspace_bytes < need)
    return fail(W4_ERR_INVALID, "%s: workspace of %zu bytes is smaller than the %zu needed for N=%lld K=%lld", fn,
                workspace_bytes, need, (long long)N, (long long)K);
  if ((reinterpret_cast<uintptr_t>(w) & 7u) || !aligned16(x) || !aligned16(out) || !aligned16(workspace))
    return fail(W4_ERR_ALIGN, "%s: w must be 8-byte and x, out, workspace 16-byte aligned", fn);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  rc = hip_status(w4::launch_dequantize(w, scale, zero, group, N, K, workspace, st), fn);
  if (rc) return rc;
  return hip_status(w4::launch_bf16_gemm_nt(x, workspace, out, M, N, K, st), fn);
}

static int nibbles(const char* fn, const uint8_t* src, int64_t N, int64_t K, uint8_t* dst, bool pack, void* stream) {
  if (N < 0 || K < 0) return fail(W4_ERR_INVALID, "%s: negative size N=%lld K=%lld", fn, (long long)N, (long long)K);
  if (K % 2) return fail(W4_ERR_ALIGN, "%s: K=%lld must be even (two codes per byte)", fn, (long long)K);
  if (N > kMaxDim || K > ((int64_t)1 << 31) || N * K > ((int64_t)1 << 40))
    return fail(W4_ERR_UNSUPPORTED, "%s: sizes too large (N=%lld K=%lld)", fn, (long long)N, (long long)K);
  if (N == 0 || K == 0) return ok();
  if (!src || !dst) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (!aligned16(src) || !aligned16(dst)) return fail(W4_ERR_ALIGN, "%s: buffers must be 16-byte aligned", fn);
  return hip_status(w4::launch_nibbles(src, dst, N, K, pack, static_cast<hipStream_t>(stream)), fn);
}

int w4_fp8_encode_range(uint32_t first_bits, int64_t n, uint8_t* codes, void* stream) {
  const char* fn = "w4_fp8_encode_range";
  if (n < 0) return fail(W4_ERR_INVALID, "%s: negative n=%lld", fn, (long long)n);
  if (n % 8) return fail(W4_ERR_ALIGN, "%s: n=%lld must be a multiple of 8", fn, (long long)n);
  if ((uint64_t)first_bits + (uint64_t)n > ((uint64_t)1 << 32))
    return fail(W4_ERR_INVALID, "%s: range of %lld patterns from 0x%08x passes 2^32", fn, (long long)n, first_bits);
  if (n == 0) return ok();
  if (!codes) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (reinterpret_cast<uintptr_t>(codes) & 7u) return fail(W4_ERR_ALIGN, "%s: codes must be 8-byte aligned", fn);
  return hip_status(w4::launch_fp8_encode_range(first_bits, n, codes, static_cast<hipStream_t>(stream)), fn);
}

int w4_probe_mfma(int kind, int64_t iters, int32_t* sink, int64_t sink_elems, double* ops, void* stream) {
  const char* fn = "w4_probe_mfma";
  if (kind < 0 || kind > 2) return fail(W4_ERR_INVALID, "%s: kind %d is not 0 (int8), 1 (fp8) or 2 (bf16)", fn, kind);
  if (iters < 1 || iters > ((int64_t)1 << 24))
    return fail(W4_ERR_INVALID, "%s: iters=%lld outside [1, 2^24]", fn, (long long)iters);
  if (!sink || !ops) return fail(W4_ERR_INVALID, "%s: null pointer argument", fn);
  if (sink_elems < w4::probe_sink_elems())
    return fail(W4_ERR_INVALID, "%s: sink of %lld int32 is smaller than the %lld needed", fn, (long long)sink_elems,
                (long long)w4::probe_sink_elems());
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return fail(W4_ERR_ALIGN, "%s: sink must be 4-byte aligned", fn);
  *ops = w4::probe_mfma_ops(kind, iters);
  return hip_status(w4::launch_probe_mfma(kind, iters, sink, static_cast<hipStream_t>(stream)), fn);
}

int w4_pack_nibbles(const uint8_t* codes, int64_t N, int64_t K, uint8_t* packed, void* stream) {
  return nibbles("w4_pack_nibbles", codes, N, K, packed, true, stream);
}

int w4_unpack_nibbles(const uint8_t* packed, int64_t N, int64_t K, uint8_t* codes, void* stream) {
  return nibbles("w4_unpack_nibbles", packed, N, K, codes, false, stream);
}

}  // extern "C"
