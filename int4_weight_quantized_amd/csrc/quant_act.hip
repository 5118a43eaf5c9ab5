// Per-token dynamic activation quantization (int8 or FP8 E4M3).
//
// Per the inc_w4a8_linear page (INCXPUW4A8LinearMethod docstring and
// apply_weights) activations are quantized per token to symmetric int8 at
// run time; per the w4afp8 page (W4AFP8Config input_quant) routed-expert
// activations are quantized per token to 8-bit float, symmetric, dynamic.
//
// One block per row. Every thread issues all its bounds-checked 16-byte
// loads (8 elements each, zero past the row end) before using any; the
// absmax is reduced with wave shuffles and LDS; then every element is
// divided by the scale and rounded: rne + clamp to [-127, 127] for int8;
// clamp to +-448, then the hardware RNE conversion to E4M3 (so it
// saturates) for FP8. Rows longer than the register cache are re-read.
//
// The division must be correctly rounded fp32, as the decision is taken on
// that quotient. For scales in [2^-90, 2^90], x is first clamped to +-b, past
// which the code is the saturated one anyway (b = 127.25 s for int8, 449 s
// for FP8), then divided by the usual reciprocal refinement: one Newton step
// on the hardware reciprocal, once per row, then two fma corrections of the
// quotient by its remainder. That is exact whenever the remainders are
// representable, which holds for |x| >= 2^-102, i.e. for every quotient
// above 2^-12; smaller ones round to a zero code whose sign comes from x.
// Other scales take the library division.
//
// HBM-bound: 2 bytes in + 1 byte out per element.
#include "w4_device.h"

namespace w4 {

constexpr int kQThreads = 256;                       // one block per row
constexpr int kQWaves = kQThreads / kWave;
constexpr int kQCache = 8;                           // passes held in registers: rows of up to 16384 elements
constexpr uint32_t kDropped = 0x80000000u;           // buffer offset past any row: the store is dropped

template <bool BF16>
__device__ __forceinline__ void unpack8(const v4i raw, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = (uint32_t)raw[i];
    if (BF16) {
      f[2 * i] = __uint_as_float(w << 16);
      f[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      f[2 * i] = f16_to_f32((uint16_t)(w & 0xFFFFu));
      f[2 * i + 1] = f16_to_f32((uint16_t)(w >> 16));
    }
  }
}

template <bool BF16>
__device__ __forceinline__ float absmax8(const v4i raw) {
  float f[8];
  unpack8<BF16>(raw, f);
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
  return a;
}

// Per-row constants of the conversion.
struct RowScale {
  float s;          // the row's scale
  float y;          // 1/s: hardware reciprocal refined by one Newton step
  float b;          // |x| beyond b decides the saturated code: x is clamped to [-b, b] first
  bool fast;        // s in [2^-90, 2^90]: divide with div_rn_row
  bool zero_row;    // s is 0 (or not a positive number): codes are 0
};

template <bool FP8>
__device__ __forceinline__ RowScale row_scale(float amax, const float* static_scale) {
  RowScale r;
  // a static (calibrated, per-tensor) scale replaces the row's own
  const float s = static_scale ? *static_scale : __fdiv_rn(amax, FP8 ? 448.0f : 127.0f);
  r.s = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s)));   // uniform over the wave
  const float y0 = __builtin_amdgcn_rcpf(r.s);
  r.y = fmaf(fmaf(-r.s, y0, 1.0f), y0, y0);
  // int8: |x/s| <= 127.25 rounds to at most 127 and beyond it the code is
  // +-127; FP8: quotients past 449 clamp to 448 like the quotient of b
  r.b = (FP8 ? 449.0f : 127.25f) * r.s;
  r.fast = r.s >= 0x1p-90f && r.s <= 0x1p90f;
  r.zero_row = !(r.s > 0.f);
  return r;
}

// x / r.s correctly rounded for r.fast rows and |x| <= r.b (a zero quotient
// may lose its sign).
__device__ __forceinline__ float div_rn_row(float x, const RowScale& r) {
  const float q0 = x * r.y;
  const float r0 = fmaf(-r.s, q0, x);
  const float q1 = fmaf(r0, r.y, q0);
  const float r1 = fmaf(-r.s, q1, x);
  return fmaf(r1, r.y, q1);
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

__device__ __forceinline__ v2i pack_fp8(const float (&v)[8]) {
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
  return v2i{w0, w1};
}

// Low bytes of four words, in order, as one word.
__device__ __forceinline__ uint32_t low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_amdgcn_perm(b, a, 0x0C0C0400u) | __builtin_amdgcn_perm(d, c, 0x04000C0Cu);
}

// Codes of one 8-element chunk; for FP8 also returns the sum of the decoded
// codes (in chunk order) when GSUM.
template <bool BF16, bool FP8, bool GSUM>
__device__ __forceinline__ float quantize_chunk(const v4i raw, const RowScale& r, v2i& out) {
  float f[8], v[8];
  unpack8<BF16>(raw, f);
  if (r.fast) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = div_rn_row(__builtin_amdgcn_fmed3f(f[i], -r.b, r.b), r);
      if (FP8) v[i] = __builtin_copysignf(v[i], f[i]);   // the quotient's sign, also for zero
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = __fdiv_rn(f[i], r.s);
      if (!FP8) v[i] = fminf(fmaxf(v[i], -127.25f), 127.25f);
    }
  }
  if (!FP8) {
    // |v| <= 127.25 (+ rounding): adding 1.5 * 2^23 rounds to the nearest
    // integer (ties to even), left in the low mantissa bits as two's complement
    uint32_t u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = __float_as_uint(v[i] + 0x1.8p23f);
    out = v2i{(int)low_bytes(u[0], u[1], u[2], u[3]), (int)low_bytes(u[4], u[5], u[6], u[7])};
    if (r.zero_row) out = v2i{0, 0};
    return 0.f;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = clamp448(v[i]);
    out = pack_fp8(v);
    if (r.zero_row) out = v2i{0, 0};
    float gs = 0.f;
    if (GSUM) {
      gs = __builtin_amdgcn_cvt_f32_fp8(out[0], 0) + __builtin_amdgcn_cvt_f32_fp8(out[0], 1);
      gs += __builtin_amdgcn_cvt_f32_fp8(out[0], 2);
      gs += __builtin_amdgcn_cvt_f32_fp8(out[0], 3);
      gs += __builtin_amdgcn_cvt_f32_fp8(out[1], 0);
      gs += __builtin_amdgcn_cvt_f32_fp8(out[1], 1);
      gs += __builtin_amdgcn_cvt_f32_fp8(out[1], 2);
      gs += __builtin_amdgcn_cvt_f32_fp8(out[1], 3);
    }
    return gs;
  }
}

// Group sums: a group covers gchunks consecutive chunks, an aligned run of
// gchunks lanes of one wave (gchunks is a power of two dividing 64); the
// first lane of the run writes the total.
__device__ __forceinline__ float group_total(float gs, int gchunks) {
  for (int off = gchunks >> 1; off > 0; off >>= 1) gs += __shfl_xor(gs, off, kWave);
  return gs;
}

template <bool BF16, bool FP8>
__global__ __launch_bounds__(kQThreads) void quant_act_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int K,
    uint8_t* __restrict__ codes, float* __restrict__ scales,
    float* __restrict__ gsums, int group, const float* __restrict__ static_scale) {
  __shared__ float red[kQWaves];
  const int m = blockIdx.x;
  const int t = threadIdx.x;
  const uint16_t* xr = x + (int64_t)m * ldx;
  uint8_t* cr = codes + (int64_t)m * K;
  const int nchunks = K >> 3;   // 8 elements per chunk
  // bounds-checked loads, all issued before any is used (zero past the end)
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xr, (uint32_t)K * 2u);
  v4i cache[kQCache];
#pragma unroll
  for (int p = 0; p < kQCache; ++p) cache[p] = buffer_load16(xrs, 16u * (uint32_t)(t + p * kQThreads));
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < kQCache; ++p) amax = fmaxf(amax, absmax8<BF16>(cache[p]));
  for (int c = t + kQCache * kQThreads; c < nchunks; c += kQThreads)
    amax = fmaxf(amax, absmax8<BF16>(buffer_load16(xrs, 16u * (uint32_t)c)));
  amax = wave_max(amax);
  if ((t & (kWave - 1)) == 0) red[t / kWave] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kQWaves; ++w) amax = fmaxf(amax, red[w]);
  amax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(amax)));
#pragma unroll
  for (int p = 0; p < kQCache; ++p) asm volatile("" : "+v"(cache[p]));

  const RowScale r = row_scale<FP8>(amax, static_scale);
  if (t == 0) scales[m] = r.s;
  const int gchunks = group >> 3;
  const int ngroups = gsums ? K / group : 0;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(cr, (uint32_t)K);
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(gsums + (int64_t)m * ngroups, (uint32_t)ngroups * 4u);

  // every lane of a wave takes part in the group-sum shuffles; stores past
  // the row end are dropped
  auto emit = [&](int c, const v4i raw) {
    v2i o;
    if (FP8 && gsums) {
      const float gs = group_total(quantize_chunk<BF16, FP8, true>(raw, r, o), gchunks);
      const bool lead = c < nchunks && (c & (gchunks - 1)) == 0;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(gs), grs, lead ? 4u * (uint32_t)(c / gchunks) : kDropped, 0, 0);
    } else {
      quantize_chunk<BF16, FP8, false>(raw, r, o);
    }
    __builtin_amdgcn_raw_buffer_store_b64(o, crs, 8u * (uint32_t)c, 0, 0);
  };
#pragma unroll
  for (int p = 0; p < kQCache; ++p) {
    if (p * kQThreads >= nchunks) break;          // uniform
    emit(t + p * kQThreads, cache[p]);
  }
  for (int base = kQCache * kQThreads; base < nchunks; base += kQThreads)
    emit(base + t, buffer_load16(xrs, 16u * (uint32_t)(base + t)));
}

// Per-token asymmetric int8 (the input_symmetric = False variant of the
// compressed-tensors W4A8 scheme; the zero output of the inc W4A8 layer's
// per-token quant op). The pages print no arithmetic for it; the grid is the
// min/max one of the cpu_int4 page's quantize_groupwise with 256 levels, in
// fp32:
//   scale  = (max - min) / 255
//   code   = clamp(rne((x - min) / scale), 0, 255) - 128
//   offset = min + 128 * scale            so that x ~ code * scale + offset
// A constant row has scale 0, codes -128 and offset = min.
// One block per row: a min/max pass (wave shuffles, then LDS), then the
// codes, 8 per 16-byte load and 8-byte store; the division is IEEE
// correctly rounded, the decision the codes are taken on. Each thread keeps
// its first kQCache 16-byte chunks in registers between the two passes
// (rows up to 16384 elements are read once); longer rows re-read the rest.
template <bool BF16>
__global__ __launch_bounds__(kQThreads) void quant_act_asym_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                   int K, uint8_t* __restrict__ codes,
                                                                   float* __restrict__ scales,
                                                                   float* __restrict__ offsets) {
  __shared__ float s_lo[kQWaves], s_hi[kQWaves];
  const int64_t m = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x + m * ldx, (uint32_t)K * 2u);
  const int nchunks = K >> 3;
  float lo = __builtin_inff(), hi = -__builtin_inff();
  auto minmax = [&](const v4i raw) {
    float f[8];
    unpack8<BF16>(raw, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo = fminf(lo, f[i]);
      hi = fmaxf(hi, f[i]);
    }
  };
  v4i cache[kQCache];
#pragma unroll
  for (int i = 0; i < kQCache; ++i)   // past the row end: out-of-range loads read zero, never used
    cache[i] = buffer_load16(xrs, 16u * (uint32_t)(t + kQThreads * i));
#pragma unroll
  for (int i = 0; i < kQCache; ++i)
    if (t + kQThreads * i < nchunks) minmax(cache[i]);
  for (int c = t + kQCache * kQThreads; c < nchunks; c += kQThreads) minmax(buffer_load16(xrs, 16u * (uint32_t)c));
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, off, kWave));
    hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
  }
  if (lane == 0) {
    s_lo[wv] = lo;
    s_hi[wv] = hi;
  }
  __syncthreads();
  lo = s_lo[0];
  hi = s_hi[0];
#pragma unroll
  for (int w = 1; w < kQWaves; ++w) {
    lo = fminf(lo, s_lo[w]);
    hi = fmaxf(hi, s_hi[w]);
  }
  const float scale = __fdiv_rn(hi - lo, 255.f);
  const float offset = lo + 128.f * scale;              // 128 * scale is exact
  if (t == 0) {
    scales[m] = scale;
    offsets[m] = offset;
  }
  uint8_t* cr = codes + m * (int64_t)K;
  auto emit = [&](int c, const v4i raw) {
    float f[8];
    unpack8<BF16>(raw, f);
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = scale > 0.f ? rintf(__fdiv_rn(f[i] - lo, scale)) : 0.f;
      b[i] = (uint32_t)((int)fminf(fmaxf(q, 0.f), 255.f) - 128) & 0xFFu;
    }
    uint2 pk;
    pk.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    pk.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    *reinterpret_cast<uint2*>(cr + 8 * (int64_t)c) = pk;
  };
#pragma unroll
  for (int i = 0; i < kQCache; ++i)
    if (t + kQThreads * i < nchunks) emit(t + kQThreads * i, cache[i]);
  for (int c = t + kQCache * kQThreads; c < nchunks; c += kQThreads) emit(c, buffer_load16(xrs, 16u * (uint32_t)c));
}

// Test hook of the FP8 encode: the fp32 values with bit patterns first,
// first + 1, ..., first + n - 1 (n a multiple of 8) go through the
// quantizer's own clamp to +-448 and pair conversion to E4M3, 8 per thread.
__global__ __launch_bounds__(kQThreads) void fp8_encode_range_kernel(uint32_t first, int64_t n8, uint8_t* __restrict__ codes) {
  const int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x;   // 8-value chunk
  if (i >= n8) return;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = clamp448(__uint_as_float(first + (uint32_t)(8 * i + e)));
  *reinterpret_cast<v2i*>(codes + 8 * i) = pack_fp8(v);
}

hipError_t launch_fp8_encode_range(uint32_t first, int64_t n, uint8_t* codes, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(fp8_encode_range_kernel, dim3((unsigned)((n8 + kQThreads - 1) / kQThreads)), dim3(kQThreads), 0,
                     stream, first, n8, codes);
  return hipGetLastError();
}

hipError_t launch_quant_act_asym(const void* x, bool bf16, int64_t M, int64_t K, int64_t ldx, void* codes,
                                 float* scales, float* offsets, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint8_t* cp = static_cast<uint8_t*>(codes);
  const dim3 grid((unsigned)M), block(kQThreads);
  if (bf16)
    hipLaunchKernelGGL((quant_act_asym_kernel<true>), grid, block, 0, stream, xp, ldx, (int)K, cp, scales, offsets);
  else
    hipLaunchKernelGGL((quant_act_asym_kernel<false>), grid, block, 0, stream, xp, ldx, (int)K, cp, scales, offsets);
  return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, bool bf16, int64_t M, int64_t K, int64_t ldx,
                            void* codes, bool fp8, float* scales, float* gsums, int group,
                            hipStream_t stream, const float* static_scale) {
  if (M == 0) return hipSuccess;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint8_t* cp = static_cast<uint8_t*>(codes);
  const dim3 grid((unsigned)M), block(kQThreads);
  const int k = (int)K;
  if (bf16 && !fp8)
    hipLaunchKernelGGL((quant_act_kernel<true, false>), grid, block, 0, stream, xp, ldx, k, cp, scales, nullptr, 8, static_scale);
  else if (!bf16 && !fp8)
    hipLaunchKernelGGL((quant_act_kernel<false, false>), grid, block, 0, stream, xp, ldx, k, cp, scales, nullptr, 8, static_scale);
  else if (bf16 && fp8)
    hipLaunchKernelGGL((quant_act_kernel<true, true>), grid, block, 0, stream, xp, ldx, k, cp, scales, gsums, group, static_scale);
  else
    hipLaunchKernelGGL((quant_act_kernel<false, true>), grid, block, 0, stream, xp, ldx, k, cp, scales, gsums, group, static_scale);
  return hipGetLastError();
}

}  // namespace w4
