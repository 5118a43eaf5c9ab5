// Per-token dynamic activation quantization (int8 or FP8 E4M3).
//
// Per the inc_w4a8_linear page (INCXPUW4A8LinearMethod docstring and
// apply_weights) activations are quantized per token to symmetric int8 at
// run time; per the w4afp8 page (W4AFP8Config input_quant) routed-expert
// activations are quantized per token to 8-bit float, symmetric, dynamic.
//
// One 256-thread block per row. The row is read once into registers
// (16-byte loads, 8 elements per thread per pass), its absmax reduced with
// wave shuffles and LDS, then every element divided by the scale with
// correctly rounded fp32 division and rounded: rne + clamp to [-127, 127]
// for int8, hardware RNE conversion to E4M3 (after clamping to +-448, so it
// saturates) for FP8. Rows longer than the register cache are re-read.
// HBM-bound: 2 bytes in + 1 byte out per element.
#include "w4_device.h"

namespace w4 {

constexpr int kQThreads = 256;
constexpr int kQCache = 8;   // passes held in registers: K <= 8 * 8 * 256 = 16384

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

// FP8 = false: int8 codes; true: E4M3 codes (+ optional group sums).
template <bool BF16, bool FP8>
__global__ __launch_bounds__(kQThreads) void quant_act_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int K,
    uint8_t* __restrict__ codes, float* __restrict__ scales,
    float* __restrict__ gsums, int group, const float* __restrict__ static_scale) {
  __shared__ float red[kQThreads / kWave];
  const int m = blockIdx.x;
  const int t = threadIdx.x;
  const uint16_t* xr = x + (int64_t)m * ldx;
  uint8_t* cr = codes + (int64_t)m * K;
  const int nchunks = K >> 3;   // 8 elements per chunk

  v4i cache[kQCache];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < kQCache; ++p) {
    const int c = t + p * kQThreads;
    if (c < nchunks) {
      cache[p] = *reinterpret_cast<const v4i*>(xr + 8 * c);
      float f[8];
      unpack8<BF16>(cache[p], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    }
  }
  for (int c = t + kQCache * kQThreads; c < nchunks; c += kQThreads) {
    float f[8];
    unpack8<BF16>(*reinterpret_cast<const v4i*>(xr + 8 * c), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = wave_max(amax);
  if ((t & (kWave - 1)) == 0) red[t / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  // a static (calibrated, per-tensor) scale replaces the row's own
  const float s = static_scale ? *static_scale : __fdiv_rn(amax, FP8 ? 448.0f : 127.0f);
  if (t == 0) scales[m] = s;
  const bool zero_row = !(s > 0.f);
  const int gchunks = group >> 3;   // chunks per group (power of two <= 64) for gsums

  auto do_chunk = [&](int c, const v4i raw) {
    float f[8];
    unpack8<BF16>(raw, f);
    uint32_t lo = 0, hi = 0;
    float gs = 0.f;
    if (!FP8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int q = zero_row ? 0 : (int)rintf(__fdiv_rn(f[i], s));
        q = min(127, max(-127, q));
        const uint32_t b = (uint32_t)(q & 0xFF);
        if (i < 4) lo |= b << (8 * i); else hi |= b << (8 * (i - 4));
      }
    } else {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = zero_row ? 0.f : __fdiv_rn(f[i], s);
        v[i] = fminf(fmaxf(v[i], -448.f), 448.f);
      }
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
      int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
      lo = (uint32_t)w0;
      hi = (uint32_t)w1;
      if (gsums) {
        gs = __builtin_amdgcn_cvt_f32_fp8(w0, 0) + __builtin_amdgcn_cvt_f32_fp8(w0, 1);
        gs += __builtin_amdgcn_cvt_f32_fp8(w0, 2);
        gs += __builtin_amdgcn_cvt_f32_fp8(w0, 3);
        gs += __builtin_amdgcn_cvt_f32_fp8(w1, 0);
        gs += __builtin_amdgcn_cvt_f32_fp8(w1, 1);
        gs += __builtin_amdgcn_cvt_f32_fp8(w1, 2);
        gs += __builtin_amdgcn_cvt_f32_fp8(w1, 3);
      }
    }
    *reinterpret_cast<v2i*>(cr + 8 * c) = v2i{(int)lo, (int)hi};
    return gs;
  };

  // Group sums: a group covers gchunks consecutive chunks, i.e. an aligned
  // run of gchunks lanes inside one wave (gchunks divides 64 and 256).
  auto emit_gsum = [&](int c, float gs) {
    if (!FP8 || !gsums) return;
    for (int off = gchunks >> 1; off > 0; off >>= 1) gs += __shfl_xor(gs, off, kWave);
    if (c < nchunks && (c % gchunks) == 0) gsums[(int64_t)m * (K / group) + c / gchunks] = gs;
  };

#pragma unroll
  for (int p = 0; p < kQCache; ++p) {
    const int c = t + p * kQThreads;
    if (p * kQThreads >= nchunks) break;          // uniform
    float gs = 0.f;
    if (c < nchunks) gs = do_chunk(c, cache[p]);
    emit_gsum(c, gs);
  }
  for (int base = kQCache * kQThreads; base < nchunks; base += kQThreads) {
    const int c = base + t;
    float gs = 0.f;
    if (c < nchunks) gs = do_chunk(c, *reinterpret_cast<const v4i*>(xr + 8 * c));
    emit_gsum(c, gs);
  }
}

hipError_t launch_quant_act(const void* x, bool bf16, int64_t M, int64_t K, int64_t ldx,
                            void* codes, bool fp8, float* scales, float* gsums, int group,
                            hipStream_t stream, const float* static_scale) {
  if (M == 0) return hipSuccess;
  dim3 grid((unsigned)M), block(kQThreads);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint8_t* cp = static_cast<uint8_t*>(codes);
  if (bf16 && !fp8)
    hipLaunchKernelGGL((quant_act_kernel<true, false>), grid, block, 0, stream, xp, ldx, (int)K, cp, scales, nullptr, 8, static_scale);
  else if (!bf16 && !fp8)
    hipLaunchKernelGGL((quant_act_kernel<false, false>), grid, block, 0, stream, xp, ldx, (int)K, cp, scales, nullptr, 8, static_scale);
  else if (bf16 && fp8)
    hipLaunchKernelGGL((quant_act_kernel<true, true>), grid, block, 0, stream, xp, ldx, (int)K, cp, scales, gsums, group, static_scale);
  else
    hipLaunchKernelGGL((quant_act_kernel<false, true>), grid, block, 0, stream, xp, ldx, (int)K, cp, scales, gsums, group, static_scale);
  return hipGetLastError();
}

}  // namespace w4
