// W4A16 decode GEMM (M <= 16) on the asymmetric grid w = (q - 8)*scale + zero.
//
// Per the cpu_int4.py page (module docstring, pack_nibbles): single-stream
// decode is bound by the bytes of the weights read per token; bf16
// activations; two codes per byte, byte j = w[2j] | w[2j+1] << 4; bf16
// scale and zero per (output row, group of K).
//
//   out[m,n] = sum_g ( scale[n,g] * sum_{k in g} x[m,k]*(q[n,k]-8)
//                    + zero[n,g]  * sum_{k in g} x[m,k] )
//
// Design (gfx950): v_mfma_f32_16x16x32_bf16 with the activations as the
// 16-row A operand (rows >= M are zero) and 16 weight rows as the B operand.
// The weights are read in their byte layout as-is: per 64-wide K unit a lane
// loads 8 bytes (16 codes) of one weight row, so every MFMA step stays inside
// one scale group. Codes become bf16 values 128+q, exact, with one mask-or
// (0x4300 | q is the bf16 bit pattern of 128+q), the pairing of K inside
// the operand being matched by a byte permute of the activations. The row
// sums sum_k x[m,k] come from the same MFMA against a ones operand, so
//   sum_k x*(q-8) = C - 136*XS   and   y_g = scale*C + (zero - 136*scale)*XS.
// Each block owns 16 output columns and splits K across its four waves
// (whole groups per wave); partial 16x16 tiles are summed through LDS.
// HBM-bound: 0.5 byte per weight + 4 bytes of scale/zero per group.
#include "w4_device.h"

namespace w4 {

constexpr int kDThreads = 256;
constexpr int kDBatch = 8;          // units (64 K each) loaded per batch

__device__ __forceinline__ v8bf as_v8bf(v4i v) { return __builtin_bit_cast(v8bf, v); }

__device__ __forceinline__ v4i unpack_bf16_128q(uint32_t w) {
  // codes c0..c7 of the word (c_{2i} low nibble of byte i) -> bf16 128+c in
  // element order [c0 c4 c1 c5 c2 c6 c3 c7]
  v4i r;
  r[0] = (int)((w & 0x000F000Fu) | 0x43004300u);
  r[1] = (int)(((w >> 4) & 0x000F000Fu) | 0x43004300u);
  r[2] = (int)(((w >> 8) & 0x000F000Fu) | 0x43004300u);
  r[3] = (int)(((w >> 12) & 0x000F000Fu) | 0x43004300u);
  return r;
}

__device__ __forceinline__ v4i permute_x(v4i raw) {
  // raw = [x0x1, x2x3, x4x5, x6x7] (bf16 pairs) -> [x0x4, x1x5, x2x6, x3x7]
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm((uint32_t)raw[2], (uint32_t)raw[0], 0x05040100u);
  r[1] = (int)__builtin_amdgcn_perm((uint32_t)raw[2], (uint32_t)raw[0], 0x07060302u);
  r[2] = (int)__builtin_amdgcn_perm((uint32_t)raw[3], (uint32_t)raw[1], 0x05040100u);
  r[3] = (int)__builtin_amdgcn_perm((uint32_t)raw[3], (uint32_t)raw[1], 0x07060302u);
  return r;
}

__global__ __launch_bounds__(kDThreads) void w4a16_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero,
    uint16_t* __restrict__ out, int M, int N, int K, int G, int upg) {
  __shared__ float red[4][64][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int l16 = lane & 15, j = lane >> 4;
  const int n = n0 + l16;                 // B column of this lane
  const bool nval = n < N;
  const bool mval = l16 < M;              // A row of this lane
  const int64_t wrow = (int64_t)(nval ? n : 0) * (K >> 1);
  const uint16_t* xrow = x + (int64_t)(mval ? l16 : 0) * K;

  // groups of this wave: g = wave, wave + 4, ...; units of a group are consecutive
  const int ng = (G > wave) ? (G - wave + 3) / 4 : 0;
  const int nu = ng * upg;                // units this wave processes
  auto unit_of = [&](int idx) { return (wave + 4 * (idx / upg)) * upg + (idx % upg); };

  auto load_batch = [&](v2i (&wb)[kDBatch], int base) {
#pragma unroll
    for (int i = 0; i < kDBatch; ++i) {
      const int idx = base + i;
      if (idx < nu && nval) {
        const int u = unit_of(idx);
        wb[i] = *reinterpret_cast<const v2i*>(w + wrow + u * 32 + 8 * j);
      } else {
        wb[i] = v2i{0, 0};
      }
    }
  };

  const v4i ones = {0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80};
  v4f yacc = {0.f, 0.f, 0.f, 0.f};
  v4f cacc = {0.f, 0.f, 0.f, 0.f}, xacc = {0.f, 0.f, 0.f, 0.f};

  auto process = [&](const v2i (&wb)[kDBatch], int base) {
#pragma unroll
    for (int i = 0; i < kDBatch; ++i) {
      const int idx = base + i;
      if (idx >= nu) break;
      const int u = unit_of(idx);
      const int kb = u * 64 + 16 * j;
      v4i xr0 = {0, 0, 0, 0}, xr1 = {0, 0, 0, 0};
      if (mval) {
        xr0 = *reinterpret_cast<const v4i*>(xrow + kb);
        xr1 = *reinterpret_cast<const v4i*>(xrow + kb + 8);
      }
      const v8bf a0 = as_v8bf(permute_x(xr0)), a1 = as_v8bf(permute_x(xr1));
      const v8bf b0 = as_v8bf(unpack_bf16_128q((uint32_t)wb[i][0]));
      const v8bf b1 = as_v8bf(unpack_bf16_128q((uint32_t)wb[i][1]));
      const bool first = (idx % upg) == 0;
      const v4f z4 = {0.f, 0.f, 0.f, 0.f};
      cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, first ? z4 : cacc, 0, 0, 0);
      cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, cacc, 0, 0, 0);
      xacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_v8bf(ones), first ? z4 : xacc, 0, 0, 0);
      xacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_v8bf(ones), xacc, 0, 0, 0);
      if ((idx % upg) == upg - 1) {
        const int g = u / upg;
        float s = 0.f, zp = 0.f;
        if (nval) {
          s = bf16_to_f32(scale[(int64_t)n * G + g]);
          const float z = zero ? bf16_to_f32(zero[(int64_t)n * G + g]) : 0.f;
          zp = fmaf(-136.f, s, z);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[r] = fmaf(s, cacc[r], fmaf(zp, xacc[r], yacc[r]));
      }
    }
  };

  // two register batches: the next batch's loads are in flight while one computes
  v2i wb0[kDBatch], wb1[kDBatch];
  if (nu > 0) load_batch(wb0, 0);
  for (int base = 0; base < nu; base += 2 * kDBatch) {
    if (base + kDBatch < nu) load_batch(wb1, base + kDBatch);
    process(wb0, base);
    if (base + kDBatch >= nu) break;
    if (base + 2 * kDBatch < nu) load_batch(wb0, base + 2 * kDBatch);
    process(wb1, base + kDBatch);
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][lane][r] = yacc[r];
  __syncthreads();
  {
    const int m = tid >> 4, nn = tid & 15;     // output element (m, n0 + nn)
    const int l = nn + 16 * (m >> 2), r = m & 3;
    const float y = red[0][l][r] + red[1][l][r] + red[2][l][r] + red[3][l][r];
    if (m < M && n0 + nn < N) out[(int64_t)m * N + n0 + nn] = f32_to_bf16_rne(y);
  }
}

hipError_t launch_w4a16(const void* x, const uint8_t* w, const void* scale, const void* zero,
                        int64_t group, void* out, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int G = (int)(K / group);
  const int upg = (int)(group / 64);
  dim3 grid((unsigned)((N + 15) / 16)), block(kDThreads);
  hipLaunchKernelGGL(w4a16_kernel, grid, block, 0, stream, static_cast<const uint16_t*>(x), w,
                     static_cast<const uint16_t*>(scale), static_cast<const uint16_t*>(zero),
                     static_cast<uint16_t*>(out), (int)M, (int)N, (int)K, G, upg);
  return hipGetLastError();
}

}  // namespace w4
