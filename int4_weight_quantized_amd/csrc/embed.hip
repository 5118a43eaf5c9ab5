// The int4 vocab table of the cpu_int4 page: its groupwise weight quantizer
// and the embedding gather, both on the asymmetric grid
// w = (q - 8) * scale + zero of the W4A16 path.
//
// quantize_groupwise (cpu_int4 page, quantize_groupwise): per row and group of
// `group` columns, in fp32: scale = max(max - min, 1e-9) / 15, zero = min +
// 8 * scale, q = clamp(rne((w - min) / scale), 0, 15); codes two per byte,
// low nibble first (pack_nibbles). One thread takes 8 consecutive values; the
// group's group/8 lanes are adjacent in one wave and reduce min and max with
// lane shuffles.
//
// Embedding (CPUInt4EmbeddingMethod.embedding): rows of the table picked by
// token id, dequantized in fp32 and cast to bf16. The table is read in the
// W4A16 tiled layout, the buffers the tied output head (w4a16_gemm) streams,
// so one copy of the weights serves both (tie_weights shares every tensor).
// One thread takes the 16 bytes that a decode lane owns in a unit pair: 32
// codes of one row, 16 consecutive K in each of the pair's two units.
#include "w4_device.h"

namespace w4 {

// ---------------------------------------------------------------- quantize_groupwise

// XT: 0 bf16, 1 fp16, 2 fp32
template <int XT>
__global__ __launch_bounds__(256) void quantize_groupwise_kernel(const void* __restrict__ w, int N, int K, int group,
                                                                 uint32_t* __restrict__ packed, void* __restrict__ scale,
                                                                 void* __restrict__ zero, bool sz_bf16) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = K / 8;
  const int64_t total = (int64_t)N * per_row;
  // threads past the end still take part in the shuffles (their group is whole
  // and entirely past the end, so nothing of theirs is stored)
  const bool live = id < total;
  const int64_t idc = live ? id : total - 1;
  const int row = (int)(idc / per_row), c8 = (int)(idc % per_row);
  float v[8];
  if constexpr (XT == 2) {
    const v4f* p = reinterpret_cast<const v4f*>(static_cast<const float*>(w) + (int64_t)row * K + 8 * c8);
    const v4f a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  } else {
    const v4i a = *reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(w) + (int64_t)row * K + 8 * c8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = (uint32_t)a[i];
      v[2 * i] = XT == 0 ? bf16_to_f32((uint16_t)(u & 0xFFFF)) : f16_to_f32((uint16_t)(u & 0xFFFF));
      v[2 * i + 1] = XT == 0 ? bf16_to_f32((uint16_t)(u >> 16)) : f16_to_f32((uint16_t)(u >> 16));
    }
  }
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  // group/8 adjacent lanes (a power of two <= 64, aligned) hold one group
  for (int off = 1; off < group / 8; off <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, 64));
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  const float s = fmaxf(mx - mn, 1e-9f) / 15.0f;      // IEEE division
  const float z = mn + 8.0f * s;                      // 8 * s is exact
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = fminf(fmaxf(rintf((v[i] - mn) / s), 0.0f), 15.0f);
    word |= (uint32_t)q << (4 * i);                   // byte j = q[2j] | q[2j+1] << 4
  }
  if (!live) return;
  packed[id] = word;
  if ((8 * c8) % group == 0) {
    const int64_t gi = (int64_t)row * (K / group) + (8 * c8) / group;
    if (sz_bf16) {
      static_cast<uint16_t*>(scale)[gi] = f32_to_bf16_rne(s);
      static_cast<uint16_t*>(zero)[gi] = f32_to_bf16_rne(z);
    } else {
      static_cast<float*>(scale)[gi] = s;
      static_cast<float*>(zero)[gi] = z;
    }
  }
}

hipError_t launch_quantize_groupwise(const void* w, int w_dtype_code, int64_t N, int64_t K, int64_t group,
                                     void* packed, void* scale, void* zero, bool sz_bf16, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int64_t total = N * (K / 8);
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
  auto P = static_cast<uint32_t*>(packed);
  switch (w_dtype_code) {
    case 0: hipLaunchKernelGGL(quantize_groupwise_kernel<0>, grid, block, 0, stream, w, (int)N, (int)K, (int)group, P,
                               scale, zero, sz_bf16); break;
    case 1: hipLaunchKernelGGL(quantize_groupwise_kernel<1>, grid, block, 0, stream, w, (int)N, (int)K, (int)group, P,
                               scale, zero, sz_bf16); break;
    default: hipLaunchKernelGGL(quantize_groupwise_kernel<2>, grid, block, 0, stream, w, (int)N, (int)K, (int)group, P,
                                scale, zero, sz_bf16); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- embedding gather

constexpr int kEWinK = 512, kEWTile = 4096, kESZTile = 512;

// One thread per (token, window, pair, j), windows whole (units past K, all
// 64-aligned, are skipped): the 16 bytes of row n at
// ((tile * KW + window) * 4096 + 1024 * pair + 16 * (n % 16 + 16 j)); words 0, 1
// hold K = 64*(2 pair) + 16 j + 0..15 of the window, words 2, 3 the same of the
// next unit. In a word nibble i < 4 is K offset 2i, nibble i >= 4 is 2(i-4)+1.
__global__ __launch_bounds__(256) void embedding_kernel(const int32_t* __restrict__ ids, int T, const uint8_t* __restrict__ wt,
                                                        const uint8_t* __restrict__ szt, int upg, int V, int K, int KW,
                                                        uint16_t* __restrict__ out) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_tok = KW * 16;                        // 32 codes per thread, whole windows
  if (id >= (int64_t)T * per_tok) return;
  const int t = (int)(id / per_tok), c = (int)(id % per_tok);
  const int w = c >> 4, p = (c >> 2) & 3, j = c & 3;  // window, pair, lane group
  const int n = ids[t];
  const int k0 = w * kEWinK + 64 * (2 * p) + 16 * j, k1 = k0 + 64;
  uint16_t* o = out + (int64_t)t * K;
  if (n < 0 || n >= V) {                              // an id outside the table gives a zero row
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (k0 + 8 * i < K) *reinterpret_cast<v4i*>(o + k0 + 8 * i) = v4i{0, 0, 0, 0};
      if (k1 + 8 * i < K) *reinterpret_cast<v4i*>(o + k1 + 8 * i) = v4i{0, 0, 0, 0};
    }
    return;
  }
  const int64_t tile = (int64_t)(n >> 4) * KW + w;
  const v4i words = *reinterpret_cast<const v4i*>(wt + tile * kEWTile + 1024 * p + 16 * ((n & 15) + 16 * j));
  const uint32_t* sz = reinterpret_cast<const uint32_t*>(szt + tile * kESZTile + 32 * (n & 15));
#pragma unroll
  for (int u = 0; u < 2; ++u) {                       // the pair's two units
    const int kb = u ? k1 : k0;
    if (kb >= K) continue;                            // past K (ragged last window)
    const uint32_t szw = sz[(2 * p + u) / upg];
    const float s = bf16_to_f32((uint16_t)(szw & 0xFFFF)), z = bf16_to_f32((uint16_t)(szw >> 16));
    uint16_t r[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t wd = (uint32_t)words[2 * u + h];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int koff = i < 4 ? 2 * i : 2 * (i - 4) + 1;
        const float q = (float)((wd >> (4 * i)) & 15u);
        r[8 * h + koff] = f32_to_bf16_rne(fmaf(q - 8.0f, s, z));
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = (int)((uint32_t)r[8 * h + 2 * e] | ((uint32_t)r[8 * h + 2 * e + 1] << 16));
      *reinterpret_cast<v4i*>(o + kb + 8 * h) = pk;
    }
  }
}

hipError_t launch_embedding(const int32_t* ids, int64_t T, const void* w_tiled, const void* sz_tiled, int64_t group,
                            int64_t V, int64_t K, void* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int KW = (int)((K + kEWinK - 1) / kEWinK);
  const int64_t total = T * KW * 16;
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
  hipLaunchKernelGGL(embedding_kernel, grid, block, 0, stream, ids, (int)T, static_cast<const uint8_t*>(w_tiled),
                     static_cast<const uint8_t*>(sz_tiled), (int)(group / 64), (int)V, (int)K, KW,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace w4

// ---------------------------------------------------------------- prefill dequantization
namespace w4 {

// cpu_int4 page (module docstring, dequantize): for many rows the weight is
// unpacked to bf16 once per call, w = (q - 8) * scale + zero in fp32, and
// handed to an ordinary GEMM. Reads the row-major byte layout [N, K/2]
// (byte j = q[2j] | q[2j+1] << 4) with bf16 scale / zero [N, K/group]; one
// thread per 16 codes (8 bytes in, 32 bytes out; group >= 64 keeps them in
// one group).
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ w, const uint16_t* __restrict__ scale,
                                                         const uint16_t* __restrict__ zero, int group, int N, int K,
                                                         uint16_t* __restrict__ out) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = K / 16;
  if (id >= (int64_t)N * per_row) return;
  const int n = (int)(id / per_row), k0 = 16 * (int)(id % per_row);
  const v2i b = *reinterpret_cast<const v2i*>(w + (int64_t)n * (K / 2) + k0 / 2);
  const int64_t gi = (int64_t)n * (K / group) + k0 / group;
  const float s = bf16_to_f32(scale[gi]), z = zero ? bf16_to_f32(zero[gi]) : 0.f;
  v4i o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t word = (uint32_t)b[h];            // codes k0 + 8h .. + 7, low nibble first
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = fmaf((float)((word >> (8 * e)) & 15u) - 8.0f, s, z);
      const float hi = fmaf((float)((word >> (8 * e + 4)) & 15u) - 8.0f, s, z);
      o[h][e] = (int)((uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16));
    }
  }
  uint16_t* op = out + (int64_t)n * K + k0;
  *reinterpret_cast<v4i*>(op) = o[0];
  *reinterpret_cast<v4i*>(op + 8) = o[1];
}

hipError_t launch_dequantize(const uint8_t* w, const void* scale, const void* zero, int64_t group, int64_t N,
                             int64_t K, void* out, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int64_t total = N * (K / 16);
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, w,
                     static_cast<const uint16_t*>(scale), static_cast<const uint16_t*>(zero), (int)group, (int)N,
                     (int)K, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace w4
