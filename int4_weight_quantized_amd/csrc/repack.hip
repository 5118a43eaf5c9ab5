// Load-time repack of int4 weights into the kernel-tiled layout.
//
// Sources: GPTQ qweight int32 [K/8, N] (inc_w4a8_linear page, the "NT"
// qweight the int8 kernel reads), compressed-tensors weight_packed int32
// [N, K/8] (zentorch page, packed along the input dim) and signed int4 two
// per byte [N, K/2] (w4afp8 page, _repack_signed_int4_to_uint4b8: XOR 0x88
// turns each signed nibble s into the uint4b8 code s + 8), and one signed
// int4 value per int8 byte [N, K] (the compressed-tensors W4A8 int scheme's
// weight_packed, created as int8 [output, input]).
//
// One thread per 32-bit word of the tiled output. The eight codes of an
// output word come from eight (k, n) positions; each is gathered from the
// source word that holds it. Load-time only, so gathers are fine here.
#include "w4_device.h"

namespace w4 {

// layout: 1 GPTQ [K/8, N], 2 CT [N, K/8], 3 signed int4 bytes [N, K/2],
// 4 int8 [N, K] holding values -8..7
__device__ __forceinline__ uint32_t code_at(const void* src, int layout, int K, int N, int k, int n) {
  if (k >= K || n >= N) return 8u;     // padding: zero weight
  if (layout == 1) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(src)[(int64_t)(k >> 3) * N + n];
    return (w >> (4 * (k & 7))) & 0xFu;
  }
  if (layout == 2) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(src)[(int64_t)n * (K >> 3) + (k >> 3)];
    return (w >> (4 * (k & 7))) & 0xFu;
  }
  if (layout == 4) {
    const uint8_t v = reinterpret_cast<const uint8_t*>(src)[(int64_t)n * K + k];
    return (v & 0xFu) ^ 0x8u;          // two's-complement low nibble of v in [-8, 7] -> v + 8
  }
  const uint8_t b = reinterpret_cast<const uint8_t*>(src)[(int64_t)n * (K >> 1) + (k >> 1)];
  const uint32_t s = (k & 1) ? (b >> 4) : (b & 0xFu);
  return s ^ 0x8u;                     // signed nibble -> uint4b8 code
}

__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ src, int layout,
                                                     int K, int N, int64_t src_stride,
                                                     uint32_t* __restrict__ dst, int64_t dst_words,
                                                     int KT) {
  const int64_t wid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int e = blockIdx.y;
  if (wid >= dst_words) return;
  const void* s = src + (int64_t)e * src_stride;
  // wid -> (tile, unit, word)
  const int64_t tile = wid / (kTileBytes / 4);
  const int in_tile = (int)(wid % (kTileBytes / 4));
  const int unit = in_tile >> 2, j = in_tile & 3;
  const int tn = (int)(tile / KT), tk = (int)(tile % KT);
  const int n = tn * kTileN + (unit >> 2);
  const int kq = unit & 3;
  const int kbase = tk * kTileK + 32 * kq + 4 * j;
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t lo = code_at(s, layout, K, N, kbase + b, n) ^ 8u;
    const uint32_t hi = code_at(s, layout, K, N, kbase + 16 + b, n) ^ 8u;
    w |= (lo | (hi << 4)) << (8 * b);
  }
  dst[(int64_t)e * dst_words + wid] = w;
}

size_t tiled_bytes(int64_t K, int64_t N) {
  const int64_t KT = (K + kTileK - 1) / kTileK, NT = (N + kTileN - 1) / kTileN;
  return (size_t)(KT * NT) * kTileBytes;
}

hipError_t launch_repack(const void* src, int layout, int64_t K, int64_t N, int64_t batch,
                         void* dst, hipStream_t stream) {
  const int64_t words = (int64_t)(tiled_bytes(K, N) / 4);
  const int KT = (int)((K + kTileK - 1) / kTileK);
  int64_t src_stride = (layout == 3) ? N * (K / 2) : (layout == 4 ? N * K : N * (K / 8) * 4);
  dim3 block(256), grid((unsigned)((words + 255) / 256), (unsigned)batch);
  hipLaunchKernelGGL(repack_kernel, grid, block, 0, stream,
                     static_cast<const uint8_t*>(src), layout, (int)K, (int)N, src_stride,
                     static_cast<uint32_t*>(dst), words, KT);
  return hipGetLastError();
}

}  // namespace w4
