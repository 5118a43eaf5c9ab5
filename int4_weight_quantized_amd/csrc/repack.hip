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

namespace w4 {

// [N, K] codes <-> [N, K/2] bytes, byte j = q[2j] | q[2j+1] << 4 (the
// cpu_int4.py page, pack_nibbles / unpack_nibbles). Rows are contiguous and K
// is even, so both are flat streams: packed byte j of the whole matrix holds
// codes 2j and 2j+1 of the whole matrix. A thread takes 16 packed bytes (32
// codes): one 16-byte load and two 16-byte stores, or the reverse; the last
// partial chunk goes byte by byte.
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b) {
  // a, b: four codes each (bytes); result: the 2-byte pairs (a0 a1)(a2 a3)(b0 b1)(b2 b3)
  const uint32_t ma = a & 0x0F0F0F0Fu, mb = b & 0x0F0F0F0Fu;
  const uint32_t pa = (ma | (ma >> 4)) & 0x00FF00FFu;     // bytes 0, 2: code 2i | code 2i+1 << 4
  const uint32_t pb = (mb | (mb >> 4)) & 0x00FF00FFu;
  return (pa & 0xFFu) | ((pa >> 8) & 0xFF00u) | ((pb & 0xFFu) << 16) | ((pb << 8) & 0xFF000000u);
}

__device__ __forceinline__ void unpack4(uint32_t p, uint32_t& a, uint32_t& b) {
  // p: 4 packed bytes -> a: codes of bytes 0, 1; b: codes of bytes 2, 3
  const uint32_t lo = p & 0x0F0F0F0Fu, hi = (p >> 4) & 0x0F0F0F0Fu;
  a = (lo & 0xFFu) | ((hi & 0xFFu) << 8) | ((lo & 0xFF00u) << 8) | ((hi & 0xFF00u) << 16);
  b = ((lo >> 16) & 0xFFu) | ((hi >> 8) & 0xFF00u) | (lo & 0xFF000000u) >> 8 | (hi & 0xFF000000u);
}

__global__ __launch_bounds__(256) void pack_nibbles_kernel(const uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ packed, int64_t nbytes) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 16-byte chunk of packed
  const int64_t b0 = 16 * c;
  if (b0 >= nbytes) return;
  if (b0 + 16 <= nbytes) {
    const v4i x0 = *reinterpret_cast<const v4i*>(codes + 2 * b0);
    const v4i x1 = *reinterpret_cast<const v4i*>(codes + 2 * b0 + 16);
    v4i r;
    r[0] = (int)pack4((uint32_t)x0[0], (uint32_t)x0[1]);
    r[1] = (int)pack4((uint32_t)x0[2], (uint32_t)x0[3]);
    r[2] = (int)pack4((uint32_t)x1[0], (uint32_t)x1[1]);
    r[3] = (int)pack4((uint32_t)x1[2], (uint32_t)x1[3]);
    *reinterpret_cast<v4i*>(packed + b0) = r;
  } else {
    for (int64_t j = b0; j < nbytes; ++j)
      packed[j] = (uint8_t)((codes[2 * j] & 0xFu) | ((codes[2 * j + 1] & 0xFu) << 4));
  }
}

__global__ __launch_bounds__(256) void unpack_nibbles_kernel(const uint8_t* __restrict__ packed,
                                                             uint8_t* __restrict__ codes, int64_t nbytes) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b0 = 16 * c;
  if (b0 >= nbytes) return;
  if (b0 + 16 <= nbytes) {
    const v4i p = *reinterpret_cast<const v4i*>(packed + b0);
    v4i r0, r1;
    uint32_t a, b;
    unpack4((uint32_t)p[0], a, b); r0[0] = (int)a; r0[1] = (int)b;
    unpack4((uint32_t)p[1], a, b); r0[2] = (int)a; r0[3] = (int)b;
    unpack4((uint32_t)p[2], a, b); r1[0] = (int)a; r1[1] = (int)b;
    unpack4((uint32_t)p[3], a, b); r1[2] = (int)a; r1[3] = (int)b;
    *reinterpret_cast<v4i*>(codes + 2 * b0) = r0;
    *reinterpret_cast<v4i*>(codes + 2 * b0 + 16) = r1;
  } else {
    for (int64_t j = b0; j < nbytes; ++j) {
      codes[2 * j] = packed[j] & 0xFu;
      codes[2 * j + 1] = packed[j] >> 4;
    }
  }
}

hipError_t launch_nibbles(const uint8_t* src, uint8_t* dst, int64_t N, int64_t K, bool pack, hipStream_t stream) {
  const int64_t nbytes = N * (K / 2);
  if (nbytes == 0) return hipSuccess;
  const int64_t chunks = (nbytes + 15) / 16;
  dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
  if (pack)
    hipLaunchKernelGGL(pack_nibbles_kernel, grid, block, 0, stream, src, dst, nbytes);
  else
    hipLaunchKernelGGL(unpack_nibbles_kernel, grid, block, 0, stream, src, dst, nbytes);
  return hipGetLastError();
}

}  // namespace w4
