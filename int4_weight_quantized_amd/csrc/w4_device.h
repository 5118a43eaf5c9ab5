// Device-side helpers shared by the gfx950 kernels of libw4.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace w4 {

constexpr int kWave = 64;

// Kernel-tiled int4 weight layout (written by w4_repack, read by the GEMMs):
// tiles of kTileN output columns x kTileK K-values, 8 KiB each, ordered
// [n_tile][k_tile]. Inside a tile, 16-byte unit u = n_local*4 + kq holds the
// 32 codes of column n_local for k = 32*kq .. 32*kq+31: in word j (0..3),
// byte b (0..3), the low nibble is the code of k = 32*kq + 4*j + b and the
// high nibble the code of k + 16. Nibbles are stored as q ^ 8, the
// two's-complement int4 of q - 8, so (w & 0xF0F0F0F0) and ((w << 4) &
// 0xF0F0F0F0) are int8 bytes equal to 16*(q - 8) in K order.
constexpr int kTileN = 128;
constexpr int kTileK = 128;
constexpr int kTileBytes = kTileN * kTileK / 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // gfx9 raw buffer: stride 0, num_records in bytes; accesses past the end
  // return zero instead of faulting.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v4i buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);   // IEEE conversion, nearest even
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Workgroup barrier without the memory wait that __syncthreads() places
// before it (s_waitcnt vmcnt(0) lgkmcnt(0), which also drains loads issued
// for later steps). The caller first waits, with a partial count, for exactly
// what the other waves need from it (its share of the next stage's LDS DMA,
// its LDS writes); loads for later steps stay in flight across the barrier.
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }

// A pair of 32-bit words (lo in the lower register) shifted as one 64-bit
// value by a constant: one v_lshlrev_b64 / v_lshrrev_b64 where two 32-bit
// shifts would otherwise be issued (the compiler splits a 64-bit shift whose
// crossing bits are masked off later; the empty asm statement takes the
// whole 64-bit result, so the shift stays whole and is still an instruction
// the compiler schedules and checks for hazards itself). The nibble unpacks
// use them on word pairs: the bits carried across the word boundary land
// where their masks clear. Pairs come from a 16-byte vector reinterpreted
// as two 64-bit lanes, so no instruction builds them.
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u64x2 as_u64x2(v4i v) { return __builtin_bit_cast(u64x2, v); }
template <int N>
__device__ __forceinline__ uint64_t shl64(uint64_t v) {
  uint64_t r = v << N;
  asm("" : "+v"(r));
  return r;
}
template <int N>
__device__ __forceinline__ uint64_t shr64(uint64_t v) {
  uint64_t r = v >> N;
  asm("" : "+v"(r));
  return r;
}

// Map a linear block id to a tile id so that blocks the hardware sends to
// the same XCD (round-robin over 8 XCDs) get a contiguous run of tile ids.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  if (nblocks % kXcd != 0) return bid;
  return (bid % kXcd) * (nblocks / kXcd) + bid / kXcd;
}

}  // namespace w4
