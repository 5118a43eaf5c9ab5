// Prefill path of the W4A16 layer: bf16 GEMM on the dequantized weights.
//
// Per the cpu_int4.py page (module docstring, dequantize, _cpu_int4_linear):
// from a batch threshold up, the int4 weight is unpacked to a bf16 matrix once
// per call (w = (q - 8) * scale + zero) and the layer is an ordinary bf16 GEMM
//   y[m, n] = sum_k x[m, k] * w[n, k]          (x: [M, K], w: [N, K], y: [M, N])
// The unpacking is dequantize_kernel (embed.hip); this file is the GEMM.
//
// Design (gfx950), bound by the bf16 matrix cores:
// - 256 threads, block tile 256 x 256 (or 256 x 224 when that fills the CUs
//   in fewer rounds), four waves of 128 x 128 (x 112), K step 64 (128-byte
//   rows), one block per CU. The fp32 accumulators of a lane (up to 256) live
//   in the accumulation registers.
// - x and w rows go straight from memory into LDS (buffer_load ... lds, one
//   KiB per wave instruction), 16-byte chunks swizzled by row & 7; the buffer
//   range check zero-fills rows past M or N. Two stages: a K step's tile is
//   requested as soon as its stage is free, about one K step before use
//   (four 32-deep stages, three steps ahead, measured slower: 448 against
//   402 us, one more barrier per 32 K).
// - v_mfma_f32_16x16x32_bf16 with the weight fragment as the first operand,
//   so each lane's four results are four consecutive output columns of one
//   row. A K step is two 32-deep substeps; the fragments of the next substep
//   (or the next step's first) are read from LDS while the current substep's
//   MFMAs run, and so are the DMAs of the tile two steps ahead: one read or
//   DMA every two to four MFMAs. With one wave per SIMD nothing else feeds
//   the matrix core, so issuing them in a burst before the MFMAs left it
//   idle while the wave waited to issue them (405 -> 335 us at M=4096,
//   K=4096, N=14336).
// - The output tile goes through LDS in two 128-row halves and leaves as
//   16-byte row segments (v_cvt_pk_bf16_f32: nearest even).
// - Tiles are visited in groups of 4 tile-rows, block ids remapped so each XCD
//   works on a contiguous range of tiles.
#include "w4_device.h"

namespace w4 {

constexpr int kPM = 256, kPK = 64;
constexpr int kPThreads = 256;
constexpr int kPRow = kPK * 2;                 // bytes per staged row
constexpr int kPStageA = kPM * kPRow;          // 32 KiB

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// acc += a (16 x 32) * b (32 x 16), the accumulator bound to accumulation
// registers for the whole kernel (a lane's 256 of them do not fit beside the
// fragments in the 256 vector registers; left to itself the allocator moves
// some between the two files on every K step). Volatile: the MFMAs keep
// their place between the loads and the barrier (measured: 430 -> 402 us at
// M=4096, K=4096, N=14336 against the compiler's own order).
__device__ __forceinline__ void mfma_acc(v4f& acc, const v8bf& a, const v8bf& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// BN: block tile columns, 256 or 224 (two waves of BN/2 = 16 NJ columns)
template <int BN>
__global__ __launch_bounds__(kPThreads, 1) void bf16_gemm_nt_kernel(const uint16_t* __restrict__ X,
                                                                     const uint16_t* __restrict__ Wb,
                                                                     uint16_t* __restrict__ Y, int M, int N, int K,
                                                                     int KT, int tilesM, int tilesN) {
  constexpr int NJ = BN / 32;                   // 16-column blocks per wave
  constexpr int kPStage = kPStageA + BN * kPRow;
  constexpr int kPORow = BN * 2 + 16;           // output row in LDS, padded
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kPStage];

  const int t = xcd_remap(blockIdx.x, gridDim.x);
  constexpr int GM = 4;
  const int per_group = GM * tilesN;
  const int first_m = (t / per_group) * GM;
  const int gsz = min(tilesM - first_m, GM);
  const int tm = first_m + (t % per_group) % gsz;
  const int tn = (t % per_group) / gsz;
  const int m0 = tm * kPM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t rowb = (uint32_t)K * 2u;      // bytes per source row

  // ---- loads: wave w's instruction i fills stage rows 64w + 8i .. +7 of x
  // (BN/4 w + 8i .. of w), lane L landing at row 64w + 8i + L/8, physical
  // chunk L%8 and fetching logical chunk (L%8) ^ (L/8) of its row. Rows past
  // the matrix read zero (range check on the per-block buffer). K is a
  // multiple of 64.
  const int rows_x = min(kPM, M - m0), rows_w = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + (int64_t)m0 * K, (uint32_t)rows_x * rowb);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wb + (int64_t)n0 * K, (uint32_t)rows_w * rowb);
  const int lrow = lane >> 3, lchunk = lane & 7;
  const uint32_t lchunk_off = 16u * (uint32_t)(lchunk ^ lrow);
  const uint32_t xoff = (uint32_t)(64 * wave + lrow) * rowb + lchunk_off;
  const uint32_t woff = (uint32_t)(BN / 4 * wave + lrow) * rowb + lchunk_off;
  // DMA instruction o of a K step: o < 8 a row group of x, else one of w
  auto gload_one = [&](int tk, int st, int o) {
    const uint32_t ks = (uint32_t)tk * kPRow;
    if (o < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (__attribute__((address_space(3))) void*)(lds + st * kPStage + (64 * wave_u + 8 * o) * kPRow), 16,
          xoff + ks + (uint32_t)(8 * o) * rowb, 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr,
          (__attribute__((address_space(3))) void*)(lds + st * kPStage + kPStageA +
                                                    (BN / 4 * wave_u + 8 * (o - 8)) * kPRow),
          16, woff + ks + (uint32_t)(8 * (o - 8)) * rowb, 0, 0, 0);
  };
  auto gload = [&](int tk, int st) {
#pragma unroll
    for (int o = 0; o < 8 + BN / 32; ++o) gload_one(tk, st, o);
  };
  constexpr int kLoads = 8 + BN / 32;           // DMA instructions per wave and K step

  // ---- fragments: lane row (lane & 15) of a 16-row block, 16-byte chunk
  // 4s + (lane >> 4) of substep s, at its swizzled place
  const int g = lane >> 4, fl = lane & 7;
  int fo[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) fo[s] = (lane & 15) * kPRow + 16 * ((4 * s + g) ^ fl);
  const int xo = 128 * wm * kPRow, wo = kPStageA + (BN / 2) * wn * kPRow;
  v8bf xf[2][8], wf[2][NJ];
  auto read_frags = [&](int st, int s, int buf) {
    const uint8_t* base = lds + st * kPStage + fo[s];
#pragma unroll
    for (int i = 0; i < 8; ++i) xf[buf][i] = *reinterpret_cast<const v8bf*>(base + xo + 16 * kPRow * i);
#pragma unroll
    for (int j = 0; j < NJ; ++j) wf[buf][j] = *reinterpret_cast<const v8bf*>(base + wo + 16 * kPRow * j);
  };
  // fragment read r of a substep: r < 8 an x row block, else a w column block
  auto read_one = [&](int st, int s, int buf, int r) {
    const uint8_t* base = lds + st * kPStage + fo[s];
    if (r < 8) xf[buf][r] = *reinterpret_cast<const v8bf*>(base + xo + 16 * kPRow * r);
    else wf[buf][r - 8] = *reinterpret_cast<const v8bf*>(base + wo + 16 * kPRow * (r - 8));
  };

  v4f acc[8][NJ];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: tiles 0 and 1 into the two stages, tile 0's first fragments
  gload(0, 0);
  gload(min(1, KT - 1), 1);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kLoads & 15) | ((kLoads >> 4) << 14));   // vmcnt(kLoads): tile 0 landed
  __syncthreads();
  read_frags(0, 0, 0);

  // step tk (stage st; tile tk + 1 already streaming into the other stage):
  // substep 0 runs while substep 1's fragments are read; then every wave's
  // tile tk + 1 has landed and every read of stage st is done (barrier), tile
  // tk + 2 starts streaming into stage st, and substep 1 runs while the next
  // step's first fragments are read. A tile has about a whole K step of MFMAs
  // to arrive.
  constexpr int kNM = 8 * NJ, kNR = 8 + NJ;   // MFMAs and fragment reads per substep
  auto kstep = [&](int tk, int st) {
    // substep 0's MFMAs with substep 1's fragment reads spread among them
#pragma unroll
    for (int r = 0; r < kNR; ++r) {
      read_one(st, 1, 1, r);
#pragma unroll
      for (int q = (r * kNM) / kNR; q < ((r + 1) * kNM) / kNR; ++q)
        mfma_acc(acc[q / NJ][q % NJ], wf[0][q % NJ], xf[0][q / NJ]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // substep 1's MFMAs with tile tk + 2's DMAs and the next step's first
    // fragment reads spread among them
    const int tn2 = min(tk + 2, KT - 1);
#pragma unroll
    for (int o = 0; o < 2 * kLoads; ++o) {
      if (o % 2 == 0) gload_one(tn2, st, o / 2);
      else read_one(st ^ 1, 0, 0, o / 2);
#pragma unroll
      for (int q = (o * kNM) / (2 * kLoads); q < ((o + 1) * kNM) / (2 * kLoads); ++q)
        mfma_acc(acc[q / NJ][q % NJ], wf[1][q % NJ], xf[1][q / NJ]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int tk = 0;
  for (; tk + 1 < KT; tk += 2) {
    kstep(tk, 0);
    kstep(tk + 1, 1);
  }
  if (tk < KT) kstep(tk, 0);
  __builtin_amdgcn_s_waitcnt(0x0070);    // the clamped last loads and reads are done
  __syncthreads();

  // ---- output: lane (row lane & 15, columns 4g..4g+3) of block (i, j); two
  // halves of 128 rows through LDS, then 16-byte row segments
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          bf2 lo, hi;
          lo[0] = (__bf16)acc[i][j][0];
          lo[1] = (__bf16)acc[i][j][1];
          hi[0] = (__bf16)acc[i][j][2];
          hi[1] = (__bf16)acc[i][j][3];
          const int row = 16 * i + (lane & 15), col = (BN / 2) * wn + 16 * j + 4 * g;
          *reinterpret_cast<v2i*>(lds + row * kPORow + 2 * col) =
              v2i{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 128 * BN / 8 / kPThreads; ++it) {
      const int c = tid + kPThreads * it, row = c / (BN / 8), seg = c % (BN / 8);
      const int m = m0 + 128 * half + row, n = n0 + 8 * seg;
      if (m < M && n < N)
        *reinterpret_cast<v4i*>(Y + (int64_t)m * N + n) = *reinterpret_cast<const v4i*>(lds + row * kPORow + 16 * seg);
    }
    __syncthreads();
  }
}

hipError_t launch_bf16_gemm_nt(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int KT = (int)(K / kPK);
  const int tilesM = (int)((M + kPM - 1) / kPM);
  // 224-column tiles when they fill the 256 CUs in fewer rounds of tile-time
  // (e.g. N = 14336: 64 of them against 56 of 256 per tile-row)
  const int64_t t256 = tilesM * ((N + 255) / 256), t224 = tilesM * ((N + 223) / 224);
  const bool use224 = ((t224 + 255) / 256) * 224 < ((t256 + 255) / 256) * 256;
  const int tilesN = (int)(use224 ? (N + 223) / 224 : (N + 255) / 256);
  auto X = static_cast<const uint16_t*>(x);
  auto Wp = static_cast<const uint16_t*>(w);
  auto Y = static_cast<uint16_t*>(y);
  if (use224)
    hipLaunchKernelGGL(bf16_gemm_nt_kernel<224>, dim3((unsigned)(tilesM * tilesN)), dim3(kPThreads), 0, stream, X, Wp,
                       Y, (int)M, (int)N, (int)K, KT, tilesM, tilesN);
  else
    hipLaunchKernelGGL(bf16_gemm_nt_kernel<256>, dim3((unsigned)(tilesM * tilesN)), dim3(kPThreads), 0, stream, X, Wp,
                       Y, (int)M, (int)N, (int)K, KT, tilesM, tilesN);
  return hipGetLastError();
}

}  // namespace w4
