// W4A8 GEMM on the int8 MFMA datapath with a fused per-group epilogue.
//
// Per the inc_w4a8_linear page (INCXPUW4A8LinearMethod docstring and
// apply_weights): int8 per-token activation codes times int4 GPTQ weights
// with fp16 per-group (or per-channel) scales, bias fused, output in the
// activation dtype; the int8 path avoids upconverting the weights.
//
//   P[m,g,n] = sum_{k in g} a[m,k] * (q[k,n] - 8)            (int32, exact)
//   out[m,n] = a_scale[m] * sum_g w_scale[g,n] * P[m,g,n] + bias[n]
//
// Design (gfx950):
// - 256 threads, block tile 128x128, four waves of 64x64, K step 128,
//   two LDS stages (64 KiB) so two blocks share a CU.
// - A (int8 codes) streams global -> LDS with 16-byte raw buffer loads
//   whose range check zero-fills rows past M and bytes past the matrix.
// - B is read from the tiled int4 layout (8 KiB contiguous per tile, fully
//   coalesced) and unpacked once per block into LDS as int8 bytes equal to
//   16*(q-8): the stored nibble is q^8, so a mask (and a 4-bit shift) is the
//   whole unpack. The MFMA therefore accumulates 16*P; the factor 1/16 is
//   folded into the final per-row scale (exact: a power of two).
// - LDS rows are 128 bytes; 16-byte chunks are XOR-swizzled by (row & 7) so
//   both the tile writes and the MFMA fragment reads are conflict-free.
// - v_mfma_i32_16x16x64_i8: each wave issues 16 MFMAs per 64-deep chunk. At
//   a K-group boundary the int32 sums are converted and FMA'd into fp32
//   accumulators with the group's fp16 scale; the next chunk restarts the
//   int32 sums with C = 0.
// - Tiles are visited in groups of 8 tile-rows, and block ids are remapped
//   so each XCD (own L2) works on a contiguous range of tiles.
#include "w4_device.h"

namespace w4 {

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kGThreads = 256;
constexpr int kStageA = kBM * kBK;               // bytes
constexpr int kStageB = kBN * kBK;
constexpr int kStage = kStageA + kStageB;

__device__ __forceinline__ int swz(int row, int kc) { return row * 128 + ((kc ^ (row & 7)) << 4); }

enum { kModeGroup = 0, kModeChannel = 1, kModePartials = 2 };

// GC: 64-deep chunks per weight group when known at compile time (1: group
// 64, 2: group 128), 0: taken from group_chunks at run time.
template <int MODE, bool OUT_BF16, int GC>
__global__ __launch_bounds__(kGThreads, 2) void w4a8_gemm_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ a_scale,
    const v4i* __restrict__ Wt, const uint16_t* __restrict__ wscale, int group_chunks_rt,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
    int32_t* __restrict__ partials, int M, int N, int K, int KT, int tilesM, int tilesN) {
  const int group_chunks = GC > 0 ? GC : group_chunks_rt;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];

  // ---- tile of this block
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  constexpr int GM = 8;
  const int per_group = GM * tilesN;
  const int first_m = (t / per_group) * GM;
  const int gsz = min(tilesM - first_m, GM);
  const int tm = first_m + (t % per_group) % gsz;
  const int tn = (t % per_group) / gsz;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nchunks = (K + 63) >> 6;
  const int G = (MODE == kModeChannel) ? 1 : nchunks / group_chunks;

  // ---- global -> register staging
  const int rows_valid = min(kBM, M - m0);
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(A + (int64_t)m0 * K, (uint32_t)rows_valid * (uint32_t)K);
  const int arow0 = tid >> 3, akc = tid & 7;
  v4i pa[4], pb[2];
  auto gload = [&](int tk) {
    const uint32_t k0 = (uint32_t)tk * kBK + 16u * akc;
#pragma unroll
    for (int i = 0; i < 4; ++i) pa[i] = buffer_load16(arsrc, (uint32_t)(arow0 + 32 * i) * (uint32_t)K + k0);
    const v4i* wt = Wt + (((int64_t)tn * KT + tk) << 9);
    pb[0] = wt[tid];
    pb[1] = wt[tid + kGThreads];
  };
  auto lstore = [&](int stage) {
    uint8_t* la = lds + stage * kStage;
    uint8_t* lb = la + kStageA;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(la + swz(arow0 + 32 * i, akc)) = pa[i];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + kGThreads * i, nl = u >> 2, kq = u & 3;
      v4i lo, hi;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lo[c] = (int)(((uint32_t)pb[i][c] << 4) & 0xF0F0F0F0u);
        hi[c] = (int)((uint32_t)pb[i][c] & 0xF0F0F0F0u);
      }
      *reinterpret_cast<v4i*>(lb + swz(nl, 2 * kq)) = lo;
      *reinterpret_cast<v4i*>(lb + swz(nl, 2 * kq + 1)) = hi;
    }
  };

  // ---- accumulators
  v4i acc[4][4];
  float facc[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) facc[i][j][r] = 0.f;
    }

  int ncol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ncol[j] = n0 + 64 * wn + 16 * j + (lane & 15);
  const int mrow0 = m0 + 64 * wm + 4 * (lane >> 4);   // + 16*i + r

  // Unconditional loads at clamped indices (no branch, no early wait); the
  // value of a column past N is never stored.
  int ncl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ncl[j] = min(ncol[j], N - 1);
  auto load_scales_raw = [&](int g, uint16_t (&raw)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = wscale[(int64_t)g * N + ncl[j]];
  };
  auto load_scales = [&](int g, float (&sc)[4]) {
    uint16_t raw[4];
    load_scales_raw(g, raw);
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = f16_to_f32(raw[j]);
  };

  auto group_end = [&](int g, const float (&sc)[4]) {
    if (MODE == kModePartials) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mrow0 + 16 * i + r;
          if (m >= M) continue;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (ncol[j] < N) partials[((int64_t)m * G + g) * N + ncol[j]] = acc[i][j][r] >> 4;
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) facc[i][j][r] = fmaf((float)acc[i][j][r], sc[j], facc[i][j][r]);
    }
  };

  auto compute_chunk = [&](int stage, int c, bool fresh) {
    const uint8_t* la = lds + stage * kStage;
    const uint8_t* lb = la + kStageA;
    const int kc = 4 * c + (lane >> 4);
    v4i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const v4i*>(la + swz(64 * wm + 16 * i + (lane & 15), kc));
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const v4i*>(lb + swz(64 * wn + 16 * j + (lane & 15), kc));
    if (fresh) {
      const v4i z = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], z, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // ---- main loop: two LDS stages, one barrier per K step. The scales of the
  // groups ending in K step tk+1 are fetched during step tk.
  uint16_t scr[2][4];
  auto fetch_step_scales = [&](int tk) {
    if (MODE != kModeGroup) return;
    const int cg0 = 2 * tk;
    load_scales_raw(min(cg0 / group_chunks, G - 1), scr[0]);
    load_scales_raw(min((cg0 + 1) / group_chunks, G - 1), scr[1]);
  };
  gload(0);
  fetch_step_scales(0);
  lstore(0);
  __syncthreads();
  for (int tk = 0; tk < KT; ++tk) {
    const int stage = tk & 1;
    const bool more = tk + 1 < KT;
    float sc[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[c][j] = f16_to_f32(scr[c][j]);
    if (more) {
      gload(tk + 1);
      fetch_step_scales(tk + 1);
    }
    const int cg0 = 2 * tk;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int cg = cg0 + c;
      if (cg >= nchunks) break;
      const bool fresh = (MODE == kModeChannel) ? (cg == 0) : (cg % group_chunks == 0);
      compute_chunk(stage, c, fresh);
      if (MODE != kModeChannel && (cg + 1) % group_chunks == 0) group_end(cg / group_chunks, sc[c]);
    }
    if (more) lstore(stage ^ 1);
    __syncthreads();
  }
  if (MODE == kModePartials) return;

  if (MODE == kModeChannel) {
    float sc[4];
    load_scales(0, sc);
    group_end(0, sc);
  }

  // ---- output: out = facc * a_scale / 16 + bias
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  if (bias) {
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = OUT_BF16 ? bf16_to_f32(bias[ncl[j]]) : f16_to_f32(bias[ncl[j]]);
  }
  float sa[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) sa[i][r] = a_scale[min(mrow0 + 16 * i + r, M - 1)] * 0.0625f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mrow0 + 16 * i + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = ncol[j];
        const float y = fmaf(facc[i][j][r], sa[i][r], bv[j]);
        if (m < M && n < N) out[(int64_t)m * N + n] = OUT_BF16 ? f32_to_bf16_rne(y) : f32_to_f16_rne(y);
      }
    }
}

hipError_t launch_w4a8_gemm(const int8_t* a, const float* a_scale, const void* w_tiled,
                            const void* w_scale, int64_t group, const void* bias, void* out,
                            bool out_bf16, int32_t* partials, int64_t M, int64_t N, int64_t K,
                            hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int KT = (int)((K + kBK - 1) / kBK);
  const int tilesM = (int)((M + kBM - 1) / kBM), tilesN = (int)((N + kBN - 1) / kBN);
  const int nchunks = (int)((K + 63) / 64);
  const int gc = (group == -1) ? nchunks : (int)(group / 64);
  dim3 grid((unsigned)(tilesM * tilesN)), block(kGThreads);
  auto W = static_cast<const v4i*>(w_tiled);
  auto S = static_cast<const uint16_t*>(w_scale);
  auto B = static_cast<const uint16_t*>(bias);
  auto O = static_cast<uint16_t*>(out);
  const int iM = (int)M, iN = (int)N, iK = (int)K;
#define W4A8_LAUNCH(MODE_, BF16_, GC_)                                                                  \
  hipLaunchKernelGGL((w4a8_gemm_kernel<MODE_, BF16_, GC_>), grid, block, 0, stream, a, a_scale, W, S, gc, B, O, \
                     partials, iM, iN, iK, KT, tilesM, tilesN)
  if (partials) {
    W4A8_LAUNCH(kModePartials, true, 0);
  } else if (group == -1) {
    if (out_bf16) W4A8_LAUNCH(kModeChannel, true, 0); else W4A8_LAUNCH(kModeChannel, false, 0);
  } else if (gc == 1) {
    if (out_bf16) W4A8_LAUNCH(kModeGroup, true, 1); else W4A8_LAUNCH(kModeGroup, false, 1);
  } else if (gc == 2) {
    if (out_bf16) W4A8_LAUNCH(kModeGroup, true, 2); else W4A8_LAUNCH(kModeGroup, false, 2);
  } else {
    if (out_bf16) W4A8_LAUNCH(kModeGroup, true, 0); else W4A8_LAUNCH(kModeGroup, false, 0);
  }
#undef W4A8_LAUNCH
  return hipGetLastError();
}

}  // namespace w4
