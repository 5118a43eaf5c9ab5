// Weight-only int4 GEMM for few rows (M <= 16) on the W4A8 kernel-tiled
// weights, activations unquantized (bf16 or fp16):
//
//   out[m,n] = sum_g w_scale[g,n] * sum_{k in g} x[m,k] * (q[k,n] - 8)  (+ bias[n])
//
// Per the inc_w4a8 page (INCXPUW4A8LinearMethod: class docstring and
// apply_weights): the int8 and the weight-only int4 kernels take bit-identical
// weights, and below a token-count threshold the layer calls the weight-only
// kernel per call, since per-token quantization would dominate there.
//
// Design (gfx950): bound by the weight stream, like the decode kernel.
// - v_mfma_f32_16x16x32_{bf16,f16}: activation rows are the 16-row A operand
//   (rows >= M read as zero), 16 weight columns the B operand.
// - Each wave loads a column group's 1 KiB unit block per 128-K tile with one
//   16-byte load per lane (lane L = unit (column L/4, K quarter L%4)) and
//   regroups it through a wave-private LDS buffer, so that lane (n, j) holds
//   word j of the units (n, kq) for kq = 0..3: one word per 32-K step. (Four
//   4-byte global loads per lane instead measured twice as slow.) A word
//   holds the codes of K offsets k..k+3 (low nibbles) and k+16..k+19 (high
//   nibbles), k = 32 kq + 4 j, stored as q ^ 8. After w ^= 0x88888888, ((w >> 4i) & 0x000F000F) | magic
//   is register i of the B fragment: the codes at bits 4i and 16 + 4i, i.e.
//   K offsets {0,2}, {16,18}, {1,3}, {17,19}. The A fragment is loaded as
//   x[k..k+3] and x[k+16..k+19] and put in the same order with v_perm_b32,
//   once per K range; every column group reuses it.
// - bf16: magic 0x4300 gives 128 + q; fp16: magic 0x5800 gives 128 + q/8;
//   both exact. Row sums XS come from an MFMA against ones, and each group's
//   accumulator starts at -(128 + 8c) XS (c = 1 or 1/8), so it ends at
//   c * sum x (q - 8); the epilogue adds (scale / c) * C.
// - A 1024-thread block owns RT groups of 16 columns. Its 16 waves take 256 K
//   each (two 128-K tiles) of a 4096-wide pass. The next column group's loads
//   are issued before the current one is computed. The 16 partial tiles are
//   summed through LDS; bias and the cast come last.
#include "w4_device.h"

namespace w4 {

constexpr int kTBlock = 1024;
constexpr int kTWaves = kTBlock / kWave;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

template <bool F16>
__device__ __forceinline__ v4f mfma16(v4i a, v4i b, v4f c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                   0);
}

// RT: column groups per block; CPG: 32-K steps per group part (2: group 64,
// 4: group 128, 8: a wave's whole 256-K range inside one group); MV:
// accumulator registers holding real rows (M == 1: 1, M == 2: 2, else 4).
template <int RT, int CPG, int MV, bool F16>
__global__ __launch_bounds__(kTBlock, 1) void w4a16_tiled_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wt, const uint16_t* __restrict__ wscale,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int M, int N, int K, int KT, int NCG, int geff) {
  constexpr int NP = 8 / CPG;                                   // group parts per wave range
  __shared__ __attribute__((aligned(16))) float red[kTWaves][RT][kWave][MV];
  // per wave: the current column group's two 1 KiB unit blocks, unit (n, kq)
  // at n * 72 + kq * 16 bytes (rows padded by 8 bytes against bank conflicts)
  __shared__ __attribute__((aligned(16))) uint8_t shuf[kTWaves][2][16 * 72];
  const int tid = threadIdx.x, lane = tid & 63;
  const int l16 = lane & 15, j = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg0 = blockIdx.x * RT;
  const int G = K / geff;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wt, (uint32_t)((int64_t)((NCG + 7) / 8) * KT * kTileBytes));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(wscale, (uint32_t)((int64_t)G * N * 2));
  const uint32_t w_lane = 16u * lane;                           // unit lane = (column lane/4, kq lane%4)
  uint8_t* const sh_w = &shuf[wave][0][0] + 72 * (lane >> 2) + 16 * (lane & 3);   // this lane's unit
  const uint8_t* const sh_r = &shuf[wave][0][0] + 72 * l16 + 4 * j;             // word j of (column l16, kq)

  // bf16: 128 + q (c = 1); fp16: 128 + q/8 (c = 1/8)
  constexpr float kInit = F16 ? -129.f : -136.f;                // -(128 + 8c)
  constexpr float kInvC = F16 ? 8.f : 1.f;
  const v4i ones = F16 ? v4i{0x3C003C00, 0x3C003C00, 0x3C003C00, 0x3C003C00}
                       : v4i{0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80};
  const v4f z4 = {0.f, 0.f, 0.f, 0.f};
  uint32_t mask_s, magic_v;
  asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(mask_s));
  if constexpr (F16)
    asm volatile("v_mov_b32 %0, 0x58005800" : "=v"(magic_v));
  else
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(magic_v));

  float y[RT][MV];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int r = 0; r < MV; ++r) y[t][r] = 0.f;

  for (int kt0 = 2 * wave; kt0 < KT; kt0 += 2 * kTWaves) {
    const int kbase = kt0 * kTileK;
    // ---- activation fragments of the 8 steps (rows >= M and K >= K read zero)
    v4i xf[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int k = kbase + 128 * (c >> 2) + 32 * (c & 3) + 4 * j;
      // K is a multiple of 8, so each 4-value run is wholly inside or past K
      const uint32_t row = (uint32_t)(l16 * K + k) * 2u;
      const uint32_t offx = (k < K) ? row : 0x80000000u, offy = (k + 16 < K) ? row + 32u : 0x80000000u;
      const v2i X = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(xr, offx, 0, 0));
      const v2i Y = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(xr, offy, 0, 0));
      xf[c] = v4i{(int)__builtin_amdgcn_perm((uint32_t)X[1], (uint32_t)X[0], 0x05040100u),
                  (int)__builtin_amdgcn_perm((uint32_t)Y[1], (uint32_t)Y[0], 0x05040100u),
                  (int)__builtin_amdgcn_perm((uint32_t)X[1], (uint32_t)X[0], 0x07060302u),
                  (int)__builtin_amdgcn_perm((uint32_t)Y[1], (uint32_t)Y[0], 0x07060302u)};
    }
    // ---- weights and scales of column group t: 8 words, NP scales
    v4i wv[RT][2];
    uint32_t sv[RT][NP];
    auto load_group = [&](int t) {
      const int cg = min(cg0 + t, NCG - 1);                     // past the last group: reload it, not stored
      const int nt = cg >> 3;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kt = min(kt0 + h, KT - 1);
        const uint32_t tile = (uint32_t)(nt * KT + kt) * kTileBytes + (uint32_t)(cg & 7) * 1024u;
        wv[t][h] = __builtin_amdgcn_raw_buffer_load_b128(wr, w_lane, tile, 0);
      }
      const uint32_t col = (uint32_t)min(16 * cg + l16, N - 1);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int g = min((kbase + 32 * CPG * p) / geff, G - 1);
        sv[t][p] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(sr, 2u * col, (uint32_t)g * (uint32_t)N * 2u, 0);
      }
    };
    load_group(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- row sums per group part; each part's accumulator starts at kInit * XS
    v4f xs_init[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      v4f run = z4;
#pragma unroll
      for (int c = CPG * p; c < CPG * (p + 1); ++c) run = mfma16<F16>(xf[c], ones, run);
#pragma unroll
      for (int r = 0; r < 4; ++r) xs_init[p][r] = (r < MV) ? kInit * run[r] : 0.f;
    }

#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if (t + 1 < RT) load_group(t + 1);        // next column group in flight while this one computes
      __builtin_amdgcn_sched_barrier(0);
      // regroup through LDS: lane (n, j) needs word j of units (n, 0..3)
      uint32_t wd[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<v2i*>(sh_w + h * 16 * 72) = v2i{wv[t][h][0], wv[t][h][1]};
        *reinterpret_cast<v2i*>(sh_w + h * 16 * 72 + 8) = v2i{wv[t][h][2], wv[t][h][3]};
      }
#pragma unroll
      for (int c = 0; c < 8; ++c)
        wd[c] = *reinterpret_cast<const uint32_t*>(sh_r + (c >> 2) * 16 * 72 + 16 * (c & 3));
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        v4f acc = xs_init[p];
#pragma unroll
        for (int c = CPG * p; c < CPG * (p + 1); ++c) {
          const uint32_t w = wd[c] ^ 0x88888888u;               // stored q ^ 8 -> q
          const v4i b = {(int)((w & mask_s) | magic_v), (int)(((w >> 4) & mask_s) | magic_v),
                         (int)(((w >> 8) & mask_s) | magic_v), (int)(((w >> 12) & mask_s) | magic_v)};
          acc = mfma16<F16>(xf[c], b, acc);
        }
        const float s = kInvC * f16_to_f32((uint16_t)sv[t][p]);
#pragma unroll
        for (int r = 0; r < MV; ++r) y[t][r] = fmaf(s, acc[r], y[t][r]);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int r = 0; r < MV; ++r) red[wave][t][lane][r] = y[t][r];
  __syncthreads();
  for (int e = tid; e < RT * 256; e += kTBlock) {
    const int t = e >> 8, m = (e >> 4) & 15, nn = e & 15;   // output (m, 16*(cg0+t) + nn)
    const int l = nn + 16 * (m >> 2), r = m & 3;
    const int n = 16 * (cg0 + t) + nn;
    if (m < M && n < N && cg0 + t < NCG) {
      float acc = 0.f;
#pragma unroll
      for (int w_ = 0; w_ < kTWaves; ++w_) acc += red[w_][t][l][r < MV ? r : 0];
      if (bias) acc += F16 ? f16_to_f32(bias[n]) : bf16_to_f32(bias[n]);
      out[(int64_t)m * N + n] = F16 ? f32_to_f16_rne(acc) : f32_to_bf16_rne(acc);
    }
  }
}

hipError_t launch_w4a16_tiled(const void* x, bool f16, const void* w_tiled, const void* w_scale, int64_t group,
                              const void* bias, void* out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int KT = (int)((K + kTileK - 1) / kTileK), NCG = (int)((N + 15) / 16);
  const int geff = (int)(group == -1 ? K : group);
  // A group part (CPG 32-K steps at a multiple of its own length) must lie in
  // one group, since it is scaled by the group of its first K: parts of 256
  // when groups are multiples of 256 (or there is one group), of 128 when
  // they are multiples of 128, else of 64 (groups are multiples of 64).
  const int cpg = (geff % 256 == 0 || geff >= K) ? 8 : (geff % 128 == 0 ? 4 : 2);
  int rt = (NCG + 255) / 256;
  rt = rt <= 1 ? 1 : (rt == 2 ? 2 : 4);
  const int mv = M == 1 ? 1 : (M == 2 ? 2 : 4);
  dim3 grid((unsigned)((NCG + rt - 1) / rt)), block(kTBlock);
  auto X = static_cast<const uint16_t*>(x);
  auto Wt = static_cast<const uint8_t*>(w_tiled);
  auto S = static_cast<const uint16_t*>(w_scale);
  auto B = static_cast<const uint16_t*>(bias);
  auto O = static_cast<uint16_t*>(out);
  const int iM = (int)M, iN = (int)N, iK = (int)K;
#define W4T_LAUNCH(RT_, CPG_, MV_, F_)                                                                          \
  hipLaunchKernelGGL((w4a16_tiled_kernel<RT_, CPG_, MV_, F_>), grid, block, 0, stream, X, Wt, S, B, O, iM, iN, iK, \
                     KT, NCG, geff)
#define W4T_F(RT_, CPG_, MV_)              \
  if (f16) W4T_LAUNCH(RT_, CPG_, MV_, true); \
  else W4T_LAUNCH(RT_, CPG_, MV_, false);
#define W4T_MV(RT_, CPG_)                      \
  switch (mv) {                                \
    case 1: W4T_F(RT_, CPG_, 1) break;         \
    case 2: W4T_F(RT_, CPG_, 2) break;         \
    default: W4T_F(RT_, CPG_, 4) break;        \
  }
#define W4T_RT(CPG_)                   \
  switch (rt) {                        \
    case 1: W4T_MV(1, CPG_) break;     \
    case 2: W4T_MV(2, CPG_) break;     \
    default: W4T_MV(4, CPG_) break;    \
  }
  switch (cpg) {
    case 2: W4T_RT(2) break;
    case 4: W4T_RT(4) break;
    default: W4T_RT(8) break;
  }
#undef W4T_RT
#undef W4T_MV
#undef W4T_F
#undef W4T_LAUNCH
  return hipGetLastError();
}

}  // namespace w4
