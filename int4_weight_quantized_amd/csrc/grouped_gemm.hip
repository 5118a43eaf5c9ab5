// Grouped W4A-FP8 GEMM over routed-expert segments.
//
// Per the w4afp8 page (W4AFP8Config, get_quant_method for RoutedExperts):
// routed experts hold int4 group-128 weights, symmetric (zero point 8), and
// take per-token dynamic FP8 activations. For routed row r of expert e with
// token t = row_token[r]:
//   out[r,n] = a_scale[t] * sum_g w_scale[e,g,n] * sum_{k in g} a[t,k]*(q[e,k,n]-8)
//
// Design (gfx950): v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 operands.
// - The weight byte q (0..15) is itself the E4M3 encoding of q * 2^-9: the
//   subnormals (0x00-0x07) and the first normal binade (0x08-0x0F) are evenly
//   spaced by 2^-9. So the int4 -> fp8 unpack is a mask, and the B block
//   scale 2^9 (E8M0 136) makes the product exact in q.
// - The zero point enters through the accumulator: the first MFMA of each
//   group starts from C[m][.] = -8 * sum_{k in g} a[t_m,k] (row sums written
//   by the activation quantizer), so D = sum_k a*(q-8) for every column.
// - The group's fp16 scale is applied with one FMA per output into fp32
//   accumulators; the token scale at the end; bf16 output in row order.
// - Block tile 128 rows x 128 columns, 4 waves of 64x64, K step 128, two LDS
//   stages; activation rows are gathered by token id while staging to LDS.
// - Work items (expert, row tile, column tile) are enumerated on the device
//   from expert_offsets; the grid is an upper bound and idle blocks exit.
#include "w4_device.h"

namespace w4 {

constexpr int kEM = 128, kEN = 128, kEK = 128;
constexpr int kEThreads = 256;
constexpr int kEStageA = kEM * kEK, kEStageB = kEN * kEK, kEStage = kEStageA + kEStageB;

__device__ __forceinline__ int eswz(int row, int kc) { return row * 128 + ((kc ^ (row & 7)) << 4); }

// GT: K steps (of 128) per weight group (group = 128 * GT)
template <int GT>
__global__ __launch_bounds__(kEThreads, 2) void grouped_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ a_scale, const float* __restrict__ gsum,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets, int E,
    const v4i* __restrict__ Wt, int64_t w_stride16, const uint16_t* __restrict__ wscale,
    uint16_t* __restrict__ out, int N, int K, int KT, int NT) {
  constexpr int group_tiles = GT;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kEStage];
  __shared__ int s_tok[kEM];                       // token of each row of the tile (-1: none)
  __shared__ __attribute__((aligned(16))) float s_gs[2][kEM];   // -8 * row sum of the staged group

  // ---- work item of this block
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  int e = -1, mt = 0, tn = 0, seg0 = 0, cnt = 0;
  {
    int cum = 0;
    for (int ee = 0; ee < E; ++ee) {
      const int o0 = offsets[ee], o1 = offsets[ee + 1];
      const int mtiles = (o1 - o0 + kEM - 1) / kEM;
      const int tiles = mtiles * NT;
      if (t < cum + tiles) {
        const int local = t - cum;
        e = ee; mt = local % mtiles; tn = local / mtiles; seg0 = o0; cnt = o1 - o0;
        break;
      }
      cum += tiles;
    }
  }
  if (e < 0) return;                       // idle block (grid is an upper bound)

  const int G = K / (group_tiles * kEK);
  const int r0 = mt * kEM, n0 = tn * kEN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- staging: activation rows gathered by token
  if (tid < kEM) s_tok[tid] = (r0 + tid < cnt) ? row_token[seg0 + r0 + tid] : -1;
  __syncthreads();
  const int arow0 = tid >> 3, akc = tid & 7;
  const uint8_t* abase = A + 16 * akc;
  const v4i* wexp = Wt + (int64_t)e * w_stride16;
  v4i pa[4], pb[2];
  float pgs = 0.f;
  auto gload = [&](int tk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk_ = s_tok[arow0 + 32 * i];          // LDS read: no live register per row
      const v4i v = *reinterpret_cast<const v4i*>(abase + (int64_t)max(tk_, 0) * K + (int64_t)tk * kEK);
      pa[i] = (tk_ >= 0) ? v : v4i{0, 0, 0, 0};
    }
    const v4i* wt = wexp + (((int64_t)tn * KT + tk) << 9);
    pb[0] = wt[tid];
    pb[1] = wt[tid + kEThreads];
    if (tid < kEM && (tk % group_tiles) == 0) {
      const int tk_ = s_tok[tid];
      const float v = gsum[(int64_t)max(tk_, 0) * G + tk / group_tiles];   // clamped: no branch
      pgs = (tk_ >= 0) ? -8.f * v : 0.f;
    }
  };
  auto lstore = [&](int stage, int tk) {
    uint8_t* la = lds + stage * kEStage;
    uint8_t* lb = la + kEStageA;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(la + eswz(arow0 + 32 * i, akc)) = pa[i];
    if (tid < kEM && (tk % group_tiles) == 0) s_gs[stage][tid] = pgs;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + kEThreads * i, nl = u >> 2, kq = u & 3;
      v4i lo, hi;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t x = (uint32_t)pb[i][c] ^ 0x88888888u;   // stored q^8 -> q
        lo[c] = (int)(x & 0x0F0F0F0Fu);
        hi[c] = (int)((x >> 4) & 0x0F0F0F0Fu);
      }
      *reinterpret_cast<v4i*>(lb + eswz(nl, 2 * kq)) = lo;
      *reinterpret_cast<v4i*>(lb + eswz(nl, 2 * kq + 1)) = hi;
    }
  };

  // ---- per-lane output rows / columns
  const int ncol0 = n0 + 64 * wn + (lane & 15);    // column of fragment j: ncol0 + 16 j
  // scales of the group that ends in a K step, fetched one step ahead
  uint16_t scr[4];
  auto fetch_scales = [&](int tk) {
    const int g = tk / group_tiles;
#pragma unroll
    for (int j = 0; j < 4; ++j) scr[j] = wscale[((int64_t)e * G + g) * N + min(ncol0 + 16 * j, N - 1)];
  };
  v4f acc[4][4];
  float facc[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) facc[i][j][r] = 0.f;

  gload(0);
  fetch_scales(0);
  lstore(0, 0);
  __syncthreads();
  for (int tk = 0; tk < KT; ++tk) {
    const int stage = tk & 1;
    const bool more = tk + 1 < KT;
    const bool fresh = (tk % group_tiles) == 0;
    const bool last = (tk % group_tiles) == group_tiles - 1;
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = f16_to_f32(scr[j]);
    if (more) {
      gload(tk + 1);
      fetch_scales(tk + 1);
    }
    const uint8_t* la = lds + stage * kEStage;
    const uint8_t* lb = la + kEStageA;
    // lane group g takes 16-byte chunks g and g + 4 of the K step (same
    // order for A and B); this read pattern is bank-conflict free
    const int kc = lane >> 4;
    v8i bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 64 * wn + 16 * j + (lane & 15);
      const v4i x0 = *reinterpret_cast<const v4i*>(lb + eswz(row, kc));
      const v4i x1 = *reinterpret_cast<const v4i*>(lb + eswz(row, kc + 4));
      bf[j] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
    if (fresh) {
      // first K step of a group: the accumulator starts at -8 * row sum
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 64 * wm + 16 * i + (lane & 15);
        const v4i x0 = *reinterpret_cast<const v4i*>(la + eswz(row, kc));
        const v4i x1 = *reinterpret_cast<const v4i*>(la + eswz(row, kc + 4));
        const v8i af = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        const v4f cinit = *reinterpret_cast<const v4f*>(&s_gs[stage][64 * wm + 16 * i + 4 * (lane >> 4)]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], cinit, 0, 0, 0, 127, 0, 136);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 64 * wm + 16 * i + (lane & 15);
        const v4i x0 = *reinterpret_cast<const v4i*>(la + eswz(row, kc));
        const v4i x1 = *reinterpret_cast<const v4i*>(la + eswz(row, kc + 4));
        const v8i af = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 0, 0, 0, 127, 0, 136);
      }
    }
    if (last) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) facc[i][j][r] = fmaf(acc[i][j][r], sc[j], facc[i][j][r]);
    }
    if (more) lstore(stage ^ 1, tk + 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = 64 * wm + 16 * i + 4 * (lane >> 4) + r;
      const int tk_ = s_tok[lr];
      if (tk_ < 0) continue;
      const int rr = seg0 + r0 + lr;
      const float sa = a_scale[tk_];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ncol0 + 16 * j < N) out[(int64_t)rr * N + ncol0 + 16 * j] = f32_to_bf16_rne(facc[i][j][r] * sa);
    }
}

hipError_t launch_grouped_fp8(const void* a, const float* a_scale, const float* gsum,
                              const int32_t* row_token, const int32_t* offsets, int64_t E,
                              const void* w_tiled, size_t w_bytes_per_expert, const void* w_scale,
                              int64_t group, void* out, int64_t T, int64_t R, int64_t N, int64_t K,
                              hipStream_t stream) {
  (void)T;
  if (R == 0 || N == 0 || E == 0) return hipSuccess;
  const int KT = (int)(K / kEK), NT = (int)((N + kEN - 1) / kEN);
  const int64_t upper = ((R + kEM - 1) / kEM + E) * NT;
  dim3 grid((unsigned)upper), block(kEThreads);
  auto Ap = static_cast<const uint8_t*>(a);
  auto Wp = static_cast<const v4i*>(w_tiled);
  auto Sp = static_cast<const uint16_t*>(w_scale);
  auto Op = static_cast<uint16_t*>(out);
  const int64_t ws = (int64_t)(w_bytes_per_expert / 16);
  switch (group / kEK) {
    case 1: hipLaunchKernelGGL((grouped_fp8_kernel<1>), grid, block, 0, stream, Ap, a_scale, gsum, row_token, offsets,
                               (int)E, Wp, ws, Sp, Op, (int)N, (int)K, KT, NT); break;
    case 2: hipLaunchKernelGGL((grouped_fp8_kernel<2>), grid, block, 0, stream, Ap, a_scale, gsum, row_token, offsets,
                               (int)E, Wp, ws, Sp, Op, (int)N, (int)K, KT, NT); break;
    default: hipLaunchKernelGGL((grouped_fp8_kernel<4>), grid, block, 0, stream, Ap, a_scale, gsum, row_token, offsets,
                                (int)E, Wp, ws, Sp, Op, (int)N, (int)K, KT, NT); break;
  }
  return hipGetLastError();
}

}  // namespace w4
