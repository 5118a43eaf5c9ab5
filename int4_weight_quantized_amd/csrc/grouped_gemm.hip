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
//   accumulators; the token scale at the end.
// - Block tile 128 rows x 128 columns, 4 waves of 64x64, K step 128, two LDS
//   stages. Activation rows are gathered by token id straight into LDS (LDS
//   DMA: each lane's source row is its token's); rows past the segment read
//   as zero. B comes through registers two K steps ahead (two register
//   sets), 8 KiB contiguous per tile, and is unpacked once per block into
//   LDS one step ahead; a step then waits only for its next A tile.
//   16-byte LDS chunks are swizzled by row & 7 and lane group g reads
//   chunks g and g + 4: bank-conflict free.
// - A two-half schedule like the W4A8 kernel's (epilogue of one half under
//   the other half's MFMAs) does not fit the registers here: the fp8
//   fragments are twice as wide, and it spills. The epilogue follows each
//   group's last MFMAs.
// - Work items (expert, row tile, column tile) are enumerated on the device
//   from expert_offsets; the grid is an upper bound and idle blocks exit.
//   The output tile goes through LDS and leaves as 16-byte row segments.
#include <type_traits>

#include "w4_device.h"

namespace w4 {

constexpr int kEM = 128, kEN = 128, kEK = 128;
constexpr int kEThreads = 256;
constexpr int kEStageA = kEM * kEK, kEStageB = kEN * kEK, kEStage = kEStageA + kEStageB;

template <int V>
using EC = std::integral_constant<int, V>;

// GT: K steps (of 128) per weight group (group = 128 * GT)
template <int GT>
__global__ __launch_bounds__(kEThreads, 2) void grouped_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ a_scale, const float* __restrict__ gsum,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets, int E,
    const uint8_t* __restrict__ Wt, int64_t w_stride, const uint16_t* __restrict__ wscale,
    uint16_t* __restrict__ out, int N, int K, int KT, int NT, int T) {
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

  const int G = K / (GT * kEK);
  const int r0 = mt * kEM, n0 = tn * kEN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  if (tid < kEM) s_tok[tid] = (r0 + tid < cnt) ? row_token[seg0 + r0 + tid] : -1;
  __syncthreads();

  // ---- loads. A: wave w's DMA i fills stage rows 32w + 8i .. +7 (one KiB),
  // lane L landing at row 32w + 8i + L/8, physical chunk L%8, and fetching
  // the logical chunk (L%8) ^ (L/8) of its row's token. A row without a
  // token gets an offset past the buffer, which reads as zero. Offsets stay
  // in the range-checked VGPR operand (T*K < 2^31, checked by the caller).
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(A, (uint32_t)((int64_t)T * K));
  const int lrow = lane >> 3, lchunk = lane & 7;
  uint32_t a_voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = s_tok[32 * wave + 8 * i + lrow];
    a_voff[i] = (tok >= 0) ? (uint32_t)tok * (uint32_t)K + 16u * (uint32_t)(lchunk ^ lrow) : 0x80000000u;
  }
  const __amdgpu_buffer_rsrc_t wrsrc =
      make_rsrc(Wt + (int64_t)e * w_stride + (int64_t)tn * KT * kTileBytes, (uint32_t)KT * kTileBytes);
  const uint32_t w_voff = 16u * tid;                   // units tid, tid + 256
  // group sums of the tile rows (threads 0..127, one row each); a row
  // without a token reads past the buffer (zero)
  const __amdgpu_buffer_rsrc_t gsrc = make_rsrc(gsum, (uint32_t)((int64_t)T * G * 4));
  const int my_tok = (tid < kEM) ? s_tok[tid] : -1;
  const uint32_t g_voff = (my_tok >= 0) ? (uint32_t)my_tok * (uint32_t)G * 4u : 0x80000000u;
  // B words and group sums of step t sit in pb[t & 1] / pgs[t & 1]: they are
  // loaded two steps ahead and stored into LDS one step ahead
  v4i pb[2][2];
  float pgs[2] = {0.f, 0.f};
  auto gload_a = [&](int tk, auto STc) {
    constexpr int ST = decltype(STc)::value;
    const uint32_t ks = (uint32_t)tk * kEK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          arsrc, (__attribute__((address_space(3))) void*)(lds + ST * kEStage + (32 * wave_u + 8 * i) * kEK), 16,
          a_voff[i] + ks, 0, 0, 0);
  };
  // three loads per call for every wave (the group sum of a row without a
  // token, or of a thread past the tile's rows, reads as zero from past the
  // buffer), so a step can wait for its A tile with a fixed vmcnt(3)
  auto gload_bg = [&](int tk, auto Pc) {
    constexpr int P = decltype(Pc)::value;
    const uint32_t ws = (uint32_t)tk * kTileBytes;
    pb[P][0] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, w_voff, ws, 0);
    pb[P][1] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, w_voff, ws + 4096u, 0);
    pgs[P] = -8.f * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gsrc, g_voff + 4u * (uint32_t)(tk / GT), 0, 0));
  };
  // B unit u (row n = u/4, K quarter q = u%4): low nibbles -> logical chunk
  // 2q (K 32q+0..15), high nibbles -> chunk 2q+1, as fp8 codes q.
  const int b_wo_lo = (tid >> 2) * kEK + 16 * ((2 * (tid & 3)) ^ ((tid >> 2) & 7));
  const int b_wo_hi = (tid >> 2) * kEK + 16 * ((2 * (tid & 3) + 1) ^ ((tid >> 2) & 7));
  auto lstore = [&](auto STc, int tk) {
    constexpr int ST = decltype(STc)::value;
    uint8_t* lb = lds + ST * kEStage + kEStageA;
    if (wave_u < 2 && (tk % GT) == 0) s_gs[ST][tid] = pgs[ST];   // stage ST holds a step of parity ST
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v4i lo, hi;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t x = (uint32_t)pb[ST][i][c] ^ 0x88888888u;   // stored q^8 -> q
        lo[c] = (int)(x & 0x0F0F0F0Fu);
        hi[c] = (int)((x >> 4) & 0x0F0F0F0Fu);
      }
      *reinterpret_cast<v4i*>(lb + b_wo_lo + 64 * kEK * i) = lo;
      *reinterpret_cast<v4i*>(lb + b_wo_hi + 64 * kEK * i) = hi;
    }
  };
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0): the DMA tile landed

  // ---- scales of group g (fp16, low half of each register), clamped columns
  const int ncol0 = n0 + 64 * wn + (lane & 15);    // column of fragment j: ncol0 + 16 j
  const __amdgpu_buffer_rsrc_t srsrc = make_rsrc(wscale + (int64_t)e * G * N, (uint32_t)((int64_t)G * N * 2));
  uint32_t s_voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s_voff[j] = 2u * (uint32_t)min(ncol0 + 16 * j, N - 1);
  auto fetch_scales = [&](int g, uint32_t (&raw)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      raw[j] = __builtin_amdgcn_raw_buffer_load_b16(srsrc, s_voff[j], (uint32_t)g * (uint32_t)N * 2u, 0);
  };

  v4f acc[4][4];
  float facc[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) facc[i][j][r] = 0.f;
    }
  auto epilogue = [&](auto I0c, auto I1c, const uint32_t (&raw)[4]) {
    constexpr int I0 = decltype(I0c)::value, I1 = decltype(I1c)::value;
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = f16_to_f32((uint16_t)raw[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) facc[i][j][r] = fmaf(acc[i][j][r], sc, facc[i][j][r]);
      }
  };

  // ---- fragments: lane row (lane & 15), lane group g = lane >> 4 takes the
  // 16-byte chunks g and g + 4 of the K step (same order for A and B)
  const int fl = lane & 7, g4 = lane >> 4;
  const int a_ro0 = (64 * wm + (lane & 15)) * kEK + 16 * (g4 ^ fl);
  const int a_ro1 = (64 * wm + (lane & 15)) * kEK + 16 * ((g4 + 4) ^ fl);
  const int b_ro0 = (64 * wn + (lane & 15)) * kEK + 16 * (g4 ^ fl);
  const int b_ro1 = (64 * wn + (lane & 15)) * kEK + 16 * ((g4 + 4) ^ fl);
  auto frag = [&](const uint8_t* base, int o0, int o1) -> v8i {
    const v4i x0 = *reinterpret_cast<const v4i*>(base + o0);
    const v4i x1 = *reinterpret_cast<const v4i*>(base + o1);
    return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  auto read_a = [&](auto STc, int i) -> v8i {
    constexpr int ST = decltype(STc)::value;
    return frag(lds + ST * kEStage + 16 * kEK * i, a_ro0, a_ro1);
  };
  auto read_b = [&](auto STc, v8i (&bf)[4]) {
    constexpr int ST = decltype(STc)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = frag(lds + ST * kEStage + kEStageA + 16 * kEK * j, b_ro0, b_ro1);
  };
  auto read_cinit = [&](auto STc, int i) -> v4f {
    constexpr int ST = decltype(STc)::value;
    return *reinterpret_cast<const v4f*>(&s_gs[ST][64 * wm + 16 * i + 4 * g4]);
  };
  auto mfma_row = [&](int i, const v8i& af, const v8i (&bf)[4], const v4f& c0, bool fresh) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], fresh ? c0 : acc[i][j], 0, 0, 0, 127,
                                                                   0, 136);
  };

  // ---- prologue
  gload_a(0, EC<0>{});
  gload_bg(0, EC<0>{});
  lstore(EC<0>{}, 0);
  gload_bg(min(1, KT - 1), EC<1>{});
  wait_loads();
  __syncthreads();

  // K step tk reads stage ST = tk & 1 while tile tk + 1 streams into the
  // other stage: A by DMA, B (loaded into registers during step tk - 1)
  // unpacked and stored at the end of the step. Past the last tile the
  // loads repeat it: the body is branch-free.
  auto kstep = [&](int tk, auto STc) {
    constexpr int ST = decltype(STc)::value;
    // this step's scales, then A of tk + 1, then B of tk + 2: the step ends
    // waiting for all but the last three loads (B and the group sums)
    const bool fresh = (tk % GT) == 0, last = (tk % GT) == GT - 1;
    uint32_t sc[4];
    fetch_scales(tk / GT, sc);
    gload_a(min(tk + 1, KT - 1), EC<ST ^ 1>{});
    gload_bg(min(tk + 2, KT - 1), EC<ST>{});        // into the registers stored last step
    v8i bf[4];
    read_b(EC<ST>{}, bf);
    // one row's A fragment and C init at a time (bounds the live registers)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mfma_row(i, read_a(EC<ST>{}, i), bf, read_cinit(EC<ST>{}, i), fresh);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (last) epilogue(EC<0>{}, EC<4>{}, sc);
    lstore(EC<ST ^ 1>{}, tk + 1);
    __builtin_amdgcn_s_waitcnt(0x0F73);   // vmcnt(3): A of step tk + 1 landed; step tk + 2's B may stay in flight
    __syncthreads();
  };

  // (the two loop shapes are equivalent; each is the one the register
  // allocator handles without spills for its group size)
  if constexpr (GT == 4) {
    int tk = 0;
    for (; tk + 1 < KT; tk += 2) {
      kstep(tk, EC<0>{});
      kstep(tk + 1, EC<1>{});
    }
    if (tk < KT) kstep(tk, EC<0>{});
  } else {
    for (int tk = 0; tk < KT; ++tk) {
      if (tk & 1) kstep(tk, EC<1>{});
      else kstep(tk, EC<0>{});
    }
  }

  // ---- output: row scale, bf16, staged through LDS (free after the last
  // barrier) and written as 16-byte row segments (N is a multiple of 8)
  constexpr int kORow = kEN * 2 + 16;
  static_assert(kEM * kORow <= 2 * kEStage, "output tile fits the stage buffers");
  const int orow0 = 64 * wm + 4 * g4, ocol0 = 64 * wn + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = s_tok[orow0 + 16 * i + r];
      const float sa = a_scale[max(tok, 0)];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint16_t*>(lds + (orow0 + 16 * i + r) * kORow + 2 * (ocol0 + 16 * j)) =
            f32_to_bf16_rne(facc[i][j][r] * sa);
    }
  __syncthreads();
  const int rows = min(kEM, cnt - r0);
#pragma unroll
  for (int it = 0; it < kEM * kEN / 8 / kEThreads; ++it) {
    const int c = tid + kEThreads * it, row = c >> 4, seg = c & 15;
    const int n = n0 + 8 * seg;
    if (row < rows && n < N)
      *reinterpret_cast<v4i*>(out + (int64_t)(seg0 + r0 + row) * N + n) =
          *reinterpret_cast<const v4i*>(lds + row * kORow + 16 * seg);
  }
}

hipError_t launch_grouped_fp8(const void* a, const float* a_scale, const float* gsum,
                              const int32_t* row_token, const int32_t* offsets, int64_t E,
                              const void* w_tiled, size_t w_bytes_per_expert, const void* w_scale,
                              int64_t group, void* out, int64_t T, int64_t R, int64_t N, int64_t K,
                              hipStream_t stream) {
  if (R == 0 || N == 0 || E == 0) return hipSuccess;
  const int KT = (int)(K / kEK), NT = (int)((N + kEN - 1) / kEN);
  const int64_t upper = ((R + kEM - 1) / kEM + E) * NT;
  dim3 grid((unsigned)upper), block(kEThreads);
  auto Ap = static_cast<const uint8_t*>(a);
  auto Wp = static_cast<const uint8_t*>(w_tiled);
  auto Sp = static_cast<const uint16_t*>(w_scale);
  auto Op = static_cast<uint16_t*>(out);
  const int64_t ws = (int64_t)w_bytes_per_expert;
  switch (group / kEK) {
    case 1: hipLaunchKernelGGL((grouped_fp8_kernel<1>), grid, block, 0, stream, Ap, a_scale, gsum, row_token, offsets,
                               (int)E, Wp, ws, Sp, Op, (int)N, (int)K, KT, NT, (int)T); break;
    case 2: hipLaunchKernelGGL((grouped_fp8_kernel<2>), grid, block, 0, stream, Ap, a_scale, gsum, row_token, offsets,
                               (int)E, Wp, ws, Sp, Op, (int)N, (int)K, KT, NT, (int)T); break;
    default: hipLaunchKernelGGL((grouped_fp8_kernel<4>), grid, block, 0, stream, Ap, a_scale, gsum, row_token, offsets,
                                (int)E, Wp, ws, Sp, Op, (int)N, (int)K, KT, NT, (int)T); break;
  }
  return hipGetLastError();
}

}  // namespace w4
