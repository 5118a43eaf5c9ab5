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
//   spaced by 2^-9. So the int4 -> fp8 unpack is a mask (one v_bitop3 per
//   word, a shift more for the high nibbles), and the B block scale 2^9 (E8M0
//   136) makes the product exact in q.
// - The zero point enters through the accumulator: the first MFMA of each
//   group starts from C[m][.] = -8 * sum_{k in g} a[t_m,k] (row sums written
//   by the activation quantizer), so D = sum_k a*(q-8) for every column.
// - The group's fp16 scale is applied with one FMA per output into fp32
//   accumulators; the token scale at the end.
// - Block tile 128 rows x 128 columns, 4 waves of 64x64, K step 128, two
//   blocks per CU (204 VGPRs, 74 KiB of LDS).
// - A: activation rows gathered by token id straight into LDS (LDS DMA: each
//   lane's source row is its token's; rows past the segment read as zero),
//   three stages. Logical 16-byte chunk 2q + s of a row sits at physical
//   chunk (4s + q) ^ (row & 7), where lane group q reads it without bank
//   conflicts.
// - B: the block's packed 8 KiB weight tile of a K step goes into the same
//   stage as A by LDS DMA, so each weight byte crosses the vector memory
//   path once per block (loaded straight into registers, each column half
//   crossed it twice, once per wave using it: 2% slower). Each wave reads
//   its own 64 columns: lane (column c, lane group q) takes the 16-byte tile
//   unit holding K 32q .. 32q+31 of column c, whose low nibbles are K
//   32q..+15 and high nibbles K 32q+16..+31 -- exactly the 32 fp8 bytes the
//   MFMA wants from that lane, matching the A fragment (logical chunks 2q,
//   2q+1).
// - With group 128 (a whole group per K step) the MFMAs are asm statements,
//   so that they keep their order, and the vector work of the step is placed
//   between them: block j's four MFMAs carry block j + 1's unpack and block
//   j - 1's epilogue (left to the compiler, the unpack all came
//   first and the epilogue all last). The stage index and the K offset of the
//   A DMA are scalar. Other group sizes use the builtin MFMA.
// - One K step per loop iteration, the stage index in a register. A step
//   first reads all of its A fragments, B words and C starts (before it
//   issues its own LDS DMA, so those reads wait for nothing newer than the
//   previous step's DMA: a tile has one step to arrive), then issues the
//   scales, sums, A and B of later steps, and works its four 16-column
//   blocks in turn, each unpacked under the previous one's MFMAs; a block's
//   group epilogue runs under the next block's MFMAs (the last block's under
//   the next step's first). (Three steps unrolled with constant stage
//   indices spilled registers; B staged unpacked in LDS, or the DMA issued
//   before the fragment reads, measured 17% and 13% slower.)
// - The group sums of a staged tile sit in LDS beside it; threads 0..127 load
//   them two steps ahead and store them one step ahead.
// - Work items (expert, row tile, column tile) are enumerated on the device
//   from expert_offsets, column tile fastest (so an XCD's run of blocks
//   shares a few gathered row tiles across all of an expert's columns: 3%
//   faster than row tile fastest); the grid is an upper bound and idle
//   blocks exit.
//   The output tile goes through LDS and leaves as 16-byte row segments.
#include "w4_device.h"

namespace w4 {

constexpr int kEM = 128, kEN = 128, kEK = 128;
constexpr int kEThreads = 256;
constexpr int kEStageA = kEM * kEK;                // 16 KiB
constexpr int kEStageB = kEN * kEK / 2;            // 8 KiB of packed weights
constexpr int kESS = kEStageA + kEStageB;          // a stage: A, then B
constexpr int kEStages = 3;

typedef _Float16 eh2 __attribute__((ext_vector_type(2)));

// GT: K steps (of 128) per weight group (group = 128 * GT)
template <int GT>
__global__ __launch_bounds__(kEThreads, 2) void grouped_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ a_scale, const float* __restrict__ gsum,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets, int E,
    const uint8_t* __restrict__ Wt, int64_t w_stride, const uint16_t* __restrict__ wscale,
    uint16_t* __restrict__ out, int N, int K, int KT, int NT, int T) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kEStages * kESS];
  __shared__ int s_tok[kEM];                                  // token of each tile row (-1: none)
  __shared__ __attribute__((aligned(16))) float s_gs[kEStages][kEM];   // -8 * group sum per staged row

  // ---- work item of this block. Block ids go to the 8 XCDs in turn; XCD x
  // takes the x-th eighth of the real work items (their count is known only
  // here), so the idle blocks of the upper-bound grid fall on every XCD
  // rather than all on the last ones. The host rounds the grid up to a
  // multiple of 8, which leaves every XCD at least an eighth of it.
  int total = 0;
  for (int ee = 0; ee < E; ++ee) total += (offsets[ee + 1] - offsets[ee] + kEM - 1) / kEM * NT;
  const int per = (total + 7) / 8, xi = (int)(blockIdx.x / 8);
  if (xi >= per) return;
  const int t = (int)(blockIdx.x % 8) * per + xi;
  if (t >= total) return;
  int e = -1, mt = 0, tn = 0, seg0 = 0, cnt = 0;
  {
    int cum = 0;
    for (int ee = 0; ee < E; ++ee) {
      const int o0 = offsets[ee], o1 = offsets[ee + 1];
      const int mtiles = (o1 - o0 + kEM - 1) / kEM;
      const int tiles = mtiles * NT;
      if (t < cum + tiles) {
        const int local = t - cum;
        e = ee; mt = local / NT; tn = local % NT; seg0 = o0; cnt = o1 - o0;
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

  // ---- A: wave w's DMA i fills stage rows 32w + 8i .. +7 (one KiB), lane L
  // landing at row 32w + 8i + L/8, physical chunk p = L%8 and fetching the
  // logical chunk vinv(p ^ (L/8)) of its row's token, vinv(u) = 2(u & 3) +
  // (u >> 2). A row without a token gets an offset past the buffer, which
  // reads as zero. Offsets stay in the range-checked VGPR operand (T*K < 2^31,
  // checked by the caller).
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(A, (uint32_t)((int64_t)T * K));
  const int lrow = lane >> 3, lchunk = lane & 7;
  const int u = lchunk ^ lrow;
  const uint32_t a_chunk = 16u * (uint32_t)(2 * (u & 3) + (u >> 2));
  uint32_t a_voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = s_tok[32 * wave + 8 * i + lrow];
    a_voff[i] = (tok >= 0) ? (uint32_t)tok * (uint32_t)K + a_chunk : 0x80000000u;
  }
  // the K offset goes in the scalar operand: a row without a token stays
  // past the buffer through its VGPR offset alone
  auto gload_a = [&](int tk, int st) {
    const uint32_t ks = (uint32_t)tk * kEK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          arsrc, (__attribute__((address_space(3))) void*)(lds + st * kESS + (32 * wave_u + 8 * i) * kEK), 16,
          a_voff[i], ks, 0, 0);
  };

  // ---- B: the block's packed 8 KiB tile of the K step into the stage after
  // A (LDS DMA, one KiB per load, two per wave), so each weight byte passes
  // the vector memory path once per block; lane (column l%16 of 16-column
  // block j, lane group l/16) then reads unit (64 wn + 16 j + l%16, l/16)
  const __amdgpu_buffer_rsrc_t wrsrc =
      make_rsrc(Wt + (int64_t)e * w_stride + (int64_t)tn * KT * kTileBytes, (uint32_t)KT * kTileBytes);
  auto gload_b = [&](int tk, int st) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wrsrc, (__attribute__((address_space(3))) void*)(lds + st * kESS + kEStageA + (2 * wave_u + i) * 1024), 16,
          16u * (uint32_t)lane + 1024u * (uint32_t)(2 * wave + i), (uint32_t)tk * kTileBytes, 0, 0);
  };
  const int b_ro = kEStageA + 4096 * wn + 64 * (lane & 15) + 16 * (lane >> 4);
  v4i pb[4];
  auto read_b = [&](int st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) pb[j] = *reinterpret_cast<const v4i*>(lds + st * kESS + b_ro + 1024 * j);
  };
  // stored q ^ 8 -> fp8 bytes q: low nibbles are K 32q..+15, high K 32q+16..+31
  auto unpack_b = [&](int j) -> v8i {
    v8i bf;
#pragma unroll
    for (int c = 0; c < 4; c += 2) {
      const uint32_t w0 = (uint32_t)pb[j][c], w1 = (uint32_t)pb[j][c + 1];
      const uint64_t h = shr64<4>(as_u64x2(pb[j])[c / 2]);   // the high nibbles of both words
      bf[c] = (int)((w0 ^ 0x88888888u) & 0x0F0F0F0Fu);
      bf[c + 1] = (int)((w1 ^ 0x88888888u) & 0x0F0F0F0Fu);
      bf[4 + c] = (int)(((uint32_t)h ^ 0x08080808u) & 0x0F0F0F0Fu);
      bf[5 + c] = (int)(((uint32_t)(h >> 32) ^ 0x08080808u) & 0x0F0F0F0Fu);
    }
    return bf;
  };

  // ---- group sums of the tile rows: thread t < 128 loads row t's sum of the
  // group of step tk + 2 (a row without a token, and threads past the rows,
  // read zero from past the buffer) and stores it one step later
  const __amdgpu_buffer_rsrc_t gsrc = make_rsrc(gsum, (uint32_t)((int64_t)T * G * 4));
  const int my_tok = (tid < kEM) ? s_tok[tid] : -1;
  const uint32_t g_voff = (my_tok >= 0) ? (uint32_t)my_tok * (uint32_t)G * 4u : 0x80000000u;
  auto gload_gs = [&](int tk) -> float {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gsrc, g_voff + 4u * (uint32_t)(tk / GT), 0, 0));
  };

  // ---- fp16 scales of the lane's 4 columns (clamped: a column past N is never stored)
  const int ncol0 = n0 + 64 * wn + (lane & 15);    // column of block j: ncol0 + 16 j
  const __amdgpu_buffer_rsrc_t srsrc = make_rsrc(wscale + (int64_t)e * G * N, (uint32_t)((int64_t)G * N * 2));
  uint32_t s_voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s_voff[j] = 2u * (uint32_t)min(ncol0 + 16 * j, N - 1);
  auto fetch_scales = [&](int tk, eh2 (&raw)[2]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      raw[j >> 1][j & 1] = __builtin_bit_cast(
          _Float16, __builtin_amdgcn_raw_buffer_load_b16(srsrc, s_voff[j], (uint32_t)(tk / GT) * (uint32_t)N * 2u, 0));
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
  // group epilogue of column block j (all four row blocks)
  auto epilogue = [&](int j, const eh2 (&raw)[2]) {
    const float sc = (float)raw[j >> 1][j & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) facc[i][j][r] = fmaf(acc[i][j][r], sc, facc[i][j][r]);
  };
  // rows [R0, R0 + 2) of block j's group epilogue
  auto epilogue_rows = [&](int j, int R0, const eh2 (&raw)[2]) {
    const float sc = (float)raw[j >> 1][j & 1];
#pragma unroll
    for (int i = R0; i < R0 + 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) facc[i][j][r] = fmaf(acc[i][j][r], sc, facc[i][j][r]);
  };
  // d = a * b + c (fp8 x fp8, block scales 2^0 and 2^9), written as asm so
  // that it keeps its place among the unpack and epilogue work around it.
  // Its result is read by vector code only four or more MFMAs later.
  const uint32_t scale_a = 127u, scale_b = 136u;
  // pins: vector work placed between two of these stays between the MFMAs
  // around them (asm statements keep their order)
  auto pin_facc = [&](int j, int R0) {
    asm volatile("" : "+v"(facc[R0][j][0]), "+v"(facc[R0][j][1]), "+v"(facc[R0][j][2]), "+v"(facc[R0][j][3]),
                 "+v"(facc[R0 + 1][j][0]), "+v"(facc[R0 + 1][j][1]), "+v"(facc[R0 + 1][j][2]),
                 "+v"(facc[R0 + 1][j][3]));
  };
  auto mfma_fresh = [&](v4f& d, const v8i& a, const v8i& b, const v4f& c) {
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %3, %4, %5 op_sel_hi:[0,0,0]"
                 : "=&v"(d)
                 : "v"(a), "v"(b), "v"(c), "v"(scale_a), "v"(scale_b));
  };
  // ---- A fragments: lane row (lane & 15), logical chunks 2g and 2g + 1 at
  // physical chunks g ^ (row & 7) and (4 + g) ^ (row & 7)
  const int fl = lane & 7, g4 = lane >> 4;
  const int a_ro0 = (64 * wm + (lane & 15)) * kEK + 16 * (g4 ^ fl);
  const int a_ro1 = (64 * wm + (lane & 15)) * kEK + 16 * ((g4 + 4) ^ fl);
  auto read_a = [&](int st, int i) -> v8i {
    const uint8_t* base = lds + st * kESS + 16 * kEK * i;
    const v4i x0 = *reinterpret_cast<const v4i*>(base + a_ro0);
    const v4i x1 = *reinterpret_cast<const v4i*>(base + a_ro1);
    return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  auto read_cinit = [&](int st, int i) -> v4f {
    return *reinterpret_cast<const v4f*>(&s_gs[st][64 * wm + 16 * i + 4 * g4]);
  };
  // ---- prologue: scales of step 0, B, sums and A of steps 0 and 1
  eh2 sc_cur[2], sc_next[2], sc_prev[2] = {eh2{0, 0}, eh2{0, 0}};
  fetch_scales(0, sc_cur);
  gload_b(0, 0);
  const float gs0 = gload_gs(0);
  gload_a(0, 0);
  float gs_pend = gload_gs(min(1, KT - 1));  // the sums of the step after the current one
  gload_b(min(1, KT - 1), 1);
  gload_a(min(1, KT - 1), 1);
  __builtin_amdgcn_s_waitcnt(0x0F77);      // vmcnt(7): all but step 1's sums, B and A
  if (tid < kEM) s_gs[0][tid] = -8.f * gs0;
  __syncthreads();

  // K step tk reads stage tk % 3 (A and B). It issues the scales of step
  // tk + 1 and the sums, A and B of step tk + 2 (into the stage read at step
  // tk - 1). The step ends once step tk + 1's A and B have landed and its
  // sums are stored (the 11 newest loads may stay in flight across the
  // barrier).
  bool last_prev = false;                  // did the previous step end a group?
  auto kstep = [&](int tk, int st_) {
    const int st = __builtin_amdgcn_readfirstlane(st_);
    const bool fresh = (tk % GT) == 0, last = (tk % GT) == GT - 1;
    const int tn1 = min(tk + 1, KT - 1);
    // this step's fragments first: read before this step's DMA is issued,
    // they wait at most for the previous step's
    v8i af[4];
    v4f ci[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = read_a(st, i);
      ci[i] = read_cinit(st, i);
    }
    read_b(st);
    fetch_scales(tn1, sc_next);
    const float gs_new = gload_gs(min(tk + 2, KT - 1));
    gload_a(min(tk + 2, KT - 1), st == 0 ? 2 : st - 1);
    gload_b(min(tk + 2, KT - 1), st == 0 ? 2 : st - 1);
    if constexpr (GT == 1) {
      // every step is one whole group: block j's four MFMAs carry block
      // j + 1's unpack and block j - 1's epilogue between them
      v8i bf = unpack_b(0);
      asm volatile("" : "+v"(bf)::"memory");
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v8i bn = bf;
        const bool epi = j > 0 || last_prev;
        const int je = j == 0 ? 3 : j - 1;
        mfma_fresh(acc[0][j], af[0], bf, ci[0]);
        if (j < 3) {
          asm volatile("" : "+v"(pb[j + 1]));
          bn = unpack_b(j + 1);
        }
        mfma_fresh(acc[1][j], af[1], bf, ci[1]);
        if (j < 3) asm volatile("" : "+v"(bn)::"memory");
        mfma_fresh(acc[2][j], af[2], bf, ci[2]);
        if (epi) {
          pin_facc(je, 0);
          epilogue_rows(je, 0, j == 0 ? sc_prev : sc_cur);
          pin_facc(je, 0);
        }
        mfma_fresh(acc[3][j], af[3], bf, ci[3]);
        if (epi) {
          pin_facc(je, 2);
          epilogue_rows(je, 2, j == 0 ? sc_prev : sc_cur);
          pin_facc(je, 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf = bn;
      }
    } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v8i bf = unpack_b(j);
      asm volatile("" : "+v"(bf)::"memory");
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, fresh ? ci[i] : acc[i][j], 0, 0, 0,
                                                                     127, 0, 136);
      if (j == 0) {
        if (last_prev) epilogue(3, sc_prev);
      } else if (last) {
        epilogue(j - 1, sc_cur);
      }
    }
    }
    last_prev = last;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc_prev[h] = sc_cur[h];
      sc_cur[h] = sc_next[h];
    }
    __builtin_amdgcn_s_waitcnt(0x0F7B);    // vmcnt(11): step tk + 1's A, B and sums landed
    if (tid < kEM) s_gs[st == 2 ? 0 : st + 1][tid] = -8.f * gs_pend;
    gs_pend = gs_new;
    __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0): sums stored (vmcnt left as is)
    barrier_keep_loads();
    __builtin_amdgcn_sched_barrier(0);
  };

  for (int tk = 0, st = 0; tk < KT; ++tk, st = (st == 2 ? 0 : st + 1)) kstep(tk, st);
  // the clamped last loads may still be streaming into LDS
  __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
  // the last MFMAs' results: wait states before vector code reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  if (last_prev) epilogue(3, sc_prev);

  // ---- output: row scale, bf16, staged through LDS and written as 16-byte
  // row segments (N is a multiple of 8)
  constexpr int kORow = kEN * 2 + 16;
  static_assert(kEM * kORow <= kEStages * kESS, "output tile fits the stage buffers");
  __syncthreads();
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
  dim3 grid((unsigned)((upper + 7) / 8 * 8)), block(kEThreads);
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
