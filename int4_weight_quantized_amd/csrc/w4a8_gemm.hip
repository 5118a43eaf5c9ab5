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
// - 256 threads, block tile 128x128, four waves of 64x64, K step 128.
//   Group 128 and per-channel: three stages of A and packed B (72 KiB), both
//   by LDS DMA two K steps ahead, so each B byte passes the vector memory
//   path once per block (that path, not the matrix core, is what the
//   per-channel kernel waits on; loading B straight into each wave's
//   registers took it twice, once per wave sharing a column half). Two
//   blocks per CU. Per-channel shapes with at least 256 blocks of 128 x 256
//   take those instead: eight waves (2 x 4 of 64x64), 96 KiB of stages, one
//   block per CU, a third fewer A and B bytes per MFMA. Other group sizes:
//   two A+B stages (64 KiB), loads one step ahead. The int32 partials test
//   hook runs each of these modes, in the block shape the GEMM of that size
//   takes, with a store in place of the epilogue.
// - Loads are raw buffer loads. A (int8 codes) goes straight from memory to
//   LDS, its range check zero-filling rows past M; B is the tiled int4
//   layout, 8 KiB contiguous per tile.
// - B (stored nibble q^8) becomes int8 bytes 16*(q-8) with a mask (and a
//   4-bit shift); the MFMA accumulates 16*P and 1/16 is folded into the row
//   scale (exact). In the three-stage modes B stays packed in LDS and each
//   wave reads its own 64 columns, one 16-byte tile unit per lane and
//   column block: lane (column c, group q) holds the 32 codes of K quarter q
//   of column c, the low nibbles serve the first 64-deep MFMA step and the
//   high nibbles the second, and the A fragments carry the same K
//   assignment (chunk 2q + step, stored where the bank-conflict-free read
//   pattern finds it). Per-channel, the int32 accumulators run over all of
//   K and the column scale is applied once after the loop. The two-stage
//   modes unpack B once per block into LDS.
// - A and B rows in LDS are 128 bytes; 16-byte chunk kc of row r sits at
//   kc ^ (r & 7). Fragment reads and tile writes are then bank-conflict free
//   (measured), and every fragment address is a base register plus an
//   immediate.
// - v_mfma_i32_16x16x64_i8. With one group per K step (group 128) a wave's
//   64x64 tile is worked in two 32-row halves: while one half's MFMAs run,
//   the other half's finished group goes through its epilogue (int32 ->
//   fp32, FMA with the group's fp16 scale), so the vector ALU work overlaps
//   the matrix core. Other group sizes apply the epilogue after each group.
// - Tiles are visited in groups of 8 tile-rows (4 for per-channel weights),
//   and block ids are remapped so each XCD (own L2) works on a contiguous
//   range of tiles.
#include <type_traits>

#include "w4_device.h"

namespace w4 {

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kGThreads = 256;
constexpr int kStageA = kBM * kBK;                 // A rows unpadded, chunks swizzled
constexpr int kStageB = kBN * kBK;                 // B rows unpadded, chunks swizzled
constexpr int kStage = kStageA + kStageB;

// kModeSplit: group 128 with K split over `splits` blocks per tile; each
// writes its fp32 partial tile (a_scale applied, no bias) to ws[split][M][N]
// and w4a8_split_finalize sums them.
enum { kModeGroup = 0, kModeChannel = 1, kModeSplit = 3 };

template <int V>
using IC = std::integral_constant<int, V>;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// GC: 64-deep chunks per weight group when known at compile time (1: group
// 64, 2: group 128), 0: taken from group_chunks at run time.
// PART: the test hook's instantiation of the same mode. Where the epilogue
// would scale a finished group it stores the exact int32 partial sum
// P[m,g,n] (the accumulator holds 16 P) to partials [M, G, N] instead, and
// the kernel ends after the K loop; loads, unpack, LDS layout, MFMAs and
// their schedule are the ones the epilogue-fused instantiation runs.
// WN: waves along N (per-channel only: 4 makes the block 128 x 256 with
// eight waves, each B and A byte then feeding twice the MFMAs).
template <int MODE, bool OUT_BF16, int GC, bool PART, int WN = 2>
__global__ __launch_bounds__(128 * WN, WN == 4 ? 1 : 2) void w4a8_gemm_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ a_scale,
    const v4i* __restrict__ Wt, const uint16_t* __restrict__ wscale, int group_chunks_rt,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
    int32_t* __restrict__ partials, int M, int N, int K, int KT, int tilesM, int tilesN,
    float* __restrict__ ws, int splits, const float* __restrict__ a_off, const float* __restrict__ w_off) {
  // three LDS stages of A and B: group 128 (its epilogue interleaved with
  // the MFMAs) and per-channel (whole K summed in the int32 accumulators,
  // scales applied once after the loop)
  constexpr bool kPingPong = ((MODE == kModeGroup || MODE == kModeSplit) && GC == 2) || MODE == kModeChannel;
  constexpr bool kStepScales = kPingPong && MODE != kModeChannel;
  static_assert(MODE != kModeSplit || GC == 2, "split K is built for group 128");
  static_assert(!PART || MODE != kModeSplit, "partials are stored by the unsplit modes");
  static_assert(WN == 2 || (WN == 4 && MODE == kModeChannel), "wide blocks are built for per-channel weights");
  constexpr int kNT = 128 * WN;                         // threads
  constexpr int kNW = 2 * WN;                           // waves
  constexpr int kBNw = 64 * WN;                         // block columns
  constexpr int kRPW = kBM / kNW;                       // A rows each wave brings into a stage
  // loads a wave issues for one three-stage K step: A (kRPW / 8 DMAs of 8
  // rows) and B (2 DMAs); the step's closing wait leaves exactly these in
  // flight (vmcnt), so everything older, the next step's tiles, has landed
  constexpr int kStepLoads = kRPW / 8 + 2;
  static_assert(kStepLoads < 16, "vmcnt immediate");

  // group 128 and per-channel: three stages of A and packed B, both by LDS
  // DMA; otherwise two stages of A and unpacked B
  constexpr bool kBL = kPingPong;
  constexpr int kSS = kBL ? kStageA + kBNw * kBK / 2 : kStage;   // bytes per stage
  constexpr int kNS = kPingPong ? 3 : 2;                // stages
  __shared__ __attribute__((aligned(16))) uint8_t lds[kNS * kSS];
  const int group_chunks = GC > 0 ? GC : group_chunks_rt;

  // ---- tile of this block (and its K range: all of K unless split)
  int t = xcd_remap(blockIdx.x, gridDim.x);
  int kt0 = 0, kt1 = KT, split = 0;
  if constexpr (MODE == kModeSplit) {
    const int ks = (KT + splits - 1) / splits;
    split = t % splits;
    t /= splits;
    kt0 = min(split * ks, KT);
    kt1 = min(kt0 + ks, KT);
  }
  // tile-rows per raster group (per-channel: 4 measured ~2% faster than 8)
  constexpr int GM = MODE == kModeChannel ? 4 : 8;
  const int per_group = GM * tilesN;
  const int first_m = (t / per_group) * GM;
  const int gsz = min(tilesM - first_m, GM);
  const int tm = first_m + (t % per_group) % gsz;
  const int tn = (t % per_group) / gsz;
  const int m0 = tm * kBM, n0 = tn * kBNw;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int nchunks = (K + 63) >> 6;
  const int G = (MODE == kModeChannel) ? 1 : nchunks / group_chunks;

  // ---- global loads: fixed per-lane offsets, K step in the scalar offset.
  // A goes straight to LDS (buffer load with the LDS destination): wave w's
  // load i fills stage rows R w + 8i .. +7 (R = 32, or 16 with eight waves),
  // one KiB, lane L landing at row R w + 8i + L/8, physical 16-byte chunk
  // L%8. The lane fetches the logical chunk that belongs there under the
  // swizzle p = kc ^ (row & 7); row & 7 is L/8 for every load, so one
  // per-lane offset serves all of them.
  const int rows_valid = min(kBM, M - m0);
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(A + (int64_t)m0 * K, (uint32_t)rows_valid * (uint32_t)K);
  // weights of the block's 128-column tiles (the second of a wide block may
  // lie past N: its loads then read zeros)
  const int wtiles = WN == 2 ? 1 : min(2, (N + 127) / 128 - 2 * tn);
  const __amdgpu_buffer_rsrc_t wrsrc =
      make_rsrc(reinterpret_cast<const uint8_t*>(Wt) + (int64_t)tn * (WN / 2) * KT * kTileBytes,
                (uint32_t)wtiles * (uint32_t)KT * kTileBytes);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int lrow = lane >> 3, lchunk = lane & 7;
  // The three-stage modes read logical chunk 2q + s for lane group q
  // and step s; it is stored at physical chunk (4s + q) ^ (row & 7), the
  // position the two-stage path reads for its own chunk 4s + q, which keeps
  // the fragment reads bank-conflict free. So the lane at physical chunk p
  // fetches logical chunk vinv(p ^ (row & 7)), vinv(u) = 2 (u & 3) + (u >> 2).
  const int a_lchunk = kPingPong ? 2 * ((lchunk ^ lrow) & 3) + ((lchunk ^ lrow) >> 2) : (lchunk ^ lrow);
  const uint32_t a_voff = (uint32_t)(kRPW * wave + lrow) * (uint32_t)K + 16u * (uint32_t)a_lchunk;
  const uint32_t w_voff = 16u * tid;                                               // units tid, tid+256
  v4i pb[2];                                        // two-stage modes: B words on their way to LDS
  auto gload_a = [&](int tk, auto STc) {
    constexpr int ST = decltype(STc)::value;
    const uint32_t ks = (uint32_t)tk * kBK;
#pragma unroll
    for (int i = 0; i < kRPW / 8; ++i)   // whole offset in the range-checked VGPR operand
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          arsrc, (__attribute__((address_space(3))) void*)(lds + ST * kSS + (kRPW * wave_u + 8 * i) * kBK), 16,
          a_voff + (ks + (uint32_t)(8 * i) * (uint32_t)K), 0, 0, 0);
  };
  // three-stage modes: the block's packed B tiles (8 KiB per 128 columns,
  // column n's 64 bytes at 64 n) straight into the stage after A, one KiB
  // per load, two per wave; KiB u of the stage is KiB u % 8 of 128-column
  // tile u / 8
  auto gload_bl = [&](int tk, auto STc) {
    constexpr int ST = decltype(STc)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t u = (uint32_t)(2 * wave + i);
      const uint32_t uo = WN == 2 ? 1024u * u : 1024u * (u & 7u) + (u >> 3) * (uint32_t)KT * kTileBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wrsrc, (__attribute__((address_space(3))) void*)(lds + ST * kSS + kStageA + (2 * wave_u + i) * 1024), 16,
          16u * (uint32_t)lane + uo, (uint32_t)tk * kTileBytes, 0, 0);
    }
  };
  auto gload = [&](int tk, auto STc) {
    constexpr int ST = decltype(STc)::value;
    const uint32_t ks = (uint32_t)tk * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i)   // whole offset in the range-checked VGPR operand
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          arsrc, (__attribute__((address_space(3))) void*)(lds + ST * kSS + (kRPW * wave_u + 8 * i) * kBK), 16,
          a_voff + (ks + (uint32_t)(8 * i) * (uint32_t)K), 0, 0, 0);
    const uint32_t ws = (uint32_t)tk * kTileBytes;
    pb[0] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, w_voff, ws, 0);
    pb[1] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, w_voff, ws + 4096u, 0);
  };
  // B unit u (row n = u/4, K quarter q = u%4): its low nibbles unpack to the
  // logical chunk 2q (K 32q+0..15), its high nibbles to chunk 2q+1.
  const int b_wo_lo = (tid >> 2) * kBK + 16 * ((2 * (tid & 3)) ^ ((tid >> 2) & 7));
  const int b_wo_hi = (tid >> 2) * kBK + 16 * ((2 * (tid & 3) + 1) ^ ((tid >> 2) & 7));
  auto lstore_b = [&](auto STc) {
    constexpr int ST = decltype(STc)::value;
    uint8_t* lb = lds + ST * kStage + kStageA;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v4i lo, hi;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lo[c] = (int)(((uint32_t)pb[i][c] << 4) & 0xF0F0F0F0u);
        hi[c] = (int)((uint32_t)pb[i][c] & 0xF0F0F0F0u);
      }
      *reinterpret_cast<v4i*>(lb + b_wo_lo + 64 * kBK * i) = lo;
      *reinterpret_cast<v4i*>(lb + b_wo_hi + 64 * kBK * i) = hi;
    }
  };
  // the step's A tile (LDS DMA) and B words must have landed before the barrier
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

  // ---- accumulators: acc[i][j] int32 16x16 sub-tiles, facc fp32
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

  // fp16 scales of group g for the lane's 4 columns, two per register, at
  // clamped columns: a column past N is never stored
  const __amdgpu_buffer_rsrc_t srsrc =
      make_rsrc(wscale, PART ? 0u : (uint32_t)((int64_t)G * N * 2));
  uint32_t s_voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s_voff[j] = 2u * (uint32_t)min(ncol[j], N - 1);
  auto fetch_scales = [&](int g, h2 (&raw)[2]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      raw[j >> 1][j & 1] = __builtin_bit_cast(
          _Float16, __builtin_amdgcn_raw_buffer_load_b16(srsrc, s_voff[j], (uint32_t)g * (uint32_t)N * 2u, 0));
  };
  // the next group's scales, loaded as four halves and paired up only once
  // the step's closing wait has seen them land: left to itself the compiler
  // may pair them mid-step, which waits there for every load issued before
  // them in the same step (the next step's B words included)
  auto fetch_scales_split = [&](int g, uint32_t (&raw)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      raw[j] = __builtin_amdgcn_raw_buffer_load_b16(srsrc, s_voff[j], (uint32_t)g * (uint32_t)N * 2u, 0);
  };
  auto pair_scales = [&](uint32_t (&raw)[4], h2 (&out)[2]) {
    asm volatile("" : "+v"(raw[0]), "+v"(raw[1]), "+v"(raw[2]), "+v"(raw[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j >> 1][j & 1] = __builtin_bit_cast(_Float16, (uint16_t)raw[j]);
  };

  // group epilogue for sub-tile rows [I0, I1)
  auto epilogue = [&](auto I0c, auto I1c, const h2 (&raw)[2], int g) {
    constexpr int I0 = decltype(I0c)::value, I1 = decltype(I1c)::value;
    if constexpr (PART) {
      if (g < 0) return;                                  // the first step's rows 2-3 hold no group yet
#pragma unroll
      for (int i = I0; i < I1; ++i)
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
      for (int i = I0; i < I1; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sc = (float)raw[j >> 1][j & 1];
#pragma unroll
          for (int r = 0; r < 4; ++r) facc[i][j][r] = fmaf((float)acc[i][j][r], sc, facc[i][j][r]);
        }
    }
  };

  // fragment reads: lane row (lane & 15), 16-byte chunk (lane >> 4); +64
  // bytes per 64-deep chunk and +16 rows per sub-tile are immediates
  const int fl = lane & 7;                                // row & 7 of the lane's fragment rows
  int a_ro[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) a_ro[c] = (64 * wm + (lane & 15)) * kBK + 16 * ((4 * c + (lane >> 4)) ^ fl);
  int b_ro[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) b_ro[c] = (64 * wn + (lane & 15)) * kBK + 16 * ((4 * c + (lane >> 4)) ^ fl);
  auto read_b = [&](auto STc, int c, v4i (&bf)[4]) {
    constexpr int ST = decltype(STc)::value;
    const uint8_t* lb = lds + ST * kStage + kStageA + b_ro[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const v4i*>(lb + 16 * kBK * j);
  };
  auto mfma_rows = [&](auto STc, int c, auto I0c, auto I1c, bool fresh, const v4i (&bf)[4]) {
    constexpr int ST = decltype(STc)::value;
    constexpr int I0 = decltype(I0c)::value, I1 = decltype(I1c)::value;
    const uint8_t* la = lds + ST * kSS + a_ro[c];
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const v4i af = *reinterpret_cast<const v4i*>(la + 16 * kBK * i);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[j], fresh ? v4i{0, 0, 0, 0} : acc[i][j], 0, 0, 0);
    }
  };

  auto read_a = [&](auto STc, int i, int c) -> v4i {
    constexpr int ST = decltype(STc)::value;
    return *reinterpret_cast<const v4i*>(lds + ST * kSS + a_ro[c] + 16 * kBK * i);
  };
  auto mfma_row = [&](int i, const v4i& af, const v4i (&bf)[4], bool fresh) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[j], fresh ? v4i{0, 0, 0, 0} : acc[i][j], 0, 0, 0);
  };
  auto interleave8 = [&]() {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
  };

  // ---- prologue: tile 0 to LDS stage 0 (three-stage modes: tiles 0 and 1
  // to stages 0 and 1)
  h2 scr_cur[2] = {h2{0, 0}, h2{0, 0}}, scr_prev[2] = {h2{0, 0}, h2{0, 0}};
  if constexpr (MODE == kModeSplit) {
    if (kt0 >= kt1) {                              // an empty split (the host avoids them): zeros
      float* wsp = ws + (int64_t)split * M * N;
      for (int e = tid; e < kBM * kBN; e += kGThreads) {
        const int m = m0 + e / kBN, n = n0 + e % kBN;
        if (m < M && n < N) wsp[(int64_t)m * N + n] = 0.f;
      }
      return;
    }
  }
  if constexpr (MODE == kModeChannel) {
    gload_bl(kt0, IC<0>{});
    gload_a(kt0, IC<0>{});
    gload_bl(min(kt0 + 1, kt1 - 1), IC<1>{});
    gload_a(min(kt0 + 1, kt1 - 1), IC<1>{});
    __builtin_amdgcn_s_waitcnt(0x0F70 | kStepLoads);   // all but tile 1's B and A
  } else if constexpr (kPingPong) {
    if constexpr (kStepScales) fetch_scales(kt0, scr_cur);
    gload_bl(kt0, IC<0>{});
    gload_a(kt0, IC<0>{});
    gload_bl(min(kt0 + 1, kt1 - 1), IC<1>{});
    gload_a(min(kt0 + 1, kt1 - 1), IC<1>{});
    __builtin_amdgcn_s_waitcnt(0x0F70 | kStepLoads);   // all but tile 1's B and A
  } else {
    gload(0, IC<0>{});
    lstore_b(IC<0>{});
    wait_loads();
  }
  __syncthreads();

  // K step tk reads LDS stage ST while the next tiles stream in: with two
  // stages tile tk + 1 into the other one (A directly, B through registers
  // stored at the end of the step); with three (group 128, per-channel) A
  // and B of tile tk + 2 by DMA into the stage read at step tk - 1. Past the
  // last tile the loads repeat it, which keeps the body branch-free.
  auto kstep = [&](int tk, auto STc) {
    constexpr int ST = decltype(STc)::value;
    // three-stage modes: this step's B words become fragments. Substep 0
    // takes the low nibbles (K 32 q + 0..15 of the lane's quarter q),
    // substep 1 the high ones (K 32 q + 16..31); the A fragments follow.
    v4i b0[4], b1[4];
    if constexpr (kBL) {
      // this wave's 64 columns from the stage: lane (column l%16 of 16-column
      // block j, K quarter l/16) reads unit (64 wn + 16 j + l%16, l/16), the
      // 64 lanes one contiguous KiB per block (bank-conflict free)
      const uint8_t* lb = lds + ST * kSS + kStageA + 4096 * wn + 64 * (lane & 15) + 16 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i wv = *reinterpret_cast<const v4i*>(lb + 1024 * j);
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          // two words shifted as one 64-bit value: the nibble carried across
          // the word boundary lands in bits the mask clears
          const uint64_t w2 = shl64<4>(as_u64x2(wv)[e / 2]);
          b0[j][e] = (int)((uint32_t)w2 & 0xF0F0F0F0u);
          b0[j][e + 1] = (int)((uint32_t)(w2 >> 32) & 0xF0F0F0F0u);
          b1[j][e] = (int)((uint32_t)wv[e] & 0xF0F0F0F0u);
          b1[j][e + 1] = (int)((uint32_t)wv[e + 1] & 0xF0F0F0F0u);
        }
      }
    }
    uint32_t scr_next[4];
    if constexpr (MODE == kModeChannel) {
      // B and A of tile tk + 2 into the stage read at step tk - 1: the step
      // ends waiting for everything but these kStepLoads loads
      gload_bl(min(tk + 2, kt1 - 1), IC<(ST + 2) % 3>{});
      gload_a(min(tk + 2, kt1 - 1), IC<(ST + 2) % 3>{});
    } else if constexpr (kPingPong) {
      // loads in this order, B and A of tile tk + 2 last, so that the step
      // can end waiting for everything but those kStepLoads loads
      if constexpr (kStepScales) fetch_scales_split(min(tk + 1, kt1 - 1), scr_next);
      gload_bl(min(tk + 2, kt1 - 1), IC<(ST + 2) % 3>{});
      gload_a(min(tk + 2, kt1 - 1), IC<(ST + 2) % 3>{});
    } else {
      gload(min(tk + 1, KT - 1), IC<ST ^ 1>{});
    }
    if constexpr (MODE == kModeChannel) {
      // per-channel: the accumulators run over all of K; low nibbles (b0)
      // serve chunk 0, high nibbles (b1) chunk 1, for rows 0-1 then 2-3
      const v4i a00 = read_a(IC<ST>{}, 0, 0), a10 = read_a(IC<ST>{}, 1, 0);
      const v4i a01 = read_a(IC<ST>{}, 0, 1), a11 = read_a(IC<ST>{}, 1, 1);
      mfma_row(0, a00, b0, false);
      mfma_row(1, a10, b0, false);
      const v4i a20 = read_a(IC<ST>{}, 2, 0), a30 = read_a(IC<ST>{}, 3, 0);
      mfma_row(0, a01, b1, false);
      mfma_row(1, a11, b1, false);
      const v4i a21 = read_a(IC<ST>{}, 2, 1), a31 = read_a(IC<ST>{}, 3, 1);
      mfma_row(2, a20, b0, false);
      mfma_row(3, a30, b0, false);
      mfma_row(2, a21, b1, false);
      mfma_row(3, a31, b1, false);
    } else if constexpr (kPingPong) {
      // Four quarters, each eight MFMAs with four vector ALU ops after each:
      //   Q1  rows 0-1, chunk 0 (fresh)  |  rows 2-3 finish group tk - 1 (row 2)
      //   Q2  rows 0-1, chunk 1          |  (row 3)
      //   Q3  rows 2-3, chunk 0 (fresh)  |  rows 0-1 finish group tk (row 0)
      //   Q4  rows 2-3, chunk 1          |  (row 1), then B unpack and store
      // At tk = 0 rows 2-3 are still zero, so their epilogue adds nothing.
      const v4i a00 = read_a(IC<ST>{}, 0, 0), a10 = read_a(IC<ST>{}, 1, 0);
      const v4i a01 = read_a(IC<ST>{}, 0, 1), a11 = read_a(IC<ST>{}, 1, 1);
      mfma_row(0, a00, b0, true);
      mfma_row(1, a10, b0, true);
      epilogue(IC<2>{}, IC<3>{}, scr_prev, tk - 1);
      __builtin_amdgcn_sched_group_barrier(0x020, 12, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      interleave8();
      __builtin_amdgcn_sched_barrier(0);

      const v4i a20 = read_a(IC<ST>{}, 2, 0), a30 = read_a(IC<ST>{}, 3, 0);
      mfma_row(0, a01, b1, false);
      mfma_row(1, a11, b1, false);
      epilogue(IC<3>{}, IC<4>{}, scr_prev, tk - 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      interleave8();
      __builtin_amdgcn_sched_barrier(0);

      const v4i a21 = read_a(IC<ST>{}, 2, 1), a31 = read_a(IC<ST>{}, 3, 1);
      mfma_row(2, a20, b0, true);
      mfma_row(3, a30, b0, true);
      epilogue(IC<0>{}, IC<1>{}, scr_cur, tk);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      interleave8();
      __builtin_amdgcn_sched_barrier(0);

      mfma_row(2, a21, b1, false);
      mfma_row(3, a31, b1, false);
      epilogue(IC<1>{}, IC<2>{}, scr_cur, tk);
      interleave8();
#pragma unroll
      for (int j = 0; j < 2; ++j) scr_prev[j] = scr_cur[j];
    } else {
      // scales of the groups ending in this step (at most two)
      h2 s0[2], s1[2];
      const int cg0 = 2 * tk;
      if constexpr (MODE == kModeGroup && !PART) {
        fetch_scales(min(cg0 / group_chunks, G - 1), s0);
        fetch_scales(min((cg0 + 1) / group_chunks, G - 1), s1);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int cg = cg0 + c;
        if (cg >= nchunks) break;
        const bool fresh = cg % group_chunks == 0;
        v4i bf[4];
        read_b(IC<ST>{}, c, bf);
        mfma_rows(IC<ST>{}, c, IC<0>{}, IC<4>{}, fresh, bf);
        if ((cg + 1) % group_chunks == 0) epilogue(IC<0>{}, IC<4>{}, c ? s1 : s0, cg / group_chunks);
      }
      lstore_b(IC<ST ^ 1>{});
    }
    if constexpr (MODE == kModeChannel) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | kStepLoads);   // tile tk + 2's B and A may stay in flight
      barrier_keep_loads();
    } else if constexpr (kPingPong) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | kStepLoads);   // tile tk + 2's B and A may stay in flight
      barrier_keep_loads();
      if constexpr (kStepScales) pair_scales(scr_next, scr_cur);
    } else {
      wait_loads();
      __syncthreads();                      // (and the B stores to LDS)
    }
  };

  int tk = kt0;
  if constexpr (kPingPong) {
    // stage (tk - kt0) % 3; tile tk + 2 streams in while tk is worked on
    for (; tk + 2 < kt1; tk += 3) {
      kstep(tk, IC<0>{});
      kstep(tk + 1, IC<1>{});
      kstep(tk + 2, IC<2>{});
    }
    if (tk < kt1) kstep(tk, IC<0>{});
    if (tk + 1 < kt1) kstep(tk + 1, IC<1>{});
  } else {
    for (; tk + 1 < KT; tk += 2) {
      kstep(tk, IC<0>{});
      kstep(tk + 1, IC<1>{});
    }
    if (tk < KT) kstep(tk, IC<0>{});
  }
  // the last steps' A tiles may still be streaming into LDS: no wave leaves
  // (or reuses LDS) with its own DMA in flight
  __builtin_amdgcn_s_waitcnt(0x0F70);                    // vmcnt(0)
  if constexpr (kStepScales) epilogue(IC<2>{}, IC<4>{}, scr_prev, kt1 - 1);
  if constexpr (PART) {
    if constexpr (MODE == kModeChannel) {                 // one group: all of K
      const h2 none[2] = {h2{0, 0}, h2{0, 0}};
      epilogue(IC<0>{}, IC<4>{}, none, 0);
    }
    return;
  }
  if constexpr (MODE == kModeSplit) {
    // fp32 partial tile with the row scale applied: rows of 16 columns are
    // 64-byte runs per store instruction
    float* wsp = ws + (int64_t)split * M * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mrow0 + 16 * i + r;
        if (m >= M) continue;
        const float sa = a_scale[m] * 0.0625f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (ncol[j] < N) wsp[(int64_t)m * N + ncol[j]] = facc[i][j][r] * sa;
      }
    return;
  }

  if constexpr (MODE == kModeChannel) {
    h2 raw[2];
    fetch_scales(0, raw);
    epilogue(IC<0>{}, IC<4>{}, raw, 0);
  }

  // ---- output: out = facc * a_scale / 16 + bias. The tile goes through LDS
  // (free after the loop's last barrier) so that each thread then writes
  // whole 16-byte row segments: 8 vector stores per thread instead of 64
  // 2-byte ones. N is a multiple of 8, so a segment is all in or all out.
  // asymmetric activations add a_off[m] * w_off[n] (activation offset times
  // the column's weight offset sum) to the bias term
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  float wo[4] = {0.f, 0.f, 0.f, 0.f}, ao[4][4] = {};
  if (a_off) {
#pragma unroll
    for (int j = 0; j < 4; ++j) wo[j] = w_off[min(ncol[j], N - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) ao[i][r] = a_off[min(mrow0 + 16 * i + r, M - 1)];
  }
  if (bias) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t b = bias[min(ncol[j], N - 1)];
      bv[j] = OUT_BF16 ? bf16_to_f32(b) : f16_to_f32(b);
    }
  }
  float sa[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) sa[i][r] = a_scale[min(mrow0 + 16 * i + r, M - 1)] * 0.0625f;
  constexpr int kORow = kBNw * 2 + 16;                   // padded output row in LDS, bytes
  static_assert(kBM * kORow <= kNS * kSS, "output tile fits the stage buffers");
  const int orow0 = 64 * wm + 4 * (lane >> 4), ocol0 = 64 * wn + (lane & 15);
  // every wave has drained its A tiles (above) before any overwrites the
  // stage buffers with the output
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = fmaf(facc[i][j][r], sa[i][r], fmaf(ao[i][r], wo[j], bv[j]));
        *reinterpret_cast<uint16_t*>(lds + (orow0 + 16 * i + r) * kORow + 2 * (ocol0 + 16 * j)) =
            OUT_BF16 ? f32_to_bf16_rne(y) : f32_to_f16_rne(y);
      }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kBM * kBNw / 8 / kNT; ++it) {
    const int c = tid + kNT * it, row = c / (kBNw / 8), seg = c % (kBNw / 8);
    const int m = m0 + row, n = n0 + 8 * seg;
    if (m < M && n < N)
      *reinterpret_cast<v4i*>(out + (int64_t)m * N + n) = *reinterpret_cast<const v4i*>(lds + row * kORow + 16 * seg);
  }
}

hipError_t launch_w4a8_gemm(const int8_t* a, const float* a_scale, const void* w_tiled,
                            const void* w_scale, int64_t group, const void* bias, void* out,
                            bool out_bf16, int32_t* partials, int64_t M, int64_t N, int64_t K,
                            hipStream_t stream, const float* a_off, const float* w_off) {
  if (M == 0 || N == 0) return hipSuccess;
  const int KT = (int)((K + kBK - 1) / kBK);
  const int tilesM = (int)((M + kBM - 1) / kBM), tilesN = (int)((N + kBN - 1) / kBN);
  const int nchunks = (int)((K + 63) / 64);
  const int gc = (group == -1) ? nchunks : (int)(group / 64);
  // per-channel: 128 x 256 blocks of eight waves once they make a full
  // round of the chip (half the A and B bytes per MFMA)
  const int tilesNw = (int)((N + 255) / 256);
  const bool wide = group == -1 && (int64_t)tilesM * tilesNw >= 256;
  dim3 grid((unsigned)(tilesM * tilesN)), block(kGThreads);
  dim3 grid_w((unsigned)(tilesM * tilesNw)), block_w(2 * kGThreads);
  auto W = static_cast<const v4i*>(w_tiled);
  auto S = static_cast<const uint16_t*>(w_scale);
  auto B = static_cast<const uint16_t*>(bias);
  auto O = static_cast<uint16_t*>(out);
  const int iM = (int)M, iN = (int)N, iK = (int)K;
#define W4A8_LAUNCH(MODE_, BF16_, GC_, PART_)                                                          \
  hipLaunchKernelGGL((w4a8_gemm_kernel<MODE_, BF16_, GC_, PART_>), grid, block, 0, stream, a, a_scale, W, S, gc, \
                     B, O, partials, iM, iN, iK, KT, tilesM, tilesN, nullptr, 1, a_off, w_off)
#define W4A8_LAUNCH_CH(BF16_, PART_)                                                                    \
  do {                                                                                                  \
    if (wide)                                                                                           \
      hipLaunchKernelGGL((w4a8_gemm_kernel<kModeChannel, BF16_, 0, PART_, 4>), grid_w, block_w, 0, stream, a, \
                         a_scale, W, S, gc, B, O, partials, iM, iN, iK, KT, tilesM, tilesNw, nullptr, 1, a_off, w_off); \
    else                                                                                                \
      W4A8_LAUNCH(kModeChannel, BF16_, 0, PART_);                                                       \
  } while (0)
  // the partials hook takes the same mode, block shape and chunk count as the GEMM
  if (partials) {
    if (group == -1) W4A8_LAUNCH_CH(true, true);
    else if (gc == 1) W4A8_LAUNCH(kModeGroup, true, 1, true);
    else if (gc == 2) W4A8_LAUNCH(kModeGroup, true, 2, true);
    else W4A8_LAUNCH(kModeGroup, true, 0, true);
  } else if (group == -1) {
    if (out_bf16) W4A8_LAUNCH_CH(true, false); else W4A8_LAUNCH_CH(false, false);
  } else if (gc == 1) {
    if (out_bf16) W4A8_LAUNCH(kModeGroup, true, 1, false); else W4A8_LAUNCH(kModeGroup, false, 1, false);
  } else if (gc == 2) {
    if (out_bf16) W4A8_LAUNCH(kModeGroup, true, 2, false); else W4A8_LAUNCH(kModeGroup, false, 2, false);
  } else {
    if (out_bf16) W4A8_LAUNCH(kModeGroup, true, 0, false); else W4A8_LAUNCH(kModeGroup, false, 0, false);
  }
#undef W4A8_LAUNCH_CH
#undef W4A8_LAUNCH
  return hipGetLastError();
}

}  // namespace w4

namespace w4 {

// Splits of K for a group-128 GEMM of this shape: enough blocks to fill the
// 512 block slots of the chip (two per CU) when the tiles alone fill at most a
// quarter of them, each split keeping at least 4 K steps. 1 = no split.
// (Measured on the up-projection weights: 112 tiles (M <= 128) split in 4 run
// 33 -> 22-33 us; 224 tiles split in 2 ran slower than unsplit, the partial
// tiles' extra traffic outweighing the fuller chip.)
int w4a8_split_count(int64_t M, int64_t N, int64_t K, int64_t group) {
  if (group != 128) return 1;
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (tiles > 128) return 1;
  const int64_t KT = (K + kBK - 1) / kBK;
  int s = 1;
  while (s < 8 && tiles * s * 2 <= 512 && KT / (s * 2) >= 4) s *= 2;
  while (s > 1 && (int64_t)(s - 1) * ((KT + s - 1) / s) >= KT) s /= 2;   // no empty split
  return s;
}

// out[m,n] = cast(sum_s ws[s][m][n] + bias[n]); 8 outputs per thread
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void split_finalize_kernel(const float* __restrict__ ws, int splits, int64_t MN, int N,
                                                             const uint16_t* __restrict__ bias,
                                                             uint16_t* __restrict__ out) {
  const int64_t e0 = 8 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (e0 >= MN) return;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  for (int s_ = 0; s_ < splits; ++s_) {
    const v4f a = *reinterpret_cast<const v4f*>(ws + s_ * MN + e0);
    const v4f b = *reinterpret_cast<const v4f*>(ws + s_ * MN + e0 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] += a[i];
      v[4 + i] += b[i];
    }
  }
  const int n0 = (int)(e0 % N);                      // N % 8 == 0: the 8 outputs share a row
  v4i pk;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = v[2 * i], hi = v[2 * i + 1];
    if (bias) {
      lo += OUT_BF16 ? bf16_to_f32(bias[n0 + 2 * i]) : f16_to_f32(bias[n0 + 2 * i]);
      hi += OUT_BF16 ? bf16_to_f32(bias[n0 + 2 * i + 1]) : f16_to_f32(bias[n0 + 2 * i + 1]);
    }
    const uint32_t l = OUT_BF16 ? f32_to_bf16_rne(lo) : f32_to_f16_rne(lo);
    const uint32_t h = OUT_BF16 ? f32_to_bf16_rne(hi) : f32_to_f16_rne(hi);
    pk[i] = (int)(l | (h << 16));
  }
  *reinterpret_cast<v4i*>(out + e0) = pk;
}

// Per-column weight offsets for asymmetric activations:
//   C[n] = sum_g w_scale[g, n] * sum_{k in g} (q[k, n] - 8)
// so that an activation offset z adds z * C[n] to output n. Load-time, from
// the tiled weights: one thread per column walks its 16-byte units (32
// codes each, stored q ^ 8 = the two's-complement nibble of q - 8), sums
// each group exactly in integers and accumulates scale * sum in fp32.
__global__ __launch_bounds__(256) void weight_offsets_kernel(const uint8_t* __restrict__ Wt,
                                                             const uint16_t* __restrict__ wscale, int N, int K,
                                                             int KT, int gsz, float* __restrict__ out) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const uint8_t* col = Wt + (int64_t)(n / kTileN) * KT * kTileBytes + 64 * (n % kTileN);
  float c = 0.f;
  int gsum = 0;
  for (int k0 = 0; k0 < K; k0 += 32) {                  // unit: 32 codes of K 32kq .. 32kq+31
    const v4i u = *reinterpret_cast<const v4i*>(col + (int64_t)(k0 / kTileK) * kTileBytes + 16 * ((k0 % kTileK) / 32));
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int v = ((uint32_t)u[e] >> (4 * i)) & 0xF;
        gsum += v - ((v & 8) << 1);                      // signed nibble = q - 8
      }
    if ((k0 + 32) % gsz == 0 || k0 + 32 >= K) {         // a group ends (per channel: K may end mid-unit, padded with zeros)
      c = fmaf(f16_to_f32(wscale[(int64_t)(k0 / gsz) * N + n]), (float)gsum, c);
      gsum = 0;
    }
  }
  out[n] = c;
}

hipError_t launch_weight_offsets(const void* w_tiled, const void* w_scale, int64_t group, int64_t K, int64_t N,
                                 float* out, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int KT = (int)((K + kBK - 1) / kBK);
  const int gsz = group == -1 ? (int)K : (int)group;
  hipLaunchKernelGGL(weight_offsets_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(w_tiled), static_cast<const uint16_t*>(w_scale), (int)N, (int)K,
                     KT, gsz, out);
  return hipGetLastError();
}

hipError_t launch_w4a8_gemm_split(const int8_t* a, const float* a_scale, const void* w_tiled, const void* w_scale,
                                  const void* bias, void* out, bool out_bf16, int64_t M, int64_t N, int64_t K,
                                  int splits, float* ws, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int KT = (int)((K + kBK - 1) / kBK);
  const int tilesM = (int)((M + kBM - 1) / kBM), tilesN = (int)((N + kBN - 1) / kBN);
  dim3 grid((unsigned)(tilesM * tilesN * splits)), block(kGThreads);
  hipLaunchKernelGGL((w4a8_gemm_kernel<kModeSplit, true, 2, false>), grid, block, 0, stream, a, a_scale,
                     static_cast<const v4i*>(w_tiled), static_cast<const uint16_t*>(w_scale), 2,
                     static_cast<const uint16_t*>(nullptr), static_cast<uint16_t*>(nullptr), nullptr, (int)M, (int)N,
                     (int)K, KT, tilesM, tilesN, ws, splits, nullptr, nullptr);
  const int64_t MN = M * N;
  dim3 fgrid((unsigned)((MN / 8 + 255) / 256));
  auto B = static_cast<const uint16_t*>(bias);
  auto O = static_cast<uint16_t*>(out);
  if (out_bf16)
    hipLaunchKernelGGL(split_finalize_kernel<true>, fgrid, dim3(256), 0, stream, ws, splits, MN, (int)N, B, O);
  else
    hipLaunchKernelGGL(split_finalize_kernel<false>, fgrid, dim3(256), 0, stream, ws, splits, MN, (int)N, B, O);
  return hipGetLastError();
}

}  // namespace w4
