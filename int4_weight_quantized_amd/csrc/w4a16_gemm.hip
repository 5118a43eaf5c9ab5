// W4A16 decode GEMM (M <= 16) on the asymmetric grid w = (q - 8)*scale + zero.
//
// Per the cpu_int4.py page (module docstring, pack_nibbles): single-stream
// decode is bound by the bytes of the weights read per token; bf16
// activations; two codes per byte, byte j = w[2j] | w[2j+1] << 4; bf16
// scale and zero per (output row, group of K). Like that page's own kernel
// layout, the weights are repacked once at load time into the layout the
// kernel streams.
//
//   out[m,n] = sum_g ( scale[n,g] * sum_{k in g} x[m,k]*(q[n,k]-8)
//                    + zero[n,g]  * sum_{k in g} x[m,k] )
//
// Tiled layout (w4a16_repack): 16-row tiles x 512-wide K windows.
//   weights  [row tile][window] 4 KiB: four 1 KiB unit pairs; in a pair, lane
//            l = n + 16 j (n: row in tile, j: 0..3) owns 16 bytes: 8 bytes of
//            unit 2p then 8 of unit 2p+1 (a unit is 64 K); each 8 bytes are
//            two words for K = 16 j + 0..7 and 16 j + 8..15 of the unit, in a
//            word nibble i < 4 holds K offset 2i and nibble i >= 4 offset
//            2(i-4)+1. Padding codes are 8.
//   scale/zero [row tile][window][row 16][8 group slots][scale, zero] bf16
//            (slots past the window's groups and padding are 0).
//
// Design (gfx950), HBM-bound: 0.5 byte per weight + 4 bytes per (row, group).
// - Every wave-wide load is 1 KiB contiguous (16-byte lanes in order).
// - v_mfma_f32_16x16x32_bf16: activations are the 16-row A operand (rows >= M
//   are zero), 16 weight rows the B operand. Word w unpacks to bf16 128+q in
//   K order with ((w >> 4i) & 0x000F000F) | 0x43004300 (one v_and_or_b32):
//   0x4300 | q is the bf16 bit pattern of 128+q, exact. Row sums XS = sum_k x
//   come from the MFMA against ones; the group's product accumulator starts
//   at -136*XS, so it ends at sum_k x*(q-8), and per group
//     y += scale*C + zero*XS.
// - A 1024-thread block owns RT row tiles; its 16 waves take the two halves
//   of the 8 windows of a 4096-wide K pass (fewer than 128 VGPRs each, so
//   four waves share a SIMD) and keep their activations in registers for all
//   RT tiles. A pass loads the activations and the first tile up front, then
//   issues each next tile's weight and scale loads just before it computes
//   the current one (raw buffer loads: masked rows/units read as zero). One
//   tile in flight per wave keeps the stream going and lets each tile's
//   unpack overlap the next tile's transfer; issuing every tile at once made
//   all of them arrive late together. Partial tiles of the 16 waves are
//   summed through LDS.
// - Up to 4 rows over K <= 4096 (decode at batch 1-4, the tied output head)
//   take w4a16_tile_kernel instead: one row tile per block and one window
//   per wave, every block resident at once and every load issued up front,
//   activations staged per wave in LDS and their group sums taken on the
//   vector ALU (no MFMA against ones). Without a chain of tiles, the work
//   left once a wave's bytes land is a single window's.
#include "w4_device.h"

namespace w4 {

constexpr int kDThreads = 512;             // one wave per window of a 4096-wide pass
constexpr int kDWaves = kDThreads / kWave; // windows per pass
constexpr int kWinK = 512;                 // K per window (8 units of 64)
constexpr int kWPW = 2;                    // waves per window
constexpr int kWTile = 4096;               // weight bytes per (row tile, window)
constexpr int kSZTile = 16 * 8 * 2 * 2;    // scale/zero bytes per (row tile, window)

__device__ __forceinline__ v8bf as_v8bf(v4i v) { return __builtin_bit_cast(v8bf, v); }
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// (a & mask) | magic in one v_and_or_b32. gfx9 VOP3 encodes no literal and
// reads at most one scalar operand, so the caller keeps the mask in an SGPR
// and the magic in a VGPR, both made opaque so the compiler cannot fold them
// back into literals; the and-or itself stays plain code.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask_s, uint32_t magic_v) {
  return (a & mask_s) | magic_v;
}

// two words -> 4 registers each of bf16 pairs 128+q, K order (see the tiled
// layout): word w gives ((w >> 4i) & 0x000F000F) | 0x43004300, i = 0..3;
// each shift is one 64-bit shift of the pair (the bits carried into the low
// word land where the mask clears them)
__device__ __forceinline__ void unpack2_bf16_128q(uint64_t w01, uint32_t mask_s, uint32_t magic_v, v4i& r0, v4i& r1) {
  const uint32_t w0 = (uint32_t)w01, w1 = (uint32_t)(w01 >> 32);
  const uint64_t s4 = shr64<4>(w01), s8 = shr64<8>(w01), s12 = shr64<12>(w01);
  r0[0] = (int)and_or(w0, mask_s, magic_v);
  r1[0] = (int)and_or(w1, mask_s, magic_v);
  r0[1] = (int)and_or((uint32_t)s4, mask_s, magic_v);
  r1[1] = (int)and_or((uint32_t)(s4 >> 32), mask_s, magic_v);
  r0[2] = (int)and_or((uint32_t)s8, mask_s, magic_v);
  r1[2] = (int)and_or((uint32_t)(s8 >> 32), mask_s, magic_v);
  r0[3] = (int)and_or((uint32_t)s12, mask_s, magic_v);
  r1[3] = (int)and_or((uint32_t)(s12 >> 32), mask_s, magic_v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// RT: row tiles per block; UPG: 64-wide units per group (1, 2, 4 or 8);
// MV: accumulator registers that hold real rows (M <= 4: rows sit in lanes
// 0-15, register r = row; M > 4: all four), the epilogue skips the rest;
// WPW: waves per 512-wide window (1 or 2): each wave takes UPW = 8/WPW units
// of its window. The epilogue is linear in a group's partial sums, so a group
// split between two waves is finished by each wave on its own part.
template <int RT, int UPG, int MV, int WPW>
__global__ __launch_bounds__(kDThreads * WPW, 1) void w4a16_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wt, const uint8_t* __restrict__ szt,
    uint16_t* __restrict__ out, int M, int N, int K, int NT16, int KW) {
  constexpr int NW = kDWaves * WPW;                 // waves per block
  constexpr int UPW = 8 / WPW;                      // units per wave and window
  constexpr int PPW = UPW / 2;                      // 1 KiB unit pairs per wave and tile
  constexpr int NG = UPW >= UPG ? UPW / UPG : 1;    // groups (or group parts) per wave
  constexpr int NSZ = (NG + 3) / 4;                 // 16-byte scale/zero registers per tile
  __shared__ __attribute__((aligned(16))) float red[NW][RT][kWave][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, j = lane >> 4;
  const int rt0 = blockIdx.x * RT;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // uniform: scalar load offsets
  const int u0 = (wave_u % WPW) * UPW;                        // first unit of this wave in a window

  // Loads: a fixed per-lane VGPR offset, the tile base in the scalar offset
  // (clamped to the last tile, so every weight and scale access is in bounds)
  // and the pair in the immediate. The activation offset keeps the window in
  // the range-checked VGPR: rows past M and the bytes past the matrix read as
  // zero. The scale/zero load starts at this wave's first group slot, so slot
  // i/UPG of the register belongs to local unit i.
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wt, (uint32_t)((int64_t)NT16 * KW * kWTile));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(szt, (uint32_t)((int64_t)NT16 * KW * kSZTile));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * K * 2));
  const uint32_t x_lane = (uint32_t)(l16 * K + 16 * j + 64 * u0) * 2u;
  const uint32_t w_lane = 16u * lane + 512u * (uint32_t)u0;
  const uint32_t s_lane = 32u * l16 + 4u * (uint32_t)(u0 / UPG);

  float y[RT][MV];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int r = 0; r < MV; ++r) y[t][r] = 0.f;
  const v4i ones = {0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80};
  const v4f z4 = {0.f, 0.f, 0.f, 0.f};
  uint32_t mask_s, magic_v;
  asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(mask_s));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(magic_v));

  auto first_of_group = [](int i) { return i % UPG == 0; };
  auto last_of_group = [](int i) { return i % UPG == UPG - 1 || i == UPW - 1; };

  for (int kw = wave_u / WPW; kw < KW; kw += kDWaves) {
    // ---- activations of this wave's units, then the first row tile
    v4i xa[UPW][2];
    const uint32_t xo = x_lane + (uint32_t)kw * (kWinK * 2);
#pragma unroll
    for (int i = 0; i < UPW; ++i)
#pragma unroll
      for (int s_ = 0; s_ < 2; ++s_) xa[i][s_] = buffer_load16(xr, xo + 128u * i + 16u * s_);
    v4i wv[RT][PPW], szv[RT][NSZ];
    auto load_tile = [&](int t) {
      // a tile past NT16 (last block) reloads the last tile; its rows are not stored
      const uint32_t tile = (uint32_t)(min(rt0 + t, NT16 - 1) * KW + kw);
#pragma unroll
      for (int p = 0; p < PPW; ++p)
        wv[t][p] = __builtin_amdgcn_raw_buffer_load_b128(wr, w_lane + 1024u * p, tile * kWTile, 0);
#pragma unroll
      for (int q = 0; q < NSZ; ++q)
        szv[t][q] = __builtin_amdgcn_raw_buffer_load_b128(sr, s_lane + 16u * q, tile * kSZTile, 0);
    };
    load_tile(0);
    __builtin_amdgcn_sched_barrier(0);       // keep these loads ahead of all compute

    // ---- activation row sums per group (shared by the row tiles): XS of
    // local group gi in xs[gi]; the group's product accumulator starts at -136*XS
    v4f xs[NG], xinit[NG];
    {
      v4f run = z4;
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        const v4f a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(xa[i][0]), as_v8bf(ones),
                                                              first_of_group(i) ? z4 : run, 0, 0, 0);
        run = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(xa[i][1]), as_v8bf(ones), a, 0, 0, 0);
        if (last_of_group(i)) {
          xs[i / UPG] = run;
#pragma unroll
          for (int r = 0; r < 4; ++r) xinit[i / UPG][r] = (r < MV) ? -136.f * run[r] : 0.f;
        }
      }
    }

    // ---- row tiles
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if (t + 1 < RT) load_tile(t + 1);        // next tile in flight while this one computes
      __builtin_amdgcn_sched_barrier(0);
      v4f c = z4;
#pragma unroll
      for (int i = 0; i < UPW; ++i) {
        // c = sum_k x*(128+q) - 136*XS = sum_k x*(q-8) over the group
        v4i u0, u1;
        unpack2_bf16_128q(as_u64x2(wv[t][i >> 1])[i & 1], mask_s, magic_v, u0, u1);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(xa[i][0]), as_v8bf(u0),
                                                    first_of_group(i) ? xinit[i / UPG] : c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(xa[i][1]), as_v8bf(u1), c, 0, 0, 0);
        if (last_of_group(i)) {
          const int gi = i / UPG;                      // local group slot
          const uint32_t sz = (uint32_t)szv[t][gi >> 2][gi & 3];
          const float s_ = bf16_lo(sz), z = bf16_hi(sz);
#pragma unroll
          for (int r = 0; r < MV; ++r) y[t][r] = fmaf(s_, c[r], fmaf(z, xs[gi][r], y[t][r]));
        }
      }
    }
  }

#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int r = 0; r < MV; ++r) red[wave][t][lane][r] = y[t][r];
  __syncthreads();
  for (int e = tid; e < RT * 256; e += kDThreads * WPW) {
    const int t = e >> 8, m = (e >> 4) & 15, nn = e & 15;   // output (m, 16*(rt0+t) + nn)
    const int l = nn + 16 * (m >> 2), r = m & 3;
    const int n = 16 * (rt0 + t) + nn;
    if (m < M && n < N) {
      float acc = 0.f;
#pragma unroll
      for (int w_ = 0; w_ < NW; ++w_) acc += red[w_][t][l][r];
      out[(int64_t)m * N + n] = f32_to_bf16_rne(acc);
    }
  }
}

// Few rows (M <= 4) over K <= 4096 (at most 8 windows): one row tile per
// block, one window per wave (NWV = 4 waves for K <= 2048, else 8). Every
// block of a 14336-row matrix is resident at once (46-66 VGPRs: seven or
// eight waves per SIMD, 896 blocks of eight waves), and each wave issues all of its
// loads up front -- its activation rows, then its scale/zero pairs, then
// its 4 KiB of weights -- so the matrix is requested in a single pass with
// no chain of tiles behind any block, and the work left once a wave's
// bytes land is one window's. The activation rows arrive one 16-byte piece
// per lane (8 consecutive K of a row); from them the wave takes the group
// sums XS (dot products with ones, a butterfly over the lanes of a group,
// read out as wave-uniform values) and stages the rows in its own LDS
// region, from which each unit's A fragments are read as the weights
// arrive (lanes of rows past M read a zero block). A group's accumulator
// starts at zero and its epilogue folds the -136 offset into the zero
// point: y += scale*C + (zero - 136*scale)*XS. A wave whose window is past
// KW reads nothing (offsets past the buffers load zero, whose share is zero).
template <int UPG, int MV, int NWV>
__global__ __launch_bounds__(64 * NWV, 32 / NWV) void w4a16_tile_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wt, const uint8_t* __restrict__ szt,
    uint16_t* __restrict__ out, int M, int N, int K, int NT16, int KW) {
  constexpr int NG = 8 / UPG;                 // groups per window
  constexpr int NSZ = (NG + 3) / 4;           // 16-byte scale/zero registers per window
  constexpr int kXRow = 1024 + 16;            // LDS bytes per staged row (512 K, padded)
  constexpr int kXWave = MV * kXRow + 16;     // a wave's rows, then its zero block
  __shared__ __attribute__((aligned(16))) uint8_t xl[NWV * kXWave];
  __shared__ __attribute__((aligned(16))) float red[NWV][16][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, j = lane >> 4;
  const int rt = blockIdx.x;
  const int kw = __builtin_amdgcn_readfirstlane(wave);     // this wave's window
  const bool have = kw < KW;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wt, (uint32_t)((int64_t)NT16 * KW * kWTile));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(szt, (uint32_t)((int64_t)NT16 * KW * kSZTile));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * K * 2));
  constexpr uint32_t kPast = 0x80000000u;     // an offset past every buffer: loads zero

  // ---- every load of the wave: activations, scale/zero pairs, weights
  v4i xv[MV], szv[NSZ], wv[4];
#pragma unroll
  for (int m = 0; m < MV; ++m)
    xv[m] = buffer_load16(xr, have ? (uint32_t)(m * K + kw * kWinK + 8 * lane) * 2u : kPast);
  {
    const uint32_t base = have ? (uint32_t)(rt * KW + kw) * kSZTile + 32u * l16 : kPast;
#pragma unroll
    for (int q = 0; q < NSZ; ++q) szv[q] = buffer_load16(sr, base + 16u * q);
  }
  {
    const uint32_t base = have ? (uint32_t)(rt * KW + kw) * kWTile + 16u * lane : kPast;
#pragma unroll
    for (int p = 0; p < 4; ++p) wv[p] = buffer_load16(wr, base + 1024u * p);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- group sums of the activation rows: lane L holds K 8L .. 8L+7 of the
  // window, so a group is 8*UPG lanes; XS of group g, row m ends up uniform
  // in xsum[m][g]
  float xsum[MV][NG];
  {
    const v2bf one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // through a scalar copy: a bit cast straight from the vector
        // element reads element 0 whatever q is (hipcc 7.2)
        const uint32_t w2 = (uint32_t)xv[m][q];
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, w2), one2, t, false);
      }
#pragma unroll
      for (int off = 1; off < 8 * UPG; off <<= 1) t += __shfl_xor(t, off, kWave);
#pragma unroll
      for (int g = 0; g < NG; ++g) xsum[m][g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 8 * UPG * g));
    }
  }

  // ---- stage the activation rows in the wave's LDS region (row m at
  // m*kXRow), and its zero block
  uint8_t* xw = xl + kw * kXWave;
#pragma unroll
  for (int m = 0; m < MV; ++m) *reinterpret_cast<v4i*>(xw + m * kXRow + 16 * lane) = xv[m];
  if (lane == 0) *reinterpret_cast<v4i*>(xw + MV * kXRow) = v4i{0, 0, 0, 0};
  // A fragment of unit i, half h: row l16, K 64i + 16j + 8h .. +7
  const int a_lane = l16 < MV ? l16 * kXRow + 32 * j : -1;
  auto read_a = [&](int i, int h) -> v4i {
    const int off = a_lane >= 0 ? a_lane + 128 * i + 16 * h : MV * kXRow;
    return *reinterpret_cast<const v4i*>(xw + off);
  };

  const v4f z4 = {0.f, 0.f, 0.f, 0.f};
  uint32_t mask_s, magic_v;
  asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(mask_s));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(magic_v));
  float y[MV];
#pragma unroll
  for (int r = 0; r < MV; ++r) y[r] = 0.f;

#pragma unroll
  for (int g = 0; g < NG; ++g) {
    v4f c = z4;                                // sum_k x*(128+q) over the group
#pragma unroll
    for (int ii = 0; ii < UPG; ++ii) {
      const int i = g * UPG + ii;
      const v4i a0 = read_a(i, 0), a1 = read_a(i, 1);
      v4i u0, u1;
      unpack2_bf16_128q(as_u64x2(wv[i >> 1])[i & 1], mask_s, magic_v, u0, u1);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(a0), as_v8bf(u0), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(a1), as_v8bf(u1), c, 0, 0, 0);
    }
    const uint32_t sz = (uint32_t)szv[g >> 2][g & 3];
    const float s_ = bf16_lo(sz), zc = fmaf(-136.f, s_, bf16_hi(sz));
#pragma unroll
    for (int r = 0; r < MV; ++r) y[r] = fmaf(s_, c[r], fmaf(zc, xsum[r][g], y[r]));
  }

  // ---- the waves' partial sums: rows m < 4 sit in lanes 0-15, register m
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < MV; ++r) red[wave][lane][r] = y[r];
  }
  __syncthreads();
  if (tid < 16 * M) {
    const int m = tid >> 4, nn = tid & 15, n = 16 * rt + nn;
    float acc = 0.f;
#pragma unroll
    for (int w_ = 0; w_ < NWV; ++w_) acc += red[w_][nn][m];
    if (n < N) out[(int64_t)m * N + n] = f32_to_bf16_rne(acc);
  }
}

// ---------------------------------------------------------------- repack

__device__ __forceinline__ uint32_t p5_code(const uint8_t* w, int N, int K, int n, int k) {
  if (n >= N || k >= K) return 8u;
  const uint8_t b = w[(int64_t)n * (K >> 1) + (k >> 1)];
  return (k & 1) ? (uint32_t)(b >> 4) : (uint32_t)(b & 0xF);
}

// one thread per 32-bit word of the weight tiles
__global__ __launch_bounds__(256) void w4a16_repack_w_kernel(const uint8_t* __restrict__ w, int N, int K, int KW,
                                                             uint32_t* __restrict__ dst, int64_t words) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= words) return;
  const int64_t tile = id / (kWTile / 4);
  const int in = (int)(id % (kWTile / 4));
  const int p = in >> 8, lane = (in >> 2) & 63, wi = in & 3;
  const int rt = (int)(tile / KW), kw = (int)(tile % KW);
  const int n = rt * 16 + (lane & 15), jj = lane >> 4;
  const int u = kw * 8 + 2 * p + (wi >> 1);
  const int kb = u * 64 + 16 * jj + 8 * (wi & 1);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = (i < 4) ? 2 * i : 2 * (i - 4) + 1;
    word |= p5_code(w, N, K, n, kb + e) << (4 * i);
  }
  dst[id] = word;
}

// one thread per (row tile, window, row, slot): scale and zero of one group
__global__ __launch_bounds__(256) void w4a16_repack_sz_kernel(const uint16_t* __restrict__ scale,
                                                              const uint16_t* __restrict__ zero, int N, int G,
                                                              int upg, int KW, uint32_t* __restrict__ dst,
                                                              int64_t entries) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= entries) return;
  const int slot = (int)(id & 7), row = (int)((id >> 3) & 15);
  const int64_t tile = id >> 7;
  const int rt = (int)(tile / KW), kw = (int)(tile % KW);
  const int n = rt * 16 + row;
  const int gpw = 8 / upg;
  const int g = kw * gpw + slot;
  uint32_t v = 0;
  if (n < N && slot < gpw && g < G) {
    const uint32_t s = scale[(int64_t)n * G + g];
    const uint32_t z = zero ? zero[(int64_t)n * G + g] : 0u;
    v = s | (z << 16);
  }
  dst[id] = v;
}

void w4a16_tiled_bytes(int64_t K, int64_t N, size_t* wbytes, size_t* szbytes) {
  const int64_t NT16 = (N + 15) / 16, KW = (K + kWinK - 1) / kWinK;
  *wbytes = (size_t)(NT16 * KW * kWTile);
  *szbytes = (size_t)(NT16 * KW * kSZTile);
}

hipError_t launch_w4a16_repack(const uint8_t* w, const void* scale, const void* zero, int64_t group, int64_t K,
                               int64_t N, void* w_tiled, void* sz_tiled, hipStream_t stream) {
  const int NT16 = (int)((N + 15) / 16), KW = (int)((K + kWinK - 1) / kWinK);
  const int64_t words = (int64_t)NT16 * KW * (kWTile / 4);
  hipLaunchKernelGGL(w4a16_repack_w_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream, w, (int)N,
                     (int)K, KW, static_cast<uint32_t*>(w_tiled), words);
  const int64_t entries = (int64_t)NT16 * KW * 128;
  hipLaunchKernelGGL(w4a16_repack_sz_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(scale), static_cast<const uint16_t*>(zero), (int)N,
                     (int)(K / group), (int)(group / 64), KW, static_cast<uint32_t*>(sz_tiled), entries);
  return hipGetLastError();
}

static hipError_t launch_w4a16_tile(const void* x, const void* w_tiled, const void* sz_tiled, int upg, void* out,
                                    int64_t M, int64_t N, int64_t K, int NT16, int KW, hipStream_t stream) {
  auto X = static_cast<const uint16_t*>(x);
  auto Wt = static_cast<const uint8_t*>(w_tiled);
  auto St = static_cast<const uint8_t*>(sz_tiled);
  auto O = static_cast<uint16_t*>(out);
  const int iM = (int)M, iN = (int)N, iK = (int)K;
  const int mv = M == 1 ? 1 : (M == 2 ? 2 : 4);
  const bool eight = KW > 4;
#define W4A16T_LAUNCH(UPG_, MV_, NWV_)                                                                     \
  hipLaunchKernelGGL((w4a16_tile_kernel<UPG_, MV_, NWV_>), dim3(NT16), dim3(64 * NWV_), 0, stream, X, Wt, St, O, iM, \
                     iN, iK, NT16, KW)
#define W4A16T_NWV(UPG_, MV_)                                            \
  { if (eight) W4A16T_LAUNCH(UPG_, MV_, 8); else W4A16T_LAUNCH(UPG_, MV_, 4); }
#define W4A16T_MV(UPG_)                                  \
  switch (mv) {                                          \
    case 1: W4A16T_NWV(UPG_, 1) break;                   \
    case 2: W4A16T_NWV(UPG_, 2) break;                   \
    default: W4A16T_NWV(UPG_, 4) break;                  \
  }
  switch (upg) {
    case 1: W4A16T_MV(1) break;
    case 2: W4A16T_MV(2) break;
    case 4: W4A16T_MV(4) break;
    default: W4A16T_MV(8) break;
  }
#undef W4A16T_MV
#undef W4A16T_NWV
#undef W4A16T_LAUNCH
  return hipGetLastError();
}

hipError_t launch_w4a16(const void* x, const void* w_tiled, const void* sz_tiled, int64_t group, void* out,
                        int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int NT16 = (int)((N + 15) / 16), KW = (int)((K + kWinK - 1) / kWinK);
  const int upg = (int)(group / 64);
  if (M <= 4 && KW <= 8) return launch_w4a16_tile(x, w_tiled, sz_tiled, upg, out, M, N, K, NT16, KW, stream);
  // row tiles per block: enough blocks to cover ~all CUs, at most 4 tiles each
  int rt = (NT16 + 255) / 256;
  rt = rt <= 1 ? 1 : (rt == 2 ? 2 : 4);
  const int mv = M == 1 ? 1 : (M == 2 ? 2 : 4);
  dim3 grid((unsigned)((NT16 + rt - 1) / rt));
  auto X = static_cast<const uint16_t*>(x);
  auto Wt = static_cast<const uint8_t*>(w_tiled);
  auto St = static_cast<const uint8_t*>(sz_tiled);
  auto O = static_cast<uint16_t*>(out);
  const int iM = (int)M, iN = (int)N, iK = (int)K;
#define W4A16_LAUNCH(RT_, UPG_, MV_) \
  hipLaunchKernelGGL((w4a16_kernel<RT_, UPG_, MV_, kWPW>), grid, dim3(kDThreads * kWPW), 0, stream, X, Wt, St, O, iM, iN, iK, NT16, KW)
#define W4A16_MV(RT_, UPG_)                             \
  switch (mv) {                                         \
    case 1: W4A16_LAUNCH(RT_, UPG_, 1); break;          \
    case 2: W4A16_LAUNCH(RT_, UPG_, 2); break;          \
    default: W4A16_LAUNCH(RT_, UPG_, 4); break;         \
  }
#define W4A16_RT(UPG_)                        \
  switch (rt) {                               \
    case 1: W4A16_MV(1, UPG_) break;          \
    case 2: W4A16_MV(2, UPG_) break;          \
    default: W4A16_MV(4, UPG_) break;         \
  }
  switch (upg) {
    case 1: W4A16_RT(1) break;
    case 2: W4A16_RT(2) break;
    case 4: W4A16_RT(4) break;
    default: W4A16_RT(8) break;
  }
#undef W4A16_RT
#undef W4A16_MV
#undef W4A16_LAUNCH
  return hipGetLastError();
}

}  // namespace w4
