// Measured matrix-core peak: pure MFMA loops (int8, fp8, bf16), eight
// independent accumulator chains per wave, 4096 waves (four per SIMD), no
// memory traffic inside the loop. The benchmark reports each GEMM's rate as
// a fraction of this measured peak beside the nominal one, and the engine
// clock the int8 rate implies (the nominal peak is quoted at 2.4 GHz).
#include "w4_device.h"

namespace w4 {

constexpr int kPBlocks = 1024, kPThreads = 256, kPChains = 8;

template <int KIND>
__global__ __launch_bounds__(kPThreads) void mfma_peak_kernel(int64_t iters, int32_t* __restrict__ sink) {
  const int t = threadIdx.x;
  const v4i a4 = {t, 3 * t, t ^ 7, 5}, b4 = {t + 1, 9, 5 * t, t ^ 3};
  const v8i a8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, t & 0x38};
  const v4i hb = {0x3F803F80 ^ (t & 1), 0x3F803F80, 0x3F803F80, 0x3F803F80};   // bf16 pairs near 1.0
  v4i ci[kPChains];
  v4f cf[kPChains];
#pragma unroll
  for (int q = 0; q < kPChains; ++q) {
    ci[q] = v4i{0, 0, 0, 0};
    cf[q] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // the MFMAs are asm statements with their accumulators in VGPRs: with the
  // builtins the register allocator moved the accumulators between VGPRs and
  // AGPRs every iteration. Nothing else in the loop touches their registers.
  const uint32_t one_scale = 127u;                 // E8M0 2^0
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < kPChains; ++q) {
      if constexpr (KIND == 0)
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+v"(ci[q]) : "v"(a4), "v"(b4));
      else if constexpr (KIND == 1)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                     : "+v"(cf[q]) : "v"(a8), "v"(a8), "v"(one_scale));
      else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(cf[q]) : "v"(hb), "v"(hb));
    }
  }
  // wait states before vector code reads the last MFMAs' results
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  int32_t s = 0;
#pragma unroll
  for (int q = 0; q < kPChains; ++q) s += ci[q][0] + ci[q][3] + (int32_t)cf[q][0] + (int32_t)cf[q][3];
  sink[(int64_t)blockIdx.x * kPThreads + t] = s;
}

// operations of one launch: blocks * waves * chains * iters * 2*16*16*K of the MFMA
double probe_mfma_ops(int kind, int64_t iters) {
  const double k = kind == 0 ? 64.0 : (kind == 1 ? 128.0 : 32.0);
  return (double)kPBlocks * (kPThreads / 64) * kPChains * (double)iters * 2.0 * 16.0 * 16.0 * k;
}

int64_t probe_sink_elems() { return (int64_t)kPBlocks * kPThreads; }

hipError_t launch_probe_mfma(int kind, int64_t iters, int32_t* sink, hipStream_t stream) {
  const dim3 grid(kPBlocks), block(kPThreads);
  if (kind == 0) hipLaunchKernelGGL((mfma_peak_kernel<0>), grid, block, 0, stream, iters, sink);
  else if (kind == 1) hipLaunchKernelGGL((mfma_peak_kernel<1>), grid, block, 0, stream, iters, sink);
  else hipLaunchKernelGGL((mfma_peak_kernel<2>), grid, block, 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace w4
