// Back-to-back bf16 MFMAs from registers: the sustained matrix rate of the
// part, against which the forward's MFMA rate is read beside the datasheet
// peak. Measurement tool only, not on the attention path.
//
// Every wave of an 8-wave workgroup (two waves per SIMD, as in the forward)
// loads four A and four B operand fragments of v_mfma_f32_32x32x16_bf16 (16
// bytes per lane each) and runs `iters` rounds of 16 MFMAs over four
// independent accumulator chains: chain c multiplies A_c by B_0 .. B_3 in turn,
// so after the loop it holds iters * sum_m A_c B_m. No memory is touched
// inside the loop. Each wave writes the sum of all its accumulator values to
// sink[workgroup * 8 + wave]; the sum of the elements of A_c B_m is
// sum_k colsum(A_c)[k] rowsum(B_m)[k] whatever the accumulator layout, which
// lets a host check that every MFMA ran with the given operands.
#include "device_common.h"
#include "launch.h"

namespace alibi {

namespace {

constexpr int kRateWaves = 8;

__global__ __launch_bounds__(kRateWaves * 64, 2) void mfma_rate_kernel(const u32x4* __restrict__ frags, int iters,
                                                                       float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, frags[i * 64 + lane]);
    b[i] = __builtin_bit_cast(bf16x8, frags[(4 + i) * 64 + lane]);
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int n = 0; n < 16; ++n)
      acc[n & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[n & 3], b[n >> 2], acc[n & 3], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  s = wave_sum(s);
  if (lane == 0) sink[blockIdx.x * kRateWaves + wave] = s;
}

}  // namespace

hipError_t launch_mfma_rate(const void* frags, int iters, float* sink, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(unsigned(workgroups)), dim3(kRateWaves * 64), 0, stream,
                     static_cast<const u32x4*>(frags), iters, sink);
  return hipGetLastError();
}

}  // namespace alibi
