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
//
// With VALU, each MFMA is followed by the vector work the forward's softmax
// issues per MFMA on an open tile (an fma, an exponential, half a bf16 pack,
// half a bf16 dot for the row sum, and an add), on data independent of the
// MFMAs: the rate of the forward's instruction mix without its memory traffic
// and without dependency stalls. That work feeds the sink only through a
// comparison that never holds, so the sums stay the MFMA sums.
#include "device_common.h"
#include "launch.h"

namespace alibi {

namespace {

constexpr int kRateWaves = 8;

template <bool VALU>
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
  // softmax-like state: eight values near the fixed point of x = 2^(x/16 - 1)
  float x[8], lsum = 0.0f, prev = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.01f * float(lane + i);
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      acc[n & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[n & 3], b[n >> 2], acc[n & 3], 0, 0, 0);
      if constexpr (VALU) {
        const float e = fast_exp2(fmaf(x[n & 7], 0.0625f, -1.0f));
        if (n & 1)
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pack_bf16x2(prev, e)), one, lsum, false);
        prev = e;
        x[n & 7] = e + 1.0e-3f;
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if constexpr (VALU) {
    float t = lsum;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += x[i];
    if (t == -1.0f) s += 1.0f;  // never: the terms are positive
  }
  s = wave_sum(s);
  if (lane == 0) sink[blockIdx.x * kRateWaves + wave] = s;
}

}  // namespace

hipError_t launch_mfma_rate(const void* frags, int iters, bool valu, float* sink, int workgroups,
                            hipStream_t stream) {
  if (valu)
    hipLaunchKernelGGL(mfma_rate_kernel<true>, dim3(unsigned(workgroups)), dim3(kRateWaves * 64), 0, stream,
                       static_cast<const u32x4*>(frags), iters, sink);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<false>, dim3(unsigned(workgroups)), dim3(kRateWaves * 64), 0, stream,
                       static_cast<const u32x4*>(frags), iters, sink);
  return hipGetLastError();
}

}  // namespace alibi
