// Largest key norm per (b, h), the data bound of the exact tile skipping in the
// forward kernel.
//
// With ALiBi every score of row i against key j is at most
//   |q_i| max_j |k_j| / sqrt(d) - m_h (i - j)
// (Cauchy-Schwarz on the content term), so keys far enough behind a query can
// be shown to give exp() values that round to zero, which is the underflow the
// blindness analysis of "When Attention Goes Blind" (Sec. 3.2-3.3, Sec. 5.1)
// describes. This pass produces max_j |k_j| for each (b, h) as P partial maxima
// (the forward takes the max of the P values; for the decode a second kernel
// reduces them to one bound per (b, h)): workgroup (b h, p) covers rows
// p N / P .. (p + 1) N / P - 1. The pass reads K once (B H N d bf16).
#include "device_common.h"
#include "launch.h"

namespace alibi {

namespace {

constexpr int kNormThreads = 256;

template <int D>
__global__ __launch_bounds__(kNormThreads) void knorm_max_kernel(const uint16_t* __restrict__ k,
                                                                 float* __restrict__ out, int N, int P) {
  constexpr int LPR = D / 8;                 // lanes per key row (16 bytes each)
  constexpr int RPP = kNormThreads / LPR;    // rows per pass of the workgroup
  __shared__ float red[kNormThreads / 64];
  const int tid = threadIdx.x;
  const long long bh = blockIdx.x / P;
  const int p = int(blockIdx.x - bh * P);
  const int r0 = int((long long)N * p / P), r1 = int((long long)N * (p + 1) / P);
  const uint16_t* kb = k + bh * (long long)N * D;
  float best = 0.0f;
  for (int r = r0 + tid / LPR; r < r1; r += RPP) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(kb + (long long)r * D + (tid % LPR) * 8);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16lo_to_f32(x[e]), b = bf16hi_to_f32(x[e]);
      s = fmaf(a, a, s);
      s = fmaf(b, b, s);
    }
    best = fmaxf(best, group_sum<LPR>(s));
  }
  best = wave_max(best);
  if ((tid & 63) == 0) red[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kNormThreads / 64; ++w) m = fmaxf(m, red[w]);
    out[blockIdx.x] = sqrtf(m);
  }
}

// out[i] = max_p part[i P + p], one thread per (b, h).
__global__ __launch_bounds__(256) void knorm_reduce_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                           long long n, int P) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float m = 0.0f;
  for (int p = 0; p < P; ++p) m = fmaxf(m, part[i * P + p]);
  out[i] = m;
}

}  // namespace

hipError_t launch_knorm_reduce(const float* part, float* out, long long n, int P, hipStream_t stream) {
  hipLaunchKernelGGL(knorm_reduce_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, part, out, n, P);
  return hipGetLastError();
}

hipError_t launch_knorm_max(const void* k, float* out, int B, int H, int N, int d, int P,
                            hipStream_t stream) {
  const unsigned grid = unsigned((long long)B * H * P);
  if (d == 128)
    hipLaunchKernelGGL(knorm_max_kernel<128>, dim3(grid), dim3(kNormThreads), 0, stream,
                       (const uint16_t*)k, out, N, P);
  else
    hipLaunchKernelGGL(knorm_max_kernel<64>, dim3(grid), dim3(kNormThreads), 0, stream,
                       (const uint16_t*)k, out, N, P);
  return hipGetLastError();
}

}  // namespace alibi
