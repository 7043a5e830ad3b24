// Generic (VALU-only) ALiBi attention forward for any head size d <= 256, in
// fp32 or bf16, plus the test-only fp32 weight materialisation.
//
// Computes, per query row i of head h (Eq. 1-3 of "When Attention Goes Blind:
// Numerical Failure in ALiBi Positional Encodings"; abhik.ai "From distance to
// a normalized weight"):
//   t_j = (q_i . k_j) / sqrt(d) - m_h * dist(i, j),   dist = i - j (causal, j <= i)
//                                                      or |i - j| (not causal)
//   out_i = sum_j softmax(t)_j v_j
// with positions shifted by the query/key offsets, and optionally the Sec. 3.4
// mitigations of the same paper (bias floor, ln(D + 1) distances, soft-capped
// content logits), evaluated with the precise device math library.
// with an fp32 online softmax in log2 units. One wave owns one query row: the
// head dimension is spread over the 64 lanes (up to 4 values per lane), the
// dot product is a wave reduction, and the keys are walked in order.
// This path serves odd head sizes and exact fp32 checks; the bf16 d = 64/128
// hot path is the MFMA kernel.
#include "device_common.h"
#include "launch.h"

#include <cmath>

namespace alibi {

template <typename T> __device__ __forceinline__ float load_f(const T* p);
template <> __device__ __forceinline__ float load_f<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <typename T> __device__ __forceinline__ void store_f(T* p, float x);
template <> __device__ __forceinline__ void store_f<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_f<uint16_t>(uint16_t* p, float x) { *p = f32_to_bf16(x); }

// Run-time description of one generic launch (natural-log units).
struct GenParams {
  int flags;        // bits 1 clamp, 2 log distance, 4 soft cap (Sec. 3.4 mitigations)
  float clamp_min;  // bias floor
  float softcap;    // z of z tanh(A / z)
  int delta;        // position of query row 0 minus position of key row 0
  float inv_sqrt_d;
  float* lse;       // optional row log-sum-exp output (natural log)
  const int* window;  // optional per-head hard window of W tokens (causal): keys with 0 <= pi - j < W
};

template <typename T>
__global__ __launch_bounds__(256) void fwd_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ out,
    int H, int Nq, int Nk, int d, long long rows, const float* __restrict__ slopes, int causal,
    GenParams gp) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const long long bh = row / Nq;
  const int i = int(row - bh * Nq);
  const int pi = i + gp.delta;  // key-index position of this query
  const int h = int(bh % H);
  const float m = slopes[h];
  const T* qr = q + row * d;
  const T* kb = k + bh * (long long)Nk * d;
  const T* vb = v + bh * (long long)Nk * d;

  float qv[4], acc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int dd = lane + 64 * e;
    qv[e] = dd < d ? load_f(qr + dd) : 0.0f;
    acc[e] = 0.0f;
  }
  float m_run = kNegInf, l_run = 0.0f;
  const int jend = causal ? max(0, min(Nk, pi + 1)) : Nk;
  int jbeg = 0;
  if (gp.window != nullptr) {  // keys j > pi - W ("When Attention Goes Blind", Sec. 5.2-5.3)
    const long long jb = (long long)pi - gp.window[h] + 1;
    jbeg = jb <= 0 ? 0 : (jb >= jend ? jend : int(jb));
  }
  for (int j = jbeg; j < jend; ++j) {
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dd = lane + 64 * e;
      if (dd < d) part += qv[e] * load_f(kb + (long long)j * d + dd);
    }
    // A = q.k / sqrt(d), soft-capped to z tanh(A / z); D = |pi - j| (= pi - j
    // under the causal mask), log-scaled to ln(D + 1); B = -m D, floored at
    // the clamp; the exponent is (A + B) in log2 units
    float a = wave_sum(part) * gp.inv_sqrt_d;
    if (gp.flags & 4) a = gp.softcap * tanhf(a / gp.softcap);
    const int dist = pi - j;
    float dd = float(dist < 0 ? -dist : dist);
    if (gp.flags & 2) dd = log1pf(dd);
    float bias = -m * dd;
    if (gp.flags & 1) bias = fmaxf(bias, gp.clamp_min);
    const float t = (a + bias) * kLog2e;
    const float m_new = fmaxf(m_run, t);
    const float alpha = fast_exp2(m_run - m_new);  // exp2(-inf) = 0 on the first key
    const float p = fast_exp2(t - m_new);
    l_run = l_run * alpha + p;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dd = lane + 64 * e;
      const float vv = dd < d ? load_f(vb + (long long)j * d + dd) : 0.0f;
      acc[e] = acc[e] * alpha + p * vv;
    }
    m_run = m_new;
  }
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;  // a row that saw no key gives 0
  if (gp.lse != nullptr && lane == 0) gp.lse[row] = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int dd = lane + 64 * e;
    if (dd < d) store_f(out + row * d + dd, acc[e] * inv);
  }
}

// Test-only: weights w[b,h,i,:] of the fp32 forward, one wave per row, N <= 1024.
__global__ __launch_bounds__(256) void weights_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, float* __restrict__ w,
    int H, int N, int d, long long rows, const float* __restrict__ slopes, int causal, float c1) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const long long bh = row / N;
  const int i = int(row - bh * N);
  const int h = int(bh % H);
  const float c2 = slopes[h] * kLog2e;
  const float* qr = q + row * d;
  const float* kb = k + bh * (long long)N * d;
  float t[16];
  float mx = kNegInf;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const int j = lane + 64 * c;
    t[c] = kNegInf;
    if (j < N && !(causal && j > i)) {
      float s = 0.0f;
      for (int e = 0; e < d; ++e) s += qr[e] * kb[(long long)j * d + e];
      const int dist = i - j;
      t[c] = s * c1 - c2 * float(dist < 0 ? -dist : dist);
    }
    mx = fmaxf(mx, t[c]);
  }
  mx = wave_max(mx);
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    t[c] = fast_exp2(t[c] - mx);  // masked: exp2(-inf) = exactly 0
    sum += t[c];
  }
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const int j = lane + 64 * c;
    if (j < N) w[row * N + j] = t[c] * inv;
  }
}

hipError_t launch_fwd_generic(const FwdArgs& a, const FwdOptions& opt, bool f32, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.Nq;
  const unsigned grid = unsigned((rows + 3) / 4);
  GenParams gp;
  gp.flags = opt.flags;
  gp.clamp_min = opt.clamp_min;
  gp.softcap = opt.softcap;
  gp.delta = opt.q_offset - opt.k_offset;
  gp.inv_sqrt_d = float(1.0 / std::sqrt(double(a.d)));
  gp.lse = opt.lse;
  gp.window = opt.window;
  if (f32)
    hipLaunchKernelGGL(fwd_generic_kernel<float>, dim3(grid), dim3(256), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.out,
                       a.H, a.Nq, a.Nk, a.d, rows, a.slopes, a.causal, gp);
  else
    hipLaunchKernelGGL(fwd_generic_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.out, a.H, a.Nq, a.Nk, a.d, rows, a.slopes, a.causal, gp);
  return hipGetLastError();
}

hipError_t launch_weights_f32(const float* q, const float* k, float* w, int B, int H, int N, int d,
                              const float* slopes, int causal, float c1, hipStream_t stream) {
  const long long rows = (long long)B * H * N;
  const unsigned grid = unsigned((rows + 3) / 4);
  hipLaunchKernelGGL(weights_f32_kernel, dim3(grid), dim3(256), 0, stream,
                     q, k, w, H, N, d, rows, slopes, causal, c1);
  return hipGetLastError();
}

}  // namespace alibi
