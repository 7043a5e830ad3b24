// Split-KV single-query ALiBi decode for gfx950.
//
// One new query per (b, h) sits at position L-1 and attends to every cached key
// j at its real position, with bias -m_h (L-1-j) (abhik.ai: with a KV cache the
// query and key positions are their actual sequence positions). The pass is
// bound by streaming the K and V caches from HBM, so the kernel is laid out for
// bandwidth: each workgroup owns one key range of one (b, h); groups of
// LPK = d/8 lanes own one key row at a time (16 bytes of K and of V per lane per
// key, so a wave reads whole contiguous rows), U keys per group are in flight
// per iteration, and keys are walked from the newest backwards so the running
// maximum settles early and the accumulator is rescaled only when the maximum
// grows by more than 2^8 (a lazy rescale, exact up to fp32 rounding).
// Partial softmax states (m, l, acc) of the key ranges are merged with the
// stable-softmax algebra of "When Attention Goes Blind", App. B.1-B.2.
//
// Exact underflow skipping (knorm != null: an upper bound of |k_j| over the
// cache of each (b, h)): every score is at most A - c2 D with
// A = |q| max|k| c1 (Cauchy-Schwarz; D the distance L - 1 - j, scores in log2
// units), and the score of key L - 1 is at least -A. The combined maximum is
// therefore at least -A, so a key range whose nearest key lies at D0 with
// c2 D0 > 2 A + 152 enters the combine with weight 2^(m_s - M) < 2^-150, an
// exact zero: it is not read at all. Inside a range, a key group's running
// maximum is at least its first key's score, at most G - 1 keys behind the
// range's nearest one, so keys beyond D0 + G - 1 + (2 A + 152) / c2 give
// exp2 values below 2^-150, exact zeros that cannot move the maximum either:
// the walk, newest keys first, stops there. The output is bit for bit the
// unskipped one whenever the bound holds (and the caches are finite); most of
// a steep head's cache is then never read ("When Attention Goes Blind",
// Sec. 3.3 and 5.1-5.2: the weights of distant keys underflow to zero).
#include "device_common.h"
#include "launch.h"

#include <mutex>

namespace alibi {

namespace {

// Scratch for the decode variant that allocates nothing: the partial softmax
// states of the split key ranges, B H S (d + 2) floats. decode_plan keeps
// B H S below 4096 + B H (S > 1 only for B H < 4096), so 8191 (256 + 2) floats
// hold every plan for d <= 256. One copy per device, alive until the process
// ends; host code uses the address resolved per device below, never the name.
constexpr size_t kScratchFloats = size_t(8191) * (256 + 2);
static __device__ __align__(256) float scratch[kScratchFloats];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

constexpr int kDecodeThreads = 256;
constexpr int kDecodeUnroll = 8;
constexpr float kLazyRescale = 8.0f;  // log2 units

template <int LPK>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    uint16_t* __restrict__ out, float* __restrict__ ws, int H, int L, int d, int splits, int chunk,
    const float* __restrict__ slopes, float c1, const float* __restrict__ knorm) {
  constexpr int G = kDecodeThreads / LPK;  // key groups per workgroup
  constexpr int U = kDecodeUnroll;
  __shared__ float sm_m[G];
  __shared__ float sm_l[G];
  __shared__ float sm_acc[G][8 * LPK + 1];

  const int tid = threadIdx.x;
  const int g = tid / LPK;
  const int sub = tid % LPK;
  // Workgroup -> (key range, head, batch), the newest range first. With the
  // exact skipping only the ranges near the query hold work, most of it in
  // the shallow heads; in this order consecutive workgroups, which are dealt
  // to the 8 XCDs round-robin, take the batches of one (range, head), so that
  // work spreads over every XCD (in pair-major order, with 4 ranges per pair,
  // range s of every pair fell on XCDs s and s + 4). The plain decode runs
  // equally fast in either order.
  const long long nbh = gridDim.x / splits;
  const int nb = int(nbh / H);
  const long long w = blockIdx.x;
  const int s = splits - 1 - int(w / nbh);
  const long long bh = (w % nb) * H + (w / nb) % H;
  const int h = int(bh % H);
  const float c2 = slopes[h] * kLog2e;
  const int jbeg = s * chunk;
  const int jend = min(L, jbeg + chunk);
  const bool dvalid = sub * 8 < d;

  // Query chunk with the softmax scale (in log2 units) folded in.
  float qf[8];
  {
    u32x4 qq = {0u, 0u, 0u, 0u};
    if (dvalid) qq = *reinterpret_cast<const u32x4*>(q + bh * d + sub * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[2 * e] = bf16lo_to_f32(qq[e]) * c1;
      qf[2 * e + 1] = bf16hi_to_f32(qq[e]) * c1;
    }
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;

  const uint16_t* kbase = kc + bh * (long long)L * d + sub * 8;
  const uint16_t* vbase = vc + bh * (long long)L * d + sub * 8;
  int n_iter = (jend - jbeg + G * U - 1) / (G * U);
  if (knorm != nullptr && c2 > 0.0f) {
    // |q| from the bf16 query (qf holds q c1), with the key bound and a
    // relative margin of 2^-8 against rounding
    float qn2 = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) qn2 = fmaf(qf[e], qf[e], qn2);
    const float A = sqrtf(group_sum<LPK>(qn2)) * knorm[bh] * (1.0f + 1.0f / 256.0f);
    const float reach = (2.0f * A + 152.0f) / c2;  // keys past a maximum's key that underflow
    const float d0 = float(L - jend);                // distance of the range's nearest key
    if (d0 > reach) {
      n_iter = 0;  // the whole range: weight zero in the combine
    } else if (reach < float(1 << 30)) {
      // iteration it starts at distance d0 + it G U: skip it once that is past
      // d0 + G - 1 + reach
      const int keep = int((float(G - 1) + reach) / float(G * U)) + 1;
      n_iter = min(n_iter, keep);
    }
  }
  for (int it = 0; it < n_iter; ++it) {
    u32x4 kr[U], vr[U];
    int jj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      jj[u] = jend - 1 - (it * G * U + u * G + g);
      kr[u] = u32x4{0u, 0u, 0u, 0u};
      vr[u] = u32x4{0u, 0u, 0u, 0u};
      if (jj[u] >= jbeg && dvalid) {
        kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (long long)jj[u] * d));
        vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + (long long)jj[u] * d));
      }
    }
    float t[U];
    float tmax = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = fmaf(qf[2 * e], bf16lo_to_f32(kr[u][e]), part);
        part = fmaf(qf[2 * e + 1], bf16hi_to_f32(kr[u][e]), part);
      }
      part = group_sum<LPK>(part);
      const float dist = float(L - 1 - jj[u]);
      t[u] = jj[u] >= jbeg ? fmaf(-c2, dist, part) : kNegInf;
      tmax = fmaxf(tmax, t[u]);
    }
    // Lazy rescale: move the running maximum only when it grows past 2^8.
    const bool need = tmax > m_run + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? tmax : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= alpha;
      m_run = m_new;
    }
    // A group that has seen no key yet keeps m_run = -inf; its t are -inf too
    // and must give p = 0, not exp2(-inf + inf).
    const float m_use = m_run == kNegInf ? 0.0f : m_run;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = fast_exp2(t[u] - m_use);
      l_run += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(p, bf16lo_to_f32(vr[u][e]), acc[2 * e]);
        acc[2 * e + 1] = fmaf(p, bf16hi_to_f32(vr[u][e]), acc[2 * e + 1]);
      }
    }
  }

  // Merge the G key groups of this workgroup.
  if (sub == 0) {
    sm_m[g] = m_run;
    sm_l[g] = l_run;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_acc[g][sub * 8 + e] = acc[e];
  __syncthreads();
  float mx = kNegInf;
  for (int gg = 0; gg < G; ++gg) mx = fmaxf(mx, sm_m[gg]);
  for (int dim = tid; dim < d; dim += kDecodeThreads) {
    float num = 0.0f, den = 0.0f;
    for (int gg = 0; gg < G; ++gg) {
      const float sc = sm_m[gg] == kNegInf ? 0.0f : fast_exp2(sm_m[gg] - mx);
      num = fmaf(sc, sm_acc[gg][dim], num);
      den = fmaf(sc, sm_l[gg], den);
    }
    if (splits == 1) {
      out[bh * d + dim] = f32_to_bf16(num / den);
    } else {
      float* p = ws + (bh * splits + s) * (long long)(d + 2);
      p[dim] = num;
      if (dim == 0) {
        p[d] = mx;
        p[d + 1] = den;
      }
    }
  }
}

// Merge the per-range partial states of one (b, h): M = max m_s,
// out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ ws, uint16_t* __restrict__ out, int d, int splits) {
  const long long bh = blockIdx.x;
  const float* p = ws + bh * splits * (long long)(d + 2);
  float mx = kNegInf;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, p[s * (d + 2) + d]);
  for (int dim = threadIdx.x; dim < d; dim += blockDim.x) {
    float num = 0.0f, den = 0.0f;
    for (int s = 0; s < splits; ++s) {
      const float* ps = p + s * (d + 2);
      const float sc = ps[d] == kNegInf ? 0.0f : fast_exp2(ps[d] - mx);
      num = fmaf(sc, ps[dim], num);
      den = fmaf(sc, ps[d + 1], den);
    }
    out[bh * d + dim] = f32_to_bf16(num / den);
  }
}

template <int LPK>
hipError_t launch_split(const void* q, const void* kc, const void* vc, void* out, float* ws,
                        int B, int H, int L, int d, int splits, int chunk, const float* slopes,
                        float c1, const float* knorm, hipStream_t stream) {
  const unsigned grid = unsigned((long long)B * H * splits);
  hipLaunchKernelGGL(decode_split_kernel<LPK>, dim3(grid), dim3(kDecodeThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)kc, (const uint16_t*)vc, (uint16_t*)out,
                     ws, H, L, d, splits, chunk, slopes, c1, knorm);
  return hipGetLastError();
}

}  // namespace

hipError_t decode_scratch(float** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    // this device's copy of the array, resolved once with the device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

void decode_plan(int B, int H, int L, int d, int* splits, int* chunk) {
  (void)d;
  // Aim for about 4096 workgroups (16 per CU on 256 CUs) so every CU has enough
  // loads in flight; never cut a range below 256 keys.
  const long long bh = (long long)B * H;
  long long s = (4096 + bh - 1) / bh;
  const long long max_s = (L + 255) / 256;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  long long c = (L + s - 1) / s;
  s = (L + c - 1) / c;  // every range non-empty
  *splits = int(s);
  *chunk = int(c);
}

hipError_t launch_decode(const void* q, const void* kc, const void* vc, void* out, float* ws,
                         int B, int H, int L, int d, int splits, int chunk,
                         const float* slopes, float c1, const float* knorm, hipStream_t stream) {
  hipError_t e;
  const int lpk = (d + 7) / 8;
  if (lpk <= 2) e = launch_split<2>(q, kc, vc, out, ws, B, H, L, d, splits, chunk, slopes, c1, knorm, stream);
  else if (lpk <= 4) e = launch_split<4>(q, kc, vc, out, ws, B, H, L, d, splits, chunk, slopes, c1, knorm, stream);
  else if (lpk <= 8) e = launch_split<8>(q, kc, vc, out, ws, B, H, L, d, splits, chunk, slopes, c1, knorm, stream);
  else if (lpk <= 16) e = launch_split<16>(q, kc, vc, out, ws, B, H, L, d, splits, chunk, slopes, c1, knorm, stream);
  else e = launch_split<32>(q, kc, vc, out, ws, B, H, L, d, splits, chunk, slopes, c1, knorm, stream);
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(unsigned((long long)B * H)), dim3(256), 0, stream,
                     (const float*)ws, (uint16_t*)out, d, splits);
  return hipGetLastError();
}

}  // namespace alibi
