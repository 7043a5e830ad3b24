// Fused causal ALiBi attention forward on gfx950 bf16 MFMA (d = 64 or 128).
//
// Per (b, h) and query i the kernel computes (Eq. 1-3 of "When Attention Goes
// Blind: Numerical Failure in ALiBi Positional Encodings"):
//   t_ij = q_i . k_j / sqrt(d) - m_h (i - j)  for j <= i,  -inf for j > i,
//   out_i = softmax_j(t_i.) V,
// or, with causal = 0, the symmetric bias -m_h |i - j| and no mask
// ("ALiBi and Relative Position Bias", quantmemo.com). The bias and the mask are
// generated in registers per tile; the (H, N, N) bias is never stored
// (abhik.ai, remark after the full-sequence example).
//
// Layout of the work
// ------------------
// * A workgroup is 4 waves and owns BM = 4 * 32 * QB consecutive query rows of
//   one (b, h); each wave owns 32 * QB rows.
// * Key/value tiles of BN = 64 rows are staged HBM -> LDS by the whole
//   workgroup: K row-major (16-byte coalesced loads, padded rows against bank
//   conflicts), V transposed to V^T[d][key] so it can feed the MFMA A operand.
// * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (M = 32 keys, N = 32 queries,
//   K = 16 of d). In the 32x32 accumulator layout lane l holds one query
//   (l % 32) and 16 of the 32 keys, so the row softmax is almost entirely
//   in-lane; one swap with lane l ^ 32 completes a row.
// * O^T += V^T P^T on the same MFMA (M = 32 of d, N = 32 queries, K = 16 keys).
//   P^T is the B operand straight from the softmax registers after packing to
//   bf16. The key order inside each 16-key step follows the accumulator layout
//   (keys 0-3, 8-11 in lanes 0-31; 4-7, 12-15 in lanes 32-63), and V^T is
//   written to LDS in that same permuted order, so the contraction pairs each
//   p with its own v row.
// * Softmax in log2 units, fp32, one online pass. Tiles are visited from the
//   diagonal backwards: the diagonal tile fixes a running maximum close to the
//   true one, older tiles carry a smaller bias, and the accumulator is rescaled
//   only when the maximum grows by more than 2^8 (lazy rescale; exact up to
//   fp32 rounding because numerator and denominator share the scale).
//   Off-diagonal tiles use a cheap upper bound of the row maximum
//   (max_j s_ij * c1 plus the largest bias in the tile) instead of the exact
//   maximum; any bound works for the algebra and this one keeps p <= 2^8.
// * The row sum is accumulated from the bf16-rounded p that the PV product
//   uses (v_dot2c_f32_bf16), so the normalisation matches the numerator.
// * Grid: one workgroup per (b, h, query block), heaviest causal blocks first
//   and blocks of one (b, h) kept on one XCD (workgroups are dealt to the 8
//   XCDs round-robin), so the K/V of a head is shared through that XCD's L2.
#include "device_common.h"
#include "launch.h"

namespace alibi {

namespace {

constexpr int kThreads = 256;
constexpr float kLazy = 8.0f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of key x (0..15) inside a 16-key group of V^T: swaps keys 4-7 with 8-11.
__device__ __forceinline__ int perm16(int x) { return ((x & 4) << 1) | ((x & 8) >> 1) | (x & 3); }

__device__ __forceinline__ float bdot2(uint32_t packed, float acc) {
  const bf16x2 a = __builtin_bit_cast(bf16x2, packed);
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  return __builtin_amdgcn_fdot2_f32_bf16(a, one, acc, false);
}

template <int D, int BN, int QB, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, int H, int N, int nqb, int total, const float* __restrict__ slopes,
    float c1) {
  constexpr int BM = 4 * 32 * QB;
  constexpr int KS = D / 16;       // MFMA k-steps of Q K^T
  constexpr int KB = BN / 32;      // 32-key blocks per tile
  constexpr int DB = D / 32;       // 32-wide d blocks of O
  constexpr int PS = BN / 16;      // MFMA k-steps of P V
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int KPITCH = D * 2 + 16;
  constexpr int VPITCH = BN * 2 + 16;
  constexpr int KBYTES = BN * KPITCH;
  constexpr int K_LOADS = BN * CPR / kThreads;
  constexpr int V_LOADS = BN * CPR / kThreads;
  static_assert(K_LOADS * kThreads == BN * CPR, "tile must split evenly");
  __shared__ __attribute__((aligned(16))) unsigned char smem[KBYTES + D * VPITCH];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Workgroup -> (b, h, query block): XCD-grouped, heaviest block first.
  const int w = blockIdx.x;
  const int lw = (total & 7) == 0 ? (w & 7) * (total >> 3) + (w >> 3) : w;
  const int bh = lw / nqb;
  const int qblk = nqb - 1 - (lw - bh * nqb);
  const int h = bh % H;
  const float c2 = slopes[h] * kLog2e;
  const long long base = (long long)bh * N * D;
  const int q0 = qblk * BM;
  const int qw0 = q0 + wave * 32 * QB;                 // first query of this wave
  const int qw_last = min(qw0 + 32 * QB, N) - 1;       // last valid query of this wave

  // Q^T fragments (MFMA B operand): lane holds query l32, d = 16 ks + 8 hi .. +7.
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int i = qw0 + 32 * qb + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (i < N) raw = *reinterpret_cast<const u32x4*>(q + base + (long long)i * D + 16 * ks + 8 * hi);
      qf[qb][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 o[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x16{};
    m_run[qb] = kNegInf;
    l_run[qb] = 0.0f;
  }

  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  unsigned char* sK = smem;
  unsigned char* sV = smem + KBYTES;

  for (int tile = ntiles - 1; tile >= 0; --tile) {
    const int j0 = tile * BN;
    __syncthreads();  // every wave is done with the previous tile
    // ---- stage K (row-major) ----
#pragma unroll
    for (int r = 0; r < K_LOADS; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / CPR, col = c % CPR;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (j0 + row < N) raw = *reinterpret_cast<const u32x4*>(k + base + (long long)(j0 + row) * D + col * 8);
      *reinterpret_cast<u32x4*>(sK + row * KPITCH + col * 16) = raw;
    }
    // ---- stage V transposed: V^T[d][perm(key)] ----
#pragma unroll
    for (int r = 0; r < V_LOADS; ++r) {
      const int key = tid % BN;
      const int col = tid / BN + (kThreads / BN) * r;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (j0 + key < N) raw = *reinterpret_cast<const u32x4*>(v + base + (long long)(j0 + key) * D + col * 8);
      const int pos = (key & ~15) | perm16(key & 15);
      unsigned char* dst = sV + (col * 8) * VPITCH + pos * 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint16_t*>(dst + (2 * e) * VPITCH) = uint16_t(raw[e] & 0xffffu);
        *reinterpret_cast<uint16_t*>(dst + (2 * e + 1) * VPITCH) = uint16_t(raw[e] >> 16);
      }
    }
    __syncthreads();

    const bool active = qw0 < N && (!CAUSAL || j0 <= qw_last);
    if (!active) continue;

    // ---- S^T = K Q^T ----
    f32x16 s[QB][KB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (32 * kb + l32) * KPITCH + (16 * ks + 8 * hi) * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(a, qf[qb][ks], s[qb][kb]);
      }
    }

    // ---- bias, mask, online softmax ----
    const bool fast = CAUSAL && (j0 + BN - 1 <= qw0) && (j0 + BN <= N);
    u32x4 pf[QB][PS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int i = qw0 + 32 * qb + l32;
      float mcand;
      if (fast) {
        float smax = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) smax = fmaxf(smax, s[qb][kb][r]);
        smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
        mcand = fmaf(smax, c1, c2 * float(j0 + BN - 1 - i));
      } else {
        float tmax = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool valid = j < N && (!CAUSAL || j <= i);
            const float dist = float(i - j);
            const float t = fmaf(s[qb][kb][r], c1, -c2 * fabsf(dist));
            s[qb][kb][r] = valid ? t : kNegInf;  // now holds t (log2 units)
            tmax = fmaxf(tmax, s[qb][kb][r]);
          }
        }
        mcand = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      }
      const bool need = mcand > m_run[qb] + kLazy;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mcand : m_run[qb];
        const float alpha = need ? fast_exp2(m_run[qb] - m_new) : 1.0f;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
        m_run[qb] = m_new;
      }
      const float m_use = m_run[qb] == kNegInf ? 0.0f : m_run[qb];
      float p[KB][16];
      if (fast) {
        const float bt = fmaf(c2, float(j0 + 4 * hi - i), -m_use);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float cr = c2 * float(32 * kb + 8 * (r >> 2) + (r & 3));
            p[kb][r] = fast_exp2(fmaf(s[qb][kb][r], c1, bt + cr));
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) p[kb][r] = fast_exp2(s[qb][kb][r] - m_use);
      }
      float lsum = l_run[qb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pk[e] = pack_bf16x2(p[kb][8 * half + 2 * e], p[kb][8 * half + 2 * e + 1]);
            lsum = bdot2(pk[e], lsum);
          }
          pf[qb][2 * kb + half] = pk;
        }
      }
      l_run[qb] = lsum;
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sV + (32 * db + l32) * VPITCH + (16 * ps + 8 * hi) * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = mfma32(a, __builtin_bit_cast(bf16x8, pf[qb][ps]), o[qb][db]);
      }
    }
  }

  // ---- epilogue: O / l -> bf16 ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int i = qw0 + 32 * qb + l32;
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    const float inv = 1.0f / lt;
    if (i < N) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 st;
          st[0] = pack_bf16x2(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv);
          st[1] = pack_bf16x2(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(out + base + (long long)i * D + 32 * db + 8 * g + 4 * hi) = st;
        }
      }
    }
  }
}

template <int D, int QB, bool CAUSAL>
hipError_t launch_cfg(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                      const float* slopes, float c1, hipStream_t stream) {
  constexpr int BM = 4 * 32 * QB;
  const int nqb = (N + BM - 1) / BM;
  const long long total = (long long)B * H * nqb;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, 64, QB, CAUSAL>), dim3(unsigned(total)), dim3(kThreads), 0,
                     stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     (uint16_t*)out, H, N, nqb, int(total), slopes, c1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, void* out,
                           int B, int H, int N, int d, const float* slopes, int causal,
                           float c1, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch_cfg<128, 1, true>(q, k, v, out, B, H, N, slopes, c1, stream)
                  : launch_cfg<128, 1, false>(q, k, v, out, B, H, N, slopes, c1, stream);
  }
  return causal ? launch_cfg<64, 1, true>(q, k, v, out, B, H, N, slopes, c1, stream)
                : launch_cfg<64, 1, false>(q, k, v, out, B, H, N, slopes, c1, stream);
}

}  // namespace alibi
