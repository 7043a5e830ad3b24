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
// * A workgroup is NW waves (8 by default) and owns BM = 32 NW consecutive
//   query rows of one (b, h); each wave owns 32 rows. Two waves share each SIMD
//   (at most 256 registers per lane), so one wave's MFMA work overlaps the
//   other's softmax arithmetic.
// * Key/value tiles of BN = 64 rows are staged HBM -> registers -> LDS by the
//   whole workgroup: K row-major (16-byte coalesced loads, rows padded by 16 B
//   against bank conflicts), V transposed to V^T[d][key] (one key per lane,
//   16-bit LDS writes) so every wave reads its MFMA A operand with 16-byte LDS
//   reads. LDS is double-buffered: the loads of the next tile are in flight
//   while the current one is computed, with one barrier per tile.
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
//   There the bias costs one add (with a wave-uniform offset held in a scalar
//   register) and one fma per score.
// * The row sum is accumulated from the bf16-rounded p that the PV product
//   uses (v_dot2c_f32_bf16), so the normalisation matches the numerator.
// * Grid: one workgroup per (b, h, query block), heaviest causal blocks first
//   and blocks of one (b, h) kept on one XCD (workgroups are dealt to the 8
//   XCDs round-robin), so the K/V of a head is shared through that XCD's L2.
#include "device_common.h"
#include "launch.h"

#include <cstdlib>

namespace alibi {

namespace {

// Waves per workgroup: 8 by default; ALIBI_FWD_NW=4 selects 4 (tuning only).
int fwd_waves() {
  static const int nw = [] {
    const char* e = std::getenv("ALIBI_FWD_NW");
    return (e != nullptr && std::atoi(e) == 4) ? 4 : 8;
  }();
  return nw;
}
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

// One K/V tile of BN keys as the workgroup stages it: each thread holds
// K_LOADS 16-byte chunks of K (row-major, coalesced) and V_LOADS chunks of V
// (one key per lane, so the transposed LDS writes of a wave cover whole rows).
template <int D, int NT>
struct TileRegs {
  static constexpr int BN = 64;
  static constexpr int CPR = D / 8;
  static constexpr int LOADS = BN * CPR / NT;
  static_assert(LOADS * NT == BN * CPR, "tile must split evenly");
  u32x4 k[LOADS];
  u32x4 v[LOADS];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                                       long long base, int j0, int N, int tid) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int c = tid + NT * r;
      const int row = c / CPR, col = c % CPR;
      k[r] = u32x4{0u, 0u, 0u, 0u};
      if (j0 + row < N) k[r] = *reinterpret_cast<const u32x4*>(kg + base + (long long)(j0 + row) * D + col * 8);
      const int key = tid % BN;
      const int vcol = tid / BN + (NT / BN) * r;
      v[r] = u32x4{0u, 0u, 0u, 0u};
      if (j0 + key < N) v[r] = *reinterpret_cast<const u32x4*>(vg + base + (long long)(j0 + key) * D + vcol * 8);
    }
  }

  template <int KPITCH, int VPITCH>
  __device__ __forceinline__ void store(unsigned char* sK, unsigned char* sV, int tid) const {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int c = tid + NT * r;
      const int row = c / CPR, col = c % CPR;
      *reinterpret_cast<u32x4*>(sK + row * KPITCH + col * 16) = k[r];
      const int key = tid % BN;
      const int vcol = tid / BN + (NT / BN) * r;
      const int pos = (key & ~15) | perm16(key & 15);
      unsigned char* dst = sV + (vcol * 8) * VPITCH + pos * 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint16_t*>(dst + (2 * e) * VPITCH) = uint16_t(v[r][e] & 0xffffu);
        *reinterpret_cast<uint16_t*>(dst + (2 * e + 1) * VPITCH) = uint16_t(v[r][e] >> 16);
      }
    }
  }
};

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, int H, int N, int nqb, int total, const float* __restrict__ slopes,
    float c1) {
  constexpr int NT = NW * 64;
  constexpr int BN = 64;
  constexpr int BM = NW * 32;
  constexpr int KS = D / 16;       // MFMA k-steps of Q K^T
  constexpr int KB = BN / 32;      // 32-key blocks per tile
  constexpr int DB = D / 32;       // 32-wide d blocks of O
  constexpr int PS = BN / 16;      // MFMA k-steps of P V
  constexpr int KPITCH = D * 2 + 16;
  constexpr int VPITCH = BN * 2 + 16;
  constexpr int KBYTES = BN * KPITCH;
  constexpr int STAGE = KBYTES + D * VPITCH;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  // The wave index is uniform across the wave; say so, so that every per-wave
  // condition below compiles to a scalar branch instead of masked execution.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int qw0 = q0 + wave * 32;                      // first query of this wave
  const int qw_last = min(qw0 + 32, N) - 1;            // last valid query of this wave
  const int i = qw0 + l32;                             // this lane's query

  // Bias offsets m log2(e) (32 kb + 8 g + r) of the accumulator registers: wave-uniform,
  // kept in scalar registers.
  float cr[KB][16];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      cr[kb][r] = __int_as_float(__builtin_amdgcn_readfirstlane(
          __float_as_int(c2 * float(32 * kb + 8 * (r >> 2) + (r & 3)))));

  // Q^T fragments (MFMA B operand): lane holds query l32, d = 16 ks + 8 hi .. +7.
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (i < N) raw = *reinterpret_cast<const u32x4*>(q + base + (long long)i * D + 16 * ks + 8 * hi);
    qf[ks] = __builtin_bit_cast(bf16x8, raw);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;

  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;

  TileRegs<D, NT> regs;
  regs.load(k, v, base, (ntiles - 1) * BN, N, tid);
  regs.template store<KPITCH, VPITCH>(smem, smem + KBYTES, tid);

  int stage = 0;
  for (int tile = ntiles - 1; tile >= 0; --tile, stage ^= 1) {
    const int j0 = tile * BN;
    // Stage `stage` holds this tile; every wave is done with the other stage.
    __syncthreads();
    if (tile > 0) regs.load(k, v, base, j0 - BN, N, tid);  // in flight during the compute
    const unsigned char* sK = smem + stage * STAGE;
    const unsigned char* sV = sK + KBYTES;

    const bool active = qw0 < N && (!CAUSAL || j0 <= qw_last);
    if (active) {
      // ---- S^T = K Q^T ----
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (32 * kb + l32) * KPITCH + (16 * ks + 8 * hi) * 2);
          s[kb] = mfma32(a, qf[ks], s[kb]);
        }
      }

      // ---- bias, mask, online softmax ----
      const bool fast = CAUSAL && (j0 + BN - 1 <= qw0) && (j0 + BN <= N);
      float mcand;
      if (fast) {
        float smax = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) smax = fmaxf(smax, s[kb][r]);
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
            const float t = fmaf(s[kb][r], c1, -c2 * fabsf(dist));
            s[kb][r] = valid ? t : kNegInf;  // now holds t (log2 units)
            tmax = fmaxf(tmax, s[kb][r]);
          }
        }
        mcand = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      }
      const bool need = mcand > m_run + kLazy;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mcand : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == kNegInf ? 0.0f : m_run;
      u32x4 pf[PS];
      float lsum = l_run;
      if (fast) {
        const float bt = fmaf(c2, float(j0 + 4 * hi - i), -m_use);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r0 = 8 * half + 2 * e;
              const float p0 = fast_exp2(fmaf(s[kb][r0], c1, bt + cr[kb][r0]));
              const float p1 = fast_exp2(fmaf(s[kb][r0 + 1], c1, bt + cr[kb][r0 + 1]));
              pk[e] = pack_bf16x2(p0, p1);
              lsum = bdot2(pk[e], lsum);
            }
            pf[2 * kb + half] = pk;
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r0 = 8 * half + 2 * e;
              pk[e] = pack_bf16x2(fast_exp2(s[kb][r0] - m_use), fast_exp2(s[kb][r0 + 1] - m_use));
              lsum = bdot2(pk[e], lsum);
            }
            pf[2 * kb + half] = pk;
          }
        }
      }
      l_run = lsum;

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int ps = 0; ps < PS; ++ps) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sV + (32 * db + l32) * VPITCH + (16 * ps + 8 * hi) * 2);
          o[db] = mfma32(a, __builtin_bit_cast(bf16x8, pf[ps]), o[db]);
        }
      }
    }
    if (tile > 0) regs.template store<KPITCH, VPITCH>(smem + (stage ^ 1) * STAGE, smem + (stage ^ 1) * STAGE + KBYTES, tid);
  }

  // ---- epilogue: O / l -> bf16 ----
  const float lt = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / lt;
  if (i < N) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 st;
        st[0] = pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
        st[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(out + base + (long long)i * D + 32 * db + 8 * g + 4 * hi) = st;
      }
    }
  }
}

template <int D, int NW, bool CAUSAL>
hipError_t launch_cfg(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                      const float* slopes, float c1, hipStream_t stream) {
  constexpr int BM = NW * 32;
  const int nqb = (N + BM - 1) / BM;
  const long long total = (long long)B * H * nqb;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, NW, CAUSAL>), dim3(unsigned(total)), dim3(NW * 64), 0,
                     stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     (uint16_t*)out, H, N, nqb, int(total), slopes, c1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, void* out,
                           int B, int H, int N, int d, const float* slopes, int causal,
                           float c1, hipStream_t stream) {
  if (fwd_waves() == 4) {
    if (d == 128)
      return causal ? launch_cfg<128, 4, true>(q, k, v, out, B, H, N, slopes, c1, stream)
                    : launch_cfg<128, 4, false>(q, k, v, out, B, H, N, slopes, c1, stream);
    return causal ? launch_cfg<64, 4, true>(q, k, v, out, B, H, N, slopes, c1, stream)
                  : launch_cfg<64, 4, false>(q, k, v, out, B, H, N, slopes, c1, stream);
  }
  if (d == 128)
    return causal ? launch_cfg<128, 8, true>(q, k, v, out, B, H, N, slopes, c1, stream)
                  : launch_cfg<128, 8, false>(q, k, v, out, B, H, N, slopes, c1, stream);
  return causal ? launch_cfg<64, 8, true>(q, k, v, out, B, H, N, slopes, c1, stream)
                : launch_cfg<64, 8, false>(q, k, v, out, B, H, N, slopes, c1, stream);
}

}  // namespace alibi
