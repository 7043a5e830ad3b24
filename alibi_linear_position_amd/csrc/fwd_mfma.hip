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
// * A workgroup is NW waves (4 by default) and owns BM = 32 NW consecutive
//   query rows of one (b, h); each wave owns 32 rows. Two waves share each SIMD
//   (at most 256 registers per lane; two 4-wave workgroups per CU), so one
//   wave's MFMA work can overlap the other's softmax arithmetic.
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
//   The first Q K^T k-step takes a constant register set as its C operand,
//   which seeds each score with its register's bias offset, so there the bias
//   costs one fma per score. Row reductions across the two lane halves use
//   v_permlane32_swap; row sums use four independent accumulators.
// * The row sum is accumulated from the bf16-rounded p that the PV product
//   uses (v_dot2c_f32_bf16), so the normalisation matches the numerator.
// * Grid: one workgroup per (b, h, query block), heaviest causal blocks first
//   and blocks of one (b, h) kept on one XCD (workgroups are dealt to the 8
//   XCDs round-robin), so the K/V of a head is shared through that XCD's L2.
#include "device_common.h"
#include "launch.h"

#include <cstdlib>
#include <type_traits>

namespace alibi {

namespace {

// Waves per workgroup: 4 by default (two workgroups share a CU);
// ALIBI_FWD_NW=8 selects one 8-wave workgroup per CU (tuning only).
int fwd_waves() {
  static const int nw = [] {
    const char* e = std::getenv("ALIBI_FWD_NW");
    return (e != nullptr && std::atoi(e) == 8) ? 8 : 4;
  }();
  return nw;
}
constexpr float kLazy = 8.0f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of key x (0..15) inside a 16-key group of V^T: swaps keys 4-7 with 8-11.
__device__ __forceinline__ int perm16(int x) { return ((x & 4) << 1) | ((x & 8) >> 1) | (x & 3); }

// Row reductions across the two lane halves (lane l and l ^ 32 hold the same
// query): v_permlane32_swap exchanges the halves in one VALU op.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum of 16 accumulator values as a shallow tree of 3-input maxima.
__device__ __forceinline__ float max16(const f32x16& a) {
  const float m0 = fmaxf(fmaxf(a[0], a[1]), a[2]);
  const float m1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
  const float m2 = fmaxf(fmaxf(a[6], a[7]), a[8]);
  const float m3 = fmaxf(fmaxf(a[9], a[10]), a[11]);
  const float m4 = fmaxf(fmaxf(a[12], a[13]), a[14]);
  return fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), a[15]));
}

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

  // A tile that lies entirely below N: no guards and no zero fill. Chunk r of
  // K sits at element (tid + NT r) * 8 of the tile (rows are contiguous), chunk
  // r of V at key * D + (tid / BN + (NT / BN) r) * 8: one per-thread offset
  // plus a constant per chunk.
  __device__ __forceinline__ void load_full(const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vt,
                                            int tid) {
    const uint32_t koff = uint32_t(tid) * 8u;
    const uint32_t voff = uint32_t(tid % BN) * D + uint32_t(tid / BN) * 8u;
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      k[r] = *reinterpret_cast<const u32x4*>(kt + koff + uint32_t(NT * 8 * r));
      v[r] = *reinterpret_cast<const u32x4*>(vt + voff + uint32_t((NT / BN) * 8 * r));
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

  // C operand of the first Q K^T k-step: seeds register r of a 32-key block
  // with its bias offset m log2(e) (8 (r / 4) + r % 4) / c1, so off-diagonal
  // tiles need one fma per score to complete the bias.
  f32x16 cinit;
  const float c21 = c2 / c1;
#pragma unroll
  for (int r = 0; r < 16; ++r) cinit[r] = c21 * float(8 * (r >> 2) + (r & 3));

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

  // One tile: S^T = K Q^T, online softmax, O^T += V^T P^T, and the LDS stores
  // of the next tile (whose global loads were issued at the top). MASKED tiles
  // may hold keys past a query or past N; the others hold none for any wave.
  int stage = 0;
  auto step = [&](int tile, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int j0 = tile * BN;
    // Stage `stage` holds this tile; every wave is done with the other stage.
    __syncthreads();
    // Only the first tile visited can be ragged, and the prologue staged it.
    if (tile > 0) regs.load_full(k + base + (long long)(j0 - BN) * D, v + base + (long long)(j0 - BN) * D, tid);
    const unsigned char* sK = smem + stage * STAGE;
    const unsigned char* sV = sK + KBYTES;
    unsigned char* const sKn = smem + (stage ^ 1) * STAGE;
    stage ^= 1;
    if (MASKED && !(qw0 < N && (!CAUSAL || j0 <= qw_last))) {
      regs.template store<KPITCH, VPITCH>(sKn, sKn + KBYTES, tid);
      return;
    }

    // ---- S^T = K Q^T ----
    f32x16 s[KB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (32 * kb + l32) * KPITCH + (16 * ks + 8 * hi) * 2);
        s[kb] = mfma32(a, qf[ks], ks == 0 ? cinit : s[kb]);
      }
    }

    // ---- bias, mask, online softmax ----
    // s = q.k + (c2 / c1)(8 (r / 4) + r % 4); the full exponent is
    // t = s c1 + c2 (j0 + 32 kb + 4 hi - i).
    const float bt0 = c2 * float(j0 + 4 * hi - i);
    const float bt1 = bt0 + 32.0f * c2;
    float mcand;
    if (!MASKED) {
      // every key is visible: max16 of s bounds the row maximum
      mcand = max_xor32(fmaxf(fmaf(max16(s[0]), c1, bt0), fmaf(max16(s[1]), c1, bt1)));
    } else {
      // masked keys become -inf in s itself, so the exponent code is shared
      float tmax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool valid = j < N && (!CAUSAL || j <= i);
          float x = s[kb][r];
          if (!CAUSAL && j > i) x -= 2.0f * c21 * float(j - i);  // symmetric bias -m |i - j|
          s[kb][r] = valid ? x : kNegInf;
          tmax = fmaxf(tmax, fmaf(s[kb][r], c1, kb ? bt1 : bt0));
        }
      }
      mcand = max_xor32(tmax);
    }
    // Lazy rescale: the running maximum moves only when a row's candidate
    // exceeds it by more than 2^kLazy, so p stays below 2^kLazy.
    const bool need = mcand > m_run + kLazy;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mcand : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    // m_run is finite after the first visible key; a row with none yet
    // (every key masked) keeps -inf and takes 0 here
    const float m_use = MASKED && m_run == kNegInf ? 0.0f : m_run;
    u32x4 pf[PS];
    float lpart[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // independent partial row sums
    const float b0 = bt0 - m_use, b1 = bt1 - m_use;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r0 = 8 * half + 2 * e;
          const float bb = kb ? b1 : b0;
          pk[e] = pack_bf16x2(fast_exp2(fmaf(s[kb][r0], c1, bb)), fast_exp2(fmaf(s[kb][r0 + 1], c1, bb)));
          lpart[e] = bdot2(pk[e], lpart[e]);
        }
        pf[2 * kb + half] = pk;
      }
    }
    l_run += (lpart[0] + lpart[1]) + (lpart[2] + lpart[3]);

    // ---- O^T += V^T P^T, with the next tile's LDS stores in the same region ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sV + (32 * db + l32) * VPITCH + (16 * ps + 8 * hi) * 2);
        o[db] = mfma32(a, __builtin_bit_cast(bf16x8, pf[ps]), o[db]);
      }
    }
    // After the last tile the registers still hold tile 0, which nobody reads
    // again; storing it keeps this region free of branches.
    regs.template store<KPITCH, VPITCH>(sKn, sKn + KBYTES, tid);
  };

  // Tiles 0 .. t_open lie wholly below the workgroup's first query q0 (so below
  // every wave's queries, and below N): no mask. The rest, at most
  // (BM + BN - 1) / BN of them under the causal mask, take the masked path.
  const int t_open = CAUSAL ? (q0 + 1) / BN - 1 : -1;
  int tile = ntiles - 1;
  for (; tile > t_open; --tile) step(tile, std::true_type{});
  for (; tile >= 0; --tile) step(tile, std::false_type{});

  // ---- epilogue: O / l -> bf16 ----
  const float lt = sum_xor32(l_run);
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
