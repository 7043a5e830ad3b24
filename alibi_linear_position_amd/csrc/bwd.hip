// Backward pass of ALiBi attention on gfx950 bf16 MFMA (d = 64 or 128).
//
// Gradients of out = softmax(Q K^T / sqrt(d) - m (i - j), causal mask) V with
// respect to q, k and v (the bias is a constant: ALiBi slopes are fixed, not
// learned -- abhik.ai, "Different heads, different distance penalties"). With
// P_ij = exp(S_ij - lse_i) recomputed from the forward's row log-sum-exp:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_d dO_i O_i,
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
// "When Attention Goes Blind" (Sec. 4.2, 5.1) trains ALiBi models and argues
// that the underflowed weights matter most in exactly this pass.
//
// Three kernels:
// * bwd_prep_kernel: D_i and the log-sum-exp in log2 units, one lane group
//   per row.
// * bwd_dkdv_kernel: one workgroup per 128 keys of one (b, h), eight waves:
//   four own dV and four own dK of 32 keys each, keeping their keys' K (or V)
//   rows as MFMA B operands in registers. Query tiles of 64 rows (or 32)
//   stream through a three-stage LDS ring: read straight for S = Q K^T and
//   dP = dO V^T (rows = queries, lane = key), and read transposed
//   (ds_read_b64_tr_b16) for dV^T += dO^T P and dK^T += Q^T dS, so P and dS go
//   from registers to the next MFMA as B operands. The dV waves compute P once
//   and hand it to the dK waves through LDS (fp16 with 64-row tiles, fp32 with
//   32-row ones); the dK waves run one query tile behind, so both roles work
//   at the same time between barriers.
// * bwd_dq_kernel: one workgroup per 128 queries, the forward's layout:
//   S^T = K Q^T and dP^T = V dO^T (lane = query, so lse and D are one value
//   per lane), dS^T packed to bf16 and dQ^T += K^T dS^T, with K^T read
//   transposed from the row-major K tile; K and V staged per 32-key tile
//   (64-key tiles need more registers than two waves per SIMD leave).
// Scores are in log2 units (c1 = log2(e) / sqrt(d), c2 = m log2(e)); masked and
// out-of-range entries get P = 0.
//
// VAR (bits 1: clamp, 2: log distance, 4: soft cap) recomputes P with the
// logits of those Sec. 3.4 mitigations: B = max(-m D*, c), D* = D or
// ln(D + 1), change only the constant bias, so the rest of the chain rule is
// the same; the soft cap A* = z tanh(A / z) of the content logit adds the
// factor dA*/dA = 1 - tanh(A / z)^2 to dS before dQ and dK (the dV waves hand
// P (1 - tanh^2) to the dK waves, and the dQ kernel scales its dS). The
// scores are then not seeded and the logit is formed per score.
//
// With the per-(b, h) norm maxima of Q and K (plain form, causal or not),
// both kernels end their walks, and each wave skips its own tiles, at the distance
// past which every P is an exact zero (live_reach below): the gradients keep
// every bit.
#include "device_common.h"
#include "launch.h"

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <type_traits>

namespace alibi {

namespace {

constexpr int kBwdClamp = 1, kBwdLog = 2, kBwdCap = 4;

// Bias of distance D >= 0 in log2 units for the VAR forms.
template <int VAR>
__device__ __forceinline__ float var_bias(float dd, float c2, float mh, float clamp2) {
  float b;
  if constexpr ((VAR & kBwdLog) != 0) {
    b = -mh * __builtin_amdgcn_logf(dd + 1.0f);  // -m ln(D + 1) log2(e) = -m log2(D + 1)
  } else {
    b = -c2 * dd;
  }
  if constexpr ((VAR & kBwdClamp) != 0) b = fmaxf(b, clamp2);
  return b;
}

// Soft-capped content logit in log2 units from the raw score s = q.k:
// z log2(e) tanh(A / z) = cap_out (1 - 2 / (e^(2 A / z) + 1)) with
// e^(2 A / z) = exp2(s cap_in); th = tanh(A / z), for dA*/dA = 1 - th^2.
__device__ __forceinline__ float cap_logit(float s, float cap_in, float cap_out, float& th) {
  th = fmaf(-2.0f, __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(s * cap_in) + 1.0f), 1.0f);
  return cap_out * th;
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family parts:
// 32-bit data format, byte-granular range check against the record count.
constexpr int kBufferFlags = 0x00020000;

// Buffer resource over `rows` rows of D bf16 (capped at 2^32 - 1 bytes, which
// no valid 16-byte chunk reaches): loads at or past the end read as zero. The
// range check covers the vector offset, so tile offsets go there.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* p, long long rows) {
  const uint32_t bytes = uint32_t(min(rows * D * 2, 0xffffffffLL));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, int(bytes), kBufferFlags);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Row-major bf16 tile in LDS, D / 8 16-byte chunks per row and no padding:
// chunk c of row r sits at chunk position c ^ x(r). The XOR pattern (a
// function of r % 16) keeps both read patterns of the backward kernels free of
// LDS bank conflicts (64 banks of 4 bytes): 16 consecutive rows read at one
// chunk with 16-byte reads, and 4 consecutive rows x 4 chunks per 32 lanes
// with ds_read_b64_tr_b16. (Row padding cannot serve both: the 16-byte row
// reads need a row stride of 4 banks times an odd number, the transposed reads
// a multiple of 16 banks.)
template <int D>
struct SwzTile {
  static constexpr int ROWB = 2 * D;
  static __host__ __device__ constexpr int x(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  // byte offset of chunk c of row r
  static __device__ __forceinline__ int off(int r, int c) { return r * ROWB + ((c ^ x(r)) << 4); }
  // 16-byte row reads: lane l reads row r0 + l % 32 (r0 a multiple of 16),
  // chunk 2 ks + l / 32, at r0 ROWB + (row_base(l) ^ 32 ks).
  static __device__ __forceinline__ int row_base(int lane) {
    const int r = lane & 31, hi = lane >> 5;
    return r * ROWB | ((hi ^ x(r)) << 4);
  }
  // Transposed reads (read_tr below): the two per-lane bases, for tile rows
  // +{0..3} (+4 for lanes >= 32) and +{8..11} (+4).
  static __device__ __forceinline__ int tr_base(int lane, int second) {
    const int j = lane & 15, g = (lane >> 4) & 1, hi = lane >> 5;
    const int r = 4 * hi + (j >> 2) + 8 * second;
    return r * ROWB | ((((2 * g) | ((j & 3) >> 1)) ^ x(r)) << 4) | (8 * (j & 1));
  }
};

// MFMA A operand (rows = 32 d values, k = 16 rows of a swizzled row-major LDS
// tile) read transposed with ds_read_b64_tr_b16: within each 16-lane group,
// lanes 4e .. 4e + 3 point at 8-byte pieces of tile row e and lane j receives
// column j of those 4 rows. Lane l gets d = dcol + l % 32 (dcol a multiple of
// 32) and tile rows r16 + {0..3, 8..11} (l < 32) or r16 + {4..7, 12..15}
// (l >= 32), r16 a multiple of 16: the row order of the 32x32 accumulator
// layout, so an accumulator used as the B operand pairs each of its rows with
// the matching tile row. tb0, tb1: SwzTile<D>::tr_base(lane, 0 / 1).
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const unsigned char* tile, int tb0, int tb1, int r16, int dcol) {
  const int m = (dcol >> 5) << 6;  // chunk 4 (dcol / 32): XOR 64 (dcol / 32) on the byte offset
  const unsigned char* t = tile + r16 * SwzTile<D>::ROWB;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (tb0 ^ m)));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (tb1 ^ m)));
  const short v8 __attribute__((ext_vector_type(8))) = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v8);
}

// Pack 8 fp32 values (registers base .. base + 7 of an accumulator) to bf16.
__device__ __forceinline__ u32x4 pack8(const f32x16& x, int base) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(x[base + 2 * e], x[base + 2 * e + 1]);
  return r;
}

// Exact underflow skipping of the plain form. With M_q and M_k the
// largest query and key norms of a (b, h) pair and A = c1 M_q M_k, every
// logit (log2 units) is at most A - c2 D at distance D = i - j
// (Cauchy-Schwarz on the content term) and every row's log-sum-exp is at
// least its diagonal logit, so at least -A. P = exp2(logit - lse2) is then
// below 2^(2A - c2 D), which rounds to an exact zero once c2 D > 2A + 152
// (a margin of 2 over the 2^-150 rounding limit of fp32, and 2^-8 relative on
// A, for the rounding of the products, of lse and of the bias). Zero P give
// zero dV terms and zero dS, hence zero dK and dQ terms: a tile whose every
// distance lies past that point adds exact zeros and is not visited.
// norms: P partial maxima of the key norms of every pair, then those of the
// query norms (nbh pairs each). Returns the largest distance that can still
// carry a nonzero P, or 2^30 (nothing skipped).
__device__ __forceinline__ int live_reach(const float* __restrict__ norms, int parts, int nbh, int bh, float c1,
                                          float c2) {
  if (norms == nullptr || !(c2 > 0.0f)) return 1 << 30;
  float km = 0.0f, qm = 0.0f;
  for (int p = 0; p < parts; ++p) {
    km = fmaxf(km, norms[(long long)bh * parts + p]);
    qm = fmaxf(qm, norms[((long long)nbh + bh) * parts + p]);
  }
  const float A = c1 * qm * km * (1.0f + 1.0f / 256.0f);
  const float reach = (2.0f * A + 152.0f) / c2;  // dead: D > reach
  return reach < 1.0e9f ? int(ceilf(reach)) : (1 << 30);
}

// ---------------------------------------------------------------- prep ------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ dsum, float* __restrict__ lse2,
                                                       long long rows) {
  constexpr int LPR = D / 8;
  const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float s = 0.0f;
  if (row < rows) {
    const u32x4 a = load16(o + row * D + sub * 8), b = load16(dout + row * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(bf16lo_to_f32(a[e]), bf16lo_to_f32(b[e]), s);
      s = fmaf(bf16hi_to_f32(a[e]), bf16hi_to_f32(b[e]), s);
    }
  }
  s = group_sum<LPR>(s);
  if (row < rows && sub == 0) {
    dsum[row] = s;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------- dK, dV ----
// Eight waves: waves 0-3 own dV and waves 4-7 own dK of the same 4 x 32 keys
// (waves w and w + 4 share a SIMD). In step t a dV wave computes S and P of
// query tile t, writes P to LDS and accumulates dV^T += dO^T P; the dK wave of
// the same keys computes dP of tile t - 1, reads that tile's P, forms
// dS = P (dP - D) and accumulates dK^T += Q^T dS. Each wave holds one
// accumulator set and one set of key rows, so two waves fit on every SIMD, and
// the two roles' MFMA and VALU work overlap within a step instead of waiting
// for each other.
//
// A query tile is QB blocks of 32 rows. With QB = 2 a step does twice the
// work per barrier and per staging round, and P goes to the dK waves as fp16
// (P <= 1; relative error 2^-11, against 2^-8 for bf16, whose hand-off
// misses the gradient bar) so that the 64-row stages and the P buffers fit in
// LDS together; with QB = 1 the hand-off is the fp32 P.
template <int D, bool CAUSAL, int VAR, int QB = 1, bool PH = (QB == 2)>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ dsum,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int H, int N, int nkb, int total,
    const float* __restrict__ slopes, float c1, float scale, float clamp2, float cap_in, float cap_out,
    const float* __restrict__ norms, int parts) {
  static_assert(QB == 1 || QB == 2, "one or two 32-row query blocks per tile");
  constexpr bool CAP = (VAR & kBwdCap) != 0;
  constexpr int NT = 512, BK = 128, BQ = 32 * QB;
  constexpr int KS = D / 16, DB = D / 32, CPR = D / 8;
  using Tile = SwzTile<D>;             // Q / dO tiles: swizzled rows of 2 D bytes
  constexpr int RBYTES = BQ * Tile::ROWB;
  constexpr int STAGE = 2 * RBYTES + 2 * BQ * 4;
  constexpr int CHUNKS = BQ * CPR;    // 16-byte chunks of Q (and of dO) per tile
  constexpr int NCH = (CHUNKS + NT - 1) / NT;  // per thread
  static_assert(CHUNKS <= NT || CHUNKS % NT == 0, "chunks split evenly over the threads");
  __shared__ __attribute__((aligned(16))) unsigned char smem[3 * STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave >> 2;  // 0: dV, 1: dK
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const WgBlock wb = schedule_block(blockIdx.x, total / nkb, nkb);
  const int bh = wb.bh;
  const int kblk = wb.rank;  // low key blocks see the most queries: scheduled first
  const int h = bh % H;
  const float mh = slopes[h];
  const float c2 = mh * kLog2e;
  const float c21 = c2 / c1;
  const long long base = (long long)bh * N * D;
  const long long rbase = (long long)bh * N;
  const int k0 = kblk * BK;
  const int kw0 = k0 + (wave & 3) * 32;
  const int j = kw0 + l32;  // this lane's key

  // S rows are queries 8 (r / 4) + 4 hi + r % 4 of a 32-row block; seeding
  // register r with -c2 / c1 (8 (r / 4) + r % 4) leaves one fma for the bias.
  f32x16 cinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) cinit[r] = VAR == 0 ? -c21 * float(8 * (r >> 2) + (r & 3)) : 0.0f;
  // per-lane byte offsets of the swizzled tile reads
  const int rb = Tile::row_base(lane), tb0 = Tile::tr_base(lane, 0), tb1 = Tile::tr_base(lane, 1);

  // Underflow skipping: queries more than R from a key give it P = 0 exactly,
  // so the tiles whose first query lies past the block's last key + R (and
  // all after them) are dropped, without the causal mask also those whose
  // last query lies more than R before its first key (and all before them),
  // and a wave skips the tiles that far from its own keys.
  const int R = VAR == 0 ? live_reach(norms, parts, total / nkb, bh, c1, c2) : (1 << 30);
  int qt0 = CAUSAL ? k0 / BQ : 0;
  if (!CAUSAL && R < (1 << 30) && k0 - R > 0) qt0 = (k0 - R) / BQ;  // tile of the first live query
  int nqt = (N + BQ - 1) / BQ;
  if (R < (1 << 30)) nqt = min(nqt, (k0 + BK - 1 + R) / BQ + 1);

  // staging registers of one query tile (NCH chunks of Q and of dO per thread)
  u32x4 rq[NCH], rdo[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) rq[c] = rdo[c] = u32x4{0u, 0u, 0u, 0u};
  float rl = 0.0f, rd = 0.0f;
  // chunk id = tid + NT c of a tile: global row q0 + id / CPR, chunk id % CPR,
  // i.e. byte 16 id past the tile's first row; rows past N read as zero
  const __amdgpu_buffer_rsrc_t rsq = rows_rsrc<D>(q + base, N), rsdo = rows_rsrc<D>(dout + base, N);
  auto load_tile = [&](int qt) {
    const int q0 = qt * BQ;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int id = tid + NT * c;
      if (id < CHUNKS) {
        const uint32_t vo = uint32_t(q0) * (D * 2) + uint32_t(id) * 16u;
        rq[c] = bload16(rsq, vo);
        rdo[c] = bload16(rsdo, vo);
      }
    }
    if (tid < BQ) {
      const bool ok = q0 + tid < N;
      rl = ok ? lse2[rbase + q0 + tid] : __builtin_huge_valf();  // rows past N: P = 0
      rd = ok ? dsum[rbase + q0 + tid] : 0.0f;
    }
  };
  auto store_tile = [&](unsigned char* st) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int id = tid + NT * c;
      if (id < CHUNKS) {
        const int o = Tile::off(id / CPR, id % CPR);
        *reinterpret_cast<u32x4*>(st + o) = rq[c];
        *reinterpret_cast<u32x4*>(st + RBYTES + o) = rdo[c];
      }
    }
    if (tid < BQ) {
      float* sL = reinterpret_cast<float*>(st + 2 * RBYTES);
      sL[tid] = rl;
      sL[BQ + tid] = rd;
    }
  };
  auto load_frags = [&](const uint16_t* src, bf16x8 (&f)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u};
      if (j < N) a = load16(src + base + (long long)j * D + 16 * ks + 8 * hi);
      f[ks] = __builtin_bit_cast(bf16x8, a);
    }
  };
  // Q K^T (or dO V^T) of the QB blocks of a tile (rows = queries, lane = key),
  // each LDS fragment read once per block; block b starts from init
  auto products = [&](const unsigned char* sX, const bf16x8 (&kf)[KS], const f32x16& init, f32x16 (&out)[QB]) {
#pragma unroll
    for (int b = 0; b < QB; ++b) out[b] = init;
    lds_mfma_ring<KS * QB, 4>(
        [&](int n) {
          return *reinterpret_cast<const bf16x8*>(sX + (n % QB) * 32 * Tile::ROWB + (rb ^ (32 * (n / QB))));
        },
        [&](int n, const bf16x8& a) { out[n % QB] = mfma32(a, kf[n / QB], out[n % QB]); });
  };
  // P = exp2(t - lse2) of block b of a tile whose first row is q0
  // with the soft cap, gc receives dA*/dA = 1 - tanh^2 per score
  auto probs = [&](f32x16& s, const float* sL, int q0, auto open_tag, f32x16& gc) {
    constexpr bool OPEN = decltype(open_tag)::value;  // no query of the tile precedes a key of the block
    const float bj = c2 * float(j - q0 - 4 * hi);  // t = s c1 + bj on the causal side
    const bool full = OPEN || (CAUSAL && q0 >= kw0 + 31);  // every query of the block sees every key of the wave
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 L = *reinterpret_cast<const f32x4*>(sL + 8 * g + 4 * hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const int i = q0 + 8 * g + 4 * hi + e;
        float t;
        if constexpr (VAR == 0) {
          t = fmaf(s[r], c1, bj);
          if (!OPEN && !full && !CAUSAL && j > i) t -= 2.0f * c2 * float(j - i);  // symmetric bias -m |i - j|
        } else if constexpr (CAP) {
          float th;
          t = cap_logit(s[r], cap_in, cap_out, th) +
              var_bias<VAR>(float(CAUSAL ? max(i - j, 0) : abs(i - j)), c2, mh, clamp2);
          gc[r] = fmaf(-th, th, 1.0f);
        } else {
          t = fmaf(s[r], c1, var_bias<VAR>(float(CAUSAL ? max(i - j, 0) : abs(i - j)), c2, mh, clamp2));
        }
        if (!OPEN && !full && CAUSAL && j > i) t = -__builtin_huge_valf();
        s[r] = fast_exp2(t - L[e]);
      }
    }
  };

  // P of a tile, computed by the dV wave of each key group and read by the dK
  // wave of the same group one step later: per buffer, group and 32-row block
  // 16 values per lane, in 16-byte pieces (four fp32 or eight fp16 values),
  // piece c of lane l at 16 (64 c + l).
  constexpr int PBYTES = PH ? 32 : 64;  // per lane and block
  __shared__ __attribute__((aligned(16))) unsigned char sP[2 * 4 * QB * 64 * PBYTES];
  auto p_slot = [&](int tile, int b) {
    return reinterpret_cast<u32x4*>(sP + ((((tile - qt0) & 1) * 4 + (wave & 3)) * QB + b) * 64 * PBYTES);
  };
  auto put_p = [&](u32x4* dst, const f32x16& p) {
    if constexpr (PH) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2 f = {p[8 * c + 2 * e], p[8 * c + 2 * e + 1]};
          w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
        }
        dst[64 * c + lane] = w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        dst[64 * c + lane] = __builtin_bit_cast(u32x4, f32x4{p[4 * c], p[4 * c + 1], p[4 * c + 2], p[4 * c + 3]});
    }
  };
  auto get_p = [&](const u32x4* src) {
    f32x16 p;
    if constexpr (PH) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4 w = src[64 * c + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the word goes through a scalar first: a bit cast taken straight
          // from the vector element compiled to element 0 for every e
          const uint32_t x = w[e];
          const f32x2 f = __builtin_convertvector(__builtin_bit_cast(f16x2, x), f32x2);
          p[8 * c + 2 * e] = f[0];
          p[8 * c + 2 * e + 1] = f[1];
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 x = __builtin_bit_cast(f32x4, src[64 * c + lane]);
#pragma unroll
        for (int e = 0; e < 4; ++e) p[4 * c + e] = x[e];
      }
    }
    return p;
  };
  // Step t: the dV waves take query tile t (S, P, dV), the dK waves tile t - 1
  // (dP, dS = P (dP - D), dK) with the P the dV waves wrote in step t - 1.
  // Tile t sits in stage t % 3; during step t the stage of tile t - 2 (free
  // after the barrier that starts the step) receives tile t + 1.
  auto stage_of = [&](int t) { return smem + ((t - qt0) % 3) * STAGE; };
  if (qt0 < nqt) {
    load_tile(qt0);
    store_tile(stage_of(qt0));
    if (qt0 + 1 < nqt) load_tile(qt0 + 1);
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  // Staging of step t, done after the step's MFMAs are issued so that the
  // wait for the loads and the LDS writes overlap them: tile t + 1 (loaded in
  // step t - 1) goes to its stage, whose last readers finished before the
  // barrier that started step t, and the loads of tile t + 2 are issued.
  auto stage_next = [&](int t) {
    if (t + 1 < nqt) {
      store_tile(stage_of(t + 1));
      if (t + 2 < nqt) load_tile(t + 2);
    }
  };
  // dV^T += dO^T P (or dK^T += Q^T dS): the A operand read transposed from the
  // tile sT, the B operand the packed accumulator rows of block n16 / 2
  auto accumulate = [&](const unsigned char* sT, const f32x16 (&x)[QB]) {
    bf16x8 xb[2 * QB];
#pragma unroll
    for (int n16 = 0; n16 < 2 * QB; ++n16) xb[n16] = __builtin_bit_cast(bf16x8, pack8(x[n16 >> 1], 8 * (n16 & 1)));
    lds_mfma_ring<2 * QB * DB, 4>(
        [&](int n) { return read_tr<D>(sT, tb0, tb1, 16 * (n % (2 * QB)), 32 * (n / (2 * QB))); },
        [&](int n, const bf16x8& a) {
          const int db = n / (2 * QB);
          acc[db] = mfma32(a, xb[n % (2 * QB)], acc[db]);
        });
  };
  if (role == 0) {
    bf16x8 kf[KS];
    load_frags(k, kf);
    auto vstep = [&](int t, auto open_tag) {
      constexpr bool OPEN = decltype(open_tag)::value;
      __syncthreads();
      if (t == nqt) return;
      const unsigned char* st = stage_of(t);
      const int q0 = t * BQ;
      if (CAUSAL ? ((OPEN || q0 + BQ - 1 >= kw0) && q0 - (kw0 + 31) <= R)
                 : (kw0 - (q0 + BQ - 1) <= R && q0 - (kw0 + 31) <= R)) {
        f32x16 p[QB], gcap[QB];
        products(st, kf, cinit, p);
        const float* sL = reinterpret_cast<const float*>(st + 2 * RBYTES);
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          probs(p[b], sL + 32 * b, q0 + 32 * b, open_tag, gcap[b]);
          if constexpr (!CAP) put_p(p_slot(t, b), p[b]);
        }
        accumulate(st + RBYTES, p);
        if constexpr (CAP) {
          // the dK waves form dS = P (1 - tanh^2) (dP - D)
#pragma unroll
          for (int b = 0; b < QB; ++b) {
            p[b] *= gcap[b];
            put_p(p_slot(t, b), p[b]);
          }
        }
      }
      stage_next(t);
    };
    // Query tiles that start at or after the block's last key see every key of
    // the block: no mask (two loops, so those tiles carry no mask arithmetic).
    const int t_open = (k0 + BK - 1 + BQ - 1) / BQ;
    int t = qt0;
    for (; t <= nqt && t < t_open; ++t) vstep(t, std::false_type{});
    for (; t <= nqt; ++t) vstep(t, std::true_type{});
  } else {
    bf16x8 vf[KS];
    load_frags(v, vf);
    for (int t = qt0; t <= nqt; ++t) {
      __syncthreads();
      if (t == qt0) {
        stage_next(t);
        continue;
      }
      const int u = t - 1;  // this wave's tile
      const unsigned char* st = stage_of(u);
      const float* sL = reinterpret_cast<const float*>(st + 2 * RBYTES);
      const int q0 = u * BQ;
      if (CAUSAL ? (q0 + BQ - 1 >= kw0 && q0 - (kw0 + 31) <= R)  // the dV wave's test
                 : (kw0 - (q0 + BQ - 1) <= R && q0 - (kw0 + 31) <= R)) {
        f32x16 dp[QB];
        products(st + RBYTES, vf, f32x16{}, dp);
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          const f32x16 p = get_p(p_slot(u, b));
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 Dv = *reinterpret_cast<const f32x4*>(sL + BQ + 32 * b + 8 * g + 4 * hi);
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[b][4 * g + e] = p[4 * g + e] * (dp[b][4 * g + e] - Dv[e]);  // dS
          }
        }
        accumulate(st, dp);
      }
      stage_next(t);
    }
  }

  // ---- epilogue: lane = key j, rows of the accumulator = d ----
  if (j < N) {
    uint16_t* dst = role == 0 ? dv : dk;
    const float sc = role == 0 ? 1.0f : scale;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 a;
        a[0] = pack_bf16x2(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc);
        a[1] = pack_bf16x2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc);
        *reinterpret_cast<u32x2*>(dst + base + (long long)j * D + 32 * db + 8 * g + 4 * hi) = a;
      }
    }
  }
}

// ---------------------------------------------------------------- dQ --------
template <int D, bool CAUSAL, int VAR>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ dsum,
    uint16_t* __restrict__ dq, int H, int N, int nqb, int total, const float* __restrict__ slopes,
    float c1, float scale, float clamp2, float cap_in, float cap_out, const float* __restrict__ norms, int parts) {
  constexpr int NT = 256, BM = 128, BN = 32;
  constexpr bool CAP = (VAR & kBwdCap) != 0;
  constexpr int KS = D / 16, KB = BN / 32, DB = D / 32, PS = BN / 16, CPR = D / 8;
  using Tile = SwzTile<D>;              // K and V tiles: swizzled rows of 2 D bytes
  constexpr int KBYTES = BN * Tile::ROWB;
  constexpr int STAGE = 2 * KBYTES;
  constexpr int LOADS = BN * CPR / NT;
  static_assert(LOADS * NT == BN * CPR, "tile must split evenly");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const WgBlock wb = schedule_block(blockIdx.x, total / nqb, nqb);
  const int bh = wb.bh;
  const int qblk = nqb - 1 - wb.rank;  // high query blocks see the most keys: scheduled first
  const int h = bh % H;
  const float mh = slopes[h];
  const float c2 = mh * kLog2e;
  const float c21 = c2 / c1;
  const long long base = (long long)bh * N * D;
  const long long rbase = (long long)bh * N;
  const int q0 = qblk * BM;
  const int qw0 = q0 + wave * 32;
  const int qw_last = min(qw0 + 32, N) - 1;
  const int i = qw0 + l32;

  bf16x8 qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (i < N) {
      a = load16(q + base + (long long)i * D + 16 * ks + 8 * hi);
      b = load16(dout + base + (long long)i * D + 16 * ks + 8 * hi);
    }
    qf[ks] = __builtin_bit_cast(bf16x8, a);
    of[ks] = __builtin_bit_cast(bf16x8, b);
  }
  const float L = i < N ? lse2[rbase + i] : __builtin_huge_valf();
  const float Dr = i < N ? dsum[rbase + i] : 0.0f;
  f32x16 cinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) cinit[r] = VAR == 0 ? c21 * float(8 * (r >> 2) + (r & 3)) : 0.0f;
  const int rb = Tile::row_base(lane), tb0 = Tile::tr_base(lane, 0), tb1 = Tile::tr_base(lane, 1);
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  f32x16 dinit;  // dP^T seeded with -D, so the MFMA yields dP - D
#pragma unroll
  for (int r = 0; r < 16; ++r) dinit[r] = -Dr;

  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  // Underflow skipping: key tiles whose last key lies more than R before the
  // block's first query carry P = 0 exactly for every query of the block: the
  // walk stops above them (t_lo); without the causal mask it also starts below
  // the tiles whose first key lies more than R after the block's last query
  // (t_hi); and a wave skips the tiles that far from its own queries.
  const int R = VAR == 0 ? live_reach(norms, parts, total / nqb, bh, c1, c2) : (1 << 30);
  const int xdead = q0 - BN - R;  // tiles with j0 <= xdead are dead
  const int t_lo = R < (1 << 30) && xdead >= 0 ? xdead / BN + 1 : 0;
  const int t_hi = !CAUSAL && R < (1 << 30) ? min(ntiles - 1, (q0 + BM - 1 + R) / BN) : ntiles - 1;

  u32x4 rk[LOADS], rv[LOADS];
  // chunk tid + NT r of a tile: byte 16 (tid + NT r) past its first row; rows
  // past N read as zero. In LDS it sits NT / CPR rows (a multiple of 16, so the
  // same swizzle) below chunk tid.
  const __amdgpu_buffer_rsrc_t rsk = rows_rsrc<D>(k + base, N), rsv = rows_rsrc<D>(v + base, N);
  const int sto = Tile::off(tid / CPR, tid % CPR);
  static_assert((NT / CPR) % 16 == 0, "row step keeps the swizzle");
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const uint32_t vo = uint32_t(j0) * (D * 2) + uint32_t(tid + NT * r) * 16u;
      rk[r] = bload16(rsk, vo);
      rv[r] = bload16(rsv, vo);
    }
  };
  auto store_tile = [&](unsigned char* st) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      *reinterpret_cast<u32x4*>(st + sto + r * (NT / CPR) * Tile::ROWB) = rk[r];
      *reinterpret_cast<u32x4*>(st + KBYTES + sto + r * (NT / CPR) * Tile::ROWB) = rv[r];
    }
  };

  if (ntiles > 0) {
    load_tile(t_hi * BN);
    store_tile(smem);
  }
  // Tiles wholly at or before the block's first query (and below N) need no
  // mask for any wave; their bias is the causal one in both modes. The others
  // (the diagonal, and without the causal mask the tiles after the queries)
  // are visited first and take the per-score mask. Two loops, so the open
  // tiles carry no mask arithmetic at all.
  int stage = 0;
  auto step = [&](int tile, auto open_tag) {
    constexpr bool OPEN = decltype(open_tag)::value;
    const int j0 = tile * BN;
    __syncthreads();
    if (tile > t_lo) load_tile(j0 - BN);
    const unsigned char* st = smem + stage * STAGE;
    const unsigned char* sK = st;
    const unsigned char* sV = st + KBYTES;
    const bool active = qw0 < N && (CAUSAL ? ((OPEN || j0 <= qw_last) && qw0 - (j0 + BN - 1) <= R)
                                           : (qw0 - (j0 + BN - 1) <= R && j0 - (qw0 + 31) <= R));
    if (active) {
      // ---- per 32-key block: S^T = K Q^T, dP^T = V dO^T (lane = query), then
      // P^T = exp2(t - lse2) and dS^T = P^T (dP^T - D) packed to bf16 ----
      const bool full = OPEN || (CAUSAL && j0 + BN - 1 <= qw0 && j0 + BN <= N);
      const float bt0 = c2 * float(j0 + 4 * hi - i) - L;
      u32x4 pf[PS];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x16 s = cinit, dp = dinit;
        // fragment 2 ks: K (for S), 2 ks + 1: V (for dP)
        lds_mfma_ring<2 * KS, 2>(
            [&](int n) {
              return *reinterpret_cast<const bf16x8*>(((n & 1) ? sV : sK) + 32 * kb * Tile::ROWB + (rb ^ (32 * (n >> 1))));
            },
            [&](int n, const bf16x8& a) {
              if (n & 1) dp = mfma32(a, of[n >> 1], dp);
              else s = mfma32(a, qf[n >> 1], s);
            });
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * half + e;
            float t, th = 0.0f;
            if constexpr (VAR == 0) {
              t = fmaf(s[r], c1, bt0 + 32.0f * kb * c2);
              if (!OPEN && !full) {
                const int jj = j0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (!CAUSAL && jj > i) t -= 2.0f * c2 * float(jj - i);
                if (jj >= N || (CAUSAL && jj > i)) t = -__builtin_huge_valf();
              }
            } else if constexpr (CAP) {
              const int jj = j0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
              t = cap_logit(s[r], cap_in, cap_out, th) +
                  (var_bias<VAR>(float(CAUSAL ? max(i - jj, 0) : abs(i - jj)), c2, mh, clamp2) - L);
              if (!OPEN && !full && (jj >= N || (CAUSAL && jj > i))) t = -__builtin_huge_valf();
            } else {
              const int jj = j0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
              t = fmaf(s[r], c1, var_bias<VAR>(float(CAUSAL ? max(i - jj, 0) : abs(i - jj)), c2, mh, clamp2) - L);
              if (!OPEN && !full && (jj >= N || (CAUSAL && jj > i))) t = -__builtin_huge_valf();
            }
            if constexpr (CAP)
              x[e] = fast_exp2(t) * fmaf(-th, th, 1.0f) * dp[r];  // dS of the content logit
            else
              x[e] = fast_exp2(t) * dp[r];
          }
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
          pf[2 * kb + half] = pk;
        }
      }
      // ---- dQ^T += K^T dS^T ----
      lds_mfma_ring<DB * PS, 2>(
          [&](int n) { return read_tr<D>(sK, tb0, tb1, 16 * (n % PS), 32 * (n / PS)); },
          [&](int n, const bf16x8& a) { acc[n / PS] = mfma32(a, __builtin_bit_cast(bf16x8, pf[n % PS]), acc[n / PS]); });
    }
    if (tile > t_lo) store_tile(smem + (stage ^ 1) * STAGE);
    stage ^= 1;
  };
  const int x_open = q0 + 1;  // keys [0, x_open) are at or before every query of the block
  const int t_open = x_open < BN ? -1 : min(min(x_open / BN - 1, N / BN - 1), ntiles - 1);
  int tile = t_hi;
  for (; tile > max(t_open, t_lo - 1); --tile) step(tile, std::false_type{});
  for (; tile >= t_lo; --tile) step(tile, std::true_type{});

  if (i < N) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 st;
        st[0] = pack_bf16x2(acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale);
        st[1] = pack_bf16x2(acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale);
        *reinterpret_cast<u32x2*>(dq + base + (long long)i * D + 32 * db + 8 * g + 4 * hi) = st;
      }
    }
  }
}

// Query blocks of 32 rows per dK/dV step: 1 or 2 (ALIBI_BWD_QB at load time,
// or set_bwd_query_blocks; 0 = automatic, which takes 2).
std::atomic<int>& bwd_qb_override() {
  static std::atomic<int> w{[] {
    const char* e = std::getenv("ALIBI_BWD_QB");
    const int n = e != nullptr ? std::atoi(e) : 0;
    return (n == 1 || n == 2) ? n : 0;
  }()};
  return w;
}
// 64-row query tiles measure faster in every form (B8 H16 N4096 d128: 2.01 vs
// 2.14 ms for the whole backward; B4 H12 N2048 d64: 0.154 vs 0.169 ms).
int bwd_query_blocks() {
  const int o = bwd_qb_override().load(std::memory_order_relaxed);
  return o != 0 ? o : 2;
}

template <int D, bool CAUSAL, int VAR>
hipError_t launch_bwd_cfg(const BwdArgs& a, float* dsum, float* lse2, float c1, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(unsigned((rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                     (const uint16_t*)a.out, (const uint16_t*)a.dout, a.lse, dsum, lse2, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale = float(1.0 / std::sqrt(double(D)));
  const int nkb = (a.N + 127) / 128;
  const long long tk = (long long)a.B * a.H * nkb;
  if (bwd_query_blocks() == 2)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VAR, 2>), dim3(unsigned(tk)), dim3(512), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, lse2, dsum, (uint16_t*)a.dk, (uint16_t*)a.dv, a.H, a.N,
                       nkb, int(tk), a.slopes, c1, scale, a.clamp2, a.cap_in, a.cap_out, a.norms, a.norm_parts);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VAR, 1>), dim3(unsigned(tk)), dim3(512), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, lse2, dsum, (uint16_t*)a.dk, (uint16_t*)a.dv, a.H, a.N,
                       nkb, int(tk), a.slopes, c1, scale, a.clamp2, a.cap_in, a.cap_out, a.norms, a.norm_parts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (a.N + 127) / 128;
  const long long tq = (long long)a.B * a.H * nqb;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, VAR>), dim3(unsigned(tq)), dim3(256), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, lse2, dsum, (uint16_t*)a.dq, a.H, a.N, nqb, int(tq),
                     a.slopes, c1, scale, a.clamp2, a.cap_in, a.cap_out, a.norms, a.norm_parts);
  return hipGetLastError();
}

}  // namespace

namespace {

template <int D, bool CAUSAL>
hipError_t launch_bwd_var(const BwdArgs& a, float* dsum, float* lse2, float c1, hipStream_t stream) {
  switch (a.flags & 7) {
    case 0: return launch_bwd_cfg<D, CAUSAL, 0>(a, dsum, lse2, c1, stream);
    case 1: return launch_bwd_cfg<D, CAUSAL, 1>(a, dsum, lse2, c1, stream);
    case 2: return launch_bwd_cfg<D, CAUSAL, 2>(a, dsum, lse2, c1, stream);
    case 3: return launch_bwd_cfg<D, CAUSAL, 3>(a, dsum, lse2, c1, stream);
    case 4: return launch_bwd_cfg<D, CAUSAL, 4>(a, dsum, lse2, c1, stream);
    case 5: return launch_bwd_cfg<D, CAUSAL, 5>(a, dsum, lse2, c1, stream);
    case 6: return launch_bwd_cfg<D, CAUSAL, 6>(a, dsum, lse2, c1, stream);
    default: return launch_bwd_cfg<D, CAUSAL, 7>(a, dsum, lse2, c1, stream);
  }
}

}  // namespace

void set_bwd_query_blocks(int qb) { bwd_qb_override().store(qb, std::memory_order_relaxed); }

hipError_t launch_bwd(const BwdArgs& a, float* ws, float c1, hipStream_t stream) {
  float* dsum = ws;
  float* lse2 = ws + (long long)a.B * a.H * a.N;
  if (a.d == 128)
    return a.causal ? launch_bwd_var<128, true>(a, dsum, lse2, c1, stream)
                    : launch_bwd_var<128, false>(a, dsum, lse2, c1, stream);
  return a.causal ? launch_bwd_var<64, true>(a, dsum, lse2, c1, stream)
                  : launch_bwd_var<64, false>(a, dsum, lse2, c1, stream);
}

}  // namespace alibi
