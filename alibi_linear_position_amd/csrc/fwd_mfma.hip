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
// * A workgroup is NW = 4 or 8 waves and owns BM = 32 NW consecutive query
//   rows of one (b, h); each wave owns 32 rows. Two waves share each SIMD (at
//   most 256 registers per lane; two 4-wave or one 8-wave workgroup per CU);
//   the barrier of every tile keeps the two in phase, so the time of a tile is
//   close to its MFMA time plus its softmax time.
// * Key/value tiles of BN = 64 rows are staged HBM -> registers -> LDS by the
//   whole workgroup through buffer resources: K row-major (16-byte coalesced
//   loads, rows padded by 16 B against bank conflicts), V transposed to
//   V^T[d][key], each thread loading the same 8 d of 2 or 4 consecutive keys
//   and writing them per d as one 4- or 8-byte store (v_perm_b32), so every
//   wave reads its MFMA A operands with 16-byte LDS reads, four fragments
//   ahead of their MFMAs. LDS is double-buffered: the loads of the next tile
//   are in flight while the current one is computed, with one barrier per
//   tile.
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
//   Tiles under the causal mask form the row maximum from the tile; tiles with
//   every key visible exponentiate against the running maximum directly and
//   form a bound of the row maximum (max_j s_ij * c1 plus the largest bias in
//   the tile) only when a lane's partial row sum leaves (0, 2^16], redoing the
//   tile then; any bound works for the algebra.
//   The first Q K^T k-step takes a constant register set as its C operand,
//   which seeds each score with its register's bias offset, so the bias costs
//   one fma per score. Row reductions across the two lane halves use
//   v_permlane32_swap; row sums use four independent accumulators.
// * The row sum is accumulated from the bf16-rounded p that the PV product
//   uses (v_dot2c_f32_bf16), so the normalisation matches the numerator.
// * Grid: one workgroup per (b, h, query block), heaviest causal blocks first
//   and blocks of one (b, h) kept on one XCD (workgroups are dealt to the 8
//   XCDs round-robin), so the K/V of a head is shared through that XCD's L2.
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <type_traits>

namespace alibi {

namespace {

// Forced waves per workgroup: 0 = automatic, else 4 or 8 (ALIBI_FWD_NW at
// load time, or set_fwd_waves).
std::atomic<int>& waves_override() {
  static std::atomic<int> w{[] {
    const char* e = std::getenv("ALIBI_FWD_NW");
    const int n = e != nullptr ? std::atoi(e) : 0;
    return (n == 4 || n == 8) ? n : 0;
  }()};
  return w;
}

// Forced key-range split of the plain causal form: 0 = automatic, 1 = never,
// 2 = always (ALIBI_FWD_SPLIT at load time, or set_fwd_split).
std::atomic<int>& split_override() {
  static std::atomic<int> w{[] {
    const char* e = std::getenv("ALIBI_FWD_SPLIT");
    const int n = e != nullptr ? std::atoi(e) : 0;
    return (n == 1 || n == 2) ? n : 0;
  }()};
  return w;
}

// The split form (two key groups of 4 waves per 128 query rows) for the plain
// causal form (with offsets, the log-sum-exp output or the exact skipping,
// which therefore stays bit-identical to the call without it), where the
// heaviest query block's walk bounds the run. A tile-step model: unsplit,
// 4-wave workgroups of 128 rows walk T_b tiles each, two per CU, so the run
// takes about max(max_b T_b, sum_b T_b / 512) steps; split, one 8-wave
// workgroup per CU walks ceil(T_b / 2), about max(max_b ceil(T_b / 2),
// sum_b ceil(T_b / 2) / 256). Measured against that model (d = 64 and 128,
// interleaved A/B), the split form pays for its second LDS stage set, its
// merge and its two rounds of workgroups when the modelled ratio is below
// ~0.7: B8 H8 N1024 d64 (0.56) 21.5 vs 24.2 us, B1 H16 N4096 d128 (0.52) 84
// vs 96 us, B4 H12 N2048 d64 (0.80) even, a 512-row chunk against 4096 keys
// (0.95) and B2 H16 N4096 d128 (1.0) 10-19% slower.
bool fwd_split(const FwdArgs& a, int flags, int delta) {
  if (!a.causal || flags != 0) return false;
  const int o = split_override().load(std::memory_order_relaxed);
  if (o != 0) return o == 2;
  if (waves_override().load(std::memory_order_relaxed) != 0) return false;
  long long t_max = 0, t_sum = 0, h_sum = 0;
  for (long long q0 = 0; q0 < a.Nq; q0 += 128) {
    const long long kend = std::max(0LL, std::min<long long>(a.Nk, q0 + 128 + delta));
    const long long t = (kend + 63) / 64;
    t_max = std::max(t_max, t);
    t_sum += t;
    h_sum += (t + 1) / 2;
  }
  const double bh = double(a.B) * a.H;
  const double unsplit = std::max(double(t_max), bh * double(t_sum) / 512.0);
  const double split = std::max(double((t_max + 1) / 2), bh * double(h_sum) / 256.0);
  return split < 0.7 * unsplit;
}

// Waves per workgroup. Two waves share each SIMD either way; 8 waves (one
// workgroup per CU) halve the K/V staging per query row and measure faster for
// d = 128 in every form (B8 H16 N4096: plain 1006 vs 939, soft cap 781 vs
// 759 TFLOP/s), while d = 64 and grids of fewer than two 8-wave workgroups per
// CU run better as two 4-wave workgroups.
int fwd_waves(const FwdArgs& a, int flags) {
  (void)flags;
  const int o = waves_override().load(std::memory_order_relaxed);
  if (o != 0) return o;
  if (a.d != 128) return 4;
  const long long wg8 = (long long)a.B * a.H * ((a.Nq + 255) / 256);
  return wg8 >= 512 ? 8 : 4;
}
constexpr float kLazy = 8.0f;
// Largest partial row sum (32 keys of one lane) accepted without a fresh bound.
constexpr float kOptLimit = 65536.0f;
// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family parts:
// 32-bit data format, byte-granular range check against the record count.
constexpr int kBufferFlags = 0x00020000;

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

// Largest |a_r| of 16 accumulator values.
__device__ __forceinline__ float absmax16(const f32x16& a) {
  float m = fabsf(a[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, fabsf(a[r]));
  return m;
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

// One K/V tile of BN keys as the workgroup stages it: each thread holds LOADS
// 16-byte chunks of K (row-major, coalesced) and LOADS chunks of V (the same 8
// d of LOADS consecutive keys, so the transposed LDS writes are LOADS keys wide).
template <int D, int NT>
struct TileRegs {
  static constexpr int BN = 64;
  static constexpr int CPR = D / 8;
  static constexpr int LOADS = BN * CPR / NT;
  static_assert(LOADS * NT == BN * CPR, "tile must split evenly");
  u32x4 k[LOADS];
  u32x4 v[LOADS];

  // Loads of one tile through buffer resources: chunk r of K sits at byte
  // 16 (tid + NT r) of the tile (rows are contiguous), chunk r of V at byte
  // 2 ((LOADS (tid % KG) + r) D + 8 (tid / KG)). Each thread's byte offset is fixed
  // and the tile's byte offset `tb` is a scalar, so a load carries no per-tile
  // vector address arithmetic. A resource whose range ends at row Nk makes
  // rows past it read as zero when the tile starts at the resource's base
  // (tb = 0: the range check covers the vector offset).
  static __device__ __forceinline__ uint32_t k_off(int tid) { return uint32_t(tid) * 16u; }
  static constexpr int KG = BN / LOADS;  // V: groups of LOADS consecutive keys
  static __device__ __forceinline__ uint32_t v_off(int tid) {
    return (uint32_t(tid % KG) * LOADS * D + uint32_t(tid / KG) * 8u) * 2u;
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t tb,
                                       uint32_t koff, uint32_t voff) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      k[r] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, int(tb + uint32_t(NT * 16 * r)), 0));
      v[r] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, int(tb + uint32_t(r * D * 2)), 0));
    }
  }

  // K rows go to LDS as loaded. V goes transposed, V^T[d][key], with the key
  // order of each 16-key group permuted (perm16) to match the accumulator
  // layout of P^T: a thread holds the same 8 d of LOADS consecutive keys, so
  // for every d it writes their LOADS values as one 2 LOADS-byte store (the
  // keys of a 4-group stay contiguous under perm16).
  template <int KPITCH, int VPITCH>
  __device__ __forceinline__ void store(unsigned char* sK, unsigned char* sV, int tid) const {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int c = tid + NT * r;
      const int row = c / CPR, col = c % CPR;
      *reinterpret_cast<u32x4*>(sK + row * KPITCH + col * 16) = k[r];
    }
    const int key = (tid % KG) * LOADS, vcol = tid / KG;
    const int pos = (key & ~15) | perm16(key & 15);
    unsigned char* dst = sV + (vcol * 8) * VPITCH + pos * 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // bf16 e of each key: the low (even e) or high (odd e) half of word e / 2
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      if constexpr (LOADS == 4) {
        u32x2 w;
        w[0] = __builtin_amdgcn_perm(v[1][e >> 1], v[0][e >> 1], sel);
        w[1] = __builtin_amdgcn_perm(v[3][e >> 1], v[2][e >> 1], sel);
        *reinterpret_cast<u32x2*>(dst + e * VPITCH) = w;
      } else if constexpr (LOADS == 2) {
        *reinterpret_cast<uint32_t*>(dst + e * VPITCH) = __builtin_amdgcn_perm(v[1][e >> 1], v[0][e >> 1], sel);
      } else {
        static_assert(LOADS == 1, "1, 2 or 4 keys per thread");
        *reinterpret_cast<uint16_t*>(dst + e * VPITCH) = uint16_t((e & 1) ? v[0][e >> 1] >> 16 : v[0][e >> 1]);
      }
    }
  }
};

// Mitigation variants (Sec. 3.4 of "When Attention Goes Blind"), as bits of the
// kernel's VAR template argument: the bias floored at a constant, the distance
// replaced by ln(D + 1), the content logit soft-capped as z tanh(A / z).
constexpr int kVarClamp = 1, kVarLog = 2, kVarSoftcap = 4;

// Run-time parameters of a variant launch, all in log2 units of the scores.
struct FwdVariant {
  int delta;      // position of query row 0 minus position of key row 0
  float clamp2;   // bias floor c_clamp log2(e)
  float cap_in;   // 2 log2(e) / (sqrt(d) z): exp2(s cap_in) = e^(2 A / z) for s = q.k
  float cap_out;  // z log2(e)
  float cap_small;  // largest |s| with |A| <= z / 4
  float cap_q[3];   // z log2(e) tanh(A / z) ~ s (q0 + q1 s^2 + q2 s^4) for |A| <= z / 4
  // Exact underflow skipping (plain form): `parts` partial maxima
  // of the key norms of each (b, h), or null.
  const float* knorm;
  int parts;
  float* lse;  // optional (B, H, Nq) row log-sum-exp output, natural log
  // Optional hard window (plain causal form): H ints, query i sees key j when
  // 0 <= pi - j < window[h] ("When Attention Goes Blind", Sec. 5.2-5.3).
  const int* window;
};

// A score whose exponent lies more than this many log2 units below the row's
// running maximum gives p < 2^-134, which rounds to zero in bf16 (the smallest
// subnormal is 2^-133); the skipping bound uses 140 plus the lazy-rescale lag.
constexpr float kDeadLog2 = 140.0f + kLazy;

// EXT = false compiles the plain call (alibi_attn_fwd: no offsets, no
// skipping, no log-sum-exp output) without those paths.
//
// SPLIT = 2 (plain causal form, 8 waves) splits the key range of a query
// block instead of its rows: the workgroup owns 4 x 32 query rows, waves 0-3
// take the block's key tiles 0, 2, 4, ... counted from the diagonal and waves
// 4-7 the tiles 1, 3, 5, ... for the same rows, each group staging its own
// tiles; at the end the two partial softmax states of a row (running maximum
// m, row sum l, unnormalised output O) are merged through LDS as
// M = max(m0, m1), l = 2^(m0 - M) l0 + 2^(m1 - M) l1, O likewise (the
// stable-softmax algebra of "When Attention Goes Blind", App. B.1-B.2). The
// heaviest causal block then walks half as many tiles, which is what bounds
// grids too small to fill the chip twice over.
template <int D, int NW, bool CAUSAL, int VAR, bool EXT, int SPLIT = 1>
__global__ __launch_bounds__(NW * 64, 2) void fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, int H, int Nq, int Nk, int nqb, int total,
    const float* __restrict__ slopes, float c1, FwdVariant var) {
  static_assert(SPLIT == 1 || (SPLIT == 2 && NW == 8 && CAUSAL && VAR == 0), "split: plain causal, 8 waves");
  constexpr int NWG = NW / SPLIT;  // waves per key group
  constexpr int NT = NWG * 64;     // threads staging one group's tiles
  constexpr int BN = 64;
  constexpr int BM = NWG * 32;
  constexpr int KS = D / 16;       // MFMA k-steps of Q K^T
  constexpr int KB = BN / 32;      // 32-key blocks per tile
  constexpr int DB = D / 32;       // 32-wide d blocks of O
  constexpr int PS = BN / 16;      // MFMA k-steps of P V
  constexpr int KPITCH = D * 2 + 16;
  constexpr int VPITCH = BN * 2 + 16;
  constexpr int KBYTES = BN * KPITCH;
  constexpr int STAGE = KBYTES + D * VPITCH;
  __shared__ __attribute__((aligned(16))) unsigned char smem_all[SPLIT * 2 * STAGE];

  // The wave index is uniform across the wave; say so, so that every per-wave
  // condition below compiles to a scalar branch instead of masked execution.
  const int wave_all = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int grp = SPLIT == 1 ? 0 : wave_all / NWG;  // key group
  const int wave = wave_all - grp * NWG;             // wave within the group
  const int tid = int(threadIdx.x) - grp * NT;       // thread within the group
  unsigned char* const smem = smem_all + grp * 2 * STAGE;  // the group's two stages
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Workgroup -> (b, h, query block): heads kept per XCD, the heaviest (last)
  // query blocks of every head first.
  const WgBlock wb = schedule_block(blockIdx.x, total / nqb, nqb);
  const int bh = wb.bh;
  const int qblk = nqb - 1 - wb.rank;
  const int h = bh % H;
  const float mh = slopes[h];
  const float c2 = mh * kLog2e;
  const long long qbase = (long long)bh * Nq * D;
  const long long kbase = (long long)bh * Nk * D;
  const int q0 = qblk * BM;
  const int qw0 = q0 + wave * 32;                      // first query row of this wave
  const int qw_last = min(qw0 + 32, Nq) - 1;           // last valid query row of this wave
  const int i = qw0 + l32;                             // this lane's query row
  // Query row i sits at key-index position pi: key j is visible to it when
  // j <= pi (causal) and lies at distance pi - j.
  const int delta = EXT ? var.delta : 0;
  const int pi = i + delta;

  // C operand of the first Q K^T k-step: seeds register r of a 32-key block
  // with its bias offset m log2(e) (8 (r / 4) + r % 4) / c1, so tiles without
  // a mask need one fma per score to complete the linear bias. Variants keep
  // the plain content score (their bias is not linear in the key index).
  // The clamp-only causal variant seeds the tiles that lie wholly inside the
  // distance where the floor starts and gives the others a zero C operand;
  // with 4 waves at d = 128 (more staging registers per lane) those extra
  // tile classes would spill, so there every clamp tile takes the per-score
  // path.
  constexpr bool SEED = VAR == 0 || (VAR == kVarClamp && CAUSAL && (NW == 8 || D == 64));
  f32x16 cinit;
  const float c21 = c2 / c1;
#pragma unroll
  for (int r = 0; r < 16; ++r) cinit[r] = SEED ? c21 * float(8 * (r >> 2) + (r & 3)) : 0.0f;
  // Log-scaled distances without the soft cap: open tiles seed every score
  // with -m_seed / c1, m_seed the row's running maximum (0 while it is
  // -inf), so the per-score fma that adds the bias yields the exponent
  // relative to the maximum directly. The seed is rebuilt where the maximum
  // moves.
  constexpr bool MSEED = (VAR & kVarLog) != 0 && (VAR & kVarSoftcap) == 0;
  // Soft-capped open tiles build the exponent relative to the running
  // maximum per score (the cap applies before the bias, so no seed can carry
  // either); with MSEED, open tiles hand the exponentials t - m directly.
  constexpr bool CAPREL = (VAR & kVarSoftcap) != 0;
  constexpr bool REL = MSEED || CAPREL;
  f32x16 mseed = f32x16{};
  float m_seed = 0.0f;
  const float rc1 = 1.0f / c1;

  // Q^T fragments (MFMA B operand): lane holds query l32, d = 16 ks + 8 hi .. +7.
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (i < Nq) raw = *reinterpret_cast<const u32x4*>(q + qbase + (long long)i * D + 16 * ks + 8 * hi);
    qf[ks] = __builtin_bit_cast(bf16x8, raw);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;

  // Keys any query of the block can see: [0, kend).
  const int kend = CAUSAL ? max(0, min(Nk, q0 + BM - 1 + delta + 1)) : Nk;
  const int ntiles = (kend + BN - 1) / BN;

  TileRegs<D, NT> regs;
  const uint32_t koff = TileRegs<D, NT>::k_off(tid), voff = TileRegs<D, NT>::v_off(tid);
  // K and V rows of this (b, h): Nk D bf16 each, at most 2^24 rows of 128
  // values (2^32 bytes); the range is capped at 2^32 - 1 bytes, which no valid
  // 16-byte chunk reaches. Byte offsets are 32-bit unsigned.
  auto rsrc = [&](const uint16_t* p, long long rows) {
    const uint32_t bytes = uint32_t(min(rows * D * 2, 0xffffffffLL));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, int(bytes), kBufferFlags);
  };
  const __amdgpu_buffer_rsrc_t rk = rsrc(k + kbase, Nk), rv = rsrc(v + kbase, Nk);
  {
    // The first tile visited is the only one that can reach past Nk: stage it
    // through resources that start at the tile, so missing rows read as zero.
    // With no tile to visit (every query before every key) tile 0 is staged
    // and never read.
    int first = ntiles - 1 - grp;
    if (!CAUSAL && Nk % BN == 0) {  // the order of the loops below
      const int x = q0 + delta + 1, nfull = Nk / BN;
      const int tl = x < BN ? -1 : min(x / BN - 1, nfull - 1);
      const int ql = q0 + BM - 1 + delta;
      const int tr = max(tl + 1, ql <= 0 ? 0 : (ql + BN - 1) / BN);
      const int mid_hi = min(tr, nfull) - 1;
      first = mid_hi > tl ? mid_hi : (tr < nfull ? tr : tl);
    }
    const int jp = max(first, 0) * BN;
    regs.load(rsrc(k + kbase + (long long)jp * D, Nk - jp), rsrc(v + kbase + (long long)jp * D, Nk - jp), 0u,
              koff, voff);
    regs.template store<KPITCH, VPITCH>(smem, smem + KBYTES, tid);
  }

  // ---- exact underflow skipping ----
  // For row i, every score against key j is at most A_i + c2 (j - pi) with
  // A_i = |q_i| max_j |k_j| c1 (Cauchy-Schwarz), and the row's running maximum
  // after its diagonal tile is at least its nearest visible key's score minus
  // the lazy lag: >= -A_i - c2 max(0, pi - Nk + 1) - kLazy. A tile whose last
  // key j_max has c2 (pi - j_max) > 140 + kLazy + 2 A_i + c2 max(0, pi - Nk + 1)
  // therefore holds only p that round to exactly zero: skipping it leaves the
  // output bit for bit unchanged. Tiles are visited from the diagonal backwards
  // and the bound only grows with the distance, so everything at or below a
  // wave's first dead tile is dead; the workgroup stops at the lowest tile any
  // of its waves still needs, and a wave skips its own dead tiles before that.
  __shared__ int s_dead[NWG];
  // Log-distance bias table of each wave's open tile: four copies of the
  // strip bias(D) for the tile's 95 distances, copy a shifted by a entries
  // (after 4 floats of padding, so that no write falls before its copy) so
  // that every lane reads its four consecutive keys with one aligned 16-byte
  // read; copies 132 floats apart so those reads hit distinct banks.
  constexpr int kTabPitch = 132;
  __shared__ __attribute__((aligned(16))) float ltab[(VAR & kVarLog) != 0 ? NW * 4 * kTabPitch : 4];
  int t_dead_wave = -1, t_dead = -1;
  // Without the causal mask (symmetric bias): the first tile past the queries
  // from which every key is dead too (2^30: none).
  int t_rdead_wave = 1 << 30, t_rdead = 1 << 30;
  __shared__ int s_rdead[NWG];
  // Hard window: keys j <= pi - W are out of row i's window. Tiles up to
  // t_wmask hold such a key for some row of the block and take the masked
  // path; tiles wholly out of a wave's window are dead for it, like the
  // skipped ones. W is clamped to +-2^30 so that pi - W stays an int.
  const bool win_on = EXT && CAUSAL && VAR == 0 && var.window != nullptr;
  const int wwin = win_on ? max(-(1 << 30), min(var.window[h], 1 << 30)) : (1 << 30);
  int t_wmask = -1;
  if (EXT && VAR == 0 && ((var.knorm != nullptr && c2 > 0.0f) || win_on)) {
    int td = -1, trd = 1 << 30;
    if (var.knorm != nullptr && c2 > 0.0f) {
    float kmax = 0.0f;
    for (int p = 0; p < var.parts; ++p) kmax = fmaxf(kmax, var.knorm[(long long)bh * var.parts + p]);
    float qn2 = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 raw = __builtin_bit_cast(u32x4, qf[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16lo_to_f32(raw[e]), b = bf16hi_to_f32(raw[e]);
        qn2 = fmaf(a, a, fmaf(b, b, qn2));
      }
    }
    // norms and their product carry a relative margin of 2^-8 against rounding
    const float A = sqrtf(sum_xor32(qn2)) * kmax * c1 * (1.0f + 1.0f / 256.0f);
    const float reach_f = (kDeadLog2 + 2.0f * A) / c2 + 1.0f;
    // the row's nearest key lies at distance max(0, pi - Nk + 1) (and, without
    // the mask, -pi for a row before every key); its score bounds the maximum
    const int dnear = CAUSAL ? max(0, pi - Nk + 1) : max(max(0, pi - Nk + 1), -pi);
    const int reach = reach_f < 1.0e9f ? int(reach_f) + dnear : (1 << 30);
    const int x = pi - reach;                                   // dead: j_max < x
    td = x >= 0 ? x / BN - 1 : -1;                               // last tile with j_max < x
    if (!CAUSAL && reach < (1 << 30)) trd = (pi + reach) / BN + 1;  // first tile with j0 > pi + reach
    }
    if (win_on) {
      const int xw = pi - wwin + 1;                              // out of the window: j < xw
      td = max(td, xw >= 0 ? xw / BN - 1 : -1);
      const int xb = min(q0 + BM, Nq) - 1 + delta - wwin + 1;    // the same for the block's last row
      t_wmask = xb >= 1 ? (xb - 1) / BN : -1;                    // tiles with j0 < xb
    }
    if (i >= Nq) td = 1 << 30, trd = -1;                         // rows past Nq do not count
    td = min(td, __shfl_xor(td, 32, 64));
    trd = max(trd, __shfl_xor(trd, 32, 64));
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
      td = min(td, __shfl_xor(td, off, 64));
      trd = max(trd, __shfl_xor(trd, off, 64));
    }
    t_dead_wave = max(__builtin_amdgcn_readfirstlane(td), -1);
    t_rdead_wave = __builtin_amdgcn_readfirstlane(trd);
    if (lane == 0 && grp == 0) {
      s_dead[wave] = t_dead_wave;  // wave w + 4 has the same rows
      s_rdead[wave] = t_rdead_wave;
    }
    __syncthreads();
    t_dead = s_dead[0];
    t_rdead = s_rdead[0];
#pragma unroll
    for (int w2 = 1; w2 < NWG; ++w2) {
      t_dead = min(t_dead, s_dead[w2]);
      t_rdead = max(t_rdead, s_rdead[w2]);
    }
  }

  // Exponent of one score (log2 units) for the variants, from the plain
  // content score s = q.k and the signed distance pi - j (an exact integer).
  // POLY (soft cap, tiles whose every |A| <= z / 4): z tanh(A / z) from a
  // polynomial instead of an exponential and a reciprocal.
  auto variant_a = [&](float s, auto poly_tag) {
    constexpr bool POLY = decltype(poly_tag)::value;
    if constexpr ((VAR & kVarSoftcap) != 0 && POLY) {
      const float u = s * s;
      return s * fmaf(fmaf(var.cap_q[2], u, var.cap_q[1]), u, var.cap_q[0]);
    } else if constexpr ((VAR & kVarSoftcap) != 0) {
      // z tanh(A / z) = z (1 - 2 / (e^(2 A / z) + 1)); saturates to +-z
      const float e2 = fast_exp2(s * var.cap_in);
      return var.cap_out * fmaf(-2.0f, __builtin_amdgcn_rcpf(e2 + 1.0f), 1.0f);
    } else {
      return s * c1;
    }
  };
  // The soft-capped score plus B (the bias minus the row's reference
  // maximum), the polynomial's last product fused with the addition.
  auto variant_rel = [&](float s, float bb, auto poly_tag) {
    constexpr bool POLY = decltype(poly_tag)::value;
    if constexpr (POLY) {
      const float u = s * s;
      return fmaf(s, fmaf(fmaf(var.cap_q[2], u, var.cap_q[1]), u, var.cap_q[0]), bb);
    } else {
      const float e2 = fast_exp2(s * var.cap_in);
      return fmaf(var.cap_out, fmaf(-2.0f, __builtin_amdgcn_rcpf(e2 + 1.0f), 1.0f), bb);
    }
  };
  auto variant_t = [&](float s, float dist, auto poly_tag) {
    const float a = variant_a(s, poly_tag);
    const float dd = CAUSAL ? dist : fabsf(dist);
    float b;
    if constexpr ((VAR & kVarLog) != 0) {
      b = -mh * __builtin_amdgcn_logf(dd + 1.0f);  // -m ln(D + 1) log2(e) = -m log2(D + 1)
    } else {
      b = -c2 * dd;
    }
    if constexpr ((VAR & kVarClamp) != 0) b = fmaxf(b, var.clamp2);
    return a + b;
  };

  // One tile: S^T = K Q^T, online softmax, O^T += V^T P^T, and the LDS stores
  // of the next tile (whose global loads were issued at the top). MASKED tiles
  // may hold keys past a query or past Nk; the others hold none for any wave.
  int stage = 0;
  // kind 0: tile needing the mask (or past Nk); 1: every key at or before
  // every query; 2 (no causal mask only): every key at or after every query.
  auto step = [&](int tile, int next, auto kind_tag) {
    constexpr int KIND = decltype(kind_tag)::value;
    constexpr bool MASKED = KIND == 0;
    constexpr bool RIGHT = KIND == 2;
    const int j0 = tile * BN;
    // Stage `stage` holds this tile; every wave is done with the other stage.
    __syncthreads();
    if (next >= 0) regs.load(rk, rv, uint32_t(next) * (BN * D * 2), koff, voff);  // in flight during this tile
    const unsigned char* sK = smem + stage * STAGE;
    const unsigned char* sV = sK + KBYTES;
    unsigned char* const sKn = smem + (stage ^ 1) * STAGE;
    stage ^= 1;
    if ((MASKED && !(qw0 < Nq && (!CAUSAL || j0 <= qw_last + delta))) || ((EXT || !MASKED) && tile <= t_dead_wave) ||
        (EXT && !CAUSAL && tile >= t_rdead_wave)) {
      regs.template store<KPITCH, VPITCH>(sKn, sKn + KBYTES, tid);
      return;
    }

    // Clamp-only causal variant, per wave and open tile: 0 = every bias lies
    // above the floor (the plain linear bias: seeded scores, as VAR = 0),
    // 1 = every bias is floored (one constant), 2 = the floor starts inside
    // the tile (per score). Only class 0 seeds the scores. The bias is linear
    // in the distance, so its extremes over the tile sit at the two extreme
    // distances (whatever the slope's sign).
    int cls = 2;
    if constexpr (SEED && VAR != 0) {
      if (!MASKED) {
        const float bf = -c2 * float(qw_last + delta - j0), bn = -c2 * float(qw0 + delta - (j0 + BN - 1));
        if (fminf(bf, bn) >= var.clamp2) cls = 0;
        else if (fmaxf(bf, bn) <= var.clamp2) cls = 1;
      }
    }

    // Log-distance open tiles left of the queries: every distance of the tile
    // is D = base + e - k >= 0 with base = qw0 + delta - j0 (>= 63 here),
    // e = l32 - 4 hi in [-4, 31] and k = 32 kb + 8 (r / 4) + r % 4 in
    // [0, 59]: 95 values from Dlow = base - 63. Lane l computes the bias of
    // Dlow + l and Dlow + l + 64 once and writes them into the four copies
    // before the Q K^T products, which hide the writes; the lanes read back
    // their 32 biases as 8 aligned 16-byte reads afterwards (same wave: LDS
    // keeps the order of its accesses).
    if constexpr ((VAR & kVarLog) != 0 && KIND == 1) {
      float* const tb = ltab + wave_all * (4 * kTabPitch);
      const int dlow = qw0 + delta - j0 - 63;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int t = lane + 64 * h2;
        float bv = -mh * __builtin_amdgcn_logf(float(dlow + t) + 1.0f);
        if constexpr ((VAR & kVarClamp) != 0) bv = fmaxf(bv, var.clamp2);
#pragma unroll
        for (int a = 0; a < 4; ++a) tb[a * kTabPitch + 4 + t - a] = bv;
      }
    }

    // ---- S^T = K Q^T ----
    f32x16 s[KB];
    auto qk = [&](const f32x16& c0) {
      lds_mfma_ring<KS * KB, 4>(
          [&](int n) {
            return *reinterpret_cast<const bf16x8*>(sK + (32 * (n % KB) + l32) * KPITCH + (16 * (n / KB) + 8 * hi) * 2);
          },
          [&](int n, const bf16x8& a) {
            const int ks = n / KB, kb = n % KB;
            s[kb] = mfma32(a, qf[ks], ks == 0 ? c0 : s[kb]);
          });
    };
    if constexpr (VAR == 0) {
      qk(cinit);
    } else if constexpr (SEED) {
      if (cls == 0)
        qk(cinit);
      else
        qk(f32x16{});
    } else if constexpr (MSEED && !MASKED) {
      qk(mseed);
    } else {
      qk(cinit);
    }

    // ---- bias, mask, online softmax ----
    // Plain ALiBi: s = q.k + (c2 / c1)(8 (r / 4) + r % 4) and the exponent is
    // t = s c1 + c2 (j0 + 32 kb + 4 hi - pi). Variants: s becomes t itself.
    const float bt0 = c2 * float(j0 + 4 * hi - pi);
    const float bt1 = bt0 + 32.0f * c2;
    const float dpos = float(pi - j0 - 4 * hi);  // distance of register 0 of key block 0
    u32x4 pf[PS];
    // scale of s in the exponent: c1 where s is the (seeded) content score, 1
    // where the per-score variant path has already turned s into the exponent
    const float sc = (VAR == 0 || (SEED && cls != 2)) ? c1 : 1.0f;
    // p = exp2(s sc + bias_kb) packed to bf16 (the P^T B operand), with the
    // row sum taken from the same bf16 values.
    // Keys after the query (RIGHT) carry -c2 (j - pi): relative to the seed
    // this is the bias of the mirrored key minus 2 c2 (8 (r / 4) + r % 4).
    // NOADD: s already holds the exponent (the seeded log-distance tiles).
    auto exp_block_t = [&](float b0, float b1, auto noadd_tag) {
      constexpr bool NOADD = decltype(noadd_tag)::value;
      float lpart[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // independent partial row sums
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r0 = 8 * half + 2 * e;
            const float bb = kb ? b1 : b0;
            float bb0 = bb, bb1 = bb;
            if constexpr (RIGHT && VAR == 0) {
              bb0 = fmaf(-2.0f * c2, float(8 * (r0 >> 2) + (r0 & 3)), bb);
              bb1 = fmaf(-2.0f * c2, float(8 * (r0 >> 2) + (r0 & 3) + 1), bb);
            }
            if constexpr (NOADD)
              pk[e] = pack_bf16x2(fast_exp2(s[kb][r0]), fast_exp2(s[kb][r0 + 1]));
            else
              pk[e] = pack_bf16x2(fast_exp2(fmaf(s[kb][r0], sc, bb0)), fast_exp2(fmaf(s[kb][r0 + 1], sc, bb1)));
            lpart[e] = bdot2(pk[e], lpart[e]);
          }
          pf[2 * kb + half] = pk;
        }
      }
      return (lpart[0] + lpart[1]) + (lpart[2] + lpart[3]);
    };
    auto exp_block = [&](float b0, float b1) { return exp_block_t(b0, b1, std::false_type{}); };
    // Lazy rescale: the running maximum moves only when a row's candidate
    // exceeds it by more than 2^kLazy.
    auto rescale = [&](float mcand) {
      const bool need = mcand > m_run + kLazy;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mcand : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m_run = m_new;
        if constexpr (MSEED) {
          m_seed = m_run == kNegInf ? 0.0f : m_run;
          const float sv = -m_seed * rc1;
#pragma unroll
          for (int r = 0; r < 16; ++r) mseed[r] = sv;
        }
      }
    };
    float lsum;
    if constexpr (VAR != 0 && !MASKED) {
      // Open tiles of the variants. Every key is visible and the tiles go
      // from the diagonal outwards, so, as in the plain path below, the
      // exponent is taken against the running maximum directly and the bound
      // and the rescale follow only when a lane's partial row sum leaves
      // (0, kOptLimit]: the row maximum of the tile is never formed otherwise.
      // Clamp-only tiles of class 0 (seeded, linear bias) and 1 (content
      // score, one constant bias) keep their scores; the others turn s into
      // the exponent per score. One rescale site (with two, the compiler
      // copies the accumulators between the paths on every tile).
      float a0 = 0.0f, a1 = 0.0f;
      bool per_score = true;
      if constexpr (SEED) {
        if (cls != 2) {
          per_score = false;
          a0 = cls == 1 ? var.clamp2 : bt0;
          a1 = cls == 1 ? var.clamp2 : bt1;
        }
      }
      // the maximum the per-score exponents of CAPREL tiles are taken against
      // (0 for a row without one yet, which then takes the bound below)
      const float mref = CAPREL ? (m_run == kNegInf ? 0.0f : m_run) : 0.0f;
      if (per_score) {
        auto per_score_t = [&](auto poly_tag) {
          if constexpr ((VAR & kVarLog) != 0 && !RIGHT) {
            // the table written before the Q K^T products
            const float* const tb = ltab + wave_all * (4 * kTabPitch);
            const int cls4 = l32 & 3, e = l32 - 4 * hi;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                // strip entries start .. start + 3 hold D_first - 3 .. D_first
                const int start = e - 8 * g - 32 * kb + 60;
                const f32x4 bv = *reinterpret_cast<const f32x4*>(tb + cls4 * kTabPitch + 4 + start - cls4);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const int r = 4 * g + 3 - q;
                  if constexpr (CAPREL)
                    s[kb][r] = variant_rel(s[kb][r], bv[q] - mref, poly_tag);
                  else
                    s[kb][r] = variant_a(s[kb][r], poly_tag) + bv[q];
                }
              }
            }
          } else if constexpr (CAPREL && (VAR & kVarLog) != 0) {
            // log-scaled distances right of the queries (no causal mask)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const float dd = fabsf(dpos - float(32 * kb + 8 * (r >> 2) + (r & 3)));
                float bb = -mh * __builtin_amdgcn_logf(dd + 1.0f);
                if constexpr ((VAR & kVarClamp) != 0) bb = fmaxf(bb, var.clamp2);
                s[kb][r] = variant_rel(s[kb][r], bb - mref, poly_tag);
              }
            }
          } else if constexpr (CAPREL) {
            // linear bias -c2 |dpos - k| for key offset k: c2 (k - dpos) left
            // of the queries, c2 (dpos - k) right of them (no causal mask)
            const float sg = RIGHT ? -c2 : c2;
            const float base = (RIGHT ? c2 : -c2) * dpos - mref;
            const float floor_rel = var.clamp2 - mref;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                float bb = fmaf(sg, float(32 * kb + 8 * (r >> 2) + (r & 3)), base);
                if constexpr ((VAR & kVarClamp) != 0) bb = fmaxf(bb, floor_rel);
                s[kb][r] = variant_rel(s[kb][r], bb, poly_tag);
              }
            }
          } else {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                s[kb][r] = variant_t(s[kb][r], dpos - float(32 * kb + 8 * (r >> 2) + (r & 3)), poly_tag);
            }
          }
        };
        bool poly = false;
        if constexpr ((VAR & kVarSoftcap) != 0) {
          // the polynomial soft cap when every content logit of the tile has
          // |A| <= z / 4 (a NaN or infinity takes the exact form)
          const float amax = fmaxf(absmax16(s[0]), absmax16(s[1]));
          poly = __builtin_amdgcn_ballot_w64(!(amax <= var.cap_small)) == 0;
        }
        if (poly)
          per_score_t(std::true_type{});
        else
          per_score_t(std::false_type{});
      }
      if constexpr (REL) {
        // s = t - m_ref (m_seed, or mref): taken as it is; a row without a
        // maximum yet (0 stands in for it) goes through the bound like an
        // overflow
        const float ms = MSEED ? m_seed : mref;
        lsum = exp_block_t(0.0f, 0.0f, std::true_type{});
        if (__builtin_amdgcn_ballot_w64(!(lsum <= kOptLimit) || m_run == kNegInf)) {
          rescale(max_xor32(fmaxf(max16(s[0]), max16(s[1]))) + ms);
          lsum = exp_block(ms - m_run, ms - m_run);
        }
      } else {
        lsum = exp_block(a0 - m_run, a1 - m_run);
        if (__builtin_amdgcn_ballot_w64(!(lsum <= kOptLimit))) {
          rescale(max_xor32(fmaxf(fmaf(max16(s[0]), sc, a0), fmaf(max16(s[1]), sc, a1))));
          lsum = exp_block(a0 - m_run, a1 - m_run);
        }
      }
    } else if (VAR == 0 && !MASKED) {
      // Every key is visible and tiles go from the diagonal outwards, so the
      // running maximum is almost always already above this tile's scores:
      // exponentiate against it directly. A lane whose partial row sum leaves
      // (0, kOptLimit] (a score above the maximum by ~2^11, an overflow, or a
      // row without a finite maximum yet) sends the wave through the bound and
      // the rescale, and the tile is redone. Right of the queries the bias of
      // block kb is at most -bt_kb (its first key), left of them at most bt_kb
      // + 31 c2, which the seed already carries.
      const float a0 = RIGHT ? -bt0 : bt0, a1 = RIGHT ? -bt1 : bt1;
      lsum = exp_block(a0 - m_run, a1 - m_run);
      if (__builtin_amdgcn_ballot_w64(!(lsum <= kOptLimit))) {
        rescale(max_xor32(fmaxf(fmaf(max16(s[0]), c1, a0), fmaf(max16(s[1]), c1, a1))));
        lsum = exp_block(a0 - m_run, a1 - m_run);
      }
    } else {
      float mcand;
      if (VAR == 0 && !MASKED) {
        // every key is visible: max16 of s bounds the row maximum
        mcand = max_xor32(fmaxf(fmaf(max16(s[0]), c1, bt0), fmaf(max16(s[1]), c1, bt1)));
      } else {
        // masked keys become -inf in s itself, so the exponent code is shared
        float tmax = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
            const int j = j0 + 4 * hi + off;
            float x;
            if constexpr (VAR == 0) {
              x = s[kb][r];
              if (!CAUSAL && j > pi) x -= 2.0f * c21 * float(j - pi);  // symmetric bias -m |i - j|
            } else {
              x = variant_t(s[kb][r], dpos - float(off), std::false_type{});
            }
            if (MASKED) x = (j < Nk && (!CAUSAL || j <= pi) && (!(EXT && CAUSAL && VAR == 0) || j > pi - wwin)) ? x : kNegInf;
            s[kb][r] = x;
            tmax = fmaxf(tmax, VAR == 0 ? fmaf(x, c1, kb ? bt1 : bt0) : x);
          }
        }
        mcand = max_xor32(tmax);
      }
      rescale(mcand);
      // m_run is finite after the first visible key; a row with none yet
      // (every key masked) keeps -inf and takes 0 here
      const float m_use = MASKED && m_run == kNegInf ? 0.0f : m_run;
      lsum = exp_block((VAR == 0 ? bt0 : 0.0f) - m_use, (VAR == 0 ? bt1 : 0.0f) - m_use);
    }
    l_run += lsum;

    // ---- O^T += V^T P^T, with the next tile's LDS stores in the same region ----
    lds_mfma_ring<DB * PS, 4>(
        [&](int n) {
          return *reinterpret_cast<const bf16x8*>(sV + (32 * (n / PS) + l32) * VPITCH + (16 * (n % PS) + 8 * hi) * 2);
        },
        [&](int n, const bf16x8& a) { o[n / PS] = mfma32(a, __builtin_bit_cast(bf16x8, pf[n % PS]), o[n / PS]); });
    // After the last tile the registers still hold tile 0, which nobody reads
    // again; storing it keeps this region free of branches.
    regs.template store<KPITCH, VPITCH>(sKn, sKn + KBYTES, tid);
  };

  // Tiles 0 .. t_open hold only keys at or before the block's first query
  // position q0 + delta (so before every wave's queries) and lie wholly below
  // Nk: no mask. The rest, at most (BM + BN - 1) / BN + 1 of them under the
  // causal mask, take the masked path; without the mask every tile does.
  using Masked = std::integral_constant<int, 0>;
  using Left = std::integral_constant<int, 1>;
  using Right = std::integral_constant<int, 2>;
  const int x = q0 + delta + 1;  // keys [0, x) are at or before every query of the block
  if (CAUSAL) {
    const int t_open = x < BN ? -1 : min(min(x / BN - 1, Nk / BN - 1), ntiles - 1);
    // With the key range split, group g takes every SPLIT-th tile from
    // ntiles - 1 - g down to min(t_open, t_dead) + 1; group 1 has one tile
    // fewer when that range has an odd length and meets group 0's last barrier
    // without a tile.
    int tile = ntiles - 1 - grp;
    for (; tile > t_open; tile -= SPLIT) step(tile, tile - SPLIT, Masked{});
    if constexpr (EXT && VAR == 0) {
      // open tiles wholly inside every row's window, then the window's edge
      const int t_lo = max(t_dead, t_wmask);
      for (; tile > t_lo; tile -= SPLIT) step(tile, tile - SPLIT, Left{});
      for (; tile > t_dead; tile -= SPLIT) step(tile, tile - SPLIT, Masked{});
    } else {
      for (; tile > t_dead; tile -= SPLIT) step(tile, tile - SPLIT, Left{});
    }
    if (SPLIT == 2 && grp == 1 && ((ntiles - 1 - min(t_open, t_dead)) & 1)) __syncthreads();
  } else {
    // Without the mask: the tiles around the diagonal and a partial last tile
    // first (masked path), then the tiles wholly after the block's queries
    // nearest first, then those wholly before them nearest first, so the
    // running maximum is set early and the bias only falls afterwards.
    const int nfull = Nk / BN;
    const int tl = x < BN ? -1 : min(x / BN - 1, nfull - 1);   // left tiles 0 .. tl
    const int ql = q0 + BM - 1 + delta;                          // last query position of the block
    const int tr = max(tl + 1, ql <= 0 ? 0 : (ql + BN - 1) / BN);  // right tiles tr .. nfull - 1
    const int mid_hi = min(tr, nfull) - 1;                        // middle tiles tl + 1 .. mid_hi
    // exact skipping: the right tiles end before t_rdead, the left ones after t_dead
    const int r_end = min(nfull, max(t_rdead, tr));
    const int after_mid = tr < r_end ? tr : tl;
    if (Nk % BN != 0) step(nfull, mid_hi > tl ? mid_hi : after_mid, Masked{});
    for (int t = mid_hi; t > tl; --t) step(t, t - 1 > tl ? t - 1 : after_mid, Masked{});
    for (int t = tr; t < r_end; ++t) step(t, t + 1 < r_end ? t + 1 : tl, Right{});
    for (int t = tl; t > t_dead; --t) step(t, t - 1, Left{});
  }

  if constexpr (SPLIT == 2) {
    // Merge the two key groups' states of each row: wave w + 4 hands its
    // lanes' (m, l, O) to wave w, which owns the same rows in the same lane
    // layout. A group that saw no key of a row has m = -inf and weighs 0.
    constexpr int NV = 16 * DB + 2;  // floats per lane
    static_assert(NWG * NV * 64 * 4 <= SPLIT * 2 * STAGE, "hand-over fits in the stages");
    float* const xs = reinterpret_cast<float*>(smem_all) + wave * NV * 64 + lane;
    __syncthreads();  // every wave is done with its stages
    if (grp == 1) {
      xs[0] = m_run;
      xs[64] = l_run;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[(2 + 16 * db + r) * 64] = o[db][r];
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xs[0], l1 = xs[64];
    const float mm = fmaxf(m_run, m1);
    const float a0 = m_run == kNegInf ? 0.0f : fast_exp2(m_run - mm);
    const float a1 = m1 == kNegInf ? 0.0f : fast_exp2(m1 - mm);
    l_run = fmaf(l_run, a0, l1 * a1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = fmaf(o[db][r], a0, xs[(2 + 16 * db + r) * 64] * a1);
    m_run = mm;
  }

  // ---- epilogue: O / l -> bf16; a row that saw no key gives 0 ----
  const float lt = sum_xor32(l_run);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (EXT && var.lse != nullptr && i < Nq && hi == 0)
    var.lse[(long long)bh * Nq + i] = lt > 0.0f ? (m_run + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
  if (i < Nq) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 st;
        st[0] = pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
        st[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(out + qbase + (long long)i * D + 32 * db + 8 * g + 4 * hi) = st;
      }
    }
  }
}

template <int D, int NW, bool CAUSAL, int VAR, bool EXT, int SPLIT = 1>
hipError_t launch_cfg(const FwdArgs& a, float c1, const FwdVariant& var, hipStream_t stream) {
  constexpr int BM = NW / SPLIT * 32;
  const int nqb = (a.Nq + BM - 1) / BM;
  const long long total = (long long)a.B * a.H * nqb;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, NW, CAUSAL, VAR, EXT, SPLIT>), dim3(unsigned(total)), dim3(NW * 64), 0,
                     stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.out, a.H, a.Nq, a.Nk, nqb, int(total), a.slopes, c1, var);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int NW>
hipError_t launch_var_nw(const FwdArgs& a, int flags, bool ext, float c1, const FwdVariant& var, hipStream_t s) {
  switch (flags) {
    case 0:
      return ext ? launch_cfg<D, NW, CAUSAL, 0, true>(a, c1, var, s)
                 : launch_cfg<D, NW, CAUSAL, 0, false>(a, c1, var, s);
    case 1: return launch_cfg<D, NW, CAUSAL, 1, true>(a, c1, var, s);
    case 2: return launch_cfg<D, NW, CAUSAL, 2, true>(a, c1, var, s);
    case 3: return launch_cfg<D, NW, CAUSAL, 3, true>(a, c1, var, s);
    case 4: return launch_cfg<D, NW, CAUSAL, 4, true>(a, c1, var, s);
    case 5: return launch_cfg<D, NW, CAUSAL, 5, true>(a, c1, var, s);
    case 6: return launch_cfg<D, NW, CAUSAL, 6, true>(a, c1, var, s);
    default: return launch_cfg<D, NW, CAUSAL, 7, true>(a, c1, var, s);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_var(const FwdArgs& a, int flags, bool ext, float c1, const FwdVariant& var, hipStream_t s) {
  if constexpr (CAUSAL) {
    if (fwd_split(a, flags, var.delta))
      return ext ? launch_cfg<D, 8, true, 0, true, 2>(a, c1, var, s) : launch_cfg<D, 8, true, 0, false, 2>(a, c1, var, s);
  }
  return fwd_waves(a, flags) == 4 ? launch_var_nw<D, CAUSAL, 4>(a, flags, ext, c1, var, s)
                                  : launch_var_nw<D, CAUSAL, 8>(a, flags, ext, c1, var, s);
}

}  // namespace

void set_fwd_waves(int nw) { waves_override().store(nw, std::memory_order_relaxed); }

int fwd_mfma_form(const FwdArgs& a, int flags, int delta) {
  if (fwd_split(a, flags & 7, delta)) return 2;
  return fwd_waves(a, flags & 7);
}
void set_fwd_split(int mode) { split_override().store(mode, std::memory_order_relaxed); }

hipError_t launch_fwd_mfma(const FwdArgs& a, const FwdOptions& opt, float c1, hipStream_t stream) {
  FwdVariant var;
  var.delta = opt.q_offset - opt.k_offset;
  var.clamp2 = opt.clamp_min * kLog2e;
  const double z = opt.softcap > 0.0f ? double(opt.softcap) : 1.0;
  var.cap_in = float(2.0 * double(c1) / z);
  var.cap_out = float(z * 1.4426950408889634);
  // tanh(y) / y ~ p0 + p1 y^2 + p2 y^4 on |y| <= 1/4: a weighted
  // least-squares (Lawson) fit for the relative error, 4.0e-7 at most there
  // (4.5e-7 evaluated in fp32); A / z = s / (sqrt(d) z) = s c1 / (z log2(e)).
  // In s itself (y = s ycoef): z log2(e) tanh(y) = s sum_i q_i s^(2i) with
  // q_i = z log2(e) p_i ycoef^(2i + 1).
  const double ycoef = double(c1) / 1.4426950408889634 / z;
  var.cap_small = float(0.25 / ycoef * (1.0 - 1e-6));
  const double pc[3] = {0.9999996043367838, -0.3332190807322682, 0.1284161017710369};
  for (int i = 0; i < 3; ++i) var.cap_q[i] = float(pc[i] * z * 1.4426950408889634 * std::pow(ycoef, 2 * i + 1));
  var.knorm = opt.knorm;
  var.parts = opt.knorm_parts;
  var.lse = opt.lse;
  var.window = opt.window;
  const int flags = opt.flags & 7;  // the mitigation bits; skipping and the window are run-time arguments
  const bool ext = var.delta != 0 || var.knorm != nullptr || var.lse != nullptr || var.window != nullptr;
  if (a.d == 128)
    return a.causal ? launch_var<128, true>(a, flags, ext, c1, var, stream)
                    : launch_var<128, false>(a, flags, ext, c1, var, stream);
  return a.causal ? launch_var<64, true>(a, flags, ext, c1, var, stream)
                  : launch_var<64, false>(a, flags, ext, c1, var, stream);
}

}  // namespace alibi
