// Device helpers shared by the gfx950 ALiBi kernels: bf16 bit conversions,
// wave64 reductions and the constants of the log2-domain softmax.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace alibi {

// exp(x) = exp2(x * log2(e)); the kernels carry scores in log2 units so that the
// hardware exp2 (v_exp_f32) is the only transcendental.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return uint16_t(pack_bf16x2(x, 0.0f) & 0xffffu);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// NF MFMAs whose A operands come from LDS: fragment n is read DEPTH MFMAs
// ahead of its use and the order is pinned (sched_barrier), so several reads
// stay in flight; left to itself the scheduler keeps one or two, and a wave
// whose SIMD partner is not issuing MFMAs then waits on LDS latency before
// most of them. frag(n) reads fragment n; op(n, a) issues MFMA n.
template <int NF, int DEPTH, typename Frag, typename Op>
__device__ __forceinline__ void lds_mfma_ring(Frag&& frag, Op&& op) {
  static_assert(NF >= DEPTH, "the prologue reads DEPTH fragments");
  bf16x8 ring[DEPTH];
#pragma unroll
  for (int n = 0; n < DEPTH; ++n) ring[n] = frag(n);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < NF; ++n) {
    const bf16x8 a = ring[n % DEPTH];
    if (n + DEPTH < NF) ring[n % DEPTH] = frag(n + DEPTH);
    op(n, a);
    __builtin_amdgcn_sched_barrier(0);
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Workgroup w -> ((b, h) pair, block rank) for nbh pairs of nblk blocks each.
// Workgroups are dealt round-robin to the 8 XCDs (w % 8). With nbh a multiple
// of 8 every XCD gets whole (b, h) pairs, so a head's K and V stay in that
// XCD's L2, and walks them in groups of kSchedGroup pairs, rank by rank inside
// a group: rank 0 (the caller's heaviest block) of the group's pairs first.
// Few pairs in flight keep the XCD's L2 on their K and V, and rank order keeps
// heavy blocks from starting late. Otherwise ranks go in order over all pairs.
// Host and device: the host side is checked to be a bijection.
constexpr int kSchedGroup = 4;
struct WgBlock {
  int bh;
  int rank;
};
__host__ __device__ inline WgBlock schedule_block(int w, int nbh, int nblk) {
  if ((nbh & 7) == 0) {
    const int per = nbh >> 3;  // pairs per XCD
    const int x = w >> 3;      // position in this XCD's queue, 0 .. per * nblk - 1
    const int G = per < kSchedGroup ? per : kSchedGroup;
    const int full = per / G;  // complete groups of G pairs
    const int span = G * nblk;
    int g, gsize, in;
    if (x < full * span) {
      g = x / span;
      gsize = G;
      in = x - g * span;
    } else {  // the last, smaller group
      g = full;
      gsize = per - full * G;
      in = x - full * span;
    }
    return {(w & 7) * per + g * G + in % gsize, in / gsize};
  }
  return {w % nbh, w / nbh};
}

// Butterfly reductions over the full 64-lane wave.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// Reductions inside aligned groups of G lanes (G = 1, 2, 4, 8, 16, 32).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace alibi
