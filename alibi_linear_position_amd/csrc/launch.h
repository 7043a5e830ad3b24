// Host-side launchers of the device kernels (internal to the library; the
// public C ABI is include/alibi.h). Each returns hipGetLastError() after the
// launch. Callers have validated every size and pointer.
#pragma once

#include <hip/hip_runtime.h>

namespace alibi {

hipError_t launch_weights_f32(const float* q, const float* k, float* w, int B, int H, int N, int d,
                              const float* slopes, int causal, float c1, hipStream_t stream);

// One forward call: q/out (B, H, Nq, d), k/v (B, H, Nk, d), device pointers.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int B, H, Nq, Nk, d;
  const float* slopes;
  int causal;
};

// Mitigations and positions (validated by the caller): flags are the
// ALIBI_CLAMP / ALIBI_LOG_DISTANCE / ALIBI_SOFTCAP bits; query row r sits at
// position q_offset + r and key row c at k_offset + c.
struct FwdOptions {
  int flags = 0;
  float clamp_min = 0.0f;
  float softcap = 0.0f;
  int q_offset = 0;
  int k_offset = 0;
  // exact underflow skipping: P partial maxima of the key norms per (b, h)
  // (launch_knorm_max), or null for no skipping
  const float* knorm = nullptr;
  int knorm_parts = 0;
  // optional output: row log-sum-exp of the logits (natural log), (B, H, Nq)
  float* lse = nullptr;
  // optional per-head hard window (device, H ints; causal form only): query i
  // sees key j when 0 <= pi - j < window[h]
  const int* window = nullptr;
};

// One backward call (bf16 tensors (B, H, N, d), lse fp32 (B, H, N)).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d;
  const float* slopes;
  int causal;
  int flags = 0;         // ALIBI_CLAMP | ALIBI_LOG_DISTANCE | ALIBI_SOFTCAP
  float clamp2 = 0.0f;   // bias floor in log2 units (ALIBI_CLAMP)
  // soft cap z (ALIBI_SOFTCAP): exp2(s cap_in) = e^(2 A / z) for the raw score
  // s = q.k, and the capped logit z tanh(A / z) in log2 units is cap_out tanh(A / z)
  float cap_in = 0.0f;
  float cap_out = 0.0f;
  // exact underflow skipping (plain form): P partial maxima of the key
  // norms of every (b, h), then those of the query norms (launch_knorm_max),
  // or null for no skipping
  const float* norms = nullptr;
  int norm_parts = 0;
};

// Backward, d in {64, 128}; ws holds 2 B H N floats (D and lse in log2 units).
hipError_t launch_bwd(const BwdArgs& a, float* ws, float c1, hipStream_t stream);
// 32-row query blocks per dK/dV step: 0 = automatic (the default: 2), 1 or 2.
void set_bwd_query_blocks(int qb);

// Generic (VALU) forward, any d <= 256: fp32 (f32 = true) or bf16 data.
hipError_t launch_fwd_generic(const FwdArgs& a, const FwdOptions& opt, bool f32, hipStream_t stream);

// MFMA forward, bf16, d in {64, 128}.
// Waves per forward workgroup: 0 = automatic (the default), 4 or 8 = forced.
void set_fwd_waves(int nw);
// Key-range split of the plain causal forward: 0 = automatic (the default),
// 1 = never, 2 = always.
void set_fwd_split(int mode);
// The form the MFMA forward launches for these arguments: 4 or 8 = waves per
// workgroup over the whole key range, 2 = the key-range split (8 waves).
int fwd_mfma_form(const FwdArgs& a, int flags, int delta);
hipError_t launch_fwd_mfma(const FwdArgs& a, const FwdOptions& opt, float c1, hipStream_t stream);

// Largest key norm of each (b, h) of k (B, H, N, d) bf16, d in {64, 128}, as P
// partial maxima: out[(b H + h) P + p].
// Streaming read of `bytes` (a multiple of 16) from buf, one XOR word per workgroup to sink.
hipError_t launch_stream_read(const void* buf, long long bytes, uint32_t* sink, int workgroups, hipStream_t stream);
// Back-to-back register-fed bf16 MFMAs: 8-wave workgroups, each wave `iters`
// rounds of 16 v_mfma_f32_32x32x16_bf16 on the 8 operand fragments at frags
// (8 x 64 lanes x 16 bytes), its accumulator sum to sink[workgroup * 8 + wave];
// valu adds the forward's per-MFMA vector work beside every MFMA.
hipError_t launch_mfma_rate(const void* frags, int iters, bool valu, float* sink, int workgroups,
                            hipStream_t stream);
hipError_t launch_knorm_max(const void* k, float* out, int B, int H, int N, int d, int P,
                            hipStream_t stream);
// out[i] = max over p of part[i P + p], i < n.
hipError_t launch_knorm_reduce(const float* part, float* out, long long n, int P, hipStream_t stream);

// Split-KV decode. `splits` key ranges of `chunk` keys each; ws holds
// B*H*splits*(d+2) floats when splits > 1 (may be null when splits == 1).
// knorm: null, or B*H upper bounds of the key norms for exact underflow
// skipping.
hipError_t launch_decode(const void* q, const void* kc, const void* vc, void* out, float* ws,
                         int B, int H, int L, int d, int splits, int chunk,
                         const float* slopes, float c1, const float* knorm, hipStream_t stream);

// Number of splits and keys per split the decode launcher will use.
void decode_plan(int B, int H, int L, int d, int* splits, int* chunk);

// The current device's file-scope decode scratch (a device address) and its
// size in bytes; resolved once per device. Allocates nothing.
hipError_t decode_scratch(float** ptr, size_t* bytes);

}  // namespace alibi
