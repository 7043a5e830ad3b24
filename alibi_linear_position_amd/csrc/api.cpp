// C-ABI entry points of libalibi (declared in include/alibi.h): argument
// validation, the host slope generator, kernel selection and the per-device
// decode workspace. Validation touches no HIP API, so argument errors are
// reported identically on machines without a GPU.
#include "alibi.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "launch.h"
#include "device_common.h"

namespace {

constexpr int kMaxLen = 1 << 24;  // token distances stay exact in fp32

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("ALIBI_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

// Softmax scale in log2 units: log2(e) / sqrt(d), evaluated in double.
float scale_log2(int d) { return float(1.4426950408889634 / std::sqrt(double(d))); }

int check_common(const void* a, const void* b, const void* c, const void* out, const float* slopes,
                 int B, int H, int N, int d, uintptr_t align) {
  if (!a || !b || !c || !out || !slopes) return ALIBI_EINVAL;
  if (B < 1 || H < 1 || N < 1 || d < 1 || N > kMaxLen) return ALIBI_EINVAL;
  if (!aligned(a, align) || !aligned(b, align) || !aligned(c, align) || !aligned(out, align))
    return ALIBI_EINVAL;
  if (!aligned(slopes, 4)) return ALIBI_EINVAL;
  // grid sizes: one wave per row (generic) or per (b, h, block) -- keep them in 32 bits
  if ((long long)B * H * N > (1LL << 31) * 4) return ALIBI_ENOTSUP;
  return ALIBI_OK;
}

// Validation of a forward call; fills *opt from opts (NULL = defaults).
int check_fwd(const void* q, const void* k, const void* v, const void* out, const float* slopes,
              int B, int H, int Nq, int Nk, int d, int causal, const alibi_fwd_opts* opts,
              uintptr_t align, alibi::FwdOptions* opt) {
  int st = check_common(q, k, v, out, slopes, B, H, Nq, d, align);
  if (st != ALIBI_OK) return st;
  if (Nk < 1 || Nk > kMaxLen) return ALIBI_EINVAL;
  if (causal != 0 && causal != 1) return ALIBI_EINVAL;
  *opt = alibi::FwdOptions{};
  if (opts != nullptr) {
    if ((opts->flags & ~(ALIBI_CLAMP | ALIBI_LOG_DISTANCE | ALIBI_SOFTCAP | ALIBI_SKIP_UNDERFLOW | ALIBI_WINDOW)) != 0)
      return ALIBI_EINVAL;
    if ((opts->flags & ALIBI_CLAMP) && !std::isfinite(opts->clamp_min)) return ALIBI_EINVAL;
    if ((opts->flags & ALIBI_SOFTCAP) && !(std::isfinite(opts->softcap) && opts->softcap > 0.0f))
      return ALIBI_EINVAL;
    if (opts->q_offset < 0 || opts->q_offset > kMaxLen || opts->k_offset < 0 || opts->k_offset > kMaxLen)
      return ALIBI_EINVAL;
    opt->flags = opts->flags;
    opt->clamp_min = opts->clamp_min;
    opt->softcap = opts->softcap;
    opt->q_offset = opts->q_offset;
    opt->k_offset = opts->k_offset;
    if (opts->lse != nullptr && !aligned(opts->lse, 4)) return ALIBI_EINVAL;
    opt->lse = opts->lse;
    if (opts->flags & ALIBI_WINDOW) {
      if (opts->window == nullptr || !aligned(opts->window, 4)) return ALIBI_EINVAL;
      if (!causal || (opts->flags & (ALIBI_CLAMP | ALIBI_LOG_DISTANCE | ALIBI_SOFTCAP)) != 0)
        return ALIBI_ENOTSUP;
      opt->window = opts->window;
    }
  }
  if ((long long)B * H * Nk > (1LL << 31) * 4) return ALIBI_ENOTSUP;
  return ALIBI_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ALIBI_OK : ALIBI_EHIP; }

// ---- library workspaces: growable buffers per device ----
// kDecode holds the decode's partial softmax states, kNorm the key-norm maxima
// of the skipping forward, kBwd the backward's row terms (and its norm maxima when it skips). All are used asynchronously on the caller's stream.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
enum { kDecode = 0, kNorm = 1, kBwd = 2, kNumWorkspaces = 3 };
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws[kNumWorkspaces];
// Test hook (alibi_debug_fail_allocations): workspace requests left to fail.
std::atomic<int> g_fail_allocs{0};

int workspace_get(int which, size_t bytes, float** out) {
  for (int n = g_fail_allocs.load(); n > 0;)
    if (g_fail_allocs.compare_exchange_weak(n, n - 1)) return ALIBI_ENOMEM;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ALIBI_EHIP;
  std::vector<Workspace>& list = g_ws[which];
  if ((size_t)dev >= list.size()) list.resize(dev + 1);
  Workspace& w = list[dev];
  if (w.bytes < bytes) {
    if (w.ptr) {
      // an earlier asynchronous call may still read the old buffer
      if (hipDeviceSynchronize() != hipSuccess) return ALIBI_EHIP;
      if (hipFree(w.ptr) != hipSuccess) return ALIBI_EHIP;
      w.ptr = nullptr;
      w.bytes = 0;
    }
    if (hipMalloc(&w.ptr, bytes) != hipSuccess) {
      w.ptr = nullptr;
      (void)hipGetLastError();
      return ALIBI_ENOMEM;
    }
    w.bytes = bytes;
  }
  *out = static_cast<float*>(w.ptr);
  return ALIBI_OK;
}

// Validation shared by the decode entry points.
int check_decode(const void* q, const void* kcache, const void* vcache, const void* out, const float* slopes,
                 int B, int H, int L, int d) {
  const int st = check_common(q, kcache, vcache, out, slopes, B, H, L, d, 16);
  if (st != ALIBI_OK) return st;
  if (d > 256 || d % 8 != 0) return ALIBI_ENOTSUP;
  return ALIBI_OK;
}

// Bytes of partial softmax states the decode needs for this shape: 0 when a
// (b, h) is not split across workgroups.
size_t decode_ws_bytes(int B, int H, int L, int d) {
  int splits = 1, chunk = L;
  alibi::decode_plan(B, H, L, d, &splits, &chunk);
  return splits > 1 ? (size_t)B * H * splits * (d + 2) * sizeof(float) : 0;
}

int launch_decode_plan(const void* q, const void* kcache, const void* vcache, void* out, int B, int H, int L,
                       int d, const float* slopes, float* ws, hipStream_t stream, const float* knorm = nullptr) {
  int splits = 1, chunk = L;
  alibi::decode_plan(B, H, L, d, &splits, &chunk);
  if (log_enabled())
    std::fprintf(stderr, "[alibi] decode B=%d H=%d L=%d d=%d splits=%d chunk=%d skip=%d\n", B, H, L, d, splits, chunk,
                 int(knorm != nullptr));
  return hip_status(alibi::launch_decode(q, kcache, vcache, out, ws, B, H, L, d, splits, chunk, slopes,
                                         scale_log2(d), knorm, stream));
}

}  // namespace

extern "C" {

int alibi_slopes(int H, float* slopes_out) {
  if (H < 1 || slopes_out == nullptr) return ALIBI_EINVAL;
  auto pow2_schedule = [](int n, int h) { return std::exp2(-8.0 * double(h + 1) / double(n)); };
  int c = 1;
  while (c * 2 <= H) c *= 2;
  for (int h = 0; h < c; ++h) slopes_out[h] = float(pow2_schedule(c, h));
  for (int t = 0; t < H - c; ++t) slopes_out[c + t] = float(pow2_schedule(2 * c, 2 * t));
  return ALIBI_OK;
}

int alibi_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                   int d, const float* slopes, int causal, hipStream_t stream) {
  return alibi_attn_fwd_ex(q, k, v, out, B, H, N, N, d, slopes, causal, nullptr, stream);
}

int alibi_attn_fwd_f32(const float* q, const float* k, const float* v, float* out, int B, int H,
                       int N, int d, const float* slopes, int causal, hipStream_t stream) {
  return alibi_attn_fwd_ex_f32(q, k, v, out, B, H, N, N, d, slopes, causal, nullptr, stream);
}

int alibi_attn_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int H, int Nq,
                      int Nk, int d, const float* slopes, int causal, const alibi_fwd_opts* opts,
                      hipStream_t stream) {
  alibi::FwdOptions opt;
  int st = check_fwd(q, k, v, out, slopes, B, H, Nq, Nk, d, causal, opts, 16, &opt);
  if (st != ALIBI_OK) return st;
  if (d > 256 || d % 8 != 0) return ALIBI_ENOTSUP;
  const alibi::FwdArgs a{q, k, v, out, B, H, Nq, Nk, d, slopes, causal};
  if (d == 64 || d == 128) {
    // Exact underflow skipping applies to the plain form, causal or not;
    // elsewhere the flag changes nothing (skipping is exact, so ignoring it is too).
    const bool mitigated = (opt.flags & (ALIBI_CLAMP | ALIBI_LOG_DISTANCE | ALIBI_SOFTCAP)) != 0;
    if ((opt.flags & ALIBI_SKIP_UNDERFLOW) && !mitigated) {
      const int parts = std::max(1, std::min(std::max(1, Nk / 256), (2048 + B * H - 1) / (B * H)));
      float* ws = nullptr;
      {
        std::lock_guard<std::mutex> lock(g_ws_mutex);
        st = workspace_get(kNorm, (size_t)B * H * parts * sizeof(float), &ws);
      }
      if (st != ALIBI_OK) return st;
      st = hip_status(alibi::launch_knorm_max(k, ws, B, H, Nk, d, parts, stream));
      if (st != ALIBI_OK) return st;
      opt.knorm = ws;
      opt.knorm_parts = parts;
    }
    if (log_enabled())
      std::fprintf(stderr, "[alibi] fwd mfma B=%d H=%d Nq=%d Nk=%d d=%d causal=%d flags=%d offsets=%d,%d\n",
                   B, H, Nq, Nk, d, causal, opt.flags, opt.q_offset, opt.k_offset);
    return hip_status(alibi::launch_fwd_mfma(a, opt, scale_log2(d), stream));
  }
  if (log_enabled()) std::fprintf(stderr, "[alibi] fwd generic bf16 B=%d H=%d Nq=%d Nk=%d d=%d\n", B, H, Nq, Nk, d);
  return hip_status(alibi::launch_fwd_generic(a, opt, false, stream));
}

int alibi_attn_fwd_ex_f32(const float* q, const float* k, const float* v, float* out, int B, int H,
                          int Nq, int Nk, int d, const float* slopes, int causal,
                          const alibi_fwd_opts* opts, hipStream_t stream) {
  alibi::FwdOptions opt;
  int st = check_fwd(q, k, v, out, slopes, B, H, Nq, Nk, d, causal, opts, 4, &opt);
  if (st != ALIBI_OK) return st;
  if (d > 256) return ALIBI_ENOTSUP;
  const alibi::FwdArgs a{q, k, v, out, B, H, Nq, Nk, d, slopes, causal};
  return hip_status(alibi::launch_fwd_generic(a, opt, true, stream));
}

int alibi_attn_bwd_ex(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                      const float* slopes, int causal, const alibi_fwd_opts* opts, hipStream_t stream) {
  int st = check_common(q, k, v, out, slopes, B, H, N, d, 16);
  if (st != ALIBI_OK) return st;
  st = check_common(dout, dq, dk, dv, slopes, B, H, N, d, 16);
  if (st != ALIBI_OK) return st;
  if (lse == nullptr || !aligned(lse, 4)) return ALIBI_EINVAL;
  if (causal != 0 && causal != 1) return ALIBI_EINVAL;
  int flags = 0;
  float clamp_min = 0.0f, softcap = 0.0f;
  bool skip = false;
  if (opts != nullptr) {
    if ((opts->flags & ~(ALIBI_CLAMP | ALIBI_LOG_DISTANCE | ALIBI_SOFTCAP | ALIBI_SKIP_UNDERFLOW | ALIBI_WINDOW)) != 0)
      return ALIBI_EINVAL;
    if ((opts->flags & ALIBI_CLAMP) && !std::isfinite(opts->clamp_min)) return ALIBI_EINVAL;
    if ((opts->flags & ALIBI_SOFTCAP) && !(std::isfinite(opts->softcap) && opts->softcap > 0.0f))
      return ALIBI_EINVAL;
    // the window and position offsets are forward-only forms
    if ((opts->flags & ALIBI_WINDOW) != 0 || opts->q_offset != 0 || opts->k_offset != 0) return ALIBI_ENOTSUP;
    flags = opts->flags & (ALIBI_CLAMP | ALIBI_LOG_DISTANCE | ALIBI_SOFTCAP);
    clamp_min = opts->clamp_min;
    softcap = opts->softcap;
    skip = (opts->flags & ALIBI_SKIP_UNDERFLOW) != 0;
  }
  if (d != 64 && d != 128) return ALIBI_ENOTSUP;
  // Exact underflow skipping acts on the plain form, causal or not (with the
  // mitigations the flag changes nothing); its bound needs the largest query
  // and key norms per (b, h), kept as partial maxima behind the row terms in
  // the workspace.
  skip = skip && flags == 0;
  const long long bh = (long long)B * H;
  const int parts = skip ? int(std::max(1LL, std::min(std::max(1LL, (long long)N / 256), (2048 + bh - 1) / bh))) : 0;
  float* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    st = workspace_get(kBwd, ((size_t)2 * B * H * N + (size_t)2 * bh * parts) * sizeof(float), &ws);
  }
  if (st != ALIBI_OK) return st;
  if (log_enabled())
    std::fprintf(stderr, "[alibi] bwd B=%d H=%d N=%d d=%d causal=%d flags=%d skip=%d\n", B, H, N, d, causal, flags,
                 int(skip));
  alibi::BwdArgs a{q, k, v, out, dout, lse, dq, dk, dv, B, H, N, d, slopes, causal};
  a.flags = flags;
  a.clamp2 = clamp_min * 1.4426950408889634f;  // as the forward forms its floor (log2 units)
  if (flags & ALIBI_SOFTCAP) {                  // as the forward forms its cap
    a.cap_in = float(2.0 * double(scale_log2(d)) / double(softcap));
    a.cap_out = float(double(softcap) * 1.4426950408889634);
  }
  if (skip) {
    float* norms = ws + (size_t)2 * B * H * N;
    st = hip_status(alibi::launch_knorm_max(k, norms, B, H, N, d, parts, stream));
    if (st != ALIBI_OK) return st;
    st = hip_status(alibi::launch_knorm_max(q, norms + bh * parts, B, H, N, d, parts, stream));
    if (st != ALIBI_OK) return st;
    a.norms = norms;
    a.norm_parts = parts;
  }
  return hip_status(alibi::launch_bwd(a, ws, scale_log2(d), stream));
}

int alibi_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   const float* slopes, int causal, hipStream_t stream) {
  return alibi_attn_bwd_ex(q, k, v, out, dout, lse, dq, dk, dv, B, H, N, d, slopes, causal, nullptr, stream);
}

int alibi_slopes_recipe(int recipe, int H, int log_distance, float* slopes_out) {
  if (H < 1 || slopes_out == nullptr) return ALIBI_EINVAL;
  if (recipe == ALIBI_SLOPES_DEFAULT) return alibi_slopes(H, slopes_out);
  double lo = 0.0, hi = 0.0;
  switch (recipe) {
    case ALIBI_SLOPES_STEEP: lo = 128.0; hi = 512.0; break;
    case ALIBI_SLOPES_SAFE: lo = 2048.0; hi = 4096.0; break;
    case ALIBI_SLOPES_WIDE: lo = 16.0; hi = 4096.0; break;
    case ALIBI_SLOPES_EXPLICIT: break;
    default: return ALIBI_EINVAL;
  }
  const double tau = 126.0 * std::log(2.0);  // |ln 2^-126|
  for (int h = 0; h < H; ++h) {
    double delta;
    if (recipe == ALIBI_SLOPES_EXPLICIT)
      delta = 32.0 * std::exp2(double(h));
    else
      delta = H == 1 ? lo : lo * std::pow(hi / lo, double(h) / double(H - 1));
    slopes_out[h] = float(log_distance ? tau / std::log(delta + 1.0) : tau / delta);
  }
  return ALIBI_OK;
}

int alibi_attn_decode(const void* q, const void* kcache, const void* vcache, void* out, int B,
                      int H, int L, int d, const float* slopes, hipStream_t stream) {
  int st = check_decode(q, kcache, vcache, out, slopes, B, H, L, d);
  if (st != ALIBI_OK) return st;
  float* ws = nullptr;
  const size_t bytes = decode_ws_bytes(B, H, L, d);
  if (bytes > 0) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    st = workspace_get(kDecode, bytes, &ws);
    if (st != ALIBI_OK) return st;
  }
  return launch_decode_plan(q, kcache, vcache, out, B, H, L, d, slopes, ws, stream);
}

int alibi_attn_decode_ex(const void* q, const void* kcache, const void* vcache, void* out, int B, int H, int L,
                         int d, const float* slopes, const alibi_decode_opts* opts, hipStream_t stream) {
  int st = check_decode(q, kcache, vcache, out, slopes, B, H, L, d);
  if (st != ALIBI_OK) return st;
  const float* knorm = nullptr;
  if (opts != nullptr) {
    if ((opts->flags & ~ALIBI_SKIP_UNDERFLOW) != 0) return ALIBI_EINVAL;
    if (opts->flags & ALIBI_SKIP_UNDERFLOW) {
      if (opts->key_norm_max == nullptr || !aligned(opts->key_norm_max, 4)) return ALIBI_EINVAL;
      knorm = opts->key_norm_max;
    }
  }
  float* ws = nullptr;
  const size_t bytes = decode_ws_bytes(B, H, L, d);
  if (bytes > 0) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    st = workspace_get(kDecode, bytes, &ws);
    if (st != ALIBI_OK) return st;
  }
  return launch_decode_plan(q, kcache, vcache, out, B, H, L, d, slopes, ws, stream, knorm);
}

int alibi_key_norm_max(const void* kcache, int B, int H, int L, int d, float* out, hipStream_t stream) {
  if (kcache == nullptr || out == nullptr || B < 1 || H < 1 || L < 1 || d < 1 || L > kMaxLen ||
      !aligned(kcache, 16) || !aligned(out, 4))
    return ALIBI_EINVAL;
  if (d != 64 && d != 128) return ALIBI_ENOTSUP;
  if ((long long)B * H * L > (1LL << 31) * 4) return ALIBI_ENOTSUP;
  // partial maxima over key ranges of at least 256 rows, enough of them to
  // keep the part's loads in flight, then one maximum per (b, h)
  const long long bh = (long long)B * H;
  const int parts = int(std::max(1LL, std::min(std::max(1LL, (long long)L / 256), (4096 + bh - 1) / bh)));
  float* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    const int st = workspace_get(kNorm, (size_t)bh * parts * sizeof(float), &ws);
    if (st != ALIBI_OK) return st;
  }
  const int st = hip_status(alibi::launch_knorm_max(kcache, ws, B, H, L, d, parts, stream));
  if (st != ALIBI_OK) return st;
  return hip_status(alibi::launch_knorm_reduce(ws, out, bh, parts, stream));
}

int alibi_attn_decode_noalloc(const void* q, const void* kcache, const void* vcache, void* out, int B, int H,
                              int L, int d, const float* slopes, hipStream_t stream) {
  int st = check_decode(q, kcache, vcache, out, slopes, B, H, L, d);
  if (st != ALIBI_OK) return st;
  const size_t bytes = decode_ws_bytes(B, H, L, d);
  float* ws = nullptr;
  if (bytes > 0) {
    size_t cap = 0;
    st = hip_status(alibi::decode_scratch(&ws, &cap));
    if (st != ALIBI_OK) return st;
    if (bytes > cap) return ALIBI_ENOTSUP;
  }
  return launch_decode_plan(q, kcache, vcache, out, B, H, L, d, slopes, ws, stream);
}

size_t alibi_decode_ws_bytes(int B, int H, int L, int d) {
  if (B < 1 || H < 1 || L < 1 || d < 1 || L > kMaxLen || d > 256 || d % 8 != 0) return 0;
  return decode_ws_bytes(B, H, L, d);
}

int alibi_attn_decode_ws(const void* q, const void* kcache, const void* vcache, void* out, int B, int H,
                         int L, int d, const float* slopes, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_decode(q, kcache, vcache, out, slopes, B, H, L, d);
  if (st != ALIBI_OK) return st;
  const size_t bytes = decode_ws_bytes(B, H, L, d);
  if (bytes > 0 && (ws == nullptr || !aligned(ws, 16) || ws_bytes < bytes)) return ALIBI_EINVAL;
  return launch_decode_plan(q, kcache, vcache, out, B, H, L, d, slopes, bytes > 0 ? static_cast<float*>(ws) : nullptr,
                            stream);
}

int alibi_attn_weights_f32(const float* q, const float* k, float* w, int B, int H, int N, int d,
                           const float* slopes, int causal, hipStream_t stream) {
  int st = check_common(q, k, k, w, slopes, B, H, N, d, 4);
  if (st != ALIBI_OK) return st;
  if (causal != 0 && causal != 1) return ALIBI_EINVAL;
  if (N > 1024 || d > 256) return ALIBI_ENOTSUP;
  return hip_status(alibi::launch_weights_f32(q, k, w, B, H, N, d, slopes, causal, scale_log2(d), stream));
}

int alibi_debug_schedule(int w, int nbh, int nblk, int* out2) {
  if (out2 == nullptr || nbh < 1 || nblk < 1 || w < 0 || (long long)w >= (long long)nbh * nblk)
    return ALIBI_EINVAL;
  const alibi::WgBlock b = alibi::schedule_block(w, nbh, nblk);
  out2[0] = b.bh;
  out2[1] = b.rank;
  return ALIBI_OK;
}

int alibi_debug_stream_read(const void* buf, long long bytes, unsigned* sink, int workgroups,
                            hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes < 16 || bytes % 16 != 0 || workgroups < 1 ||
      workgroups > 65536 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return ALIBI_EINVAL;
  return hip_status(alibi::launch_stream_read(buf, bytes, sink, workgroups, stream));
}

int alibi_debug_mfma_rate(const void* frags, int iters, int valu, float* sink, int workgroups,
                          hipStream_t stream) {
  if (frags == nullptr || sink == nullptr || iters < 1 || iters > (1 << 20) || (valu != 0 && valu != 1) ||
      workgroups < 1 || workgroups > 65536 || (reinterpret_cast<uintptr_t>(frags) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return ALIBI_EINVAL;
  return hip_status(alibi::launch_mfma_rate(frags, iters, valu != 0, sink, workgroups, stream));
}

int alibi_debug_fail_allocations(int count) {
  if (count < 0) return ALIBI_EINVAL;
  g_fail_allocs.store(count);
  return ALIBI_OK;
}

int alibi_debug_fwd_waves(int nw) {
  if (nw != 0 && nw != 4 && nw != 8) return ALIBI_EINVAL;
  alibi::set_fwd_waves(nw);
  return ALIBI_OK;
}

int alibi_debug_fwd_form(int B, int H, int Nq, int Nk, int d, int causal, int flags, int delta, int* form) {
  if (form == nullptr || B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || (flags & ~15) != 0) return ALIBI_EINVAL;
  if (d != 64 && d != 128) {
    *form = 0;
    return ALIBI_OK;
  }
  alibi::FwdArgs a{};
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.causal = causal != 0;
  *form = alibi::fwd_mfma_form(a, flags, delta);
  return ALIBI_OK;
}

int alibi_debug_bwd_query_blocks(int qb) {
  if (qb < 0 || qb > 2) return ALIBI_EINVAL;
  alibi::set_bwd_query_blocks(qb);
  return ALIBI_OK;
}

int alibi_debug_fwd_split(int mode) {
  if (mode < 0 || mode > 2) return ALIBI_EINVAL;
  alibi::set_fwd_split(mode);
  return ALIBI_OK;
}

const char* alibi_status_string(int status) {
  switch (status) {
    case ALIBI_OK: return "ALIBI_OK: success";
    case ALIBI_EINVAL: return "ALIBI_EINVAL: invalid argument (size, null or misaligned pointer)";
    case ALIBI_ENOTSUP: return "ALIBI_ENOTSUP: request not supported by this library";
    case ALIBI_EHIP: return "ALIBI_EHIP: HIP runtime or launch failure";
    case ALIBI_ENOMEM: return "ALIBI_ENOMEM: workspace allocation failed";
    default: return "ALIBI: unknown status";
  }
}

int alibi_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int st = ALIBI_OK;
  int cur = 0;
  bool any = false;
  for (auto& list : g_ws) any = any || !list.empty();
  if (any && hipGetDevice(&cur) != hipSuccess) return ALIBI_EHIP;
  for (auto& list : g_ws) {
    for (size_t dev = 0; dev < list.size(); ++dev) {
      if (!list[dev].ptr) continue;
      if (hipSetDevice(int(dev)) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
          hipFree(list[dev].ptr) != hipSuccess)
        st = ALIBI_EHIP;
      list[dev].ptr = nullptr;
      list[dev].bytes = 0;
    }
  }
  if (any) (void)hipSetDevice(cur);
  return st;
}

}  // extern "C"
