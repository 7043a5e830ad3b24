/*
 * alibi.h -- C ABI of the MI355X (gfx950) causal ALiBi attention library.
 *
 * What is computed (per batch b, head h, query i, key j):
 *   score(i, j) = q_i . k_j / sqrt(d) - m_h * (i - j)      for j <= i
 *   score(i, j) = -inf                                     for j >  i (causal mask)
 *   w(i, .)     = softmax over keys of score(i, .)
 *   out_i       = sum_j w(i, j) v_j
 * Sources: "When Attention Goes Blind: Numerical Failure in ALiBi Positional
 * Encodings" (arXiv 2608.03994), Sec. 3.1, Eq. 1-3, and Sec. 3.2, Eq. 4;
 * "ALiBi: Attention with Linear Biases" (abhik.ai), section "From distance to
 * a normalized weight". The bias is generated inside the kernels' tiles; no
 * (H, N, N) bias tensor is ever stored (abhik.ai, remark after the
 * full-sequence example).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Return value: ALIBI_OK (0) or a negative alibi_status. No exception or
 *   abort crosses the ABI. Arguments are validated before anything is enqueued;
 *   on an error nothing is launched and outputs are untouched.
 * - Device pointers (q, k, v, out, caches, slopes on the attention calls) are
 *   caller-owned HIP device allocations on the current device. The library
 *   keeps no pointer past the call's stream order.
 * - Tensors are dense and contiguous, row-major, head dimension fastest:
 *   (B, H, N, d) for q/k/v/out, (B, H, L, d) for KV caches, (B, H, d) for the
 *   decode query and output. Every data pointer must be 16-byte aligned.
 * - `slopes` holds H fp32 values, one per head, for the GLOBAL head index
 *   (normally the output of alibi_slopes copied to the device). The library
 *   cannot detect a mismatched schedule.
 * - Work is enqueued asynchronously on `stream` (0 = the null stream). A
 *   launch failure is reported as ALIBI_EHIP; faults inside a kernel surface
 *   at the caller's next synchronisation.
 * - Sizes: B, H, N (or L), d >= 1 and N, L <= 2^24 (token distances stay
 *   exact in fp32). Element offsets are computed in 64-bit.
 */
#ifndef ALIBI_H_
#define ALIBI_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum alibi_status {
  ALIBI_OK = 0,
  ALIBI_EINVAL = -1,   /* bad size, null or misaligned pointer */
  ALIBI_ENOTSUP = -2,  /* valid request the library does not handle (e.g. d > 256) */
  ALIBI_EHIP = -3,     /* a HIP runtime call or kernel launch failed */
  ALIBI_ENOMEM = -4    /* the library could not allocate one of its workspaces */
} alibi_status;

/*
 * Per-head slopes (host only; no device work).
 * Power-of-two H: m_h = 2^(-8 (h + 1) / H), h = 0 .. H-1. Other H: the
 * schedule of c = the largest power of two below H, followed by entries
 * 0, 2, 4, ... of the schedule for 2c until H slopes are listed, in that
 * order (abhik.ai, "Different heads, different distance penalties"; dev.to
 * "ALiBi: give a Transformer position sense with one line", "Per-head slopes
 * form a geometric ladder"). Each power is evaluated in double and rounded
 * to nearest-even fp32.
 * slopes_out: caller-owned HOST array of at least H floats.
 * Errors: H < 1 or slopes_out == NULL -> ALIBI_EINVAL.
 */
int alibi_slopes(int H, float* slopes_out);

/*
 * Fused multi-head ALiBi attention forward, bf16 in / bf16 out, fp32
 * accumulation and fp32 online softmax.
 * q, k, v, out: device, bf16, (B, H, N, d) contiguous. out may not alias q/k/v.
 * slopes: device, H fp32.
 * causal = 1: the causal form above (Eq. 2-3 of "When Attention Goes Blind").
 * causal = 0: no mask and the symmetric bias -m_h |i - j| ("ALiBi and Relative
 *   Position Bias", quantmemo.com, "The mechanics").
 * d in {64, 128} runs the MFMA kernel; other d that are multiples of 8 up to
 * 256 run a slower generic kernel. Errors: ALIBI_EINVAL for bad sizes,
 * pointers or causal not in {0, 1}; ALIBI_ENOTSUP for d > 256 or d % 8 != 0.
 */
int alibi_attn_fwd(const void* q, const void* k, const void* v, void* out,
                   int B, int H, int N, int d, const float* slopes, int causal,
                   hipStream_t stream);

/*
 * Same operation in fp32 (inputs, output and all arithmetic), for any
 * 1 <= d <= 256 (pointers need only 4-byte alignment). Generic kernel; meant
 * for small and exact checks such as the 4-head, 8-token, d = 16 example of
 * "ALiBi in Attention: Complete Implementation" (mbrenndoerfer.com).
 */
int alibi_attn_fwd_f32(const float* q, const float* k, const float* v, float* out,
                       int B, int H, int N, int d, const float* slopes, int causal,
                       hipStream_t stream);

/*
 * Single-query decode against a KV cache, bf16 in / bf16 out.
 * q, out: device bf16 (B, H, d); kcache, vcache: device bf16 (B, H, L, d).
 * The query is the newest token at position L - 1 and key j keeps its real
 * position j, so the bias is -m_h (L - 1 - j) and every cached key is allowed
 * (abhik.ai, KV-cache remark after the full-sequence example).
 * The key range is split across workgroups; partial softmax states are merged
 * by a second kernel through a library-owned per-device workspace (see
 * alibi_release). Errors: as alibi_attn_fwd; ALIBI_ENOMEM if the workspace
 * cannot be allocated. Calls on one device are serialised by a mutex while
 * they size the workspace; the work itself stays asynchronous, and every
 * decode on one device uses the same workspace: order such calls on one
 * stream (or synchronise between them), or give each stream its own workspace
 * through alibi_attn_decode_ws.
 */
int alibi_attn_decode(const void* q, const void* kcache, const void* vcache, void* out,
                      int B, int H, int L, int d, const float* slopes,
                      hipStream_t stream);

/*
 * The same decode with a caller-owned workspace instead of the library's: no
 * allocation, no lock, and concurrent decodes on different streams stay
 * independent as long as each has its own workspace.
 * alibi_decode_ws_bytes(B, H, L, d) gives the bytes the call needs for a shape
 * (the partial softmax states of a key range split, B H S (d + 2) fp32 values
 * for S ranges per (b, h); 0 when no (b, h) is split, and 0 for arguments the
 * decode rejects). ws: device memory of at least that many bytes, 16-byte
 * aligned, owned by the caller and used asynchronously on `stream` (keep it
 * alive until the call's work completes); may be NULL when 0 bytes are needed.
 * Errors: as alibi_attn_decode, plus ALIBI_EINVAL for a missing, misaligned or
 * too small workspace. Source: the KV-cache remark of abhik.ai after the
 * full-sequence example (serving-style decode, where concurrent streams occur).
 */
size_t alibi_decode_ws_bytes(int B, int H, int L, int d);
int alibi_attn_decode_ws(const void* q, const void* kcache, const void* vcache, void* out,
                         int B, int H, int L, int d, const float* slopes,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): it
 * calls no allocating routine. Instead of a workspace it uses a fixed scratch
 * array compiled into the library, one per device, of 8191 (256 + 2) fp32
 * values (8.45 MB), which holds the partial states of every split the decode
 * makes for d <= 256; each device keeps its copy until the process ends. Its
 * address is looked up once per device, on the first call with that device
 * current. Arguments and results as alibi_attn_decode. Every call on one
 * device shares that device's scratch: calls whose work overlaps on one device
 * (other streams, other threads) race and must be ordered by the caller. No
 * part of the scratch needs to start at zero. ALIBI_ENOTSUP if a shape would
 * need more scratch than the array holds; ALIBI_EHIP if the lookup fails.
 */
int alibi_attn_decode_noalloc(const void* q, const void* kcache, const void* vcache, void* out,
                              int B, int H, int L, int d, const float* slopes, hipStream_t stream);

/*
 * Options of alibi_attn_decode_ex. flags: 0 or ALIBI_SKIP_UNDERFLOW (defined
 * below with the forward's options); other bits -> ALIBI_EINVAL.
 */
typedef struct alibi_decode_opts {
  int flags;
  const float* key_norm_max; /* device, B H fp32 (4-byte aligned): for each (b, h) an upper
                                bound of |k_j| over the whole key cache, e.g. from
                                alibi_key_norm_max; required with ALIBI_SKIP_UNDERFLOW */
} alibi_decode_opts;

/*
 * The decode with options (opts NULL or flags 0: alibi_attn_decode).
 * ALIBI_SKIP_UNDERFLOW skips, exactly, the cached keys whose weights round to
 * zero: every score is at most A - m_h D with A = |q| key_norm_max / sqrt(d)
 * and D the key's distance, and the newest key's score is at least -A, so a
 * key more than (2 A + 152 ln 2) / m_h behind the keys that set the running
 * maxima has exp() below 2^-150 relative to them, an exact zero in fp32 ("When
 * Attention Goes Blind", Sec. 3.3 and 5.1-5.2: distant weights underflow). Key
 * ranges past that distance are not read, and the walk inside a range stops
 * there, so a steep head reads only its last few hundred keys. The output is
 * bitwise the output of alibi_attn_decode when key_norm_max bounds every key
 * norm of its (b, h) and the caches are finite; a smaller bound gives a wrong
 * result, not a fault. A caller that appends keys keeps the bound current as
 * max(bound, |k_new|). Uses the library's decode workspace (ordering as
 * alibi_attn_decode). Errors: as alibi_attn_decode, plus ALIBI_EINVAL for an
 * unknown flag or a missing or misaligned key_norm_max.
 */
int alibi_attn_decode_ex(const void* q, const void* kcache, const void* vcache, void* out,
                         int B, int H, int L, int d, const float* slopes, const alibi_decode_opts* opts,
                         hipStream_t stream);

/*
 * The bound alibi_attn_decode_ex's skipping takes: out[b H + h] (device fp32,
 * 4-byte aligned) = max_j |k_j| over the L keys of (b, h) of a bf16 cache
 * (B, H, L, d), d in {64, 128} (ALIBI_ENOTSUP otherwise), computed in fp32 from
 * the bf16 values (the decode adds a relative margin of 2^-8 against
 * rounding). Reads the cache once; partial maxima go through the library's
 * key-norm workspace (ordering as the other workspaces, ALIBI_ENOMEM if it
 * cannot be allocated). Asynchronous on `stream`. ALIBI_EINVAL for NULL or
 * misaligned pointers or sizes < 1.
 */
int alibi_key_norm_max(const void* kcache, int B, int H, int L, int d, float* out, hipStream_t stream);

/*
 * TEST ONLY, not on the hot path: materialises the fp32 attention weights
 * w (B, H, N, N) of the fp32 forward, so the printed weight matrices of the
 * 4-head seed-42 example can be checked on the device. Masked weights are
 * written as exact zeros. Rejects N > 1024 (ALIBI_ENOTSUP) and d > 256.
 */
int alibi_attn_weights_f32(const float* q, const float* k, float* w,
                           int B, int H, int N, int d, const float* slopes, int causal,
                           hipStream_t stream);

/*
 * Extended forward: mitigation variants and query/key position offsets.
 *
 * Mitigations (Sec. 3.4 of "When Attention Goes Blind", settings of Sec. 4.3):
 *   ALIBI_CLAMP         bias floored at a constant: B* = max(B, clamp_min)
 *   ALIBI_LOG_DISTANCE  distance compressed: D* = ln(D + 1), so B = -m ln(D + 1)
 *   ALIBI_SOFTCAP       content logit capped: A* = softcap * tanh(A / softcap),
 *                       A = q.k / sqrt(d); the bias is not capped
 * Any combination is allowed; per score the order is A -> A*, D -> D*,
 * B = -m D*, B -> B*, logit = A* + B*, then the causal mask and the softmax.
 */
#define ALIBI_CLAMP 1
#define ALIBI_LOG_DISTANCE 2
#define ALIBI_SOFTCAP 4
/*
 * ALIBI_SKIP_UNDERFLOW: exact skipping of key tiles whose every weight would
 * round to zero ("When Attention Goes Blind": the underflow of Sec. 3.2-3.3
 * and the wasted work of Sec. 5.1-5.2). A first pass stores max_j |k_j| per
 * (b, h) in a library-owned per-device workspace; the forward then bounds each
 * score by |q_i| max|k| / sqrt(d) - m (i - j) and stops, per workgroup, at the
 * first key tile where that bound lies more than 148 log2 units under the
 * row's guaranteed running maximum (without the causal mask, the symmetric
 * bias -m |i - j| lets it stop on both sides of the queries). The output is
 * bit-identical to the call without the flag. It acts on the plain form with
 * d in {64, 128}, causal or not; with mitigations or on the generic kernel it
 * is accepted and changes nothing. Calls with this flag on one device share the workspace:
 * order them on one stream (or synchronise between them).
 */
#define ALIBI_SKIP_UNDERFLOW 8
/*
 * ALIBI_WINDOW: a hard per-head sliding window ("When Attention Goes Blind",
 * Sec. 5.2: steep heads already act as sliding windows, and Sec. 5.3: a hard
 * window lets the computation ignore out-of-window entries instead of
 * computing and discarding them). opts->window holds H ints on the device: a
 * window of W tokens keeps key c for query r when 0 <= pos(r) - pos(c) < W,
 * so W = 1 keeps the query's own key and W <= 0 none (a zero output row).
 * This changes results wherever a weight falls outside the window. Key tiles
 * wholly out of a wave's window are skipped. Causal form only
 * (ALIBI_ENOTSUP with causal = 0) and without the mitigation bits
 * (ALIBI_ENOTSUP); offsets, opts->lse and ALIBI_SKIP_UNDERFLOW combine with it.
 */
#define ALIBI_WINDOW 16

typedef struct alibi_fwd_opts {
  int flags;         /* OR of the ALIBI_* bits above; other bits -> ALIBI_EINVAL */
  float clamp_min;   /* bias floor in logit units (e.g. -87); finite; used with ALIBI_CLAMP */
  float softcap;     /* z > 0, finite (e.g. 50); used with ALIBI_SOFTCAP */
  int q_offset;      /* position of query row 0, 0 .. 2^24 */
  int k_offset;      /* position of key row 0, 0 .. 2^24 */
  float* lse;        /* optional device fp32 (B, H, Nq) output: each row's natural-log
                        log-sum-exp of its logits (-inf for a row that sees no key),
                        what alibi_attn_bwd needs; NULL = not written; 4-byte aligned */
  const int* window; /* device, H ints: the per-head window in tokens; used with
                        ALIBI_WINDOW (non-NULL, 4-byte aligned), ignored otherwise */
} alibi_fwd_opts;

/*
 * q, out: device bf16 (B, H, Nq, d); k, v: device bf16 (B, H, Nk, d).
 * Query row r sits at position q_offset + r and key row c at k_offset + c; the
 * distance is the difference of the positions (abhik.ai, KV-cache remark: a
 * cached query keeps its real position). With causal = 1 key c is visible to
 * query r when its position is not later; a query that sees no key gets a zero
 * output row. A chunk of Nq new tokens after Nk - Nq cached ones is
 * q_offset = Nk - Nq, k_offset = 0 (chunked prefill).
 * opts may be NULL (no mitigation, both offsets 0); alibi_attn_fwd is this call
 * with Nq = Nk = N and opts = NULL. d in {64, 128} runs the MFMA kernel (each
 * mitigation mix is its own compiled variant); other d (multiples of 8 up to
 * 256) the generic kernel. Errors: as alibi_attn_fwd, plus ALIBI_EINVAL for an
 * unknown flag bit, a non-finite clamp, a soft cap that is not positive and
 * finite, or an offset outside 0 .. 2^24.
 */
int alibi_attn_fwd_ex(const void* q, const void* k, const void* v, void* out,
                      int B, int H, int Nq, int Nk, int d, const float* slopes, int causal,
                      const alibi_fwd_opts* opts, hipStream_t stream);

/*
 * Same operation in fp32 through the generic kernel, with the mitigations
 * evaluated by the precise device math library (tanhf, log1pf); for exact
 * checks. Any 1 <= d <= 256, 4-byte aligned pointers.
 */
int alibi_attn_fwd_ex_f32(const float* q, const float* k, const float* v, float* out,
                          int B, int H, int Nq, int Nk, int d, const float* slopes, int causal,
                          const alibi_fwd_opts* opts, hipStream_t stream);

/*
 * Backward pass: gradients of the plain ALiBi forward (no mitigation, no
 * offsets) with respect to q, k and v; the bias is a constant (the slopes are
 * fixed, abhik.ai "Different heads, different distance penalties").
 * With P = exp(logits - lse) recomputed per tile from the forward's lse:
 *   dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dO * O)),
 *   dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
 * q, k, v, out (the forward's output), dout, dq, dk, dv: device bf16
 * (B, H, N, d) contiguous, 16-byte aligned; lse: device fp32 (B, H, N) from
 * alibi_attn_fwd_ex's opts->lse; slopes: device, H fp32; causal as in the
 * forward. d must be 64 or 128 (ALIBI_ENOTSUP otherwise). Uses a
 * library-owned per-device workspace of 2 B H N floats: order calls on one
 * device on one stream. dq, dk, dv may not alias the inputs.
 */
int alibi_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, const float* slopes, int causal,
                   hipStream_t stream);

/*
 * Backward pass of the forward with the mitigations of Sec. 3.4 of "When
 * Attention Goes Blind" (the paper trains with them): opts->flags may hold
 * ALIBI_CLAMP (opts->clamp_min, finite) and ALIBI_LOG_DISTANCE, which change
 * only the constant bias, B = max(-m D*, c) with D* = D or ln(D + 1), so the
 * gradients follow the same chain rule with P recomputed under that bias; and
 * ALIBI_SOFTCAP (opts->softcap = z, finite and > 0), whose capped content
 * logit z tanh(A / z) adds the factor 1 - tanh(A / z)^2 to dS before dQ and dK
 * are formed. lse must come from alibi_attn_fwd_ex with the same opts.
 * Everything else as alibi_attn_bwd (which is this call with opts = NULL).
 * ALIBI_WINDOW and nonzero offsets: ALIBI_ENOTSUP (forward-only forms);
 * unknown bits, a non-finite clamp or a soft cap that is not finite and
 * positive: ALIBI_EINVAL.
 * ALIBI_SKIP_UNDERFLOW (plain form, causal or not; accepted and without
 * effect with the mitigations): a first pass takes max|q_i|
 * and max|k_j| per (b, h); every logit is then at most A - m D (A =
 * max|q| max|k| / sqrt(d)) and every row's log-sum-exp at least -A (its
 * diagonal logit), so query-key pairs further apart than D with
 * m D log2(e) > 2 A log2(e) + 152 have P = exp(logit - lse) rounding to an
 * exact zero, and so add exact zeros to dq, dk and dv: the tiles made only of
 * such pairs are not visited. For finite inputs and lse from the matching
 * forward the gradients are bit-identical to the call without the flag. The
 * workspace then also holds 2 B H P floats of norm maxima (P <= 2048 / (B H)
 * rounded up, at least 1).
 */
int alibi_attn_bwd_ex(const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, const float* slopes, int causal,
                      const alibi_fwd_opts* opts, hipStream_t stream);

/*
 * Slope recipes from target blindness distances (host only). A head whose bias
 * should reach the fp32 underflow limit ln 2^-126 at distance delta gets
 * m = 126 ln(2) / delta ("When Attention Goes Blind": Sec. 3.2 blindness
 * distance, Sec. 3.4 "Robust Slopes", Sec. 4.2 configurations, App. F Table 8;
 * the printed distances follow that threshold). Targets, steepest head first,
 * spaced geometrically from the first to the last:
 *   ALIBI_SLOPES_STEEP     128 .. 512
 *   ALIBI_SLOPES_SAFE      2048 .. 4096
 *   ALIBI_SLOPES_WIDE      16 .. 4096
 *   ALIBI_SLOPES_EXPLICIT  32, 64, 128, ... (doubling, as Table 8 lists them)
 *   ALIBI_SLOPES_DEFAULT   the geometric schedule of alibi_slopes
 * log_distance != 0 adapts a target recipe to ALIBI_LOG_DISTANCE:
 * m = 126 ln(2) / ln(delta + 1) (Sec. 4.3); it does not change the default.
 * Each slope is evaluated in double and rounded to nearest-even fp32.
 * slopes_out: HOST array of H floats. Errors: H < 1, an unknown recipe or a
 * NULL pointer -> ALIBI_EINVAL.
 */
#define ALIBI_SLOPES_DEFAULT 0
#define ALIBI_SLOPES_STEEP 1
#define ALIBI_SLOPES_SAFE 2
#define ALIBI_SLOPES_WIDE 3
#define ALIBI_SLOPES_EXPLICIT 4
int alibi_slopes_recipe(int recipe, int H, int log_distance, float* slopes_out);

/*
 * TEST ONLY, host only: the workgroup -> ((b, h) pair, block rank) schedule the
 * forward and backward kernels use (heads kept per XCD, heaviest blocks first
 * within small groups of heads), for workgroup w of nbh pairs x nblk blocks.
 * Writes {pair, rank} to out2 (host array of 2 ints). ALIBI_EINVAL for w
 * outside [0, nbh nblk), sizes < 1 or NULL.
 */
int alibi_debug_schedule(int w, int nbh, int nblk, int* out2);

/*
 * TEST ONLY: the next `count` requests for a library-owned workspace (decode,
 * skipping forward, backward) fail with ALIBI_ENOMEM as if the device
 * allocation had failed, before any HIP call; 0 turns the hook off.
 * Process-wide. ALIBI_EINVAL for count < 0.
 */
int alibi_debug_fail_allocations(int count);

/*
 * TEST AND TUNING ONLY: waves per workgroup of the bf16 MFMA forward kernel,
 * process-wide. 0 = automatic (the default: 8 for d = 128 when the grid has at
 * least 512 eight-wave workgroups, else 4), 4 or 8 =
 * forced for every later call. The two differ only by rounding: a row's tiles
 * are visited in the same order, but which of them take the exact or the
 * bounded running maximum depends on the block height. The environment variable
 * ALIBI_FWD_NW=4|8, read once at load, sets the same override. Not
 * synchronised with launches in flight on other threads. ALIBI_EINVAL for
 * other values.
 */
int alibi_debug_fwd_waves(int nw);

/*
 * TEST AND TUNING ONLY: the key-range split of the plain causal bf16 forward
 * (no mitigation; offsets, the log-sum-exp output and the exact skipping
 * allowed), process-wide. 0 = automatic (the default, when no wave count is
 * forced: split where a tile-step model of the run, the heaviest query
 * block's walk against the total work per CU, says the split form takes under
 * 0.7 of the unsplit time; alibi_debug_fwd_form reports the choice),
 * 1 = never, 2 = always. The split form runs 8-wave workgroups over 128 query
 * rows, waves 0-3 and 4-7 taking alternate key tiles of those rows and merging
 * their partial softmax states (m, l, O) at the end (the stable-softmax algebra
 * of "When Attention Goes Blind", App. B.1-B.2); its output differs from the
 * unsplit form's by rounding only. The environment variable ALIBI_FWD_SPLIT=1|2,
 * read once at load, sets the same override. Not synchronised with launches in
 * flight on other threads. ALIBI_EINVAL for other values.
 */
int alibi_debug_fwd_split(int mode);

/*
 * TEST AND TUNING ONLY: 32-row query blocks per step of the backward's dK/dV
 * kernel, process-wide. 0 = automatic (the default, which takes 2), 1 or 2 =
 * forced for every later call. With 2, each step takes a 64-row query tile and the weights P
 * pass from the dV to the dK waves as fp16 (fp32 with 1); the gradients
 * differ by rounding only. The environment variable ALIBI_BWD_QB=1|2, read
 * once at load, sets the same override. Not synchronised with launches in
 * flight on other threads. ALIBI_EINVAL for other values.
 */
int alibi_debug_bwd_query_blocks(int qb);

/*
 * TEST AND TUNING ONLY: the form a bf16 forward call with these sizes would
 * launch, under the current overrides. flags: the ALIBI_* option bits; delta:
 * q_offset - k_offset. *form: 0 = the generic kernel (d not 64 or 128), 4 or 8
 * = MFMA kernel with that many waves per workgroup over the whole key range,
 * 2 = the key-range split (8 waves). Host only. ALIBI_EINVAL for sizes < 1,
 * unknown flags or a NULL form.
 */
int alibi_debug_fwd_form(int B, int H, int Nq, int Nk, int d, int causal, int flags, int delta, int* form);

/*
 * MEASUREMENT ONLY: a plain streaming read of `bytes` bytes of device memory
 * at `buf` (16-byte aligned, bytes a positive multiple of 16), the practical
 * HBM read ceiling against which the decode's bandwidth is read. Each of
 * `workgroups` (1 .. 65536) workgroups of 256 threads writes the XOR of the
 * 32-bit words it read to sink[workgroup] (device memory, 4-byte aligned, room
 * for `workgroups` words), so the XOR of the sink equals the XOR of the buffer.
 * Asynchronous on `stream`. ALIBI_EINVAL for bad arguments (checked before
 * anything is enqueued).
 */
int alibi_debug_stream_read(const void* buf, long long bytes, unsigned* sink, int workgroups,
                            hipStream_t stream);

/*
 * MEASUREMENT ONLY: the sustained bf16 matrix rate of the part, against which
 * the forward's MFMA rate is read beside the datasheet peak. Each of
 * `workgroups` (1 .. 65536) workgroups of 8 waves (two per SIMD, as in the
 * forward) runs, per wave, `iters` (1 .. 2^20) rounds of 16 back-to-back
 * v_mfma_f32_32x32x16_bf16 from registers, over four independent accumulator
 * chains; one round is 16 x 32768 flop per wave. `frags` (device memory,
 * 16-byte aligned) holds the operand fragments as 8 x 64 lanes x 8 bf16: A_0 ..
 * A_3 then B_0 .. B_3, lane l of A holding row l % 32, k = 8 (l / 32) .. + 7,
 * and lane l of B column l % 32 at the same k; chain c accumulates A_c B_m for
 * m = 0 .. 3 in turn. valu = 1 adds, beside every MFMA, the vector work the
 * forward's softmax issues per MFMA (an fma, an exponential, half a bf16
 * pack, half a bf16 dot, an add) on independent data; valu = 0 runs the
 * MFMAs alone. Wave w of workgroup g writes the sum of all its accumulator
 * values, iters * sum_m sum(A_c B_m) summed over c, to sink[8 g + w] (device
 * memory, 4-byte aligned, room for 8 workgroups fp32) either way.
 * Asynchronous on `stream`. ALIBI_EINVAL for bad arguments (checked before
 * anything is enqueued).
 */
int alibi_debug_mfma_rate(const void* frags, int iters, int valu, float* sink, int workgroups,
                          hipStream_t stream);

/* Static, never-NULL description of a status code. */
const char* alibi_status_string(int status);

/*
 * Frees the library-owned workspaces (decode partial states, key-norm maxima
 * of the skipping forward, the backward's row terms) on every device after a
 * device synchronisation. Safe to call at any time; later calls re-allocate.
 */
int alibi_release(void);

#ifdef __cplusplus
}
#endif

#endif /* ALIBI_H_ */
