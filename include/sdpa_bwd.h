/*
 * sdpa_bwd.h -- C ABI of the MI355X (gfx950) scaled-dot-product-attention backward library.
 *
 * The operation ("SDPA Backward (SM120)", sections "Overview" and "API Usage"): from the forward
 * pass's inputs and output (Q, K, V, O), the gradient that reaches O (dO) and the forward's
 * log-sum-exp in natural log (LSE), compute dQ, dK, dV of softmax(scale * Q K^T + mask) V, with
 *     P     = exp(scale * Q K^T - LSE)                (replayed from LSE; masked pairs give 0)
 *     delta = rowsum(O * dO)                           ("The kernel chain")
 *     dS    = P * (dO V^T - delta)                     (unscaled softmax VJP)
 *     dV    = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K
 * (scale placement as printed in "NVFP4 Attention QAT Backward", section "Overview").
 * GQA/MQA: H_kv divides H_q, query head h uses KV head h / (H_q / H_kv), and dK/dV of a KV head
 * sum over its query-head group in a fixed order ("GQA/MQA group reduction").
 *
 * Layout and types.  Every tensor is contiguous (B, H, S, D) with the head dim innermost (any other
 * dense layout with a contiguous head dim through sdpa_bwd_flex):
 *   q, dq : (B, Hq,  Sq,  Dqk) bf16       k, dk : (B, Hkv, Skv, Dqk) bf16
 *   v, dv : (B, Hkv, Skv, Dv)  bf16       o, dO : (B, Hq,  Sq,  Dv)  bf16
 *   lse   : (B, Hq,  Sq)       fp32, natural log; -inf marks a row that saw no key
 * bf16 values are passed as their 16-bit patterns.  All pointers are device pointers; tensor
 * pointers must be 16-byte aligned (lse 4-byte aligned) and the workspace 256-byte aligned; a
 * tensor with no elements may be NULL.  Head dims ("Support surface"): Dqk and Dv multiples of 8
 * with 8 <= Dv <= Dqk <= 256.  A call computes on the kernel head dims (Kqk, Kv), the first of
 * (32,32), (64,64), (128,128), (192,128), (256,256) that covers (Dqk, Dv): those five run as they
 * are, any other pair reads the operand columns past its head dims as zeros and writes no column
 * past them (so the gaps of a strided layout are left untouched).  Empty problems (B, Sq or Skv zero) need
 * no workspace: the gradients that have elements are written as zeros.
 *
 * Masks ("API Usage" and "Causal, sliding-window, and padding masks"): query q and key k are
 * visible together when q < seq_q, k < seq_kv, causal => k <= q + diag + window_right, and
 * window_left >= 0 => k >= q + diag - window_left; diag = 0 (top-left) or seq_kv - seq_q
 * (bottom-right).  dq rows at or past seq_q and dk/dv rows at or past seq_kv are written as 0;
 * every element of dq, dk and dv is overwritten.
 *
 * Ownership and streams.  The caller owns every buffer, including one workspace of at least
 * sdpa_bwd_workspace_size() bytes; the library allocates nothing and keeps no state between calls.
 * All work is enqueued on `stream` (a hipStream_t; 0 = the null stream) and the call returns
 * without synchronising.  Calls that share a workspace must be ordered on one stream.
 *
 * Errors.  Functions return SDPA_BWD_OK (0) or a status code; validation happens before the first
 * launch, so a rejected call leaves every output untouched.  Nothing aborts or throws.
 *
 * Determinism ("Determinism", "Deterministic vs. non-deterministic dQ"): the `deterministic`
 * argument selects how dQ is formed (SDPA_BWD_DQ_*):
 *   0  fp32 atomic adds into an fp32 accumulator, converted once; the low bits of dq may vary
 *      between runs;
 *   2  dS panels: the main kernel stores the bf16 dS tiles in the workspace and a second kernel
 *      forms dQ = scale * dS K in ascending KV order;
 *   3  dQ partials: the main kernel stores one fp32 dQ partial per (KV tile, 32-row q tile) in
 *      the workspace and a second kernel sums them in ascending KV order;
 *   4  ordered relay ("Deterministic vs. non-deterministic dQ", ordered-reduction relay): the
 *      main kernel keeps one fp32 running sum per (query head, 32-row q tile) in the workspace and
 *      the key tiles that see the q tile add into it one after another in ascending KV order,
 *      passing a turn counter; a conversion kernel then writes dq.  The workspace stays linear in
 *      the sequence lengths.  The key tiles of one query head run on one XCD (of the device's
 *      hipDeviceAttributeNumberOfXccs), taking their work from per-XCD queues; if a wait for a
 *      turn is ever abandoned (it is bounded), or not every work item ran, dq is written as NaN;
 *   1  deterministic, the library's choice: 3 where its workspace holds fewer bytes per
 *      (KV tile, q row) (Kqk fp32 partials against the key tile's bf16 dS values), else 2
 *      (kernel head dims 32 and 64 take 3; 128, 192 and 256 take 2); and 4 when that route's
 *      buffer, quadratic in the sequence lengths, would exceed 4 GiB ("Determinism": shapes whose
 *      dS buffer does not fit fall back to the relay).  The bound is fixed, so the choice depends
 *      on the call's arguments only; sdpa_bwd_dq_route reports it.
 * Routes 1-4 make dq, dk, dv bitwise reproducible run to run; dK and dV are reproducible on every
 * route.  Any other value gives SDPA_BWD_INVALID_ARG.
 */
#ifndef SDPA_BWD_H
#define SDPA_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* values of the `deterministic` argument */
enum {
  SDPA_BWD_DQ_ATOMIC = 0,
  SDPA_BWD_DQ_DETERMINISTIC = 1,
  SDPA_BWD_DQ_DS_PANELS = 2,
  SDPA_BWD_DQ_PARTIALS = 3,
  SDPA_BWD_DQ_RELAY = 4
};

enum {
  SDPA_BWD_OK = 0,
  SDPA_BWD_INVALID_ARG = 1,          /* null pointer, negative size, H_kv not dividing H_q, ... */
  SDPA_BWD_UNSUPPORTED = 2,          /* head dims outside the supported set, misaligned pointer */
  SDPA_BWD_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below sdpa_bwd_workspace_size()        */
  SDPA_BWD_LAUNCH_FAILED = 4,        /* the HIP runtime reported an error at launch             */
  SDPA_BWD_SCRATCH_TOO_SMALL = 5     /* sdpa_bwd_noalloc: the problem's workspace exceeds
                                        SDPA_BWD_NOALLOC_SCRATCH_BYTES                           */
};

/* Bytes of workspace needed by a call with these arguments: a 256-byte-aligned carve of the
 * per-row statistics (LSE * log2 e and delta, B*Hq*Sq_pad float pairs, Sq_pad = Sq rounded up to
 * 32), then the dQ route's buffer: the fp32 dQ accumulator (B*Hq*Sq*Kqk floats, route 0), the
 * bf16 dS panels (B*Hq*Sq_pad*Skv_pad, route 2), the fp32 dQ partials
 * (B*Hq*(Skv_pad/BC)*Sq_pad*Kqk floats, route 3) or the relay's running sums (B*Hq*Sq_pad*Kqk
 * floats), its turn counters (B*Hq*Sq_pad/32 int32) and 16 int32 control words (route 4), where (Kqk, Kv) are the kernel head dims of
 * the call (see above), BC is the key tile (256 keys for kernel head dims up to 192, 128 for 256)
 * and Skv_pad is Skv rounded up to BC; then, under GQA or when the main grid splits its q ranges,
 * the bf16 per-(query head, part) dK/dV partials (Kqk + Kv per key row).  Returns 0 for arguments
 * sdpa_bwd rejects and for empty problems. */
size_t sdpa_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv,
                               int causal, int window_left, int deterministic, int has_seqlens);

/* The dQ route a call of sdpa_bwd, sdpa_bwd_ex or sdpa_bwd_flex with these sizes and this
 * `deterministic` value takes: SDPA_BWD_DQ_ATOMIC, SDPA_BWD_DQ_DS_PANELS, SDPA_BWD_DQ_PARTIALS or
 * SDPA_BWD_DQ_RELAY (never SDPA_BWD_DQ_DETERMINISTIC, which resolves to one of the last three
 * by head dim and by the size of its quadratic buffer, see above); -1 for sizes or head dims
 * sdpa_bwd rejects or an unknown value.  Host only, no GPU work.  sdpa_bwd_workspace_size sizes
 * the same route's buffers. */
int sdpa_bwd_dq_route(int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv,
                      int deterministic);

/* The backward pass with top-left causal masking, no padding and no right band.
 * scale <= 0 selects 1/sqrt(Dqk) ("API Usage": None -> 1/sqrt(D)).  window_left = -1 disables the
 * left window.  `workspace` must hold sdpa_bwd_workspace_size(...) bytes (not checked here; use
 * sdpa_bwd_ex to have it checked).  `stream` is a hipStream_t. */
int sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv,
             float scale, int causal, int window_left, int deterministic,
             void* workspace, void* stream);

/* Superset of sdpa_bwd: per-batch padding lengths seq_q_lens / seq_kv_lens (device int32 (B,)
 * arrays or NULL = full length; values are clamped to [0, S]), bottom-right causal alignment,
 * a right band window_right >= 0 widening the causal diagonal, and a checked workspace size. */
int sdpa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dO,
                const float* lse, void* dq, void* dk, void* dv,
                int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv,
                float scale, int causal, int window_left, int deterministic,
                const int* seq_q_lens, const int* seq_kv_lens, int causal_bottom_right,
                int window_right, void* workspace, size_t workspace_bytes, void* stream);

/* sdpa_bwd_ex that also records five HIP events (hipEvent_t, created by the caller) on `stream`:
 * before the preprocess, after the preprocess, after the main kernel, after the GQA reduce (same
 * point as the previous one when there is none) and after the dQ convert / dq2k / dq_reduce kernel.  A NULL
 * entry is skipped (each recorded event is one more packet on the stream).  For measuring each
 * kernel's share of the chain; the arithmetic is identical to sdpa_bwd_ex. */
int sdpa_bwd_ex_events(const void* q, const void* k, const void* v, const void* o, const void* dO,
                       const float* lse, void* dq, void* dk, void* dv,
                       int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv,
                       float scale, int causal, int window_left, int deterministic,
                       const int* seq_q_lens, const int* seq_kv_lens, int causal_bottom_right,
                       int window_right, void* workspace, size_t workspace_bytes, void* stream,
                       void* const* events);

/* Size of the static device scratch of sdpa_bwd_noalloc, per device (256 MiB). */
#define SDPA_BWD_NOALLOC_SCRATCH_BYTES (256u * 1024u * 1024u)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): sdpa_bwd_ex without a workspace argument.  The
 * workspace is carved from a static device array of SDPA_BWD_NOALLOC_SCRATCH_BYTES that the
 * library holds on every device it runs on until the process ends; the call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  The caller still owns every tensor.
 * Arguments, layout, masks, routes, stream and status rules are those of sdpa_bwd_ex, and the
 * arithmetic is the same.  A problem whose workspace (sdpa_bwd_workspace_size) exceeds the scratch
 * gives SDPA_BWD_SCRATCH_TOO_SMALL before any GPU call.  `stream` must belong to the current
 * device; the scratch's device address is looked up on the first call made with a device current.
 * Every call on one device shares that device's scratch and finds the previous call's contents
 * (the chain clears what it accumulates into on its own stream), so calls that overlap on one
 * device race: order them (one stream, or events).  No stage events. */
int sdpa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv,
                     float scale, int causal, int window_left, int deterministic,
                     const int* seq_q_lens, const int* seq_kv_lens, int causal_bottom_right,
                     int window_right, void* stream);

/* element types: the io type of sdpa_bwd_flex (BF16, FP16); a bias may also be FP32 */
enum { SDPA_BWD_BF16 = 0, SDPA_BWD_FP16 = 1, SDPA_BWD_FP32 = 2 };

/* Strides, in elements, of one logical (B, H, S, D) tensor whose head dim is contiguous (stride 1):
 * "dense_flex" layouts ("SDPA Backward (SM120)", section "API Usage": any dense layout with the
 * head dim innermost-contiguous, addressed in place).  BHSD contiguous is {H*S*D, S*D, D}; BSHD
 * (B, S, H, D) storage viewed as (B, H, S, D) is {S*H*D, D, H*D}. */
typedef struct sdpa_bwd_layout {
  int64_t batch, head, seq;
} sdpa_bwd_layout;

/* sdpa_bwd_ex_events with per-tensor layouts and an io dtype.
 * layouts: NULL (every tensor contiguous BHSD) or 8 entries, in the order q, k, v, o, dO, dq, dk,
 *   dv.  Each stride must be a multiple of 8 elements (with 16-byte-aligned base pointers every
 *   row is 16-byte aligned; else SDPA_BWD_UNSUPPORTED), batch/head strides >= 0 and the seq
 *   stride >= the head dim (else SDPA_BWD_INVALID_ARG), and one head's span,
 *   ((S - 1) * seq + D) * 2 bytes, below 2^31 (else SDPA_BWD_UNSUPPORTED).  Outputs must not
 *   overlap each other or the inputs.  lse stays contiguous (B, Hq, Sq); the workspace is the
 *   same as for sdpa_bwd_ex.
 * dtype: the element type of q, k, v, o, dO, dq, dk, dv ("Support surface": FP16 / BF16, LSE
 *   fp32): SDPA_BWD_BF16, or SDPA_BWD_FP16, for which P and dS enter the MFMAs as fp16 and the
 *   GQA partials and the deterministic dS workspace are fp16 too (accumulation stays fp32);
 *   any other value gives SDPA_BWD_UNSUPPORTED.
 * events: NULL or five entries as for sdpa_bwd_ex_events. */
int sdpa_bwd_flex(const void* q, const void* k, const void* v, const void* o, const void* dO,
                  const float* lse, void* dq, void* dk, void* dv,
                  int B, int Hq, int Hkv, int Sq, int Skv, int Dqk, int Dv,
                  float scale, int causal, int window_left, int deterministic,
                  const int* seq_q_lens, const int* seq_kv_lens, int causal_bottom_right,
                  int window_right, const sdpa_bwd_layout* layouts, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/* Every argument of one backward call, for sdpa_bwd_run.  The fields mean what the arguments of
 * the same names mean for sdpa_bwd_flex (layouts NULL = every tensor contiguous BHSD; events NULL
 * or five entries), plus the sink tokens ("SDPA Backward (SM120)", "API Usage" sink_token,
 * "The kernel chain" dsink, "Support surface" sink tokens):
 *   sink   (Hq,) fp32 device array of per-query-head sink logits, 4-byte aligned, or NULL.  The
 *          forward's LSE already folds the sink into each row's softmax denominator, so dq, dk
 *          and dv do not depend on it.
 *   dsink  (Hq,) fp32 device output, 4-byte aligned, or NULL (then sink is not read):
 *          dsink[h] = -sum over batch entries b and query rows q < seq_q_lens[b] whose LSE is
 *          finite of exp(sink[h] - lse[b,h,q]) * rowsum(O * dO)[b,h,q], summed in a fixed order
 *          (bitwise reproducible on every dQ route).  Overwritten, not accumulated into; 0 when
 *          B or Sq is 0.  A non-NULL dsink with a NULL sink gives SDPA_BWD_INVALID_ARG.
 * The dsink kernel runs right after the preprocess (inside the first event interval).
 * And the additive bias ("API Usage" bias_tensor, "Support surface" bias):
 *   bias        (bias_batch, Hq, Sq, Skv) contiguous device array added to the scores after the
 *               softmax scale and before the softmax (the forward's LSE must include it), or
 *               NULL; elements of the io type (bias_dtype = dtype, 2-byte aligned) or fp32
 *               (bias_dtype = SDPA_BWD_FP32, 4-byte aligned); another bias_dtype gives
 *               SDPA_BWD_UNSUPPORTED.
 *   bias_batch  1 (one bias shared by every batch entry) or B; another value gives
 *               SDPA_BWD_INVALID_ARG.
 *   dbias       (bias_batch, Hq, Sq, Skv) fp32 device output, 4-byte aligned, or NULL (needs bias,
 *               else SDPA_BWD_INVALID_ARG): dBias = dS, the unscaled softmax VJP, 0 on masked
 *               pairs and padded rows/keys; every element is overwritten.  With bias_batch = 1 and
 *               B > 1 it sums over the batch entries through fp32 atomics, so it is not bitwise
 *               reproducible, and the deterministic dQ routes then give SDPA_BWD_UNSUPPORTED
 *               (use a per-batch bias).  Otherwise each element is written once (reproducible).
 *   dbias_io    0: dbias holds fp32 elements (above).  1: dbias holds elements of the io type
 *               (dtype), 2-byte aligned ("The kernel chain" dbias_cvt, "Support surface" bias: an
 *               io-dtype output adds a cast).  Each element is the fp32 dBias rounded once to the
 *               io type: written directly by the main kernel when it is written once (a per-batch
 *               bias, or B == 1); for a bias summed over the batch (bias_batch == 1, B > 1) it is
 *               accumulated in fp32 in the workspace (Hq*Sq*Skv floats, 256-byte aligned, after
 *               the other pieces) and rounded by the dbias_cvt kernel right after the main kernel
 *               (inside the main kernel's event interval).  Read only when dbias is not NULL.
 * With a bias the key tile depends on the bias (256 keys with an io-type bias staged in LDS at
 * kernel head dims up to 128, else 128), so the workspace can differ from the one
 * sdpa_bwd_workspace_size reports: size it with sdpa_bwd_run_workspace_size. */
typedef struct sdpa_bwd_args {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Sq, Skv, Dqk, Dv;
  float scale;
  int causal, causal_bottom_right, window_left, window_right;
  int deterministic;
  const int* seq_q_lens;
  const int* seq_kv_lens;
  const sdpa_bwd_layout* layouts;
  int dtype;
  const float* sink;
  float* dsink;
  const void* bias;
  int bias_dtype;
  int bias_batch;
  float* dbias;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
  void* const* events;
  int dbias_io;
} sdpa_bwd_args;

/* The superset entry point: everything sdpa_bwd_flex does, plus the sink gradient.  Same
 * validation, workspace (sdpa_bwd_workspace_size; dsink needs none), stream and status rules;
 * args NULL gives SDPA_BWD_INVALID_ARG. */
int sdpa_bwd_run(const sdpa_bwd_args* args);

/* Bytes of workspace sdpa_bwd_run needs for these arguments (the workspace, workspace_bytes,
 * stream and events fields are not read); 0 for arguments it rejects and for empty problems. */
size_t sdpa_bwd_run_workspace_size(const sdpa_bwd_args* args);

/* The dQ route sdpa_bwd_run takes for these arguments (values as for sdpa_bwd_dq_route; with a
 * bias held in registers the 128-key tiles can change the choice of `deterministic` = 1); -1 for
 * arguments it rejects by size or head dim, an unknown `deterministic` value, or args NULL.
 * Host only. */
int sdpa_bwd_run_dq_route(const sdpa_bwd_args* args);

/* NVFP4 attention-QAT backward ("NVFP4 Attention QAT Backward", "Overview", "Tensor contract",
 * "Current support and limitations").  Q, K and V are fake-quantised to NVFP4 (every 16
 * consecutive head-dim values: E2M1 values times one E4M3 scale E4M3(amax / 6), round to nearest
 * even after correctly rounded fp32 divisions, then dequantised) into bf16 copies Q^, K^, V^ in the
 * workspace, and the chain computes
 *     P = softmax(scale Q^ K^T),  dS = P * (dO V^T - rowsum(o_hp * dO)),
 *     dq = scale dS K^,  dk = scale dS^T Q^   (unquantised P: straight-through estimator),
 *     dv = fake_nvfp4(P)^T dO                 (P fake-quantised in groups of 16 consecutive keys of a
 *                                              row, after masking)
 * o_hp is the forward's softmax(scale Q^ K^T) V^ before any probability quantisation, lse its
 * natural-log statistic (B, H, Sq) fp32.  Tensors: contiguous (B, H, S, 128) bf16 device buffers
 * (q, o_hp, dO, dq with Sq rows; k, v, dk, dv with Skv rows), 16-byte aligned.  Supported: MHA,
 * D = 128 (else SDPA_BWD_UNSUPPORTED), causal only with Sq == Skv (top-left, self-attention; else
 * SDPA_BWD_UNSUPPORTED), non-causal cross-attention with any lengths.  scale <= 0 selects
 * 1/sqrt(128).  `deterministic` selects the dQ route as for sdpa_bwd.  The workspace (256-byte
 * aligned, at least sdpa_bwd_nvfp4_qat_workspace_size() bytes) holds Q^, K^, V^ first, then the
 * chain's buffers.  Validation happens before any launch; the work is ordered on `stream`.
 * `events` (or NULL) are the five stage events of sdpa_bwd_ex_events, recorded around the chain
 * after the quantisation. */
int sdpa_bwd_nvfp4_qat(const void* q, const void* k, const void* v, const void* o_hp,
                       const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                       int H, int Sq, int Skv, int D, float scale, int causal, int deterministic,
                       void* workspace, size_t workspace_bytes, void* stream,
                       void* const* events);
/* Bytes of workspace sdpa_bwd_nvfp4_qat needs; 0 for rejected arguments and empty problems. */
size_t sdpa_bwd_nvfp4_qat_workspace_size(int B, int H, int Sq, int Skv, int D, int causal,
                                         int deterministic);

/* Step 1 of the chain alone ("The kernel chain", dot), as the chain runs it: for every query row
 * (rows padded to Sq_pad = Sq rounded up to 32 per (b, h)) write the pair
 *     stats[(b*Hq + h)*Sq_pad + s] = { LSE * log2(e),  rowsum(O * dO) in fp32 }
 * and { +inf, 0 } for padding rows, rows at or past seq_q_lens[b] and rows whose LSE is -inf.
 * When dq_accum is not NULL, also zero its rows s < seq_q_lens[b] (all Sq rows when seq_q_lens is
 * NULL), Dqk floats each: the main kernel adds into no other row and the chain writes the other
 * rows of dQ as zeros without reading them.  stats holds B*Hq*Sq_pad*2
 * floats.  (Dqk, Dv) as for sdpa_bwd; o, dO, stats, dq_accum 16-byte aligned, lse 4-byte
 * aligned. */
int sdpa_bwd_preprocess(const void* o, const void* dO, const float* lse, float* stats,
                        float* dq_accum, const int* seq_q_lens, int B, int Hq, int Sq, int Dv,
                        int Dqk, void* stream);

/* Human-readable name of a status code (static storage). */
const char* sdpa_bwd_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_BWD_H */
