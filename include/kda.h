/* kda.h -- C ABI of the MI355X (gfx950) KDA / gated-delta-rule decode library.
 *
 * The library runs one Kimi Delta Attention layer, or a pre-norm residual stack of them,
 * for three call shapes: a one-token decode step, a multi-token verify with a later
 * commit of an accepted prefix, and a chunked prefill.  The step it computes is the
 * list under "Where the time goes" in "Thirty tiny kernels per layer: a 16% decode win
 * for GLM-5.3-Flash on Apple Silicon" (frederic.ai), written there as the pure function
 * (x, conv_state, state) -> (out, new_conv_state, new_state):
 *   p = [W_q u; W_k u; W_v u]                      (u = x, or RMSNorm(x) in a stack)
 *   a = SiLU(causal depthwise conv over the last conv_k-1 tokens and p);  window <- p
 *   q_h = l2norm(a_q,h) * d_k^-1/2,  k_h = l2norm(a_k,h),  v_h = a_v,h
 *   alpha = exp(-exp(A_log[h]) * softplus(F_b F_a u + dt_bias))   (per key channel)
 *   beta_h = sigmoid((W_beta u)_h),  gate = sigmoid(G_b G_a u)
 *   S' = diag(alpha) S;  delta = beta (v - S'^T k);  S = S' + k delta^T;  o = S^T q
 *   n_h = RMSNorm(o_h) * o_norm_w * gate_h   (per head; torad-labs/llama.cpp PR #84,
 *                                             the KDA output-gate commit)
 *   out = W_o n;   stack: x <- x + out
 *
 * Conventions for every entry point:
 *  - Pointers named *_dev are HIP device memory owned by the caller; pointers named
 *    *_host are host memory owned by the caller.  The library never frees caller memory.
 *    Device pointers must be 16-byte aligned (KDA_E_ALIGN otherwise).
 *  - Calls that take a `stream` (a hipStream_t passed as void*, NULL = the null stream)
 *    are asynchronous on that stream unless stated otherwise.
 *  - Arguments are validated before anything is enqueued.  On a non-OK return nothing
 *    was enqueued and no caller buffer was modified; kda_last_error() gives detail.
 *    Device faults surface at the caller's next synchronisation.
 *  - Matrices are row-major [out][in]; a GEMV contracts along the contiguous in-dim.
 *  - One kda_model may be used by one host thread at a time.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 3

typedef enum {
  KDA_OK = 0,
  KDA_E_ARG = 1,          /* null pointer / bad enum / bad option */
  KDA_E_SHAPE = 2,        /* unsupported or inconsistent sizes */
  KDA_E_ALIGN = 3,        /* a device pointer is not 16-byte aligned */
  KDA_E_DTYPE = 4,        /* unsupported data type for this call */
  KDA_E_WORKSPACE = 5,    /* workspace / log buffer too small */
  KDA_E_HIP = 6,          /* a HIP runtime call failed */
  KDA_E_UNSUPPORTED = 7
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1, KDA_Q8_0 = 2, KDA_MXFP4 = 3 } kda_dtype;

typedef enum { KDA_OP_DECODE = 0, KDA_OP_VERIFY = 1, KDA_OP_PREFILL = 2, KDA_OP_SCAN = 3 } kda_op;

/* Forget-gate forms.  f is the gate input F_b F_a u + dt_bias.
 * KDA_GATE_KDA    per key channel: alpha = exp(-exp(A_log[h]) softplus(f))   (the workload
 *                 text's gate); F_b [H*d_k][rank_f], dt_bias [H*d_k].
 * KDA_GATE_SAFE   per key channel, lower-bounded: alpha = exp(gate_lb sigmoid(-f a[h])),
 *                 with the a_log array's value of head h used as given (not exponentiated)
 *                 and gate_lb < 0, so e^gate_lb < alpha < 1 (torad-labs/llama.cpp PR #84,
 *                 the decay-precompute commit, which writes KDA's decay as
 *                 exp(raw_lb * sigmoid(-(g * raw_a[h]))); "Thirty tiny kernels per layer"
 *                 lists a "safe gate" transform in the step).  Shapes as KDA_GATE_KDA.
 * KDA_GATE_SCALAR one gate per head (the gated delta rule's scalar gate, which the chunk_kda
 *                 commit of the same PR contrasts with KDA's per-channel gate):
 *                 alpha_h = exp(-exp(A_log[h]) softplus(f_h)) on every key channel of head
 *                 h; F_b [H][rank_f], dt_bias [H]. */
typedef enum { KDA_GATE_KDA = 0, KDA_GATE_SAFE = 1, KDA_GATE_SCALAR = 2 } kda_gate;

typedef struct kda_model kda_model;   /* opaque */

int kda_abi_version(void);
const char* kda_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* kda_last_error(void);

/* ------------------------------------------------------------------------------------
 * Weight packing.
 * KDA_F32  : [rows][cols] fp32, as given.
 * KDA_BF16 : [rows][cols] bfloat16 bit patterns, round to nearest even.
 * KDA_Q8_0 : blocks of 32 consecutive values along a row with one fp16 scale (antirez/ds4
 *            PR #964, the commit that requantises KDA's projections to Q8_0):
 *              amax = max|x|, d = fp32(amax/127), d16 = fp16_rne(d),
 *              q = clamp(round_half_away(fp32(x / d16)), -127, 127), all q = 0 if d16 = 0.
 *            Device layout: a plane of rows*cols bytes holding q+128, then (at the next
 *            256-byte boundary) a plane of rows*(cols/32) fp16 scales.  cols % 32 == 0.
 * KDA_MXFP4: one of the 4-bit block formats the quant-format commit of torad-labs/llama.cpp
 *            PR #84 ranks at the KDA projection shapes, as the OCP Microscaling (MX)
 *            specification v1.0 defines it: blocks of 32 consecutive values along a row
 *            share an E8M0 scale X = 2^s, s = floor(log2(max|x|)) - 2 (clamped to
 *            [-127, 127]; -127 for a block of zeros); each element is the E2M1 value
 *            (0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives) nearest to x / X, ties to
 *            the even mantissa bit, clamped to +-6; code = sign << 3 | grid index.
 *            Device layout: rows*cols/2 bytes of codes (codes 2i and 2i+1 of a row in
 *            byte i, low nibble first), then (at the next 256-byte boundary) a plane of
 *            rows*(cols/32) scale bytes s + 127.  cols % 32 == 0.  Decode and verify run
 *            it through the per-layer kernels (vector dots, as the page notes for one
 *            row; from 2 columns the matrix cores, after gfx950's exact scaled FP4 ->
 *            BF16 conversion); the one-launch decode of an eligible stack (see
 *            kda_model_query) takes it as the Q8_0 copy holding the same values; the
 *            chunked prefill does not take it.
 * ---------------------------------------------------------------------------------- */
/* Bytes a packed [rows][cols] matrix occupies (0 on an invalid request). */
size_t kda_packed_bytes(int dtype, int64_t rows, int64_t cols);

/* Pack fp32 src_host [rows][cols] (host memory) into dst_dev (kda_packed_bytes bytes):
 * the format is applied on the host, then the bytes are copied on `stream`; the call
 * returns once the copy is complete (synchronous), so src_host may be freed at once.
 * Errors: KDA_E_DTYPE (unknown dtype), KDA_E_SHAPE (rows/cols <= 0, Q8_0 with
 * cols % 32 != 0), KDA_E_ALIGN (dst_dev), KDA_E_HIP. */
int kda_pack(int dtype, const float* src_host, int64_t rows, int64_t cols, void* dst_dev,
             void* stream);

/* The same packing from fp32 src_dev [rows][cols] in device memory, by a kernel;
 * asynchronous on `stream`.  Bit-identical to kda_pack. */
int kda_pack_device(int dtype, const float* src_dev, int64_t rows, int64_t cols, void* dst_dev,
                    void* stream);

/* Canonical view of a Q8_0-packed matrix in host memory: d16_host [rows][cols/32] fp16 bit
 * patterns and qs_host [rows][cols] int8.  Synchronous: the packed bytes are copied back
 * on `stream` and unpacked on the host before the call returns. */
int kda_unpack_q8_0(const void* packed_dev, int64_t rows, int64_t cols, uint16_t* d16_host,
                    int8_t* qs_host, void* stream);

/* Canonical view of an MXFP4-packed matrix in host memory: e8m0_host [rows][cols/32] (the
 * scale bytes s + 127) and codes_host [rows][cols] (one 4-bit code a byte).  Synchronous. */
int kda_unpack_mxfp4(const void* packed_dev, int64_t rows, int64_t cols, uint8_t* e8m0_host,
                     uint8_t* codes_host, void* stream);

/* The same view written to device memory (d16_dev, qs_dev), asynchronous on `stream`. */
int kda_unpack_q8_0_device(const void* packed_dev, int64_t rows, int64_t cols,
                           uint16_t* d16_dev, int8_t* qs_dev, void* stream);

/* ------------------------------------------------------------------------------------
 * Model description.  The library keeps the pointers; it does not copy weights.
 * ---------------------------------------------------------------------------------- */
typedef struct {
  int32_t d_model;           /* D */
  int32_t n_heads;           /* H */
  int32_t d_k;               /* 64 or 128 */
  int32_t d_v;               /* == d_k */
  int32_t conv_k;            /* 4 */
  int32_t rank_f;            /* low rank of the forget gate (F_a: [rank_f][D]) */
  int32_t rank_g;            /* low rank of the output gate (G_a: [rank_g][D]) */
  int32_t n_layers;
  int32_t prenorm_residual;  /* 0: y = layer(x); 1: x <- x + layer(RMSNorm(x)) per layer */
  float norm_eps;            /* RMSNorm eps (pre-norm and output norm) */
  float l2_eps;              /* q/k L2-norm eps: x / sqrt(sum x^2 + l2_eps) */
  int32_t wtype;             /* kda_dtype of every projection matrix */
  int32_t gate;              /* kda_gate: forget-gate form (0 = KDA) */
  float gate_lb;             /* KDA_GATE_SAFE: lower bound of log(alpha), < 0 (else unused) */
} kda_dims;

typedef struct {
  /* packed by kda_pack with dims.wtype; shapes [out][in]:
   * wq, wk: [H*d_k][D]  wv: [H*d_v][D]  wo: [D][H*d_v]  fa: [rank_f][D]
   * fb: [H*d_k][rank_f] ([H][rank_f] for KDA_GATE_SCALAR)  wbeta: [H][D]
   * ga: [rank_g][D]  gb: [H*d_v][rank_g] */
  const void *wq, *wk, *wv, *wo, *fa, *fb, *wbeta, *ga, *gb;
  const float* conv_w;    /* [C][conv_k] fp32, C = 2*H*d_k + H*d_v; tap conv_k-1 = current */
  const float* a_log;     /* [H] (KDA_GATE_SAFE: the per-head factor a, used as given) */
  const float* dt_bias;   /* [H*d_k] ([H] for KDA_GATE_SCALAR) */
  const float* o_norm_w;  /* [d_v] or NULL (ones) */
} kda_layer;

/* Recurrent state of all layers for `batch` sequences. */
typedef struct {
  float* S_dev;     /* [n_layers][batch][H][d_k][d_v] fp32, row = key channel */
  float* conv_dev;  /* [n_layers][batch][conv_k-1][C] fp32, oldest token first */
  int32_t batch;
} kda_state;

/* Create a model over caller-owned packed weights (layers[n_layers]).
 * Ownership: a Q8_0 KDA-gate model eligible for the one-launch decode (kda_model_query,
 * KDA_Q_OWNS_WEIGHTS = 1) copies every packed matrix into its own matrix-core order
 * during this call, and every kernel of every call on it reads only that copy: the
 * caller's packed buffers (wq .. gb) may be freed or reused once this call has returned,
 * so the weights sit in device memory once.  Any other model reads the caller's packed
 * buffers in every call (an eligible MXFP4, safe- or scalar-gate model too, in its
 * per-layer kernels; its one-launch decode reads a copy of its own), and they must stay
 * valid and unchanged until kda_model_destroy.  conv_w, a_log, dt_bias and o_norm_w are always read from the
 * caller's buffers.  Errors: KDA_E_ARG, KDA_E_SHAPE (d_k != d_v, d_k not 64/128,
 * conv_k != 4, D % 32, ranks % 32 for Q8_0, ...), KDA_E_ALIGN, KDA_E_HIP. */
int kda_model_create(const kda_dims* dims, const kda_layer* layers, kda_model** out);
void kda_model_destroy(kda_model* m);

/* Options. */
typedef enum {
  KDA_OPT_GRAPH = 0,       /* 1: decode, verify and commit replay a captured hipGraph of
                              all layers, re-captured when a pointer or the batch changes;
                              0 (default): the same kernels launched directly.  On MI355X
                              with ROCm 7.2 a replay measured no faster than the launches
                              (a single layer 2x slower a token, 34 layers 0.7-1.4 %
                              slower); it is for callers that need a fixed host cost a
                              step.  The one-launch decode never uses a graph. */
  KDA_OPT_TIMING = 1,      /* 1: record hipEvents around every kernel launch (no graph) */
  KDA_OPT_PERSISTENT = 2,  /* 1 (default): batch-1 decode of an eligible model runs every
                              layer in one launch (see kda_model_query) */
  KDA_OPT_WAIT_US = 3,     /* bound of every wait between blocks of the one-launch decode, in
                              microseconds of wall clock; <= 0 (default) = 50 ms.  A step
                              whose wait runs out leaves through the bound and
                              kda_model_status reports it; limits under 100 us make the waits
                              look at the clock after every poll round (for exercising that
                              path) */
  KDA_OPT_COOPERATIVE = 4  /* 0 (default): the one-launch decode is a plain launch of one
                              block per CU, co-resident when the stream has the GPU to itself;
                              on a GPU shared with other work a block that cannot start leaves
                              the rest to their bounded waits and kda_model_status reports the
                              step.  1: a cooperative launch, which guarantees co-residency
                              and costs ~17 us more per step */
} kda_option;
int kda_model_set_option(kda_model* m, int option, int64_t value);

/* Queries.  KDA_Q_OWNS_WEIGHTS: 1 if the model reads only its own copy of the packed
 * matrices (see kda_model_create), else 0.
 * KDA_Q_PERSISTENT: number of blocks of the one-launch decode, 0 if the model is
 * not eligible (it needs Q8_0 weights, or MXFP4 weights whose nonzero blocks all have a
 * scale 2^(e - 127) with e - 128 in [-24, 15], any of the three gate forms, a pre-norm
 * residual stack, d_k = d_v = 128,
 * H*d_v = D in {1024, 2048}, rank_f = rank_g in {32, 64, 128}, H <= 32, and one
 * co-resident block per CU with 2 H + D/32 + C/48 + ceil((proj_rows - C)/16) <= CUs).  For it kda_model_create allocates
 * ~130 KB of exchange words, flags and layer table, and a copy of every layer's projection
 * rows, W_o, F_b and G_b rearranged for the matrix cores (about
 * (D*(proj_rows + D) + 2*D*rank)*17/16 bytes per layer; 19.0 MB at D = 2048, rank 128;
 * MXFP4 matrices enter it as the Q8_0 holding the same values, twice each E2M1 value as
 * the int8 code and half the block scale as the fp16 one; the scalar gate's one F_b row
 * and dt_bias a head enter repeated over the head's d_k channels): for a Q8_0 KDA-gate
 * stack the one-launch decode and every per-layer kernel read that copy
 * (KDA_Q_OWNS_WEIGHTS), for MXFP4 or the other gate forms the one-launch decode alone, so
 * later changes to the caller's weights reach it only through a new model. */
typedef enum { KDA_Q_PERSISTENT = 0, KDA_Q_OWNS_WEIGHTS = 1 } kda_query;
int kda_model_query(const kda_model* m, int what);

/* Synchronises the device and reports whether a one-launch decode since the last call hit
 * its bounded wait between blocks (KDA_E_HIP; that step's outputs and state are invalid
 * and the exchange buffers are reset).  KDA_OK otherwise.
 * Such a step leaves its error word set until this call: the one-launch kernel leaves at
 * once, touching nothing, in every step enqueued after the failed one, and once the host
 * can see the word (after the failed step has completed, e.g. at the caller's next
 * synchronisation) kda_decode_step, kda_verify_steps, kda_verify_commit,
 * kda_prefill_chunked and kda_conv_window_canonical refuse with KDA_E_HIP and enqueue
 * nothing.  A caller must therefore call kda_model_status after such a refusal (and should
 * before trusting a state after a step that ran with a short KDA_OPT_WAIT_US). */
int kda_model_status(kda_model* m);

/* Kernel kinds reported by kda_timing_query. */
typedef enum { KDA_K_PROJ = 0, KDA_K_HEAD = 1, KDA_K_OUT = 2, KDA_K_COMMIT = 3,
               KDA_K_PREFILL = 4, KDA_K_GATES = 5, KDA_K_STEP = 6, KDA_K_GEMM = 7,
               KDA_K_CHUNK = 8, KDA_K_COUNT = 9 } kda_kernel_kind;
/* Sum of event-timed durations (ms) and launch count per kernel kind since the last
 * reset; synchronises on the recorded events.  reset != 0 clears the counters. */
int kda_timing_query(kda_model* m, int kind, double* total_ms, int64_t* launches, int reset);

/* Measurement utility (not part of the step): the device's sequential-read ceiling.
 * Reads `bytes` of buf_dev (16-byte aligned; its first 4 bytes per block may be
 * overwritten with a checksum in the rare case it takes one value) `reps` times after one
 * warm-up read, with 4 blocks per CU of 16-byte non-temporal loads, and returns the mean
 * milliseconds per read in *ms_per_read (hipEvents on `stream`; synchronous).  A buffer
 * larger than the 256 MB last-level cache measures HBM.  Errors: KDA_E_ARG, KDA_E_ALIGN,
 * KDA_E_HIP. */
int kda_stream_read_probe(const void* buf_dev, size_t bytes, int reps, void* stream,
                          float* ms_per_read);

/* Device workspace bytes an op needs for `batch` sequences and `tokens` tokens each
 * (decode: tokens = 1; verify: T; prefill: L). */
size_t kda_workspace_bytes(const kda_model* m, int op, int32_t batch, int64_t tokens);

/* One decode token for every sequence of the batch (the pure step above, on all layers).
 * x_dev [B][D] fp32 in, y_dev [B][D] fp32 out (layer output, or the final residual
 * stream of a stack); st is read and advanced in place.  x_dev and y_dev must not
 * overlap.  Errors: KDA_E_ARG, KDA_E_ALIGN, KDA_E_SHAPE (st->batch < 1),
 * KDA_E_WORKSPACE, KDA_E_HIP. */
int kda_decode_step(kda_model* m, const float* x_dev, float* y_dev, const kda_state* st,
                    void* ws_dev, size_t ws_bytes, void* stream);

/* kda_decode_step for callers that cannot allocate device memory (code under hipGraph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same step, with its
 * workspace in a static device array of the library (8 MiB per GPU, held by the process
 * until it ends) instead of a caller's buffer.  It calls no hipMalloc, hipFree or other
 * allocating routine: the kernels run as plain launches (no graph of the library's own, no
 * timing events).  Every call on one GPU shares that array, which keeps the last call's
 * contents; no part of it needs to start at zero.  Calls that overlap on one GPU (two
 * streams, two threads, two models) race on it: serialise them.  Errors as
 * kda_decode_step, and KDA_E_WORKSPACE when the batch needs more than the array holds
 * (kda_workspace_bytes(m, KDA_OP_DECODE, batch, 1) > 8 MiB). */
int kda_decode_step_static(kda_model* m, const float* x_dev, float* y_dev, const kda_state* st,
                           void* stream);

/* Batched decode with ragged or left-padded sequences ("Thirty tiny kernels per layer",
 * section "Taking it upstream, and finding out why it's worth less there": a left-padded
 * batch mask and ragged per-row lengths).  active_dev: device int32 [B]; a sequence with
 * active_dev[b] == 0 takes no token this step: its state and conv window are left exactly
 * as they were (bit for bit), and its y_dev row is the layer (stack) output its x_dev row
 * would have had (computed from the unchanged state; callers normally ignore it).  A
 * sequence with a nonzero entry is decoded exactly as by kda_decode_step.  Left padding is
 * a mask that is 0 until a sequence's first token, ragged lengths one that is 0 after its
 * last.  Runs the per-layer kernels (never the one-launch kernel); with KDA_OPT_GRAPH = 1
 * they replay as a hipGraph keyed also on active_dev.  Errors as kda_decode_step, KDA_E_ARG for a null mask and
 * KDA_E_ALIGN for a mask that is not 4-byte aligned. */
int kda_decode_step_masked(kda_model* m, const float* x_dev, float* y_dev, const kda_state* st,
                           const int32_t* active_dev, void* ws_dev, size_t ws_bytes,
                           void* stream);

/* Verify (multi-token, read-only on the state): T tokens per sequence, x_dev [B][T][D],
 * run in order through every layer from the state in st.  Writes y_dev [B][T][D] for
 * every token and a replay log that kda_verify_commit uses.  The read-only verify and the
 * later commit of an accepted prefix are the verify / commit-after-k modes of the gdn_step
 * kernel in the regolith GDN audit (opus_gdn_qsa, section 2).  1 <= T <= 8.
 *
 * Folded commit.  kda_verify_commit only records the accepted lengths; the next
 * kda_verify_steps on the same state and log applies them first, inside its own kernels:
 * per (sequence, layer, head) the state is read once, the accepted tokens of the previous
 * verify are replayed from the log, the state is written once, and the new tokens run from
 * it in registers; the conv window moves on in the projection kernel the same way.  So the
 * state is read once and written once per step, and st holds the state after the last
 * applied commit.  Every other call that reads or writes st (kda_decode_step and its
 * variants, kda_prefill_scan, kda_prefill_chunked, kda_conv_window_canonical) and
 * kda_state_flush apply a pending commit first, and a verify on st through another log
 * applies that log's; a verify of another state through the same log applies a commit
 * pending in it first.  A caller that reads st's buffers itself, copies them (a snapshot)
 * or frees them, or frees or reuses the log, calls kda_state_flush first (and synchronises
 * as for any asynchronous call).
 *
 * log_dev: device memory of log_bytes >= kda_verify_log_bytes(m, B, T), 16-byte aligned,
 * owned by the caller and left to the library between a verify and the call that applies
 * its commit: a header of the accepted lengths ([B] int32) and two halves that
 * consecutive verifies alternate (the one being written, the one whose commit is folded
 * in), each holding per layer the pre-conv projections, alpha and gate, and the activated
 * q|k|v of the B*T tokens.  A commit must follow the verify it commits on that state and
 * log, with no call that writes st in between (such a call retires the verify).  Errors:
 * KDA_E_ARG, KDA_E_ALIGN, KDA_E_SHAPE, KDA_E_WORKSPACE (log or workspace too small; a log
 * sized for T serves every T' <= T), KDA_E_HIP; after a failed call the state is
 * undefined. */
size_t kda_verify_log_bytes(const kda_model* m, int32_t batch, int32_t T);
int kda_verify_steps(kda_model* m, const float* x_dev, int32_t T, float* y_dev,
                     const kda_state* st, void* log_dev, size_t log_bytes, void* ws_dev,
                     size_t ws_bytes, void* stream);
/* Commit: st becomes the state and conv window reached after accept_dev[b] tokens (device
 * int32 [B], each in 1..T) of the last kda_verify_steps on this state and log; the result
 * equals decoding those tokens.  Recorded, not run: the lengths are copied into the log
 * header on `stream` (accept_dev may be reused once the stream has passed this call) and
 * applied by the next call on st (above).  T must be the verify's T and log_bytes the size
 * it was given.  KDA_E_ARG if no verify of T tokens on this state and log waits for a
 * commit (none made, one already committed, or retired by a call that wrote st); at most
 * 64 commits may be pending on one model.  The accept lengths are device data, which the
 * host cannot read without a synchronisation: the kernels clamp a value outside 1..T to
 * that range. */
int kda_verify_commit(kda_model* m, const kda_state* st, const void* log_dev, size_t log_bytes,
                      int32_t T, const int32_t* accept_dev, void* stream);
/* Apply the commit pending on st, if any (the replay of the accepted tokens into the
 * state and the window, enqueued on `stream`); nothing to do otherwise.  Needed before the
 * caller reads, copies or frees st's buffers or the log itself.  Errors: KDA_E_ARG,
 * KDA_E_ALIGN, KDA_E_HIP. */
int kda_state_flush(kda_model* m, const kda_state* st, void* stream);

/* Sequential-scan prefill of L tokens per sequence, for prompts too short for the
 * chunked form to pay (the sequential prompt scan gdn_scan_r of the regolith audit
 * opus_gdn_qsa, section 3): every layer of any model (any weight format and gate form,
 * a single layer or a pre-norm stack, any batch) runs the tokens in order, layer by layer
 * over blocks of Tc tokens (B * Tc <= 64): the projections of a block's B * Tc token
 * columns in one pass over the weights, then per (sequence, head, 32 value columns) one
 * wave holds its state tile in registers across the block's tokens (one read and one
 * write of the state per block, two register passes per token), then the output
 * projection.  The window is rolled by the block's tokens in the same launch.
 * x_dev [B][L][D] fp32 in, y_dev [B][L][D] fp32 out (layer output, or the final
 * residual stream of a stack); st is read as the initial state and advanced to the state
 * after all L tokens.  The result equals L calls of kda_decode_step.  Workspace:
 * kda_workspace_bytes(m, KDA_OP_SCAN, B, L).  Errors: KDA_E_ARG, KDA_E_ALIGN,
 * KDA_E_SHAPE (L < 1), KDA_E_WORKSPACE, KDA_E_HIP. */
int kda_prefill_scan(kda_model* m, const float* x_dev, int64_t L, float* y_dev,
                     const kda_state* st, void* ws_dev, size_t ws_bytes, void* stream);

/* The conv windows of every layer and sequence in the canonical layout
 * out_dev [n_layers][B][conv_k - 1][C] fp32, oldest token first (the "conv_state" of the
 * pure decode step in "Thirty tiny kernels per layer", section "Why mx.compile fits here
 * and not elsewhere").  Asynchronous device-to-device copy on `stream`, after a pending
 * commit on st is applied. */
int kda_conv_window_canonical(kda_model* m, const kda_state* st, float* out_dev, void* stream);

/* Chunked prefill of L tokens per sequence through a single-layer model (n_layers == 1,
 * prenorm_residual == 0): x_dev [B][L][D] (x_dtype KDA_BF16 bit patterns or KDA_F32),
 * y_dev [B][L][D] fp32; st is read as the initial state and overwritten with the final
 * state and window.  The delta rule runs in the chunked WY/UT form of the chunk_kda
 * commit of torad-labs/llama.cpp PR #84 with an fp32 state carried across chunks;
 * chunk must be 64.  Any L >= 1 (partial last chunk allowed).  Needs BF16 weights,
 * rank_f of 64 or 128, and D, rank_g and H*d_v multiples of 64 (KDA_E_SHAPE,
 * KDA_E_DTYPE otherwise).  The products run on matrix cores with fp32 operands split into
 * two BF16 terms (about 16 significant bits per product, fp32 accumulation). */
int kda_prefill_chunked(kda_model* m, const void* x_dev, int x_dtype, int64_t L,
                        int32_t chunk, float* y_dev, const kda_state* st, void* ws_dev,
                        size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
