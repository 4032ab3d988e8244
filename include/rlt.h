/*
 * rlt.h - C ABI of the Recurrent Looped Transformer decoder-step library
 * (librlt.so, HIP, gfx950).
 *
 * The library computes the recurrent decoder state transition
 *     H_{t-1} = (s_{t-1}, C_{t-1})  ->  H_t = (s_t, C_t),  logits_t = W_o RMSNorm_o(s_t)
 * for a batch of independent sequences, each at its own position.
 *
 * Pages this follows (cited by title):
 *   [Tutorial]  "Understanding and Applying the Recurrent Looped Transformer
 *               Architecture": "How the Architecture Works" (H_t, H_0, the
 *               state-transition equation, the next-token distribution),
 *               "Three forms of context", "Basic Usage", "Prompt prefill",
 *               "Autoregressive generation", "Advanced Implementation Tips".
 *   [Princeton] "Princeton Researcher Proposes Recurrent Looped Transformer to
 *               Carry Decoder State Across Tokens": architecture paragraph
 *               (gated merge, block contents, memory groups, window), design
 *               principles paragraph (batching independent sequences),
 *               training/serving paragraph (prefix snapshot contents).
 *   [Article]   "Recurrent Looped Transformer: A New Architecture for Infinite
 *               Context Reasoning in Language Models": "The Recurrent Decoder
 *               State", "The Critical Boundary", "Multi-Turn Serving".
 *
 * One step, per sequence consuming token t (t = 1 is BOS):
 *   g   = sigmoid(W_g [e_t ; s_{t-1}] + b_g);  x = g*e_t + (1-g)*s_{t-1}
 *   per layer l = 0..L-1 (pre-RMSNorm, residual adds):
 *     x += W_O  SWA(W_Q a, W_K a, W_V a),  a = RMSNorm(x; g1[l])
 *          window: positions max(1, t-W+1)..t, current token included
 *     x += W_Oc Attn(W_Qc RMSNorm(x; g2[l]), memory group g(l), positions 1..t)
 *     x += W_2 GELU(W_1 RMSNorm(x; g3[l]))
 *   s_t = x;  logits = W_o RMSNorm(s_t; g_o)
 * The gate formula, the pre-norm block layout, RMSNorm eps, the exact (erf)
 * GELU, and "no positional encoding besides the window and memory bounds" are
 * readings where the pages leave the step open.  Attention scale 1/sqrt(dh).
 *
 * Precision: dtype RLT_DTYPE_F32 computes and stores everything in fp32.
 * RLT_DTYPE_BF16 stores weights, e_t, encoder memory, the decoder window cache,
 * q/k/v, attention outputs, normalised GEMM inputs and the FFN hidden layer in
 * bf16 (round to nearest even); accumulation, softmax, the residual stream,
 * s_t and logits are fp32.
 *
 * Conventions for every function below:
 *   - All device memory is owned by the caller.  The library only lays out
 *     the buffers it is given (sizes from the *_bytes queries) and never
 *     allocates device memory.  Handles hold host-side metadata only.
 *   - Pointers named dev_* are device pointers; host_* are host pointers.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call that
 *     takes a stream only enqueues work on it and returns; nothing
 *     synchronises except rlt_state_import (see there).  Inputs must stay
 *     valid until the stream has passed the enqueued work.
 *   - Functions return rlt_status and never throw.  All validation happens on
 *     the host before any device work, so a call that fails has no effect.
 *     A detail message for the calling thread is in rlt_last_error().
 *   - A model may be shared by several states and streams.  One state must be
 *     used by one stream at a time; calls on one state that overlap race.
 */
#ifndef RLT_H
#define RLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RLT_ABI_VERSION 4

typedef enum {
  RLT_OK = 0,
  RLT_ERR_INVALID_ARG = 1,   /* null pointer, bad count, duplicate or out-of-range slot */
  RLT_ERR_SHAPE = 2,         /* buffer too small, dimension not supported by the layout */
  RLT_ERR_RANGE = 3,         /* a position would pass the memory capacity or max_tokens */
  RLT_ERR_STALE = 4,         /* state built for another model version: weights changed,
                                caches are invalid [Article, "Multi-Turn Serving"] */
  RLT_ERR_CONVENTION = 5,    /* snapshot of another shape / window / dtype / version */
  RLT_ERR_UNSUPPORTED = 6,   /* configuration the kernels do not implement */
  RLT_ERR_DEVICE = 7         /* a HIP call failed (also: an earlier asynchronous fault) */
} rlt_status;

enum { RLT_DTYPE_F32 = 0, RLT_DTYPE_BF16 = 1 };
enum { RLT_LOGITS_ALL = 0, RLT_LOGITS_LAST = 1, RLT_LOGITS_NONE = 2 };

/* Model dimensions.  head_dim must equal d_model / n_heads and be one of
 * 16, 32, 64, 128, 256; d_model and d_ffn must be multiples of 32;
 * mem_groups is 1 (one memory read by every layer) or n_layers (layer l reads
 * group l) [Princeton, architecture paragraph].  window >= 1 counts the
 * current token.  attn_chunk: positions an attention workgroup loads per step
 * of its double-buffered loop, spread over its 4 wavefronts, each of which
 * keeps its own running softmax (0 = the largest the kernel takes for the
 * head size: 64 positions for bf16 with head_dim 128; larger values are cut
 * to that).  It fixes the order of the softmax sums and so is part of the
 * model's numerics: a state and its model must agree on it. */
typedef struct {
  int32_t vocab, d_model, n_heads, head_dim, n_layers, d_ffn, window, mem_groups, dtype;
  float rms_eps;
  int32_t attn_chunk;
} rlt_config;

/* Canonical parameters, device pointers, row-major, torch Linear convention
 * W[out][in] (y = W x).  Matrices in the model dtype; vectors always fp32.
 * Per-layer tensors are stacked on a leading [L] axis.  Read once by
 * rlt_model_create (repacked into the model buffer); not retained. */
typedef struct {
  const void *s_star;           /* [d]       fp32: learned start state s*       */
  const void *wg;               /* [d][2d]   gate weights, input order [e ; s]  */
  const void *bg;               /* [d]       fp32 gate bias                     */
  const void *g1, *g2, *g3;     /* [L][d]    fp32 RMSNorm gains (SWA, cross, FFN) */
  const void *wq, *wk, *wv, *wo;/* [L][d][d] self-attention                     */
  const void *wqc, *woc;        /* [L][d][d] cross-attention query / output     */
  const void *w1;               /* [L][F][d] FFN up                             */
  const void *w2;               /* [L][d][F] FFN down                           */
  const void *go;               /* [d]       fp32 output RMSNorm gain           */
  const void *wout;             /* [V][d]    output head                        */
} rlt_params;

/* Encoder memory M (read only, caller owned), already split per head:
 * element (group g, sequence j, head h, position p (0-based), c) is at
 * k[g*stride_group + j*stride_seq + h*stride_head + p*stride_pos + c]
 * (strides in elements, head_dim contiguous, model dtype).  Sequence index
 * j = state slot.  Entries 0..t-1 of a slot must be valid before the step that
 * consumes its token t [Tutorial, "Three forms of context": memory is read only
 * through the current position]. */
typedef struct {
  const void *k, *v;
  int64_t stride_group, stride_seq, stride_head, stride_pos;
  int32_t capacity;             /* positions available per sequence            */
  int32_t n_seq;                /* sequences available (> every slot used)     */
  int32_t n_groups;             /* groups available (>= mem_groups)            */
} rlt_memory;

typedef struct rlt_model rlt_model;
typedef struct rlt_state rlt_state;

int32_t     rlt_abi_version(void);
const char *rlt_status_str(rlt_status s);
const char *rlt_last_error(void);          /* thread-local; "" if none */

/* ------------------------------------------------------------------ model */
/* Bytes of device memory a model needs (0 if the config is invalid): the
 * decoder's parameters -- gate W_g, b_g and s*; per layer the three RMSNorm
 * gains, W_Q, W_K, W_V, W_O, W_Qc, W_Oc, W_1, W_2; the output norm and head
 * [Princeton, architecture; Tutorial, "How the Architecture Works"] -- in the
 * packed tile layout the kernels read. */
size_t rlt_model_bytes(const rlt_config *cfg);

/* Validate cfg, repack `src` into dev_buf (>= rlt_model_bytes, 256-byte
 * aligned) with kernels on `stream`, and return a host handle in *out.
 * model_version tags every state made from this model: a state is valid only
 * under the weights that produced it, and a call with a state of another
 * version fails with RLT_ERR_STALE [Tutorial, "Current-Policy Reinforcement
 * Learning Replay": states are rebuilt under the current weights]. */
rlt_status rlt_model_create(const rlt_config *cfg, const rlt_params *src,
                            uint64_t model_version, void *dev_buf, size_t bytes,
                            void *stream, rlt_model **out);
void rlt_model_destroy(rlt_model *m);       /* frees the host handle only */

/* ------------------------------------------------------------------ state */
/* The state of a sequence is H_t = (s_t, C_t): the decoder output carried to
 * the next token's gate and the window cache of every layer [Tutorial, "How
 * the Architecture Works": the state and its transition; Article, "The
 * Recurrent Decoder State"].
 * Bytes for a state of `batch` slots whose positions stay <= max_tokens
 * (max_tokens is checked by the calls, it does not change the size): s [B][d]
 * fp32, positions [B] int32, the window cache K,V [L][B][H][W][dh] in the
 * model dtype (a ring: position p lives in entry (p-1) mod W), and the
 * per-step scratch the kernels use (residual stream, normalised GEMM inputs,
 * attention outputs, FFN hidden layer, sum-of-squares partials). */
size_t rlt_state_bytes(const rlt_config *cfg, int32_t batch, int32_t max_tokens);

/* Lay out a state in dev_buf and set every slot to H_0 = (s*, empty cache),
 * position 0 [Tutorial, "How the Architecture Works": initial state]. */
rlt_status rlt_state_init(const rlt_model *m, int32_t batch, int32_t max_tokens,
                          void *dev_buf, size_t bytes, void *stream, rlt_state **out);
void rlt_state_destroy(rlt_state *st);

/* Return the listed slots to H_0.  For a document boundary only: the prompt /
 * response boundary is never a reset [Article, "The Critical Boundary"]. */
rlt_status rlt_state_reset(const rlt_model *m, rlt_state *st, int32_t n,
                           const int32_t *host_slots, void *stream);

/* One decoder step for n listed slots (host_slots NULL = slots 0..n-1):
 *   dev_e      [n][d] model dtype, row i = e_t of slot host_slots[i]
 *   mem        encoder memory (sequence index = slot)
 *   dev_logits [n][V] fp32 out (may be NULL: no logits; the state still advances)
 * Each listed slot consumes exactly one token and its position advances by 1
 * [Tutorial, "Autoregressive generation"].  Slots must be distinct.  Results
 * for a slot do not depend on which other slots share the call. */
rlt_status rlt_decoder_step(const rlt_model *m, rlt_state *st, int32_t n,
                            const int32_t *host_slots, const void *dev_e,
                            const rlt_memory *mem, float *dev_logits, void *stream);

/* rlt_decoder_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, kernels and results (bitwise), but the per-step working
 * memory -- residual stream, sum-of-squares partials, packed normed GEMM
 * inputs, q, attention output, FFN hidden layer, staged slot list and row
 * order -- lives in a static array of 16 MiB per device that the library holds
 * until the process ends, instead of in the state's scratch region.  It calls
 * no allocating routine.  Every call on one device shares that array: calls
 * that overlap on one GPU (two streams, or two host threads) race and must
 * not be issued; calls in stream order are safe, and nothing in the array
 * needs to start at zero.  The model's device must be current on the first
 * call on that device.  Errors: those of rlt_decoder_step, plus RLT_ERR_RANGE
 * when the n rows need more than the 16 MiB, with no side effects.  The need
 * is about n * (8 + 4.25 d + 3 es d + es F) bytes (es = 2 for bf16, 4 for
 * fp32; packed buffers round n up to 16 rows): up to 448 rows at d = 2048,
 * F = 8192 and 224 rows at d = 4096, F = 16384 in bf16. */
rlt_status rlt_decoder_step_noalloc(const rlt_model *m, rlt_state *st, int32_t n,
                                    const int32_t *host_slots, const void *dev_e,
                                    const rlt_memory *mem, float *dev_logits, void *stream);

/* T steps for all B slots with no reset anywhere (prompt prefill and decode are
 * the same transition) [Tutorial, "Prompt prefill"; Article, "The Critical
 * Boundary"].  dev_e [B][T][d]; logits: RLT_LOGITS_ALL -> [B][T][V],
 * RLT_LOGITS_LAST -> [B][V] of the last step, RLT_LOGITS_NONE -> none (NULL ok).
 * Bitwise identical to T calls of rlt_decoder_step on all slots. */
rlt_status rlt_run_sequence(const rlt_model *m, rlt_state *st, int32_t T,
                            const void *dev_e, const rlt_memory *mem, float *dev_logits,
                            int32_t logits_mode, void *stream);

/* rlt_run_sequence with each decoder step as one persistent launch: the
 * step's phases (gated merge; per layer QKV, window attention, O, Qc,
 * cross-attention, Oc, FFN-up, FFN-down; the head) run inside one cooperative
 * kernel, one workgroup per compute unit, instead of 2 + 8L separate launches
 * -- the kernel fusion the pages list among the implementation targets
 * [Princeton, design-principles paragraph; Article, "Principle 2: Co-Design
 * Between Model and Hardware"].  There is no grid barrier: each work item of a
 * phase (a GEMM tile of 16 rows, or an attention row and head) waits only for
 * the items of the phase before it that it reads, through per-item ready
 * flags, and issues its weights (or memory keys and values) before it waits.
 * Each item runs the launch chain's own per-workgroup code with the same K
 * split and summation order, so logits and state are bitwise those of
 * rlt_run_sequence.
 *   dev_workspace  caller-owned device buffer of
 *                  rlt_persistent_workspace_bytes(cfg, B) bytes (256-byte
 *                  aligned): the error word, one flag per item of a step,
 *                  the phase tables, and one output buffer per phase of a
 *                  step (no address is written twice within a launch).  It
 *                  must not be shared by calls that overlap.
 * Supported: bf16 with head_dim 32, 64, 128; fp32 with head_dim 16, 32, 64
 * (RLT_ERR_UNSUPPORTED otherwise).  Every wait is bounded (0.2 s): on timeout
 * the kernel sets an error word and every later wait returns at once, so the
 * launch ends; results are then undefined and rlt_persistent_check reports
 * RLT_ERR_DEVICE.  Other errors as rlt_run_sequence, plus RLT_ERR_SHAPE for a
 * short workspace. */
size_t rlt_persistent_workspace_bytes(const rlt_config *cfg, int32_t batch);
rlt_status rlt_run_sequence_persistent(const rlt_model *m, rlt_state *st, int32_t T,
                                       const void *dev_e, const rlt_memory *mem,
                                       float *dev_logits, int32_t logits_mode,
                                       void *dev_workspace, size_t workspace_bytes,
                                       void *stream);
/* Synchronize the stream and report whether a wait of the last
 * rlt_run_sequence_persistent call on this workspace timed out
 * (RLT_ERR_DEVICE) or not (RLT_OK).  The word is cleared by the next call. */
rlt_status rlt_persistent_check(void *dev_workspace, void *stream);
/* For tests of the time-out path only: while on (nonzero, process-wide),
 * the waits of later rlt_run_sequence_persistent calls look for an epoch
 * that no item stores, so each such call's first wait times out after its
 * bound (0.2 s), sets the error word, and the call's launches end at once;
 * rlt_persistent_check then reports RLT_ERR_DEVICE and the state's contents
 * and positions are undefined until it is reset. */
void rlt_persistent_test_stall(int32_t on);

/* rlt_run_sequence for small fp32 models, as one launch for the whole call:
 * workgroup b runs all T steps of slot b (the recurrence is sequential
 * within a sequence and sequences never interact [Princeton, architecture
 * and design-principles paragraphs]), with the model's weights unpacked once
 * into its LDS and the slot's window cache mirrored there, so the phases of
 * a step are separated by workgroup barriers only -- the kernel fusion the
 * pages list among the implementation targets, for models where the launch
 * chain would pay a kernel boundary for a few hundred multiply-adds.
 * Arguments, semantics and errors as rlt_run_sequence (the state, window
 * cache and positions it leaves are those the launch chain would leave, up
 * to rounding), plus RLT_ERR_UNSUPPORTED unless rlt_fused_supported(cfg).
 * With one memory group, the memory positions the call reads are held in
 * LDS for the whole call when they fit beside the rest; otherwise they are
 * read from the memory in chunks in every layer (the same values either way).
 * Results: fp32 sums in a fixed order per output (not the chain's MFMA
 * order), so they match the chain and the CPU oracle up to rounding, and
 * splitting a run into calls changes no bit. */
int32_t rlt_fused_supported(const rlt_config *cfg);   /* 1: fp32, at most 16 layers,
                                                          heads * window <= 256, and
                                                          weights, gains, one slot's window
                                                          cache and activations in 160 KiB */
rlt_status rlt_run_sequence_fused(const rlt_model *m, rlt_state *st, int32_t T, const void *dev_e,
                                  const rlt_memory *mem, float *dev_logits, int32_t logits_mode,
                                  void *stream);

/* Replay scoring [Tutorial, "Current-Policy Reinforcement Learning Replay":
 * rebuild the states from the sequence start under the current weights,
 * evaluate each action from the preceding state, then consume it once].
 * T steps for all B slots exactly as rlt_run_sequence (no reset; the state
 * ends bitwise where rlt_run_sequence would leave it), and for each step t
 * the log-probability of the realized next token under that step's logits:
 *   dev_logprob[b][t] = log softmax(logits of slot b after consuming e_t)[dev_tokens[b][t]]
 * dev_e       [B][T][d] model dtype
 * dev_tokens  [B][T] int32: the token slot b consumes at step t + 1; a token
 *             < 0 is not scored (0 written), a token >= vocab gives NaN
 * dev_logprob [B][T] fp32 out
 * The logits are formed in the state's scratch and not returned; the log
 * softmax is taken in fp32 with the maximum taken out first. */
rlt_status rlt_score_sequence(const rlt_model *m, rlt_state *st, int32_t T, const void *dev_e,
                              const rlt_memory *mem, const int32_t *dev_tokens,
                              float *dev_logprob, void *stream);

/* --------------------------------------------------------- generation */
/* Stand-in incremental encoder for generation: lookup tables of the token.
 * A generated token's e_t and memory entry come from these tables (device
 * pointers, model dtype); the causal encoder (rlt_encode) is not run inside
 * this loop:
 *   e  [V][d]            e_t of token v
 *   k, v [G][V][H][dh]   memory K / V entry of token v in group g */
typedef struct {
  const void *e, *k, *v;
} rlt_encoder_table;

/* Sampling distribution: p(v) proportional to exp(logit_v / temperature)
 * over the kept tokens, those whose logit is >= the top_k-th largest logit
 * (top_k >= vocab keeps all).  temperature > 0, top_k >= 1. */
typedef struct {
  float temperature;
  int32_t top_k;
} rlt_sampling;

/* Autoregressive generation of n_steps tokens for all B slots [Tutorial,
 * "Autoregressive generation": use the preceding state's distribution,
 * sample, encode the sampled token, consume it through the decoder exactly
 * once].  For j = 0 .. n_steps-1 and every slot b:
 *   1. sample x from the preceding state's logits (j = 0: dev_logits0 [B][V],
 *      e.g. the last logits of the prompt from rlt_run_sequence; later: the
 *      previous step's) with u = dev_u[b][j] in [0, 1): the first token v in
 *      token order whose cumulative weight exceeds u times the total;
 *   2. record dev_tokens[b][j] = x and dev_logprob[b][j] = its log-probability
 *      under that distribution (the behaviour log-probability);
 *   3. encode x with the stand-in tables: e_t = enc->e[x], and memory entry
 *      pos (0-based; pos = the slot's position before the step) of every
 *      group set to enc->k[g][x], enc->v[g][x] -- this call WRITES those
 *      entries of the caller's memory buffers mem->k, mem->v;
 *   4. consume x: one decoder step of all slots.
 * dev_logits_last [B][V] fp32 (may be NULL) receives the last step's logits.
 * Each slot's position advances by n_steps; RLT_ERR_RANGE if that would pass
 * the memory capacity or max_tokens.  The state, scores and memory entries
 * are bitwise those of rlt_run_sequence over the same tokens' table rows. */
rlt_status rlt_generate(const rlt_model *m, rlt_state *st, int32_t n_steps,
                        const float *dev_logits0, const rlt_encoder_table *enc,
                        const rlt_memory *mem, const rlt_sampling *smp, const float *dev_u,
                        int32_t *dev_tokens, float *dev_logprob, float *dev_logits_last,
                        void *stream);

/* ------------------------------------------------------------ encoder */
/* The causal encoder [Article, "Encoder-Decoder Pairing with Shared Weights"
 * and "Principle 2: Co-Design Between Model and Hardware"; Princeton,
 * architecture paragraph; Tutorial, "Prompt prefill"]: all known tokens of a
 * sequence at once under a causal mask, as many layers as the decoder, layer l
 * using decoder layer l's attention and feed-forward weights; the memory
 * M_<=t is projected from e_t once per memory group.  For token x at encoder
 * position p (0-based) of its sequence:
 *   x = emb[x]
 *   per layer l = 0..L-1:
 *     x += W_O[l] CausalAttn(W_Q[l] a, W_K[l] a, W_V[l] a),  a = RMSNorm(x; g1[l])
 *          over positions 0..p of the sequence (itself included; keys and
 *          values of earlier calls come from the encoder cache)
 *     x += W_2[l] GELU(W_1[l] RMSNorm(x; g3[l]))
 *   e = RMSNorm(x; g_e)
 *   memory entry p of group g: K = W_Km[g] e, V = W_Vm[g] e, split into heads
 * Readings where the pages leave the step open: a learned token embedding, no
 * positional encoding, the tied weights include the two RMSNorm gains, the
 * encoder's own final gain g_e, memory projections without bias.  Precision as
 * for the decoder; e and the memory entries are stored in the model dtype (the
 * bf16 attention also rounds its softmax weights to bf16 for the P V product). */
typedef struct {
  const void *emb;              /* [V][d]    token embedding, model dtype         */
  const void *ge;               /* [d]       fp32 final RMSNorm gain g_e           */
  const void *wkm, *wvm;        /* [G][d][d] memory K / V projections, model dtype */
} rlt_encoder_params;

typedef struct rlt_encoder rlt_encoder;
typedef struct rlt_encoder_state rlt_encoder_state;

/* Bytes of device memory the encoder-only weights need; 0 if the model is
 * NULL or its configuration is outside the encoder kernels (bf16 needs
 * head_dim >= 32). */
size_t rlt_encoder_bytes(const rlt_model *m);

/* Copy and repack `src` into dev_buf (>= rlt_encoder_bytes, 256-byte aligned)
 * with kernels on `stream`; src is not retained.  The encoder reads the tied
 * layer weights from m's buffer: m must outlive it. */
rlt_status rlt_encoder_create(const rlt_model *m, const rlt_encoder_params *src, void *dev_buf,
                              size_t bytes, void *stream, rlt_encoder **out);
void rlt_encoder_destroy(rlt_encoder *enc);   /* frees the host handle only */

/* Bytes for an encoder state of `batch` slots: the encoder cache K, V
 * [L][B][H][max_tokens][dh] (model dtype; position p of slot b, layer l, head h
 * at ((l*B + b)*H + h)*max_tokens + p), a slot table, and scratch for up to
 * max_rows tokens per rlt_encode call (fp32 residual stream [rows][d];
 * normalised inputs, q, attention output and e rows [rows][d] and the FFN
 * hidden layer [rows][F] in the model dtype).  0 on a bad argument. */
size_t rlt_encoder_state_bytes(const rlt_config *cfg, int32_t batch, int32_t max_tokens,
                               int32_t max_rows);

/* Lay out an encoder state in dev_buf with every slot at position 0 (no
 * tokens encoded).  The only device work is clearing the small array of tile
 * counters the fast short-call mode uses (a memset of
 * 8 * ceil(max(3 d_model, d_ffn) / 32) bytes on the null stream, waited for
 * before the call returns); RLT_ERR_DEVICE if it fails. */
rlt_status rlt_encoder_state_init(const rlt_encoder *enc, int32_t batch, int32_t max_tokens,
                                  int32_t max_rows, void *dev_buf, size_t bytes,
                                  rlt_encoder_state **out);
void rlt_encoder_state_destroy(rlt_encoder_state *es);

/* Set the listed slots back to position 0 (a new document).  Host only. */
rlt_status rlt_encoder_state_reset(rlt_encoder_state *es, int32_t n, const int32_t *host_slots);

/* Kernel forms of the state's short calls [Tutorial, "Autoregressive
 * generation": each sampled token is encoded incrementally, and kernels that
 * share the execution semantics need not agree numerically].
 *   RLT_ENC_EXACT (the default): every call runs the prompt kernels'
 *     arithmetic, so a prompt gives bitwise the same values however it is
 *     split into calls.
 *   RLT_ENC_FAST: the bf16 GEMMs of calls of at most 64 token rows split K
 *     over 2 or 4 workgroups where N leaves room (a function of N and K only;
 *     the parts added in a fixed order), and calls of one token per sequence
 *     take the decoder's attention form (independent wavefront streams);
 *     values agree with the exact mode up to rounding, do not depend on the
 *     other rows of a call and are the same on every run.  Calls in fast mode
 *     on one state must not overlap (the split's tile counters live in it).
 * Applies to the calls made after it, rlt_generate_encoded's included.
 * Selecting RLT_ENC_FAST also clears the tile counters (a memset on the null
 * stream, waited for before the call returns; every complete launch leaves
 * them clear, so this only matters after a device error).  RLT_ERR_INVALID_ARG for another mode, RLT_ERR_DEVICE if the
 * memset fails. */
#define RLT_ENC_EXACT 0
#define RLT_ENC_FAST 1
rlt_status rlt_encoder_state_set_mode(rlt_encoder_state *es, int32_t mode);

/* Tokens encoded so far in a slot; -1 on a bad argument. */
int32_t rlt_encoder_position(const rlt_encoder_state *es, int32_t slot);

/* Encode the next T tokens of each of n listed slots (host_slots NULL = slots
 * 0..n-1; slots distinct):
 *   dev_tokens [n][T] int32: row i holds the next T tokens of slot host_slots[i];
 *              a token outside 0..V-1 makes its sequence's outputs NaN from that
 *              token on (earlier tokens of that sequence in the same call may be
 *              NaN too); other sequences are not affected
 *   dev_e      [n][T][d] model dtype out, 16-byte aligned (NULL: e is kept in
 *              the state's scratch only)
 *   mem        caller memory, WRITTEN: for sequence index = slot, positions
 *              p0..p0+T-1 of every group, p0 = the slot's position before the call
 * Token j of slot s is encoder position p0_s + j and attends to positions
 * 0..p0_s + j, so a prompt encoded in one call or in several chunks gives the
 * same values up to the summation order of the softmax.  Each slot's position
 * advances by T.  RLT_ERR_SHAPE if n*T > max_rows; RLT_ERR_RANGE if a position
 * would pass max_tokens or the memory capacity.  A prompt's prefill is this
 * call followed by rlt_run_sequence over dev_e (the decoder recurrence over
 * every prompt token [Tutorial, "Prompt prefill"]). */
rlt_status rlt_encode(const rlt_encoder *enc, rlt_encoder_state *es, int32_t n,
                      const int32_t *host_slots, int32_t T, const int32_t *dev_tokens,
                      void *dev_e, const rlt_memory *mem, void *stream);

/* Autoregressive generation with the causal encoder in the loop [Tutorial,
 * "Autoregressive generation": sample, encode the sampled token
 * incrementally, consume it once]: rlt_generate with step 3 replaced by
 * rlt_encode of each slot's new token (T = 1, slots 0..B-1 of es): the
 * encoder attends to its cache of the slot's earlier tokens, writes e_t and
 * memory entry pos of every group (pos = the slot's position before the
 * step) into the caller's memory, and advances es.  Before the call every
 * slot must have as many tokens encoded as consumed (es position == st
 * position, e.g. after prefill: rlt_encode of the prompt, then
 * rlt_run_sequence over its e rows); RLT_ERR_RANGE otherwise or when a
 * position would pass either state's max_tokens or the memory capacity.
 * enc must belong to m (RLT_ERR_INVALID_ARG), es to m's version
 * (RLT_ERR_STALE), es->batch >= B and its max_rows >= B (RLT_ERR_SHAPE).
 * The state, logits and memory entries are bitwise those of encoding the
 * generated tokens in one rlt_encode call and running rlt_run_sequence over
 * their e rows. */
rlt_status rlt_generate_encoded(const rlt_model *m, rlt_state *st, int32_t n_steps,
                                const float *dev_logits0, const rlt_encoder *enc,
                                rlt_encoder_state *es, const rlt_memory *mem,
                                const rlt_sampling *smp, const float *dev_u, int32_t *dev_tokens,
                                float *dev_logprob, float *dev_logits_last, void *stream);

/* Exact prefix snapshot of the encoder cache [Article, "Multi-Turn Serving":
 * the snapshot of a prefix carries the encoder's cached state with the
 * decoder's; Princeton, training/serving paragraph].  With the decoder's
 * record (rlt_state_export) and the memory entries (caller buffers, copied by
 * the caller), a conversation resumes in another slot or process bitwise.
 * Per slot one record of rlt_encoder_snapshot_bytes(cfg, capacity, 1) bytes:
 *   256-byte header: uint32 magic 0x454C5452, format 1, d_model, n_heads,
 *         head_dim, n_layers, dtype, position p (tokens encoded), capacity,
 *         0, then the model version as two uint32 (low, high); rest zero
 *   then  K: [L][H][capacity][dh] model dtype, positions 0..p-1, later zero
 *   then  V: same layout as K
 * (each of K and V starts at a 256-byte boundary).  Export: RLT_ERR_RANGE if
 * a listed slot holds more than `capacity` positions.  Import checks every
 * header first and changes nothing on a mismatch (RLT_ERR_CONVENTION: not a
 * record, another shape, dtype, capacity or model version, or a position past
 * the state's max_tokens); it synchronises the stream once to read them.
 * Both: RLT_ERR_STALE for an encoder state of another model version,
 * RLT_ERR_INVALID_ARG for bad or repeated slots, RLT_ERR_SHAPE for a
 * dev_snap that is not 256-byte aligned. */
size_t rlt_encoder_snapshot_bytes(const rlt_config *cfg, int32_t capacity, int32_t n);
rlt_status rlt_encoder_state_export(const rlt_encoder *enc, rlt_encoder_state *es, int32_t n,
                                    const int32_t *host_slots, int32_t capacity, void *dev_snap,
                                    void *stream);
rlt_status rlt_encoder_state_import(const rlt_encoder *enc, rlt_encoder_state *es, int32_t n,
                                    const int32_t *host_slots, int32_t capacity,
                                    const void *dev_snap, void *stream);

/* Encoder kernel timing, as rlt_profile_begin with every call one step:
 * RLT_E_GEMM = the token-parallel GEMMs, RLT_E_ATTN = causal attention,
 * RLT_E_OTHER = embedding and RMSNorm.  Collect returns the recorded launch
 * durations (ms), their count, their algorithmic FLOPs (2 per multiply-add of
 * the GEMMs, 4 * d per attended position of attention; 0 for OTHER) and bytes
 * (weights, activations in and out, cache positions read once per sequence). */
enum { RLT_E_GEMM = 0, RLT_E_ATTN = 1, RLT_E_OTHER = 2, RLT_E_NCLASSES = 3 };
rlt_status rlt_encoder_profile_begin(rlt_encoder_state *es, int32_t class_mask,
                                     int32_t max_launches);
rlt_status rlt_encoder_profile_collect(rlt_encoder_state *es, int32_t kclass, double *total_ms,
                                       int32_t *launches, double *flops, double *bytes_moved);

/* Host mirror of a slot's position (tokens consumed); -1 on a bad argument.
 * Does not synchronise. */
int32_t rlt_state_position(const rlt_state *st, int32_t slot);

/* ------------------------------------------------------------- snapshots */
/* Exact prefix snapshot of the decoder state [Article, "Multi-Turn Serving";
 * Princeton, training/serving paragraph]: per slot one record of
 * rlt_snapshot_bytes(cfg, 1) bytes, independent of the ring phase:
 *   +0    header: uint32 magic 0x534C5452 ("RTLS"), uint32 format 1,
 *         int32 d_model, n_heads, head_dim, n_layers, window, dtype, pos,
 *         int32 0, uint64 model_version (48 bytes; 256 reserved)
 *   +256  s: fp32 [d]
 *   then  K: [L][H][W-1][dh] model dtype, logical order: entry e < n_hist =
 *         min(pos, W-1) holds position pos - n_hist + 1 + e; later entries 0
 *   then  V: same layout as K
 * (each section starts at a 256-byte boundary). */
size_t rlt_snapshot_bytes(const rlt_config *cfg, int32_t n);

/* Write records of the listed slots to dev_snap (record i = host_slots[i]). */
rlt_status rlt_state_export(const rlt_model *m, const rlt_state *st, int32_t n,
                            const int32_t *host_slots, void *dev_snap, void *stream);

/* Restore the listed slots from dev_snap.  Reads the n headers back to the host
 * (synchronising `stream`) to check them: RLT_ERR_CONVENTION if a record's
 * shape, window, dtype, magic or model_version differ from the model's, or
 * its position exceeds the state's max_tokens; nothing is written then. */
rlt_status rlt_state_import(const rlt_model *m, rlt_state *st, int32_t n,
                            const int32_t *host_slots, const void *dev_snap, void *stream);

/* ------------------------------------------------------------- training */
/* Backpropagation through time [Article, "Training Methodology"; Tutorial,
 * "Pretraining and supervised fine-tuning"; Forget, its note on truncated
 * BPTT].  B sequences run from H_0 over T steps (the step of this header, fp32,
 * on the canonical parameters: the decode path's packed model is not used),
 * with the loss
 *   loss = sum over b, t with dev_targets[b][t] >= 0 of -log softmax(logits_{b,t})[dev_targets[b][t]]
 * (a target < 0 removes the loss term only: the step still updates the state,
 * and gradients from later losses flow through it; a target >= vocab makes the
 * loss NaN), then the exact gradient of that loss w.r.t. every parameter, the
 * e rows and the memory.  Gradients flow through s_t and through every window
 * cache entry to each later step that reads it (the cross terms of the
 * state-to-state Jacobian).  Truncation names what it cuts: with opts->chunk = k
 * > 0, at each boundary between steps k*j and k*j + 1 the parts of H listed in
 * opts->detach are detached, RLT_DETACH_S (s) and/or RLT_DETACH_KV (every cache
 * entry carried across the boundary); the forward values never change.
 * opts NULL or chunk 0 = full BPTT.
 * Activation checkpointing [Tutorial, "Key Design Principles": checkpointing
 * around the recurrent decoder; Princeton, design-principles paragraph]:
 * with opts->segment = S in [1, T), the intermediates of only S steps are
 * held at once.  Every step runs forward once; then the segments go in
 * reverse, each recomputed forward from its first state (the same kernels on
 * the same inputs: the same bits) before its backward.  Kept for every step:
 * the keys and values of every layer and their gradient rows, s_t and the
 * per-row losses.  The loss, dev_de and the memory gradients are bitwise
 * those of segment 0 (= T: everything kept); the parameter gradients are
 * sums over the segments' rows in reverse segment order, so they differ from
 * segment 0 only by the grouping of those sums. */
enum { RLT_DETACH_S = 1, RLT_DETACH_KV = 2 };
typedef struct {
  int32_t chunk;                /* truncation length in steps; 0 = none */
  int32_t detach;               /* RLT_DETACH_* bits cut at each chunk boundary */
  int32_t segment;              /* steps whose intermediates are held at once; 0 = all T */
} rlt_bptt_opts;

/* Workspace bytes for rlt_bptt with every intermediate of the T steps kept
 * (about (22 d + 3 F) * L + 7 d + V floats per sequence and step); 0 if the
 * config is invalid, not fp32, or T exceeds 4096. */
size_t rlt_bptt_workspace_bytes(const rlt_config *cfg, int32_t batch, int32_t T);
/* The same for opts->segment = segment (0 = T): about 4 d L + d floats per
 * sequence and step for all T steps plus (18 d + 3 F) * L + 6 d + V per
 * sequence and step of one segment; 0 also for segment < 0. */
size_t rlt_bptt_workspace_bytes_segmented(const rlt_config *cfg, int32_t batch, int32_t T,
                                          int32_t segment);

/* params: fp32 canonical device tensors as for rlt_model_create (read only).
 * grads:  buffers of the same shapes, OVERWRITTEN with d loss / d param.
 * dev_e [B][T][d] fp32; mem: fp32 memory, sequence index = b, capacity >= T.
 * dev_de [B][T][d] (written) or NULL; dmem: memory gradients with mem's
 * strides and 16-byte aligned pointers (RLT_ERR_SHAPE otherwise; ACCUMULATED
 * into: zero them first) or NULL; dev_loss [1] (written).
 * dev_workspace: >= rlt_bptt_workspace_bytes_segmented(cfg, batch, T,
 * opts->segment), 256-byte aligned, caller owned.
 * RLT_ERR_UNSUPPORTED for a bf16 config. */
rlt_status rlt_bptt(const rlt_config *cfg, const rlt_params *params, int32_t batch, int32_t T,
                    const float *dev_e, const rlt_memory *mem, const int32_t *dev_targets,
                    const rlt_bptt_opts *opts, const rlt_params *grads, float *dev_de,
                    const rlt_memory *dmem, float *dev_loss, void *dev_workspace,
                    size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------- profiling */
/* Kernel classes for per-class timing: RLT_K_EXTRA = the replay-scoring,
 * sampling and stand-in encoder kernels; GEMM = every projection and the head;
 * SWA = window attention; CROSS = memory attention. */
enum { RLT_K_EXTRA = 0, RLT_K_GEMM = 1, RLT_K_SWA = 2, RLT_K_CROSS = 3, RLT_K_NCLASSES = 4 };

/* Start recording a HIP event pair around every launch of the kernel classes
 * in class_mask (bit 1 << RLT_K_*) on this state, during every step_stride-th
 * step (step_stride >= 1), up to max_launches pairs; class_mask = 0 stops.
 * Events come from a pool kept by the state.  Meant for measurement runs: each
 * recorded pair adds two event records to the stream. */
rlt_status rlt_profile_begin(rlt_state *st, int32_t class_mask, int32_t max_launches,
                             int32_t step_stride);
/* For kernel class kclass: the sum of the recorded launch durations (ms), their
 * count, and the algorithmic bytes those launches move (weights, window cache
 * and memory entries read once, activations in and out, as stored).  Waits for
 * the recorded events, then clears that class's records. */
rlt_status rlt_profile_collect(rlt_state *st, int32_t kclass, double *total_ms,
                               int32_t *launches, double *bytes_moved);

/* Achievable peaks of the device, measured on it (the survey's measurement
 * contract asks for them beside the published figures; they price the
 * path's kernels against what the part delivers).  Both return RLT_OK,
 * RLT_ERR_INVALID_ARG for a null pointer or bad count, RLT_ERR_SHAPE for a
 * bad size, RLT_ERR_DEVICE for a HIP error; they set no rlt_last_error text.
 * Each runs `reps` launches on the stream and reports the fastest (HIP events
 * bound to the launch's own dispatch); the call synchronises with them.
 *   rlt_peak_bandwidth: read (copy = 0) or copy to dev_dst (copy = 1) `bytes`
 *     bytes of dev_src (a multiple of 64 KiB, at least 64 MiB; both buffers
 *     16-byte aligned, dev_dst at least `bytes` long for a copy and 4 KiB for
 *     a read) with 16-byte non-temporal loads and stores, one contiguous
 *     64 KiB span per workgroup; *gb_per_s = bytes moved (read, or read plus
 *     written) / time, in 1e9 bytes per second.
 *   rlt_peak_mfma: dense loops of v_mfma_f32_32x32x16_bf16 (shape 0, four
 *     independent accumulator chains per wavefront) or v_mfma_f32_16x16x32_bf16
 *     (shape 1, eight chains), `iters` rounds, two 256-thread workgroups per
 *     compute unit; dev_sink receives one float per thread (2 * CUs * 256
 *     floats, sink_bytes at least that); *tflops in 1e12 FLOP per second. */
rlt_status rlt_peak_bandwidth(const void *dev_src, void *dev_dst, size_t bytes, int32_t copy,
                              int32_t reps, double *gb_per_s, void *stream);
rlt_status rlt_peak_mfma(int32_t shape, int32_t iters, int32_t reps, float *dev_sink,
                         size_t sink_bytes, double *tflops, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* RLT_H */
