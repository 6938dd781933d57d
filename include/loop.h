/*
 * loop.h - C ABI of libloop.so: the forward pass (prefill and decode) of a
 * looped weight-shared decoder on one AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The model stores n_layers decoder layers.  Layers
 * [0, loop_start) run once, the block [loop_start, loop_end) runs n_passes
 * times with every pass fed the previous pass's output, and layers
 * [loop_end, n_layers) and the output head finish (pages: "SenseTime's Loop-9B
 * runs its own layers twice, and gets a deeper model for free", section "The
 * trick: run the middle of the network twice"; "How Does SenseNova-Loop Get
 * More Depth Without More Parameters?", section "What is the looped decoder in
 * SenseNova-Loop?").  The Loop-9B shape is 32 stored layers, block [4, 28)
 * twice: 56 layer executions.  The loop range, the pass count and the
 * hyper-connection parameters are part of the model's execution config, which
 * a compatible engine must load and honour (same page, section "How do you
 * run SenseNova-Loop-9B-Preview?"): they are fields of loop_config below.
 *
 * Inside the block the hidden state is two residual streams X0, X1 joined by
 * hyper-connection maps (section "What does two-stream mHC do?").  Every
 * sublayer (attention, then FFN) of a looped layer is one site with learned
 * float32 parameters W [8][2C], b [8]:
 *   x_hat = [X0, X1] / rms([X0, X1]);  l = W x_hat + b
 *   H_pre = sigmoid(l0, l1), H_post = 2 sigmoid(l2, l3),
 *   H_res = Sinkhorn_iters(exp([[l4, l5], [l6, l7]] - max))  (rows, then columns)
 *   u = RMSNorm(H_pre0 X0 + H_pre1 X1; gamma);  y = f(u)
 *   X_i <- sum_j H_res[i][j] X_j + H_post[i] y
 * The streams are entered as two copies of h before the first looped layer
 * and left as their mean after the last pass.  Outside the block every layer
 * is two pre-norm residual sublayers h <- h + f(RMSNorm(h; gamma)).
 * Attention follows a period of attn_period layers: layer i is full causal
 * softmax attention when i % attn_period == attn_period - 1 and causal linear
 * attention otherwise ("How does the hybrid attention pattern work?").  The
 * linear attention uses the elu+1 feature map with normaliser la_eps; each
 * (layer, pass) owns its own KV cache or linear state.  The FFN is SwiGLU.
 * The pages leave these internals open; the choices above are this library's
 * documented reading.
 *
 * Conventions.
 *  - All tensors are row-major.  "dtype" means float (LOOP_FP32) or bf16
 *    (LOOP_BF16) for the whole backbone; RMSNorm gains and the mHC
 *    parameters are always float32; logits are always float32.
 *  - Device pointers are HIP device memory owned by the caller, 16-byte
 *    aligned (torch and hipMalloc allocations are 256-byte aligned), valid
 *    for as long as the calls that use them run.
 *  - Every call is asynchronous on the given stream (a hipStream_t passed as
 *    void*; NULL = the default stream).  Calls that share a state must be
 *    issued on one stream, in order.
 *  - Results are deterministic: no floating-point atomics are used.
 *  - Return codes are LOOP_OK (0) or a negative loop_status; a failed call
 *    has launched nothing and changed no state.  loop_last_error() gives a
 *    message for the calling thread.  Device-side input errors (a token id
 *    out of range) are flagged in the state and read by loop_state_check().
 */
#ifndef LOOP_H
#define LOOP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOOP_OK = 0,
  LOOP_ERR_INVALID_ARG = -1,  /* null pointer or a value out of range */
  LOOP_ERR_SHAPE = -2,        /* shapes the kernels do not support */
  LOOP_ERR_ALIGN = -3,        /* a pointer not 16-byte aligned */
  LOOP_ERR_CAPACITY = -4,     /* batch or positions beyond the state's capacity */
  LOOP_ERR_WORKSPACE = -5,    /* workspace smaller than loop_workspace_bytes() */
  LOOP_ERR_NO_DEVICE = -6,    /* no HIP device */
  LOOP_ERR_HIP = -7,          /* a HIP runtime call failed */
  LOOP_ERR_DEVICE_FLAG = -8,  /* loop_state_check(): a device-side input error was flagged */
  LOOP_ERR_STATE = -9         /* decode before any prefill, or a state of another model */
} loop_status;

enum { LOOP_FP32 = 0, LOOP_BF16 = 1 };

/* loop_prefill flags */
enum {
  LOOP_ALL_LOGITS = 1,  /* logits for every position [B][S][V] (default: last position [B][V]) */
  LOOP_HIDDEN_OUT = 2,  /* return the final residual h [B][S][C] in dtype instead of logits */
  LOOP_CONTINUE = 4     /* append to the state's sequences (chunked prefill) instead of restarting */
};

typedef struct loop_config {
  int vocab;           /* V */
  int hidden;          /* C; a multiple of 8, at most 4096 */
  int ffn;             /* F (SwiGLU width) */
  int n_heads;         /* Hq query heads */
  int n_kv_heads;      /* Hkv KV heads; Hq % Hkv == 0, Hq / Hkv <= 8 (bf16: 1, 2, 4 or 8; 1, 2, 4 at d 256) */
  int head_dim;        /* d: float32 64 or 128; bf16 128 or 256 */
  int n_layers;        /* stored layers */
  int loop_start;      /* first looped layer */
  int loop_end;        /* one past the last looped layer */
  int n_passes;        /* >= 1 */
  int sinkhorn_iters;  /* Sinkhorn iterations of H_res (20 for Loop-9B) */
  int attn_period;     /* layer i is full attention iff i % attn_period == attn_period - 1 */
  float rms_eps;       /* RMSNorm epsilon (mHC rms included) */
  float la_eps;        /* linear-attention normaliser epsilon */
  int dtype;           /* LOOP_FP32 or LOOP_BF16 */
} loop_config;

typedef struct loop_layer_weights {
  const float* attn_norm;  /* [C] */
  const float* ffn_norm;   /* [C] */
  const void* qkv;         /* [(Hq + 2 Hkv) d][C]: q rows, then k rows, then v rows */
  const void* o;           /* [C][Hq d] */
  const void* gate_up;     /* [2F][C]: gate rows, then up rows */
  const void* down;        /* [C][F] */
  const float* mhc_w[2];   /* looped layers only: [8][2C] per site (0 = attention, 1 = FFN) */
  const float* mhc_b[2];   /* looped layers only: [8] per site */
} loop_layer_weights;

typedef struct loop_weights {
  const void* embed;               /* [V][C] */
  const float* final_norm;         /* [C] */
  const void* head;                /* [V][C] (untied) */
  const loop_layer_weights* layers;  /* host array of n_layers entries (copied) */
  int n_layers;
} loop_weights;

typedef struct loop_model loop_model;  /* host object: config, weight pointers, schedule */
typedef struct loop_state loop_state;  /* host handle on caller-owned device state */

/* Validates the config and records the weight pointers (no copy, no launch).
 * Errors: INVALID_ARG, SHAPE, ALIGN, NO_DEVICE. */
int loop_model_create(const loop_config* cfg, const loop_weights* w, loop_model** out);
int loop_model_destroy(loop_model* m);

/* The execution schedule: for e < n, layer[e], pass[e] and kind[e] (1 = full,
 * 0 = linear) and slot[e] (index among full or among linear executions).
 * Any output array may be NULL; *n receives the number of executions. */
int loop_model_schedule(const loop_model* m, int max, int* layer, int* pass, int* kind, int* slot, int* n);

/* Device bytes of a state for `batch` sequences of up to `max_seq` positions:
 * a 256-byte header, then per full-attention execution K [batch][Hkv][S_max][d]
 * and V^T [batch][Hkv][d][S_max] (dtype), then per linear execution
 * S [batch][Hkv][d][d] and z [batch][Hkv][d] (float32), then the parked
 * cohorts of loop_decode_pipelined (X [batch][2][C], y [batch][C] in dtype,
 * maps [batch][8] float32), then the start positions of a ragged decode step
 * (int32 [batch]); regions start on 256-byte boundaries; S_max is max_seq
 * rounded up to a multiple of 64. */
int loop_state_bytes(const loop_model* m, int batch, int max_seq, size_t* bytes);

/* Device bytes of the workspace for one call over up to `max_tokens` new
 * positions in total (batch x positions per sequence) of `batch` sequences
 * whose state holds up to `max_seq` positions. */
int loop_workspace_bytes(const loop_model* m, int batch, int max_tokens, int max_seq, size_t* bytes);

/* Wraps caller-owned device memory (>= loop_state_bytes) as a state of length 0.
 * The memory is not cleared; a prefill without LOOP_CONTINUE ignores its
 * contents.  Clear the header once (hipMemset to 0) before the first
 * loop_state_check(). */
int loop_state_create(const loop_model* m, void* state_dev, size_t bytes, int batch, int max_seq, loop_state** out);
int loop_state_destroy(loop_state* st);
/* Paged KV caches, for serving.  Serving shared-weight loops is the gap one
 * page names ("SenseTime Open-Sources Loop-9B: Same Layers, Run Twice", its
 * closing paragraphs on costs): a looped model needs one cache per (layer,
 * pass), so a paged state gives every full-attention (layer, pass) slot its
 * own pool of n_pages pages of 64 positions, K [n_pages][Hkv][64][d] and V^T
 * [n_pages][Hkv][d][64], and one block table maps each sequence's positions
 * to pages for all slots at once: positions [64 j, 64 j + 64) of sequence b
 * live in page block_table_dev[b * ceil(max_seq / 64) + j] of every pool.
 * block_table_dev is caller-owned device memory, int32 [batch][ceil(max_seq /
 * 64)], read by the kernels of every call (the caller may change entries
 * between calls, for example to give a growing sequence its next page); an
 * entry outside [0, n_pages) is clamped into it, so a bad entry gives wrong
 * results but no access outside the pools.  Two sequences that write the
 * same page race; sharing pages that no call writes (a common prefix) is
 * allowed.  Everything else (linear states, lengths, ragged batches, every
 * prefill and decode entry point) is as for loop_state_create.
 * loop_state_bytes_paged: device bytes of such a state (the pools replace the
 * per-sequence slots; the rest as loop_state_bytes).  loop_state_create_paged:
 * max_seq <= 524,288.  Errors: INVALID_ARG (n_pages <= 0, null table), ALIGN,
 * CAPACITY. */
int loop_state_bytes_paged(const loop_model* m, int batch, int max_seq, int n_pages, size_t* bytes);
int loop_state_create_paged(const loop_model* m, void* state_dev, size_t bytes, int batch, int max_seq, int n_pages,
                            const int32_t* block_table_dev, loop_state** out);

/* Every sequence of a state has its own length (the positions its KV caches
 * and linear states hold).  Sequences of one state may differ (a ragged
 * batch): loop_prefill_rows fills a subset, and loop_decode_step advances
 * each sequence from its own length (contiguous or paged caches).
 *
 * loop_state_length: the shortest sequence's length (the common length when
 * all agree).  loop_state_seq_length: sequence `seq`'s length. */
int loop_state_length(const loop_state* st, int* length);
int loop_state_seq_length(const loop_state* st, int seq, int* length);
/* Declares that every sequence (loop_state_set_length) or sequence `seq`
 * (loop_state_set_seq_length) holds `length` valid positions, for example
 * after filling the regions directly; 0 <= length <= max_seq.  Only the KV
 * caches are indexed by position: a linear-attention state holds every
 * position it has taken in, so a shorter length is only consistent once the
 * caller has restored those regions (or with length 0, which the next
 * prefill starts from).  Either call resets loop_decode_pipelined (tokens in
 * flight are dropped).  Errors: INVALID_ARG (seq outside [0, batch)),
 * CAPACITY. */
int loop_state_set_length(loop_state* st, int length);
int loop_state_set_seq_length(loop_state* st, int seq, int length);
/* Device pointer and byte size of one region of the state: kind 0 = K, 1 = V^T
 * (slot = full-attention execution index; a page pool for a paged state),
 * 2 = S, 3 = z (slot = linear execution index), 4 = header (slot ignored;
 * word 0 = error flags). */
int loop_state_region(const loop_state* st, int kind, int slot, void** ptr, size_t* bytes);
/* Synchronises the stream, reads and clears the device error word.
 * Returns LOOP_OK or LOOP_ERR_DEVICE_FLAG (token id out of range: row 0 used). */
int loop_state_check(loop_state* st, void* stream);

/* Prefill of B sequences of S new positions each (B <= state batch).
 * tokens_dev: int32 [B][S] (or NULL with embeds_dev: dtype [B][S][C]).
 * out_dev: float32 logits [B][V] (last position), [B][S][V] with
 * LOOP_ALL_LOGITS, or dtype h [B][S][C] with LOOP_HIDDEN_OUT.
 * Without LOOP_CONTINUE the sequences restart at position 0; with it they
 * continue at their length, which must be the same for all B (else STATE).
 * Each sequence's length becomes its start position + S.
 * Errors: INVALID_ARG, ALIGN, CAPACITY, WORKSPACE, STATE, HIP. */
int loop_prefill(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes,
                 const int32_t* tokens_dev, const void* embeds_dev, int B, int S,
                 unsigned flags, void* out_dev, void* stream);
/* loop_prefill over sequences [seq0, seq0 + B) of the state (their slots and
 * lengths); the other sequences are untouched.  This is how a ragged batch is
 * built: prompts of different lengths prefilled per group, then decoded
 * together by loop_decode_step.  tokens/embeds/out are laid out as for
 * loop_prefill with B rows.  Errors: as loop_prefill; INVALID_ARG when seq0
 * lies outside [0, batch), CAPACITY when seq0 + B > batch. */
int loop_prefill_rows(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes, int seq0,
                      const int32_t* tokens_dev, const void* embeds_dev, int B, int S,
                      unsigned flags, void* out_dev, void* stream);

/* One decode step: one new token per sequence, tokens_dev int32 [B]; logits
 * float32 [B][V].  Sequence b in [0, B) takes its token at its own length
 * (ragged batches allowed); appends one position to each of its KV caches
 * and updates every linear state.  A ragged step first writes the B start
 * positions into the state's position region (one small kernel launch).
 * Errors: as loop_prefill, plus STATE when any of the B sequences is empty. */
int loop_decode_step(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes,
                     const int32_t* tokens_dev, int B, float* logits_dev, void* stream);

/* loop_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the workspace is the library's own device array of
 * LOOP_NOALLOC_WORKSPACE_BYTES (64 MiB), one per GPU, held until the process
 * ends; its address on a device is looked up once (loop_model_create, or the
 * first call on that device).  The call allocates nothing and computes what
 * loop_decode_step computes with the same kernels.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from several threads without ordering) race and give wrong
 * results.  No kernel relies on the array's previous contents.
 * Errors: as loop_decode_step; WORKSPACE (nothing launched) when the step
 * needs more than the array holds, that is when
 * loop_workspace_bytes(m, B, B, max_seq) > LOOP_NOALLOC_WORKSPACE_BYTES. */
enum { LOOP_NOALLOC_WORKSPACE_BYTES = 64 << 20 };
int loop_decode_step_noalloc(loop_model* m, loop_state* st, const int32_t* tokens_dev, int B, float* logits_dev,
                             void* stream);

/* Decode with the passes of the looped block co-scheduled over cohorts, so
 * that every call reads each shared layer's weights once for several tokens'
 * passes.  One page expects the shared block's weights to be fetched once
 * and kept for the second pass ("SenseTime open-sourced its experimental
 * SenseNova-Loop-9B-Preview" (frontword.com), section "Why parameter reuse
 * matters for inference"); at 9.3 GB per block pass no cache holds them, and
 * this schedule is what makes one weight read serve two passes.
 *
 * The state holds n_passes cohorts of B sequences: cohort g is sequences
 * [g B, (g + 1) B) (state batch = n_passes x B, prefilled as usual).  A token
 * enters its cohort with the layers before the block and pass 1 of the block,
 * advances one pass per call (parked inside the block between calls), and
 * leaves after the last pass with the layers after the block and the head.
 * Cohorts enter in the order 0, 1, ..., n_passes - 1, 0, ...; a cohort can
 * take its next token once its previous one has left.  Each call runs every
 * stored layer of the block once over all cohorts' rows (each cohort on its own
 * (layer, pass) KV cache or linear state and its own position).
 *
 * tokens_dev: int32 [B] for the entering cohort, or NULL (no cohort enters:
 * drains the pipeline).  logits_dev: float32 [B][V], written for the cohort
 * whose token leaves in this call.  cohorts (host int[2]): [0] the cohort
 * that entered (-1: none), [1] the cohort whose logits were written (-1: none;
 * the first n_passes - 1 calls after a prefill write none).  Results per
 * token equal loop_decode_step's up to summation order.  The workspace is
 * loop_workspace_bytes(m, n_passes x B, n_passes x B, max_seq).  While a
 * cohort has a token in flight, loop_prefill and loop_decode_step return
 * STATE; loop_state_set_length resets the pipeline (tokens in flight are
 * dropped).  Each cohort's sequences must share one length (else STATE when
 * it enters); cohorts may differ.  A cohort's lengths grow when its token
 * leaves, so loop_state_length reports the shortest cohort's length.
 * Errors: INVALID_ARG, SHAPE (batch != n_passes x B), ALIGN, CAPACITY,
 * WORKSPACE, STATE (nothing to run, a cohort not ready, or no prefill), HIP. */
int loop_decode_pipelined(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes,
                          const int32_t* tokens_dev, int B, float* logits_dev, int* cohorts, void* stream);

const char* loop_status_string(int status);
const char* loop_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LOOP_H */
