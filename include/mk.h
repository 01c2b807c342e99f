/*
 * mk.h -- C ABI of the persistent MoE decode megakernel for MI355X (gfx950).
 *
 * One call to mk_decode_step runs one BF16 autoregressive decode step of a
 * parallel-block mixture-of-experts decoder, or of its sequential-block form
 * (mk_config.block_style) (RMSNorm, QKV projection, rotary
 * embedding, paged split-KV attention, router top-k, expert gather with
 * gate/up/down projections, residuals, LM head) as a single persistent kernel:
 * one workgroup per compute unit works through a task table that the host
 * built ahead of time, and tasks wait on counters in global memory instead of
 * on kernel boundaries.
 *
 * Where the operations come from (the Cohere megakernel pages):
 *  - latestnews.news, "Cohere speeds up North Mini Code with new megakernel",
 *    paragraphs 2-3: the whole decode forward pass in one persistent kernel,
 *    a host-built static schedule, global-memory counters, paged attention
 *    and ragged sequence lengths;
 *  - ainews.surl.tw, paragraph 2: a fine-grained task table of GEMM tiles and
 *    attention splits assigned to compute units in advance; attention and MoE
 *    run concurrently from the same normalized input;
 *  - aiweekly.co, paragraphs 2-4: the fused operation kinds (QKV projection,
 *    attention, MoE routing, gather, GEMMs, normalization), fixed-size task
 *    descriptors, a consumer waiting on a single count, and prefetch of
 *    immutable weights.
 *
 * Conventions for every entry point:
 *  - Return MK_OK (0) or a negative MK_ERR_* code; no exception crosses the ABI.
 *    mk_last_error_message() returns a thread-local description of the last
 *    failure on the calling thread.
 *  - "device pointer" = memory the caller allocated on the GPU (e.g. through
 *    PyTorch); the library never allocates or frees device memory.  It owns
 *    its host-side state and one static device array per GPU, used only by
 *    mk_bind_scratch.
 *  - "stream" = a hipStream_t passed as void*; NULL means the default stream.
 *    Work is enqueued asynchronously on it.
 *  - Matrices are row-major [out][in] bfloat16 (raw 16-bit patterns), or, in
 *    the FP8 / FP4 weight formats, E4M3 / packed E2M1 codes with per-row
 *    scales (mk_bind).
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mk_ctx mk_ctx;

enum {
  MK_OK = 0,
  MK_ERR_INVALID_ARG = -1,   /* bad argument detected on the host; nothing enqueued */
  MK_ERR_UNSUPPORTED = -2,   /* configuration outside what the kernels handle */
  MK_ERR_STATE = -3,         /* call out of order (no schedule, not bound, reset needed) */
  MK_ERR_SCHEDULE = -4,      /* schedule failed validation (deadlock or bad fan-in) */
  MK_ERR_HIP = -5,           /* a HIP runtime call failed; the message names it */
  MK_ERR_DEVICE_PAGE = -10,  /* kernel met a page id outside [0, num_pages) */
  MK_ERR_DEVICE_SEQ = -11,   /* kernel met seq_len < 0 or seq_len + 1 > max_pages_per_seq * page_size */
  MK_ERR_DEVICE_TOKEN = -12, /* kernel met a token id outside [0, vocab) */
  MK_ERR_DEVICE_TIMEOUT = -13 /* a dependency wait exceeded the spin limit; the grid drained */
};

/* Model shape and capacity.  Supported: hidden, n_q_heads*head_dim and inter
 * multiples of 128; head_dim 64 or 128; n_q_heads a multiple of n_kv_heads
 * with at most 8 q heads per kv head; n_experts <= 128; top_k <= 8;
 * page_size == 16; 1 <= max_batch <= 8. */
typedef struct mk_config {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, inter, vocab;
  int32_t page_size;          /* tokens per KV page (16) */
  int32_t max_batch;          /* largest batch a step may carry */
  int32_t max_pages_per_seq;  /* page-table row stride; a sequence holds at most this many pages */
  int32_t num_pages;          /* pages in each layer's K pool and V pool */
  float rms_eps;              /* RMSNorm epsilon (1e-6) */
  double rope_theta;          /* RoPE base (1e4) */
  int32_t weight_format;      /* MK_WEIGHTS_BF16 (0), MK_WEIGHTS_FP8_E4M3 (1) or MK_WEIGHTS_FP4_E2M1 (2), see mk_bind */
  int32_t block_style;        /* MK_BLOCK_PARALLEL (0) or MK_BLOCK_SEQUENTIAL (1) */
} mk_config;

/* Layer forms.  PARALLEL: attention and the MoE path both read
 * bf16(rmsnorm(x, attn_norm)) and the layer leaves x + attention + moe, the
 * model the pages describe (latestnews.news, paragraph 1).  SEQUENTIAL: the
 * MoE path reads bf16(rmsnorm(x + attention, moe_norm)) with a gain of its own
 * and the layer leaves (x + attention) + moe: the pre-norm layer of other MoE
 * models, to which the pages ask whether the engine generalizes
 * (ainews.surl.tw, paragraph 4).  Its router rows wait for the layer's Wo
 * rows, so a layer's attention and experts run one after the other. */
enum { MK_BLOCK_PARALLEL = 0, MK_BLOCK_SEQUENTIAL = 1 };

/* Weight formats.  FP8_E4M3: the LM head, wqkv, wo, w_gate, w_up and w_down
 * are OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, no infinities) with one fp32 scale per row: the weight is
 * code * scale.  The pages list FP8 weights as a next step (aiweekly.co,
 * paragraph 6) and fix no format; per-row scales are this library's reading.
 * FP4_E2M1: the same matrices as OCP FP4 E2M1 codes (1 sign, 2 exponent bits
 * with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two a
 * byte (element 2j in the low nibble of byte j), with one fp32 scale per row.
 * Router, norm gains, embedding and the KV cache stay bfloat16. */
enum { MK_WEIGHTS_BF16 = 0, MK_WEIGHTS_FP8_E4M3 = 1, MK_WEIGHTS_FP4_E2M1 = 2 };

/* Creates a context for one model shape.  Host only, no GPU call.
 * cfg is copied.  *out receives the context (free with mk_destroy).
 * max_batch is part of the shape, not of the schedule: the workspace layout,
 * the LDS carve-up and the matrix-core tiles are all sized by it, so one
 * context serves one batch capacity (steps may carry 1..max_batch sequences).
 * Source: the 30B-total / 3.3B-active MoE decoder served at batch 1 to 8
 * (latestnews.news, paragraph 1; ainews.surl.tw, paragraph 4). */
int mk_create(const mk_config* cfg, mk_ctx** out);

/* How the static schedule is cut.  All-zero (or a NULL pointer) gives the
 * defaults; no field changes what a step computes, only which compute unit
 * computes it and how much is staged in LDS before a wait.
 *  num_cus: persistent workgroups, one per compute unit (0 = every compute
 *    unit of the current device, which also sets the LDS capacity from the
 *    device; otherwise 160 KB is assumed and no GPU call is made).
 *  attn_units: compute units that run the attention split and the Wo rows
 *    (0 = from ctx_hint: the smaller of the split where attention's K/V
 *    bytes meet the experts' gate/up/down bytes and the split where the QKV
 *    rows plus the K/V reads take least time).  Clamped to
 *    [max_batch*n_kv_heads + 1, num_cus - 2].
 *  router_units: stage-1 units that compute the router rows (0 = default).
 *    Clamped to [1, stage-1 units - 1].
 *  prefetch_bytes: upper bound on the LDS region that receives weight tiles
 *    and K/V pages before a task's wait (0 = all LDS left over by the other
 *    regions; > 0 = at most this many bytes; < 0 = no such region).
 *  pool_64ths: share of each layer's expert gate/up rows, in 64ths, that is
 *    not assigned ahead but claimed at run time, 16 rows at a time, by
 *    whichever unit is idle: the gate/up units once their own rows are done
 *    and the attention units past their chunk (0 or < 0 = none, the default;
 *    at most 63).  On the 30B shape at batch 1 and 8K, 8 to 24 64ths cost
 *    about 11% per step: every claimer's final claim is one more device
 *    round trip, and the attention units' own top-k and normalization before
 *    their pool items delay their Wo rows.  With MK_BLOCK_SEQUENTIAL the
 *    attention units claim after their Wo rows (the router waits for them).
 *    Source: idle units take over tail-end work from the other path
 *    (ainews.surl.tw, paragraph 2).
 *  qkv_units: stage-1 units that take the Wqkv rows and no gate/up rows
 *    (0 = none: the Wqkv rows go to every stage-1 unit but the router's, each
 *    of which then also takes gate/up rows).  With qkv_units > 0 the other
 *    stage-1 units normalize and go straight to the router poll and their
 *    gate/up rows.  Clamped to [1, stage-1 units - router units - 1].
 *    MK_ERR_UNSUPPORTED with MK_BLOCK_SEQUENTIAL.
 *  ctx_hint: expected cached tokens per sequence (0 = 4096); used only to
 *    size attn_units when that is 0. */
typedef struct mk_schedule_params {
  int32_t num_cus;
  int32_t attn_units;
  int32_t router_units;
  int32_t prefetch_bytes;
  int32_t pool_64ths;
  int32_t qkv_units;
  int64_t ctx_hint;
} mk_schedule_params;

/* Fills *p with the defaults (all fields zero). */
void mk_schedule_params_default(mk_schedule_params* p);

/* Builds the static task table (host only apart from the device query,
 * deterministic, integer only), validates it by simulating every queue on the
 * host (deadlock freedom, the fan-in of each counter, signal slots), and
 * reports the size of the device workspace the caller must provide to
 * mk_bind.  params may be NULL (defaults).  Source: the host builds a task
 * table in advance that assigns GEMM tiles and attention splits to the
 * compute units (ainews.surl.tw, paragraph 2; latestnews.news, paragraph 3);
 * every descriptor is 32 int32 (aiweekly.co, paragraph 2). */
int mk_build_schedule(mk_ctx* ctx, const mk_schedule_params* params, size_t* workspace_bytes);

/* Binds caller-owned device buffers and uploads the task table into the
 * workspace on `stream` (synchronizes that stream before returning).
 *  weights: host array of n_weights device pointers, n_weights = 3 + 7*n_layers
 *    (3 + 8*n_layers with MK_BLOCK_SEQUENTIAL),
 *    in this order: embed [vocab][hidden], lm_head [vocab][hidden],
 *    final_norm [hidden], then per layer: attn_norm [hidden],
 *    wqkv [(n_q+2*n_kv)*head_dim][hidden] (q rows, then k rows, then v rows),
 *    wo [hidden][n_q*head_dim], router [n_experts][hidden],
 *    w_gate [n_experts][inter][hidden], w_up [n_experts][inter][hidden],
 *    w_down [n_experts][hidden][inter]; with MK_BLOCK_SEQUENTIAL then, after
 *    every layer's seven, one moe_norm [hidden] per layer.
 *    With weight_format MK_WEIGHTS_FP8_E4M3 each of lm_head, wqkv, wo,
 *    w_gate, w_up and w_down is one buffer: the [rows][cols] E4M3 codes
 *    (one byte each, same row order as above; an expert tensor's rows are
 *    [n_experts * rows]) followed at byte rows*cols by rows fp32 row scales.
 *    With MK_WEIGHTS_FP4_E2M1 the same, with cols / 2 bytes of E2M1 codes per
 *    row and the scales at byte rows*cols/2.
 *  k_pool: device, [n_layers][num_pages][n_kv_heads][page_size][head_dim] bf16.
 *  v_pool: device, [n_layers][num_pages][n_kv_heads][head_dim][page_size] bf16
 *    (dims-major inside a page, the layout the P*V matrix-core product reads).
 *  workspace: device, at least the size mk_build_schedule reported, 256-byte aligned.
 * The buffers must stay valid until the context is destroyed or bound again.
 * Errors: MK_ERR_STATE before mk_build_schedule; MK_ERR_INVALID_ARG for a
 * wrong weight count, a null or misaligned pointer (weights and pools 16
 * bytes) or a short workspace; MK_ERR_HIP if the upload fails.
 * Source: BF16 weights of the 30B-total mixture-of-experts decoder and a paged
 * KV cache (latestnews.news, paragraphs 1 and 3; ainews.surl.tw, paragraph 2);
 * the V layout inside a page is this library's choice for the matrix cores. */
int mk_bind(mk_ctx* ctx, const void* const* weights, int32_t n_weights, void* k_pool, void* v_pool,
            void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code that will be captured
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc): the
 * same as mk_bind, but the workspace is the library's static one, a 256-byte
 * aligned array of mk_scratch_capacity() bytes (64 MiB) that every GPU the
 * library runs on holds until the process ends.  Binds on the current device;
 * makes no device or host allocation (no hipMalloc, hipFree or allocating
 * library call).  Uploads the task table and clears the counters, tickets,
 * error word and epoch-tagged words, like mk_bind.
 * Errors: MK_ERR_INVALID_ARG if the workspace mk_build_schedule reported is
 * larger than mk_scratch_capacity() (nothing is bound then), or for the
 * argument errors of mk_bind; MK_ERR_HIP if the array's device address cannot
 * be found.
 * One array per GPU: binding another context on the same device overwrites
 * this one's table and state, after which this context's calls fail with
 * MK_ERR_STATE until it is bound again.  Calls that overlap on one GPU (two
 * contexts' steps in flight on different streams, or a bind while a step
 * runs) race on the array and give wrong results. */
int mk_bind_scratch(mk_ctx* ctx, const void* const* weights, int32_t n_weights, void* k_pool, void* v_pool,
                    void* stream);

/* Size in bytes of the static workspace mk_bind_scratch uses (host only). */
size_t mk_scratch_capacity(void);

/* Enqueues one decode step for a ragged batch of n sequences (1 <= n <= max_batch).
 *  d_tokens: device int32[n], the new token of each sequence.
 *  d_page_table: device int32[n][max_pages_per_seq], physical page of each
 *    logical page (-1 = none).  Shared by all layers.
 *  d_seq_lens: device int32[n], tokens already cached; the new token sits at
 *    position seq_lens[b].  Its K/V are written to slot seq_lens[b] % page_size
 *    of page page_table[b][seq_lens[b] / page_size]; attention covers
 *    positions 0..seq_lens[b].  seq_lens is not modified: the caller advances it.
 *    The page that receives a sequence's new token must not appear in another
 *    sequence's row of the page table in the same step (pages are read before
 *    the new entries are written; shared prefix pages are fine).
 *  d_logits: device float[n][vocab], written.
 *  d_next_tokens: device int32[n] receiving the next token (the greedy argmax,
 *    lowest id on ties, or the draw mk_set_sampling asks for), or NULL.
 * Asynchronous.  One step per context may be in flight at a time; steps on
 * one stream are ordered.  Device-detected errors (bad token, page or length;
 * a dependency wait past the spin limit) are sticky: read them with
 * mk_get_error.  Host-side errors: MK_ERR_STATE (not bound, or a device error
 * not yet cleared by mk_reset), MK_ERR_INVALID_ARG (n outside [1, max_batch],
 * a null buffer), MK_ERR_HIP (the launch failed).
 * Source: one persistent kernel runs the whole decode forward pass of a
 * ragged batch of 1 to 8 sequences over a paged KV cache (latestnews.news,
 * paragraph 3; ainews.surl.tw, paragraphs 1, 2 and 4). */
int mk_decode_step(mk_ctx* ctx, int32_t n, const int32_t* d_tokens, const int32_t* d_page_table,
                   const int32_t* d_seq_lens, float* d_logits, int32_t* d_next_tokens, void* stream);

/* Enqueues `steps` decode steps of the same ragged batch in ONE launch
 * of the persistent kernel: step s (0-based) feeds each sequence the token
 * step s - 1 picked (greedy or sampled, mk_set_sampling; step 0: d_tokens), writes K/V at position
 * seq_lens[b] + s and attends over 0..seq_lens[b] + s.  No host round trip
 * and no kernel boundary between steps.
 *  d_next_tokens: device int32[steps][n], required when steps > 1: the
 *    token every step picked.
 *  d_logits: device float[n][vocab]: the logits of the last step.
 *  The page table must hold every position up to seq_lens[b] + steps - 1;
 *  seq_lens is not modified (the caller advances it by `steps`).
 * The result equals `steps` calls of mk_decode_step that feed back the picked
 * token, bit for bit.  Not combinable with mk_set_layer_inputs.
 * Errors: as mk_decode_step; MK_ERR_INVALID_ARG for steps outside
 * [1, 2^20] or a missing d_next_tokens with steps > 1; MK_ERR_STATE with
 * the layer-input hook set.
 * Source: the whole decode loop in one persistent kernel with no launch or
 * host synchronization between operations (aiweekly.co, paragraph 2;
 * ainews.surl.tw, paragraph 1); a step-after-step loop is the next step of
 * that idea. */
int mk_decode_steps(mk_ctx* ctx, int32_t n, int32_t steps, const int32_t* d_tokens, const int32_t* d_page_table,
                    const int32_t* d_seq_lens, float* d_logits, int32_t* d_next_tokens, void* stream);

/* One step whose batch entries may belong to the same sequence: chunked
 * prefill mixed with decode.  Arguments as mk_decode_step; each entry b is
 * one token at position seq_lens[b] of the sequence its page-table row
 * names.  Entries of one sequence give it the same row and distinct
 * positions (a chunk of its prompt, say positions p .. p + k - 1 in k
 * entries); entries of other sequences decode as usual in the same launch.
 * Every entry's new K/V is written before any entry's attention reads the
 * pages, and entry b attends over positions 0..seq_lens[b] of its row, so a
 * chunk entry sees the earlier tokens of its chunk: the result equals running
 * the entries one at a time, in order of position within each sequence, as
 * single-token decode steps.  Every position below seq_lens[b] must hold K/V
 * (written before, or by an entry of this step).  Logits and next tokens are
 * written for every entry (a prefill chunk's last entry gives the first
 * generated token).  This step reads no K/V page before its waits, so it is
 * slower per token than mk_decode_step.  Errors: as mk_decode_step.
 * Source: the pages list prefill running apart from decode, which it pauses,
 * as a limit of the engine and mixed prefill and decode as what to watch next
 * (ainews.surl.tw, paragraph 4; aiweekly.co, paragraph 6). */
int mk_mixed_step(mk_ctx* ctx, int32_t n, const int32_t* d_tokens, const int32_t* d_page_table,
                  const int32_t* d_seq_lens, float* d_logits, int32_t* d_next_tokens, void* stream);

/* Synchronizes `stream`, reads the sticky device error word and clears it.
 * *code receives 0 or an MK_ERR_DEVICE_* code; *cu and *task (may be NULL)
 * the workgroup and task that raised it.  After a device error the context
 * needs mk_reset before the next step.  Errors: MK_ERR_STATE when not bound,
 * MK_ERR_HIP when the read fails.  Source: the dependency counters live in
 * global memory (ainews.surl.tw, paragraph 2; aiweekly.co, paragraph 3); the
 * pages say nothing of failures: a bounded wait and a sticky error word that
 * makes every other wait give up (so the grid drains) are this library's
 * reading of how such a kernel must fail. */
int mk_get_error(mk_ctx* ctx, int32_t* code, int32_t* cu, int32_t* task, void* stream);

/* Clears counters, tickets, the error word and the epoch-tagged words on
 * `stream` with a fill kernel, and restarts the epoch.  Errors: MK_ERR_STATE
 * when not bound, MK_ERR_HIP when the fill cannot be launched.  Source: as
 * mk_get_error (the counters of ainews.surl.tw, paragraph 2, are never reset
 * between steps: each step waits for epoch times fan-in). */
int mk_reset(mk_ctx* ctx, void* stream);

/* Sets the bound of every dependency wait in microseconds (default 2e6);
 * a wait past it raises MK_ERR_DEVICE_TIMEOUT and the grid drains.  Errors:
 * MK_ERR_INVALID_ARG for a bound below 1.  Host only; applies from the next
 * step.  Source: as mk_get_error. */
int mk_set_spin_limit_us(mk_ctx* ctx, int64_t microseconds);

/* Test hook for checking each layer in isolation: when d_x is not NULL,
 * every layer l >= 1 and the final RMSNorm read their input residual from
 * the caller's device buffer d_x (float [n_layers+1][max_batch][hidden],
 * slot 0 unused) instead of the residual the previous layer wrote, so each
 * layer runs on inputs the caller chose (e.g. a reference implementation's).
 * Layer outputs are still written to the workspace (mk_get_ws_offsets).
 * NULL restores normal operation.  Host only; applies from the next step.
 * Errors: MK_ERR_INVALID_ARG for a pointer not 4-byte aligned.  A test hook
 * with no counterpart in the pages: it lets each layer be compared with a
 * reference on the reference's own inputs. */
int mk_set_layer_inputs(mk_ctx* ctx, const float* d_x);

/* Per-task timeline: when d_records is not NULL, every task q < capacity
 * writes eight uint64 at d_records[8*q], readings of the constant 100 MHz
 * clock (s_memrealtime): [0] its workgroup fetched it, [1] its dependencies
 * were met, [2..5] phase marks inside the task body (0 where the body has
 * fewer phases), [6] it had signalled, [7] unused.  Tasks are numbered as
 * in mk_copy_schedule.  NULL turns tracing off.  Host only; applies from
 * the next step.  Errors: MK_ERR_INVALID_ARG for capacity < 1 or a pointer
 * not 8-byte aligned.  Instrumentation with no counterpart in the pages. */
int mk_set_trace(mk_ctx* ctx, uint64_t* d_records, int64_t capacity);

/* How each step picks the next token (d_next_tokens, and the token fed to the
 * next step of a multi-step launch).  temperature 0 (the default): the greedy
 * argmax of the logits, ties to the lowest id.  temperature T > 0: a draw
 * from softmax(logits / T) by the Gumbel-max rule, the argmax over i of
 * logits_i / T + g_i (ties to the lowest id), with g_i = -log(-log(u_i)) and
 * u_i = (top 53 bits of SplitMix64 output n + 1/2) / 2^53, where output n of
 * the generator seeded with `seed` is its finalizer applied to
 * seed + (n + 1) * 0x9E3779B97F4A7C15, and n = (p * max_batch + b) * vocab + i
 * for batch slot b whose step input token sits at position p.  The draw
 * depends only on (seed, p, b, i) and the logits, so it repeats exactly.
 * The logits written to d_logits stay the unscaled ones.  Source: the pages
 * call the engine's sampling options incomplete (ainews.surl.tw, the
 * paragraph on limitations); this is the plainest sampling that needs no
 * sort of the vocabulary.  Errors: MK_ERR_INVALID_ARG for a negative, NaN or
 * infinite temperature, or one so small that 1/T overflows.  Host only;
 * applies from the next step. */
int mk_set_sampling(mk_ctx* ctx, double temperature, uint64_t seed);

/* Top-p (nucleus) sampling on top of mk_set_sampling's temperature draw:
 * with temperature T > 0 and top_p < 1, the draw is the same Gumbel-max rule
 * restricted to the nucleus, every token whose logit / T is at least the
 * largest threshold that keeps probability mass >= top_p of softmax(logits / T)
 * (tokens tied at the threshold included).  The masses are summed as 32-bit
 * fixed-point integers, so the threshold does not depend on summation order;
 * it can differ from an exact-arithmetic one only where the mass of the tokens
 * at a threshold is within that rounding of top_p.  top_p = 1 (the default)
 * switches it off; it has no effect at temperature 0.
 * Errors: MK_ERR_INVALID_ARG for a null context or top_p outside (0, 1].
 * Source: the pages call the engine's sampling options incomplete
 * (ainews.surl.tw, paragraph 4); the nucleus rule is this library's reading. */
int mk_set_top_p(mk_ctx* ctx, float top_p);

/* Thread-local text of the last failure on the calling thread. */
const char* mk_last_error_message(void);
/* Frees the context's host state (device buffers stay the caller's); NULL is a no-op. */
void mk_destroy(mk_ctx* ctx);

/* ---- host-only introspection (no GPU call; for tests and tooling) ----
 * The task table they expose is the host-built schedule of ainews.surl.tw,
 * paragraph 2, with 32-int32 descriptors (aiweekly.co, paragraph 2).  The
 * calls that take a context return MK_ERR_STATE before mk_build_schedule
 * (or when it is NULL); the others MK_ERR_INVALID_ARG for a null input, and
 * all MK_ERR_INVALID_ARG for a short output buffer (mk_copy_schedule skips a
 * NULL one). */

typedef struct mk_schedule_info {
  int32_t num_cus;
  int32_t n_tasks;
  int32_t n_counters;
  int32_t n_attn;      /* attention split tasks per layer */
  int32_t n_gateup;    /* expert gate/up tasks per layer */
  int32_t n_out;       /* output-row tasks per layer */
  int32_t n_lmhead;    /* LM head tasks */
  int32_t task_int32s; /* int32 fields per task descriptor (32) */
  int64_t lds_bytes;   /* dynamic LDS per workgroup */
  int64_t workspace_bytes;
} mk_schedule_info;

int mk_get_schedule_info(const mk_ctx* ctx, mk_schedule_info* out);

/* Copies the task table (n_tasks * 32 int32) and the per-CU queue offsets
 * (num_cus + 1 int32) into host buffers of the given capacities. */
int mk_copy_schedule(const mk_ctx* ctx, int32_t* tasks, int64_t tasks_cap, int32_t* queue_off, int64_t off_cap);

/* Re-runs the host simulation of the built table.  Returns MK_OK or
 * MK_ERR_SCHEDULE; *completed receives the number of tasks that ran. */
int mk_validate_schedule(const mk_ctx* ctx, int32_t* completed);

/* Simulates an arbitrary task table (n_tasks * 32 int32, queue offsets of
 * num_cus + 1 int32, n_counters counters) the way mk_validate_schedule does:
 * every wait must name the full fan-in of its counter, and running each
 * queue in order, a task at a time whenever its waits are met, must finish
 * every task.  Returns MK_OK or MK_ERR_SCHEDULE (MK_ERR_INVALID_ARG for a
 * malformed table); *completed receives the number of tasks that ran. */
int mk_simulate_table(const int32_t* tasks, int32_t n_tasks, const int32_t* queue_off, int32_t num_cus,
                      int32_t n_counters, int32_t* completed);

/* Host mirror of the kernel's runtime attention split: for seq_lens[0..n),
 * n_kv heads and n_tasks split tasks of which the first n_lead (>= n * n_kv)
 * lead one (sequence, kv head) segment each, writes the chunk length in
 * tokens to *chunk and, per task, (b, kv head, first token, end token) into
 * plan[n_tasks][4] (b = -1 for an idle task).  Lead task m < n * n_kv takes
 * the first chunk of segment m (b = m / n_kv, head m % n_kv); tasks n_lead ..
 * take the other chunks of all segments in order.  The megakernel uses
 * n_lead = max_batch * n_kv and n_tasks = the schedule's n_attn. */
int mk_attn_plan(const int32_t* seq_lens, int32_t n, int32_t n_kv, int32_t n_tasks, int32_t n_lead, int32_t page_size,
                 int32_t* chunk, int32_t* plan);

/* Offsets (bytes from the workspace base) of the per-layer activation
 * buffers, for debugging and layer-by-layer comparison.  The normalized input
 * of a layer is not among them: it lives only in each unit's LDS.  The router
 * logits (the router rows times it, in fp32) and the new K/V entries pin it
 * down, and the top-k margin of a layer is the gap between its k-th and
 * (k+1)-th router logit in the `router` buffer.
 *  x: float [n_layers+1][max_batch][hidden] residual entering each layer l >= 1 and the
 *     final norm (slot 0 unused), as the step summed it from layer l-1's outputs, also when
 *     mk_set_layer_inputs feeds the layers other inputs
 *  qkv: float [n_layers][max_batch][(n_q+2*n_kv)*head_dim] before rotation
 *  router: float [n_layers][max_batch][n_experts]
 *  attn_out: bf16 [n_layers][max_batch][n_q*head_dim]
 *  h: bf16 [n_layers][max_batch*top_k][inter] (row b*top_k+j: j-th expert of token b)
 *  sel: int32 [n_layers][max_batch][top_k] experts chosen for each token, best first
 *  moe_half: float [n_layers+1][max_batch][hidden]: slot l+1 holds x_l + moe_l, layer l's
 *     residual plus its expert sum (slot 0 unused)
 *  attn_half: float [n_layers][max_batch][hidden]: layer l's attention output times Wo;
 *     x_{l+1} is moe_half[l+1] + attn_half[l] */
typedef struct mk_ws_offsets {
  int64_t x, qkv, router, attn_out, h, sel, moe_half, attn_half;
} mk_ws_offsets;

int mk_get_ws_offsets(const mk_ctx* ctx, mk_ws_offsets* out);

#ifdef __cplusplus
}
#endif

#endif /* MK_H */
