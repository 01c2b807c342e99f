// Internal types shared by the host scheduler (mk_host.cpp) and the
// megakernel (mk_kernel.hip): the task descriptor, counter numbering, the
// kernel argument block and the runtime attention-split function.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MK_HD __host__ __device__ inline
#else
#define MK_HD inline
#endif

namespace mk {

constexpr int kThreads = 512;      // 8 wave64 per workgroup, one workgroup per CU
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBatch = 8;
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 128;   // the top-k's expert pass covers lanes e and e + 64 of one wave
constexpr int kMaxGroup = 8;       // q heads per kv head
constexpr int kTaskInts = 32;      // 128-byte descriptor
constexpr int kGuPass = 256;       // gate/up virtual rows per pass of one task
constexpr int kGuItem = 16;        // gate/up virtual rows per item of the shared pool
constexpr int kLmPass = 512;       // LM head rows per pass of one task
constexpr int kMfmaRedBytes = 16 * 1024; // region C bytes for the matrix-core path's partial tiles (batch >= 2)
constexpr int kTopPBins = 2048;  // top-p threshold search: buckets per radix pass (11 bits)
constexpr int kTraceWords = 8;     // per task: fetch, ready, 4 phase marks, done, spare
constexpr int kLdsB = 8192;        // LDS region B: top-k state, flags, reductions, router logits
constexpr int kTopKScratch = 4 * kMaxExperts + kMaxBatch * kMaxExperts + kWaves * 4 * kMaxTopK * 4;  // region C bytes the top-k borrows

enum Op : int32_t {
  OP_PRE = 1,     // RMSNorm + rows of [Wq; Wk; Wv] or of the router
  OP_ATTN = 2,    // paged split-KV attention chunk; a (seq, kv head) segment's lead combines
  OP_GATEUP = 3,  // router top-k + rows of the selected experts' gate/up + SwiGLU
  OP_OUT = 4,     // rows of the selected experts' down projection + residual update
  OP_LMHEAD = 5,  // final RMSNorm + LM head rows; last arriver takes the argmax
  OP_WO = 6,      // rows of Wo times the merged attention output (run by the attention units)
  OP_GUTAIL = 7,  // an attention unit past its chunk takes gate/up rows from the layer's shared pool
  OP_KVW = 8,     // a segment lead's unit: (mixed steps) the new K/V of its (sequence, kv head), then its signal
};

// One task: 32 int32 (128 bytes, one cache line).
struct Task {
  int32_t op;
  int32_t layer;
  int32_t wait[2];    // counter index or -1
  int32_t fanin[2];   // signals per step on that counter
  int32_t signal;     // counter this task adds one to when done, or -1
  int32_t r0, r1;     // row range (PRE, OUT, LMHEAD)
  int32_t idx, count; // index of this task among the op's tasks of the layer, and their number
  int32_t late_wait;  // host simulator only: a counter the task's body waits on after its first
  int32_t late_fanin; // part (-1 = none); the kernel waits there by other means (a segment ticket)
  int32_t slot;       // this task's index among the tasks signalling its counter: 0 .. (signals) - 1
  int32_t tagged;     // 1: consumers read this task's output as epoch-tagged words (value | epoch << 32),
                      // so its signal is an edge for the host simulator only: on the device no counter
                      // add and no wait for the stores to complete
  int32_t next_layer, next_r0, next_r1;  // OUT: the PRE task that follows on this queue (rows; r1 = 0: none),
                                         // whose weight tile the OUT task copies into LDS while it waits
  int32_t report;     // host simulator only: a counter this task feeds by other means (a non-lead
                      // attention chunk reports to its segment's ticket), or -1
  int32_t pad[13];
};
static_assert(sizeof(Task) == kTaskInts * 4, "task descriptor is 128 bytes");

// Counters: per layer l, kCtrPerLayer of them.  A counter is kSubCounters
// words, each in its own 128-byte line; the task with slot s adds one to word
// s % kSubCounters, and a wait is over when the words sum to epoch * fan-in
// (no reset between steps).  Spreading the adds keeps any one line from
// serializing many of them, and a waiter reads only kSubCounters lines.
enum CtrSlot : int32_t { C_QKV = 0, C_ROUTER = 1, C_ATTN = 2, C_GATEUP = 3, C_XNEXT = 4, C_DONE = 5, C_WO = 6,
                         C_CHUNK = 7,   // simulation only (the leads' ticket waits)
                         C_KVW = 8 };   // the step's new K/V written (every lead signals; mixed steps wait)
constexpr int kCtrPerLayer = 9;
constexpr int kSubCounters = 16;
constexpr int kSubStride = 32;                           // words between sub-counters (128 bytes)
constexpr int kCounterWords = kSubCounters * kSubStride;

MK_HD int ctr_index(int layer, int slot) { return layer * kCtrPerLayer + slot; }

// Error word layout (int32): code, cu, task, aux, abort flag.
enum ErrSlot : int32_t { E_CODE = 0, E_CU = 1, E_TASK = 2, E_AUX = 3, E_ABORT = 4, E_WORDS = 8 };

struct KArgs {
  // shape
  int32_t L, H, nq, nkv, d, E, topk, I, V, ps, max_batch, max_pages, num_pages;
  int32_t qkv_rows, group;
  float eps;
  // schedule
  int32_t n_attn, n_gu, n_lm;
  int32_t gu_rows_max, out_rows_max, lm_rows_max;  // largest row range of one task
  int32_t lds_b, lds_c, lds_p;                     // LDS region offsets (bytes)
  int32_t pf_bytes;                                // size of the prefetch region P (K/V pages, merge partials)
  int32_t pf_wide;                                 // bytes of the PRE / WO weight tile region, which starts tile_off
                                                   // bytes into region C and runs to the end of LDS
  int32_t tile_off;                                // (region C below it: the output task's expert contributions)
  int32_t gu_pool;                                 // 64ths of a layer's gate/up virtual rows in the shared pool
  int32_t gu_items;                                // pool items per layer at the largest expert count
  int32_t gu_parts;                                // tasks per layer that claim from the pool
  const Task* tasks;
  const int32_t* queue_off;
  uint32_t* flags;      // counters: [(L + 1) * kCtrPerLayer][kCounterWords]
  uint32_t* tickets;    // attention tickets [L][max_batch][nkv], then 1 for the LM head
  int32_t* err;         // E_WORDS
  uint64_t* rll;        // router logits as epoch-tagged words [L][max_batch][E] (zeroed with the counters)
  uint32_t* claims;     // per layer: items of the shared gate/up pool claimed so far (zeroed with the counters)
  const uint64_t* wtab; // device pointers of the weights
  const double* inv_freq; // [d/2]
  // activations
  float* x;             // [L+1][max_batch][H]: index l+1 holds x_l + moe_l (the expert half of x_{l+1})
  float* xr;            // [L+1][max_batch][H]: x_l for l >= 1 as the kernel summed it (a record for the caller)
  float* qkv;           // [L][max_batch][qkv_rows]
  float* rlog;          // [L][max_batch][E]
  float* attn_part;     // [L][n_attn][attn_part_stride(group, d)]
  uint16_t* attn_out;   // [L][max_batch][nq*d]
  float* wo_out;        // [L][max_batch][H] attention output times Wo (the attention half of x_{l+1})
  uint16_t* h;          // [L][max_batch*topk][I]
  float* lm_part;       // [n_lm][max_batch][2] (value, index as float bits)
  int32_t* sel_out;     // [L][max_batch][topk] experts chosen per token
  const float* x_in;    // test hook: layer inputs [L+1][max_batch][H] read instead of x (NULL = off)
  uint64_t* trace;      // per task: s_memrealtime at fetch, dependencies met, done (NULL = off)
  int64_t trace_cap;    // tasks the trace buffer holds
  // KV pools
  uint16_t* k_pool;
  uint16_t* v_pool;
  // step
  int32_t n;
  uint32_t epoch;
  const int32_t* tokens;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* logits;
  int32_t* next_tok;         // [nsteps][n] greedy tokens (step s > 0 reads step s - 1's), or NULL at one step
  uint64_t spin_limit_ticks; // s_memrealtime ticks (100 MHz)
  double inv_temp;           // sampling: 1 / temperature, or 0 for the greedy argmax
  uint64_t seed;             // sampling: generator seed
  float top_p;               // sampling: nucleus mass (1: every token)
  int32_t nsteps;            // decode steps in this launch
  int32_t kv_sync;           // mixed step: entries may share a sequence; attention reads pages only after
                             // every entry's new K/V is written (the KVW tasks), and no page is read before
  int32_t step;              // the step being run (set by the kernel: epoch + step, positions + step)
  int32_t seq_block;         // sequential block: attention-side norms read x_l alone, the MoE path's norm
                             // reads x_l + this layer's Wo rows with its own gain, and the output tasks
                             // write the whole next residual
};

// Weight table order.
enum WIdx : int32_t { W_EMBED = 0, W_LM_HEAD = 1, W_FINAL_NORM = 2, W_LAYER0 = 3 };
enum WLayer : int32_t { WL_NORM = 0, WL_QKV = 1, WL_O = 2, WL_ROUTER = 3, WL_GATE = 4, WL_UP = 5, WL_DOWN = 6, WL_COUNT = 7 };
MK_HD int widx(int layer, int which) { return W_LAYER0 + layer * WL_COUNT + which; }
// the sequential block's MoE norm gain of a layer, after every layer's WL_COUNT tensors
MK_HD int widx_moe_norm(int n_layers, int layer) { return W_LAYER0 + n_layers * WL_COUNT + layer; }

// Floats per attention partial (one split task): outputs [group][d], then the
// running maxima [kMaxGroup] and sums [kMaxGroup]; a multiple of 4, so every
// partial starts 16-byte aligned.
MK_HD int attn_part_stride(int group, int d) { return group * d + 2 * kMaxGroup; }

// Pages of a split task's chunk copied into LDS before its inputs are ready
// (flag words hold one valid bit per page).
constexpr int kMaxLdsPages = 64;

// ---------------------------------------------------------------------------
// Runtime attention split (identical on host and device).
//
// Every (sequence b, kv head g) pair is a segment of n_b = seq_len_b + 1
// positions.  All segments are cut into chunks of C tokens (C a multiple of
// the page size, so chunks start on page boundaries; the last chunk of a
// segment is shorter), C being the smallest multiple of the page size for
// which the number of chunks fits in n_tasks.  Chunks are numbered segment
// by segment (b major, g minor); chunk number i goes to split task i.

MK_HD int64_t attn_count_chunks(const int32_t* lens1, int n, int nkv, int64_t C) {
  int64_t c = 0;
  for (int b = 0; b < n; ++b) c += (int64_t)nkv * ((lens1[b] + C - 1) / C);
  return c;
}

// lens1[b] = positions of sequence b (seq_len + 1, already clamped >= 1).
// Requires n * nkv <= n_tasks.  The number of chunks is at most n_tasks.
MK_HD int64_t attn_chunk_len(const int32_t* lens1, int n, int nkv, int n_tasks, int ps) {
  int64_t maxlen = 1;
  for (int b = 0; b < n; ++b) maxlen = lens1[b] > maxlen ? lens1[b] : maxlen;
  int64_t hi = (maxlen + ps - 1) / ps;  // chunk = whole segment: n*nkv chunks
  int64_t lo = 1;
  while (lo < hi) {                      // smallest page count per chunk that fits
    int64_t mid = (lo + hi) / 2;
    if (attn_count_chunks(lens1, n, nkv, mid * ps) <= n_tasks) hi = mid; else lo = mid + 1;
  }
  return lo * ps;
}

// Split task i -> chunk.  Tasks 0 .. nlead - 1 are the segment leads: task
// m < n * nkv takes the first chunk of segment m (b = m / nkv, g = m % nkv)
// and later merges the segment; tasks nlead .. take the other chunks of all
// segments in chunk order.  *chunk is the chunk's number in segment order
// (segment b major, g minor; the segment's chunks are first .. first + nch - 1).
// With n_tasks split tasks, chunk lengths come from
// attn_chunk_len(..., n_tasks - nlead + n * nkv, ...), so the non-first
// chunks fit in tasks nlead .. n_tasks - 1.  Returns false for an idle task.
MK_HD bool attn_task_chunk(const int32_t* lens1, int n, int nkv, int64_t C, int i, int nlead, int* b, int* g, int* t0,
                           int* t1, int* first_chunk, int* nchunks, int* chunk) {
  int64_t base = 0;
  if (i < nlead) {
    if (i >= n * nkv) return false;
    const int bb = i / nkv;
    for (int s = 0; s < i; ++s) base += (lens1[s / nkv] + C - 1) / C;
    *b = bb;
    *g = i % nkv;
    *t0 = 0;
    *t1 = (int)(C < lens1[bb] ? C : lens1[bb]);
    *first_chunk = (int)base;
    *nchunks = (int)((lens1[bb] + C - 1) / C);
    *chunk = (int)base;
    return true;
  }
  int64_t k = i - nlead;
  for (int bb = 0; bb < n; ++bb) {
    const int64_t per = (lens1[bb] + C - 1) / C;
    for (int gg = 0; gg < nkv; ++gg) {
      if (k < per - 1) {
        const int64_t j = k + 1;
        *b = bb;
        *g = gg;
        *t0 = (int)(j * C);
        const int64_t e = (j + 1) * C;
        *t1 = (int)(e < lens1[bb] ? e : lens1[bb]);
        *first_chunk = (int)base;
        *nchunks = (int)per;
        *chunk = (int)(base + j);
        return true;
      }
      k -= per - 1;
      base += per;
    }
  }
  return false;
}

}  // namespace mk
