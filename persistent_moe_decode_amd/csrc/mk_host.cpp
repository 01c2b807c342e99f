// Host half of the C ABI in include/mk.h: argument checks, the static
// schedule builder and its simulator, the workspace layout, binding of
// caller-owned buffers and the per-step launch.
//
// The schedule follows the pages' description of the table (ainews.surl.tw,
// paragraph 2: tiles and attention splits assigned to compute units in
// advance; aiweekly.co, paragraphs 2-3: fixed-size descriptors, a task waits
// on one count) with its own layout: one queue per compute unit, per layer
//   attention units:  ATTN (a chunk; leads merge)  ->  WO (Wo rows: the attention half)
//   stage-1 units:    PRE (norm + Wqkv / router rows)  ->  GATEUP  ->  OUT (down rows: the expert half)
// then LM head rows on every unit.  (Opt-in: pool tasks on the attention units
// after their chunk; dedicated Wqkv units.)  A counter is a set of sub-counters in separate lines;
// the task with slot s (its index among the counter's signallers) adds one to
// sub-counter s mod 16, and a wait ends when they sum to epoch * fan-in, so
// nothing is reset between steps.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_types.h"

using namespace mk;

extern "C" int mkk_launch_step(const KArgs* a, int grid, size_t lds_bytes, hipStream_t stream);
extern "C" int mkk_launch_step_fp8(const KArgs* a, int grid, size_t lds_bytes, hipStream_t stream);
extern "C" int mkk_launch_step_fp4(const KArgs* a, int grid, size_t lds_bytes, hipStream_t stream);
extern "C" int mkk_launch_step_seq(const KArgs* a, int grid, size_t lds_bytes, hipStream_t stream);
extern "C" int mkk_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t stream);
extern "C" size_t mkk_scratch_bytes();
extern "C" int mkk_scratch(int* device, void** ptr);

namespace {

thread_local std::string g_msg;

int fail(int code, const std::string& m) {
  g_msg = m;
  return code;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t state = 0, n_state_u32 = 0;  // counter flags, tickets, error word (zeroed by mk_reset)
  size_t ctr = 0, tickets = 0, err = 0, rll = 0, claims = 0;  // (u32 offsets in the state region)
  size_t tasks = 0, queue_off = 0, wtab = 0, inv_freq = 0;
  size_t x = 0, xr = 0, qkv = 0, rlog = 0, attn_part = 0, attn_out = 0, wo_out = 0, h = 0, lm_part = 0, sel = 0;
  size_t total = 0;
};

}  // namespace

struct mk_ctx {
  mk_config cfg{};
  bool built = false, bound = false, need_reset = false;
  int ncu = 0, n_attn = 0, n_gu = 0, n_out = 0, n_lm = 0, n_ctr = 0, n_tickets = 0, n_slots = 0;
  int out_rows_max = 0, gu_rows_max = 0, lm_rows_max = 0, pre_rows_max = 0;
  int lds_b = 0, lds_c = 0, lds_p = 0, pf_bytes = 0, pf_wide = 0, tile_off = 0;
  int gu_pool = 0, gu_items = 0, gu_parts = 0;  // the shared gate/up pool
  size_t lds_bytes = 0;
  std::vector<Task> tasks;
  std::vector<int32_t> qoff;
  std::vector<double> inv_freq;  // rotary frequencies theta^(-2i/d), uploaded by bind
  WsLayout ws;
  // bound state
  uint8_t* wsp = nullptr;
  int scratch_dev = -1;  // device whose static workspace this context is bound to, else -1
  uint16_t* kpool = nullptr;
  uint16_t* vpool = nullptr;
  uint32_t epoch = 0;
  int64_t spin_us = 2000000;
  double inv_temp = 0.0;  // sampling (0: greedy)
  float top_p = 1.0f;     // sampling: nucleus mass (1: off)
  uint64_t seed = 0;
  const float* x_in = nullptr;
  uint64_t* trace = nullptr;
  int64_t trace_cap = 0;
};

static int check_config(const mk_config& c) {
  auto bad = [](const char* what) { return fail(MK_ERR_UNSUPPORTED, std::string("unsupported config: ") + what); };
  if (c.n_layers < 1 || c.hidden < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.n_experts < 1 || c.top_k < 1 ||
      c.inter < 1 || c.vocab < 2 || c.num_pages < 1 || c.max_pages_per_seq < 1 || c.max_batch < 1)
    return fail(MK_ERR_INVALID_ARG, "config has a non-positive size");
  if (c.hidden % 128) return bad("hidden % 128 != 0");
  if (c.inter % 128) return bad("inter % 128 != 0");
  if ((c.n_q_heads * c.head_dim) % 128) return bad("n_q_heads*head_dim % 128 != 0");
  if (c.head_dim != 64 && c.head_dim != 128) return bad("head_dim must be 64 or 128");
  if (c.n_q_heads % c.n_kv_heads) return bad("n_q_heads % n_kv_heads != 0");
  if (c.n_q_heads / c.n_kv_heads > kMaxGroup) return bad("more than 8 q heads per kv head");
  if (c.n_experts > kMaxExperts) return bad("n_experts > 128");
  if (c.top_k > kMaxTopK || c.top_k > c.n_experts) return bad("top_k > 8 or > n_experts");
  if (c.page_size != 16) return bad("page_size must be 16");
  if (c.max_batch > kMaxBatch) return bad("max_batch > 8");
  if (!(c.rms_eps >= 0.f) || !(c.rope_theta > 0.0)) return fail(MK_ERR_INVALID_ARG, "bad rms_eps or rope_theta");
  if ((int64_t)c.max_pages_per_seq * c.page_size > (1 << 30)) return bad("context bound too large");
  if (c.weight_format != MK_WEIGHTS_BF16 && c.weight_format != MK_WEIGHTS_FP8_E4M3 &&
      c.weight_format != MK_WEIGHTS_FP4_E2M1)
    return fail(MK_ERR_INVALID_ARG, "unknown weight_format");
  if (c.block_style != MK_BLOCK_PARALLEL && c.block_style != MK_BLOCK_SEQUENTIAL)
    return fail(MK_ERR_INVALID_ARG, "unknown block_style");
  if (c.block_style == MK_BLOCK_SEQUENTIAL && c.weight_format != MK_WEIGHTS_BF16)
    return bad("the sequential block is built for bf16 weights only");
  return MK_OK;
}

// Weight pointers mk_bind takes: 3 global, 7 per layer, and with the
// sequential block one more per layer (the MoE norm gains, after the rest).
static int n_weights_of(const mk_config& f) {
  return 3 + (f.block_style == MK_BLOCK_SEQUENTIAL ? 8 : 7) * f.n_layers;
}

extern "C" int mk_create(const mk_config* cfg, mk_ctx** out) {
  if (!cfg || !out) return fail(MK_ERR_INVALID_ARG, "null argument");
  int r = check_config(*cfg);
  if (r) return r;
  mk_ctx* c = new (std::nothrow) mk_ctx();
  if (!c) return fail(MK_ERR_INVALID_ARG, "out of host memory");
  c->cfg = *cfg;
  *out = c;
  return MK_OK;
}

// Which context each device's static workspace is bound to: binding another context there
// overwrites the table and state of the previous one, whose later calls then fail.
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
mk_ctx* g_scratch_owner[kMaxDevices] = {};
}  // namespace

static void release_scratch(mk_ctx* c) {
  if (c->scratch_dev < 0) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_owner[c->scratch_dev] == c) g_scratch_owner[c->scratch_dev] = nullptr;
  c->scratch_dev = -1;
}

static bool scratch_lost(const mk_ctx* c) {
  if (c->scratch_dev < 0) return false;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_owner[c->scratch_dev] != c;
}

extern "C" void mk_destroy(mk_ctx* ctx) {
  if (!ctx) return;
  release_scratch(ctx);
  delete ctx;
}

extern "C" const char* mk_last_error_message(void) { return g_msg.c_str(); }

// ---------------------------------------------------------------------------
// schedule

static void split_rows(int rows, int parts, int i, int* r0, int* r1) {
  *r0 = (int)((int64_t)rows * i / parts);
  *r1 = (int)((int64_t)rows * (i + 1) / parts);
}

static Task make_task(int op, int layer) {
  Task t;
  std::memset(&t, 0, sizeof t);
  t.op = op;
  t.layer = layer;
  t.wait[0] = t.wait[1] = -1;
  t.late_wait = -1;
  t.signal = -1;
  t.report = -1;
  return t;
}

static int simulate_raw(const Task* tasks, int nt, const int32_t* qoff, int ncu, int n_ctr, int32_t* completed) {
  if (completed) *completed = 0;
  if (nt < 0 || ncu < 1 || n_ctr < 0 || qoff[0] != 0 || qoff[ncu] != nt)
    return fail(MK_ERR_INVALID_ARG, "malformed task table");
  for (int q = 0; q < ncu; ++q)
    if (qoff[q + 1] < qoff[q]) return fail(MK_ERR_INVALID_ARG, "queue offsets not ascending");
  // a task's waits: the two before its body and the one inside it (which, for
  // progress, counts like the others: the task signals only after all three)
  auto waits = [](const Task& t, int k, int* ctr_out, int* fan_out) {
    *ctr_out = k < 2 ? t.wait[k] : t.late_wait;
    *fan_out = k < 2 ? t.fanin[k] : t.late_fanin;
  };
  std::vector<int64_t> ctr(n_ctr, 0), signals(n_ctr, 0);
  for (int i = 0; i < nt; ++i) {
    const Task& t = tasks[i];
    if (t.signal >= n_ctr || t.wait[0] >= n_ctr || t.wait[1] >= n_ctr || t.late_wait >= n_ctr || t.report >= n_ctr)
      return fail(MK_ERR_INVALID_ARG, "counter index out of range");
    if (t.signal >= 0) signals[t.signal]++;
    if (t.report >= 0) signals[t.report]++;
  }
  // the signalling tasks of a counter hold slots 0 .. signals - 1, one each (slots spread the adds over sub-counters)
  std::vector<std::vector<char>> owned(n_ctr);
  for (int c = 0; c < n_ctr; ++c) owned[c].assign((size_t)signals[c], 0);
  for (int i = 0; i < nt; ++i) {
    const Task& t = tasks[i];
    if (t.signal < 0) continue;
    if (t.slot < 0 || t.slot >= signals[t.signal] || owned[t.signal][t.slot])
      return fail(MK_ERR_SCHEDULE, "schedule: task " + std::to_string(i) + " has a signal slot that is out of range or taken");
    owned[t.signal][t.slot] = 1;
  }
  // every wait must name the full fan-in of its counter
  for (int i = 0; i < nt; ++i)
    for (int k = 0; k < 3; ++k) {
      int w, f;
      waits(tasks[i], k, &w, &f);
      if (w >= 0 && signals[w] != f)
        return fail(MK_ERR_SCHEDULE, "schedule: task " + std::to_string(i) +
                                         " waits for a fan-in that differs from the signals on its counter");
    }
  std::vector<int> head(qoff, qoff + ncu);
  int done = 0;
  bool progress = true;
  while (progress) {
    progress = false;
    for (int q = 0; q < ncu; ++q) {
      while (head[q] < qoff[q + 1]) {
        const Task& t = tasks[head[q]];
        bool ready = true;
        for (int k = 0; k < 3; ++k) {
          int w, f;
          waits(t, k, &w, &f);
          if (w >= 0 && ctr[w] < f) ready = false;
        }
        if (!ready) break;
        if (t.signal >= 0) ctr[t.signal]++;
        if (t.report >= 0) ctr[t.report]++;
        head[q]++;
        done++;
        progress = true;
      }
    }
  }
  if (completed) *completed = done;
  if (done != nt) return fail(MK_ERR_SCHEDULE, "schedule: deadlock in host simulation (" + std::to_string(done) +
                                                   " of " + std::to_string(nt) + " tasks ran)");
  return MK_OK;
}

static int simulate(const mk_ctx* c, int32_t* completed) {
  return simulate_raw(c->tasks.data(), (int)c->tasks.size(), c->qoff.data(), c->ncu, c->n_ctr, completed);
}

extern "C" int mk_simulate_table(const int32_t* tasks, int32_t n_tasks, const int32_t* queue_off, int32_t num_cus,
                                 int32_t n_counters, int32_t* completed) {
  if (!tasks || !queue_off) return fail(MK_ERR_INVALID_ARG, "null table");
  return simulate_raw((const Task*)tasks, n_tasks, queue_off, num_cus, n_counters, completed);
}

static WsLayout layout_workspace(const mk_ctx* c) {
  const mk_config& f = c->cfg;
  WsLayout w;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  const size_t B = f.max_batch, L = f.n_layers;
  const size_t qkv_rows = (size_t)(f.n_q_heads + 2 * f.n_kv_heads) * f.head_dim;
  const size_t group = f.n_q_heads / f.n_kv_heads;
  w.state = o;
  w.ctr = 0;
  w.tickets = (size_t)c->n_ctr * kCounterWords;
  w.err = w.tickets + c->n_tickets;
  // epoch-tagged words (8-byte aligned): router logits; then the pool claim counters
  w.rll = align_up(w.err + E_WORDS, 2);
  w.claims = w.rll + 2 * L * B * (size_t)f.n_experts;
  w.n_state_u32 = w.claims + L;
  take(4 * w.n_state_u32);
  w.tasks = take(sizeof(Task) * c->tasks.size());
  w.queue_off = take(4 * (c->ncu + 1));
  w.wtab = take(8 * (size_t)n_weights_of(c->cfg));
  w.inv_freq = take(8 * (f.head_dim / 2));
  w.x = take(4 * (L + 1) * B * f.hidden);
  w.xr = take(4 * (L + 1) * B * f.hidden);
  w.qkv = take(4 * L * B * qkv_rows);
  w.rlog = take(4 * L * B * f.n_experts);
  w.attn_part = take((size_t)4 * L * c->n_attn * attn_part_stride(group, f.head_dim));
  w.attn_out = take(2 * L * B * f.n_q_heads * f.head_dim);
  w.wo_out = take(4 * L * B * f.hidden);
  w.h = take(2 * L * B * f.top_k * f.inter);
  w.lm_part = take(4 * 2 * c->n_lm * B);
  w.sel = take(4 * L * B * f.top_k);
  w.total = o;
  return w;
}

extern "C" void mk_schedule_params_default(mk_schedule_params* p) {
  if (p) std::memset(p, 0, sizeof *p);
}

extern "C" int mk_build_schedule(mk_ctx* c, const mk_schedule_params* params, size_t* workspace_bytes) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  mk_schedule_params p{};
  if (params) p = *params;
  int32_t num_cus = p.num_cus;
  const int64_t ctx_hint = p.ctx_hint;
  if (num_cus < 0 || ctx_hint < 0 || p.attn_units < 0 || p.router_units < 0)
    return fail(MK_ERR_INVALID_ARG, "negative num_cus, ctx_hint, attn_units or router_units");
  const mk_config& f = c->cfg;
  size_t lds_cap = 160 * 1024;
  if (num_cus == 0) {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess)
      return fail(MK_ERR_HIP, "cannot query the current device");
    num_cus = p.multiProcessorCount;
    lds_cap = p.sharedMemPerBlock;
  }
  const int ncu = num_cus;
  const int L = f.n_layers, H = f.hidden, E = f.n_experts, B = f.max_batch;
  const int qkv_rows = (f.n_q_heads + 2 * f.n_kv_heads) * f.head_dim;
  const int group = f.n_q_heads / f.n_kv_heads;
  if (ncu < 2) return fail(MK_ERR_UNSUPPORTED, "need at least 2 compute units");

  // Compute units 0 .. n_attn - 1 run the attention split and no stage-1
  // rows, so their K/V loads are in flight while the other units normalize
  // and project, and then the Wo rows; units n_attn .. ncu - 1 run the
  // stage-1 rows, the selected experts' gate/up rows and the output rows.
  // A stage-1 unit streams weight rows about 2.25x as fast as an attention
  // unit streams K/V pages, so a layer takes at least the longer of
  //   the expert path:    (gate/up + down bytes) / (2.25 * (ncu - n_attn))
  //   the attention path: QKV bytes / (2.25 * (ncu - n_attn)) + K/V bytes / n_attn
  // (the attention of a layer waits for its QKV rows).  The first grows with
  // n_attn; the second is least at n_attn / (ncu - n_attn) =
  // sqrt(2.25 * K/V bytes / QKV bytes).  So n_attn is the smaller of the
  // point where the expert path meets the attention chunks and that minimum:
  // short contexts take the first, long single-sequence contexts the second.
  // FP8 rows at batch 1 count as 1.5 bytes per element: half the bytes of
  // bf16, but a stage-1 unit takes about three quarters of the bf16 time over
  // them (measured on the gate/up rows), the code conversion being the rest.
  // At larger batches each row's conversion is repeated per token and FP8
  // rows cost about what bf16 rows do (measured: the bf16 split is best).
  // FP4 rows take the FP8 figure: with a quarter of the bf16 bytes the
  // stage-1 time is no longer set by the bytes (measured at 8K, batch 1:
  // 103 units, the 1.5 split, beat 90, 115, 128 and 140).
  // The split never changes results.
  const double hint = ctx_hint > 0 ? (double)ctx_hint : 4096.0;
  const double kRate = 2.25;
  const double wb = B == 1 && f.weight_format != MK_WEIGHTS_BF16 ? 1.5 : 2.0;  // per streamed-matrix element
  const double kv_bytes = kRate * hint * B * f.n_kv_heads * f.head_dim * 4.0;
  const double expert_bytes = (double)std::min(E, B * f.top_k) * 3.0 * f.inter * H * wb;
  const double qkv_bytes = (double)qkv_rows * H * wb;
  const double chain = std::sqrt(kv_bytes / qkv_bytes);
  const double n_fit = std::min(ncu * kv_bytes / (kv_bytes + expert_bytes), ncu * chain / (1.0 + chain));
  // The sequential block runs a layer's phases one after another (attention,
  // then the experts).  From batch 2 every unit takes part in every phase in
  // turn: attention on all units (or the first attn_units), the stage-1 rows
  // too.  At batch 1 the parallel block's split does better (measured at 8K:
  // 311.5 against 265.0 tok/s): its attention units issue their next chunk's
  // K/V page copies right after their Wo rows, so those pages stream in while
  // the other units run the experts; at batch 8 the expert phase is long and
  // all units sharing it win (807.1 against 611.4 tok/s).
  const bool seq = f.block_style == MK_BLOCK_SEQUENTIAL;
  const bool all_units = seq && B >= 2;
  int n_attn = all_units ? ncu : (int)std::lround(n_fit);
  if (p.attn_units > 0) n_attn = p.attn_units;
  // attention units 0 .. n_lead - 1 lead a (sequence, kv head) segment each:
  // first chunk and merge, no Wo rows; the others take the remaining chunks
  // and the Wo rows
  const int n_lead = B * f.n_kv_heads;
  n_attn = std::max(n_attn, n_lead + 1);
  // (parallel block: at least one unit each left for the QKV and the router rows)
  n_attn = std::min(n_attn, all_units ? ncu : ncu - 2);
  if (n_attn < n_lead + 1) return fail(MK_ERR_UNSUPPORTED, "too few compute units for the attention split");
  // Stage-1 units n_attn ..: the router's rows go to the last n_rcu of them.
  // Without dedicated QKV units every other stage-1 unit takes Wqkv rows and
  // then gate/up rows; with qkv_units = n_q > 0 the first n_q take only Wqkv
  // rows and the rest (router units included) only gate/up rows, the ones
  // without router rows running a PRE task that just normalizes (no rows, no
  // signal), so their gate/up rows start as soon as the routing is in.
  const int R1 = qkv_rows + E;
  const int s1 = all_units ? 0 : n_attn;  // first stage-1 unit
  const int m1 = ncu - s1;
  int n_rcu = (int)(((int64_t)m1 * E + R1 - 1) / R1);
  if (p.router_units > 0) n_rcu = p.router_units;
  n_rcu = std::min(m1 - 1, std::max(1, n_rcu));
  const int n_q = p.qkv_units > 0 ? std::max(1, std::min(p.qkv_units, m1 - n_rcu - 1)) : 0;
  const int n_qcu = n_q > 0 ? n_q : m1 - n_rcu;  // units with Wqkv rows
  const int gu0 = s1 + n_q;                      // first unit with gate/up rows
  const int n_gu = ncu - gu0;

  // The shared gate/up pool: the last pool/64 of a layer's virtual gate/up rows
  // (one expert's gate and up row each) go out in items of kGuItem rows, claimed
  // at run time by the gate/up tasks once their own rows are done and by a pool
  // task on every non-lead attention unit right after its chunk.  Every claimer
  // ends with one failed claim, so a step adds exactly items + claimers to the
  // layer's claim counter whatever the order: the kernel subtracts
  // (epoch - 1) * (items + claimers) to number this step's items.
  if (seq && (p.qkv_units > 0 || p.pool_64ths > 0))
    return fail(MK_ERR_UNSUPPORTED, "qkv_units and pool_64ths are not supported with the sequential block");
  const int pool = std::max(0, std::min(p.pool_64ths, 63));
  const int64_t rows_max = (int64_t)std::min(E, B * f.top_k) * f.inter;
  const int gu_items = pool > 0 ? (int)((rows_max * pool / 64 + kGuItem - 1) / kGuItem) : 0;
  const int n_pool_tasks = gu_items > 0 ? n_attn - n_lead : 0;
  c->gu_pool = gu_items > 0 ? pool : 0;
  c->gu_items = gu_items;
  c->gu_parts = n_gu + n_pool_tasks;

  c->tasks.clear();
  c->qoff.assign(ncu + 1, 0);
  c->ncu = ncu;
  c->n_attn = n_attn;
  c->n_gu = n_gu;
  c->n_ctr = (L + 1) * kCtrPerLayer;
  c->n_tickets = L * B * f.n_kv_heads + 1;  // attention (seq, kv head) merges, LM argmax

  // Stage-1 rows: no unit has two stage-1 tasks, and the routing is ready as
  // early as the QKV rows.
  auto pre_rows = [&](int q, int* r0, int* r1) {
    *r0 = *r1 = 0;
    if (q < s1) return;
    q -= s1;
    if (q < n_qcu) {
      split_rows(qkv_rows, n_qcu, q, r0, r1);
    } else if (q >= m1 - n_rcu) {
      split_rows(E, n_rcu, q - (m1 - n_rcu), r0, r1);
      *r0 += qkv_rows;
      *r1 += qkv_rows;
    }
  };
  // Output rows (expert down projections, residual) over the stage-1 units;
  // the Wo rows over the attention units, which run them once the chunk
  // groups are merged, while the experts are still in flight.
  auto out_rows = [&](int q, int* r0, int* r1) {
    *r0 = *r1 = 0;
    if (q >= s1) split_rows(H, ncu - s1, q - s1, r0, r1);
  };
  auto wo_rows = [&](int q, int* r0, int* r1) {
    *r0 = *r1 = 0;
    if (q >= n_lead && q < n_attn) split_rows(H, n_attn - n_lead, q - n_lead, r0, r1);
  };
  std::vector<int> n_qkv_tasks(L, 0), n_router_tasks(L, 0), n_out_tasks(L, 0), n_wo_tasks(L, 0);
  int n_lm = 0;
  c->out_rows_max = 0;
  c->lm_rows_max = 0;
  c->pre_rows_max = 0;
  for (int q = 0; q < ncu; ++q) {
    int r0, r1;
    pre_rows(q, &r0, &r1);
    if (r1 > r0) (r0 < qkv_rows ? n_qkv_tasks[0] : n_router_tasks[0])++;
    c->pre_rows_max = std::max(c->pre_rows_max, r1 - r0);
    out_rows(q, &r0, &r1);
    if (r1 > r0) n_out_tasks[0]++;
    c->out_rows_max = std::max(c->out_rows_max, r1 - r0);
    wo_rows(q, &r0, &r1);
    if (r1 > r0) n_wo_tasks[0]++;
    split_rows(f.vocab, ncu, q, &r0, &r1);
    if (r1 > r0) n_lm++;
    c->lm_rows_max = std::max(c->lm_rows_max, r1 - r0);
  }
  for (int l = 1; l < L; ++l) {
    n_qkv_tasks[l] = n_qkv_tasks[0];
    n_router_tasks[l] = n_router_tasks[0];
    n_out_tasks[l] = n_out_tasks[0];
    n_wo_tasks[l] = n_wo_tasks[0];
  }
  c->n_out = n_out_tasks[0];
  c->n_lm = n_lm;

  int lm_i = 0;
  for (int q = 0; q < ncu; ++q) {
    c->qoff[q] = (int)c->tasks.size();
    for (int l = 0; l < L; ++l) {
      int r0, r1;
      pre_rows(q, &r0, &r1);
      const bool has_pre = r1 > r0 || (n_q > 0 && q >= gu0);
      Task pre = make_task(OP_PRE, l);
      if (has_pre) {
        const bool router = r0 >= qkv_rows;
        Task& t = pre;
        if (l > 0) {
          // x_l is the sum of the expert half (output tasks) and the attention half (Wo tasks)
          t.wait[0] = ctr_index(l - 1, C_XNEXT);
          t.fanin[0] = n_out_tasks[l - 1];
          t.wait[1] = ctr_index(l - 1, C_WO);
          t.fanin[1] = n_wo_tasks[l - 1];
        }
        t.r0 = r0;
        t.r1 = r1;
        if (r1 > r0) {
          t.signal = ctr_index(l, router ? C_ROUTER : C_QKV);
          t.tagged = router ? 1 : 0;  // gate/up and output tasks poll the tagged router logits
        }
        if (seq && router) {
          // sequential block: the router reads the norm of x_l + this layer's Wo rows
          t.wait[1] = ctr_index(l, C_WO);
          t.fanin[1] = n_wo_tasks[l];
        }
      }
      // (sequential block: a unit's router rows come after its own Wo rows, which they wait for)
      const bool pre_late = seq && has_pre && r0 >= qkv_rows;
      if (has_pre && !pre_late) c->tasks.push_back(pre);
      // stage 2: attention units run their chunk, the others gate/up rows
      if (q < n_attn) {
        if (q < n_lead) {
          // the new K/V of lead q's (sequence, kv head): written here in mixed steps (the kernel
          // waits for the QKV rows only then), signalled in every step so the counter's targets hold
          Task k = make_task(OP_KVW, l);
          k.wait[0] = ctr_index(l, C_QKV);
          k.fanin[0] = n_qkv_tasks[l];
          k.idx = q;
          k.signal = ctr_index(l, C_KVW);
          c->tasks.push_back(k);
        }
        Task t = make_task(OP_ATTN, l);
        t.wait[0] = ctr_index(l, C_QKV);
        t.fanin[0] = n_qkv_tasks[l];
        t.wait[1] = ctr_index(l, C_KVW);  // waited in mixed steps only
        t.fanin[1] = n_lead;
        t.idx = q;
        t.count = n_attn;
        // leads signal once their segment is merged; the other chunks report
        // to their segment's ticket instead.  Which chunks feed which lead is
        // decided at run time (the split follows the sequence lengths), so the
        // simulator takes the superset: every lead waits, inside its body, for
        // every other chunk task of the layer
        t.signal = q < n_lead ? ctr_index(l, C_ATTN) : -1;
        if (q < n_lead) {
          t.late_wait = ctr_index(l, C_CHUNK);
          t.late_fanin = n_attn - n_lead;
        } else {
          t.report = ctr_index(l, C_CHUNK);
        }
        c->tasks.push_back(t);
        if (n_pool_tasks > 0 && q >= n_lead) {
          // gate/up rows from the shared pool (needs the router logits; polls them itself)
          Task g = make_task(OP_GUTAIL, l);
          g.wait[0] = ctr_index(l, C_ROUTER);
          g.fanin[0] = n_router_tasks[l];
          g.signal = ctr_index(l, C_GATEUP);
          c->tasks.push_back(g);
        }
        wo_rows(q, &r0, &r1);
        if (r1 > r0) {
          Task w = make_task(OP_WO, l);
          w.wait[0] = ctr_index(l, C_ATTN);
          w.fanin[0] = n_lead;
          w.r0 = r0;
          w.r1 = r1;
          w.signal = ctr_index(l, C_WO);
          c->tasks.push_back(w);
        }
      }
      if (pre_late) c->tasks.push_back(pre);
      if (q >= gu0) {
        Task t = make_task(OP_GATEUP, l);
        t.wait[0] = ctr_index(l, C_ROUTER);
        t.fanin[0] = n_router_tasks[l];
        t.idx = q - gu0;
        t.count = n_gu;
        t.signal = ctr_index(l, C_GATEUP);
        c->tasks.push_back(t);
      }
      // OUT
      out_rows(q, &r0, &r1);
      if (r1 > r0) {
        // expert rows (needs gate/up), then the expert half of the residual
        // update, x_l + moe_l; the next layer adds the Wo rows' half
        Task t = make_task(OP_OUT, l);
        t.wait[0] = ctr_index(l, C_GATEUP);
        t.fanin[0] = c->gu_parts;
        t.wait[1] = ctr_index(l, C_ROUTER);  // for the top-k, where no gate/up task left it in LDS
        t.fanin[1] = n_router_tasks[l];
        t.r0 = r0;
        t.r1 = r1;
        t.signal = ctr_index(l, C_XNEXT);
        c->tasks.push_back(t);
      }
    }
    int r0, r1;
    split_rows(f.vocab, ncu, q, &r0, &r1);
    if (r1 > r0) {
      Task t = make_task(OP_LMHEAD, L);
      t.wait[0] = ctr_index(L - 1, C_XNEXT);
      t.fanin[0] = n_out_tasks[L - 1];
      t.wait[1] = ctr_index(L - 1, C_WO);
      t.fanin[1] = n_wo_tasks[L - 1];
      t.r0 = r0;
      t.r1 = r1;
      t.idx = lm_i++;
      t.count = n_lm;
      t.signal = ctr_index(L, C_DONE);
      c->tasks.push_back(t);
    }
  }
  c->qoff[ncu] = (int)c->tasks.size();
  // each output task learns the PRE task that follows it on its queue (its weight tile is copied
  // into LDS while the output task waits for the Wo rows)
  for (int q = 0; q < ncu; ++q)
    for (int i = c->qoff[q]; i + 1 < c->qoff[q + 1]; ++i) {
      Task& t = c->tasks[i];
      const Task& nx = c->tasks[i + 1];
      if (t.op == OP_OUT && nx.op == OP_PRE) {
        t.next_layer = nx.layer;
        t.next_r0 = nx.r0;
        t.next_r1 = nx.r1;
      }
    }
  // signal slots: the k-th task (in table order) that signals a counter has slot k
  {
    std::vector<int> used(c->n_ctr, 0);
    for (Task& t : c->tasks)
      if (t.signal >= 0) t.slot = used[t.signal]++;
    c->n_slots = std::max(1, *std::max_element(used.begin(), used.end()));
  }

  // LDS: region A (input vectors), B (top-k state, reductions), C (per-op arrays)
  const int maxU = std::min(E, B * f.top_k);
  c->gu_rows_max = (int)(((int64_t)maxU * f.inter + n_gu - 1) / n_gu) + 1;
  // (the normalization stages its input rows and gain behind xs: fp32 [B][H], then [H] bf16)
  size_t a_bytes = std::max({align_up((size_t)B * H * 2, 256) + (size_t)B * H * 4 + (size_t)H * 2,
                             (size_t)B * f.n_q_heads * f.head_dim * 2, (size_t)B * f.top_k * f.inter * 2,
                             (size_t)(group + 1) * f.head_dim * 2});  // attention: rotated q heads + the new k
  a_bytes = align_up(a_bytes, 256);
  const size_t b_bytes = kLdsB;
  size_t c_gu = (size_t)std::max(std::min(c->gu_rows_max, kGuPass), c->gu_items > 0 ? kGuItem : 0) * B * 2 * 4;
  size_t c_out = (size_t)c->out_rows_max * B * f.top_k * 4;  // the experts' contributions to the task's rows
  size_t c_lm = (size_t)std::min(c->lm_rows_max, kLmPass) * B * 4;
  // attention: the waves' partial results, or (a segment's lead) the (max, sum) of all chunks plus one float4 per thread
  size_t c_attn = std::max((size_t)kWaves * (group * f.head_dim + 2 * kMaxGroup) * 4,
                           align_up((size_t)n_attn * kMaxGroup * 2 * 4, 16) + (size_t)kThreads * 16);
  const size_t c_mfma = B >= 2 ? (size_t)kMfmaRedBytes : 0;  // partial tiles of split dense rows
  // the top-p histogram and block sums of the last LM-head unit (whole KiB, so the region that
  // follows keeps the KiB alignment the prefetch region is cut in)
  const size_t c_topp = align_up((size_t)(kTopPBins + kWaves) * 8, 1024);
  size_t c_bytes = align_up(std::max({c_gu, c_out, c_lm, c_attn, c_mfma, c_topp, (size_t)kTopKScratch}), 256);
  c->lds_b = (int)a_bytes;
  c->lds_c = (int)(a_bytes + b_bytes);
  c->lds_p = (int)(a_bytes + b_bytes + c_bytes);
  if ((size_t)c->lds_p > lds_cap)
    return fail(MK_ERR_UNSUPPORTED, "LDS need " + std::to_string(c->lds_p) + " exceeds " + std::to_string(lds_cap));
  // region P: the rest of LDS, for the first weight tile of PRE and OUT tasks
  // (rows of Wqkv / router / Wo) and the first K/V pages of attention chunks
  size_t pf = lds_cap - (size_t)c->lds_p;
  if (p.prefetch_bytes > 0) pf = std::min(pf, (size_t)p.prefetch_bytes);
  if (p.prefetch_bytes < 0) pf = 0;
  c->pf_bytes = (int)(pf / 1024 * 1024);
  c->lds_bytes = (size_t)c->lds_p + c->pf_bytes;
  // PRE and WO weight tiles start in region C past the output task's expert contributions (at batch 1
  // nothing else in C is live across those tasks' start, or while an output task copies the tile)
  c->tile_off = (int)align_up(c_out, 256);
  size_t wide = c->lds_bytes - (size_t)c->lds_c - (size_t)c->tile_off;
  if (p.prefetch_bytes > 0) wide = std::min(wide, (size_t)p.prefetch_bytes);
  if (p.prefetch_bytes < 0) wide = 0;
  c->pf_wide = (int)(wide / 1024 * 1024);

  int r = simulate(c, nullptr);
  if (r) return r;
  c->ws = layout_workspace(c);
  c->inv_freq.resize(f.head_dim / 2);
  for (int i = 0; i < f.head_dim / 2; ++i) c->inv_freq[i] = std::pow(f.rope_theta, -(2.0 * i) / f.head_dim);
  release_scratch(c);
  c->built = true;
  c->bound = false;
  if (workspace_bytes) *workspace_bytes = c->ws.total;
  return MK_OK;
}

extern "C" int mk_validate_schedule(const mk_ctx* c, int32_t* completed) {
  if (!c || !c->built) return fail(MK_ERR_STATE, "no schedule built");
  return simulate(c, completed);
}

extern "C" int mk_get_schedule_info(const mk_ctx* c, mk_schedule_info* out) {
  if (!c || !out) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->built) return fail(MK_ERR_STATE, "no schedule built");
  out->num_cus = c->ncu;
  out->n_tasks = (int32_t)c->tasks.size();
  out->n_counters = c->n_ctr;
  out->n_attn = c->n_attn;
  out->n_gateup = c->n_gu;
  out->n_out = c->n_out;
  out->n_lmhead = c->n_lm;
  out->task_int32s = kTaskInts;
  out->lds_bytes = (int64_t)c->lds_bytes;
  out->workspace_bytes = (int64_t)c->ws.total;
  return MK_OK;
}

extern "C" int mk_copy_schedule(const mk_ctx* c, int32_t* tasks, int64_t tasks_cap, int32_t* queue_off, int64_t off_cap) {
  if (!c || !c->built) return fail(MK_ERR_STATE, "no schedule built");
  const int64_t need = (int64_t)c->tasks.size() * kTaskInts;
  if (tasks) {
    if (tasks_cap < need) return fail(MK_ERR_INVALID_ARG, "task buffer too small");
    std::memcpy(tasks, c->tasks.data(), need * 4);
  }
  if (queue_off) {
    if (off_cap < c->ncu + 1) return fail(MK_ERR_INVALID_ARG, "offset buffer too small");
    std::memcpy(queue_off, c->qoff.data(), (c->ncu + 1) * 4);
  }
  return MK_OK;
}

extern "C" int mk_attn_plan(const int32_t* seq_lens, int32_t n, int32_t n_kv, int32_t n_tasks, int32_t n_lead,
                            int32_t page_size, int32_t* chunk, int32_t* plan) {
  if (!seq_lens || !chunk || !plan || n < 1 || n > kMaxBatch || n_kv < 1 || page_size < 1 || n_lead < n * n_kv ||
      n_tasks < n_lead)
    return fail(MK_ERR_INVALID_ARG, "bad attention plan arguments");
  int32_t lens1[kMaxBatch];
  for (int b = 0; b < n; ++b) {
    if (seq_lens[b] < 0) return fail(MK_ERR_INVALID_ARG, "negative seq_len");
    lens1[b] = seq_lens[b] + 1;
  }
  const int64_t C = attn_chunk_len(lens1, n, n_kv, n_tasks - n_lead + n * n_kv, page_size);
  *chunk = (int32_t)C;
  for (int i = 0; i < n_tasks; ++i) {
    int b, g, t0, t1, first, nch, ch;
    if (attn_task_chunk(lens1, n, n_kv, C, i, n_lead, &b, &g, &t0, &t1, &first, &nch, &ch)) {
      plan[4 * i + 0] = b;
      plan[4 * i + 1] = g;
      plan[4 * i + 2] = t0;
      plan[4 * i + 3] = t1;
    } else {
      plan[4 * i + 0] = -1;
      plan[4 * i + 1] = plan[4 * i + 2] = plan[4 * i + 3] = 0;
    }
  }
  return MK_OK;
}

extern "C" int mk_get_ws_offsets(const mk_ctx* c, mk_ws_offsets* out) {
  if (!c || !out) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->built) return fail(MK_ERR_STATE, "no schedule built");
  out->x = (int64_t)c->ws.xr;
  out->qkv = (int64_t)c->ws.qkv;
  out->router = (int64_t)c->ws.rlog;
  out->attn_out = (int64_t)c->ws.attn_out;
  out->h = (int64_t)c->ws.h;
  out->sel = (int64_t)c->ws.sel;
  out->moe_half = (int64_t)c->ws.x;
  out->attn_half = (int64_t)c->ws.wo_out;
  return MK_OK;
}

extern "C" int mk_set_layer_inputs(mk_ctx* c, const float* d_x) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (d_x && ((uintptr_t)d_x) % 4) return fail(MK_ERR_INVALID_ARG, "layer inputs not 4-byte aligned");
  c->x_in = d_x;
  return MK_OK;
}

extern "C" int mk_set_sampling(mk_ctx* c, double temperature, uint64_t seed) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (!(temperature >= 0.0) || temperature == HUGE_VAL) return fail(MK_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  if (temperature > 0.0 && !(1.0 / temperature < HUGE_VAL)) return fail(MK_ERR_INVALID_ARG, "temperature too small");
  c->inv_temp = temperature > 0.0 ? 1.0 / temperature : 0.0;
  c->seed = seed;
  return MK_OK;
}

extern "C" int mk_set_top_p(mk_ctx* c, float top_p) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(MK_ERR_INVALID_ARG, "top_p must be in (0, 1]");
  c->top_p = top_p;
  return MK_OK;
}

extern "C" int mk_set_trace(mk_ctx* c, uint64_t* d_records, int64_t capacity) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (d_records && capacity < 1) return fail(MK_ERR_INVALID_ARG, "trace capacity must be positive");
  if (d_records && ((uintptr_t)d_records) % 8) return fail(MK_ERR_INVALID_ARG, "trace buffer not 8-byte aligned");
  c->trace = d_records;
  c->trace_cap = d_records ? capacity : 0;
  return MK_OK;
}

extern "C" int mk_set_spin_limit_us(mk_ctx* c, int64_t us) {
  if (!c || us < 1) return fail(MK_ERR_INVALID_ARG, "bad spin limit");
  c->spin_us = us;
  return MK_OK;
}

// ---------------------------------------------------------------------------
// device binding and launch

static int hip_fail(hipError_t e, const char* what) {
  return fail(MK_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

static int zero_state(mk_ctx* c, hipStream_t s) {
  int r = mkk_fill_u32((uint32_t*)(c->wsp + c->ws.state), 0u, c->ws.n_state_u32, s);
  if (r) return fail(MK_ERR_HIP, "state fill kernel launch failed");
  c->epoch = 0;
  c->need_reset = false;
  return MK_OK;
}

// Checks the bound buffers; the workspace is checked by the caller.
static int check_bind_args(const mk_ctx* c, const void* const* weights, int32_t n_weights, const void* k_pool,
                           const void* v_pool) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (!c->built) return fail(MK_ERR_STATE, "mk_build_schedule must run before binding");
  const mk_config& f = c->cfg;
  if (!weights || n_weights != n_weights_of(f))
    return fail(MK_ERR_INVALID_ARG, "weights must hold 3 + 7*n_layers pointers (3 + 8*n_layers for the sequential block)");
  for (int i = 0; i < n_weights; ++i)
    if (!weights[i]) return fail(MK_ERR_INVALID_ARG, "null weight pointer " + std::to_string(i));
  if (!k_pool || !v_pool) return fail(MK_ERR_INVALID_ARG, "null pool");
  for (int i = 0; i < n_weights; ++i)
    if (((uintptr_t)weights[i]) % 16) return fail(MK_ERR_INVALID_ARG, "weight pointer not 16-byte aligned");
  if (((uintptr_t)k_pool) % 16 || ((uintptr_t)v_pool) % 16) return fail(MK_ERR_INVALID_ARG, "pool not 16-byte aligned");
  return MK_OK;
}

// Uploads the task table, queue offsets, weight table and rotary frequencies into the
// workspace and clears its state region.  Makes no allocation: the uploads read the
// context's own tables and the caller's pointer array.
static int bind_workspace(mk_ctx* c, const void* const* weights, int32_t n_weights, void* k_pool, void* v_pool,
                          uint8_t* ws, hipStream_t s) {
  static_assert(sizeof(const void*) == sizeof(uint64_t), "the weight table holds 64-bit device addresses");
  c->bound = false;
  c->wsp = ws;
  c->kpool = (uint16_t*)k_pool;
  c->vpool = (uint16_t*)v_pool;
  hipError_t e;
  if ((e = hipMemcpyAsync(c->wsp + c->ws.tasks, c->tasks.data(), sizeof(Task) * c->tasks.size(), hipMemcpyHostToDevice, s)) ||
      (e = hipMemcpyAsync(c->wsp + c->ws.queue_off, c->qoff.data(), 4 * c->qoff.size(), hipMemcpyHostToDevice, s)) ||
      (e = hipMemcpyAsync(c->wsp + c->ws.wtab, weights, 8 * (size_t)n_weights, hipMemcpyHostToDevice, s)) ||
      (e = hipMemcpyAsync(c->wsp + c->ws.inv_freq, c->inv_freq.data(), 8 * c->inv_freq.size(), hipMemcpyHostToDevice, s)))
    return hip_fail(e, "hipMemcpyAsync (schedule upload)");
  int r = zero_state(c, s);
  if (r) return r;
  if ((e = hipStreamSynchronize(s))) return hip_fail(e, "hipStreamSynchronize (bind)");
  c->bound = true;
  return MK_OK;
}

extern "C" int mk_bind(mk_ctx* c, const void* const* weights, int32_t n_weights, void* k_pool, void* v_pool,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int r = check_bind_args(c, weights, n_weights, k_pool, v_pool);
  if (r) return r;
  if (!workspace) return fail(MK_ERR_INVALID_ARG, "null workspace");
  if (workspace_bytes < c->ws.total) return fail(MK_ERR_INVALID_ARG, "workspace smaller than reported");
  if (((uintptr_t)workspace) % 256) return fail(MK_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  release_scratch(c);
  return bind_workspace(c, weights, n_weights, k_pool, v_pool, (uint8_t*)workspace, (hipStream_t)stream);
}

extern "C" size_t mk_scratch_capacity(void) { return mkk_scratch_bytes(); }

extern "C" int mk_bind_scratch(mk_ctx* c, const void* const* weights, int32_t n_weights, void* k_pool, void* v_pool,
                               void* stream) {
  int r = check_bind_args(c, weights, n_weights, k_pool, v_pool);
  if (r) return r;
  const size_t cap = mkk_scratch_bytes();
  if (c->ws.total > cap)
    return fail(MK_ERR_INVALID_ARG, "workspace of " + std::to_string(c->ws.total) +
                                        " bytes exceeds the static workspace of " + std::to_string(cap) + " bytes");
  int dev = -1;
  void* p = nullptr;
  int e = mkk_scratch(&dev, &p);
  if (e) return hip_fail((hipError_t)e, "static workspace address");
  if (dev >= kMaxDevices) return fail(MK_ERR_HIP, "device index beyond the static workspace table");
  release_scratch(c);
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    g_scratch_owner[dev] = c;
  }
  c->scratch_dev = dev;
  return bind_workspace(c, weights, n_weights, k_pool, v_pool, (uint8_t*)p, (hipStream_t)stream);
}

static int launch_steps(mk_ctx* c, int32_t n, int32_t steps, const int32_t* d_tokens,
                        const int32_t* d_page_table, const int32_t* d_seq_lens, float* d_logits,
                        int32_t* d_next_tokens, void* stream, int32_t kv_sync) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (!c->bound) return fail(MK_ERR_STATE, "context not bound");
  if (scratch_lost(c)) return fail(MK_ERR_STATE, "the static workspace was bound to another context since");
  if (c->need_reset) return fail(MK_ERR_STATE, "a device error was reported; call mk_reset first");
  const mk_config& f = c->cfg;
  if (n < 1 || n > f.max_batch) return fail(MK_ERR_INVALID_ARG, "batch outside [1, max_batch]");
  if (!d_tokens || !d_page_table || !d_seq_lens || !d_logits) return fail(MK_ERR_INVALID_ARG, "null step buffer");
  if (steps < 1 || steps > (1 << 20)) return fail(MK_ERR_INVALID_ARG, "steps outside [1, 2^20]");
  if (steps > 1 && !d_next_tokens) return fail(MK_ERR_INVALID_ARG, "several steps need the token buffer");
  if (steps > 1 && c->x_in) return fail(MK_ERR_STATE, "the layer-input hook applies to single steps only");

  KArgs a;
  std::memset(&a, 0, sizeof a);
  a.L = f.n_layers;
  a.H = f.hidden;
  a.nq = f.n_q_heads;
  a.nkv = f.n_kv_heads;
  a.d = f.head_dim;
  a.E = f.n_experts;
  a.topk = f.top_k;
  a.I = f.inter;
  a.V = f.vocab;
  a.ps = f.page_size;
  a.max_batch = f.max_batch;
  a.max_pages = f.max_pages_per_seq;
  a.num_pages = f.num_pages;
  a.qkv_rows = (f.n_q_heads + 2 * f.n_kv_heads) * f.head_dim;
  a.group = f.n_q_heads / f.n_kv_heads;
  a.eps = f.rms_eps;
  a.n_attn = c->n_attn;
  a.n_gu = c->n_gu;
  a.n_lm = c->n_lm;
  a.gu_rows_max = c->gu_rows_max;
  a.out_rows_max = c->out_rows_max;
  a.lm_rows_max = c->lm_rows_max;
  a.lds_b = c->lds_b;
  a.lds_c = c->lds_c;
  a.lds_p = c->lds_p;
  a.pf_bytes = c->pf_bytes;
  a.pf_wide = c->pf_wide;
  a.tile_off = c->tile_off;
  a.gu_pool = c->gu_pool;
  a.seq_block = c->cfg.block_style == MK_BLOCK_SEQUENTIAL ? 1 : 0;
  a.gu_items = c->gu_items;
  a.gu_parts = c->gu_parts;
  uint8_t* w = c->wsp;
  a.tasks = (const Task*)(w + c->ws.tasks);
  a.queue_off = (const int32_t*)(w + c->ws.queue_off);
  uint32_t* st = (uint32_t*)(w + c->ws.state);
  a.flags = st + c->ws.ctr;
  a.tickets = st + c->ws.tickets;
  a.err = (int32_t*)(st + c->ws.err);
  a.rll = (uint64_t*)(st + c->ws.rll);
  a.claims = st + c->ws.claims;
  a.wtab = (const uint64_t*)(w + c->ws.wtab);
  a.inv_freq = (const double*)(w + c->ws.inv_freq);
  a.x = (float*)(w + c->ws.x);
  a.xr = (float*)(w + c->ws.xr);
  a.qkv = (float*)(w + c->ws.qkv);
  a.rlog = (float*)(w + c->ws.rlog);
  a.attn_part = (float*)(w + c->ws.attn_part);
  a.attn_out = (uint16_t*)(w + c->ws.attn_out);
  a.wo_out = (float*)(w + c->ws.wo_out);
  a.h = (uint16_t*)(w + c->ws.h);
  a.lm_part = (float*)(w + c->ws.lm_part);
  a.sel_out = (int32_t*)(w + c->ws.sel);
  a.x_in = c->x_in;
  a.trace = c->trace;
  a.trace_cap = c->trace_cap;
  a.k_pool = c->kpool;
  a.v_pool = c->vpool;
  a.n = n;
  a.nsteps = steps;
  a.kv_sync = kv_sync;
  a.step = 0;
  a.epoch = c->epoch + 1;
  a.tokens = d_tokens;
  a.page_table = d_page_table;
  a.seq_lens = d_seq_lens;
  a.logits = d_logits;
  a.next_tok = d_next_tokens;
  a.spin_limit_ticks = (uint64_t)c->spin_us * 100;  // s_memrealtime runs at 100 MHz
  a.inv_temp = c->inv_temp;
  a.seed = c->seed;
  a.top_p = c->top_p;
  const hipStream_t hs = (hipStream_t)stream;
  int r = c->cfg.weight_format == MK_WEIGHTS_FP8_E4M3   ? mkk_launch_step_fp8(&a, c->ncu, c->lds_bytes, hs)
          : c->cfg.weight_format == MK_WEIGHTS_FP4_E2M1 ? mkk_launch_step_fp4(&a, c->ncu, c->lds_bytes, hs)
          : c->cfg.block_style == MK_BLOCK_SEQUENTIAL   ? mkk_launch_step_seq(&a, c->ncu, c->lds_bytes, hs)
                                                        : mkk_launch_step(&a, c->ncu, c->lds_bytes, hs);
  if (r) return fail(MK_ERR_HIP, std::string("cooperative launch failed: ") + hipGetErrorString((hipError_t)r));
  c->epoch += (uint32_t)steps;
  return MK_OK;
}

extern "C" int mk_decode_steps(mk_ctx* c, int32_t n, int32_t steps, const int32_t* d_tokens,
                               const int32_t* d_page_table, const int32_t* d_seq_lens, float* d_logits,
                               int32_t* d_next_tokens, void* stream) {
  return launch_steps(c, n, steps, d_tokens, d_page_table, d_seq_lens, d_logits, d_next_tokens, stream, 0);
}

extern "C" int mk_decode_step(mk_ctx* c, int32_t n, const int32_t* d_tokens, const int32_t* d_page_table,
                              const int32_t* d_seq_lens, float* d_logits, int32_t* d_next_tokens, void* stream) {
  return launch_steps(c, n, 1, d_tokens, d_page_table, d_seq_lens, d_logits, d_next_tokens, stream, 0);
}

extern "C" int mk_mixed_step(mk_ctx* c, int32_t n, const int32_t* d_tokens, const int32_t* d_page_table,
                             const int32_t* d_seq_lens, float* d_logits, int32_t* d_next_tokens, void* stream) {
  return launch_steps(c, n, 1, d_tokens, d_page_table, d_seq_lens, d_logits, d_next_tokens, stream, 1);
}

extern "C" int mk_get_error(mk_ctx* c, int32_t* code, int32_t* cu, int32_t* task, void* stream) {
  if (!c || !code) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!c->bound) return fail(MK_ERR_STATE, "context not bound");
  if (scratch_lost(c)) return fail(MK_ERR_STATE, "the static workspace was bound to another context since");
  hipStream_t s = (hipStream_t)stream;
  int32_t ew[E_WORDS];
  hipError_t e;
  uint32_t* st = (uint32_t*)(c->wsp + c->ws.state);
  if ((e = hipMemcpyAsync(ew, st + c->ws.err, sizeof ew, hipMemcpyDeviceToHost, s))) return hip_fail(e, "hipMemcpyAsync (error word)");
  if ((e = hipStreamSynchronize(s))) return hip_fail(e, "hipStreamSynchronize (error word)");
  *code = ew[E_CODE];
  if (cu) *cu = ew[E_CU];
  if (task) *task = ew[E_TASK];
  if (ew[E_CODE] != 0 || ew[E_ABORT] != 0) {
    c->need_reset = true;
    int r = mkk_fill_u32(st + c->ws.err, 0u, E_WORDS, s);
    if (r) return fail(MK_ERR_HIP, "error-word fill kernel launch failed");
  }
  return MK_OK;
}

extern "C" int mk_reset(mk_ctx* c, void* stream) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null context");
  if (!c->bound) return fail(MK_ERR_STATE, "context not bound");
  if (scratch_lost(c)) return fail(MK_ERR_STATE, "the static workspace was bound to another context since");
  return zero_state(c, (hipStream_t)stream);
}
