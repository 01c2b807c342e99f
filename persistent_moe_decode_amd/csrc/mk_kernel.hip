// The persistent decode megakernel for MI355X (gfx950, wave64).
//
// One workgroup of 512 threads (8 wave64) runs on each compute unit and walks
// the queue the host built for it (the pages' host-built static task table:
// latestnews.news paragraph 3, ainews.surl.tw paragraph 2).  Before a task it
// waits until one counter in global memory reaches epoch * fan-in, and after
// the task it adds one to one counter (aiweekly.co paragraph 3: a consumer
// waits on a single count, signalling and waiting are O(1) whatever the
// fan-in).  Task bodies:
//   PRE     RMSNorm of the residual, then rows of [Wq; Wk; Wv] or of the router;
//   ATTN    one chunk of paged split-KV attention for a (sequence, kv head);
//           the last chunk to finish merges all chunks (log-sum-exp combine);
//   GATEUP  top-k of the router logits, then rows of the selected experts'
//           gate and up projections and SwiGLU;
//   OUT     rows of Wo and of the selected experts' down projections, weighted
//           expert sum and residual add (parallel block: x += attn + moe);
//   LMHEAD  final RMSNorm, rows of the LM head, greedy argmax (last arriver).
// Weight rows stream from HBM with 128-bit loads, lanes accumulate in fp32
// with v_dot2_f32_bf16, and groups of lanes reduce through DPP.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"
#include "mk_types.h"

using namespace mk;

#define DEV __device__ __forceinline__

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

static constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// scalar helpers

DEV float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bfloat16 bits, round to nearest even (NaN kept quiet).
DEV uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

DEV float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w), __builtin_bit_cast(bf16x2_v, x), acc, false);
}

DEV float dot8(const uint4& w, const uint4& x, float acc) {
  acc = dot2(w.x, x.x, acc);
  acc = dot2(w.y, x.y, acc);
  acc = dot2(w.z, x.z, acc);
  acc = dot2(w.w, x.w, acc);
  return acc;
}

template <int CTRL>
DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes; every lane of a group gets the sum.
// quad_perm [1,0,3,2] and [2,3,0,1] pair lanes within a quad, row_half_mirror
// pairs the two quads of 8 lanes, row_mirror the two halves of a 16-lane row.
template <int N>
DEV float group_sum(float v) {
  v += dpp<0xB1>(v);
  if (N >= 4) v += dpp<0x4E>(v);
  if (N >= 8) v += dpp<0x141>(v);
  if (N >= 16) v += dpp<0x140>(v);
  if (N >= 32) v += __shfl_xor(v, 16);
  if (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

// ---------------------------------------------------------------------------
// LDS carve-up.  Region A: input vectors.  Region B: top-k state, flags and
// reduction scratch.  Region C: per-op arrays.

struct TopK {
  int32_t sel[kMaxBatch][kMaxTopK];
  float w[kMaxBatch][kMaxTopK];
  int32_t nU, maxtok;
  int32_t U[kMaxBatch * kMaxTopK];                // distinct experts, ascending
  int32_t ntok[kMaxBatch * kMaxTopK];             // tokens routed to U[u]
  int32_t pair[kMaxBatch * kMaxTopK][kMaxBatch];  // b*topk+j of each of them, ascending b
};
static_assert(sizeof(TopK) <= 3584, "top-k state fits region B");

struct Lds {
  uint8_t* base;
  uint8_t* A;
  TopK* tk;
  int32_t* flags;  // [16]
  float* red;      // [16]
  uint8_t* C;
};

DEV Lds carve(uint8_t* lds, const KArgs& a) {
  Lds s;
  s.base = lds;
  s.A = lds;
  s.tk = (TopK*)(lds + a.lds_b);
  s.flags = (int32_t*)(lds + a.lds_b + 3584);
  s.red = (float*)(lds + a.lds_b + 3584 + 64);
  s.C = lds + a.lds_c;
  return s;
}

// All threads get the block-wide sum; the order of the partial sums is fixed.
DEV float block_sum(float v, float* red) {
  v = group_sum<64>(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += red[w];
  return t;
}

// ---------------------------------------------------------------------------
// errors, waits and signals

DEV void raise_error(const KArgs& a, int code, int task, int aux) {
  if (atomicCAS(&a.err[E_CODE], 0, code) == 0) {
    __hip_atomic_store(&a.err[E_CU], (int)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.err[E_TASK], task, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.err[E_AUX], aux, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __hip_atomic_store(&a.err[E_ABORT], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

DEV bool aborting(const KArgs& a) {
  return __hip_atomic_load(&a.err[E_ABORT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Thread 0 spins (relaxed agent-scope loads, s_sleep between polls) until
// counter idx reaches epoch * fanin, then takes one agent-scope acquire fence;
// the barrier hands the result to the other waves.  The wait is bounded: past
// the spin limit the task raises MK_ERR_DEVICE_TIMEOUT and the grid drains.
// Returns false when the grid is aborting.
DEV bool wait_counter(const KArgs& a, int idx, int fanin, int task, int32_t* slot) {
  if (threadIdx.x == 0) {
    int ok = aborting(a) ? 0 : 1;
    if (ok && idx >= 0) {
      const uint32_t want = a.epoch * (uint32_t)fanin;
      uint32_t* c = a.ctr + idx;
      const uint64_t t0 = wall_clock64();
      uint32_t it = 0;
      while ((int32_t)(__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - want) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if ((++it & 31) == 0) {
          if (aborting(a)) {
            ok = 0;
            break;
          }
          if (wall_clock64() - t0 > a.spin_limit_ticks) {
            raise_error(a, MK_ERR_DEVICE_TIMEOUT, task, idx);
            ok = 0;
            break;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    *slot = ok;
  }
  __syncthreads();
  return *slot != 0;
}

// Every wave waits for its own stores, the barrier orders them before thread
// 0's agent-scope release, and the add publishes the task.
DEV void signal_counter(const KArgs& a, int idx) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0 && idx >= 0) __hip_atomic_fetch_add(a.ctr + idx, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Ticket for "last of count arrivals does the merge": returns true in every
// thread of the last arriving workgroup, which also resets the ticket.
DEV bool arrive_last(uint32_t* ticket, uint32_t count, int32_t* slot) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == count - 1;
    if (last) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *slot = last;
  }
  __syncthreads();
  return *slot != 0;
}

// ---------------------------------------------------------------------------
// inputs

DEV const uint16_t* wptr(const KArgs& a, int i) { return (const uint16_t*)(uintptr_t)a.wtab[i]; }

DEV const uint16_t* token_row(const KArgs& a, int b, int task) {
  int tok = a.tokens[b];
  if (tok < 0 || tok >= a.V) {
    raise_error(a, MK_ERR_DEVICE_TOKEN, task, b);
    tok = 0;
  }
  return wptr(a, W_EMBED) + (size_t)tok * a.H;
}

// Residual entering `layer` (layer 0: the embedding row).
// With the layer-input hook set, layers >= 1 (and the final norm) read the
// residual the caller supplied instead of the one the previous layer wrote.
DEV float load_x(const KArgs& a, int layer, int b, int i, const uint16_t* emb) {
  if (layer == 0) return bf2f(emb[i]);
  const float* src = a.x_in ? a.x_in : a.x;
  return src[((size_t)layer * a.max_batch + b) * a.H + i];
}

// xs[b][H] = bf16(x_b / sqrt(mean(x_b^2) + eps) * g) for b < n.
DEV void norm_inputs(const KArgs& a, int layer, const uint16_t* gain, uint16_t* xs, float* red, int task) {
  const int H = a.H;
  for (int b = 0; b < a.n; ++b) {
    const uint16_t* emb = layer == 0 ? token_row(a, b, task) : nullptr;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += kThreads) {
      const float v = load_x(a, layer, b, i, emb);
      ss += v * v;
    }
    const float tot = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(tot / (float)H + a.eps);
    for (int i = threadIdx.x; i < H; i += kThreads)
      xs[(size_t)b * H + i] = f2bf(load_x(a, layer, b, i, emb) * inv * bf2f(gain[i]));
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Row dot products: each job is one weight row of K bf16 dotted with up to
// maxnx input vectors held in LDS.  LPR lanes share a row; each lane loads
// CPL 16-byte chunks (strided by LPR chunks, so a row's loads coalesce) before
// any arithmetic, so a whole pass of rows is in flight at once.

template <int LPR, int CPL, class Job>
DEV void rowdots(int njobs, int maxnx, const Job& job) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int RPW = 64 / LPR;
  const int sub = lane / LPR, li = lane % LPR;
  for (int base = 0; base < njobs; base += kWaves * RPW) {
    const int i = base + wave * RPW + sub;
    const bool act = i < njobs;
    const int ic = act ? i : 0;
    const uint4* wr = job.row(ic) + li;
    uint4 wv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) wv[c] = act ? wr[LPR * c] : make_uint4(0, 0, 0, 0);
    const int nx = act ? job.nx(ic) : 0;
    for (int t = 0; t < maxnx; ++t) {
      const bool on = t < nx;
      const uint4* xr = job.x(ic, on ? t : 0) + li;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc = dot8(wv[c], xr[LPR * c], acc);
      acc = group_sum<LPR>(acc);
      if (on && li == 0) job.emit(i, t, acc);
    }
  }
}

// Any K that is a multiple of 128: 16 lanes per row, runtime chunk count.
template <class Job>
DEV void rowdots_generic(int K, int njobs, int maxnx, const Job& job) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / 16, li = lane % 16;
  const int cpl = K / 128;
  for (int base = 0; base < njobs; base += kWaves * 4) {
    const int i = base + wave * 4 + sub;
    const bool act = i < njobs;
    const int ic = act ? i : 0;
    const int nx = act ? job.nx(ic) : 0;
    const uint4* wr = job.row(ic) + li;
    for (int t = 0; t < maxnx; ++t) {
      const bool on = t < nx;
      const uint4* xr = job.x(ic, on ? t : 0) + li;
      float acc = 0.f;
      for (int c = 0; c < cpl; ++c) acc = dot8(act ? wr[16 * c] : make_uint4(0, 0, 0, 0), xr[16 * c], acc);
      acc = group_sum<16>(acc);
      if (on && li == 0) job.emit(i, t, acc);
    }
  }
}

template <class Job>
DEV void run_rowdots(int K, int njobs, int maxnx, const Job& job) {
  if (njobs <= 0 || maxnx <= 0) return;
  const int ch = K / 8;  // 16-byte chunks per row
  if (njobs <= 8 && ch == 512) return rowdots<64, 8>(njobs, maxnx, job);
  if (njobs <= 8 && ch == 256) return rowdots<64, 4>(njobs, maxnx, job);
  if (njobs <= 16 || ch > 256) {
    switch (ch) {
      case 64: return rowdots<32, 2>(njobs, maxnx, job);
      case 96: return rowdots<32, 3>(njobs, maxnx, job);
      case 128: return rowdots<32, 4>(njobs, maxnx, job);
      case 256: return rowdots<32, 8>(njobs, maxnx, job);
      case 512: return rowdots<32, 16>(njobs, maxnx, job);
      default: break;
    }
  }
  switch (ch) {
    case 16: return rowdots<16, 1>(njobs, maxnx, job);
    case 32: return rowdots<16, 2>(njobs, maxnx, job);
    case 64: return rowdots<16, 4>(njobs, maxnx, job);
    case 96: return rowdots<16, 6>(njobs, maxnx, job);
    case 128: return rowdots<16, 8>(njobs, maxnx, job);
    case 256: return rowdots<16, 16>(njobs, maxnx, job);
    default: return rowdots_generic(K, njobs, maxnx, job);
  }
}

// ---------------------------------------------------------------------------
// Router top-k: per token, the top_k logits ordered by (value desc, index
// asc), their softmax, the distinct experts in ascending order and, for each
// of them, the (token, slot) pairs routed to it.  Wave 0 computes, all read.

DEV bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

DEV void compute_topk(const KArgs& a, int layer, TopK* tk) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == 0) {
    const int E = a.E, K = a.topk;
    for (int b = 0; b < a.n; ++b) {
      const float* r = a.rlog + ((size_t)layer * a.max_batch + b) * E;
      float v0 = lane < E ? r[lane] : kNegInf;
      float v1 = lane + 64 < E ? r[lane + 64] : kNegInf;
      if (v0 != v0) v0 = kNegInf;  // NaN never outranks a number
      if (v1 != v1) v1 = kNegInf;
      bool t0 = lane >= E, t1 = lane + 64 >= E;
      float selv0 = 0.f;
      float wsum = 0.f;
      for (int j = 0; j < K; ++j) {
        float bv = kNegInf;
        int bi = 0x7fffffff;
        if (!t0 && better(v0, lane, bv, bi)) { bv = v0; bi = lane; }
        if (!t1 && better(v1, lane + 64, bv, bi)) { bv = v1; bi = lane + 64; }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
          const float ov = __shfl_xor(bv, m);
          const int oi = __shfl_xor(bi, m);
          if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        if (bi == lane) t0 = true;
        if (bi == lane + 64) t1 = true;
        if (j == 0) selv0 = bv;
        const float e = __expf(bv - selv0);
        wsum += e;
        if (lane == 0) {
          tk->sel[b][j] = bi;
          tk->w[b][j] = e;
        }
      }
      if (lane == 0)
        for (int j = 0; j < K; ++j) tk->w[b][j] = tk->w[b][j] / wsum;
    }
    // distinct experts, ascending
    const int np = a.n * K;
    bool in0 = false, in1 = false;
    for (int p = 0; p < np; ++p) {
      const int e = tk->sel[p / K][p % K];
      in0 |= e == lane;
      in1 |= e == lane + 64;
    }
    const uint64_t m0 = __ballot(in0), m1 = __ballot(in1);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int c0 = __popcll(m0);
    if (in0) tk->U[__popcll(m0 & below)] = lane;
    if (in1) tk->U[c0 + __popcll(m1 & below)] = lane + 64;
    // pairs of each expert, in ascending pair order
    int mytok = 0;
    if (lane < np) {
      const int e = tk->sel[lane / K][lane % K];
      const uint64_t bm = e < 64 ? m0 : m1;
      const int eb = e & 63;
      const uint64_t lower = eb == 0 ? 0ull : (~0ull >> (64 - eb));
      const int u = (e < 64 ? 0 : c0) + __popcll(bm & lower);
      int t = 0, tot = 0;
      for (int p = 0; p < np; ++p) {
        const int ep = tk->sel[p / K][p % K];
        if (ep == e) {
          t += p < lane;
          tot++;
        }
      }
      tk->pair[u][t] = lane;
      if (t == 0) tk->ntok[u] = tot;
      mytok = tot;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mytok = max(mytok, __shfl_xor(mytok, m));
    if (lane == 0) {
      tk->nU = c0 + __popcll(m1);
      tk->maxtok = mytok;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// PRE: RMSNorm + rows [r0, r1) of the stacked [Wq; Wk; Wv; Wr] matrix.

struct JobPre {
  const uint16_t* W;
  int r0, K;
  const uint16_t* xs;
  float* out;  // [b][ld] + r0 already applied
  int ld;
  DEV const uint4* row(int i) const { return (const uint4*)(W + (size_t)(r0 + i) * K); }
  DEV int nx(int) const { return 1 << 30; }
  DEV const uint4* x(int, int t) const { return (const uint4*)(xs + (size_t)t * K); }
  DEV void emit(int i, int t, float v) const { out[(size_t)t * ld + i] = v; }
};

DEV void task_pre(const KArgs& a, const Task& t, const Lds& s, int qi) {
  const int l = t.layer;
  uint16_t* xs = (uint16_t*)s.A;
  norm_inputs(a, l, wptr(a, widx(l, WL_NORM)), xs, s.red, qi);
  JobPre j;
  j.K = a.H;
  j.xs = xs;
  if (t.r0 < a.qkv_rows) {
    j.W = wptr(a, widx(l, WL_QKV));
    j.r0 = t.r0;
    j.out = a.qkv + (size_t)l * a.max_batch * a.qkv_rows + t.r0;
    j.ld = a.qkv_rows;
  } else {
    j.W = wptr(a, widx(l, WL_ROUTER));
    j.r0 = t.r0 - a.qkv_rows;
    j.out = a.rlog + (size_t)l * a.max_batch * a.E + j.r0;
    j.ld = a.E;
  }
  run_rowdots(a.H, t.r1 - t.r0, a.n, j);
}

// ---------------------------------------------------------------------------
// ATTN: one chunk [t0, t1) of the positions of (sequence b, kv head g).

DEV void task_attn(const KArgs& a, const Task& t, const Lds& s, int qi) {
  const int l = t.layer, G = a.group, d = a.d, ps = a.ps;
  int32_t* plan = s.flags + 2;  // b, g, t0, t1, first, nch, ok
  int32_t* lens1 = (int32_t*)s.C;
  if (threadIdx.x == 0) {
    const int cap = a.max_pages * ps;
    for (int b = 0; b < a.n; ++b) {
      int p = a.seq_lens[b];
      if (p < 0 || p + 1 > cap) {
        raise_error(a, MK_ERR_DEVICE_SEQ, qi, b);
        p = p < 0 ? 0 : cap - 1;
      }
      lens1[b] = p + 1;
    }
    const int64_t C = attn_chunk_len(lens1, a.n, a.nkv, a.n_attn, ps);
    int b, g, t0, t1, first, nch;
    const bool ok = attn_chunk_of(lens1, a.n, a.nkv, C, t.idx, &b, &g, &t0, &t1, &first, &nch);
    plan[0] = b; plan[1] = g; plan[2] = t0; plan[3] = t1; plan[4] = first; plan[5] = nch; plan[6] = ok;
    plan[7] = lens1[ok ? b : 0] - 1;
  }
  __syncthreads();
  if (!plan[6]) return;
  const int b = plan[0], g = plan[1], t0 = plan[2], t1 = plan[3], first = plan[4], nch = plan[5], p = plan[7];
  __syncthreads();  // plan and lens1 read before region C is reused below

  const int half = d / 2;
  uint16_t* q_s = (uint16_t*)s.A;  // [G][d] rotated q, bf16
  const float* qkv = a.qkv + ((size_t)l * a.max_batch + b) * a.qkv_rows;
  for (int e = threadIdx.x; e < G * half; e += kThreads) {
    const int hh = e / half, i = e % half;
    double sd, cd;
    sincos((double)p * a.inv_freq[i], &sd, &cd);
    const float cf = (float)cd, sf = (float)sd;
    const float* q = qkv + (size_t)(g * G + hh) * d;
    const float x0 = q[i], x1 = q[i + half];
    q_s[hh * d + i] = f2bf(x0 * cf - x1 * sf);
    q_s[hh * d + i + half] = f2bf(x0 * sf + x1 * cf);
  }
  // the chunk holding position p writes the new token's K (rotated) and V
  if (t1 == p + 1) {
    const int page = a.page_table[(size_t)b * a.max_pages + p / ps];
    if (page < 0 || page >= a.num_pages) {
      if (threadIdx.x == 0) raise_error(a, MK_ERR_DEVICE_PAGE, qi, page);
    } else {
      const size_t off = ((((size_t)l * a.num_pages + page) * a.nkv + g) * ps + p % ps) * d;
      const float* kk = qkv + (size_t)a.nq * d + (size_t)g * d;
      const float* vv = qkv + (size_t)(a.nq + a.nkv) * d + (size_t)g * d;
      for (int i = threadIdx.x; i < half; i += kThreads) {
        double sd, cd;
        sincos((double)p * a.inv_freq[i], &sd, &cd);
        const float cf = (float)cd, sf = (float)sd;
        const float x0 = kk[i], x1 = kk[i + half];
        a.k_pool[off + i] = f2bf(x0 * cf - x1 * sf);
        a.k_pool[off + i + half] = f2bf(x0 * sf + x1 * cf);
      }
      for (int i = threadIdx.x; i < d; i += kThreads) a.v_pool[off + i] = f2bf(vv[i]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __threadfence_block();
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float scale = 1.0f / sqrtf((float)d);
  float m[kMaxGroup], ls[kMaxGroup], o0[kMaxGroup], o1[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m[h] = kNegInf;
    ls[h] = 0.f;
    o0[h] = 0.f;
    o1[h] = 0.f;
  }
  float* pbuf = (float*)s.C + wave * 16 * kMaxGroup;  // [h][16] probabilities of this wave's block
  const int tl = lane >> 2, qd = lane & 3;
  const int nblk = (t1 - t0 + 15) / 16;
  for (int blk = wave; blk < nblk; blk += kWaves) {
    const int tb = t0 + blk * 16;
    const int page = a.page_table[(size_t)b * a.max_pages + tb / ps];
    if (page < 0 || page >= a.num_pages) {
      if (lane == 0) raise_error(a, MK_ERR_DEVICE_PAGE, qi, page);
      continue;
    }
    const size_t boff = (((size_t)l * a.num_pages + page) * a.nkv + g) * (size_t)ps * d;
    const uint16_t* kb = a.k_pool + boff;
    const uint16_t* vb = a.v_pool + boff;
    const bool valid = tb + tl < t1;
    // scores: 4 lanes per position, d/4 dims each
    const uint4* kr = (const uint4*)(kb + tl * d + qd * (d / 4));
    uint4 kv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) kv[c] = (valid && c < d / 32) ? kr[c] : make_uint4(0, 0, 0, 0);
    float sc[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      float acc = 0.f;
      if (h < G) {
        const uint4* qr = (const uint4*)(q_s + h * d + qd * (d / 4));
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (c < d / 32) acc = dot8(kv[c], qr[c], acc);
      }
      acc += dpp<0xB1>(acc);
      acc += dpp<0x4E>(acc);
      sc[h] = valid ? acc * scale : kNegInf;
    }
    // V rows of the block (lane owns d/64 consecutive dims)
    uint32_t vr[16];
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const bool ok = tb + tt < t1;
      if (d == 128)
        vr[tt] = ok ? *(const uint32_t*)(vb + tt * d + 2 * lane) : 0u;
      else
        vr[tt] = ok ? (uint32_t)vb[tt * d + lane] : 0u;
    }
    // online softmax over the block's 16 positions
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h >= G) break;
      float bm = sc[h];
      bm = fmaxf(bm, __shfl_xor(bm, 4));
      bm = fmaxf(bm, __shfl_xor(bm, 8));
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mn = fmaxf(m[h], bm);
      const float alpha = __expf(m[h] - mn);
      const float pr = valid ? __expf(sc[h] - mn) : 0.f;
      float bs = pr;
      bs += __shfl_xor(bs, 4);
      bs += __shfl_xor(bs, 8);
      bs += __shfl_xor(bs, 16);
      bs += __shfl_xor(bs, 32);
      ls[h] = ls[h] * alpha + bs;
      m[h] = mn;
      o0[h] *= alpha;
      o1[h] *= alpha;
      if (qd == 0) pbuf[h * 16 + tl] = pr;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const float v0 = d == 128 ? bf2f(vr[tt] & 0xffffu) : bf2f(vr[tt]);
      const float v1 = d == 128 ? bf2f(vr[tt] >> 16) : 0.f;
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < G) {
          const float pp = pbuf[h * 16 + tt];
          o0[h] += pp * v0;
          o1[h] += pp * v1;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // merge the 8 waves' running states into this chunk's partial
  float* mrg = (float*)s.C + kWaves * 16 * kMaxGroup;  // [wave][G][d+2]
  const int DPV = d / 64;
  for (int h = 0; h < G; ++h) {
    float* row = mrg + ((size_t)wave * G + h) * (d + 2);
    row[lane * DPV] = o0[h];
    if (DPV == 2) row[lane * DPV + 1] = o1[h];
    if (lane == 0) {
      row[d] = m[h];
      row[d + 1] = ls[h];
    }
  }
  __syncthreads();
  float* part = a.attn_part + ((size_t)l * a.n_attn + t.idx) * G * (d + 2);
  for (int e = threadIdx.x; e < G * d; e += kThreads) {
    const int hh = e / d, dim = e % d;
    float M = kNegInf;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrg[((size_t)w * G + hh) * (d + 2) + d]);
    float O = 0.f, Ls = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float* row = mrg + ((size_t)w * G + hh) * (d + 2);
      const float sc = row[d] == kNegInf ? 0.f : __expf(row[d] - M);
      O += row[dim] * sc;
      Ls += row[d + 1] * sc;
    }
    part[hh * (d + 2) + dim] = O;
    if (dim == 0) {
      part[hh * (d + 2) + d] = M;
      part[hh * (d + 2) + d + 1] = Ls;
    }
  }
  // last chunk of (b, g) merges all chunks: o = sum_j e^(m_j - M) o_j / sum_j e^(m_j - M) l_j
  uint32_t* ticket = a.tickets + ((size_t)l * a.max_batch + b) * a.nkv + g;
  if (arrive_last(ticket, (uint32_t)nch, s.flags + 10)) {
    const float* parts = a.attn_part + ((size_t)l * a.n_attn + first) * G * (d + 2);
    uint16_t* out = a.attn_out + ((size_t)l * a.max_batch + b) * a.nq * d + (size_t)g * G * d;
    for (int e = threadIdx.x; e < G * d; e += kThreads) {
      const int hh = e / d, dim = e % d;
      float M = kNegInf;
      for (int j = 0; j < nch; ++j) M = fmaxf(M, parts[((size_t)j * G + hh) * (d + 2) + d]);
      float O = 0.f, Ls = 0.f;
      for (int j = 0; j < nch; ++j) {
        const float* row = parts + ((size_t)j * G + hh) * (d + 2);
        const float sc = __expf(row[d] - M);
        O += row[dim] * sc;
        Ls += row[d + 1] * sc;
      }
      out[hh * d + dim] = f2bf(O / Ls);
    }
  }
}

// ---------------------------------------------------------------------------
// GATEUP: the distinct selected experts' rows, flattened expert-major into
// nU * I virtual rows, are cut evenly over the gate/up tasks.

struct JobGateUp {
  const TopK* tk;
  const uint16_t *wg, *wu, *xs;
  float* gs;
  int64_t v0;
  int H, I, maxB, topk;
  DEV int urow(int i, int* r) const {
    const int64_t vr = v0 + (i >> 1);
    *r = (int)(vr % I);
    return (int)(vr / I);
  }
  DEV const uint4* row(int i) const {
    int r;
    const int u = urow(i, &r);
    return (const uint4*)(((i & 1) ? wu : wg) + ((size_t)tk->U[u] * I + r) * H);
  }
  DEV int nx(int i) const {
    int r;
    return tk->ntok[urow(i, &r)];
  }
  DEV const uint4* x(int i, int t) const {
    int r;
    const int u = urow(i, &r);
    return (const uint4*)(xs + (size_t)(tk->pair[u][t] / topk) * H);
  }
  DEV void emit(int i, int t, float v) const { gs[((size_t)(i >> 1) * maxB + t) * 2 + (i & 1)] = v; }
};

DEV void task_gateup(const KArgs& a, const Task& t, const Lds& s, int qi) {
  const int l = t.layer;
  compute_topk(a, l, s.tk);
  uint16_t* xs = (uint16_t*)s.A;
  norm_inputs(a, l, wptr(a, widx(l, WL_NORM)), xs, s.red, qi);
  const TopK* tk = s.tk;
  if (t.idx == 0 && threadIdx.x < a.n * a.topk)
    a.sel_out[(size_t)l * a.max_batch * a.topk + threadIdx.x] = tk->sel[threadIdx.x / a.topk][threadIdx.x % a.topk];
  const int64_t R = (int64_t)tk->nU * a.I;
  const int64_t va = R * t.idx / a.n_gu, vb = R * (t.idx + 1) / a.n_gu;
  JobGateUp j;
  j.tk = tk;
  j.wg = wptr(a, widx(l, WL_GATE));
  j.wu = wptr(a, widx(l, WL_UP));
  j.xs = xs;
  j.gs = (float*)s.C;
  j.H = a.H;
  j.I = a.I;
  j.maxB = a.max_batch;
  j.topk = a.topk;
  const int mt = tk->maxtok;
  uint16_t* hl = a.h + (size_t)l * a.max_batch * a.topk * a.I;
  // virtual rows in passes of at most kGuPass (bounds the LDS of gate/up results)
  for (int64_t v0 = va; v0 < vb; v0 += kGuPass) {
    const int nvr = (int)((vb - v0) < kGuPass ? (vb - v0) : kGuPass);
    j.v0 = v0;
    run_rowdots(a.H, 2 * nvr, mt, j);
    __syncthreads();
    for (int e = threadIdx.x; e < nvr * mt; e += kThreads) {
      const int vi = e / mt, tt = e % mt;
      const int64_t vr = v0 + vi;
      const int u = (int)(vr / a.I), r = (int)(vr % a.I);
      if (tt < tk->ntok[u]) {
        const float gg = j.gs[((size_t)vi * a.max_batch + tt) * 2];
        const float uu = j.gs[((size_t)vi * a.max_batch + tt) * 2 + 1];
        const float hv = gg / (1.0f + __expf(-gg)) * uu;
        hl[(size_t)tk->pair[u][tt] * a.I + r] = f2bf(hv);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// OUT: rows [r0, r1) of the hidden state.

struct JobO {
  const uint16_t* W;
  int r0, K, maxB;
  const uint16_t* xs;
  float* ao;
  DEV const uint4* row(int i) const { return (const uint4*)(W + (size_t)(r0 + i) * K); }
  DEV int nx(int) const { return 1 << 30; }
  DEV const uint4* x(int, int t) const { return (const uint4*)(xs + (size_t)t * K); }
  DEV void emit(int i, int t, float v) const { ao[(size_t)i * maxB + t] = v; }
};

struct JobDown {
  const TopK* tk;
  const uint16_t* W;
  const uint16_t* hs;
  float* contrib;
  int r0, H, I, nU, maxBK;
  DEV const uint4* row(int i) const {
    const int rr = i / nU, u = i % nU;
    return (const uint4*)(W + ((size_t)tk->U[u] * H + r0 + rr) * I);
  }
  DEV int nx(int i) const { return tk->ntok[i % nU]; }
  DEV const uint4* x(int i, int t) const { return (const uint4*)(hs + (size_t)tk->pair[i % nU][t] * I); }
  DEV void emit(int i, int t, float v) const { contrib[(size_t)(i / nU) * maxBK + tk->pair[i % nU][t]] = v; }
};

DEV void copy_to_lds(uint16_t* dst, const uint16_t* src, int elems) {
  const uint4* s4 = (const uint4*)src;
  uint4* d4 = (uint4*)dst;
  for (int i = threadIdx.x; i < elems / 8; i += kThreads) d4[i] = s4[i];
}

DEV void task_out(const KArgs& a, const Task& t, const Lds& s, int qi) {
  const int l = t.layer, nr = t.r1 - t.r0, n = a.n, AD = a.nq * a.d;
  float* ao = (float*)s.C;                                    // [out_rows_max][maxB]
  float* contrib = ao + (size_t)a.out_rows_max * a.max_batch;  // [out_rows_max][maxB*topk]
  const int maxBK = a.max_batch * a.topk;
  // attention output projection
  uint16_t* xs = (uint16_t*)s.A;
  copy_to_lds(xs, a.attn_out + (size_t)l * a.max_batch * AD, n * AD);
  __syncthreads();
  JobO jo;
  jo.W = wptr(a, widx(l, WL_O));
  jo.r0 = t.r0;
  jo.K = AD;
  jo.maxB = a.max_batch;
  jo.xs = xs;
  jo.ao = ao;
  run_rowdots(AD, nr, n, jo);
  // expert down projections
  compute_topk(a, l, s.tk);  // begins and ends with barriers, so xs is free afterwards
  const TopK* tk = s.tk;
  copy_to_lds(xs, a.h + (size_t)l * a.max_batch * a.topk * a.I, n * a.topk * a.I);
  __syncthreads();
  JobDown jd;
  jd.tk = tk;
  jd.W = wptr(a, widx(l, WL_DOWN));
  jd.hs = xs;
  jd.contrib = contrib;
  jd.r0 = t.r0;
  jd.H = a.H;
  jd.I = a.I;
  jd.nU = tk->nU;
  jd.maxBK = maxBK;
  run_rowdots(a.I, nr * tk->nU, tk->maxtok, jd);
  __syncthreads();
  // x_{l+1} = (x_l + attn) + sum_j w_j y_j
  for (int e = threadIdx.x; e < nr * n; e += kThreads) {
    const int rr = e / n, b = e % n;
    float moe = 0.f;
    for (int j = 0; j < a.topk; ++j) moe += tk->w[b][j] * contrib[(size_t)rr * maxBK + b * a.topk + j];
    const uint16_t* emb = l == 0 ? token_row(a, b, qi) : nullptr;
    const float xo = load_x(a, l, b, t.r0 + rr, emb);
    a.x[((size_t)(l + 1) * a.max_batch + b) * a.H + t.r0 + rr] = (xo + ao[(size_t)rr * a.max_batch + b]) + moe;
  }
}

// ---------------------------------------------------------------------------
// LMHEAD: rows [r0, r1) of the vocabulary, then the greedy argmax.

struct JobLM {
  const uint16_t* W;
  int r0, K, V, maxB;
  const uint16_t* xs;
  float* lmv;
  float* logits;
  DEV const uint4* row(int i) const { return (const uint4*)(W + (size_t)(r0 + i) * K); }
  DEV int nx(int) const { return 1 << 30; }
  DEV const uint4* x(int, int t) const { return (const uint4*)(xs + (size_t)t * K); }
  DEV void emit(int i, int t, float v) const {
    logits[(size_t)t * V + r0 + i] = v;
    lmv[(size_t)i * maxB + t] = v;
  }
};

// Block-wide argmax (value desc, index asc); result valid in all threads.
DEV void block_argmax(float& v, int& i, float* red) {
  if (v != v) v = kNegInf;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(v, m);
    const int oi = __shfl_xor(i, m);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = v;
    ((int*)red)[8 + (threadIdx.x >> 6)] = i;
  }
  __syncthreads();
  v = red[0];
  i = ((int*)red)[8];
  for (int w = 1; w < kWaves; ++w)
    if (better(red[w], ((int*)red)[8 + w], v, i)) { v = red[w]; i = ((int*)red)[8 + w]; }
}

DEV void task_lmhead(const KArgs& a, const Task& t, const Lds& s, int qi) {
  const int L = a.L, nr = t.r1 - t.r0;
  uint16_t* xs = (uint16_t*)s.A;
  norm_inputs(a, L, wptr(a, W_FINAL_NORM), xs, s.red, qi);
  JobLM j;
  j.W = wptr(a, W_LM_HEAD);
  j.r0 = t.r0;
  j.K = a.H;
  j.V = a.V;
  j.maxB = a.max_batch;
  j.xs = xs;
  j.lmv = (float*)s.C;
  j.logits = a.logits;
  run_rowdots(a.H, nr, a.n, j);
  __syncthreads();
  for (int b = 0; b < a.n; ++b) {
    float v = kNegInf;
    int i = 0x7fffffff;
    for (int r = threadIdx.x; r < nr; r += kThreads) {
      float x = j.lmv[(size_t)r * a.max_batch + b];
      if (x != x) x = kNegInf;
      if (better(x, t.r0 + r, v, i)) { v = x; i = t.r0 + r; }
    }
    block_argmax(v, i, s.red);
    if (threadIdx.x == 0) {
      a.lm_part[((size_t)t.idx * a.max_batch + b) * 2] = v;
      ((int*)a.lm_part)[((size_t)t.idx * a.max_batch + b) * 2 + 1] = i;
    }
  }
  uint32_t* ticket = a.tickets + (size_t)a.L * a.max_batch * a.nkv;
  if (arrive_last(ticket, (uint32_t)a.n_lm, s.flags + 11)) {
    for (int b = 0; b < a.n; ++b) {
      float v = kNegInf;
      int i = 0x7fffffff;
      for (int k = threadIdx.x; k < a.n_lm; k += kThreads) {
        const float x = a.lm_part[((size_t)k * a.max_batch + b) * 2];
        const int xi = ((const int*)a.lm_part)[((size_t)k * a.max_batch + b) * 2 + 1];
        if (better(x, xi, v, i)) { v = x; i = xi; }
      }
      block_argmax(v, i, s.red);
      if (threadIdx.x == 0 && a.next_tok) a.next_tok[b] = i;
    }
  }
}

// ---------------------------------------------------------------------------

extern "C" __global__ void __launch_bounds__(kThreads, 1) mk_megakernel(KArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  const Lds s = carve(lds_raw, a);
  const int cu = blockIdx.x;
  const int q0 = a.queue_off[cu], q1 = a.queue_off[cu + 1];
  for (int q = q0; q < q1; ++q) {
    const Task t = a.tasks[q];
    bool ok = wait_counter(a, t.wait[0], t.fanin[0], q, s.flags + 0);
    if (ok && t.wait[1] >= 0) ok = wait_counter(a, t.wait[1], t.fanin[1], q, s.flags + 1);
    if (ok) {
      switch (t.op) {
        case OP_PRE: task_pre(a, t, s, q); break;
        case OP_ATTN: task_attn(a, t, s, q); break;
        case OP_GATEUP: task_gateup(a, t, s, q); break;
        case OP_OUT: task_out(a, t, s, q); break;
        case OP_LMHEAD: task_lmhead(a, t, s, q); break;
        default: break;
      }
    }
    signal_counter(a, t.signal);
  }
}

__global__ void mk_fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

extern "C" int mkk_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t stream) {
  size_t blocks = (n + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(mk_fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, v, n);
  return (int)hipGetLastError();
}

extern "C" int mkk_launch_step(const KArgs* a, int grid, size_t lds_bytes, hipStream_t stream) {
  static size_t attr_bytes = 0;
  if (lds_bytes > attr_bytes) {
    hipError_t e = hipFuncSetAttribute((const void*)mk_megakernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return (int)e;
    attr_bytes = lds_bytes;
  }
  KArgs copy = *a;
  void* args[] = {&copy};
  return (int)hipLaunchCooperativeKernel((const void*)mk_megakernel, dim3(grid), dim3(kThreads), args,
                                         (unsigned)lds_bytes, stream);
}
