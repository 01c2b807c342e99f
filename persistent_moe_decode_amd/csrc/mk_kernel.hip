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
//           the segment's lead (which took its first chunk) merges all
//           chunks once the others have reported (log-sum-exp combine);
//   GATEUP  top-k of the router logits, then rows of the selected experts'
//           gate and up projections and SwiGLU;
//   WO      rows of Wo times the merged attention output: the attention half
//           of the residual;
//   OUT     rows of the selected experts' down projections, weighted expert
//           sum added to the residual rows: the expert half (parallel block:
//           the next layer's readers add the two halves, x + moe + attn);
//   GUTAIL  (opt-in) gate/up rows claimed from the layer's shared pool;
//   LMHEAD  final RMSNorm, rows of the LM head, greedy or sampled argmax
//           (last arriver).
// Weight rows stream from HBM with 128-bit loads; at batch 1 lanes accumulate
// in fp32 with v_dot2_f32_bf16 and groups of lanes reduce through DPP, at
// batch >= 2 rows that every token uses run as 16-row matrix-core tiles.
//
// This file is compiled four times.  With MK_WFMT = 0 it is the kernel for
// bf16 weights (and with MK_SEQ = 1, mk_kernel_seq.hip, the same for the
// sequential block); with MK_WFMT = 1 (mk_kernel_fp8.hip) or 2 (mk_kernel_fp4.hip)
// the LM head, Wqkv, Wo and the expert gate/up/down matrices are FP8 (OCP
// E4M3) or FP4 (OCP E2M1, two codes a byte) codes with one fp32 scale per row
// after each matrix's codes: the row loops convert the codes to bf16 in
// registers (exact: every E4M3 and E2M1 value is a bf16 value), accumulate as
// for bf16 weights and multiply the row's sum by its scale.  Router, norm
// gains, embedding and the KV cache stay bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mk.h"
#include "mk_types.h"

using namespace mk;

#define DEV __device__ __forceinline__
#define TASK __device__ __forceinline__

#ifndef MK_WFMT
#define MK_WFMT 0  // weight format: 0 bf16, 1 FP8 E4M3, 2 FP4 E2M1
#endif
#ifndef MK_SEQ
#define MK_SEQ 0   // 1: the sequential block (attention, then the MoE path behind its own norm)
#endif
#if MK_SEQ && MK_WFMT != 0
#error "the sequential block is built for bf16 weights only"
#endif
#if MK_WFMT == 1
#define MKK(name) name##_fp8
#elif MK_WFMT == 2
#define MKK(name) name##_fp4
#elif MK_SEQ
#define MKK(name) name##_seq
#else
#define MKK(name) name
#endif
// a separate build, so the parallel block's kernel carries none of the sequential block's branches
constexpr bool kSeq = MK_SEQ != 0;
// the streamed matrices (LM head, Wqkv, Wo, experts): quantized or not, bits per element
constexpr bool kWQ = MK_WFMT != 0;
constexpr int kWBits = MK_WFMT == 1 ? 8 : (MK_WFMT == 2 ? 4 : 16);
// bits per element of a row: WQ (the kernel's quantized format) or bf16
template <bool WQ>
constexpr int row_bits() { return WQ ? kWBits : 16; }
// bytes of a K-element streamed-matrix row in the kernel's format
DEV constexpr int wrow_bytes(int K) { return K * kWBits / 8; }

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// Weights are addressed through global-address-space pointers and LDS tiles
// through LDS pointers.  A generic pointer (one the compiler cannot place)
// becomes a FLAT access, which counts against both the memory and the LDS
// wait counters, so every later LDS read would wait for all weight loads in
// flight.
#define AS_GLOBAL __attribute__((address_space(1)))
#define AS_LDS __attribute__((address_space(3)))
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
typedef const AS_GLOBAL uint16_t gu16;
typedef const AS_GLOBAL u32x4_v gu4;
typedef const AS_LDS u32x4_v lu4;

// Data that one compute unit writes and another reads within a launch goes
// through device-coherent accesses: relaxed agent-scope atomic stores and
// loads (the store is written through past the writer's L2, the load never
// hits a stale line in the reader's L2), and LDS copies with the same cache
// policy.  Ordering comes from the flags: a task waits for its own stores to
// complete before it sets its flag, and readers load only after they have
// seen every flag they need.  No cache-wide write-back or invalidate is
// needed, which keeps a wait-and-signal hop to about one memory round trip.
constexpr int kCohPolicy = 16;  // sc1: device-scope coherent (cache policy operand of the LDS copy)
// Weights and K/V are read once per step: their loads carry the non-temporal
// hint (nt), so they do not push code, page tables and activations out of L2.
constexpr int kStreamPolicy = 2;
DEV void st_coh(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV void st_coh(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV void st_coh(uint16_t* p, uint16_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Epoch-tagged words: a value and the step's epoch stored together by one
// 64-bit device-coherent store, so a reader that sees the tag sees the value
// (each aligned 8-byte store is single-copy atomic).  A consumer polls the
// words themselves: the producer needs no counter and no wait for its stores
// to complete, and the consumer no second round trip after the flag.
DEV void st_tag(uint64_t* p, float v, uint32_t epoch) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes at byte offset `off` of [base, base + nbytes), read with the same
// device-coherent cache policy as the atomic loads above (sc1): data another
// compute unit wrote in this launch, read after its flag was seen.  One
// 16-byte load per lane (the LDS copy engine moves data at a fraction of this
// rate per compute unit); offsets past nbytes read as zero.  base and nbytes
// must be the same in every lane (they form a scalar buffer resource).
DEV u32x4_v ld_coh16(const void* base, uint32_t nbytes, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCohPolicy);
}

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

typedef float float2_v __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 bit patterns (round to nearest even), low half
// first: one gfx950 v_cvt_pk_bf16_f32.  Finite values round exactly as f2bf.
DEV uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_v){a, b}, bf16x2_v));
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

#if MK_WFMT == 1
// Two E4M3 codes (bytes 0, 1, or with HI bytes 2, 3 of w) as a bf16 pair, exactly (scale 1).
template <bool HI>
DEV uint32_t fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// 16 E4M3 codes (one 16-byte chunk) dotted with 16 bf16 inputs (x[0]: the first 8).
DEV float dotq(const uint4& w, const uint4* x, float acc) {
  acc = dot2(fp8x2_bf16<false>(w.x), x[0].x, acc);
  acc = dot2(fp8x2_bf16<true>(w.x), x[0].y, acc);
  acc = dot2(fp8x2_bf16<false>(w.y), x[0].z, acc);
  acc = dot2(fp8x2_bf16<true>(w.y), x[0].w, acc);
  acc = dot2(fp8x2_bf16<false>(w.z), x[1].x, acc);
  acc = dot2(fp8x2_bf16<true>(w.z), x[1].y, acc);
  acc = dot2(fp8x2_bf16<false>(w.w), x[1].z, acc);
  acc = dot2(fp8x2_bf16<true>(w.w), x[1].w, acc);
  return acc;
}

// The 8 bf16 values of codes 8j .. 8j + 7 of a 16-byte chunk (j = 0, 1).
DEV uint4 q8_bf16(const uint4& w, int j) {
  const uint32_t a = j ? w.z : w.x, b = j ? w.w : w.y;
  return make_uint4(fp8x2_bf16<false>(a), fp8x2_bf16<true>(a), fp8x2_bf16<false>(b), fp8x2_bf16<true>(b));
}
#elif MK_WFMT == 2
// The two E2M1 codes of byte B of w (low nibble first) as a bf16 pair, exactly (scale 1).
template <int B>
DEV uint32_t fp4x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
}

// The 8 bf16 values of the 8 E2M1 codes of one 32-bit word.
DEV uint4 fp4x8_bf16(uint32_t w) {
  return make_uint4(fp4x2_bf16<0>(w), fp4x2_bf16<1>(w), fp4x2_bf16<2>(w), fp4x2_bf16<3>(w));
}

// 32 E2M1 codes (one 16-byte chunk) dotted with 32 bf16 inputs (x[0..3], 8 each).
DEV float dotq(const uint4& w, const uint4* x, float acc) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc = dot2(fp4x2_bf16<0>(ws[k]), x[k].x, acc);
    acc = dot2(fp4x2_bf16<1>(ws[k]), x[k].y, acc);
    acc = dot2(fp4x2_bf16<2>(ws[k]), x[k].z, acc);
    acc = dot2(fp4x2_bf16<3>(ws[k]), x[k].w, acc);
  }
  return acc;
}

// The 8 bf16 values of codes 8j .. 8j + 7 of a 16-byte chunk (j = 0..3).
DEV uint4 q8_bf16(const uint4& w, int j) { return fp4x8_bf16(j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w); }
#endif

// One 16-byte weight chunk dotted with its inputs: 8 bf16 weights with x[0],
// or (WQ) the chunk's 16 / kWBits * 8 codes with x[0 .. 16 / kWBits - 1].
template <bool WQ>
DEV float dotw(const uint4& w, const uint4* x, float acc) {
#if MK_WFMT != 0
  if constexpr (WQ) return dotq(w, x, acc);
#endif
  return dot8(w, x[0], acc);
}

// w, passed through an empty volatile asm: its conversion to bf16 inside a loop
// over tokens then stays in that loop instead of being hoisted out of it as
// XM times as many live registers.
DEV void opaque(uint4& w) { asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w)); }

// The thread's index, read through an empty volatile asm: the compiler then
// cannot hoist per-lane arithmetic out of the persistent task loop, where it
// would stay live across every task body and spill.
DEV int tid() {
  int t = (int)__builtin_amdgcn_workitem_id_x();
  asm volatile("" : "+v"(t));
  return t;
}

template <int CTRL>
DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
DEV uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
DEV double dpp_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = dpp_u<CTRL>((uint32_t)u), hi = dpp_u<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}

// The gfx950 row swaps: with both operands the same register,
// permlane16_swap returns (even row, odd row) of each pair of 16-lane rows in
// every lane, permlane32_swap (lower half, upper half).  Sums of the two, in
// that order, at VALU speed (no LDS round trip as with a shuffle).
DEV float xrow16_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto t = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
DEV float xrow32_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
DEV double xrow_sum_d(double v, bool half) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  const auto l = half ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false) : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h = half ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false) : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const double a = __longlong_as_double((long long)(((uint64_t)h[0] << 32) | l[0]));
  const double b = __longlong_as_double((long long)(((uint64_t)h[1] << 32) | l[1]));
  return a + b;
}

// Sum over aligned groups of N lanes; every lane of a group gets the sum.
// quad_perm [1,0,3,2] and [2,3,0,1] pair lanes within a quad, row_half_mirror
// pairs the two quads of 8 lanes, row_mirror the two halves of a 16-lane row;
// row swaps then pair 16-lane rows and the two halves of the wave.
template <int N>
DEV float group_sum(float v) {
  v += dpp<0xB1>(v);
  if (N >= 4) v += dpp<0x4E>(v);
  if (N >= 8) v += dpp<0x141>(v);
  if (N >= 16) v += dpp<0x140>(v);
  if (N >= 32) v = xrow16_sum(v);
  if (N >= 64) v = xrow32_sum(v);
  return v;
}

// Sum over the whole wave of a double, in every lane.
DEV double wave_sum_d(double v) {
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x141>(v);
  v += dpp_d<0x140>(v);
  v = xrow_sum_d(v, false);
  return xrow_sum_d(v, true);
}

// ---------------------------------------------------------------------------
// LDS carve-up.  Region A: input vectors.  Region B: top-k state, flags and
// reduction scratch.  Region C: per-op arrays.

struct TopK {
  int32_t sel[kMaxBatch][kMaxTopK];
  float w[kMaxBatch][kMaxTopK];
  int32_t nU, maxtok, pad_[2];
  int32_t U[kMaxBatch * kMaxTopK];                // distinct experts, ascending
  int32_t ntok[kMaxBatch * kMaxTopK];             // tokens routed to U[u]
  int32_t pair[kMaxBatch * kMaxTopK][kMaxBatch];  // b*topk+j of each of them, ascending b
};
constexpr int kTopKBytes = 3136;
static_assert(sizeof(TopK) <= kTopKBytes && sizeof(TopK) % 16 == 0, "top-k state fits region B, 16-byte multiple");

struct Lds {
  uint8_t* base;
  uint8_t* A;
  TopK* tk;
  int32_t* flags;  // [32]
  float* red;      // [16]
  double* red8;    // [kWaves][kMaxBatch]
  float* rot;      // attention units: cos, sin of the rotation at the chunk's position [2][64] (with the plan)
  uint8_t* C;
  uint8_t* P;      // prefetched weight tile
};

// Region B (kLdsB bytes): top-k state | flags | red | red8 | ... | rotation table at +4096.
DEV Lds carve(uint8_t* lds, const KArgs& a) {
  Lds s;
  s.base = lds;
  s.A = lds;
  s.tk = (TopK*)(lds + a.lds_b);
  s.flags = (int32_t*)(lds + a.lds_b + kTopKBytes);
  s.red = (float*)(lds + a.lds_b + kTopKBytes + 128);
  s.red8 = (double*)(lds + a.lds_b + kTopKBytes + 192);
  s.rot = (float*)(lds + a.lds_b + 4096);
  s.C = lds + a.lds_c;
  s.P = lds + a.lds_p;
  return s;
}
static_assert(kTopKBytes + 192 + 8 * kWaves * kMaxBatch <= 4096, "region B head fits");
static_assert(4096 + 2 * 64 * 4 <= kLdsB, "rotation table fits region B");

// All threads get the block-wide sum; the order of the partial sums is fixed.
DEV float block_sum(float v, float* red) {
  v = group_sum<64>(v);
  __syncthreads();
  if ((tid() & 63) == 0) red[tid() >> 6] = v;
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

// Sum of a counter's sub-counters, in every lane of the calling wave.
// The sub-counters sit in lanes 0..15 (the wave's first row): DPP sums the
// row, lane 0 hands the total to the wave.
static_assert(kSubCounters == 16, "counter_sum sums one 16-lane row");
DEV uint32_t counter_sum(const KArgs& a, int idx) {
  const int lane = tid() & 63;
  uint32_t v = lane < kSubCounters ? ld_coh(a.flags + (size_t)idx * kCounterWords + lane * kSubStride) : 0u;
  v += dpp_u<0xB1>(v);
  v += dpp_u<0x4E>(v);
  v += dpp_u<0x141>(v);
  v += dpp_u<0x140>(v);
  return __builtin_amdgcn_readfirstlane(v);
}

// Wave 0 polls the counter (relaxed device-coherent loads of its
// sub-counters, s_sleep between polls) until it sums to want (mod 2^32,
// compared as a signed difference; a full wait is epoch * fanin); the
// barrier hands the result to the other waves.  The wait is bounded: past
// the spin limit the task raises MK_ERR_DEVICE_TIMEOUT and the grid drains.
// The abort flag is read every 32 polls, not before the first one (that
// would put a dependent round trip in front of every wait).  Returns false
// when the grid is aborting or the wait timed out.
DEV bool wait_counter_until(const KArgs& a, int idx, uint32_t want, int task, int32_t* slot) {
  if (tid() < 64) {
    const int lane = tid();
    int ok = 1;
    if (idx >= 0) {
      const uint64_t t0 = wall_clock64();
      uint32_t it = 0;
      while ((int32_t)(counter_sum(a, idx) - want) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if ((++it & 31) == 0) {
          int stop = 0;
          if (lane == 0) stop = aborting(a) ? 1 : (wall_clock64() - t0 > a.spin_limit_ticks ? 2 : 0);
          stop = __shfl(stop, 0);
          if (stop) {
            if (lane == 0 && stop == 2) raise_error(a, MK_ERR_DEVICE_TIMEOUT, task, idx);
            ok = 0;
            break;
          }
        }
      }
    }
    if (lane == 0) *slot = ok;
  }
  __syncthreads();
  return *slot != 0;
}

DEV bool wait_counter_at(const KArgs& a, int idx, int fanin, int task, int32_t* slot, uint32_t epoch) {
  return wait_counter_until(a, idx, epoch * (uint32_t)fanin, task, slot);
}

DEV bool wait_counter(const KArgs& a, int idx, int fanin, int task, int32_t* slot) {
  return wait_counter_at(a, idx, fanin, task, slot, a.epoch);
}

// Until need of this step's fanin signals of counter idx are in.
DEV bool wait_counter_part(const KArgs& a, int idx, int fanin, int need, int task, int32_t* slot) {
  return wait_counter_until(a, idx, (a.epoch - 1u) * (uint32_t)fanin + (uint32_t)need, task, slot);
}

// A workgroup barrier that orders LDS accesses only: each wave waits for its
// own LDS reads and writes, not for its vector-memory loads.  __syncthreads()
// also waits for every LDS copy-engine transfer the wave has in flight (they
// write LDS), which would hold a wave up for a whole weight tile that nobody
// reads before a later full barrier.
DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waves 0 .. wait_waves - 1 (those that stored what the consumers read) wait
// for their stores to complete, the barrier orders them before thread 0's
// add; the other waves may leave loads in flight (an LDS copy for the next
// task, waited there), which the LDS-only barrier does not wait for.
DEV void signal_counter(const KArgs& a, int idx, int slot, int wait_waves = kWaves) {
  if ((tid() >> 6) < wait_waves) __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  if (tid() == 0 && idx >= 0)
    __hip_atomic_fetch_add(a.flags + (size_t)idx * kCounterWords + (slot % kSubCounters) * kSubStride, 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Ticket for "last of count arrivals does the merge": returns true in every
// thread of the last arriving workgroup, which also resets the ticket.  Each
// arrival's stores are complete before its add.
DEV bool arrive_last(uint32_t* ticket, uint32_t count, int32_t* slot) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid() == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == count - 1;
    if (last) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *slot = last;
  }
  __syncthreads();
  return *slot != 0;
}

// Wave 0 polls a ticket word until it holds `want`, then resets it for the
// next step; bounded like wait_counter (abort flag read every 32 polls).  Returns false when the grid is
// aborting or the wait timed out.
DEV bool wait_ticket(const KArgs& a, uint32_t* ticket, uint32_t want, int task, int32_t* slot) {
  if (tid() < 64) {
    const int lane = tid();
    int ok = 1;
    {
      const uint64_t t0 = wall_clock64();
      uint32_t it = 0;
      while (__builtin_amdgcn_readfirstlane(ld_coh(ticket)) != want) {
        __builtin_amdgcn_s_sleep(1);
        if ((++it & 31) == 0) {
          int stop = 0;
          if (lane == 0) stop = aborting(a) ? 1 : (wall_clock64() - t0 > a.spin_limit_ticks ? 2 : 0);
          stop = __shfl(stop, 0);
          if (stop) {
            if (lane == 0 && stop == 2) raise_error(a, MK_ERR_DEVICE_TIMEOUT, task, -1);
            ok = 0;
            break;
          }
        }
      }
      if (ok && lane == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) *slot = ok;
  }
  __syncthreads();
  return *slot != 0;
}


// ---------------------------------------------------------------------------
// inputs

DEV const gu16* wptr(const KArgs& a, int i) { return (const gu16*)(uintptr_t)a.wtab[i]; }

// The gain of the norm in front of layer l's MoE path: the attention norm's
// (parallel block), or the MoE path's own (sequential block).
DEV const gu16* moe_gain(const KArgs& a, int l) {
  return wptr(a, kSeq ? widx_moe_norm(a.L, l) : widx(l, WL_NORM));
}
// a streamed matrix as bytes (bf16 elements, or FP8 codes followed by the rows' fp32 scales)
typedef const AS_GLOBAL uint8_t gu8;
DEV const gu8* wbytes(const KArgs& a, int i) { return (const gu8*)(uintptr_t)a.wtab[i]; }
// row scales of a quantized matrix of `rows` rows of `cols` codes
DEV const AS_GLOBAL float* wscales(const KArgs& a, int i, size_t rows, int cols) {
  return (const AS_GLOBAL float*)(wbytes(a, i) + rows * (size_t)wrow_bytes(cols));
}

// Trace mark k (0..3) of task qi: the clock when thread 0 passes this point.
DEV void mark(const KArgs& a, int qi, int k) {
  if (a.trace && tid() == 0 && qi < a.trace_cap) a.trace[kTraceWords * (size_t)qi + 2 + k] = wall_clock64();
}

// The token of sequence b in this step: the caller's at step 0, the greedy
// token of the previous step (written in this launch) after that.
DEV const gu16* token_row(const KArgs& a, int b, int task) {
  int tok = a.step == 0 ? a.tokens[b] : (int)ld_coh((const uint32_t*)a.next_tok + (size_t)(a.step - 1) * a.n + b);
  if (tok < 0 || tok >= a.V) {
    raise_error(a, MK_ERR_DEVICE_TOKEN, task, b);
    tok = 0;
  }
  return wptr(a, W_EMBED) + (size_t)tok * a.H;
}

// Residual entering `layer` >= 1, from the previous layer's two halves:
// x_layer = (x_{layer-1} + moe) + attn, the expert half written by the
// output tasks, the attention half (attention output times Wo) by the Wo
// tasks.  Neither kind of task waits for the other; whoever reads x adds them.
DEV float resid(const KArgs& a, int layer, int b, int i) {
  const size_t o = (size_t)b * a.H + i;
  return ld_coh(a.x + (size_t)layer * a.max_batch * a.H + o) +
         ld_coh(a.wo_out + (size_t)(layer - 1) * a.max_batch * a.H + o);
}

// Residual entering `layer` (layer 0: the embedding row).
// With the layer-input hook set, layers >= 1 (and the final norm) read the
// residual the caller supplied instead of the one the previous layer wrote.
// Sequential block: the residual the MoE path starts from, x_layer plus this
// layer's Wo rows (x_layer itself whole in the x buffer).
DEV float load_x(const KArgs& a, int layer, int b, int i, const gu16* emb) {
  if constexpr (!kSeq) {
    if (layer == 0) return bf2f(emb[i]);
    if (a.x_in) return a.x_in[((size_t)layer * a.max_batch + b) * a.H + i];
    return resid(a, layer, b, i);
  } else {
    const size_t o = ((size_t)layer * a.max_batch + b) * a.H + i;
    const float x = layer == 0 ? bf2f(emb[i]) : (a.x_in ? a.x_in[o] : ld_coh(a.x + o));
    return x + ld_coh(a.wo_out + o);
  }
}

DEV u32x4_v add4(u32x4_v u, u32x4_v v) {
  u32x4_v r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = __float_as_uint(__uint_as_float(u[k]) + __uint_as_float(v[k]));
  return r;
}

// double -> bfloat16 bits, round to nearest even: round the 52-bit mantissa to
// 7 fraction bits, dropping 45 (add half-minus-one plus the kept lsb; carries
// run into the exponent as they should), then the value is exact in float and
// its upper half is the bfloat16.
DEV uint16_t d2bf(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  if ((u & 0x7fffffffffffffffull) > 0x7ff0000000000000ull) return 0x7fc0;
  u += 0x00000fffffffffffull + ((u >> 45) & 1ull);
  u &= ~0x00001fffffffffffull;
  return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)u)) >> 16);
}

// xs[b][H] = bf16(x_b / sqrt(mean(x_b^2) + eps) * g) for b < n, evaluated in
// double so the one rounding to bf16 is the only one (the normalized input
// feeds every projection of the layer).
// The input rows (this layer's x, fp32, or at layer 0 the tokens' embedding
// rows, bf16) and the gain are copied into LDS behind xs with register
// loads by all threads.  The sums of squares
// of all rows are reduced together: one barrier for the whole batch.  The
// loops run over the batch at run time, which keeps the code short: it runs
// once per layer and is fetched anew each time.

// All threads copy nbytes (a multiple of 16) from global memory into LDS with
// 16-byte register loads, up to 8 per thread in flight before the LDS
// writes (the LDS copy engine moves far fewer bytes per compute unit).  Coh:
// the data was written by other compute units in this launch (sc1 loads);
// otherwise plain loads of data written before the launch.  In LDS after the
// next barrier.
template <bool Coh>
DEV void copy_to_lds(void* dst, const void* src, uint32_t nbytes) {
  const uint32_t n16 = nbytes / 16;
  u32x4_v* d = (u32x4_v*)dst;
  for (uint32_t q0 = 0; q0 < n16; q0 += 8 * kThreads) {
    u32x4_v v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t q = q0 + k * kThreads + tid();
      if constexpr (Coh) v[k] = ld_coh16(src, nbytes, q * 16);  // past nbytes: zero, not stored
      else v[k] = q < n16 ? ((const gu4*)src)[q] : u32x4_v{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t q = q0 + k * kThreads + tid();
      if (q < n16) d[q] = v[k];
    }
  }
}

// The staging area behind xs in region A: [max_batch][H] fp32 rows, then the gain [H].
DEV uint8_t* norm_stage(const KArgs& a, uint16_t* xs) {
  return (uint8_t*)xs + (((size_t)a.max_batch * a.H * 2 + 255) & ~(size_t)255);
}

// Elements 4c .. 4c + 3 of rows 0 .. n - 1 of the staged input (fp32 rows,
// or bf16 embedding rows at layer 0); rows >= n read as zero.
DEV void norm_row4(const uint8_t* stage, bool emb, int H, int n, int c, float (&v)[kMaxBatch][4]) {
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) {
    if (b < n && emb) {
      const uint2 u = *(const uint2*)(stage + ((size_t)b * H + 4 * c) * 2);
      v[b][0] = bf2f(u.x & 0xffffu);
      v[b][1] = bf2f(u.x >> 16);
      v[b][2] = bf2f(u.y & 0xffffu);
      v[b][3] = bf2f(u.y >> 16);
    } else if (b < n) {
      const float4 f = *(const float4*)(stage + ((size_t)b * H + 4 * c) * 4);
      v[b][0] = f.x;
      v[b][1] = f.y;
      v[b][2] = f.z;
      v[b][3] = f.w;
    } else {
      v[b][0] = v[b][1] = v[b][2] = v[b][3] = 0.f;
    }
  }
}

// mk >= 0: trace mark mk of the task once the inputs are in LDS.  rec (or
// NULL): where to record the residual entering `layer` (>= 1) as summed here
// from the previous layer's halves, also when the hook supplies the input.
// side: kParallel, the residual entering `layer` as the sum of the previous
// layer's halves (x + moe, and its Wo rows); kAlone (sequential block:
// attention side and final norm), x_layer as the previous layer's output
// tasks wrote it whole; kWithWo (sequential block: the MoE path), x_layer
// plus this layer's Wo rows.  The layer-input hook, where set, supplies
// x_layer for layers >= 1.
enum NormSide : int { kParallel = 0, kAlone = 1, kWithWo = 2 };

DEV void norm_inputs(const KArgs& a, int layer, const gu16* gain, uint16_t* xs, double* red8, int task, int mk,
                     float* rec = nullptr, int side = kParallel) {
  const int H = a.H, n = a.n, lane = tid() & 63, wave = tid() >> 6;
  uint8_t* stage = norm_stage(a, xs);
  uint16_t* gs = (uint16_t*)(stage + (size_t)a.max_batch * H * 4);
  const bool emb = layer == 0 && side != kWithWo;
  {
    if constexpr (!kSeq) {
      // the input rows (the two halves of x: one 16-byte load each per thread
      // and row at hidden 2048) and the gain, all in flight before any is
      // written to LDS
      const uint32_t nx16 = emb ? 0u : (uint32_t)n * H / 4, ng16 = (uint32_t)H / 8;
      const size_t o = (size_t)layer * a.max_batch * H;
      const float* xh = a.x + o;                                  // x + moe of the previous layer
      const float* wh = a.wo_out + o - (size_t)a.max_batch * H;   // its attention output times Wo
      u32x4_v* st = (u32x4_v*)stage;
      for (uint32_t q0 = 0; q0 < nx16 + ng16; q0 += 4 * kThreads) {
        u32x4_v v[4], w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t q = q0 + k * kThreads + tid();
          if (q < nx16 && a.x_in) {
            v[k] = ((const gu4*)(a.x_in + o))[q];
          } else if (q < nx16) {
            v[k] = ld_coh16(xh, nx16 * 16, q * 16);
            w[k] = ld_coh16(wh, nx16 * 16, q * 16);
          } else if (q < nx16 + ng16) {
            v[k] = ((const gu4*)gain)[q - nx16];
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t q = q0 + k * kThreads + tid();
          if (q < nx16) {
            const u32x4_v x = a.x_in ? v[k] : add4(v[k], w[k]);
            st[q] = x;
            if (rec && !a.x_in) ((u32x4_v*)(rec + o))[q] = x;
          } else if (q < nx16 + ng16) {
            ((u32x4_v*)gs)[q - nx16] = v[k];
          }
        }
      }
      if (rec && a.x_in)
        for (uint32_t q = tid(); q < nx16; q += kThreads)
          ((u32x4_v*)(rec + o))[q] = add4(ld_coh16(xh, nx16 * 16, q * 16), ld_coh16(wh, nx16 * 16, q * 16));
    } else {
      // the input rows (x and, where added, the Wo rows: one 16-byte load each
      // per thread and row at hidden 2048) and the gain, all in flight before
      // any is written to LDS
      const uint32_t nx16 = emb ? 0u : (uint32_t)n * H / 4, ng16 = (uint32_t)H / 8;
      const size_t o = (size_t)layer * a.max_batch * H;
      const float* xh = a.x + o;                                  // x as the previous layer's output tasks wrote it
      const float* wh = side == kWithWo ? a.wo_out + o            // this layer's attention output times Wo
                                        : a.wo_out + o - (size_t)a.max_batch * H;  // the previous layer's
      // whether the Wo rows are added: the parallel block's halves (unless the
      // hook supplies their sum), the sequential block's MoE side always
      const bool add_w = side == kWithWo || (side == kParallel && !a.x_in);
      const bool emb_w = layer == 0 && side == kWithWo;           // the embedding row plus layer 0's Wo rows
      u32x4_v* st = (u32x4_v*)stage;
      if (emb_w)
        for (int b = 0; b < n; ++b) {
          const gu16* er = token_row(a, b, task);
          for (int c = tid(); 4 * c < H; c += kThreads) {
            const uint2 e = *(const uint2*)(er + 4 * c);
            const u32x4_v v = {__float_as_uint(bf2f(e.x & 0xffffu)), __float_as_uint(bf2f(e.x >> 16)),
                               __float_as_uint(bf2f(e.y & 0xffffu)), __float_as_uint(bf2f(e.y >> 16))};
            const uint32_t q = (uint32_t)(b * (H / 4) + c);
            st[q] = add4(v, ld_coh16(wh, nx16 * 16, q * 16));
          }
        }
      for (uint32_t q0 = emb_w ? nx16 : 0u; q0 < nx16 + ng16; q0 += 4 * kThreads) {
        u32x4_v v[4], w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t q = q0 + k * kThreads + tid();
          if (q < nx16) {
            v[k] = a.x_in ? ((const gu4*)(a.x_in + o))[q] : ld_coh16(xh, nx16 * 16, q * 16);
            if (add_w) w[k] = ld_coh16(wh, nx16 * 16, q * 16);
          } else if (q < nx16 + ng16) {
            v[k] = ((const gu4*)gain)[q - nx16];
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t q = q0 + k * kThreads + tid();
          if (q < nx16) {
            const u32x4_v x = add_w ? add4(v[k], w[k]) : v[k];
            st[q] = x;
            if (rec && !a.x_in) ((u32x4_v*)(rec + o))[q] = x;
          } else if (q < nx16 + ng16) {
            ((u32x4_v*)gs)[q - nx16] = v[k];
          }
        }
      }
      // the record of the residual as this kernel computed it (the hook's input aside)
      if (rec && a.x_in)
        for (uint32_t q = tid(); q < nx16; q += kThreads)
          ((u32x4_v*)(rec + o))[q] = side == kParallel ? add4(ld_coh16(xh, nx16 * 16, q * 16), ld_coh16(wh, nx16 * 16, q * 16))
                                                       : ld_coh16(xh, nx16 * 16, q * 16);
    }
    if (emb)
      for (int b = 0; b < n; ++b)
        copy_to_lds<false>(stage + (size_t)b * H * 2, (const void*)(uintptr_t)token_row(a, b, task), H * 2);
  }
  __syncthreads();
  if (mk >= 0) mark(a, task, mk);
  if (n == 1) {
    // one row: thread t takes elements t, t + 512, ... (measured faster than
    // the vector path below at one row)
    const float* xf = (const float*)stage;
    const uint16_t* xb = (const uint16_t*)stage;
    for (int b = 0; b < n; ++b) {
      double ss = 0.0;
      for (int i = tid(); i < H; i += kThreads) {
        const double v = emb ? (double)bf2f(xb[(size_t)b * H + i]) : (double)xf[(size_t)b * H + i];
        ss += v * v;
      }
      ss = wave_sum_d(ss);
      if (lane == 0) red8[wave * kMaxBatch + b] = ss;
    }
    __syncthreads();
    for (int b = 0; b < n; ++b) {
      double tot = 0.0;
      for (int w = 0; w < kWaves; ++w) tot += red8[w * kMaxBatch + b];
      const double inv = 1.0 / sqrt(tot / (double)H + (double)a.eps);
      for (int i = tid(); i < H; i += kThreads) {
        const double v = emb ? (double)bf2f(xb[(size_t)b * H + i]) : (double)xf[(size_t)b * H + i];
        xs[(size_t)b * H + i] = d2bf(v * inv * (double)bf2f(gs[i]));
      }
    }
  } else {
    // thread t takes elements 4c .. 4c + 3 of every row, c = t, t + 512, ...
    // (H is a multiple of 128); the loads of all rows are issued before any
    // arithmetic, so the LDS round trips overlap instead of adding up
    double ss[kMaxBatch];
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) ss[b] = 0.0;
    for (int c = tid(); 4 * c < H; c += kThreads) {
      float v[kMaxBatch][4];
      norm_row4(stage, emb, H, n, c, v);
#pragma unroll
      for (int b = 0; b < kMaxBatch; ++b)
        if (b < n)
#pragma unroll
          for (int e = 0; e < 4; ++e) ss[b] += (double)v[b][e] * (double)v[b][e];
    }
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      if (b >= n) break;
      const double t = wave_sum_d(ss[b]);
      if (lane == 0) red8[wave * kMaxBatch + b] = t;
    }
    __syncthreads();
    // lane b < n of each wave works out row b's scale (one division per wave,
    // whatever the batch), the others read it from that lane
    double my = 0.0;
    if (lane < n) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) my += red8[w * kMaxBatch + lane];
      my = 1.0 / sqrt(my / (double)H + (double)a.eps);
    }
    double inv[kMaxBatch];
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      const uint64_t u = (uint64_t)__double_as_longlong(my);
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, b);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), b);
      inv[b] = b < n ? __longlong_as_double((long long)(((uint64_t)hi << 32) | lo)) : 0.0;
    }
    for (int c = tid(); 4 * c < H; c += kThreads) {
      float v[kMaxBatch][4];
      norm_row4(stage, emb, H, n, c, v);
      const uint2 gw = *(const uint2*)(gs + 4 * c);
      const double g4[4] = {(double)bf2f(gw.x & 0xffffu), (double)bf2f(gw.x >> 16), (double)bf2f(gw.y & 0xffffu),
                            (double)bf2f(gw.y >> 16)};
#pragma unroll
      for (int b = 0; b < kMaxBatch; ++b) {
        if (b >= n) break;
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = d2bf((double)v[b][e] * inv[b] * g4[e]);
        *(uint2*)(xs + (size_t)b * H + 4 * c) =
            make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Row dot products: each job is one weight row of K bf16 dotted with up to
// maxnx input vectors held in LDS.  LPR lanes share a row; each lane loads
// CPL 16-byte chunks (strided by LPR chunks, so a row's loads coalesce) before
// any arithmetic, so a whole pass of rows is in flight at once.  Rows
// [i0, i1) are done; they come from HBM (job.row, global loads) or, with
// FromLds, from a weight tile already in LDS (job.lrow).

template <bool FromLds, int CPL, int STRIDE, class Job>
DEV void load_row(const Job& job, int i, int li, bool act, uint4 (&wv)[CPL]) {
  if constexpr (FromLds) {
    const lu4* wr = job.lrow(i) + li;
#pragma unroll
    for (int c = 0; c < CPL; ++c) wv[c] = __builtin_bit_cast(uint4, act ? wr[STRIDE * c] : u32x4_v{0, 0, 0, 0});
  } else {
    const gu4* wr = job.row(i) + li;
#pragma unroll
    for (int c = 0; c < CPL; ++c) wv[c] = __builtin_bit_cast(uint4, act ? __builtin_nontemporal_load(wr + STRIDE * c) : u32x4_v{0, 0, 0, 0});
  }
}

// A row's sum times its scale (WQ: quantized rows), or as it is (bf16 rows).
template <bool WQ, class Job>
DEV float scaled(const Job& job, int i, float v) {
  if constexpr (WQ) return v * job.scale(i);
  return v;
}

// WQ: a 16-byte chunk holds 128 / kWBits codes, so it meets XM = 16 / kWBits
// 16-byte input chunks.
template <int LPR, int CPL, bool FromLds, bool WQ, class Job>
DEV void rowdots(int i0, int i1, int maxnx, const Job& job) {
  const int lane = tid() & 63, wave = tid() >> 6;
  constexpr int RPW = 64 / LPR, XM = 16 / row_bits<WQ>();
  const int sub = lane / LPR, li = lane % LPR;
  for (int base = i0; base < i1; base += kWaves * RPW) {
    const int i = base + wave * RPW + sub;
    const bool act = i < i1;
    const int ic = act ? i : i0;
    uint4 wv[CPL];
    load_row<FromLds, CPL, LPR>(job, ic, li, act, wv);
    const int nx = act ? job.nx(ic) : 0;
    for (int t = 0; t < maxnx; ++t) {
      const bool on = t < nx;
      const uint4* xr = job.x(ic, on ? t : 0) + XM * li;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        uint4 w = wv[c];
        if constexpr (WQ) opaque(w);
        acc = dotw<WQ>(w, xr + XM * LPR * c, acc);
      }
      acc = group_sum<LPR>(acc);
      if (on && li == 0) job.emit(i, t, scaled<WQ>(job, i, acc));
    }
  }
}

// Any row of a multiple of 128 elements: 16 lanes per row (bf16), 8 (FP8) or
// 4 (FP4), one 16-byte chunk per lane per load.
template <bool FromLds, bool WQ, class Job>
DEV void rowdots_generic(int K, int i0, int i1, int maxnx, const Job& job) {
  constexpr int LPR = row_bits<WQ>(), RPW = 64 / LPR, XM = 16 / row_bits<WQ>();  // 128 elements per lane-group chunk
  const int lane = tid() & 63, wave = tid() >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  const int cpl = K * row_bits<WQ>() / (128 * LPR);
  for (int base = i0; base < i1; base += kWaves * RPW) {
    const int i = base + wave * RPW + sub;
    const bool act = i < i1;
    const int ic = act ? i : i0;
    const int nx = act ? job.nx(ic) : 0;
    for (int t = 0; t < maxnx; ++t) {
      const bool on = t < nx;
      const uint4* xr = job.x(ic, on ? t : 0) + XM * li;
      float acc = 0.f;
      for (int c = 0; c < cpl; ++c) {
        uint4 w[1];
        load_row<FromLds, 1, LPR>(job, ic, li + LPR * c, act, w);
        acc = dotw<WQ>(w[0], xr + XM * LPR * c, acc);
      }
      acc = group_sum<LPR>(acc);
      if (on && li == 0) job.emit(i, t, scaled<WQ>(job, i, acc));
    }
  }
}

// Dense jobs (every row dotted with all n >= 2 token vectors) on the matrix
// cores: a wave takes a tile of 16 rows and contracts it with the n token
// vectors, v_mfma_f32_16x16x32_bf16 per 32 columns:
//   D[16 rows][16 tokens] += W[16 rows][32] * X^T[32][16 tokens]
// lane l holds row l % 16 of the weights and token l % 16 of the inputs at
// columns 8 * (l / 16) .. + 7 of each 32-column block (tokens >= n are zero),
// and receives D[4 * (l / 16) + q][l % 16] in component q.  Weight rows
// stream from HBM, eight 16-byte loads per lane in flight per batch.  With
// fewer tiles than waves the columns are split into kp parts whose partial
// tiles are summed in LDS (red: kMfmaRedBytes of region C) in part order.
// WQ: one 16-byte load holds XM * 8 consecutive columns of a block of
// 32 * XM columns (XM = 16 / kWBits), converted to bf16 and contracted as XM
// products, each with the inputs at the same 8 columns: the sum over the
// block is the same, only its order differs.
constexpr int kMfmaBatch = 8;                   // 16-byte loads per lane per batch

template <bool WQ, class Job>
DEV void rowdots_mfma(int K, int i0, int i1, int n, const Job& job, float* red) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int XM = 16 / row_bits<WQ>();       // products (8 columns each) per 16-byte load
  constexpr int CB = 32 * XM;                   // columns per block (one load per lane)
  const int lane = tid() & 63, wave = tid() >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int ntile = (i1 - i0 + 15) / 16;
  int kp = 1;
  while (red && kp < 8 && ntile * kp < kWaves && (K / (2 * kp)) % (CB * kMfmaBatch) == 0) kp *= 2;
  const int kl = K / kp;                        // columns per part
  const int nitem = ntile * kp;
  const uint4* xb = job.x(i0, r < n ? r : 0);   // token r's input vector (LDS)
  for (int it = wave; it < nitem; it += kWaves) {
    const int tile = it / kp, part = it - tile * kp;
    const int row = i0 + tile * 16 + r;
    const gu4* wr = job.row(row < i1 ? row : i0) + (size_t)part * (kl / (CB / 4)) + grp;
    const uint4* xr = xb + (size_t)part * (kl / 8) + XM * grp;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < kl / CB; kb += kMfmaBatch) {
      uint4 wa[kMfmaBatch];
#pragma unroll
      for (int u = 0; u < kMfmaBatch; ++u) wa[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(wr + 4 * (kb + u)));
#pragma unroll
      for (int u = 0; u < kMfmaBatch; ++u) {
#pragma unroll
        for (int j = 0; j < XM; ++j) {
          const uint4 xv = r < n ? xr[4 * XM * (kb + u) + j] : make_uint4(0, 0, 0, 0);
          uint4 av = wa[u];
#if MK_WFMT != 0
          if constexpr (WQ) av = q8_bf16(wa[u], j);
#endif
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                        __builtin_bit_cast(bf16x8_t, xv), acc, 0, 0, 0);
        }
      }
    }
    if (kp == 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rq = i0 + tile * 16 + 4 * grp + q;
        if (rq < i1 && r < n) job.emit(rq, r, scaled<WQ>(job, rq, acc[q]));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) red[it * 256 + (4 * grp + q) * 16 + r] = acc[q];
    }
  }
  if (kp > 1) {
    __syncthreads();
    for (int e = tid(); e < ntile * 256; e += kThreads) {
      const int tile = e >> 8, rt = (e >> 4) & 15, tok = e & 15;
      const int rq = i0 + tile * 16 + rt;
      float v = 0.f;
      for (int part = 0; part < kp; ++part) v += red[(tile * kp + part) * 256 + rt * 16 + tok];
      if (rq < i1 && tok < n) job.emit(rq, tok, scaled<WQ>(job, rq, v));
    }
    __syncthreads();
  }
}

// Rows [i0, i1) of a job with K-element rows; WQ: the rows are in the
// kernel's quantized format.
template <bool FromLds, bool WQ, class Job>
DEV void rowdots_range(int K, int i0, int i1, int maxnx, const Job& job) {
  const int nj = i1 - i0;
  if (nj <= 0 || maxnx <= 0) return;
  if constexpr (!FromLds && Job::kDense)
    if (maxnx >= 2 && K % (32 * (16 / row_bits<WQ>()) * kMfmaBatch) == 0)
      return rowdots_mfma<WQ>(K, i0, i1, maxnx, job, job.red);
  const int ch = K * row_bits<WQ>() / 128;  // 16-byte chunks per row
  if (nj <= 8 && ch == 512) return rowdots<64, 8, FromLds, WQ>(i0, i1, maxnx, job);
  if (nj <= 8 && ch == 256) return rowdots<64, 4, FromLds, WQ>(i0, i1, maxnx, job);
  if (nj <= 16 || ch > 256) {
    switch (ch) {
      case 64: return rowdots<32, 2, FromLds, WQ>(i0, i1, maxnx, job);
      case 96: return rowdots<32, 3, FromLds, WQ>(i0, i1, maxnx, job);
      case 128: return rowdots<32, 4, FromLds, WQ>(i0, i1, maxnx, job);
      case 256: return rowdots<32, 8, FromLds, WQ>(i0, i1, maxnx, job);
      case 512: return rowdots<32, 16, FromLds, WQ>(i0, i1, maxnx, job);
      default: break;
    }
  }
  switch (ch) {
    case 4:
      if constexpr (WQ && kWBits == 4) return rowdots<4, 1, FromLds, WQ>(i0, i1, maxnx, job);
      break;
    case 8:
      if constexpr (WQ) return rowdots<8, 1, FromLds, WQ>(i0, i1, maxnx, job);
      break;
    case 16: return rowdots<16, 1, FromLds, WQ>(i0, i1, maxnx, job);
    case 24:
      if constexpr (WQ && kWBits == 4) return rowdots<8, 3, FromLds, WQ>(i0, i1, maxnx, job);
      break;
    case 32: return rowdots<16, 2, FromLds, WQ>(i0, i1, maxnx, job);
    case 48:
      if constexpr (WQ) return rowdots<16, 3, FromLds, WQ>(i0, i1, maxnx, job);
      break;
    case 64: return rowdots<16, 4, FromLds, WQ>(i0, i1, maxnx, job);
    case 96: return rowdots<16, 6, FromLds, WQ>(i0, i1, maxnx, job);
    case 128: return rowdots<16, 8, FromLds, WQ>(i0, i1, maxnx, job);
    case 256: return rowdots<16, 16, FromLds, WQ>(i0, i1, maxnx, job);
    default: break;
  }
  rowdots_generic<FromLds, WQ>(K, i0, i1, maxnx, job);
}

// All rows of a job from HBM.
template <bool WQ, class Job>
DEV void run_rowdots(int K, int njobs, int maxnx, const Job& job) {
  rowdots_range<false, WQ>(K, 0, njobs, maxnx, job);
}

// Rows [0, npf) from the LDS tile, the rest from HBM.
template <bool WQ, class Job>
DEV void run_rowdots_pf(int K, int njobs, int npf, int maxnx, const Job& job) {
  rowdots_range<true, WQ>(K, 0, npf, maxnx, job);
  rowdots_range<false, WQ>(K, npf, njobs, maxnx, job);
}

// ---------------------------------------------------------------------------
// Router top-k: per token, the top_k logits ordered by (value desc, index
// asc), their softmax, the distinct experts in ascending order and, for each
// of them, the (token, slot) pairs routed to it.
//
// Wave b takes token b: it polls the token's epoch-tagged router logits
// (lanes hold experts lane and lane + 64) until every tag is this step's,
// then picks the winners in top_k rounds: the largest remaining key (an
// order-preserving 32-bit image of the logit, NaN ranking as -inf) by a
// wave-wide max, the lowest expert holding it by a ballot, which is removed
// before the next round.  Slot j is round j's winner.

// The order of (value, index) pairs used by every selection here: larger
// value first, then smaller index.
DEV bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

DEV uint32_t topk_key(float v) {
  const uint32_t u = __float_as_uint(v != v ? kNegInf : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Unsigned maximum over the wave, in every lane: DPP within 16-lane rows,
// then the gfx950 row swaps across rows and halves.
DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  v = max(v, dpp_u<0x140>(v));
  const auto t = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(t[0], t[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(h[0], h[1]);
}

// The calling wave polls token b's tagged router logits of `layer` until all
// carry this step's epoch (bounded like wait_counter); lanes get experts lane
// and lane + 64.  False when the grid is aborting or the wait timed out.
DEV bool poll_router(const KArgs& a, int layer, int b, int task, float& v0, float& v1) {
  const int lane = tid() & 63;
  const uint64_t* base = a.rll + ((size_t)layer * a.max_batch + b) * a.E;
  const bool h0 = lane < a.E, h1 = lane + 64 < a.E;
  const uint64_t t0 = wall_clock64();
  uint32_t it = 0;
  while (true) {
    const uint64_t w0 = h0 ? ld_tag(base + lane) : 0ull;
    const uint64_t w1 = h1 ? ld_tag(base + lane + 64) : 0ull;
    const bool ok = (!h0 || (uint32_t)(w0 >> 32) == a.epoch) && (!h1 || (uint32_t)(w1 >> 32) == a.epoch);
    if (__ballot(!ok) == 0ull) {
      v0 = __uint_as_float((uint32_t)w0);
      v1 = __uint_as_float((uint32_t)w1);
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
    if ((++it & 31) == 0) {
      int stop = 0;
      if (lane == 0) stop = aborting(a) ? 1 : (wall_clock64() - t0 > a.spin_limit_ticks ? 2 : 0);
      stop = __shfl(stop, 0);
      if (stop) {
        if (lane == 0 && stop == 2) raise_error(a, MK_ERR_DEVICE_TIMEOUT, task, -1);
        return false;
      }
    }
  }
}

// scratch: region C, per-expert token masks [kMaxExperts], then slots
// [kMaxBatch][kMaxExperts].  fail: an LDS word.  Returns false in every
// thread when a token's router logits never arrived (abort or time-out).
// With a trace, wave 0 records when its logits arrived as the task's ready time.
DEV bool compute_topk(const KArgs& a, int layer, TopK* tk, uint8_t* scratch, int task, int32_t* fail, int mk) {
  const int lane = tid() & 63, wave = tid() >> 6;
  const int E = a.E, K = a.topk, n = a.n;
  int32_t* emask = (int32_t*)scratch;
  uint8_t* eslot = scratch + 4 * kMaxExperts;
  for (int e = tid(); e < kMaxExperts; e += kThreads) emask[e] = 0;
  if (tid() == 0) *fail = 0;
  __syncthreads();
  if (wave < n) {
    const int b = wave;
    float v0, v1;
    if (!poll_router(a, layer, b, task, v0, v1)) {
      if (lane == 0) *fail = 1;
    } else {
      if (wave == 0 && lane == 0 && a.trace && task < a.trace_cap) a.trace[kTraceWords * (size_t)task + 1] = wall_clock64();
      v0 = v0 != v0 ? kNegInf : v0;
      v1 = v1 != v1 ? kNegInf : v1;
      uint32_t k0 = lane < E ? topk_key(v0) : 0u, k1 = lane + 64 < E ? topk_key(v1) : 0u;
      int ej = 0;
      float vj = 0.f;
      for (int j = 0; j < K; ++j) {
        // every valid key exceeds 0 (the image of -inf is 0x007fffff), so a removed or absent expert never wins
        const uint32_t m = wave_max_u32(max(k0, k1));
        const uint64_t b0 = __ballot(k0 == m), b1 = __ballot(k1 == m);
        const int e = b0 ? __ffsll((long long)b0) - 1 : 64 + __ffsll((long long)b1) - 1;
        const float ve = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e < 64 ? v0 : v1), e & 63));
        if (lane == j) {
          ej = e;
          vj = ve;
        }
        if (lane == (e & 63)) {
          if (e < 64) k0 = 0u;
          else k1 = 0u;
        }
      }
      // softmax in slot order, relative to the largest logit (slot 0's)
      const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vj), 0));
      const float ex = lane < K ? __expf(vj - vmax) : 0.f;
      float wsum = 0.f;
      for (int j = 0; j < K; ++j) wsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
      if (lane < K) {
        tk->sel[b][lane] = ej;
        tk->w[b][lane] = ex / wsum;
        eslot[b * kMaxExperts + ej] = (uint8_t)lane;
        atomicOr(emask + ej, 1 << b);
      }
      if (mk >= 0 && wave == 0) mark(a, task, mk);
    }
  }
  __syncthreads();
  if (*fail) return false;
  if (wave == 0) {
    // distinct experts in ascending order (lane e and e + 64), each with its
    // tokens in ascending order as pairs b * top_k + slot
    const int m_lo = emask[lane], m_hi = emask[lane + 64];
    const uint64_t b0 = __ballot(m_lo != 0), b1 = __ballot(m_hi != 0);
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int c0 = __popcll(b0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = h ? m_hi : m_lo, e = lane + 64 * h;
      if (m) {
        const int u = h ? c0 + __popcll(b1 & below) : __popcll(b0 & below);
        tk->U[u] = e;
        tk->ntok[u] = __popc(m);
        int t = 0;
        for (int bb = 0; bb < n; ++bb)
          if ((m >> bb) & 1) tk->pair[u][t++] = bb * K + eslot[bb * kMaxExperts + e];
      }
    }
    // the most tokens any selected expert has (at most kMaxBatch): one ballot per count
    const int myt = max(__popc(m_lo), __popc(m_hi));
    int mytok = 0;
#pragma unroll
    for (int k = 1; k <= kMaxBatch; ++k)
      if (__ballot(myt >= k) != 0ull) mytok = k;
    if (lane == 0) {
      tk->nU = c0 + __popcll(b1);
      tk->maxtok = mytok;
    }
  }
  __syncthreads();
  return true;
}

// The experts chosen per token, reported to the caller (written by one task per layer).
DEV void write_sel(const KArgs& a, int layer, const TopK* tk) {
  if (tid() < a.n * a.topk)
    a.sel_out[(size_t)layer * a.max_batch * a.topk + tid()] = tk->sel[tid() / a.topk][tid() % a.topk];
}

// ---------------------------------------------------------------------------
// PRE: RMSNorm + rows [r0, r1) of the stacked [Wq; Wk; Wv; Wr] matrix.

// Immutable weight tiles are prefetched into LDS before the task waits for
// its inputs (the pages' third-ranked gain: weights start streaming before
// dependencies resolve).  Rows [0, npf) of a job's matrix are then read from
// LDS, the rest from HBM.
// Waves 1..7 issue the copies with the LDS copy engine (asynchronous: the
// waves go on at once, the data lands while the task waits): wave 0, whose thread 0 polls the flags right
// after, keeps its load queue short (a wave's loads complete in order).
// Each of waves 1..7 copies one contiguous run of 1 KB chunks: measured on
// this part, that runs at about 2.5x the rate of dealing the chunks to the
// waves round robin.
DEV void prefetch_to_lds(const gu8* src, uint8_t* dst_lds, int nbytes) {
  const int lane = tid() & 63, wave = tid() >> 6;
  const AS_GLOBAL uint8_t* s8 = (const AS_GLOBAL uint8_t*)src;
  const int nchunk = (nbytes + 1023) >> 10;
  const int per = (nchunk + kWaves - 2) / (kWaves - 1);
  const int c0 = (wave - 1) * per, c1 = min(c0 + per, nchunk);
  for (int c = c0; wave > 0 && c < c1; ++c) {
    const int off = (c << 10) + (lane << 4);
    if (off < nbytes)
      __builtin_amdgcn_global_load_lds((AS_GLOBAL void*)(s8 + off), (AS_LDS void*)(dst_lds + (c << 10)), 16, 0, kStreamPolicy);
  }
}


// Work a task can do before its inputs are ready: the first weight tile of
// PRE and WO tasks (rows [r0, r1) of Wqkv / router / Wo) starts streaming
// into LDS, from tile_off bytes into region C to the end (at batch 1
// nothing below the end of LDS from there is live across this point: an
// output task keeps only its expert contributions, below tile_off).  A PRE
// task that follows an output task finds its tile already copied by it.
// Returns the rows in LDS.
// The first rows of a PRE task (Wqkv rows in the kernel's weight format,
// router rows bf16): start and bytes per row.
DEV const gu8* pre_rows_src(const KArgs& a, int layer, int r0, int* rowb) {
  if (r0 < a.qkv_rows) {
    *rowb = wrow_bytes(a.H);
    return wbytes(a, widx(layer, WL_QKV)) + (size_t)r0 * *rowb;
  }
  *rowb = a.H * 2;
  return wbytes(a, widx(layer, WL_ROUTER)) + (size_t)(r0 - a.qkv_rows) * *rowb;
}

DEV int task_prefetch(const KArgs& a, const Task& t, const Lds& s, int qi) {
  const gu8* src;
  int rowb, nrows = t.r1 - t.r0;
  if (t.op == OP_PRE) {
    src = pre_rows_src(a, t.layer, t.r0, &rowb);
  } else if (t.op == OP_WO) {
    rowb = wrow_bytes(a.nq * a.d);
    src = wbytes(a, widx(t.layer, WL_O)) + (size_t)t.r0 * rowb;
  } else {
    return 0;
  }
  // (with several tokens the rows go to the matrix cores straight from HBM)
  const int npf = a.n == 1 ? min(nrows, a.pf_wide / rowb) : 0;
  // flags[18] = layer + 1 of a PRE tile the preceding output task has already copied
  if (npf > 0 && !(t.op == OP_PRE && s.flags[18] == t.layer + 1)) prefetch_to_lds(src, s.C + a.tile_off, npf * rowb);
  return npf;
}

// Makes every wave's prefetched tile visible to the whole workgroup.
DEV void prefetch_wait() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

struct JobPre {
  static constexpr bool kDense = true;  // every row is dotted with every token
  const gu8* W;                     // the matrix (bytes)
  const AS_GLOBAL float* sc = nullptr;  // FP8 rows: the matrix's row scales
  const AS_LDS uint8_t* pf;         // prefetched rows [0, npf)
  float* red;                       // LDS for the matrix-core path's partial tiles (region C)
  int npf;
  int r0, K, rowb;                  // rowb: bytes per row (K * 2, or K for FP8 rows)
  const uint16_t* xs;
  float* out;  // [b][ld] + r0 already applied
  int ld;
  uint64_t* tag_out = nullptr;  // router rows: the same values as epoch-tagged words ([b][ld] + r0 applied)
  uint32_t epoch = 0;
  DEV const gu4* row(int i) const { return (const gu4*)(W + (size_t)(r0 + i) * rowb); }
  DEV const lu4* lrow(int i) const { return (const lu4*)(pf + (size_t)i * rowb); }
  DEV float scale(int i) const { return sc[r0 + i]; }
  DEV int nx(int) const { return 1 << 30; }
  DEV const uint4* x(int, int t) const { return (const uint4*)(xs + (size_t)t * K); }
  DEV void emit(int i, int t, float v) const {
    st_coh(out + (size_t)t * ld + i, v);
    if (tag_out) st_tag(tag_out + (size_t)t * ld + i, v, epoch);
  }
};

TASK void task_pre(const KArgs& a, const Task& t, const Lds& s, int qi, int npf) {
  const int l = t.layer;
  uint16_t* xs = (uint16_t*)s.A;
  // sequential block: the Wqkv rows read the attention side's norm, the router rows the MoE path's
  const bool moe_side = kSeq && t.r0 >= a.qkv_rows;
  norm_inputs(a, l, moe_side ? moe_gain(a, l) : wptr(a, widx(l, WL_NORM)), xs, s.red8, qi, 0, nullptr,
              kSeq ? (moe_side ? kWithWo : kAlone) : kParallel);
  prefetch_wait();
  mark(a, qi, 1);
  JobPre j;
  j.K = a.H;
  j.xs = xs;
  j.pf = (const AS_LDS uint8_t*)(s.C + a.tile_off);
  j.npf = npf;
  j.red = (float*)s.C;
  if (t.r0 < a.qkv_rows) {
    j.W = wbytes(a, widx(l, WL_QKV));
    j.rowb = wrow_bytes(a.H);
    if constexpr (kWQ) j.sc = wscales(a, widx(l, WL_QKV), a.qkv_rows, a.H);
    j.r0 = t.r0;
    j.out = a.qkv + (size_t)l * a.max_batch * a.qkv_rows + t.r0;
    j.ld = a.qkv_rows;
  } else {
    j.W = wbytes(a, widx(l, WL_ROUTER));
    j.rowb = a.H * 2;
    j.r0 = t.r0 - a.qkv_rows;
    j.out = a.rlog + (size_t)l * a.max_batch * a.E + j.r0;
    j.tag_out = a.rll + (size_t)l * a.max_batch * a.E + j.r0;
    j.epoch = a.epoch;
    j.ld = a.E;
  }
  // Wqkv rows in the kernel's weight format, router rows always bf16
  if (t.r0 < a.qkv_rows) run_rowdots_pf<kWQ>(a.H, t.r1 - t.r0, npf, a.n, j);
  else run_rowdots_pf<false>(a.H, t.r1 - t.r0, npf, a.n, j);
  mark(a, qi, 2);
}

// ---------------------------------------------------------------------------
// ATTN: one chunk [t0, t1) of the positions of (sequence b, kv head g).
//
// Per page of 16 positions a wave runs two MFMA contractions:
//   S^T[16 pos][16 heads] = K[16 pos][d] * Q^T[d][16 heads]   (v_mfma_f32_16x16x32_bf16,
//     the group's q heads padded to 16 with zero rows), so lane l holds the
//     scores of positions 4*(l/16)..+3 for head l%16;
//   O^T[d][16 heads] += V^T[d][16 pos] * P^T[16 pos][16 heads] (v_mfma_f32_16x16x16_bf16,
//     d/16 tiles), where the probabilities above are already in the B-operand
//     layout (column = head l%16, k = positions 4*(l/16)..+3), and lane l's
//     output column is head l%16 too, so the online softmax rescales each lane
//     by its own factor (no cross-lane exchange).
// The A operand of the second product needs 4 consecutive positions of one
// dim per lane, which is why V pages are stored dims-major.  Softmax is online
// per page (running max and sum per head, O columns rescaled), in fp32; the
// probabilities enter the MFMA as a bf16 pair (high part + remainder), so the
// P*V product is as accurate as the fp32 sum it is divided by.  K/V of the
// next page are loaded while the current one is processed.

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef short short4_v __attribute__((ext_vector_type(4)));
typedef float float4_v __attribute__((ext_vector_type(4)));

// One rotated pair (i, i + d/2) of a head at angle (cos cf, sin sf), each half rounded to bf16.
DEV void rope_pair(float x0, float x1, float cf, float sf, uint16_t& lo, uint16_t& hi) {
  lo = f2bf(x0 * cf - x1 * sf);
  hi = f2bf(x0 * sf + x1 * cf);
}

template <int D>
struct AttnPage {
  uint4 k[D / 32];  // lane l: K[pos l%16][32c + 8*(l/16) .. +7]
  uint2 v[D / 16];  // lane l: V[pos 4*(l/16) .. +3][dim 16t + l%16]
  int nvalid;       // positions of the page inside the chunk
};

// The last nl blocks of a chunk, [bl0, bl0 + nl), are copied into LDS region
// P before the task waits for q (K/V of earlier positions never change during a step; the block that
// receives the new token is patched after the wait):
// K blocks [nl][16][D], then V blocks [nl][D][16].  In a K block the 16-byte
// pieces of position r are stored XOR-swizzled by r, so the 16 positions a
// wave reads at one dim offset sit in different banks.
template <int D>
DEV int kslot(int r, int cc) {
  constexpr int NC = D / 8;  // 16-byte pieces per K row
  return r * NC + (cc ^ (r & (NC - 1)));
}

template <int D>
DEV int attn_lds_pages(const KArgs& a, int nblk) {
  return min(min(nblk, kMaxLdsPages), a.pf_bytes / (2 * 16 * D * 2));
}

// Waves 1..7 issue the copies (wave 0, whose thread 0 polls the counters,
// keeps its load queue short); wave 0 records which of the blocks' pages are
// valid and raises the error for the others.
template <int D>
DEV void attn_prefetch(const KArgs& a, const Lds& s, int qi, int l, int b, int g, int t0, int bl0, int nl) {
  constexpr int NI = 16 * D * 2 / 1024;  // 1 KB copies per K (or V) block
  const int lane = tid() & 63, wave = tid() >> 6;
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages + t0 / 16 + bl0;
  // one contiguous run of copies per wave (see prefetch_to_lds)
  const int nq = nl * 2 * NI, per = (nq + kWaves - 2) / (kWaves - 1);
  const int q0 = (wave - 1) * per, q1 = min(q0 + per, nq);
  for (int q = q0; wave > 0 && q < q1; ++q) {
    const int pi = q / (2 * NI), isv = (q / NI) & 1, k = q % NI;
    const int page = pt[pi];
    if (page < 0 || page >= a.num_pages) continue;
    const size_t boff = (((size_t)l * a.num_pages + page) * a.nkv + g) * (size_t)16 * D;
    const int slot = 64 * k + lane;
    const int piece = isv ? slot : kslot<D>(slot / (D / 8), slot % (D / 8));  // the swizzle is its own inverse
    const uint16_t* src = (isv ? a.v_pool : a.k_pool) + boff + (size_t)piece * 8;
    uint8_t* dst = s.P + (isv ? (size_t)nl * 16 * D * 2 : 0) + (size_t)pi * 16 * D * 2 + k * 1024;
    __builtin_amdgcn_global_load_lds((AS_GLOBAL void*)src, (AS_LDS void*)dst, 16, 0, kStreamPolicy);
  }
  if (wave == 0) {
    // lane pi checks page pi; one load per lane, one ballot
    const int page = lane < nl ? pt[lane] : 0;
    const bool ok = lane < nl && page >= 0 && page < a.num_pages;
    if (lane < nl && !ok) raise_error(a, MK_ERR_DEVICE_PAGE, qi, page);
    const uint64_t m = __ballot(ok);
    if (lane == 0) {
      s.flags[14] = (int32_t)(uint32_t)m;
      s.flags[15] = (int32_t)(uint32_t)(m >> 32);
    }
  }
}

template <int D>
DEV void attn_fetch(const KArgs& a, AttnPage<D>& P, int l, int b, int g, int tb, int t1, int qi) {
  const int lane = tid() & 63, r = lane & 15, grp = lane >> 4;
  const int page = a.page_table[(size_t)b * a.max_pages + tb / a.ps];
  const bool pg_ok = page >= 0 && page < a.num_pages;
  if (!pg_ok && lane == 0) raise_error(a, MK_ERR_DEVICE_PAGE, qi, page);
  P.nvalid = pg_ok ? min(16, t1 - tb) : 0;
  const size_t boff = (((size_t)l * a.num_pages + (pg_ok ? page : 0)) * a.nkv + g) * (size_t)16 * D;
  const uint16_t* kb = a.k_pool + boff;
  const uint16_t* vb = a.v_pool + boff;
  const bool krow = r < P.nvalid, vcol = 4 * grp < P.nvalid;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    P.k[c] = krow ? __builtin_bit_cast(uint4, __builtin_nontemporal_load((const AS_GLOBAL u32x4_v*)(kb + r * D + 32 * c + 8 * grp))) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    P.v[t] = vcol ? __builtin_bit_cast(uint2, __builtin_nontemporal_load((const AS_GLOBAL uint64_t*)(vb + (16 * t + r) * 16 + 4 * grp))) : make_uint2(0, 0);
}

typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));

// Page pi of the chunk from its LDS copy.
template <int D>
DEV void attn_fetch_lds(const Lds& s, AttnPage<D>& P, int npp, int pi, int tb, int t1) {
  const int lane = tid() & 63, r = lane & 15, grp = lane >> 4;
  const uint32_t mask = (uint32_t)s.flags[pi < 32 ? 14 : 15];
  P.nvalid = ((mask >> (pi & 31)) & 1u) ? min(16, t1 - tb) : 0;
  const AS_LDS uint8_t* kb = (const AS_LDS uint8_t*)s.P + (size_t)pi * 16 * D * 2;
  const AS_LDS uint8_t* vb = (const AS_LDS uint8_t*)s.P + (size_t)(npp + pi) * 16 * D * 2;
  const bool krow = r < P.nvalid, vcol = 4 * grp < P.nvalid;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    P.k[c] = __builtin_bit_cast(uint4, krow ? *(const lu4*)(kb + 16 * kslot<D>(r, 4 * c + grp)) : u32x4_v{0, 0, 0, 0});
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    P.v[t] = __builtin_bit_cast(
        uint2, vcol ? *(const AS_LDS u32x2_v*)(vb + 2 * ((16 * t + r) * 16 + 4 * grp)) : u32x2_v{0, 0});
}

// Max / sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48), every lane getting the result, through the gfx950 row-swap
// instructions: with both operands the same register, permlane16_swap returns
// (even row, odd row) of each row pair in every lane, permlane32_swap (lower
// half, upper half); no LDS round trip as with a shuffle.
DEV float rows4_max(float v) {
  const uint32_t u = __float_as_uint(v);
  auto t = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float w = fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
  const uint32_t uw = __float_as_uint(w);
  auto h = __builtin_amdgcn_permlane32_swap(uw, uw, false, false);
  return fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
}

DEV float rows4_sum(float v) { return xrow32_sum(xrow16_sum(v)); }

template <int D>
DEV void attn_page(const AttnPage<D>& P, const bf16x8_v (&qb)[D / 32], float scale, float& m, float& lsum,
                   float4_v (&o)[D / 16]) {
  const int lane = tid() & 63, grp = lane >> 4;
  float4_v sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, P.k[c]), qb[c], sacc, 0, 0, 0);
  float sv[4];
  float bm = kNegInf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = (4 * grp + i < P.nvalid) ? sacc[i] * scale : kNegInf;  // select: poison slots never enter
    bm = fmaxf(bm, sv[i]);
  }
  bm = rows4_max(bm);
  const float mn = fmaxf(m, bm);
  const float alpha = mn == kNegInf ? 1.f : __expf(m - mn);
  float pf[4];
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pf[i] = sv[i] == kNegInf ? 0.f : __expf(sv[i] - mn);
    ps += pf[i];
  }
  // p = p_hi + p_lo, both bf16: two matrix-core products keep P*V at ~2^-16 relative
  const uint32_t h01 = pack_bf16(pf[0], pf[1]), h23 = pack_bf16(pf[2], pf[3]);
  const uint32_t l01 = pack_bf16(pf[0] - bf2f(h01 & 0xffffu), pf[1] - bf2f(h01 >> 16));
  const uint32_t l23 = pack_bf16(pf[2] - bf2f(h23 & 0xffffu), pf[3] - bf2f(h23 >> 16));
  const short4_v pa = __builtin_bit_cast(short4_v, make_uint2(h01, h23));
  const short4_v pl = __builtin_bit_cast(short4_v, make_uint2(l01, l23));
  lsum = lsum * alpha + ps;
  m = mn;
  // O^T[dim][head] = V^T P^T: the lane's column is its own head, so its
  // rescale factor is its own alpha
#pragma unroll
  for (int t = 0; t < D / 16; ++t) o[t] *= alpha;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    short4_v vb4;
    const uint2 vv = P.v[t];
    vb4[0] = (4 * grp + 0 < P.nvalid) ? (short)(vv.x & 0xffffu) : (short)0;
    vb4[1] = (4 * grp + 1 < P.nvalid) ? (short)(vv.x >> 16) : (short)0;
    vb4[2] = (4 * grp + 2 < P.nvalid) ? (short)(vv.y & 0xffffu) : (short)0;
    vb4[3] = (4 * grp + 3 < P.nvalid) ? (short)(vv.y >> 16) : (short)0;
    o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb4, pa, o[t], 0, 0, 0);
    o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb4, pl, o[t], 0, 0, 0);
  }
}

// Per-wave results of a chunk in region C: outputs [wave][G][d], maxima and
// sums [wave][kMaxGroup].
struct AttnMerge {
  float* o;
  float* m;
  float* l;
};

DEV AttnMerge attn_merge_area(const Lds& s, int G, int d) {
  AttnMerge r;
  r.o = (float*)s.C;
  r.m = r.o + (size_t)kWaves * G * d;
  r.l = r.m + kWaves * kMaxGroup;
  return r;
}

// This wave's pages of the chunk: its early blocks, already in ring[0] and
// ring[1] (waves 1..7: blocks wave - 1 and wave + 6, of [0, ne)), then the
// LDS blocks [bl0, nblk) and HBM blocks [ne, bl0) congruent to the wave mod
// 8.  The pages go through a ring of kAttnRing page registers: while page j
// is processed, pages j + 1 .. j + kAttnDepth are being fetched (a long
// chunk streams most of its pages from HBM this way).  Leaves (o, m, sum)
// per head in the merge area.
constexpr int kAttnDepth = 2, kAttnRing = kAttnDepth + 1;

template <int D>
DEV void attn_wave(const KArgs& a, const Lds& s, int qi, const uint16_t* q_s, int l, int b, int g, int t0, int t1,
                   int ne, int bl0, int nl, AttnPage<D> (&ring)[kAttnRing], const AttnMerge& mrg) {
  const int lane = tid() & 63, wave = tid() >> 6, r = lane & 15, grp = lane >> 4;
  const int G = a.group;
  bf16x8_v qb[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const uint4 qv = r < G ? *(const uint4*)(q_s + r * D + 32 * c + 8 * grp) : make_uint4(0, 0, 0, 0);
    qb[c] = __builtin_bit_cast(bf16x8_v, qv);
  }
  const float scale = 1.0f / sqrtf((float)D);
  float m = kNegInf, lsum = 0.f;
  float4_v o[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) o[t] = float4_v{0.f, 0.f, 0.f, 0.f};
  // this wave's pages in order: its early blocks (registers), its LDS blocks,
  // its HBM blocks; one call site processes them all (the code runs once per
  // layer: fewer copies, fewer instruction fetches)
  const int nblk = (t1 - t0 + 15) / 16;
  const int n_e = (wave >= 1 && wave - 1 < ne) + (wave >= 1 && wave + kWaves - 2 < ne);
  const int l0 = bl0 + (wave - bl0 % kWaves + kWaves) % kWaves;  // first LDS block of the wave
  const int n_l = l0 < nblk ? (nblk - l0 + kWaves - 1) / kWaves : 0;
  const int h0 = ne + (wave - ne % kWaves + kWaves) % kWaves;    // first HBM block of the wave
  const int n_h = h0 < bl0 ? (bl0 - h0 + kWaves - 1) / kWaves : 0;
  const int total = n_e + n_l + n_h;
  // pages [0, n_e) are in ring[0 .. n_e) already (n_e <= 2 <= kAttnDepth)
  auto fetch = [&](int jn, AttnPage<D>& dst) {
    if (jn < n_e + n_l) {
      const int blk = l0 + kWaves * (jn - n_e);
      attn_fetch_lds<D>(s, dst, nl, blk - bl0, t0 + 16 * blk, t1);
    } else {
      const int blk = h0 + kWaves * (jn - n_e - n_l);
      attn_fetch<D>(a, dst, l, b, g, t0 + 16 * blk, t1, qi);
    }
  };
#pragma unroll
  for (int k = 0; k < kAttnDepth; ++k)
    if (k >= n_e && k < total) fetch(k, ring[k]);
  for (int j0 = 0; j0 < total; j0 += kAttnRing) {
#pragma unroll
    for (int k = 0; k < kAttnRing; ++k) {
      const int j = j0 + k;
      if (j < total) {
        if (j + kAttnDepth < total) fetch(j + kAttnDepth, ring[(k + kAttnDepth) % kAttnRing]);
        attn_page<D>(ring[k], qb, scale, m, lsum, o);
      }
    }
  }
  // per-head totals over the 4 lane groups, then this wave's part of the merge area
  lsum = rows4_sum(lsum);
  if (grp == 0 && r < G) {
    mrg.m[wave * kMaxGroup + r] = m;
    mrg.l[wave * kMaxGroup + r] = lsum;
  }
  // lane (r, grp) holds O^T[16 t + 4 grp + i][head r]
  if (r < G) {
    float* row = mrg.o + ((size_t)wave * G + r) * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) *(float4_v*)(row + 16 * t + 4 * grp) = o[t];
  }
}

// The chunk of split task t.idx, from the step's sequence lengths only, so it
// runs before the task's wait; thread 0 writes it to plan = flags[2..9] and
// its chunk number to flags[17].
DEV void attn_plan(const KArgs& a, const Task& t, const Lds& s, int qi) {
  int32_t* plan = s.flags + 2;  // b, g, t0, t1, first, nch, ok, p; [15]: chunk number
  if (tid() == 0) {
    int32_t lens1[kMaxBatch];
    const int cap = a.max_pages * a.ps;
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      int p = b < a.n ? a.seq_lens[b] + a.step : 0;
      if (b < a.n && (p < 0 || p + 1 > cap)) {
        raise_error(a, MK_ERR_DEVICE_SEQ, qi, b);
        p = p < 0 ? 0 : cap - 1;
      }
      lens1[b] = p + 1;
    }
    const int nlead = a.max_batch * a.nkv;
    const int64_t C = attn_chunk_len(lens1, a.n, a.nkv, a.n_attn - nlead + a.n * a.nkv, a.ps);
    int b = 0, g = 0, t0 = 0, t1 = 0, first = 0, nch = 0, ch = 0;
    const bool ok = attn_task_chunk(lens1, a.n, a.nkv, C, t.idx, nlead, &b, &g, &t0, &t1, &first, &nch, &ch);
    plan[0] = b; plan[1] = g; plan[2] = t0; plan[3] = t1; plan[4] = first; plan[5] = nch; plan[6] = ok;
    plan[7] = lens1[ok ? b : 0] - 1;
    plan[15] = ch;
  }
}

// The lead of segment (b, g) merges all chunks j of the segment:
//   o_h = sum_j e^(m_jh - M_h) o_jh / sum_j e^(m_jh - M_h) l_jh,  M_h = max_j m_jh.
// Thread (slice sl, float4 f) takes chunks sl, sl + S, ...; slices are summed
// in a fixed order.  Every partial is read with 16-byte coherent loads, the
// chunks' maxima and sums first (through LDS), the outputs in batches of R
// loads in flight before any is used.
DEV void attn_combine(const KArgs& a, const Lds& s, const float* parts, int nch, uint16_t* out) {
  const int G = a.group, d = a.d, GD = G * d, CS = attn_part_stride(G, d);
  const int nf4 = GD / 4, S = kThreads / nf4;
  const int sl = tid() / nf4, f = tid() - sl * nf4;
  const bool act = sl < S;
  const int hh = 4 * f / d;
  const uint32_t nbytes = (uint32_t)nch * CS * 4;
  float* mj = (float*)s.C;                                                 // [nch][kMaxGroup]
  float* lj = mj + (size_t)nch * kMaxGroup;                                // [nch][kMaxGroup]
  float4* red = (float4*)(s.C + ((2 * (size_t)nch * kMaxGroup * 4 + 15) & ~(size_t)15));  // [kThreads]
  // the maxima and sums: 4 float4 per chunk (G <= kMaxGroup = 8 each)
  for (int q = tid(); q < 4 * nch; q += kThreads) {
    const int j = q >> 2, k = q & 3;
    const u32x4_v v = ld_coh16(parts, nbytes, (uint32_t)(j * CS + GD + 4 * k) * 4);
    *(u32x4_v*)((k < 2 ? mj : lj) + j * kMaxGroup + 4 * (k & 1)) = v;
  }
  constexpr int R = 8;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  u32x4_v v[R];
  auto load = [&](int k0) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int j = sl + S * (k0 + k);
      v[k] = (act && j < nch) ? ld_coh16(parts, nbytes, (uint32_t)(j * CS + 4 * f) * 4) : u32x4_v{0, 0, 0, 0};
    }
  };
  load(0);
  __syncthreads();
  float M = kNegInf, Ls = 0.f;
  for (int j = 0; j < nch; ++j) M = fmaxf(M, mj[j * kMaxGroup + hh]);
  for (int j = 0; j < nch; ++j) Ls += lj[j * kMaxGroup + hh] * __expf(mj[j * kMaxGroup + hh] - M);
  for (int k0 = 0;; k0 += R) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int j = sl + S * (k0 + k);
      if (act && j < nch) {
        const float sc = __expf(mj[j * kMaxGroup + hh] - M);
        acc.x += __uint_as_float(v[k][0]) * sc;
        acc.y += __uint_as_float(v[k][1]) * sc;
        acc.z += __uint_as_float(v[k][2]) * sc;
        acc.w += __uint_as_float(v[k][3]) * sc;
      }
    }
    if (sl + S * (k0 + R) >= nch) break;
    load(k0 + R);
  }
  red[tid()] = acc;
  __syncthreads();
  if (tid() < nf4) {
    float4 o = red[f];
    for (int k = 1; k < S; ++k) {
      const float4 w = red[k * nf4 + f];
      o.x += w.x;
      o.y += w.y;
      o.z += w.z;
      o.w += w.w;
    }
    st_coh((uint32_t*)(out + 4 * f), pack_bf16(o.x / Ls, o.y / Ls));
    st_coh((uint32_t*)(out + 4 * f + 2), pack_bf16(o.z / Ls, o.w / Ls));
  }
}

// Attention waits for its inputs itself: before the wait it works out its
// chunk (once per launch), starts the LDS copies of the chunk's last blocks
// and loads its first blocks into registers, so little of the chunk's K/V
// traffic is left once q is ready.
template <int D>
DEV void attn_task(const KArgs& a, const Task& t, const Lds& s, int qi) {
  // flags[16] (the split task whose plan flags[2..9] holds) was last written
  // before an earlier barrier, so every thread takes the same branch
  if (s.flags[16] != t.idx) {
    attn_plan(a, t, s, qi);
    __syncthreads();
    // the rotation of the chunk's sequence at its position p (fixed for the
    // launch): angles in double, cos / sin rounded to float
    if (tid() < D / 2) {
      double sd, cd;
      sincos((double)s.flags[2 + 7] * a.inv_freq[tid()], &sd, &cd);
      s.rot[tid()] = (float)cd;
      s.rot[64 + tid()] = (float)sd;
    }
    __syncthreads();
    if (tid() == 0) s.flags[16] = t.idx;
  }
  const int32_t* plan = s.flags + 2;
  if (!plan[6]) {  // idle split task
    if (a.trace && tid() == 0 && qi < a.trace_cap) a.trace[kTraceWords * (size_t)qi + 1] = wall_clock64();
    return;
  }
  const int l = t.layer, G = a.group, ps = a.ps;
  const int b = plan[0], g = plan[1], t0 = plan[2], t1 = plan[3], first = plan[4], nch = plan[5], p = plan[7];
  const int nblk = (t1 - t0 + 15) / 16;
  // a mixed step reads no page before every entry's new K/V is in (they may
  // share a sequence): no LDS copies or early blocks then
  const int nl = a.kv_sync ? 0 : attn_lds_pages<D>(a, nblk);
  const int bl0 = nblk - nl;
  // early blocks never include the last one (it receives the new token); wave
  // 0, whose thread 0 polls the flags, loads none
  const int ne = a.kv_sync ? 0 : max(0, min(bl0 - (nl == 0 ? 1 : 0), 2 * (kWaves - 1)));
  attn_prefetch<D>(a, s, qi, l, b, g, t0, bl0, nl);
  const int wave = tid() >> 6;
  AttnPage<D> ring[kAttnRing];
  if (wave >= 1 && wave - 1 < ne) attn_fetch<D>(a, ring[0], l, b, g, t0 + 16 * (wave - 1), t1, qi);
  if (wave >= 1 && wave + kWaves - 2 < ne) attn_fetch<D>(a, ring[1], l, b, g, t0 + 16 * (wave + kWaves - 2), t1, qi);
  // the chunk holding position p writes the new token's K (rotated) and V, to
  // HBM and, when its block was copied, to the LDS copy as well
  const bool mine = t1 == p + 1;
  const int page = mine ? a.page_table[(size_t)b * a.max_pages + p / ps] : 0;
  const bool pg_ok = page >= 0 && page < a.num_pages;
  if (mine && !pg_ok && tid() == 0) raise_error(a, MK_ERR_DEVICE_PAGE, qi, page);
  const bool put = mine && pg_ok && !a.kv_sync;  // (a mixed step's KVW tasks wrote it)
  const size_t koff = ((((size_t)l * a.num_pages + page) * a.nkv + g) * ps + p % ps) * D;
  constexpr int half = D / 2;
  const int nrot = (G + (put ? 1 : 0)) * half;  // pairs: q heads, then (put) the new k
  if (!wait_counter(a, t.wait[0], t.fanin[0], qi, s.flags + 0)) return;
  if (a.kv_sync && !wait_counter(a, t.wait[1], t.fanin[1], qi, s.flags + 0)) return;
  if (a.trace && tid() == 0 && qi < a.trace_cap) a.trace[kTraceWords * (size_t)qi + 1] = wall_clock64();
  // q of the group's heads, the new k and v (all loads in flight before any use)
  const float* qkv = a.qkv + ((size_t)l * a.max_batch + b) * a.qkv_rows;
  float x0[2] = {0.f, 0.f}, x1[2] = {0.f, 0.f}, vval = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = tid() + k * kThreads;
    if (e < nrot) {
      const int hh = e / half, i = e % half;
      const float* src = qkv + (hh < G ? (size_t)(g * G + hh) * D : (size_t)a.nq * D + (size_t)g * D);
      x0[k] = ld_coh(src + i);
      x1[k] = ld_coh(src + i + half);
    }
  }
  if (put && tid() < D) vval = ld_coh(qkv + (size_t)(a.nq + a.nkv) * D + (size_t)g * D + tid());

  // rotated q heads, and (put) the new k as head G, bf16 in region A
  uint16_t* q_s = (uint16_t*)s.A;  // [G + 1][D]
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = tid() + k * kThreads;
    if (e < nrot) {
      const int hh = e / half, i = e % half;
      uint16_t lo, hi;
      rope_pair(x0[k], x1[k], s.rot[i], s.rot[64 + i], lo, hi);
      q_s[hh * D + i] = lo;
      q_s[hh * D + i + half] = hi;
      if (hh == G) {
        a.k_pool[koff + i] = lo;
        a.k_pool[koff + i + half] = hi;
      }
    }
  }
  // V pages are stored dims-major: element (dim, slot) of a (page, head) block at dim*page_size + slot
  uint16_t v_i = 0;  // thread i < D: V dim i
  if (put && tid() < D) {
    const size_t voff = (((size_t)l * a.num_pages + page) * a.nkv + g) * (size_t)ps * D + p % ps;
    v_i = f2bf(vval);
    a.v_pool[voff + (size_t)tid() * ps] = v_i;
  }
  mark(a, qi, 0);
  // copied blocks have landed, q is complete, the new K/V are in HBM
  __builtin_amdgcn_s_waitcnt(0);
  __threadfence_block();
  __syncthreads();
  const int pp = (p - t0) / 16;
  if (put && pp >= bl0 && tid() < D) {
    const int i = tid(), r = p % 16;
    uint16_t* kb = (uint16_t*)(s.P + (size_t)(pp - bl0) * 16 * D * 2);
    uint16_t* vb = (uint16_t*)(s.P + (size_t)(nl + pp - bl0) * 16 * D * 2);
    kb[8 * kslot<D>(r, i / 8) + i % 8] = q_s[G * D + i];
    vb[i * 16 + r] = v_i;
  }
  __syncthreads();
  mark(a, qi, 1);

  // positions of the chunk, 16 (one page) at a time, pages dealt to waves round robin
  const AttnMerge mrg = attn_merge_area(s, G, D);
  attn_wave<D>(a, s, qi, q_s, l, b, g, t0, t1, ne, bl0, nl, ring, mrg);
  mark(a, qi, 2);
  __syncthreads();
  // this chunk's partial: the waves' results merged, as [G][D] outputs, G maxima, G sums
  const int GD = G * D, CS = attn_part_stride(G, D);
  const int chunk = plan[15];
  float* part = a.attn_part + ((size_t)l * a.n_attn + chunk) * CS;
  for (int e4 = tid(); e4 < GD / 4; e4 += kThreads) {
    const int hh = 4 * e4 / D;
    float M = kNegInf;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrg.m[w * kMaxGroup + hh]);
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    float Ls = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float mw = mrg.m[w * kMaxGroup + hh];
      const float sc = mw == kNegInf ? 0.f : __expf(mw - M);
      const float4 ow = *(const float4*)(mrg.o + (size_t)w * GD + 4 * e4);
      O.x += ow.x * sc;
      O.y += ow.y * sc;
      O.z += ow.z * sc;
      O.w += ow.w * sc;
      Ls += mrg.l[w * kMaxGroup + hh] * sc;
    }
    st_coh(part + 4 * e4, O.x);
    st_coh(part + 4 * e4 + 1, O.y);
    st_coh(part + 4 * e4 + 2, O.z);
    st_coh(part + 4 * e4 + 3, O.w);
    if ((4 * e4) % D == 0) {
      st_coh(part + GD + hh, M);
      st_coh(part + GD + kMaxGroup + hh, Ls);
    }
  }
  uint32_t* ticket = a.tickets + ((size_t)l * a.max_batch + b) * a.nkv + g;
  mark(a, qi, 3);
  if (t.idx >= a.max_batch * a.nkv) {
    // one of the other chunks: report to the segment's ticket (the partial's
    // stores are complete before the add)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid() == 0) __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // the segment's lead: its own partial's stores complete, then it waits for
  // the other nch - 1 chunks and merges them all
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nch > 1 && !wait_ticket(a, ticket, (uint32_t)(nch - 1), qi, s.flags + 10)) return;
  const float* parts = a.attn_part + ((size_t)l * a.n_attn + first) * CS;
  uint16_t* out = a.attn_out + ((size_t)l * a.max_batch + b) * a.nq * D + (size_t)g * G * D;
  attn_combine(a, s, parts, nch, out);
  return;
}

// Mixed steps only: the new K (rotated) and V of lead t.idx's (sequence, kv
// head), written through to memory before the task's signal, so that every
// attention task of the layer, which waits for all of them, reads them from
// the pages.  In other steps the task only signals.
TASK void task_kvw(const KArgs& a, const Task& t, const Lds& s, int qi) {
  if (a.kv_sync && !wait_counter(a, t.wait[0], t.fanin[0], qi, s.flags + 0)) return;
  // the trace's ready time: after the wait, or at once in a plain decode step (nothing to write)
  if (a.trace && tid() == 0 && qi < a.trace_cap) a.trace[kTraceWords * (size_t)qi + 1] = wall_clock64();
  if (!a.kv_sync) return;
  const int m = t.idx, b = m / a.nkv, g = m % a.nkv;
  if (b >= a.n) return;
  const int D = a.d, half = D / 2, ps = a.ps, l = t.layer;
  const int p = a.seq_lens[b] + a.step;
  if (p < 0 || p + 1 > a.max_pages * ps) {
    if (tid() == 0) raise_error(a, MK_ERR_DEVICE_SEQ, qi, b);
    return;
  }
  const int page = a.page_table[(size_t)b * a.max_pages + p / ps];
  if (page < 0 || page >= a.num_pages) {
    if (tid() == 0) raise_error(a, MK_ERR_DEVICE_PAGE, qi, page);
    return;
  }
  const float* qkv = a.qkv + ((size_t)l * a.max_batch + b) * a.qkv_rows;
  const float* kr = qkv + (size_t)a.nq * D + (size_t)g * D;
  const float* vr = qkv + (size_t)(a.nq + a.nkv) * D + (size_t)g * D;
  const size_t koff = ((((size_t)l * a.num_pages + page) * a.nkv + g) * ps + p % ps) * D;
  const size_t voff = (((size_t)l * a.num_pages + page) * a.nkv + g) * (size_t)ps * D + p % ps;
  const int i = tid();
  if (i < half) {
    // the rotation at position p as the attention tasks compute it (angle in double, cos / sin in float)
    double sd, cd;
    sincos((double)p * a.inv_freq[i], &sd, &cd);
    uint16_t lo, hi;
    rope_pair(ld_coh(kr + i), ld_coh(kr + i + half), (float)cd, (float)sd, lo, hi);
    st_coh(a.k_pool + koff + i, lo);
    st_coh(a.k_pool + koff + i + half, hi);
  }
  if (i < D) st_coh(a.v_pool + voff + (size_t)i * ps, f2bf(ld_coh(vr + i)));
}

TASK void task_attn(const KArgs& a, const Task& t, const Lds& s, int qi) {
  if (a.d == 128) attn_task<128>(a, t, s, qi);
  else attn_task<64>(a, t, s, qi);
}

// ---------------------------------------------------------------------------
// GATEUP: the distinct selected experts' rows, flattened expert-major into
// nU * I virtual rows, are cut evenly over the gate/up tasks.

struct JobGateUp {
  static constexpr bool kDense = false;  // rows see a varying token subset
  float* red = nullptr;
  const TopK* tk;
  const gu8 *wg, *wu;                       // gate and up matrices (bytes)
  const AS_GLOBAL float *sg = nullptr, *su = nullptr;  // FP8: their row scales
  const uint16_t* xs;
  float* gs;
  int64_t v0;
  int H, I, maxB, topk;
  DEV int urow(int i, int* r) const {
    const int64_t vr = v0 + (i >> 1);
    *r = (int)(vr % I);
    return (int)(vr / I);
  }
  DEV const gu4* row(int i) const {
    int r;
    const int u = urow(i, &r);
    return (const gu4*)(((i & 1) ? wu : wg) + ((size_t)tk->U[u] * I + r) * wrow_bytes(H));
  }
  DEV float scale(int i) const {
    int r;
    const int u = urow(i, &r);
    return ((i & 1) ? su : sg)[(size_t)tk->U[u] * I + r];
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

// Every gate/up task takes the layer's top-k itself from the router logits
// (once the router rows are done), which spares the routing a hop of its own.
// have_xs: region A still holds this layer's normalized input, left there by
// the PRE task that ran just before on this compute unit.
// Virtual gate/up rows [va, vb) of layer l (row v: expert U[v / I], row
// v % I of its gate and up matrices), in passes of at most kGuPass (bounds the
// LDS of the gate/up results): SwiGLU of each token's pair into h.
DEV void gateup_range(const KArgs& a, const Lds& s, int l, const uint16_t* xs, int64_t va, int64_t vb) {
  const TopK* tk = s.tk;
  JobGateUp j;
  j.tk = tk;
  j.wg = wbytes(a, widx(l, WL_GATE));
  j.wu = wbytes(a, widx(l, WL_UP));
  if constexpr (kWQ) {
    j.sg = wscales(a, widx(l, WL_GATE), (size_t)a.E * a.I, a.H);
    j.su = wscales(a, widx(l, WL_UP), (size_t)a.E * a.I, a.H);
  }
  j.xs = xs;
  j.gs = (float*)s.C;
  j.H = a.H;
  j.I = a.I;
  j.maxB = a.max_batch;
  j.topk = a.topk;
  const int mt = tk->maxtok;
  uint16_t* hl = a.h + (size_t)l * a.max_batch * a.topk * a.I;
  for (int64_t v0 = va; v0 < vb; v0 += kGuPass) {
    const int nvr = (int)((vb - v0) < kGuPass ? (vb - v0) : kGuPass);
    j.v0 = v0;
    run_rowdots<kWQ>(a.H, 2 * nvr, mt, j);
    __syncthreads();
    for (int e = tid(); e < nvr * mt; e += kThreads) {
      const int vi = e / mt, tt = e % mt;
      const int64_t vr = v0 + vi;
      const int u = (int)(vr / a.I), r = (int)(vr % a.I);
      if (tt < tk->ntok[u]) {
        const float gg = j.gs[((size_t)vi * a.max_batch + tt) * 2];
        const float uu = j.gs[((size_t)vi * a.max_batch + tt) * 2 + 1];
        const float hv = gg / (1.0f + __expf(-gg)) * uu;
        st_coh(hl + (size_t)tk->pair[u][tt] * a.I + r, f2bf(hv));
      }
    }
    __syncthreads();
  }
}

// The split of layer l's R = nU * I virtual rows: [0, Rs) cut evenly over the
// gate/up tasks, [Rs, R) the shared pool in items of kGuItem rows.
DEV int64_t gateup_static_rows(const KArgs& a, int64_t R, int* n_items) {
  int64_t items = a.gu_items ? (R * a.gu_pool / 64 + kGuItem - 1) / kGuItem : 0;
  if (items > a.gu_items) items = a.gu_items;
  if (items * kGuItem > R) items = R / kGuItem;
  *n_items = (int)items;
  return R - items * kGuItem;
}

// Claims items of layer l's shared pool until none is left.  The claim counter
// is never reset: every claimer of a step ends with one failed claim, so each
// step adds exactly gu_items + gu_parts, and this step's items are numbered
// from (epoch - 1) times that (mod 2^32).  Items past this step's count (fewer
// distinct experts than the most there can be) are claimed and skipped.
DEV void gateup_pool(const KArgs& a, const Lds& s, int l, const uint16_t* xs, int64_t R) {
  if (a.gu_items == 0) return;
  int n_items;
  const int64_t Rs = gateup_static_rows(a, R, &n_items);
  const uint32_t base = (a.epoch - 1u) * (uint32_t)(a.gu_items + a.gu_parts);
  for (;;) {
    if (tid() == 0)
      s.flags[12] = (int32_t)(__hip_atomic_fetch_add(a.claims + l, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - base);
    __syncthreads();
    const int k = s.flags[12];
    __syncthreads();
    if (k < 0 || k >= a.gu_items) break;
    if (k < n_items) {
      const int64_t v0 = Rs + (int64_t)k * kGuItem;
      gateup_range(a, s, l, xs, v0, v0 + kGuItem);
    }
  }
}

// Returns whether region B holds this layer's top-k afterwards (false when the
// router logits never arrived: abort or time-out).
TASK bool task_gateup(const KArgs& a, const Task& t, const Lds& s, int qi, bool have_xs) {
  const int l = t.layer;
  if (!compute_topk(a, l, s.tk, s.C, qi, s.flags + 0, 0)) return false;
  if (t.idx == 0) write_sel(a, l, s.tk);
  mark(a, qi, 1);
  uint16_t* xs = (uint16_t*)s.A;
  if (!have_xs) norm_inputs(a, l, moe_gain(a, l), xs, s.red8, qi, -1, nullptr, kSeq ? kWithWo : kParallel);
  mark(a, qi, 2);
  const int64_t R = (int64_t)s.tk->nU * a.I;
  int n_items;
  const int64_t Rs = gateup_static_rows(a, R, &n_items);
  gateup_range(a, s, l, xs, Rs * t.idx / a.n_gu, Rs * (t.idx + 1) / a.n_gu);
  mark(a, qi, 3);
  gateup_pool(a, s, l, xs, R);
  return true;
}

// An attention unit past its chunk: the layer's top-k and normalized input,
// then items of the shared gate/up pool.  Returns as task_gateup.
TASK bool task_gutail(const KArgs& a, const Task& t, const Lds& s, int qi) {
  const int l = t.layer;
  if (!compute_topk(a, l, s.tk, s.C, qi, s.flags + 0, 0)) return false;
  uint16_t* xs = (uint16_t*)s.A;
  norm_inputs(a, l, moe_gain(a, l), xs, s.red8, qi, 1, nullptr, kSeq ? kWithWo : kParallel);
  gateup_pool(a, s, l, xs, (int64_t)s.tk->nU * a.I);
  mark(a, qi, 2);
  return true;
}

// ---------------------------------------------------------------------------
// OUT: rows [r0, r1) of the hidden state.

struct JobDown {
  static constexpr bool kDense = false;  // rows see a varying token subset
  float* red = nullptr;
  const TopK* tk;
  const gu8* W;                           // down matrices (bytes)
  const AS_GLOBAL float* sc = nullptr;    // FP8: their row scales
  const uint16_t* hs;
  float* contrib;
  int r0, H, I, nU, maxBK;
  DEV const gu4* row(int i) const {
    const int rr = i / nU, u = i % nU;
    return (const gu4*)(W + ((size_t)tk->U[u] * H + r0 + rr) * wrow_bytes(I));
  }
  DEV float scale(int i) const {
    const int rr = i / nU, u = i % nU;
    return sc[(size_t)tk->U[u] * H + r0 + rr];
  }
  DEV int nx(int i) const { return tk->ntok[i % nU]; }
  DEV const uint4* x(int i, int t) const { return (const uint4*)(hs + (size_t)tk->pair[i % nU][t] * I); }
  DEV void emit(int i, int t, float v) const { contrib[(size_t)(i / nU) * maxBK + tk->pair[i % nU][t]] = v; }
};

// Down-projection rows held in registers across the gate/up wait: kDownL
// lanes per row (16; 8 for FP4, whose 768-element rows are 24 chunks), up to
// kDownC 16-byte chunks per lane, kDownGroups groups of 64 / kDownL rows per
// wave (the 96 rows of a 12-row task at 8 experts fit).
constexpr int kDownC = 6;
constexpr int kDownGroups = 4;
constexpr int kDownL = kWBits == 4 ? 8 : 16;

// Output tasks wait for their inputs themselves: the residual rows and the
// top-k (from LDS, or computed once the router rows are done) first; the
// first down-projection rows once nine tenths of the gate/up tasks are in,
// and the gate/up results after the last one.
// have_tk: region B still holds this layer's top-k, left there by the gate/up
// task that ran just before on this compute unit.  tk_layer: set to the layer
// whose top-k region B holds when the task ends (-1: none).
// Returns the number of leading waves that must wait for their stores before
// the task signals (the others may still be copying the next task's tile).
TASK int task_out(const KArgs& a, const Task& t, const Lds& s, int qi, bool have_tk, int& tk_layer) {
  const int l = t.layer, nr = t.r1 - t.r0, n = a.n;
  float* contrib = (float*)s.C;  // [out_rows_max][maxB*topk]
  const int maxBK = a.max_batch * a.topk;
  uint16_t* xs = (uint16_t*)s.A;
  // the residual rows this task updates are final already: their loads go out first
  float x_first = 0.f;
  if (tid() < nr * n) {
    const int rr = tid() / n, b = tid() % n;
    x_first = load_x(a, l, b, t.r0 + rr, l == 0 ? token_row(a, b, qi) : nullptr);
  }
  if (!have_tk) {
    tk_layer = compute_topk(a, l, s.tk, s.C, qi, s.flags + 1, -1) ? l : -1;
    if (tk_layer < 0) return kWaves;
  }
  const TopK* tk = s.tk;
  JobDown jd;
  jd.tk = tk;
  jd.W = wbytes(a, widx(l, WL_DOWN));
  if constexpr (kWQ) jd.sc = wscales(a, widx(l, WL_DOWN), (size_t)a.E * a.H, a.I);
  jd.hs = xs;
  jd.contrib = contrib;
  jd.r0 = t.r0;
  jd.H = a.H;
  jd.I = a.I;
  jd.nU = tk->nU;
  jd.maxBK = maxBK;
  // 16-byte chunks per lane of a down row (kDownL lanes per row)
  const int nd = nr * jd.nU, cpl = wrow_bytes(a.I) / (16 * kDownL);
  // waves 1..7 hold them (wave 0, whose thread 0 polls the flags, loads none)
  constexpr int kGroupRows = (kWaves - 1) * (64 / kDownL);
  const int npre = (wrow_bytes(a.I) % (16 * kDownL) == 0 && cpl <= kDownC) ? min(nd, kDownGroups * kGroupRows) : 0;
  // the down rows go out once nine tenths of the gate/up tasks are done: issued
  // earlier, by the units that finish first, they take bandwidth from the last
  // gate/up tasks, which every output task waits for
  if (!wait_counter_part(a, t.wait[0], t.fanin[0], (t.fanin[0] * 9 + 9) / 10, qi, s.flags + 0)) return kWaves;
  const int lane = tid() & 63, wave = tid() >> 6, li = lane % kDownL;
  const int ig = wave >= 1 ? (wave - 1) * (64 / kDownL) + lane / kDownL : kDownGroups * kGroupRows;  // row within a group
  uint4 dp[kDownGroups][kDownC];
#pragma unroll
  for (int g = 0; g < kDownGroups; ++g) {
    const int i = g * kGroupRows + ig;
    const bool act = i < npre;
    const gu4* wr = jd.row(act ? i : 0) + li;
#pragma unroll
    for (int c = 0; c < kDownC; ++c)
      dp[g][c] = __builtin_bit_cast(uint4, act && c < cpl ? __builtin_nontemporal_load(wr + kDownL * c) : u32x4_v{0, 0, 0, 0});
  }
  if (!wait_counter(a, t.wait[0], t.fanin[0], qi, s.flags + 0)) return kWaves;
  if (a.trace && tid() == 0 && qi < a.trace_cap) a.trace[kTraceWords * (size_t)qi + 1] = wall_clock64();
  copy_to_lds<true>(xs, a.h + (size_t)l * a.max_batch * a.topk * a.I, (uint32_t)n * a.topk * a.I * 2);
  prefetch_wait();
  mark(a, qi, 0);
  // expert down projections: the register rows, then the rest from HBM
  const int mt = tk->maxtok;
  constexpr int XM = 16 / kWBits;                    // input chunks per weight chunk
  constexpr int kDC = 768 * kWBits / (128 * kDownL);  // chunks per lane of a 768-element row
  if (cpl == kDC) {
    // every chunk present: a row's LDS reads go out together, then the
    // arithmetic (a guard per chunk would make each read wait for the last)
#pragma unroll
    for (int g = 0; g < kDownGroups; ++g) {
      const int i = g * kGroupRows + ig;
      const bool act = i < npre;
      const int nx = act ? jd.nx(i) : 0;
      for (int tt = 0; tt < mt; ++tt) {
        const bool on = tt < nx;
        const uint4* xr = jd.x(act ? i : 0, on ? tt : 0) + XM * li;
        uint4 xv[kDC * XM];
#pragma unroll
        for (int c = 0; c < kDC; ++c)
#pragma unroll
          for (int m = 0; m < XM; ++m) xv[XM * c + m] = xr[XM * kDownL * c + m];
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < kDC; ++c) acc = dotw<kWQ>(dp[g][c], xv + XM * c, acc);
        acc = group_sum<kDownL>(acc);
        if (on && li == 0) jd.emit(i, tt, scaled<kWQ>(jd, i, acc));
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < kDownGroups; ++g) {
      const int i = g * kGroupRows + ig;
      const bool act = i < npre;
      const int nx = act ? jd.nx(i) : 0;
      for (int tt = 0; tt < mt; ++tt) {
        const bool on = tt < nx;
        const uint4* xr = jd.x(act ? i : 0, on ? tt : 0) + XM * li;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < kDownC; ++c)
          if (c < cpl) acc = dotw<kWQ>(dp[g][c], xr + XM * kDownL * c, acc);
        acc = group_sum<kDownL>(acc);
        if (on && li == 0) jd.emit(i, tt, scaled<kWQ>(jd, i, acc));
      }
    }
  }
  rowdots_range<false, kWQ>(a.I, npre, nd, mt, jd);
  mark(a, qi, 1);
  // batch 1, wave 0 alone storing the residual rows: meanwhile waves 1..7
  // copy the weight tile of the PRE task that follows on this unit into LDS
  // (above tile_off, clear of the contributions); that task then finds it
  // there instead of issuing it in front of its own wait
  const bool early = n == 1 && nr <= 64 && t.next_r1 > t.next_r0 && a.pf_wide > 0;
  if (early) {
    int rowb;
    const gu8* src = pre_rows_src(a, t.next_layer, t.next_r0, &rowb);
    const int npf = min(t.next_r1 - t.next_r0, a.pf_wide / rowb);
    prefetch_to_lds(src, s.C + a.tile_off, npf * rowb);
    if (tid() == 0) s.flags[18] = t.next_layer + 1;
  }
  // the expert half of x_{l+1}: x_l + sum_j w_j y_j (the next layer adds the
  // Wo rows' half); the record of x_l (layers >= 1) for the caller.  The
  // contributions in LDS come from every wave: barrier first (LDS only: waves
  // 1..7 may have the next tile's copy in flight).
  lds_barrier();
  mark(a, qi, 2);
  for (int e = tid(); e < nr * n; e += kThreads) {
    const int rr = e / n, b = e % n;
    float moe = 0.f;
    for (int j = 0; j < a.topk; ++j) moe += tk->w[b][j] * contrib[(size_t)rr * maxBK + b * a.topk + j];
    const float xo = e == tid() ? x_first : load_x(a, l, b, t.r0 + rr, l == 0 ? token_row(a, b, qi) : nullptr);
    const size_t o = ((size_t)l * a.max_batch + b) * a.H + t.r0 + rr;
    st_coh(a.x + o + (size_t)a.max_batch * a.H, xo + moe);
    if (l > 0) a.xr[o] = kSeq ? ld_coh(a.x + o) : (a.x_in ? resid(a, l, b, t.r0 + rr) : xo);
  }
  mark(a, qi, 3);
  // waves whose stores the consumers read must see them complete before the signal
  return early ? 1 : kWaves;
}

// ---------------------------------------------------------------------------
// WO: rows [r0, r1) of Wo times the merged attention output, for the output
// tasks' residual update.  The task waits for the merges itself: before that
// the first rows of Wo are in LDS already (copied at task start) and the next
// (kWaves - 1) * 2 are loaded into registers by waves 1..7 (32 lanes per row,
// kWoC 16-byte chunks per lane), so mostly arithmetic is left once the
// attention output is in.
constexpr int kWoC = 16;

TASK void task_wo(const KArgs& a, const Task& t, const Lds& s, int qi, int npf) {
  const int l = t.layer, AD = a.nq * a.d, nr = t.r1 - t.r0, n = a.n;
  const int lane = tid() & 63, wave = tid() >> 6, li = lane & 31;
  constexpr int kWC = kWoC * kWBits / 16;  // chunks per lane of a register row
  const int rowb = wrow_bytes(AD);
  const int nreg = rowb == 32 * kWC * 16 && n == 1 ? min(nr - npf, (kWaves - 1) * 2) : 0;
  const int ir = npf + (wave >= 1 ? (wave - 1) * 2 + (lane >> 5) : nreg);  // this lane's register row
  const bool act = ir < npf + nreg;
  const gu8* W = wbytes(a, widx(l, WL_O));
  const gu4* wsrc = (const gu4*)(W + (size_t)(t.r0 + (act ? ir : 0)) * rowb) + li;
  uint4 wr[kWC];
#pragma unroll
  for (int c = 0; c < kWC; ++c)
    wr[c] = __builtin_bit_cast(uint4, act ? __builtin_nontemporal_load(wsrc + 32 * c) : u32x4_v{0, 0, 0, 0});
  if (!wait_counter(a, t.wait[0], t.fanin[0], qi, s.flags + 0)) return;
  if (a.trace && tid() == 0 && qi < a.trace_cap) a.trace[kTraceWords * (size_t)qi + 1] = wall_clock64();
  uint16_t* xs = (uint16_t*)s.A;
  copy_to_lds<true>(xs, a.attn_out + (size_t)l * a.max_batch * AD, (uint32_t)n * AD * 2);
  prefetch_wait();
  mark(a, qi, 0);
  JobPre j;
  j.pf = (const AS_LDS uint8_t*)(s.C + a.tile_off);
  j.npf = npf;
  j.red = (float*)s.C;
  j.W = W;
  if constexpr (kWQ) j.sc = wscales(a, widx(l, WL_O), a.H, AD);
  j.r0 = t.r0;
  j.K = AD;
  j.rowb = rowb;
  j.xs = xs;
  j.out = a.wo_out + (size_t)l * a.max_batch * a.H + t.r0;
  j.ld = a.H;
  rowdots_range<true, kWQ>(AD, 0, npf, n, j);
  constexpr int XM = 16 / kWBits;
  for (int b = 0; b < n; ++b) {
    const uint4* xr = (const uint4*)(xs + (size_t)b * AD) + XM * li;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < kWC; ++c) acc = dotw<kWQ>(wr[c], xr + XM * 32 * c, acc);
    acc = group_sum<32>(acc);
    if (act && li == 0) j.emit(ir, b, scaled<kWQ>(j, ir, acc));
  }
  rowdots_range<false, kWQ>(AD, npf + nreg, nr, n, j);
  mark(a, qi, 1);
}

// ---------------------------------------------------------------------------
// LMHEAD: rows [r0, r1) of the vocabulary, then the greedy or sampled argmax.

struct JobLM {
  static constexpr bool kDense = true;
  float* red = nullptr;  // region C holds the logits for the argmax: no column split
  const gu8* W;                           // the LM head (bytes)
  const AS_GLOBAL float* sc = nullptr;    // FP8: its row scales
  int r0, K, V, maxB;
  const uint16_t* xs;
  float* lmv;
  float* logits;
  bool coh;  // top-p: the last LM-head unit reads every unit's logits, so they go out device-coherent
  DEV const gu4* row(int i) const { return (const gu4*)(W + (size_t)(r0 + i) * wrow_bytes(K)); }
  DEV float scale(int i) const { return sc[r0 + i]; }
  DEV int nx(int) const { return 1 << 30; }
  DEV const uint4* x(int, int t) const { return (const uint4*)(xs + (size_t)t * K); }
  DEV void emit(int i, int t, float v) const {
    if (coh) st_coh(logits + (size_t)t * V + r0 + i, v);
    else logits[(size_t)t * V + r0 + i] = v;
    lmv[(size_t)i * maxB + t] = v;
  }
};

// Sampling at temperature T by the Gumbel-max rule: the next token is
// argmax_i (logit_i / T + g_i) with g_i ~ Gumbel(0, 1), which draws token i
// with probability softmax(logits / T)_i.  The noise comes from SplitMix64
// (Steele, Lea and Flood 2014) used as a counter-based generator: output n of
// the generator seeded with `seed` is the finalizer applied to
// seed + (n + 1) * 0x9E3779B97F4A7C15; token i of batch slot b whose step input
// sits at position p takes n = (p * max_batch + b) * V + i, u = (top 53 bits +
// 1/2) / 2^53 in (0, 1), and g = -log(-log(u)) in double.
DEV uint64_t splitmix64_at(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The score the argmax compares for logit x of token i, slot b: the logit
// itself (greedy) or x / T + g_i, rounded to float.
DEV float sample_score(const KArgs& a, float x, int b, int i) {
  if (a.inv_temp == 0.0) return x;
  const uint64_t p = (uint64_t)(a.seq_lens[b] + a.step);
  const uint64_t n = (p * (uint64_t)a.max_batch + (uint64_t)b) * (uint64_t)a.V + (uint64_t)i;
  const double u = ((double)(splitmix64_at(a.seed, n) >> 11) + 0.5) * 0x1.0p-53;
  return (float)((double)x * a.inv_temp - log(-log(u)));
}

// Top-p sampling for slot b, by the last LM-head unit once every unit's logits
// are stored: the nucleus is every token whose scaled logit s = x / T is at
// least the largest threshold keeping mass >= top_p of softmax(s), tokens tied
// at it included; the draw is the Gumbel-max argmax within it.  No sort: the
// masses exp(s - max) as 32-bit fixed point (integer sums, so no order
// dependence) go into a histogram over the ordered bits of s, 11 bits a pass
// from the top (three passes), which pins the threshold's key; one more pass
// takes the argmax of the scores of the tokens at or above it.  hist: LDS,
// kTopPBins 64-bit words.  Returns the token, in every thread.
DEV void block_argmax(float& v, int& i, float* red);

DEV float scaled_logit(const KArgs& a, const float* lg, int i) {
  const float x = ld_coh(lg + i);
  return x != x ? kNegInf : (float)((double)x * a.inv_temp);
}

DEV uint64_t block_sum_u64(uint64_t v, uint64_t* scratch) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  __syncthreads();
  if ((tid() & 63) == 0) scratch[tid() >> 6] = v;
  __syncthreads();
  uint64_t t = 0;
  for (int w = 0; w < kWaves; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

DEV int top_p_draw(const KArgs& a, int b, uint64_t* hist, float* red) {
  const int V = a.V;
  const float* lg = a.logits + (size_t)b * V;
  uint64_t* scratch = hist + kTopPBins;           // kWaves words for the block sums
  // the largest scaled logit
  float smax = kNegInf;
  int imax = 0;
  for (int i = tid(); i < V; i += kThreads) {
    const float sv = scaled_logit(a, lg, i);
    if (better(sv, i, smax, imax)) { smax = sv; imax = i; }
  }
  block_argmax(smax, imax, red);
  // three radix passes: 11, 11 and 10 bits of the key, each among the tokens whose
  // higher bits equal the threshold's so far; `above` is the mass of the tokens
  // whose key lies above every bucket of this pass
  uint32_t prefix = 0;
  uint64_t above = 0, need = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int k = tid(); k < nb; k += kThreads) hist[k] = 0;
    __syncthreads();
    uint64_t mine = 0;
    for (int i = tid(); i < V; i += kThreads) {
      const float sv = scaled_logit(a, lg, i);
      const uint32_t key = topk_key(sv);
      if (pass > 0 && (key >> (shift + (pass == 1 ? 11 : 10))) != prefix) continue;
      const uint64_t m = (uint64_t)(__expf(sv - smax) * 4294967296.0f);
      atomicAdd((unsigned long long*)(hist + ((key >> shift) & (uint32_t)(nb - 1))), (unsigned long long)m);
      mine += m;
    }
    if (pass == 0) {
      const uint64_t z = block_sum_u64(mine, scratch);
      need = (uint64_t)ceil((double)a.top_p * (double)z);
    }
    __syncthreads();
    if (tid() == 0) {
      // the highest bucket at which the mass from the top reaches `need`
      uint64_t acc = above;
      int k = nb - 1;
      for (; k > 0; --k) {
        if (acc + hist[k] >= need) break;
        acc += hist[k];
      }
      scratch[0] = (uint64_t)k;
      scratch[1] = acc;
    }
    __syncthreads();
    prefix = (prefix << (pass == 2 ? 10 : 11)) | (uint32_t)scratch[0];
    above = scratch[1];
    __syncthreads();
  }
  // prefix is now the threshold's whole key: the draw among the tokens at or above it
  float v = kNegInf;
  int pick = 0x7fffffff;
  for (int i = tid(); i < V; i += kThreads) {
    const float sv = scaled_logit(a, lg, i);
    if (topk_key(sv) < prefix) continue;
    float x = ld_coh(lg + i);
    if (x != x) x = kNegInf;
    const float sc = sample_score(a, x, b, i);
    if (better(sc, i, v, pick)) { v = sc; pick = i; }
  }
  block_argmax(v, pick, red);
  return pick;
}

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
  if ((tid() & 63) == 0) {
    red[tid() >> 6] = v;
    ((int*)red)[8 + (tid() >> 6)] = i;
  }
  __syncthreads();
  v = red[0];
  i = ((int*)red)[8];
  for (int w = 1; w < kWaves; ++w)
    if (better(red[w], ((int*)red)[8 + w], v, i)) { v = red[w]; i = ((int*)red)[8 + w]; }
}

TASK void task_lmhead(const KArgs& a, const Task& t, const Lds& s, int qi) {
  const int L = a.L, nr = t.r1 - t.r0;
  uint16_t* xs = (uint16_t*)s.A;
  norm_inputs(a, L, wptr(a, W_FINAL_NORM), xs, s.red8, qi, -1, t.idx == 0 ? a.xr : nullptr,
              kSeq ? kAlone : kParallel);
  mark(a, qi, 0);
  JobLM j;
  j.W = wbytes(a, W_LM_HEAD);
  if constexpr (kWQ) j.sc = wscales(a, W_LM_HEAD, a.V, a.H);
  j.K = a.H;
  j.V = a.V;
  j.maxB = a.max_batch;
  j.xs = xs;
  j.lmv = (float*)s.C;
  j.logits = a.logits;
  const bool top_p = a.inv_temp != 0.0 && a.top_p < 1.0f;
  j.coh = top_p;
  // rows in passes of at most kLmPass (bounds the LDS copy of the logits); thread 0
  // keeps the running best of each sequence
  float best_v[kMaxBatch];
  int best_i[kMaxBatch];
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) {
    best_v[b] = kNegInf;
    best_i[b] = 0x7fffffff;
  }
  for (int p0 = 0; p0 < nr; p0 += kLmPass) {
    const int np = min(kLmPass, nr - p0);
    j.r0 = t.r0 + p0;
    run_rowdots<kWQ>(a.H, np, a.n, j);
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      if (b >= a.n) break;
      float v = kNegInf;
      int i = 0x7fffffff;
      for (int r = tid(); r < np; r += kThreads) {
        float x = j.lmv[(size_t)r * a.max_batch + b];
        if (x != x) x = kNegInf;
        x = sample_score(a, x, b, j.r0 + r);
        if (better(x, j.r0 + r, v, i)) { v = x; i = j.r0 + r; }
      }
      block_argmax(v, i, s.red);
      if (better(v, i, best_v[b], best_i[b])) { best_v[b] = v; best_i[b] = i; }
    }
  }
  mark(a, qi, 1);
  if (tid() == 0) {
    for (int b = 0; b < a.n; ++b) {
      st_coh(a.lm_part + ((size_t)t.idx * a.max_batch + b) * 2, best_v[b]);
      st_coh((uint32_t*)a.lm_part + ((size_t)t.idx * a.max_batch + b) * 2 + 1, (uint32_t)best_i[b]);
    }
  }
  uint32_t* ticket = a.tickets + (size_t)a.L * a.max_batch * a.nkv;
  mark(a, qi, 2);
  if (arrive_last(ticket, (uint32_t)a.n_lm, s.flags + 11)) {
    for (int b = 0; b < a.n; ++b) {
      float v = kNegInf;
      int i = 0x7fffffff;
      if (top_p) {
        i = top_p_draw(a, b, (uint64_t*)s.C, s.red);
      } else {
        for (int k = tid(); k < a.n_lm; k += kThreads) {
          const float x = ld_coh(a.lm_part + ((size_t)k * a.max_batch + b) * 2);
          const int xi = (int)ld_coh((const uint32_t*)a.lm_part + ((size_t)k * a.max_batch + b) * 2 + 1);
          if (better(x, xi, v, i)) { v = x; i = xi; }
        }
        block_argmax(v, i, s.red);
      }
      if (tid() == 0 && a.next_tok) st_coh((uint32_t*)a.next_tok + (size_t)a.step * a.n + b, (uint32_t)i);
    }
  }
}

// ---------------------------------------------------------------------------

// Runs a.nsteps decode steps: step s uses epoch a.epoch + s (counter targets,
// tags) and positions seq_lens + s; its layer-0 tasks wait for step s - 1's
// LM head (the greedy token).  Every queue ends with its LM head task, so a
// queue starts step s + 1 only after its share of step s.
extern "C" __global__ void __launch_bounds__(kThreads, 1) MKK(mk_megakernel)(KArgs a0) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  KArgs a = a0;
  const Lds s = carve(lds_raw, a);
  const int cu = blockIdx.x;
  const int q0 = a.queue_off[cu], q1 = a.queue_off[cu + 1];
  for (int step = 0; step < a0.nsteps; ++step) {
    a.step = step;
    a.epoch = a0.epoch + (uint32_t)step;
    if (tid() == 0) {
      s.flags[16] = -1;  // no attention plan cached yet (positions moved)
      s.flags[18] = 0;   // no PRE tile copied ahead
    }
    __syncthreads();
    int xs_layer = -1;                 // layer whose normalized input region A holds
    int tk_layer = -1;                 // layer whose top-k region B holds
    for (int q = q0; q < q1; ++q) {
      const Task t = a.tasks[q];
      uint64_t t_fetch = 0, t_ready = 0;
      if (a.trace && tid() == 0) t_fetch = wall_clock64();
      // immutable weights start streaming into LDS before the inputs are ready
      const int npf = task_prefetch(a, t, s, q);
      bool ok = true;
      // after the first step, layer 0 needs the previous step's greedy token
      if (step > 0 && t.layer == 0 && (t.op == OP_PRE || t.op == OP_OUT))
        ok = wait_counter_at(a, ctr_index(a.L, C_DONE), a.n_lm, q, s.flags + 1, a.epoch - 1);
      // attention, Wo and output tasks wait inside, once their loads are in flight; gate/up
      // tasks poll the tagged router logits inside
      const bool own_wait = t.op == OP_ATTN || t.op == OP_OUT || t.op == OP_WO || t.op == OP_GATEUP ||
                            t.op == OP_GUTAIL || t.op == OP_KVW;
      if (ok && !own_wait) ok = wait_counter(a, t.wait[0], t.fanin[0], q, s.flags + 0);
      if (ok && !own_wait && t.wait[1] >= 0) ok = wait_counter(a, t.wait[1], t.fanin[1], q, s.flags + 1);
      if (a.trace && tid() == 0) t_ready = wall_clock64();
      int wait_waves = kWaves;
      if (ok) {
        switch (t.op) {
          case OP_PRE: task_pre(a, t, s, q, npf); break;
          case OP_ATTN: task_attn(a, t, s, q); break;
          case OP_GATEUP: tk_layer = task_gateup(a, t, s, q, xs_layer == t.layer) ? t.layer : -1; break;
          case OP_OUT: wait_waves = task_out(a, t, s, q, tk_layer == t.layer, tk_layer); break;
          case OP_WO: task_wo(a, t, s, q, npf); break;
          case OP_KVW: task_kvw(a, t, s, q); break;
          case OP_GUTAIL: tk_layer = task_gutail(a, t, s, q) ? t.layer : -1; break;
          case OP_LMHEAD: task_lmhead(a, t, s, q); break;
          default: break;
        }
      }
      // (sequential block: only a router task's norm is the one the gate/up task needs)
      xs_layer = ok && t.op == OP_PRE && (!kSeq || t.r0 >= a.qkv_rows) ? t.layer
                                                                            : (ok && t.op == OP_GATEUP ? xs_layer : -1);
      // region B holds a layer's top-k only after a top-k that succeeded (a failed one, on
      // abort or time-out, leaves whatever an earlier task or kernel left there)
      if (t.op == OP_LMHEAD) tk_layer = -1;
      if (t.tagged) __syncthreads();  // consumers poll the tagged output itself
      else signal_counter(a, t.signal, t.slot, wait_waves);
      if (a.trace && tid() == 0 && q < a.trace_cap) {
        uint64_t* r = a.trace + kTraceWords * (size_t)q;
        r[0] = t_fetch;
        if (!own_wait) r[1] = t_ready;
        r[6] = wall_clock64();
      }
    }
  }
}

#if MK_WFMT == 0 && !MK_SEQ
// One copy of what follows (not per weight format): the fill kernel and the static workspace.
__global__ void mk_fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + tid(); i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

extern "C" int mkk_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t stream) {
  size_t blocks = (n + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(mk_fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, v, n);
  return (int)hipGetLastError();
}

// Workspace for callers that cannot allocate device memory (mk_bind_scratch).
// Each GPU that loads this library holds one copy until the process ends; host
// code never passes the name `scratch` to a kernel (on the host it is only a
// stand-in), it asks mkk_scratch for this device's address instead.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

extern "C" size_t mkk_scratch_bytes() { return kScratchBytes; }

// Device address of the current device's copy of `scratch`, looked up once per
// device with that device current.
extern "C" int mkk_scratch(int* device, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p || ((uintptr_t)p) % 256) return (int)hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *device = dev;
  *ptr = addr[dev];
  return 0;
}
#endif  // MK_WFMT == 0

extern "C" int MKK(mkk_launch_step)(const KArgs* a, int grid, size_t lds_bytes, hipStream_t stream) {
  static size_t attr_bytes = 0;
  if (lds_bytes > attr_bytes) {
    hipError_t e = hipFuncSetAttribute((const void*)MKK(mk_megakernel), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return (int)e;
    attr_bytes = lds_bytes;
  }
  KArgs copy = *a;
  void* args[] = {&copy};
  return (int)hipLaunchCooperativeKernel((const void*)MKK(mk_megakernel), dim3(grid), dim3(kThreads), args,
                                         (unsigned)lds_bytes, stream);
}
