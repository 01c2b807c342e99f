// Streaming-read probe for MI355X (gfx950): how fast one workgroup of 512
// threads, and a grid of them, reads HBM with the two load forms the decode
// kernel uses: 16-byte non-temporal register loads (DEPTH in flight per lane)
// and 16-byte LDS DMA copies (global_load_lds, an LDS ring of RING KB).
// Each workgroup reads its own disjoint range of `per_wg` bytes once and
// records s_memrealtime (100 MHz) at start and end.  The bytes read are known
// exactly, so the same runs also calibrate the FETCH_SIZE counter for these
// load forms.  Host-visible entry points take plain device pointers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define AS_GLOBAL __attribute__((address_space(1)))
#define AS_LDS __attribute__((address_space(3)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DEPTH>
__global__ void __launch_bounds__(512, 1) reg_stream(const u32x4* src, size_t per_wg, uint64_t* times, uint32_t* sink) {
  const size_t n16 = per_wg / 16;                     // 16-byte pieces of this workgroup
  const AS_GLOBAL u32x4* p = (const AS_GLOBAL u32x4*)(src + (size_t)blockIdx.x * n16);
  const int t = threadIdx.x;
  uint64_t t0 = wall_clock64();
  u32x4 acc = {0, 0, 0, 0};
  // pass: every lane loads DEPTH pieces 512 apart (a wave reads 1 KB per load), then uses them
  for (size_t base = 0; base < n16; base += (size_t)512 * DEPTH) {
    u32x4 v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const size_t i = base + (size_t)d * 512 + t;
      v[d] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= v[d];
  }
  __syncthreads();
  if (t == 0) { times[2 * blockIdx.x] = t0; times[2 * blockIdx.x + 1] = wall_clock64(); }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) sink[t] = 1;   // keep the loads
}

// gfx9 s_waitcnt immediate: vmcnt <= n (bits 3:0 and 15:14), expcnt and lgkmcnt left at their maxima.
constexpr int waitcnt_vm(int n) { return (n & 0xf) | 0x70 | 0xf00 | ((n >> 4) << 14); }

// LDS DMA ring of 8 slots, CPW 1 KB copies per wave per slot (slot = 8 * CPW KB,
// ring = 64 * CPW KB): the copies of slot s + 7 are issued before slot s is
// consumed, so 7 slots are in flight while one is read.
template <int CPW>
__global__ void __launch_bounds__(512, 1) lds_stream(const uint8_t* src, size_t per_wg, uint64_t* times, uint32_t* sink) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const AS_GLOBAL uint8_t* p = (const AS_GLOBAL uint8_t*)(src + (size_t)blockIdx.x * per_wg);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  constexpr int slot_bytes = 8 * CPW * 1024;
  const int nslot = (int)(per_wg / slot_bytes);
  uint64_t t0 = wall_clock64();
  uint32_t acc = 0;
  auto issue = [&](int s) {  // wave w copies 1 KB pieces w * CPW .. w * CPW + CPW - 1 of slot s
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int piece = wave * CPW + c;
      const size_t off = (size_t)s * slot_bytes + (size_t)piece * 1024 + lane * 16;
      __builtin_amdgcn_global_load_lds((AS_GLOBAL void*)(p + off), (AS_LDS void*)(lds + (s & 7) * slot_bytes + piece * 1024),
                                       16, 0, 2);
    }
  };
  for (int s = 0; s < 7 && s < nslot; ++s) issue(s);
  for (int s = 0; s < nslot; ++s) {
    if (s + 7 < nslot) {
      issue(s + 7);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(7 * CPW));  // this wave's copies of slot s have landed
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    acc ^= *(const uint32_t*)(lds + (s & 7) * slot_bytes + (t * 16) % slot_bytes);
    __syncthreads();
  }
  if (t == 0) { times[2 * blockIdx.x] = t0; times[2 * blockIdx.x + 1] = wall_clock64(); }
  if (acc == 0x12345678u) sink[t] = 1;
}

extern "C" int probe_reg_stream(const void* src, size_t per_wg, int nwg, int depth, uint64_t* times, uint32_t* sink,
                                void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (depth) {
    case 8: hipLaunchKernelGGL(reg_stream<8>, dim3(nwg), dim3(512), 0, s, (const u32x4*)src, per_wg, times, sink); break;
    case 16: hipLaunchKernelGGL(reg_stream<16>, dim3(nwg), dim3(512), 0, s, (const u32x4*)src, per_wg, times, sink); break;
    case 32: hipLaunchKernelGGL(reg_stream<32>, dim3(nwg), dim3(512), 0, s, (const u32x4*)src, per_wg, times, sink); break;
    case 48: hipLaunchKernelGGL(reg_stream<48>, dim3(nwg), dim3(512), 0, s, (const u32x4*)src, per_wg, times, sink); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

extern "C" int probe_lds_stream(const void* src, size_t per_wg, int nwg, int cpw, uint64_t* times, uint32_t* sink,
                                void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const size_t lds = (size_t)cpw * 64 * 1024;
  if (per_wg % ((size_t)cpw * 8 * 1024)) return -3;
  if (cpw == 1) {
    if (hipFuncSetAttribute((const void*)lds_stream<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) return -2;
    hipLaunchKernelGGL(lds_stream<1>, dim3(nwg), dim3(512), lds, s, (const uint8_t*)src, per_wg, times, sink);
  } else if (cpw == 2) {
    if (hipFuncSetAttribute((const void*)lds_stream<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) return -2;
    hipLaunchKernelGGL(lds_stream<2>, dim3(nwg), dim3(512), lds, s, (const uint8_t*)src, per_wg, times, sink);
  } else {
    return -1;
  }
  return (int)hipGetLastError();
}
