// Pieces shared by the gfx950 GEMM kernels (integer and MX): LDS chunk swizzles,
// explicit vmcnt waits, a fence-free barrier, direct global->LDS loads, the tile order
// over XCDs and the persistent grid size.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dev_common.h"

namespace vqk {

// Chunk swizzles: 16-byte chunk c of row r is stored at position c ^ swz(r).
// Both depend only on r & 15, so a fragment read of rows 16*blk + (lane & 15) can use
// the lane's constant swizzle for every block.
__device__ __forceinline__ int swz64(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz32(int r) { return (r >> 3) & 1; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS at ldst + 16 * lane (ldst is
// wave-uniform).  Written as inline asm: the compiler cannot tell these LDS writes from
// the fragment reads of other stages and would otherwise drain every outstanding load
// (vmcnt(0)) before each read.  The instruction has no register outputs (the data goes
// to LDS), its completion is tracked with explicit vmcnt waits, and m0 is set inside
// the statement; no other code of this kernel reads m0.
__device__ __forceinline__ void dma16(const void* gsrc, void* ldst) {
  const unsigned la = (unsigned)(size_t)(lds_ptr_t)ldst;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(la), "v"(gsrc) : "memory");
}

// Four consecutive float32 outputs of one row (16 B when aligned and whole).
__device__ __forceinline__ void store4_f32(void* y, int64_t off, const float v[4], int cnt, bool vec) {
  float* p = reinterpret_cast<float*>(y) + off;
  if (vec && cnt == 4) {
    *reinterpret_cast<v4f*>(p) = v4f{v[0], v[1], v[2], v[3]};
  } else {
    for (int i = 0; i < cnt; ++i) p[i] = v[i];
  }
}

// Block b -> tile (tm, tn): contiguous tile ranges per XCD, grouped order inside.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int q = T >> 3, r = T & 7;
  const int x = b & 7, j = b >> 3;
  const int t = x * q + min(x, r) + j;
  constexpr int GROUP = 8;
  const int width = GROUP * tiles_n;
  const int first_m = (t / width) * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  tm = first_m + (t % width) % gsz;
  tn = (t % width) / gsz;
}

// ---- remainder split: exchange of a K range's partial accumulators.
// A lane's accumulators (MB x NB blocks of 16 32-bit values) travel as 64-bit words; word
// w of thread t sits at part[w * nt + t], so each wave-wide access is contiguous.  The
// words move with device-scope relaxed atomic stores and loads (write-through, no L2
// write-back or invalidate), a store being performed device-wide once vmcnt reaches 0.
template <typename V, int MB, int NB>
__device__ __forceinline__ void split_publish(uint64_t* part, int nt, int tid, const V (&acc)[MB][NB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // Elements are copied out first: a bit cast applied to a vector element in place
        // reads the vector's first element whatever the index.
        const auto lo = acc[mb][nb][2 * i], hi = acc[mb][nb][2 * i + 1];
        const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, lo) | ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
        __hip_atomic_store(part + (int64_t)((mb * NB + nb) * 8 + i) * nt + tid, v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
}

template <typename V, int MB, int NB>
__device__ __forceinline__ void split_accumulate(const uint64_t* part, int nt, int tid, V (&acc)[MB][NB]) {
  typedef decltype(acc[0][0][0] + 0) E;  // int or float
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    // All words of a row of blocks are requested before any is added: these loads bypass
    // the L2, and issued one at a time each would wait out the full memory latency.
    uint64_t v[NB][8];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[nb][i] = __hip_atomic_load(part + (int64_t)((mb * NB + nb) * 8 + i) * nt + tid, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[mb][nb][2 * i] += __builtin_bit_cast(E, (uint32_t)v[nb][i]);
        acc[mb][nb][2 * i + 1] += __builtin_bit_cast(E, (uint32_t)(v[nb][i] >> 32));
      }
  }
}

// After this workgroup's partial is published: bump the tile's arrival count once the
// stores are performed; true (for the whole workgroup) in the last of `parts` arrivals.
__device__ __forceinline__ bool split_arrive(int32_t* cnt, int parts, int* s_flag) {
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == parts - 1;
  __syncthreads();
  return *s_flag != 0;
}

// The last arrival, having added the other partials, leaves the count at zero.
__device__ __forceinline__ void split_reset(int32_t* cnt) {
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace vqk

namespace vq_internal {

// One persistent workgroup per compute unit (each needs most of a CU's LDS).  The count
// is read once per process (thread-safe static initialization); without a visible device
// it is taken as MI355X's 256.
inline int persistent_blocks() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    return cus;
  }();
  return n;
}

}  // namespace vq_internal
