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

// Swizzle and direct-load lane mapping of a row width: a 1 KB load covers 1024/W rows,
// lane -> (row, 16-byte position), the position holding chunk position ^ swz(row).
// A 16-lane group of 16-byte fragment reads covers the 64 banks once when the chunks of
// its 16 rows land on distinct 16-byte bank groups: with 128-byte rows, rows r and r+1
// start half a bank line apart, so the eight chunk positions are spread over r >> 1.
template <int W>
__device__ __forceinline__ int swz_row(int r) {
  if constexpr (W == 32) return swz32(r);
  else if constexpr (W == 64) return swz64(r);
  else return (r >> 1) & 7;
}
template <int W>
__device__ __forceinline__ void dma_lane(int q, int lane, int& row, int& col) {
  constexpr int LPR = W / 16;  // lanes per row
  row = (1024 / W) * q + lane / LPR;
  col = 16 * ((lane % LPR) ^ swz_row<W>(row));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// The same barrier with no instruction moved across it by the scheduler: the ping-pong
// schedules rely on the phases staying where they are written.
__device__ __forceinline__ void sched_barrier_all() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

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

// 4 bytes per lane from global memory straight into LDS at ldst + 4 * lane (the same
// form as dma16, one dword per lane): used for the tile's scales.
__device__ __forceinline__ void dma4(const void* gsrc, void* ldst) {
  const unsigned la = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_ptr_t)ldst);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(la), "v"(gsrc) : "memory");
}

// Two float32 values rounded (to nearest even) to a pair of 16-bit values in one dword,
// the first in the low half: one v_cvt_pk_{bf16,f16}_f32.  The inputs are fenced so that
// each is a rounded float32 product before it is narrowed.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <int OUT_DT>
__device__ __forceinline__ unsigned cvt_pair(float a, float b) {
  const f32x2_t v = {f32_fence(a), f32_fence(b)};
  if constexpr (OUT_DT == DT_BF16) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
  } else {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2_t));
  }
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

// Work item w of a persistent GEMM with the remainder split: items [0, dp_items) are
// whole tiles, the rest are `split` consecutive K ranges of each remaining tile.  Written
// with selects only: with an if/else that assigns the fields on both sides, the compiler
// merged the stores into a store through a selected address and kept the fields in
// scratch memory, whose reload at every tile start drained all outstanding loads.
struct WorkItem {
  int tile;   // tile index for tile_of
  int kb0;    // first K stage
  int nks;    // K stages of the item
  int part;   // K range (-1: whole tile)
  int rslot;  // index among the remaining tiles (0 for a whole tile)
};
__device__ __forceinline__ WorkItem item_of(int w, int dp_items, int split, int nk) {
  const bool whole = w < dp_items;
  const int j = whole ? 0 : w - dp_items;
  const int rs = j / split;
  const int pt = j - rs * split;
  const int b0 = pt * nk / split;
  WorkItem it;
  it.tile = whole ? w : dp_items + rs;
  it.kb0 = whole ? 0 : b0;
  it.nks = whole ? nk : (pt + 1) * nk / split - b0;
  it.part = whole ? -1 : pt;
  it.rslot = rs;
  return it;
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
// words are plain stores and loads; the tile's arrival counter orders them by the memory
// model: each workgroup bumps it with a device-scope release (after a workgroup barrier
// that orders every wave's stores before it), and the last arrival takes a device-scope
// acquire fence before anyone reads the other partials (the barrier after it orders the
// reads of every wave after the fence).
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
        part[(int64_t)((mb * NB + nb) * 8 + i) * nt + tid] = v;
      }
}

template <typename V, int MB, int NB>
__device__ __forceinline__ void split_accumulate(const uint64_t* part, int nt, int tid, V (&acc)[MB][NB]) {
  typedef decltype(acc[0][0][0] + 0) E;  // int or float
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    // All words of a row of blocks are requested before any is added: the partial was
    // written back past the L2 by its publisher, and loads issued one at a time would each
    // wait out the full memory latency.
    uint64_t v[NB][8];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[nb][i] = part[(int64_t)((mb * NB + nb) * 8 + i) * nt + tid];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[mb][nb][2 * i] += __builtin_bit_cast(E, (uint32_t)v[nb][i]);
        acc[mb][nb][2 * i + 1] += __builtin_bit_cast(E, (uint32_t)(v[nb][i] >> 32));
      }
  }
}

// After this workgroup's partial is stored: bump the tile's arrival count with a release
// (every wave's stores done first); true (for the whole workgroup) in the last of `parts`
// arrivals, which acquires before the barrier that lets its waves read the partials.
__device__ __forceinline__ bool split_arrive(int32_t* cnt, int parts, int* s_flag) {
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == parts - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_flag = last;
  }
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
