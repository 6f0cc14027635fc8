// Integer GEMM with fused dequantization for gfx950 (int8 MFMA).
//
// Q-ARVD (aitrends.kr), Technical details: quantized activations and weights meet in a
// GEMM whose integer result is dequantized with the activation scale (per tensor or per
// token) times the per-output-channel weight scale; Methodology: the outlier input
// channels carry their own scales (Q_dual), so the K sum splits into two partitions
// with separate scale pairs.  6Bit-Diffusion (gist.science arXiv 2603.18742),
// Methodology B.1: 4-bit weights; gfx950 has no 4-bit integer MFMA, so 4-bit weights
// are unpacked to int8 operands (each nibble placed in the high half of its byte, i.e.
// 16 * code, and the accumulator shifted right by 4 afterwards, which is exact).
//
// Tiling: a 512-thread workgroup (8 waves, two per SIMD) computes a 256 (M) x 256 (N)
// tile; the waves form a 2 (M) x 4 (N) grid, each wave 128 x 64 as 4 x 2 blocks of
// v_mfma_i32_32x32x32_i8 (on gfx950 this form keeps the matrix pipe busier than
// 16x16x64).  Two waves per SIMD let one wave's MFMAs cover the other's waits, and they
// double the LDS read rate a CU reaches (one wave per SIMD cannot issue reads fast
// enough).  The weights are the MFMA's A operand and the activations its B operand, so
// each group of four accumulators of a lane holds four consecutive output columns of one
// row.
//
// Pipeline: K advances 64 codes per step through a ring of NST LDS stages filled by
// gfx950's direct global->LDS loads (global_load_lds_dwordx4) issued NST-1 steps ahead,
// so several steps of HBM/L2 latency hide behind the MFMAs without staging registers.
// Each wave waits for its own loads with an explicit vmcnt, then a plain s_barrier (no
// fence) publishes the stage to the other waves.  LDS rows are dense (64 B of int8
// codes, 32 B of packed nibbles) with the 16-byte chunks XOR-swizzled by the row index
// so that the 16-row fragment reads hit distinct banks.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2; block b is mapped so that every XCD walks a contiguous range of tiles in a grouped
// order (8 M-tiles per sweep over N), keeping the A and B slices it reuses in its L2.
//
// Remainder split: the tiles fill whole rounds of the persistent grid except the last
// round, which would leave most CUs idle.  With a workspace, each remaining tile is split
// into S ranges of K stages handled by different workgroups; each stores its int32
// partial tile, then bumps an atomic count with a device-scope release, and the
// workgroup that arrives last acquires, adds the other partials and runs the epilogue.
// Integer sums are exact in any order, so the result is bit-identical to the unsplit
// tile, and no workgroup ever waits for another.  The last arrival resets the tile's counter, so
// the workspace is left zeroed for the next call.
#include <mutex>
#include <type_traits>

#include "dev_common.h"
#include "gemm_common.h"
#include "vq_internal.h"

namespace vqk {

constexpr int BM = 256, BN = 256;
constexpr int64_t QGEMM_WS_COUNTERS = 4096;  // arrival counters of up to 1024 remaining tiles
// Largest remainder-split workspace the scratch-free entry serves (40 MiB): the counters
// plus two 256 KB partials for each of up to 159 remaining tiles.
constexpr int64_t QGEMM_SCRATCH_BYTES = (int64_t)40 << 20;
constexpr int NT = 512;           // threads per workgroup
constexpr int WTM = 128, WTN = 64;  // wave tile
constexpr int MBLK = WTM / 32, NBLK = WTN / 32;

// A ring stage holds H k-halves of 32 codes (BK = 32 H codes); one barrier per stage.
template <int BBITS, int H>
struct GCfg {
  static constexpr int BK = 32 * H;
  static constexpr int A_ROW = BK;                            // int8 codes
  static constexpr int B_ROW = BBITS == 8 ? BK : BK / 2;      // int8 codes or packed nibbles
  static constexpr int A_BYTES = BM * A_ROW;
  static constexpr int B_BYTES = BN * B_ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int NST = H == 4 ? 3 : (BBITS == 8 ? 4 : 5);
  static constexpr int LA = A_BYTES / (NT * 16);  // 16-byte loads per thread per stage
  static constexpr int LB = B_BYTES / (NT * 16);
  static constexpr int L = LA + LB;
};


struct GArgs {
  const int8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* y;
  int32_t* accd;
  int m, n, kp, k0;
  int64_t ldy;
  int sa_tok;
  int vec_store;  // 16-byte stores are aligned (y 16-byte aligned, row pitch a multiple of 16 B)
  int tiles_m, tiles_n;
  int dp_items;      // whole tiles: items [0, dp_items) are tiles [0, dp_items)
  int split;         // K ranges per remaining tile (1: no split)
  int items;         // dp_items + (tiles - dp_items) * split
  int32_t* ws_cnt;   // [tiles - dp_items] arrival counters (zero between calls)
  uint64_t* ws_part;  // [(tiles - dp_items) * split][64][NT] partial accumulators (int32 pairs)
  int64_t b_kp;  // weights in 64-byte K pieces: bytes from one piece to the next (64 n)
};

// Weight addressing, fixed per kernel instance (KB: the layout of 64-byte K pieces, piece
// j of every row stored together).  Bytes from one row to the next, and the offset of byte
// c of a row from the row's first byte.
template <bool KB>
__device__ __forceinline__ int64_t wrow(const GArgs& g, int bbits) {
  return KB ? 64 : (bbits == 8 ? g.kp : g.kp / 2);
}
template <bool KB>
__device__ __forceinline__ int64_t wofs(const GArgs& g, int c) {
  if constexpr (KB) return (int64_t)(c >> 6) * g.b_kp + (c & 63);
  else return c;
}

__device__ __forceinline__ v4i unpack_int4x16(u2v w) {
  const unsigned h0 = w.x & 0xF0F0F0F0u, l0 = (w.x << 4) & 0xF0F0F0F0u;
  const unsigned h1 = w.y & 0xF0F0F0F0u, l1 = (w.y << 4) & 0xF0F0F0F0u;
  v4i r;
  r.x = (int)__builtin_amdgcn_perm(h0, l0, 0x05010400u);
  r.y = (int)__builtin_amdgcn_perm(h0, l0, 0x07030602u);
  r.z = (int)__builtin_amdgcn_perm(h1, l1, 0x05010400u);
  r.w = (int)__builtin_amdgcn_perm(h1, l1, 0x07030602u);
  return r;
}

template <int BBITS, int OUT_DT, bool DUAL, int H, bool KB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_qgemm(GArgs g) {
  static_assert(!DUAL || H == 2 || (H == 4 && BBITS == 4),
                "the outlier partition is staged in 64-code stages, or in one 128-code stage");
  using C = GCfg<BBITS, H>;
  constexpr int BK = C::BK;
  constexpr int P = DUAL ? 2 : 1;
  constexpr bool HALF_OUT = OUT_DT != DT_F32;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NST * C::STAGE];
  __shared__ float s_sa[2][P][BM];
  __shared__ float s_sb[2][P][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // wave grid 2 (M) x 4 (N)
  const int nk = g.k0 / BK;
  __shared__ int s_last;

  // ---- direct-load assignment: instruction q of this wave fills 1 KB of a stage.
  int ra[C::LA], rb[C::LB];  // tile-local rows loaded by this lane
  int la_off[C::LA], lb_off[C::LB], ca[C::LA], cb[C::LB];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int q = wave * C::LA + i;
    dma_lane<C::A_ROW>(q, lane, ra[i], ca[i]);
    la_off[i] = q * 1024;
  }
#pragma unroll
  for (int i = 0; i < C::LB; ++i) {
    const int q = wave * C::LB + i;
    dma_lane<C::B_ROW>(q, lane, rb[i], cb[i]);
    lb_off[i] = C::A_BYTES + q * 1024;
  }
  const int8_t* ga[C::LA];
  const uint8_t* gb[C::LB];
  int m0 = 0, n0 = 0;
  int kb0 = 0, nks = nk;    // the item's first stage and stage count
  int part = -1, rslot = 0;  // K range of a split tile (-1: whole tile) and its remainder index
  auto set_tile = [&](int w) {
    const WorkItem it = item_of(w, g.dp_items, g.split, nk);
    kb0 = it.kb0;
    nks = it.nks;
    part = it.part;
    rslot = it.rslot;
    int tm, tn;
    tile_of(it.tile, g.tiles_m, g.tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) ga[i] = g.a + (int64_t)min(m0 + ra[i], g.m - 1) * g.kp + ca[i];
#pragma unroll
    for (int i = 0; i < C::LB; ++i) gb[i] = g.b + (int64_t)min(n0 + rb[i], g.n - 1) * wrow<KB>(g, BBITS) + cb[i];
  };
  auto issue = [&](int k, int slot) {
    uint8_t* base = lds + slot * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) dma16(ga[i] + k, base + la_off[i]);
    const int kb = BBITS == 8 ? k : k / 2;
#pragma unroll
    for (int i = 0; i < C::LB; ++i) dma16(gb[i] + wofs<KB>(g, kb), base + lb_off[i]);
  };
  // The outlier partition [k0, kp) of 64 or 128 codes as one 128-code stage: columns past
  // the partition wrap to its start (mask), so every load stays inside the row's
  // partition; the wrapped chunks are never read.
  auto issue_part = [&](int amask, int bmask) {
#pragma unroll
    for (int i = 0; i < C::LA; ++i) dma16(ga[i] - ca[i] + (ca[i] & amask) + g.k0, lds + la_off[i]);
#pragma unroll
    for (int i = 0; i < C::LB; ++i) dma16(gb[i] - cb[i] + (cb[i] & bmask) + wofs<KB>(g, g.k0 / 2), lds + lb_off[i]);
  };
  auto issue_prologue = [&]() {
#pragma unroll
    for (int s = 0; s < C::NST - 1; ++s)
      if (s < nks) issue((kb0 + s) * BK, s);
  };
  // Scales of a tile's rows and columns.  With 64-code stages they go straight to LDS by
  // direct loads (64 lanes x 4 bytes per instruction, P per wave), issued before the
  // tile's first stage so that the waits for that stage cover them: loaded into registers
  // instead, they are the only loads the compiler tracks, and it drains every direct load
  // in flight (vmcnt(0)) before their first use.  The 128-code-stage kernels, whose scalar
  // registers are spoken for by their wider ring, load them into registers early and write
  // them to LDS late.
  constexpr bool SC_DMA = H == 2;
  // Register path: threads below BM hold a row scale, the others a column scale, both in
  // sc[] (one array: conditional stores to two arrays were merged through a selected
  // address and kept in scratch memory).
  float sc[P];
  const int srow = tid & (BM - 1);  // register path: each thread loads one row or column scale
  auto load_scales = [&](int buf) {
    if constexpr (SC_DMA) {
      const int r = 64 * (wave & 3) + lane;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (wave < 4) {
          const float* src = g.sa_tok ? g.sa + (int64_t)min(m0 + r, g.m - 1) * P + p : g.sa + p;
          dma4(src, &s_sa[buf][p][64 * wave]);
        } else {
          dma4(g.sb + (int64_t)min(n0 + r, g.n - 1) * P + p, &s_sb[buf][p][64 * (wave - 4)]);
        }
      }
    } else {
      const float* src = tid < BM ? (g.sa_tok ? g.sa + (int64_t)min(m0 + srow, g.m - 1) * P : g.sa)
                                  : g.sb + (int64_t)min(n0 + srow, g.n - 1) * P;
#pragma unroll
      for (int p = 0; p < P; ++p) sc[p] = src[p];
    }
  };
  auto store_scales = [&](int buf) {
    if constexpr (!SC_DMA) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (tid < BM)
          s_sa[buf][p][srow] = sc[p];
        else
          s_sb[buf][p][srow] = sc[p];
      }
    }
  };

  // ---- fragment offsets (per lane, constant): rows 32*blk + (lane & 31), k-half h:
  // 16-byte chunk 2h + (lane >> 5) of the int8 row; 8 bytes (lane >> 5) of chunk h of a
  // packed 4-bit row.
  const int rl = lane & 31;
  const int kc = lane >> 5;
  int fa[H], fb[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    fa[h] = (wm * WTM + rl) * C::A_ROW + 16 * ((2 * h + kc) ^ swz_row<C::A_ROW>(rl));
    if constexpr (BBITS == 8) {
      fb[h] = C::A_BYTES + (wn * WTN + rl) * C::B_ROW + 16 * ((2 * h + kc) ^ swz_row<C::B_ROW>(rl));
    } else {
      fb[h] = C::A_BYTES + (wn * WTN + rl) * C::B_ROW + 16 * (h ^ swz_row<C::B_ROW>(rl)) + 8 * kc;
    }
  }
  auto afrag = [&](int slot, int h, int mb) -> v4i {
    return *reinterpret_cast<const v4i*>(lds + slot * C::STAGE + fa[h] + mb * 32 * C::A_ROW);
  };
  // B fragment as stored (int8 codes, or the 8 packed bytes in .xy for 4-bit weights).
  auto braw = [&](int slot, int h, int nb) -> v4i {
    if constexpr (BBITS == 8) {
      return *reinterpret_cast<const v4i*>(lds + slot * C::STAGE + fb[h] + nb * 32 * C::B_ROW);
    } else {
      const u2v w = *reinterpret_cast<const u2v*>(lds + slot * C::STAGE + fb[h] + nb * 32 * C::B_ROW);
      return v4i{(int)w.x, (int)w.y, 0, 0};
    }
  };
  auto bval = [&](v4i raw) -> v4i {
    if constexpr (BBITS == 8) {
      return raw;
    } else {
      return unpack_int4x16(u2v{(unsigned)raw.x, (unsigned)raw.y});
    }
  };
  auto bfrag = [&](int slot, int h, int nb) -> v4i { return bval(braw(slot, h, nb)); };

  v16i acc[MBLK][NBLK];

  // Fragments of one k-half (32 codes) of a stage.
  struct Frag {
    v4i a[MBLK];
    v4i b[NBLK];
  };
  auto load_half = [&](int slot, int h, Frag& f) {
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) f.b[nb] = braw(slot, h, nb);
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) f.a[mb] = afrag(slot, h, mb);
  };
  auto mma_half = [&](const Frag& f) {
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
      const v4i bv = bval(f.b[nb]);
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bv, f.a[mb], acc[mb][nb], 0, 0, 0);
    }
  };
  auto wait_loads = [&](int later) {  // at most `later` load groups may stay in flight
    if (later >= 3) {
      wait_vmcnt<3 * C::L>();
    } else if (later == 2) {
      wait_vmcnt<2 * C::L>();
    } else if (later == 1) {
      wait_vmcnt<C::L>();
    } else {
      wait_vmcnt<0>();
    }
  };

  // Persistent loop: block b takes tiles b, b + gridDim.x, ...  The next tile's scales
  // and first NST-1 stages are requested before the current tile's epilogue, so its
  // load latency and this tile's output stores overlap.
  int vt = blockIdx.x;
  if (vt >= g.items) return;
  set_tile(vt);
  if constexpr (SC_DMA) {
    load_scales(0);  // ahead of the first stage, whose waits then cover it
    issue_prologue();
  } else {
    issue_prologue();
    load_scales(0);
    store_scales(0);
  }
  int buf = 0;
  for (;;) {
#pragma unroll
    for (int i = 0; i < MBLK; ++i)
#pragma unroll
      for (int j = 0; j < NBLK; ++j) acc[i][j] = v16i{};

    // Software pipeline over k-halves.  Stage kt holds H k-halves; each half's MFMAs run
    // while the next half's fragments are read.  Before the last half every wave waits for
    // its loads of stage kt+1 and meets the others at a barrier, which publishes stage
    // kt+1 and certifies that stage kt-1 is no longer read; that stage then receives stage
    // kt+NST-1, and the first half of stage kt+1 is read while the last half of stage kt
    // runs.  (H is even, so the next stage's first half lands in F[0].)
    Frag F[2];
    wait_loads(min(C::NST - 2, nks - 1));
    barrier_nofence();
    load_half(0, 0, F[0]);
    int kt = 0, slot = 0;
    // Order of a half-step's MFMAs and next-half fragment reads.  With 64-code stages
    // (two halves) reads go one after each MFMA from the first on; with 128-code stages
    // the two spare MFMAs go first.  Measured at the workload shapes: issuing the reads
    // any earlier was 1-6% slower, and the later order for 64-code stages 1% slower at
    // 17776 x 3072 x 12288, while it made 17776 x 12288 x 3072 (128-code stages) 2.7%
    // faster.
    auto interleave = [&]() {
      if constexpr (H == 4)
        __builtin_amdgcn_sched_group_barrier(0x008, MBLK * NBLK - (MBLK + NBLK), 0);
#pragma unroll
      for (int i = 0; i < MBLK + NBLK; ++i) {
        if constexpr (H == 4) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
      }
      if constexpr (H != 4)
        __builtin_amdgcn_sched_group_barrier(0x008, MBLK * NBLK - (MBLK + NBLK), 0);
    };
    // Steady state: every stage refills a stage and keeps NST-3 load groups in flight.
    // The body has no branch, so the waits the compiler inserts for the fragments stay
    // partial (lgkmcnt of the reads issued later) instead of draining all LDS reads.
    for (; kt < nks - (C::NST - 1); ++kt) {
      const int next = slot + 1 == C::NST ? 0 : slot + 1;
      const int refill = slot == 0 ? C::NST - 1 : slot - 1;
#pragma unroll
      for (int h = 0; h < H - 1; ++h) {
        load_half(slot, h + 1, F[(h + 1) & 1]);
        mma_half(F[h & 1]);
        interleave();
      }
      wait_vmcnt<(C::NST - 3) * C::L>();
      barrier_nofence();
      issue((kb0 + kt + C::NST - 1) * BK, refill);
      load_half(next, 0, F[0]);
      mma_half(F[(H - 1) & 1]);
      interleave();
      slot = next;
    }
    // Last NST-1 stages: nothing left to load; fewer groups in flight each stage.
    for (; kt < nks; ++kt) {
      const int next = slot + 1 == C::NST ? 0 : slot + 1;
#pragma unroll
      for (int h = 0; h < H - 1; ++h) {
        load_half(slot, h + 1, F[(h + 1) & 1]);
        mma_half(F[h & 1]);
      }
      if (kt + 1 < nks) {
        wait_loads(nks - 2 - kt);
        barrier_nofence();
        load_half(next, 0, F[0]);
      }
      mma_half(F[(H - 1) & 1]);
      slot = next;
    }

    // ------------------------------------------------------------ remainder split
    if (part >= 0) {
      // Every item after a split one is split too and belongs to another workgroup, so
      // this is the block's last item and nothing is in flight.  The partials are plain
      // stores; the count is bumped with a device-scope release and the last arrival
      // acquires before it loads the other partials (split_arrive).  Only these last-round
      // items pay the release's L2 write-back and the acquire's invalidate.
      split_publish(g.ws_part + (int64_t)(rslot * g.split + part) * (64 * NT), NT, tid, acc);
      if (!split_arrive(&g.ws_cnt[rslot], g.split, &s_last)) break;
      for (int p2 = 0; p2 < g.split; ++p2)
        if (p2 != part) split_accumulate(g.ws_part + (int64_t)(rslot * g.split + p2) * (64 * NT), NT, tid, acc);
      split_reset(&g.ws_cnt[rslot]);
    }

    // ------------------------------------------------------------ epilogue
    const int nvt = vt + (int)gridDim.x;
    const bool has_next = nvt < g.items;
    const int cm0 = m0, cn0 = n0;  // this tile
    barrier_nofence();             // every wave is done with the ring
    int steps1 = 0;
    if constexpr (DUAL) {
      // Outlier partition [k0, kp): at most two 64-code steps, staged in stages 0-1.
      if constexpr (H == 2) {
        steps1 = (g.kp - g.k0) / BK;
        issue(g.k0, 0);
        if (steps1 > 1) issue(g.k0 + BK, 1);
      } else {
        steps1 = (g.kp - g.k0) / 32;  // k-halves of the partition: 2 or 4
        issue_part(g.kp - g.k0 - 1, (g.kp - g.k0) / 2 - 1);
      }
      wait_vmcnt<0>();
      barrier_nofence();
    } else {
      if (has_next) {
        set_tile(nvt);
        load_scales(buf ^ 1);
        issue_prologue();
      }
    }

    // Output layout of a 32 x 32 block: lane holds column m = lane & 31 (activation row)
    // and, for group q = 0..3, rows n = 8q + 4 * (lane >> 5) + 0..3 (weight rows).  16-bit
    // outputs leave straight from registers, 16 B per lane (32 contiguous bytes per row
    // and instruction); a detour through LDS for full-row stores measured slower.
    const int mrow = wm * WTM + (lane & 31);
    const int ncol = wn * WTN + 4 * (lane >> 5);
    const int64_t mn = (int64_t)g.m * g.n;
    typedef typename std::conditional<OUT_DT == DT_BF16, __bf16, _Float16>::type h_t;
    // A tile inside the output with aligned rows stores without per-lane guards.
    const bool full = g.vec_store && cm0 + BM <= g.m && cn0 + BN <= g.n && !g.accd;

    if (!DUAL && g.accd) {  // test hook: the int32 accumulators (with the 4-bit shift), before any scaling
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = cm0 + mrow + mb * 32;
            const int n = cn0 + ncol + nb * 32 + 8 * (e >> 2) + (e & 3);
            int a0 = acc[mb][nb][e];
            if constexpr (BBITS == 4) a0 >>= 4;
            if (m < g.m && n < g.n) g.accd[(int64_t)m * g.n + n] = a0;
          }
    }
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
      const int ml = mrow + mb * 32;
      const int m = cm0 + ml;
      float sa0[P];
#pragma unroll
      for (int p = 0; p < P; ++p) sa0[p] = s_sa[buf][p][ml];
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) {
        v16i t1 = v16i{};
        if constexpr (DUAL) {
          if constexpr (H == 2) {
#pragma unroll
            for (int s1 = 0; s1 < 2; ++s1) {
              if (s1 < steps1) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                  t1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(bfrag(s1, h, nb), afrag(s1, h, mb), t1, 0, 0, 0);
              }
            }
          } else {
#pragma unroll
            for (int h = 0; h < H; ++h)
              if (h < steps1)
                t1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(bfrag(0, h, nb), afrag(0, h, mb), t1, 0, 0, 0);
          }
        }
        unsigned pk[8];  // 16-bit outputs of group q as pairs: columns 8q + 4 * (lane >> 5) + 0..3
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = ncol + nb * 32 + 8 * q;
          const int n = cn0 + nl;
          const v4f sb0 = *reinterpret_cast<const v4f*>(&s_sb[buf][0][nl]);
          v4f sb1 = sb0;
          if constexpr (DUAL) sb1 = *reinterpret_cast<const v4f*>(&s_sb[buf][1][nl]);
          float out[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int a0 = acc[mb][nb][4 * q + r];
            if constexpr (BBITS == 4) a0 >>= 4;
            const float t0 = sa0[0] * sb0[r];
            float yv = (float)a0 * t0;
            if constexpr (DUAL) {
              int a1 = t1[4 * q + r];
              if constexpr (BBITS == 4) a1 >>= 4;
              const float tt = sa0[P - 1] * sb1[r];
              const float y1 = (float)a1 * tt;
              yv = yv + y1;
              if (g.accd && m < g.m && n + r < g.n) g.accd[mn + (int64_t)m * g.n + n + r] = a1;
            }
            if (DUAL && g.accd && m < g.m && n + r < g.n) g.accd[(int64_t)m * g.n + n + r] = a0;
            out[r] = yv;
          }
          if constexpr (HALF_OUT) {
            pk[2 * q] = cvt_pair<OUT_DT>(out[0], out[1]);
            pk[2 * q + 1] = cvt_pair<OUT_DT>(out[2], out[3]);
          } else {
            if (m < g.m && n < g.n) store4_f32(g.y, (int64_t)m * g.ldy + n, out, min(4, g.n - n), g.vec_store != 0);
          }
        }
        if constexpr (HALF_OUT) {
          // Groups (q, q+2) of the two half-waves are exchanged so that each lane holds eight
          // consecutive columns: lanes 0-31 columns 16pr + 0..7, lanes 32-63 16pr + 8..15.
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const auto s0 = __builtin_amdgcn_permlane32_swap(pk[4 * pr], pk[4 * pr + 2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(pk[4 * pr + 1], pk[4 * pr + 3], false, false);
            const u4v w = {s0[0], s1[0], s0[1], s1[1]};
            const int no = cn0 + wn * WTN + nb * 32 + 16 * pr + 8 * (lane >> 5);
            h_t* dst = reinterpret_cast<h_t*>(g.y) + (int64_t)m * g.ldy + no;
            if (full) {
              *reinterpret_cast<u4v*>(dst) = w;
            } else if (m < g.m && no < g.n) {
              if (g.vec_store && no + 8 <= g.n) {
                *reinterpret_cast<u4v*>(dst) = w;
              } else {
                for (int e = 0; e < 8 && no + e < g.n; ++e) {
                  const unsigned d = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
                  dst[e] = __builtin_bit_cast(h_t, (unsigned short)(d >> (16 * (e & 1))));
                }
              }
            }
          }
        }
      }
    }

    if (!has_next) break;
    if constexpr (DUAL) {
      barrier_nofence();  // stages 0-1 (outlier partition) are no longer read
      set_tile(nvt);
      load_scales(buf ^ 1);
      issue_prologue();
    }
    store_scales(buf ^ 1);  // register path: the next tile's epilogue reads them after several barriers
    buf ^= 1;
    vt = nvt;
  }
}

// ---------------------------------------------------------------------------------------
// Ping-pong schedule for int8 weights without an outlier partition and without the
// remainder split (the W8A8 layers).  The two waves of a SIMD alternate between a memory
// phase (the fragment reads of a whole 64-code stage and the refill loads) and a compute
// phase (that stage's 16 MFMAs from registers), so each matrix pipe is fed by one wave
// while the other reads LDS.  Waves 0-3 (one per SIMD) lead and waves 4-7 follow one
// phase behind; two barriers per stage keep the phases apart.  The ring holds 4 stages,
// refilled 2 stages ahead: a refill goes into the slot of the stage read 2 stages
// earlier, whose last reader finished before the barrier that precedes the refill.
// Measured at the fused-QKV shape (17776 x 1920 x 5760): 7-8% faster than the
// interleaved schedule of k_qgemm.
namespace ppc {
constexpr int NST = 4, D = 2;
constexpr int ROW = 64;                 // 64 int8 codes per row and stage
constexpr int A_BYTES = BM * ROW;       // activations of a stage (16 KB)
constexpr int STAGE = A_BYTES + BN * ROW;
constexpr int LA = A_BYTES / (NT * 16);  // direct loads per wave per operand and stage (2)
constexpr int L = 2 * LA;
}  // namespace ppc

template <int OUT_DT, bool KB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_qgemm_pp(GArgs g) {
  using namespace ppc;
  constexpr bool HALF_OUT = OUT_DT != DT_F32;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * STAGE];
  __shared__ float s_sa[2][BM];
  __shared__ float s_sb[2][BN];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // waves w and w + 4 share a SIMD
  const int wm = wave & 1, wn = wave >> 1;
  const int nk = g.k0 / ROW;

  int ra[LA], rb[LA], ca[LA], cb[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    dma_lane<ROW>(wave * LA + i, lane, ra[i], ca[i]);
    dma_lane<ROW>(wave * LA + i, lane, rb[i], cb[i]);
  }
  const int8_t* ga[LA];
  const uint8_t* gb[LA];
  int m0 = 0, n0 = 0;
  auto set_tile = [&](int t) {
    int tm, tn;
    tile_of(t, g.tiles_m, g.tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      ga[i] = g.a + (int64_t)min(m0 + ra[i], g.m - 1) * g.kp + ca[i];
      gb[i] = g.b + (int64_t)min(n0 + rb[i], g.n - 1) * wrow<KB>(g, 8) + cb[i];
    }
  };
  auto issue = [&](int k, int slot) {
    uint8_t* base = lds + slot * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i) dma16(ga[i] + k, base + (wave * LA + i) * 1024);
#pragma unroll
    for (int i = 0; i < LA; ++i) dma16(gb[i] + wofs<KB>(g, k), base + A_BYTES + (wave * LA + i) * 1024);
  };
  // Scales straight to LDS, one direct load per wave, ahead of the tile's first stage.
  auto load_scales = [&](int buf) {
    const int r = 64 * (wave & 3) + lane;
    if (wave < 4)
      dma4(g.sa_tok ? g.sa + min(m0 + r, g.m - 1) : g.sa, &s_sa[buf][64 * wave]);
    else
      dma4(g.sb + min(n0 + r, g.n - 1), &s_sb[buf][64 * (wave - 4)]);
  };
  const int rl = lane & 31, kc = lane >> 5;
  int fa[2], fb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    fa[h] = (wm * WTM + rl) * ROW + 16 * ((2 * h + kc) ^ swz64(rl));
    fb[h] = A_BYTES + (wn * WTN + rl) * ROW + 16 * ((2 * h + kc) ^ swz64(rl));
  }
  v16i acc[MBLK][NBLK];
  v4i fA[2][MBLK], fB[2][NBLK];
  auto read_stage = [&](int slot) {
    const uint8_t* base = lds + slot * STAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) fB[h][nb] = *reinterpret_cast<const v4i*>(base + fb[h] + nb * 32 * ROW);
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb) fA[h][mb] = *reinterpret_cast<const v4i*>(base + fa[h] + mb * 32 * ROW);
    }
  };
  auto compute = [&]() {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
          acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fB[h][nb], fA[h][mb], acc[mb][nb], 0, 0, 0);
  };
  auto lds_reads_done = [&]() { __builtin_amdgcn_s_waitcnt(0xC07F); };  // lgkmcnt(0)
  auto wait_groups = [&](int later) {  // at most `later` stages of loads in flight
    if (later >= 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
  };

  int t = blockIdx.x;
  if (t >= g.items) return;
  // Staggered start: every CU changes tiles at the same moment, so their output stores
  // would fall into the same few microseconds.  When the last round is partial, the
  // workgroups with one tile fewer than the others (a whole tile of slack) start late,
  // spread evenly over about a quarter of a tile (about 360 counter ticks per 64-code
  // stage plus the tile change; measured at the fused-QKV shape), so that the critical
  // path, the workgroups with the extra tile, is not delayed.
  {
    const int G = (int)gridDim.x, rem = g.items % G;
    if (rem > 0 && g.items > G && t >= rem) {
      const uint64_t quarter = (uint64_t)nk * 360 + 3100;
      const uint64_t delay = quarter * (uint64_t)(t - rem) / (uint64_t)(G - rem);
      const uint64_t s0 = __builtin_amdgcn_s_memtime();
      while (__builtin_amdgcn_s_memtime() - s0 < delay) __builtin_amdgcn_s_sleep(8);
    }
  }
  set_tile(t);
  load_scales(0);
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < nk) issue(s * ROW, s);
  typedef typename std::conditional<OUT_DT == DT_BF16, __bf16, _Float16>::type h_t;
  int buf = 0;
  // pend: the number of output stores (16, PD or 0) the previous tile issued after this
  // tile's first loads, so that waits for this tile's first stages leave them in flight
  // (vmcnt retires in order).
  int pend = 0;
  // The stores of the last NDEF / 4 row blocks of a whole 16-bit tile are deferred into the next
  // tile's first NDEF stages, one per stage after that stage's own loads: all CUs finish
  // their tiles together, and storing a whole tile at once made every CU's tile change
  // wait for the same burst of writes.  dq holds their payloads, dptr the first one's
  // address; dcnt is NDEF while they are pending, else 0.
  constexpr int NDEF = 4;
  constexpr int MB_DEF = MBLK - NDEF / 4;  // first deferred row block
  constexpr int PD = 4 * NBLK * MBLK / 2 - NDEF;  // stores issued at a tile change that defers (of 16)
  u4v dq[NDEF];
  h_t* dptr = nullptr;
  int dcnt = 0;
  const int64_t d_mb = (int64_t)32 * g.ldy;  // elements from one row block to the next
  auto def_store = [&](int j) {  // deferred store j = 4 * (mb - MB_DEF) + 2 * nb + pr
    *reinterpret_cast<u4v*>(dptr + (j >> 2) * d_mb + ((j >> 1) & 1) * 32 + (j & 1) * 16) = dq[j];
  };
  // One K stage of the ping-pong loop.  wsel: loads and stores allowed in flight beyond
  // the next stage's own loads (0; 1: a deferred store issued in the previous stage;
  // PD or 16: the previous tile's last stores).
  auto stage = [&](int p, int wsel, int dj) {
    // memory phase (leaders: while the followers compute stage p - 1)
    read_stage(p % NST);
    issue((p + D) * ROW, (p + D) % NST);
    auto wait_next = [&]() {
      if (wsel == 16) wait_vmcnt<(D - 1) * L + 16>();
      else if (wsel == PD) wait_vmcnt<(D - 1) * L + PD>();
      else if (wsel == 1) wait_vmcnt<(D - 1) * L + 1>();
      else wait_vmcnt<(D - 1) * L>();
    };
    if (grp == 1) wait_next();
    lds_reads_done();
    sched_barrier_all();
    // compute phase
    compute();
    if (grp == 0) wait_next();
    if (dj >= 0) def_store(dj);
    sched_barrier_all();
  };
  for (;;) {
#pragma unroll
    for (int i = 0; i < MBLK; ++i)
#pragma unroll
      for (int j = 0; j < NBLK; ++j) acc[i][j] = v16i{};
    if (pend == 16 && nk > D) wait_vmcnt<(D - 1) * L + 16>();
    else if (pend == PD && nk > D) wait_vmcnt<(D - 1) * L + PD>();
    else wait_groups(min(D, nk) - 1);
    sched_barrier_all();
    if (grp == 1) sched_barrier_all();
    int p = 0;
    // stage 0 waits past the previous tile's last stores (pend); stages 1 .. NDEF past the
    // deferred store of the stage before
    if (dcnt) {
#pragma unroll
      for (int j = 0; j < NDEF; ++j) stage(j, j == 0 ? pend : 1, j);
      p = NDEF;
      stage(p, 1, -1);
      ++p;
    } else if (p + D < nk) {
      stage(0, pend, -1);
      ++p;
    }
    for (; p + D < nk; ++p) stage(p, 0, -1);
    for (; p < nk; ++p) {
      read_stage(p % NST);
      const int later = nk - p - 2;
      if (grp == 1) wait_groups(later < 0 ? 0 : later);
      lds_reads_done();
      sched_barrier_all();
      compute();
      if (grp == 0) wait_groups(later < 0 ? 0 : later);
      sched_barrier_all();
    }
    if (grp == 0) sched_barrier_all();

    const int nt = t + (int)gridDim.x;
    const bool has_next = nt < g.items;
    const int cm0 = m0, cn0 = n0;
    if (has_next) {
      set_tile(nt);
      load_scales(buf ^ 1);
#pragma unroll
      for (int s = 0; s < D; ++s)
        if (s < nk) issue(s * ROW, s);
    }
    const bool full = g.vec_store && cm0 + BM <= g.m && cn0 + BN <= g.n && !g.accd;
    // deferral needs the next tile's loop to have more than NDEF + 1 stages before its tail
    const bool defer = HALF_OUT && has_next && full && nk > NDEF + 1 + D;
    pend = HALF_OUT && has_next && full ? (defer ? PD : 16) : 0;
    dcnt = defer ? NDEF : 0;
    if (defer) dptr = reinterpret_cast<h_t*>(g.y) + (int64_t)(cm0 + wm * WTM + rl + 32 * MB_DEF) * g.ldy + cn0 + wn * WTN + 8 * kc;
    // The lane's row and column scales, read once per tile and waited for once: its
    // columns are the same for every row block.
    float sa_r[MBLK];
    v4f sb_r[NBLK][4];
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) sa_r[mb] = s_sa[buf][wm * WTM + rl + mb * 32];
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) sb_r[nb][q] = *reinterpret_cast<const v4f*>(&s_sb[buf][wn * WTN + 4 * kc + nb * 32 + 8 * q]);
    if (g.accd) {  // test hook: the int32 accumulators, before any scaling
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = cm0 + wm * WTM + rl + mb * 32;
            const int n = cn0 + wn * WTN + 4 * kc + nb * 32 + 8 * (e >> 2) + (e & 3);
            if (m < g.m && n < g.n) g.accd[(int64_t)m * g.n + n] = acc[mb][nb][e];
          }
    }
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
      const int ml = wm * WTM + rl + mb * 32;
      const int m = cm0 + ml;
      const float sa0 = sa_r[mb];
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) {
        unsigned pk[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn * WTN + 4 * kc + nb * 32 + 8 * q;
          const int n = cn0 + nl;
          const v4f sb0 = sb_r[nb][q];
          float out[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int a0 = acc[mb][nb][4 * q + r];
            const float t0 = sa0 * sb0[r];
            out[r] = (float)a0 * t0;
          }
          if constexpr (HALF_OUT) {
            pk[2 * q] = cvt_pair<OUT_DT>(out[0], out[1]);
            pk[2 * q + 1] = cvt_pair<OUT_DT>(out[2], out[3]);
          } else {
            if (m < g.m && n < g.n) store4_f32(g.y, (int64_t)m * g.ldy + n, out, min(4, g.n - n), g.vec_store != 0);
          }
        }
        if constexpr (HALF_OUT) {
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const auto s0 = __builtin_amdgcn_permlane32_swap(pk[4 * pr], pk[4 * pr + 2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(pk[4 * pr + 1], pk[4 * pr + 3], false, false);
            const u4v w = {s0[0], s1[0], s0[1], s1[1]};
            const int no = cn0 + wn * WTN + nb * 32 + 16 * pr + 8 * kc;
            h_t* dst = reinterpret_cast<h_t*>(g.y) + (int64_t)m * g.ldy + no;
            if (defer && mb >= MB_DEF) {
              dq[4 * (mb - MB_DEF) + 2 * nb + pr] = w;
            } else if (full) {
              *reinterpret_cast<u4v*>(dst) = w;
            } else if (m < g.m && no < g.n) {
              if (g.vec_store && no + 8 <= g.n) {
                *reinterpret_cast<u4v*>(dst) = w;
              } else {
                for (int e = 0; e < 8 && no + e < g.n; ++e) {
                  const unsigned d = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
                  dst[e] = __builtin_bit_cast(h_t, (unsigned short)(d >> (16 * (e & 1))));
                }
              }
            }
          }
        }
      }
    }
    if (!has_next) break;
    buf ^= 1;
    t = nt;
  }
}

// ---------------------------------------------------------------------------------------
// Few-tile layers (int8 weights, no outlier partition): a 256 x 256 tile per CU would leave
// the part nearly idle and run every 64-code stage at the latency of the LDS ring, so each
// wave computes one 32 x 32 output block on its own, with its A and B fragments loaded
// straight from global memory into registers (16 codes per lane and operand per 32-deep
// MFMA, two batches of SMALL_KB steps in flight), no LDS and no barriers.
// Each workgroup is one wave, so the blocks spread over as many CUs as there are blocks
// (the operand loads of a 32-row fragment touch 32 lines each and are the per-CU cost).
// The scales are requested before the K loop.  Epilogue arithmetic as in the tiled kernels.
constexpr int SMALL_KB = 8;           // 32-deep steps per load batch
constexpr int SMALL_MAX_TILES = 16;   // 256 x 256 tiles up to which this kernel is taken

template <int OUT_DT, bool KB>
__global__ __launch_bounds__(64) void k_qgemm_small(GArgs g) {
  const int lane = threadIdx.x;
  const int m0 = blockIdx.x * 32;
  const int n0 = blockIdx.y * 32;
  const int rl = lane & 31, kc = lane >> 5;
  // Scales first: their latency hides behind the K loop.
  const int m = m0 + rl;
  const float sa0 = g.sa_tok ? g.sa[min(m, g.m - 1)] : g.sa[0];
  float sbv[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) sbv[q][r] = g.sb[min(n0 + 8 * q + 4 * kc + r, g.n - 1)];
  const int8_t* pa = g.a + (int64_t)min(m0 + rl, g.m - 1) * g.kp + 16 * kc;
  const uint8_t* pb = g.b + (int64_t)min(n0 + rl, g.n - 1) * wrow<KB>(g, 8) + 16 * kc;
  const int nks = g.k0 / 32;
  v16i acc = v16i{};
  v4i fa[2][SMALL_KB], fb[2][SMALL_KB];
  auto load = [&](int set, int kb) {
#pragma unroll
    for (int u = 0; u < SMALL_KB; ++u) {
      const int ks = min(kb * SMALL_KB + u, nks - 1);  // past the end: a valid step, not used
      fa[set][u] = *reinterpret_cast<const v4i*>(pa + 32 * ks);
      fb[set][u] = *reinterpret_cast<const v4i*>(pb + wofs<KB>(g, 32 * ks));
    }
  };
  auto mma = [&](int set, int kb) {
#pragma unroll
    for (int u = 0; u < SMALL_KB; ++u)
      if (kb * SMALL_KB + u < nks) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[set][u], fa[set][u], acc, 0, 0, 0);
  };
  const int nkb = (nks + SMALL_KB - 1) / SMALL_KB;
  load(0, 0);
  for (int kb = 0; kb < nkb; kb += 2) {
    if (kb + 1 < nkb) load(1, kb + 1);
    mma(0, kb);
    if (kb + 2 < nkb) load(0, kb + 2);
    if (kb + 1 < nkb) mma(1, kb + 1);
  }

  if (m >= g.m) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = n0 + 8 * q + 4 * kc;
    if (n >= g.n) continue;
    const int cnt = min(4, g.n - n);
    float out[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int a0 = acc[4 * q + r];
      const float t0 = sa0 * sbv[q][r];
      out[r] = (float)a0 * t0;
      if (g.accd && r < cnt) g.accd[(int64_t)m * g.n + n + r] = a0;
    }
    if constexpr (OUT_DT == DT_F32) {
      store4_f32(g.y, (int64_t)m * g.ldy + n, out, cnt, g.vec_store != 0);
    } else {
      typedef typename std::conditional<OUT_DT == DT_BF16, __bf16, _Float16>::type h_t;
      const unsigned p0 = cvt_pair<OUT_DT>(out[0], out[1]), p1 = cvt_pair<OUT_DT>(out[2], out[3]);
      h_t* dst = reinterpret_cast<h_t*>(g.y) + (int64_t)m * g.ldy + n;
      if (g.vec_store && cnt == 4) {
        *reinterpret_cast<u2v*>(dst) = u2v{p0, p1};
      } else {
        for (int e = 0; e < cnt; ++e)
          dst[e] = __builtin_bit_cast(h_t, (unsigned short)((e < 2 ? p0 : p1) >> (16 * (e & 1))));
      }
    }
  }
}

template <int BBITS, int OUT_DT, bool KB>
static hipError_t launch_dual(const GArgs& a, bool dual, int grid, hipStream_t st) {
  const int part = a.kp - a.k0;
  if (dual && BBITS == 4 && a.k0 % 128 == 0 && (part == 64 || part == 128))  // 128-code stages
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, true, BBITS == 4 ? 4 : 2, KB>), dim3(grid), dim3(NT), 0, st, a);
  else if (dual)
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, true, 2, KB>), dim3(grid), dim3(NT), 0, st, a);
  else if (BBITS == 4 && a.k0 % 128 == 0)  // 4-bit weights: 128-code stages
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, false, BBITS == 4 ? 4 : 2, KB>), dim3(grid), dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, false, 2, KB>), dim3(grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int BBITS, bool KB>
static hipError_t launch_out(const GArgs& a, int out_dt, bool dual, int grid, hipStream_t st) {
  switch (out_dt) {
    case DT_F16: return launch_dual<BBITS, DT_F16, KB>(a, dual, grid, st);
    case DT_BF16: return launch_dual<BBITS, DT_BF16, KB>(a, dual, grid, st);
    default: return launch_dual<BBITS, DT_F32, KB>(a, dual, grid, st);
  }
}

template <bool KB>
static hipError_t launch_small(const GArgs& a, int out_dt, dim3 sg, hipStream_t st) {
  switch (out_dt) {
    case DT_F16: hipLaunchKernelGGL((k_qgemm_small<DT_F16, KB>), sg, dim3(64), 0, st, a); break;
    case DT_BF16: hipLaunchKernelGGL((k_qgemm_small<DT_BF16, KB>), sg, dim3(64), 0, st, a); break;
    default: hipLaunchKernelGGL((k_qgemm_small<DT_F32, KB>), sg, dim3(64), 0, st, a); break;
  }
  return hipGetLastError();
}

template <bool KB>
static hipError_t launch_pp(const GArgs& a, int out_dt, int grid, hipStream_t st) {
  switch (out_dt) {
    case DT_F16: hipLaunchKernelGGL((k_qgemm_pp<DT_F16, KB>), dim3(grid), dim3(NT), 0, st, a); break;
    case DT_BF16: hipLaunchKernelGGL((k_qgemm_pp<DT_BF16, KB>), dim3(grid), dim3(NT), 0, st, a); break;
    default: hipLaunchKernelGGL((k_qgemm_pp<DT_F32, KB>), dim3(grid), dim3(NT), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace vqk

namespace vq_internal {

using namespace vqk;

// Remainder split of a tile grid: K ranges per remaining tile (1: none).  A range's
// partial (256 KB of int32) is stored and reloaded through one CU.  Measured at the
// workload shapes, two ranges pay off once K has at least 96 stages of 64 codes
// (17776 x 12288 x 3072: 5-6% faster), while at 30 or 48 stages two or three ranges are
// slower or even: the last round's whole tiles, run on a few CUs, already go faster
// than tiles of a full round.
static int split_of(int tiles, int grid, int nk) {
  const int rem = tiles % grid;
  if (rem == 0 || nk < 96 || grid > QGEMM_WS_COUNTERS / 4) return 1;
  return grid / rem >= 2 ? 2 : 1;
}

int64_t qgemm_workspace_bytes(int64_t m, int64_t n, int64_t k0) {
  const int tiles = (int)(((m + BM - 1) / BM) * ((n + BN - 1) / BN));
  const int grid = persistent_blocks();
  const int s = split_of(tiles, grid, (int)(k0 / 64));
  if (s == 1) return 0;
  const int64_t rem = tiles % grid;
  return QGEMM_WS_COUNTERS + rem * s * (int64_t)(32 * NT * 16);
}

hipError_t launch_qgemm(const GemmParams& p, hipStream_t st) {
  GArgs a{};
  a.a = p.a;
  a.sa = p.sa;
  a.b = reinterpret_cast<const uint8_t*>(p.b);
  a.sb = p.sb;
  a.y = p.y;
  a.accd = p.acc_debug;
  a.m = (int)p.m;
  a.n = (int)p.n;
  a.kp = (int)p.kp;
  a.k0 = (int)p.k0;
  a.ldy = p.ldy;
  a.sa_tok = p.sa_per_token;
  a.b_kp = 64 * p.n;
  const int64_t esize = p.out_dt == DT_F32 ? 4 : 2;
  a.vec_store = ((reinterpret_cast<uintptr_t>(p.y) & 15u) == 0 && (p.ldy * esize) % 16 == 0) ? 1 : 0;
  a.tiles_m = (int)((p.m + BM - 1) / BM);
  a.tiles_n = (int)((p.n + BN - 1) / BN);
  const int tiles = a.tiles_m * a.tiles_n;
  const int pb = persistent_blocks();
  // The split is chosen on 64-code stages; a kernel with 128-code stages still gets at
  // least two stages per range.
  const int split = p.ws ? split_of(tiles, pb, (int)(p.k0 / 64)) : 1;
  a.split = split;
  a.dp_items = split > 1 ? tiles - tiles % pb : tiles;
  a.items = a.dp_items + (tiles - a.dp_items) * split;
  a.ws_cnt = split > 1 ? reinterpret_cast<int32_t*>(p.ws) : nullptr;
  a.ws_part = split > 1 ? reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(p.ws) + QGEMM_WS_COUNTERS) : nullptr;
  const int grid = a.items < pb ? a.items : pb;
  const bool dual = p.k0 < p.kp;
  const bool kb = p.b_kblock != 0;
  if (p.b_bits == 8 && !dual && tiles <= SMALL_MAX_TILES) {
    const dim3 sg((unsigned)((p.m + 31) / 32), (unsigned)((p.n + 31) / 32));
    return kb ? launch_small<true>(a, p.out_dt, sg, st) : launch_small<false>(a, p.out_dt, sg, st);
  }
  if (p.b_bits == 8 && !dual && split == 1)
    return kb ? launch_pp<true>(a, p.out_dt, grid, st) : launch_pp<false>(a, p.out_dt, grid, st);
  if (p.b_bits == 8)
    return kb ? launch_out<8, true>(a, p.out_dt, dual, grid, st) : launch_out<8, false>(a, p.out_dt, dual, grid, st);
  return kb ? launch_out<4, true>(a, p.out_dt, dual, grid, st) : launch_out<4, false>(a, p.out_dt, dual, grid, st);
}

// ---- scratch-free entry: the remainder split's workspace in a static device array.
// Each GPU the library runs on holds its own copy from the code object's load until the
// process ends.  Host code never uses the array's name as an address (on the host it is a
// stand-in): the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[QGEMM_SCRATCH_BYTES];

int64_t qgemm_scratch_bytes() { return QGEMM_SCRATCH_BYTES; }

static hipError_t scratch_address(void** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_qgemm_noalloc(const GemmParams& p, hipStream_t st) {
  GemmParams q = p;
  q.ws = nullptr;
  if (qgemm_workspace_bytes(p.m, p.n, p.k0) > 0) {
    hipError_t e = scratch_address(&q.ws);
    if (e != hipSuccess) return e;
    // The arrival counters must start at zero.  Every call leaves them zero, but the
    // array's first contents are not the library's to rely on, so each call clears them
    // with a fill kernel (which, unlike a memset node, also replays correctly in a graph).
    e = launch_fill_u32(reinterpret_cast<unsigned*>(q.ws), (int)(QGEMM_WS_COUNTERS / 4), 0u, st);
    if (e != hipSuccess) return e;
  }
  return launch_qgemm(q, st);
}

}  // namespace vq_internal
