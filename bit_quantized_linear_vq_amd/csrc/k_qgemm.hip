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
// partial tile (device-coherent stores), then bumps an atomic count, and the workgroup
// that arrives last adds the other partials and runs the epilogue.  Integer
// sums are exact in any order, so the result is bit-identical to the unsplit tile, and
// no workgroup ever waits for another.  The last arrival resets the tile's counter, so
// the workspace is left zeroed for the next call.
#include <type_traits>

#include "dev_common.h"
#include "gemm_common.h"
#include "vq_internal.h"

namespace vqk {

constexpr int BM = 256, BN = 256;
constexpr int64_t QGEMM_WS_COUNTERS = 4096;  // arrival counters of up to 1024 remaining tiles
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
};

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

template <int BBITS, int OUT_DT, bool DUAL, int H>
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
  const int64_t ldb = BBITS == 8 ? g.kp : g.kp / 2;
  const int8_t* ga[C::LA];
  const uint8_t* gb[C::LB];
  int m0 = 0, n0 = 0;
  int kb0 = 0, nks = nk;    // the item's first stage and stage count
  int part = -1, rslot = 0;  // K range of a split tile (-1: whole tile) and its remainder index
  auto set_tile = [&](int w) {
    int ti = w;
    if (w < g.dp_items) {
      kb0 = 0;
      nks = nk;
      part = -1;
    } else {
      const int j = w - g.dp_items;
      rslot = j / g.split;
      part = j - rslot * g.split;
      ti = g.dp_items + rslot;
      kb0 = part * nk / g.split;
      nks = (part + 1) * nk / g.split - kb0;
    }
    int tm, tn;
    tile_of(ti, g.tiles_m, g.tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) ga[i] = g.a + (int64_t)min(m0 + ra[i], g.m - 1) * g.kp + ca[i];
#pragma unroll
    for (int i = 0; i < C::LB; ++i) gb[i] = g.b + (int64_t)min(n0 + rb[i], g.n - 1) * ldb + cb[i];
  };
  auto issue = [&](int k, int slot) {
    uint8_t* base = lds + slot * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) dma16(ga[i] + k, base + la_off[i]);
    const int kb = BBITS == 8 ? k : k / 2;
#pragma unroll
    for (int i = 0; i < C::LB; ++i) dma16(gb[i] + kb, base + lb_off[i]);
  };
  // The outlier partition [k0, kp) of 64 or 128 codes as one 128-code stage: columns past
  // the partition wrap to its start (mask), so every load stays inside the row's
  // partition; the wrapped chunks are never read.
  auto issue_part = [&](int amask, int bmask) {
#pragma unroll
    for (int i = 0; i < C::LA; ++i) dma16(ga[i] - ca[i] + (ca[i] & amask) + g.k0, lds + la_off[i]);
#pragma unroll
    for (int i = 0; i < C::LB; ++i) dma16(gb[i] - cb[i] + (cb[i] & bmask) + g.k0 / 2, lds + lb_off[i]);
  };
  auto issue_prologue = [&]() {
#pragma unroll
    for (int s = 0; s < C::NST - 1; ++s)
      if (s < nks) issue((kb0 + s) * BK, s);
  };
  // Scales of a tile's rows and columns: loaded into registers early, written to LDS late.
  float sc_a[P], sc_b[P];
  const int srow = tid & (BM - 1);  // 512 threads: each loads one row scale or one column scale
  auto load_scales = [&]() {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (tid < BM)
        sc_a[p] = g.sa_tok ? g.sa[(int64_t)min(m0 + srow, g.m - 1) * P + p] : g.sa[p];
      else
        sc_b[p] = g.sb[(int64_t)min(n0 + srow, g.n - 1) * P + p];
    }
  };
  auto store_scales = [&](int buf) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (tid < BM)
        s_sa[buf][p][srow] = sc_a[p];
      else
        s_sb[buf][p][srow] = sc_b[p];
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
  issue_prologue();
  load_scales();
  store_scales(0);
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
      // this is the block's last item and nothing is in flight.  The partials move with
      // device-scope relaxed atomic stores and loads, which write through and bypass the
      // per-XCD L2: a device-scope fence would instead write back and invalidate the whole
      // L2 under every other workgroup of the XCD.  A store is performed device-wide once
      // vmcnt reaches 0, and the count is bumped only after that; the last arrival loads
      // the other partials only after it has read the count.
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
        load_scales();
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
        u2v hw[4];  // 16-bit outputs of group q: columns 8q + 4 * (lane >> 5) + 0..3
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
            if (g.accd && m < g.m && n + r < g.n) g.accd[(int64_t)m * g.n + n + r] = a0;
            out[r] = yv;
          }
          if constexpr (HALF_OUT) {
            h_t hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) hv[r] = (h_t)f32_fence(out[r]);
            hw[q] = u2v{(unsigned)__builtin_bit_cast(unsigned short, hv[0]) |
                            ((unsigned)__builtin_bit_cast(unsigned short, hv[1]) << 16),
                        (unsigned)__builtin_bit_cast(unsigned short, hv[2]) |
                            ((unsigned)__builtin_bit_cast(unsigned short, hv[3]) << 16)};
          } else {
            if (m < g.m && n < g.n) store4_f32(g.y, (int64_t)m * g.ldy + n, out, min(4, g.n - n), g.vec_store != 0);
          }
        }
        if constexpr (HALF_OUT) {
          // Groups (q, q+1) of the two half-waves are exchanged so that each lane holds eight
          // consecutive columns: lanes 0-31 columns 16pr + 0..7, lanes 32-63 16pr + 8..15.
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const u2v X = hw[2 * pr], Y = hw[2 * pr + 1];
            const auto s0 = __builtin_amdgcn_permlane32_swap(X.x, Y.x, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(X.y, Y.y, false, false);
            const u4v w = {s0[0], s1[0], s0[1], s1[1]};
            const int no = cn0 + wn * WTN + nb * 32 + 16 * pr + 8 * (lane >> 5);
            if (m < g.m && no < g.n) {
              h_t* dst = reinterpret_cast<h_t*>(g.y) + (int64_t)m * g.ldy + no;
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
      load_scales();
      issue_prologue();
    }
    store_scales(buf ^ 1);  // the next tile's epilogue reads them after several barriers
    buf ^= 1;
    vt = nvt;
  }
}

template <int BBITS, int OUT_DT>
static hipError_t launch_dual(const GArgs& a, bool dual, int grid, hipStream_t st) {
  const int part = a.kp - a.k0;
  if (dual && BBITS == 4 && a.k0 % 128 == 0 && (part == 64 || part == 128))  // 128-code stages
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, true, BBITS == 4 ? 4 : 2>), dim3(grid), dim3(NT), 0, st, a);
  else if (dual)
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, true, 2>), dim3(grid), dim3(NT), 0, st, a);
  else if (BBITS == 4 && a.k0 % 128 == 0)  // 4-bit weights: 128-code stages
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, false, BBITS == 4 ? 4 : 2>), dim3(grid), dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, false, 2>), dim3(grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int BBITS>
static hipError_t launch_out(const GArgs& a, int out_dt, bool dual, int grid, hipStream_t st) {
  switch (out_dt) {
    case DT_F16: return launch_dual<BBITS, DT_F16>(a, dual, grid, st);
    case DT_BF16: return launch_dual<BBITS, DT_BF16>(a, dual, grid, st);
    default: return launch_dual<BBITS, DT_F32>(a, dual, grid, st);
  }
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
  if (p.b_bits == 8) return launch_out<8>(a, p.out_dt, dual, grid, st);
  return launch_out<4>(a, p.out_dt, dual, grid, st);
}

}  // namespace vq_internal
