// Unquantized FP16/BF16 linear layer for gfx950: Y = X . W^T with float32 accumulation
// on the 16-bit MFMA, for the layers the precision override runs unquantized.
//
// 6Bit-Diffusion (gist.science, arXiv 2603.18742), Methodology B.3 (PDR): a layer whose
// input has a high outlier ratio is computed in FP16/BF16 (precision code 16 of the step
// control).
//
// The schedule is the ping-pong one of the W8A8 kernel (k_qgemm.hip): 256 x 256 tiles,
// 8 waves of 128 x 64, the two waves of a SIMD alternating between a memory phase (the
// fragment reads of a stage and its share of the direct loads) and a compute phase (the
// stage's MFMAs from registers).  A stage holds 32 elements of K (64-byte rows, the same
// byte layout and swizzle as the int8 kernel's 64-code stages): two 32 x 32 x 16 steps,
// lane l holding row l mod 32 and elements 8 (l div 32) .. +7 of each step.  Ring of 4
// stages, refilled 2 stages ahead.  The epilogue rounds the float32 accumulators once to
// the output type (round to nearest even).
#include "dev_common.h"
#include "gemm_common.h"
#include "vq_internal.h"

namespace vqk {

namespace dn {
constexpr int BM = 256, BN = 256, NT = 512;
constexpr int WTM = 128, WTN = 64, MBLK = WTM / 32, NBLK = WTN / 32;
constexpr int ROW = 64;                    // bytes per row and stage: 32 16-bit elements
constexpr int A_BYTES = BM * ROW, STAGE = A_BYTES + BN * ROW;
constexpr int NST = 4, D = 2;
constexpr int LA = A_BYTES / (NT * 16);    // direct loads per wave and operand (2)
constexpr int L = 2 * LA;
}  // namespace dn

struct DArgs {
  const uint16_t* x;  // [m x k], row pitch ldx elements
  const uint16_t* w;  // [n x k], row pitch ldw elements
  void* y;
  int m, n, k;
  int64_t ldx, ldw, ldy;
  int vec_store;
  int tiles_m, tiles_n, items;
};

__device__ __forceinline__ void dn_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int IN_DT, int OUT_DT>
__global__ __launch_bounds__(dn::NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_dense(DArgs g) {
  using namespace dn;
  typedef typename std::conditional<IN_DT == DT_BF16, __bf16, _Float16>::type in_t;
  typedef in_t in8 __attribute__((ext_vector_type(8)));
  constexpr bool HALF_OUT = OUT_DT != DT_F32;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // waves w and w + 4 share a SIMD
  const int wm = wave & 1, wn = wave >> 1;
  const int nk = g.k / 32;

  int ra[LA], rb[LA], ca[LA], cb[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    dma_lane<ROW>(wave * LA + i, lane, ra[i], ca[i]);
    dma_lane<ROW>(wave * LA + i, lane, rb[i], cb[i]);
  }
  const uint8_t* ga[LA];
  const uint8_t* gb[LA];
  int m0 = 0, n0 = 0;
  auto set_tile = [&](int t) {
    int tm, tn;
    tile_of(t, g.tiles_m, g.tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      ga[i] = reinterpret_cast<const uint8_t*>(g.x + (int64_t)min(m0 + ra[i], g.m - 1) * g.ldx) + ca[i];
      gb[i] = reinterpret_cast<const uint8_t*>(g.w + (int64_t)min(n0 + rb[i], g.n - 1) * g.ldw) + cb[i];
    }
  };
  auto issue = [&](int s, int slot) {
    const int kb = s * ROW;
    uint8_t* base = lds + slot * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i) dma16(ga[i] + kb, base + (wave * LA + i) * 1024);
#pragma unroll
    for (int i = 0; i < LA; ++i) dma16(gb[i] + kb, base + A_BYTES + (wave * LA + i) * 1024);
  };
  const int rl = lane & 31, kc = lane >> 5;
  int fa[2], fb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    fa[h] = (wm * WTM + rl) * ROW + 16 * ((2 * h + kc) ^ swz_row<ROW>(rl));
    fb[h] = A_BYTES + (wn * WTN + rl) * ROW + 16 * ((2 * h + kc) ^ swz_row<ROW>(rl));
  }
  v16f acc[MBLK][NBLK];
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
        for (int mb = 0; mb < MBLK; ++mb) {
          const in8 b = __builtin_bit_cast(in8, fB[h][nb]);
          const in8 a = __builtin_bit_cast(in8, fA[h][mb]);
          if constexpr (IN_DT == DT_BF16)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[mb][nb], 0, 0, 0);
          else
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, acc[mb][nb], 0, 0, 0);
        }
  };
  auto lds_reads_done = [&]() { __builtin_amdgcn_s_waitcnt(0xC07F); };  // lgkmcnt(0)
  auto wait_groups = [&](int later) {  // at most `later` stages of loads in flight
    if (later >= 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
  };

  int t = blockIdx.x;
  if (t >= g.items) return;
  set_tile(t);
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < nk) issue(s, s);
  // pend: the previous tile issued exactly 16 vector stores after this tile's first loads,
  // so waits for this tile's first stages leave those stores in flight (vmcnt is in order).
  bool pend = false;
  for (;;) {
#pragma unroll
    for (int i = 0; i < MBLK; ++i)
#pragma unroll
      for (int j = 0; j < NBLK; ++j) acc[i][j] = v16f{};
    if (pend && nk > D) wait_vmcnt<(D - 1) * L + 16>();
    else wait_groups(min(D, nk) - 1);
    dn_barrier();
    if (grp == 1) dn_barrier();
    int p = 0;
    for (; p + D < nk; ++p) {
      read_stage(p % NST);
      issue(p + D, (p + D) % NST);
      const bool early = pend && p < D - 1;  // stage p + 1 was loaded before the stores
      if (grp == 1) {
        if (early) wait_vmcnt<(D - 1) * L + 16>();
        else wait_vmcnt<(D - 1) * L>();
      }
      lds_reads_done();
      dn_barrier();
      compute();
      if (grp == 0) {
        if (early) wait_vmcnt<(D - 1) * L + 16>();
        else wait_vmcnt<(D - 1) * L>();
      }
      dn_barrier();
    }
    for (; p < nk; ++p) {
      read_stage(p % NST);
      const int later = nk - p - 2;
      if (grp == 1) wait_groups(later < 0 ? 0 : later);
      lds_reads_done();
      dn_barrier();
      compute();
      if (grp == 0) wait_groups(later < 0 ? 0 : later);
      dn_barrier();
    }
    if (grp == 0) dn_barrier();

    const int nt = t + (int)gridDim.x;
    const bool has_next = nt < g.items;
    const int cm0 = m0, cn0 = n0;
    if (has_next) {
      set_tile(nt);
#pragma unroll
      for (int s = 0; s < D; ++s)
        if (s < nk) issue(s, s);
    }
    const bool full = g.vec_store && cm0 + BM <= g.m && cn0 + BN <= g.n;
    pend = HALF_OUT && has_next && full;
    typedef typename std::conditional<OUT_DT == DT_BF16, __bf16, _Float16>::type h_t;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
      const int m = cm0 + wm * WTM + rl + mb * 32;
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) {
        if constexpr (HALF_OUT) {
          // Lanes l and l + 32 swap column groups so that each holds 8 consecutive outputs.
          unsigned pk[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            pk[2 * q] = cvt_pair<OUT_DT>(acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1]);
            pk[2 * q + 1] = cvt_pair<OUT_DT>(acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]);
          }
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const auto s0 = __builtin_amdgcn_permlane32_swap(pk[4 * pr], pk[4 * pr + 2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(pk[4 * pr + 1], pk[4 * pr + 3], false, false);
            const u4v wv = {s0[0], s1[0], s0[1], s1[1]};
            const int no = cn0 + wn * WTN + nb * 32 + 16 * pr + 8 * kc;
            h_t* dst = reinterpret_cast<h_t*>(g.y) + (int64_t)m * g.ldy + no;
            if (full) {
              *reinterpret_cast<u4v*>(dst) = wv;
            } else if (m < g.m && no < g.n) {
              if (g.vec_store && no + 8 <= g.n) {
                *reinterpret_cast<u4v*>(dst) = wv;
              } else {
                for (int e = 0; e < 8 && no + e < g.n; ++e) {
                  const unsigned d = e < 2 ? wv.x : e < 4 ? wv.y : e < 6 ? wv.z : wv.w;
                  dst[e] = __builtin_bit_cast(h_t, (unsigned short)(d >> (16 * (e & 1))));
                }
              }
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = cn0 + wn * WTN + 4 * kc + nb * 32 + 8 * q;
            const float out[4] = {acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1], acc[mb][nb][4 * q + 2],
                                  acc[mb][nb][4 * q + 3]};
            if (m < g.m && n < g.n) store4_f32(g.y, (int64_t)m * g.ldy + n, out, min(4, g.n - n), g.vec_store != 0);
          }
        }
      }
    }
    if (!has_next) break;
    t = nt;
  }
}

}  // namespace vqk

namespace vq_internal {

using namespace vqk;

hipError_t launch_gemm_dense(const DenseParams& p, hipStream_t st) {
  DArgs a{};
  a.x = reinterpret_cast<const uint16_t*>(p.x);
  a.w = reinterpret_cast<const uint16_t*>(p.w);
  a.y = p.y;
  a.m = (int)p.m;
  a.n = (int)p.n;
  a.k = (int)p.k;
  a.ldx = p.ldx;
  a.ldw = p.ldw;
  a.ldy = p.ldy;
  const int64_t esize = p.out_dt == DT_F32 ? 4 : 2;
  a.vec_store = ((reinterpret_cast<uintptr_t>(p.y) & 15u) == 0 && (p.ldy * esize) % 16 == 0) ? 1 : 0;
  a.tiles_m = (int)((p.m + dn::BM - 1) / dn::BM);
  a.tiles_n = (int)((p.n + dn::BN - 1) / dn::BN);
  a.items = a.tiles_m * a.tiles_n;
  const int pb = persistent_blocks();
  const int grid = a.items < pb ? a.items : pb;
#define VQ_DENSE(I, O) hipLaunchKernelGGL((k_gemm_dense<I, O>), dim3(grid), dim3(dn::NT), 0, st, a)
  if (p.in_dt == DT_BF16) {
    switch (p.out_dt) {
      case DT_F16: VQ_DENSE(DT_BF16, DT_F16); break;
      case DT_BF16: VQ_DENSE(DT_BF16, DT_BF16); break;
      default: VQ_DENSE(DT_BF16, DT_F32); break;
    }
  } else {
    switch (p.out_dt) {
      case DT_F16: VQ_DENSE(DT_F16, DT_F16); break;
      case DT_BF16: VQ_DENSE(DT_F16, DT_BF16); break;
      default: VQ_DENSE(DT_F16, DT_F32); break;
    }
  }
#undef VQ_DENSE
  return hipGetLastError();
}

}  // namespace vq_internal
