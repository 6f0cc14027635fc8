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
// Tiling: a 256-thread workgroup (4 waves) computes a 256 (M) x 256 (N) tile, each wave
// 128 x 128 as 8 x 8 blocks of v_mfma_i32_16x16x64_i8.  The weights are the MFMA's A
// operand and the activations its B operand, so a lane's four accumulators are four
// consecutive output columns of one row: the epilogue stores 4 outputs per lane.
// K advances 64 codes per step through a double-buffered LDS stage whose rows are
// padded (80 B for 64 int8 codes, 40 B for 32 packed bytes) so that the 16-lane row
// groups of the fragment reads fall in distinct banks.
#include <type_traits>

#include "dev_common.h"
#include "vq_internal.h"

namespace vqk {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int PA = 80;  // LDS pitch of a 64-code int8 row
constexpr int A_ST = BM * PA;

template <int BBITS>
struct BTile {
  static constexpr int PITCH = BBITS == 8 ? 80 : 40;
  static constexpr int ST = BN * PITCH;
  static constexpr int STAGE = A_ST + ST;
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
  int vec_store;  // 4-wide stores are aligned (y 16-byte aligned, ldy % 4 == 0)
  int tiles_m, tiles_n;
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

template <int OUT_DT>
__device__ __forceinline__ void store4(void* y, int64_t off, const float v[4], int cnt, bool vec) {
  if constexpr (OUT_DT == DT_F32) {
    float* p = reinterpret_cast<float*>(y) + off;
    if (vec && cnt == 4) {
      v4f w = {v[0], v[1], v[2], v[3]};
      *reinterpret_cast<v4f*>(p) = w;
    } else {
      for (int i = 0; i < cnt; ++i) p[i] = v[i];
    }
  } else {
    typedef typename std::conditional<OUT_DT == DT_BF16, __bf16, _Float16>::type h_t;
    h_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = (h_t)f32_fence(v[i]);
    h_t* p = reinterpret_cast<h_t*>(y) + off;
    if (vec && cnt == 4) {
      u2v w = {(unsigned)__builtin_bit_cast(unsigned short, h[0]) | ((unsigned)__builtin_bit_cast(unsigned short, h[1]) << 16),
               (unsigned)__builtin_bit_cast(unsigned short, h[2]) | ((unsigned)__builtin_bit_cast(unsigned short, h[3]) << 16)};
      *reinterpret_cast<u2v*>(p) = w;
    } else {
      for (int i = 0; i < cnt; ++i) p[i] = h[i];
    }
  }
}

template <int BBITS, int OUT_DT, bool DUAL>
__global__ __launch_bounds__(256, 1) void k_qgemm(GArgs g) {
  using BT = BTile<BBITS>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BT::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // Grouped tile order: 8 M-tiles share each sweep over N.
  constexpr int GROUP = 8;
  const int tile = blockIdx.x;
  const int width = GROUP * g.tiles_n;
  const int first_m = (tile / width) * GROUP;
  const int gsz = min(g.tiles_m - first_m, GROUP);
  const int tm = first_m + (tile % width) % gsz;
  const int tn = (tile % width) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  // Global -> LDS copy assignment.
  const int8_t* ga[4];
  int la[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 2) + 64 * i;
    const int c16 = tid & 3;
    const int gr = min(m0 + row, g.m - 1);
    ga[i] = g.a + (int64_t)gr * g.kp + 16 * c16;
    la[i] = row * PA + 16 * c16;
  }
  constexpr int NB = BBITS == 8 ? 4 : 2;
  const uint8_t* gb[NB];
  int lb[NB];
  const int64_t ldb = BBITS == 8 ? g.kp : g.kp / 2;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = BBITS == 8 ? (tid >> 2) + 64 * i : (tid >> 1) + 128 * i;
    const int c16 = BBITS == 8 ? (tid & 3) : (tid & 1);
    const int gr = min(n0 + row, g.n - 1);
    gb[i] = g.b + (int64_t)gr * ldb + 16 * c16;
    lb[i] = A_ST + row * BT::PITCH + 16 * c16;
  }

  u4v ra[4], rb[NB];
  auto gload = [&](int k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const u4v*>(ga[i] + k);
    const int kb = BBITS == 8 ? k : k / 2;
#pragma unroll
    for (int i = 0; i < NB; ++i) rb[i] = *reinterpret_cast<const u4v*>(gb[i] + kb);
  };
  auto swrite = [&](int stage) {
    uint8_t* base = lds + stage * BT::STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u4v*>(base + la[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (BBITS == 8) {
        *reinterpret_cast<u4v*>(base + lb[i]) = rb[i];
      } else {
        u2v lo = {rb[i].x, rb[i].y}, hi = {rb[i].z, rb[i].w};
        *reinterpret_cast<u2v*>(base + lb[i]) = lo;
        *reinterpret_cast<u2v*>(base + lb[i] + 8) = hi;
      }
    }
  };

  // Fragment addresses inside a stage.
  const int fa = (wm * 128 + (lane & 15)) * PA + 16 * (lane >> 4);
  const int fb = A_ST + (wn * 128 + (lane & 15)) * BT::PITCH + (BBITS == 8 ? 16 : 8) * (lane >> 4);

  auto afrag = [&](int stage, int mb) -> v4i {
    return *reinterpret_cast<const v4i*>(lds + stage * BT::STAGE + fa + mb * 16 * PA);
  };
  auto bfrag = [&](int stage, int nb) -> v4i {
    const uint8_t* p = lds + stage * BT::STAGE + fb + nb * 16 * BT::PITCH;
    if constexpr (BBITS == 8) {
      return *reinterpret_cast<const v4i*>(p);
    } else {
      return unpack_int4x16(*reinterpret_cast<const u2v*>(p));
    }
  };

  v4i acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int nk = g.k0 / BK;
  gload(0);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    v4i af[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) af[mb] = afrag(cur, mb);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const v4i bf = bfrag(cur, nb);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf, af[mb], acc[mb][nb], 0, 0, 0);
    }
    if (kt + 1 < nk) swrite(cur ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // Each 16 x 16 block is dequantized and stored on its own; with dual scale the
  // outlier partition [k0, kp) (at most two 64-code steps) is staged in LDS first and
  // its block product is added in float32: y = fl(y_0 + y_1).
  int steps1 = 0;
  if constexpr (DUAL) {
    steps1 = (g.kp - g.k0) / BK;
    gload(g.k0);
    swrite(0);
    if (steps1 > 1) {
      gload(g.k0 + BK);
      swrite(1);
    }
    __syncthreads();
  }

  constexpr int P = DUAL ? 2 : 1;
  const int mrow0 = m0 + wm * 128 + (lane & 15);
  const int ncol0 = n0 + wn * 128 + 4 * (lane >> 4);
  const int64_t mn = (int64_t)g.m * g.n;

  float sa_r[8][P];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int mc = min(mrow0 + mb * 16, g.m - 1);
#pragma unroll
    for (int p = 0; p < P; ++p) sa_r[mb][p] = g.sa_tok ? g.sa[(int64_t)mc * P + p] : g.sa[p];
  }

#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int n = ncol0 + nb * 16;
    float sb_r[4][P];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int p = 0; p < P; ++p) sb_r[r][p] = g.sb[(int64_t)min(n + r, g.n - 1) * P + p];
    v4i bf1[2];
    if constexpr (DUAL) {
      bf1[0] = bfrag(0, nb);
      bf1[1] = steps1 > 1 ? bfrag(1, nb) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int m = mrow0 + mb * 16;
      v4i t1 = v4i{0, 0, 0, 0};
      if constexpr (DUAL) {
        t1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf1[0], afrag(0, mb), t1, 0, 0, 0);
        if (steps1 > 1) t1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf1[1], afrag(1, mb), t1, 0, 0, 0);
      }
      float out[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int a0 = acc[mb][nb][r];
        if constexpr (BBITS == 4) a0 >>= 4;
        const float t0 = sa_r[mb][0] * sb_r[r][0];
        float yv = (float)a0 * t0;
        if constexpr (DUAL) {
          int a1 = t1[r];
          if constexpr (BBITS == 4) a1 >>= 4;
          const float tt = sa_r[mb][P - 1] * sb_r[r][P - 1];
          const float y1 = (float)a1 * tt;
          yv = yv + y1;
          if (g.accd && m < g.m && n + r < g.n) g.accd[mn + (int64_t)m * g.n + n + r] = a1;
        }
        if (g.accd && m < g.m && n + r < g.n) g.accd[(int64_t)m * g.n + n + r] = a0;
        out[r] = yv;
      }
      if (m < g.m && n < g.n) store4<OUT_DT>(g.y, (int64_t)m * g.ldy + n, out, min(4, g.n - n), g.vec_store != 0);
    }
  }
}

template <int BBITS, int OUT_DT>
static hipError_t launch_dual(const GArgs& a, bool dual, int grid, hipStream_t st) {
  if (dual)
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, true>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_qgemm<BBITS, OUT_DT, false>), dim3(grid), dim3(256), 0, st, a);
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
  a.vec_store = ((reinterpret_cast<uintptr_t>(p.y) & 15u) == 0 && p.ldy % 4 == 0) ? 1 : 0;
  a.tiles_m = (int)((p.m + BM - 1) / BM);
  a.tiles_n = (int)((p.n + BN - 1) / BN);
  const int grid = a.tiles_m * a.tiles_n;
  const bool dual = p.k0 < p.kp;
  if (p.b_bits == 8) return launch_out<8>(a, p.out_dt, dual, grid, st);
  return launch_out<4>(a, p.out_dt, dual, grid, st);
}

}  // namespace vq_internal
