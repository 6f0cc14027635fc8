// MX block-format route for gfx950: MXFP4 / MXFP6 quantization and the GEMM on the
// scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// 6Bit-Diffusion (gist.science, arXiv 2603.18742), Introduction and Methodology B.1:
// recent GPUs replaced INT4 by a 4-bit floating-point block format, DMPQ routes
// activations between INT8 and that format, and the weights are kept in it offline.
// gfx950's counterpart is the OCP MX family: blocks of 32 elements along K share one
// E8M0 scale 2^e, e = floor(log2(max|v|)) - emax (emax = 2 for FP4 E2M1 and FP6 E2M3),
// and each element is v / 2^e rounded to nearest even and clamped to the largest value
// (6 for E2M1, 7.5 for E2M3).  The matrix cores take the element codes and the scale
// bytes directly, at twice the int8 rate.
//
// Layouts (both operands K-contiguous, "TN"):
//   codes   row-major, element p of a row at bits [w*p, w*p+w) of the row's little-endian
//           bit string (w = 4: two per byte, low nibble first; w = 6: 3 bytes per 4);
//   scales  E8M0 bytes in k-step-major order [K/64][rows8][2] (rows8 = rows rounded up to
//           8): the two block scales of every row for each 64-deep step are adjacent, so
//           a tile's scales for one step are 512 contiguous bytes that the GEMM moves into
//           LDS with the same direct loads as the codes.
//
// Measured on gfx950 (lane-layout probe of the scaled MFMA): for FP4 and FP6 E2M3 the
// A operand of lane l holds row l % 32 and K values 32 * (l / 32) + p, the B operand
// column l % 32 likewise, and each lane's scale byte applies to its 32 values (one MX
// block); the 32 x 32 float32 result is laid out as for the other 32x32 MFMA forms.
#include <type_traits>

#include "dev_common.h"
#include "gemm_common.h"
#include "vq_internal.h"

namespace vqk {

enum : int { MX_FP6 = 2, MX_FP4 = 4 };  // the scaled MFMA's operand format codes

template <int FMT>
struct MxFmt {
  static constexpr int M = FMT == MX_FP4 ? 1 : 3;  // mantissa bits (both have 2 exponent bits, bias 1)
  static constexpr int W = 3 + M;                  // bits per element
  static constexpr int STEP_BYTES = 64 * W / 8;    // bytes of one row per 64-deep step
};

// ------------------------------------------------------------------ quantization
//
// The element codes come from gfx950's MX conversion instructions
// (v_cvt_scalef32_pk_fp4_{bf16,f16}: two elements; v_cvt_scalef32_pk32_fp6_{bf16,f16}: a
// whole 32-element block).  Given the scale 2^e as a float, they divide by it (only its
// exponent field is read, so the bit pattern 0 stands for 2^-127 as in E8M0), round to
// the nearest value with ties to even, saturate at the largest magnitude, keep the sign of
// a value that rounds to zero, and pack element p at bits [w*p, w*p + w) of the output.
// A probe of 40,000 blocks (tie grids of both formats, signed zeros, subnormal inputs, a
// zero block, scales 2^-127 .. 2^125, random bf16 bit patterns) matched the rounding rule
// above element for element; the bit-exact tests against the oracle hold it to that.

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));
typedef _Float16 f16x32_t __attribute__((ext_vector_type(32)));
typedef unsigned u32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x6_t __attribute__((ext_vector_type(6)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

// One block: E8M0 exponent from its largest magnitude, scale byte, element codes.
template <int DT, int FMT>
__device__ __forceinline__ void mxq_block(const unsigned (&d)[16], int64_t row, int blk, int64_t rows8,
                                          uint8_t* codes_blk, uint8_t* scales) {
  using F = MxFmt<FMT>;
  // Largest magnitude: with the sign bit cleared, bf16 and fp16 magnitudes order like their
  // 16-bit patterns (finite inputs), so a packed 16-bit integer maximum finds it.
  u16x2_t m = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, d[i] & 0x7FFF7FFFu));
  const unsigned a16 = m.x > m.y ? m.x : m.y;
  int ex;  // float32 exponent field of the maximum
  if constexpr (DT == DT_BF16) {
    ex = (int)(a16 >> 7);
  } else {
    ex = (int)((f_bits((float)__builtin_bit_cast(_Float16, (unsigned short)a16)) >> 23) & 0xFF);
  }
  // E8M0 exponent: floor(log2 max) - 2 (emax of E2M1 and E2M3), -127 for a zero block.
  int e = ex == 0 ? -127 : ex - 127 - 2;
  e = e < -127 ? -127 : e;
  scales[((int64_t)(blk >> 1) * rows8 + row) * 2 + (blk & 1)] = (uint8_t)(e + 127);
  const float sc = bits_f((unsigned)(e + 127) << 23);  // 2^e (bit pattern 0 for 2^-127)
  u2v* dst = reinterpret_cast<u2v*>(codes_blk);
  if constexpr (FMT == MX_FP4) {
    unsigned o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unsigned r = 0;
      if constexpr (DT == DT_BF16) {
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, d[4 * q + 0]), sc, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, d[4 * q + 1]), sc, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, d[4 * q + 2]), sc, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, d[4 * q + 3]), sc, 3);
      } else {
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(r, __builtin_bit_cast(f16x2_t, d[4 * q + 0]), sc, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(r, __builtin_bit_cast(f16x2_t, d[4 * q + 1]), sc, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(r, __builtin_bit_cast(f16x2_t, d[4 * q + 2]), sc, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f16(r, __builtin_bit_cast(f16x2_t, d[4 * q + 3]), sc, 3);
      }
      o[q] = r;
    }
    dst[0] = u2v{o[0], o[1]};
    dst[1] = u2v{o[2], o[3]};
  } else {
    const u32x16_t all = {d[0], d[1], d[2], d[3], d[4], d[5], d[6], d[7], d[8], d[9], d[10], d[11], d[12], d[13], d[14], d[15]};
    u32x6_t o;
    if constexpr (DT == DT_BF16) {
      o = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(__builtin_bit_cast(bf16x32_t, all), sc);
    } else {
      o = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(__builtin_bit_cast(f16x32_t, all), sc);
    }
    dst[0] = u2v{o[0], o[1]};
    dst[1] = u2v{o[2], o[3]};
    dst[2] = u2v{o[4], o[5]};
  }
}

// One block of float32 values (the rotated route): E8M0 exponent from the float32
// largest magnitude, scale byte, element codes from the fp32-input conversions
// (v_cvt_scalef32_pk_fp4_f32: two elements; v_cvt_scalef32_2xpk16_fp6_f32: the block).
template <int FMT>
__device__ __forceinline__ void mxq_block_f32(const float (&v)[32], int64_t row, int blk, int64_t rows8,
                                              uint8_t* codes_blk, uint8_t* scales) {
  using F = MxFmt<FMT>;
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  const int ex = (int)((f_bits(m) >> 23) & 0xFF);
  int e = ex == 0 ? -127 : ex - 127 - 2;  // floor(log2 max) - 2; zero or subnormal maxima clamp to -127
  e = e < -127 ? -127 : e;
  scales[((int64_t)(blk >> 1) * rows8 + row) * 2 + (blk & 1)] = (uint8_t)(e + 127);
  const float sc = bits_f((unsigned)(e + 127) << 23);
  u2v* dst = reinterpret_cast<u2v*>(codes_blk);
  if constexpr (FMT == MX_FP4) {
    unsigned o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unsigned r = 0;
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 0], v[8 * q + 1], sc, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 2], v[8 * q + 3], sc, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 4], v[8 * q + 5], sc, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 6], v[8 * q + 7], sc, 3);
      o[q] = r;
    }
    dst[0] = u2v{o[0], o[1]};
    dst[1] = u2v{o[2], o[3]};
  } else {
    // The instruction interleaves its two sources (output element 2i from the first, 2i + 1
    // from the second; lane-layout probe), and its destination must not overlap them: the
    // compiler allocated overlapping registers for the builtin, and the result then held a
    // value written before it was read.  Hence inline asm with an early-clobber output.
    v16f ev, od;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ev[i] = v[2 * i];
      od[i] = v[2 * i + 1];
    }
    u32x6_t o;
    asm volatile("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(o) : "v"(ev), "v"(od), "v"(sc));
    dst[0] = u2v{o[0], o[1]};
    dst[1] = u2v{o[2], o[3]};
    dst[2] = u2v{o[4], o[5]};
  }
}

// 128-point block Hadamard rotation of the four 32-element blocks held by a lane quad
// (lane q of the quad holds elements 32q .. 32q + 31 of the 128-element block): float32
// butterflies with distances 1, 2, 4, 8, 16 inside the lane, then 32 and 64 across the
// quad, each pair (i, i + h) becoming (z_i + z_{i+h}, z_i - z_{i+h}), in ascending order.
// Across lanes the lower lane of a pair computes fl(mine + partner) and the upper lane
// fl(partner - mine), both as one fma with the exact product mine * (+-1).
__device__ __forceinline__ void fwht128_quad(float (&v)[32], int q) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  const float c32 = (q & 1) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(v[i], c32, dpp_f<0xB1>(v[i]));  // quad_perm [1,0,3,2]
  const float c64 = (q & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf(v[i], c64, dpp_f<0x4E>(v[i]));  // quad_perm [2,3,0,1]
}

// A wave takes tiles of 8 rows x 8 blocks (tile t: row group t / nbg, block group t % nbg,
// nbg = ceil(nb / 8), nb = k / 32), so that the scale bytes it writes for one 64-deep step
// are 16 contiguous bytes of the step-major layout (8 rows x 2 blocks).  The loads are
// contiguous 16-byte pieces: piece p = 64u + l of load u in lane l is quarter p % 4 of
// block p / 4 of the tile (row p / 32, 512 contiguous bytes per row), and a pass through
// the wave's 4 KB of LDS hands lane L its block L (row L / 8, block L % 8) whole.
// Quarter j of block B sits at byte 64 B + 16 ((j + B + B / 4) mod 4): the 16 lanes of a
// 16-byte LDS access then cover all banks, for the writes and for the reads.  (Loading
// each block straight into its lane, 64 bytes per lane, measured 1.5x slower; 64
// consecutive blocks of one row per wave wrote each step's scale bytes two at a time into
// 32 different cache lines, 42% more bytes written than the codes and scales.)
// HAD: the rows are first rotated by 128-point Hadamard blocks (each a lane quad, K a
// multiple of 128) and scaled by pscale (an exact power of two); the block scales then
// come from the float32 rotated values.
// KB (FP4 codes only): the codes go out in 64-byte K pieces, four blocks of a row per
// piece and piece j of every row together (byte c of row r at (c / 64) * 64 rows + 64 r +
// c % 64), the weight layout whose GEMM stages read whole cache lines.
template <int DT, int FMT, bool HAD, bool KB>
__global__ __launch_bounds__(256) void k_mxquant(const void* x, int64_t ldx, int64_t rows, int k, int64_t rows8,
                                                 uint8_t* codes, uint8_t* scales, float pscale) {
  using F = MxFmt<FMT>;
  static_assert(!KB || FMT == MX_FP4, "K pieces hold whole FP4 blocks only");
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * 4096];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // the tile index stays scalar
  uint8_t* wl = lds + wave * 4096;
  const int nb = k / 32;
  const int nbg = (nb + 7) / 8;
  const int64_t tiles = (rows + 7) / 8 * nbg;
  const int64_t row_bytes = (int64_t)k * F::W / 8;
  // Destination of block blk of row `row`.
  auto block_at = [&](int64_t row, int blk) -> uint8_t* {
    if constexpr (KB) return codes + (int64_t)(blk >> 2) * rows * 64 + row * 64 + (blk & 3) * 16;
    else return codes + row * row_bytes + (int64_t)blk * (32 * F::W / 8);
  };
  const int64_t step = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t < tiles; t += step) {
    const int64_t row0 = t / nbg * 8;  // wave-uniform
    const int blk0 = (int)(t % nbg) * 8;
    u4v raw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = 64 * u + lane;
      const int64_t row = row0 + (p >> 5);
      const int blk = blk0 + ((p & 31) >> 2);
      if (row < rows && blk < nb) {
        raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(
            reinterpret_cast<const char*>(x) + (row * ldx + blk * 32) * 2 + (p & 3) * 16));
      } else {
        raw[u] = u4v{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int B = 16 * u + (lane >> 2), Q = lane & 3;
      *reinterpret_cast<u4v*>(wl + B * 64 + 16 * ((Q + B + (B >> 2)) & 3)) = raw[u];
    }
    // Plain array, not a vector: a bit cast applied in place to an element of an
    // ext-vector reads the vector's first element whatever the index.
    unsigned d[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u4v w = *reinterpret_cast<const u4v*>(wl + lane * 64 + 16 * ((j + lane + (lane >> 2)) & 3));
      d[4 * j + 0] = w.x;
      d[4 * j + 1] = w.y;
      d[4 * j + 2] = w.z;
      d[4 * j + 3] = w.w;
    }
    const int64_t row = row0 + (lane >> 3);
    const int blk = blk0 + (lane & 7);
    if constexpr (HAD) {
      // Every lane of the quad takes part in the butterflies (a quad lies entirely inside
      // or entirely past the row's blocks; rows past the end hold zeros and are not stored).
      float v[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) decode2<DT>(d[i], v[2 * i], v[2 * i + 1]);
      fwht128_quad(v, lane & 3);
      if (pscale != 1.0f) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] *= pscale;
      }
      if (row < rows && blk < nb) mxq_block_f32<FMT>(v, row, blk, rows8, block_at(row, blk), scales);
    } else {
      if (row < rows && blk < nb) mxq_block<DT, FMT>(d, row, blk, rows8, block_at(row, blk), scales);
    }
    // LDS operations of one wave complete in order, so the next pass's writes cannot pass
    // these reads; this only keeps the compiler from moving them across.
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------------ GEMM

constexpr int MX_BM = 256, MX_BN = 256, MX_BK = 64;
constexpr int MX_NT = 512;
constexpr int MX_WTM = 128, MX_WTN = 64;
constexpr int MX_MBLK = MX_WTM / 32, MX_NBLK = MX_WTN / 32;

// A ring stage holds S consecutive 64-deep MFMA steps ("sub-steps") of both operands and
// their scales; one barrier per stage, so S = 2 halves the synchronization per MFMA.
template <int FA, int S>
struct MxCfg {
  static constexpr int A_ROW = MxFmt<FA>::STEP_BYTES * S;  // 32/64 (FP4) or 48/96 (FP6) bytes
  static constexpr int B_ROW = 32 * S;
  static constexpr int A_BYTES = MX_BM * A_ROW;
  static constexpr int B_BYTES = MX_BN * B_ROW;
  static constexpr int SA_OFF = A_BYTES + B_BYTES;  // per sub-step: 256 x 2 scale bytes of A, then of B
  static constexpr int STAGE = SA_OFF + 1024 * S;
  static constexpr int NST = (160 * 1024) / STAGE > 6 ? 6 : (160 * 1024) / STAGE;
  // Direct loads per wave and stage: A slots (1 KB, or 768 B of dense FP6 rows), B slots,
  // and one 8-lane scale slot per sub-step.
  static constexpr int LA = FA == MX_FP4 ? A_BYTES / 8192 : A_BYTES / (8 * 768);
  static constexpr int LB = B_BYTES / 8192;
  static constexpr int L = LA + LB + S;
};

struct MxArgs {
  const uint8_t* a;   // activations: codes [m x row bytes], scales [k/64][m8][2]
  const uint8_t* sa;
  const uint8_t* b;   // weights: FP4 codes [n x k/2], scales [k/64][n8][2]
  const uint8_t* sb;
  void* y;
  int m, n, k;
  int64_t m8, n8;
  int64_t ldy;
  int vec_store;
  int tiles_m, tiles_n;
  // Remainder split (as in the integer GEMM): items [0, dp_items) are whole tiles, then
  // every remaining tile as `split` ranges of K stages whose float32 partials meet in
  // the workspace.  Two ranges at most: adding two partials is commutative, so the
  // result does not depend on which range arrives last.
  int dp_items, split, items;
  int32_t* ws_cnt;
  uint64_t* ws_part;
  int64_t b_kp;  // weights in 64-byte K pieces: bytes from one piece to the next (64 n)
};

// Two schedules of the same K loop.  Interleaved (PP false, S = 1): every wave reads the
// next stage's fragments while the MFMAs of the current one run, one barrier per stage.
// Ping-pong (PP true, S = 2): the two waves of a SIMD (w and w + 4) alternate between a
// memory phase (the fragment reads of a whole stage and this wave's share of the refill
// loads) and a compute phase (the stage's MFMAs from registers), waves 0-3 one phase
// ahead of waves 4-7, two barriers per stage; the refill of stage p + 2 is issued in the
// memory phase of stage p into the slot read at stage p + 2 - NST, whose readers passed
// a barrier before.
// KB: the weights in 64-byte K pieces (vq_mx_quant with VQ_W_KBLOCK); a stage's weight
// bytes of a row (32 or 64) then lie in one piece, and a tile's rows are consecutive.
template <int FA, int S, int OUT_DT, bool PP, bool KB>
__global__ __launch_bounds__(MX_NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_mxgemm(MxArgs g) {
  using C = MxCfg<FA, S>;
  static_assert(PP ? (S == 2 && C::NST >= 3) : S == 1,
                "ping-pong: two sub-steps, three stages; interleaved: one sub-step");
  constexpr int PD = 2;                         // ping-pong refill distance (stages)
  constexpr int PRO = PP ? PD : C::NST - 1;     // stages requested ahead of a tile
  constexpr bool HALF_OUT = OUT_DT != DT_F32;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NST * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // wave grid 2 (M) x 4 (N)
  const int nk = g.k / (MX_BK * S);  // ring stages along K
  __shared__ int s_last;
  const int64_t a_rowb = (int64_t)g.k * MxFmt<FA>::W / 8;
  const int64_t b_rowb = KB ? 64 : g.k / 2;
  // Offset of byte c of a weight row from the row's first byte.
  auto bofs = [&](int64_t c) -> int64_t { return KB ? (c >> 6) * g.b_kp + (c & 63) : c; };

  // ---- direct-load assignment (per lane, per stage).
  // 64-byte rows (FP4, S = 2): 1 KB slot = 16 rows, lane -> row lane/4, chunk (lane & 3)
  //   ^ swz64(row), as in the integer kernel.  32-byte rows (FP4, S = 1): 1 KB = 32 rows,
  //   lane -> row lane/2, chunk (lane & 1) ^ swz32(row).  Dense FP6 rows of 48 or 96 B:
  //   768 B slots (lanes 0-47), lane -> row and 16-byte piece in row order.
  // Scales: per sub-step 128 B per wave (lanes 0-7): waves 0-3 carry the A scales of rows
  //   64w .. 64w+63, waves 4-7 the B scales.
  auto assign64 = [&](int q, int& r, int& c) {
    if constexpr (S == 2) {
      r = 16 * q + (lane >> 2);
      c = 16 * ((lane & 3) ^ swz64(r));
    } else {
      r = 32 * q + (lane >> 1);
      c = 16 * ((lane & 1) ^ swz32(r));
    }
  };
  int ra[C::LA], ca[C::LA], la_off[C::LA];
  bool a_on[C::LA];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int q = wave * C::LA + i;
    if constexpr (FA == MX_FP4) {
      assign64(q, ra[i], ca[i]);
      la_off[i] = q * 1024;
      a_on[i] = true;
    } else {
      constexpr int PIECES = C::A_ROW / 16;  // 3 or 6 pieces per row
      constexpr int ROWS = 48 / PIECES;      // rows per 768 B slot
      ra[i] = ROWS * q + lane / PIECES;
      ca[i] = 16 * (lane % PIECES);
      la_off[i] = q * 768;
      a_on[i] = lane < 48;
    }
  }
  int rb[C::LB], cb[C::LB], lb_off[C::LB];
#pragma unroll
  for (int i = 0; i < C::LB; ++i) {
    const int q = wave * C::LB + i;
    assign64(q, rb[i], cb[i]);
    lb_off[i] = C::A_BYTES + q * 1024;
  }
  const bool s_on = lane < 8;
  const bool s_is_a = wave < 4;
  const int s_row0 = 64 * (wave & 3) + 8 * lane;  // first tile row of this lane's 16 scale bytes
  const int ls_off = C::SA_OFF + wave * 128;

  const uint8_t* ga[C::LA];
  const uint8_t* gb[C::LB];
  const uint8_t* gs;
  int64_t s_pitch = 0;  // bytes between the scale slabs of consecutive steps
  int m0 = 0, n0 = 0;
  int kb0 = 0, nks = nk;     // the item's first stage and stage count
  int part = -1, rslot = 0;  // K range of a split tile (-1: whole tile) and its remainder index
  auto set_tile = [&](int w) {
    const WorkItem it = item_of(w, g.dp_items, g.split, nk);
    kb0 = it.kb0;
    nks = it.nks;
    part = it.part;
    rslot = it.rslot;
    int tm, tn;
    tile_of(it.tile, g.tiles_m, g.tiles_n, tm, tn);
    m0 = tm * MX_BM;
    n0 = tn * MX_BN;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) ga[i] = g.a + (int64_t)min(m0 + ra[i], g.m - 1) * a_rowb + ca[i];
#pragma unroll
    for (int i = 0; i < C::LB; ++i) gb[i] = g.b + (int64_t)min(n0 + rb[i], g.n - 1) * b_rowb + cb[i];
    // Scale chunk of 8 rows: clamped to the last whole chunk of the (8-padded) slab.
    if (s_is_a) {
      const int64_t r = min((int64_t)m0 + s_row0, g.m8 - 8);
      gs = g.sa + r * 2;
      s_pitch = g.m8 * 2;
    } else {
      const int64_t r = min((int64_t)n0 + s_row0, g.n8 - 8);
      gs = g.sb + r * 2;
      s_pitch = g.n8 * 2;
    }
  };
  auto issue = [&](int kt, int slot) {
    uint8_t* base = lds + slot * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::LA; ++i)
      if (a_on[i]) dma16(ga[i] + (int64_t)kt * C::A_ROW, base + la_off[i]);
#pragma unroll
    for (int i = 0; i < C::LB; ++i) dma16(gb[i] + bofs((int64_t)kt * C::B_ROW), base + lb_off[i]);
#pragma unroll
    for (int sub = 0; sub < S; ++sub)
      if (s_on) dma16(gs + (int64_t)(kt * S + sub) * s_pitch, base + ls_off + sub * 1024);
  };
  auto issue_prologue = [&]() {
#pragma unroll
    for (int s = 0; s < PRO; ++s)
      if (s < nks) issue(kb0 + s, s);
  };

  // ---- fragment offsets: rows 32*blk + (lane & 31); sub-step u, K half lane >> 5.
  const int rl = lane & 31;
  const int kh = lane >> 5;
  int fa_off[S], fb_off[S];
#pragma unroll
  for (int u = 0; u < S; ++u) {
    if constexpr (FA == MX_FP4) {
      fa_off[u] = (wm * MX_WTM + rl) * C::A_ROW +
                  16 * (S == 2 ? ((2 * u + kh) ^ swz64(rl)) : (kh ^ swz32(rl)));
    } else {
      fa_off[u] = (wm * MX_WTM + rl) * C::A_ROW + 48 * u + 24 * kh;
    }
    fb_off[u] = C::A_BYTES + (wn * MX_WTN + rl) * C::B_ROW +
                16 * (S == 2 ? ((2 * u + kh) ^ swz64(rl)) : (kh ^ swz32(rl)));
  }
  const int fsa_off = C::SA_OFF + (wm * MX_WTM + rl) * 2 + kh;
  const int fsb_off = C::SA_OFF + 512 + (wn * MX_WTN + rl) * 2 + kh;

  // Operands of one sub-step: A fragments (4 or 6 dwords), B fragments, scale bytes.
  struct Frag {
    v8i a[MX_MBLK];
    v8i b[MX_NBLK];
    int sa[MX_MBLK];
    int sb[MX_NBLK];
  };
  auto load_sub = [&](int slot, int u, Frag& f) {
    const uint8_t* st = lds + slot * C::STAGE;
#pragma unroll
    for (int nb = 0; nb < MX_NBLK; ++nb) {
      const v4i w = *reinterpret_cast<const v4i*>(st + fb_off[u] + nb * 32 * C::B_ROW);
      f.b[nb] = v8i{w.x, w.y, w.z, w.w, 0, 0, 0, 0};
      f.sb[nb] = st[fsb_off + u * 1024 + nb * 32 * 2];
    }
#pragma unroll
    for (int mb = 0; mb < MX_MBLK; ++mb) {
      if constexpr (FA == MX_FP4) {
        const v4i w = *reinterpret_cast<const v4i*>(st + fa_off[u] + mb * 32 * C::A_ROW);
        f.a[mb] = v8i{w.x, w.y, w.z, w.w, 0, 0, 0, 0};
      } else {
        const uint8_t* p = st + fa_off[u] + mb * 32 * C::A_ROW;
        const u2v w0 = *reinterpret_cast<const u2v*>(p);
        const u2v w1 = *reinterpret_cast<const u2v*>(p + 8);
        const u2v w2 = *reinterpret_cast<const u2v*>(p + 16);
        f.a[mb] = v8i{(int)w0.x, (int)w0.y, (int)w1.x, (int)w1.y, (int)w2.x, (int)w2.y, 0, 0};
      }
      f.sa[mb] = st[fsa_off + u * 1024 + mb * 32 * 2];
    }
  };

  v16f acc[MX_MBLK][MX_NBLK];
  // Weights are the MFMA's A operand (FP4), activations its B operand (FA).
  auto mma_nb = [&](const Frag& f, int nb) {
#pragma unroll
    for (int mb = 0; mb < MX_MBLK; ++mb)
      acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[nb], f.a[mb], acc[mb][nb], MX_FP4, FA, 0,
                                                                    f.sb[nb], 0, f.sa[mb]);
  };
  auto mma_sub = [&](const Frag& f) {
#pragma unroll
    for (int nb = 0; nb < MX_NBLK; ++nb) mma_nb(f, nb);
  };
  auto wait_loads = [&](int later) {  // at most `later` load groups may stay in flight
    if (later >= 4) {
      wait_vmcnt<4 * C::L>();
    } else if (later == 3) {
      wait_vmcnt<3 * C::L>();
    } else if (later == 2) {
      wait_vmcnt<2 * C::L>();
    } else if (later == 1) {
      wait_vmcnt<C::L>();
    } else {
      wait_vmcnt<0>();
    }
  };

  int vt = blockIdx.x;
  if (vt >= g.items) return;
  set_tile(vt);
  issue_prologue();
  // pend (ping-pong): the previous tile's 16 output stores were issued after this tile's
  // first loads, so the first waits of this tile leave them in flight (vmcnt is in order).
  bool pend = false;
  for (;;) {
#pragma unroll
    for (int i = 0; i < MX_MBLK; ++i)
#pragma unroll
      for (int j = 0; j < MX_NBLK; ++j) acc[i][j] = v16f{};

    if constexpr (PP) {
      const int grp = wave >> 2;
      auto reads_done = [&]() { __builtin_amdgcn_s_waitcnt(0xC07F); };  // lgkmcnt(0)
      if (nks >= 2) {
        if (pend) wait_vmcnt<C::L + 16>();
        else wait_vmcnt<C::L>();
      } else {
        if (pend) wait_vmcnt<16>();
        else wait_vmcnt<0>();
      }
      sched_barrier_all();
      if (grp == 1) sched_barrier_all();
      Frag f[S];
      int p = 0, slot = 0;
      for (; p + PD < nks; ++p) {
        // memory phase (waves 0-3: while waves 4-7 compute stage p - 1)
#pragma unroll
        for (int u = 0; u < S; ++u) load_sub(slot, u, f[u]);
        const int fill = slot + PD >= C::NST ? slot + PD - C::NST : slot + PD;
        issue(kb0 + p + PD, fill);
        const bool early = pend && p == 0;  // stage 1 was requested before the stores
        if (grp == 1) {
          if (early) wait_vmcnt<C::L + 16>();
          else wait_vmcnt<C::L>();
        }
        reads_done();
        sched_barrier_all();
        // compute phase
#pragma unroll
        for (int u = 0; u < S; ++u) mma_sub(f[u]);
        if (grp == 0) {
          if (early) wait_vmcnt<C::L + 16>();
          else wait_vmcnt<C::L>();
        }
        sched_barrier_all();
        slot = slot + 1 == C::NST ? 0 : slot + 1;
      }
      for (; p < nks; ++p) {
#pragma unroll
        for (int u = 0; u < S; ++u) load_sub(slot, u, f[u]);
        if (grp == 1) {
          if (pend && p == 0) wait_vmcnt<16>();
          else wait_vmcnt<0>();
        }
        reads_done();
        sched_barrier_all();
#pragma unroll
        for (int u = 0; u < S; ++u) mma_sub(f[u]);
        if (grp == 0) {
          if (pend && p == 0) wait_vmcnt<16>();
          else wait_vmcnt<0>();
        }
        sched_barrier_all();
        slot = slot + 1 == C::NST ? 0 : slot + 1;
      }
      if (grp == 0) sched_barrier_all();
    } else {
      Frag f0, f1;
      wait_loads(min(C::NST - 2, nks - 1));
      barrier_nofence();
      load_sub(0, 0, f0);
      int kt = 0, slot = 0;
      // One sub-step per stage: the MFMAs of weight block 0 run on operands read during
      // stage kt-1; then every wave waits for its loads of stage kt+1 and meets the others
      // at a barrier, which publishes stage kt+1 and certifies that stage kt-1 is no longer
      // read (that slot receives stage kt+NST-1); then the operands of stage kt+1 are read
      // while the MFMAs of weight block 1 run.
      for (; kt < nks - (C::NST - 1); ++kt) {
        const int next = slot + 1 == C::NST ? 0 : slot + 1;
        const int refill = slot == 0 ? C::NST - 1 : slot - 1;
        mma_nb(f0, 0);
        wait_vmcnt<(C::NST - 3) * C::L>();
        barrier_nofence();
        issue(kb0 + kt + C::NST - 1, refill);
        load_sub(next, 0, f1);
        mma_nb(f0, 1);
        f0 = f1;
        slot = next;
      }
      for (; kt < nks; ++kt) {
        const int next = slot + 1 == C::NST ? 0 : slot + 1;
        mma_nb(f0, 0);
        if (kt + 1 < nks) {
          wait_loads(nks - 2 - kt);
          barrier_nofence();
          load_sub(next, 0, f1);
        }
        mma_nb(f0, 1);
        f0 = f1;
        slot = next;
      }
    }  // interleaved schedule

    // ------------------------------------------------------------ remainder split
    if (part >= 0) {  // the block's last item: nothing is in flight
      constexpr int WORDS = MX_MBLK * MX_NBLK * 8;
      split_publish(g.ws_part + (int64_t)(rslot * g.split + part) * (WORDS * MX_NT), MX_NT, tid, acc);
      if (!split_arrive(&g.ws_cnt[rslot], g.split, &s_last)) break;
      for (int p2 = 0; p2 < g.split; ++p2)
        if (p2 != part)
          split_accumulate(g.ws_part + (int64_t)(rslot * g.split + p2) * (WORDS * MX_NT), MX_NT, tid, acc);
      split_reset(&g.ws_cnt[rslot]);
    }

    // ------------------------------------------------------------ epilogue
    const int nvt = vt + (int)gridDim.x;
    const bool has_next = nvt < g.items;
    const int cm0 = m0, cn0 = n0;
    barrier_nofence();  // every wave is done with the ring
    if (has_next) {
      set_tile(nvt);
      issue_prologue();
    }
    // A whole tile with aligned rows stores exactly MBLK * NBLK * 2 = 16 times per wave.
    pend = PP && HALF_OUT && has_next && g.vec_store && cm0 + MX_BM <= g.m && cn0 + MX_BN <= g.n;
    // Output layout of a 32 x 32 block: lane holds column m = lane & 31 (activation row)
    // and, for group q = 0..3, rows n = 8q + 4 * (lane >> 5) + 0..3 (weight rows); the
    // block scales are already applied by the matrix cores.
    const int mrow = wm * MX_WTM + (lane & 31);
    const int ncol = wn * MX_WTN + 4 * (lane >> 5);
    typedef typename std::conditional<OUT_DT == DT_BF16, __bf16, _Float16>::type h_t;
#pragma unroll
    for (int mb = 0; mb < MX_MBLK; ++mb) {
      const int m = cm0 + mrow + mb * 32;
#pragma unroll
      for (int nb = 0; nb < MX_NBLK; ++nb) {
        u2v hw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = cn0 + ncol + nb * 32 + 8 * q;
          float out[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) out[r] = acc[mb][nb][4 * q + r];
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
          // Lanes l and l+32 exchange column groups so that each holds eight consecutive
          // outputs of its row (one 16-byte store).
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const u2v X = hw[2 * pr], Y = hw[2 * pr + 1];
            const auto s0 = __builtin_amdgcn_permlane32_swap(X.x, Y.x, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(X.y, Y.y, false, false);
            const u4v w = {s0[0], s1[0], s0[1], s1[1]};
            const int no = cn0 + wn * MX_WTN + nb * 32 + 16 * pr + 8 * (lane >> 5);
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
    vt = nvt;
  }
}

}  // namespace vqk

namespace vq_internal {

using namespace vqk;

int64_t mx_rows8(int64_t rows) { return (rows + 7) / 8 * 8; }

hipError_t launch_mx_quant(const void* x, int dtype, int64_t ldx, int64_t rows, int64_t k, int fmt, uint8_t* codes,
                           uint8_t* scales, hipStream_t st, bool had, int exp_offset, bool kblock) {
  if (kblock && fmt != MX_FP4) return hipErrorInvalidValue;
  const int64_t tiles = (rows + 7) / 8 * ((k / 32 + 7) / 8);
  const int64_t wgs = (tiles + 3) / 4;  // four waves, one 8 x 8-block tile each, per workgroup and pass
  const unsigned grid = (unsigned)(wgs < 8192 ? wgs : 8192);
  const int64_t r8 = mx_rows8(rows);
  const float pscale = ldexpf(1.0f, exp_offset);  // exact: |exp_offset| <= 64
#define MXQ(DTV, FV, H, KBV)                                                                                  \
  hipLaunchKernelGGL((k_mxquant<DTV, FV, H, KBV>), dim3(grid), dim3(256), 0, st, x, ldx, rows, (int)k, r8, codes, \
                     scales, pscale)
#define MXQ4(DTV, H) \
  if (kblock) MXQ(DTV, MX_FP4, H, true); else MXQ(DTV, MX_FP4, H, false)
  if (dtype == DT_F16) {
    if (fmt == MX_FP4) {
      if (had) { MXQ4(DT_F16, true); } else { MXQ4(DT_F16, false); }
    } else {
      if (had) MXQ(DT_F16, MX_FP6, true, false); else MXQ(DT_F16, MX_FP6, false, false);
    }
  } else {
    if (fmt == MX_FP4) {
      if (had) { MXQ4(DT_BF16, true); } else { MXQ4(DT_BF16, false); }
    } else {
      if (had) MXQ(DT_BF16, MX_FP6, true, false); else MXQ(DT_BF16, MX_FP6, false, false);
    }
  }
#undef MXQ4
#undef MXQ
  return hipGetLastError();
}

// Remainder split of the MX GEMM: two K ranges per tile past the last whole round, when
// K has at least 96 steps of 64 (the integer GEMM's measured break-even) and the ranges
// fit in one round.
static int mx_split_of(int tiles, int grid, int64_t k) {
  const int rem = tiles % grid;
  if (rem == 0 || k / 64 < 96 || grid > 1024 || grid / rem < 2) return 1;
  return 2;
}

int64_t mx_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const int tiles = (int)(((m + MX_BM - 1) / MX_BM) * ((n + MX_BN - 1) / MX_BN));
  const int grid = persistent_blocks();
  if (mx_split_of(tiles, grid, k) == 1) return 0;
  return 4096 + (int64_t)(tiles % grid) * 2 * (MX_MBLK * MX_NBLK * 8) * MX_NT * 8;
}

hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* sa, int fa, const uint8_t* b, const uint8_t* sb, int64_t m,
                          int64_t n, int64_t k, void* y, int out_dt, int64_t ldy, void* ws, hipStream_t st,
                          bool b_kblock) {
  MxArgs g{};
  g.a = a;
  g.sa = sa;
  g.b = b;
  g.sb = sb;
  g.y = y;
  g.m = (int)m;
  g.n = (int)n;
  g.k = (int)k;
  g.m8 = mx_rows8(m);
  g.n8 = mx_rows8(n);
  g.ldy = ldy;
  g.b_kp = 64 * n;
  const int64_t esize = out_dt == DT_F32 ? 4 : 2;
  g.vec_store = ((reinterpret_cast<uintptr_t>(y) & 15u) == 0 && (ldy * esize) % 16 == 0) ? 1 : 0;
  g.tiles_m = (int)((m + MX_BM - 1) / MX_BM);
  g.tiles_n = (int)((n + MX_BN - 1) / MX_BN);
  const int tiles = g.tiles_m * g.tiles_n;
  const int pb = persistent_blocks();
  g.split = ws ? mx_split_of(tiles, pb, k) : 1;
  g.dp_items = g.split > 1 ? tiles - tiles % pb : tiles;
  g.items = g.dp_items + (tiles - g.dp_items) * g.split;
  g.ws_cnt = g.split > 1 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  g.ws_part = g.split > 1 ? reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(ws) + 4096) : nullptr;
  const int grid = g.items < pb ? g.items : pb;
  // FP4 activations: two 64-deep sub-steps per ring stage on the ping-pong schedule when K
  // allows it.  FP6 activations stay at one sub-step on the interleaved schedule: with two
  // sub-steps (42 KB stages, three in the ring) the ping-pong form measured 19% slower.
  const bool two = fa == MX_FP4 && k % 128 == 0;
#define MXG(F, SS, O)                                                                          \
  if (b_kblock)                                                                                \
    hipLaunchKernelGGL((k_mxgemm<F, SS, O, SS == 2, true>), dim3(grid), dim3(MX_NT), 0, st, g); \
  else                                                                                         \
    hipLaunchKernelGGL((k_mxgemm<F, SS, O, SS == 2, false>), dim3(grid), dim3(MX_NT), 0, st, g)
#define MXO(F, SS)              \
  if (out_dt == DT_F16) {       \
    MXG(F, SS, DT_F16);         \
  } else if (out_dt == DT_BF16) { \
    MXG(F, SS, DT_BF16);        \
  } else {                      \
    MXG(F, SS, DT_F32);         \
  }
  if (fa == MX_FP4) {
    if (two) { MXO(MX_FP4, 2); } else { MXO(MX_FP4, 1); }
  } else {
    MXO(MX_FP6, 1);
  }
#undef MXO
#undef MXG
  return hipGetLastError();
}

}  // namespace vq_internal
