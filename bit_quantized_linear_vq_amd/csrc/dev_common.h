// Device helpers shared by the gfx950 kernels of the quantized linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));

enum : int { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2 };

__device__ __forceinline__ float bits_f(unsigned u) { return __builtin_bit_cast(float, u); }

// Materializes a float32 value in a register before it is narrowed: without it the
// compiler may fold fptrunc(fmul) into v_fma_mix*, rounding the exact product once to
// 16 bits instead of first to float32 and then to 16 bits.
__device__ __forceinline__ float f32_fence(float v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ unsigned f_bits(float f) { return __builtin_bit_cast(unsigned, f); }

// Two packed 16-bit values of a dword -> floats (element 2i in the low half).
template <int DT>
__device__ __forceinline__ void decode2(unsigned u, float& lo, float& hi) {
  if constexpr (DT == DT_BF16) {
    lo = bits_f(u << 16);
    hi = bits_f(u & 0xFFFF0000u);
  } else {
    _Float16 a = __builtin_bit_cast(_Float16, (unsigned short)(u & 0xFFFFu));
    _Float16 b = __builtin_bit_cast(_Float16, (unsigned short)(u >> 16));
    lo = (float)a;
    hi = (float)b;
  }
}

// One element of a storage dtype as float.
template <int DT>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
  if constexpr (DT == DT_BF16) {
    return bits_f(((unsigned)reinterpret_cast<const unsigned short*>(p)[i]) << 16);
  } else if constexpr (DT == DT_F16) {
    return (float)reinterpret_cast<const _Float16*>(p)[i];
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return bits_f((unsigned)__builtin_amdgcn_update_dpp(0, (int)f_bits(v), CTRL, 0xF, 0xF, false));
}

// Wave-wide maximum of non-negative floats (exact: max is order independent).  Register
// moves instead of LDS permutes: two quad swaps, the half-row and row mirrors make every
// lane hold its 16-lane row's maximum, and the four rows are combined from lanes 0, 16,
// 32 and 48 in scalar registers.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  const int b = (int)f_bits(v);
  const float r0 = bits_f((unsigned)__builtin_amdgcn_readlane(b, 0));
  const float r1 = bits_f((unsigned)__builtin_amdgcn_readlane(b, 16));
  const float r2 = bits_f((unsigned)__builtin_amdgcn_readlane(b, 32));
  const float r3 = bits_f((unsigned)__builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// 128-point Sylvester Hadamard butterflies held in registers.
//
// A 128-element block is spread over 8 consecutive lanes as two 8-element pieces per
// lane, 64 elements apart: lane slot l (0..7) holds elements 8g .. 8g+7 (v[0..7]) and
// 64 + 8g .. 64 + 8g+7 (v[8..15]), with g = perm8(l) and perm8 = (0,1,2,3,7,6,5,4).  A
// wave's load of one piece then covers whole 128-byte lines (8 lanes x 16 bytes per
// block half).  Butterfly distances 1, 2, 4 are inside a piece, 64 pairs the two pieces
// of a lane, and with the slot assignment above the three cross-lane distances map onto
// single DPP moves:
//   h = 8  (group bit 0): lane xor 1      -> quad_perm [1,0,3,2]
//   h = 16 (group bit 1): lane xor 2      -> quad_perm [2,3,0,1]
//   h = 32 (group bit 2): lane 7 - lane   -> row_half_mirror
// The stages run in ascending h, as the transform's definition does them.
//
// Cross-lane stages keep a per-lane sign: the lane holding the lower index of a pair
// computes fl(mine + partner); the upper lane computes fl(mine - partner), which is
// exactly -(z_lo - z_hi).  Partners always carry the same sign, so the stored value is
// sigma * z with sigma = (-1)^popcount(g); the last stage pairs two values of one lane,
// which carry the same sign; negation is exact in IEEE arithmetic, so sigma is folded
// into the consumer's multiplier.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int perm8(int l) { return l < 4 ? l : 11 - l; }

__device__ __forceinline__ float had_sigma(int g) { return (__builtin_popcount(g) & 1) ? -1.0f : 1.0f; }

// All seven stages; g = this lane's element group (0..7).  Returns sigma.
// Cross-lane stage: v = fl(partner * c + mine) with c = +1 on the lower lane of the
// pair and -1 on the upper lane; partner * c is exact, so the fma rounds once.
// FUSED_DPP: each cross-lane stage as one v_fmac_f32 reading the partner through DPP
// (inline asm: the compiler keeps the DPP move and the fma apart), for the quantizer, whose
// fused rotation is VALU-bound; the memory-bound standalone rotation keeps the compiler's
// two-instruction form, which measured faster there.
template <bool FUSED_DPP>
__device__ __forceinline__ float fwht128(float v[16], int g) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  const float c0 = (g & 1) ? -1.0f : 1.0f;
  const float c1 = (g & 2) ? -1.0f : 1.0f;
  const float c2 = (g & 4) ? -1.0f : 1.0f;
  if constexpr (FUSED_DPP) {
    // v = fl(partner * c + v) in one instruction, exact product.  A DPP read needs two wait
    // states after a VALU write of the same register: the first stage's inputs come from
    // compiler-scheduled code, so each of its instructions starts with an s_nop; in the
    // later stages every input was written by the previous stage's (ordered, volatile)
    // instruction for the same element, 15 instructions earlier.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float src = v[i];
      asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                   : "+v"(v[i]) : "v"(src), "v"(c0));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float src = v[i];
      asm volatile("v_fmac_f32_dpp %0, %1, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
                   : "+v"(v[i]) : "v"(src), "v"(c1));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float src = v[i];
      asm volatile("v_fmac_f32_dpp %0, %1, %2 row_half_mirror row_mask:0xf bank_mask:0xf"
                   : "+v"(v[i]) : "v"(src), "v"(c2));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(dpp_f<0xB1>(v[i]), c0, v[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(dpp_f<0x4E>(v[i]), c1, v[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(dpp_f<0x141>(v[i]), c2, v[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float a = v[i], b = v[i + 8];
    v[i] = a + b;
    v[i + 8] = a - b;
  }
  return had_sigma(g);
}

// ---------------------------------------------------------------------------
// Round-half-even quantization through the float32 magic constant 1.5 * 2^23:
// for |t| <= 2^22, fl(t + 12582912) = 12582912 + rne(t) exactly (the sum is
// rounded once, to an integer, and 12582912 is even), so the code's two's
// complement byte is the low byte of the sum's bit pattern.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned qbyte(float x, float r, float qf) {
  float t = x * r;
  t = __builtin_amdgcn_fmed3f(t, -qf, qf);
  return f_bits(t + 12582912.0f);
}

// r and s of a dynamic group with absolute maximum amax (a = 0 or an overflowing
// reciprocal give r = s = 0, so every code is 0).
__device__ __forceinline__ void dyn_scale(float amax, float qf, float& r, float& s) {
  r = qf / amax;
  s = amax / qf;
  if (!(amax > 0.0f) || __builtin_isinf(r)) {
    r = 0.0f;
    s = 0.0f;
  }
}

// Low bytes of four dwords -> one dword (byte i from u_i).
__device__ __forceinline__ unsigned pack4_lo(unsigned u0, unsigned u1, unsigned u2, unsigned u3) {
  unsigned lo = __builtin_amdgcn_perm(u1, u0, 0x0c0c0400u);
  unsigned hi = __builtin_amdgcn_perm(u3, u2, 0x04000c0cu);
  return lo | hi;
}

// Low nibbles of the low bytes of u[0..7] -> one dword of 8 packed 4-bit codes,
// element 2j in the low nibble of byte j.
__device__ __forceinline__ unsigned pack8_nibbles(const unsigned u[8]) {
  unsigned r = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    unsigned b = (u[2 * j] & 0xFu) | ((u[2 * j + 1] & 0xFu) << 4);
    r |= b << (8 * j);
  }
  return r;
}

}  // namespace vqk
