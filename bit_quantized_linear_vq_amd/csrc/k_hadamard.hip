// Standalone 128-point block Hadamard rotation for gfx950 (6Bit-Diffusion,
// gist.science arXiv 2603.18742, Methodology B.1: online block Hadamard transform of
// activations against outliers).
//
// Every 128-element block of every row is one unit of work for 8 lanes (two 8-element
// pieces per lane, 64 elements apart, see fwht128: each load and store of a wave
// then covers whole 128-byte lines); the blocks of all rows are numbered flat, so a wave
// transforms 8 blocks and lanes are never idle on ragged rows.  HBM-bound: 2 + 2 bytes
// per element for bf16 in and out, about ten VALU operations per element.
#include "dev_common.h"
#include "vq_internal.h"

namespace vqk {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned pack2(float a, float b, int dt) {
  a = f32_fence(a);
  b = f32_fence(b);
  if (dt == DT_BF16) {
    f2_t f = {a, b};
    bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(unsigned, h);
  }
  f2_t f = {a, b};
  f16x2_t h = __builtin_convertvector(f, f16x2_t);
  return __builtin_bit_cast(unsigned, h);
}

// Eight consecutive outputs.
template <int OUT_DT>
__device__ __forceinline__ void store8(void* p, const float* v) {
  u4v* q = reinterpret_cast<u4v*>(p);
  if constexpr (OUT_DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 2; ++i) q[i] = u4v{f_bits(v[4 * i]), f_bits(v[4 * i + 1]), f_bits(v[4 * i + 2]), f_bits(v[4 * i + 3])};
  } else {
    q[0] = u4v{pack2(v[0], v[1], OUT_DT), pack2(v[2], v[3], OUT_DT), pack2(v[4], v[5], OUT_DT), pack2(v[6], v[7], OUT_DT)};
  }
}

template <int IN_DT, int OUT_DT>
__global__ __launch_bounds__(256) void k_hadamard(const void* __restrict__ x, int64_t ldx, void* __restrict__ y,
                                                  int64_t ldy, int64_t rows, int64_t bpr, float cnorm) {
  const int lane = threadIdx.x & 63;
  const int g = perm8(lane & 7);
  const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3;
  const bool ok = blk < rows * bpr;
  const int64_t row = ok ? blk / bpr : 0;
  // The two 8-element pieces of this lane (see fwht128): elements 8g.. and 64+8g..
  const int64_t col = (ok ? blk - row * bpr : 0) * 128 + 8 * g;
  constexpr int ISZ = IN_DT == DT_F32 ? 4 : 2;
  constexpr int OSZ = OUT_DT == DT_F32 ? 4 : 2;
  constexpr int NW = IN_DT == DT_F32 ? 2 : 1;  // 16-byte words per piece
  // Both pieces' loads first (a lane past the end reads row 0 and discards it).
  u4v raw[2][NW];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int w = 0; w < NW; ++w)
      raw[h][w] = __builtin_nontemporal_load(
          reinterpret_cast<const u4v*>(reinterpret_cast<const char*>(x) + (row * ldx + col + 64 * h) * ISZ) + w);
  float v[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (IN_DT == DT_F32) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        v[8 * h + 4 * w + 0] = bits_f(raw[h][w].x);
        v[8 * h + 4 * w + 1] = bits_f(raw[h][w].y);
        v[8 * h + 4 * w + 2] = bits_f(raw[h][w].z);
        v[8 * h + 4 * w + 3] = bits_f(raw[h][w].w);
      }
    } else {
      decode2<IN_DT>(raw[h][0].x, v[8 * h + 0], v[8 * h + 1]);
      decode2<IN_DT>(raw[h][0].y, v[8 * h + 2], v[8 * h + 3]);
      decode2<IN_DT>(raw[h][0].z, v[8 * h + 4], v[8 * h + 5]);
      decode2<IN_DT>(raw[h][0].w, v[8 * h + 6], v[8 * h + 7]);
    }
  }
  const float sigma = fwht128<false>(v, g);
  const float c = sigma * cnorm;  // exact: sigma = +-1
#pragma unroll
  for (int t = 0; t < 16; ++t) v[t] = v[t] * c;
  if (ok) {
#pragma unroll
    for (int h = 0; h < 2; ++h) store8<OUT_DT>(reinterpret_cast<char*>(y) + (row * ldy + col + 64 * h) * OSZ, v + 8 * h);
  }
}

template <int IN_DT>
static hipError_t launch_out(int out_dt, const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows,
                             int64_t bpr, float cnorm, hipStream_t st) {
  const int64_t threads = rows * bpr * 8;
  const int64_t grid = (threads + 255) / 256;
  switch (out_dt) {
    case DT_F16:
      hipLaunchKernelGGL((k_hadamard<IN_DT, DT_F16>), dim3((unsigned)grid), dim3(256), 0, st, x, ldx, y, ldy, rows,
                         bpr, cnorm);
      break;
    case DT_BF16:
      hipLaunchKernelGGL((k_hadamard<IN_DT, DT_BF16>), dim3((unsigned)grid), dim3(256), 0, st, x, ldx, y, ldy,
                         rows, bpr, cnorm);
      break;
    default:
      hipLaunchKernelGGL((k_hadamard<IN_DT, DT_F32>), dim3((unsigned)grid), dim3(256), 0, st, x, ldx, y, ldy, rows,
                         bpr, cnorm);
      break;
  }
  return hipGetLastError();
}

}  // namespace vqk

namespace vq_internal {

using namespace vqk;

hipError_t launch_hadamard(const void* x, int in_dt, int64_t ldx, void* y, int out_dt, int64_t ldy, int64_t rows,
                           int64_t cols, int normalize, hipStream_t st) {
  // fl32(1/sqrt(128)) = 0x3DB504F3
  const float cnorm = normalize ? __builtin_bit_cast(float, 0x3DB504F3u) : 1.0f;
  const int64_t bpr = cols / 128;
  switch (in_dt) {
    case DT_F16: return launch_out<DT_F16>(out_dt, x, ldx, y, ldy, rows, bpr, cnorm, st);
    case DT_BF16: return launch_out<DT_BF16>(out_dt, x, ldx, y, ldy, rows, bpr, cnorm, st);
    default: return launch_out<DT_F32>(out_dt, x, ldx, y, ldy, rows, bpr, cnorm, st);
  }
}

}  // namespace vq_internal
