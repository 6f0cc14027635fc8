// Activation decomposition for gfx950: residual re-quantization of selected tokens.
//
// SemanticDialect (gist.science, arXiv 2603.02883), Methodology 2.2: after an activation
// is quantized, the quantization error that remains is quantized once more and its
// contribution is added to the layer output; only selected (salient) tokens are
// decomposed, to keep the bit budget.
//
// Per listed row x (one 256-thread workgroup per row, the row read three times, the
// second and third times from L2):
//   pass 1: a1 = max|x|; r1 = fl32(Q1/a1), s1 = fl32(a1/Q1)
//   pass 2: q1 = clamp(rne(fl32(x*r1)), -Q1, Q1) exactly as the per-token quantizer;
//           deq = fl32(q1*s1), res = fl32(x - deq), a2 = max|res|; r2, s2 from a2 and Q2
//   pass 3: q1 and q2 = clamp(rne(fl32(res*r2)), -Q2, Q2), stored one per int8
// The codes form a stacked operand of 2R rows (row i: q1 of listed row i, row R+i: its
// q2), so that one small GEMM yields both terms of every listed row; a merge kernel then
// writes y = fl32(y1 + y2) rounded once over the plain GEMM's row.  The maxima are exact
// (order-independent) and every other step is elementwise, so codes, scales and outputs
// are bit-identical to any correct evaluation of the same steps.
#include <type_traits>

#include "dev_common.h"
#include "vq_internal.h"

namespace vqk {

constexpr int RQ_THREADS = 256;

// Signed code of clamp(rne(x * r), -qf, qf) (the low bits of fl(t + 1.5 * 2^23)).
__device__ __forceinline__ int qcode(float x, float r, float qf) {
  return (int)(qbyte(x, r, qf) - 0x4B400000u);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
  for (int w = 1; w < RQ_THREADS / 64; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

template <int DT>
__global__ __launch_bounds__(RQ_THREADS) void k_residual_quant(const void* x, int64_t ldx, int64_t m, int k,
                                                                const int32_t* rows, int64_t n_rows, float qf1,
                                                                float qf2, int8_t* codes, float* scales) {
  __shared__ float red[RQ_THREADS / 64];
  const int i = blockIdx.x;
  const int64_t row = rows[i];
  int8_t* out1 = codes + (int64_t)i * k;
  int8_t* out2 = codes + (int64_t)(n_rows + i) * k;
  if (row < 0 || row >= m) {  // not a row of x: zero codes and scales (block-uniform exit)
    for (int c = threadIdx.x; c < k / 8; c += RQ_THREADS) {
      *reinterpret_cast<u2v*>(out1 + (int64_t)c * 8) = u2v{0u, 0u};
      *reinterpret_cast<u2v*>(out2 + (int64_t)c * 8) = u2v{0u, 0u};
    }
    if (threadIdx.x == 0) {
      scales[i] = 0.0f;
      scales[n_rows + i] = 0.0f;
    }
    return;
  }
  const char* xr = reinterpret_cast<const char*>(x) + row * ldx * 2;
  const int chunks = k / 8;  // 8 elements (16 bytes) per chunk

  auto load8 = [&](int c, float v[8]) {
    const u4v w = *reinterpret_cast<const u4v*>(xr + (int64_t)c * 16);
    decode2<DT>(w.x, v[0], v[1]);
    decode2<DT>(w.y, v[2], v[3]);
    decode2<DT>(w.z, v[4], v[5]);
    decode2<DT>(w.w, v[6], v[7]);
  };

  float m1 = 0.0f;
  for (int c = threadIdx.x; c < chunks; c += RQ_THREADS) {
    float v[8];
    load8(c, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) m1 = fmaxf(m1, fabsf(v[t]));
  }
  float r1, s1;
  dyn_scale(block_max(m1, red), qf1, r1, s1);

  auto residual = [&](float v) {
    const float deq = (float)qcode(v, r1, qf1) * s1;
    return v - deq;
  };
  float m2 = 0.0f;
  for (int c = threadIdx.x; c < chunks; c += RQ_THREADS) {
    float v[8];
    load8(c, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) m2 = fmaxf(m2, fabsf(residual(v[t])));
  }
  float r2, s2;
  dyn_scale(block_max(m2, red), qf2, r2, s2);

  for (int c = threadIdx.x; c < chunks; c += RQ_THREADS) {
    float v[8];
    load8(c, v);
    unsigned u[8], w[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u[t] = qbyte(v[t], r1, qf1);
      w[t] = qbyte(residual(v[t]), r2, qf2);
    }
    *reinterpret_cast<u2v*>(out1 + (int64_t)c * 8) = u2v{pack4_lo(u[0], u[1], u[2], u[3]), pack4_lo(u[4], u[5], u[6], u[7])};
    *reinterpret_cast<u2v*>(out2 + (int64_t)c * 8) = u2v{pack4_lo(w[0], w[1], w[2], w[3]), pack4_lo(w[4], w[5], w[6], w[7])};
  }
  if (threadIdx.x == 0) {
    scales[i] = s1;
    scales[n_rows + i] = s2;
  }
}

// y[rows[i], j] = RNE(fl32(y12[i, j] + y12[R + i, j])) for the listed rows that exist;
// y12 is float32 [2R x n] (row pitch n): the two dequantized terms of each listed row.
constexpr int MERGE_COLS = 1024;  // columns per workgroup

template <int OUT_DT>
__global__ void k_residual_merge(const float* y12, int64_t n_rows, int64_t n, const int32_t* rows, int64_t m,
                                 void* y, int64_t ldy) {
  const int64_t cb = (n + MERGE_COLS - 1) / MERGE_COLS;
  const int64_t i = blockIdx.x / cb;
  const int64_t j0 = (blockIdx.x % cb) * MERGE_COLS;
  const int64_t row = rows[i];
  if (row < 0 || row >= m) return;
  const float* a = y12 + i * n;
  const float* b = y12 + (n_rows + i) * n;
  const int64_t j1 = j0 + MERGE_COLS < n ? j0 + MERGE_COLS : n;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += blockDim.x) {
    const float v = a[j] + b[j];
    if constexpr (OUT_DT == DT_F32) {
      reinterpret_cast<float*>(y)[row * ldy + j] = v;
    } else {
      typedef typename std::conditional<OUT_DT == DT_BF16, __bf16, _Float16>::type h_t;
      reinterpret_cast<h_t*>(y)[row * ldy + j] = (h_t)f32_fence(v);
    }
  }
}

}  // namespace vqk

namespace vq_internal {

using namespace vqk;

hipError_t launch_residual_quant(const void* x, int dtype, int64_t ldx, int64_t m, int64_t k, const int32_t* rows,
                                 int64_t n_rows, int bits1, int bits2, int8_t* codes, float* scales,
                                 hipStream_t st) {
  const float qf1 = (float)((1 << (bits1 - 1)) - 1), qf2 = (float)((1 << (bits2 - 1)) - 1);
  if (dtype == 0)
    hipLaunchKernelGGL(k_residual_quant<DT_F16>, dim3((unsigned)n_rows), dim3(RQ_THREADS), 0, st, x, ldx, m, (int)k,
                       rows, n_rows, qf1, qf2, codes, scales);
  else
    hipLaunchKernelGGL(k_residual_quant<DT_BF16>, dim3((unsigned)n_rows), dim3(RQ_THREADS), 0, st, x, ldx, m, (int)k,
                       rows, n_rows, qf1, qf2, codes, scales);
  return hipGetLastError();
}

hipError_t launch_residual_merge(const float* y12, int64_t n_rows, int64_t n, const int32_t* rows, int64_t m, void* y,
                                 int out_dt, int64_t ldy, hipStream_t st) {
  const dim3 grid((unsigned)(n_rows * ((n + MERGE_COLS - 1) / MERGE_COLS)));
  switch (out_dt) {
    case DT_F16: hipLaunchKernelGGL(k_residual_merge<DT_F16>, grid, dim3(256), 0, st, y12, n_rows, n, rows, m, y, ldy); break;
    case DT_BF16: hipLaunchKernelGGL(k_residual_merge<DT_BF16>, grid, dim3(256), 0, st, y12, n_rows, n, rows, m, y, ldy); break;
    default: hipLaunchKernelGGL(k_residual_merge<DT_F32>, grid, dim3(256), 0, st, y12, n_rows, n, rows, m, y, ldy); break;
  }
  return hipGetLastError();
}

}  // namespace vq_internal
