// Column sums of squares for outlier-channel detection, and the relative-L1 routing
// statistic, for gfx950.
//
// Q-ARVD (aitrends.kr), Methodology: the L2 norm of every input channel feeds the
// modified z-score.  The squares are accumulated in float64 in a fixed order (rows in
// ascending chunks, chunks summed in ascending order), so the result is reproducible
// run to run; the median and MAD are taken on the host.
//
// 6Bit-Diffusion (gist.science arXiv 2603.18742), Key Insights 1 and Methodology B.1:
// Gamma = sum|y - x| / sum|x| of a block's input and output at the previous timestep,
// compared with a threshold to route the block's activations to INT8 or 4 bits.  Both
// sums are float64 with a fixed reduction order; the decision is written to device
// memory for the quantization kernel, with no host round trip.
#include "dev_common.h"
#include "vq_internal.h"

namespace vqk {

constexpr int DET_MAX_CHUNKS = 256;

// Grid (column groups of 8 per thread, row chunks).  ws[chunk * cols + col].
template <int DT>
__global__ __launch_bounds__(256) void k_colsumsq_partial(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                          int64_t ldx, int64_t rows_per_chunk, double* ws) {
  const int64_t c0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  const int64_t chunk = blockIdx.y;
  if (c0 >= cols) return;
  const int64_t r0 = chunk * rows_per_chunk;
  const int64_t r1 = r0 + rows_per_chunk < rows ? r0 + rows_per_chunk : rows;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const unsigned short* xs = reinterpret_cast<const unsigned short*>(x);
  const bool full = c0 + 8 <= cols;
  for (int64_t r = r0; r < r1; ++r) {
    const unsigned short* p = xs + r * ldx + c0;
    if (full) {
      u4v w = *reinterpret_cast<const u4v*>(p);
      float f[8];
      decode2<DT>(w.x, f[0], f[1]);
      decode2<DT>(w.y, f[2], f[3]);
      decode2<DT>(w.z, f[4], f[5]);
      decode2<DT>(w.w, f[6], f[7]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double d = (double)f[i];
        acc[i] = __builtin_fma(d, d, acc[i]);  // d*d is exact in float64
      }
    } else {
      for (int i = 0; i < 8 && c0 + i < cols; ++i) {
        const double d = (double)load1<DT>(x, r * ldx + c0 + i);
        acc[i] = __builtin_fma(d, d, acc[i]);
      }
    }
  }
  for (int i = 0; i < 8 && c0 + i < cols; ++i) ws[chunk * cols + c0 + i] = acc[i];
}

__global__ __launch_bounds__(256) void k_colsumsq_final(double* ws, int64_t cols, int chunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  double s = 0.0;
  for (int i = 0; i < chunks; ++i) s += ws[(int64_t)i * cols + c];
  ws[(int64_t)chunks * cols + c] = s;
}

constexpr int ROUTE_BLOCKS = 512;

template <int DT>
__device__ __forceinline__ double ld_d(const void* p, int64_t i) {
  return (double)load1<DT>(p, i);
}

// Partial sums per block (grid-stride over elements): ws[2b] = sum|y-x|, ws[2b+1] = sum|x|.
template <int DT>
__global__ __launch_bounds__(256) void k_route_partial(const void* __restrict__ x, const void* __restrict__ y,
                                                       int64_t n, double* ws) {
  __shared__ double s_d[4], s_x[4];
  double sd = 0.0, sx = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const double xv = ld_d<DT>(x, i);
    const double yv = ld_d<DT>(y, i);
    sd += fabs(yv - xv);  // exact: both are 16-bit floats widened to float64
    sx += fabs(xv);
  }
  sd = wave_sum_d(sd);
  sx = wave_sum_d(sx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_d[wave] = sd;
    s_x[wave] = sx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, b = 0.0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      a += s_d[w];
      b += s_x[w];
    }
    ws[2 * blockIdx.x] = a;
    ws[2 * blockIdx.x + 1] = b;
  }
}

__global__ void k_route_final(const double* ws, int blocks, double threshold, int hi, int lo, double* gamma,
                              int32_t* bits) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double a = 0.0, b = 0.0;
  for (int i = 0; i < blocks; ++i) {
    a += ws[2 * i];
    b += ws[2 * i + 1];
  }
  const double g = b > 0.0 ? a / b : __builtin_inf();
  if (gamma) *gamma = g;
  *bits = g > threshold ? hi : lo;
}

}  // namespace vqk

namespace vq_internal {

using namespace vqk;

int detect_row_chunks(int64_t rows) { return rows < DET_MAX_CHUNKS ? (int)rows : DET_MAX_CHUNKS; }

hipError_t launch_colsumsq(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, double* ws,
                           hipStream_t st) {
  const int chunks = detect_row_chunks(rows);
  const int64_t rpc = (rows + chunks - 1) / chunks;
  const int64_t threads = (cols + 7) / 8;
  dim3 grid((unsigned)((threads + 255) / 256), (unsigned)chunks);
  if (dt == DT_F16)
    hipLaunchKernelGGL(k_colsumsq_partial<DT_F16>, grid, dim3(256), 0, st, x, rows, cols, ldx, rpc, ws);
  else
    hipLaunchKernelGGL(k_colsumsq_partial<DT_BF16>, grid, dim3(256), 0, st, x, rows, cols, ldx, rpc, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_colsumsq_final, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, st, ws, cols, chunks);
  return hipGetLastError();
}

int route_blocks() { return ROUTE_BLOCKS; }

hipError_t launch_route(const void* x, const void* y, int dt, int64_t n, double threshold, int hi, int lo,
                        double* ws, double* gamma, int32_t* bits, hipStream_t st) {
  int64_t want = (n + 2047) / 2048;
  const int blocks = (int)(want < ROUTE_BLOCKS ? (want < 1 ? 1 : want) : ROUTE_BLOCKS);
  switch (dt) {
    case DT_F16: hipLaunchKernelGGL(k_route_partial<DT_F16>, dim3(blocks), dim3(256), 0, st, x, y, n, ws); break;
    case DT_BF16: hipLaunchKernelGGL(k_route_partial<DT_BF16>, dim3(blocks), dim3(256), 0, st, x, y, n, ws); break;
    default: hipLaunchKernelGGL(k_route_partial<DT_F32>, dim3(blocks), dim3(256), 0, st, x, y, n, ws); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_route_final, dim3(1), dim3(64), 0, st, ws, blocks, threshold, hi, lo, gamma, bits);
  return hipGetLastError();
}

}  // namespace vq_internal
