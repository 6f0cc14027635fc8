// Histogram of |x| for the static-scale calibration (clipping-percentile search).
//
// Q-ARVD (aitrends.kr), Technical details: activations are quantized per tensor with a
// clipping percentile and a scale learned during reconstruction.  For a 16-bit float
// tensor, |x| is its 15 low bits, and those patterns order like the magnitudes, so a
// histogram of 32768 bins holds every order statistic of |x| exactly; the percentile
// clips and the reconstruction error of each candidate scale then follow from the bins.
#include "dev_common.h"
#include "gemm_common.h"
#include "vq_internal.h"

namespace vqk {

constexpr int HIST_BINS = 32768;
constexpr int HIST_THREADS = 1024;

// One workgroup per CU: a private LDS histogram (128 KB), then one global atomic add per
// non-empty bin.  Elements are read 8 at a time (16 bytes per lane).
__global__ __launch_bounds__(HIST_THREADS) void k_abs_hist(const uint16_t* x, int64_t rows, int64_t cols,
                                                           int64_t ldx, unsigned* hist) {
  __shared__ unsigned h[HIST_BINS];
  for (int i = threadIdx.x; i < HIST_BINS; i += HIST_THREADS) h[i] = 0u;
  __syncthreads();
  const int64_t cpr = cols / 8;
  const int64_t total = rows * cpr;
  for (int64_t c = (int64_t)blockIdx.x * HIST_THREADS + threadIdx.x; c < total; c += (int64_t)gridDim.x * HIST_THREADS) {
    const int64_t r = c / cpr, j = c - r * cpr;
    const u4v w = *reinterpret_cast<const u4v*>(x + r * ldx + j * 8);
    const unsigned d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      atomicAdd(&h[d[t] & 0x7FFFu], 1u);
      atomicAdd(&h[(d[t] >> 16) & 0x7FFFu], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HIST_BINS; i += HIST_THREADS)
    if (h[i]) atomicAdd(&hist[i], h[i]);
}

}  // namespace vqk

namespace vq_internal {

using namespace vqk;

int calib_hist_bins() { return HIST_BINS; }

hipError_t launch_abs_hist(const void* x, int64_t rows, int64_t cols, int64_t ldx, unsigned* hist, hipStream_t st) {
  hipError_t e = hipMemsetAsync(hist, 0, HIST_BINS * sizeof(unsigned), st);
  if (e != hipSuccess) return e;
  const int grid = persistent_blocks();  // one workgroup per CU
  hipLaunchKernelGGL(k_abs_hist, dim3(grid), dim3(HIST_THREADS), 0, st, reinterpret_cast<const uint16_t*>(x), rows,
                     cols, ldx, hist);
  return hipGetLastError();
}

}  // namespace vq_internal
