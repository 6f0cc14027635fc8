// Static-scale calibration by clipping-percentile search, on the device.
//
// Q-ARVD (aitrends.kr), Technical details: activations are quantized per tensor with a
// clipping percentile and a scale learned during reconstruction.  For a 16-bit float
// tensor, |x| is its 15 low bits, and those patterns order like the magnitudes, so a
// histogram of 32768 bins holds every order statistic of |x| exactly, and the
// reconstruction error of any scale is a sum over the bins (x and -x quantize
// symmetrically, so they have the same error).
//
//   k_abs_hist       one pass over x: the histogram (HBM-bound)
//   k_calib_search   one workgroup per candidate: the clip at rank ceil(p/100*N), the
//                    scale s = fl32(clip/Q), r = fl32(1/s), and the float64 error of the
//                    static quantizer summed over the bins in a fixed order
//   k_calib_pick     the candidate of smallest error (the first one on a tie)
#include "dev_common.h"
#include "gemm_common.h"
#include "vq_internal.h"

namespace vqk {

constexpr int HIST_BINS = 32768;
constexpr int HIST_THREADS = 1024;
constexpr int SEARCH_THREADS = 1024;
constexpr int BINS_PER_THREAD = HIST_BINS / SEARCH_THREADS;  // 32 consecutive bins per lane

struct CalibCands {
  double pct[vq_internal::CALIB_MAX_CAND];
};

// One workgroup per CU: a private LDS histogram (128 KB), then one global atomic add per
// non-empty bin.  A lane takes 16-byte chunks (8 elements) and keeps HIST_UNROLL of them
// in flight before its LDS atomics.  The tensor has fewer than 2^32 elements, so chunk
// indices fit in 32 bits; a dense tensor (ldx == cols) is read as one flat array.
constexpr int HIST_UNROLL = 4;

template <bool FLAT>
__global__ __launch_bounds__(HIST_THREADS) void k_abs_hist(const uint16_t* x, unsigned chunks, unsigned cpr,
                                                           int64_t ldx, unsigned* hist) {
  __shared__ unsigned h[HIST_BINS];
  for (int i = threadIdx.x; i < HIST_BINS; i += HIST_THREADS) h[i] = 0u;
  __syncthreads();
  const unsigned stride = gridDim.x * HIST_THREADS;
  for (unsigned base = blockIdx.x * HIST_THREADS + threadIdx.x; base < chunks; base += HIST_UNROLL * stride) {
    u4v w[HIST_UNROLL];
#pragma unroll
    for (int u = 0; u < HIST_UNROLL; ++u) {
      const unsigned c = base + u * stride;
      if (c < chunks) {
        const uint16_t* p;
        if constexpr (FLAT) {
          p = x + (size_t)c * 8;
        } else {
          const unsigned r = c / cpr;
          p = x + (int64_t)r * ldx + (int64_t)(c - r * cpr) * 8;
        }
        w[u] = *reinterpret_cast<const u4v*>(p);
      }
    }
#pragma unroll
    for (int u = 0; u < HIST_UNROLL; ++u) {
      if (base + u * stride < chunks) {
        const unsigned d[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          atomicAdd(&h[d[t] & 0x7FFFu], 1u);
          atomicAdd(&h[(d[t] >> 16) & 0x7FFFu], 1u);
        }
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HIST_BINS; i += HIST_THREADS)
    if (h[i]) atomicAdd(&hist[i], h[i]);
}

// Value of a 15-bit magnitude pattern of a 16-bit float (exact in float32).
template <int DT>
__device__ __forceinline__ float mag_value(unsigned pat) {
  if constexpr (DT == DT_BF16) {
    return __uint_as_float(pat << 16);
  } else {
    const unsigned short u = (unsigned short)pat;
    return (float)__builtin_bit_cast(_Float16, u);
  }
}

template <int DT>
__global__ __launch_bounds__(SEARCH_THREADS) void k_calib_search(const unsigned* hist, CalibCands cand, double n,
                                                                 float qf, float* clips, float* scales,
                                                                 double* mse) {
  __shared__ unsigned wave_tot[SEARCH_THREADS / 64];
  __shared__ double wave_err[SEARCH_THREADS / 64];
  __shared__ int s_bin;
  const int c = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b0 = threadIdx.x * BINS_PER_THREAD;

  unsigned cnt[BINS_PER_THREAD];
  unsigned own = 0;
#pragma unroll
  for (int i = 0; i < BINS_PER_THREAD; ++i) {
    cnt[i] = hist[b0 + i];
    own += cnt[i];
  }
  // Inclusive prefix of the per-lane totals in bin order (N < 2^32, so 32 bits suffice).
  unsigned incl = own;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const unsigned v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wave_tot[wave] = incl;
  if (threadIdx.x == 0) s_bin = HIST_BINS - 1;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wave_tot[w];
  const unsigned excl = incl - own;

  // Rank of the percentile among the N magnitudes, 1-based and clamped to [1, N].
  double rk = ceil(cand.pct[c] / 100.0 * n);
  rk = fmin(fmax(rk, 1.0), n);
  const unsigned rank = (unsigned)rk;
  if (excl < rank && rank <= incl) {  // exactly one lane holds the crossing
    unsigned cum = excl;
    for (int i = 0; i < BINS_PER_THREAD; ++i) {
      cum += cnt[i];
      if (cum >= rank) {
        s_bin = b0 + i;
        break;
      }
    }
  }
  __syncthreads();

  const float clip = mag_value<DT>((unsigned)s_bin);
  const float s = clip / qf;
  float r = 1.0f / s;
  if (!(s != 0.0f) || __builtin_isinf(r)) r = 0.0f;  // a zero scale quantizes everything to 0

  double err = 0.0;
#pragma unroll 4
  for (int i = 0; i < BINS_PER_THREAD; ++i) {
    if (!cnt[i]) continue;
    const float v = mag_value<DT>((unsigned)(b0 + i));
    float t = v * r;
    t = fminf(fmaxf(t, -qf), qf);
    const float q = __builtin_rintf(t);
    const float deq = q * s;
    const double d = (double)v - (double)deq;
    err += (double)cnt[i] * (d * d);
  }
  // Fixed-order reduction: butterfly within each wave, then the waves in order.
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) err += __shfl_xor(err, d, 64);
  if (lane == 0) wave_err[wave] = err;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int w = 0; w < SEARCH_THREADS / 64; ++w) tot += wave_err[w];
    clips[c] = clip;
    scales[c] = s;
    mse[c] = tot / n;
  }
}

__global__ void k_calib_pick(const float* scales, const double* mse, int n_cand, int32_t* best, float* scale_out) {
  if (threadIdx.x != 0) return;
  int b = 0;
  for (int c = 1; c < n_cand; ++c)
    if (mse[c] < mse[b]) b = c;
  *best = b;
  if (scale_out) *scale_out = scales[b];
}

}  // namespace vqk

namespace vq_internal {

using namespace vqk;

int calib_hist_bins() { return HIST_BINS; }

hipError_t launch_calib(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int bits,
                        const double* pct, int n_cand, unsigned* hist, float* clips, float* scales, double* mse,
                        int32_t* best, float* scale_out, hipStream_t st) {
  hipError_t e = launch_fill_u32(hist, HIST_BINS, 0u, st);
  if (e != hipSuccess) return e;
  // rows * cols < 2^32 (checked by the caller), so the 16-byte chunk count fits in 32 bits.
  const unsigned cpr = (unsigned)(cols / 8), chunks = (unsigned)(rows * (cols / 8));
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x);
  if (ldx == cols)
    hipLaunchKernelGGL(k_abs_hist<true>, dim3(persistent_blocks()), dim3(HIST_THREADS), 0, st, xp, chunks, cpr, ldx,
                       hist);
  else
    hipLaunchKernelGGL(k_abs_hist<false>, dim3(persistent_blocks()), dim3(HIST_THREADS), 0, st, xp, chunks, cpr, ldx,
                       hist);
  CalibCands cand{};
  for (int i = 0; i < n_cand; ++i) cand.pct[i] = pct[i];
  const double n = (double)rows * (double)cols;
  const float qf = (float)((1 << (bits - 1)) - 1);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_calib_search<DT_BF16>, dim3(n_cand), dim3(SEARCH_THREADS), 0, st, hist, cand, n, qf, clips,
                       scales, mse);
  else
    hipLaunchKernelGGL(k_calib_search<DT_F16>, dim3(n_cand), dim3(SEARCH_THREADS), 0, st, hist, cand, n, qf, clips,
                       scales, mse);
  hipLaunchKernelGGL(k_calib_pick, dim3(1), dim3(64), 0, st, scales, mse, n_cand, best, scale_out);
  return hipGetLastError();
}

}  // namespace vq_internal
