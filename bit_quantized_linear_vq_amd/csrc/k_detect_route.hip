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
constexpr int COLSUM_BATCH = 16;  // rows loaded together per thread in the column sums
constexpr int COLFIN_BATCH = 32;  // chunk partials loaded together per thread in the final sums

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
  auto add_row = [&](const u4v& w) {
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
  };
  int64_t r = r0;
  if (full) {
    // Rows in groups of COLSUM_BATCH: all loads of a group are issued before the first
    // addition, which still runs in ascending row order.
    for (; r + COLSUM_BATCH <= r1; r += COLSUM_BATCH) {
      u4v w[COLSUM_BATCH];
#pragma unroll
      for (int j = 0; j < COLSUM_BATCH; ++j) w[j] = *reinterpret_cast<const u4v*>(xs + (r + j) * ldx + c0);
#pragma unroll
      for (int j = 0; j < COLSUM_BATCH; ++j) add_row(w[j]);
    }
  }
  for (; r < r1; ++r) {
    const unsigned short* p = xs + r * ldx + c0;
    if (full) {
      add_row(*reinterpret_cast<const u4v*>(p));
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
  int i = 0;
  // Loads in groups of COLFIN_BATCH (issued together), added in ascending chunk order.
  for (; i + COLFIN_BATCH <= chunks; i += COLFIN_BATCH) {
    double v[COLFIN_BATCH];
#pragma unroll
    for (int j = 0; j < COLFIN_BATCH; ++j) v[j] = ws[(int64_t)(i + j) * cols + c];
#pragma unroll
    for (int j = 0; j < COLFIN_BATCH; ++j) s += v[j];
  }
  for (; i < chunks; ++i) s += ws[(int64_t)i * cols + c];
  ws[(int64_t)chunks * cols + c] = s;
}

// ---- outlier statistics and flags (one workgroup): norms, median, MAD, the flag rule and
// the outlier-first index list.  The median and MAD are exact order statistics, found by
// radix selection over the float64 bit patterns (non-negative doubles order like their
// bits), so they equal any correct sort of the same norms.
constexpr int SEL_THREADS = 1024;
constexpr int SEL_LDS_VALUES = 16384;  // norms kept in LDS when cols <= this

struct DetectOut {
  double* norms;  // [cols]
  double* stats;  // [2]: median, MAD
  int32_t* n_out; // [1]
  int32_t* idx;   // [cols]
  uint8_t* mask;  // [cols]
};

// The rank0-th and rank1-th smallest (0-based) of val(0..n-1), all non-negative and
// finite, found together: eight passes over 8-bit digits from the top, each building one
// 256-bin histogram per rank of the values that share that rank's prefix so far (the two
// middle ranks of an even count share most of their digits).  hist holds 512 bins,
// s_sel and s_rem two entries.
template <class F>
__device__ void select_ranks(F val, int n, int rank0, int rank1, unsigned* hist, int* s_sel, int* s_rem,
                             double& out0, double& out1) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t prefix[2] = {0ull, 0ull};
  int rem[2] = {rank0, rank1};
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 512; i += SEL_THREADS) hist[i] = 0u;
    __syncthreads();
    const uint64_t hi = shift == 56 ? 0ull : (~0ull << (shift + 8));
    // The leading digits of the norms mostly agree, and one LDS atomic per lane on a single
    // bin serializes the pass: the lanes holding the digit of the wave's first active lane
    // add their count with one atomic, the others (diverse digits) one each.
    for (int base = 0; base < n; base += SEL_THREADS) {
      const int i = base + tid;
      uint64_t b = 0;
      if (i < n) b = (uint64_t)__double_as_longlong(val(i));
      const unsigned dig = (unsigned)(b >> shift) & 255u;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bool act = i < n && (b & hi) == prefix[q];
        const uint64_t am = __ballot(act);
        if (am) {
          const int leader = __ffsll((unsigned long long)am) - 1;
          const unsigned d = __shfl(dig, leader, 64);
          const bool mine = act && dig == d;
          const uint64_t same = __ballot(mine);
          if (lane == leader) atomicAdd(&hist[256 * q + d], (unsigned)__popcll(same));
          if (act && !mine) atomicAdd(&hist[256 * q + dig], 1u);
        }
      }
    }
    __syncthreads();
    if (wave < 2) {  // wave q: the digit whose cumulative count passes rem[q]; lane l holds digits 4l..4l+3
      const int q = wave;
      const int r = rem[q];
      unsigned c[4], own = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[256 * q + 4 * lane + j];
        own += c[j];
      }
      unsigned incl = own;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const unsigned v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      const unsigned excl = incl - own;
      if (excl <= (unsigned)r && (unsigned)r < incl) {
        unsigned cum = excl;
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] > (unsigned)r) {
            s_sel[q] = 4 * lane + j;
            s_rem[q] = r - (int)cum;
            break;
          }
          cum += c[j];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      prefix[q] |= (uint64_t)s_sel[q] << shift;
      rem[q] = s_rem[q];
    }
    __syncthreads();
  }
  out0 = __longlong_as_double((long long)prefix[0]);
  out1 = __longlong_as_double((long long)prefix[1]);
}

// Median: the middle value of an odd count, the mean of the two middle values of an even one.
template <class F>
__device__ double median_of(F val, int n, unsigned* hist, int* s_sel, int* s_rem) {
  double a, b;
  select_ranks(val, n, (n - 1) / 2, n / 2, hist, s_sel, s_rem, a, b);
  return (n & 1) ? b : 0.5 * (a + b);
}

__global__ __launch_bounds__(SEL_THREADS) void k_detect_flags(const double* sums, int cols, double tau, double alpha,
                                                              double kfac, DetectOut o) {
  __shared__ double sv[SEL_LDS_VALUES];
  __shared__ unsigned hist[512];
  __shared__ int s_sel[2], s_rem[2];
  __shared__ int s_wcnt[SEL_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool in_lds = cols <= SEL_LDS_VALUES;
  for (int i = tid; i < cols; i += SEL_THREADS) {
    const double v = sqrt(sums[i]);
    o.norms[i] = v;
    if (in_lds) sv[i] = v;
  }
  __syncthreads();
  const double* vg = o.norms;
  auto V = [&](int i) { return in_lds ? sv[i] : vg[i]; };
  const double med = median_of(V, cols, hist, s_sel, s_rem);
  auto D = [&](int i) { return fabs(V(i) - med); };
  const double mad = median_of(D, cols, hist, s_sel, s_rem);
  const double amin = alpha * med;

  // Outliers in ascending order, then the normal channels in ascending order.
  int base = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int c0 = 0; c0 < cols; c0 += SEL_THREADS) {
      const int i = c0 + tid;
      bool f = false;
      if (i < cols) {
        bool out;
        if (pass == 0) {
          const double v = V(i);
          double z;
          if (mad == 0.0)
            z = v > med ? __builtin_inf() : 0.0;
          else
            z = kfac * (v - med) / mad;
          out = z > tau && v > amin;
          o.mask[i] = out ? 1 : 0;
        } else {
          out = o.mask[i] != 0;  // written by this thread in the first pass
        }
        f = pass == 0 ? out : !out;
      }
      const uint64_t bal = __ballot(f);
      const int pre = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) s_wcnt[wave] = __popcll(bal);
      __syncthreads();
      int off = 0, tot = 0;
      for (int w = 0; w < SEL_THREADS / 64; ++w) {
        if (w < wave) off += s_wcnt[w];
        tot += s_wcnt[w];
      }
      if (f) o.idx[base + off + pre] = i;
      base += tot;
      __syncthreads();
    }
    if (pass == 0 && tid == 0) *o.n_out = base;
  }
  if (tid == 0) {
    o.stats[0] = med;
    o.stats[1] = mad;
  }
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

// Sums of the per-block partial pairs (ws[2i], ws[2i + 1]) by one wave in a fixed order:
// lane l adds the pairs l, l + 64, ... in turn, then a butterfly over the lanes.  Every
// lane returns the totals.
__device__ __forceinline__ void sum_pairs_wave(const double* ws, int blocks, double& a, double& b) {
  const int lane = threadIdx.x & 63;
  a = 0.0;
  b = 0.0;
  for (int i = lane; i < blocks; i += 64) {
    a += ws[2 * i];
    b += ws[2 * i + 1];
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    a += __shfl_xor(a, d, 64);
    b += __shfl_xor(b, d, 64);
  }
}

__global__ void k_route_final(const double* ws, int blocks, double threshold, int hi, int lo, double* gamma,
                              int32_t* bits) {
  if (threadIdx.x >= 64 || blockIdx.x != 0) return;
  double a, b;
  sum_pairs_wave(ws, blocks, a, b);
  if (threadIdx.x != 0) return;
  const double g = b > 0.0 ? a / b : __builtin_inf();
  if (gamma) *gamma = g;
  *bits = g > threshold ? hi : lo;
}

// ---- per-block step control (TDC skip test, PDR overrides, DMPQ route).
struct ControlParams {
  double skip_threshold, drift_threshold, route_threshold, outlier_ratio_max;
  int max_skips, bits_hi, bits_lo;
};

// ws_e / ws_g: partial sums of the two relative-L1 statistics (blocks_e / blocks_g = 0 when
// absent).  state[0] = consecutive skips (int32), state + 8 = accumulated error (double).
__global__ void k_control_final(const double* ws_e, int blocks_e, const double* ws_g, int blocks_g,
                                const int32_t* n_out, int64_t channels, ControlParams p, uint8_t* state,
                                int32_t* skip, int32_t* bits, double* e_out, double* g_out) {
  if (threadIdx.x >= 64 || blockIdx.x != 0) return;
  double e = __builtin_nan(""), g = __builtin_nan("");
  if (blocks_e) {
    double num, den;
    sum_pairs_wave(ws_e, blocks_e, num, den);
    e = num == 0.0 ? 0.0 : (den > 0.0 ? num / den : __builtin_inf());
  }
  if (blocks_g) {
    double num, den;
    sum_pairs_wave(ws_g, blocks_g, num, den);
    g = den > 0.0 ? num / den : __builtin_inf();
  }
  if (threadIdx.x != 0) return;
  int32_t* skips = reinterpret_cast<int32_t*>(state);
  double* drift = reinterpret_cast<double*>(state + 8);
  if (e_out) *e_out = e;
  if (g_out) *g_out = g;
  const int s = *skips;
  const double d = *drift;
  if (blocks_e && s < p.max_skips && e <= p.skip_threshold && d + e <= p.drift_threshold) {
    *skips = s + 1;
    *drift = d + e;
    *skip = 1;
    *bits = 0;
    return;
  }
  int b;
  if (n_out && channels > 0 && (double)*n_out / (double)channels > p.outlier_ratio_max)
    b = 16;
  else if (s > 0)
    b = 8;
  else if (!blocks_g)
    b = p.bits_hi;
  else
    b = g > p.route_threshold ? p.bits_hi : p.bits_lo;
  *skips = 0;
  *drift = 0.0;
  *skip = 0;
  *bits = b;
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

int64_t detect_result_bytes(int64_t cols) { return 13 * cols + 32; }

hipError_t launch_detect_flags(double* ws, int64_t cols, int chunks, double tau, double alpha, double kfac,
                               hipStream_t st) {
  const double* sums = ws + (int64_t)chunks * cols;
  uint8_t* r = reinterpret_cast<uint8_t*>(ws + (int64_t)(chunks + 1) * cols);
  DetectOut o;
  o.norms = reinterpret_cast<double*>(r);
  o.stats = reinterpret_cast<double*>(r + 8 * cols);
  o.n_out = reinterpret_cast<int32_t*>(r + 8 * cols + 16);
  o.idx = reinterpret_cast<int32_t*>(r + 8 * cols + 32);
  o.mask = r + 12 * cols + 32;
  hipLaunchKernelGGL(k_detect_flags, dim3(1), dim3(SEL_THREADS), 0, st, sums, (int)cols, tau, alpha, kfac, o);
  return hipGetLastError();
}

int route_blocks() { return ROUTE_BLOCKS; }

static int route_grid(int64_t n) {
  const int64_t want = (n + 2047) / 2048;
  return (int)(want < ROUTE_BLOCKS ? (want < 1 ? 1 : want) : ROUTE_BLOCKS);
}

static void launch_route_partial(const void* x, const void* y, int dt, int64_t n, int blocks, double* ws,
                                 hipStream_t st) {
  switch (dt) {
    case DT_F16: hipLaunchKernelGGL(k_route_partial<DT_F16>, dim3(blocks), dim3(256), 0, st, x, y, n, ws); break;
    case DT_BF16: hipLaunchKernelGGL(k_route_partial<DT_BF16>, dim3(blocks), dim3(256), 0, st, x, y, n, ws); break;
    default: hipLaunchKernelGGL(k_route_partial<DT_F32>, dim3(blocks), dim3(256), 0, st, x, y, n, ws); break;
  }
}

hipError_t launch_control(const void* d1, const void* d2, int d_dt, int64_t n_d, const void* x, const void* y,
                          int xy_dt, int64_t n_xy, const int32_t* n_out, int64_t channels, double skip_thr,
                          double drift_thr, int max_skips, double route_thr, int hi, int lo, double ratio_max,
                          uint8_t* state, double* ws, int32_t* skip, int32_t* bits, double* e, double* g,
                          hipStream_t st) {
  // E = sum|d1 - d2| / sum|d2| is the relative-L1 form with x = d2 (older), y = d1 (newer).
  const int be = d1 ? route_grid(n_d) : 0;
  const int bg = x ? route_grid(n_xy) : 0;
  double* ws_e = ws;
  double* ws_g = ws + 2 * ROUTE_BLOCKS;
  if (be) launch_route_partial(d2, d1, d_dt, n_d, be, ws_e, st);
  if (bg) launch_route_partial(x, y, xy_dt, n_xy, bg, ws_g, st);
  ControlParams p{skip_thr, drift_thr, route_thr, ratio_max, max_skips, hi, lo};
  hipLaunchKernelGGL(k_control_final, dim3(1), dim3(64), 0, st, ws_e, be, ws_g, bg, n_out, channels, p, state, skip,
                     bits, e, g);
  return hipGetLastError();
}

hipError_t launch_route(const void* x, const void* y, int dt, int64_t n, double threshold, int hi, int lo,
                        double* ws, double* gamma, int32_t* bits, hipStream_t st) {
  const int blocks = route_grid(n);
  launch_route_partial(x, y, dt, n, blocks, ws, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_route_final, dim3(1), dim3(64), 0, st, ws, blocks, threshold, hi, lo, gamma, bits);
  return hipGetLastError();
}

}  // namespace vq_internal
