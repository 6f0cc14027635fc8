// Launch interface between the C-ABI layer (vq_api.cpp) and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vq_internal {

struct RowQuantParams {
  const void* x;
  int dtype;  // 0 f16, 1 bf16
  int64_t ldx;
  int64_t rows;
  int64_t k;
  int64_t kp;
  int bits;
  const int32_t* bits_dev;
  const int32_t* idx;
  int n_out;
  int p1;
  const float* gsrc;
  float scale_mul;
  void* codes;
  float* scales;
  int mode;  // 0 per row dynamic, 1 global dynamic (absmax in gsrc), 2 static (scales in gsrc)
  bool had;
  bool out4;
  bool maxonly;
  bool kblock;  // codes in the 64-byte K-piece layout (weights, MODE_ROW only)
};

int row_quant_max_k();
hipError_t launch_row_quant(const RowQuantParams& p, hipStream_t st);
hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t st);
// Dynamic per-tensor quantization of at most tensor_small_max_elems() elements in one launch
// (no outlier partition, no rotation, int8 code rows of length k).
int64_t tensor_small_max_elems();
// Atomic maximum of |x| over a whole tensor of at most tensor_absmax_max_pieces() 8-element
// pieces into *maxbits (float bit pattern, cleared by the caller).
int64_t tensor_absmax_max_pieces();
hipError_t launch_tensor_absmax(const void* x, int dtype, int64_t ldx, int64_t rows, int64_t k, unsigned* maxbits,
                                hipStream_t st);
hipError_t launch_tensor_small(const void* x, int dtype, int64_t ldx, int64_t rows, int64_t k, int bits,
                               const int32_t* bits_dev, int8_t* codes, float* scales, hipStream_t st);
hipError_t launch_tensor_finalize(float* scales, int parts, int qbits, const int32_t* bits_dev, hipStream_t st);

hipError_t launch_hadamard(const void* x, int in_dt, int64_t ldx, void* y, int out_dt, int64_t ldy,
                           int64_t rows, int64_t cols, int normalize, hipStream_t st);

struct GemmParams {
  const int8_t* a;
  const float* sa;
  int sa_per_token;
  const void* b;
  int b_bits;    // 8 or 4
  int b_kblock;  // b in the 64-byte K-piece layout (VQ_W_KBLOCK)
  const float* sb;
  int64_t m, n, kp, k0;
  void* y;
  int out_dt;
  int64_t ldy;
  int32_t* acc_debug;
  void* ws;  // remainder-split workspace or nullptr
};
int64_t qgemm_workspace_bytes(int64_t m, int64_t n, int64_t k0);
hipError_t launch_qgemm(const GemmParams& g, hipStream_t st);
// Scratch-free launch: the split workspace is the library's static device array.
int64_t qgemm_scratch_bytes();
hipError_t launch_qgemm_noalloc(const GemmParams& g, hipStream_t st);

hipError_t launch_residual_quant(const void* x, int dtype, int64_t ldx, int64_t m, int64_t k, const int32_t* rows,
                                 int64_t n_rows, int bits1, int bits2, int8_t* codes2, float* scales2,
                                 hipStream_t st);
hipError_t launch_residual_merge(const float* y12, int64_t n_rows, int64_t n, const int32_t* rows, int64_t m, void* y,
                                 int out_dt, int64_t ldy, hipStream_t st);

int64_t mx_rows8(int64_t rows);
hipError_t launch_mx_quant(const void* x, int dtype, int64_t ldx, int64_t rows, int64_t k, int fmt, uint8_t* codes,
                           uint8_t* scales, hipStream_t st, bool had = false, int exp_offset = 0,
                           bool kblock = false);
int64_t mx_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* sa, int fa, const uint8_t* b, const uint8_t* sb, int64_t m,
                          int64_t n, int64_t k, void* y, int out_dt, int64_t ldy, void* ws, hipStream_t st,
                          bool b_kblock);

struct DenseParams {
  const void* x;
  const void* w;
  int in_dt;  // 0 f16, 1 bf16
  int64_t m, n, k, ldx, ldw;
  void* y;
  int out_dt;
  int64_t ldy;
};
hipError_t launch_gemm_dense(const DenseParams& p, hipStream_t st);

int calib_hist_bins();
constexpr int CALIB_MAX_CAND = 64;
hipError_t launch_calib(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int bits,
                        const double* pct, int n_cand, unsigned* hist, float* clips, float* scales, double* mse,
                        int32_t* best, float* scale_out, hipStream_t st);

int detect_row_chunks(int64_t rows);
// Result block of the detection, after the (chunks + 1) * cols partial and total sums in
// the workspace: norms f64 [cols], median and MAD f64, n_out i32 (+12 pad), idx i32 [cols],
// mask u8 [cols].
int64_t detect_result_bytes(int64_t cols);
hipError_t launch_detect_flags(double* ws, int64_t cols, int chunks, double tau, double alpha, double kfac,
                               hipStream_t st);
hipError_t launch_colsumsq(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, double* ws,
                           hipStream_t st);

int route_blocks();
hipError_t launch_control(const void* d1, const void* d2, int d_dt, int64_t n_d, const void* x, const void* y,
                          int xy_dt, int64_t n_xy, const int32_t* n_out, int64_t channels, double skip_thr,
                          double drift_thr, int max_skips, double route_thr, int hi, int lo, double ratio_max,
                          uint8_t* state, double* ws, int32_t* skip, int32_t* bits, double* e, double* g,
                          hipStream_t st);
hipError_t launch_route(const void* x, const void* y, int dt, int64_t n, double threshold, int hi, int lo,
                        double* ws, double* gamma, int32_t* bits, hipStream_t st);

}  // namespace vq_internal
