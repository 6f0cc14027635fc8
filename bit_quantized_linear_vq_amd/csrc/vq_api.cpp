// C ABI of the quantized linear layer: argument validation, launch selection and
// error mapping.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/vq.h"
#include "vq_internal.h"

namespace {

thread_local int g_last_hip = 0;

vq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return VQ_OK;
  g_last_hip = (int)e;
  return VQ_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(vq_dtype dt) { return dt == VQ_F32 ? 4 : 2; }

bool is_16bit(vq_dtype dt) { return dt == VQ_F16 || dt == VQ_BF16; }

bool valid_dt(vq_dtype dt) { return dt == VQ_F16 || dt == VQ_BF16 || dt == VQ_F32; }

int64_t part_len(int32_t n_out) { return n_out > 0 ? ((int64_t)n_out + VQ_K_ALIGN - 1) / VQ_K_ALIGN * VQ_K_ALIGN : 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;
// The GEMM kernels count 256 x 256 tiles (and split items, at most twice as many) in
// 32-bit integers.
bool too_many_tiles(int64_t m, int64_t n) { return ((m + 255) / 256) * ((n + 255) / 256) > ((int64_t)1 << 28); }

// Shared checks of the row-quantization entry points.
vq_status check_rows(const void* x, vq_dtype dt, int64_t rows, int64_t k, int64_t ldx, const int32_t* idx,
                     int32_t n_out, int had_block, const void* codes, const float* scales) {
  if (!x || !codes || !scales) return VQ_ERR_INVALID_ARG;
  if (!is_16bit(dt)) return VQ_ERR_INVALID_ARG;
  if (rows < 1 || k < 1 || rows >= kMaxDim || k >= kMaxDim || ldx < k) return VQ_ERR_INVALID_ARG;
  if (n_out < 0 || (n_out > 0 && !idx)) return VQ_ERR_INVALID_ARG;
  if (had_block != 0 && had_block != VQ_HAD_BLOCK) return VQ_ERR_UNSUPPORTED;
  if (k % VQ_K_ALIGN) return VQ_ERR_SHAPE;
  if (had_block && k % VQ_HAD_BLOCK) return VQ_ERR_SHAPE;
  if (had_block && n_out > 0) return VQ_ERR_UNSUPPORTED;
  if (n_out > VQ_MAX_OUTLIERS || n_out >= k) return VQ_ERR_UNSUPPORTED;
  if (k > vq_internal::row_quant_max_k()) return VQ_ERR_UNSUPPORTED;
  if (!aligned16(x) || ldx % 8 || !aligned16(codes)) return VQ_ERR_SHAPE;
  return VQ_OK;
}

}  // namespace

extern "C" {

int64_t vq_outlier_part_len(int32_t n_out) { return part_len(n_out); }

int64_t vq_packed_k(int64_t k, int32_t n_out) { return k + part_len(n_out); }

namespace {
// A weight format: the width (4 or 8) with or without VQ_W_KBLOCK.
bool wfmt_ok(int wfmt) {
  const int bits = wfmt & ~VQ_W_KBLOCK;
  return bits == 4 || bits == 8;
}
int64_t weight_row_bytes(int64_t kp, int wfmt) { return (wfmt & ~VQ_W_KBLOCK) == 8 ? kp : kp / 2; }
}  // namespace

int64_t vq_weight_bytes(int64_t n, int64_t kp, int wfmt) {
  if (n < 1 || kp < 1 || n >= kMaxDim || kp >= kMaxDim || kp % VQ_K_ALIGN || !wfmt_ok(wfmt)) return 0;
  const int64_t rb = weight_row_bytes(kp, wfmt);
  return (wfmt & VQ_W_KBLOCK) ? (rb + 63) / 64 * 64 * n : rb * n;
}

const char* vq_status_string(vq_status s) {
  switch (s) {
    case VQ_OK: return "ok";
    case VQ_ERR_INVALID_ARG: return "invalid argument";
    case VQ_ERR_SHAPE: return "shape, stride or alignment not allowed by the layout";
    case VQ_ERR_UNSUPPORTED: return "unsupported combination";
    case VQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int vq_last_hip_error(void) { return g_last_hip; }

const char* vq_version(void) { return "vq 0.1 gfx950"; }

// ------------------------------------------------------------------ detection

int64_t vq_detect_workspace_elems(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1) return 0;
  return ((int64_t)vq_internal::detect_row_chunks(rows) + 1) * cols +
         (vq_internal::detect_result_bytes(cols) + 7) / 8;
}

vq_status vq_detect_outliers(const void* x, vq_dtype dt, int64_t rows, int64_t cols, int64_t ldx, double tau,
                             double alpha, double kfac, double* ws_dev, double* norms_host, uint8_t* mask_host,
                             int32_t* idx_host, int32_t* n_out, int32_t* n_out_dev, hipStream_t stream) {
  if (!x || !ws_dev || !mask_host || !idx_host || !n_out) return VQ_ERR_INVALID_ARG;
  if (!is_16bit(dt)) return VQ_ERR_INVALID_ARG;
  if (rows < 1 || cols < 1 || ldx < cols || rows >= kMaxDim || cols >= kMaxDim) return VQ_ERR_INVALID_ARG;
  if (!std::isfinite(tau) || !std::isfinite(alpha) || !std::isfinite(kfac)) return VQ_ERR_INVALID_ARG;
  if (!aligned16(x) || ldx % 8) return VQ_ERR_SHAPE;

  // Every step runs on the device; the host only receives the results, because the
  // outlier count fixes the packed layout that the caller allocates next.
  hipError_t e = vq_internal::launch_colsumsq(x, (int)dt, rows, cols, ldx, ws_dev, stream);
  if (e != hipSuccess) return hip_status(e);
  const int chunks = vq_internal::detect_row_chunks(rows);
  e = vq_internal::launch_detect_flags(ws_dev, cols, chunks, tau, alpha, kfac, stream);
  if (e != hipSuccess) return hip_status(e);
  const uint8_t* res = reinterpret_cast<const uint8_t*>(ws_dev + (int64_t)(chunks + 1) * cols);
  if (n_out_dev) {
    e = hipMemcpyAsync(n_out_dev, res + 8 * cols + 16, sizeof(int32_t), hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  std::vector<uint8_t> h((size_t)vq_internal::detect_result_bytes(cols));
  e = hipMemcpyAsync(h.data(), res, h.size(), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e);
  if (norms_host) std::memcpy(norms_host, h.data(), sizeof(double) * (size_t)cols);
  std::memcpy(n_out, h.data() + 8 * cols + 16, sizeof(int32_t));
  std::memcpy(idx_host, h.data() + 8 * cols + 32, sizeof(int32_t) * (size_t)cols);
  std::memcpy(mask_host, h.data() + 12 * cols + 32, (size_t)cols);
  return VQ_OK;
}

// ------------------------------------------------------------------ weights

vq_status vq_pack_weights(const void* w, vq_dtype dt, int64_t n, int64_t k, int64_t ldw, int bits,
                          const int32_t* idx_dev, int32_t n_out, int had_block, void* codes, float* scales,
                          hipStream_t stream) {
  vq_status s = check_rows(w, dt, n, k, ldw, idx_dev, n_out, had_block, codes, scales);
  if (s != VQ_OK) return s;
  if (!wfmt_ok(bits)) return VQ_ERR_UNSUPPORTED;
  const bool kblock = (bits & VQ_W_KBLOCK) != 0;
  bits &= ~VQ_W_KBLOCK;
  vq_internal::RowQuantParams p{};
  p.x = w;
  p.dtype = (int)dt;
  p.ldx = ldw;
  p.rows = n;
  p.k = k;
  p.kp = k + part_len(n_out);
  p.bits = bits;
  p.idx = idx_dev;
  p.n_out = n_out;
  p.p1 = (int)part_len(n_out);
  p.scale_mul = had_block ? 1.0f / (float)had_block : 1.0f;
  p.codes = codes;
  p.scales = scales;
  p.mode = 0;
  p.had = had_block != 0;
  p.out4 = bits == 4;
  p.kblock = kblock;
  return hip_status(vq_internal::launch_row_quant(p, stream));
}

// ------------------------------------------------------------------ activations

vq_status vq_quant_act(const void* x, vq_dtype dt, int64_t m, int64_t k, int64_t ldx, int bits,
                       const int32_t* bits_dev, vq_gran gran, int had_block, const int32_t* idx_dev, int32_t n_out,
                       const float* static_scale_dev, int8_t* codes, float* scales, hipStream_t stream) {
  vq_status s = check_rows(x, dt, m, k, ldx, idx_dev, n_out, had_block, codes, scales);
  if (s != VQ_OK) return s;
  if (bits != 4 && bits != 6 && bits != 8) return VQ_ERR_UNSUPPORTED;
  if (gran != VQ_PER_TENSOR && gran != VQ_PER_TOKEN && gran != VQ_PER_TENSOR_STATIC) return VQ_ERR_INVALID_ARG;
  if (gran == VQ_PER_TENSOR_STATIC && !static_scale_dev) return VQ_ERR_INVALID_ARG;

  const int parts = n_out > 0 ? 2 : 1;
  vq_internal::RowQuantParams p{};
  p.x = x;
  p.dtype = (int)dt;
  p.ldx = ldx;
  p.rows = m;
  p.k = k;
  p.kp = k + part_len(n_out);
  p.bits = bits;
  p.bits_dev = bits_dev;
  p.idx = idx_dev;
  p.n_out = n_out;
  p.p1 = (int)part_len(n_out);
  p.scale_mul = 1.0f;
  p.codes = codes;
  p.scales = scales;
  p.had = had_block != 0;
  p.out4 = false;

  hipError_t e = hipSuccess;
  if (gran == VQ_PER_TOKEN) {
    p.mode = 0;
    return hip_status(vq_internal::launch_row_quant(p, stream));
  }
  if (gran == VQ_PER_TENSOR) {
    if (parts == 1 && !had_block && m * k <= vq_internal::tensor_small_max_elems())
      return hip_status(vq_internal::launch_tensor_small(x, (int)dt, ldx, m, k, bits, bits_dev, codes, scales,
                                                         stream));
    e = vq_internal::launch_fill_u32(reinterpret_cast<unsigned*>(scales), parts, 0u, stream);
    if (e != hipSuccess) return hip_status(e);
    if (parts == 1 && !had_block && m * (k / 8) <= vq_internal::tensor_absmax_max_pieces()) {
      e = vq_internal::launch_tensor_absmax(x, (int)dt, ldx, m, k, reinterpret_cast<unsigned*>(scales), stream);
    } else {
      vq_internal::RowQuantParams q = p;
      q.maxonly = true;
      e = vq_internal::launch_row_quant(q, stream);
    }
    if (e != hipSuccess) return hip_status(e);
    p.mode = 1;
    p.gsrc = scales;
    e = vq_internal::launch_row_quant(p, stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(vq_internal::launch_tensor_finalize(scales, parts, bits, bits_dev, stream));
  }
  p.mode = 2;
  p.gsrc = static_scale_dev;
  return hip_status(vq_internal::launch_row_quant(p, stream));
}

// ------------------------------------------------------------------ Hadamard

vq_status vq_hadamard_block(const void* x, vq_dtype in_dt, int64_t ldx, void* y, vq_dtype out_dt, int64_t ldy,
                            int64_t rows, int64_t cols, int block, int normalize, hipStream_t stream) {
  if (!x || !y) return VQ_ERR_INVALID_ARG;
  if (!valid_dt(in_dt) || !valid_dt(out_dt)) return VQ_ERR_INVALID_ARG;
  if (rows < 1 || cols < 1 || ldx < cols || ldy < cols || rows >= kMaxDim || cols >= kMaxDim)
    return VQ_ERR_INVALID_ARG;
  if (normalize != 0 && normalize != 1) return VQ_ERR_INVALID_ARG;
  if (block != VQ_HAD_BLOCK) return VQ_ERR_UNSUPPORTED;
  if (cols % VQ_HAD_BLOCK) return VQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y) || (ldx * elem_size(in_dt)) % 16 || (ldy * elem_size(out_dt)) % 16)
    return VQ_ERR_SHAPE;
  if (x == y) return VQ_ERR_INVALID_ARG;
  return hip_status(vq_internal::launch_hadamard(x, (int)in_dt, ldx, y, (int)out_dt, ldy, rows, cols, normalize,
                                                 stream));
}

// ------------------------------------------------------------------ GEMM

int64_t vq_qgemm_workspace_bytes(int64_t m, int64_t n, int64_t k0) {
  if (m < 1 || n < 1 || k0 < 1 || m >= kMaxDim || n >= kMaxDim || k0 >= kMaxDim || too_many_tiles(m, n)) return 0;
  return vq_internal::qgemm_workspace_bytes(m, n, k0);
}

namespace {
vq_status check_gemm(const int8_t* a, const float* sa, int sa_per_token, const void* b, int b_bits, const float* sb,
                     int64_t m, int64_t n, int64_t kp, int64_t k0, void* y, vq_dtype out_dt, int64_t ldy) {
  if (!a || !sa || !b || !sb || !y) return VQ_ERR_INVALID_ARG;
  if (!valid_dt(out_dt)) return VQ_ERR_INVALID_ARG;
  if (sa_per_token != 0 && sa_per_token != 1) return VQ_ERR_INVALID_ARG;
  if (m < 1 || n < 1 || kp < 1 || k0 < 1 || ldy < n || m >= kMaxDim || n >= kMaxDim || kp >= kMaxDim)
    return VQ_ERR_INVALID_ARG;
  if (!wfmt_ok(b_bits)) return VQ_ERR_UNSUPPORTED;
  if (too_many_tiles(m, n)) return VQ_ERR_UNSUPPORTED;
  if (kp % VQ_K_ALIGN || k0 % VQ_K_ALIGN || k0 > kp || kp - k0 > VQ_MAX_OUTLIERS) return VQ_ERR_SHAPE;
  // The int32 accumulators must hold any sum of the longer partition (partition 0): 127
  // per activation code times 127 per int8 weight code, or 112 = 16 * 7 per 4-bit weight
  // code, which enters the MFMA as 16 times its value.
  if ((double)k0 * 127.0 * ((b_bits & ~VQ_W_KBLOCK) == 8 ? 127.0 : 112.0) >= 2147483648.0) return VQ_ERR_SHAPE;
  if (!aligned16(a) || !aligned16(b)) return VQ_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(y) % (uintptr_t)elem_size(out_dt)) return VQ_ERR_SHAPE;
  return VQ_OK;
}

vq_internal::GemmParams gemm_params(const int8_t* a, const float* sa, int sa_per_token, const void* b, int b_bits,
                                    const float* sb, int64_t m, int64_t n, int64_t kp, int64_t k0, void* y,
                                    vq_dtype out_dt, int64_t ldy) {
  vq_internal::GemmParams p{};
  p.a = a;
  p.sa = sa;
  p.sa_per_token = sa_per_token;
  p.b = b;
  p.b_bits = b_bits & ~VQ_W_KBLOCK;
  p.b_kblock = (b_bits & VQ_W_KBLOCK) != 0;
  p.sb = sb;
  p.m = m;
  p.n = n;
  p.kp = kp;
  p.k0 = k0;
  p.y = y;
  p.out_dt = (int)out_dt;
  p.ldy = ldy;
  return p;
}
}  // namespace

vq_status vq_qgemm_dequant(const int8_t* a, const float* sa, int sa_per_token, const void* b, int b_bits,
                           const float* sb, int64_t m, int64_t n, int64_t kp, int64_t k0, void* y, vq_dtype out_dt,
                           int64_t ldy, int32_t* acc_debug, void* ws, hipStream_t stream) {
  vq_status s = check_gemm(a, sa, sa_per_token, b, b_bits, sb, m, n, kp, k0, y, out_dt, ldy);
  if (s != VQ_OK) return s;
  if (ws && !aligned16(ws)) return VQ_ERR_SHAPE;
  vq_internal::GemmParams p = gemm_params(a, sa, sa_per_token, b, b_bits, sb, m, n, kp, k0, y, out_dt, ldy);
  p.acc_debug = acc_debug;
  p.ws = ws;
  return hip_status(vq_internal::launch_qgemm(p, stream));
}

int64_t vq_qgemm_scratch_bytes(void) { return vq_internal::qgemm_scratch_bytes(); }

vq_status vq_qgemm_dequant_noalloc(const int8_t* a, const float* sa, int sa_per_token, const void* b, int b_bits,
                                   const float* sb, int64_t m, int64_t n, int64_t kp, int64_t k0, void* y,
                                   vq_dtype out_dt, int64_t ldy, hipStream_t stream) {
  vq_status s = check_gemm(a, sa, sa_per_token, b, b_bits, sb, m, n, kp, k0, y, out_dt, ldy);
  if (s != VQ_OK) return s;
  if (vq_internal::qgemm_workspace_bytes(m, n, k0) > vq_internal::qgemm_scratch_bytes()) return VQ_ERR_SHAPE;
  return hip_status(vq_internal::launch_qgemm_noalloc(
      gemm_params(a, sa, sa_per_token, b, b_bits, sb, m, n, kp, k0, y, out_dt, ldy), stream));
}

// ------------------------------------------------------------------ decomposition

namespace {
bool ok_bits(int b) { return b == 4 || b == 6 || b == 8; }
}  // namespace

int64_t vq_residual_workspace_bytes(int64_t m, int64_t n_rows, int64_t n) {
  if (m < 1 || n_rows < 0 || n < 1 || m >= kMaxDim || n >= kMaxDim || n_rows > m) return 0;
  return 8 * n_rows * n;  // float32 [2 * n_rows x n]: the two terms of every listed row
}

vq_status vq_quant_residual(const void* x, vq_dtype dt, int64_t m, int64_t k, int64_t ldx, int bits1, int bits2,
                            const int32_t* rows_dev, int64_t n_rows, int8_t* codes, float* scales,
                            hipStream_t stream) {
  if (!x) return VQ_ERR_INVALID_ARG;
  if (n_rows > 0 && (!rows_dev || !codes || !scales)) return VQ_ERR_INVALID_ARG;
  if (!is_16bit(dt)) return VQ_ERR_INVALID_ARG;
  if (m < 1 || k < 1 || m >= kMaxDim || k >= kMaxDim || ldx < k || n_rows < 0 || n_rows > m)
    return VQ_ERR_INVALID_ARG;
  if (!ok_bits(bits1) || !ok_bits(bits2)) return VQ_ERR_UNSUPPORTED;
  if (k % VQ_K_ALIGN) return VQ_ERR_SHAPE;
  if (!aligned16(x) || ldx % 8 || (n_rows > 0 && reinterpret_cast<uintptr_t>(codes) % 8)) return VQ_ERR_SHAPE;
  if (n_rows == 0) return VQ_OK;
  return hip_status(vq_internal::launch_residual_quant(x, (int)dt, ldx, m, k, rows_dev, n_rows, bits1, bits2, codes,
                                                       scales, stream));
}

vq_status vq_qgemm_dequant_residual(const int8_t* a, const float* sa, const void* b, int b_bits, const float* sb,
                                    int64_t m, int64_t n, int64_t kp, const int8_t* a2, const float* sa2,
                                    const int32_t* rows_dev, int64_t n_rows, void* y, vq_dtype out_dt, int64_t ldy,
                                    void* ws, hipStream_t stream) {
  if (n_rows < 0 || n_rows > m) return VQ_ERR_INVALID_ARG;
  if (n_rows > 0 && (!a2 || !sa2 || !rows_dev || !ws)) return VQ_ERR_INVALID_ARG;
  if (n_rows > 0 && (2 * n_rows >= kMaxDim || (n >= 1 && n_rows * ((n + 1023) / 1024) >= kMaxDim)))
    return VQ_ERR_UNSUPPORTED;
  if (n_rows > 0 && (!aligned16(a2) || !aligned16(ws))) return VQ_ERR_SHAPE;
  // Every row as without decomposition (this also validates a, sa, b, sb, y and the sizes).
  vq_status st = vq_qgemm_dequant(a, sa, 1, b, b_bits, sb, m, n, kp, kp, y, out_dt, ldy, nullptr, nullptr, stream);
  if (st != VQ_OK || n_rows == 0) return st;
  // Both terms of every listed row in float32: y12 = fl32(acc * fl32(s * sw)) over the
  // stacked operand [q1 rows; q2 rows].
  float* y12 = reinterpret_cast<float*>(ws);
  st = vq_qgemm_dequant(a2, sa2, 1, b, b_bits, sb, 2 * n_rows, n, kp, kp, y12, VQ_F32, n, nullptr, nullptr,
                        stream);
  if (st != VQ_OK) return st;
  return hip_status(vq_internal::launch_residual_merge(y12, n_rows, n, rows_dev, m, y, (int)out_dt, ldy, stream));
}

// ------------------------------------------------------------------ MX formats

namespace {
bool mx_fmt_ok(vq_mx_fmt f) { return f == VQ_MXFP4 || f == VQ_MXFP6 || f == VQ_MXFP4_KBLOCK; }
bool mx_kblock(vq_mx_fmt f) { return f == VQ_MXFP4_KBLOCK; }
int mx_base(vq_mx_fmt f) { return (int)f & ~VQ_W_KBLOCK; }  // the element format (MFMA code)
int mx_bits(vq_mx_fmt f) { return mx_base(f) == VQ_MXFP4 ? 4 : 6; }
}  // namespace

int64_t vq_mx_code_bytes(int64_t rows, int64_t k, vq_mx_fmt fmt) {
  if (rows < 1 || k < 1 || k % VQ_K_ALIGN || !mx_fmt_ok(fmt)) return 0;
  const int64_t row_bytes = k * mx_bits(fmt) / 8;
  return mx_kblock(fmt) ? (row_bytes + 63) / 64 * 64 * rows : rows * row_bytes;
}

int64_t vq_mx_scale_bytes(int64_t rows, int64_t k) {
  if (rows < 1 || k < 1 || k % VQ_K_ALIGN) return 0;
  return (k / 64) * vq_internal::mx_rows8(rows) * 2;
}

vq_status vq_mx_quant(const void* x, vq_dtype dt, int64_t rows, int64_t k, int64_t ldx, vq_mx_fmt fmt, uint8_t* codes,
                      uint8_t* scales, hipStream_t stream) {
  if (!x || !codes || !scales) return VQ_ERR_INVALID_ARG;
  if (!is_16bit(dt)) return VQ_ERR_INVALID_ARG;
  if (rows < 1 || k < 1 || rows >= kMaxDim || k >= kMaxDim || ldx < k) return VQ_ERR_INVALID_ARG;
  if (!mx_fmt_ok(fmt)) return VQ_ERR_UNSUPPORTED;
  if (k % VQ_K_ALIGN) return VQ_ERR_SHAPE;
  if (!aligned16(x) || ldx % 8 || reinterpret_cast<uintptr_t>(codes) % 8) return VQ_ERR_SHAPE;
  return hip_status(vq_internal::launch_mx_quant(x, (int)dt, ldx, rows, k, mx_base(fmt), codes, scales, stream, false,
                                                 0, mx_kblock(fmt)));
}

vq_status vq_mx_quant_rotated(const void* x, vq_dtype dt, int64_t rows, int64_t k, int64_t ldx, vq_mx_fmt fmt,
                              int exp_offset, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (!x || !codes || !scales) return VQ_ERR_INVALID_ARG;
  if (!is_16bit(dt)) return VQ_ERR_INVALID_ARG;
  if (rows < 1 || k < 1 || rows >= kMaxDim || k >= kMaxDim || ldx < k) return VQ_ERR_INVALID_ARG;
  if (exp_offset < -64 || exp_offset > 64) return VQ_ERR_INVALID_ARG;
  if (!mx_fmt_ok(fmt)) return VQ_ERR_UNSUPPORTED;
  if (k % VQ_HAD_BLOCK) return VQ_ERR_SHAPE;
  if (!aligned16(x) || ldx % 8 || reinterpret_cast<uintptr_t>(codes) % 8) return VQ_ERR_SHAPE;
  return hip_status(
      vq_internal::launch_mx_quant(x, (int)dt, ldx, rows, k, mx_base(fmt), codes, scales, stream, true, exp_offset,
                                   mx_kblock(fmt)));
}

int64_t vq_mx_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 1 || n < 1 || k < 1 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim || k % VQ_K_ALIGN ||
      too_many_tiles(m, n))
    return 0;
  return vq_internal::mx_gemm_workspace_bytes(m, n, k);
}

vq_status vq_mx_gemm(const uint8_t* a, const uint8_t* sa, vq_mx_fmt fa, const uint8_t* b, const uint8_t* sb,
                     vq_mx_fmt fb, int64_t m, int64_t n, int64_t k, void* y, vq_dtype out_dt, int64_t ldy,
                     void* ws, hipStream_t stream) {
  if (!a || !sa || !b || !sb || !y) return VQ_ERR_INVALID_ARG;
  if (!valid_dt(out_dt)) return VQ_ERR_INVALID_ARG;
  if (m < 1 || n < 1 || k < 1 || ldy < n || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim) return VQ_ERR_INVALID_ARG;
  if ((fa != VQ_MXFP4 && fa != VQ_MXFP6) || (fb != VQ_MXFP4 && fb != VQ_MXFP4_KBLOCK)) return VQ_ERR_UNSUPPORTED;
  if (too_many_tiles(m, n)) return VQ_ERR_UNSUPPORTED;
  if (k % VQ_K_ALIGN) return VQ_ERR_SHAPE;
  if (!aligned16(a) || !aligned16(b) || !aligned16(sa) || !aligned16(sb)) return VQ_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(y) % (uintptr_t)elem_size(out_dt)) return VQ_ERR_SHAPE;
  if (ws && !aligned16(ws)) return VQ_ERR_SHAPE;
  return hip_status(
      vq_internal::launch_mx_gemm(a, sa, (int)fa, b, sb, m, n, k, y, (int)out_dt, ldy, ws, stream, mx_kblock(fb)));
}

// ------------------------------------------------------------------ unquantized layer

vq_status vq_gemm_dense(const void* x, const void* w, vq_dtype dt, int64_t m, int64_t n, int64_t k,
                        int64_t ldx, int64_t ldw, void* y, vq_dtype out_dt, int64_t ldy, hipStream_t stream) {
  if (!x || !w || !y) return VQ_ERR_INVALID_ARG;
  if (!is_16bit(dt) || !valid_dt(out_dt)) return VQ_ERR_INVALID_ARG;
  if (m < 1 || n < 1 || k < 1 || m >= kMaxDim || n >= kMaxDim || k >= kMaxDim) return VQ_ERR_INVALID_ARG;
  if (ldx < k || ldw < k || ldy < n) return VQ_ERR_INVALID_ARG;
  if (too_many_tiles(m, n)) return VQ_ERR_UNSUPPORTED;
  if (k % VQ_K_ALIGN) return VQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || ldx % 8 || ldw % 8) return VQ_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(y) % (uintptr_t)elem_size(out_dt)) return VQ_ERR_SHAPE;
  vq_internal::DenseParams p{x, w, dt == VQ_BF16 ? 1 : 0, m, n, k, ldx, ldw, y, (int)out_dt, ldy};
  return hip_status(vq_internal::launch_gemm_dense(p, stream));
}

// ------------------------------------------------------------------ calibration

int64_t vq_calib_hist_bins(void) { return vq_internal::calib_hist_bins(); }

vq_status vq_calib_static_scale(const void* x, vq_dtype dt, int64_t rows, int64_t cols, int64_t ldx, int bits,
                                const double* percentiles_host, int32_t n_cand, uint32_t* hist_dev,
                                float* clips_dev, float* scales_dev, double* mse_dev, int32_t* best_dev,
                                float* scale_dev, hipStream_t stream) {
  if (!x || !percentiles_host || !hist_dev || !clips_dev || !scales_dev || !mse_dev || !best_dev)
    return VQ_ERR_INVALID_ARG;
  if (!is_16bit(dt)) return VQ_ERR_INVALID_ARG;
  if (rows < 1 || cols < 1 || ldx < cols || rows >= kMaxDim || cols >= kMaxDim) return VQ_ERR_INVALID_ARG;
  if (n_cand < 1 || n_cand > vq_internal::CALIB_MAX_CAND) return VQ_ERR_INVALID_ARG;
  if ((double)rows * (double)cols >= 4294967296.0) return VQ_ERR_UNSUPPORTED;  // 32-bit bin counts
  if (!ok_bits(bits)) return VQ_ERR_UNSUPPORTED;
  for (int i = 0; i < n_cand; ++i)
    if (!(percentiles_host[i] > 0.0 && percentiles_host[i] <= 100.0)) return VQ_ERR_INVALID_ARG;
  if (cols % 8 || ldx % 8 || !aligned16(x)) return VQ_ERR_SHAPE;
  return hip_status(vq_internal::launch_calib(x, dt == VQ_BF16 ? 1 : 0, rows, cols, ldx, bits, percentiles_host,
                                              n_cand, hist_dev, clips_dev, scales_dev, mse_dev, best_dev,
                                              scale_dev, stream));
}

// ------------------------------------------------------------------ routing

int64_t vq_route_workspace_elems(int64_t n) { return n < 1 ? 0 : 2 * (int64_t)vq_internal::route_blocks(); }

vq_status vq_route_rel_l1(const void* x, const void* y, vq_dtype dt, int64_t n, double threshold, int bits_hi,
                          int bits_lo, double* ws_dev, double* gamma_dev, int32_t* bits_dev, hipStream_t stream) {
  if (!x || !y || !ws_dev || !bits_dev) return VQ_ERR_INVALID_ARG;
  if (!valid_dt(dt) || n < 1) return VQ_ERR_INVALID_ARG;
  auto ok_bits = [](int b) { return b == 4 || b == 6 || b == 8; };
  if (!ok_bits(bits_hi) || !ok_bits(bits_lo) || !std::isfinite(threshold)) return VQ_ERR_INVALID_ARG;
  return hip_status(vq_internal::launch_route(x, y, (int)dt, n, threshold, bits_hi, bits_lo, ws_dev, gamma_dev,
                                              bits_dev, stream));
}

static_assert(sizeof(vq_control_params) == 48 && offsetof(vq_control_params, max_skips) == 16 &&
                  offsetof(vq_control_params, route_threshold) == 32,
              "vq_control_params layout is part of the ABI");

int64_t vq_control_workspace_elems(void) { return 4 * (int64_t)vq_internal::route_blocks(); }

vq_status vq_step_control(const void* delta_new, const void* delta_old, vq_dtype delta_dt, int64_t n_delta,
                          const void* x_prev, const void* y_prev, vq_dtype xy_dt, int64_t n_xy,
                          const int32_t* n_out_dev, int64_t channels, const vq_control_params* params,
                          void* state_dev, double* ws_dev, int32_t* skip_dev, int32_t* bits_dev, double* e_dev,
                          double* gamma_dev, hipStream_t stream) {
  if (!params || !state_dev || !ws_dev || !skip_dev || !bits_dev) return VQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(state_dev) % 8) return VQ_ERR_INVALID_ARG;
  if (!delta_new != !delta_old || !x_prev != !y_prev) return VQ_ERR_INVALID_ARG;
  if (delta_new && (!valid_dt(delta_dt) || n_delta < 1)) return VQ_ERR_INVALID_ARG;
  if (x_prev && (!valid_dt(xy_dt) || n_xy < 1)) return VQ_ERR_INVALID_ARG;
  if (n_out_dev && channels < 1) return VQ_ERR_INVALID_ARG;
  const vq_control_params& p = *params;
  if (std::isnan(p.skip_threshold) || std::isnan(p.drift_threshold) || std::isnan(p.route_threshold) ||
      std::isnan(p.outlier_ratio_max) || p.max_skips < 0 || !ok_bits(p.bits_hi) || !ok_bits(p.bits_lo))
    return VQ_ERR_INVALID_ARG;
  return hip_status(vq_internal::launch_control(
      delta_new, delta_old, (int)delta_dt, n_delta, x_prev, y_prev, (int)xy_dt, n_xy, n_out_dev, channels,
      p.skip_threshold, p.drift_threshold, p.max_skips, p.route_threshold, p.bits_hi, p.bits_lo,
      p.outlier_ratio_max, static_cast<uint8_t*>(state_dev), ws_dev, skip_dev, bits_dev, e_dev, gamma_dev, stream));
}

}  // extern "C"
