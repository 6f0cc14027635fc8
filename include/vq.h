/*
 * vq.h - C ABI of the MI355X (gfx950) quantized linear layer for video diffusion
 * transformers: online activation quantization, block Hadamard rotation, dual-scale
 * outlier channels, packed INT8/INT4 weights, integer MFMA GEMM with a fused
 * dequantization epilogue, and per-layer INT8-vs-4-bit routing.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers marked "device" are device memory owned by the caller; the
 *    library never allocates, frees or keeps them past the call.  Pointers marked
 *    "host" are ordinary host memory owned by the caller.
 *  - Tensors are row-major; K (input channels) is the contiguous dimension.  Strides
 *    (ld*) are in elements and must be at least the row length.
 *  - Every call enqueues its work asynchronously on `stream` (0 = the null stream)
 *    and returns without waiting, except vq_detect_outliers, which waits on `stream`
 *    because its result is host memory.
 *  - Arguments are validated before anything is enqueued; on an error nothing is
 *    enqueued and outputs are untouched.  Faults inside kernels are reported by the
 *    caller's next synchronization, as for any HIP kernel.
 *  - Element types: VQ_F16 = IEEE binary16, VQ_BF16 = bfloat16, VQ_F32 = binary32.
 *  - Quantized codes: Q = 2^(bits-1) - 1 (127, 31, 7); code = clamp(rne(x * r), -Q, Q)
 *    with r = fl32(Q / a) for the group absolute maximum a and scale s = fl32(a / Q);
 *    a group whose maximum is 0 gets s = 0 and zero codes.  Activation codes of every
 *    width are stored one per int8.  4-bit weight codes are packed two per byte, low
 *    nibble = even k.
 *  - Dual-scale layout: with n_out > 0 outlier input channels the K axis of both
 *    operands has two partitions: partition 0 = the K channels in place with the
 *    outlier positions holding code 0, partition 1 = the outlier channels gathered
 *    in ascending channel order, zero-padded to vq_outlier_part_len(n_out).  Codes are
 *    [rows x vq_packed_k(K, n_out)] and every group has two scales (row-major [rows x 2]).
 *
 * Sources: Q-ARVD (aitrends.kr article, "Q-ARVD: quantization of autoregressive video
 * diffusion models"), sections Methodology and Technical details; 6Bit-Diffusion
 * (gist.science summary of arXiv 2603.18742), Key Insights 1 and Methodology B.1 (DMPQ);
 * S2Q-VDiT (gist.science summary of arXiv 2508.04016), the W4A6 setting; SemanticDialect
 * (gist.science summary of arXiv 2603.02883), Methodology 2.2 (activation decomposition);
 * the OCP Microscaling (MX) v1.0 format definition for the MX block formats.
 */
#ifndef VQ_H
#define VQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vq_status {
  VQ_OK = 0,
  VQ_ERR_INVALID_ARG = 1, /* null pointer, unknown enum, non-positive size, bad stride */
  VQ_ERR_SHAPE = 2,       /* sizes that the layout forbids (K not a multiple of 64, ...) */
  VQ_ERR_UNSUPPORTED = 3, /* a valid but unimplemented combination */
  VQ_ERR_HIP = 4          /* a HIP runtime call failed; see vq_last_hip_error() */
} vq_status;

typedef enum vq_dtype { VQ_F16 = 0, VQ_BF16 = 1, VQ_F32 = 2 } vq_dtype;

typedef enum vq_gran {
  VQ_PER_TENSOR = 0,       /* one dynamic scale per partition over the whole tensor */
  VQ_PER_TOKEN = 1,        /* one dynamic scale per row (token) and partition */
  VQ_PER_TENSOR_STATIC = 2 /* caller-given scale per partition: r = fl32(1 / s) */
} vq_gran;

/* MX element formats: the codes of the scaled MFMA's operand formats. */
typedef enum vq_mx_fmt {
  VQ_MXFP6 = 2, /* FP6 E2M3: sign, 2 exponent bits (bias 1), 3 mantissa bits; largest 7.5 */
  VQ_MXFP4 = 4, /* FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; largest 6 */
  /* FP4 codes in 64-byte K pieces (weights): the layout of VQ_W_KBLOCK below, four MX
   * blocks of a row per piece. */
  VQ_MXFP4_KBLOCK = 4 | 0x100
} vq_mx_fmt;

#define VQ_K_ALIGN 64        /* K and each K partition are multiples of this */
#define VQ_HAD_BLOCK 128     /* the only Hadamard block size */
#define VQ_MAX_OUTLIERS 128  /* largest n_out of the dual-scale path */

/* Length of the outlier partition: n_out rounded up to a multiple of 64 (0 for 0). */
int64_t vq_outlier_part_len(int32_t n_out);

/* Total code length of a K-channel operand with n_out outlier channels. */
int64_t vq_packed_k(int64_t k, int32_t n_out);

/*
 * Weight layout flag, OR'ed into the weight width (bits of vq_pack_weights, b_bits of the
 * GEMM entry points; the same value goes to both).  A row of packed weight codes has
 * row_bytes = kp (8-bit weights) or kp / 2 (4-bit).  Without the flag the codes are
 * [n x row_bytes] row-major.  With it they are cut into 64-byte K pieces (64 int8 codes
 * or 128 4-bit codes) and piece j of every row is stored together: byte c of row r is at
 * (c / 64) * n * 64 + r * 64 + c % 64, for ceil(row_bytes / 64) pieces (the last one
 * padded to 64 bytes when row_bytes % 64 == 32; its padding is never read).  A GEMM stage
 * of a 256-row weight tile is then one contiguous block of whole 128-byte lines, where
 * the row-major layout gives it half lines at the row pitch.
 */
#define VQ_W_KBLOCK 0x100

/* Bytes of packed weights [n rows, kp codes] in format wfmt (4 or 8, optionally OR
 * VQ_W_KBLOCK); 0 for invalid arguments. */
int64_t vq_weight_bytes(int64_t n, int64_t kp, int wfmt);

/*
 * Outlier input-channel detection (Q-ARVD, Methodology: outlier-aware adaptive
 * dual-scale quantization).  For each column k of x [rows x cols]:
 *   v_k = sqrt(sum_r x[r,k]^2)                       (float64 accumulation)
 *   M_k = kfac * (v_k - median(v)) / MAD,  MAD = median(|v - median(v)|)
 *   outlier  <=>  M_k > tau  and  v_k > alpha * median(v)     (both strict)
 * An even count's median is the mean of the two middle values; MAD = 0 makes
 * M_k = +inf where v_k > median, else 0.  kfac = 1 is the page's formula (0.6745 the
 * textbook variant); typical tau = 3.5, alpha = 2.
 *   x          device, dt in {F16, BF16}, [rows x cols], stride ldx
 *   ws_dev     device scratch of vq_detect_workspace_elems(rows, cols) doubles
 *   norms_host host [cols] or NULL: receives v
 *   mask_host  host [cols]: 1 for an outlier channel, else 0
 *   idx_host   host [cols]: first *n_out entries = outlier channels, ascending, then
 *              the other channels, ascending
 *   n_out      host: number of outlier channels
 *   n_out_dev  device int32 [1] or NULL: receives the same count (for vq_step_control)
 * The norms, the median and MAD (exact order statistics of the norms) and the flags are
 * computed on the device; the call then copies the results to the host and waits on
 * `stream`, since the count fixes the packed layout the caller allocates next.
 * Errors: INVALID_ARG for null pointers / rows or cols < 1 / ldx < cols / bad dtype.
 */
int64_t vq_detect_workspace_elems(int64_t rows, int64_t cols);
vq_status vq_detect_outliers(const void* x, vq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                             double tau, double alpha, double kfac, double* ws_dev,
                             double* norms_host, uint8_t* mask_host, int32_t* idx_host,
                             int32_t* n_out, int32_t* n_out_dev, hipStream_t stream);

/*
 * Offline per-output-channel weight quantization (Q-ARVD, Methodology and Technical
 * details: per-channel weights, dual scale; 6Bit-Diffusion, Methodology B.1: weights
 * quantized offline to 4 bits and activations rotated by an online block Hadamard).
 *   w          device, dt in {F16, BF16}, [n x k], stride ldw; k % 64 == 0
 *   bits       8 (codes int8 [n x kp]) or 4 (codes uint8 [n x kp/2], two per byte),
 *              optionally OR VQ_W_KBLOCK for the K-piece layout
 *   idx_dev    device int32 [n_out] outlier channels (ascending, < k), or NULL with n_out = 0
 *   had_block  0, or 128: each row is first rotated by the unnormalized 128-point
 *              Sylvester Hadamard butterflies; the scale then carries the exact 1/128
 *              so that products with rotated activations equal the normalized rotation.
 *              Not combined with n_out > 0.
 *   codes      device, vq_weight_bytes(n, kp, bits) bytes, kp = vq_packed_k(k, n_out)
 *   scales     device float [n] (n_out = 0) or [n x 2] (partition 0, partition 1)
 * Errors: INVALID_ARG, SHAPE (k % 64, k % 128 with had_block), UNSUPPORTED (bits other
 * than 4/8 with or without VQ_W_KBLOCK, had_block other than 0/128, had_block with
 * n_out, n_out > VQ_MAX_OUTLIERS or >= k).
 */
vq_status vq_pack_weights(const void* w, vq_dtype dt, int64_t n, int64_t k, int64_t ldw, int bits,
                          const int32_t* idx_dev, int32_t n_out, int had_block, void* codes,
                          float* scales, hipStream_t stream);

/*
 * Online activation quantization (Q-ARVD, Technical details: activation-quantization
 * kernel, per-tensor activations; per-token rows; 6Bit-Diffusion, Methodology B.1:
 * INT8 or 4-bit activations per block, online block Hadamard; S2Q-VDiT: 6-bit).
 *   x          device, dt in {F16, BF16}, [m x k], stride ldx; k % 64 == 0
 *   bits       4, 6 or 8
 *   bits_dev   device int32 or NULL: when given, the kernels read the bit width from it
 *              at run time (4, 6 or 8; any other value acts as 8) -- the DMPQ route
 *              decided on the device by vq_route_rel_l1 without a host round trip
 *   gran       VQ_PER_TOKEN, VQ_PER_TENSOR (dynamic) or VQ_PER_TENSOR_STATIC
 *   had_block  0 or 128 (unnormalized rotation before quantizing; not with n_out > 0)
 *   idx_dev    device int32 [n_out] outlier channels (ascending), or NULL with n_out = 0
 *   static_scale_dev  device float [1 or 2] (static granularity only), else NULL
 *   codes      device int8 [m x kp], row stride kp = vq_packed_k(k, n_out)
 *   scales     device float: per token [m] or [m x 2]; per tensor [1] or [2]
 * Launches: per token, one kernel; dynamic per tensor, one kernel for at most 2^18
 * elements without outlier partition or rotation (every workgroup reduces the whole
 * maximum itself), else a fill kernel that clears the maximum, a maximum pass, the code
 * pass and a one-thread finalize; static per tensor, the code pass alone (it also copies
 * the given scales to scales, which may alias static_scale_dev).  No memset is enqueued, so a call may be captured in a
 * graph.
 * Errors: INVALID_ARG, SHAPE, UNSUPPORTED as for vq_pack_weights.
 */
vq_status vq_quant_act(const void* x, vq_dtype dt, int64_t m, int64_t k, int64_t ldx, int bits,
                       const int32_t* bits_dev, vq_gran gran, int had_block, const int32_t* idx_dev,
                       int32_t n_out, const float* static_scale_dev, int8_t* codes, float* scales,
                       hipStream_t stream);

/*
 * Standalone block Hadamard rotation (6Bit-Diffusion, Methodology B.1: online block
 * Hadamard transform).  Per row and per contiguous 128-element block, z = H x by
 * float32 butterflies with distances h = 1, 2, ..., 64 in that order, each pair
 * (i, i+h) becoming (z_i + z_{i+h}, z_i - z_{i+h}).  normalize = 1 returns
 * fl32(z * fl32(1/sqrt(128))), normalize = 0 returns z; then RNE to out_dt.
 *   x   device, in_dt in {F16, BF16, F32}, [rows x cols], stride ldx
 *   y   device, out_dt in {F16, BF16, F32}, [rows x cols], stride ldy; may not alias x
 * Errors: INVALID_ARG, SHAPE (cols % 128), UNSUPPORTED (block != 128).
 */
vq_status vq_hadamard_block(const void* x, vq_dtype in_dt, int64_t ldx, void* y, vq_dtype out_dt,
                            int64_t ldy, int64_t rows, int64_t cols, int block, int normalize,
                            hipStream_t stream);

/*
 * Integer GEMM with fused dequantization (Q-ARVD, Technical details: GEMM and
 * dequantization kernel; Methodology: Q_dual keeps separate scales for outlier and
 * normal channels).  acc_P[i,j] = sum_{k in P} a[i,k] * b[j,k] exactly in int32 over
 * partition 0 = [0, k0) and, when k0 < kp, partition 1 = [k0, kp).  Then, in float32
 * without fused multiply-add: y_P = fl32(fl32(acc_P) * fl32(sa_P[i] * sb_P[j])),
 * y = y_0 (+ y_1 when dual, added in float32), RNE to out_dt.
 *   a        device int8 [m x kp] (row stride kp)
 *   sa       device float: sa_per_token ? [m] or [m x 2] : [1] or [2]
 *   b        device: b_bits 8 -> int8 [n x kp]; b_bits 4 -> uint8 [n x kp/2] packed nibbles;
 *            with VQ_W_KBLOCK OR'ed into b_bits, the K-piece layout of those codes
 *            (vq_weight_bytes bytes), as vq_pack_weights wrote it with the same flag
 *   sb       device float [n] or [n x 2]
 *   kp, k0   kp % 64 == 0, k0 % 64 == 0, 0 < k0 <= kp, kp - k0 <= 128; the int32
 *            accumulators bound k0: k0 * 127 * 127 < 2^31 (int8 weights, k0 <= 133120) or
 *            k0 * 127 * 112 < 2^31 (4-bit weights, which enter the MFMA as 16 * code,
 *            k0 <= 150976); longer K is rejected with VQ_ERR_SHAPE
 *   y        device out_dt in {F16, BF16, F32}, [m x n], row stride ldy (element aligned;
 *            a 16-byte aligned y whose row pitch is a multiple of 16 bytes takes the
 *            vector-store path)
 *   acc_debug device int32 [P x m x n] or NULL: receives the raw accumulators
 *   ws       device workspace of vq_qgemm_workspace_bytes(m, n, k0) bytes (16-byte
 *            aligned, zero-filled before its first use), or NULL.  With it, the 256 x 256
 *            tiles that do not fill a whole round of the persistent grid are split into
 *            ranges of K handled by different workgroups; each range's int32 partial goes
 *            through the workspace and the last one to finish adds them, so the result is
 *            bit-identical to the unsplit GEMM.  Every call leaves the workspace
 *            zero-filled; calls that share one must not overlap.  A size of 0 means the
 *            shape gains nothing from the split (ws is then not used).
 * Errors: INVALID_ARG, SHAPE, UNSUPPORTED (b_bits not 4/8 with or without VQ_W_KBLOCK,
 * out_dt, or more than 2^28 output tiles of 256 x 256, which the kernels' 32-bit tile
 * counts cannot hold).
 */
int64_t vq_qgemm_workspace_bytes(int64_t m, int64_t n, int64_t k0);
vq_status vq_qgemm_dequant(const int8_t* a, const float* sa, int sa_per_token, const void* b,
                           int b_bits, const float* sb, int64_t m, int64_t n, int64_t kp, int64_t k0,
                           void* y, vq_dtype out_dt, int64_t ldy, int32_t* acc_debug, void* ws,
                           hipStream_t stream);

/*
 * vq_qgemm_dequant without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  It computes exactly what vq_qgemm_dequant computes (bit-identical
 * output) and allocates nothing: the remainder split's workspace is a static device array
 * of vq_qgemm_scratch_bytes() bytes (40 MiB) that the library holds on each GPU it runs
 * on until the process ends.  Each call clears the array's arrival counters with a fill
 * kernel on `stream` before the GEMM, and leaves them zero.  Calls that overlap on one GPU
 * (on different streams, or from different threads) share the array and race; serialize
 * them.  Arguments as for vq_qgemm_dequant, without acc_debug and ws.
 * Errors: as vq_qgemm_dequant, plus SHAPE when the shape's split needs more than the
 * array holds (vq_qgemm_workspace_bytes(m, n, k0) > vq_qgemm_scratch_bytes()).
 */
int64_t vq_qgemm_scratch_bytes(void);
vq_status vq_qgemm_dequant_noalloc(const int8_t* a, const float* sa, int sa_per_token, const void* b,
                                   int b_bits, const float* sb, int64_t m, int64_t n, int64_t kp,
                                   int64_t k0, void* y, vq_dtype out_dt, int64_t ldy,
                                   hipStream_t stream);

/*
 * Activation decomposition (SemanticDialect, gist.science summary of arXiv 2603.02883,
 * Methodology 2.2: the quantization error of the activation is quantized again and its
 * contribution added to the output, for selected tokens only).  For each listed row
 * x = rows_dev[i]: (q1, s1) = the per-token quantizer with bits1 (exactly the codes and
 * scale of vq_quant_act with VQ_PER_TOKEN, no rotation, no dual scale); deq =
 * fl32(q1 * s1); residual r = fl32(x - deq); (q2, s2) = the per-token quantizer of r with
 * bits2.  The output is a stacked operand of 2 * n_rows rows:
 *   codes  device int8 [2 n_rows x k] (8-byte aligned): row i = q1 of listed row i,
 *          row n_rows + i = its q2
 *   scales device float [2 n_rows]: s1 of listed row i, then s2
 *   x      device, dt in {F16, BF16}, [m x k], stride ldx; 16-byte aligned, ldx % 8 == 0
 *   rows_dev  device int32 [n_rows]: distinct rows of x (the salient tokens, chosen by
 *          the caller); an index outside [0, m) yields zero codes and scales
 * n_rows = 0 enqueues nothing.  Errors: INVALID_ARG, SHAPE (k % 64, alignment),
 * UNSUPPORTED (bits not 4/6/8).
 */
vq_status vq_quant_residual(const void* x, vq_dtype dt, int64_t m, int64_t k, int64_t ldx, int bits1,
                            int bits2, const int32_t* rows_dev, int64_t n_rows, int8_t* codes,
                            float* scales, hipStream_t stream);

/*
 * GEMM with the decomposed rows added back (same passage).  Every row i first gets
 * vq_qgemm_dequant's output (single partition, per-token scales):
 *   y1 = fl32(fl32(acc1[i,j]) * fl32(sa[i] * sb[j])),  acc1 = a . b,  rounded to out_dt;
 * then every listed row i = rows_dev[t] is rewritten as
 *   y = RNE_out(fl32(y1 + y2)),  y2 = fl32(fl32(acc2[t,j]) * fl32(s2[t] * sb[j])),
 * with acc1 and acc2 taken from the stacked operand of vq_quant_residual (one small GEMM
 * over its 2 n_rows rows, float32 results in ws, then a merge kernel).
 *   a, sa     the per-token codes [m x kp] and scales [m] of vq_quant_act (kp % 64 == 0)
 *   b, sb     packed weights as for vq_qgemm_dequant (b_bits 8 or 4, optionally OR
 *             VQ_W_KBLOCK), scales [n]
 *   a2, sa2   the stacked codes [2 n_rows x kp] and scales [2 n_rows] of vq_quant_residual
 *   rows_dev  device int32 [n_rows], distinct, the same list as for vq_quant_residual
 *   y         as for vq_qgemm_dequant
 *   ws        device scratch, 16-byte aligned, vq_residual_workspace_bytes(m, n_rows, n)
 *             bytes (float32 [2 n_rows x n]); contents not kept
 * Launches on `stream`: the GEMM of all rows, the GEMM of the stacked rows, the merge.
 * n_rows = 0 is vq_qgemm_dequant.  Errors: INVALID_ARG, SHAPE, UNSUPPORTED as for
 * vq_qgemm_dequant, plus UNSUPPORTED when 2 n_rows does not fit the launch grid.
 */
int64_t vq_residual_workspace_bytes(int64_t m, int64_t n_rows, int64_t n);
vq_status vq_qgemm_dequant_residual(const int8_t* a, const float* sa, const void* b, int b_bits,
                                    const float* sb, int64_t m, int64_t n, int64_t kp, const int8_t* a2,
                                    const float* sa2, const int32_t* rows_dev, int64_t n_rows, void* y,
                                    vq_dtype out_dt, int64_t ldy, void* ws, hipStream_t stream);

/*
 * MX block formats (6Bit-Diffusion, Introduction and Methodology B.1: GPUs that dropped
 * INT4 offer a 4-bit floating-point block format, and DMPQ routes activations between
 * INT8 and it, with the weights in it offline).  The gfx950 form is OCP MX: per row,
 * blocks of 32 consecutive K elements share a scale 2^e stored as an E8M0 byte
 * (e + 127), e = floor(log2(max|v|)) - 2 clamped to [-127, 127] (a zero block gets
 * e = -127); each element is v / 2^e rounded to nearest even and clamped to +-6 (FP4)
 * or +-7.5 (FP6); a negative value that rounds to zero keeps its sign bit.
 *   codes   row-major [rows x k*w/8] bytes, w = 4 or 6; element p of a row at bits
 *           [w*p, w*p+w) of the row's little-endian bit string.  VQ_MXFP4_KBLOCK: the
 *           same FP4 bytes in 64-byte K pieces (byte c of row r at (c / 64) * rows * 64 +
 *           r * 64 + c % 64, the last piece padded when k % 128 == 64), for weights
 *   scales  E8M0 bytes in step-major order [k/64][rows8][2], rows8 = rows rounded up to a
 *           multiple of 8 (byte (t * rows8 + r) * 2 + h = block 2t + h of row r); bytes
 *           of the padding rows are not written
 * vq_mx_code_bytes / vq_mx_scale_bytes give the buffer sizes (0 for invalid sizes).
 *
 * vq_mx_quant: x device, dt in {F16, BF16}, [rows x k], stride ldx; 16-byte aligned,
 *   ldx % 8 == 0, k % 64 == 0, codes 8-byte aligned.  Finite inputs.  The element codes come from the matrix unit's MX conversion
 *   instructions (round to nearest even, saturation), which match the rule above.
 *   Errors: INVALID_ARG, SHAPE, UNSUPPORTED (fmt).
 * vq_mx_gemm: y[i,j] = sum_k dec(a[i,k]) * dec(b[j,k]) on the matrix cores (block scales
 *   applied there, float32 accumulation), then RNE to out_dt.  a: activations [m x k]
 *   in fa (MXFP4 or MXFP6); b: weights [n x k], fb MXFP4 or MXFP4_KBLOCK; codes and scales
 *   16-byte aligned; y as for vq_qgemm_dequant.  The sums are accumulated in float32 by
 *   the hardware, so y equals the exact sum rounded to float32 only up to the
 *   accumulation's rounding.  ws: device workspace of vq_mx_gemm_workspace_bytes(m, n,
 *   k) bytes (16-byte aligned, zero-filled before its first use) or NULL; with it, the
 *   tiles past the last whole round of the persistent grid are split into two K ranges
 *   whose float32 partials are added once (y then differs from the unsplit GEMM by that
 *   one rounding, within the same bound, and does not depend on the order the ranges
 *   finish).  Every call leaves the workspace zeroed; calls sharing one must not
 *   overlap.  Errors: INVALID_ARG, SHAPE (k % 64, alignment), UNSUPPORTED (fa other than
 *   MXFP4/MXFP6, fb other than MXFP4/MXFP4_KBLOCK, or more than 2^28 output tiles of
 *   256 x 256).
 */
int64_t vq_mx_code_bytes(int64_t rows, int64_t k, vq_mx_fmt fmt);
int64_t vq_mx_scale_bytes(int64_t rows, int64_t k);
vq_status vq_mx_quant(const void* x, vq_dtype dt, int64_t rows, int64_t k, int64_t ldx, vq_mx_fmt fmt,
                      uint8_t* codes, uint8_t* scales, hipStream_t stream);
/*
 * MX quantization of rotated rows: the 4-bit floating-point route with the online block
 * Hadamard transform (6Bit-Diffusion, Methodology B.1).  Each row is first rotated by the
 * unnormalized 128-point Sylvester Hadamard butterflies (float32, distances 1, 2, ..., 64
 * in that order, as vq_hadamard_block with normalize = 0), scaled by 2^exp_offset
 * (exact), and the float32 result is quantized as by vq_mx_quant (same layouts).
 * Activations take exp_offset = 0; weights rotated offline take -7, so that the MX GEMM
 * of the two returns sum_k (Hx)_k (Hw)_k / 128 = sum_k x_k w_k up to quantization.
 *   x, codes, scales as for vq_mx_quant; k % 128 == 0; -64 <= exp_offset <= 64.
 * Errors: INVALID_ARG, SHAPE (k % 128, alignment), UNSUPPORTED (fmt).
 */
vq_status vq_mx_quant_rotated(const void* x, vq_dtype dt, int64_t rows, int64_t k, int64_t ldx, vq_mx_fmt fmt,
                              int exp_offset, uint8_t* codes, uint8_t* scales, hipStream_t stream);
int64_t vq_mx_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
vq_status vq_mx_gemm(const uint8_t* a, const uint8_t* sa, vq_mx_fmt fa, const uint8_t* b,
                     const uint8_t* sb, vq_mx_fmt fb, int64_t m, int64_t n, int64_t k, void* y,
                     vq_dtype out_dt, int64_t ldy, void* ws, hipStream_t stream);

/*
 * Unquantized FP16/BF16 layer for the precision override (6Bit-Diffusion, Methodology
 * B.3, PDR: a layer whose input has a high outlier ratio is computed in FP16/BF16; the
 * step control reports it as precision code 16).
 *   y[i, j] = sum_k x[i, k] * w[j, k], accumulated in float32 on the matrix cores (the
 *   products of 16-bit values are exact), then rounded once to out_dt (round to nearest
 *   even).  The sum is the exact one only up to the float32 accumulation's rounding:
 *   |y - exact| <= (k + 2) * 2^-24 * sum_k |x_k w_k| before the output rounding.
 *   x      device, dt in {F16, BF16}, [m x k], row stride ldx elements
 *   w      device, same dt, [n x k], row stride ldw elements
 *   y      device, out_dt in {F16, BF16, F32}, [m x n], row stride ldy elements; aligned
 *          to its element size (16-byte rows store faster)
 *   k % 64 == 0; x and w 16-byte aligned, ldx % 8 == 0, ldw % 8 == 0.
 * Asynchronous on `stream`; nothing is allocated.  Errors: INVALID_ARG (null pointers,
 * dtypes, sizes, strides), SHAPE (k % 64, alignment), UNSUPPORTED (more than 2^28 output
 * tiles of 256 x 256).
 */
vq_status vq_gemm_dense(const void* x, const void* w, vq_dtype dt, int64_t m, int64_t n, int64_t k,
                        int64_t ldx, int64_t ldw, void* y, vq_dtype out_dt, int64_t ldy, hipStream_t stream);

/*
 * Static per-tensor activation scale by clipping-percentile search (Q-ARVD, Technical
 * details: per-tensor activations with a clipping percentile and a scale learned during
 * reconstruction).  One pass builds the histogram of |x| over its 32768 16-bit magnitude
 * patterns; then, on the device, for each candidate percentile p:
 *   clip  = the order statistic of |x| at rank ceil(p/100 * N) (1-based, N = rows*cols)
 *   s     = fl32(clip / Q),  r = fl32(1 / s)   (Q = 2^(bits-1) - 1)
 *   mse   = sum over x of (x - fl32(clamp(rne(fl32(x * r)), -Q, Q) * s))^2 / N  (float64)
 * and the candidate of smallest mse wins (the first one on a tie).  The reconstruction
 * objective is the activation quantizer's own (the page's frame-weighted layer loss needs
 * a model); the result feeds vq_quant_act's VQ_PER_TENSOR_STATIC.
 *   x              device, dt in {F16, BF16}, [rows x cols], stride ldx; finite values;
 *                  16-byte aligned, cols % 8 == 0, ldx % 8 == 0, rows * cols < 2^32
 *   percentiles_host  host double [n_cand], each in (0, 100], 1 <= n_cand <= 64
 *                  (read during the call; kernel arguments carry them)
 *   hist_dev       device uint32 [vq_calib_hist_bins()] scratch: receives the histogram
 *   clips_dev, scales_dev (float), mse_dev (double): device [n_cand]
 *   best_dev       device int32 [1]: index of the chosen candidate
 *   scale_dev      device float [1] or NULL: receives scales_dev[best]
 * Asynchronous on `stream` (no host synchronization).  Errors: INVALID_ARG, SHAPE,
 * UNSUPPORTED (bits not 4/6/8, too many elements).
 */
int64_t vq_calib_hist_bins(void);
vq_status vq_calib_static_scale(const void* x, vq_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                                int bits, const double* percentiles_host, int32_t n_cand,
                                uint32_t* hist_dev, float* clips_dev, float* scales_dev,
                                double* mse_dev, int32_t* best_dev, float* scale_dev,
                                hipStream_t stream);

/*
 * DMPQ routing on the device (6Bit-Diffusion, Key Insights 1 and Methodology B.1):
 * Gamma = sum|y - x| / sum|x| over n elements (float64, fixed reduction order), then
 * bits = Gamma > threshold ? bits_hi : bits_lo (strict: a tie takes bits_lo).  x and y
 * are the block's input and output at the previous timestep.  sum|x| = 0 gives
 * Gamma = +inf.
 *   x, y       device, dt in {F16, BF16, F32}, [n]
 *   ws_dev     device scratch of vq_route_workspace_elems(n) doubles
 *   gamma_dev  device double [1] or NULL
 *   bits_dev   device int32 [1]: the routed bit width, ready for vq_quant_act's bits_dev
 * Errors: INVALID_ARG (null, n < 1, bits not 4/6/8).
 */
int64_t vq_route_workspace_elems(int64_t n);
vq_status vq_route_rel_l1(const void* x, const void* y, vq_dtype dt, int64_t n, double threshold,
                          int bits_hi, int bits_lo, double* ws_dev, double* gamma_dev,
                          int32_t* bits_dev, hipStream_t stream);

/*
 * One block's runtime decision at a denoising step (6Bit-Diffusion, Methodology B.1-B.3:
 * DMPQ route, TDC skip with drift control, PDR precision overrides).  On the device:
 *   E     = sum|delta_new - delta_old| / sum|delta_old|  (float64; 0 when the numerator
 *           is 0, +inf when only the denominator is 0), from the block's two cached
 *           residual deltas (output minus input at the two previous computed steps);
 *   Gamma = sum|y_prev - x_prev| / sum|x_prev|  (as vq_route_rel_l1);
 *   skip  <=>  deltas given, skips < max_skips, E <= skip_threshold and
 *              drift + E <= drift_threshold; then skips += 1, drift += E, bits = 0;
 *   else compute, skips = drift = 0, and bits =
 *     16       if n_out / channels > outlier_ratio_max (unquantized layer),
 *     8        else if the previous step was skipped (no routing information),
 *     bits_hi  else if Gamma is unknown (no x_prev/y_prev) or Gamma > route_threshold,
 *     bits_lo  otherwise.
 * The readings (delta definition, the form of E, the accumulated error, the precedence)
 * are this library's: the page states the rules without formulas.  bits_dev feeds
 * vq_quant_act's bits_dev directly (it quantizes a 16 as 8: a caller that honours the
 * flag runs the layer unquantized instead, with vq_gemm_dense).
 *   delta_new, delta_old  device [n_delta] of delta_dt (F16/BF16/F32), or both NULL
 *   x_prev, y_prev        device [n_xy] of xy_dt, or both NULL
 *   n_out_dev             device int32 [1] (e.g. vq_detect_outliers' n_out_dev) or NULL;
 *                         channels >= 1 when given
 *   state_dev             device, VQ_CONTROL_STATE_BYTES, 8-byte aligned, zero for a
 *                         fresh block: consecutive skips (int32) and the accumulated
 *                         error (double at byte 8); updated in place
 *   ws_dev                device scratch of vq_control_workspace_elems() doubles
 *   skip_dev, bits_dev    device int32 [1]: 1 to skip the block; the precision code
 *   e_dev, gamma_dev      device double [1] or NULL (NaN when not computed)
 * Asynchronous.  Calls for one block must be ordered (they share its state).
 * Errors: INVALID_ARG (null state/ws/outputs/params, an unpaired input, n < 1, a NaN
 * threshold, max_skips < 0, widths not 4/6/8, channels < 1 with n_out_dev).
 */
typedef struct vq_control_params {
  double skip_threshold;
  double drift_threshold;
  int32_t max_skips;
  int32_t bits_hi;
  int32_t bits_lo;
  double route_threshold;
  double outlier_ratio_max;
} vq_control_params;
#define VQ_CONTROL_STATE_BYTES 16
int64_t vq_control_workspace_elems(void);
vq_status vq_step_control(const void* delta_new, const void* delta_old, vq_dtype delta_dt, int64_t n_delta,
                          const void* x_prev, const void* y_prev, vq_dtype xy_dt, int64_t n_xy,
                          const int32_t* n_out_dev, int64_t channels, const vq_control_params* params,
                          void* state_dev, double* ws_dev, int32_t* skip_dev, int32_t* bits_dev,
                          double* e_dev, double* gamma_dev, hipStream_t stream);

/* Text of a status code (static storage). */
const char* vq_status_string(vq_status s);

/* The hipError_t of the last failed HIP call on this thread (0 if none). */
int vq_last_hip_error(void);

/* Library version string (static storage). */
const char* vq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VQ_H */
