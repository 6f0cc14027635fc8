// Row quantization kernels for gfx950: online activation quantization (per token,
// per tensor, static), the dual-scale outlier partition, the fused 128-point block
// Hadamard rotation, and offline per-output-channel weight packing (int8 / int4).
//
// Q-ARVD (aitrends.kr), Methodology and Technical details: per-tensor activation and
// per-channel weight quantizers, Q_dual = [Q_outlier | Q_normal] over input channels,
// an activation-quantization kernel ahead of the GEMM.  6Bit-Diffusion (gist.science,
// arXiv 2603.18742), Methodology B.1: INT8 or 4-bit activations per block, online block
// Hadamard, weights quantized offline to 4 bits.
//
// Work layout: a row of K elements is read in passes of 1024 elements; in a pass each
// of the 64 lanes of a wave owns 16 elements as two 8-element pieces (one 16-byte load
// and one 8-byte store of codes each).  Without rotation lane l owns elements 8l..8l+7
// of each 512-element half of the pass, so every load and store instruction of a wave
// covers one contiguous span; with the rotation the 8 lanes of a 128-element block own
// 8-element pieces of its two halves (see fwht128), so every load covers whole
// 128-byte lines.  A row is owned by W waves (W = 1, 2, 4 or 8) so that every lane keeps at
// most 4 passes (64 floats) in registers: the row is read from HBM once, reduced to its
// absolute maximum, and quantized from registers.  All loads of a row are issued before
// any of them is used (addresses past the row end are clamped into the row and their
// values discarded), so a wave waits for one memory latency per row, not one per pass.
#include "dev_common.h"
#include "vq_internal.h"

namespace vqk {

enum : int { MODE_ROW = 0, MODE_GLOBAL = 1, MODE_STATIC = 2 };
constexpr int NPMAX = 4;
constexpr int MAX_MASK_WORDS = 32768 / 32;

struct RowArgs {
  const void* x;
  int64_t ldx;
  int64_t rows;
  int k;               // row length of x
  int kp;              // code row length (k + p1)
  int W;               // waves per row
  int np;              // passes per wave
  int qbits;           // bit width when bits_dev is null
  const int32_t* bits_dev;
  const int32_t* idx;  // dual: outlier channels (ascending)
  int n_out;
  int p1;              // outlier partition length (multiple of 64, <= 128)
  const float* gsrc;   // MODE_GLOBAL: absmax bit patterns [P]; MODE_STATIC: scales [P]
  float scale_mul;     // exact factor folded into the stored scale (1/128 after rotation)
  void* codes;         // int8 [rows x kp] or packed uint8 [rows x kp/2]
  float* scales;       // MODE_ROW: [rows] or [rows x 2]; MAXONLY: absmax target [P]
  int64_t c_kp;        // KBLK: bytes between 64-byte K pieces (64 rows)
};

__device__ __forceinline__ float qmax_f(const RowArgs& a) {
  int b = a.bits_dev ? *a.bits_dev : a.qbits;
  b = (b == 4 || b == 6) ? b : 8;
  return (float)((1 << (b - 1)) - 1);
}

__device__ __forceinline__ void static_scale(float sgiven, float& r, float& s) {
  s = sgiven;
  r = 1.0f / sgiven;
  if (!(sgiven != 0.0f) || __builtin_isinf(r)) r = 0.0f;
}

// Eight storage elements (one 16-byte word) as float.
template <int DT>
__device__ __forceinline__ void decode8(const u4v& w, float* v) {
  decode2<DT>(w.x, v[0], v[1]);
  decode2<DT>(w.y, v[2], v[3]);
  decode2<DT>(w.z, v[4], v[5]);
  decode2<DT>(w.w, v[6], v[7]);
}

// KBLK: the codes go out in 64-byte K pieces (byte c of row r at (c / 64) * c_kp +
// 64 r + c % 64), the weight layout whose GEMM stages are whole cache lines.
template <int DT, bool HAD, bool DUAL, int MODE, bool OUT4, bool MAXONLY, int NP, bool KBLK>
__global__ __launch_bounds__(512) void k_rowquant(RowArgs a) {
  static_assert(!(HAD && DUAL), "the rotation and the outlier partition are not combined");
  __shared__ float s_red[8][2];
  // Per wave: the outlier bits of the wave's NP passes (32 words of 32 channels each).
  __shared__ unsigned s_mask[DUAL ? 8 * NPMAX * 32 : 1];
  // Dual scale with one wave per row: per row of the block, an image of the loaded row
  // (K 16-bit words, dynamic LDS sized at launch).
  extern __shared__ u4v s_rowimg_v[];
  unsigned short* s_rowimg = reinterpret_cast<unsigned short*>(s_rowimg_v);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int rpb = nwaves / a.W;  // rows per block
  const int rib = wave / a.W;
  const int wr = wave - rib * a.W;
  const float sigma = HAD ? had_sigma(perm8(lane & 7)) : 1.0f;
  const float qf = qmax_f(a);
  // First element of piece h (0, 1) of pass j in this lane.
  auto piece = [&](int j, int h) {
    const int p0 = (wr + a.W * j) * 1024;
    return HAD ? p0 + 128 * (lane >> 3) + 64 * h + 8 * perm8(lane & 7) : p0 + 512 * h + 8 * lane;
  };

  // Outlier channels gathered by this lane (the same for every row).
  int oidx[2] = {0, 0};
  if constexpr (DUAL) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (lane + 64 * i < a.n_out) oidx[i] = a.idx[lane + 64 * i];
  }
  // Outlier bits of this lane's pieces (bit t: element t of the piece is an outlier), from
  // the wave's own mask in LDS: cleared, outliers of its passes set, pieces read.  LDS
  // operations of one wave complete in program order, so no barrier is involved (the
  // fences keep the compiler from moving them across one another).  Built once the first
  // row's loads are in flight.
  unsigned obits[NP][2] = {};
  bool bits_ready = !DUAL;
  auto build_bits = [&]() {
    unsigned* wm = s_mask + wave * (NPMAX * 32);
    for (int i = lane; i < NP * 32; i += 64) wm[i] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int o = oidx[i];
      const int pass = o >> 10;
      if (lane + 64 * i < a.n_out && pass % a.W == wr && pass / a.W < NP)
        atomicOr(&wm[(pass / a.W) * 32 + ((o & 1023) >> 5)], 1u << (o & 31));
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = piece(j, h) & 1023;
        obits[j][h] = (wm[j * 32 + (e >> 5)] >> (e & 31)) & 0xFFu;
      }
  };

  // Scales common to the whole tensor.
  float r_g[2] = {0.0f, 0.0f}, s_g[2] = {0.0f, 0.0f};
  if constexpr (MODE == MODE_GLOBAL && !MAXONLY) {
    for (int p = 0; p < (DUAL ? 2 : 1); ++p) dyn_scale(a.gsrc[p], qf, r_g[p], s_g[p]);
  } else if constexpr (MODE == MODE_STATIC && !MAXONLY) {
    for (int p = 0; p < (DUAL ? 2 : 1); ++p) static_scale(a.gsrc[p], r_g[p], s_g[p]);
    // The stored scale is the given one, bit for bit (so even an output that aliases the
    // input keeps its value while other workgroups read it): no finalizing launch.
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      a.scales[0] = s_g[0];
      if constexpr (DUAL) a.scales[1] = s_g[1];
    }
  }

  float run_max[2] = {0.0f, 0.0f};  // MAXONLY running maxima

  // Byte c of row `row`'s codes.
  auto code_at = [&](int64_t row, int c) -> uint8_t* {
    uint8_t* base = reinterpret_cast<uint8_t*>(a.codes);
    if constexpr (KBLK) return base + (int64_t)(c >> 6) * a.c_kp + row * 64 + (c & 63);
    else return base + row * (OUT4 ? a.kp / 2 : a.kp) + c;
  };

  for (int64_t rowbase = (int64_t)blockIdx.x * rpb; rowbase < a.rows; rowbase += (int64_t)gridDim.x * rpb) {
    const int64_t row = rowbase + rib;
    const bool row_ok = row < a.rows;
    const char* xrow = reinterpret_cast<const char*>(a.x) + (row_ok ? row : 0) * a.ldx * 2;

    // Every load first (clamped into the row), then the decoding.
    u4v raw[NP][2];
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = piece(j, h);
        raw[j][h] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(xrow + (int64_t)(e < a.k ? e : 0) * 2));
      }
    // The row's loads go out before anything that waits for the outlier indices.
    __builtin_amdgcn_sched_barrier(0);
    // Outlier partition, at most 128 values.  A row held by several waves: gathered from
    // memory by its wave 0.  A row held by one wave (K <= 4096): taken from the row's own
    // loads through LDS (below), so no extra memory request is made.
    unsigned short oraw[2] = {0, 0};
    if constexpr (DUAL) {
      if (wr == 0 && a.W > 1) {
#pragma unroll
        for (int i = 0; i < 2; ++i) oraw[i] = reinterpret_cast<const unsigned short*>(xrow)[oidx[i]];
      }
    }

    if constexpr (DUAL) {
      if (!bits_ready) {  // wave-uniform
        build_bits();
        bits_ready = true;
      }
      if (a.W == 1) {
        // Each piece holding an outlier channel is copied, as loaded, into the wave's row
        // image in LDS (channel-indexed 16-bit words); then lane i reads outlier i.  The
        // LDS operations of one wave complete in program order; the fences keep the
        // compiler from moving them across one another.
        unsigned short* img = s_rowimg + rib * a.k;
#pragma unroll
        for (int j = 0; j < NP; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int e = piece(j, h);
            if (obits[j][h] != 0u && e < a.k) *reinterpret_cast<u4v*>(img + e) = raw[j][h];
          }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (lane + 64 * i < a.n_out) oraw[i] = img[oidx[i]];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      }
    }

    float v[NP][16];
    float lmax = 0.0f;
    // Pieces past the row end hold clamped reads: a piece (and, with the rotation, its whole
    // 128-element block) lies entirely inside or entirely past the row end, nothing past
    // it is stored, so only the row maximum has to leave them out.  (A row past the last
    // one is computed from row 0 and not stored at all.)
#pragma unroll
    for (int j = 0; j < NP; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) decode8<DT>(raw[j][h], &v[j][8 * h]);
      if constexpr (HAD) {
        fwht128<true>(v[j], perm8(lane & 7));
      }
      if constexpr (DUAL) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if ((obits[j][h] >> t) & 1u) v[j][8 * h + t] = 0.0f;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float pm = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) pm = fmaxf(pm, fabsf(v[j][8 * h + t]));
        lmax = fmaxf(lmax, piece(j, h) < a.k ? pm : 0.0f);
      }
    }

    float ov[2] = {0.0f, 0.0f};
    float omax = 0.0f;
    if constexpr (DUAL) {
      if (wr == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float lo, hi;
          decode2<DT>((unsigned)oraw[i], lo, hi);
          ov[i] = (row_ok && lane + 64 * i < a.n_out) ? lo : 0.0f;
          omax = fmaxf(omax, fabsf(ov[i]));
        }
        omax = wave_max(omax);
      }
    }

    float amax = wave_max(lmax);
    if (a.W > 1) {
      if (lane == 0) s_red[wave][0] = amax;
      __syncthreads();
      float m = 0.0f;
      for (int w = 0; w < a.W; ++w) m = fmaxf(m, s_red[rib * a.W + w][0]);
      amax = m;
      __syncthreads();
    }

    if constexpr (MAXONLY) {
      if (row_ok) {
        run_max[0] = fmaxf(run_max[0], amax);
        run_max[1] = fmaxf(run_max[1], omax);
      }
      continue;
    }

    float r0, s0, r1 = 0.0f, s1 = 0.0f;
    if constexpr (MODE == MODE_ROW) {
      dyn_scale(amax, qf, r0, s0);
      if constexpr (DUAL) dyn_scale(omax, qf, r1, s1);
    } else {
      r0 = r_g[0];
      s0 = s_g[0];
      r1 = r_g[1];
      s1 = s_g[1];
    }
    const float rr = r0 * sigma;  // exact: sigma = +-1

    if (row_ok) {
#pragma unroll
      for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = piece(j, h);
          if (e < a.k) {
            unsigned u[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) u[t] = qbyte(v[j][8 * h + t], rr, qf);
            if constexpr (OUT4) {
              reinterpret_cast<unsigned*>(code_at(row, e / 2))[0] = pack8_nibbles(u);
            } else {
              *reinterpret_cast<u2v*>(code_at(row, e)) =
                  u2v{pack4_lo(u[0], u[1], u[2], u[3]), pack4_lo(u[4], u[5], u[6], u[7])};
            }
          }
        }
      if constexpr (DUAL) {
        if (wr == 0) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int jj = lane + 64 * i;
            const unsigned c = qbyte(ov[i], r1, qf) & 0xFFu;
            if constexpr (OUT4) {
              const unsigned nb = __shfl_down(c, 1, 64);
              if (jj < a.p1 && (jj & 1) == 0)
                *code_at(row, (a.k + jj) / 2) = (uint8_t)((c & 0xFu) | ((nb & 0xFu) << 4));
            } else {
              if (jj < a.p1) *code_at(row, a.k + jj) = (uint8_t)c;
            }
          }
        }
      }
      if constexpr (MODE == MODE_ROW) {
        if (wr == 0 && lane == 0) {
          if constexpr (DUAL) {
            a.scales[2 * row] = s0 * a.scale_mul;
            a.scales[2 * row + 1] = s1 * a.scale_mul;
          } else {
            a.scales[row] = s0 * a.scale_mul;
          }
        }
      }
    }
  }

  if constexpr (MAXONLY) {
    // Block maximum, then one atomic per block and partition (non-negative floats
    // order like their bit patterns, so an unsigned max is the float max).
    float m0 = wave_max(run_max[0]);
    float m1 = run_max[1];  // already a wave max (lanes agree)
    if (lane == 0) {
      s_red[wave][0] = m0;
      s_red[wave][1] = m1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float b0 = 0.0f, b1 = 0.0f;
      for (int w = 0; w < nwaves; ++w) {
        b0 = fmaxf(b0, s_red[w][0]);
        b1 = fmaxf(b1, s_red[w][1]);
      }
      atomicMax(reinterpret_cast<unsigned*>(a.scales), f_bits(b0));
      if constexpr (DUAL) atomicMax(reinterpret_cast<unsigned*>(a.scales) + 1, f_bits(b1));
    }
  }
}

__global__ void k_fill_u32(unsigned* p, int n, unsigned v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Dynamic per-tensor scales after the codes: the maxima the code pass read are replaced
// by s = fl32(amax / Q).
__global__ void k_tensor_finalize(float* scales, int parts, int qbits, const int32_t* bits_dev) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int b = bits_dev ? *bits_dev : qbits;
  b = (b == 4 || b == 6) ? b : 8;
  const float qf = (float)((1 << (b - 1)) - 1);
  for (int p = 0; p < parts; ++p) {
    float r, s;
    dyn_scale(scales[p], qf, r, s);
    scales[p] = s;
  }
}

// Dynamic per-tensor quantization of a small tensor in one launch.  Every workgroup
// reduces the whole tensor's absolute maximum by itself (a maximum is exact in any order,
// so all workgroups find the same value), derives r = fl32(Q/a) and s = fl32(a/Q) as the
// two-pass path does, and quantizes its own range of 8-element pieces; workgroup 0 stores
// s.  Each workgroup starts its pass at its own range, so the pieces it quantizes are
// among its first loads and are still in registers when the maximum is known: one memory
// latency for the whole kernel.  No clearing, no atomics and no finalizing launch: at a few
// hundred KB the launches of the two-pass path cost more than the redundant reads, which
// the L2 serves.
constexpr int SMALL_THREADS = 1024;
constexpr int SMALL_UNROLL = 8;
constexpr int SMALL_MAX_GRID = 16;

template <int DT, bool CONTIG>
__global__ __launch_bounds__(SMALL_THREADS) void k_tensorquant_small(const void* x, int64_t ldx, int rows, int k,
                                                                     int qbits, const int32_t* bits_dev,
                                                                     int8_t* codes, float* scales) {
  __shared__ float s_red[SMALL_THREADS / 64];
  const int ppr = k / 8;  // pieces per row
  const int n = rows * ppr;
  const int tid = threadIdx.x;
  const int per = (n + (int)gridDim.x - 1) / (int)gridDim.x;  // at most SMALL_THREADS * SMALL_UNROLL
  const int lo = min(n, (int)blockIdx.x * per);
  const int hi = min(n, lo + per);
  auto piece_of = [&](int j) {  // j-th piece of this workgroup's pass (j < n): starts at lo, wraps
    const int i = lo + j;
    return i < n ? i : i - n;
  };
  auto load = [&](int i) {
    int64_t off = (int64_t)i * 8;
    if constexpr (!CONTIG) {
      const int r = i / ppr;
      off = (int64_t)r * ldx + 8 * (i - r * ppr);
    }
    return *reinterpret_cast<const u4v*>(reinterpret_cast<const uint16_t*>(x) + off);
  };
  float m = 0.0f;
  u4v own[SMALL_UNROLL];  // the first batch: this workgroup's own pieces
#pragma unroll
  for (int u = 0; u < SMALL_UNROLL; ++u) {
    const int j = u * SMALL_THREADS + tid;
    own[u] = load(piece_of(j < n ? j : 0));
  }
  for (int j0 = SMALL_THREADS * SMALL_UNROLL; j0 < n; j0 += SMALL_THREADS * SMALL_UNROLL) {
    u4v w[SMALL_UNROLL];
#pragma unroll
    for (int u = 0; u < SMALL_UNROLL; ++u) {
      const int j = j0 + u * SMALL_THREADS + tid;
      w[u] = load(piece_of(j < n ? j : 0));  // a piece loaded again cannot raise the maximum
    }
#pragma unroll
    for (int u = 0; u < SMALL_UNROLL; ++u) {
      float v[8];
      decode8<DT>(w[u], v);
#pragma unroll
      for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(v[t]));
    }
  }
  float vo[SMALL_UNROLL][8];
#pragma unroll
  for (int u = 0; u < SMALL_UNROLL; ++u) {
    decode8<DT>(own[u], vo[u]);
#pragma unroll
    for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(vo[u][t]));
  }
  m = wave_max(m);
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  float amax = 0.0f;
#pragma unroll
  for (int w = 0; w < SMALL_THREADS / 64; ++w) amax = fmaxf(amax, s_red[w]);

  int b = bits_dev ? *bits_dev : qbits;
  b = (b == 4 || b == 6) ? b : 8;
  const float qf = (float)((1 << (b - 1)) - 1);
  float r, sc;
  dyn_scale(amax, qf, r, sc);

#pragma unroll
  for (int u = 0; u < SMALL_UNROLL; ++u) {
    const int i = lo + u * SMALL_THREADS + tid;
    if (i < hi) {
      unsigned q[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) q[t] = qbyte(vo[u][t], r, qf);
      // code rows are k long, so piece i starts at code 8i
      *reinterpret_cast<u2v*>(codes + (int64_t)i * 8) =
          u2v{pack4_lo(q[0], q[1], q[2], q[3]), pack4_lo(q[4], q[5], q[6], q[7])};
    }
  }
  if (blockIdx.x == 0 && tid == 0) scales[0] = sc;
}

// Absolute maximum of a whole tensor (no outlier partition, no rotation) for the dynamic
// per-tensor scale: a flat grid-stride pass over 8-element pieces with eight 16-byte loads
// in flight per lane, one workgroup of 1024 lanes per CU and one atomic maximum per
// workgroup (non-negative floats order like their bit patterns).  The row-structured
// maximum pass needs a row's loads per wave and thousands of workgroups, each ending in
// an atomic on the same word.
constexpr int AMAX_THREADS = 1024;
constexpr int AMAX_UNROLL = 8;

template <int DT, bool CONTIG>
__global__ __launch_bounds__(AMAX_THREADS) void k_tensor_absmax(const void* x, int64_t ldx, int rows, int k,
                                                                unsigned* maxbits) {
  __shared__ float s_red[AMAX_THREADS / 64];
  const int ppr = k / 8;
  const int n = rows * ppr;
  const int stride = (int)gridDim.x * AMAX_THREADS;
  const int tid = threadIdx.x;
  auto load = [&](int i) {
    int64_t off;
    if constexpr (CONTIG) {
      off = (int64_t)i * 8;
    } else {
      const int r = i / ppr;
      off = (int64_t)r * ldx + 8 * (i - r * ppr);
    }
    return __builtin_nontemporal_load(reinterpret_cast<const u4v*>(reinterpret_cast<const uint16_t*>(x) + off));
  };
  float m = 0.0f;
  for (int i0 = (int)blockIdx.x * AMAX_THREADS + tid; i0 < n; i0 += stride * AMAX_UNROLL) {
    u4v w[AMAX_UNROLL];
#pragma unroll
    for (int u = 0; u < AMAX_UNROLL; ++u) {
      const int i = i0 + u * stride;
      w[u] = load(i < n ? i : i0);  // piece i0 again past the end: cannot raise the maximum
    }
#pragma unroll
    for (int u = 0; u < AMAX_UNROLL; ++u) {
      float v[8];
      decode8<DT>(w[u], v);
#pragma unroll
      for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(v[t]));
    }
  }
  m = wave_max(m);
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    float b = 0.0f;
#pragma unroll
    for (int w = 0; w < AMAX_THREADS / 64; ++w) b = fmaxf(b, s_red[w]);
    atomicMax(maxbits, f_bits(b));
  }
}

template <int DT, bool HAD, bool DUAL, int MODE, bool OUT4, bool MAXONLY, bool KBLK = false>
static hipError_t launch_row(const RowArgs& a, int grid, int block, hipStream_t st) {
  // The pass count is a compile-time constant so that a lane holds exactly its passes.
  const size_t shm = (DUAL && a.W == 1) ? (size_t)(block / 64) * a.k * 2 : 0;  // rows per block x K words
  switch (a.np) {
    case 1: hipLaunchKernelGGL((k_rowquant<DT, HAD, DUAL, MODE, OUT4, MAXONLY, 1, KBLK>), dim3(grid), dim3(block), shm, st, a); break;
    case 2: hipLaunchKernelGGL((k_rowquant<DT, HAD, DUAL, MODE, OUT4, MAXONLY, 2, KBLK>), dim3(grid), dim3(block), shm, st, a); break;
    case 3: hipLaunchKernelGGL((k_rowquant<DT, HAD, DUAL, MODE, OUT4, MAXONLY, 3, KBLK>), dim3(grid), dim3(block), shm, st, a); break;
    default: hipLaunchKernelGGL((k_rowquant<DT, HAD, DUAL, MODE, OUT4, MAXONLY, NPMAX, KBLK>), dim3(grid), dim3(block), shm, st, a); break;
  }
  return hipGetLastError();
}

template <int DT, bool HAD, bool DUAL>
static hipError_t dispatch_mode(const RowArgs& a, int mode, bool out4, bool maxonly, bool kblock, int grid,
                                int block, hipStream_t st) {
  if (maxonly) return launch_row<DT, HAD, DUAL, MODE_ROW, false, true>(a, grid, block, st);
  if (kblock) {  // weights: per-row (output-channel) scales
    if (out4) return launch_row<DT, HAD, DUAL, MODE_ROW, true, false, true>(a, grid, block, st);
    return launch_row<DT, HAD, DUAL, MODE_ROW, false, false, true>(a, grid, block, st);
  }
  if (out4) return launch_row<DT, HAD, DUAL, MODE_ROW, true, false>(a, grid, block, st);
  switch (mode) {
    case MODE_ROW: return launch_row<DT, HAD, DUAL, MODE_ROW, false, false>(a, grid, block, st);
    case MODE_GLOBAL: return launch_row<DT, HAD, DUAL, MODE_GLOBAL, false, false>(a, grid, block, st);
    default: return launch_row<DT, HAD, DUAL, MODE_STATIC, false, false>(a, grid, block, st);
  }
}

template <int DT>
static hipError_t dispatch_dt(const RowArgs& a, bool had, bool dual, int mode, bool out4, bool maxonly, bool kblock,
                              int grid, int block, hipStream_t st) {
  if (had) return dispatch_mode<DT, true, false>(a, mode, out4, maxonly, kblock, grid, block, st);
  if (dual) return dispatch_mode<DT, false, true>(a, mode, out4, maxonly, kblock, grid, block, st);
  return dispatch_mode<DT, false, false>(a, mode, out4, maxonly, kblock, grid, block, st);
}

}  // namespace vqk

namespace vq_internal {

using namespace vqk;

static void row_geometry(int k, int& W, int& np, int& block) {
  const int passes = (k + 1023) / 1024;
  W = passes <= 4 ? 1 : passes <= 8 ? 2 : passes <= 16 ? 4 : 8;
  np = (passes + W - 1) / W;
  block = W == 8 ? 512 : 256;
}

int row_quant_max_k() { return 8 * NPMAX * 1024; }

static RowArgs make_args(const RowQuantParams& p) {
  RowArgs a{};
  a.x = p.x;
  a.ldx = p.ldx;
  a.rows = p.rows;
  a.k = (int)p.k;
  a.kp = (int)p.kp;
  a.qbits = p.bits;
  a.bits_dev = p.bits_dev;
  a.idx = p.idx;
  a.n_out = p.n_out;
  a.p1 = p.p1;
  a.gsrc = p.gsrc;
  a.scale_mul = p.scale_mul;
  a.codes = p.codes;
  a.scales = p.scales;
  a.c_kp = p.kblock ? 64 * p.rows : 64;
  return a;
}

hipError_t launch_row_quant(const RowQuantParams& p, hipStream_t st) {
  if (p.kblock && (p.mode != 0 || p.maxonly)) return hipErrorInvalidValue;  // a weight layout
  RowArgs a = make_args(p);
  int W, np, block;
  row_geometry(a.k, W, np, block);
  a.W = W;
  a.np = np;
  const int rpb = (block / 64) / W;
  int64_t blocks = (p.rows + rpb - 1) / rpb;
  if (p.maxonly && blocks > 2048) blocks = 2048;
  // With the outlier partition every wave first waits for the outlier indices (its
  // gathers need them); a bounded grid lets each wave pay that once over several rows.
  // At 17776 x 3072: 512 blocks 31.2 us, 1024 30.6, 2048 29.9, no bound 30.2.
  if (p.n_out > 0 && blocks > 2048) blocks = 2048;
  if (blocks > (1 << 30)) blocks = 1 << 30;
  const int grid = (int)blocks;
  const int mode = p.mode;
  switch (p.dtype) {
    case DT_F16: return dispatch_dt<DT_F16>(a, p.had, p.n_out > 0, mode, p.out4, p.maxonly, p.kblock, grid, block, st);
    case DT_BF16: return dispatch_dt<DT_BF16>(a, p.had, p.n_out > 0, mode, p.out4, p.maxonly, p.kblock, grid, block, st);
    default: return hipErrorInvalidValue;
  }
}

int64_t tensor_small_max_elems() { return (int64_t)1 << 18; }

hipError_t launch_tensor_small(const void* x, int dtype, int64_t ldx, int64_t rows, int64_t k, int bits,
                               const int32_t* bits_dev, int8_t* codes, float* scales, hipStream_t st) {
  if (rows * k > tensor_small_max_elems() || k % 8) return hipErrorInvalidValue;
  // One piece per thread where the grid allows it; every workgroup's range must fit in
  // its first batch of loads (2^18 elements: 32768 pieces, 2048 per workgroup).
  const int64_t pieces = rows * (k / 8);
  int grid = (int)((pieces + SMALL_THREADS - 1) / SMALL_THREADS);
  grid = grid < 1 ? 1 : grid > SMALL_MAX_GRID ? SMALL_MAX_GRID : grid;
  if ((pieces + grid - 1) / grid > (int64_t)SMALL_THREADS * SMALL_UNROLL) return hipErrorInvalidValue;
  const bool contig = ldx == k;
  const int r = (int)rows, kk = (int)k;
#define VQ_SMALLQ(D, C)                                                                                          \
  hipLaunchKernelGGL((k_tensorquant_small<D, C>), dim3(grid), dim3(SMALL_THREADS), 0, st, x, ldx, r, kk, bits, \
                     bits_dev, codes, scales)
  switch (dtype) {
    case DT_F16: if (contig) VQ_SMALLQ(DT_F16, true); else VQ_SMALLQ(DT_F16, false); break;
    case DT_BF16: if (contig) VQ_SMALLQ(DT_BF16, true); else VQ_SMALLQ(DT_BF16, false); break;
    default: return hipErrorInvalidValue;
  }
#undef VQ_SMALLQ
  return hipGetLastError();
}

int64_t tensor_absmax_max_pieces() { return (int64_t)1 << 30; }  // 32-bit piece indices

hipError_t launch_tensor_absmax(const void* x, int dtype, int64_t ldx, int64_t rows, int64_t k, unsigned* maxbits,
                                hipStream_t st) {
  const int64_t pieces = rows * (k / 8);
  if (k % 8 || pieces > tensor_absmax_max_pieces()) return hipErrorInvalidValue;
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    return n;
  }();
  int64_t grid = (pieces + (int64_t)AMAX_THREADS * AMAX_UNROLL - 1) / ((int64_t)AMAX_THREADS * AMAX_UNROLL);
  grid = grid < 1 ? 1 : grid > cus ? cus : grid;
  const bool contig = ldx == k;
  const int r = (int)rows, kk = (int)k;
#define VQ_AMAX(D, C) hipLaunchKernelGGL((k_tensor_absmax<D, C>), dim3((int)grid), dim3(AMAX_THREADS), 0, st, x, ldx, r, kk, maxbits)
  switch (dtype) {
    case DT_F16: if (contig) VQ_AMAX(DT_F16, true); else VQ_AMAX(DT_F16, false); break;
    case DT_BF16: if (contig) VQ_AMAX(DT_BF16, true); else VQ_AMAX(DT_BF16, false); break;
    default: return hipErrorInvalidValue;
  }
#undef VQ_AMAX
  return hipGetLastError();
}

hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t st) {
  hipLaunchKernelGGL(k_fill_u32, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_tensor_finalize(float* scales, int parts, int qbits, const int32_t* bits_dev, hipStream_t st) {
  hipLaunchKernelGGL(k_tensor_finalize, dim3(1), dim3(64), 0, st, scales, parts, qbits, bits_dev);
  return hipGetLastError();
}

}  // namespace vq_internal
