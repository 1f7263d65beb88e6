// qemb.hip -- row-wise INT4/INT8 quantized embedding tables on gfx950.
//
// Kernels and the C ABI declared in include/qemb.h:
//   * quantize_range_kernel   row range -> fp16 scale/bias -> codes -> packed row
//   * quantize_greedy_kernel  greedy clip search on the row's squared error,
//                             then the same encoding
//   * dequant_kernel          packed rows -> fp32
//   * bag_kernel              fused decode + (weighted) sum pooling over CSR bags
//   * l2_partial/l2_final     normalized l2 error, fixed-order reduction
//
// The method: row-wise uniform quantization with fp16 scale and bias, clip
// thresholds from the row range or from a greedy search over the squared
// error ("Post-Training 4-bit Quantization on Embedding Tables", review page,
// "Proposed method" / "Main findings"); 4-bit codes bit-packed two per byte
// (DQRM repository page, Android demo paragraph); pooled lookups of sparse
// ids through many tables ("Deep Learning Recommendation Model for
// Personalization and Recommendation Systems", review page, "Proposed
// method").  The bit-level rules are spelled out in include/qemb.h.
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off (no fast-math):
// the quantizer must round exactly as the rules say (IEEE division, one
// rounding per operation, fp32 denormals kept, which is gfx950's default).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qemb.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t half_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float half_value(uint32_t b16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(b16 & 0xffffu));  // exact
}

// Quantization window: stored fp16 scale/bias and the reciprocal of the
// stored scale (0 when the stored scale is 0, which makes every code 0).
struct Window {
  uint32_t s16, b16;
  float sf, bf, r;
};

template <int BITS>
__device__ __forceinline__ Window make_window(float lo, float hi) {
  constexpr float Qf = (float)((1 << BITS) - 1);
  float s = (hi - lo) / Qf;
  if (!(s > 0.0f)) s = 0.0f;
  Window w;
  w.s16 = half_bits(s);
  w.b16 = half_bits(lo);
  w.sf = half_value(w.s16);
  w.bf = half_value(w.b16);
  w.r = (w.sf == 0.0f) ? 0.0f : 1.0f / w.sf;
  return w;
}

// Code of one element as a float in [0, Q] (integral).
template <int BITS>
__device__ __forceinline__ float code_of(float x, const Window& w) {
  constexpr float Qf = (float)((1 << BITS) - 1);
  float t = (x - w.bf) * w.r;
  float q = __builtin_rintf(t);
  return fminf(fmaxf(q, 0.0f), Qf);
}

// The 4 parameter bytes (s16 | b16 << 16) start at byte C of the row; this
// returns their contribution to the row dword that starts at byte 4j, given
// off = C - 4j.
__device__ __forceinline__ uint32_t param_part(uint32_t p32, int off) {
  if (off >= 4 || off <= -4) return 0u;
  return off >= 0 ? (p32 << (8 * off)) : (p32 >> (-8 * off));
}

// Load the 4 parameter bytes at byte C of a 16-byte aligned row.
__device__ __forceinline__ uint32_t load_params(const uint8_t* row, int C) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + (C & ~3));
  const int sh = C & 3;
  if (sh == 0) return p[0];
  return __builtin_amdgcn_alignbyte(p[1], p[0], (uint32_t)sh);
}

template <int N>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) v = fminf(v, __shfl_xor(v, m));
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ int64_t load_index(const void* p, int64_t k, int idx64) {
  return idx64 ? reinterpret_cast<const int64_t*>(p)[k]
               : (int64_t)reinterpret_cast<const int32_t*>(p)[k];
}

// ---------------------------------------------------------------------------
// range quantizer: LPR lanes per row, 8 contiguous elements per lane per
// chunk, NCH chunks per lane.  Memory-bound: one streaming read of the row,
// one write of the packed row.
// ---------------------------------------------------------------------------

template <int BITS, int LPR, int NCH>
__global__ __launch_bounds__(kBlock) void quantize_range_kernel(
    const float* __restrict__ x, int64_t rows, int dim, int C, int S, int vec4,
    uint8_t* __restrict__ packed) {
  constexpr int EPL = 8;
  constexpr int ND = EPL * BITS / 32;  // code dwords per chunk (1 or 2)
  const int s = threadIdx.x % LPR;
  const int64_t groups = (int64_t)gridDim.x * (kBlock / LPR);
  const int nwords = S / (4 * ND);
  for (int64_t row = (int64_t)blockIdx.x * (kBlock / LPR) + threadIdx.x / LPR; row < rows;
       row += groups) {
    const float* xr = x + row * dim;
    float v[NCH][EPL];
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = (c * LPR + s) * EPL;
      if (vec4 && e0 + EPL <= dim) {
        const float4 a = *reinterpret_cast<const float4*>(xr + e0);
        const float4 b = *reinterpret_cast<const float4*>(xr + e0 + 4);
        v[c][0] = a.x; v[c][1] = a.y; v[c][2] = a.z; v[c][3] = a.w;
        v[c][4] = b.x; v[c][5] = b.y; v[c][6] = b.z; v[c][7] = b.w;
      } else {
#pragma unroll
        for (int k = 0; k < EPL; ++k) v[c][k] = (e0 + k < dim) ? xr[e0 + k] : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        if (e0 + k < dim) {
          mn = fminf(mn, v[c][k]);
          mx = fmaxf(mx, v[c][k]);
        }
      }
    }
    mn = group_min<LPR>(mn);
    mx = group_max<LPR>(mx);
    const Window w = make_window<BITS>(mn + 0.0f, mx + 0.0f);
    const uint32_t p32 = w.s16 | (w.b16 << 16);
    uint8_t* prow = packed + row * (int64_t)S;
    // word wd (ND dwords) of the row belongs to lane wd % LPR, chunk wd / LPR;
    // words past the code chunks hold only parameter bytes and zero padding
#pragma unroll
    for (int c = 0; c < NCH + 6; ++c) {
      const int wd = c * LPR + s;
      if (wd >= nwords) break;
      uint32_t cw[ND];
#pragma unroll
      for (int dd = 0; dd < ND; ++dd) cw[dd] = 0u;
      if (c < NCH) {
        const int e0 = (c * LPR + s) * EPL;
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
          if (e0 + k < dim) {
            const uint32_t q = (uint32_t)code_of<BITS>(v[c < NCH ? c : 0][k], w);
            cw[(k * BITS) / 32] |= q << ((k * BITS) % 32);
          }
        }
      }
#pragma unroll
      for (int dd = 0; dd < ND; ++dd) cw[dd] |= param_part(p32, C - 4 * (wd * ND + dd));
      if (ND == 1) {
        *reinterpret_cast<uint32_t*>(prow + 4 * wd) = cw[0];
      } else {
        *reinterpret_cast<uint2*>(prow + 8 * wd) = make_uint2(cw[0], cw[ND - 1]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// greedy quantizer: EPL contiguous elements per lane held in registers, LPR
// lanes per row (LPR = 1 up to 64 elements).  ALU-bound: every step evaluates
// two candidate windows, each a full encode / decode / squared error.
// ---------------------------------------------------------------------------

// Squared error of the lane's row (or row slice) at window [lo, hi]: the
// pairwise sum of contiguous halves, in-lane first, then across the LPR
// lanes (xor 1, 2, 4, ...), which forms the same tree.
template <int BITS, int EPL, int LPR, bool PAD>
__device__ __forceinline__ float window_sse(const float (&v)[EPL], int valid, float lo, float hi) {
  const Window w = make_window<BITS>(lo, hi);
  float u[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    const float q = code_of<BITS>(v[k], w);
    const float y = __builtin_fmaf(w.sf, q, w.bf);
    const float e = v[k] - y;
    u[k] = e * e;
    if (PAD && k >= valid) u[k] = 0.0f;
  }
#pragma unroll
  for (int h = 1; h < EPL; h <<= 1) {
#pragma unroll
    for (int k = 0; k < EPL; k += 2 * h) u[k] = u[k] + u[k + h];
  }
  float tot = u[0];
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) tot = tot + __shfl_xor(tot, m);
  return tot;
}

template <int BITS, int EPL, int LPR, bool PAD>
__global__ __launch_bounds__(kBlock) void quantize_greedy_kernel(
    const float* __restrict__ x, int64_t rows, int dim, int C, int S, int vec4, int n_bins,
    int n_steps, uint8_t* __restrict__ packed) {
  constexpr int CODE_DW = (EPL * BITS + 31) / 32;  // code dwords held by a lane
  constexpr int S_MAX = 16 * ((((EPL * LPR * BITS + 7) / 8) + 4 + 15) / 16);
  const int s = threadIdx.x % LPR;
  const int64_t groups = (int64_t)gridDim.x * (kBlock / LPR);
  for (int64_t row = (int64_t)blockIdx.x * (kBlock / LPR) + threadIdx.x / LPR; row < rows;
       row += groups) {
    const float* xr = x + row * dim;
    const int e0 = s * EPL;
    const int valid = min(max(dim - e0, 0), EPL);
    float v[EPL];
    if (EPL >= 4 && vec4 && valid == EPL) {
#pragma unroll
      for (int k = 0; k < EPL; k += 4) {
        const float4 a = *reinterpret_cast<const float4*>(xr + e0 + k);
        v[k] = a.x; v[k + 1] = a.y; v[k + 2] = a.z; v[k + 3] = a.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPL; ++k) v[k] = (k < valid) ? xr[e0 + k] : 0.0f;
    }
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      if (!PAD || k < valid) {
        mn = fminf(mn, v[k]);
        mx = fmaxf(mx, v[k]);
      }
    }
    const float xmin = group_min<LPR>(mn) + 0.0f;
    const float xmax = group_max<LPR>(mx) + 0.0f;
    int bi = 0, bj = 0;
    if (xmax != xmin) {
      const float delta = (xmax - xmin) / (float)n_bins;
      int i = 0, j = 0;
      float lo_i = __builtin_fmaf(0.0f, delta, xmin) + 0.0f;
      float hi_j = __builtin_fmaf(-0.0f, delta, xmax) + 0.0f;
      float best = window_sse<BITS, EPL, LPR, PAD>(v, valid, lo_i, hi_j);
      for (int step = 0; step < n_steps; ++step) {
        const float lo_n = __builtin_fmaf((float)(i + 1), delta, xmin) + 0.0f;
        const float hi_n = __builtin_fmaf(-(float)(j + 1), delta, xmax) + 0.0f;
        const float la = window_sse<BITS, EPL, LPR, PAD>(v, valid, lo_n, hi_j);
        const float lb = window_sse<BITS, EPL, LPR, PAD>(v, valid, lo_i, hi_n);
        const bool move_lo = la < lb;  // a tie moves the high end
        const float cur = move_lo ? la : lb;
        i += move_lo ? 1 : 0;
        j += move_lo ? 0 : 1;
        lo_i = move_lo ? lo_n : lo_i;
        hi_j = move_lo ? hi_j : hi_n;
        const bool better = cur < best;
        best = better ? cur : best;
        bi = better ? i : bi;
        bj = better ? j : bj;
      }
    }
    // kept window; (0, 0) is the row's range (also when the row is constant)
    const float delta_k = (xmax - xmin) / (float)n_bins;
    const float lo = __builtin_fmaf((float)bi, delta_k, xmin) + 0.0f;
    const float hi = __builtin_fmaf(-(float)bj, delta_k, xmax) + 0.0f;
    const Window w = make_window<BITS>(lo, hi);
    const uint32_t p32 = w.s16 | (w.b16 << 16);
    uint32_t cw[CODE_DW];
#pragma unroll
    for (int dd = 0; dd < CODE_DW; ++dd) cw[dd] = 0u;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      if (k < valid) {
        const uint32_t q = (uint32_t)code_of<BITS>(v[k], w);
        cw[(k * BITS) / 32] |= q << ((k * BITS) % 32);
      }
    }
    uint8_t* prow = packed + row * (int64_t)S;
    if (LPR == 1) {
      // one lane owns the whole row
#pragma unroll
      for (int U = 0; U < S_MAX / 16; ++U) {
        if (16 * U < S) {
          uint32_t d4[4];
#pragma unroll
          for (int dd = 0; dd < 4; ++dd) {
            const int j = 4 * U + dd;
            d4[dd] = (j < CODE_DW ? cw[j < CODE_DW ? j : 0] : 0u) | param_part(p32, C - 4 * j);
          }
          *reinterpret_cast<uint4*>(prow + 16 * U) = make_uint4(d4[0], d4[1], d4[2], d4[3]);
        }
      }
    } else {
      // lane s owns the 16-byte units of its code dwords; the units past all
      // lanes' code dwords (parameters / padding) go round robin
      constexpr int UPL = CODE_DW / 4;
#pragma unroll
      for (int u = 0; u < UPL; ++u) {
        const int U = s * UPL + u;
        if (16 * U < S) {
          uint32_t d4[4];
#pragma unroll
          for (int dd = 0; dd < 4; ++dd) d4[dd] = cw[4 * u + dd] | param_part(p32, C - 4 * (4 * U + dd));
          *reinterpret_cast<uint4*>(prow + 16 * U) = make_uint4(d4[0], d4[1], d4[2], d4[3]);
        }
      }
      for (int U = LPR * UPL + s; 16 * U < S; U += LPR) {
        uint32_t d4[4];
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) d4[dd] = param_part(p32, C - 4 * (4 * U + dd));
        *reinterpret_cast<uint4*>(prow + 16 * U) = make_uint4(d4[0], d4[1], d4[2], d4[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dequantize: LPR lanes per row, 8 elements per lane per chunk
// ---------------------------------------------------------------------------

template <int BITS, int LPR, int NCH>
__global__ __launch_bounds__(kBlock) void dequant_kernel(const uint8_t* __restrict__ packed,
                                                         int64_t rows, int dim, int C, int S,
                                                         int vec4, float* __restrict__ y) {
  constexpr int EPL = 8;
  const int s = threadIdx.x % LPR;
  const int64_t groups = (int64_t)gridDim.x * (kBlock / LPR);
  for (int64_t row = (int64_t)blockIdx.x * (kBlock / LPR) + threadIdx.x / LPR; row < rows;
       row += groups) {
    const uint8_t* prow = packed + row * (int64_t)S;
    const uint32_t p = load_params(prow, C);
    const float sf = half_value(p), bf = half_value(p >> 16);
    float* yr = y + row * dim;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = (c * LPR + s) * EPL;
      if (e0 >= dim) break;
      float o[EPL];
      if (BITS == 4) {
        const uint32_t wd = *reinterpret_cast<const uint32_t*>(prow + e0 / 2);
#pragma unroll
        for (int k = 0; k < EPL; ++k) o[k] = __builtin_fmaf(sf, (float)((wd >> (4 * k)) & 15u), bf);
      } else {
        const uint2 wd = *reinterpret_cast<const uint2*>(prow + e0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o[k] = __builtin_fmaf(sf, (float)((wd.x >> (8 * k)) & 255u), bf);
          o[k + 4] = __builtin_fmaf(sf, (float)((wd.y >> (8 * k)) & 255u), bf);
        }
      }
      if (vec4 && e0 + EPL <= dim) {
        *reinterpret_cast<float4*>(yr + e0) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(yr + e0 + 4) = make_float4(o[4], o[5], o[6], o[7]);
      } else {
#pragma unroll
        for (int k = 0; k < EPL; ++k)
          if (e0 + k < dim) yr[e0 + k] = o[k];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// pooled lookup.  A bag is owned by a slice of LPR*RG lanes: RG row groups of
// LPR lanes; lane (g, s) reads VEC code bytes at byte s*VEC of rows
// p0+g, p0+g+RG, ...  U rows per group are in flight per iteration (all their
// loads are issued before any is used).  The RG partial vectors are reduced
// across the slice by xor shuffles.
// ---------------------------------------------------------------------------

template <int BITS, int VEC>
struct CodeChunk;
template <int BITS>
struct CodeChunk<BITS, 8> {
  uint2 v;
  __device__ __forceinline__ void load(const uint8_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint2(0u, 0u); }
  __device__ __forceinline__ uint32_t dw(int i) const { return i == 0 ? v.x : v.y; }
};
template <int BITS>
struct CodeChunk<BITS, 16> {
  uint4 v;
  __device__ __forceinline__ void load(const uint8_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ uint32_t dw(int i) const {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
  }
};

// acc[k] += w * fmaf(sf, code_k, bf): each term is the decoded value (one
// rounding, as a standalone decode gives) times the weight, so the fp32
// accumulation error stays relative to sum |w * y| even when the bias is much
// larger than the decoded values.
template <int BITS, int VEC>
__device__ __forceinline__ void accumulate(float* acc, const CodeChunk<BITS, VEC>& c, float w,
                                           float sf, float bf) {
#pragma unroll
  for (int d = 0; d < VEC / 4; ++d) {
    const uint32_t wd = c.dw(d);
    if (BITS == 4) {
      const uint32_t lo = wd & 0x0f0f0f0fu;         // elements 0, 2, 4, 6 of this dword
      const uint32_t hi = (wd >> 4) & 0x0f0f0f0fu;  // elements 1, 3, 5, 7
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float y0 = __builtin_fmaf(sf, (float)((lo >> (8 * b)) & 255u), bf);
        const float y1 = __builtin_fmaf(sf, (float)((hi >> (8 * b)) & 255u), bf);
        acc[8 * d + 2 * b] = __builtin_fmaf(w, y0, acc[8 * d + 2 * b]);
        acc[8 * d + 2 * b + 1] = __builtin_fmaf(w, y1, acc[8 * d + 2 * b + 1]);
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float y = __builtin_fmaf(sf, (float)((wd >> (8 * b)) & 255u), bf);
        acc[4 * d + b] = __builtin_fmaf(w, y, acc[4 * d + b]);
      }
    }
  }
}

template <int BITS, int VEC, int LPR, int RG, int U>
__global__ __launch_bounds__(kBlock) void bag_kernel(
    const uint8_t* __restrict__ packed, int64_t S, int64_t total_rows,
    const int64_t* __restrict__ table_offsets, int T, int64_t B, int dim, int C,
    const void* __restrict__ indices, const void* __restrict__ offsets, int idx64, int64_t nnz,
    const float* __restrict__ weights, float* __restrict__ out, int32_t* __restrict__ err_count,
    int64_t n_bags, int vec4) {
  constexpr int EPL = VEC * 8 / BITS;
  constexpr int SLICE = LPR * RG;
  const int lane = threadIdx.x & (kWave - 1);
  const int sl = lane % SLICE;
  const int g = sl / LPR;
  const int s = sl % LPR;
  const int64_t bag = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / SLICE;
  if (bag >= n_bags) return;  // whole slices leave together
  const int64_t t = bag / B;
  const int64_t b = bag - t * B;
  int errs = 0;
  int64_t p0 = load_index(offsets, bag, idx64);
  int64_t p1 = load_index(offsets, bag + 1, idx64);
  if (!(p0 >= 0 && p1 >= p0 && p1 <= nnz)) {
    errs += (sl == 0);
    p0 = p1 = 0;
  }
  const int64_t t0 = table_offsets[t], t1 = table_offsets[t + 1];
  const bool table_ok = t0 >= 0 && t1 >= t0 && t1 <= total_rows;
  const int64_t n_t = table_ok ? t1 - t0 : 0;
  const bool has_codes = s * VEC < C;
  const uint8_t* tbase = packed + (table_ok ? t0 : 0) * S + s * VEC;
  const uint8_t* pbase = packed + (table_ok ? t0 : 0) * S;

  float acc[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) acc[k] = 0.0f;

  for (int64_t base = p0; base < p1; base += RG * U) {
    int64_t id[U];
    float w[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = base + u * RG + g;
      const bool in = p < p1;
      id[u] = in ? load_index(indices, p, idx64) : 0;
      w[u] = in ? (weights ? weights[p] : 1.0f) : 0.0f;
      ok[u] = in && id[u] >= 0 && id[u] < n_t;
      errs += (in && !ok[u] && s == 0);
    }
    CodeChunk<BITS, VEC> cc[U];
    uint32_t pr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ok[u] && has_codes) {
        cc[u].load(tbase + id[u] * S);
      } else {
        cc[u].zero();
      }
      pr[u] = ok[u] ? load_params(pbase + id[u] * S, C) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      accumulate<BITS, VEC>(acc, cc[u], w[u], half_value(pr[u]), half_value(pr[u] >> 16));
    }
  }

#pragma unroll
  for (int m = LPR; m < SLICE; m <<= 1) {
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[k] += __shfl_xor(acc[k], m);
  }

  if (g == 0) {
    float* o = out + (b * T + t) * (int64_t)dim;
    const int e0 = s * EPL;
    if (vec4 && e0 + EPL <= dim) {
#pragma unroll
      for (int k = 0; k < EPL; k += 4)
        *reinterpret_cast<float4*>(o + e0 + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
    } else {
#pragma unroll
      for (int k = 0; k < EPL; ++k)
        if (e0 + k < dim) o[e0 + k] = acc[k];
    }
  }
  if (errs && err_count) atomicAdd(err_count, errs);
}

// ---------------------------------------------------------------------------
// normalized l2 error: one thread per row, fixed grid, fixed reduction order
// ---------------------------------------------------------------------------

constexpr int kL2Blocks = 1024;

__device__ __forceinline__ void block_sum4(double (&a)[4], double* sh) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < 4; ++c) sh[c * kBlock + tid] = a[c];
  __syncthreads();
  for (int h = kBlock / 2; h > 0; h >>= 1) {
    if (tid < h) {
#pragma unroll
      for (int c = 0; c < 4; ++c) sh[c * kBlock + tid] += sh[c * kBlock + tid + h];
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBlock) void l2_partial_kernel(const float* __restrict__ x,
                                                            const uint8_t* __restrict__ packed,
                                                            int64_t rows, int dim, int bits, int C,
                                                            int S, double* __restrict__ part) {
  __shared__ double sh[4 * kBlock];
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  for (int64_t row = (int64_t)blockIdx.x * kBlock + threadIdx.x; row < rows;
       row += (int64_t)gridDim.x * kBlock) {
    const float* xr = x + row * dim;
    const uint8_t* prow = packed + row * (int64_t)S;
    const uint32_t p = load_params(prow, C);
    const float sf = half_value(p), bf = half_value(p >> 16);
    double e2 = 0.0, x2 = 0.0;
    for (int k = 0; k < dim; ++k) {
      uint32_t q = bits == 8 ? prow[k] : ((prow[k >> 1] >> ((k & 1) * 4)) & 15u);
      const double yk = (double)__builtin_fmaf(sf, (float)q, bf);
      const double xk = (double)xr[k];
      const double e = xk - yk;
      e2 += e * e;
      x2 += xk * xk;
    }
    a[2] += e2;
    a[3] += x2;
    if (x2 > 0.0) {
      a[0] += sqrt(e2) / sqrt(x2);
      a[1] += 1.0;
    }
  }
  block_sum4(a, sh);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) part[4 * blockIdx.x + c] = sh[c * kBlock];
  }
}

__global__ __launch_bounds__(kBlock) void l2_final_kernel(const double* __restrict__ part,
                                                          double* __restrict__ out4) {
  __shared__ double sh[4 * kBlock];
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  for (int k = threadIdx.x; k < kL2Blocks; k += kBlock) {
#pragma unroll
    for (int c = 0; c < 4; ++c) a[c] += part[4 * k + c];
  }
  block_sum4(a, sh);
  if (threadIdx.x == 0) {
    const double n = sh[kBlock];
    out4[0] = n > 0.0 ? sh[0] / n : 0.0;
    out4[1] = n;
    out4[2] = sh[2 * kBlock];
    out4[3] = sh[3 * kBlock];
  }
}

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------

inline int64_t code_bytes(int dim, int bits) { return ((int64_t)dim * bits + 7) / 8; }

inline int next_pow2(int64_t v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int launched() { return hipGetLastError() == hipSuccess ? QEMB_OK : QEMB_E_LAUNCH; }

inline unsigned grid_for(int64_t items, int per_block, int64_t cap) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (unsigned)g;
}

constexpr int64_t kGridCap = 1 << 20;

template <int BITS, int LPR, int NCH>
int launch_range(const float* x, int64_t rows, int dim, int C, int S, int vec4, uint8_t* packed,
                 hipStream_t st) {
  hipLaunchKernelGGL((quantize_range_kernel<BITS, LPR, NCH>),
                     dim3(grid_for(rows, kBlock / LPR, kGridCap)), dim3(kBlock), 0, st, x, rows,
                     dim, C, S, vec4, packed);
  return launched();
}

template <int BITS>
int dispatch_range(const float* x, int64_t rows, int dim, int C, int S, int vec4, uint8_t* packed,
                   hipStream_t st) {
  const int chunks = (dim + 7) / 8;
  const int lpr = chunks >= 64 ? 64 : next_pow2(chunks);
  const int nch = (chunks + lpr - 1) / lpr;
  switch (lpr) {
    case 1: return launch_range<BITS, 1, 1>(x, rows, dim, C, S, vec4, packed, st);
    case 2: return launch_range<BITS, 2, 1>(x, rows, dim, C, S, vec4, packed, st);
    case 4: return launch_range<BITS, 4, 1>(x, rows, dim, C, S, vec4, packed, st);
    case 8: return launch_range<BITS, 8, 1>(x, rows, dim, C, S, vec4, packed, st);
    case 16: return launch_range<BITS, 16, 1>(x, rows, dim, C, S, vec4, packed, st);
    case 32: return launch_range<BITS, 32, 1>(x, rows, dim, C, S, vec4, packed, st);
    default:
      return nch == 1 ? launch_range<BITS, 64, 1>(x, rows, dim, C, S, vec4, packed, st)
                      : launch_range<BITS, 64, 2>(x, rows, dim, C, S, vec4, packed, st);
  }
}

template <int BITS, int EPL, int LPR>
int launch_greedy(const float* x, int64_t rows, int dim, int C, int S, int vec4, int n_bins,
                  int n_steps, uint8_t* packed, hipStream_t st) {
  const unsigned grid = grid_for(rows, kBlock / LPR, kGridCap);
  if (dim == EPL * LPR) {
    hipLaunchKernelGGL((quantize_greedy_kernel<BITS, EPL, LPR, false>), dim3(grid), dim3(kBlock), 0,
                       st, x, rows, dim, C, S, vec4, n_bins, n_steps, packed);
  } else {
    hipLaunchKernelGGL((quantize_greedy_kernel<BITS, EPL, LPR, true>), dim3(grid), dim3(kBlock), 0,
                       st, x, rows, dim, C, S, vec4, n_bins, n_steps, packed);
  }
  return launched();
}

template <int BITS>
int dispatch_greedy(const float* x, int64_t rows, int dim, int C, int S, int vec4, int n_bins,
                    int n_steps, uint8_t* packed, hipStream_t st) {
  const int n = next_pow2(dim);
  switch (n) {
    case 1: return launch_greedy<BITS, 1, 1>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    case 2: return launch_greedy<BITS, 2, 1>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    case 4: return launch_greedy<BITS, 4, 1>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    case 8: return launch_greedy<BITS, 8, 1>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    case 16: return launch_greedy<BITS, 16, 1>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    case 32: return launch_greedy<BITS, 32, 1>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    case 64: return launch_greedy<BITS, 64, 1>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    case 128: return launch_greedy<BITS, 64, 2>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    case 256: return launch_greedy<BITS, 64, 4>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    case 512: return launch_greedy<BITS, 64, 8>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
    default: return launch_greedy<BITS, 64, 16>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
  }
}

template <int BITS, int LPR, int NCH>
int launch_dequant(const uint8_t* packed, int64_t rows, int dim, int C, int S, int vec4, float* y,
                   hipStream_t st) {
  hipLaunchKernelGGL((dequant_kernel<BITS, LPR, NCH>), dim3(grid_for(rows, kBlock / LPR, kGridCap)),
                     dim3(kBlock), 0, st, packed, rows, dim, C, S, vec4, y);
  return launched();
}

template <int BITS>
int dispatch_dequant(const uint8_t* packed, int64_t rows, int dim, int C, int S, int vec4, float* y,
                     hipStream_t st) {
  const int chunks = (dim + 7) / 8;
  const int lpr = chunks >= 64 ? 64 : next_pow2(chunks);
  const int nch = (chunks + lpr - 1) / lpr;
  switch (lpr) {
    case 1: return launch_dequant<BITS, 1, 1>(packed, rows, dim, C, S, vec4, y, st);
    case 2: return launch_dequant<BITS, 2, 1>(packed, rows, dim, C, S, vec4, y, st);
    case 4: return launch_dequant<BITS, 4, 1>(packed, rows, dim, C, S, vec4, y, st);
    case 8: return launch_dequant<BITS, 8, 1>(packed, rows, dim, C, S, vec4, y, st);
    case 16: return launch_dequant<BITS, 16, 1>(packed, rows, dim, C, S, vec4, y, st);
    case 32: return launch_dequant<BITS, 32, 1>(packed, rows, dim, C, S, vec4, y, st);
    default:
      return nch == 1 ? launch_dequant<BITS, 64, 1>(packed, rows, dim, C, S, vec4, y, st)
                      : launch_dequant<BITS, 64, 2>(packed, rows, dim, C, S, vec4, y, st);
  }
}

struct BagArgs {
  const uint8_t* packed;
  int64_t S, total_rows;
  const int64_t* table_offsets;
  int T;
  int64_t B;
  int dim, C;
  const void* indices;
  const void* offsets;
  int idx64;
  int64_t nnz;
  const float* weights;
  float* out;
  int32_t* err_count;
  int64_t n_bags;
  int vec4;
};

constexpr int kBagUnroll = 4;

template <int BITS, int VEC, int LPR, int RG>
int launch_bag(const BagArgs& a, hipStream_t st) {
  constexpr int SLICE = LPR * RG;
  const int64_t threads = a.n_bags * SLICE;
  const int64_t blocks = (threads + kBlock - 1) / kBlock;
  if (blocks > 0x7fffffff) return QEMB_E_UNSUPPORTED;
  hipLaunchKernelGGL((bag_kernel<BITS, VEC, LPR, RG, kBagUnroll>), dim3((unsigned)blocks),
                     dim3(kBlock), 0, st, a.packed, a.S, a.total_rows, a.table_offsets, a.T, a.B,
                     a.dim, a.C, a.indices, a.offsets, a.idx64, a.nnz, a.weights, a.out,
                     a.err_count, a.n_bags, a.vec4);
  return launched();
}

template <int BITS, int VEC, int LPR>
int dispatch_bag_rg(const BagArgs& a, int rg, hipStream_t st) {
  constexpr int MAXRG = (64 / LPR) < 16 ? (64 / LPR) : 16;
  if (rg > MAXRG) rg = MAXRG;
  switch (rg) {
    case 1: return launch_bag<BITS, VEC, LPR, 1>(a, st);
    case 2: return launch_bag<BITS, VEC, LPR, (2 <= MAXRG ? 2 : 1)>(a, st);
    case 4: return launch_bag<BITS, VEC, LPR, (4 <= MAXRG ? 4 : 1)>(a, st);
    case 8: return launch_bag<BITS, VEC, LPR, (8 <= MAXRG ? 8 : 1)>(a, st);
    default: return launch_bag<BITS, VEC, LPR, (16 <= MAXRG ? 16 : 1)>(a, st);
  }
}

template <int BITS, int VEC>
int dispatch_bag_lpr(const BagArgs& a, int lpr, int rg, hipStream_t st) {
  switch (lpr) {
    case 1: return dispatch_bag_rg<BITS, VEC, 1>(a, rg, st);
    case 2: return dispatch_bag_rg<BITS, VEC, 2>(a, rg, st);
    case 4: return dispatch_bag_rg<BITS, VEC, 4>(a, rg, st);
    case 8: return dispatch_bag_rg<BITS, VEC, 8>(a, rg, st);
    case 16: return dispatch_bag_rg<BITS, VEC, 16>(a, rg, st);
    case 32: return dispatch_bag_rg<BITS, VEC, 32>(a, rg, st);
    default: return dispatch_bag_rg<BITS, VEC, 64>(a, rg, st);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int qemb_abi_version(void) { return QEMB_ABI_VERSION; }

const char* qemb_strerror(int code) {
  switch (code) {
    case QEMB_OK: return "ok";
    case QEMB_E_INVALID_ARG: return "invalid argument";
    case QEMB_E_MISALIGNED: return "array not 16-byte aligned";
    case QEMB_E_UNSUPPORTED: return "unsupported size";
    case QEMB_E_LAUNCH: return "kernel launch failed";
    default: return "unknown error";
  }
}

int64_t qemb_row_stride(int32_t dim, int32_t bits) {
  if (dim < 1 || dim > QEMB_MAX_DIM || (bits != 4 && bits != 8)) return -1;
  return (code_bytes(dim, bits) + 4 + 15) / 16 * 16;
}

int qemb_quantize_rowwise(const float* x, int64_t rows, int32_t dim, int32_t bits,
                          int32_t clip_mode, int32_t n_bins, int32_t n_steps, uint8_t* packed,
                          qemb_stream_t stream) {
  if (rows < 0 || dim < 1 || (bits != 4 && bits != 8)) return QEMB_E_INVALID_ARG;
  if (clip_mode != QEMB_CLIP_RANGE && clip_mode != QEMB_CLIP_GREEDY) return QEMB_E_INVALID_ARG;
  if (clip_mode == QEMB_CLIP_GREEDY && (n_bins < 1 || n_steps < 0 || n_steps >= n_bins))
    return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (rows == 0) return QEMB_OK;
  if (!x || !packed) return QEMB_E_INVALID_ARG;
  if (!aligned16(x) || !aligned16(packed)) return QEMB_E_MISALIGNED;
  const int C = (int)code_bytes(dim, bits);
  const int S = (int)qemb_row_stride(dim, bits);
  const int vec4 = (dim % 4 == 0);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (clip_mode == QEMB_CLIP_RANGE) {
    return bits == 4 ? dispatch_range<4>(x, rows, dim, C, S, vec4, packed, st)
                     : dispatch_range<8>(x, rows, dim, C, S, vec4, packed, st);
  }
  return bits == 4 ? dispatch_greedy<4>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st)
                   : dispatch_greedy<8>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
}

int qemb_dequantize(const uint8_t* packed, int64_t rows, int32_t dim, int32_t bits, float* y,
                    qemb_stream_t stream) {
  if (rows < 0 || dim < 1 || (bits != 4 && bits != 8)) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (rows == 0) return QEMB_OK;
  if (!packed || !y) return QEMB_E_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(y)) return QEMB_E_MISALIGNED;
  const int C = (int)code_bytes(dim, bits);
  const int S = (int)qemb_row_stride(dim, bits);
  const int vec4 = (dim % 4 == 0);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return bits == 4 ? dispatch_dequant<4>(packed, rows, dim, C, S, vec4, y, st)
                   : dispatch_dequant<8>(packed, rows, dim, C, S, vec4, y, st);
}

int qemb_bag_forward(const uint8_t* packed, int64_t total_rows, const int64_t* table_offsets,
                     int32_t T, int64_t B, int32_t dim, int32_t bits, const void* indices,
                     const void* offsets, int64_t nnz, int32_t index_type, int32_t pool_mode,
                     const float* weights, float* out, int32_t* err_count,
                     qemb_stream_t stream) {
  if (T < 0 || B < 0 || dim < 1 || (bits != 4 && bits != 8) || total_rows < 0 || nnz < 0)
    return QEMB_E_INVALID_ARG;
  if (index_type != QEMB_INDEX_INT32 && index_type != QEMB_INDEX_INT64) return QEMB_E_INVALID_ARG;
  if (pool_mode != QEMB_POOL_SUM && pool_mode != QEMB_POOL_WEIGHTED_SUM) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (T == 0 || B == 0) return QEMB_OK;
  if (B > INT64_MAX / T) return QEMB_E_INVALID_ARG;
  if (!table_offsets || !offsets || !out) return QEMB_E_INVALID_ARG;
  if (nnz > 0 && !indices) return QEMB_E_INVALID_ARG;
  if (total_rows > 0 && !packed) return QEMB_E_INVALID_ARG;
  if (pool_mode == QEMB_POOL_WEIGHTED_SUM && nnz > 0 && !weights) return QEMB_E_INVALID_ARG;
  if ((packed && !aligned16(packed)) || !aligned16(out)) return QEMB_E_MISALIGNED;
  BagArgs a;
  a.packed = packed;
  a.S = qemb_row_stride(dim, bits);
  a.total_rows = total_rows;
  a.table_offsets = table_offsets;
  a.T = T;
  a.B = B;
  a.dim = dim;
  a.C = (int)code_bytes(dim, bits);
  a.indices = indices;
  a.offsets = offsets;
  a.idx64 = index_type == QEMB_INDEX_INT64;
  a.nnz = nnz;
  a.weights = pool_mode == QEMB_POOL_WEIGHTED_SUM ? weights : nullptr;
  a.out = out;
  a.err_count = err_count;
  a.n_bags = (int64_t)T * B;
  a.vec4 = (dim % 4 == 0);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // lanes per row: 8-byte code chunks (16-byte for INT8 rows wider than 512)
  const int64_t chunks8 = (a.C + 7) / 8;
  const int vec = chunks8 > 64 ? 16 : 8;
  const int lpr = next_pow2((a.C + vec - 1) / vec);
  // row groups per bag: about kBagUnroll rows per group for the mean bag
  const int64_t mean_len = (nnz + a.n_bags - 1) / a.n_bags;
  const int rg = next_pow2((mean_len + kBagUnroll - 1) / kBagUnroll);
  if (bits == 4) return dispatch_bag_lpr<4, 8>(a, lpr, rg, st);
  if (vec == 8) return dispatch_bag_lpr<8, 8>(a, lpr, rg, st);
  return dispatch_bag_rg<8, 16, 64>(a, rg, st);  // only rows wider than 512 codes get here
}

size_t qemb_l2_error_workspace_bytes(void) { return (size_t)kL2Blocks * 4 * sizeof(double); }

int qemb_l2_error(const float* x, const uint8_t* packed, int64_t rows, int32_t dim, int32_t bits,
                  void* workspace, double* out4, qemb_stream_t stream) {
  if (rows < 0 || dim < 1 || (bits != 4 && bits != 8)) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (!workspace || !out4 || (rows > 0 && (!x || !packed))) return QEMB_E_INVALID_ARG;
  if ((x && !aligned16(x)) || (packed && !aligned16(packed)) || !aligned16(workspace))
    return QEMB_E_MISALIGNED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  double* part = reinterpret_cast<double*>(workspace);
  hipLaunchKernelGGL(l2_partial_kernel, dim3(kL2Blocks), dim3(kBlock), 0, st, x, packed, rows, dim,
                     bits, (int)code_bytes(dim, bits), (int)qemb_row_stride(dim, bits), part);
  if (launched() != QEMB_OK) return QEMB_E_LAUNCH;
  hipLaunchKernelGGL(l2_final_kernel, dim3(1), dim3(kBlock), 0, st, part, out4);
  return launched();
}

}  // extern "C"
