// qemb.hip -- row-wise INT4/INT8 quantized embedding tables on gfx950.
//
// Kernels and the C ABI declared in include/qemb.h:
//   * quantize_range_kernel   row range -> fp16 scale/bias -> codes -> packed row
//   * quantize_greedy_kernel  greedy clip search on the row's squared error,
//                             then the same encoding
//   * dequant_kernel          packed rows -> fp32
//   * bag_stream_kernel       fused decode + (weighted) sum pooling of multi-hot
//                             bags, pipelined over batches of ids
//   * bag_wave_kernel         the same for rows wider than 8 lanes
//   * bag_slice_kernel        the same for short bags, several bags per wave
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

#include <type_traits>

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

// Load the 4 parameter bytes at byte C of a 16-byte aligned row of stride S
// bytes.  Both dwords are loaded unconditionally (the second address is
// clamped inside the row; alignbyte by 0 keeps the first), so no branch sits
// between a load and its use and the loads of many rows stay in flight.
__device__ __forceinline__ uint32_t load_params(const uint8_t* row, int C, int S) {
  const int c4 = C & ~3;
  const uint32_t lo = *reinterpret_cast<const uint32_t*>(row + c4);
  const uint32_t hi = *reinterpret_cast<const uint32_t*>(row + (c4 + 4 < S ? c4 + 4 : S - 4));
  return __builtin_amdgcn_alignbyte(hi, lo, (uint32_t)(C & 3));
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

template <typename IdxT>
__device__ __forceinline__ int64_t load_index(const void* p, int64_t k) {
  return (int64_t) reinterpret_cast<const IdxT*>(p)[k];
}

// ---------------------------------------------------------------------------
// decode + accumulate.  A code placed in the low bits of a binary16 half is
// the denormal code * 2^-24, so v_fma_mix_f32(scale * 2^24, half, bias) is
// fmaf(scale, code, bias) with the same single rounding and no int->float
// conversion; unpacking 8 nibbles into such halves takes 7 ALU ops.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float h16(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}

// sfs = scale * 2^24 (exact), bf = bias; y_k = fmaf(scale, code_k, bias)
template <int BITS>
__device__ __forceinline__ void decode_dword(uint32_t wd, float sfs, float bf, float (&y)[32 / BITS]) {
  if (BITS == 4) {
    const uint32_t r04 = wd & 0x000f000fu;
    const uint32_t r15 = (wd >> 4) & 0x000f000fu;
    const uint32_t r26 = (wd >> 8) & 0x000f000fu;
    const uint32_t r37 = (wd >> 12) & 0x000f000fu;
    y[0] = __builtin_fmaf(sfs, h16(r04), bf);
    y[1] = __builtin_fmaf(sfs, h16(r15), bf);
    y[2] = __builtin_fmaf(sfs, h16(r26), bf);
    y[3] = __builtin_fmaf(sfs, h16(r37), bf);
    y[4] = __builtin_fmaf(sfs, h16(r04 >> 16), bf);
    y[5] = __builtin_fmaf(sfs, h16(r15 >> 16), bf);
    y[6] = __builtin_fmaf(sfs, h16(r26 >> 16), bf);
    y[7] = __builtin_fmaf(sfs, h16(r37 >> 16), bf);
  } else {
    const uint32_t r02 = wd & 0x00ff00ffu;
    const uint32_t r13 = (wd >> 8) & 0x00ff00ffu;
    y[0] = __builtin_fmaf(sfs, h16(r02), bf);
    y[1] = __builtin_fmaf(sfs, h16(r13), bf);
    y[2] = __builtin_fmaf(sfs, h16(r02 >> 16), bf);
    y[3] = __builtin_fmaf(sfs, h16(r13 >> 16), bf);
  }
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
    const uint32_t p = load_params(prow, C, S);
    const float sfs = half_value(p) * 16777216.0f, bf = half_value(p >> 16);
    float* yr = y + row * dim;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = (c * LPR + s) * EPL;
      if (e0 >= dim) break;
      float o[EPL];
      if (BITS == 2) {
        // 8 two-bit codes in 2 bytes; a code under a binary16 zero exponent
        // reads as code * 2^-24, as in decode_dword
        const uint32_t wd = *reinterpret_cast<const uint16_t*>(prow + e0 / 4);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = __builtin_fmaf(sfs, h16((wd >> (2 * k)) & 3u), bf);
      } else if (BITS == 4) {
        float yk[8];
        decode_dword<4>(*reinterpret_cast<const uint32_t*>(prow + e0 / 2), sfs, bf, yk);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = yk[k];
      } else {
        const uint2 wd = *reinterpret_cast<const uint2*>(prow + e0);
        float y0[4], y1[4];
        decode_dword<8>(wd.x, sfs, bf, y0);
        decode_dword<8>(wd.y, sfs, bf, y1);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o[k] = y0[k];
          o[k + 4] = y1[k];
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
// pooled lookup
//
// acc[k] += w * fmaf(sf, code_k, bf): each term is the decoded value (one
// rounding, as a standalone decode gives) times the weight, so the fp32
// accumulation error stays relative to sum |w * y| even when the bias is much
// larger than the decoded values.
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

template <int BITS, int VEC, bool INIT = false>
__device__ __forceinline__ void accumulate(float* acc, const CodeChunk<BITS, VEC>& c, float w,
                                           uint32_t prm) {
  constexpr int PER = 32 / BITS;  // elements per dword
  const float sfs = h16(prm) * 16777216.0f;
  const float bf = h16(prm >> 16);
#pragma unroll
  for (int d = 0; d < VEC / 4; ++d) {
    float y[PER];
    decode_dword<BITS>(c.dw(d), sfs, bf, y);
#pragma unroll
    for (int k = 0; k < PER; ++k)
      acc[PER * d + k] = INIT ? w * y[k] : __builtin_fmaf(w, y[k], acc[PER * d + k]);
  }
}

// Short bags (few ids per bag): a bag is owned by a slice of LPR*RG lanes,
// RG row groups of LPR lanes; lane (g, s) reads VEC code bytes at byte s*VEC
// of rows p0+g, p0+g+RG, ...  U rows per group are in flight per iteration.
// The RG partial vectors are reduced across the slice by xor shuffles.
template <int BITS, int VEC, int LPR, int RG, int U, typename IdxT>
__global__ __launch_bounds__(kBlock) void bag_slice_kernel(
    const uint8_t* __restrict__ packed, int64_t S, int64_t total_rows,
    const int64_t* __restrict__ table_offsets, int T, int64_t B, int dim, int C,
    const void* __restrict__ indices, const void* __restrict__ offsets, int64_t nnz,
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
  int64_t p0 = load_index<IdxT>(offsets, bag);
  int64_t p1 = load_index<IdxT>(offsets, bag + 1);
  if (!(p0 >= 0 && p1 >= p0 && p1 <= nnz)) {
    errs += (sl == 0);
    p0 = p1 = 0;
  }
  const int64_t t0 = table_offsets[t], t1 = table_offsets[t + 1];
  const bool table_ok = t0 >= 0 && t1 >= t0 && t1 <= total_rows;
  const int64_t n_t = table_ok ? t1 - t0 : 0;
  const bool has_codes = s * VEC < C;
  const uint8_t* tbase = packed + (table_ok ? t0 : 0) * S;

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
      id[u] = in ? load_index<IdxT>(indices, p) : 0;
      ok[u] = in && id[u] >= 0 && id[u] < n_t;
      w[u] = ok[u] ? (weights ? weights[p] : 1.0f) : 0.0f;
      errs += (in && !ok[u] && s == 0);
    }
    CodeChunk<BITS, VEC> cc[U];
    uint32_t pr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint8_t* row = tbase + id[u] * S;
      if (ok[u] && has_codes) {
        cc[u].load(row + s * VEC);
      } else {
        cc[u].zero();
      }
      pr[u] = ok[u] ? load_params(row, C, (int)S) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) accumulate<BITS, VEC>(acc, cc[u], w[u], pr[u]);
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

// Multi-hot bags: each wave walks kWave consecutive bags.  Lane i holds the
// CSR bounds of bag i of the run; for the current bag, lane L validates id L
// (64 ids at a time) once and leaves its row offset and weight in LDS, while
// the ids of the next bag are already being fetched.  The 64 lanes form
// RG = 64/LPR row groups of LPR lanes (LPR*VEC code bytes cover a row); group
// g takes rows g, g+RG, ... of the batch, with all of them (up to UMAX per
// group) in flight at once and the batch sized to the rows left.  Each lane
// accumulates EPL = 16 elements; the RG partial vectors are summed through
// LDS in a fixed order and written with coalesced stores.  Consecutive blocks
// go round-robin over the 8 XCDs, so block ids are remapped to give each XCD
// a contiguous run of bags (a few tables): each XCD's L2 then holds fewer
// tables' hot rows.
constexpr int kWPB = kBlock / kWave;
constexpr int kBagUMax = 8;

template <int BITS, int LPR>
struct WaveBag {
  static constexpr int VEC = 2 * BITS;  // bytes per lane per row: 16 codes
  static constexpr int EPL = VEC * 8 / BITS;
  static constexpr int RG = kWave / LPR;
};

// Rows j0 + u*RG + g (u < U) of the current id batch.  Every lane loads
// unconditionally: a slot without a valid row reads the table's first row
// (`safe`) at byte 0 and gets zero scale and bias, so it adds exactly 0; a
// lane whose chunk lies past the row's code bytes also reads at byte 0 (its
// elements are never stored).
template <int BITS, int LPR, int U>
__device__ __forceinline__ void wave_bag_rows(float* acc, const uint8_t* safe, int C, int S, int code_off,
                                              int g, int j0, int n, const int64_t* moff,
                                              const float* mw) {
  using W = WaveBag<BITS, LPR>;
  int64_t off[U];
  float w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int slot = j0 + u * W::RG + g;
    off[u] = slot < n ? moff[slot] : -1;
    w[u] = slot < n ? mw[slot] : 0.0f;
  }
  CodeChunk<BITS, W::VEC> cc[U];
  uint32_t pr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint8_t* row = safe + (off[u] >= 0 ? off[u] : 0);
    cc[u].load(row + (off[u] >= 0 ? code_off : 0));
    pr[u] = load_params(row, C, (int)S);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    accumulate<BITS, W::VEC>(acc, cc[u], w[u], off[u] >= 0 ? pr[u] : 0u);
}

template <int BITS, int LPR>
__device__ __forceinline__ void wave_bag_batch(float* acc, const uint8_t* safe, int C, int S, int code_off,
                                               int g, int n, const int64_t* moff, const float* mw) {
  constexpr int RG = WaveBag<BITS, LPR>::RG;
  for (int j0 = 0; j0 < n; j0 += kBagUMax * RG) {
    const int u = (n - j0 + RG - 1) / RG;
    switch (u < kBagUMax ? u : kBagUMax) {
      case 1: wave_bag_rows<BITS, LPR, 1>(acc, safe, C, S, code_off, g, j0, n, moff, mw); break;
      case 2: wave_bag_rows<BITS, LPR, 2>(acc, safe, C, S, code_off, g, j0, n, moff, mw); break;
      case 3: wave_bag_rows<BITS, LPR, 3>(acc, safe, C, S, code_off, g, j0, n, moff, mw); break;
      case 4: wave_bag_rows<BITS, LPR, 4>(acc, safe, C, S, code_off, g, j0, n, moff, mw); break;
      case 5: wave_bag_rows<BITS, LPR, 5>(acc, safe, C, S, code_off, g, j0, n, moff, mw); break;
      case 6: wave_bag_rows<BITS, LPR, 6>(acc, safe, C, S, code_off, g, j0, n, moff, mw); break;
      case 7: wave_bag_rows<BITS, LPR, 7>(acc, safe, C, S, code_off, g, j0, n, moff, mw); break;
      default: wave_bag_rows<BITS, LPR, 8>(acc, safe, C, S, code_off, g, j0, n, moff, mw); break;
    }
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int64_t lane_i64(int64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), lane);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <int BITS, int LPR, typename IdxT>
__global__ __launch_bounds__(kBlock) void bag_wave_kernel(
    const uint8_t* __restrict__ packed, int64_t S, int64_t total_rows,
    const int64_t* __restrict__ table_offsets, int T, int64_t B, int dim, int C,
    const void* __restrict__ indices, const void* __restrict__ offsets, int64_t nnz,
    const float* __restrict__ weights, float* __restrict__ out, int32_t* __restrict__ err_count,
    int64_t n_bags) {
  using W = WaveBag<BITS, LPR>;
  constexpr int EPL = W::EPL, RG = W::RG;
  __shared__ int64_t meta_off[kWPB][kWave];
  __shared__ float meta_w[kWPB][kWave];
  __shared__ float red[RG > 1 ? kWPB : 1][RG > 1 ? kWave * EPL : 1];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane / LPR, s = lane % LPR;
  // XCD-aware block order (a bijection on [0, gridDim.x))
  const int64_t nbk = gridDim.x, x = blockIdx.x % 8, k = blockIdx.x / 8;
  const int64_t qf = nbk / 8, r = nbk % 8;
  const int64_t blk = x * qf + (x < r ? x : r) + k;
  const int64_t bag0 = (blk * kWPB + wv) * kWave;
  if (bag0 >= n_bags) return;  // whole waves leave together
  const int nb = (int)((n_bags - bag0) < kWave ? (n_bags - bag0) : kWave);
  int errs = 0;

  // CSR bounds of the run's bags, one bag per lane; bad bounds -> empty bag
  int64_t lp0 = 0, lp1 = 0;
  if (lane < nb) {
    lp0 = load_index<IdxT>(offsets, bag0 + lane);
    lp1 = load_index<IdxT>(offsets, bag0 + lane + 1);
    if (!(lp0 >= 0 && lp1 >= lp0 && lp1 <= nnz)) {
      errs += 1;
      lp0 = lp1 = 0;
    }
  }
  const int code_off = s * W::VEC < C ? s * W::VEC : 0;
  int64_t* moff = meta_off[wv];
  float* mw = meta_w[wv];

  // table of the current bag (bags are table-major)
  int64_t t = bag0 / B;
  int64_t t_end = (t + 1) * B;  // first bag of the next table
  int64_t t0 = 0, n_t = 0;
  const uint8_t* tbase = packed;
  auto enter_table = [&](int64_t tt) {
    const int64_t a0 = table_offsets[tt], a1 = table_offsets[tt + 1];
    const bool ok = a0 >= 0 && a1 >= a0 && a1 <= total_rows;
    t0 = ok ? a0 : 0;
    n_t = ok ? a1 - a0 : 0;
    tbase = packed + t0 * S;
  };
  enter_table(t);

  // first id batch of bag 0
  int64_t p0 = lane_i64(lp0, 0), p1 = lane_i64(lp1, 0);
  int64_t nid = 0;
  float nw = 0.0f;
  if (lane < p1 - p0) {
    nid = load_index<IdxT>(indices, p0 + lane);
    nw = weights ? weights[p0 + lane] : 1.0f;
  }

  for (int i = 0; i < nb; ++i) {
    const int64_t bag = bag0 + i;
    if (bag >= t_end) {
      t = bag / B;
      t_end = (t + 1) * B;
      enter_table(t);
    }
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    // this bag's first id batch was prefetched; start fetching the next
    // bag's (also when this bag is empty)
    const int64_t fid = nid;
    const float fw = nw;
    if (i + 1 < nb) {
      const int64_t q0 = lane_i64(lp0, i + 1), q1 = lane_i64(lp1, i + 1);
      nid = 0;
      nw = 0.0f;
      if (lane < q1 - q0) {
        nid = load_index<IdxT>(indices, q0 + lane);
        nw = weights ? weights[q0 + lane] : 1.0f;
      }
    }
    for (int64_t c0 = p0; c0 < p1; c0 += kWave) {
      const int n = (int)((p1 - c0) < kWave ? (p1 - c0) : kWave);
      int64_t id = fid;
      float wl = fw;
      if (c0 != p0 && lane < n) {
        id = load_index<IdxT>(indices, c0 + lane);
        wl = weights ? weights[c0 + lane] : 1.0f;
      }
      int64_t off = -1;
      if (lane < n) {
        if (id >= 0 && id < n_t) {
          off = id * S;
        } else {
          errs += 1;
          wl = 0.0f;
        }
      }
      moff[lane] = off;
      mw[lane] = wl;
      wave_sync_lds();
      if (n_t > 0) wave_bag_batch<BITS, LPR>(acc, tbase, C, (int)S, code_off, g, n, moff, mw);
      wave_sync_lds();  // the next batch overwrites the metadata
    }
    if (i + 1 < nb) {
      p0 = lane_i64(lp0, i + 1);
      p1 = lane_i64(lp1, i + 1);
    }

    const int64_t b = bag - t * B;
    float* o = out + (b * T + t) * (int64_t)dim;
    if (RG > 1) {
      float* rw = red[RG > 1 ? wv : 0];
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(rw + g * (LPR * EPL) + s * EPL + e) =
            make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
      wave_sync_lds();
      for (int e = lane; e < dim; e += kWave) {
        float v = rw[e];
#pragma unroll
        for (int gg = 1; gg < RG; ++gg) v += rw[gg * (LPR * EPL) + e];
        o[e] = v;
      }
      wave_sync_lds();
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        if (s * EPL + e < dim) o[s * EPL + e] = acc[e];
    }
  }
  if (errs && err_count) atomicAdd(err_count, errs);
}

// v_permlane32_swap_b32 / v_permlane16_swap_b32: exchange lanes 32..63 of a
// with lanes 0..31 of b (resp. the odd 16-lane rows of a with the even rows
// of b).  Written as two-operand asm with both registers read-write: this
// compiler's two-result builtins for these instructions drop the second
// result (it reuses the first), so the builtins are not used.  The compiler
// inserts no wait states before inline asm, and on gfx950 these swaps read
// their operands wrongly within 2 wait states of a VALU write to them (4 of
// a v_cmpx write to exec), so each swap starts with s_nop 3 (4 wait states).
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 3\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm volatile("s_nop 3\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Sum 16 partial elements over the 8 row groups of a wave whose lanes are
// (group g = lane bits 3..5, chunk s = bits 0..2), halving the elements kept
// at each step: bit 5 by permlane32_swap, bit 4 by permlane16_swap, bit 3 by
// a DPP row rotation by 8.  Afterwards lane L holds the sums of elements
// s*16 + b5*8 + b4*4 + b3*2 + {0, 1} (b = lane bits) in r0, r1.
__device__ __forceinline__ void reduce_scatter_g8(float (&acc)[16], int lane, float& r0, float& r1) {
  // in place: acc is consumed
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    permlane32_swap(acc[k], acc[k + 8]);
    acc[k] += acc[k + 8];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    permlane16_swap(acc[k], acc[k + 4]);
    acc[k] += acc[k + 4];
  }
  const bool h3 = (lane >> 3) & 1;
  const float k0 = h3 ? acc[2] : acc[0], k1 = h3 ? acc[3] : acc[1];  // kept
  const float s0 = h3 ? acc[0] : acc[2], s1 = h3 ? acc[1] : acc[3];  // sent to lane ^ 8
  r0 = k0 + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                          0, __builtin_bit_cast(int, s0), 0x128, 0xf, 0xf, false));
  r1 = k1 + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                          0, __builtin_bit_cast(int, s1), 0x128, 0xf, 0xf, false));
}

// Multi-hot bags of narrow rows (LPR <= 8): each wave streams the ids of a
// run of 64 consecutive bags as a sequence of batches of up to BATCH ids
// (BATCH = RG row groups x SLOTS rows per lane, at most 64).  A bag is one or
// more batches (an empty bag is one empty batch), so long bags need no
// special path.  The batch stream is software pipelined DEPTH batches deep:
// while batch k is decoded, the rows of batches k+1 .. k+DEPTH are loading
// into rotating register buffers and the ids of batch k+DEPTH+1 are being
// fetched.  A bag's accumulators carry across its batches; at its last batch
// the RG partial vectors are summed and stored.  All batch bookkeeping
// (positions, bag and table cursors, flags) is wave-uniform and lives in
// scalar registers.
//
// Lane L of a batch owns id L: it validates it, computes the row's byte
// offset, and loads the row's scale/bias dword; the lanes that read row L's
// codes (and later decode them) get the offset, the weight and the scale/bias
// from lane L by ds_bpermute.
//
// The vector-memory counter completes in issue order, so a use can wait for
// exactly the loads it needs only if the number of loads issued after them
// is fixed.  Every step therefore issues the same loads in straight-line
// code: the next batch's ids (and weights) through a buffer descriptor that
// spans exactly that batch (lanes past it read 0), then the scale/bias dword
// and all SLOTS row slots.  The ids go out before the rows, so waiting for
// them (next step) does not wait for the rows still in flight.  No loaded
// value is used inside a branch.
//
// Rows are read through a buffer descriptor of the batch's table with 32-bit
// byte offsets; a slot without a valid row gets an offset past the
// descriptor's range, so the hardware returns zero codes and zero scale and
// bias.  Tables of 2 GB or more use 64-bit addresses instead (such a slot
// reads the table's first row).  Either way a lane whose id is not a valid
// row has weight 0 and its scale/bias is replaced by 0 before it is handed
// out, so the row adds exactly 0.  PA4: the scale/bias starts on a 4-byte
// boundary (one dword), else two dwords are merged.
// A wave-uniform condition from a 64-bit signed comparison (evaluated by the
// VALU into VCC), turned into a 0/1 integer in an SGPR that the compiler
// cannot see through.  Used where such a condition feeds scalar selects: this
// compiler has emitted s_cselect on a stale SCC for them (after dropping the
// s_and of VCC with EXEC that sets SCC) in unrolled copies of the loop.
__device__ __forceinline__ bool uniform_flag(bool c) {
  int v = __builtin_amdgcn_readfirstlane(c ? 1 : 0);
  asm volatile("" : "+s"(v));
  return v != 0;
}

template <int BITS, int LPR>
struct StreamGeo {
  static constexpr int RG = kWave / LPR;
  static constexpr int SLOTS = LPR;          // RG * SLOTS = 64 ids per batch
  static constexpr int BATCH = RG * SLOTS;
  static constexpr int VEC = WaveBag<BITS, LPR>::VEC;
  static constexpr int EPL = WaveBag<BITS, LPR>::EPL;
  // batches whose rows are in flight beyond the one being decoded (64-id
  // batches: one more batch keeps about 2x32 rows per wave in flight; deeper
  // rings cost registers, hence occupancy, and measured no faster)
  static constexpr int DEPTH = 1;
};

// PX: each lane's slot load also takes the 4 bytes after its codes, which in
// a row's last lane are the row's scale and bias (rows whose codes fill the
// LPR lanes exactly and end on a 4-byte boundary).  Otherwise lane L loads
// the scale/bias of batch row L itself, one dword from each of 64 rows.
template <int BITS, int LPR, bool PA4, bool PX>
struct StreamRows {
  CodeChunk<BITS, StreamGeo<BITS, LPR>::VEC> cc[StreamGeo<BITS, LPR>::SLOTS];
  uint32_t px[PX ? StreamGeo<BITS, LPR>::SLOTS : 1];  // PX: the dword after each lane's codes
  uint32_t plo, phi;  // not PX: scale/bias dword(s) of batch row `lane`
  float w;            // weight of batch row `lane` (0 without a valid row)
};

// Centered decode.  A row's decoded values are y = bf + sf*q.  With m the
// code nearest the row's zero crossing (clamped to [0, Q]) and
// c = fma(sf, m, bf), y = c + sf*(q - m), and |c| <= |y| for every code of the
// row (either c is the value of code m itself, at most sf/2 from zero, or the
// whole row lies on one side of zero and c is its value nearest zero), while
// |sf*(q - m)| <= |y| + |c| <= 2|y|.  A bag's pooled element is accumulated
// as sum_r fl(w_r sf_r)*(q - m_r) per element plus sum_r fl(w_r c_r) once per
// bag, so every summed quantity is bounded by 2|w y| and the fp32 rounding
// error stays a small multiple of eps * sum|w y| -- the bound the direct form
// sum fl(w * fl(bf + sf*q)) has -- while the per-element work drops to one
// v_fma_mix (fp32 ws times an fp16 integer) plus the unpack.
//
// Unpack: a code k placed in the low mantissa bits of fp16 0x6400 reads as
// 1024 + k; one packed fp16 add of -(1024 + m) (-(1024 + 16 m) for a code in
// bits 4..7, which reads as 1024 + 16k) leaves k - m (16(k - m)) exactly, two
// elements per instruction.  The 16(k - m) halves are scaled by ws/16, which
// is exact, so every element's product is ws*(k - m) exactly before the one
// rounding of its fma.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

// The masks and the 0x64006400 pattern are passed in registers (UnpackK):
// with both as literals the compiler splits each v_and_or_b32 in two.
struct UnpackK {
  uint32_t m_lo, m_hi, m_byte, one;
};

template <int BITS, int VEC, bool INIT = false>
__device__ __forceinline__ void accumulate_centered(float* acc, const CodeChunk<BITS, VEC>& c, float ws,
                                                    uint32_t nlo, uint32_t nhi, const UnpackK& K) {
  const half2v hlo = as_h2(nlo);
#pragma unroll
  for (int d = 0; d < VEC / 4; ++d) {
    const uint32_t x = c.dw(d), x8 = x >> 8;
    if constexpr (BITS == 4) {
      const half2v hhi = as_h2(nhi);
      const float ws16 = ws * 0.0625f;
      const half2v a = as_h2((x & K.m_lo) | K.one) + hlo;   // elements 0, 4
      const half2v b = as_h2((x & K.m_hi) | K.one) + hhi;   // 1, 5 (x16)
      const half2v e = as_h2((x8 & K.m_lo) | K.one) + hlo;  // 2, 6
      const half2v f = as_h2((x8 & K.m_hi) | K.one) + hhi;  // 3, 7 (x16)
      float* o = acc + 8 * d;
      o[0] = __builtin_fmaf(ws, (float)a.x, INIT ? 0.0f : o[0]);
      o[1] = __builtin_fmaf(ws16, (float)b.x, INIT ? 0.0f : o[1]);
      o[2] = __builtin_fmaf(ws, (float)e.x, INIT ? 0.0f : o[2]);
      o[3] = __builtin_fmaf(ws16, (float)f.x, INIT ? 0.0f : o[3]);
      o[4] = __builtin_fmaf(ws, (float)a.y, INIT ? 0.0f : o[4]);
      o[5] = __builtin_fmaf(ws16, (float)b.y, INIT ? 0.0f : o[5]);
      o[6] = __builtin_fmaf(ws, (float)e.y, INIT ? 0.0f : o[6]);
      o[7] = __builtin_fmaf(ws16, (float)f.y, INIT ? 0.0f : o[7]);
    } else {
      const half2v a = as_h2((x & K.m_byte) | K.one) + hlo;   // elements 0, 2
      const half2v b = as_h2((x8 & K.m_byte) | K.one) + hlo;  // 1, 3
      float* o = acc + 4 * d;
      o[0] = __builtin_fmaf(ws, (float)a.x, INIT ? 0.0f : o[0]);
      o[1] = __builtin_fmaf(ws, (float)b.x, INIT ? 0.0f : o[1]);
      o[2] = __builtin_fmaf(ws, (float)a.y, INIT ? 0.0f : o[2]);
      o[3] = __builtin_fmaf(ws, (float)b.y, INIT ? 0.0f : o[3]);
    }
  }
}

// Sum of v over the 64 lanes of the wave, in every lane: DPP within each
// 16-lane row, then the permlane swaps across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xf, 0xf, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  float a = v, b = v;
  permlane32_swap(a, b);
  v = a + b;
  a = v;
  b = v;
  permlane16_swap(a, b);
  return a + b;
}

constexpr uint32_t kBufLimit = 0x7fffff00u;  // tables below this many bytes use descriptors
constexpr uint32_t kBufOut = 0x80000000u;    // offset of a slot without a row (out of range)
constexpr int kBufWord3 = 0x00020000;        // gfx9 raw-buffer descriptor word 3

__device__ __forceinline__ uint32_t bperm(int addr, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v);
}

template <int BITS, int LPR, typename IdxT, bool PA4, bool WEIGHTED, bool PX>
__global__ __launch_bounds__(kBlock) void bag_stream_kernel(
    const uint8_t* __restrict__ packed, int64_t S, int64_t total_rows,
    const int64_t* __restrict__ table_offsets, int T, int64_t B, int dim, int C,
    const void* __restrict__ indices, const void* __restrict__ offsets, int64_t nnz,
    const float* __restrict__ weights, float* __restrict__ out, int32_t* __restrict__ err_count,
    int64_t n_bags) {
  using G = StreamGeo<BITS, LPR>;
  using Rows = StreamRows<BITS, LPR, PA4, PX>;
  static_assert(!PX || (StreamGeo<BITS, LPR>::VEC == 8 && PA4), "PX: 8-byte lane chunks, aligned scale/bias");
  constexpr int EPL = G::EPL, RG = G::RG, SLOTS = G::SLOTS, BATCH = G::BATCH, VEC = G::VEC;
  constexpr int DEPTH = G::DEPTH, NBUF = DEPTH + 1;
  static_assert(LPR <= 8 && EPL == 16, "stream lookup: 16 elements per lane, <= 8 lanes per row");
  __shared__ float red[LPR == 8 ? 1 : kWPB][LPR == 8 ? 1 : kWave * EPL];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane / LPR, s = lane % LPR;
  // XCD-aware block order (a bijection on [0, gridDim.x)): consecutive block
  // ids go round-robin over the 8 XCDs, so each XCD gets a contiguous run of
  // bags -- a few tables at a time -- and its L2 holds fewer tables' hot rows
  const int64_t nbk = gridDim.x, xcd = blockIdx.x % 8, kk = blockIdx.x / 8;
  const int64_t qf = nbk / 8, rr = nbk % 8;
  const int64_t blk = xcd * qf + (xcd < rr ? xcd : rr) + kk;
  const int64_t bag0 = (blk * kWPB + wv) * kWave;
  if (bag0 >= n_bags) return;  // whole waves leave together
  const int nb = (int)((n_bags - bag0) < kWave ? (n_bags - bag0) : kWave);
  const int c4 = C & ~3;
  const int c4n = c4 + 4 < (int)S ? c4 + 4 : (int)S - 4;
  const uint32_t csh = (uint32_t)(C & 3);
  const IdxT* ids = reinterpret_cast<const IdxT*>(indices);
  int errs = 0;

  int64_t lp0 = 0, lp1 = 0;
  if (lane < nb) {
    lp0 = load_index<IdxT>(offsets, bag0 + lane);
    lp1 = load_index<IdxT>(offsets, bag0 + lane + 1);
    if (!(lp0 >= 0 && lp1 >= lp0 && lp1 <= nnz)) {
      errs += 1;
      lp0 = lp1 = 0;
    }
  }
  const int64_t t0 = bag0 / B, b0 = bag0 - t0 * B;

  if (nnz == 0 || total_rows == 0) {
    // no id, or no row to read: every term is skipped, every bag is +0
    errs += (int)(lp1 - lp0);
    for (int i = 0; i < nb; ++i) {
      const int64_t bag = bag0 + i, t = bag / B, b = bag - t * B;
      float* o = out + (b * T + t) * (int64_t)dim;
      for (int e = lane; e < dim; e += kWave) o[e] = 0.0f;
    }
    if (errs && err_count) atomicAdd(err_count, errs);
    return;
  }
  const int code_off = s * VEC < C ? s * VEC : 0;
  int baddr[SLOTS];  // ds_bpermute address of batch row u*RG + g
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) baddr[u] = (u * RG + g) * 4;
  const int aown = ((lane % RG) * LPR + LPR - 1) * 4;  // PX: the lane holding row lane's scale/bias

  // ---- producer cursor: the next batch to generate (wave-uniform) ----
  int gj = 0;                                            // its bag within the run
  int64_t gpos = lane_i64(lp0, 0), gend = lane_i64(lp1, 0);
  int gfirst = 1;
  int64_t gt = t0, gb = b0;                              // table, row of the bag
  // a batch: its id count, its table (-1: past the run) and flags
  constexpr int kFirst = 1, kLast = 2, kReal = 4;  // first / last batch of its bag; in the run
  struct Batch {
    int n, t, f;
  };
  auto next_batch = [&](IdxT& id, float& wl) {
    Batch bt;
    int64_t q = 0;
    if (gj < nb) {
      const int64_t rem = gend - gpos;
      const bool last = uniform_flag(rem <= BATCH);
      q = gpos;
      bt.n = last ? (int)rem : BATCH;
      bt.t = (int)gt;
      bt.f = gfirst | (last ? kLast : 0) | kReal;
      if (last) {
        ++gj;
        if (++gb == B) {
          gb = 0;
          ++gt;
        }
        gfirst = kFirst;
        if (gj < nb) {
          gpos = lane_i64(lp0, gj);
          gend = lane_i64(lp1, gj);
        }
      } else {
        gpos += BATCH;
        gfirst = 0;
      }
    } else {
      bt.n = 0;
      bt.t = -1;  // keeps the current table
      bt.f = 0;
    }
    // this batch's ids (and weights) through a descriptor of exactly n ids
    const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ids + q), (short)0, bt.n * (int)sizeof(IdxT), kBufWord3);
    if constexpr (sizeof(IdxT) == 8) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(ri, lane * 8, 0, 0);
      id = (IdxT)(((uint64_t)v[1] << 32) | v[0]);
    } else {
      id = (IdxT)__builtin_amdgcn_raw_buffer_load_b32(ri, lane * 4, 0, 0);
    }
    if constexpr (WEIGHTED) {
      const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(weights + q), (short)0, bt.n * 4, kBufWord3);
      wl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, lane * 4, 0, 0));
    } else {
      wl = 1.0f;
    }
    return bt;
  };

  // ---- the current table (the one of the batch being issued) ----
  int tab_t = -1;
  int64_t tab_nt = 0;
  const uint8_t* tab_base = packed;
  __amdgpu_buffer_rsrc_t tab_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)packed, (short)0, 0, kBufWord3);
  auto use_table = [&](int t) {
    if (t >= 0 && t != tab_t) {
      tab_t = t;
      const int64_t a0 = table_offsets[t], a1 = table_offsets[t + 1];
      const bool ok = uniform_flag(a0 >= 0 && a1 > a0 && a1 <= total_rows);
      tab_nt = ok ? a1 - a0 : 0;
      tab_base = packed + (ok ? a0 : 0) * S;
      const int64_t bytes = tab_nt * S;
      tab_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)tab_base, (short)0, uniform_flag(bytes < (int64_t)kBufLimit) ? (int)bytes : 0, kBufWord3);
    }
  };

  // validate lane's id of a batch; issue its scale/bias load and all slots
  // (BUF: through the table's descriptor, else with 64-bit addresses)
  auto issue = [&](Rows& R, const Batch& bt, IdxT idr, float wl, auto BUF_) {
    const bool in = lane < bt.n;
    bool ok;
    if constexpr (sizeof(IdxT) == 8) {
      ok = in && idr >= 0 && (int64_t)idr < tab_nt;
    } else {
      ok = in && (uint32_t)idr < (uint64_t)tab_nt;
    }
    errs += (in && !ok) ? 1 : 0;  // the id's owner lane counts it
    R.w = ok ? wl : 0.0f;
    if constexpr (decltype(BUF_)::value) {
      const uint32_t own = ok ? (uint32_t)idr * (uint32_t)S : kBufOut;
      if constexpr (!PX) {
        R.plo = __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, own, c4, 0);
        if constexpr (!PA4) R.phi = __builtin_amdgcn_raw_buffer_load_b32(tab_rsrc, own, c4n, 0);
      }
#pragma unroll
      for (int u = 0; u < SLOTS; ++u) {
        const uint32_t bo = bperm(baddr[u], own) + (uint32_t)code_off;
        if constexpr (PX) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b96(tab_rsrc, bo, 0, 0);
          R.cc[u].v = make_uint2(v[0], v[1]);
          R.px[u] = v[2];
        } else if constexpr (VEC == 8) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(tab_rsrc, bo, 0, 0);
          R.cc[u].v = make_uint2(v[0], v[1]);
        } else {
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(tab_rsrc, bo, 0, 0);
          R.cc[u].v = make_uint4(v[0], v[1], v[2], v[3]);
        }
      }
    } else {
      const uint64_t own = ok ? (uint64_t)(int64_t)idr * (uint64_t)S : 0;
      const uint8_t* orow = tab_base + own;
      if constexpr (!PX) {
        R.plo = *reinterpret_cast<const uint32_t*>(orow + c4);
        if constexpr (!PA4) R.phi = *reinterpret_cast<const uint32_t*>(orow + c4n);
      }
      const uint32_t olo = (uint32_t)own, ohi = (uint32_t)(own >> 32);
#pragma unroll
      for (int u = 0; u < SLOTS; ++u) {
        const uint64_t o = ((uint64_t)bperm(baddr[u], ohi) << 32) | bperm(baddr[u], olo);
        if constexpr (PX) {
          const uint3 v = *reinterpret_cast<const uint3*>(tab_base + o + code_off);
          R.cc[u].v = make_uint2(v.x, v.y);
          R.px[u] = v.z;
        } else {
          R.cc[u].load(tab_base + o + code_off);
        }
      }
    }
  };

  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  float accb = 0.0f;  // this lane's share of the bag's sum of w * c
  bool bag_empty = false;
  constexpr float kQ = (float)((1 << BITS) - 1);
  UnpackK K{0x000F000Fu, 0x00F000F0u, 0x00FF00FFu, 0x64006400u};
  asm volatile("" : "+s"(K.m_lo), "+s"(K.m_hi), "+s"(K.m_byte), "+v"(K.one));
  // decode and accumulate a batch; its first batch starts the bag's sums (an
  // empty bag adds nothing and is written as +0)
  auto consume = [&](Rows& R, int nf) {
    const int U = ((nf & 0xff) + RG - 1) / RG;
    const bool first = nf & (kFirst << 8);
    if (first) bag_empty = U == 0;
    if (U == 0) return;
    // lane L prepares batch row L: m, c, ws (zeros without a valid row:
    // its scale/bias read as 0, or its weight is 0)
    uint32_t pown;
    if constexpr (PX) {
      // row L = u*RG + g: its scale/bias came with slot u, in lane g*LPR + LPR-1
      pown = 0u;
#pragma unroll
      for (int u = 0; u < SLOTS; ++u) {
        const uint32_t t = bperm(aown, R.px[u]);
        pown = lane / RG == u ? t : pown;
      }
    } else {
      pown = PA4 ? R.plo : __builtin_amdgcn_alignbyte(R.phi, R.plo, csh);
    }
    const float sf = h16(pown), bf = h16(pown >> 16);
    float mf = __builtin_rintf(-bf * __builtin_amdgcn_rcpf(sf));
    mf = sf > 0.0f ? __builtin_fminf(__builtin_fmaxf(mf, 0.0f), kQ) : 0.0f;
    const float cb = __builtin_fmaf(sf, mf, bf);
    const float wl = R.w;
    accb = first ? wl * cb : __builtin_fmaf(wl, cb, accb);
    const uint32_t mi = (uint32_t)mf;
    const uint32_t wsb = __builtin_bit_cast(uint32_t, wl * sf);
    const uint32_t nlo = (0xE400u + mi) * 0x00010001u;       // fp16 -(1024 + m), twice
    const uint32_t nhi = (0xE400u + 16u * mi) * 0x00010001u; // fp16 -(1024 + 16 m), twice
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      if (u < U) {
        const float ws = __builtin_bit_cast(float, bperm(baddr[u], wsb));
        const uint32_t lo = bperm(baddr[u], nlo);
        const uint32_t hi = BITS == 4 ? bperm(baddr[u], nhi) : 0u;
        if (u == 0 && first) {
          accumulate_centered<BITS, VEC, true>(acc, R.cc[u], ws, lo, hi, K);
        } else {
          accumulate_centered<BITS, VEC>(acc, R.cc[u], ws, lo, hi, K);
        }
      }
    }
  };
  // ---- consumer cursor: the bag whose sums are accumulating ----
  int64_t ct = t0, cb = b0;
  auto finish = [&]() {
    float* o = out + (cb * T + ct) * (int64_t)dim;
    if (++cb == B) {
      cb = 0;
      ++ct;
    }
    const float bias = wave_sum(accb);
    if constexpr (LPR == 8) {
      float r0, r1;
      reduce_scatter_g8(acc, lane, r0, r1);
      r0 = bag_empty ? 0.0f : r0 + bias;
      r1 = bag_empty ? 0.0f : r1 + bias;
      const int e0 = s * 16 + ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2;
      if (dim == LPR * EPL) {
        *reinterpret_cast<float2*>(o + e0) = make_float2(r0, r1);
      } else {
        if (e0 < dim) o[e0] = r0;
        if (e0 + 1 < dim) o[e0 + 1] = r1;
      }
    } else {
      float* rw = red[LPR == 8 ? 0 : wv];
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(rw + g * (LPR * EPL) + s * EPL + e) =
            make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
      wave_sync_lds();
      for (int e = lane; e < dim; e += kWave) {
        float v = rw[e];
#pragma unroll
        for (int gg = 1; gg < RG; ++gg) v += rw[gg * (LPR * EPL) + e];
        o[e] = bag_empty ? 0.0f : v + bias;
      }
      wave_sync_lds();
    }
  };

  // the pipelined batch loop; BUF: every table of the run is under kBufLimit
  // bytes, so all rows go through descriptors (a wave-uniform choice made
  // once, keeping the loop free of a per-batch branch between the two forms)
  auto run = [&](auto BUF_) {
    // ring buffers indexed by batch number mod NBUF: ids (and weights, and
    // the batch's metadata) are requested DEPTH steps before the batch's rows
    // are issued, and rows are consumed DEPTH steps after they are issued.
    // Waiting for a batch's ids then leaves the DEPTH batches of rows issued
    // after them in flight.
    Rows R[NBUF];
    int rnf[NBUF];  // id count | flags << 8 of the batch in rows buffer j
    IdxT bid[NBUF];
    float bw[NBUF];
    Batch bi[NBUF];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) bi[j] = next_batch(bid[j], bw[j]);
    // step k (I = k mod NBUF): request the ids of batch k + DEPTH, issue the
    // rows of batch k
    auto produce_issue = [&](auto I_) {
      constexpr int I = decltype(I_)::value, P = (I + NBUF - 1) % NBUF;
      bi[P] = next_batch(bid[P], bw[P]);
      use_table(bi[I].t);
      issue(R[I], bi[I], bid[I], bw[I], BUF_);
      rnf[I] = bi[I].n | (bi[I].f << 8);
    };
    // ... and consume batch k - DEPTH; false once every batch is consumed
    auto step = [&](auto I_) {
      constexpr int C = (decltype(I_)::value + 1) % NBUF;
      produce_issue(I_);
      consume(R[C], rnf[C]);
      if (rnf[C] & (kLast << 8)) finish();
      return (rnf[C] & (kReal << 8)) != 0;
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    produce_issue(I0{});
    if constexpr (DEPTH == 1) {
      while (step(I1{}) && step(I0{})) {
      }
    } else if constexpr (DEPTH == 2) {
      produce_issue(I1{});
      while (step(I2{}) && step(I0{}) && step(I1{})) {
      }
    } else {
      produce_issue(I1{});
      produce_issue(I2{});
      while (step(I3{}) && step(I0{}) && step(I1{}) && step(I2{})) {
      }
    }
  };
  // tables of the run: t0 .. the table of its last bag
  bool run_buf = true;
  for (int64_t t = t0; t <= (bag0 + nb - 1) / B; ++t) {
    const int64_t a0 = table_offsets[t], a1 = table_offsets[t + 1];
    const bool ok = uniform_flag(a0 >= 0 && a1 > a0 && a1 <= total_rows);
    run_buf = run_buf && uniform_flag((ok ? (a1 - a0) * S : 0) < (int64_t)kBufLimit);
  }
  if (run_buf) {
    run(std::true_type{});
  } else {
    run(std::false_type{});
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
    const uint32_t p = load_params(prow, C, S);
    const float sf = half_value(p), bf = half_value(p >> 16);
    double e2 = 0.0, x2 = 0.0;
    for (int k = 0; k < dim; ++k) {
      uint32_t q = bits == 8   ? prow[k]
                   : bits == 4 ? ((prow[k >> 1] >> ((k & 1) * 4)) & 15u)
                               : ((prow[k >> 2] >> ((k & 3) * 2)) & 3u);
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
// quantizer baselines ("Post-Training 4-bit Quantization on Embedding
// Tables", review page, "Proposed method": the comparison with symmetric
// quantization, histogram-based clipping and ACIQ), in the packed row format:
//   SYMMETRIC   y = s q, q in [-(2^(b-1) - 1), 2^(b-1) - 1], s = max|x| /
//               (2^(b-1) - 1) in fp16 (at most 65504 / 2^(b-1)); stored as
//               code q + 2^(b-1) with bias -2^(b-1) s (exact in fp16)
//   PERCENTILE  window = the row's (1 - p) and p quantiles, linear between
//               order statistics (h = (d - 1) q, fmaf(h - i, v[i+1] - v[i], v[i]))
//   ACIQ        window = mean +- W(3 4^b) * mean|x - mean| (Laplace prior),
//               inside the row range; both means are pairwise sums of the row
//               padded with +0 to a power of two, divided by d
// LPR lanes per row, EPL contiguous elements per lane (the row padded with
// +0 to P = EPL * LPR, a power of two), so a lane's pairwise sum followed by
// xor butterflies is the contiguous-halves pairwise sum of the padded row.
// ---------------------------------------------------------------------------

constexpr int kBaseSym = 0, kBasePct = 1, kBaseAciq = 2;
constexpr int kBaseRange = 3;  // the row range: the range rule's window (used for 2-bit rows)

// W(3 4^b) as binary32: 2.8306830 (b = 2), 5.0286403 (b = 4), 9.8967600 (b = 8)
template <int BITS>
__device__ __forceinline__ float aciq_ratio() {
  return __builtin_bit_cast(float, BITS == 2 ? 0x403529e9u : BITS == 4 ? 0x40a0ea9fu : 0x411e5921u);
}

template <int EPL, int LPR>
__device__ __forceinline__ float lane_pairwise_group_sum(const float (&u0)[EPL]) {
  float u[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) u[e] = u0[e];
#pragma unroll
  for (int h = 1; h < EPL; h <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; e += 2 * h) u[e] = u[e] + u[e + h];
  }
  float t = u[0];
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) t = t + __shfl_xor(t, m);
  return t;
}

template <int LPR>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v |= (uint32_t)__shfl_xor((int)v, m);
  return v;
}

template <int BITS, int EPL, int LPR, int METHOD>
__global__ __launch_bounds__(kBlock) void quantize_baseline_kernel(
    const float* __restrict__ x, int64_t rows, int dim, int C, int S, int vec4, float param,
    uint8_t* __restrict__ packed) {
  constexpr int H = 1 << (BITS - 1), Qs = H - 1;
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
    uint32_t s16, b16;
    float sf, bf, r;
    if constexpr (METHOD == kBaseSym) {
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < EPL; ++k)
        if (k < valid) m = fmaxf(m, __builtin_fabsf(v[k]));
      m = group_max<LPR>(m);
      s16 = half_bits(m / (float)Qs);
      sf = half_value(s16);
      constexpr float smax = 65504.0f / (float)H;
      if (sf > smax) {
        s16 = half_bits(smax);
        sf = smax;
      }
      // the product stays an fp32 multiply: fused into the fp16 conversion it
      // became v_fma_mix with a +0 addend, which turns -8 * (+0) into +0
      float nb = -(float)H * sf;
      asm volatile("" : "+v"(nb));
      b16 = half_bits(nb);
      bf = half_value(b16);
      r = sf == 0.0f ? 0.0f : 1.0f / sf;
    } else {
      float lo, hi;
      float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        if (k < valid) {
          mn = fminf(mn, v[k]);
          mx = fmaxf(mx, v[k]);
        }
      }
      mn = group_min<LPR>(mn) + 0.0f;
      mx = group_max<LPR>(mx) + 0.0f;
      if constexpr (METHOD == kBaseRange) {
        lo = mn;
        hi = mx;
      } else if constexpr (METHOD == kBaseAciq) {
        float u[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) u[k] = k < valid ? v[k] : 0.0f;
        const float mu = lane_pairwise_group_sum<EPL, LPR>(u) / (float)dim;
#pragma unroll
        for (int k = 0; k < EPL; ++k) u[k] = k < valid ? __builtin_fabsf(v[k] - mu) : 0.0f;
        const float bsc = lane_pairwise_group_sum<EPL, LPR>(u) / (float)dim;
        const float a = aciq_ratio<BITS>() * bsc;
        const float l = mu - a, h = mu + a;
        lo = (l > mn ? l : mn) + 0.0f;
        hi = (h < mx ? h : mx) + 0.0f;
      } else {
        // ranks by value, ties by position: the order of a stable sort
        int rk[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) rk[k] = 0;
        const int gbase = (threadIdx.x % kWave) - s;
        for (int t = 0; t < LPR; ++t) {
#pragma unroll
          for (int kk = 0; kk < EPL; ++kk) {
            const float o = __shfl(v[kk], gbase + t);
            const int j = t * EPL + kk;
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
              const int i = e0 + k;
              rk[k] += (j < dim && (o < v[k] || (o == v[k] && j < i))) ? 1 : 0;
            }
          }
        }
        auto order_stat = [&](int want) {
          uint32_t b = 0u;
#pragma unroll
          for (int k = 0; k < EPL; ++k)
            b |= (k < valid && rk[k] == want) ? __builtin_bit_cast(uint32_t, v[k]) : 0u;
          return __builtin_bit_cast(float, group_or<LPR>(b));
        };
        auto quantile = [&](float q) {
          const float hq = (float)(dim - 1) * q;
          const int i = (int)__builtin_floorf(hq);
          if (i >= dim - 1) return order_stat(dim - 1);
          const float f = hq - (float)i;
          const float v0 = order_stat(i), v1 = order_stat(i + 1);
          return __builtin_fmaf(f, v1 - v0, v0);
        };
        lo = quantile(1.0f - param) + 0.0f;
        hi = quantile(param) + 0.0f;
      }
      const Window w = make_window<BITS>(lo, hi);
      s16 = w.s16;
      b16 = w.b16;
      sf = w.sf;
      bf = w.bf;
      r = w.r;
    }
    // codes of this lane's elements (padding elements 0)
    constexpr int LW = (EPL * BITS + 31) / 32;  // code words of one lane
    uint32_t cw[LW];
#pragma unroll
    for (int j = 0; j < LW; ++j) cw[j] = 0u;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      if (k < valid) {
        uint32_t q;
        if constexpr (METHOD == kBaseSym) {
          const float t = sf == 0.0f ? 0.0f : __builtin_rintf(v[k] * r);
          q = (uint32_t)(int)(fminf(fmaxf(t, -(float)Qs), (float)Qs) + (float)H);
        } else {
          constexpr float Qf = (float)((1 << BITS) - 1);
          q = (uint32_t)fminf(fmaxf(__builtin_rintf((v[k] - bf) * r), 0.0f), Qf);
        }
        cw[(k * BITS) / 32] |= q << ((k * BITS) % 32);
      }
    }
    (void)bf;
    const uint32_t p32 = s16 | (b16 << 16);
    uint8_t* prow = packed + row * (int64_t)S;
    const int nwords = S / 4;
    // the lane's own words, then the words past every lane's codes (scale,
    // bias and padding) round robin
#pragma unroll
    for (int j = 0; j < LW; ++j) {
      const int wd = s * LW + j;
      if (wd < nwords) *reinterpret_cast<uint32_t*>(prow + 4 * wd) = cw[j] | param_part(p32, C - 4 * wd);
    }
    for (int wd = LPR * LW + s; wd < nwords; wd += LPR)
      *reinterpret_cast<uint32_t*>(prow + 4 * wd) = param_part(p32, C - 4 * wd);
  }
}

// ---------------------------------------------------------------------------
// codebook rows: 16 fp32 levels per row (1-D k-means), 4-bit codes
// ("Post-Training 4-bit Quantization on Embedding Tables", review page,
// "Proposed method": codebook quantization by k-means clustering; "Main
// findings": 18.8%-37.5% of the fp32 size, lowest normalized l2 loss).
// Row: levels c_0..c_15 (64 bytes) | codes (element 2k in the low nibble of
// byte 64 + k) | zero padding to a multiple of 16 bytes.
// ---------------------------------------------------------------------------

constexpr int kCbLevels = 16;

// smallest k minimizing |x - c_k| (one fp32 subtraction each, exact |.|)
__device__ __forceinline__ int nearest_level(float x, const float (&c)[kCbLevels]) {
  int best = 0;
  float bd = __builtin_fabsf(x - c[0]);
#pragma unroll
  for (int k = 1; k < kCbLevels; ++k) {
    const float dk = __builtin_fabsf(x - c[k]);
    const bool b = dk < bd;
    bd = b ? dk : bd;
    best = b ? k : best;
  }
  return best;
}

// LPR lanes per row, lane s holding the contiguous elements [s*EPL,
// (s+1)*EPL) of the row padded with +0 to P = EPL*LPR (a power of two), so a
// lane's pairwise sum of its chunk followed by xor butterflies over the LPR
// lanes is the contiguous-halves pairwise sum of the padded row.
//   1. levels start on the row's uniform grid c_k = fma(k, (hi-lo)/15, lo) + 0;
//   2. n_iter times: nearest level of every element; every level with
//      members becomes (pairwise sum of the members' values, +0 elsewhere) /
//      member count + 0; a level without members keeps its value;
//   3. codes: nearest level with the final levels.
template <int EPL, int LPR>
__global__ __launch_bounds__(kBlock) void quantize_codebook_kernel(
    const float* __restrict__ x, int64_t rows, int dim, int S, int vec4, int n_iter,
    uint8_t* __restrict__ packed) {
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
      if (k < valid) {
        mn = fminf(mn, v[k]);
        mx = fmaxf(mx, v[k]);
      }
    }
    const float lo = group_min<LPR>(mn) + 0.0f;
    const float hi = group_max<LPR>(mx) + 0.0f;
    const float delta = (hi - lo) / (float)(kCbLevels - 1);
    float c[kCbLevels];
#pragma unroll
    for (int k = 0; k < kCbLevels; ++k) c[k] = __builtin_fmaf((float)k, delta, lo) + 0.0f;
    int a[EPL];
    for (int it = 0; it < n_iter; ++it) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) a[e] = e < valid ? nearest_level(v[e], c) : -1;
      float nx[kCbLevels];
#pragma unroll
      for (int k = 0; k < kCbLevels; ++k) {
        float u[EPL];
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const bool m = a[e] == k;
          u[e] = m ? v[e] : 0.0f;
          cnt += m ? 1 : 0;
        }
#pragma unroll
        for (int h = 1; h < EPL; h <<= 1) {
#pragma unroll
          for (int e = 0; e < EPL; e += 2 * h) u[e] = u[e] + u[e + h];
        }
        float tot = u[0];
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) {
          tot = tot + __shfl_xor(tot, m);
          cnt += __shfl_xor(cnt, m);
        }
        nx[k] = cnt > 0 ? tot / (float)cnt + 0.0f : c[k];
      }
#pragma unroll
      for (int k = 0; k < kCbLevels; ++k) c[k] = nx[k];
    }
    // codes of this lane's elements (padding elements code 0)
    uint32_t cw[(EPL + 7) / 8];
#pragma unroll
    for (int j = 0; j < (EPL + 7) / 8; ++j) cw[j] = 0u;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if (e < valid) cw[e / 8] |= (uint32_t)nearest_level(v[e], c) << (4 * (e % 8));
    uint8_t* prow = packed + row * (int64_t)S;
    // levels: 4 units of 16 bytes, round robin over the row's lanes
#pragma unroll
    for (int U = 0; U < 4; ++U)
      if (U % LPR == s)
        *reinterpret_cast<float4*>(prow + 16 * U) =
            make_float4(c[4 * U], c[4 * U + 1], c[4 * U + 2], c[4 * U + 3]);
    if constexpr (LPR >= 2) {
      // EPL == 16: this lane's 8 code bytes at 64 + 8s (the lanes cover
      // every byte from 64 to the stride; lanes past it store nothing)
      if (64 + 8 * s < S) *reinterpret_cast<uint2*>(prow + 64 + 8 * s) = make_uint2(cw[0], cw[1]);
    } else {
      // one lane per row: codes (at most 8 bytes) and padding, 16-byte units
      for (int U = 4; 16 * U < S; ++U)
        *reinterpret_cast<uint4*>(prow + 16 * U) =
            make_uint4(U == 4 ? cw[0] : 0u, U == 4 && EPL > 8 ? cw[(EPL + 7) / 8 - 1] : 0u, 0u, 0u);
    }
  }
}

// Dequantize codebook rows: groups of 16 lanes per row, lane k holding level
// k; lane k decodes elements [EPL k, EPL k + EPL) of each pass of 16 EPL
// elements (EPL = 4 for d <= 64, else 8), each by one ds_bpermute from the
// lane that holds its level (the pre-masked nibble addresses of the codebook
// lookup).  Every lane of a wave runs the same number of passes (rows past
// the end are clamped and not stored), so the cross-lane reads see all lanes
// active.
template <int EPL>
__global__ __launch_bounds__(kBlock) void dequant_codebook_kernel(
    const uint8_t* __restrict__ packed, int64_t rows, int dim, int S, float* __restrict__ y) {
  const int lane = threadIdx.x % kWave;
  const int k = lane % kCbLevels, grp = lane / kCbLevels;
  const uint32_t gsel = (uint32_t)(grp * 64) * 0x01010101u;
  const int64_t gpb = kBlock / kCbLevels;  // row groups per block
  const int64_t stride_rows = (int64_t)gridDim.x * gpb;
  const int64_t first = (int64_t)blockIdx.x * gpb + threadIdx.x / kCbLevels;
  const int64_t nrounds = (rows + stride_rows - 1) / stride_rows;
  constexpr int PASS = 16 * EPL;
  const int npass = (dim + PASS - 1) / PASS;
  const bool vec = dim % 4 == 0;
  for (int64_t rd = 0; rd < nrounds; ++rd) {
    const int64_t row = first + rd * stride_rows;
    const bool live = row < rows;
    const uint8_t* prow = packed + (live ? row : 0) * (int64_t)S;
    const uint32_t lvb = *reinterpret_cast<const uint32_t*>(prow + 4 * k);
    for (int pss = 0; pss < npass; ++pss) {
      const int e0 = pss * PASS + EPL * k;
      uint32_t cw = 0u;
      if (e0 < dim) {
        if constexpr (EPL == 8) {
          cw = *reinterpret_cast<const uint32_t*>(prow + 64 + e0 / 2);
        } else {
          cw = *reinterpret_cast<const uint16_t*>(prow + 64 + e0 / 2);
        }
      }
      const uint32_t ev = ((cw << 2) & 0x3C3C3C3Cu) | gsel;  // elements 0, 2, ...
      const uint32_t od = ((cw >> 2) & 0x3C3C3C3Cu) | gsel;  // elements 1, 3, ...
      float o[EPL];
#pragma unroll
      for (int h = 0; h < EPL / 2; ++h) {
        o[2 * h] = __builtin_bit_cast(float, bperm((int)(ev >> (8 * h)), lvb));
        o[2 * h + 1] = __builtin_bit_cast(float, bperm((int)(od >> (8 * h)), lvb));
      }
      if (live && e0 < dim) {
        float* yr = y + row * dim + e0;
        if (e0 + EPL <= dim && vec) {
#pragma unroll
          for (int j = 0; j < EPL; j += 4)
            *reinterpret_cast<float4*>(yr + j) = make_float4(o[j], o[j + 1], o[j + 2], o[j + 3]);
        } else {
#pragma unroll
          for (int j = 0; j < EPL; ++j)
            if (e0 + j < dim) yr[j] = o[j];
        }
      }
    }
  }
}

// Pooled lookup over codebook rows: one wave per bag, 4 row groups of 16
// lanes; lane k of a group holds level k of the group's current row and the
// code word of elements [8k, 8k+8) of every 128-element pass.  The bag's ids
// are read 64 at a time, one per owner lane, which checks it; row offsets and
// weights reach the groups by ds_bpermute, so 4*U rows are in flight after
// one wait for the ids.  Tables below kBufLimit bytes are read through a
// buffer descriptor with 32-bit offsets (an absent row reads zeros), larger
// ones with 64-bit addresses.
//
// Decoding an element is one ds_bpermute from the lane that holds its level:
// ds_bpermute selects the source lane by address bits [7:2] and ignores the
// bits above, so a byte holding (group lane base + code) * 4 is an address
// as it stands; a code word gives two words of four such bytes each (even
// and odd elements), and a shift moves each byte to the bottom.
template <typename IdxT, int NP, int U>
__global__ __launch_bounds__(kBlock) void bag_codebook_kernel(
    const uint8_t* __restrict__ packed, int64_t S, int64_t total_rows,
    const int64_t* __restrict__ table_offsets, int T, int64_t B, int dim,
    const void* __restrict__ indices, const void* __restrict__ offsets, int64_t nnz,
    const float* __restrict__ weights, float* __restrict__ out, int32_t* __restrict__ err_count,
    int64_t n_bags) {
  static_assert(16 % U == 0, "U divides the 16 rounds of a 64-id chunk");
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int k = lane % kCbLevels, grp = lane / kCbLevels;
  const int64_t bag = (int64_t)blockIdx.x * kWPB + wv;
  if (bag >= n_bags) return;  // whole waves leave together
  const int64_t t = bag / B, b = bag - t * B;
  int errs = 0;
  int64_t p0 = load_index<IdxT>(offsets, bag), p1 = load_index<IdxT>(offsets, bag + 1);
  if (!uniform_flag(p0 >= 0 && p1 >= p0 && p1 <= nnz)) {
    errs = lane == 0 ? 1 : 0;
    p0 = p1 = 0;
  }
  const int64_t a0 = table_offsets[t], a1 = table_offsets[t + 1];
  const bool tab_ok = uniform_flag(a0 >= 0 && a1 > a0 && a1 <= total_rows);
  const int64_t nt = tab_ok ? a1 - a0 : 0;
  const uint8_t* base = packed + (tab_ok ? a0 : 0) * S;
  const IdxT* ids = reinterpret_cast<const IdxT*>(indices);
  if (total_rows == 0) {
    // no row to read: every id is skipped and counted
    errs += lane == 0 ? (int)(p1 - p0) : 0;
    p1 = p0;
  }
  const int64_t tab_bytes = nt * S;
  const bool use_buf = uniform_flag(tab_bytes < (int64_t)kBufLimit);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)base, (short)0, use_buf ? (int)tab_bytes : 0, kBufWord3);
  const uint32_t gsel = (uint32_t)(grp * 64) * 0x01010101u;  // group lane base * 4, every byte
  const uint32_t kmask = 0x3C3C3C3Cu;
  float acc[NP][8];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[pp][j] = 0.0f;

  auto body = [&](auto BUF_) {
    constexpr bool BUF = decltype(BUF_)::value;
    for (int64_t c = p0; c < p1; c += kWave) {
      const int n = (int)min<int64_t>(kWave, p1 - c);
      const bool in = lane < n;
      const int64_t id = in ? (int64_t)ids[c + lane] : 0;
      const bool ok = in && id >= 0 && id < nt;
      errs += (in && !ok) ? 1 : 0;
      const int wt = __builtin_bit_cast(int, ok ? (weights ? weights[c + lane] : 1.0f) : 0.0f);
      uint32_t own_lo, own_hi = 0;
      if constexpr (BUF) {
        own_lo = ok ? (uint32_t)id * (uint32_t)S : kBufOut;
      } else {
        const int64_t off = (ok ? id : 0) * S;  // absent: row 0, weight 0
        own_lo = (uint32_t)off;
        own_hi = (uint32_t)(off >> 32);
      }
      const int nr = (n + 3) / 4;  // rounds of 4 rows, one per group
      for (int r0 = 0; r0 < nr; r0 += U) {
        float lv[U], wl[U];
        uint32_t cwd[U][NP];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (r0 + u < nr) {
            const int src = 16 * (r0 + u) + 4 * grp;  // owner lane 4(r0+u) + grp
            wl[u] = __builtin_bit_cast(float, (int)bperm(src, (uint32_t)wt));
            const uint32_t o = bperm(src, own_lo);
            if constexpr (BUF) {
              const uint32_t vo = o + 4 * k;
              lv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, vo, 0, 0));
#pragma unroll
              for (int pp = 0; pp < NP; ++pp)
                cwd[u][pp] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, vo + 64 + 64 * pp, 0, 0);
            } else {
              const uint64_t hi = bperm(src, own_hi);
              const uint8_t* prow = base + ((hi << 32) | o);
              lv[u] = *reinterpret_cast<const float*>(prow + 4 * k);
#pragma unroll
              for (int pp = 0; pp < NP; ++pp) {
                const int e0 = pp * 128 + 8 * k;
                cwd[u][pp] = e0 < dim ? *reinterpret_cast<const uint32_t*>(prow + 64 + e0 / 2) : 0u;
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (r0 + u < nr) {
            const uint32_t lvb = __builtin_bit_cast(uint32_t, lv[u]);
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) {
              const uint32_t ev = ((cwd[u][pp] << 2) & kmask) | gsel;  // elements 0,2,4,6
              const uint32_t od = ((cwd[u][pp] >> 2) & kmask) | gsel;  // elements 1,3,5,7
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                const float y0 = __builtin_bit_cast(float, bperm((int)(ev >> (8 * h)), lvb));
                const float y1 = __builtin_bit_cast(float, bperm((int)(od >> (8 * h)), lvb));
                acc[pp][2 * h] = __builtin_fmaf(wl[u], y0, acc[pp][2 * h]);
                acc[pp][2 * h + 1] = __builtin_fmaf(wl[u], y1, acc[pp][2 * h + 1]);
              }
            }
          }
        }
      }
    }
  };
  if (use_buf) {
    body(std::true_type{});
  } else {
    body(std::false_type{});
  }
  // the 4 groups' partial sums: lanes i, i^32, i^16, i^48
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x0 = acc[pp][j], x1 = acc[pp][j];
      permlane32_swap(x0, x1);
      const float h = x0 + x1;
      float y0 = h, y1 = h;
      permlane16_swap(y0, y1);
      acc[pp][j] = y0 + y1;
    }
  if (grp == 0) {
    float* o = out + (b * T + t) * (int64_t)dim;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int e0 = pp * 128 + 8 * k;
      if (e0 + 8 <= dim && (dim % 4) == 0) {
        *reinterpret_cast<float4*>(o + e0) = make_float4(acc[pp][0], acc[pp][1], acc[pp][2], acc[pp][3]);
        *reinterpret_cast<float4*>(o + e0 + 4) = make_float4(acc[pp][4], acc[pp][5], acc[pp][6], acc[pp][7]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (e0 + j < dim) o[e0 + j] = acc[pp][j];
      }
    }
  }
  for (int m = 1; m < kWave; m <<= 1) errs += __shfl_xor(errs, m);
  if (lane == 0 && errs && err_count) atomicAdd(err_count, errs);
}

// Pooled lookup over 2-bit rows: the mapping of bag_codebook_kernel (one
// wave per bag, 4 groups of 16 lanes, owner-lane ids, buffer-descriptor
// rows), lane k of a group decoding elements [8k, 8k + 8) of each
// 128-element pass from 2 code bytes; the term is w * fmaf(sf, q, bf) (the
// decoded value times the weight, as the other uniform-row lookups).
template <typename IdxT, int NP, int U>
__global__ __launch_bounds__(kBlock) void bag_int2_kernel(
    const uint8_t* __restrict__ packed, int64_t S, int64_t total_rows,
    const int64_t* __restrict__ table_offsets, int T, int64_t B, int dim, int C,
    const void* __restrict__ indices, const void* __restrict__ offsets, int64_t nnz,
    const float* __restrict__ weights, float* __restrict__ out, int32_t* __restrict__ err_count,
    int64_t n_bags) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int k = lane % 16, grp = lane / 16;
  const int64_t bag = (int64_t)blockIdx.x * kWPB + wv;
  if (bag >= n_bags) return;
  const int64_t t = bag / B, b = bag - t * B;
  int errs = 0;
  int64_t p0 = load_index<IdxT>(offsets, bag), p1 = load_index<IdxT>(offsets, bag + 1);
  if (!uniform_flag(p0 >= 0 && p1 >= p0 && p1 <= nnz)) {
    errs = lane == 0 ? 1 : 0;
    p0 = p1 = 0;
  }
  const int64_t a0 = table_offsets[t], a1 = table_offsets[t + 1];
  const bool tab_ok = uniform_flag(a0 >= 0 && a1 > a0 && a1 <= total_rows);
  const int64_t nt = tab_ok ? a1 - a0 : 0;
  const uint8_t* base = packed + (tab_ok ? a0 : 0) * S;
  const IdxT* ids = reinterpret_cast<const IdxT*>(indices);
  if (total_rows == 0) {
    errs += lane == 0 ? (int)(p1 - p0) : 0;
    p1 = p0;
  }
  const int c4 = C & ~3, c4n = c4 + 4 < (int)S ? c4 + 4 : (int)S - 4;
  const uint32_t csh = (uint32_t)(C & 3);
  float acc[NP][8];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[pp][j] = 0.0f;
  for (int64_t c = p0; c < p1; c += kWave) {
    const int n = (int)min<int64_t>(kWave, p1 - c);
    const bool in = lane < n;
    const int64_t id = in ? (int64_t)ids[c + lane] : 0;
    const bool ok = in && id >= 0 && id < nt;
    errs += (in && !ok) ? 1 : 0;
    const int64_t off = (ok ? id : 0) * S;  // absent: row 0, weight 0
    const uint32_t own_lo = (uint32_t)off, own_hi = (uint32_t)(off >> 32);
    const int wt = __builtin_bit_cast(int, ok ? (weights ? weights[c + lane] : 1.0f) : 0.0f);
    const int nr = (n + 3) / 4;
    for (int r0 = 0; r0 < nr; r0 += U) {
      float wl[U], sf[U], bf[U];
      uint32_t cwd[U][NP];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (r0 + u < nr) {
          const int src = 16 * (r0 + u) + 4 * grp;
          wl[u] = __builtin_bit_cast(float, (int)bperm(src, (uint32_t)wt));
          const uint64_t hi = bperm(src, own_hi);
          const uint8_t* prow = base + ((hi << 32) | bperm(src, own_lo));
          const uint32_t plo = *reinterpret_cast<const uint32_t*>(prow + c4);
          const uint32_t phi = *reinterpret_cast<const uint32_t*>(prow + c4n);
          const uint32_t p32 = __builtin_amdgcn_alignbyte(phi, plo, csh);
          sf[u] = half_value(p32);
          bf[u] = half_value(p32 >> 16);
#pragma unroll
          for (int pp = 0; pp < NP; ++pp) {
            const int e0 = pp * 128 + 8 * k;
            cwd[u][pp] = e0 < dim ? *reinterpret_cast<const uint16_t*>(prow + e0 / 4) : 0u;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (r0 + u < nr) {
#pragma unroll
          for (int pp = 0; pp < NP; ++pp) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float y = __builtin_fmaf(sf[u], (float)((cwd[u][pp] >> (2 * j)) & 3u), bf[u]);
              acc[pp][j] = __builtin_fmaf(wl[u], y, acc[pp][j]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x0 = acc[pp][j], x1 = acc[pp][j];
      permlane32_swap(x0, x1);
      const float h = x0 + x1;
      float y0 = h, y1 = h;
      permlane16_swap(y0, y1);
      acc[pp][j] = y0 + y1;
    }
  if (grp == 0) {
    float* o = out + (b * T + t) * (int64_t)dim;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int e0 = pp * 128 + 8 * k;
      if (e0 + 8 <= dim && (dim % 4) == 0) {
        *reinterpret_cast<float4*>(o + e0) = make_float4(acc[pp][0], acc[pp][1], acc[pp][2], acc[pp][3]);
        *reinterpret_cast<float4*>(o + e0 + 4) = make_float4(acc[pp][4], acc[pp][5], acc[pp][6], acc[pp][7]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (e0 + j < dim) o[e0 + j] = acc[pp][j];
      }
    }
  }
  for (int m = 1; m < kWave; m <<= 1) errs += __shfl_xor(errs, m);
  if (lane == 0 && errs && err_count) atomicAdd(err_count, errs);
}

__global__ __launch_bounds__(kBlock) void l2_partial_codebook_kernel(
    const float* __restrict__ x, const uint8_t* __restrict__ packed, int64_t rows, int dim, int S,
    double* __restrict__ part) {
  __shared__ double sh[4 * kBlock];
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  for (int64_t row = (int64_t)blockIdx.x * kBlock + threadIdx.x; row < rows;
       row += (int64_t)gridDim.x * kBlock) {
    const float* xr = x + row * dim;
    const uint8_t* prow = packed + row * (int64_t)S;
    const float* lv = reinterpret_cast<const float*>(prow);
    double e2 = 0.0, x2 = 0.0;
    for (int e = 0; e < dim; ++e) {
      const uint32_t q = (prow[64 + (e >> 1)] >> ((e & 1) * 4)) & 15u;
      const double xk = (double)xr[e];
      const double d = xk - (double)lv[q];
      e2 += d * d;
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

// ---------------------------------------------------------------------------
// dot interaction of the pooled embeddings ("Deep Learning Recommendation
// Model ..." review page, "Proposed method": second-order interactions are
// the dot products between the embedding vectors and the processed dense
// features, concatenated with the dense features).  Per sample b the rows of
// Z are the dense vector (row 0) and the T pooled vectors (rows 1..T, the
// lookup's [B][T][d] output); out[b] = dense[b], then <z_i, z_j> for
// i = 1..T, j = 0..i-1 in that order: the pair (t1 + 1, t2 + 1) of pooled
// rows t2 < t1 sits at d + (t1 + 1) t1 / 2 + t2 + 1, the pair (t + 1, 0)
// with the dense vector at d + (t + 1) t / 2.
//
// Pooled x pooled dots are 16 x 16 tiles of the Gram matrix on the matrix
// cores (v_mfma_f32_16x16x4_f32, fp32 in and out): lane l supplies row l % 16
// of each operand block at k-slot l / 16, so a lane holding the float4 of
// columns [16s + 4g, 16s + 4g + 4) of its row feeds four MFMAs, and the
// result tile leaves rows 4g..4g+3 of column l % 16 in the lane.  Only the
// tiles on or below the diagonal are computed.  The dense dots are plain
// FMAs on the vector ALU with a reduction across the four k-slots.
// ---------------------------------------------------------------------------

using f32x4 = __attribute__((ext_vector_type(4))) float;
using u32x4 = __attribute__((ext_vector_type(4))) unsigned int;

// columns [k, k+4) of a row (zeros past dim or for an absent row)
__device__ __forceinline__ float4 ix_chunk(const float* row, int k, int dim, bool vec4) {
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (row != nullptr) {
    if (vec4 && k + 4 <= dim) {
      v = *reinterpret_cast<const float4*>(row + k);
    } else {
      if (k < dim) v.x = row[k];
      if (k + 1 < dim) v.y = row[k + 1];
      if (k + 2 < dim) v.z = row[k + 2];
      if (k + 3 < dim) v.w = row[k + 3];
    }
  }
  return v;
}

__device__ __forceinline__ f32x4 mfma4(float4 a, float4 b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
  return c;
}

// sum over the four lanes of a column (lanes c, c+16, c+32, c+48)
__device__ __forceinline__ float ix_col_sum(float v) {
  float a = v, b = v;
  permlane32_swap(a, b);
  const float h = a + b;
  float c = h, d = h;
  permlane16_swap(c, d);
  return c + d;
}

__device__ __forceinline__ void ix_store_tile(float* ob, f32x4 acc, int I, int J, int r, int g, int T,
                                              int dim) {
  const int t2 = 16 * J + r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t1 = 16 * I + 4 * g + v;
    if (t2 < t1 && t1 < T) ob[dim + (int64_t)(t1 + 1) * t1 / 2 + t2 + 1] = acc[v];
  }
}

// NBP blocks of 16 pooled rows (T <= 16 NBP) and KC chunks of 16 columns
// (dim <= 16 KC), all held in registers: each row is read once.
template <int NBP, int KC>
__global__ __launch_bounds__(kBlock) void interaction_kernel(
    const float* __restrict__ dense, const float* __restrict__ pooled, int64_t B, int T, int dim,
    int vec4, float* __restrict__ out) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r = lane % 16, g = lane / 16;
  const int64_t b = (int64_t)blockIdx.x * kWPB + wv;
  if (b >= B) return;  // whole waves leave together
  const int64_t W = dim + (int64_t)T * (T + 1) / 2;
  const float* xb = dense + b * dim;
  const float* eb = pooled + b * (int64_t)T * dim;
  float* ob = out + b * W;
  float4 z[NBP][KC], xv[KC];
#pragma unroll
  for (int I = 0; I < NBP; ++I) {
    const int t = 16 * I + r;
    const float* row = t < T ? eb + (int64_t)t * dim : nullptr;
#pragma unroll
    for (int s = 0; s < KC; ++s) z[I][s] = ix_chunk(row, 16 * s + 4 * g, dim, vec4);
  }
#pragma unroll
  for (int s = 0; s < KC; ++s) xv[s] = ix_chunk(xb, 16 * s + 4 * g, dim, vec4);
  for (int k = lane; k < dim; k += kWave) ob[k] = xb[k];
  // dots with the dense vector
#pragma unroll
  for (int I = 0; I < NBP; ++I) {
    float p = 0.0f;
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      p = __builtin_fmaf(z[I][s].x, xv[s].x, p);
      p = __builtin_fmaf(z[I][s].y, xv[s].y, p);
      p = __builtin_fmaf(z[I][s].z, xv[s].z, p);
      p = __builtin_fmaf(z[I][s].w, xv[s].w, p);
    }
    p = ix_col_sum(p);
    const int t = 16 * I + r;
    if (g == 0 && t < T) ob[dim + (int64_t)(t + 1) * t / 2] = p;
  }
  // pooled x pooled: tiles on or below the diagonal
#pragma unroll
  for (int I = 0; I < NBP; ++I) {
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KC; ++s) acc = mfma4(z[I][s], z[J][s], acc);
      ix_store_tile(ob, acc, I, J, r, g, T, dim);
    }
  }
}

// Persistent workgroups of 4 waves, one sample at a time.  The sample being
// computed sits in LDS; the next two are in flight in two register sets
// (about 43 KB of LDS per workgroup at d = 128: three workgroups per CU).
// Every global access is unconditional and goes through a per-sample buffer
// descriptor (an absent row or a column past dim takes an out-of-range
// offset: loads read zeros, stores are dropped), and the results are staged
// in an LDS output row written out with coalesced stores after a barrier, so
// the number of memory operations between a sample's loads and their use is
// static and the wait before each LDS fill covers exactly that sample.
// Rows sit in LDS at a stride of 16 KC + 8 floats (measured: no padding costs
// about 40 % in bank conflicts).  Wave w takes tiles w,
// w+4, ... of the lower triangle and the dense dots of block rows w, w+4, ...;
// results are bitwise those of interaction_kernel (same operation order).
// Needs dim % 4 == 0; ST4: the output row width is a multiple of 4.
template <int NBP, int KC, bool ST4>
__global__ __launch_bounds__(kBlock) void interaction_lds_kernel(
    const float* __restrict__ dense, const float* __restrict__ pooled, int64_t B, int T, int dim,
    float* __restrict__ out) {
  constexpr int ROWS = 16 * NBP, C4 = 4 * KC, RS = C4 + 2;  // row stride in float4
  constexpr int SLOTS = ROWS * C4, PER = (SLOTS + kBlock - 1) / kBlock;
  constexpr int NT = NBP * (NBP + 1) / 2;
  constexpr int WMAX = 16 * KC + ROWS * (ROWS + 1) / 2;  // widest output row
  constexpr int OUTW = (WMAX + 3) / 4 * 4;
  static_assert(C4 <= kBlock, "the dense row fits one pass");
  __shared__ float4 buf[1][(ROWS + 1) * RS];
  __shared__ float obuf[OUTW];
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int r = lane % 16, g = lane / 16;
  const int W = dim + T * (T + 1) / 2;
  const int c4n = dim / 4;
  const int rowb = dim * 4;  // bytes per row
  float4 va[PER], vb[PER], xa, xb;
  auto fetch = [&](int64_t smp, float4 (&v)[PER], float4& xd) {
    const bool live = smp < B;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(pooled + (live ? smp : 0) * T * (int64_t)dim), (short)0, live ? T * rowb : 0, kBufWord3);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(dense + (live ? smp : 0) * dim), (short)0, live ? rowb : 0, kBufWord3);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int f = tid + kBlock * u, row = f / C4, c4 = f % C4;
      const uint32_t off = (f < SLOTS && c4 < c4n) ? (uint32_t)(row * rowb + 16 * c4) : kBufOut;
      v[u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, 0));
    }
    xd = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                        rx, tid < c4n ? (uint32_t)(16 * tid) : kBufOut, 0, 0));
  };
  auto put = [&](int bs, const float4 (&v)[PER], const float4& xd) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int f = tid + kBlock * u;
      if (f < SLOTS) buf[bs][(f / C4) * RS + f % C4] = v[u];
    }
    if (tid < C4) buf[bs][ROWS * RS + tid] = xd;
  };
  auto compute = [&](int bs) {
    const float* xs = reinterpret_cast<const float*>(&buf[bs][ROWS * RS]);
    for (int k = tid; k < dim; k += kBlock) obuf[k] = xs[k];
#pragma unroll
    for (int I = 0; I < NBP; ++I) {
      if (I % kWPB == wv) {
        float p = 0.0f;
#pragma unroll
        for (int s = 0; s < KC; ++s) {
          const float4 zi = buf[bs][(16 * I + r) * RS + 4 * s + g];
          const float4 xv = buf[bs][ROWS * RS + 4 * s + g];
          p = __builtin_fmaf(zi.x, xv.x, p);
          p = __builtin_fmaf(zi.y, xv.y, p);
          p = __builtin_fmaf(zi.z, xv.z, p);
          p = __builtin_fmaf(zi.w, xv.w, p);
        }
        p = ix_col_sum(p);
        const int t = 16 * I + r;
        if (g == 0 && t < T) obuf[dim + (t + 1) * t / 2] = p;
      }
    }
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
      if (tau % kWPB == wv) {
        int I = 0, J = tau;
        while (J > I) {
          J -= I + 1;
          ++I;
        }
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KC; ++s)
          acc = mfma4(buf[bs][(16 * I + r) * RS + 4 * s + g], buf[bs][(16 * J + r) * RS + 4 * s + g], acc);
        const int t2 = 16 * J + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t1 = 16 * I + 4 * g + v;
          if (t2 < t1 && t1 < T) obuf[dim + (t1 + 1) * t1 / 2 + t2 + 1] = acc[v];
        }
      }
    }
  };
  auto copy_out = [&](int64_t smp) {
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(out + smp * (int64_t)W), (short)0, W * 4, kBufWord3);
    if constexpr (ST4) {
#pragma unroll
      for (int u = 0; u < (OUTW / 4 + kBlock - 1) / kBlock; ++u) {
        const int q4 = tid + kBlock * u;
        const float4 vv = q4 < OUTW / 4 ? reinterpret_cast<const float4*>(obuf)[q4]
                                        : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, vv), ro,
                                               4 * q4 < W ? (uint32_t)(16 * q4) : kBufOut, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < (OUTW + kBlock - 1) / kBlock; ++u) {
        const int q1 = tid + kBlock * u;
        const float vv = q1 < OUTW ? obuf[q1] : 0.0f;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, vv), ro,
                                              q1 < W ? (uint32_t)(4 * q1) : kBufOut, 0, 0);
      }
    }
  };
  // the barrier after compute orders the LDS fill after every wave's reads,
  // and the barrier after the fill orders it before the next compute
  const int64_t G = gridDim.x;
  int64_t smp = blockIdx.x;
  fetch(smp, va, xa);
  fetch(smp + G, vb, xb);
  put(0, va, xa);
  fetch(smp + 2 * G, va, xa);
  __syncthreads();
  while (true) {
    compute(0);
    __syncthreads();
    copy_out(smp);
    put(0, vb, xb);
    fetch(smp + 3 * G, vb, xb);
    __syncthreads();
    smp += G;
    if (smp >= B) break;
    compute(0);
    __syncthreads();
    copy_out(smp);
    put(0, va, xa);
    fetch(smp + 3 * G, va, xa);
    __syncthreads();
    smp += G;
    if (smp >= B) break;
  }
}

// Any T and dim: the same tiles, operands re-read for every tile.
__global__ __launch_bounds__(kBlock) void interaction_stream_kernel(
    const float* __restrict__ dense, const float* __restrict__ pooled, int64_t B, int T, int dim,
    int vec4, float* __restrict__ out) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r = lane % 16, g = lane / 16;
  const int64_t b = (int64_t)blockIdx.x * kWPB + wv;
  if (b >= B) return;
  const int64_t W = dim + (int64_t)T * (T + 1) / 2;
  const float* xb = dense + b * dim;
  const float* eb = pooled + b * (int64_t)T * dim;
  float* ob = out + b * W;
  for (int k = lane; k < dim; k += kWave) ob[k] = xb[k];
  const int nbp = (T + 15) / 16;
  for (int I = 0; I < nbp; ++I) {
    const int ti = 16 * I + r;
    const float* ri = ti < T ? eb + (int64_t)ti * dim : nullptr;
    float p = 0.0f;
    for (int k0 = 0; k0 < dim; k0 += 16) {
      const float4 a = ix_chunk(ri, k0 + 4 * g, dim, vec4), x = ix_chunk(xb, k0 + 4 * g, dim, vec4);
      p = __builtin_fmaf(a.x, x.x, p);
      p = __builtin_fmaf(a.y, x.y, p);
      p = __builtin_fmaf(a.z, x.z, p);
      p = __builtin_fmaf(a.w, x.w, p);
    }
    p = ix_col_sum(p);
    if (g == 0 && ti < T) ob[dim + (int64_t)(ti + 1) * ti / 2] = p;
    for (int J = 0; J <= I; ++J) {
      const int tj = 16 * J + r;
      const float* rj = tj < T ? eb + (int64_t)tj * dim : nullptr;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int k0 = 0; k0 < dim; k0 += 16)
        acc = mfma4(ix_chunk(ri, k0 + 4 * g, dim, vec4), ix_chunk(rj, k0 + 4 * g, dim, vec4), acc);
      ix_store_tile(ob, acc, I, J, r, g, T, dim);
    }
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

template <int BITS, int VEC, int LPR, int RG, typename IdxT>
int launch_bag_slice_t(const BagArgs& a, hipStream_t st) {
  constexpr int SLICE = LPR * RG;
  const int64_t threads = a.n_bags * SLICE;
  const int64_t blocks = (threads + kBlock - 1) / kBlock;
  if (blocks > 0x7fffffff) return QEMB_E_UNSUPPORTED;
  hipLaunchKernelGGL((bag_slice_kernel<BITS, VEC, LPR, RG, kBagUnroll, IdxT>), dim3((unsigned)blocks),
                     dim3(kBlock), 0, st, a.packed, a.S, a.total_rows, a.table_offsets, a.T, a.B,
                     a.dim, a.C, a.indices, a.offsets, a.nnz, a.weights, a.out,
                     a.err_count, a.n_bags, a.vec4);
  return launched();
}

template <int BITS, int VEC, int LPR, int RG>
int launch_bag_slice(const BagArgs& a, hipStream_t st) {
  if (a.idx64) return launch_bag_slice_t<BITS, VEC, LPR, RG, int64_t>(a, st);
  return launch_bag_slice_t<BITS, VEC, LPR, RG, int32_t>(a, st);
}

template <int BITS, int VEC, int LPR>
int dispatch_slice_rg(const BagArgs& a, int rg, hipStream_t st) {
  constexpr int MAXRG = (64 / LPR) < 16 ? (64 / LPR) : 16;
  if (rg > MAXRG) rg = MAXRG;
  switch (rg) {
    case 1: return launch_bag_slice<BITS, VEC, LPR, 1>(a, st);
    case 2: return launch_bag_slice<BITS, VEC, LPR, (2 <= MAXRG ? 2 : 1)>(a, st);
    case 4: return launch_bag_slice<BITS, VEC, LPR, (4 <= MAXRG ? 4 : 1)>(a, st);
    case 8: return launch_bag_slice<BITS, VEC, LPR, (8 <= MAXRG ? 8 : 1)>(a, st);
    default: return launch_bag_slice<BITS, VEC, LPR, (16 <= MAXRG ? 16 : 1)>(a, st);
  }
}

template <int BITS, int VEC>
int dispatch_slice(const BagArgs& a, int lpr, int rg, hipStream_t st) {
  switch (lpr) {
    case 1: return dispatch_slice_rg<BITS, VEC, 1>(a, rg, st);
    case 2: return dispatch_slice_rg<BITS, VEC, 2>(a, rg, st);
    case 4: return dispatch_slice_rg<BITS, VEC, 4>(a, rg, st);
    case 8: return dispatch_slice_rg<BITS, VEC, 8>(a, rg, st);
    case 16: return dispatch_slice_rg<BITS, VEC, 16>(a, rg, st);
    case 32: return dispatch_slice_rg<BITS, VEC, 32>(a, rg, st);
    default: return dispatch_slice_rg<BITS, VEC, 64>(a, rg, st);
  }
}

template <int BITS, int LPR, typename IdxT>
int launch_bag_wave_t(const BagArgs& a, hipStream_t st) {
  const int64_t blocks = (a.n_bags + kWPB * kWave - 1) / (kWPB * kWave);
  if (blocks > 0x7fffffff) return QEMB_E_UNSUPPORTED;
  hipLaunchKernelGGL((bag_wave_kernel<BITS, LPR, IdxT>), dim3((unsigned)blocks), dim3(kBlock), 0, st,
                     a.packed, a.S, a.total_rows, a.table_offsets, a.T, a.B, a.dim, a.C, a.indices,
                     a.offsets, a.nnz, a.weights, a.out, a.err_count, a.n_bags);
  return launched();
}

template <int BITS, int LPR, typename IdxT, bool PA4, bool WEIGHTED, bool PX>
int launch_bag_stream_w(const BagArgs& a, hipStream_t st) {
  const int64_t blocks = (a.n_bags + kWPB * kWave - 1) / (kWPB * kWave);
  if (blocks > 0x7fffffff) return QEMB_E_UNSUPPORTED;
  hipLaunchKernelGGL((bag_stream_kernel<BITS, LPR, IdxT, PA4, WEIGHTED, PX>), dim3((unsigned)blocks),
                     dim3(kBlock), 0, st, a.packed, a.S, a.total_rows, a.table_offsets, a.T, a.B,
                     a.dim, a.C, a.indices, a.offsets, a.nnz, a.weights, a.out, a.err_count,
                     a.n_bags);
  return launched();
}

template <int BITS, int LPR, typename IdxT, bool PA4, bool PX>
int launch_bag_stream_t(const BagArgs& a, hipStream_t st) {
  return a.weights ? launch_bag_stream_w<BITS, LPR, IdxT, PA4, true, PX>(a, st)
                   : launch_bag_stream_w<BITS, LPR, IdxT, PA4, false, PX>(a, st);
}

template <int BITS, int LPR>
int launch_bag_wave(const BagArgs& a, hipStream_t st) {
  return a.idx64 ? launch_bag_wave_t<BITS, LPR, int64_t>(a, st)
                 : launch_bag_wave_t<BITS, LPR, int32_t>(a, st);
}

template <int BITS, int LPR>
int launch_bag_stream(const BagArgs& a, hipStream_t st) {
  constexpr int VEC = StreamGeo<BITS, LPR>::VEC;
  if constexpr (VEC == 8) {
    if (a.C == LPR * VEC)  // codes fill the lanes; the scale/bias follows the last lane's codes
      return a.idx64 ? launch_bag_stream_t<BITS, LPR, int64_t, true, true>(a, st)
                     : launch_bag_stream_t<BITS, LPR, int32_t, true, true>(a, st);
  }
  if (a.C % 4 == 0)
    return a.idx64 ? launch_bag_stream_t<BITS, LPR, int64_t, true, false>(a, st)
                   : launch_bag_stream_t<BITS, LPR, int32_t, true, false>(a, st);
  return a.idx64 ? launch_bag_stream_t<BITS, LPR, int64_t, false, false>(a, st)
                 : launch_bag_stream_t<BITS, LPR, int32_t, false, false>(a, st);
}

template <int BITS>
int dispatch_wave(const BagArgs& a, hipStream_t st) {
  constexpr int VEC = WaveBag<BITS, 1>::VEC;
  const int lpr = next_pow2((a.C + VEC - 1) / VEC);
  switch (lpr) {
    case 1: return launch_bag_stream<BITS, 1>(a, st);
    case 2: return launch_bag_stream<BITS, 2>(a, st);
    case 4: return launch_bag_stream<BITS, 4>(a, st);
    case 8: return launch_bag_stream<BITS, 8>(a, st);
    case 16: return launch_bag_wave<BITS, 16>(a, st);
    case 32: return launch_bag_wave<BITS, 32>(a, st);
    default: return launch_bag_wave<BITS, 64>(a, st);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

int dispatch_bag_int2(const BagArgs& a, hipStream_t st) {
  const int64_t blocks = (a.n_bags + kWPB - 1) / kWPB;
  if (blocks > 0x7fffffff) return QEMB_E_UNSUPPORTED;
  const int np = (a.dim + 127) / 128;
  auto go = [&](auto idx_tag, auto np_tag) {
    using IdxT = decltype(idx_tag);
    constexpr int NP = decltype(np_tag)::value;
    constexpr int U = NP <= 2 ? 8 : NP == 4 ? 4 : 2;
    hipLaunchKernelGGL((bag_int2_kernel<IdxT, NP, U>), dim3((unsigned)blocks), dim3(kBlock), 0, st,
                       a.packed, a.S, a.total_rows, a.table_offsets, a.T, a.B, a.dim, a.C, a.indices,
                       a.offsets, a.nnz, a.weights, a.out, a.err_count, a.n_bags);
    return launched();
  };
  auto by_np = [&](auto idx_tag) {
    switch (np) {
      case 1: return go(idx_tag, std::integral_constant<int, 1>{});
      case 2: return go(idx_tag, std::integral_constant<int, 2>{});
      case 3:
      case 4: return go(idx_tag, std::integral_constant<int, 4>{});
      default: return go(idx_tag, std::integral_constant<int, 8>{});
    }
  };
  return a.idx64 ? by_np(int64_t{}) : by_np(int32_t{});
}

template <int BITS, int EPL, int LPR, int METHOD>
int launch_baseline(const float* x, int64_t rows, int dim, int C, int S, int vec4, float param,
                    uint8_t* packed, hipStream_t st) {
  hipLaunchKernelGGL((quantize_baseline_kernel<BITS, EPL, LPR, METHOD>),
                     dim3(grid_for(rows, kBlock / LPR, kGridCap)), dim3(kBlock), 0, st, x, rows, dim,
                     C, S, vec4, param, packed);
  return launched();
}

template <int BITS, int METHOD>
int baseline_by_dim(const float* x, int64_t rows, int dim, int C, int S, int vec4, float param,
                    uint8_t* packed, hipStream_t st) {
  switch (next_pow2(dim)) {
    case 1: return launch_baseline<BITS, 1, 1, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    case 2: return launch_baseline<BITS, 2, 1, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    case 4: return launch_baseline<BITS, 4, 1, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    case 8: return launch_baseline<BITS, 8, 1, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    case 16: return launch_baseline<BITS, 16, 1, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    case 32: return launch_baseline<BITS, 16, 2, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    case 64: return launch_baseline<BITS, 16, 4, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    case 128: return launch_baseline<BITS, 16, 8, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    case 256: return launch_baseline<BITS, 16, 16, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    case 512: return launch_baseline<BITS, 16, 32, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
    default: return launch_baseline<BITS, 16, 64, METHOD>(x, rows, dim, C, S, vec4, param, packed, st);
  }
}

template <int BITS>
int baseline_by_method(int method, const float* x, int64_t rows, int dim, int C, int S, int vec4,
                       float param, uint8_t* packed, hipStream_t st) {
  if (method == QEMB_BASE_SYMMETRIC)
    return baseline_by_dim<BITS, kBaseSym>(x, rows, dim, C, S, vec4, param, packed, st);
  if (method == QEMB_BASE_PERCENTILE)
    return baseline_by_dim<BITS, kBasePct>(x, rows, dim, C, S, vec4, param, packed, st);
  return baseline_by_dim<BITS, kBaseAciq>(x, rows, dim, C, S, vec4, param, packed, st);
}

template <int EPL, int LPR>
int launch_codebook(const float* x, int64_t rows, int dim, int S, int vec4, int n_iter,
                    uint8_t* packed, hipStream_t st) {
  hipLaunchKernelGGL((quantize_codebook_kernel<EPL, LPR>),
                     dim3(grid_for(rows, kBlock / LPR, kGridCap)), dim3(kBlock), 0, st, x, rows, dim,
                     S, vec4, n_iter, packed);
  return launched();
}

// P = next power of two >= dim: one lane per row up to 16 elements, else
// 16 elements per lane and P/16 lanes per row
int dispatch_codebook(const float* x, int64_t rows, int dim, int S, int vec4, int n_iter,
                      uint8_t* packed, hipStream_t st) {
  switch (next_pow2(dim)) {
    case 1: return launch_codebook<1, 1>(x, rows, dim, S, vec4, n_iter, packed, st);
    case 2: return launch_codebook<2, 1>(x, rows, dim, S, vec4, n_iter, packed, st);
    case 4: return launch_codebook<4, 1>(x, rows, dim, S, vec4, n_iter, packed, st);
    case 8: return launch_codebook<8, 1>(x, rows, dim, S, vec4, n_iter, packed, st);
    case 16: return launch_codebook<16, 1>(x, rows, dim, S, vec4, n_iter, packed, st);
    case 32: return launch_codebook<16, 2>(x, rows, dim, S, vec4, n_iter, packed, st);
    case 64: return launch_codebook<16, 4>(x, rows, dim, S, vec4, n_iter, packed, st);
    case 128: return launch_codebook<16, 8>(x, rows, dim, S, vec4, n_iter, packed, st);
    case 256: return launch_codebook<16, 16>(x, rows, dim, S, vec4, n_iter, packed, st);
    case 512: return launch_codebook<16, 32>(x, rows, dim, S, vec4, n_iter, packed, st);
    default: return launch_codebook<16, 64>(x, rows, dim, S, vec4, n_iter, packed, st);
  }
}

template <int NBP, int KC>
int launch_interaction(const float* dense, const float* pooled, int64_t B, int T, int dim, int vec4,
                       float* out, hipStream_t st) {
  hipLaunchKernelGGL((interaction_kernel<NBP, KC>), dim3((unsigned)((B + kWPB - 1) / kWPB)),
                     dim3(kBlock), 0, st, dense, pooled, B, T, dim, vec4, out);
  return launched();
}

template <int NBP, int KC>
int launch_interaction_lds(const float* dense, const float* pooled, int64_t B, int T, int dim,
                           float* out, hipStream_t st) {
  // three workgroups per CU (about 43 KB of LDS each at d = 128)
  const int64_t grid = B < 768 ? B : 768;
  const int64_t W = dim + (int64_t)T * (T + 1) / 2;
  if (W % 4 == 0 && ((uintptr_t)out & 15) == 0)
    hipLaunchKernelGGL((interaction_lds_kernel<NBP, KC, true>), dim3((unsigned)grid), dim3(kBlock), 0,
                       st, dense, pooled, B, T, dim, out);
  else
    hipLaunchKernelGGL((interaction_lds_kernel<NBP, KC, false>), dim3((unsigned)grid), dim3(kBlock), 0,
                       st, dense, pooled, B, T, dim, out);
  return launched();
}

template <int NBP>
int interaction_by_kc(const float* dense, const float* pooled, int64_t B, int T, int dim, int vec4,
                      float* out, hipStream_t st) {
  const int kc = (dim + 15) / 16;
  if (kc <= 2) return launch_interaction<NBP, 2>(dense, pooled, B, T, dim, vec4, out, st);
  if (kc <= 4) return launch_interaction<NBP, 4>(dense, pooled, B, T, dim, vec4, out, st);
  return launch_interaction<NBP, 8>(dense, pooled, B, T, dim, vec4, out, st);
}

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
  if (dim < 1 || dim > QEMB_MAX_DIM || (bits != 2 && bits != 4 && bits != 8)) return -1;
  return (code_bytes(dim, bits) + 4 + 15) / 16 * 16;
}

int qemb_quantize_rowwise(const float* x, int64_t rows, int32_t dim, int32_t bits,
                          int32_t clip_mode, int32_t n_bins, int32_t n_steps, uint8_t* packed,
                          qemb_stream_t stream) {
  if (rows < 0 || dim < 1 || (bits != 2 && bits != 4 && bits != 8)) return QEMB_E_INVALID_ARG;
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
    if (bits == 2) return baseline_by_dim<2, kBaseRange>(x, rows, dim, C, S, vec4, 0.0f, packed, st);
    return bits == 4 ? dispatch_range<4>(x, rows, dim, C, S, vec4, packed, st)
                     : dispatch_range<8>(x, rows, dim, C, S, vec4, packed, st);
  }
  if (bits == 2) return dispatch_greedy<2>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
  return bits == 4 ? dispatch_greedy<4>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st)
                   : dispatch_greedy<8>(x, rows, dim, C, S, vec4, n_bins, n_steps, packed, st);
}

int qemb_dequantize(const uint8_t* packed, int64_t rows, int32_t dim, int32_t bits, float* y,
                    qemb_stream_t stream) {
  if (rows < 0 || dim < 1 || (bits != 2 && bits != 4 && bits != 8)) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (rows == 0) return QEMB_OK;
  if (!packed || !y) return QEMB_E_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(y)) return QEMB_E_MISALIGNED;
  const int C = (int)code_bytes(dim, bits);
  const int S = (int)qemb_row_stride(dim, bits);
  const int vec4 = (dim % 4 == 0);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (bits == 2) return dispatch_dequant<2>(packed, rows, dim, C, S, vec4, y, st);
  return bits == 4 ? dispatch_dequant<4>(packed, rows, dim, C, S, vec4, y, st)
                   : dispatch_dequant<8>(packed, rows, dim, C, S, vec4, y, st);
}

int qemb_bag_forward(const uint8_t* packed, int64_t total_rows, const int64_t* table_offsets,
                     int32_t T, int64_t B, int32_t dim, int32_t bits, const void* indices,
                     const void* offsets, int64_t nnz, int32_t index_type, int32_t pool_mode,
                     const float* weights, float* out, int32_t* err_count,
                     qemb_stream_t stream) {
  if (T < 0 || B < 0 || dim < 1 || (bits != 2 && bits != 4 && bits != 8) || total_rows < 0 || nnz < 0)
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
  if (bits == 2) return dispatch_bag_int2(a, st);
  // multi-hot bags (8+ ids on average): one wave per bag
  const int64_t mean_len = (nnz + a.n_bags - 1) / a.n_bags;
  if (mean_len >= 8) return bits == 4 ? dispatch_wave<4>(a, st) : dispatch_wave<8>(a, st);
  // short bags: several bags per wave; 8-byte code chunks per lane (16-byte
  // for INT8 rows wider than 512 codes), about kBagUnroll rows per group
  const int64_t chunks8 = (a.C + 7) / 8;
  const int vec = chunks8 > 64 ? 16 : 8;
  const int lpr = next_pow2((a.C + vec - 1) / vec);
  const int rg = next_pow2((mean_len + kBagUnroll - 1) / kBagUnroll);
  if (bits == 4) return dispatch_slice<4, 8>(a, lpr, rg, st);
  if (vec == 8) return dispatch_slice<8, 8>(a, lpr, rg, st);
  return dispatch_slice_rg<8, 16, 64>(a, rg, st);  // only rows wider than 512 codes get here
}

size_t qemb_l2_error_workspace_bytes(void) { return (size_t)kL2Blocks * 4 * sizeof(double); }

int qemb_quantize_baseline(const float* x, int64_t rows, int32_t dim, int32_t bits, int32_t method,
                           float param, uint8_t* packed, qemb_stream_t stream) {
  if (rows < 0 || dim < 1 || (bits != 2 && bits != 4 && bits != 8)) return QEMB_E_INVALID_ARG;
  if (method != QEMB_BASE_SYMMETRIC && method != QEMB_BASE_PERCENTILE && method != QEMB_BASE_ACIQ)
    return QEMB_E_INVALID_ARG;
  if (method == QEMB_BASE_PERCENTILE && !(param >= 0.5f && param <= 1.0f)) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (rows == 0) return QEMB_OK;
  if (!x || !packed) return QEMB_E_INVALID_ARG;
  if (!aligned16(x) || !aligned16(packed)) return QEMB_E_MISALIGNED;
  const int C = (int)code_bytes(dim, bits), S = (int)qemb_row_stride(dim, bits);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int vec4 = dim % 4 == 0;
  if (bits == 2) return baseline_by_method<2>(method, x, rows, dim, C, S, vec4, param, packed, st);
  return bits == 4 ? baseline_by_method<4>(method, x, rows, dim, C, S, vec4, param, packed, st)
                   : baseline_by_method<8>(method, x, rows, dim, C, S, vec4, param, packed, st);
}

int64_t qemb_codebook_row_stride(int32_t dim) {
  if (dim < 1 || dim > QEMB_MAX_DIM) return -1;
  return (64 + ((int64_t)dim + 1) / 2 + 15) / 16 * 16;
}

int qemb_quantize_codebook(const float* x, int64_t rows, int32_t dim, int32_t n_iter,
                           uint8_t* packed, qemb_stream_t stream) {
  if (rows < 0 || dim < 1 || n_iter < 0) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (rows == 0) return QEMB_OK;
  if (!x || !packed) return QEMB_E_INVALID_ARG;
  if (!aligned16(x) || !aligned16(packed)) return QEMB_E_MISALIGNED;
  return dispatch_codebook(x, rows, dim, (int)qemb_codebook_row_stride(dim), dim % 4 == 0, n_iter,
                           packed, reinterpret_cast<hipStream_t>(stream));
}

int qemb_dequantize_codebook(const uint8_t* packed, int64_t rows, int32_t dim, float* y,
                             qemb_stream_t stream) {
  if (rows < 0 || dim < 1) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (rows == 0) return QEMB_OK;
  if (!packed || !y) return QEMB_E_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(y)) return QEMB_E_MISALIGNED;
  constexpr int kRowsPerBlock = kBlock / kCbLevels;
  const dim3 grid(grid_for(rows, kRowsPerBlock, kGridCap));
  const int S = (int)qemb_codebook_row_stride(dim);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dim <= 64)
    hipLaunchKernelGGL(dequant_codebook_kernel<4>, grid, dim3(kBlock), 0, st, packed, rows, dim, S, y);
  else
    hipLaunchKernelGGL(dequant_codebook_kernel<8>, grid, dim3(kBlock), 0, st, packed, rows, dim, S, y);
  return launched();
}

int qemb_bag_forward_codebook(const uint8_t* packed, int64_t total_rows,
                              const int64_t* table_offsets, int32_t T, int64_t B, int32_t dim,
                              const void* indices, const void* offsets, int64_t nnz,
                              int32_t index_type, int32_t pool_mode, const float* weights,
                              float* out, int32_t* err_count, qemb_stream_t stream) {
  if (T < 0 || B < 0 || dim < 1 || total_rows < 0 || nnz < 0) return QEMB_E_INVALID_ARG;
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
  const int64_t n_bags = (int64_t)T * B;
  const int64_t blocks = (n_bags + kWPB - 1) / kWPB;
  if (blocks > 0x7fffffff) return QEMB_E_UNSUPPORTED;
  const float* w = pool_mode == QEMB_POOL_WEIGHTED_SUM ? weights : nullptr;
  const int64_t S = qemb_codebook_row_stride(dim);
  const int np = (dim + 127) / 128;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  auto go = [&](auto idx_tag, auto np_tag) {
    using IdxT = decltype(idx_tag);
    constexpr int NP = decltype(np_tag)::value;
    constexpr int U = NP == 1 ? 8 : NP == 2 ? 4 : NP == 4 ? 4 : 2;
    hipLaunchKernelGGL((bag_codebook_kernel<IdxT, NP, U>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       st, packed, S, total_rows, table_offsets, T, B, dim, indices, offsets, nnz,
                       w, out, err_count, n_bags);
    return launched();
  };
  auto by_np = [&](auto idx_tag) {
    switch (np) {
      case 1: return go(idx_tag, std::integral_constant<int, 1>{});
      case 2: return go(idx_tag, std::integral_constant<int, 2>{});
      case 3:
      case 4: return go(idx_tag, std::integral_constant<int, 4>{});
      default: return go(idx_tag, std::integral_constant<int, 8>{});
    }
  };
  return index_type == QEMB_INDEX_INT64 ? by_np(int64_t{}) : by_np(int32_t{});
}

int64_t qemb_interaction_width(int32_t T, int32_t dim) {
  if (T < 0 || T > QEMB_MAX_INTERACTION_T || dim < 1 || dim > QEMB_MAX_DIM) return -1;
  return (int64_t)dim + (int64_t)T * (T + 1) / 2;
}

int qemb_dot_interaction(const float* dense, const float* pooled, int64_t B, int32_t T,
                         int32_t dim, float* out, qemb_stream_t stream) {
  if (B < 0 || T < 0 || dim < 1) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM || T > QEMB_MAX_INTERACTION_T) return QEMB_E_UNSUPPORTED;
  if (B == 0) return QEMB_OK;
  if (!dense || !out || (T > 0 && !pooled)) return QEMB_E_INVALID_ARG;
  if (!aligned16(dense) || (pooled && !aligned16(pooled)) || !aligned16(out)) return QEMB_E_MISALIGNED;
  if ((B + kWPB - 1) / kWPB > 0x7fffffff) return QEMB_E_UNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int vec4 = dim % 4 == 0;
  if (vec4 && dim > 64 && dim <= 128 && T > 48 && T <= 64)
    return launch_interaction_lds<4, 8>(dense, pooled, B, T, dim, out, st);
  if (dim <= 128 && T <= 64) {
    switch ((T + 15) / 16) {
      case 0:
      case 1: return interaction_by_kc<1>(dense, pooled, B, T, dim, vec4, out, st);
      case 2: return interaction_by_kc<2>(dense, pooled, B, T, dim, vec4, out, st);
      case 3: return interaction_by_kc<3>(dense, pooled, B, T, dim, vec4, out, st);
      default: return interaction_by_kc<4>(dense, pooled, B, T, dim, vec4, out, st);
    }
  }
  hipLaunchKernelGGL(interaction_stream_kernel, dim3((unsigned)((B + kWPB - 1) / kWPB)), dim3(kBlock),
                     0, st, dense, pooled, B, T, dim, vec4, out);
  return launched();
}

int qemb_l2_error_codebook(const float* x, const uint8_t* packed, int64_t rows, int32_t dim,
                           void* workspace, double* out4, qemb_stream_t stream) {
  if (rows < 0 || dim < 1) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (!workspace || !out4 || (rows > 0 && (!x || !packed))) return QEMB_E_INVALID_ARG;
  if ((x && !aligned16(x)) || (packed && !aligned16(packed)) || !aligned16(workspace))
    return QEMB_E_MISALIGNED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  double* part = reinterpret_cast<double*>(workspace);
  hipLaunchKernelGGL(l2_partial_codebook_kernel, dim3(kL2Blocks), dim3(kBlock), 0, st, x, packed,
                     rows, dim, (int)qemb_codebook_row_stride(dim), part);
  if (launched() != QEMB_OK) return QEMB_E_LAUNCH;
  hipLaunchKernelGGL(l2_final_kernel, dim3(1), dim3(kBlock), 0, st, part, out4);
  return launched();
}

int qemb_l2_error(const float* x, const uint8_t* packed, int64_t rows, int32_t dim, int32_t bits,
                  void* workspace, double* out4, qemb_stream_t stream) {
  if (rows < 0 || dim < 1 || (bits != 2 && bits != 4 && bits != 8)) return QEMB_E_INVALID_ARG;
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
