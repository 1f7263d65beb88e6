// qemb.hip -- row-wise INT4/INT8 quantized embedding tables on gfx950.
//
// Kernels and the C ABI declared in include/qemb.h:
//   * quantize_range_kernel   row range -> fp16 scale/bias -> codes -> packed row
//   * quantize_greedy_kernel  greedy clip search on the row's squared error,
//                             then the same encoding
//   * dequant_kernel          packed rows -> fp32
//   * bag_stream_kernel       fused decode + (weighted) sum pooling of multi-hot
//                             bags, pipelined over batches of ids
//   * bag_pack_kernel         the same over runs of 64 bags whose ids are packed
//                             into full batches (bags of a few to a few tens of ids)
//   * bag_seg_kernel          the same for rows of 128 codes in 8 lanes (INT4,
//                             INT2): runs of bags cut into equal chunks per row
//                             group, bag sums kept in LDS
//   * bag_wave_kernel         the same for rows wider than 8 lanes
//   * bag_slice_kernel        the same for short bags, several bags per wave
//   * l2_partial/l2_final     normalized l2 error, fixed-order reduction
//   * compress_* / decompress error-bounded compression of pooled vectors
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

#include <mutex>
#include <type_traits>
#include <utility>

#include "qemb.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;

#include "common.inc"
#include "quantize.inc"
#include "lookup.inc"
#include "pack.inc"
#include "seg.inc"
#include "l2_error.inc"
#include "baselines.inc"
#include "codebook.inc"
#include "interaction.inc"
#include "compress.inc"
#include "host.inc"

}  // namespace

// Workspace of qemb_compress_pooled_noalloc: the per-block record sizes and
// the per-vector widths of up to QEMB_COMPRESS_NOALLOC_MAX_VECTORS vectors.
// In host code `scratch` is only a handle; its device address on each GPU
// comes from hipGetSymbolAddress (scratch_device_ptr).
constexpr int64_t kNoAllocBlocks = (QEMB_COMPRESS_NOALLOC_MAX_VECTORS + kCmpVPB - 1) / kCmpVPB;
constexpr size_t kNoAllocScratchBytes =
    8 * kNoAllocBlocks + ((QEMB_COMPRESS_NOALLOC_MAX_VECTORS + 15) / 16) * 16;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (null until looked up)

// The device address of `scratch` on the device of `st` (the current device
// for the null stream), looked up once per device with that device current.
int scratch_device_ptr(hipStream_t st, void** ptr) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return QEMB_E_LAUNCH;
  int dev = cur;
  if (st != nullptr && hipStreamGetDevice(st, &dev) != hipSuccess) return QEMB_E_INVALID_ARG;
  if (dev < 0 || dev >= kMaxDevices) return QEMB_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return QEMB_E_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return QEMB_E_LAUNCH;
    if (e != hipSuccess || p == nullptr) return QEMB_E_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return QEMB_OK;
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
    case QEMB_E_TOO_LARGE: return "more vectors than the no-allocation entry point's maximum";
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
  // Kernel choice by row width (lanes of 16 codes per row) and mean bag
  // length, from timings of the bag kernels over bag-length mixes:
  //   rows of 128 codes in 8 lanes (INT4 d 127..128, INT2 d 125..128), two
  //     or more ids per bag on average: runs of 24 bags cut into equal
  //     chunks per row group, bag sums in LDS;
  //   rows of 4..8 lanes, mean length up to 16 (24 for INT4): runs of 64
  //     bags packed into full id batches;
  //   rows of 1..2 lanes, mean length up to 16, and wider rows with bags of
  //     under 8 ids: several bags per wave;
  //   longer bags: one wave per bag (the stream kernel up to 8 lanes per
  //     row, the wave kernel beyond).
  const int64_t mean_len = (nnz + a.n_bags - 1) / a.n_bags;
  if (seg_fits(a, bits) && nnz >= 2 * a.n_bags)
    return bits == 4 ? dispatch_seg<4>(a, st) : dispatch_seg<2>(a, st);
  if (bits == 2) {
    const int lpr = pack_lanes<2>(a);
    if (lpr >= 4 && mean_len <= 16) return dispatch_pack<2>(a, st);
    if (mean_len > 16 || (lpr < 0 && mean_len >= 8)) return dispatch_wave<2>(a, st);
    // several bags per wave, 4-byte code chunks (16 codes) per lane
    return dispatch_slice<2, 4>(a, next_pow2((a.C + 3) / 4), next_pow2((mean_len + kBagUnroll - 1) / kBagUnroll),
                                st);
  }
  const int lpr = bits == 4 ? pack_lanes<4>(a) : pack_lanes<8>(a);
  if (lpr >= 4 && mean_len <= (bits == 4 ? 24 : 16))
    return bits == 4 ? dispatch_pack<4>(a, st) : dispatch_pack<8>(a, st);
  if (mean_len > 16 || (lpr < 0 && mean_len >= 8))
    return bits == 4 ? dispatch_wave<4>(a, st) : dispatch_wave<8>(a, st);
  // several bags per wave; 8-byte code chunks per lane (16-byte for INT8
  // rows wider than 512 codes), about kBagUnroll rows per group
  const int64_t chunks8 = (a.C + 7) / 8;
  const int vec = chunks8 > 64 ? 16 : 8;
  const int slpr = next_pow2((a.C + vec - 1) / vec);
  const int rg = next_pow2((mean_len + kBagUnroll - 1) / kBagUnroll);
  if (bits == 4) return dispatch_slice<4, 8>(a, slpr, rg, st);
  if (vec == 8) return dispatch_slice<8, 8>(a, slpr, rg, st);
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
  // short bags (fewer than 8 ids on average): four bags per wave
  const bool short_bags = (nnz + n_bags - 1) / n_bags < 8;
  auto go = [&](auto idx_tag, auto np_tag) {
    using IdxT = decltype(idx_tag);
    constexpr int NP = decltype(np_tag)::value;
    constexpr int U = NP == 1 ? 8 : NP == 2 ? 4 : NP == 4 ? 4 : 2;
    if (short_bags) {
      hipLaunchKernelGGL((bag_codebook_short_kernel<IdxT, NP>),
                         dim3((unsigned)((n_bags + kBlock / kCbLevels - 1) / (kBlock / kCbLevels))), dim3(kBlock),
                         0, st, packed, S, total_rows, table_offsets, T, B, dim, indices, offsets, nnz, w, out,
                         err_count, n_bags);
    } else {
      hipLaunchKernelGGL((bag_codebook_kernel<IdxT, NP, U>), dim3((unsigned)blocks), dim3(kBlock), 0,
                         st, packed, S, total_rows, table_offsets, T, B, dim, indices, offsets, nnz,
                         w, out, err_count, n_bags);
    }
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

int64_t qemb_compress_record_bytes(int32_t dim, int32_t w) {
  if (dim < 1 || dim > QEMB_MAX_DIM || w < 0 || w > QEMB_COMPRESS_VERBATIM) return -1;
  return 4 + 4 * (w == QEMB_COMPRESS_VERBATIM ? (int64_t)dim : ((int64_t)dim * w + 31) / 32);
}

int64_t qemb_compress_bound(int64_t n, int32_t dim) {
  if (n < 0 || dim < 1 || dim > QEMB_MAX_DIM || n > INT64_MAX / (4 + 4 * (int64_t)dim)) return -1;
  return n * (4 + 4 * (int64_t)dim);
}

size_t qemb_compress_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  const int64_t nblk = (n + kCmpVPB - 1) / kCmpVPB;
  return (size_t)(8 * nblk + ((n + 15) / 16) * 16);
}

int qemb_compress_pooled(const float* x, int64_t n, int32_t dim, int32_t T, const float* eb,
                         uint8_t* out, int64_t* offs, void* workspace, qemb_stream_t stream) {
  if (n < 0 || dim < 1 || T < 1) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (!offs || (n > 0 && (!x || !eb || !out || !workspace))) return QEMB_E_INVALID_ARG;
  if ((x && !aligned16(x)) || ((uintptr_t)out & 3u) || ((uintptr_t)offs & 7u) ||
      ((uintptr_t)eb & 3u) || (workspace && !aligned16(workspace)))
    return QEMB_E_MISALIGNED;
  const int64_t nblk = (n + kCmpVPB - 1) / kCmpVPB;
  if (nblk > 0x7fffffff) return QEMB_E_UNSUPPORTED;
  int64_t* bsum = reinterpret_cast<int64_t*>(workspace);
  uint8_t* wbuf = reinterpret_cast<uint8_t*>(workspace) + 8 * nblk;
  return dispatch_compress(x, n, dim, T, eb, out, offs, bsum, wbuf, reinterpret_cast<hipStream_t>(stream));
}

int qemb_compress_pooled_noalloc(const float* x, int64_t n, int32_t dim, int32_t T, const float* eb,
                                 uint8_t* out, int64_t* offs, qemb_stream_t stream) {
  if (n < 0 || dim < 1 || T < 1) return QEMB_E_INVALID_ARG;
  if (n > QEMB_COMPRESS_NOALLOC_MAX_VECTORS) return QEMB_E_TOO_LARGE;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (!offs || (n > 0 && (!x || !eb || !out))) return QEMB_E_INVALID_ARG;
  if ((x && !aligned16(x)) || ((uintptr_t)out & 3u) || ((uintptr_t)offs & 7u) || ((uintptr_t)eb & 3u))
    return QEMB_E_MISALIGNED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const int rc = scratch_device_ptr(st, &ws);
  if (rc != QEMB_OK) return rc;
  const int64_t nblk = (n + kCmpVPB - 1) / kCmpVPB;  // <= kNoAllocBlocks
  int64_t* bsum = reinterpret_cast<int64_t*>(ws);
  uint8_t* wbuf = reinterpret_cast<uint8_t*>(ws) + 8 * nblk;
  return dispatch_compress(x, n, dim, T, eb, out, offs, bsum, wbuf, st);
}

int qemb_decompress_pooled(const uint8_t* in, int64_t in_bytes, const int64_t* offs, int64_t n,
                           int32_t dim, int32_t T, const float* eb, float* y, int32_t* err_count,
                           qemb_stream_t stream) {
  if (n < 0 || dim < 1 || T < 1 || in_bytes < 0) return QEMB_E_INVALID_ARG;
  if (dim > QEMB_MAX_DIM) return QEMB_E_UNSUPPORTED;
  if (n == 0) return QEMB_OK;
  if (!offs || !eb || !y || (in_bytes > 0 && !in)) return QEMB_E_INVALID_ARG;
  if (((uintptr_t)in & 3u) || ((uintptr_t)offs & 7u) || ((uintptr_t)eb & 3u) || !aligned16(y))
    return QEMB_E_MISALIGNED;
  const int64_t nblk = (n + kCmpVPB - 1) / kCmpVPB;
  if (nblk > 0x7fffffff) return QEMB_E_UNSUPPORTED;
  return dispatch_decompress(in, in_bytes, offs, n, dim, T, eb, y, err_count,
                             reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
