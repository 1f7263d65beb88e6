// gather_floor.hip -- libqemb_floor.so, a measurement aid beside libqemb.so
// (not part of the library's C ABI; bench.py --gather-floor runs it, and
// every bench run times its streaming ceilings, at the end of this file).
//
// The memory traffic of one pooled lookup call over packed rows of up to 8
// lanes x 8 code bytes (INT4 rows of d <= 128), with none of its arithmetic:
// every id of the batch is read once, contiguously (the cheapest order the
// CSR layout allows), with its weight; every row it names is read the way the
// lookup reads rows (8 lanes per row, each lane 12 bytes: 8 code bytes and
// the next 4, which for the last lane are the row's fp16 scale and bias);
// and as many output bytes as the lookup writes are written, in coalesced
// wave-wide stores.  No decode, no pooling, no bag bookkeeping: the time of
// this kernel is a floor for any lookup kernel that reads rows this way.
//
// Work mapping as in the lookup: a wave takes `run` batches of 64 ids of one
// table (the table's ids are contiguous in the batch), waves of a table are
// consecutive, and consecutive block ids go round-robin over the 8 XCDs so
// that each XCD works through a contiguous range of tables.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWave = 64;
constexpr int kWPB = 4;
constexpr int kLPR = 8;                  // lanes per row
constexpr int kRG = kWave / kLPR;        // rows per load instruction
constexpr uint32_t kBufWord3 = 0x00020000u;
constexpr uint32_t kBufOut = 0x80000000u;  // an offset past every descriptor's range

__device__ __forceinline__ uint32_t bperm(int byte_addr, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(byte_addr, (int)v);
}

struct Rows {
  uint32_t v[kLPR][3];
};

// wave w: table wave_table[w], chunk w - wave_start[table] of that table's ids
__global__ __launch_bounds__(kWPB * kWave) void gather_floor_kernel(
    const uint8_t* __restrict__ packed, int64_t S, const int64_t* __restrict__ table_offsets,
    const int64_t* __restrict__ id_start, const int32_t* __restrict__ wave_table,
    const int64_t* __restrict__ wave_start, int64_t n_waves, const int32_t* __restrict__ ids,
    const float* __restrict__ weights, int run, uint8_t* __restrict__ out, int64_t out_bytes,
    int64_t out_per_wave, uint32_t* __restrict__ sink) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane / kLPR, s = lane % kLPR;
  const int64_t nbk = gridDim.x, xcd = blockIdx.x % 8, kk = blockIdx.x / 8;
  const int64_t qf = nbk / 8, rr = nbk % 8;
  const int64_t blk = xcd * qf + (xcd < rr ? xcd : rr) + kk;
  const int64_t w = blk * kWPB + wv;
  if (w >= n_waves) return;
  const int t = wave_table[w];
  const int64_t i0 = id_start[t] + (w - wave_start[t]) * (int64_t)kWave * run;  // first id of the chunk
  const int64_t i1 = id_start[t + 1];
  const int64_t n_ids = (i1 - i0) < (int64_t)kWave * run ? (i1 - i0) : (int64_t)kWave * run;
  const int64_t r0 = table_offsets[t], n_rows = table_offsets[t + 1] - r0;
  const __amdgpu_buffer_rsrc_t tab = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(packed + r0 * S), (short)0, (int)(n_rows * S), kBufWord3);
  const __amdgpu_buffer_rsrc_t rid = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ids + i0), (short)0, (int)(n_ids * 4), kBufWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(weights + i0), (short)0, (int)(n_ids * 4), kBufWord3);
  // this wave's share of the output: out_per_wave bytes per wave
  const int64_t o0 = w * out_per_wave;
  const int64_t o1 = (o0 + out_per_wave) < out_bytes ? o0 + out_per_wave : out_bytes;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(out + (o0 < out_bytes ? o0 : 0)), (short)0, (int)(o1 > o0 ? o1 - o0 : 0), kBufWord3);
  const int store_bytes = (int)(out_per_wave / (run > 0 ? run : 1)) & ~511;  // per batch

  uint32_t acc = 0;
  auto issue = [&](Rows& R, uint32_t id) {
    const uint32_t own = id < (uint32_t)n_rows ? id * (uint32_t)S : kBufOut;
#pragma unroll
    for (int u = 0; u < kLPR; ++u) {
      const uint32_t bo = bperm((u * kRG + g) * 4, own) + (uint32_t)(s * 8);
      const auto v = __builtin_amdgcn_raw_buffer_load_b96(tab, bo, 0, 0);
      R.v[u][0] = v[0];
      R.v[u][1] = v[1];
      R.v[u][2] = v[2];
    }
  };
  auto consume = [&](const Rows& R) {
#pragma unroll
    for (int u = 0; u < kLPR; ++u) acc += R.v[u][0] ^ R.v[u][1] ^ R.v[u][2];
  };
  // two batches of rows in flight: step k issues batch k + 1's rows (its ids
  // came one step earlier), requests batch k + 2's ids and weights, reads
  // batch k's rows and writes batch k's share of the output.  Steps run in
  // pairs (run is even) so both row buffers keep fixed registers.
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  Rows R[2];
  uint32_t idb[2];
  idb[0] = __builtin_amdgcn_raw_buffer_load_b32(rid, lane * 4, 0, 0);
  idb[1] = __builtin_amdgcn_raw_buffer_load_b32(rid, (kWave + lane) * 4, 0, 0);
  acc += __builtin_amdgcn_raw_buffer_load_b32(rw, lane * 4, 0, 0);
  acc += __builtin_amdgcn_raw_buffer_load_b32(rw, (kWave + lane) * 4, 0, 0);
  issue(R[0], idb[0]);
  auto step = [&](Rows& cur, Rows& nxt, uint32_t& idn, int k) {
    issue(nxt, idn);
    idn = __builtin_amdgcn_raw_buffer_load_b32(rid, ((k + 2) * kWave + lane) * 4, 0, 0);
    acc += __builtin_amdgcn_raw_buffer_load_b32(rw, ((k + 2) * kWave + lane) * 4, 0, 0);
    consume(cur);
    for (int b = 0; b < store_bytes; b += 512)
      __builtin_amdgcn_raw_buffer_store_b64(u2{acc, acc ^ 1u}, ro, k * store_bytes + b + lane * 8, 0, 2);
  };
  for (int k = 0; k < run; k += 2) {
    step(R[0], R[1], idb[1], k);
    step(R[1], R[0], idb[0], k + 1);
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads live
}

// Streaming ceilings: HBM rates of the plainest access patterns, for the
// rooflines of the streaming kernels.  mode 0 reads n 16-byte words (folded
// into one word per workgroup), mode 1 writes them, mode 2 copies them; each
// lane moves U words per round with non-temporal loads and stores, rounds
// strided over the whole grid.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void stream_ceiling_kernel(const v4u* __restrict__ in, v4u* __restrict__ out,
                                                             int64_t n, int mode, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    if (mode == 1) {
#pragma unroll
      for (int r = 0; r < U; ++r) __builtin_nontemporal_store(v4u{(unsigned)r, 0u, 0u, 0u}, out + i + r * stride);
    } else {
      v4u v[U];
#pragma unroll
      for (int r = 0; r < U; ++r) v[r] = __builtin_nontemporal_load(in + i + r * stride);
      if (mode == 2) {
#pragma unroll
        for (int r = 0; r < U; ++r) __builtin_nontemporal_store(v[r], out + i + r * stride);
      } else {
#pragma unroll
        for (int r = 0; r < U; ++r) acc ^= v[r].x ^ v[r].y ^ v[r].z ^ v[r].w;
      }
    }
  }
  for (; i < n; i += stride) {
    if (mode == 1) {
      out[i] = v4u{0u, 0u, 0u, 0u};
    } else {
      const v4u v = in[i];
      if (mode == 2) {
        out[i] = v;
      } else {
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
  }
  if (mode == 0 && acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads live
}

}  // namespace

extern "C" {

// Launch the floor kernel (see the top of this file).  All arrays are device
// arrays: packed [rows][S]; table_offsets [T + 1]; id_start [T + 1] (table
// t's ids are ids[id_start[t] .. id_start[t + 1])); wave_table [n_waves],
// wave_start [T + 1] (table t's waves are wave_start[t] .. wave_start[t + 1]
// - 1, each taking up to 64 * run ids, run even); out of out_bytes bytes, of which wave
// w writes bytes [w out_bytes_per_wave, (w + 1) out_bytes_per_wave) (clipped
// to out_bytes); sink one uint32.  Every table must be under 2 GB of rows
// (rows are read through a buffer descriptor).  Returns 0, or -1 on bad
// arguments, -4 if the launch failed.
int qemb_floor_gather(const uint8_t* packed, int64_t S, const int64_t* table_offsets, const int64_t* id_start,
                      const int32_t* wave_table, const int64_t* wave_start, int64_t n_waves, const int32_t* ids,
                      const float* weights, int32_t run, uint8_t* out, int64_t out_bytes,
                      int64_t out_bytes_per_wave, uint32_t* sink, hipStream_t stream) {
  if (!packed || S < 12 || !table_offsets || !id_start || !wave_table || !wave_start || n_waves < 0 || !ids ||
      !weights || run < 2 || run % 2 != 0 || !out || out_bytes < 0 || out_bytes_per_wave < 0 || !sink)
    return -1;
  if (n_waves == 0) return 0;
  const int64_t blocks = (n_waves + kWPB - 1) / kWPB;
  if (blocks > 0x7fffffff) return -1;
  hipLaunchKernelGGL(gather_floor_kernel, dim3((unsigned)blocks), dim3(kWPB * kWave), 0, stream, packed, S,
                     table_offsets, id_start, wave_table, wave_start, n_waves, ids, weights, (int)run, out,
                     out_bytes, out_bytes_per_wave, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Launch the streaming-ceiling kernel (see above) on `grid` workgroups of
// 256 lanes with u (2, 4 or 8) words per lane and round: in and out device
// arrays of n 16-byte words (in unused for mode 1, out for mode 0), sink one
// uint32.  Returns 0, -1 on bad arguments, -4 if the launch failed.
int qemb_floor_stream(const void* in, void* out, int64_t n, int32_t mode, int32_t grid, int32_t u, uint32_t* sink,
                      hipStream_t stream) {
  if (n < 0 || mode < 0 || mode > 2 || grid < 1 || !sink || (mode != 1 && !in) || (mode != 0 && !out) ||
      (u != 2 && u != 4 && u != 8))
    return -1;
  if (n == 0) return 0;
  const v4u* src = static_cast<const v4u*>(in);
  v4u* dst = static_cast<v4u*>(out);
  if (u == 2) {
    hipLaunchKernelGGL(stream_ceiling_kernel<2>, dim3(grid), dim3(256), 0, stream, src, dst, n, (int)mode, sink);
  } else if (u == 4) {
    hipLaunchKernelGGL(stream_ceiling_kernel<4>, dim3(grid), dim3(256), 0, stream, src, dst, n, (int)mode, sink);
  } else {
    hipLaunchKernelGGL(stream_ceiling_kernel<8>, dim3(grid), dim3(256), 0, stream, src, dst, n, (int)mode, sink);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
