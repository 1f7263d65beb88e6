/*
 * qemb.h -- C ABI of libqemb: row-wise INT4/INT8 quantized embedding tables
 * on AMD Instinct MI355X (gfx950).
 *
 * Operations (the pages state them in prose; the exact numeric rules are the
 * project's readings of those passages):
 *
 *  - Row-wise uniform quantization: every table row gets its own scale and
 *    bias, stored as binary16, and 4- or 8-bit codes; the clipping window is
 *    either the row's range or the result of a greedy search that lowers the
 *    row's squared error ("Post-Training 4-bit Quantization on Embedding
 *    Tables", review page, sections "Proposed method" and "Main findings").
 *  - 4-bit codes are bit-packed two per byte (DQRM repository page, the
 *    paragraph on the Android demo); 2-bit codes, one of the widths the
 *    quantizer comparison uses, four per byte.
 *  - Pooled lookup: sparse categorical ids select rows of many embedding
 *    tables and each bag of ids is reduced to one dense vector ("Deep
 *    Learning Recommendation Model for Personalization and Recommendation
 *    Systems", review page, "Proposed method").
 *  - Normalized l2 quantization error ("Post-Training 4-bit Quantization on
 *    Embedding Tables", review page, "Proposed method").
 *  - Codebook rows (16 fp32 levels from 1-D k-means, 4-bit codes) and the
 *    quantizer baselines the same page compares against; the dot
 *    interaction of the pooled vectors (DLRM page, "Proposed method"); the
 *    error-bounded compression of the pooled vectors a table-sharded model
 *    exchanges ("Avancées dans les recommandations en Deep Learning",
 *    scisimple page).  Each is stated with its entry points below.
 *
 * Packed row layout (stride S bytes, S = 16 * ceil((C + 4) / 16),
 * C = ceil(dim * bits / 8)):
 *     bytes [0, C)      codes; INT4: element 2k in the low nibble of byte k,
 *                       element 2k+1 in the high nibble (0 for odd dim);
 *                       INT8: element k in byte k; INT2: element 4k+j in
 *                       bits [2j, 2j+2) of byte k
 *     bytes [C, C+2)    scale, binary16, little-endian
 *     bytes [C+2, C+4)  bias,  binary16, little-endian
 *     bytes [C+4, S)    zero
 * Element k of a row decodes to fmaf(scale, (float)code_k, bias).
 *
 * Numeric rules of the quantizer (bit-exact; binary32 round-to-nearest-even,
 * one rounding per operation, no contraction, IEEE division, denormals kept):
 *     Q = 2^bits - 1
 *     window [lo, hi]; range mode: lo = min(row) + 0, hi = max(row) + 0
 *     s = (hi - lo) / Q, replaced by +0 unless s > 0
 *     s16 = fp16_rne(s), b16 = fp16_rne(lo); sf, bf = their binary32 values
 *     code_k = 0 if sf == 0, else min(max(rint((x_k - bf) * (1 / sf)), 0), Q)
 *              with rint rounding half to even
 *     row error = pairwise sum (contiguous halves, length padded with +0 to a
 *                 power of two) of (x_k - decoded_k)^2
 *     greedy mode (n_bins = Bn, n_steps = K, 0 <= K < Bn): from the row's
 *       range, delta = (max - min) / Bn; window (i, j) is
 *       lo = fmaf(i, delta, min) + 0, hi = fmaf(-j, delta, max) + 0; starting
 *       at (0, 0), each of K steps evaluates (i+1, j) and (i, j+1) and moves to
 *       the one with the smaller error (a tie moves j); the window with the
 *       smallest error seen (only a strictly smaller error replaces it) is
 *       encoded.  K = 0 gives the range encoding.
 * Preconditions: every input value finite with |x| <= 65504; otherwise the
 * codes of the affected rows are unspecified (no fault).
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller; the
 *    library allocates nothing, frees nothing, keeps no state between calls
 *    and never synchronizes.  Work is enqueued on `stream` (NULL = the
 *    default stream) and errors that can be seen on the host are returned
 *    synchronously before anything is enqueued.
 *  - Inputs are read-only; outputs are fully overwritten; inputs and outputs
 *    must not overlap.
 *  - Return codes: QEMB_OK, or a negative QEMB_E_* value (qemb_strerror).
 *  - Calls from several host threads are safe; calls whose outputs overlap
 *    race.
 */
#ifndef QEMB_H
#define QEMB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* qemb_stream_t; /* the same type as hipStream_t */

#define QEMB_ABI_VERSION 1

#define QEMB_OK 0
#define QEMB_E_INVALID_ARG -1 /* NULL where required, bad size, mode or type */
#define QEMB_E_MISALIGNED -2  /* an array is not aligned as documented */
#define QEMB_E_UNSUPPORTED -3 /* dim above QEMB_MAX_DIM */
#define QEMB_E_LAUNCH -4      /* the HIP runtime rejected a kernel launch */
#define QEMB_E_TOO_LARGE -5   /* n above the no-allocation entry point's maximum */

#define QEMB_MAX_DIM 1024
#define QEMB_MAX_INTERACTION_T 1024 /* tables per sample in qemb_dot_interaction */

#define QEMB_CLIP_RANGE 0
#define QEMB_CLIP_GREEDY 1

#define QEMB_COMPRESS_VERBATIM 32 /* record header of a vector stored verbatim */
#define QEMB_COMPRESS_NOALLOC_MAX_VECTORS (1 << 21) /* n limit of qemb_compress_pooled_noalloc */

#define QEMB_BASE_SYMMETRIC 0
#define QEMB_BASE_PERCENTILE 1
#define QEMB_BASE_ACIQ 2

#define QEMB_POOL_SUM 0
#define QEMB_POOL_WEIGHTED_SUM 1

#define QEMB_INDEX_INT32 0
#define QEMB_INDEX_INT64 1

/* ABI version of the loaded library (QEMB_ABI_VERSION). */
int qemb_abi_version(void);

/* Static description of a return code. */
const char* qemb_strerror(int code);

/* Packed row stride S in bytes for (dim, bits), or -1 if dim < 1,
 * dim > QEMB_MAX_DIM or bits is not 2, 4 or 8. */
int64_t qemb_row_stride(int32_t dim, int32_t bits);

/*
 * Row-wise quantization of an fp32 table (the post-training quantizer of the
 * "Post-Training 4-bit Quantization on Embedding Tables" review page,
 * "Proposed method": row-wise uniform quantization, range or greedy clip,
 * fp16 scale and bias).
 *   x       [rows][dim] fp32, row-major, 16-byte aligned
 *   rows    >= 0 (0 = nothing to do)
 *   dim     1 .. QEMB_MAX_DIM
 *   bits    2, 4 or 8 (every other entry point taking `bits` accepts the
 *           same three widths)
 *   clip_mode  QEMB_CLIP_RANGE or QEMB_CLIP_GREEDY
 *   n_bins, n_steps  greedy only: 1 <= n_bins, 0 <= n_steps < n_bins
 *                    (ignored for range mode)
 *   packed  [rows][S] bytes, 16-byte aligned, written in full
 */
int qemb_quantize_rowwise(const float* x, int64_t rows, int32_t dim, int32_t bits,
                          int32_t clip_mode, int32_t n_bins, int32_t n_steps,
                          uint8_t* packed, qemb_stream_t stream);

/*
 * Quantizer baselines the same page compares the greedy search against
 * ("Proposed method": ACIQ, histogram-based clipping, symmetric
 * quantization; "Main findings"), writing the packed rows of
 * qemb_quantize_rowwise, so qemb_dequantize and qemb_bag_forward read them
 * unchanged.  Bit-exact, deterministic.
 *   QEMB_BASE_SYMMETRIC   y = s q, q in [-(2^(bits-1) - 1), 2^(bits-1) - 1],
 *       s = max|x| / (2^(bits-1) - 1) rounded to fp16 and capped at
 *       65504 / 2^(bits-1); q = rint(x * (1/s)) clamped; stored as code
 *       q + 2^(bits-1) with bias -2^(bits-1) s (exact), so y = s q exactly
 *   QEMB_BASE_PERCENTILE  window [Q(1 - p), Q(p)] of the row's values, p =
 *       param in [0.5, 1]; Q(q): h = (dim - 1) q (fp32), i = floor(h), the
 *       i-th smallest value v_i (ties in position order), Q = fmaf(h - i,
 *       v_{i+1} - v_i, v_i) (Q = v_{dim-1} when i >= dim - 1); then encoded as
 *       the range rule does for [lo, hi]
 *   QEMB_BASE_ACIQ  window [max(min, mu - a), min(max, mu + a)], mu = the
 *       row mean, b = mean |x - mu| (each a contiguous-halves pairwise fp32
 *       sum of the row padded with +0 to a power of two, divided by dim),
 *       a = t b with t = W(3 * 4^bits) as fp32 (Lambert W: the clip that
 *       minimizes the clipping plus rounding error of a Laplace(b) source)
 *   x, rows, dim, bits, packed: as qemb_quantize_rowwise; param ignored
 *   except for PERCENTILE.
 */
int qemb_quantize_baseline(const float* x, int64_t rows, int32_t dim, int32_t bits, int32_t method,
                           float param, uint8_t* packed, qemb_stream_t stream);

/*
 * Decode packed rows to fp32: y[r][k] = fmaf(scale_r, code_rk, bias_r)
 * (same passage as above: fp16 scale and bias per row).
 *   packed  [rows][S], 16-byte aligned;  y  [rows][dim] fp32, 16-byte aligned
 */
int qemb_dequantize(const uint8_t* packed, int64_t rows, int32_t dim, int32_t bits,
                    float* y, qemb_stream_t stream);

/*
 * Fused dequantize + pooled embedding-bag lookup over many tables ("Deep
 * Learning Recommendation Model ..." review page, "Proposed method": sparse
 * ids are mapped to dense vectors through embedding tables).
 *   packed         all tables' packed rows back to back, [total_rows][S],
 *                  16-byte aligned
 *   total_rows     rows in `packed`
 *   table_offsets  [T+1] int64, table t owns rows [table_offsets[t],
 *                  table_offsets[t+1])
 *   T, B           tables and bags per table (batch); bag g = t * B + b
 *   indices        [nnz] row ids local to the bag's table (int32 or int64)
 *   offsets        [T*B + 1] CSR offsets into indices (same type as indices);
 *                  bag g covers positions [offsets[g], offsets[g+1])
 *   index_type     QEMB_INDEX_INT32 or QEMB_INDEX_INT64
 *   pool_mode      QEMB_POOL_SUM (every weight 1) or QEMB_POOL_WEIGHTED_SUM
 *   weights        [nnz] fp32 per-index weights; required for WEIGHTED_SUM,
 *                  ignored (may be NULL) for SUM
 *   out            [B][T][dim] fp32, 16-byte aligned:
 *                  out[b][t][:] = sum over p in bag g of w_p * decode(row)
 *                  accumulated in fp32 (any order); an empty bag gives +0
 *   err_count      nullable int32 counter (device); the caller zeroes it.
 * Bad device data never faults: a term whose id lies outside its table, or
 * whose table range leaves [0, total_rows), is skipped; a bag whose offsets
 * decrease or leave [0, nnz] is empty; each such event adds 1 to *err_count.
 */
int qemb_bag_forward(const uint8_t* packed, int64_t total_rows, const int64_t* table_offsets,
                     int32_t T, int64_t B, int32_t dim, int32_t bits, const void* indices,
                     const void* offsets, int64_t nnz, int32_t index_type, int32_t pool_mode,
                     const float* weights, float* out, int32_t* err_count,
                     qemb_stream_t stream);

/* Bytes of device workspace that qemb_l2_error needs (a fixed size). */
size_t qemb_l2_error_workspace_bytes(void);

/*
 * Normalized l2 error of a quantized table against its fp32 source ("Post-
 * Training 4-bit Quantization on Embedding Tables", review page, "Proposed
 * method": quantization error measured by a normalized l2 loss), binary64:
 *   out4[0] = mean over rows with ||x_r|| > 0 of ||x_r - y_r|| / ||x_r||
 *   out4[1] = number of such rows
 *   out4[2] = sum over rows of ||x_r - y_r||^2
 *   out4[3] = sum over rows of ||x_r||^2
 * x [rows][dim] fp32 and packed [rows][S], both 16-byte aligned; workspace
 * of qemb_l2_error_workspace_bytes() bytes, 16-byte aligned; out4 double[4]
 * (device).  The reduction order is fixed, so results repeat exactly.
 */
int qemb_l2_error(const float* x, const uint8_t* packed, int64_t rows, int32_t dim,
                  int32_t bits, void* workspace, double* out4, qemb_stream_t stream);

/*
 * Codebook rows ("Post-Training 4-bit Quantization on Embedding Tables",
 * review page, "Proposed method": per-row codebook quantization by k-means
 * clustering with 4-bit codes; "Main findings": 18.8%-37.5% of the fp32
 * size).  A row is 16 fp32 levels (64 bytes, little-endian) followed by
 * ceil(dim/2) code bytes (element 2k in the low nibble of byte 64 + k) and
 * zero padding to a multiple of 16 bytes.
 */

/* Codebook row stride in bytes: 16 * ceil((64 + ceil(dim/2)) / 16), or -1 if
 * dim < 1 or dim > QEMB_MAX_DIM. */
int64_t qemb_codebook_row_stride(int32_t dim);

/*
 * Per-row 1-D k-means codebook quantization (same passage):
 *   levels start on the row's uniform grid c_k = fmaf(k, (max-min)/15, min)
 *   (+0, fp32); then n_iter rounds of: assign every element to its nearest
 *   level (smallest k on ties), and move every level that has members to
 *   their mean (pairwise sum of the member values, +0 for the other elements,
 *   over the row padded with +0 to a power of two, divided by the member
 *   count, fp32); levels without members stay.  The codes are the nearest
 *   levels after the last round.  Results are bit-exact and deterministic.
 *   x       [rows][dim] fp32, 16-byte aligned (finite values)
 *   rows    >= 0 (0 = nothing to do);  dim 1 .. QEMB_MAX_DIM
 *   n_iter  >= 0 rounds (0 = the uniform grid)
 *   packed  [rows][qemb_codebook_row_stride(dim)] bytes, 16-byte aligned,
 *           written in full
 */
int qemb_quantize_codebook(const float* x, int64_t rows, int32_t dim, int32_t n_iter,
                           uint8_t* packed, qemb_stream_t stream);

/* Decode codebook rows: y[r][k] = level_r[code_rk] (exact copies).
 *   packed [rows][S] and y [rows][dim] fp32, both 16-byte aligned. */
int qemb_dequantize_codebook(const uint8_t* packed, int64_t rows, int32_t dim, float* y,
                             qemb_stream_t stream);

/*
 * Fused decode + pooled embedding-bag lookup over codebook rows: the same
 * arguments, output, accumulation and error handling as qemb_bag_forward,
 * with `packed` holding codebook rows (stride qemb_codebook_row_stride(dim))
 * and no `bits` argument.
 */
int qemb_bag_forward_codebook(const uint8_t* packed, int64_t total_rows,
                              const int64_t* table_offsets, int32_t T, int64_t B, int32_t dim,
                              const void* indices, const void* offsets, int64_t nnz,
                              int32_t index_type, int32_t pool_mode, const float* weights,
                              float* out, int32_t* err_count, qemb_stream_t stream);

/*
 * Normalized l2 error of codebook rows against their fp32 source: the same
 * four binary64 results, workspace and alignment as qemb_l2_error.
 */
int qemb_l2_error_codebook(const float* x, const uint8_t* packed, int64_t rows, int32_t dim,
                           void* workspace, double* out4, qemb_stream_t stream);

/*
 * Dot interaction of the pooled embeddings ("Deep Learning Recommendation
 * Model for Personalization and Recommendation Systems", review page,
 * "Proposed method": explicit second-order interactions are the dot products
 * between the embedding vectors and the processed dense features, and they
 * are concatenated with those dense features).
 *
 * Per sample b, Z is the (T+1) x dim matrix whose row 0 is dense[b] and
 * whose row 1 + t is pooled[b][t].  The output row is
 *   out[b] = [ dense[b][0..dim) , <z_i, z_j> for i = 1..T, j = 0..i-1 ]
 * (pairs row by row over the strict lower triangle: (1,0), (2,0), (2,1),
 * (3,0), ...), dim + T(T+1)/2 floats; see qemb_interaction_width.
 *   dense   [B][dim] fp32 (the bottom MLP's output), 16-byte aligned
 *   pooled  [B][T][dim] fp32, 16-byte aligned: exactly the output layout of
 *           qemb_bag_forward / qemb_bag_forward_codebook
 *   out     [B][dim + T(T+1)/2] fp32, 16-byte aligned base (rows are packed
 *           back to back, so a row is 16-byte aligned only when its width is
 *           a multiple of 4)
 *   B >= 0 (0 = nothing to do), 0 <= T <= QEMB_MAX_INTERACTION_T,
 *   1 <= dim <= QEMB_MAX_DIM
 * The dense part is copied exactly.  Each dot is accumulated in fp32 (the
 * pooled-pooled ones on the matrix cores) in a fixed order, so results
 * repeat exactly; the error of each is within dim * 2^-23 * sum_k |z_ik z_jk|.
 */
int64_t qemb_interaction_width(int32_t T, int32_t dim);
int qemb_dot_interaction(const float* dense, const float* pooled, int64_t B, int32_t T,
                         int32_t dim, float* out, qemb_stream_t stream);

/*
 * Error-bounded compression of pooled vectors, the payload a table-sharded
 * model exchanges in its all-to-all ("Avancées dans les recommandations en
 * Deep Learning", scisimple page, "Méthodes de Compression des Données": a
 * lossy method whose reconstruction error stays within a maximum the user
 * sets; "Stratégies de Compression Adaptative": one bound per table, which
 * may change from call to call).  Per element, in binary32 with one
 * rounding per operation:
 *   step = 2 eb, inv = 1 / step (IEEE division, once per vector),
 *   q = rint(x * inv) (ties to even), x' = step * (float)q, and
 *   |x - x'| <= eb is checked;
 *   u = 2q for q >= 0, -2q - 1 for q < 0.
 * A vector's width w (0 .. 31) is the bit length of its largest u; element i's
 * u sits at bits [i w, i w + w) of a little-endian stream of dwords.  A vector
 * with an element that is not finite, has |q| >= 2^30 or misses the bound
 * after rounding, or whose table's eb is not a positive finite number (or
 * makes step overflow), is stored verbatim instead: every decompressed
 * element is then within eb of the input (verbatim ones bit-exact), and the
 * decompressed zeros of coded vectors are +0.
 * Record of a vector: a uint32 header (w, or QEMB_COMPRESS_VERBATIM), then
 * ceil(dim w / 32) payload dwords, or dim fp32 values for a verbatim one;
 * qemb_compress_record_bytes gives its size.  Records follow in vector order.
 *
 * qemb_compress_pooled
 *   x     [n][dim] fp32, 16-byte aligned; vector v belongs to table v mod T
 *         (the [B][T][dim] output of qemb_bag_forward has n = B T)
 *   eb    [T] fp32 device array (4-byte aligned), the tables' bounds
 *   out   device buffer of qemb_compress_bound(n, dim) bytes, 4-byte aligned;
 *         the first offs[n] bytes are written
 *   offs  [n + 1] int64 device array, 8-byte aligned: offs[v] is the byte
 *         offset of record v, offs[0] = 0, offs[n] the total size (the rank
 *         chunk [v0, v1) of an all-to-all is bytes [offs[v0], offs[v1]))
 *   workspace  qemb_compress_workspace_bytes(n) bytes of device memory,
 *         16-byte aligned, owned by the caller (contents need no clearing)
 *   n >= 0 (0 writes offs[0] = 0), 1 <= dim <= QEMB_MAX_DIM, T >= 1
 * Deterministic and bit-exact; three kernel launches on the stream.
 *
 * qemb_decompress_pooled
 *   in    in_bytes bytes of records, 4-byte aligned; offs [n + 1] as written
 *         by the compressor (relative to in); eb the same bounds
 *   y     [n][dim] fp32, 16-byte aligned, fully written
 *   err_count  device int32, nullable, incremented (the caller zeroes it)
 *         once per malformed record: offsets out of order or outside
 *         [0, in_bytes], a header above 32, or a size that differs from
 *         what the header implies; such a vector is written as zeros.  No
 *         read leaves [in, in + in_bytes).
 */
int64_t qemb_compress_record_bytes(int32_t dim, int32_t w);
int64_t qemb_compress_bound(int64_t n, int32_t dim);
size_t qemb_compress_workspace_bytes(int64_t n);
int qemb_compress_pooled(const float* x, int64_t n, int32_t dim, int32_t T, const float* eb,
                         uint8_t* out, int64_t* offs, void* workspace, qemb_stream_t stream);
int qemb_decompress_pooled(const uint8_t* in, int64_t in_bytes, const int64_t* offs, int64_t n,
                           int32_t dim, int32_t T, const float* eb, float* y, int32_t* err_count,
                           qemb_stream_t stream);

/* qemb_compress_pooled_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): qemb_compress_pooled with the same arguments, results
 * and kernels, minus the workspace argument.  It allocates nothing: its
 * workspace is a fixed array inside the library, 2.25 MiB per GPU, which
 * every GPU the library runs on holds until the process ends.
 *   n <= QEMB_COMPRESS_NOALLOC_MAX_VECTORS (2^21 vectors: two of the
 *   multi-hot workload's pooled outputs of 16384 x 64); larger n returns
 *   QEMB_E_TOO_LARGE before any GPU work.
 * The caller still passes out and offs.  Every call on a GPU shares that
 * GPU's array, which keeps the last call's contents (nothing in it needs to
 * start at zero): calls that overlap on one GPU -- on two streams, or from
 * two threads without ordering -- race on it and must be serialized by the
 * caller.  The first call on a device looks up the array's address there
 * (with the stream's device current), which is not an allocation.
 */
int qemb_compress_pooled_noalloc(const float* x, int64_t n, int32_t dim, int32_t T, const float* eb,
                                 uint8_t* out, int64_t* offs, qemb_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QEMB_H */
