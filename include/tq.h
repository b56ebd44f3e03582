/*
 * libtq: rotation + Lloyd-Max weight quantization and its fused quantized linear layers,
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (turboquant-mlx, "How it works"):
 *   - "Quantizing a weight, with no data": every weight row w (length K, the input
 *     dimension) is rotated, w' = R w with R = H_K diag(s) / sqrt(K) (random +-1 signs s,
 *     then a Hadamard matrix); the rotated row is cut into groups of 16/32/64/128 along K,
 *     each group is divided by its root-mean-square, every value snaps to the nearest
 *     centroid of a fixed Lloyd-Max codebook for N(0,1) (2, 3 or 4 bits), and the indices
 *     are bit-packed into 32-bit words with per-group scales stored alongside.
 *   - "The ternary tier (1.58 bits)": a 3-level codebook {-c, 0, +c}; twenty base-3
 *     digits per 32-bit word. The codebook size tells which packing is used.
 *   - "Running a quantized layer": R is orthonormal, so the layer rotates its input,
 *     x' = R x, and multiplies by the packed weights, decoding them inline:
 *         y_i = sum_g scale_{i,g} sum_{j in g} c[idx_ij] x'_j .
 *     Mixture-of-Experts layers use gather_qmv (one token, shared input),
 *     multi_gather_qmv (a different input per expert) and gather_qmm (a large batch
 *     sorted by expert).
 *   - "Quantizing a weight, with no data", last paragraph: all experts of a layer share
 *     the rotation signs and the codebook.
 *
 * Conventions shared by every entry point
 *   Memory    Pointers marked "device" are HIP device pointers; "host" are host pointers.
 *             The caller owns all memory, including workspaces. The library never
 *             allocates and keeps no pointer after a call returns.
 *   Streams   `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *             Calls only enqueue work on it and never synchronize; routing ids and offsets
 *             stay on the device.
 *   Errors    Arguments are checked on the host before anything is launched. A failed
 *             check returns a negative tq_status and sets a thread-local message readable
 *             with tq_last_error(). A launch failure returns TQ_ERR_HIP. Nothing aborts
 *             and nothing throws across this interface. TQ_OK is 0.
 *   Shapes    K = m * 2^k with m in {1, 12, 20, 28}, K a multiple of 32 in [64, 8192];
 *             group in {16, 32, 64, 128} dividing K; n_levels in {3, 4, 8, 16} (and 256
 *             for KV-cache rows, see tq_kv_fetch);
 *             E in [1, 8192]. Other shapes return TQ_ERR_UNSUPPORTED.
 *   Layout    codes  uint32 [E][N][words_per_row], rows packed independently;
 *                    words_per_row = ceil(K * b / 32) for b = log2(n_levels) bits, element
 *                    j of a row in bits [b*j, b*j + b) of the row's little-endian
 *                    bitstream (bit p is bit p%32 of word p/32), unused bits zero;
 *                    n_levels = 3: words_per_row = ceil(K / 20), word w holds elements
 *                    20w..20w+19 as sum_k t_k 3^k (element 20w+k is digit k), padding
 *                    digits 0. Index 0 is the most negative centroid.
 *             scales fp16 bit patterns [E][N][K / group]: the group RMS rounded to
 *                    nearest even, saturating at 65504.
 *             signs  uint32 [ceil(K / 32)]: bit i (bit i%32 of word i/32) set means
 *                    s_i = -1. Produced by tq_signs from the seed.
 *   Signs     s_i = -1 iff the top bit of SplitMix64 output i of the generator seeded with
 *             `seed` is set: output i = mix64(seed + (i + 1) * 0x9E3779B97F4A7C15) with the
 *             SplitMix64 finalizer (Steele, Lea, Flood 2014). The pages only say the
 *             rotation comes from a seed; this generator is this library's choice.
 *   Hadamard  H_K = H_m (x) H_{2^k}: natural-order Sylvester H_{2^k}; H_12 and H_20 from
 *             Paley's first construction (q = 11, 19), H_28 from Paley's second (q = 13),
 *             with Jacobsthal matrix Q[a][b] = chi(a - b).
 *   Dtypes    Activations and outputs are fp32, bf16 or fp16 (tq_dtype). Accumulation is
 *             fp32. Weights for tq_encode are fp32, bf16 or fp16. Activations x are read
 *             with 16-byte loads and must be 16-byte aligned; outputs y need the alignment
 *             of their dtype.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

typedef enum {
  TQ_OK = 0,
  TQ_ERR_ARG = -1,          /* null pointer, bad size, bad dtype */
  TQ_ERR_UNSUPPORTED = -2,  /* K, group or n_levels outside the supported set */
  TQ_ERR_ALIGN = -3,        /* a pointer is not aligned as documented */
  TQ_ERR_WORKSPACE = -4,    /* workspace missing or smaller than tq_workspace_bytes */
  TQ_ERR_HIP = -5           /* the HIP runtime reported an error */
} tq_status;

/* flags for the qmv family */
enum { TQ_X_ROTATED = 1 }; /* x is already R x: skip the input rotation */

/* operation ids for tq_workspace_bytes */
enum { TQ_OP_QMV = 1, TQ_OP_GATHER_QMV = 2, TQ_OP_MULTI_GATHER_QMV = 3, TQ_OP_GATHER_QMM = 4,
       TQ_OP_ENCODE_DENSE = 5 };

/* A packed quantized weight: E experts of N x K (E = 1 for a dense layer). Read only
 * during the call.
 * The rotation of the weight is given by one thing only, `signs`: the kernels rotate the
 * input with R = H_K diag(s) / sqrt(K) for the s these bits hold. The rotation is recorded
 * by its seed ("Configuration that converter and loader share": rotation, seed and group
 * sizes), so a caller makes `signs` with tq_signs(seed, K) for the seed that tq_encode was
 * given; the descriptor carries no seed, so it cannot name a second, disagreeing rotation. */
typedef struct {
  const uint32_t *codes;  /* device, [E][N][words_per_row], 16-byte aligned */
  const uint16_t *scales; /* device, [E][N][K / group], fp16 bits, 2-byte aligned */
  const uint32_t *signs;  /* device, [ceil(K / 32)] rotation sign bits (tq_signs) */
  int32_t n_levels;       /* 3 -> trit packed; 4 / 8 / 16 -> 2 / 3 / 4-bit bitstream */
  int32_t group;          /* 16, 32, 64 or 128 */
  int64_t K, N, E;        /* input dim, output dim, number of experts */
} tq_qweight;

/* Number of uint32 words per packed row, or 0 for an unsupported (K, n_levels). */
int64_t tq_words_per_row(int64_t K, int32_t n_levels);

/* Centroids (ascending, n_levels floats) and, if `thresholds` is not NULL, the n_levels-1
 * decision thresholds (midpoints of neighbouring centroids), both binary32, host memory.
 * n_levels 3, 4, 8, 16 or 256.
 * The codebook is the Lloyd-Max quantizer of N(0,1) ("Quantizing a weight, with no data",
 * third bullet; "The ternary tier"), computed by Lloyd iteration in double precision when
 * the library loads and rounded once. Returns TQ_OK or TQ_ERR_UNSUPPORTED. */
int tq_codebook(int32_t n_levels, float *centroids, float *thresholds);

/* Rotation sign bits for (seed, K) into device memory `bits` (ceil(K/32) words). */
int tq_signs(uint64_t seed, int64_t K, uint32_t *bits, void *stream);

/* Encode `rows` weight rows of length K (device, row-major, dtype w_dtype) into codes
 * (device, [rows][words_per_row]) and scales (device, [rows][K/group]). For an expert
 * stack pass rows = E * N. Steps ("Quantizing a weight, with no data"): v = R w; per
 * group r = sqrt(mean v^2), scale = fp16(r); u = v / r (u = 0 when r = 0);
 * idx = #{k : u > t_k} with u and t_k in binary32; pack. Rotation and RMS are computed in
 * double precision. Deterministic and independent of how rows are split across calls. */
int tq_encode(const void *W, tq_dtype w_dtype, int64_t rows, int64_t K, int32_t n_levels,
              int32_t group, uint64_t seed, uint32_t *codes, uint16_t *scales, void *stream);

/* tq_encode of weight rows that live in HOST memory, streamed through a caller-owned device
 * staging buffer, so that device memory holds the encoded weight plus the staging buffer
 * and never the whole unquantized weight (turboquant-mlx "How it works", "Two converters":
 * the streaming converter keeps memory near one shard and writes the same bytes as the
 * in-memory one). The rows go up in chunks: each chunk is copied on `copy_stream` into one
 * half of `staging` and encoded on `stream` into its rows of codes and scales; the halves
 * alternate, ordered by events, so the copy of chunk i + 1 overlaps the encode of chunk i
 * when W_host is pinned (a pageable W_host is copied as the runtime allows). The output is
 * byte-identical to one tq_encode of all rows.
 *   W_host         host, [rows][K] of w_dtype; must stay valid and unchanged until the
 *                  work enqueued on `stream` has completed
 *   staging        device, 256-byte aligned, staging_bytes >= 2 * 256-byte-rounded K row
 *                  bytes (a chunk is as many rows as half of it holds)
 *   copy_stream    hipStream_t as void*, or NULL to copy on `stream` (no overlap)
 * The first copies wait for all work enqueued on `stream` before the call (an event
 * recorded on `stream` at entry), so a staging buffer that earlier encodes on `stream`
 * still read, for example the previous call's, is not overwritten early; work on other
 * streams that uses `staging` is the caller's to order. Like every call here it enqueues
 * and returns; it creates five HIP events and releases them before returning (the runtime
 * frees them once the work has used them).
 * Errors: the tq_encode argument errors; TQ_ERR_ARG for a NULL W_host or staging, or a
 * staging buffer that holds fewer than two rows; TQ_ERR_ALIGN for a misaligned staging;
 * TQ_ERR_HIP if the runtime fails, in which case some chunks may already be enqueued. */
int tq_encode_stream(const void *W_host, tq_dtype w_dtype, int64_t rows, int64_t K,
                     int32_t n_levels, int32_t group, uint64_t seed, uint32_t *codes,
                     uint16_t *scales, void *staging, size_t staging_bytes, void *stream,
                     void *copy_stream);

/* out[r] = R x[r] for `rows` rows of length K (device, row-major). Computed in fp32.
 * ("Running a quantized layer": the input is rotated with the weights' rotation.) */
int tq_fwht(const void *x, tq_dtype x_dtype, int64_t rows, int64_t K, uint64_t seed,
            void *out, tq_dtype out_dtype, void *stream);

/* Bytes of workspace an operation needs (0 if none). `count` is n (ids) for
 * gather_qmv, P (pairs) for multi_gather_qmv, M (rows) for gather_qmm, the number of rows
 * for encode_dense (w gives K; its other fields must be valid); T is the number of input
 * rows of gather_qmm. Returns SIZE_MAX for invalid arguments. Workspaces are
 * 16-byte aligned (multi_gather_qmv) or 256-byte aligned (gather_qmm). */
size_t tq_workspace_bytes(int32_t op, const tq_qweight *w, int64_t count, int64_t T);

/* Dense layer (E must be 1): y[N] = W R x, x device [K]. Workspace: none. */
int tq_qmv(const tq_qweight *w, const void *x, tq_dtype x_dtype, void *y, tq_dtype y_dtype,
           uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* One token through n routed experts sharing one input ("Running a quantized layer",
 * kernel table, first row): y[k][N] = W_{ids[k]} R x for k < n. ids device int32 [n].
 * An id outside [0, E) yields a row of NaN (no out-of-range access). */
int tq_gather_qmv(const tq_qweight *w, const int32_t *ids, int32_t n, const void *x,
                  tq_dtype x_dtype, void *y, tq_dtype y_dtype, uint32_t flags, void *ws,
                  size_t ws_bytes, void *stream);

/* tq_gather_qmv of two weights that read the same token through the same routed experts,
 * in one launch: a Mixture-of-Experts layer's gate and up projections ("Running a
 * quantized layer", kernel table, first row: one token, shared input; both projections of
 * an expert see that token). y[k][N] = W1_{ids[k]} R x and y[n + k][N] = W2_{ids[k]} R x
 * for k < n; y device [2n][N]. The input is rotated once for both, so the two weights must
 * have the same n_levels, group, K, N and E and share one rotation: the same `signs`
 * pointer (encoded with the same seed); with TQ_X_ROTATED no signs are read. Results are
 * those of two tq_gather_qmv calls, bit for bit. An id outside [0, E) yields NaN rows.
 * Workspace: none. Errors: the tq_gather_qmv ones; TQ_ERR_ARG when the weights differ in
 * format or shape, do not share their signs array, or n is above 65535. */
int tq_gather_qmv_pair(const tq_qweight *w1, const tq_qweight *w2, const int32_t *ids,
                       int32_t n, const void *x, tq_dtype x_dtype, void *y, tq_dtype y_dtype,
                       uint32_t flags, void *stream);

/* P (input, expert) pairs, each with its own input ("Running a quantized layer", kernel
 * table, second row): y[p] = W_{ids[p]} R x[p]. x device [P][K], y device [P][N]. Pairs
 * are bucketed by expert on the device so that each W_e is streamed once; y keeps the
 * caller's pair order. Ids outside [0, E) yield NaN rows. Workspace: tq_workspace_bytes. */
int tq_multi_gather_qmv(const tq_qweight *w, const int32_t *ids, int64_t P, const void *x,
                        tq_dtype x_dtype, void *y, tq_dtype y_dtype, uint32_t flags, void *ws,
                        size_t ws_bytes, void *stream);

/* tq_multi_gather_qmv of two weights over the same pairs, in one call: a Mixture-of-Experts
 * layer's gate and up projections, which read each token's input through the same routed
 * experts ("Running a quantized layer", kernel table, second row: per-expert inputs).
 * y[p][N] = W1_{ids[p]} R x[p] and y[P + p][N] = W2_{ids[p]} R x[p]; y device [2P][N].
 * The inputs are rotated and the pairs bucketed once for both weights, and the trit kernel
 * takes the row blocks of both in one launch. The weights must have the same n_levels,
 * group, K, N and E and share one `signs` array (with TQ_X_ROTATED none is read). Results
 * are those of two tq_multi_gather_qmv calls, bit for bit; a pair with an id outside
 * [0, E) gets NaN rows in both halves. Workspace: tq_workspace_bytes(TQ_OP_MULTI_GATHER_QMV,
 * w1, P, 0) bytes, 16-byte aligned. Errors: the tq_multi_gather_qmv ones; TQ_ERR_ARG when
 * the weights differ in format or shape or do not share their signs array, or P > 2^29. */
int tq_multi_gather_qmv_pair(const tq_qweight *w1, const tq_qweight *w2, const int32_t *ids,
                             int64_t P, const void *x, tq_dtype x_dtype, void *y,
                             tq_dtype y_dtype, uint32_t flags, void *ws, size_t ws_bytes,
                             void *stream);

/* tq_multi_gather_qmv with no workspace argument and no allocation of any kind, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Its workspace is one fixed array of 8 MiB per GPU,
 * held from the first such call on that GPU until the process ends; the call uses the
 * array of the device current on the calling thread (`stream` must belong to it). Arguments,
 * kernels and results are those of tq_multi_gather_qmv. Limit: the workspace
 * tq_workspace_bytes(TQ_OP_MULTI_GATHER_QMV, w, P, 0) must fit in 8 MiB (about
 * 2 (P + 1) (K + 4) bytes: about 2000 pairs at K = 2048, or 500 at K = 8192); a larger call returns
 * TQ_ERR_WORKSPACE before anything is launched. Every call on one GPU shares the array and
 * nothing in it must start at zero (each call writes all it reads); calls that overlap in
 * time on one GPU (different streams, or several host threads) race on it and give wrong
 * results; calls on one stream are ordered and safe. */
int tq_multi_gather_qmv_static(const tq_qweight *w, const int32_t *ids, int64_t P,
                               const void *x, tq_dtype x_dtype, void *y, tq_dtype y_dtype,
                               uint32_t flags, void *stream);

/* Batched gather-GEMM over rows sorted by expert ("Running a quantized layer", kernel
 * table, third row): for offsets[e] <= m < offsets[e+1], y[m] = W_e R x[row_token[m]].
 * x device [T][K]; row_token device int32 [M]; expert_offsets device int32 [E+1],
 * non-decreasing, offsets[0] = 0, offsets[E] = M; y device [M][N] in sorted-row order.
 * Inputs are rotated once into fp16 rows (each scaled by a power of two), weights are
 * decoded to fp16 (centroid times group scale) and multiplied on the matrix cores with fp32
 * accumulation. A row_token outside [0, T) yields a row of NaN. Workspace:
 * tq_workspace_bytes (it depends on M, T and E). */
int tq_gather_qmm(const tq_qweight *w, const void *x, tq_dtype x_dtype, int64_t T,
                  const int32_t *row_token, const int32_t *expert_offsets, int64_t M, void *y,
                  tq_dtype y_dtype, uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* tq_gather_qmm of two weights over the same sorted rows: a Mixture-of-Experts layer's gate
 * and up projections, which multiply the same token rows by the same experts' weights
 * ("Running a quantized layer", kernel table, third row). y[m] = W1_e R x[row_token[m]] and
 * y[M + m] = W2_e R x[row_token[m]] for offsets[e] <= m < offsets[e+1]; y device [2M][N].
 * The rows are rotated and the tiles scheduled once, then each weight's matrix kernel runs.
 * The weights must have the same n_levels, group, K, N and E and share one `signs` array
 * (with TQ_X_ROTATED none is read). Results are those of two tq_gather_qmm calls, bit for
 * bit; a row_token outside [0, T) gives NaN rows in both halves. Workspace:
 * tq_workspace_bytes(TQ_OP_GATHER_QMM, w1, M, T). Errors: the
 * tq_gather_qmm ones; TQ_ERR_ARG when the weights differ in format or shape or do not share
 * their signs array, or M >= 2^30. */
int tq_gather_qmm_pair(const tq_qweight *w1, const tq_qweight *w2, const void *x,
                       tq_dtype x_dtype, int64_t T, const int32_t *row_token,
                       const int32_t *expert_offsets, int64_t M, void *y, tq_dtype y_dtype,
                       uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* Decoded weights of n experts in the rotated basis, for the shapes of work the fused
 * kernels above do not cover ("Running a quantized layer", kernel table, fourth row:
 * dequantize the experts, then a regular matrix multiply):
 *   out[k][i][j] = scale[e][i][j / group] * c[idx[e][i][j]],  e = ids[k] (k if ids is NULL),
 * the fp32 centroid times the fp16 scale, rounded once to out_dtype, so that out[k] times
 * the rotated input (tq_fwht) is W_e R x up to rounding. ids: device int32 [n], or NULL with
 * n <= E. out: device [n][N][K], aligned to 16 bytes. An id outside [0, E) yields a block of
 * NaN. n must be at most 65535. Workspace: none. */
int tq_dequant(const tq_qweight *w, const int32_t *ids, int64_t n, void *out,
               tq_dtype out_dtype, void *stream);

/* Dense rotations, for input dimensions the Hadamard transform does not cover (VeloxQuant-MLX,
 * "What already existed" and "Where the time actually went": a rotation derived by QR from a
 * seeded random matrix for dimensions such as 4864, which is neither a power of two nor a
 * multiple of the transform's special sizes). The rotation is a caller-owned K x K binary32
 * matrix R (device, row-major, R[i][k]); the library applies it and never makes it, so the
 * page's "persist the matrix or regenerate it from the seed" choice stays with the caller.
 * A layer with a dense rotation is encoded with tq_encode_dense, its inputs are rotated with
 * tq_rotate_dense, and the qmv family then runs with TQ_X_ROTATED on a descriptor of that K
 * (K any multiple of 32 in [64, 8192]; the signs pointer may be NULL). */

/* out[r] = R x[r] for `rows` rows of length K (x device [rows][K] of x_dtype; out device
 * [rows][K] of out_dtype). Computed on the fp64 matrix cores (exact products, fp64 sums) and
 * rounded once to out_dtype. K a multiple of 32 in [64, 8192]; rows below 64 * 65536. */
int tq_rotate_dense(const void *x, tq_dtype x_dtype, int64_t rows, int64_t K, const float *R,
                    void *out, tq_dtype out_dtype, void *stream);

/* tq_encode with the dense rotation R in place of the randomized Hadamard one: v = R w per
 * row, computed in fp64 as tq_encode computes its rotation, then group RMS, fp16 scale, snap
 * and pack as in tq_encode (scale = fp16(r), R being orthonormal). ws: device, 8-byte
 * aligned, at least K * 8 bytes; rows go through it in chunks of ws_bytes / (K * 8) rows
 * (tq_workspace_bytes(TQ_OP_ENCODE_DENSE, ...) gives the size for all rows at once).
 * n_levels 3, 4, 8 or 16; group dividing K; K a multiple of 32 in [64, 8192]. */
int tq_encode_dense(const void *W, tq_dtype w_dtype, int64_t rows, int64_t K, const float *R,
                    int32_t n_levels, int32_t group, uint32_t *codes, uint16_t *scales,
                    void *ws, size_t ws_bytes, void *stream);

/* KV-cache compression (turboquant-mlx "How it works", "The KV cache": the weights' rotation
 * and codebook compress the cache at run time, 8-bit keys and 3-bit values; "your SSD is a
 * GPU", KV-cache section: rotate, quantize, store; dequantize, de-rotate on the way out).
 * A cache of T tokens x H heads is rows = T * H rows of head_dim = K:
 *   store  tq_encode(x, dtype, rows, K, n_levels, group, seed, codes, scales, stream), with
 *          n_levels = 256 (8-bit keys: one byte per code, four per word) or 8 (3-bit values),
 *          or any other level count; 256 levels need K a power of two in [64, 4096] and a
 *          16-byte aligned x (TQ_ERR_UNSUPPORTED / TQ_ERR_ALIGN otherwise);
 *   fetch  tq_kv_fetch below.
 * The 256-level codebook is the Lloyd-Max quantizer of N(0,1) like the others (tq_codebook
 * accepts 256); the qmv family, tq_dequant and tq_gather_qmm do not take it. */

/* Fetch: out[r] = R^T w'_r for every row r < E * N of w, w'_r[j] = c[idx_rj] * scale_{r, j /
 * group} (the dequantized row) and R^T = diag(s) H_K / sqrt(K) the inverse rotation (the
 * signs of w). w: n_levels 4, 8, 16 or 256 (bit formats), K a power of two in [64, 2048],
 * any group. out: device [E * N][K] of out_dtype, 16-byte aligned. Computed in fp32 and
 * rounded once to out_dtype. Returns TQ_ERR_UNSUPPORTED for other formats or K. */
int tq_kv_fetch(const tq_qweight *w, void *out, tq_dtype out_dtype, void *stream);

/* Expert streaming (turboquant-mlx "How it works", "Expert streaming": experts are read on
 * demand through an LRU cache, with results bit-identical to a model held in memory). The
 * packed experts stay in HOST memory; a caller-owned device pool of `slots` expert slots
 * holds the ones in use, and a caller-owned host state (tq_expert_cache_bytes) keeps which
 * expert sits in which slot. Each fetch makes the routed experts resident and writes their
 * slot numbers to the device, so the usual layer calls run on the pool:
 *     tq_expert_cache_fetch(state, host, pool, ids, n, slot_ids_dev, ...);
 *     tq_gather_qmv(pool, slot_ids_dev, n, x, ...);   (or tq_multi_gather_qmv)
 * and their outputs are bit-identical to the same calls on all E experts in device memory. */

/* Bytes of host state for `slots` slots over E experts (SIZE_MAX for slots or E outside
 * [1, 8192]). */
size_t tq_expert_cache_bytes(int32_t slots, int64_t E);

/* Empties the cache: `state` host, 8-byte aligned, state_bytes >= tq_expert_cache_bytes.
 * Returns TQ_OK, TQ_ERR_ARG or TQ_ERR_ALIGN. */
int tq_expert_cache_init(void *state, size_t state_bytes, int32_t slots, int64_t E);

/* Makes experts ids_host[0..n) resident (n <= 512; repeats allowed; the distinct ones must
 * fit the slots) and writes the slot of ids_host[k] to slot_ids_dev[k] (device int32 [n])
 * and, when not NULL, to slot_ids_host[k]. Experts already resident are kept; each missing
 * one takes the least recently used slot that this call does not need, and its codes and
 * scales are copied from `host` into that slot of `pool`.
 *   host   the packed weight with codes and scales in HOST memory, [E][N][..] as usual
 *          (pinned memory lets the copies run asynchronously); its signs pointer is not
 *          read here and may be the pool's
 *   pool   a device weight of E = slots experts with the same n_levels, group, K and N;
 *          its codes and scales are written here, its signs are those of the weight
 *   copied when not NULL, the number of experts copied by this call
 * Copies go on `copy_stream` (NULL: on `stream`) after the work already on `stream`, and
 * `stream` waits for them, so a following call on `stream` sees the slots filled and no
 * earlier one sees them change; the slot numbers are written on `stream`. `host` must stay
 * valid and unchanged until the copies have run. Host-side errors (bad ids, too many
 * distinct experts, mismatched descriptors) are found before anything is enqueued and leave
 * the state unchanged; TQ_ERR_HIP leaves the state recording the new residency. */
int tq_expert_cache_fetch(void *state, const tq_qweight *host, const tq_qweight *pool,
                          const int32_t *ids_host, int32_t n, int32_t *slot_ids_dev,
                          int32_t *slot_ids_host, int32_t *copied, void *stream,
                          void *copy_stream);

/* Total hits and misses (experts found resident / copied) since tq_expert_cache_init. */
int tq_expert_cache_stats(const void *state, int64_t *hits, int64_t *misses);

/* Message of the last failed call on this thread ("" if none). */
const char *tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
