/*
 * osm.h -- C ABI of libosm: online softmax, the fused attention forward and
 * its backward on AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (cited by page title and section):
 *   [Ch6]   "Ch.6 Softmax and Online Softmax", yangyitao.com CUDA
 *           FlashAttention-v2 book.
 *   [xxqk]  m.xxqk.cn article on parallelising softmax, Online Softmax and
 *           FlashAttention.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE memory owned by the caller.  The library
 *     allocates nothing and frees nothing.  Between calls it keeps only
 *     per-device facts it looks up once (the compute-unit count, the
 *     addresses of two fixed device arrays: osm_attn_bwd_noalloc's scratch
 *     and the attention forward's work-queue counters) and those arrays'
 *     content.  Calls from several host threads are safe, except overlapping
 *     osm_attn_bwd_noalloc calls on one GPU (see there).
 *   - The attention forward hands out its work through 64 queue slots per
 *     GPU, one per launch in turn, each reset by the launch that used it: at
 *     most 64 forward launches may run at the same time on one GPU.  A
 *     launch enqueued on a stream that is being captured into a HIP graph
 *     uses no slot (it takes a fixed schedule), so graph replays may run
 *     concurrently with each other and with eager launches.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *     the call returns without waiting.  The caller synchronises.
 *   - Arguments are validated on the host before any HIP call.  An invalid call
 *     returns OSM_ERR_INVALID_ARG or OSM_ERR_UNSUPPORTED and launches nothing.
 *     A launch failure reported by the runtime returns OSM_ERR_HIP.  Nothing is
 *     printed and nothing aborts.
 *   - Results are deterministic: reductions use a fixed order and no atomics,
 *     so the same inputs give bitwise-identical outputs on the same device.
 *     (The forward's queue counters only decide which workgroup computes an
 *     item, never how.)
 */
#ifndef OSM_H_
#define OSM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OSM_F32 = 0,  /* IEEE binary32 */
  OSM_BF16 = 1  /* bfloat16 (8-bit exponent, 7-bit stored mantissa) */
} osm_dtype;

typedef enum {
  OSM_OK = 0,
  OSM_ERR_INVALID_ARG = 1,  /* null pointer, negative size, unknown dtype, overflow */
  OSM_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement */
  OSM_ERR_HIP = 3           /* the HIP runtime reported an error at launch */
} osm_status;

/*
 * osm_softmax_rows -- row-wise softmax of a row-major [rows, cols] matrix.
 *
 * Computes out[r, i] = exp(in[r, i] - m_r) / sum_j exp(in[r, j] - m_r) with
 * m_r the row maximum: the safe softmax of [Ch6 §6.2], evaluated with the
 * online normaliser of [Ch6 §6.3.1] (a running max m and a rescaled sum l per
 * lane) and the associative (m, l) combine of [Ch6 §6.4.1] across lanes and
 * wavefronts.  Each row is read from HBM once and written once.
 *
 *   in, out  device pointers to contiguous row-major [rows, cols] arrays of
 *            `dtype` (no row stride).  in == out (in place) is allowed; any
 *            other overlap is not.  Element alignment is required; 16-byte
 *            alignment with cols a multiple of 16 bytes takes the vector path.
 *   rows     number of rows, >= 0.
 *   cols     row length, >= 0 and < 2^31.  rows == 0 or cols == 0 is a
 *            successful no-op (pointers may then be NULL).
 *   dtype    OSM_F32 or OSM_BF16; input and output share it.  Arithmetic is
 *            float32; bfloat16 outputs are rounded to nearest even.
 *   stream   hipStream_t to enqueue on.
 *
 * Values: -inf entries contribute 0 and produce 0.  A row whose entries are
 * all -inf produces all zeros (where an unguarded 0/0 would give NaN,
 * [Ch6 §6.7.3]).  +inf and NaN inputs are outside the contract.
 *
 * Returns OSM_OK, or OSM_ERR_INVALID_ARG (null pointer with nonzero size,
 * negative or too large size, unknown dtype, misaligned pointer), or
 * OSM_ERR_HIP.
 */
int osm_softmax_rows(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                     void* stream);

/*
 * osm_softmax_rows_ex -- row softmax with a fused additive mask and/or
 * per-row lengths.
 *
 * The fused form of [Ch6 §6.7.3]: each logit is in[r, i] + mask[r % mask_rows,
 * i] (a mask of 0 / -inf hides entries, other finite values bias them), and
 * with row_len only the first row_len[r] entries of row r take part; the
 * outputs past a row's length are 0.  Everything else is as in
 * osm_softmax_rows (one read of in and mask, one write of out).
 *
 *   mask       device pointer, same dtype as in, contiguous [mask_rows, cols];
 *              NULL for no mask.  mask_rows >= 1 when mask is given (1
 *              broadcasts one mask row to every row).  The sum is formed in
 *              float32.
 *   row_len    device pointer to int32 [rows], or NULL for full rows; values
 *              are clamped to [0, cols] (0 gives an all-zero row).
 *
 * Returns as osm_softmax_rows, plus OSM_ERR_INVALID_ARG for mask_rows < 1
 * with a mask, or a misaligned mask / row_len pointer.
 */
int osm_softmax_rows_ex(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                        const void* mask, int64_t mask_rows, const int32_t* row_len,
                        void* stream);

/*
 * osm_softmax_rows_split -- row softmax for rows too long for one workgroup.
 *
 * The same result as osm_softmax_rows_ex, computed the split-row way of
 * [Ch6 §6.7.1]: every row is cut into 8192-element chunks, one workgroup per
 * (row, chunk).  A first kernel reduces each chunk to an online state (m, l)
 * and stores it in `workspace`; a second merges the row's states with the
 * combine of [Ch6 §6.4.1] in a fixed order and writes exp(x - M) / L for its
 * chunk.  The input is read twice and the output written once; use it when
 * rows * (cols / 8192) is large next to rows alone (a few very long rows).
 *
 *   in, out, rows, cols, dtype, mask, mask_rows, row_len
 *              as osm_softmax_rows_ex (in == out allowed).
 *   workspace  device memory owned by the caller, 8-byte aligned, at least
 *              osm_softmax_rows_split_workspace(rows, cols) bytes; its content
 *              on entry does not matter and is overwritten.  Calls that share
 *              a workspace must be ordered (same stream).
 *   workspace_bytes  its size.
 *
 * Returns as osm_softmax_rows_ex, plus OSM_ERR_INVALID_ARG for a missing,
 * misaligned or too small workspace.
 */
int osm_softmax_rows_split(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                           const void* mask, int64_t mask_rows, const int32_t* row_len,
                           void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of workspace osm_softmax_rows_split needs: 8 * rows * ceil(cols / 8192);
 * -1 for invalid sizes. */
int64_t osm_softmax_rows_split_workspace(int64_t rows, int64_t cols);

/*
 * osm_attn_fwd -- fused attention forward with per-row log-sum-exp.
 *
 * For every batch b, head h and query row i:
 *   S[i, j] = scale * dot(q[b,h,i,:], k[b,h,j,:])            ([xxqk §4.1])
 *   with causal != 0, S[i, j] = -inf for j > i              ([xxqk §6.3])
 *   o[b,h,i,:] = sum_j softmax_j(S[i, :]) * v[b,h,j,:]
 *   lse[b,h,i] = log sum_j exp(S[i, j])                     ([Ch6 §6.5])
 * The scores are never written to memory: key/value tiles stream through
 * on-chip memory and the running (m, l) and the output accumulator are
 * rescaled per tile ([Ch6 §6.6], [xxqk §4.1]); the division by l happens once
 * at the end.
 *
 *   q, k, v  device pointers, contiguous [B, H, N, D] bfloat16.
 *   o        device pointer, contiguous [B, H, N, D] bfloat16 (rounded to
 *            nearest even).  Must not overlap q, k, v or lse.
 *   lse      device pointer, contiguous [B, H, N] float32: natural log of the
 *            sum of exp over the scaled, unmasked scores (-inf if none).
 *   B, H, N  >= 0; any N (tails are masked).  B*H*N == 0 is a no-op.
 *   D        head dimension: 64 or 128 (others return OSM_ERR_UNSUPPORTED).
 *   scale    multiplier applied to q.k (e.g. 1/sqrt(D)); finite and > 0.
 *   causal   0: every key visible; nonzero: key j visible to query i iff j <= i.
 *   stream   hipStream_t to enqueue on.
 *
 * Returns OSM_OK, OSM_ERR_INVALID_ARG (null pointer with nonzero size, negative
 * size, B*H*N*D overflowing int64, non-finite or non-positive scale, pointer
 * not 16-byte aligned), OSM_ERR_UNSUPPORTED (D not 64 or 128; (N + 64) * D * 2
 * >= 2^31 bytes per head; more than 2^24 workgroups), or OSM_ERR_HIP.
 */
int osm_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int H, int N, int D, float scale, int causal, void* stream);

/*
 * osm_attn_fwd_ex -- fused attention forward with key padding and an
 * additive score bias.
 *
 *   S[i, j] = scale * dot(q[b,h,i,:], k[b,h,j,:]) + bias[b,h,i,j]
 *   hidden (-inf) when j >= kv_len[b], or when causal and j > i
 * ([xxqk §6.3]: additive -inf masks; [Ch6 §6.7.3]: the mask fused into the
 * softmax).  o and lse are then as in osm_attn_fwd; a query row with no
 * visible key gets o = 0 and lse = -inf.
 *
 *   kv_len          device pointer to int32 [B] (valid keys per batch,
 *                   clamped to [0, N]), or NULL for N.  Key tiles past a
 *                   batch's length are not visited.
 *   bias            device pointer to float32, element (b, h, i, j) at
 *                   bias[b * bias_stride_b + h * bias_stride_h + i * N + j]
 *                   (strides in elements, >= 0; 0 broadcasts), or NULL.
 *                   4-byte alignment required; 16-byte alignment with N and
 *                   both strides multiples of 4 takes 16-byte loads.
 *   bias_stride_b, bias_stride_h   ignored when bias is NULL.
 *
 * Returns as osm_attn_fwd, plus OSM_ERR_INVALID_ARG for negative strides or a
 * misaligned kv_len / bias pointer.
 */
int osm_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int N, int D, float scale, int causal, const int32_t* kv_len,
                    const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                    void* stream);

/*
 * osm_attn_fwd_split -- the fused attention forward with the key range of
 * every query tile split over several workgroups (split-K).
 *
 * The same result as osm_attn_fwd_ex.  Workgroup (b, h, query tile, split)
 * runs the online softmax over its share of the key tiles and writes its own
 * normalised partial output O_s (float32) and log-sum-exp LSE_s to
 * `workspace`; a second kernel merges the splits of every query row with the
 * combine of [Ch6 §6.4.1] written for normalised partials:
 *   LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 * Useful when B * H * ceil(N / 128) is small next to the number of compute
 * units (few heads, long sequences).
 *
 *   q .. stride_h   as osm_attn_fwd_ex.
 *   splits          1 .. 64 workgroups per query tile.
 *   workspace       device memory owned by the caller, 16-byte aligned, at
 *                   least osm_attn_fwd_split_workspace(B, H, N, D, splits)
 *                   bytes; its content on entry does not matter.  Calls that
 *                   share a workspace must be ordered (same stream).
 *
 * Returns as osm_attn_fwd_ex, plus OSM_ERR_INVALID_ARG for splits outside
 * 1..64 or a missing, misaligned or too small workspace, and
 * OSM_ERR_UNSUPPORTED when splits > 1 and B * H * N * D / 4 >= 2^32 (the merge
 * runs one work-item per query row and 4 dimensions).
 */
int osm_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int N, int D, float scale, int causal, const int32_t* kv_len,
                       const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                       int splits, void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of workspace osm_attn_fwd_split needs: 4 * splits * B * H * N * (D + 1);
 * -1 for invalid arguments. */
int64_t osm_attn_fwd_split_workspace(int B, int H, int N, int D, int splits);

/*
 * osm_attn_bwd -- attention backward from the forward's output and
 * log-sum-exp, with the scores recomputed instead of stored ([Ch6 §6.5]: the
 * forward keeps one LSE per row for the backward; [xxqk §5.2]: the backward
 * recomputes S, trading compute for memory).
 *
 * For O = softmax(S) V with S as in osm_attn_fwd (scale, optional causal
 * mask) and an upstream gradient dO, with P = exp(S - LSE):
 *   dv = P^T dO
 *   dS = P * (dO V^T - Delta),   Delta[i] = dot(dO[i, :], O[i, :])
 *   dq = scale * dS K,   dk = scale * dS^T Q
 * per batch and head.  P and dS enter the products as bfloat16, products
 * accumulate in float32, Delta is formed in float32 from o and dout.
 *
 *   q, k, v     device pointers, contiguous [B, H, N, D] bfloat16 (the
 *               forward's inputs).
 *   o, lse      the forward's outputs for these inputs, same scale and causal
 *               flag: o [B, H, N, D] bfloat16, lse [B, H, N] float32 (a row
 *               with lse = -inf contributes nothing).
 *   dout        device pointer, [B, H, N, D] bfloat16: dL/do.
 *   dq, dk, dv  device pointers, [B, H, N, D] bfloat16, written (rounded to
 *               nearest even).  They must not overlap each other, any input
 *               or the workspace.
 *   B, H, N, D, scale, causal   as osm_attn_fwd.
 *   workspace   device memory owned by the caller, 16-byte aligned, at least
 *               osm_attn_bwd_workspace(B, H, N, D) bytes; its content on
 *               entry does not matter.  Calls that share a workspace must be
 *               ordered (same stream).
 *   stream      hipStream_t to enqueue on (two kernels, in order).
 *
 * The result does not depend on the launch (no atomics): equal inputs give
 * bitwise equal gradients.  Returns as osm_attn_fwd, plus OSM_ERR_INVALID_ARG
 * for a missing, misaligned or too small workspace.
 */
int osm_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int D,
                 float scale, int causal, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * osm_attn_bwd_ex -- osm_attn_bwd for a forward run with key padding
 * (osm_attn_fwd_ex with the same kv_len and no bias).
 *
 *   kv_len   device pointer to int32 [B] (valid keys per batch, clamped to
 *            [0, N]), or NULL for N.  Keys at or past a batch's length get
 *            dk = dv = 0 and contribute nothing to dq; key blocks wholly
 *            past the length are not visited.
 *
 * Returns as osm_attn_bwd, plus OSM_ERR_INVALID_ARG for a misaligned kv_len.
 */
int osm_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int D,
                    float scale, int causal, const int32_t* kv_len, void* workspace,
                    int64_t workspace_bytes, void* stream);

/* Bytes of workspace osm_attn_bwd and osm_attn_bwd_ex need: 8 * B * H * (N
 * rounded up to a multiple of 128); -1 for invalid arguments. */
int64_t osm_attn_bwd_workspace(int B, int H, int N, int D);

/*
 * osm_attn_bwd_noalloc -- osm_attn_bwd_ex with no workspace argument, for
 * callers that cannot allocate device memory: code being captured into a HIP
 * graph, tight serving or training loops, and harnesses that forbid
 * hipMalloc.  The call allocates and frees nothing.
 *
 * The per-row scratch (-Delta and LSE * log2 e, osm_attn_bwd_workspace bytes)
 * lives in a fixed array of OSM_ATTN_BWD_SCRATCH_BYTES bytes inside the
 * library.  Every GPU the library runs on holds its own copy from the first
 * call on that GPU until the process ends.  Its content on entry does not
 * matter: the first kernel writes every entry the second reads.  The call
 * uses the array of the current device, which must be the device of the
 * pointers and the stream.
 *
 * All calls on one GPU share that array: calls that overlap in time on one
 * GPU (on different streams, or from host threads without ordering) race and
 * give wrong gradients.  Calls ordered on one stream are safe.
 *
 *   q .. kv_len, stream   as osm_attn_bwd_ex.
 *
 * Returns as osm_attn_bwd_ex, plus OSM_ERR_UNSUPPORTED when
 * osm_attn_bwd_workspace(B, H, N, D) exceeds OSM_ATTN_BWD_SCRATCH_BYTES
 * (B * H * (N rounded up to 128) above 4194304 rows), checked before any HIP
 * call, and OSM_ERR_HIP when the runtime cannot give the array's address.
 */
#define OSM_ATTN_BWD_SCRATCH_BYTES ((int64_t)32 << 20)
int osm_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                         int H, int N, int D, float scale, int causal, const int32_t* kv_len,
                         void* stream);

/*
 * osm_stream_copy -- copy `bytes` bytes from src to dst on the device with
 * the memory access pattern of the row softmax (16-byte non-temporal loads
 * and stores, every byte read once and written once).  A measurement
 * utility, not a step of the method: its rate on the softmax's bytes is the
 * practical ceiling of a kernel that moves one read and one write per
 * element, the traffic [Ch6 §6.2] and [Ch6 §6.7.4] give as the softmax's
 * lower bound.
 *
 *   src, dst  device pointers, 16-byte aligned; the ranges must not overlap.
 *   bytes     0 .. 2^44 (0 is a no-op).
 *
 * Returns OSM_OK, OSM_ERR_INVALID_ARG (null or misaligned pointer,
 * overlapping ranges, size out of range) or OSM_ERR_HIP.
 */
int osm_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Human-readable name of a status code; never NULL, static storage. */
const char* osm_status_string(int status);

/* Library version as "major.minor.patch"; static storage. */
const char* osm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OSM_H_ */
