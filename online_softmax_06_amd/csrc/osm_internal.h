// Launchers behind the C ABI (include/osm.h).  Arguments are validated by the
// caller in osm_api.cpp; these functions only pick a kernel and enqueue it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osm {

// Row softmax.  dtype 0 = float32, 1 = bfloat16.  `vector_path` requires all
// pointers 16-byte aligned and cols a multiple of the 16-byte vector.  `mask`
// (nullable, input dtype, [mask_rows, cols]) is added to the input; `row_len`
// (nullable, int32 [rows]) limits each row.
hipError_t softmax_rows_launch(const void* in, void* out, int64_t rows, int cols, int dtype,
                               bool vector_path, const void* mask, int64_t mask_rows,
                               const int32_t* row_len, hipStream_t stream);

// Split-row softmax: bytes of workspace needed, and the two-stage launch
// (workspace holds one float2 state per (row, 8192-element chunk)).
int64_t softmax_split_workspace(int64_t rows, int64_t cols);
hipError_t softmax_rows_split_launch(const void* in, void* out, int64_t rows, int cols, int dtype,
                                     bool vector_path, const void* mask, int64_t mask_rows,
                                     const int32_t* row_len, void* workspace,
                                     hipStream_t stream);

// Fused attention forward, bfloat16 [B, H, N, D] in/out, float32 LSE [B, H, N].
// D must be 64 or 128.  kv_len (nullable, int32 [B]) limits the keys of each
// batch; bias (nullable, fp32) is added to the scaled scores, element
// (b, h, i, j) at bias[b * bias_stride_b + h * bias_stride_h + i * N + j].
hipError_t attn_fwd_launch(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int D, float scale, bool causal,
                           const int32_t* kv_len, const float* bias, int64_t bias_stride_b,
                           int64_t bias_stride_h, hipStream_t stream);

// Split-K attention: workspace bytes (partial O in float32 plus partial LSE
// for every split), and the launch of the partial and merge kernels.
int64_t attn_split_workspace(int B, int H, int N, int D, int splits);
hipError_t attn_fwd_split_launch(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int H, int N, int D, float scale, bool causal,
                                 const int32_t* kv_len, const float* bias, int64_t bias_stride_b,
                                 int64_t bias_stride_h, int splits, void* workspace,
                                 hipStream_t stream);

// Attention backward: workspace bytes (Delta and LSE * log2 e per query row,
// float32, rows padded to a multiple of 128 per head), and the launch of the
// two kernels (dQ, which also fills the workspace, then dK/dV).  D must be 64 or 128; kv_len (nullable,
// int32 [B]) limits the keys of each batch as in the forward.
int64_t attn_bwd_workspace(int B, int H, int N);

// Size of the library's own scratch array for the allocation-free backward
// (one per GPU), and its device address on the current device (looked up
// once per device; hipSuccess or the runtime's error).
constexpr int64_t kAttnBwdScratchBytes = (int64_t)32 << 20;
hipError_t attn_bwd_scratch(void** ptr);
hipError_t attn_bwd_launch(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                           int H, int N, int D, float scale, bool causal, const int32_t* kv_len,
                           void* workspace, hipStream_t stream);

// Streaming copy of `bytes` bytes (16-byte aligned src and dst), the
// practical bandwidth ceiling of one read and one write per byte.
hipError_t stream_copy_launch(const void* src, void* dst, int64_t bytes, hipStream_t stream);

}  // namespace osm
