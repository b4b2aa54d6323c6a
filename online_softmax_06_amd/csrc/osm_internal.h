// Launchers behind the C ABI (include/osm.h).  Arguments are validated by the
// caller in osm_api.cpp; these functions only pick a kernel and enqueue it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osm {

// Row softmax.  dtype 0 = float32, 1 = bfloat16.  `vector_path` requires both
// pointers 16-byte aligned and cols a multiple of the 16-byte vector.
hipError_t softmax_rows_launch(const void* in, void* out, int64_t rows, int cols, int dtype,
                               bool vector_path, hipStream_t stream);

// Fused attention forward, bfloat16 [B, H, N, D] in/out, float32 LSE [B, H, N].
// D must be 64 or 128.
hipError_t attn_fwd_launch(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int D, float scale, bool causal,
                           hipStream_t stream);

}  // namespace osm
