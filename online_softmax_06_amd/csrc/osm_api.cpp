// C ABI of libosm (declared in include/osm.h): host-side validation and
// dispatch.  No HIP call is made before the arguments have been checked, so
// invalid calls return a status without touching the device.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "osm.h"
#include "osm_internal.h"

static_assert(OSM_ATTN_BWD_SCRATCH_BYTES == osm::kAttnBwdScratchBytes,
              "the header states the size of the library's scratch array");

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? OSM_OK : OSM_ERR_HIP; }

}  // namespace

extern "C" {

const char* osm_status_string(int status) {
  switch (status) {
    case OSM_OK: return "OSM_OK";
    case OSM_ERR_INVALID_ARG: return "OSM_ERR_INVALID_ARG: invalid argument";
    case OSM_ERR_UNSUPPORTED: return "OSM_ERR_UNSUPPORTED: unsupported configuration";
    case OSM_ERR_HIP: return "OSM_ERR_HIP: HIP runtime error at launch";
    default: return "OSM_ERR_UNKNOWN: unknown status code";
  }
}

const char* osm_version(void) { return "0.1.0"; }

int osm_softmax_rows_ex(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                        const void* mask, int64_t mask_rows, const int32_t* row_len,
                        void* stream) {
  if (dtype != OSM_F32 && dtype != OSM_BF16) return OSM_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0 || cols > INT32_MAX) return OSM_ERR_INVALID_ARG;
  if (mask != nullptr && mask_rows < 1) return OSM_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return OSM_OK;
  if (in == nullptr || out == nullptr) return OSM_ERR_INVALID_ARG;
  const int64_t esize = dtype == OSM_F32 ? 4 : 2;
  if (rows > INT64_MAX / cols / esize) return OSM_ERR_INVALID_ARG;
  if (mask != nullptr && mask_rows > INT64_MAX / cols / esize) return OSM_ERR_INVALID_ARG;
  if (!aligned(in, esize) || !aligned(out, esize)) return OSM_ERR_INVALID_ARG;
  if (mask != nullptr && !aligned(mask, esize)) return OSM_ERR_INVALID_ARG;
  if (row_len != nullptr && !aligned(row_len, 4)) return OSM_ERR_INVALID_ARG;
  const int64_t vec = 16 / esize;
  const bool vector_path = aligned(in, 16) && aligned(out, 16) && (cols % vec) == 0 &&
                           (mask == nullptr || aligned(mask, 16));
  return from_hip(osm::softmax_rows_launch(in, out, rows, (int)cols, dtype, vector_path, mask,
                                           mask_rows, row_len, static_cast<hipStream_t>(stream)));
}

int64_t osm_softmax_rows_split_workspace(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0 || cols > INT32_MAX) return -1;
  if (rows > INT64_MAX / 16 / (cols / 8192 + 1)) return -1;
  return osm::softmax_split_workspace(rows, cols);
}

int osm_softmax_rows_split(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                           const void* mask, int64_t mask_rows, const int32_t* row_len,
                           void* workspace, int64_t workspace_bytes, void* stream) {
  if (dtype != OSM_F32 && dtype != OSM_BF16) return OSM_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0 || cols > INT32_MAX) return OSM_ERR_INVALID_ARG;
  if (mask != nullptr && mask_rows < 1) return OSM_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return OSM_OK;
  if (in == nullptr || out == nullptr) return OSM_ERR_INVALID_ARG;
  const int64_t esize = dtype == OSM_F32 ? 4 : 2;
  if (rows > INT64_MAX / cols / esize) return OSM_ERR_INVALID_ARG;
  if (mask != nullptr && mask_rows > INT64_MAX / cols / esize) return OSM_ERR_INVALID_ARG;
  const int64_t need = osm_softmax_rows_split_workspace(rows, cols);
  if (need < 0 || workspace == nullptr || workspace_bytes < need) return OSM_ERR_INVALID_ARG;
  if (!aligned(workspace, 8)) return OSM_ERR_INVALID_ARG;
  if (!aligned(in, esize) || !aligned(out, esize)) return OSM_ERR_INVALID_ARG;
  if (mask != nullptr && !aligned(mask, esize)) return OSM_ERR_INVALID_ARG;
  if (row_len != nullptr && !aligned(row_len, 4)) return OSM_ERR_INVALID_ARG;
  const int64_t vec = 16 / esize;
  const bool vector_path = aligned(in, 16) && aligned(out, 16) && (cols % vec) == 0 &&
                           (mask == nullptr || aligned(mask, 16));
  return from_hip(osm::softmax_rows_split_launch(in, out, rows, (int)cols, dtype, vector_path,
                                                 mask, mask_rows, row_len, workspace,
                                                 static_cast<hipStream_t>(stream)));
}

int osm_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes > ((int64_t)1 << 44)) return OSM_ERR_INVALID_ARG;
  if (bytes == 0) return OSM_OK;
  if (src == nullptr || dst == nullptr) return OSM_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return OSM_ERR_INVALID_ARG;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + (uint64_t)bytes && b < a + (uint64_t)bytes) return OSM_ERR_INVALID_ARG;
  return from_hip(osm::stream_copy_launch(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

int osm_softmax_rows(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                     void* stream) {
  return osm_softmax_rows_ex(in, out, rows, cols, dtype, nullptr, 0, nullptr, stream);
}

}  // extern "C"

namespace {

// Argument checks shared by the attention entry points; OSM_OK when the call
// may proceed (a call with B*H*N == 0 returns OSM_OK and does nothing).
int check_attn(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
               int H, int N, int D, float scale, const int32_t* kv_len, const float* bias,
               int64_t bias_stride_b, int64_t bias_stride_h, int splits) {
  if (B < 0 || H < 0 || N < 0 || D < 0) return OSM_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return OSM_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return OSM_ERR_UNSUPPORTED;
  const int64_t bh = (int64_t)B * (int64_t)H;  // < 2^62: no overflow
  if (bh > INT32_MAX) return OSM_ERR_INVALID_ARG;
  const int64_t bhn = bh * (int64_t)N;         // < 2^62: no overflow
  if (bhn == 0) return OSM_OK;
  if (bhn > INT64_MAX / (2 * (int64_t)D)) return OSM_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !lse) return OSM_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return OSM_ERR_INVALID_ARG;
  if (kv_len != nullptr && !aligned(kv_len, 4)) return OSM_ERR_INVALID_ARG;
  if (bias != nullptr) {
    if (!aligned(bias, 4) || bias_stride_b < 0 || bias_stride_h < 0) return OSM_ERR_INVALID_ARG;
  }
  // Key/value tiles are addressed with 32-bit buffer offsets within one head.
  if (((int64_t)N + 64) * D * 2 >= ((int64_t)1 << 31)) return OSM_ERR_UNSUPPORTED;
  // One 256-thread workgroup per 128 query rows of each (batch, head) and
  // split: the launch must stay below 2^32 work-items.
  const int64_t workgroups = bh * (((int64_t)N + 127) / 128) * splits;
  if (workgroups * 256 >= ((int64_t)1 << 32)) return OSM_ERR_UNSUPPORTED;
  // The split merge runs one work-item per (query row, 4 dims).
  if (splits > 1 && bhn * (D / 4) >= ((int64_t)1 << 32)) return OSM_ERR_UNSUPPORTED;
  return OSM_OK;
}

}  // namespace

extern "C" {

int osm_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int N, int D, float scale, int causal, const int32_t* kv_len,
                    const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                    void* stream) {
  const int st = check_attn(q, k, v, o, lse, B, H, N, D, scale, kv_len, bias, bias_stride_b,
                            bias_stride_h, 1);
  if (st != OSM_OK || (int64_t)B * H * N == 0) return st;
  return from_hip(osm::attn_fwd_launch(q, k, v, o, lse, B, H, N, D, scale, causal != 0, kv_len,
                                       bias, bias_stride_b, bias_stride_h,
                                       static_cast<hipStream_t>(stream)));
}

int64_t osm_attn_fwd_split_workspace(int B, int H, int N, int D, int splits) {
  if (B < 0 || H < 0 || N < 0 || splits < 1 || splits > 64) return -1;
  if (D != 64 && D != 128) return -1;
  const int64_t rows = (int64_t)B * H * N;  // < 2^93 cannot happen: each factor < 2^31
  if ((int64_t)B * H > INT32_MAX || rows > INT64_MAX / 64 / (D + 1) / 4) return -1;
  return osm::attn_split_workspace(B, H, N, D, splits);
}

int osm_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int N, int D, float scale, int causal, const int32_t* kv_len,
                       const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                       int splits, void* workspace, int64_t workspace_bytes, void* stream) {
  if (splits < 1 || splits > 64) return OSM_ERR_INVALID_ARG;
  const int st = check_attn(q, k, v, o, lse, B, H, N, D, scale, kv_len, bias, bias_stride_b,
                            bias_stride_h, splits);
  if (st != OSM_OK || (int64_t)B * H * N == 0) return st;
  const int64_t need = osm_attn_fwd_split_workspace(B, H, N, D, splits);
  if (need < 0 || workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
    return OSM_ERR_INVALID_ARG;
  return from_hip(osm::attn_fwd_split_launch(q, k, v, o, lse, B, H, N, D, scale, causal != 0,
                                             kv_len, bias, bias_stride_b, bias_stride_h, splits,
                                             workspace, static_cast<hipStream_t>(stream)));
}

int64_t osm_attn_bwd_workspace(int B, int H, int N, int D) {
  if (B < 0 || H < 0 || N < 0) return -1;
  if (D != 64 && D != 128) return -1;
  if ((int64_t)B * H > INT32_MAX) return -1;
  return osm::attn_bwd_workspace(B, H, N);  // < 8 * 2^31 * 2^31: no overflow
}

int osm_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int D,
                    float scale, int causal, const int32_t* kv_len, void* workspace,
                    int64_t workspace_bytes, void* stream) {
  const int st = check_attn(q, k, v, o, lse, B, H, N, D, scale, kv_len, nullptr, 0, 0, 1);
  if (st != OSM_OK || (int64_t)B * H * N == 0) return st;
  if (!dout || !dq || !dk || !dv) return OSM_ERR_INVALID_ARG;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return OSM_ERR_INVALID_ARG;
  const int64_t need = osm_attn_bwd_workspace(B, H, N, D);
  if (need < 0 || workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
    return OSM_ERR_INVALID_ARG;
  return from_hip(osm::attn_bwd_launch(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale,
                                       causal != 0, kv_len, workspace,
                                       static_cast<hipStream_t>(stream)));
}

int osm_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                         int H, int N, int D, float scale, int causal, const int32_t* kv_len,
                         void* stream) {
  const int st = check_attn(q, k, v, o, lse, B, H, N, D, scale, kv_len, nullptr, 0, 0, 1);
  if (st != OSM_OK || (int64_t)B * H * N == 0) return st;
  if (!dout || !dq || !dk || !dv) return OSM_ERR_INVALID_ARG;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return OSM_ERR_INVALID_ARG;
  const int64_t need = osm_attn_bwd_workspace(B, H, N, D);
  if (need < 0) return OSM_ERR_INVALID_ARG;
  if (need > OSM_ATTN_BWD_SCRATCH_BYTES) return OSM_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  if (osm::attn_bwd_scratch(&scratch) != hipSuccess) return OSM_ERR_HIP;
  return from_hip(osm::attn_bwd_launch(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale,
                                       causal != 0, kv_len, scratch,
                                       static_cast<hipStream_t>(stream)));
}

int osm_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int D,
                 float scale, int causal, void* workspace, int64_t workspace_bytes, void* stream) {
  return osm_attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale, causal, nullptr,
                         workspace, workspace_bytes, stream);
}

int osm_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int D, float scale, int causal, void* stream) {
  return osm_attn_fwd_ex(q, k, v, o, lse, B, H, N, D, scale, causal, nullptr, nullptr, 0, 0,
                         stream);
}

}  // extern "C"
