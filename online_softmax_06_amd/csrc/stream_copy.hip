// Streaming copy on gfx950: the practical HBM ceiling for a kernel that reads
// every byte once and writes every byte once, the traffic of the row softmax
// ("Ch.6 Softmax and Online Softmax" §6.2 and §6.7.4 count one read and one
// write per element as its lower bound).
//
// The access pattern is the softmax's: 16-byte non-temporal loads and stores,
// lane t of a workgroup owning vectors t, t + T, t + 2T, ... of its chunk.
// The shape is the fastest of a sweep on MI355X (64 to 512 threads, 2 to 32
// vectors per lane, normal or non-temporal accesses): 512 threads with two
// vectors each, 16 KiB per workgroup; each wave waits for all its loads and
// sleeps ~256 clocks before its first store.  That
// separation of the read and write phases (the softmax has its arithmetic
// there) is worth 6% over storing each vector as soon as it arrives.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "osm_device.h"
#include "osm_internal.h"

namespace osm {
namespace {

constexpr int kCopyThreads = 512;
constexpr int kCopyVecs = 2;  // 16-byte vectors per lane: 16 KiB per workgroup
constexpr int64_t kCopyChunk = (int64_t)kCopyThreads * kCopyVecs * 16;

__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                    u32x4* __restrict__ dst,
                                                                    int64_t nvec) {
  const int64_t base = (int64_t)blockIdx.x * (kCopyThreads * kCopyVecs) + threadIdx.x;
  u32x4 w[kCopyVecs];
#pragma unroll
  for (int k = 0; k < kCopyVecs; ++k) {
    const int64_t i = base + (int64_t)k * kCopyThreads;
    if (i < nvec) w[k] = __builtin_nontemporal_load(src + i);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_sleep(4);
#pragma unroll
  for (int k = 0; k < kCopyVecs; ++k) {
    const int64_t i = base + (int64_t)k * kCopyThreads;
    if (i < nvec) __builtin_nontemporal_store(w[k], dst + i);
  }
}

// Bytes past the last whole 16-byte vector (fewer than 16).
__global__ void stream_copy_tail_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                        int n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

hipError_t stream_copy_launch(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t nvec = bytes / 16;
  if (nvec > 0) {
    const int64_t blocks = (nvec * 16 + kCopyChunk - 1) / kCopyChunk;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int tail = (int)(bytes - nvec * 16);
  if (tail > 0) {
    hipLaunchKernelGGL(stream_copy_tail_kernel, dim3(1), dim3(16), 0, s,
                       static_cast<const uint8_t*>(src) + nvec * 16,
                       static_cast<uint8_t*>(dst) + nvec * 16, tail);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace osm
