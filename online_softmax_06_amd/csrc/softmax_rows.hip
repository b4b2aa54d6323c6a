// Row softmax on gfx950: one read and one write of every element.
//
// Method ("Ch.6 Softmax and Online Softmax", §6.3-§6.4; xxqk §3.2): every lane
// keeps an online state (m, l) over the values it owns, the states are merged
// across the 64-lane wavefront with DPP / permlane moves and across the
// wavefronts of a row through LDS, and each output is exp(x - m_row) / l_row.
//
// Unlike the chapter's kernel, which re-reads the row from memory for its
// normalisation pass, the resident kernel keeps the whole row in VGPRs:
// each lane holds NV vectors of VEC elements, already turned into
// e = exp(x - m_lane).  After the merge a lane needs one scale factor,
// exp(m_lane - m_row) / l_row, and one multiply per element.  HBM traffic is
// the 1 read + 1 write lower bound of §6.2 / §6.7.4.
//
// Layout: input and output are contiguous row-major [rows, cols].  Lane t of a
// row's thread group owns vectors t, t + T, t + 2T, ... (T threads per row), so
// consecutive lanes touch consecutive 16-byte chunks: every load and store is
// a fully coalesced global_load_dwordx4 / global_store_dwordx4.
//
// Rows longer than the resident capacity use the looping kernel, which is the
// chapter's two-read design (an online pass, then a normalising pass).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "osm_device.h"
#include "osm_internal.h"

namespace osm {
namespace {

// Element traits: how a 16-byte vector unpacks to floats and packs back.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  __device__ static void unpack(const u32x4& w, float* f) {
    f[0] = __uint_as_float(w[0]);
    f[1] = __uint_as_float(w[1]);
    f[2] = __uint_as_float(w[2]);
    f[3] = __uint_as_float(w[3]);
  }
  __device__ static u32x4 pack(const float* f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
  __device__ static float load1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static void store1(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
};

struct Bf16 {};  // tag: bfloat16 storage

template <>
struct Elem<Bf16> {
  __device__ static void unpack(const u32x4& w, float* f) {
    f[0] = bf16_lo(w[0]); f[1] = bf16_hi(w[0]);
    f[2] = bf16_lo(w[1]); f[3] = bf16_hi(w[1]);
    f[4] = bf16_lo(w[2]); f[5] = bf16_hi(w[2]);
    f[6] = bf16_lo(w[3]); f[7] = bf16_hi(w[3]);
  }
  __device__ static u32x4 pack(const float* f) {
    return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
  }
  __device__ static float load1(const void* p, int64_t i) {
    return bf16_lo(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static void store1(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xFFFFu);
  }
};

// Pairwise sum of a register array (keeps the rounding error at log2(n) ulps).
template <int N>
__device__ __forceinline__ float tree_sum(const float* v) {
  if constexpr (N == 1) {
    return v[0];
  } else {
    constexpr int H = N / 2;
    return tree_sum<H>(v) + tree_sum<N - H>(v + H);
  }
}

// Optional fused inputs ([Ch6 §6.7.3]): an additive mask of the input dtype,
// row r using mask row r % mask_rows, and per-row lengths (entries at or past
// len[r] count as -inf).  Both pointers may be null.
struct RowOptions {
  const void* mask;
  int64_t mask_rows;
  const int32_t* lens;
  __device__ int length(int64_t row, int cols) const {
    if (lens == nullptr) return cols;
    const int n = lens[row];
    return n < 0 ? 0 : (n > cols ? cols : n);
  }
};

// Load one vector (or scalar) of a row with the mask added and the length
// applied.
template <typename E, int VEC>
__device__ __forceinline__ void load_masked(const void* in, int64_t base, int64_t mbase, int v,
                                            int len, const RowOptions& opt, float* x) {
  if constexpr (VEC == 1) {
    x[0] = E::load1(in, base + v);
    if (opt.mask) x[0] += E::load1(opt.mask, mbase + v);
  } else {
    E::unpack(*reinterpret_cast<const u32x4*>(static_cast<const char*>(in) +
                                               (base + (int64_t)v * VEC) * (16 / VEC)),
              x);
    if (opt.mask) {
      float mv[VEC];
      E::unpack(*reinterpret_cast<const u32x4*>(static_cast<const char*>(opt.mask) +
                                                 (mbase + (int64_t)v * VEC) * (16 / VEC)),
                mv);
#pragma unroll
      for (int j = 0; j < VEC; ++j) x[j] += mv[j];
    }
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) x[j] = v * VEC + j < len ? x[j] : kNegInf;
}

// Merge the per-wave states of one row through LDS.  `slot` holds one (m, l)
// per wave of the row; every lane reads all of them and folds them in wave
// order, so the result is identical on every lane and on every run.
template <int kWaves>
__device__ __forceinline__ void lds_combine(float& m, float& l, float2* slot, int wave) {
  if (__lane_id() == 0) slot[wave] = make_float2(m, l);
  __syncthreads();
  float2 s = slot[0];
  m = s.x;
  l = s.y;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    s = slot[w];
    combine_state(m, l, s.x, s.y);
  }
}

// Resident kernel.  T threads per row (a multiple of 64), NV vectors of VEC
// elements per lane (VEC = 1 is the scalar path for unaligned inputs).  A
// 256-thread workgroup serves 256 / T rows (or one row when T >= 256).
template <typename E, int VEC, int NV, int T, bool kOpt>
__global__ __launch_bounds__(T >= 256 ? T : 256) void softmax_resident_kernel(
    const void* in, void* out, int64_t rows, int cols, RowOptions opt) {
  constexpr int kBlock = T >= 256 ? T : 256;
  constexpr int kRowsPerBlock = kBlock / T;
  constexpr int kWavesPerRow = T / 64;
  constexpr int kN = NV * VEC;
  __shared__ float2 slots[2][kRowsPerBlock * kWavesPerRow];

  const int tid = threadIdx.x;
  const int row_in_block = tid / T;
  const int t = tid % T;
  const int wave_in_row = t / 64;
  const int vcols = cols / VEC;  // whole vectors per row (cols % VEC == 0 here)

  int parity = 0;
  for (int64_t row0 = (int64_t)blockIdx.x * kRowsPerBlock; row0 < rows;
       row0 += (int64_t)gridDim.x * kRowsPerBlock, parity ^= 1) {
    const int64_t row = row0 + row_in_block;
    const bool live_row = row < rows;
    const int64_t base = row * (int64_t)cols;
    const int len = kOpt ? (live_row ? opt.length(row, cols) : 0) : cols;
    const int64_t mbase = kOpt && opt.mask ? (row % opt.mask_rows) * (int64_t)cols : 0;

    // R1: load the row into registers; missing elements take the identity -inf.
    float x[kN];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = k * T + t;
      if (live_row && v < vcols) {
        if constexpr (VEC == 1) {
          x[k] = E::load1(in, base + v);
          if (kOpt && opt.mask) x[k] += E::load1(opt.mask, mbase + v);
        } else {
          const u32x4 w = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(static_cast<const char*>(in) +
                                             (base + (int64_t)v * VEC) * (16 / VEC)));
          E::unpack(w, &x[k * VEC]);
          if (kOpt && opt.mask) {
            float mv[VEC];
            E::unpack(*reinterpret_cast<const u32x4*>(static_cast<const char*>(opt.mask) +
                                                      (mbase + (int64_t)v * VEC) * (16 / VEC)),
                      mv);
#pragma unroll
            for (int j = 0; j < VEC; ++j) x[k * VEC + j] += mv[j];
          }
        }
        // Entries past the row's length take part as -inf (output 0).
        if constexpr (kOpt) {
#pragma unroll
          for (int j = 0; j < VEC; ++j)
            x[k * VEC + j] = v * VEC + j < len ? x[k * VEC + j] : kNegInf;
        }
      } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) x[k * VEC + j] = kNegInf;
      }
    }

    // R2: the lane's own state.  e_i = exp(x_i - m_lane), kept in place of x.
    float m_lane = kNegInf;
#pragma unroll
    for (int i = 0; i < kN; ++i) m_lane = fmaxf(m_lane, x[i]);
    const float ref = finite_ref(m_lane);
#pragma unroll
    for (int i = 0; i < kN; ++i) x[i] = exp2_hw((x[i] - ref) * kLog2e);
    float l = tree_sum<kN>(x);
    float m = m_lane;

    // R3: wavefront butterfly.  R4: merge the row's wavefronts through LDS.
    wave_combine_state(m, l);
    if constexpr (kWavesPerRow > 1) {
      lds_combine<kWavesPerRow>(m, l, &slots[parity][row_in_block * kWavesPerRow], wave_in_row);
    }

    // R5: one scale per lane, one multiply per element, one store.
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float s = exp2_hw((m_lane - finite_ref(m)) * kLog2e) * inv;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = k * T + t;
      if (live_row && v < vcols) {
        float y[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) y[j] = x[k * VEC + j] * s;
        if constexpr (VEC == 1) {
          E::store1(out, base + v, y[0]);
        } else {
          __builtin_nontemporal_store(
              E::pack(y), reinterpret_cast<u32x4*>(static_cast<char*>(out) +
                                                   (base + (int64_t)v * VEC) * (16 / VEC)));
        }
      }
    }
  }
}

// Looping kernel for rows longer than the resident capacity: 1024 threads per
// row, an online pass over the row (per element, §6.3.1), the merge, then a
// second pass that re-reads the row and writes exp(x - m) / l.
template <typename E, int VEC>
__global__ __launch_bounds__(1024) void softmax_looping_kernel(const void* in, void* out,
                                                                int64_t rows, int cols,
                                                                RowOptions opt) {
  constexpr int T = 1024;
  __shared__ float2 slots[2][T / 64];
  const int t = threadIdx.x;
  const int vcols = cols / VEC;
  int parity = 0;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x, parity ^= 1) {
    const int64_t base = row * (int64_t)cols;
    const int len = opt.length(row, cols);
    const int64_t mbase = opt.mask ? (row % opt.mask_rows) * (int64_t)cols : 0;
    float m = kNegInf, l = 0.0f;
    for (int v = t; v < vcols; v += T) {
      float x[VEC];
      load_masked<E, VEC>(in, base, mbase, v, len, opt, x);
      float mv = kNegInf;
#pragma unroll
      for (int j = 0; j < VEC; ++j) mv = fmaxf(mv, x[j]);
      const float m_new = fmaxf(m, mv);
      const float r = finite_ref(m_new);
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < VEC; ++j) acc += exp2_hw((x[j] - r) * kLog2e);
      l = l * exp2_hw((m - r) * kLog2e) + acc;
      m = m_new;
    }
    wave_combine_state(m, l);
    lds_combine<T / 64>(m, l, slots[parity], t / 64);
    const float r = finite_ref(m);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    for (int v = t; v < vcols; v += T) {
      float x[VEC];
      load_masked<E, VEC>(in, base, mbase, v, len, opt, x);
#pragma unroll
      for (int j = 0; j < VEC; ++j) x[j] = exp2_hw((x[j] - r) * kLog2e) * inv;
      if constexpr (VEC == 1) {
        E::store1(out, base + v, x[0]);
      } else {
        *reinterpret_cast<u32x4*>(static_cast<char*>(out) + (base + (int64_t)v * VEC) * (16 / VEC)) =
            E::pack(x);
      }
    }
    // In-place calls: every read of this row above must finish before a later
    // iteration of this workgroup could write; rows are disjoint, so only the
    // LDS slots need the parity double-buffer.
  }
}

// Workgroups to launch: enough to fill the chip many times over, capped so
// the grid stays far below the 2^32 work-item limit; the kernels loop over
// any remaining rows.
inline unsigned grid_for(int64_t row_groups) {
  const int64_t cap = 1 << 20;
  return (unsigned)(row_groups < cap ? row_groups : cap);
}

// `reserve_lds` bytes of dynamic LDS per workgroup, which the kernel does not
// use, cap the workgroups resident on a CU (LDS is 160 KiB per CU): a way to
// bound the loads in flight per CU.
template <typename E, int VEC, int NV, int T>
hipError_t launch_resident(const void* in, void* out, int64_t rows, int cols,
                           const RowOptions& opt, hipStream_t s, size_t reserve_lds = 0) {
  constexpr int kBlock = T >= 256 ? T : 256;
  constexpr int kRowsPerBlock = kBlock / T;
  const int64_t groups = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (opt.mask != nullptr || opt.lens != nullptr) {
    hipLaunchKernelGGL((softmax_resident_kernel<E, VEC, NV, T, true>), dim3(grid_for(groups)),
                       dim3(kBlock), reserve_lds, s, in, out, rows, cols, opt);
  } else {
    hipLaunchKernelGGL((softmax_resident_kernel<E, VEC, NV, T, false>), dim3(grid_for(groups)),
                       dim3(kBlock), reserve_lds, s, in, out, rows, cols, opt);
  }
  return hipGetLastError();
}

// Pick the smallest resident configuration that holds `nvec` vectors per row:
// one wavefront per row for short rows, 128 or 256 threads for medium rows,
// 1024 threads for long rows, at most 64 values per lane (so that 1024-thread
// workgroups fit in 128 VGPRs); otherwise the looping kernel.
template <typename E, int VEC>
hipError_t dispatch(const void* in, void* out, int64_t rows, int cols, const RowOptions& opt,
                    hipStream_t s) {
  constexpr int kMaxNV = (64 / VEC) < 16 ? (64 / VEC) : 16;
  const int nvec = cols / VEC;
  if (nvec <= 64 * 1) return launch_resident<E, VEC, 1, 64>(in, out, rows, cols, opt, s);
  if (nvec <= 64 * 2) return launch_resident<E, VEC, 2, 64>(in, out, rows, cols, opt, s);
  if (nvec <= 64 * 4) return launch_resident<E, VEC, 4, 64>(in, out, rows, cols, opt, s);
  if constexpr (kMaxNV >= 8) {
    if (nvec <= 64 * 8) return launch_resident<E, VEC, 8, 64>(in, out, rows, cols, opt, s);
  }
  if constexpr (VEC == 4) {
    // Float32 rows of 4097..8192 values: two rows per workgroup, 128 threads
    // and 64 values per lane (measured 4% above one row per 256 threads).
    // At most two such workgroups per CU (60 KiB of LDS reserved each): 128
    // KiB of loads in flight per CU instead of 256 KiB at the four that the
    // registers allow, measured 3.7% faster at 32768 x 8192 (three per CU
    // are level with four, one is 2% slower).
    if (nvec > 256 * 4 && nvec <= 128 * 16)
      return launch_resident<E, VEC, 16, 128>(in, out, rows, cols, opt, s, 60 << 10);
  }
  if constexpr (VEC == 8) {
    // Bfloat16 rows of 4097..8192 values: 512 threads and 16 values per lane
    // (measured 4% above 256 threads; 128 or 1024 threads are slower).
    if (nvec > 64 * 8 && nvec <= 512 * 2)
      return launch_resident<E, VEC, 2, 512>(in, out, rows, cols, opt, s);
  }
  if (nvec <= 256 * 4) return launch_resident<E, VEC, 4, 256>(in, out, rows, cols, opt, s);
  if (nvec <= 256 * kMaxNV / 2 && kMaxNV / 2 > 4)
    return launch_resident<E, VEC, kMaxNV / 2 < 4 ? 4 : kMaxNV / 2, 256>(in, out, rows, cols, opt, s);
  if (nvec <= 256 * kMaxNV) return launch_resident<E, VEC, kMaxNV, 256>(in, out, rows, cols, opt, s);
  if (nvec <= 1024 * kMaxNV) return launch_resident<E, VEC, kMaxNV, 1024>(in, out, rows, cols, opt, s);
  hipLaunchKernelGGL((softmax_looping_kernel<E, VEC>), dim3(grid_for(rows)), dim3(1024), 0, s, in,
                     out, rows, cols, opt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split rows ("Ch.6" §6.7.1: a row too long for one block is shared by several
// blocks, with a second stage to merge).  Each workgroup owns one chunk of
// kSplitChunk elements of one row.
//   stage 1: load the chunk, reduce it to one online state (m, l) -- the same
//            lane state, wavefront butterfly and LDS merge as above -- and
//            store it in the workspace at [row][chunk];
//   stage 2: merge the row's chunk states (lane i folds states i, i + 256, ...,
//            then the same butterfly and LDS merge, in a fixed order), reload
//            the chunk and write exp(x - M) / L.
// Traffic: 2 reads + 1 write per element, spread over rows x chunks workgroups.
// ---------------------------------------------------------------------------
constexpr int kSplitThreads = 256;
constexpr int kSplitChunk = 8192;  // elements per workgroup

template <typename E, int VEC>
__device__ __forceinline__ void load_chunk(const void* in, int64_t base, int64_t mbase, int c0,
                                           int cols, int len, const RowOptions& opt, int t,
                                           float (&x)[kSplitChunk / kSplitThreads]) {
  constexpr int NV = kSplitChunk / kSplitThreads / VEC;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int e0 = c0 + (k * kSplitThreads + t) * VEC;  // first element of the vector
    if (e0 < cols) {
      load_masked<E, VEC>(in, base, mbase, e0 / VEC, len, opt, &x[k * VEC]);
    } else {
#pragma unroll
      for (int j = 0; j < VEC; ++j) x[k * VEC + j] = kNegInf;
    }
  }
}

template <typename E, int VEC>
__global__ __launch_bounds__(kSplitThreads) void softmax_split_stats_kernel(
    const void* in, int64_t rows, int cols, int chunks, RowOptions opt, float2* state) {
  constexpr int kN = kSplitChunk / kSplitThreads;
  __shared__ float2 slots[2][kSplitThreads / 64];
  const int t = threadIdx.x;
  int parity = 0;
  for (int64_t w = blockIdx.x; w < rows * chunks; w += gridDim.x, parity ^= 1) {
    const int64_t row = w / chunks;
    const int c0 = (int)(w % chunks) * kSplitChunk;
    const int len = opt.length(row, cols);
    const int64_t mbase = opt.mask ? (row % opt.mask_rows) * (int64_t)cols : 0;
    float x[kN];
    load_chunk<E, VEC>(in, row * (int64_t)cols, mbase, c0, cols, len, opt, t, x);
    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < kN; ++i) m = fmaxf(m, x[i]);
    const float ref = finite_ref(m);
#pragma unroll
    for (int i = 0; i < kN; ++i) x[i] = exp2_hw((x[i] - ref) * kLog2e);
    float l = tree_sum<kN>(x);
    wave_combine_state(m, l);
    lds_combine<kSplitThreads / 64>(m, l, slots[parity], t / 64);
    if (t == 0) state[w] = make_float2(m, l);
  }
}

template <typename E, int VEC>
__global__ __launch_bounds__(kSplitThreads) void softmax_split_norm_kernel(
    const void* in, void* out, int64_t rows, int cols, int chunks, RowOptions opt,
    const float2* state) {
  constexpr int kN = kSplitChunk / kSplitThreads;
  constexpr int NV = kN / VEC;
  __shared__ float2 slots[2][kSplitThreads / 64];
  const int t = threadIdx.x;
  int parity = 0;
  for (int64_t w = blockIdx.x; w < rows * chunks; w += gridDim.x, parity ^= 1) {
    const int64_t row = w / chunks;
    const int c0 = (int)(w % chunks) * kSplitChunk;
    // Merge the row's chunk states.
    float m = kNegInf, l = 0.0f;
    for (int c = t; c < chunks; c += kSplitThreads) {
      const float2 st = state[row * chunks + c];
      combine_state(m, l, st.x, st.y);
    }
    wave_combine_state(m, l);
    lds_combine<kSplitThreads / 64>(m, l, slots[parity], t / 64);
    const float r = finite_ref(m);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    // Normalise this chunk.
    const int len = opt.length(row, cols);
    const int64_t base = row * (int64_t)cols;
    const int64_t mbase = opt.mask ? (row % opt.mask_rows) * (int64_t)cols : 0;
    float x[kN];
    load_chunk<E, VEC>(in, base, mbase, c0, cols, len, opt, t, x);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int e0 = c0 + (k * kSplitThreads + t) * VEC;
      if (e0 < cols) {
        float y[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) y[j] = exp2_hw((x[k * VEC + j] - r) * kLog2e) * inv;
        if constexpr (VEC == 1) {
          E::store1(out, base + e0, y[0]);
        } else {
          __builtin_nontemporal_store(
              E::pack(y),
              reinterpret_cast<u32x4*>(static_cast<char*>(out) + (base + e0) * (16 / VEC)));
        }
      }
    }
  }
}

template <typename E, int VEC>
hipError_t launch_split(const void* in, void* out, int64_t rows, int cols, const RowOptions& opt,
                        float2* state, hipStream_t s) {
  const int chunks = (cols + kSplitChunk - 1) / kSplitChunk;
  const unsigned grid = grid_for(rows * chunks);
  hipLaunchKernelGGL((softmax_split_stats_kernel<E, VEC>), dim3(grid), dim3(kSplitThreads), 0, s,
                     in, rows, cols, chunks, opt, state);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((softmax_split_norm_kernel<E, VEC>), dim3(grid), dim3(kSplitThreads), 0, s,
                     in, out, rows, cols, chunks, opt, state);
  return hipGetLastError();
}

}  // namespace

hipError_t softmax_rows_launch(const void* in, void* out, int64_t rows, int cols, int dtype,
                               bool vector_path, const void* mask, int64_t mask_rows,
                               const int32_t* row_len, hipStream_t s) {
  const RowOptions opt{mask, mask_rows > 0 ? mask_rows : 1, row_len};
  if (dtype == 0) {
    return vector_path ? dispatch<Elem<float>, 4>(in, out, rows, cols, opt, s)
                       : dispatch<Elem<float>, 1>(in, out, rows, cols, opt, s);
  }
  return vector_path ? dispatch<Elem<Bf16>, 8>(in, out, rows, cols, opt, s)
                     : dispatch<Elem<Bf16>, 1>(in, out, rows, cols, opt, s);
}

}  // namespace osm

namespace osm {

int64_t softmax_split_workspace(int64_t rows, int64_t cols) {
  const int64_t chunks = (cols + kSplitChunk - 1) / kSplitChunk;
  return rows * chunks * (int64_t)sizeof(float2);
}

hipError_t softmax_rows_split_launch(const void* in, void* out, int64_t rows, int cols, int dtype,
                                     bool vector_path, const void* mask, int64_t mask_rows,
                                     const int32_t* row_len, void* workspace, hipStream_t s) {
  const RowOptions opt{mask, mask_rows > 0 ? mask_rows : 1, row_len};
  float2* state = static_cast<float2*>(workspace);
  if (dtype == 0) {
    return vector_path ? launch_split<Elem<float>, 4>(in, out, rows, cols, opt, state, s)
                       : launch_split<Elem<float>, 1>(in, out, rows, cols, opt, state, s);
  }
  return vector_path ? launch_split<Elem<Bf16>, 8>(in, out, rows, cols, opt, state, s)
                     : launch_split<Elem<Bf16>, 1>(in, out, rows, cols, opt, state, s);
}

}  // namespace osm
