// Fused attention forward on gfx950: S = scale * Q K^T, optional causal mask,
// online softmax, O = P V, and the per-row log-sum-exp, with S and P living
// only in registers.
//
// Method ("Ch.6 Softmax and Online Softmax" §6.5-§6.6; xxqk §4.1): a workgroup
// owns a tile of BM query rows and streams the key/value tiles of its
// (batch, head) through LDS.  Per tile it forms the scores on the matrix
// cores, updates the running max m and rescaled sum l of every query row,
// rescales the output accumulator by alpha = e^(m_old - m_new), and adds
// P V_j with P = e^(S - m_new) (the form that needs no second correction
// factor).  The division by l happens once, after the last tile.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, wave64).  Each wavefront owns
// 32 query rows and computes the TRANSPOSED products
//     S^T (keys x queries)  = K   * Q^T      A = K tile (LDS), B = Q (VGPRs)
//     O^T (dims x queries) += V^T * P^T      A = V^T tile (LDS), B = P (VGPRs)
// With this orientation every lane holds values of exactly one query row
// (lane % 32), split with its partner lane (lane ^ 32): row max, row sum and
// the alpha rescale of the accumulator are per-lane operations plus one
// permlane32 swap, and P is fed to the second product straight from the
// registers that received S.  The key order inside each 16-key slice of a
// tile follows the MFMA output layout; the V^T tile in LDS is stored in that
// same order, so no register shuffle is needed between the two products.
//
// Data layout in LDS (double-buffered, one barrier per key tile):
//   K tile   [BN keys][D] bf16, 16-byte units XOR-swizzled by (key & 7).
//   V^T tile [D][BN keys] bf16, V transposed while it is written, key
//            positions permuted as above, 16-byte units XOR-swizzled by (d & 7).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "osm_device.h"
#include "osm_internal.h"

namespace osm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;     // query rows per workgroup
constexpr int kBN = 64;      // keys per tile
constexpr int kWaves = 4;    // wavefronts per workgroup, 32 query rows each
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Byte offset of 16-byte unit `u` of key row `key` in a K tile.
template <int D>
__device__ __forceinline__ int k_lds_off(int key, int u) {
  return key * (D * 2) + ((u ^ (key & 7)) << 4);
}

// Byte offset of the 8-byte chunk holding key positions [4c, 4c+4) of row d
// in a V^T tile.  Chunks are XOR-swizzled by 2 * (d & 7) so that 16-byte
// reads stay aligned.
__device__ __forceinline__ int vt_lds_off(int d, int c) {
  return d * (kBN * 2) + ((c ^ ((d & 7) << 1)) << 3);
}

// Position of key `kk` (0..63) inside a V^T row: bits 2 and 3 swapped, which
// makes the 8 keys one lane feeds to the P V product contiguous.
__device__ __forceinline__ int vt_pos(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// Per-thread staging registers for one K/V tile.
template <int D>
struct TileRegs {
  static constexpr int kKUnits = kBN * D / 8 / kThreads;  // 16-byte units of K per thread
  static constexpr int kVThreads = (kBN / 4) * (D / 8);   // threads that carry V (4 keys x 8 dims)
  uint4 k[kKUnits];
  uint4 v[4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const uint16_t* kg, const uint16_t* vg,
                                          int k0, int N, int tid) {
  constexpr int kUnitsPerRow = D / 8;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kKUnits; ++i) {
    const int U = tid + i * kThreads;
    const int key = U / kUnitsPerRow, u = U % kUnitsPerRow;
    const int gk = k0 + key;
    r.k[i] = gk < N ? *reinterpret_cast<const uint4*>(kg + (int64_t)gk * D + u * 8)
                    : make_uint4(0, 0, 0, 0);
  }
  if (tid < TileRegs<D>::kVThreads) {
    const int kgrp = tid % (kBN / 4), dg = tid / (kBN / 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int gk = k0 + kgrp * 4 + rr;
      r.v[rr] = gk < N ? *reinterpret_cast<const uint4*>(vg + (int64_t)gk * D + dg * 8)
                       : make_uint4(0, 0, 0, 0);
    }
  }
}

// Write the staged tile to LDS: K as is (swizzled), V transposed.
template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, char* k_lds, char* vt_lds,
                                           int tid) {
  constexpr int kUnitsPerRow = D / 8;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kKUnits; ++i) {
    const int U = tid + i * kThreads;
    const int key = U / kUnitsPerRow, u = U % kUnitsPerRow;
    *reinterpret_cast<uint4*>(k_lds + k_lds_off<D>(key, u)) = r.k[i];
  }
  if (tid < TileRegs<D>::kVThreads) {
    const int kgrp = tid % (kBN / 4), dg = tid / (kBN / 4);
    const int chunk = vt_pos(kgrp * 4) >> 2;
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r.v[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r.v[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r.v[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r.v[3]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // dims 8*dg + j of keys 4*kgrp .. 4*kgrp+3 -> one 8-byte chunk of row d.
      const int w = j >> 1;
      // v_perm_b32 selectors: low halves (bytes 1:0 of each source) for even
      // j, high halves (bytes 3:2) for odd j.
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      uint2 out;
      out.x = __builtin_amdgcn_perm(w1[w], w0[w], sel);
      out.y = __builtin_amdgcn_perm(w3[w], w2[w], sel);
      const int d = dg * 8 + j;
      *reinterpret_cast<uint2*>(vt_lds + vt_lds_off(d, chunk)) = out;
    }
  }
}

// Map a linear workgroup id to (batch*head, query tile).  Workgroups are
// dispatched round-robin over the 8 XCDs; when B*H is a multiple of 8 all
// query tiles of one head land on one XCD (its L2 holds that head's K and
// V), visited heaviest first when causal.
__device__ __forceinline__ void tile_of(int L, int nqt, int BH, bool causal, int& bh, int& qt) {
  int rank;
  if ((BH & 7) == 0) {
    const int xcd = L & 7, idx = L >> 3;
    bh = (idx / nqt) * 8 + xcd;
    rank = idx % nqt;
  } else {
    bh = L / nqt;
    rank = L % nqt;
  }
  qt = causal ? nqt - 1 - rank : rank;
}

template <int D, bool kCausal>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int BH,
    int N, float scale_log2) {
  constexpr int kDC = D / 16;  // 16-wide slices of the head dimension
  constexpr int kDB = D / 32;  // 32-row blocks of O^T
  constexpr int kKBytes = kBN * D * 2;
  constexpr int kVBytes = D * kBN * 2;
  __shared__ __attribute__((aligned(16))) char smem[2 * (kKBytes + kVBytes)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // the query row this lane works on (within the wave)
  const int half = lane >> 5;  // which 8-element half of each 16-wide slice

  const int nqt = (N + kBM - 1) / kBM;
  int bh, qt;
  tile_of(blockIdx.x, nqt, BH, kCausal, bh, qt);
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* qg = q + head_off;
  const uint16_t* kg = k + head_off;
  const uint16_t* vg = v + head_off;

  const int q0 = qt * kBM;
  const int qw = q0 + wave * 32;  // first query row of this wave
  const int qrow = qw + col;      // this lane's query row
  const bool wave_live = qw < N;

  // A1: this lane's part of Q as the B operand of S^T = K Q^T.
  uint4 qreg[kDC];
#pragma unroll
  for (int c = 0; c < kDC; ++c) {
    qreg[c] = qrow < N ? *reinterpret_cast<const uint4*>(qg + (int64_t)qrow * D + c * 16 + half * 8)
                       : make_uint4(0, 0, 0, 0);
  }

  f32x16 oacc[kDB];
#pragma unroll
  for (int b = 0; b < kDB; ++b) oacc[b] = f32x16{};
  float m_run = kNegInf;  // running max, in units of log2(e) * scale * S
  float l_run = 0.0f;     // this lane's half of the running sum

  const int kv_end = kCausal ? min(N, q0 + kBM) : N;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  TileRegs<D> stage;
  load_tile<D>(stage, kg, vg, 0, N, tid);
  store_tile<D>(stage, smem, smem + kKBytes, tid);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * kBN;
    char* k_lds = smem + (j & 1) * (kKBytes + kVBytes);
    char* vt_lds = k_lds + kKBytes;
    const bool has_next = j + 1 < ntiles;
    // A2: prefetch the next tile into registers while this one is used.
    if (has_next) load_tile<D>(stage, kg, vg, k0 + kBN, N, tid);

    const bool visible = wave_live && (!kCausal || k0 <= qw + 31);
    if (visible) {
      // A3: S^T for keys [k0, k0+64) x this wave's 32 queries.
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int c = 0; c < kDC; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint4 a =
              *reinterpret_cast<const uint4*>(k_lds + k_lds_off<D>(kb * 32 + col, 2 * c + half));
          sacc[kb] = mfma32(a, qreg[c], sacc[kb]);
        }
      }
      // A4: mask keys past the causal diagonal or past the end of the sequence.
      const bool need_mask = (kCausal && k0 + kBN - 1 > qw) || (k0 + kBN > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            const bool hide = key >= N || (kCausal && key > qrow);
            if (hide) sacc[kb][i] = kNegInf;
          }
        }
      }
      // A5: online-softmax update of (m, l) for this lane's query row.
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float ref = finite_ref(m_new);
      const float alpha = exp2_hw(m_run - ref);
      float psum = 0.0f;
      uint4 pb[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        float p[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          p[jj] = exp2_hw(__builtin_fmaf(sacc[kc >> 1][(kc & 1) * 8 + jj], scale_log2, -ref));
          psum += p[jj];
        }
        pb[kc] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                            pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      // A6: rescale the accumulator, then O^T += V^T P^T.
#pragma unroll
      for (int b = 0; b < kDB; ++b) oacc[b] *= alpha;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int b = 0; b < kDB; ++b) {
          const uint4 a = *reinterpret_cast<const uint4*>(
              vt_lds + vt_lds_off(b * 32 + col, (kc * 16 + half * 8) >> 2));
          oacc[b] = mfma32(a, pb[kc], oacc[b]);
        }
      }
    }

    if (has_next) {
      store_tile<D>(stage, smem + ((j + 1) & 1) * (kKBytes + kVBytes),
                    smem + ((j + 1) & 1) * (kKBytes + kVBytes) + kKBytes, tid);
    }
    __syncthreads();
  }

  // A7: O = O / l (deferred division), LSE = ln 2 * (m + log2 l).
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qrow < N) {
    uint16_t* orow = o + head_off + (int64_t)qrow * D;
#pragma unroll
    for (int b = 0; b < kDB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // O^T rows b*32 + g*8 + half*4 + (0..3): four consecutive dims.
        uint2 w;
        w.x = pack_bf16x2(oacc[b][g * 4 + 0] * inv, oacc[b][g * 4 + 1] * inv);
        w.y = pack_bf16x2(oacc[b][g * 4 + 2] * inv, oacc[b][g * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + b * 32 + g * 8 + half * 4) = w;
      }
    }
    if (half == 0) {
      lse[(int64_t)bh * N + qrow] =
          l_tot > 0.0f ? (finite_ref(m_run) + log2_hw(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <int D, bool kCausal>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                  float scale, hipStream_t s) {
  const int nqt = (N + kBM - 1) / kBM;
  const float scale_log2 = scale * kLog2e;
  hipLaunchKernelGGL((attn_fwd_kernel<D, kCausal>), dim3(nqt * BH), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, BH, N,
                     scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_fwd_launch(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int D, float scale, bool causal,
                           hipStream_t stream) {
  const int BH = B * H;
  if (D == 64) {
    return causal ? launch<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch<64, false>(q, k, v, o, lse, BH, N, scale, stream);
  }
  return causal ? launch<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch<128, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace osm
