// Fused attention forward on gfx950: S = scale * Q K^T, optional causal mask,
// online softmax, O = P V, and the per-row log-sum-exp, with S and P living
// only in registers.
//
// Method ("Ch.6 Softmax and Online Softmax" §6.5-§6.6; xxqk §4.1): a workgroup
// owns a tile of 128 query rows and streams the key/value tiles of its
// (batch, head) through LDS.  Per tile it forms the scores on the matrix
// cores, updates the running max m and rescaled sum l of every query row,
// rescales the output accumulator by alpha = 2^(m_old - m_new), and adds
// P V_j with P = 2^(S' - m_new) (S' = S * scale * log2 e), the form that needs
// no second correction factor.  The division by l happens once at the end.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, wave64).  Each wavefront owns
// 32 query rows and computes the TRANSPOSED products
//     S^T (keys x queries)  = K   * Q^T      A = K tile (LDS), B = Q (VGPRs)
//     O^T (dims x queries) += V^T * P^T      A = V^T (LDS),    B = P (VGPRs)
// so every lane holds values of exactly one query row (lane % 32), shared with
// its partner lane (lane ^ 32): row max, row sum and the alpha rescale are
// per-lane operations plus one v_permlane32_swap, and P enters the second
// product straight from the registers that received S.
//
// Memory path.  K and V tiles go from HBM to LDS with buffer_load ... lds
// (no VGPR staging); keys past the end of the sequence fall outside the
// buffer descriptor's range and arrive as zeros.  Both tiles are stored
// row-major ([64 keys][D]) with 16-byte units XOR-swizzled per row.  K rows
// feed the A operand of the first product with ds_read_b128; V feeds the A
// operand of the second product through ds_read_b64_tr_b16, which returns
// each lane four consecutive keys of one head dimension, already transposed.
// The key order inside every 16-key slice follows the MFMA output layout of
// S^T, so P needs no register shuffle.  Two LDS stages alternate; one barrier
// per key tile.
//
// Exponent reference.  The reference m used in P = 2^(S' - m) is raised only
// when a tile's row max exceeds it by more than kLag (in log2 units); P then
// stays below 2^kLag, which float32 sums and bfloat16 P hold without loss of
// range, and alpha is exactly 1 on most tiles, so the O rescale is skipped
// whenever it is 1 for the whole wavefront.  In exact arithmetic the result
// does not depend on the reference (the combine of §6.4.1 holds for any
// finite one); the pages' recurrence is the special case kLag = 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "osm_device.h"
#include "osm_internal.h"

namespace osm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;     // query rows per workgroup
constexpr int kBN = 64;      // keys per tile
constexpr int kWaves = 4;    // wavefronts per workgroup, 32 query rows each
constexpr int kThreads = kWaves * 64;
constexpr float kLag = 8.0f;  // allowed lag of the exponent reference (log2 units)

// Buffer descriptor word 3 for raw (untyped) buffer loads on gfx950.
constexpr int kBufferFlags = 0x00020000;

#define OSM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tile geometry for head dimension D.
template <int D>
struct Tile {
  static constexpr int kUnits = D / 8;                // 16-byte units per key row
  static constexpr int kBytes = kBN * D * 2;          // one K or V tile
  static constexpr int kLoadsPerWave = kBN * kUnits / 64 / kWaves;  // 1 KB each
  // Row swizzles of the 16-byte units (LDS has 64 four-byte banks).
  // K rows are read 16 bytes per lane, 16 consecutive rows per 256-byte bank
  // sweep: XOR by row & 15 (row & 7 at D = 64) spreads them over all banks.
  // V rows are read 8 bytes per lane through the transpose read: each 32-lane
  // half reads 4 consecutive rows x 64 bytes, so rows r..r+3 are XORed by
  // 0, 4, 8, 12 units (one 64-byte quarter each) and rows 4..7 of an 8-row
  // group additionally by 2.  Every swizzle depends on row & 7 or row & 15
  // only, so rows 32 apart (K) and 8 or 16 apart (V) share one lane offset.
  __device__ static int k_swz(int row) { return row & (kUnits - 1); }
  __device__ static int v_swz(int row) {
    return D == 128 ? (((row & 3) << 2) | ((row & 4) >> 1)) : ((row & 3) << 1);
  }
};

// Issue the global->LDS copy of one K or V tile (keys [k0, k0 + 64)) into
// `buf`.  Instruction i of wave w fills LDS units [(w * kLoadsPerWave + i) *
// 64, +64) of the tile, one 16-byte unit per lane; `swz` is the tile's row
// swizzle.  Keys at or past the end of the head read as zeros.
template <int D, int (*Swz)(int)>
__device__ __forceinline__ void issue_tile(char* buf, const uint16_t* base, int head_bytes, int k0,
                                           int wave, int lane) {
  // The buffer-to-LDS builtins exist only for the device; the host pass of
  // this single-source file sees an empty body.
#if defined(__HIP_DEVICE_COMPILE__)
  using T = Tile<D>;
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, head_bytes, kBufferFlags);
#pragma unroll
  for (int i = 0; i < T::kLoadsPerWave; ++i) {
    const int inst = wave * T::kLoadsPerWave + i;
    const int p = inst * 64 + lane;                 // physical unit in the tile
    const int row = p / T::kUnits, pu = p % T::kUnits;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, OSM_LDS(buf + inst * 1024), 16,
                                             (k0 + row) * (D * 2) + ((pu ^ Swz(row)) << 4), 0, 0,
                                             0);
  }
#endif
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

// Split-K variant: each (head, query tile) owns `splits` consecutive ids, so
// the splits of one query tile are dispatched together.
__device__ __forceinline__ void tile_of_split(int L, int nqt, int splits, int BH, bool causal,
                                              int& bh, int& qt, int& split) {
  int vt;
  tile_of(L, nqt * splits, BH, false, bh, vt);
  split = vt % splits;
  const int rank = vt / splits;
  qt = causal ? nqt - 1 - rank : rank;
}

// Per-lane LDS byte offsets inside a K or V buffer, computed once per
// workgroup.
// K: lane reads row `col` (and col + 32), 16-byte unit (2c + half) ^ swz(col);
// since the swizzle keeps bit 0 of the unit apart from c's bits, the offset
// for slice c is k ^ (c << 5), and rows col + 32 sit 32 rows further.
// V: lane reads key row `vkey` (+ 16 kc + 8 part) at dims b*32 + vd; the
// swizzle depends on row & 7 only, so the other rows are constant offsets.
template <int D>
struct LaneOffsets {
  int k;
  int v[D / 32];
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int lane) {
  using T = Tile<D>;
  const int col = lane & 31, half = lane >> 5;
  LaneOffsets<D> off;
  off.k = col * (D * 2) + ((half ^ T::k_swz(col)) << 4);
  const int g = lane >> 4, r = lane & 15;
  const int vkey = half * 4 + (r >> 2);        // 0..7 within a 16-key slice
  const int vd = (g & 1) * 16 + 4 * (r & 3);   // dim offset within a 32-dim block
#pragma unroll
  for (int b = 0; b < D / 32; ++b) {
    const int d = b * 32 + vd;
    off.v[b] = vkey * (D * 2) + (((d >> 3) ^ T::v_swz(vkey)) << 4) + (d & 7) * 2;
  }
  return off;
}

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
}

// A3: S^T = K Q^T for one key tile (16 products at D = 128) from `kbuf`.
// K operands are read two slices ahead of the products that use them.
template <int D>
__device__ __forceinline__ void compute_scores(const char* kbuf, const LaneOffsets<D>& off,
                                               const bf16x8 (&qreg)[D / 16], f32x16 (&s)[2]) {
  constexpr int kDC = D / 16;
  constexpr int kRow = D * 2;
  s[0] = f32x16{};
  s[1] = f32x16{};
  bf16x8 ka[3][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const char* pk = kbuf + (off.k ^ (c << 5));
    ka[c][0] = *reinterpret_cast<const bf16x8*>(pk);
    ka[c][1] = *reinterpret_cast<const bf16x8*>(pk + 32 * kRow);
  }
#pragma unroll
  for (int c = 0; c < kDC; ++c) {
    if (c + 2 < kDC) {
      const char* pk = kbuf + (off.k ^ ((c + 2) << 5));
      ka[(c + 2) % 3][0] = *reinterpret_cast<const bf16x8*>(pk);
      ka[(c + 2) % 3][1] = *reinterpret_cast<const bf16x8*>(pk + 32 * kRow);
    }
    s[0] = mfma32(ka[c % 3][0], qreg[c], s[0]);
    s[1] = mfma32(ka[c % 3][1], qreg[c], s[1]);
  }
}

// One key tile j for one wavefront: mask and softmax the scores S_j held in
// `scur`, then O^T += V_j^T P_j^T; with kNext, then form the scores of tile
// j + 1 into `snext`, so 32 matrix products run back to back per tile.
// Optional fused inputs: per-batch key lengths (keys at or past kv_len are
// hidden) and an additive fp32 bias on the scaled scores, element (b, h, i, j)
// at bias[b * stride_b + h * stride_h + i * N + j].
struct AttnOptions {
  const int32_t* kv_len;
  const float* bias;
  int64_t bias_stride_b, bias_stride_h;
  float inv_scale;  // the bias enters the raw scores as bias / scale
  bool bias_vec;    // N, strides and base allow 16-byte bias loads
};

// Add the bias of this lane's query row to its 32 raw scores of tile k0.
__device__ __forceinline__ void add_bias(f32x16 (&s)[2], const float* brow, int k0, int half,
                                         int N, const AttnOptions& opt) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int key = k0 + kb * 32 + g * 8 + half * 4;  // 4 consecutive keys
      float b4[4];
      if (opt.bias_vec) {
        if (key < N) {
          const float4 f = *reinterpret_cast<const float4*>(brow + key);
          b4[0] = f.x; b4[1] = f.y; b4[2] = f.z; b4[3] = f.w;
        } else {
          b4[0] = b4[1] = b4[2] = b4[3] = 0.0f;
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) b4[t] = key + t < N ? brow[key + t] : 0.0f;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) s[kb][g * 4 + t] += b4[t] * opt.inv_scale;
    }
  }
}

template <int D, bool kCausal, bool kNext, bool kBias>
__device__ __forceinline__ void tile_step(const char* kbuf_next, const char* vbuf,
                                          const LaneOffsets<D>& off, int j, int N, int kvlen,
                                          int qw, int qrow, int half, float scale_log2,
                                          const float* brow, const AttnOptions& opt,
                                          const bf16x8 (&qreg)[D / 16], f32x16 (&scur)[2],
                                          f32x16 (&snext)[2], f32x16 (&oacc)[D / 32],
                                          float& m_run, float& l_run) {
  constexpr int kDC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kRow = D * 2;  // bytes per key row
  const int k0 = j * kBN;

  if constexpr (kBias) {
    if (qrow < N) add_bias(scur, brow, k0, half, N, opt);
  }
  // A4: hide keys past the causal diagonal or past the valid keys.
  const bool need_mask = (kCausal && k0 + kBN - 1 > qw) || (k0 + kBN > kvlen);
  if (need_mask) {
    // Keys k0 + (i / 4) * 8 + half * 4 + i % 4 (+ 32) are visible when below
    // lim; compare the constant part against lim - k0 - 4 * half.
    const int lim = (kCausal ? min(kvlen, qrow + 1) : kvlen) - k0 - half * 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = (i >> 2) * 8 + (i & 3);
      scur[0][i] = kk < lim ? scur[0][i] : kNegInf;
      scur[1][i] = kk + 32 < lim ? scur[1][i] : kNegInf;
    }
  }

  // A5: online-softmax update for this lane's query row.
  float mx = __builtin_fmaxf(scur[0][0], scur[1][0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = max3(mx, scur[0][i], scur[1][i]);
  mx = __builtin_fmaxf(mx, swap_halves(mx));
  const float mt = mx * scale_log2;
  const float m_new = mt > m_run + kLag ? mt : m_run;
  const float ref = finite_ref(m_new);
  const float alpha = exp2_hw(m_run - ref);
  float psum = 0.0f;
  bf16x8 pb[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    uint32_t w[4];
#pragma unroll
    for (int jj = 0; jj < 8; jj += 2) {
      const float sa = scur[kc >> 1][(kc & 1) * 8 + jj];
      const float sb = scur[kc >> 1][(kc & 1) * 8 + jj + 1];
      const float pa = exp2_hw(__builtin_fmaf(sa, scale_log2, -ref));
      const float pbv = exp2_hw(__builtin_fmaf(sb, scale_log2, -ref));
      psum += pa + pbv;
      w[jj / 2] = pack_bf16x2(pa, pbv);
    }
    pb[kc] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  l_run = l_run * alpha + psum;
  m_run = m_new;

  // A6: rescale the accumulator (skipped when alpha is 1 on every lane),
  // then O^T += V^T P^T.
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
    // The empty asm keeps this a branch: without it the compiler would
    // multiply unconditionally, since scaling by 1 is harmless.
    asm volatile("");
#pragma unroll
    for (int b = 0; b < kDB; ++b) oacc[b] *= alpha;
  }
  // Transposed V reads: lane (group g = lane / 16, r = lane % 16) supplies the
  // address of dims [d0 + 4 (r % 4), +4) of key row base + r / 4; it receives
  // dims d0 + r of keys base .. base + 3 (d0 = 32 b + 16 (g % 2)).
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
    for (int b = 0; b < kDB; ++b) {
      const char* p0 = vbuf + off.v[b] + kc * 16 * kRow;
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(p0));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(p0 + 8 * kRow));
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[b] = mfma32(a, pb[kc], oacc[b]);
    }
  }
  // A3 for tile j + 1: its products follow this tile's in one stream.
  if constexpr (kNext) compute_scores<D>(kbuf_next, off, qreg, snext);
}

// With kSplit, workgroup (head, query tile, split) covers only its share of
// the key tiles and writes a partial result normalised by its own l -- O_s in
// float32 and LSE_s -- to o_part / lse_part; attn_split_merge_kernel combines
// the splits.
template <int D, bool kCausal, bool kBias, bool kSplit>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int BH,
    int H, int N, float scale_log2, AttnOptions opt, int splits, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  using T = Tile<D>;
  constexpr int kDC = D / 16;
  constexpr int kDB = D / 32;
  // Two K buffers and two V buffers: tile j's K sits in kbuf[j & 1], its V in
  // vbuf[j & 1].
  __shared__ __attribute__((aligned(1024))) char kbuf0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char kbuf1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char vbuf0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char vbuf1[T::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // the query row this lane works on (within the wave)
  const int half = lane >> 5;  // which 8-element half of each 16-wide slice

  const int nqt = (N + kBM - 1) / kBM;
  int bh, qt, split = 0;
  if constexpr (kSplit) {
    tile_of_split(blockIdx.x, nqt, splits, BH, kCausal, bh, qt, split);
  } else {
    tile_of(blockIdx.x, nqt, BH, kCausal, bh, qt);
  }
  const int64_t head_off = (int64_t)bh * N * D;
  const int head_bytes = N * D * 2;
  const uint16_t* kh = k + head_off;
  const uint16_t* vh = v + head_off;

  const int q0 = qt * kBM;
  const int qw = q0 + wave * 32;  // first query row of this wave
  const int qrow = qw + col;      // this lane's query row
  const int b = bh / H, h = bh % H;
  const int kvlen = opt.kv_len ? min(max(opt.kv_len[b], 0), N) : N;
  const float* brow = kBias ? opt.bias + b * opt.bias_stride_b + h * opt.bias_stride_h +
                                  (int64_t)min(qrow, N - 1) * N
                            : nullptr;

  const int kv_end = kCausal ? min(kvlen, q0 + kBM) : kvlen;
  const int ntiles_all = (kv_end + kBN - 1) / kBN;
  // Key tiles [j_begin, j_end) of this workgroup (all of them without splits).
  int j_begin = 0, j_end = ntiles_all;
  if constexpr (kSplit) {
    const int per = (ntiles_all + splits - 1) / splits;
    j_begin = min(split * per, ntiles_all);
    j_end = min(j_begin + per, ntiles_all);
  }
  const int ntiles = j_end - j_begin;
  // Last key tile with work for this wave (below j_begin: none).
  const int jw_last =
      (qw >= N || ntiles == 0) ? -1 : (kCausal ? min(j_end - 1, (qw + 31) / kBN) : j_end - 1);

  // A2 prologue: K and V of the first tile and K of the second in flight.
  issue_tile<D, T::k_swz>(kbuf0, kh, head_bytes, j_begin * kBN, wave, lane);
  issue_tile<D, T::v_swz>(vbuf0, vh, head_bytes, j_begin * kBN, wave, lane);
  if (ntiles > 1) issue_tile<D, T::k_swz>(kbuf1, kh, head_bytes, (j_begin + 1) * kBN, wave, lane);

  // A1: this lane's part of Q as the B operand of S^T = K Q^T.
  bf16x8 qreg[kDC];
  const uint16_t* qg = q + head_off + (int64_t)qrow * D + half * 8;
#pragma unroll
  for (int c = 0; c < kDC; ++c) {
    qreg[c] = qrow < N ? *reinterpret_cast<const bf16x8*>(qg + c * 16) : bf16x8{};
  }

  const LaneOffsets<D> off = lane_offsets<D>(lane);
  f32x16 oacc[kDB];
#pragma unroll
  for (int b = 0; b < kDB; ++b) oacc[b] = f32x16{};
  float m_run = kNegInf;  // exponent reference, in units of log2(e) * scale * S
  float l_run = 0.0f;     // this lane's half of the running sum
  f32x16 sA[2], sB[2];    // scores of the current and the next tile

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (jw_last >= j_begin) compute_scores<D>(kbuf0, off, qreg, sA);

  // A2: at the top of step j, K_{j+1} and V_j have landed and every wave is
  // done with the buffers of K_j and V_{j-1}, which then receive K_{j+2} and
  // V_{j+1}.  One barrier per key tile.
  for (int j = j_begin; j < j_end; j += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 2 < j_end) issue_tile<D, T::k_swz>(kbuf0, kh, head_bytes, (j + 2) * kBN, wave, lane);
    if (j + 1 < j_end) issue_tile<D, T::v_swz>(vbuf1, vh, head_bytes, (j + 1) * kBN, wave, lane);
    if (j < jw_last) {
      tile_step<D, kCausal, true, kBias>(kbuf1, vbuf0, off, j, N, kvlen, qw, qrow, half,
                                         scale_log2, brow, opt, qreg, sA, sB, oacc, m_run, l_run);
    } else if (j == jw_last) {
      tile_step<D, kCausal, false, kBias>(kbuf1, vbuf0, off, j, N, kvlen, qw, qrow, half,
                                          scale_log2, brow, opt, qreg, sA, sB, oacc, m_run, l_run);
    }
    if (j + 1 >= j_end) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 3 < j_end) issue_tile<D, T::k_swz>(kbuf1, kh, head_bytes, (j + 3) * kBN, wave, lane);
    if (j + 2 < j_end) issue_tile<D, T::v_swz>(vbuf0, vh, head_bytes, (j + 2) * kBN, wave, lane);
    if (j + 1 < jw_last) {
      tile_step<D, kCausal, true, kBias>(kbuf0, vbuf1, off, j + 1, N, kvlen, qw, qrow, half,
                                         scale_log2, brow, opt, qreg, sB, sA, oacc, m_run, l_run);
    } else if (j + 1 == jw_last) {
      tile_step<D, kCausal, false, kBias>(kbuf0, vbuf1, off, j + 1, N, kvlen, qw, qrow, half,
                                          scale_log2, brow, opt, qreg, sB, sA, oacc, m_run, l_run);
    }
  }

  // A7: O = O / l (deferred division), LSE = ln 2 * (m + log2 l).
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_val = l_tot > 0.0f ? (finite_ref(m_run) + log2_hw(l_tot)) * kLn2 : kNegInf;
  if (qrow < N) {
    if constexpr (kSplit) {
      const int64_t prow = ((int64_t)split * BH + bh) * N + qrow;
      float* orow = o_part + prow * D;
#pragma unroll
      for (int b = 0; b < kDB; ++b) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const float4 w = make_float4(oacc[b][gq * 4 + 0] * inv, oacc[b][gq * 4 + 1] * inv,
                                       oacc[b][gq * 4 + 2] * inv, oacc[b][gq * 4 + 3] * inv);
          *reinterpret_cast<float4*>(orow + b * 32 + gq * 8 + half * 4) = w;
        }
      }
      if (half == 0) lse_part[prow] = lse_val;
    } else {
      uint16_t* orow = o + head_off + (int64_t)qrow * D;
#pragma unroll
      for (int b = 0; b < kDB; ++b) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          // O^T rows b*32 + gq*8 + half*4 + (0..3): four consecutive dims.
          uint2 w;
          w.x = pack_bf16x2(oacc[b][gq * 4 + 0] * inv, oacc[b][gq * 4 + 1] * inv);
          w.y = pack_bf16x2(oacc[b][gq * 4 + 2] * inv, oacc[b][gq * 4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + b * 32 + gq * 8 + half * 4) = w;
        }
      }
      if (half == 0) lse[(int64_t)bh * N + qrow] = lse_val;
    }
  }
}

// Merge the splits of every query row: with M = max_s LSE_s and
// w_s = e^(LSE_s - M), LSE = M + log sum_s w_s and O = sum_s w_s O_s / sum_s w_s
// -- the (m, l) combine of §6.4.1 written for normalised partial outputs.
// One thread per (row, 4 dims); splits are folded in index order.
template <int D>
__global__ __launch_bounds__(256) void attn_split_merge_kernel(const float* __restrict__ o_part,
                                                                const float* __restrict__ lse_part,
                                                                uint16_t* __restrict__ o,
                                                                float* __restrict__ lse,
                                                                int64_t rows, int splits) {
  constexpr int kQuads = D / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * kQuads) return;
  const int64_t row = idx / kQuads;
  const int dq = (int)(idx % kQuads);
  float M = kNegInf;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, lse_part[s * rows + row]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.0f;
  if (M != kNegInf) {
    for (int s = 0; s < splits; ++s) {
      const float w = exp2_hw((lse_part[s * rows + row] - M) * kLog2e);
      const float4 p = *reinterpret_cast<const float4*>(o_part + (s * rows + row) * D + dq * 4);
      acc.x += w * p.x;
      acc.y += w * p.y;
      acc.z += w * p.z;
      acc.w += w * p.w;
      L += w;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint2 out;
  out.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  out.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(o + row * D + dq * 4) = out;
  if (dq == 0) lse[row] = L > 0.0f ? M + log2_hw(L) * kLn2 : kNegInf;
}

template <int D, bool kCausal, bool kBias, bool kSplit>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int H,
                  int N, float scale, const AttnOptions& opt, int splits, float* o_part,
                  float* lse_part, hipStream_t s) {
  const int nqt = (N + kBM - 1) / kBM;
  const float scale_log2 = scale * kLog2e;
  hipLaunchKernelGGL((attn_fwd_kernel<D, kCausal, kBias, kSplit>),
                     dim3(nqt * BH * (kSplit ? splits : 1)), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, BH, H, N,
                     scale_log2, opt, splits, o_part, lse_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !kSplit) return e;
  const int64_t rows = (int64_t)BH * N;
  const int64_t threads = rows * (D / 4);
  hipLaunchKernelGGL((attn_split_merge_kernel<D>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, s, o_part, lse_part, static_cast<uint16_t*>(o), lse, rows,
                     splits);
  return hipGetLastError();
}

template <int D, bool kSplit>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                    int H, int N, float scale, bool causal, const AttnOptions& opt, int splits,
                    float* o_part, float* lse_part, hipStream_t s) {
  if (opt.bias != nullptr) {
    return causal ? launch<D, true, true, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt, splits,
                                                  o_part, lse_part, s)
                  : launch<D, false, true, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt, splits,
                                                   o_part, lse_part, s);
  }
  return causal ? launch<D, true, false, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt, splits,
                                                 o_part, lse_part, s)
                : launch<D, false, false, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt, splits,
                                                  o_part, lse_part, s);
}

AttnOptions make_options(int N, float scale, const int32_t* kv_len, const float* bias,
                         int64_t bias_stride_b, int64_t bias_stride_h) {
  AttnOptions opt;
  opt.kv_len = kv_len;
  opt.bias = bias;
  opt.bias_stride_b = bias_stride_b;
  opt.bias_stride_h = bias_stride_h;
  opt.inv_scale = 1.0f / scale;
  opt.bias_vec = bias != nullptr && (N % 4) == 0 && (bias_stride_b % 4) == 0 &&
                 (bias_stride_h % 4) == 0 && (reinterpret_cast<uintptr_t>(bias) % 16) == 0;
  return opt;
}

}  // namespace

hipError_t attn_fwd_launch(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int D, float scale, bool causal,
                           const int32_t* kv_len, const float* bias, int64_t bias_stride_b,
                           int64_t bias_stride_h, hipStream_t stream) {
  const int BH = B * H;
  const AttnOptions opt = make_options(N, scale, kv_len, bias, bias_stride_b, bias_stride_h);
  if (D == 64)
    return launch_d<64, false>(q, k, v, o, lse, BH, H, N, scale, causal, opt, 1, nullptr, nullptr,
                               stream);
  return launch_d<128, false>(q, k, v, o, lse, BH, H, N, scale, causal, opt, 1, nullptr, nullptr,
                              stream);
}

int64_t attn_split_workspace(int B, int H, int N, int D, int splits) {
  return (int64_t)splits * B * H * N * (D + 1) * (int64_t)sizeof(float);
}

hipError_t attn_fwd_split_launch(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int H, int N, int D, float scale, bool causal,
                                 const int32_t* kv_len, const float* bias, int64_t bias_stride_b,
                                 int64_t bias_stride_h, int splits, void* workspace,
                                 hipStream_t stream) {
  const int BH = B * H;
  const AttnOptions opt = make_options(N, scale, kv_len, bias, bias_stride_b, bias_stride_h);
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = o_part + (int64_t)splits * BH * N * D;
  if (D == 64)
    return launch_d<64, true>(q, k, v, o, lse, BH, H, N, scale, causal, opt, splits, o_part,
                              lse_part, stream);
  return launch_d<128, true>(q, k, v, o, lse, BH, H, N, scale, causal, opt, splits, o_part,
                             lse_part, stream);
}

}  // namespace osm
