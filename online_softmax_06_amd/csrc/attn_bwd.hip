// Fused attention backward on gfx950: dQ, dK, dV of O = softmax(scale Q K^T) V
// from Q, K, V, the output O, its per-row log-sum-exp and the upstream
// gradient dO, with the scores recomputed on the matrix cores and no N x N
// matrix in HBM.
//
// Method.  The forward keeps only O and one log-sum-exp per query row
// ("Ch.6 Softmax and Online Softmax" §6.5), and the backward rebuilds the
// probabilities from them instead of reading a stored S (xxqk §5.2: compute
// traded for memory):  P = 2^(S' - LSE log2 e) with S' = S * scale * log2 e,
// which is the normalised softmax without any running max.  The gradients are
// those of the forward map:
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Delta),   Delta_i = sum_j P_ij dP_ij,
//     dQ = scale dS K,   dK = scale dS^T Q,
// with Delta_i computed as the row dot product dO_i . O_i (equal to the sum
// above because O_i = sum_j P_ij V_j), so it costs one pass over O and dO.
//
// Two launches, no atomics (the result is deterministic):
//   dq    a workgroup owns 128 query rows (32 per wavefront), computes their
//         Delta and LSE * log2 e from its own loads of O, dO and LSE and
//         writes -Delta and LSE * log2 e to a padded workspace for dkdv
//         (padding rows get 0 and +inf, so their P is exactly 0), keeps Q,
//         dO, Delta, LSE and the dQ^T accumulator in registers and streams
//         the 64-key tiles of K and V: S^T = K Q^T, dP^T = V dO^T, P, dS,
//         then dQ^T += K^T dS^T;
//   dkdv  a workgroup owns 128 keys (32 per wavefront), keeps their K rows
//         in LDS, their V fragments and the dK^T, dV^T accumulators in
//         registers, and streams 32-row tiles of Q and dO (plus their -Delta
//         and LSE) through LDS: per tile S = Q K^T, dP = dO V^T, P, dS, then
//         dV^T += dO^T P and dK^T += Q^T dS (two workgroups per CU).
// Both kernels start the dP accumulator from -Delta instead of zero, so the
// products leave dP - Delta and dS = P * dP costs one multiply.
// dkdv repeats two of the dq kernel's products (the scores and dP) instead
// of adding partial dQ into HBM with atomics.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, wave64).  A product whose
// output has lanes = the index kept by the wavefront and registers = the
// streamed index feeds the next product directly as its B operand, when that
// product contracts over the streamed index.  The streamed tiles are read
// twice: row-wise (16 bytes per lane, A operand of the first products) and
// transposed (ds_read_b64_tr_b16, A operand of the accumulating products).
// One XOR swizzle of the 16-byte units serves both reads without bank
// conflicts (see Geo::swz).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "osm_device.h"
#include "osm_internal.h"

// Scratch memory of the allocation-free backward (osm_attn_bwd_noalloc): the
// per-row -Delta and LSE * log2 e arrays live here instead of in a caller's
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it names a stand-in, not device memory): it uses the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[osm::kAttnBwdScratchBytes];

namespace osm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlk = 128;  // keys per dK/dV workgroup; query rows per dQ workgroup
constexpr int kTile = 64;  // rows of a streamed tile (query rows or keys)
constexpr int kPad = 128;  // per-head row padding of the Delta / LSE arrays

// Buffer descriptor word 3 for raw (untyped) buffer loads on gfx950.
constexpr int kBufferFlags = 0x00020000;

#define OSM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Geometry of the streamed tiles: rows of D bfloat16, row-major in LDS, with
// 16-byte units swizzled per row (kBytes: one kTile-row tile).
template <int D>
struct Geo {
  static constexpr int kUnits = D / 8;     // 16-byte units per row
  static constexpr int kRow = D * 2;       // bytes per row
  static constexpr int kBytes = kTile * kRow;
  static constexpr int kDC = D / 16;       // 16-wide slices of the head dimension
  static constexpr int kDB = D / 32;       // 32-wide blocks of the head dimension
  // Unit u of row r sits at unit u ^ swz(r).
  //  * Row reads: 16 lanes read one unit of 16 consecutive rows; swz takes 16
  //    distinct values on them (D = 128: 16 units per 256-byte row) or 8
  //    distinct values on the rows of each parity (D = 64: two rows per
  //    256-byte bank sweep), so the 16 units hit disjoint banks.
  //  * Transposed reads: 32 lanes read 64 contiguous bytes of 4 consecutive
  //    rows; swz moves the four rows to four different 64-byte quarters of
  //    the bank space.
  // Rows r and r + 8 differ by kPartXor in their byte offset.
  __device__ static int swz(int r) {
    if constexpr (D == 128) return (((r & 3) << 2) | ((r & 4) >> 1)) ^ ((r >> 3) & 1);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  static constexpr int kPartXor = D == 128 ? 16 : 32;
};

// Global->LDS copy of rows [row0, row0 + kRows) of one head (row-major,
// D bfloat16 per row) into `lds`, swizzled: copy i of wave w fills LDS bytes
// [(w * kPerWave + i) * 1024, +1024), one 16-byte unit per lane at the
// per-lane source offset off[i].  The buffer descriptor starts at row0 and
// ends with the head, so rows past the head arrive as zeros.
template <int D, int kRows>
struct RowCopy {
  static constexpr int kPerWave = kRows * (D / 8) / 64 / kWaves;
  static_assert(kPerWave >= 1, "every wave issues at least one copy");
  __device__ static void offsets(int wave, int lane, int (&off)[kPerWave]) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int p = (wave * kPerWave + i) * 64 + lane;  // physical unit in the block
      const int r = p / (D / 8), u = p % (D / 8);
      off[i] = r * (D * 2) + ((u ^ Geo<D>::swz(r)) << 4);
    }
  }
  __device__ static void issue(char* lds, const uint16_t* head, int head_bytes, int row0,
                               int wave, const int (&off)[kPerWave]) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int left = head_bytes - row0 * (D * 2);
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(head + (int64_t)row0 * D), 0,
                                                        left > 0 ? left : 0, kBufferFlags);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, OSM_LDS(lds + (wave * kPerWave + i) * 1024),
                                               16, off[i], 0, 0, 0);
#endif
  }
};

// Global->LDS copy of n <= 64 floats starting at `src` into lds[0, 64): lane i
// copies element i; lanes at or past n store zeros (outside the descriptor).
__device__ __forceinline__ void copy_vec(float* lds, const float* src, int n, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, n * 4, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, OSM_LDS(lds), 4, lane * 4, 0, 0, 0);
#endif
}

// Per-lane LDS byte offsets for the two reads of a streamed tile.
//   row: lane reads row (lane % 32) of a 32-row sub-tile, unit 2 c + half of
//        slice c at offset row ^ (c << 5).
//   tr[b]: transposed read of dim block b: lane (g = lane / 16, r = lane % 16)
//        supplies the address of dims [32 b + 16 (g % 2) + 4 (r % 4), +4) of
//        row 4 half + r / 4 of a 16-row slice (rows +8 for the second read of
//        the slice) and receives dim 32 b + lane % 32 of four consecutive rows.
template <int D>
struct ReadOffsets {
  int row;
  int tr[D / 32];
  int trx[D / 32];  // tr[b] ^ kPartXor: the same read 8 rows further down
};

template <int D>
__device__ __forceinline__ ReadOffsets<D> read_offsets(int lane) {
  using G = Geo<D>;
  const int col = lane & 31, half = lane >> 5;
  ReadOffsets<D> o;
  o.row = col * G::kRow + ((half ^ G::swz(col)) << 4);
  const int g = lane >> 4, r = lane & 15;
  const int trow = half * 4 + (r >> 2);
  const int td = (g & 1) * 16 + 4 * (r & 3);
#pragma unroll
  for (int b = 0; b < G::kDB; ++b) {
    const int d = b * 32 + td;
    o.tr[b] = trow * G::kRow + (((d >> 3) ^ G::swz(trow)) << 4) + (d & 7) * 2;
    o.trx[b] = o.tr[b] ^ G::kPartXor;
  }
  return o;
}

// A operand of an accumulating product: dims [32 b, +32) x rows
// {r0 + 4 half + 0..3, r0 + 8 + 4 half + 0..3} of a streamed tile (r0 a
// multiple of 16), transposed; the row order is the register order of a
// 32 x 32 product output, so P and dS enter as B operands unchanged.
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char* tile, const ReadOffsets<D>& off, int b,
                                          int r0) {
  using G = Geo<D>;
  // Adding whole rows leaves the bits of kPartXor alone, so both offsets are
  // a per-lane register plus a constant.
  const int o0 = off.tr[b] + r0 * G::kRow;
  const int o1 = off.trx[b] + (r0 + 8) * G::kRow;
  const s16x4 v0 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + o0));
  const s16x4 v1 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + o1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand of a first product: rows [r0, r0 + 32) of a streamed tile, slice c.
template <int D>
__device__ __forceinline__ bf16x8 read_row(const char* tile, const ReadOffsets<D>& off, int c,
                                           int r0) {
  return *reinterpret_cast<const bf16x8*>(tile + r0 * Geo<D>::kRow + (off.row ^ (c << 5)));
}

// Registers 8 kc2 .. 8 kc2 + 7 of a 32 x 32 product output, as a bfloat16
// B operand.
__device__ __forceinline__ bf16x8 pack8(const float (&x)[16], int kc2) {
  const int o = kc2 * 8;
  return __builtin_bit_cast(
      bf16x8, make_uint4(pack_bf16x2(x[o + 0], x[o + 1]), pack_bf16x2(x[o + 2], x[o + 3]),
                         pack_bf16x2(x[o + 4], x[o + 5]), pack_bf16x2(x[o + 6], x[o + 7])));
}

// Output register i of a 32 x 32 product sits in row rho(i) + 4 half.
__device__ __forceinline__ constexpr int rho(int i) { return (i >> 2) * 8 + (i & 3); }

// The two first products of a 32-row sub-tile, s1 = A1 B1 and
// s2 = s2_init + A2 B2 over the kDC slices of the head dimension: A rows
// [r0, r0 + 32) of the
// streamed tiles t1 and t2, B in registers.  Each region (fenced by
// sched_barrier) issues one product of each and the LDS reads of the next
// slice, so few operands are live at a time.
template <int D, int kAhead>
__device__ __forceinline__ void first_products(const char* t1, const char* t2,
                                               const ReadOffsets<D>& off, int r0,
                                               const bf16x8 (&b1)[D / 16],
                                               const bf16x8 (&b2)[D / 16], f32x16& s1,
                                               f32x16& s2, const f32x16& s2_init) {
  constexpr int kDC = D / 16, kBuf = kAhead + 1;
  bf16x8 a1[kBuf], a2[kBuf];
#pragma unroll
  for (int c = 0; c < kAhead; ++c) {
    a1[c] = read_row<D>(t1, off, c, r0);
    a2[c] = read_row<D>(t2, off, c, r0);
  }
  s1 = f32x16{};
  s2 = s2_init;
#pragma unroll
  for (int c = 0; c < kDC; ++c) {
    if (c + kAhead < kDC) {
      a1[(c + kAhead) % kBuf] = read_row<D>(t1, off, c + kAhead, r0);
      a2[(c + kAhead) % kBuf] = read_row<D>(t2, off, c + kAhead, r0);
    }
    s1 = mfma32(a1[c % kBuf], b1[c], s1);
    s2 = mfma32(a2[c % kBuf], b2[c], s2);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The accumulating products of a 32-row sub-tile: for each 16-row slice kc2
// and dim block b, acc1[b] += T1^T B1[kc2] (and acc2[b] += T2^T B2[kc2] when
// kTwo), the A operands read transposed from the streamed tiles one step
// ahead, in fenced regions.
template <int D, bool kTwo, int kAhead>
__device__ __forceinline__ void acc_products(const char* t1, const char* t2,
                                             const ReadOffsets<D>& off, int r0,
                                             const bf16x8 (&b1)[2], const bf16x8 (&b2)[2],
                                             f32x16 (&acc1)[D / 32], f32x16 (&acc2)[D / 32]) {
  constexpr int kDB = D / 32, kSteps = 2 * kDB, kBuf = kAhead + 1;
  bf16x8 x1[kBuf], x2[kBuf];
  auto fetch = [&](int i) __attribute__((always_inline)) {
    const int rn = r0 + 16 * (i / kDB), bn = i % kDB;
    x1[i % kBuf] = read_tr<D>(t1, off, bn, rn);
    if constexpr (kTwo) x2[i % kBuf] = read_tr<D>(t2, off, bn, rn);
  };
#pragma unroll
  for (int i = 0; i < kAhead; ++i) fetch(i);
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int kc2 = i / kDB, b = i % kDB;
    if (i + kAhead < kSteps) fetch(i + kAhead);
    acc1[b] = mfma32(x1[i % kBuf], b1[kc2], acc1[b]);
    if constexpr (kTwo) acc2[b] = mfma32(x2[i % kBuf], b2[kc2], acc2[b]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Map a linear workgroup id to (batch*head, block rank); rank 0 is the
// heaviest block under the causal mask.  Workgroups go round-robin over the 8
// XCDs; when B*H is a multiple of 8, the heads an XCD owns are those with
// bh mod 8 equal to it, so its L2 holds their streamed tiles.
//   kCausal: the heads of an XCD in groups of kGroup; within a group
//            rank-major (every head's rank-0 block, then every rank-1
//            block, ...), groups in order.  Heavy blocks then start first
//            and no heavy block is dispatched late to set the end of the
//            launch, while an XCD still streams the tiles of few heads at a
//            time.
//   otherwise: head-major, all blocks of a head together (equal work; the
//            fewest heads in flight per XCD).
// Measured interleaved, causal D = 128: B8 H40 N2048 1136 us against 1246
// us head-major and 1183 us rank-major over all of an XCD's heads (which
// also fetched 3.4x the bytes from beyond L2); B16 H40 N1024 +11%,
// B8 H40 N2048 D = 64 +6%.  Without the mask, head-major is fastest.
constexpr int kGroup = 8;

template <bool kCausal>
__device__ __forceinline__ void block_of(int L, int per_head, int BH, int& bh, int& rank) {
  if ((BH & 7) == 0) {
    const int xcd = L & 7, idx = L >> 3;
    const int hpx = BH >> 3;
    if constexpr (kCausal) {
      const int grp = idx / (kGroup * per_head);
      const int gsz = min(kGroup, hpx - grp * kGroup);  // heads in this group
      const int r = idx - grp * kGroup * per_head;
      bh = (grp * kGroup + r % gsz) * 8 + xcd;
      rank = r / gsz;
    } else {
      bh = (idx / per_head) * 8 + xcd;
      rank = idx % per_head;
    }
  } else if constexpr (kCausal) {
    const int grp = L / (kGroup * per_head);
    const int gsz = min(kGroup, BH - grp * kGroup);
    const int r = L - grp * kGroup * per_head;
    bh = grp * kGroup + r % gsz;
    rank = r / gsz;
  } else {
    bh = L / per_head;
    rank = L % per_head;
  }
}

// ---------------------------------------------------------------------------
// dkdv: dK and dV of 128 keys per workgroup (32 per wavefront), two
// workgroups per CU.  The block's K rows stay in LDS (B operand of the
// scores, read like a streamed tile), its V fragments in registers, and the
// query rows stream through LDS 32 at a time, double-buffered.
// ---------------------------------------------------------------------------
template <int D, bool kCausal>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ delta, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int BH, int H, int N, int Np, const int32_t* __restrict__ kv_len,
    float scale, float scale_log2) {
  using G = Geo<D>;
  constexpr int kDC = G::kDC, kDB = G::kDB;
  constexpr int kSub = 32;  // query rows per streamed tile
  using KCopy = RowCopy<D, kBlk>;
  using QCopy = RowCopy<D, kSub>;
  // K of the block, and two stages of Q, dO, LSE and Delta tiles, each its
  // own array so that every copy names its target at compile time.
  __shared__ __attribute__((aligned(1024))) char ks[kBlk * G::kRow];
  __shared__ __attribute__((aligned(1024))) char qs0[kSub * G::kRow];
  __shared__ __attribute__((aligned(1024))) char qs1[kSub * G::kRow];
  __shared__ __attribute__((aligned(1024))) char gs0[kSub * G::kRow];
  __shared__ __attribute__((aligned(1024))) char gs1[kSub * G::kRow];
  __shared__ __attribute__((aligned(256))) float ls0[64];
  __shared__ __attribute__((aligned(256))) float ls1[64];
  __shared__ __attribute__((aligned(256))) float es0[64];
  __shared__ __attribute__((aligned(256))) float es1[64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int nkb = (N + kBlk - 1) / kBlk;
  int bh, kb;
  block_of<kCausal>(blockIdx.x, nkb, BH, bh, kb);  // causal: kb = rank, the heaviest first
  const int64_t head = (int64_t)bh * N * D;
  const int head_bytes = N * D * 2;
  const int kw = kb * kBlk + wave * 32;  // first key of this wave
  const int key = kw + col;              // this lane's key
  // Keys at or past the batch's key length are hidden from every row.
  const int kvlen = kv_len ? min(max(kv_len[bh / H], 0), N) : N;
  f32x16 dka[kDB], dva[kDB];
#pragma unroll
  for (int b = 0; b < kDB; ++b) dka[b] = dva[b] = f32x16{};
  // A block wholly past the key length has dK = dV = 0 (uniform over the
  // workgroup: no barrier is skipped by part of it).
  if (kb * kBlk < kvlen) {

  {
    int koff[KCopy::kPerWave];
    KCopy::offsets(wave, lane, koff);
    KCopy::issue(ks, k + head, head_bytes, kb * kBlk, wave, koff);
  }
  // B operand of dP = dO V^T: key `key`, dims 16 c + 8 half + 0..7.
  bf16x8 vreg[kDC];
#pragma unroll
  for (int c = 0; c < kDC; ++c) {
    const int64_t e = head + (int64_t)key * D + c * 16 + half * 8;
    vreg[c] = key < N ? *reinterpret_cast<const bf16x8*>(v + e) : bf16x8{};
  }

  int coff[QCopy::kPerWave];
  QCopy::offsets(wave, lane, coff);
  const ReadOffsets<D> off = read_offsets<D>(lane);
  const float* lse2_h = lse2 + (int64_t)bh * Np;
  const float* delta_h = delta + (int64_t)bh * Np;
  const char* krows = ks + wave * 32 * G::kRow;  // this wave's 32 keys

  const int nst = (N + kSub - 1) / kSub;
  // Causal: query rows below the block's first key see none of its keys.
  const int t_begin = kCausal ? kb * (kBlk / kSub) : 0;

  auto issue = [&](char* qb, char* gb, float* lb, float* eb, int t) __attribute__((always_inline)) {
    const int row0 = t * kSub;
    QCopy::issue(qb, q + head, head_bytes, row0, wave, coff);
    QCopy::issue(gb, dout + head, head_bytes, row0, wave, coff);
    if (wave == 0) copy_vec(lb, lse2_h + row0, kSub, lane);
    if (wave == 1) copy_vec(eb, delta_h + row0, kSub, lane);
  };

  // One 32-row tile: S = Q K^T and dP = dO V^T, P and dS, then
  // dV^T += dO^T P and dK^T += Q^T dS.
  auto compute = [&](auto masked, const char* qb, const char* gb, const float* lb,
                     const float* eb, int t) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
    const int qbase = t * kSub;  // first query row of the tile
    // Masked tiles: skip when every key of this wave is hidden from every
    // row of the tile (causal: all rows before the keys; or all keys past
    // the key length).
    if (kMasked && ((kCausal && kw > qbase + 31) || kw >= kvlen)) return;
    // dP starts from -Delta of its rows (register i: row rho(i) + 4 half, four
    // rows per 16-byte read), so the products leave dP - Delta.
    f32x16 sc = f32x16{}, dp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 e4 = *reinterpret_cast<const f32x4*>(eb + 8 * j + 4 * half);
#pragma unroll
      for (int r = 0; r < 4; ++r) dp[4 * j + r] = e4[r];
    }
    {
      constexpr int kAhead = 2, kBuf = kAhead + 1;
      bf16x8 a1[kBuf], a2[kBuf], bk[kBuf];
      auto fetch = [&](int c) __attribute__((always_inline)) {
        a1[c % kBuf] = read_row<D>(qb, off, c, 0);
        bk[c % kBuf] = read_row<D>(krows, off, c, 0);
        a2[c % kBuf] = read_row<D>(gb, off, c, 0);
      };
#pragma unroll
      for (int c = 0; c < kAhead; ++c) fetch(c);
#pragma unroll
      for (int c = 0; c < kDC; ++c) {
        if (c + kAhead < kDC) fetch(c + kAhead);
        sc = mfma32(a1[c % kBuf], bk[c % kBuf], sc);
        dp = mfma32(a2[c % kBuf], vreg[c], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Key `key` is visible from row qbase + 4 half + rho when rho >= lim.
    const int lim = key - qbase - 4 * half;
    // P (into sc) and dS (into dp), four rows at a time: rows 8 j + 4 half +
    // 0..3, whose LSE is one 16-byte read.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lb + 8 * j + 4 * half);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * j + r;
        float x = exp2_hw(__builtin_fmaf(sc[i], scale_log2, -l4[r]));
        if (kMasked && ((kCausal && rho(i) < lim) || key >= kvlen)) x = 0.0f;
        sc[i] = x;
        dp[i] = x * dp[i];
      }
    }
    float p[16], ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = sc[i];
      ds[i] = dp[i];
    }
    const bf16x8 pb[2] = {pack8(p, 0), pack8(p, 1)};
    const bf16x8 db[2] = {pack8(ds, 0), pack8(ds, 1)};
    __builtin_amdgcn_sched_barrier(0);
    acc_products<D, true, 2>(gb, qb, off, 0, pb, db, dva, dka);
  };

  using Masked = std::integral_constant<bool, true>;
  using Plain = std::integral_constant<bool, false>;
  using Stage0 = std::integral_constant<int, 0>;
  using Stage1 = std::integral_constant<int, 1>;
  // Tile t sits in stage (t - t_begin) & 1.  A step waits for its tile,
  // starts the copy of the next one into the other stage and computes.
  auto step = [&](auto masked, auto stage, int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (decltype(stage)::value == 0) {
      if (t + 1 < nst) issue(qs1, gs1, ls1, es1, t + 1);
      compute(masked, qs0, gs0, ls0, es0, t);
    } else {
      if (t + 1 < nst) issue(qs0, gs0, ls0, es0, t + 1);
      compute(masked, qs1, gs1, ls1, es1, t);
    }
  };

  issue(qs0, gs0, ls0, es0, t_begin);
  int t = t_begin;
  if (kb * kBlk + kBlk > kvlen) {
    // The block holds the key length: every tile masks its keys.
    for (; t + 1 < nst; t += 2) {
      step(Masked{}, Stage0{}, t);
      step(Masked{}, Stage1{}, t + 1);
    }
    if (t < nst) step(Masked{}, Stage0{}, t);
  } else {
    if constexpr (kCausal) {
      // The four tiles over the block's own key range cross the diagonal.
      step(Masked{}, Stage0{}, t);
      if (t + 1 < nst) step(Masked{}, Stage1{}, t + 1);
      if (t + 2 < nst) step(Masked{}, Stage0{}, t + 2);
      if (t + 3 < nst) step(Masked{}, Stage1{}, t + 3);
      t += 4;
    }
    for (; t + 1 < nst; t += 2) {
      step(Plain{}, Stage0{}, t);
      step(Plain{}, Stage1{}, t + 1);
    }
    if (t < nst) step(Plain{}, Stage0{}, t);
  }
  }  // kb * kBlk < kvlen

  // dK^T and dV^T: lane = key, register i of block b = dim 32 b + 8 (i / 4)
  // + 4 half + i % 4.
  if (key < N) {
    uint16_t* dkr = dk + head + (int64_t)key * D;
    uint16_t* dvr = dv + head + (int64_t)key * D;
#pragma unroll
    for (int b = 0; b < kDB; ++b) {
      store_block_bf16(dkr + b * 32, dka[b], half, scale);
      store_block_bf16(dvr + b * 32, dva[b], half, 1.0f);
    }
  }
}

// ---------------------------------------------------------------------------
// dq: dQ of 128 query rows per workgroup.
// ---------------------------------------------------------------------------
template <int D, bool kCausal>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ o,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ lse2,
    float* __restrict__ delta, uint16_t* __restrict__ dq, int BH, int H, int N, int Np,
    const int32_t* __restrict__ kv_len, float scale, float scale_log2) {
  using G = Geo<D>;
  constexpr int kDC = G::kDC, kDB = G::kDB;
  __shared__ __attribute__((aligned(1024))) char ks0[G::kBytes];
  __shared__ __attribute__((aligned(1024))) char ks1[G::kBytes];
  __shared__ __attribute__((aligned(1024))) char vs0[G::kBytes];
  __shared__ __attribute__((aligned(1024))) char vs1[G::kBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int nqb = (N + kBlk - 1) / kBlk;
  int bh, rank;
  block_of<kCausal>(blockIdx.x, nqb, BH, bh, rank);
  const int qt = kCausal ? nqb - 1 - rank : rank;  // causal: the heaviest blocks first
  const int64_t head = (int64_t)bh * N * D;
  const int head_bytes = N * D * 2;
  const int qw = qt * kBlk + wave * 32;  // first query row of this wave
  const int qrow = qw + col;             // this lane's query row (< Np)

  // B operands of S^T = K Q^T and dP^T = V dO^T: row `qrow`, dims
  // 16 c + 8 half + 0..7.  The same dims of O give this lane's half of
  // Delta = dO . O; the lane 32 apart holds the other half.
  bf16x8 qreg[kDC], oreg[kDC];
  float dl = 0.0f;
#pragma unroll
  for (int c = 0; c < kDC; ++c) {
    const int64_t e = head + (int64_t)qrow * D + c * 16 + half * 8;
    qreg[c] = qrow < N ? *reinterpret_cast<const bf16x8*>(q + e) : bf16x8{};
    oreg[c] = qrow < N ? *reinterpret_cast<const bf16x8*>(dout + e) : bf16x8{};
    if (qrow < N) {
      const uint4 a = *reinterpret_cast<const uint4*>(o + e);
      const uint4 g = __builtin_bit_cast(uint4, oreg[c]);
      dl = __builtin_fmaf(bf16_lo(a.x), bf16_lo(g.x), dl);
      dl = __builtin_fmaf(bf16_hi(a.x), bf16_hi(g.x), dl);
      dl = __builtin_fmaf(bf16_lo(a.y), bf16_lo(g.y), dl);
      dl = __builtin_fmaf(bf16_hi(a.y), bf16_hi(g.y), dl);
      dl = __builtin_fmaf(bf16_lo(a.z), bf16_lo(g.z), dl);
      dl = __builtin_fmaf(bf16_hi(a.z), bf16_hi(g.z), dl);
      dl = __builtin_fmaf(bf16_lo(a.w), bf16_lo(g.w), dl);
      dl = __builtin_fmaf(bf16_hi(a.w), bf16_hi(g.w), dl);
    }
  }
  dl += __shfl_xor(dl, 32);
  // A row without a visible key (LSE = -inf) and a padding row get +inf:
  // every P of the row is then 2^-inf = 0.
  const float lv = qrow < N ? lse[(int64_t)bh * N + qrow] : kNegInf;
  const float l2 = lv == kNegInf ? __builtin_inff() : lv * kLog2e;
  // The grid covers the padded rows [0, Np) of every head exactly once.
  if (half == 0) {
    delta[(int64_t)bh * Np + qrow] = -dl;
    lse2[(int64_t)bh * Np + qrow] = l2;
  }
  // dP^T starts from -Delta, so its products leave dP - Delta.
  f32x16 ndl;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndl[i] = -dl;
  f32x16 dqa[kDB];
#pragma unroll
  for (int b = 0; b < kDB; ++b) dqa[b] = f32x16{};

  using KVCopy = RowCopy<D, kTile>;
  int coff[KVCopy::kPerWave];
  KVCopy::offsets(wave, lane, coff);
  const ReadOffsets<D> off = read_offsets<D>(lane);

  // Keys at or past the batch's key length are hidden from every row.
  const int kvlen = kv_len ? min(max(kv_len[bh / H], 0), N) : N;
  const int nkt = (kvlen + kTile - 1) / kTile;
  // Causal: keys past the block's last query row are hidden from all of it.
  const int t_end = kCausal ? min(nkt, (qt + 1) * (kBlk / kTile)) : nkt;
  // The last key visible from this lane's row, plus one.
  const int vis_end = kCausal ? min(qrow + 1, kvlen) : kvlen;

  auto issue = [&](char* kbuf, char* vbuf, int t) __attribute__((always_inline)) {
    KVCopy::issue(kbuf, k + head, head_bytes, t * kTile, wave, coff);
    KVCopy::issue(vbuf, v + head, head_bytes, t * kTile, wave, coff);
  };

  auto compute = [&](auto masked, const char* kbuf, const char* vbuf, int t) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r0 = s * 32;
      const int kbase = t * kTile + r0;  // first key of the sub-tile
      // Masked tiles: every key of the sub-tile is hidden from this wave.
      if (kMasked && (kbase >= kvlen || (kCausal && kbase > qw + 31))) continue;
      f32x16 sc, dp;
      // Operands read two slices ahead.
      first_products<D, 2>(kbuf, vbuf, off, r0, qreg, oreg, sc, dp, ndl);
      // Key kbase + 4 half + rho is visible from this row when rho < lim.
      const int lim = vis_end - kbase - 4 * half;
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = exp2_hw(__builtin_fmaf(sc[i], scale_log2, -l2));
        if (kMasked && rho(i) >= lim) x = 0.0f;
        ds[i] = x * dp[i];
      }
      const bf16x8 db[2] = {pack8(ds, 0), pack8(ds, 1)};
      __builtin_amdgcn_sched_barrier(0);
      acc_products<D, false, 2>(kbuf, kbuf, off, r0, db, db, dqa, dqa);
    }
  };
  using Masked = std::integral_constant<bool, true>;
  using Plain = std::integral_constant<bool, false>;
  using Stage0 = std::integral_constant<int, 0>;
  using Stage1 = std::integral_constant<int, 1>;
  // Tile t sits in stage t & 1.  A step waits for its tile, starts the copy
  // of the next one into the other stage and computes.
  auto step = [&](auto masked, auto stage, int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (decltype(stage)::value == 0) {
      if (t + 1 < t_end) issue(ks1, vs1, t + 1);
      compute(masked, ks0, vs0, t);
    } else {
      if (t + 1 < t_end) issue(ks0, vs0, t + 1);
      compute(masked, ks1, vs1, t);
    }
  };
  // Masked tiles, those crossing the causal diagonal or the end of the keys,
  // all come after the plain ones.  Each kind runs in a loop of its own, so
  // the accumulators keep one register assignment through every iteration.
  const int t_plain_end = min(min(kCausal ? qt * (kBlk / kTile) : nkt, kvlen / kTile), t_end);

  if (t_end > 0) issue(ks0, vs0, 0);
  int t = 0;
  for (; t + 1 < t_plain_end; t += 2) {
    step(Plain{}, Stage0{}, t);
    step(Plain{}, Stage1{}, t + 1);
  }
  if (t < t_plain_end) {
    step(Plain{}, Stage0{}, t);
    ++t;
    if (t < t_end) step(Masked{}, Stage1{}, t++);
  }
  for (; t + 1 < t_end; t += 2) {
    step(Masked{}, Stage0{}, t);
    step(Masked{}, Stage1{}, t + 1);
  }
  if (t < t_end) step(Masked{}, Stage0{}, t);

  // dQ^T: lane = query row, register i of block b = dim 32 b + 8 (i / 4) +
  // 4 half + i % 4.
  if (qrow < N) {
    uint16_t* dqr = dq + head + (int64_t)qrow * D;
#pragma unroll
    for (int b = 0; b < kDB; ++b) store_block_bf16(dqr + b * 32, dqa[b], half, scale);
  }
}

template <int D, bool kCausal>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int BH, int H, int N,
                      float scale, const int32_t* kv_len, void* workspace, hipStream_t stream) {
  const int Np = (N + kPad - 1) / kPad * kPad;
  float* delta = static_cast<float*>(workspace);
  float* lse2 = delta + (int64_t)BH * Np;
  const float scale_log2 = scale * kLog2e;
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  const auto* g16 = static_cast<const uint16_t*>(dout);
  // Np == number of dQ workgroups per head * kBlk: the dQ kernel writes
  // Delta and LSE * log2 e for every padded row, which dK/dV then reads.
  static_assert(kPad == kBlk, "one dQ workgroup per padded block of rows");
  const unsigned blocks = (unsigned)((int64_t)BH * ((N + kBlk - 1) / kBlk));
  attn_bwd_dq_kernel<D, kCausal><<<dim3(blocks), dim3(kThreads), 0, stream>>>(
      q16, k16, v16, static_cast<const uint16_t*>(o), g16, lse, lse2, delta,
      static_cast<uint16_t*>(dq), BH, H, N, Np, kv_len, scale, scale_log2);
  attn_bwd_dkdv_kernel<D, kCausal><<<dim3(blocks), dim3(kThreads), 0, stream>>>(
      q16, k16, v16, g16, lse2, delta, static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), BH,
      H, N, Np, kv_len, scale, scale_log2);
  return hipGetLastError();
}

}  // namespace

int64_t attn_bwd_workspace(int B, int H, int N) {
  const int64_t Np = ((int64_t)N + kPad - 1) / kPad * kPad;
  return 2 * 4 * (int64_t)B * H * Np;
}

hipError_t attn_bwd_scratch(void** ptr) {
  // One lookup per device, with that device current; the addresses are
  // kept for the life of the process.
  constexpr int kMaxDevices = 64;
  static std::mutex lock;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(lock);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t attn_bwd_launch(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                           int H, int N, int D, float scale, bool causal, const int32_t* kv_len,
                           void* workspace, hipStream_t stream) {
  const int BH = B * H;
  if (D == 128) {
    return causal ? launch_bwd<128, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, H, N, scale,
                                          kv_len, workspace, stream)
                  : launch_bwd<128, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, H, N, scale,
                                           kv_len, workspace, stream);
  }
  return causal ? launch_bwd<64, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, H, N, scale, kv_len,
                                       workspace, stream)
                : launch_bwd<64, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, H, N, scale,
                                        kv_len, workspace, stream);
}

}  // namespace osm
