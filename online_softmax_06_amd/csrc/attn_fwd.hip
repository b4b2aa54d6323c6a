// Fused attention forward on gfx950: S = scale * Q K^T, optional causal mask,
// online softmax, O = P V, and the per-row log-sum-exp, with S and P living
// only in registers.
//
// Method ("Ch.6 Softmax and Online Softmax" §6.5-§6.6; xxqk §4.1): a workgroup
// owns a tile of 128 or 256 query rows and streams the key/value tiles of its
// (batch, head) through LDS (grids too small to fill the GPU: 32 rows, the
// keys split over the four wavefronts and their partial states combined).  Per tile it forms the scores on the matrix
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
// Exponent reference.  In exact arithmetic the result does not depend on the
// reference m used in P = 2^(S' - m): the combine of §6.4.1 holds for any
// finite one, and the pages' recurrence (m = the running max) is one choice.
// Here no sub-tile computes a max as a rule: P is formed against the current
// reference (the row max of the item's first unmasked sub-tile) and summed,
// and only when a lane's partial sum leaves [0, 2^64] (a score far above the
// reference) or a row has no finite reference yet does the wavefront take
// the max, raise the reference (only when the max exceeds it by more than
// kLag, in log2 units), rescale O and l and form P again.  P <= 2^64 keeps
// every float32 sum and product in range and bfloat16 P loses no precision;
// the rescale is rare, and masked sub-tiles differ only by hiding keys
// (-inf) before their exponentials.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "osm_device.h"
#include "osm_internal.h"

// Work queues of the persistent forward launches: per launch slot, one claim
// counter per XCD partition (8) and one exit counter per partition (8).
// Launches take slots in turn; the last workgroup of a partition to leave
// resets both of its counters, so every launch finds its slot at zero.
constexpr int kQueueSlots = 64;
static __device__ unsigned fwd_queue[kQueueSlots * 16];

namespace osm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kBN = 64;      // keys per tile
constexpr float kLag = 8.0f;  // allowed lag of the exponent reference (log2 units)

// Workgroup shape: kW wavefronts of 32 query rows each.  With kW = 4 two
// workgroups share a CU; with kW = 8 (D = 128 only: a K sub-tile must give
// every wavefront a copy instruction) one workgroup fills it, two
// wavefronts per SIMD.  Both have two wavefronts per SIMD, but with two
// workgroups the one dispatched second runs about a fifth slower on the same
// work and sets the end of a persistent launch; with one workgroup the two
// wavefronts of a SIMD advance together and every K/V tile in LDS serves
// twice the rows.  Its 256-row query tiles cost more on the causal diagonal,
// where a wavefront idles over the sub-tiles above its rows, so the launch
// takes kW = 8 for long or unmasked rows (when its tiles fill the compute
// units) and kW = 4 for short causal rows and small grids.
template <int D, int kW>
struct Shape {
  static_assert(kW == 4 || (kW == 8 && D == 128), "supported shapes");
  static constexpr int kWaves = kW;
  static constexpr int kThreads = kW * 64;
  static constexpr int kBM = kW * 32;          // query rows per workgroup
  static constexpr int kPerCU = kW == 8 ? 1 : 2;  // resident workgroups per CU
};

// Resident workgroups per CU that a kernel is compiled for (it bounds the
// registers): three at D = 64 without a bias or splits, where the kernel
// fits in 168 VGPRs and a third wavefront per SIMD overlaps more vector work
// with the products (8-14% faster than two); Shape::kPerCU otherwise.
template <int D, int kW, bool kBias, bool kSplit>
constexpr int per_cu() {
  return (D == 64 && kW == 4 && !kBias && !kSplit) ? 3 : Shape<D, kW>::kPerCU;
}

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

// Global->LDS copy of kRows key rows [k0, k0 + kRows) of K or V into `buf`
// (row-major, 16-byte units XOR-swizzled by `Swz`), one instruction at a
// time: instruction i of wave w fills LDS units [(w * kPerWave + i) * 64,
// +64), one 16-byte unit per lane at a loop-invariant per-lane offset.  The
// buffer descriptor (one per item) spans the head, so rows at or past the end
// of the head fall outside its range and arrive as zeros; k0 = N turns an
// instruction into a zero fill without memory traffic.  The row offset goes
// into the lane offset (one vector add) rather than into a new descriptor
// per copy, which took a dozen scalar instructions per copy.
template <int D, int kRows, int kW>
struct RowCopy {
  static constexpr int kUnits = D / 8;
  static constexpr int kPerWave = kRows * kUnits / 64 / kW;
  static_assert(kPerWave >= 1, "every wave issues at least one load");
  template <int (*Swz)(int)>
  __device__ static int lane_offset(int wave, int lane, int i) {
    const int p = (wave * kPerWave + i) * 64 + lane;  // physical unit in the block
    const int row = p / kUnits, pu = p % kUnits;
    return row * (D * 2) + ((pu ^ Swz(row)) << 4);
  }
  template <typename Rsrc>
  __device__ static void issue(char* buf, Rsrc head, int k0, int wave, int i, int voff) {
    // The buffer-to-LDS builtins exist only for the device; the host pass of
    // this single-source file sees an empty body.
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(head, OSM_LDS(buf + (wave * kPerWave + i) * 1024), 16,
                                             voff + k0 * (D * 2), 0, 0, 0);
#endif
  }
};

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

// Per-lane LDS byte offsets, computed once per workgroup.
// K: lane reads row `col` of a 32-row slot, 16-byte unit (2c + half) ^
// swz(col); since the swizzle keeps bit 0 of the unit apart from c's bits,
// the offset for slice c is k ^ (c << 5).
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

// A3 for one 32-key sub-tile: S^T (32 keys x 32 queries) = K Q^T from the
// 32-row K slot `kslot` (kDC products; K operands read two slices ahead).
template <int D>
__device__ __forceinline__ f32x16 sub_scores(const char* kslot, const LaneOffsets<D>& off,
                                             const bf16x8 (&qreg)[D / 16]) {
  constexpr int kDC = D / 16;
  f32x16 s = f32x16{};
  bf16x8 ka[3];
  ka[0] = *reinterpret_cast<const bf16x8*>(kslot + off.k);
  ka[1] = *reinterpret_cast<const bf16x8*>(kslot + (off.k ^ (1 << 5)));
#pragma unroll
  for (int c = 0; c < kDC; ++c) {
    if (c + 2 < kDC) ka[(c + 2) % 3] = *reinterpret_cast<const bf16x8*>(kslot + (off.k ^ ((c + 2) << 5)));
    s = mfma32(ka[c % 3], qreg[c], s);
  }
  return s;
}

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

// Add the bias of this lane's query row to its 16 raw scores of the sub-tile
// starting at key k0.  Score i is key k0 + (i / 4) * 8 + half * 4 + i % 4.
__device__ __forceinline__ void add_bias(f32x16& s, const float* brow, int k0, int half, int N,
                                         const AttnOptions& opt) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int key = k0 + g * 8 + half * 4;  // 4 consecutive keys
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
    for (int t = 0; t < 4; ++t) s[g * 4 + t] += b4[t] * opt.inv_scale;
  }
}

// Per-wavefront state of the key loop.
template <int D>
struct WaveState {
  bf16x8 qreg[D / 16];   // this lane's part of Q: B operand of S^T = K Q^T
  f32x16 oacc[D / 32];   // O^T accumulators (32 dims x 32 queries each)
  f32x16 sc;             // scores of the current 32-key sub-tile
  float m_run;           // exponent reference, in units of log2(e) * scale * S
  float l_run;           // this lane's half of the running sum
};

// One 32-key sub-tile s (keys [32 s, 32 s + 32), the half kKb of its 64-key
// tile) for one wavefront, in two phases.
//   Phase 1: the vector unit exponentiates the current scores (on masked
//            sub-tiles, kMask, after hiding keys) and sums them, while the
//            scores of sub-tile s + 1 (with kNext) are formed on the matrix
//            core from `kslot_next` (neither depends on the other, so both
//            units work side by side).  Rarely, O and the sums are then
//            rescaled to a new exponent reference.
//   Phase 2: O^T += V^T P^T on the two 16-key slices of this sub-tile, fed
//            by transposed V reads from `vtile`, while the vector unit packs
//            P to bfloat16.
// Each phase is a sequence of short regions (one or two products, the LDS
// reads they need two regions later, a share of the vector work) fenced by
// sched_barrier, so the compiler keeps this interleaving.  `copy(i)` issues
// this wave's i-th global->LDS copy instruction of the sub-step (if any).
template <int D, bool kCausal, int kKb, bool kNext, bool kMask, bool kBias, typename Copy>
__device__ __forceinline__ void sub_step(WaveState<D>& st, const char* kslot_next,
                                         const char* vtile, const LaneOffsets<D>& off, int s,
                                         int N, int kvlen, int qrow, int half, float scale_log2,
                                         const float* brow, const AttnOptions& opt,
                                         const Copy& copy) {
  constexpr int kDC = D / 16;   // 16-wide slices of the head dimension
  constexpr int kDB = D / 32;   // 32-dim blocks of O^T
  constexpr int kPV = 2 * kDB;  // products of phase 2
  constexpr int kRow = D * 2;   // bytes per key row
  const int k0 = s * 32;
  f32x16& sc = st.sc;

  if constexpr (kBias) {
    if (qrow < N) add_bias(sc, brow, k0, half, N, opt);
  }

  // Phase 1.
  bf16x8 ka[3];
  auto read_k = [&](int c) {
    ka[c % 3] = *reinterpret_cast<const bf16x8*>(kslot_next + (off.k ^ (c << 5)));
  };
  // V operands of phase 2, two products ahead; product i is (kc2, b) =
  // (i / kDB, i % kDB), key slice kc = 2 kKb + kc2 of the 64-key tile.
  bf16x8 va[3];
  auto read_v = [&](int i) {
    const int kc = 2 * kKb + i / kDB, b = i % kDB;
    const char* p0 = vtile + off.v[b] + kc * 16 * kRow;
    // Transposed V reads: lane (group g = lane / 16, r = lane % 16) supplies
    // the address of dims [d0 + 4 (r % 4), +4) of key row base + r / 4; it
    // receives dims d0 + r of keys base .. base + 3 (d0 = 32 b + 16 (g % 2)).
    const s16x4 v0 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p0 + 8 * kRow));
    va[i % 3] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  f32x16 sn = f32x16{};
  if constexpr (kNext) {
    read_k(0);
    read_k(1);
  }
  float p[16];
  float alpha = 1.0f;
  float ps0 = 0.0f, ps1 = 0.0f;  // this lane's half of the sub-tile's row sum
  {
    // No row max: P is formed against the current reference right away and
    // summed; the reference moves only when a lane's partial sum leaves
    // [0, 2^64] (a score far above the reference: too large for the sums, or
    // +inf) or a row has no finite reference yet (its first visible keys).
    // Any finite reference gives the same result in exact arithmetic, and
    // P <= 2^64 keeps every sum and product in range.
    const float ref = finite_ref(st.m_run);
    // A4 (masked sub-tiles, the last key tiles): score i is key k0 + (i / 4)
    // * 8 + half * 4 + i % 4, hidden (-inf, so P = 0) unless (i / 4) * 8 +
    // i % 4 is below lim; each region hides its scores before their
    // exponentials.
    const int lim = kMask ? (kCausal ? min(kvlen, qrow + 1) : kvlen) - k0 - half * 4 : 0;
    constexpr int kPer = 16 / kDC;  // exponentials per region
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      if constexpr (kNext) {
        if (c + 2 < kDC) read_k(c + 2);
        sn = mfma32(ka[c % 3], st.qreg[c], sn);
      }
      if (c > 0) copy(c - 1);
#pragma unroll
      for (int t = 0; t < kPer; ++t) {
        const int i = c * kPer + t;
        if constexpr (kMask) sc[i] = (i >> 2) * 8 + (i & 3) < lim ? sc[i] : kNegInf;
        p[i] = exp2_hw(__builtin_fmaf(sc[i], scale_log2, -ref));
        // The sums start as p0 + p2 and p1 + p3: no add of 0 and no copy.
        if (i == 2) ps0 = p[0] + p[2];
        if (i == 3) ps1 = p[1] + p[3];
        if (i >= 4) {
          if (t & 1) ps1 += p[i]; else ps0 += p[i];
        }
      }
      // Keep this region's exponentials and sums in the region (once both
      // sums exist).
      if (c * kPer + kPer > 3) asm volatile("" : "+v"(ps0), "+v"(ps1));
      if (c == kDC - 1) {
        read_v(0);
        read_v(1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::"v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]),
                 "v"(p[6]), "v"(p[7]), "v"(p[8]), "v"(p[9]), "v"(p[10]), "v"(p[11]),
                 "v"(p[12]), "v"(p[13]), "v"(p[14]), "v"(p[15]));
    // One ballot per condition: each compare then feeds the branch directly.
    const float ps = ps0 + ps1;
    if ((__builtin_amdgcn_ballot_w64(!(ps <= 0x1p64f)) |
         __builtin_amdgcn_ballot_w64(st.m_run == kNegInf)) != 0) {
      // Rare: the row max, a new reference (raised only past kLag), the
      // rescale of O and l, and P again.
      asm volatile("");
      float mx = max3(sc[0], sc[1], sc[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mx = max3(mx, sc[i], sc[i + 1]);
      mx = __builtin_fmaxf(mx, sc[15]);
      mx = __builtin_fmaxf(mx, swap_halves(mx));
      const float mt = mx * scale_log2;
      const float m_new = mt > st.m_run + kLag ? mt : st.m_run;
      const float ref2 = finite_ref(m_new);
      alpha = exp2_hw(st.m_run - ref2);
      st.m_run = m_new;
      ps0 = 0.0f;
      ps1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = exp2_hw(__builtin_fmaf(sc[i], scale_log2, -ref2));
        if (i & 1) ps1 += p[i]; else ps0 += p[i];
      }
#pragma unroll
      for (int b = 0; b < kDB; ++b) st.oacc[b] *= alpha;
    }
  }

  // Phase 2 (A6): O^T += V^T P^T.
  // P in the B-operand layout: slice kc2 holds scores kc2 * 8 + 0..7, i.e.
  // keys 16 kc2 + {0..3, 8..11} + 4 half, the order the V reads follow.
  bf16x8 pb[2];
  auto pack_p = [&](int kc2) {
    const int o = kc2 * 8;
    pb[kc2] = __builtin_bit_cast(
        bf16x8, make_uint4(pack_bf16x2(p[o + 0], p[o + 1]), pack_bf16x2(p[o + 2], p[o + 3]),
                           pack_bf16x2(p[o + 4], p[o + 5]), pack_bf16x2(p[o + 6], p[o + 7])));
  };
  pack_p(0);
#pragma unroll
  for (int i = 0; i < kPV; ++i) {
    const int kc2 = i / kDB, b = i % kDB;
    if (i + 2 < kPV) read_v(i + 2);
    if (i == 0) pack_p(1);
    st.oacc[b] = mfma32(va[i % 3], pb[kc2], st.oacc[b]);
    __builtin_amdgcn_sched_barrier(0);
  }
  st.l_run = st.l_run * alpha + (ps0 + ps1);
  if constexpr (kNext) st.sc = sn;
}

// Which (head, query tile) items a workgroup processes.
//   kOnePerGroup: item = the workgroup's own id, mapped by tile_of /
//                 tile_of_split (split-K launches, and grids with no more
//                 query tiles than resident workgroups).
//   kPairsXcd:    a persistent grid, `workers` workgroups per XCD.  Items are
//                 folded in pairs (query tiles p and nqt - 1 - p of one head,
//                 so with a causal mask every pair holds the same number of
//                 key tiles) and the pairs of the heads an XCD owns (bh = x
//                 mod 8) are dealt round-robin to its workgroups: every
//                 workgroup gets the same work, one head's pairs run side by
//                 side on one XCD (its L2 holds that head's K and V), and no
//                 workgroup waits to be dispatched behind a longer one.
//   kPairsAll:    the same over all heads and the whole grid (B * H not a
//                 multiple of 8).
//   kQueue:       a persistent grid whose workgroups claim items one at a
//                 time from an atomic counter of their partition (the heads
//                 bh = x mod 8 for workgroups x mod 8, or all heads), in the
//                 order of queue_item.  With two or three workgroups per CU
//                 the first dispatched one gets the larger share of the
//                 SIMDs; with a fixed share of items each, the other then
//                 finished its last items alone, one wavefront per SIMD, for
//                 about a fifth of the launch.  Claiming lets the faster one
//                 take more items.  Used for 4-wavefront launches without a
//                 bias, except those captured into a graph; with one
//                 8-wavefront workgroup per CU kPairsXcd keeps fewer heads in
//                 flight per L2 and is faster, and so it is with a bias (whose
//                 score tiles the pairs also share).
enum : int { kOnePerGroup = 0, kPairsXcd = 1, kPairsAll = 2, kQueue = 3 };

struct Schedule {
  int mode;
  int nqt;            // query tiles per head
  int pairs;          // pairs per head: ceil(nqt / 2)
  int heads_per_xcd;  // kPairsXcd: B * H / 8
  int workers;        // kPairsXcd: workgroups per XCD; kPairsAll: grid size;
                      // kQueue: workgroups per partition
  int parts;          // kQueue: partitions (8 when B * H is a multiple of 8, else 1)
  int heads;          // kQueue: heads per partition
  int group;          // kQueue: heads visited together
  int total;          // kQueue: items per partition
};

// kQueue: item `idx` of partition `part`.  The heads of a partition (bh =
// part mod parts) are visited in groups of `group`; inside a group the
// query tiles go rank-major (every head's heaviest tile, then every head's
// next, ...), so a group's heads share the L2 and the lightest tiles come
// last, where they even out the end of the launch.
__device__ __forceinline__ void queue_item(const Schedule& sc, int idx, int part, bool causal,
                                           int& bh, int& qt) {
  const int per_group = sc.group * sc.nqt;
  const int grp = idx / per_group, in = idx - grp * per_group;
  const int gh = min(sc.group, sc.heads - grp * sc.group);
  const int r = in / gh, h = in - r * gh;
  bh = (grp * sc.group + h) * sc.parts + part;
  qt = causal ? sc.nqt - 1 - r : r;
}

// Item k of workgroup g: returns 1 and sets (bh, qt, split), 0 when the
// workgroup has no item k (nor any later one), -1 for an empty slot (the
// second half of the middle pair when nqt is odd).
__device__ __forceinline__ int item_of(const Schedule& sc, int g, int k, int BH, int splits,
                                       bool causal, int& bh, int& qt, int& split) {
  split = 0;
  if (sc.mode == kOnePerGroup) {
    if (k > 0) return 0;
    if (splits > 1) {
      tile_of_split(g, sc.nqt, splits, BH, causal, bh, qt, split);
    } else {
      tile_of(g, sc.nqt, BH, causal, bh, qt);
    }
    return 1;
  }
  int pi, p;
  if (sc.mode == kPairsXcd) {
    const int xcd = g & 7, w = g >> 3;
    pi = w + (k >> 1) * sc.workers;
    if (pi >= sc.heads_per_xcd * sc.pairs) return 0;
    bh = (pi / sc.pairs) * 8 + xcd;
    p = pi % sc.pairs;
  } else {
    pi = g + (k >> 1) * sc.workers;
    if (pi >= BH * sc.pairs) return 0;
    bh = pi / sc.pairs;
    p = pi % sc.pairs;
  }
  const int heavy = sc.nqt - 1 - p;  // the query tile with more key tiles first
  if (k & 1) {
    if (p == heavy) return -1;
    qt = p;
  } else {
    qt = heavy;
  }
  return 1;
}

// With kSplit, item (head, query tile, split) covers only its share of the
// key tiles and writes a partial result normalised by its own l -- O_s in
// float32 and LSE_s -- to o_part / lse_part; attn_split_merge_kernel combines
// the splits.
template <int D, int kW, bool kCausal, bool kBias, bool kSplit>
__global__ __launch_bounds__((Shape<D, kW>::kThreads),
                             (per_cu<D, kW, kBias, kSplit>())) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int BH,
    int H, int N, float scale_log2, AttnOptions opt, Schedule sched, int splits,
    float* __restrict__ o_part, float* __restrict__ lse_part, unsigned* __restrict__ queue) {
  using T = Tile<D>;
  constexpr int kDC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kSlot = 32 * D * 2;  // one 32-row K slot
  // K streams through four 32-row slots (sub-tile t in slot t & 3); V through
  // two 64-row buffers (tile j in buffer j & 1).  Each is its own array, and
  // every copy into LDS names its target at compile time: the compiler then
  // knows that a copy in flight does not alias the slots being read, and
  // waits for it only at the barrier.
  __shared__ __attribute__((aligned(1024))) char ks0[kSlot];
  __shared__ __attribute__((aligned(1024))) char ks1[kSlot];
  __shared__ __attribute__((aligned(1024))) char ks2[kSlot];
  __shared__ __attribute__((aligned(1024))) char ks3[kSlot];
  __shared__ __attribute__((aligned(1024))) char vb0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char vb1[T::kBytes];
  // Q staging (D = 128, 4 wavefronts, no splits): every wave's 32 query
  // rows pass through LDS; waves 0-2 use the V buffer and the K slot that
  // the prologue leaves free, wave 3 this array.  (With 8 wavefronts, at
  // D = 64 and in the split kernels, measured level or slower, or spilling.)
  constexpr bool kQLds = D == 128 && kW == 4 && !kSplit;
  constexpr int kQStage = 32 * D * 2;
  __shared__ __attribute__((aligned(256))) char qx[kQLds ? kQStage : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;   // the query row this lane works on (within the wave)
  const int half = lane >> 5;  // which 8-element half of each 16-wide slice
  const int head_bytes = N * D * 2;
  const LaneOffsets<D> off = lane_offsets<D>(lane);
  using KCopy = RowCopy<D, 32, kW>;
  using VCopy = RowCopy<D, 64, kW>;
  static_assert(2 * KCopy::kPerWave <= kDC - 1 && VCopy::kPerWave <= kDC - 1,
                "a sub-step has a phase-1 region for each of its copies");
  int koff[KCopy::kPerWave], voff[VCopy::kPerWave];
#pragma unroll
  for (int i = 0; i < KCopy::kPerWave; ++i)
    koff[i] = KCopy::template lane_offset<T::k_swz>(wave, lane, i);
#pragma unroll
  for (int i = 0; i < VCopy::kPerWave; ++i)
    voff[i] = VCopy::template lane_offset<T::v_swz>(wave, lane, i);
  WaveState<D> st;

  // kQueue (4-wavefront launches without bias or splits): thread 0 claims
  // the items and hands each index to the workgroup through LDS (two slots,
  // one per item parity).
  constexpr bool kMayQueue = kW == 4 && !kBias && !kSplit;
  const bool queued = kMayQueue && sched.mode == kQueue;
  __shared__ int s_item[2];
  const int part = (queued && sched.parts == 8) ? (blockIdx.x & 7) : 0;
  int qidx = 0;
  if (queued) {
    if (tid == 0) s_item[0] = (int)atomicAdd(queue + part, 1u);
    __syncthreads();
    qidx = __builtin_amdgcn_readfirstlane(s_item[0]);
  }

  for (int item = 0;; ++item) {
    int bh, qt, split = 0;
    unsigned next = 0;
    // kQueue: the next item is claimed at the first of the last tiles, late
    // enough that the claims follow the order in which workgroups become
    // free, early enough that the atomic's round trip hides behind a tile.
    bool claim = false;
    if (queued) {
      if (qidx >= sched.total) break;
      queue_item(sched, qidx, part, kCausal, bh, qt);
      claim = true;
    } else {
      const int have = item_of(sched, blockIdx.x, item, BH, splits, kCausal, bh, qt, split);
      if (have == 0) break;
      if (have < 0) continue;
      // Every wave is done with the LDS slots of the previous item.
      if (item > 0) __syncthreads();
    }

    const int64_t head_off = (int64_t)bh * N * D;
    const uint16_t* kh = k + head_off;
    const uint16_t* vh = v + head_off;
    const int q0 = qt * Shape<D, kW>::kBM;
    const int qw = q0 + wave * 32;  // first query row of this wave
    const int qrow = qw + col;      // this lane's query row
    const int b = bh / H, h = bh % H;
    const int kvlen = opt.kv_len ? min(max(opt.kv_len[b], 0), N) : N;
    const float* brow = kBias ? opt.bias + b * opt.bias_stride_b + h * opt.bias_stride_h +
                                    (int64_t)min(qrow, N - 1) * N
                              : nullptr;

    const int kv_end = kCausal ? min(kvlen, q0 + Shape<D, kW>::kBM) : kvlen;
    const int ntiles_all = (kv_end + kBN - 1) / kBN;
    // Key tiles [j_begin, j_end) of this item (all of them without splits).
    int j_begin = 0, j_end = ntiles_all;
    if constexpr (kSplit) {
      const int per = (ntiles_all + splits - 1) / splits;
      j_begin = min(split * per, ntiles_all);
      j_end = min(j_begin + per, ntiles_all);
    }
    // Last 32-key sub-tile with a visible key for this wave (below 2 j_begin:
    // none).  Causal: the diagonal sub-tile, 32-aligned like the wave's rows.
    int sw_last = min(2 * j_end, (kvlen + 31) / 32) - 1;
    if constexpr (kCausal) sw_last = min(sw_last, qw / 32);
    if (qw >= N || j_end <= j_begin) sw_last = -1;
    const int s_end = 2 * j_end;
    const int s0 = 2 * j_begin;

    // Copies of 32-row K sub-tiles and 64-row V tiles; a sub-tile or tile
    // outside this item's range becomes a zero fill (k0 = N).
#if defined(__HIP_DEVICE_COMPILE__)
    const auto krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kh, 0, head_bytes, kBufferFlags);
    const auto vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vh, 0, head_bytes, kBufferFlags);
#else
    const int krsrc = 0, vrsrc = 0;
#endif
    auto copy_k = [&](char* slot, int t, int i) {
      KCopy::issue(slot, krsrc, t < s_end ? t * 32 : N, wave, i, koff[i]);
    };
    auto copy_v = [&](char* buf, int jj, int i) {
      VCopy::issue(buf, vrsrc, jj < j_end ? jj * kBN : N, wave, i, voff[i]);
    };

    // A2 prologue: the first three K sub-tiles and the first V tile in flight.
#pragma unroll
    for (int i = 0; i < KCopy::kPerWave; ++i) {
      if ((j_begin & 1) == 0) {
        copy_k(ks0, s0, i);
        copy_k(ks1, s0 + 1, i);
        copy_k(ks2, s0 + 2, i);
      } else {
        copy_k(ks2, s0, i);
        copy_k(ks3, s0 + 1, i);
        copy_k(ks0, s0 + 2, i);
      }
    }
#pragma unroll
    for (int i = 0; i < VCopy::kPerWave; ++i) {
      if ((j_begin & 1) == 0) copy_v(vb0, j_begin, i); else copy_v(vb1, j_begin, i);
    }

    // A1: this lane's part of Q as the B operand of S^T = K Q^T.  Loaded
    // directly, each instruction touches 32 rows in 32-byte pieces; with
    // kQLds the wave copies its rows into LDS like a K sub-tile (whole
    // 128-byte lines per instruction, the K swizzle) and reads them back in
    // the operand layout after the barrier.  Rows past N arrive as zeros.
    char* qst = qx;
    if constexpr (kQLds) {
      if (wave < 2) qst = ((j_begin & 1) ? vb0 : vb1) + wave * kQStage;
      else if (wave == 2) qst = (j_begin & 1) ? ks1 : ks3;
#if defined(__HIP_DEVICE_COMPILE__)
      const auto qrsrc =
          __builtin_amdgcn_make_buffer_rsrc((void*)(q + head_off), 0, head_bytes, kBufferFlags);
#pragma unroll
      for (int i = 0; i < 32 * T::kUnits / 64; ++i) {
        const int row = (i * 64 + lane) / T::kUnits, pu = (i * 64 + lane) % T::kUnits;
        const int vo = (qw + row) * (D * 2) + ((pu ^ T::k_swz(row)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, OSM_LDS(qst + i * 1024), 16, vo, 0, 0, 0);
      }
#endif
    } else {
      const uint16_t* qg = q + head_off + (int64_t)qrow * D + half * 8;
#pragma unroll
      for (int c = 0; c < kDC; ++c) {
        st.qreg[c] = qrow < N ? *reinterpret_cast<const bf16x8*>(qg + c * 16) : bf16x8{};
      }
    }
#pragma unroll
    for (int i = 0; i < kDB; ++i) st.oacc[i] = f32x16{};
    st.m_run = kNegInf;
    st.l_run = 0.0f;
    st.sc = f32x16{};

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (kQLds) {
      // The staging slots are next written by the copies of the first tile,
      // issued after its barrier, which every wave reaches only once these
      // reads have completed.
#pragma unroll
      for (int c = 0; c < kDC; ++c) {
        st.qreg[c] = *reinterpret_cast<const bf16x8*>(qst + (off.k ^ (c << 5)));
      }
    }
    if (sw_last >= s0) st.sc = sub_scores<D>((j_begin & 1) ? ks2 : ks0, off, st.qreg);

    int full_end = min(j_end, kvlen / kBN);
    // Causal: tiles below this wave's first row are unmasked for it (other
    // waves of the workgroup may mask them).
    if constexpr (kCausal) full_end = min(full_end, qw / kBN);
    if (sw_last < 0) full_end = j_begin;
    const int main_end = max(j_begin, min(full_end, j_end - 1));
    if constexpr (!kBias) {
      // When the item starts with an unmasked tile, its first sub-tile's row
      // max becomes the exponent reference: the first sub-step then forms P
      // once, instead of taking the re-reference branch that a reference of
      // -inf forces (a second round of exponentials and a rescale of the
      // empty accumulator).  With a bias the scores are complete only inside
      // the sub-step, which keeps the branch.
      if (main_end > j_begin) {
        const f32x16& sc = st.sc;
        float mx = max3(sc[0], sc[1], sc[2]);
#pragma unroll
        for (int i = 3; i < 15; i += 2) mx = max3(mx, sc[i], sc[i + 1]);
        mx = __builtin_fmaxf(mx, sc[15]);
        mx = __builtin_fmaxf(mx, swap_halves(mx));
        st.m_run = mx * scale_log2;
      }
    }

    // A2: at the top of the step for tile j, K sub-tiles 2j + 1 and 2j + 2
    // and V_j have landed and every wave is done with sub-tiles 2j - 1 and 2j
    // and with V_{j-1}, whose places receive sub-tiles 2j + 3, 2j + 4 (copied
    // during the tile's first sub-step) and V_{j+1} (during its second).  One
    // barrier per 64-key tile.  Tile j even: its sub-tiles read the next
    // scores from slots 1 and 2 and V from buffer 0; j odd: slots 3, 0 and
    // buffer 1.
#define OSM_TILE_COPIES(J, ODD)                                                               \
  auto cp0 = [&](int i) {                                                                     \
    if (i < KCopy::kPerWave)                                                                  \
      copy_k(ODD ? ks1 : ks3, 2 * (J) + 3, i);                                                \
    else if (i < 2 * KCopy::kPerWave)                                                         \
      copy_k(ODD ? ks2 : ks0, 2 * (J) + 4, i - KCopy::kPerWave);                              \
  };                                                                                          \
  auto cp1 = [&](int i) {                                                                     \
    if (i < VCopy::kPerWave) copy_v(ODD ? vb0 : vb1, (J) + 1, i);                             \
  }
    // Main part: tiles this wave does not mask (keys below its first query
    // row when causal, whole tiles below the key length) and whose sub-tiles
    // are all followed by another: one code path.  The waves of a workgroup
    // may run different numbers of main tiles; every tile, main or not, has
    // its one barrier.
#define OSM_MAIN_TILE(J, ODD)                                                                 \
  do {                                                                                        \
    __builtin_amdgcn_s_waitcnt(0);                                                            \
    __syncthreads();                                                                          \
    OSM_TILE_COPIES(J, ODD);                                                                  \
    sub_step<D, kCausal, 0, true, false, kBias>(st, ODD ? ks3 : ks1, ODD ? vb1 : vb0, off,    \
                                                2 * (J), N, kvlen, qrow, half, scale_log2,    \
                                                brow, opt, cp0);                              \
    sub_step<D, kCausal, 1, true, false, kBias>(st, ODD ? ks0 : ks2, ODD ? vb1 : vb0, off,    \
                                                2 * (J) + 1, N, kvlen, qrow, half,            \
                                                scale_log2, brow, opt, cp1);                  \
  } while (0)
    // The last tiles (those crossing the diagonal or the key length, and the
    // final one): always masked, and per wave in three wave-uniform runs --
    // tiles whose two sub-tiles the wave computes (up to its last visible
    // sub-tile sw_last), at most one tile whose first sub-tile only it
    // computes, then tiles where it only issues its share of the copies.
    // Every tile still has its one barrier for every wave.  With a branch per
    // sub-tile instead, the compiler gave the two paths different register
    // assignments and copied 64-80 VGPRs at every join.  A masked sub-step
    // always forms the next scores, also on the wave's last sub-tile, where
    // they are not used: one code path for every computed sub-tile.
#define OSM_TAIL_FULL(J, ODD)                                                                 \
  do {                                                                                        \
    __builtin_amdgcn_s_waitcnt(0);                                                            \
    __syncthreads();                                                                          \
    if (claim) {                                                                              \
      claim = false;                                                                          \
      if (tid == 0) next = atomicAdd(queue + part, 1u);                                       \
    }                                                                                         \
    OSM_TILE_COPIES(J, ODD);                                                                  \
    sub_step<D, kCausal, 0, true, true, kBias>(st, ODD ? ks3 : ks1, ODD ? vb1 : vb0, off,     \
                                               2 * (J), N, kvlen, qrow, half, scale_log2,     \
                                               brow, opt, cp0);                               \
    sub_step<D, kCausal, 1, true, true, kBias>(st, ODD ? ks0 : ks2, ODD ? vb1 : vb0, off,     \
                                               2 * (J) + 1, N, kvlen, qrow, half,             \
                                               scale_log2, brow, opt, cp1);                   \
  } while (0)
#define OSM_TAIL_HALF(J, ODD)                                                                 \
  do {                                                                                        \
    __builtin_amdgcn_s_waitcnt(0);                                                            \
    __syncthreads();                                                                          \
    if (claim) {                                                                              \
      claim = false;                                                                          \
      if (tid == 0) next = atomicAdd(queue + part, 1u);                                       \
    }                                                                                         \
    OSM_TILE_COPIES(J, ODD);                                                                  \
    sub_step<D, kCausal, 0, true, true, kBias>(st, ODD ? ks3 : ks1, ODD ? vb1 : vb0, off,     \
                                               2 * (J), N, kvlen, qrow, half, scale_log2,     \
                                               brow, opt, cp0);                               \
    _Pragma("unroll") for (int i = 0; i < kDC - 1; ++i) cp1(i);                               \
  } while (0)
#define OSM_TAIL_EMPTY(J, ODD)                                                                \
  do {                                                                                        \
    __builtin_amdgcn_s_waitcnt(0);                                                            \
    __syncthreads();                                                                          \
    if (claim) {                                                                              \
      claim = false;                                                                          \
      if (tid == 0) next = atomicAdd(queue + part, 1u);                                       \
    }                                                                                         \
    OSM_TILE_COPIES(J, ODD);                                                                  \
    _Pragma("unroll") for (int i = 0; i < kDC - 1; ++i) {                                     \
      cp0(i);                                                                                 \
      cp1(i);                                                                                 \
    }                                                                                         \
  } while (0)

    int j = j_begin;
    if ((j & 1) && j < main_end) {
      OSM_MAIN_TILE(j, true);
      ++j;
    }
    for (; j + 1 < main_end; j += 2) {
      OSM_MAIN_TILE(j, false);
      OSM_MAIN_TILE(j + 1, true);
    }
    if (j < main_end) {
      OSM_MAIN_TILE(j, false);
      ++j;
    }
    // Tail tiles j with 2j + 1 <= sw_last: both sub-tiles computed.
    int tail_full = min(j_end, (sw_last + 1) / 2);
    tail_full = max(tail_full, j);
    if ((j & 1) && j < tail_full) {
      OSM_TAIL_FULL(j, true);
      ++j;
    }
    for (; j + 1 < tail_full; j += 2) {
      OSM_TAIL_FULL(j, false);
      OSM_TAIL_FULL(j + 1, true);
    }
    if (j < tail_full) {
      OSM_TAIL_FULL(j, false);
      ++j;
    }
    // The tile holding sw_last as its first sub-tile.
    if (j < j_end && 2 * j == sw_last) {
      if (j & 1) {
        OSM_TAIL_HALF(j, true);
      } else {
        OSM_TAIL_HALF(j, false);
      }
      ++j;
    }
    // Tiles past the wave's last visible sub-tile: copies only.
    if ((j & 1) && j < j_end) {
      OSM_TAIL_EMPTY(j, true);
      ++j;
    }
    for (; j + 1 < j_end; j += 2) {
      OSM_TAIL_EMPTY(j, false);
      OSM_TAIL_EMPTY(j + 1, true);
    }
    if (j < j_end) {
      OSM_TAIL_EMPTY(j, false);
      ++j;
    }
#undef OSM_TAIL_EMPTY
#undef OSM_TAIL_HALF
#undef OSM_TAIL_FULL
#undef OSM_MAIN_TILE
#undef OSM_TILE_COPIES
    // The last tile's copies (zero fills of slots past the item) land before
    // this wave reaches the next item's barrier, after which other waves
    // copy the next item's tiles into the same slots: an early copy can then
    // not overwrite a later one.  They carry no memory traffic, so this wait
    // is short.
    __builtin_amdgcn_s_waitcnt(0);

    // A7: O = O / l (deferred division), LSE = ln 2 * (m + log2 l).  The
    // stores are not waited for: the next item's loads go out behind them.
    const float l_tot = st.l_run + swap_halves(st.l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse_val = l_tot > 0.0f ? (finite_ref(st.m_run) + log2_hw(l_tot)) * kLn2 : kNegInf;
    if (qrow < N) {
      if constexpr (kSplit) {
        const int64_t prow = ((int64_t)split * BH + bh) * N + qrow;
        float* orow = o_part + prow * D;
#pragma unroll
        for (int bb = 0; bb < kDB; ++bb) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const f32x16& oa = st.oacc[bb];
            const float4 w = make_float4(oa[gq * 4 + 0] * inv, oa[gq * 4 + 1] * inv,
                                         oa[gq * 4 + 2] * inv, oa[gq * 4 + 3] * inv);
            *reinterpret_cast<float4*>(orow + bb * 32 + gq * 8 + half * 4) = w;
          }
        }
        if (half == 0) lse_part[prow] = lse_val;
      } else {
        // O^T block bb holds dims bb*32 + 8 (i / 4) + 4 half + i % 4; the
        // stores trade columns with the partner lane first (16 bytes per lane).
        uint16_t* orow = o + head_off + (int64_t)qrow * D;
#pragma unroll
        for (int bb = 0; bb < kDB; ++bb) store_block_bf16(orow + bb * 32, st.oacc[bb], half, inv);
        if (half == 0) lse[(int64_t)bh * N + qrow] = lse_val;
      }
    }
    if (queued) {
      // Hand over the next index; the barrier also tells every wave that the
      // others are done with this item's LDS slots.  An item without key
      // tiles (a batch whose key length is 0) has made no claim yet.
      if (claim && tid == 0) next = atomicAdd(queue + part, 1u);
      if (tid == 0) s_item[(item + 1) & 1] = (int)next;
      __syncthreads();
      qidx = __builtin_amdgcn_readfirstlane(s_item[(item + 1) & 1]);
    }
  }
  if (queued && tid == 0) {
    // Every workgroup of the partition has made its last claim once the exit
    // counter reaches `workers`: the last one resets the slot.
    if (atomicAdd(queue + 8 + part, 1u) == (unsigned)sched.workers - 1) {
      queue[part] = 0u;
      queue[8 + part] = 0u;
    }
  }
}

// Grids too small to fill the GPU (few heads and query tiles): a workgroup
// owns only 32 query rows and its four wavefronts split their key range
// into four consecutive parts.  Every wavefront streams its own part through
// LDS areas of its own (no barrier inside the key loop), each sub-tile
// handled by the masked sub-step (keys past the causal diagonal or the key
// length hidden), and ends with a partial state (reference, sum, O) of the
// same rows.  Wavefronts 1-3 leave theirs in LDS and wavefront 0 folds the
// four in order with the (m, l) combine of §6.4.1 before the epilogue.
// Four times the workgroups of the 128-row kernel, each with a quarter of
// the key loop.
template <int D, bool kCausal>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void attn_fwd_small_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, int BH,
    int H, int N, float scale_log2, AttnOptions opt) {
  using T = Tile<D>;
  using SubCopy = RowCopy<D, 32, 1>;  // one wavefront copies a 32-row sub-tile
  constexpr int kDC = D / 16, kDB = D / 32;
  constexpr int kSub = 32 * D * 2;  // bytes of a 32-row sub-tile
  // Per wavefront: two K and two V sub-tile slots (double buffering).
  __shared__ __attribute__((aligned(1024))) char area[4][4][kSub];
  static_assert(kDB * 16 * 64 * 4 + 2 * 64 * 4 <= 4 * kSub, "partial state fits the area");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // All 32-row groups of a head on one XCD when B * H is a multiple of 8
  // (the L2 of that XCD then fetches the head's K and V once), causal groups
  // heaviest first.
  const int ngroups = (N + 31) / 32;
  int bh, grp;
  tile_of(blockIdx.x, ngroups, BH, kCausal, bh, grp);
  const int q0 = grp * 32;
  const int qrow = q0 + col;
  const int64_t head_off = (int64_t)bh * N * D;
  const int head_bytes = N * D * 2;
  const int kvlen = opt.kv_len ? min(max(opt.kv_len[bh / H], 0), N) : N;
  const LaneOffsets<D> off = lane_offsets<D>(lane);

  // This wavefront's sub-tiles [s_lo, s_hi) of the rows' visible keys.
  const int kv_end = kCausal ? min(kvlen, q0 + 32) : kvlen;
  const int nsub = (kv_end + 31) / 32;
  const int per = (nsub + 3) / 4;
  const int s_lo = min(wave * per, nsub), s_hi = min(s_lo + per, nsub);

  WaveState<D> st;
  {
    const uint16_t* qg = q + head_off + (int64_t)qrow * D + half * 8;
#pragma unroll
    for (int c = 0; c < kDC; ++c)
      st.qreg[c] = qrow < N ? *reinterpret_cast<const bf16x8*>(qg + c * 16) : bf16x8{};
  }
#pragma unroll
  for (int b = 0; b < kDB; ++b) st.oacc[b] = f32x16{};
  st.m_run = kNegInf;
  st.l_run = 0.0f;
  st.sc = f32x16{};

  char* const kslot[2] = {area[wave][0], area[wave][1]};
  char* const vslot[2] = {area[wave][2], area[wave][3]};
#if defined(__HIP_DEVICE_COMPILE__)
  const auto krsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k + head_off), 0, head_bytes, kBufferFlags);
  const auto vrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v + head_off), 0, head_bytes, kBufferFlags);
#else
  const int krsrc = 0, vrsrc = 0;
#endif
  int koff[SubCopy::kPerWave], voff[SubCopy::kPerWave];
#pragma unroll
  for (int i = 0; i < SubCopy::kPerWave; ++i) {
    koff[i] = SubCopy::template lane_offset<T::k_swz>(0, lane, i);
    voff[i] = SubCopy::template lane_offset<T::v_swz>(0, lane, i);
  }
  // Rows past the head fall outside the descriptors and arrive as zeros.
  auto copy_sub = [&](int slot, int s) {
#pragma unroll
    for (int i = 0; i < SubCopy::kPerWave; ++i) {
      SubCopy::issue(kslot[slot], krsrc, s * 32, 0, i, koff[i]);
      SubCopy::issue(vslot[slot], vrsrc, s * 32, 0, i, voff[i]);
    }
  };
  auto no_copy = [](int) {};

  if (s_lo < s_hi) copy_sub(0, s_lo);
  for (int s = s_lo; s < s_hi; ++s) {
    const int slot = (s - s_lo) & 1;
    // This wavefront's copies of sub-tile s have landed in LDS; the other
    // slot was last read by sub-tile s - 1, whose products have consumed it.
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    if (s + 1 < s_hi) copy_sub(slot ^ 1, s + 1);
    st.sc = sub_scores<D>(kslot[slot], off, st.qreg);
    sub_step<D, kCausal, 0, false, true, false>(st, kslot[slot], vslot[slot], off, s, N, kvlen,
                                                qrow, half, scale_log2, nullptr, opt, no_copy);
  }

  // Partial state of this wavefront's part: P was formed against
  // ref = finite_ref(m_run), so the part's sum is l * 2^ref and its output O.
  const float ref = finite_ref(st.m_run);
  const float l_tot = st.l_run + swap_halves(st.l_run);
  __syncthreads();  // every wavefront is done with its key loop
  float* part = reinterpret_cast<float*>(area[wave][0]);
  if (wave > 0) {
#pragma unroll
    for (int b = 0; b < kDB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) part[(b * 16 + i) * 64 + lane] = st.oacc[b][i];
    part[kDB * 16 * 64 + lane] = ref;
    part[kDB * 16 * 64 + 64 + lane] = l_tot;
  }
  __syncthreads();
  if (wave != 0) return;

  // A7 after the combine, parts in order 0..3: M = the largest reference of
  // the parts with keys, weights 2^(ref_w - M) <= 1.
  float refs[4], ls[4];
  refs[0] = ref;
  ls[0] = l_tot;
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const float* pw = reinterpret_cast<const float*>(area[w][0]);
    refs[w] = pw[kDB * 16 * 64 + lane];
    ls[w] = pw[kDB * 16 * 64 + 64 + lane];
  }
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = ls[w] > 0.0f ? fmaxf(M, refs[w]) : M;
  float wgt[4];
  float l_all = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wgt[w] = ls[w] > 0.0f ? exp2_hw(refs[w] - M) : 0.0f;
    l_all += wgt[w] * ls[w];
  }
#pragma unroll
  for (int b = 0; b < kDB; ++b) {
    st.oacc[b] *= wgt[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float* pw = reinterpret_cast<const float*>(area[w][0]);
#pragma unroll
      for (int i = 0; i < 16; ++i) st.oacc[b][i] += wgt[w] * pw[(b * 16 + i) * 64 + lane];
    }
  }
  const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
  if (qrow < N) {
    uint16_t* orow = o + head_off + (int64_t)qrow * D;
#pragma unroll
    for (int b = 0; b < kDB; ++b) store_block_bf16(orow + b * 32, st.oacc[b], half, inv);
    if (half == 0) lse[(int64_t)bh * N + qrow] = l_all > 0.0f ? (M + log2_hw(l_all)) * kLn2 : kNegInf;
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

// Compute units of the current device (cached per device; relaxed atomics,
// since calls from several host threads may fill the same entry).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The queue slot of the next persistent launch on the current device (the
// array's address is looked up once per device).
hipError_t queue_slot(unsigned** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex lock;
  static unsigned* addr[kMaxDevices] = {};
  static unsigned seq[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(lock);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(fwd_queue));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<unsigned*>(p);
  }
  *ptr = addr[dev] + (seq[dev]++ % kQueueSlots) * 16;
  return hipSuccess;
}

// Whether `s` is being captured into a graph.  A captured launch keeps its
// kernel arguments, queue slot included, for every replay, while eager
// launches go on taking the slots in turn: such a launch could meet another
// on the same slot, so captured launches take a fixed schedule instead.
// If the query itself fails, its error is cleared and the stream is taken
// as captured.
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return st != hipStreamCaptureStatusNone;
}

template <int D, int kW, bool kCausal, bool kBias, bool kSplit>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int H,
                  int N, float scale, const AttnOptions& opt, int splits, float* o_part,
                  float* lse_part, hipStream_t s) {
  using Sh = Shape<D, kW>;
  const int nqt = (N + Sh::kBM - 1) / Sh::kBM;
  const float scale_log2 = scale * kLog2e;
  Schedule sc;
  sc.nqt = nqt;
  sc.pairs = (nqt + 1) / 2;
  sc.heads_per_xcd = BH / 8;
  sc.parts = 1;
  sc.heads = 0;
  sc.group = 8;
  sc.total = 0;
  unsigned* queue = nullptr;
  int64_t grid;
  if (kSplit) {
    sc.mode = kOnePerGroup;
    sc.workers = 0;
    grid = (int64_t)nqt * BH * splits;
  } else {
    // Resident workgroups: per_cu() per compute unit.
    const int slots = per_cu<D, kW, kBias, kSplit>() * device_cus();
    const int64_t items = (int64_t)nqt * BH;
    if (items <= slots) {
      // Small grid: every query tile gets a workgroup of its own (heaviest
      // first when causal); folding pairs would run two tiles back to back
      // while compute units stay idle.
      sc.mode = kOnePerGroup;
      sc.workers = 0;
      grid = items;
    } else if (kW == 4 && !kBias && slots >= 8 && !capturing(s)) {
      sc.mode = kQueue;
      sc.parts = (BH & 7) == 0 ? 8 : 1;
      sc.heads = BH / sc.parts;
      sc.total = sc.heads * nqt;
      const int per_part = slots / sc.parts;
      sc.workers = sc.total < per_part ? sc.total : per_part;
      grid = (int64_t)sc.parts * sc.workers;
      const hipError_t e = queue_slot(&queue);
      if (e != hipSuccess) return e;
    } else if ((BH & 7) == 0 && slots >= 8) {
      sc.mode = kPairsXcd;
      const int64_t per_xcd = (int64_t)sc.heads_per_xcd * sc.pairs;
      sc.workers = (int)(per_xcd < slots / 8 ? per_xcd : slots / 8);
      grid = 8 * (int64_t)sc.workers;
    } else {
      sc.mode = kPairsAll;
      const int64_t total = (int64_t)BH * sc.pairs;
      sc.workers = (int)(total < slots ? total : slots);
      grid = sc.workers;
    }
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D, kW, kCausal, kBias, kSplit>), dim3((unsigned)grid),
                     dim3(Sh::kThreads), 0, s, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<uint16_t*>(o), lse, BH, H, N, scale_log2, opt, sc, splits, o_part,
                     lse_part, queue);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !kSplit) return e;
  const int64_t rows = (int64_t)BH * N;
  const int64_t threads = rows * (D / 4);
  hipLaunchKernelGGL((attn_split_merge_kernel<D>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, s, o_part, lse_part, static_cast<uint16_t*>(o), lse, rows,
                     splits);
  return hipGetLastError();
}

template <int D, bool kCausal>
hipError_t launch_small(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                        int H, int N, float scale, const AttnOptions& opt, hipStream_t s) {
  const int64_t grid = (int64_t)BH * ((N + 31) / 32);
  hipLaunchKernelGGL((attn_fwd_small_kernel<D, kCausal>), dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, BH, H, N,
                     scale * kLog2e, opt);
  return hipGetLastError();
}

template <int D, bool kSplit>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                    int H, int N, float scale, bool causal, const AttnOptions& opt, int splits,
                    float* o_part, float* lse_part, hipStream_t s) {
  if constexpr (!kSplit) {
    // Grids whose 128-row query tiles would leave half the compute units
    // idle (so B * H * N <= 16384 * 128): 32-row workgroups with the key
    // range split over their wavefronts, at D = 64 always and at D = 128 up
    // to 1024 keys.  Measured against the 128-row kernel: B1 H8 N1024 D64
    // 30% faster, B1 H1 N16384 D64 causal 34%, B1 H8 N1024 D128 13%; at
    // D = 128 with 2048 keys or more level to 50% slower (each wavefront
    // streams its own K/V, and 128 KiB of LDS leave one wavefront per SIMD).
    const int64_t tiles = (int64_t)BH * ((N + 127) / 128);
    const bool short_rows = D == 64 || N <= 1024;
    if (opt.bias == nullptr && short_rows && 2 * tiles <= device_cus()) {
      return causal ? launch_small<D, true>(q, k, v, o, lse, BH, H, N, scale, opt, s)
                    : launch_small<D, false>(q, k, v, o, lse, BH, H, N, scale, opt, s);
    }
  }
  if (opt.bias != nullptr) {
    return causal ? launch<D, 4, true, true, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt, splits,
                                                     o_part, lse_part, s)
                  : launch<D, 4, false, true, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt,
                                                      splits, o_part, lse_part, s);
  }
  // Eight wavefronts for rows without a causal diagonal or with many key
  // tiles per diagonal (the crossover measured at N = 4096), when their
  // 256-row tiles still give every compute unit one (else the 128-row tiles
  // of four wavefronts spread the work over twice as many workgroups).
  if constexpr (D == 128 && !kSplit) {
    const bool fills = (int64_t)((N + 255) / 256) * BH >= device_cus();
    if (!causal && fills) {
      return launch<D, 8, false, false, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt, splits,
                                                o_part, lse_part, s);
    }
    if (causal && fills && N >= 4096) {
      return launch<D, 8, true, false, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt, splits,
                                               o_part, lse_part, s);
    }
  }
  return causal ? launch<D, 4, true, false, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt, splits,
                                                    o_part, lse_part, s)
                : launch<D, 4, false, false, kSplit>(q, k, v, o, lse, BH, H, N, scale, opt,
                                                     splits, o_part, lse_part, s);
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
