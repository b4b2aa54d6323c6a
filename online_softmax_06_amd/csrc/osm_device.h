// Device-side helpers shared by the row-softmax and attention kernels (gfx950).
//
// The online-softmax state of a lane is a pair (m, l): the largest value seen
// and the sum of exp(x - m) over the values seen ("Ch.6 Softmax and Online
// Softmax", §6.3.1).  The empty state is (-inf, 0).  Two states merge with
//   M = max(m1, m2),  l = l1 * e^(m1 - M) + l2 * e^(m2 - M)            (§6.4.1)
// which is commutative and associative with the empty state as identity, so
// any reduction tree gives the same result up to rounding.
//
// The chapter guards the merge with a branch ("if the new max is -inf, keep the
// state"), because e^(-inf - (-inf)) is NaN.  Here the guard is branch-free:
// the exponent reference is M when M is finite and 0 otherwise, so an empty
// side contributes e^(-inf) = 0 and two empty sides give (-inf, 0) again.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osm {

// Native 16-byte vector (usable with the nontemporal load/store builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// log2(x) on the hardware unit (v_log_f32); log2(0) = -inf.
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Exponent reference for a running maximum: m itself, or 0 while nothing
// finite has been seen.
__device__ __forceinline__ float finite_ref(float m) { return m == kNegInf ? 0.0f : m; }

// Merge (m2, l2) into (m, l), natural-log units (the row kernel works on raw
// inputs).  The subtraction comes before the scaling by log2(e), so that
// values near 1000 keep their small differences exactly.
__device__ __forceinline__ void combine_state(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  const float r = finite_ref(M);
  l = l * exp2_hw((m - r) * kLog2e) + l2 * exp2_hw((m2 - r) * kLog2e);
  m = M;
}

// ---------------------------------------------------------------------------
// Cross-lane moves on a 64-wide wavefront.
//
// DPP handles the four steps inside a 16-lane row (quad_perm for lane^1 and
// lane^2, row_half_mirror and row_mirror to pair the 4-lane and 8-lane groups);
// gfx950's v_permlane16_swap and v_permlane32_swap exchange whole rows between
// the 16-lane and 32-lane halves.  After a butterfly that uses all six, every
// lane holds the reduction over the wavefront.
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadXor1 = 0xB1,   // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,   // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141,
  kDppRowMirror = 0x140,
};

template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Value of the lane 16 positions away inside its 32-lane half (lane ^ 16).
__device__ __forceinline__ float swap_rows16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // r[0]: odd rows replaced by the even rows of the source; r[1]: even rows
  // replaced by the odd rows.  Each lane wants the other row of its pair.
  const unsigned lane = __lane_id();
  return __uint_as_float(((lane >> 4) & 1) ? r[0] : r[1]);
}

// Value of the lane 32 positions away (lane ^ 32).
__device__ __forceinline__ float swap_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const unsigned lane = __lane_id();
  return __uint_as_float((lane >> 5) ? r[0] : r[1]);
}

// Butterfly all-reduce of online-softmax states over the 64 lanes.
__device__ __forceinline__ void wave_combine_state(float& m, float& l) {
  combine_state(m, l, dpp_move<kDppQuadXor1>(m), dpp_move<kDppQuadXor1>(l));
  combine_state(m, l, dpp_move<kDppQuadXor2>(m), dpp_move<kDppQuadXor2>(l));
  combine_state(m, l, dpp_move<kDppHalfMirror>(m), dpp_move<kDppHalfMirror>(l));
  combine_state(m, l, dpp_move<kDppRowMirror>(m), dpp_move<kDppRowMirror>(l));
  combine_state(m, l, swap_rows16(m), swap_rows16(l));
  combine_state(m, l, swap_halves(m), swap_halves(l));
}

// ---------------------------------------------------------------------------
// bfloat16 <-> float32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats to two bfloat16 in one dword, round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// Stores one 32-column block of a transposed 32x32 matrix-core accumulator
// (lane = row, shared with the partner lane ^ 32; register i = column
// 8 (i / 4) + 4 half + i % 4, half = lane / 32) times `mul` as bfloat16 to
// row[0..31].  One v_permlane32_swap per register pair first trades four of
// this lane's columns for four of the partner's, so that every lane holds 8
// consecutive columns (16 p + 8 half + 0..7 in registers 8 p .. 8 p + 7) and
// writes them with one 16-byte store: half the store instructions of 8-byte
// stores, and each covers 32 contiguous bytes of every row.  Both lanes of a
// row must be active.
template <typename V>
__device__ __forceinline__ void store_block_bf16(uint16_t* row, V a, int half, float mul) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[8 * p + t]),
                                                      __float_as_uint(a[8 * p + 4 + t]), false,
                                                      false);
      a[8 * p + t] = __uint_as_float(r[0]);
      a[8 * p + 4 + t] = __uint_as_float(r[1]);
    }
    uint4 w;
    w.x = pack_bf16x2(a[8 * p + 0] * mul, a[8 * p + 1] * mul);
    w.y = pack_bf16x2(a[8 * p + 2] * mul, a[8 * p + 3] * mul);
    w.z = pack_bf16x2(a[8 * p + 4] * mul, a[8 * p + 5] * mul);
    w.w = pack_bf16x2(a[8 * p + 6] * mul, a[8 * p + 7] * mul);
    *reinterpret_cast<uint4*>(row + 16 * p + 8 * half) = w;
  }
}

}  // namespace osm
