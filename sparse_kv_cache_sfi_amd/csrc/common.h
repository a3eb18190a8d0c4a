// Device helpers shared by the SFI kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfi {

constexpr int kPage = 16;     // tokens per KV page
constexpr int kWave = 64;     // CDNA wavefront width
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;   // one 16-byte load
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// bfloat16 is the upper half of a float32: widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// v_dot2_f32_bf16: a.x*b.x + a.y*b.y + c with bf16 pairs (products are exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// Inclusive prefix sum over the 64 lanes of a wave, in lane order: DPP row shifts by
// 1, 2, 4 and 8 within each row of 16 lanes (a lane shifted in from outside the row
// contributes 0), then the totals of the lower rows, read with readlane.  Every lane
// of the wave must be active.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (int)(threadIdx.x & 63) >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// v_exp_f32 computes 2^x; exp2(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of N consecutive lanes (N in {1,2,4,8,16}); every
// lane of the group receives the group sum.  DPP quad_perm xor-1 / xor-2, then
// row_half_mirror (pairs the two quads of 8 lanes), then row_mirror (pairs the
// two halves of a 16-lane row).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);
  if constexpr (N >= 16) x += dpp_mov<0x140>(x);
  return x;
}

// The values x holds in lanes (lane & ~OFF) and (lane | OFF), for OFF 16 or 32, as
// (lo, hi): v_permlane16_swap / v_permlane32_swap (gfx950), VALU operations that
// exchange 16-lane rows or 32-lane halves without a trip through the LDS unit.
template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float& lo, float& hi) {
  static_assert(OFF == 16 || OFF == 32, "row or half-wave pairs");
  const uint32_t u = __float_as_uint(x);
  if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  }
}

// The value of x held by lane (lane ^ OFF), for a power of two OFF < 64: DPP
// quad_perm for 1 and 2, DPP row_ror:8 for 8 (a rotation by 8 inside a 16-lane row
// is the xor-8 exchange), for 4 the rotations by 4 and by 12 inside the row (lane i
// receives lane i - 4 or i + 4, and a lane keeps the one that is its xor-4 partner),
// the permlane swaps for 16 and 32: VALU operations, none through the LDS unit.  Every
// lane must be active (blocks are whole waves, so lane = threadIdx.x mod 64).
template <int OFF>
__device__ __forceinline__ float lane_xor(float x) {
  static_assert(OFF > 0 && OFF < 64 && (OFF & (OFF - 1)) == 0, "power of two below the wave width");
  if constexpr (OFF == 1) return dpp_mov<0xB1>(x);
  else if constexpr (OFF == 2) return dpp_mov<0x4E>(x);
  else if constexpr (OFF == 8) return dpp_mov<0x128>(x);
  else if constexpr (OFF == 16 || OFF == 32) {
    float lo, hi;
    lane_pair<OFF>(x, lo, hi);
    return (threadIdx.x & OFF) ? lo : hi;
  } else {
    const float down = dpp_mov<0x124>(x);   // row_ror:4: lane i receives lane i - 4 (mod 16)
    const float up = dpp_mov<0x12C>(x);     // row_ror:12: lane i receives lane i + 4 (mod 16)
    return (threadIdx.x & 4) ? down : up;
  }
}

// x combined by op with the lanes at xor distance FROM, 2 FROM, ..., 32, in that
// order: every lane ends with op over the lanes that share its bits below FROM (op
// commutative: the 16 and 32 steps combine the pair as op(lo, hi) in every lane).
template <int FROM, typename Op>
__device__ __forceinline__ float xor_fold(float x, Op op) {
  if constexpr (FROM < kWave) {
    if constexpr (FROM == 16 || FROM == 32) {
      float lo, hi;
      lane_pair<FROM>(x, lo, hi);
      x = op(lo, hi);
    } else {
      x = op(x, lane_xor<FROM>(x));
    }
    return xor_fold<FROM * 2>(x, op);
  } else {
    return x;
  }
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Request length as the kernels use it: never beyond what the block table or the
// launch plan can address.
__device__ __forceinline__ int clamp_len(int L, int max_seq_len, int max_pages) {
  return clampi(L, 0, min(max_seq_len, max_pages * kPage));
}

// Candidate range [lo, hi) of a slow step / verification with t_q query tokens.
__device__ __forceinline__ void candidate_bounds(int L, int t_q, int n_sink, int n_recent, int* lo, int* hi) {
  const int l = n_sink;
  const int h = L - t_q + 1 - n_recent;
  *lo = l;
  *hi = h > l ? h : l;
}

}  // namespace sfi
