// qs_wave.h -- wave64 cross-lane primitives for gfx950 built from DPP moves
// and the v_permlane16/32_swap instructions, so reductions and scans stay in
// the VALU instead of going through the LDS crossbar (ds_bpermute).
//
// Butterfly partner of stage s for lane l:
//   s=0: l^1 (quad_perm), s=1: l^2 (quad_perm),
//   s=2: 7-l within each 8-lane half row (row_half_mirror),
//   s=3: 15-l within each 16-lane row (row_mirror),
//   s=4: l^16 (permlane16_swap), s=5: l^32 (permlane32_swap).
// Stages 2 and 3 are not xor partners, but after stages 0..1 (resp. 0..2)
// every lane of a quad (half row) holds the same value, so combining with the
// mirrored lane combines two disjoint groups.  After stages 0..n-1 every lane
// of an aligned group of 2^n lanes holds the group's result, computed in the
// same order on every lane.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qs {

// Every control used here reads a valid lane for every lane, so the move
// needs no "old" value; that lets the compiler fold it into the consuming
// VALU instruction as a DPP operand.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Partner value of butterfly stage S (see above).
template <int S>
__device__ __forceinline__ uint32_t partner_u32(uint32_t v) {
  if constexpr (S == 0) return dpp_mov<0xB1>(v);
  else if constexpr (S == 1) return dpp_mov<0x4E>(v);
  else if constexpr (S == 2) return dpp_mov<0x141>(v);
  else if constexpr (S == 3) return dpp_mov<0x140>(v);
  else if constexpr (S == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
  }
}

template <int S>
__device__ __forceinline__ float partner_f32(float v) {
  return __uint_as_float(partner_u32<S>(__float_as_uint(v)));
}

template <int S>
__device__ __forceinline__ double partner_f64(double v) {
  const uint32_t lo = (uint32_t)__double2loint(v), hi = (uint32_t)__double2hiint(v);
  return __hiloint2double((int)partner_u32<S>(hi), (int)partner_u32<S>(lo));
}

// Sum over aligned groups of 2^N lanes; every lane gets its group's sum.
template <int N>
__device__ __forceinline__ float bfly_sum(float v) {
  if constexpr (N > 0) v += partner_f32<0>(v);
  if constexpr (N > 1) v += partner_f32<1>(v);
  if constexpr (N > 2) v += partner_f32<2>(v);
  if constexpr (N > 3) v += partner_f32<3>(v);
  if constexpr (N > 4) v += partner_f32<4>(v);
  if constexpr (N > 5) v += partner_f32<5>(v);
  return v;
}

template <int N>
__device__ __forceinline__ double bfly_sum_f64(double v) {
  if constexpr (N > 0) v += partner_f64<0>(v);
  if constexpr (N > 1) v += partner_f64<1>(v);
  if constexpr (N > 2) v += partner_f64<2>(v);
  if constexpr (N > 3) v += partner_f64<3>(v);
  if constexpr (N > 4) v += partner_f64<4>(v);
  if constexpr (N > 5) v += partner_f64<5>(v);
  return v;
}

template <int N>
__device__ __forceinline__ float bfly_max(float v) {
  if constexpr (N > 0) v = fmaxf(v, partner_f32<0>(v));
  if constexpr (N > 1) v = fmaxf(v, partner_f32<1>(v));
  if constexpr (N > 2) v = fmaxf(v, partner_f32<2>(v));
  if constexpr (N > 3) v = fmaxf(v, partner_f32<3>(v));
  if constexpr (N > 4) v = fmaxf(v, partner_f32<4>(v));
  if constexpr (N > 5) v = fmaxf(v, partner_f32<5>(v));
  return v;
}

template <int N>
__device__ __forceinline__ int bfly_sum_i32(int v) {
  if constexpr (N > 0) v += (int)partner_u32<0>((uint32_t)v);
  if constexpr (N > 1) v += (int)partner_u32<1>((uint32_t)v);
  if constexpr (N > 2) v += (int)partner_u32<2>((uint32_t)v);
  if constexpr (N > 3) v += (int)partner_u32<3>((uint32_t)v);
  if constexpr (N > 4) v += (int)partner_u32<4>((uint32_t)v);
  if constexpr (N > 5) v += (int)partner_u32<5>((uint32_t)v);
  return v;
}

// Runtime group width (power of two, 1..64).
__device__ __forceinline__ float bfly_sum_dyn(float v, int width) {
  switch (width) {
    case 1: return v;
    case 2: return bfly_sum<1>(v);
    case 4: return bfly_sum<2>(v);
    case 8: return bfly_sum<3>(v);
    case 16: return bfly_sum<4>(v);
    case 32: return bfly_sum<5>(v);
    default: return bfly_sum<6>(v);
  }
}

// (value desc, index asc) better-than, for arg-max with ties to the lower index.
__device__ __forceinline__ bool better(double ov, int oi, double v, int i) {
  return ov > v || (ov == v && oi < i);
}

template <int S>
__device__ __forceinline__ void argmax_stage(double& v, int& i) {
  const double ov = partner_f64<S>(v);
  const int oi = (int)partner_u32<S>((uint32_t)i);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Wave-wide arg-max of (v, i); every lane receives the winner.
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
  argmax_stage<0>(v, i);
  argmax_stage<1>(v, i);
  argmax_stage<2>(v, i);
  argmax_stage<3>(v, i);
  argmax_stage<4>(v, i);
  argmax_stage<5>(v, i);
}

// Inclusive prefix sum over the 64 lanes (row shifts, then row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}

}  // namespace qs
