// Wave-level (64-lane) reductions and prefix sums for gfx950 device code.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace up {
namespace {

// Wave-wide reductions and scans on the VALU: DPP row operations within each
// 16-lane row, then the gfx950 row swaps (v_permlane16_swap /
// v_permlane32_swap) across rows — no LDS permutes in the dependent chains.
// Every lane of the wave must be active.
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;    // lane i <- lane 15-i of its row
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i of its half row
constexpr int kDppRowShr = 0x110;       // + n: lane i <- lane i-n of its row
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of a row -> the next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 -> rows 2 and 3

// Lanes whose source is outside the row, or whose row is not in ROW_MASK,
// read `old`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// f over all 64 lanes, in every lane (f commutative and associative; for
// 64-bit values see the u64 overloads).
template <typename F>
__device__ __forceinline__ uint32_t wave_allreduce32(uint32_t v, F f) {
  v = f(v, dpp<kDppQuadXor1>(v, v));
  v = f(v, dpp<kDppQuadXor2>(v, v));
  v = f(v, dpp<kDppRowHalfMirror>(v, v));
  v = f(v, dpp<kDppRowMirror>(v, v));
  auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows (0,1), (2,3)
  v = f(r16[0], r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // halves
  return f(r32[0], r32[1]);
}

__device__ __forceinline__ uint64_t u64_of(uint32_t lo, uint32_t hi) {
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
  auto step = [&](uint64_t a, uint64_t b) { return a + b; };
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
#define UP_U64_STEP(CTRL)                                                              \
  {                                                                                    \
    v = step(v, u64_of(dpp<CTRL>(lo, lo), dpp<CTRL>(hi, hi)));                         \
    lo = (uint32_t)v;                                                                  \
    hi = (uint32_t)(v >> 32);                                                          \
  }
  UP_U64_STEP(kDppQuadXor1)
  UP_U64_STEP(kDppQuadXor2)
  UP_U64_STEP(kDppRowHalfMirror)
  UP_U64_STEP(kDppRowMirror)
#undef UP_U64_STEP
  auto l16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto h16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  v = u64_of(l16[0], h16[0]) + u64_of(l16[1], h16[1]);
  lo = (uint32_t)v;
  hi = (uint32_t)(v >> 32);
  auto l32 = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto h32 = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return u64_of(l32[0], h32[0]) + u64_of(l32[1], h32[1]);
}

__device__ __forceinline__ int wave_sum(int v) {
  return (int)wave_allreduce32((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Inclusive prefix sums over the 64 lanes (lane order): shifts by 1, 2, 4, 8
// within each row, then each row adds the totals of the rows before it.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
  v += dpp<kDppRowShr + 1>(0u, v);
  v += dpp<kDppRowShr + 2>(0u, v);
  v += dpp<kDppRowShr + 4>(0u, v);
  v += dpp<kDppRowShr + 8>(0u, v);
  v += dpp<kDppRowBcast15, 0xa>(0u, v);
  v += dpp<kDppRowBcast31, 0xc>(0u, v);
  return v;
}

__device__ __forceinline__ uint64_t wave_scan_incl(uint64_t v) {
#define UP_U64_SCAN(CTRL, ROWS) \
  v += u64_of(dpp<CTRL, ROWS>(0u, (uint32_t)v), dpp<CTRL, ROWS>(0u, (uint32_t)(v >> 32)));
  UP_U64_SCAN(kDppRowShr + 1, 0xf)
  UP_U64_SCAN(kDppRowShr + 2, 0xf)
  UP_U64_SCAN(kDppRowShr + 4, 0xf)
  UP_U64_SCAN(kDppRowShr + 8, 0xf)
  UP_U64_SCAN(kDppRowBcast15, 0xa)
  UP_U64_SCAN(kDppRowBcast31, 0xc)
#undef UP_U64_SCAN
  return v;
}

// Sum of a float over the 64 lanes, in every lane (a fixed order of
// additions, so every caller gets the same bits for the same inputs).
__device__ __forceinline__ float wave_sum_f32(float v) {
  return __uint_as_float(wave_allreduce32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

}  // namespace
}  // namespace up
