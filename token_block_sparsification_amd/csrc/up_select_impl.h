// Top-p block selection for one request, shared by the stand-alone selection
// kernel and the scoring epilogue that runs it in its last workgroup.
//
// Method (UniPrefill page "中国科学院与腾讯微信合作解决AI排队等待问题", §二 step 2 and
// Q&A 1; §三 for the binary mask): blocks are ranked by score, the smallest
// set holding p of the total importance is kept, and the blocks covering the
// first and the last 128 tokens are exempt from pruning.
//
// Rule: forced blocks count toward the mass; optional blocks are taken in
// (score desc, index asc) order while the kept mass is below p * total.  The
// kept optional blocks are therefore exactly those ranked before a cutoff
// block, so no full sort is needed, only the cutoff:
//
//   1. One workgroup per request.  Each block's score becomes an integer mass
//      m = floor(score / max_score * 2^S) (S chosen so the sum fits 63 bits),
//      so every sum below is exact and independent of summation order: the
//      result is bitwise deterministic.
//   2. R = ceil(p * total) - forced mass is the optional mass still needed.
//   3. Radix select, most significant 8-bit digit first, over the 32-bit
//      order-preserving key of each optional block's score: an LDS histogram
//      of (count, mass) per digit, then one wave scans the 256 buckets from
//      the top and finds the bucket where the mass from above reaches R.
//      Four passes give the exact cutoff score v* and the mass above it.
//   4. Blocks with score v* are tied; the lowest-index ones are kept until the
//      mass reaches R (a block-wide prefix count over index order).
// Fixed point differs from exact fp64 sums by < N * 2^-S of the top score, so
// a decision can differ from an fp64 evaluation only when the cumulative
// mass is within that distance of p * total.
#pragma once

#include <math.h>

#include "up_internal.h"

namespace up {
namespace {

constexpr int kSelectThreads = 256;
constexpr int kSelectWaves = kSelectThreads / 64;
constexpr int64_t kMaxBlocksPerRequest = 1 << 24;

struct SelectArgs {
  const int32_t* cu_seqlens;
  const int32_t* cu_blocks;
  const float* scores;
  uint8_t* mask;
  int32_t* kept;
  int block, sink, tail;
  double top_p;
};

__device__ __forceinline__ uint32_t orderable(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool is_forced(int i, int L, int G, int sink, int tail) {
  const int j0 = i * G;
  const int j1 = min(j0 + G, L);
  return j0 < sink || j1 > L - tail;
}

__device__ __forceinline__ uint64_t mass_of(float s, double scale) {
  const double m = (double)s * scale;
  return m > 0.0 ? (uint64_t)m : 0ull;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

struct SelectShared {
  uint32_t cnt[256];
  uint64_t mass[256];
  uint64_t red[kSelectWaves];
  float redf[kSelectWaves];
  int redi[kSelectWaves];
  // decision state (written by wave 0, read by all after a barrier)
  uint32_t prefix;       // known high digits of the cutoff key
  uint64_t above;        // optional mass with key above the current bucket range
  int64_t need;          // R: optional mass still needed (<= 0: none)
  int all_optional;      // the optional mass never reaches R: keep every block
  uint64_t tie_mass;     // mass of one block at the cutoff key
  uint64_t tie_keep;     // how many tied blocks (lowest index first) are kept
};

// Block-wide reductions (fixed order: wave butterfly, then waves in order).
__device__ uint64_t block_sum_u64(uint64_t v, SelectShared& sh) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t s = 0;
  for (int w = 0; w < kSelectWaves; ++w) s += sh.red[w];
  return s;
}

__device__ float block_max(float v, SelectShared& sh) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.redf[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = sh.redf[0];
  for (int w = 1; w < kSelectWaves; ++w) m = fmaxf(m, sh.redf[w]);
  return m;
}

// Wave 0: scan buckets 255..0 (descending keys) for the first bucket where
// above + (mass of this and higher buckets) >= need; refine the state.
__device__ void pick_bucket(SelectShared& sh, int shift) {
  const int lane = threadIdx.x & 63;
  // lane l owns buckets 255-4l .. 252-4l, highest first
  uint64_t m[4];
  uint64_t local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = sh.mass[255 - 4 * lane - i];
    local += m[i];
  }
  uint64_t incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  const uint64_t before = sh.above + (incl - local);  // mass of buckets above this lane's first
  const uint64_t need = (uint64_t)sh.need;
  const bool crosses = before + local >= need;
  const uint64_t ballot = __ballot(crosses);
  if (ballot == 0) {  // the candidates never reach R (only possible on the first pass)
    if (lane == 0) sh.all_optional = 1;
    return;
  }
  const int first = __ffsll((unsigned long long)ballot) - 1;
  if (lane == first) {
    uint64_t acc = before;
    int i = 0;
    for (; i < 3; ++i) {
      if (acc + m[i] >= need) break;
      acc += m[i];
    }
    const uint32_t digit = (uint32_t)(255 - 4 * lane - i);
    sh.prefix |= digit << shift;
    sh.above = acc;
    if (shift == 0) {
      const uint32_t c = sh.cnt[digit];
      sh.tie_mass = c ? m[i] / c : 0;
      const uint64_t rest = need - acc;  // > 0, <= m[i]
      sh.tie_keep = sh.tie_mass ? (rest + sh.tie_mass - 1) / sh.tie_mass : c;
    }
  }
}

// Selection of one request by the whole (kSelectThreads-thread) workgroup.
// Uniform over the workgroup; every thread must call it.
__device__ void select_request(const SelectArgs& a, int req, SelectShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s0 = a.cu_seqlens[req];
  const int L = a.cu_seqlens[req + 1] - s0;
  const int cb0 = a.cu_blocks[req];
  const int nb = a.cu_blocks[req + 1] - cb0;
  if (nb <= 0) {
    if (tid == 0) a.kept[req] = 0;
    return;
  }
  __syncthreads();  // the shared state may still be read by a previous call
  const int G = a.block;
  const float* sc = a.scores + cb0;

  // 1. fixed-point scale from the request's largest score
  float mx = 0.f;
  for (int i = tid; i < nb; i += kSelectThreads) mx = fmaxf(mx, sc[i]);
  mx = block_max(mx, sh);
  int lg = 0;
  while ((1ll << lg) < (int64_t)nb + 1) ++lg;
  const int S = 62 - lg;
  const double scale = mx > 0.f ? ldexp(1.0, S) / (double)mx : 0.0;

  // 2. total and forced mass
  uint64_t tot = 0, forced = 0;
  for (int i = tid; i < nb; i += kSelectThreads) {
    const uint64_t m = mass_of(sc[i], scale);
    tot += m;
    if (is_forced(i, L, G, a.sink, a.tail)) forced += m;
  }
  tot = block_sum_u64(tot, sh);
  forced = block_sum_u64(forced, sh);
  if (tid == 0) {
    const uint64_t target = (uint64_t)ceil(a.top_p * (double)tot);
    sh.need = (int64_t)target - (int64_t)forced;
    sh.prefix = 0;
    sh.above = 0;
    sh.all_optional = 0;
    sh.tie_mass = 0;
    sh.tie_keep = 0;
  }
  __syncthreads();
  const bool any_optional = sh.need > 0;

  // 3. radix select of the cutoff key over optional blocks, MSB digit first
  if (any_optional) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int d = tid; d < 256; d += kSelectThreads) {
        sh.cnt[d] = 0;
        sh.mass[d] = 0;
      }
      __syncthreads();
      const uint32_t hi_mask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
      const uint32_t prefix = sh.prefix;
      for (int i = tid; i < nb; i += kSelectThreads) {
        if (is_forced(i, L, G, a.sink, a.tail)) continue;
        const float s = sc[i];
        const uint32_t key = orderable(s);
        if ((key & hi_mask) != (prefix & hi_mask)) continue;
        const uint32_t d = (key >> shift) & 0xFFu;
        atomicAdd(&sh.cnt[d], 1u);
        atomicAdd((unsigned long long*)&sh.mass[d], (unsigned long long)mass_of(s, scale));
      }
      __syncthreads();
      if (wave == 0) pick_bucket(sh, shift);
      __syncthreads();
      if (sh.all_optional) break;
    }
  }

  // 4. mask: forced, above the cutoff, or among the first tie_keep ties
  const uint32_t vstar = sh.prefix;
  const bool keep_all = sh.all_optional != 0;
  const uint64_t tie_keep = sh.tie_keep;
  int kept_tokens = 0;
  uint64_t ties_before = 0;  // ties at lower indices in earlier rounds
  for (int base = 0; base < nb; base += kSelectThreads) {
    const int i = base + tid;
    bool keep = false, tie = false;
    if (i < nb) {
      const bool f = is_forced(i, L, G, a.sink, a.tail);
      const uint32_t key = orderable(sc[i]);
      tie = any_optional && !keep_all && !f && key == vstar;
      keep = f || (any_optional && (keep_all || key > vstar));
    }
    // rank of this tie among ties in index order
    const uint64_t bal = __ballot(tie);
    const int below_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) sh.redi[wave] = __popcll(bal);
    __syncthreads();
    int below_waves = 0, round_ties = 0;
    for (int w = 0; w < kSelectWaves; ++w) {
      if (w < wave) below_waves += sh.redi[w];
      round_ties += sh.redi[w];
    }
    if (tie) keep = (ties_before + below_waves + below_in_wave) < tie_keep;
    ties_before += round_ties;
    if (i < nb) {
      a.mask[cb0 + i] = keep ? 1 : 0;
      if (keep) kept_tokens += min(i * G + G, L) - i * G;
    }
  }
  kept_tokens = wave_sum(kept_tokens);
  __syncthreads();
  if (lane == 0) sh.redi[wave] = kept_tokens;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < kSelectWaves; ++w) s += sh.redi[w];
    a.kept[req] = s;
  }
}

}  // namespace
}  // namespace up
