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
//   3. Radix select, most significant digit first, over the 32-bit
//      order-preserving key of each optional block's score.  The bits that
//      the smallest and the largest optional key share are common to every
//      optional key, so the digits start at their highest differing bit
//      (near-uniform scores differ only in low mantissa bits).  Per digit of
//      8 bits: an LDS histogram of (count, mass), then one wave scans
//      the buckets from the top and finds the bucket where the mass from
//      above reaches R.  One to four passes give the exact cutoff score v*
//      and the mass above it.  The histograms alternate between two LDS
//      buffers, so clearing the next one overlaps building the current one.
//   4. Blocks with score v* are tied; the lowest-index ones are kept until the
//      mass reaches R: each thread takes a contiguous run of blocks, and one
//      block-wide exclusive scan of the runs' tie counts ranks every tie (only
//      when some tied blocks are dropped; the last radix pass counts them).
// A request with at most STAGE blocks has its keys and fixed-point masses
// computed once into LDS (every later pass reads them there); longer requests
// recompute them from the scores in memory on every pass.  The workgroup
// size NTH and STAGE are template arguments, so another kernel (the fused
// entry point's block-mean kernel) can run the selection in its workgroups.
// Fixed point differs from exact fp64 sums by < N * 2^-S of the top score, so
// a decision can differ from an fp64 evaluation only when the cumulative
// mass is within that distance of p * total.
#pragma once

#include <math.h>

#include "up_internal.h"
#include "up_wave.h"

namespace up {
namespace {

#ifndef UP_SEL_THREADS
#define UP_SEL_THREADS 512
#endif
constexpr int kSelectThreads = UP_SEL_THREADS;
constexpr int64_t kMaxBlocksPerRequest = 1 << 24;
constexpr int kStageMax = 4096;         // blocks staged in LDS by the stand-alone kernel
#ifndef UP_SEL_DIGIT_BITS
#define UP_SEL_DIGIT_BITS 8
#endif
constexpr int kDigitBits = UP_SEL_DIGIT_BITS;
constexpr int kBuckets = 1 << kDigitBits;
constexpr int kBucketsPerLane = kBuckets / 64;
// Histogram slot of bucket d: one pad slot per kBucketsPerLane buckets, so the
// wave that scans the buckets (lane l reads kBucketsPerLane consecutive ones
// from the top) spreads each step's reads over the LDS banks.
constexpr int kBucketSlots = kBuckets + kBuckets / kBucketsPerLane;
__device__ __forceinline__ int bslot(int d) { return d + d / kBucketsPerLane; }

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

template <int NTH, int STAGE>
struct SelectShared {
  static constexpr int kWaves = NTH / 64;
  static constexpr int kStage = STAGE;
  uint32_t skey[STAGE];   // staged: order-preserving key (0 for forced blocks)
  uint64_t smass[STAGE];  // staged: fixed-point mass
  uint32_t cnt[2][kBucketSlots];
  uint64_t mass[2][kBucketSlots];
  uint64_t red64[2][kWaves];
  float redf[kWaves];
  uint32_t redu[2][kWaves];
  int redi[kWaves];
  // decision state (written by wave 0, read by all after a barrier)
  uint32_t prefix;       // known high bits of the cutoff key
  uint64_t above;        // optional mass with key above the current bucket range
  int all_optional;      // the optional mass never reaches R: keep every block
  uint64_t tie_mass;     // mass of one block at the cutoff key
  uint64_t tie_keep;     // how many tied blocks (lowest index first) are kept
  uint32_t tie_count;    // optional blocks at the cutoff key
};

// Wave 0: scan the buckets from the top (descending keys) for the first
// bucket where above + (mass of this and higher buckets) >= need; refine the
// state.  Bucket d of this pass holds keys whose bits [shift, shift + width)
// equal d (higher bits equal the known prefix).
template <typename Shared>
__device__ void pick_bucket(Shared& sh, int buf, int shift, int width, uint64_t need) {
  const int lane = threadIdx.x & 63;
  const int nbk = 1 << width;
  // lane l owns buckets top-kBucketsPerLane*l ... (highest first)
  uint64_t m[kBucketsPerLane];
  uint64_t local = 0;
#pragma unroll
  for (int i = 0; i < kBucketsPerLane; ++i) {
    const int d = nbk - 1 - kBucketsPerLane * lane - i;
    m[i] = d >= 0 ? sh.mass[buf][bslot(d)] : 0;
    local += m[i];
  }
  const uint64_t incl = wave_scan_incl(local);
  const uint64_t before = sh.above + (incl - local);  // mass of buckets above this lane's first
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
    for (; i < kBucketsPerLane - 1; ++i) {
      if (acc + m[i] >= need) break;
      acc += m[i];
    }
    const uint32_t digit = (uint32_t)(nbk - 1 - kBucketsPerLane * lane - i);
    sh.prefix |= digit << shift;
    sh.above = acc;
    if (shift == 0) {
      const uint32_t c = sh.cnt[buf][bslot(digit)];
      sh.tie_count = c;
      sh.tie_mass = c ? m[i] / c : 0;
      const uint64_t rest = need - acc;  // > 0, <= m[i]
      sh.tie_keep = sh.tie_mass ? (rest + sh.tie_mass - 1) / sh.tie_mass : c;
    }
  }
}

// Block score i of a request: COHERENT reads it with a relaxed device-scope
// atomic load, for scores written earlier in the same kernel by workgroups
// on other XCDs (the block-mean kernel of the fused entry point).
template <bool COHERENT>
__device__ __forceinline__ float score_at(const float* sc, int i) {
  if constexpr (COHERENT)
    return __hip_atomic_load(sc + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return sc[i];
}

// Selection of one request by the whole (NTH-thread) workgroup.
// STAGED: the request has at most STAGE blocks; their keys and masses are
// computed once into LDS and every later pass reads them from there.
template <bool STAGED, int NTH, int STAGE, bool COHERENT>
__device__ void select_impl(const SelectArgs& a, int req, int nb, SelectShared<NTH, STAGE>& sh) {
  constexpr int kSelectThreads = NTH;
  constexpr int kSelectWaves = NTH / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s0 = a.cu_seqlens[req];
  const int L = a.cu_seqlens[req + 1] - s0;
  const int cb0 = a.cu_blocks[req];
  const int G = a.block;
  const float* sc = a.scores + cb0;

  // 1. largest score, smallest / largest optional key (staging the scores)
  float mx = 0.f;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  auto visit = [&](int i, float s) {
    if (STAGED) sh.skey[i] = __float_as_uint(s);
    mx = fmaxf(mx, s);
    if (!is_forced(i, L, G, a.sink, a.tail)) {
      const uint32_t k = orderable(s);
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    }
  };
  if constexpr (STAGED) {
    // at most STAGE / NTH scores per thread: all loads issued before the
    // first is used (one round trip instead of one per score)
    constexpr int PER = (STAGE + kSelectThreads - 1) / kSelectThreads;
    float v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSelectThreads;
      v[u] = i < nb ? score_at<COHERENT>(sc, i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSelectThreads;
      if (i < nb) visit(i, v[u]);
    }
  } else {
    for (int i = tid; i < nb; i += kSelectThreads) visit(i, score_at<COHERENT>(sc, i));
  }
  mx = __uint_as_float(wave_allreduce32(__float_as_uint(mx), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
  kmin = wave_allreduce32(kmin, [](uint32_t a, uint32_t b) { return min(a, b); });
  kmax = wave_allreduce32(kmax, [](uint32_t a, uint32_t b) { return max(a, b); });
  if (lane == 0) {
    sh.redf[wave] = mx;
    sh.redu[0][wave] = kmin;
    sh.redu[1][wave] = kmax;
  }
  __syncthreads();
  mx = sh.redf[0];
  kmin = sh.redu[0][0];
  kmax = sh.redu[1][0];
  for (int w = 1; w < kSelectWaves; ++w) {
    mx = fmaxf(mx, sh.redf[w]);
    kmin = min(kmin, sh.redu[0][w]);
    kmax = max(kmax, sh.redu[1][w]);
  }
  int lg = 0;
  while ((1ll << lg) < (int64_t)nb + 1) ++lg;
  const int S = 62 - lg;
  const double scale = mx > 0.f ? ldexp(1.0, S) / (double)mx : 0.0;

  // Key of an optional block (forced: false) and its mass.
  auto key_mass = [&](int i, uint32_t& key, uint64_t& m) -> bool {
    if (STAGED) {
      key = sh.skey[i];
      if (key == 0) return false;  // forced
      m = sh.smass[i];
      return true;
    }
    if (is_forced(i, L, G, a.sink, a.tail)) return false;
    const float s = score_at<COHERENT>(sc, i);
    key = orderable(s);
    m = mass_of(s, scale);
    return true;
  };

  // 2. total and forced mass (one two-value reduction); staged: keys and
  //    masses into LDS (each thread rewrites the entries it staged)
  uint64_t tot = 0, forced = 0;
  for (int i = tid; i < nb; i += kSelectThreads) {
    const float s = STAGED ? __uint_as_float(sh.skey[i]) : score_at<COHERENT>(sc, i);
    const uint64_t m = mass_of(s, scale);
    const bool f = is_forced(i, L, G, a.sink, a.tail);
    tot += m;
    if (f) forced += m;
    if (STAGED) {
      sh.smass[i] = m;
      sh.skey[i] = f ? 0u : orderable(s);  // real scores never map to key 0
    }
  }
  tot = wave_sum(tot);
  forced = wave_sum(forced);
  if (lane == 0) {
    sh.red64[0][wave] = tot;
    sh.red64[1][wave] = forced;
  }
  // state for the radix passes (read after the next barrier)
  if (tid == 0) {
    sh.above = 0;
    sh.all_optional = 0;
    sh.tie_mass = 0;
    sh.tie_keep = 0;
    sh.tie_count = 0;
  }
  // the digits start at the highest bit where optional keys differ
  const uint32_t diff = kmin ^ kmax;
  const int top = diff ? 31 - __clz(diff) : 0;        // highest differing bit
  int width = min(kDigitBits, top + 1);
  int shift = top + 1 - width;
  const uint32_t common = (top == 31) ? 0u : (kmin & (0xFFFFFFFFu << (top + 1)));
  if (tid == 0) sh.prefix = common;
  for (int d = tid; d < (1 << width); d += kSelectThreads) {
    sh.cnt[0][bslot(d)] = 0;
    sh.mass[0][bslot(d)] = 0;
  }
  __syncthreads();
  tot = 0;
  forced = 0;
  for (int w = 0; w < kSelectWaves; ++w) {
    tot += sh.red64[0][w];
    forced += sh.red64[1][w];
  }
  const uint64_t target = (uint64_t)ceil(a.top_p * (double)tot);
  const int64_t need = (int64_t)target - (int64_t)forced;
  const bool any_optional = need > 0 && kmin <= kmax;

  // 3. radix select of the cutoff key over optional blocks, most significant
  //    digit first; histogram buffers alternate (the next one is cleared
  //    while the current one is built)
  if (any_optional) {
    for (int pass = 0;; ++pass) {
      const int buf = pass & 1;
      const uint32_t hi_mask = (shift + width >= 32) ? 0u : (0xFFFFFFFFu << (shift + width));
      const uint32_t prefix = sh.prefix;
      const int next_width = min(kDigitBits, shift);
      for (int d = tid; d < (1 << next_width) && shift > 0; d += kSelectThreads) {
        sh.cnt[buf ^ 1][bslot(d)] = 0;
        sh.mass[buf ^ 1][bslot(d)] = 0;
      }
      // counts are needed by the last digit only (tied blocks)
      const bool last = shift == 0;
      for (int i = tid; i < nb; i += kSelectThreads) {
        uint32_t key;
        uint64_t m;
        if (!key_mass(i, key, m)) continue;
        if ((key & hi_mask) != (prefix & hi_mask)) continue;
        const int d = bslot((int)((key >> shift) & ((1u << width) - 1u)));
        if (last) atomicAdd(&sh.cnt[buf][d], 1u);
        atomicAdd((unsigned long long*)&sh.mass[buf][d], (unsigned long long)m);
      }
      __syncthreads();
      if (wave == 0) pick_bucket(sh, buf, shift, width, (uint64_t)need);
      __syncthreads();
      if (sh.all_optional || shift == 0) break;
      width = next_width;
      shift -= width;
    }
  }

  // 4. mask: forced, above the cutoff, or among the first tie_keep ties;
  //    thread t takes the contiguous run of blocks [t*run, (t+1)*run)
  const uint32_t vstar = sh.prefix;
  const bool keep_all = sh.all_optional != 0;
  const uint64_t tie_keep = sh.tie_keep;
  // ranks among the blocks at the cutoff key matter only when some of them
  // are dropped (uniform over the workgroup)
  const bool rank_ties = any_optional && !keep_all && tie_keep < (uint64_t)sh.tie_count;
  const int run = (nb + kSelectThreads - 1) / kSelectThreads;
  const int i0 = min(nb, tid * run), i1 = min(nb, i0 + run);
  int64_t rank = 0;
  if (rank_ties) {
    int my_ties = 0;
    for (int i = i0; i < i1; ++i) {
      uint32_t key;
      uint64_t m;
      my_ties += (key_mass(i, key, m) && key == vstar) ? 1 : 0;
    }
    // exclusive scan of the tie counts in thread (= block index) order
    const int incl = (int)wave_scan_incl((uint32_t)my_ties);
    if (lane == 63) sh.redi[wave] = incl;
    __syncthreads();
    rank = incl - my_ties;
    for (int w = 0; w < wave; ++w) rank += sh.redi[w];
  }
  int kept_tokens = 0;
  for (int i = i0; i < i1; ++i) {
    uint32_t key;
    uint64_t m;
    const bool opt = key_mass(i, key, m);
    bool keep = !opt || (any_optional && (keep_all || key >= vstar));
    if (rank_ties && opt && key == vstar) keep = (uint64_t)(rank++) < tie_keep;
    a.mask[cb0 + i] = keep ? 1 : 0;
    if (keep) kept_tokens += min(i * G + G, L) - i * G;
  }
  kept_tokens = wave_sum(kept_tokens);
  __syncthreads();  // every wave has read redi
  if (lane == 0) sh.redi[wave] = kept_tokens;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < kSelectWaves; ++w) s += sh.redi[w];
    a.kept[req] = s;
  }
}

// Selection of one request by the whole (NTH-thread) workgroup.
// Uniform over the workgroup; every thread must call it.
template <int NTH, int STAGE, bool COHERENT = false>
__device__ void select_request(const SelectArgs& a, int req, SelectShared<NTH, STAGE>& sh) {
  const int nb = a.cu_blocks[req + 1] - a.cu_blocks[req];
  if (nb <= 0) {
    if (threadIdx.x == 0) a.kept[req] = 0;
    return;
  }
  __syncthreads();  // the shared state may still be read by a previous call
  if (nb <= STAGE) select_impl<true, NTH, STAGE, COHERENT>(a, req, nb, sh);
  else select_impl<false, NTH, STAGE, COHERENT>(a, req, nb, sh);
}

}  // namespace
}  // namespace up
