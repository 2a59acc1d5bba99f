// Step 4 of the pruning path: Top-p block selection with forced blocks.
//
// Method (UniPrefill page "中国科学院与腾讯微信合作解决AI排队等待问题", §二 step 2 and
// Q&A 1; §三 for the binary mask): blocks are ranked by score, the smallest
// set holding p of the total importance is kept, and the blocks covering the
// first and the last 128 tokens are exempt from pruning.
//
// One workgroup per request.  Each block becomes a 64-bit key
//   (forced ? 0xFFFFFFFF : order-preserving bits of its score) << 32 | ~index
// so a descending sort puts the forced blocks first and the rest in
// (score desc, index asc) order.  The keys are sorted in LDS with a bitonic
// network; an fp64 exclusive scan over the sorted scores (fixed order, no
// atomics) then keeps position k iff it is forced or its exclusive prefix is
// still below p * total.
#include "up_internal.h"

namespace up {
namespace {

constexpr int kSelectThreads = 1024;
constexpr int kSelectWaves = kSelectThreads / 64;
constexpr int kMaxBlocksPerRequest = 16384;

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

// Block-wide exclusive scan of one double per thread (fixed order).
__device__ double block_exclusive_scan(double x, double* wave_tot, double* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int w = 0; w < kSelectWaves; ++w) {
      const double t = wave_tot[w];
      wave_tot[w] = acc;
      acc += t;
    }
    wave_tot[kSelectWaves] = acc;
  }
  __syncthreads();
  const double excl = wave_tot[wave] + (incl - x);
  *total = wave_tot[kSelectWaves];
  return excl;
}

__global__ void __launch_bounds__(kSelectThreads) up_select_kernel(SelectArgs a) {
  extern __shared__ uint64_t keys[];
  __shared__ double wave_tot[kSelectWaves + 1];
  __shared__ int wave_kept[kSelectWaves];

  const int req = blockIdx.x;
  const int tid = threadIdx.x;
  const int s0 = a.cu_seqlens[req];
  const int L = a.cu_seqlens[req + 1] - s0;
  const int cb0 = a.cu_blocks[req];
  const int nb = a.cu_blocks[req + 1] - cb0;
  if (nb <= 0) {
    if (tid == 0) a.kept[req] = 0;
    return;
  }
  const int G = a.block;
  int np = 1;
  while (np < nb) np <<= 1;

  for (int i = tid; i < np; i += kSelectThreads) {
    uint64_t key = 0;
    if (i < nb) {
      const uint32_t hi =
          is_forced(i, L, G, a.sink, a.tail) ? 0xFFFFFFFFu : orderable(a.scores[cb0 + i]);
      key = ((uint64_t)hi << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
    }
    keys[i] = key;
  }
  __syncthreads();

  // Bitonic sort, descending.
  for (int k = 2; k <= np; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < np; i += kSelectThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = keys[i], y = keys[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  // Each thread owns a contiguous run of sorted positions.
  const int per = (np + kSelectThreads - 1) / kSelectThreads;
  const int p0 = tid * per, p1 = min(p0 + per, nb);
  double local = 0.0;
  for (int p = p0; p < p1; ++p) {
    const int idx = (int)(0xFFFFFFFFu - (uint32_t)(keys[p] & 0xFFFFFFFFu));
    local += (double)a.scores[cb0 + idx];
  }
  double total;
  double excl = block_exclusive_scan(local, wave_tot, &total);
  const double target = a.top_p * total;

  int kept_tokens = 0;
  for (int p = p0; p < p1; ++p) {
    const int idx = (int)(0xFFFFFFFFu - (uint32_t)(keys[p] & 0xFFFFFFFFu));
    const bool forced = is_forced(idx, L, G, a.sink, a.tail);
    const bool keep = forced || (excl < target);
    a.mask[cb0 + idx] = keep ? 1 : 0;
    if (keep) kept_tokens += min(idx * G + G, L) - idx * G;
    excl += (double)a.scores[cb0 + idx];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) kept_tokens += __shfl_xor(kept_tokens, off);
  if ((tid & 63) == 0) wave_kept[tid >> 6] = kept_tokens;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < kSelectWaves; ++w) s += wave_kept[w];
    a.kept[req] = s;
  }
}

}  // namespace
}  // namespace up

extern "C" up_status up_select_topp(int num_seqs, const int32_t* cu_seqlens_h,
                                    const int32_t* cu_seqlens_d, const int32_t* cu_blocks_d,
                                    const float* block_scores, int block, double top_p, int sink,
                                    int tail, uint8_t* block_mask, int32_t* kept_tokens,
                                    hipStream_t stream) {
  up::clear_error();
  int64_t T;
  int max_len;
  up_status st = up::check_cu_seqlens(num_seqs, cu_seqlens_h, &T, &max_len);
  if (st != UP_OK) return st;
  if (block < 1) return up::set_error(UP_ERR_INVALID, "block < 1");
  if (!(top_p > 0.0 && top_p <= 1.0)) return up::set_error(UP_ERR_INVALID, "top_p not in (0, 1]");
  if (sink < 0 || tail < 0) return up::set_error(UP_ERR_INVALID, "sink and tail must be >= 0");
  if (num_seqs == 0) return UP_OK;
  if (!cu_seqlens_d || !cu_blocks_d || !kept_tokens || (T > 0 && (!block_scores || !block_mask)))
    return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  const int64_t max_nb = up::ceil_div(max_len, block);
  if (max_nb > up::kMaxBlocksPerRequest)
    return up::set_error(UP_ERR_UNSUPPORTED, "%lld blocks in one request > %d",
                         (long long)max_nb, up::kMaxBlocksPerRequest);
  st = up::check_device();
  if (st != UP_OK) return st;
  int np = 1;
  while (np < max_nb) np <<= 1;
  const size_t lds = (size_t)np * sizeof(uint64_t);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(up::up_select_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(up::kMaxBlocksPerRequest * sizeof(uint64_t)));
    (void)hipGetLastError();
    attr_set = true;
  }
  up::SelectArgs a{cu_seqlens_d, cu_blocks_d, block_scores, block_mask, kept_tokens,
                   block, sink, tail, top_p};
  hipLaunchKernelGGL(up::up_select_kernel, dim3((unsigned)num_seqs), dim3(up::kSelectThreads), lds,
                     stream, a);
  return up::check_launch("up_select_kernel");
}
