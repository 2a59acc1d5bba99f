// Step 4 of the pruning path: Top-p block selection with forced blocks, one
// workgroup per request (the rule and the algorithm are described in
// up_select_impl.h, which the block-mean kernel of the fused entry point
// shares).
#include "up_select_impl.h"

namespace up {
namespace {

__global__ void __launch_bounds__(kSelectThreads) up_select_kernel(SelectArgs a) {
  __shared__ SelectShared<kSelectThreads, kStageMax> sh;
  select_request(a, blockIdx.x, sh);
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
    return up::set_error(UP_ERR_UNSUPPORTED, "%lld blocks in one request > %lld",
                         (long long)max_nb, (long long)up::kMaxBlocksPerRequest);
  st = up::check_device();
  if (st != UP_OK) return st;
  up::SelectArgs a{cu_seqlens_d, cu_blocks_d, block_scores, block_mask, kept_tokens,
                   block, sink, tail, top_p};
  hipLaunchKernelGGL(up::up_select_kernel, dim3((unsigned)num_seqs), dim3(up::kSelectThreads), 0,
                     stream, a);
  return up::check_launch("up_select_kernel");
}
