/*
 * uniprefill.h — C ABI of the UniPrefill token-block pruning hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * Method source: the UniPrefill article page
 * "中国科学院与腾讯微信合作解决AI排队等待问题" (CAS Institute of Automation, UCAS
 * and Tencent WeChat; arXiv 2605.06221).  Section marks (§二, §三, Q&A 1)
 * refer to that page.
 *
 * One pass of the path over a packed batch of B requests:
 *   up_score        tail-query importance scores, per-token and per-block
 *   up_select_topp  Top-p block mask with forced sink / tail blocks
 *   up_compact      gather of the kept rows + positions, new cu_seqlens
 *                   (up_compact_status: its workspace's status bits)
 *   up_drop_history append (layer id, kept tokens) to each request's ledger
 * and, around it,
 *   up_kv_len       per-layer KV length read back from the ledger
 *   up_revive       scatter of packed kept rows back into the full buffer
 * and, fused:
 *   up_score_select     up_score + up_select_topp, selecting in the block-mean kernel
 *   up_compact_record   up_compact + up_drop_history, appending in the copy kernel
 * and, fused into the next layer's first reads (no compacted copy),
 *   up_compact_rmsnorm  normalised input operand of the kept rows
 *   up_gather_add       residual sum with the residual read from frozen rows
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Packing.   Request r owns tokens cu_seqlens[r] .. cu_seqlens[r+1]-1 of a
 *            packed token axis of length T = cu_seqlens[B]; cu_seqlens is
 *            int32, non-decreasing, cu_seqlens[0] == 0.  Its blocks of
 *            `block` (G) consecutive tokens are request-local, the last one
 *            possibly shorter; block-indexed arrays are packed the same way
 *            with cu_blocks[r+1]-cu_blocks[r] = ceil(L_r / G) (see
 *            up_make_cu_blocks).  Most calls take both the host copy (`_h`,
 *            used to validate and to size the launch) and the device copy
 *            (`_d`, read by the kernels); the two must hold the same values.
 * Memory.    Every buffer is owned by the caller.  Pointers named `_h` are
 *            host memory; all others are device memory of the current HIP
 *            device.  The library never allocates device memory and keeps no
 *            pointer after a call returns (work still queued on the stream
 *            aside).
 * Streams.   Calls only enqueue work on `stream` (a hipStream_t; 0 is the
 *            null stream) and never synchronise.  Results are valid once the
 *            stream reaches them.  Calls that share a workspace or ledger
 *            must not overlap.
 * Layout.    Row-major with a contiguous last dimension; strides are in
 *            elements unless the name says bytes.
 * Errors.    Every entry point returns an up_status and never aborts.
 *            Arguments are checked on the host before anything is enqueued;
 *            on failure nothing is enqueued and up_last_error() (a
 *            thread-local string) says why.  UP_ERR_HIP reports a launch
 *            failure returned by the HIP runtime.
 */
#ifndef UNIPREFILL_H
#define UNIPREFILL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UP_ABI_VERSION 1

typedef enum up_status {
  UP_OK = 0,
  UP_ERR_INVALID = 1,     /* bad argument (null pointer, bad size, bad packing) */
  UP_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement      */
  UP_ERR_WORKSPACE = 3,   /* workspace smaller than the *_workspace_size query */
  UP_ERR_CAPACITY = 4,    /* output capacity smaller than the worst case       */
  UP_ERR_HIP = 5          /* the HIP runtime reported an error                 */
} up_status;

/* Element type of the entry points that compute on row elements (the
 * compaction and revival copies move bytes and take no element type).  They
 * take it as an int holding one of these values, so an out-of-range value is
 * rejected (UP_ERR_INVALID) rather than read as an enum. */
typedef enum up_dtype {
  UP_DTYPE_BF16 = 0,
  UP_DTYPE_F16 = 1,
  UP_DTYPE_F32 = 2
} up_dtype;

/* ABI version of the loaded library (UP_ABI_VERSION of its build). */
int up_abi_version(void);

/* Message for the last failing call on this thread ("" if none). */
const char* up_last_error(void);

/* Static name of a status code. */
const char* up_status_string(int status);

/*
 * Host helper: block offsets of a packed batch.
 * cu_blocks_h[0] = 0, cu_blocks_h[r+1] = cu_blocks_h[r] + ceil(L_r / block).
 * cu_seqlens_h: host int32 [num_seqs+1]; cu_blocks_h: host int32 [num_seqs+1]
 * (written).  *num_blocks receives N = cu_blocks_h[num_seqs].
 * Errors: UP_ERR_INVALID for null pointers, num_seqs < 0, block < 1 or
 * non-monotone cu_seqlens_h.
 */
up_status up_make_cu_blocks(int num_seqs, const int32_t* cu_seqlens_h, int block,
                            int32_t* cu_blocks_h, int64_t* num_blocks);

/* ------------------------------------------------------------------------ */
/* Steps 1-3: tail-query importance scores (§二 steps 1-2, §三)              */
/* ------------------------------------------------------------------------ */

/*
 * Workspace bytes up_score needs for this batch and shape.
 */
up_status up_score_workspace_size(int num_seqs, const int32_t* cu_seqlens_h, int hq, int hkv,
                                  int head_dim, int n_query, size_t* bytes);

/*
 * up_score — importance estimation (§二 step 1: the last n tokens of each
 * request query every key of the request; §三: scores, online normalisation,
 * block aggregation) and block means (§二 step 2).
 *
 * For request r of length L, n_eff = min(n_query, L) tail rows
 * i in [L-n_eff, L) (request-local), query head h and KV head
 * g = h / (hq/hkv):
 *     p[h,i,j] = exp(s[h,i,j]) / sum_{j' <= i} exp(s[h,i,j']),
 *     s[h,i,j] = scale * <q[i,h,:], k[j,g,:]>        for keys j <= i,
 *     token_scores[j] = sum_h sum_i p[h,i,j],
 *     block_scores[b] = mean of token_scores over block b's tokens.
 * So each request's token scores sum to hq * n_eff.
 *
 * q      bf16 [T, hq, head_dim]; element (t, h, c) at q[t*q_tok_stride +
 *        h*q_head_stride + c].  Only the n_eff tail rows of each request are
 *        read.  q and both strides must be 16-byte / 8-element aligned.
 * k      bf16 [T, hkv, head_dim], same convention; every row is read.
 *        k_tok_stride <= 2^24 elements (UP_ERR_UNSUPPORTED otherwise).
 * head_dim  64, 128 or 256.    hq % hkv == 0, 1 <= hq <= 1024.
 * n_query   tail queries n, 1..4096.   block  G, a power of two in [16, 256].
 * scale  softmax scale; 0 selects 1/sqrt(head_dim).
 * token_scores  fp32 [T] or NULL.    block_scores  fp32 [N].
 * cu_blocks_d   device int32 [B+1] from up_make_cu_blocks (same block).
 * workspace     device, >= up_score_workspace_size bytes, 256-byte aligned.
 * Deterministic: no floating-point atomics; repeated calls give identical
 * bits.  Calling it on a subset of heads (q/k offset, local hq/hkv) gives
 * partial scores whose sum over disjoint subsets is the full score, up to
 * fp32 rounding (§三: per-device scores are summed before selection).
 */
up_status up_score(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                   const int32_t* cu_blocks_d,
                   const void* q, int64_t q_tok_stride, int64_t q_head_stride, int hq,
                   const void* k, int64_t k_tok_stride, int64_t k_head_stride, int hkv,
                   int head_dim, int n_query, int block, float scale,
                   float* token_scores, float* block_scores,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Step 4: Top-p block selection (§二 step 2, Q&A 1, §三 binary mask)         */
/* ------------------------------------------------------------------------ */

/*
 * up_select_topp — for each request: blocks overlapping the first `sink` or
 * the last `tail` tokens are forced; with total = sum of the request's block
 * scores, the remaining blocks are added in (score desc, index asc) order
 * while the kept mass (forced blocks included) is below top_p * total.
 * The result is the smallest block set that contains the forced blocks and
 * holds at least top_p of the mass.
 *
 * block_scores  fp32 [N], finite and >= 0.
 * block_mask    uint8 [N] (written: 1 keep, 0 drop).
 * kept_tokens   int32 [B] (written: tokens in kept blocks).
 * top_p in (0, 1]; sink, tail >= 0; at most 2^24 blocks per request.
 * Masses are summed exactly as 63-bit fixed point relative to the request's
 * largest score (deterministic in any order); a decision can differ from
 * exact real arithmetic only when the cumulative mass lies within
 * N * 2^-(62 - ceil(log2(N+1))) of the largest score from p * total.
 */
up_status up_select_topp(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                         const int32_t* cu_blocks_d, const float* block_scores, int block,
                         double top_p, int sink, int tail,
                         uint8_t* block_mask, int32_t* kept_tokens, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Step 5: compaction (§二 step 3, §三 metadata update)                       */
/* ------------------------------------------------------------------------ */

/* Workspace bytes up_compact needs for this batch (control and status words,
 * one 16-byte copy descriptor per block).
 *
 * The first 256 bytes of a compaction workspace are its control block, uint32
 * words:
 *   [0] scan tile ticket and [1] done counter (zero between calls);
 *   [2] status bits, sticky until read by up_compact_status (bit 0: a
 *       look-back gave up waiting for a predecessor tile, so that call's
 *       cu_seqlens_out and copy offsets are wrong; the copies stay within
 *       out_capacity_rows);
 *   [3] look-back poll limit: polls of one predecessor's status word before
 *       giving up; 0 (what up_compact_workspace_init leaves) selects 2^24;
 *   [4] call epoch, advanced by every call (a tile's status word counts only
 *       with the current epoch, so nothing an earlier call left behind, for
 *       any batch size, is taken for this call's).
 * The rest is per-tile scan state and the copy descriptors. */
up_status up_compact_workspace_size(int num_seqs, const int32_t* cu_seqlens_h, int block,
                                    size_t* bytes);

/*
 * Prepare a compaction workspace once, before its first up_compact call
 * (zeroes workspace_bytes bytes on `stream`).  Every up_compact call leaves
 * the workspace prepared again when it completes (counters zero, epoch
 * advanced), so one workspace serves any number of calls and any batch it is
 * large enough for, in any order of sizes.
 * workspace: 256-byte aligned, >= 256 bytes.
 */
up_status up_compact_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * up_compact — stream compaction of the kept blocks.  Kept tokens keep their
 * order (request, then token); dropped rows are never read.  The input is
 * not modified (the dropped rows stay in place, "frozen", §二 step 3).
 *
 * block_mask       uint8 [N] (nonzero = keep).
 * hidden           [T rows], row t at hidden + t*row_stride_bytes, row_bytes
 *                  bytes each; copied byte for byte (any dtype).
 * positions        int32 [T] or NULL.
 * hidden_out       [out_capacity_rows, row_bytes] contiguous (written).
 * positions_out    int32 [out_capacity_rows] or NULL (written).
 * cu_seqlens_out   int32 [B+1] (written): packing of the kept batch.
 * out_capacity_rows must be >= T (the all-kept case), else UP_ERR_CAPACITY.
 * workspace        >= up_compact_workspace_size bytes, 256-byte aligned,
 *                  prepared by up_compact_workspace_init (and then only
 *                  used by up_compact calls, one at a time).
 * Two kernel launches: a scan that writes each block's output row and
 * cu_seqlens_out — one workgroup for a batch of at most 4096 blocks, else a
 * single-pass decoupled look-back scan (Merrill & Garland 2016) over tiles
 * of 1024 blocks (tiles are claimed in order from an atomic counter, so
 * every predecessor a tile waits on has started; a wait that still exceeds
 * the poll limit gives up and sets status bit 0, read with
 * up_compact_status; the last tile to finish restores the workspace's
 * counters and tile state for the next call), then a copy kernel moves each
 * kept block in 4 KiB pieces (32 KiB of rows when rows are strided).
 */
up_status up_compact(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                     const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                     const void* hidden, int64_t row_bytes, int64_t row_stride_bytes,
                     const int32_t* positions,
                     void* hidden_out, int32_t* positions_out, int32_t* cu_seqlens_out,
                     int64_t out_capacity_rows, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * up_compact_record — up_compact followed by up_drop_history in one call of
 * two launches (§二 step 3 and §三: the compaction and its ledger entry, the
 * metadata update of the same step).  Arguments: those of up_compact, then
 * the ledger, its capacity and the layer id as for up_drop_history.  The
 * copy kernel's first workgroup appends every request's (layer_id, kept
 * tokens) entry from the cu_seqlens_out the scan wrote; a batch with no
 * blocks appends through the ledger kernel instead.  Outputs (rows,
 * positions, cu_seqlens_out, ledger words and status bits) are identical to
 * up_compact then up_drop_history with the same arguments.
 * ledger     device int32, as for up_drop_history (not NULL).
 * capacity   >= 1 (UP_ERR_INVALID otherwise).
 */
up_status up_compact_record(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                            const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                            const void* hidden, int64_t row_bytes, int64_t row_stride_bytes,
                            const int32_t* positions, void* hidden_out, int32_t* positions_out,
                            int32_t* cu_seqlens_out, int64_t out_capacity_rows, void* workspace,
                            size_t workspace_bytes, void* ledger, int capacity, int layer_id,
                            hipStream_t stream);

/*
 * up_compact_noalloc — up_compact without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, outputs
 * and kernels as up_compact, except:
 * - the scan's control block, tile status words and copy descriptors live in
 *   a device array inside the library (about 8 MiB, held by every GPU the
 *   library runs on until the process ends); the call allocates nothing;
 * - at most 2^19 blocks per call (UP_ERR_CAPACITY beyond that);
 * - every call on one GPU shares that array, so calls that overlap on one GPU
 *   (different streams without ordering) race; order them;
 * - status   device int32 [1] or NULL: receives the array's status bits
 *            accumulated since the last call that passed one (bit 0: a
 *            look-back gave up, as for up_compact_status) and clears them.
 * The first call on a device looks up the array's device address and clears
 * its control words with a kernel on `stream`.
 */
up_status up_compact_noalloc(int num_seqs, const int32_t* cu_seqlens_h,
                             const int32_t* cu_seqlens_d, const int32_t* cu_blocks_d, int block,
                             const uint8_t* block_mask, const void* hidden, int64_t row_bytes,
                             int64_t row_stride_bytes, const int32_t* positions, void* hidden_out,
                             int32_t* positions_out, int32_t* cu_seqlens_out,
                             int64_t out_capacity_rows, int32_t* status, hipStream_t stream);

/*
 * up_compact_status — the status bits of a compaction workspace (control word
 * 2: bit 0 = a look-back gave up, see up_compact_workspace_size) as left by
 * the calls enqueued before it on `stream` (up_compact, up_revive and the
 * fused row operations share the scan).  The page requires the metadata
 * update to be exact (§三), so a caller that must be sure checks this word.
 * status   device int32 [1] (written).
 * clear    nonzero: also clear the bits (the word keeps accumulating
 *          otherwise).
 */
up_status up_compact_status(void* workspace, size_t workspace_bytes, int32_t* status, int clear,
                            hipStream_t stream);

/*
 * up_set_copy_events — measurement aid.  While set, every call that runs the
 * compaction copy kernel (up_compact, up_compact_record, up_compact_noalloc,
 * up_revive) records `start` on its stream immediately before enqueuing that
 * kernel and `stop` immediately after it, so hipEventElapsedTime(start, stop)
 * times the copy kernel alone (the scan before it excluded).  Per host
 * thread; NULL, NULL clears it (both or neither must be NULL, else
 * UP_ERR_INVALID).  The events are the caller's (created on the device the
 * calls run on, kept valid while set); a failed record returns UP_ERR_HIP.
 */
up_status up_set_copy_events(hipEvent_t start, hipEvent_t stop);

/* ------------------------------------------------------------------------ */
/* Step 5 (cont.): drop-history ledger (§三)                                  */
/* ------------------------------------------------------------------------ */

/*
 * Ledger layout (int32 words, device memory):
 *   [0] status bits (bit 0: an append found a request's record full;
 *       bit 1: a call found a ledger set up for another num_seqs/capacity)
 *   [1] num_seqs   [2] capacity   [3] reserved
 *   [4 + r]                          entries used by request r
 *   [4 + B + 2*(r*capacity + e)]     entry e of request r: layer id
 *   [4 + B + 2*(r*capacity + e) + 1]                       kept tokens
 */
size_t up_history_bytes(int num_seqs, int capacity);

/* Clear a ledger (header written, all counts zero).  capacity >= 1. */
up_status up_history_init(void* ledger, int num_seqs, int capacity, hipStream_t stream);

/*
 * up_drop_history — for every request r append (layer_id,
 * cu_seqlens_out[r+1] - cu_seqlens_out[r]) to its record (§三: each drop
 * records the layer and the number of kept tokens).  A full record keeps its
 * entries, drops the new one and sets status bit 0.
 */
up_status up_drop_history(void* ledger, int num_seqs, int capacity, int layer_id,
                          const int32_t* cu_seqlens_out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Consumers of the ledger and of the frozen rows (§三, §二 step 3)            */
/* ------------------------------------------------------------------------ */

/*
 * up_kv_len — KV length of every request for layer layer_id, read back from
 * the ledger (§三: at generation time the ledger tells each layer how many
 * cache entries it holds).  Reading: a drop at layer l already applies to
 * layer l, so kv_len[r] is the kept count of the latest-appended entry of
 * request r whose layer id is <= layer_id, else the prompt length
 * cu_seqlens[r+1] - cu_seqlens[r].
 * ledger        as written by up_history_init / up_drop_history (status bit
 *               1 is set, and prompt lengths written, if its num_seqs or
 *               capacity differ from the arguments).
 * cu_seqlens_d  device int32 [B+1], the prompt packing.
 * kv_len        device int32 [B] (written).
 */
up_status up_kv_len(void* ledger, int num_seqs, int capacity, int layer_id,
                    const int32_t* cu_seqlens_d, int32_t* kv_len, hipStream_t stream);

/*
 * up_revive — revival of frozen tokens (§二 step 3: dropped tokens are kept
 * aside, frozen, so they can be brought back).  The inverse of up_compact's
 * gather for the same mask: row i of `packed` (the i-th kept token in
 * request-then-token order, as up_compact wrote it, possibly updated since)
 * is written to its own row of `full`; rows of dropped blocks keep their
 * (frozen) contents, so `full` holds a complete sequence again.
 * block, block_mask, cu_*  as for up_compact.
 * packed     [kept rows, row_bytes] contiguous (read); must not overlap full.
 * full       [T rows], row t at full + t*row_stride_bytes, row_bytes bytes
 *            each (kept rows written in place).
 * workspace  a prepared up_compact workspace of at least
 *            up_compact_workspace_size bytes; calls sharing it run one at a
 *            time (it is left prepared again).
 * Two launches: up_compact's scan (without cu_seqlens_out) and its copy
 * kernel with source and destination swapped.
 */
up_status up_revive(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                    const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                    const void* packed, void* full, int64_t row_bytes, int64_t row_stride_bytes,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Fused pipeline: selection inside the block-mean kernel (§三)             */
/* ------------------------------------------------------------------------ */

/*
 * up_score_select — up_score followed by up_select_topp in one call of
 * three launches (§三: scores, block aggregation and the binary mask without
 * a round trip): the two scoring passes, then one kernel that computes the
 * token and block scores and, in the workgroup that writes a request's last
 * block mean, selects that request's blocks.
 * Outputs are bit-identical to up_score then up_select_topp with the same
 * arguments (same sums in the same order; the same selection code on the
 * same block scores).  Arguments: those of up_score, then those of
 * up_select_topp.  The workspace is up_score's (it holds the arrival
 * counters, reset by every call; calls sharing a workspace run one at a
 * time).  Requests with no tokens get kept_tokens 0.  At most 2^24 blocks
 * per request, as for up_select_topp.
 */
up_status up_score_select(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                          const int32_t* cu_blocks_d, const void* q, int64_t q_tok_stride,
                          int64_t q_head_stride, int hq, const void* k, int64_t k_tok_stride,
                          int64_t k_head_stride, int hkv, int head_dim, int n_query, int block,
                          float scale, float* token_scores, float* block_scores, double top_p,
                          int sink, int tail, uint8_t* block_mask, int32_t* kept_tokens,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Fused pipeline: the next layer reads the kept rows itself (§二 step 3)    */
/* ------------------------------------------------------------------------ */
/*
 * Later layers work on the kept tokens only while the dropped ones stay
 * frozen in place (§二 step 3).  The first reads of the next layer are its
 * input normalisation and, at its end, the residual that its output is
 * added to.  These two calls perform those reads straight from the frozen
 * buffer through the compaction's row map, so no compacted copy of the
 * hidden states has to be written and read back: the gather costs the kept
 * rows' read only (the normalised operand and the residual sum are written
 * by the next layer in any case).  Reading: the next layer is pre-norm with
 * an RMS normalisation, as in the models the page evaluates.
 *
 * Both take the packing arguments of up_compact (block, block_mask, cu_*),
 * share its workspace (prepared by up_compact_workspace_init, one call at a
 * time) and run its scan first; rows are `hidden_dim` elements of `dtype`,
 * a multiple of 16 bytes and at most 16 KiB; every row buffer is 16-byte
 * aligned and strides are in elements (multiples of 16 bytes); otherwise
 * UP_ERR_UNSUPPORTED.  Arithmetic is fp32; results are rounded to dtype
 * (nearest even).  Two launches each: the scan, then one wave per row.
 */

/*
 * up_compact_rmsnorm — the next layer's normalised input operand for the
 * kept tokens, read from the frozen rows:
 *   normed_out[i] = hidden[t_i] / sqrt(mean_k hidden[t_i][k]^2 + eps) * gamma
 * where t_i is the i-th kept token (request, then token order), plus the
 * kept positions and cu_seqlens_out exactly as up_compact writes them.
 * hidden        [T rows], row t at hidden + t*row_stride (elements).
 * gamma         [hidden_dim] of dtype, or NULL for a gain of 1.
 * eps           >= 0 (an all-zero row with eps = 0 gives NaN, as the formula).
 * normed_out    [out_capacity_rows, hidden_dim] contiguous (written).
 * residual_out  [out_capacity_rows, hidden_dim] contiguous, or NULL: when set,
 *               also receives the kept rows unchanged (the compacted copy).
 * positions, positions_out, cu_seqlens_out, out_capacity_rows  as up_compact.
 */
up_status up_compact_rmsnorm(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                             const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                             int dtype, const void* hidden, int64_t hidden_dim,
                             int64_t row_stride, const void* gamma, float eps,
                             const int32_t* positions, void* normed_out, void* residual_out,
                             int32_t* positions_out, int32_t* cu_seqlens_out,
                             int64_t out_capacity_rows, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * up_gather_add — the next layer's residual sum for the kept tokens, with
 * the residual read from the frozen rows:
 *   out[i] = frozen[t_i] + delta[i]     (i over the kept tokens)
 * frozen   [T rows], row t at frozen + t*row_stride (elements).
 * delta    [out_rows, hidden_dim] contiguous, e.g. the layer's output
 *          projection of the rows up_compact_rmsnorm normalised.
 * out      [out_rows, hidden_dim] contiguous (written); may be the same
 *          buffer as delta (in-place residual add), must not overlap frozen.
 * out_rows should be >= the number of kept tokens (cu_seqlens_out[B] of the
 *          same mask); a kept block that would end past out_rows is skipped,
 *          so nothing is read or written beyond out_rows.
 */
up_status up_gather_add(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                        const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                        int dtype, const void* frozen, int64_t hidden_dim, int64_t row_stride,
                        const void* delta, void* out, int64_t out_rows, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* UNIPREFILL_H */
