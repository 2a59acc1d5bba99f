// Step 5 of the pruning path: stream compaction and the drop-history ledger.
//
// Method (UniPrefill page "中国科学院与腾讯微信合作解决AI排队等待问题", §二 step 3 and
// §三): tokens of dropped blocks are skipped by every later layer, so the
// kept rows (hidden states and positions) are gathered into a packed batch
// with updated per-request lengths, and each drop appends (layer id, kept
// tokens) to the request's drop-history ledger.
//
// up_compact is two kernels.
//   up_compact_scan_kernel   a batch of at most 4096 blocks is one tile that
//     one 1024-thread workgroup scans alone; larger ones run a single-pass
//     decoupled look-back scan (Merrill &
//     Garland, "Single-pass Parallel Prefix Scan with Decoupled Look-back",
//     2016) over tiles of 1024 blocks: each workgroup claims the next tile
//     from an atomic ticket (so every tile it may wait on has already
//     started), publishes its kept-token count, walks back over its
//     predecessors' published counts to get its output offset, publishes the
//     inclusive count, and writes one copy descriptor per block (destination
//     row, source row, rows) plus cu_seqlens_out.  Every status word carries
//     its state and its count in one 64-bit atomic and no tile reads data
//     another tile wrote, so relaxed device-scope atomics are enough:
//     release/acquire at device scope would write back / invalidate the XCD's
//     L2 on every publish and poll.  The last workgroup to finish (a done
//     counter) clears the status words and both counters, so the next call
//     starts from a clean workspace without a separate clearing launch.
//   up_compact_copy_kernel   one workgroup per (block, 4 KiB piece): a kept
//     block is a run of G consecutive rows, copied as one flat byte range with
//     16-byte non-temporal loads and stores; dropped rows are never read.
// Splitting the gather from the scan lets the copy use small, uniform work
// items (the shape a plain device copy runs fastest with) instead of one
// workgroup per scan tile.  up_compact_record is up_compact whose copy kernel
// also appends the ledger entries (workgroup 0, before its piece), so the
// step needs no separate ledger launch.
#include <math.h>

#include <initializer_list>
#include <mutex>

#include "up_internal.h"
#include "up_wave.h"

namespace up {
namespace {

constexpr int kCompactThreads = 256;
constexpr int kScanPerThread = 4;
constexpr int kScanTileBlocks = kCompactThreads * kScanPerThread;  // blocks per scan tile
// Batches of at most kScan1Blocks blocks are scanned by one workgroup of
// kScan1Threads threads (one tile, nothing to look back on).
constexpr int kScan1Threads = 1024;
constexpr int kScan1Blocks = kScan1Threads * kScanPerThread;
// Copy work items: 4 KiB per 128-thread workgroup, one 16-byte vector in
// flight per lane (two rounds).  Many short-lived workgroups keep more HBM
// requests in flight across the chip than fewer long ones.  Per up_compact
// call at L = 131072, D = 4096 bf16 (16-request batch in brackets): 128 x 4 KiB
// 341 us (1376), 128 x 2 KiB 372, 128 x 4 KiB with both vectors in flight 352,
// 64 x 4 KiB 348 (1421), 64 x 2 KiB 348 (1406), 256 x 8 KiB 358 (1462),
// 256 x 32 KiB with four vectors in flight 377 (1663), 512 x 16 KiB 380 (1590).
#ifndef UP_PIECE_KIB
#define UP_PIECE_KIB 4
#endif
#ifndef UP_COPY_UNROLL
#define UP_COPY_UNROLL 1
#endif
constexpr int64_t kPieceBytes = (int64_t)UP_PIECE_KIB << 10;       // bytes per copy work item
constexpr int64_t kRowPieceBytes = 32 << 10;  // per work item when rows are strided (a wave per row)
#ifndef UP_COPY_THREADS
#define UP_COPY_THREADS 128
#endif
constexpr int kCopyThreads = UP_COPY_THREADS;  // threads per copy workgroup
// Tile status word: state in bits 63..62 (1 = aggregate, 2 = inclusive
// prefix), the call's epoch in bits 61..31, the count in bits 30..0 (counts
// are at most T < 2^31).  A word counts as published only with a state of 1
// or 2 and this call's epoch, so nothing left in the status-word region by
// earlier calls reads as published: their status words carry an older epoch,
// and copy descriptors that a call with fewer tiles wrote there decode to
// state 0 or 3 (their upper halves are a row count, a non-negative row or
// -1).
constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagIncl = 2ull << 62;
constexpr int kEpochShift = 31;
constexpr uint64_t kEpochMask = (1ull << 31) - 1;
constexpr uint64_t kValueMask = (1ull << 31) - 1;
// Polls of one predecessor's status word before a look-back gives up (when
// control word 3 is 0).  Tiles are claimed in ticket order, so every
// predecessor has started and publishes within a few microseconds; the
// limit only bounds the wait if one never does.
constexpr uint32_t kSpinLimit = 1u << 24;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Copy descriptor of one block: dst < 0 marks a dropped block (or one that
// would not fit the output capacity).
struct __attribute__((aligned(16))) BlockCopy {
  int64_t dst;  // first output row
  int32_t src;  // first input row
  int32_t rows;
};
static_assert(sizeof(BlockCopy) == 16, "descriptor is one 16-byte load");

struct CompactArgs {
  const int32_t* cu_seqlens;
  const int32_t* cu_blocks;
  const uint8_t* mask;
  const char* hidden;
  const int32_t* positions;
  char* hidden_out;
  int32_t* positions_out;
  int32_t* cu_out;    // NULL: not written (revival)
  uint64_t* flags;    // [num_tiles] scan tile status words
  uint32_t* ctl;      // [0] tile ticket, [1] done counter, [2] status bits, [3] poll limit, [4] epoch
  BlockCopy* desc;    // [num_blocks]
  int64_t row_bytes, row_stride, capacity, num_blocks, num_tiles;
  int64_t pieces;      // copy work items per block
  int64_t piece_bytes; // bytes per work item when rows are packed
  int64_t piece_rows;  // rows per work item when rows are strided
  int num_seqs, block;
  int32_t* ledger;     // NULL, or the drop-history ledger the copy kernel appends to
  int led_capacity, layer_id;
};

// Status bit of control word 2: a look-back gave up on a predecessor tile.
constexpr uint32_t kStatusLookbackGaveUp = 1u;

// Zero a whole compaction workspace (control words and tile status words).
__global__ void up_compact_init_kernel(uint32_t* ws, int64_t nwords) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nwords) ws[i] = 0;
}

// Copy the status bits of a compaction workspace, optionally clearing them.
__global__ void up_compact_status_kernel(uint32_t* ctl, int32_t* out, int clear) {
  if (threadIdx.x == 0) {
    out[0] = (int32_t)ctl[2];
    if (clear) ctl[2] = 0;
  }
}

// Request owning block b: the last r with cu_blocks[r] <= b.
__device__ __forceinline__ int block_request(const int32_t* cu_blocks, int num_seqs, int64_t b) {
  int lo = 0, hi = num_seqs;  // cu_blocks[lo] <= b < cu_blocks[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_blocks[mid] <= b) lo = mid; else hi = mid;
  }
  return lo;
}

// NTH threads, kScanPerThread blocks each, per tile.  ONE: the whole batch
// is one tile of one workgroup (at most kScan1Blocks blocks), so there is no
// ticket, no look-back and no done counter; that form leaves the control
// words and the tile status words untouched (it writes descriptors and
// cu_seqlens_out only), which keeps the workspace as prepared.
template <int NTH, bool ONE>
__global__ void __launch_bounds__(NTH) up_compact_scan_kernel(CompactArgs a) {
  constexpr int kTileBlocks = NTH * kScanPerThread;
  __shared__ int64_t s_tile;
  __shared__ int64_t s_excl;
  __shared__ int64_t s_wave[NTH / 64];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (!ONE) {
    if (tid == 0) s_tile = (int64_t)atomicAdd(&a.ctl[0], 1u);
    __syncthreads();
  }
  const int64_t t = ONE ? 0 : s_tile;
  const uint32_t poll_limit = a.ctl[3] ? a.ctl[3] : kSpinLimit;
  // This call's epoch: the last workgroup advances it only after every
  // workgroup of the call has counted itself done, so all read one value.
  const uint64_t epoch = a.ctl[4] & kEpochMask;
  const uint64_t tag = epoch << kEpochShift;

  if (t == 0 && tid == 0 && a.cu_out) {
    // Output packing starts at 0; requests with no blocks before the first
    // block end at 0 as well.
    a.cu_out[0] = 0;
    for (int r = 0; r < a.num_seqs && a.cu_blocks[r + 1] == 0; ++r) a.cu_out[r + 1] = 0;
  }

  if (ONE || t < a.num_tiles) {
    // This thread's blocks: kScanPerThread consecutive ones.
    const int64_t b0 = t * kTileBlocks + (int64_t)tid * kScanPerThread;
    int req[kScanPerThread], rows[kScanPerThread], src[kScanPerThread];
    bool ends[kScanPerThread];
    int64_t kept[kScanPerThread];
    int64_t mine = 0;
    if (b0 < a.num_blocks) {
      // The mask bytes and the first block's request bounds are loaded
      // together (one round trip); a thread's blocks rarely cross a request
      // boundary, and only then does it load the next request's bounds.
      int r = block_request(a.cu_blocks, a.num_seqs, b0);
      int cb_lo = a.cu_blocks[r], cb_hi = a.cu_blocks[r + 1];
      int s_lo = a.cu_seqlens[r], s_hi = a.cu_seqlens[r + 1];
      uint8_t mk[kScanPerThread];
      if (b0 + kScanPerThread <= a.num_blocks) {  // straight-line loads, one wait
#pragma unroll
        for (int i = 0; i < kScanPerThread; ++i) mk[i] = a.mask[b0 + i];
      } else {
#pragma unroll
        for (int i = 0; i < kScanPerThread; ++i) mk[i] = b0 + i < a.num_blocks ? a.mask[b0 + i] : 0;
      }
#pragma unroll
      for (int i = 0; i < kScanPerThread; ++i) {
        const int64_t b = b0 + i;
        req[i] = -1;
        rows[i] = 0;
        src[i] = 0;
        ends[i] = false;
        kept[i] = 0;
        if (b < a.num_blocks) {
          while (cb_hi <= b) {  // skip to the owning request
            ++r;
            cb_lo = cb_hi;
            cb_hi = a.cu_blocks[r + 1];
            s_lo = s_hi;
            s_hi = a.cu_seqlens[r + 1];
          }
          const int lb = (int)(b - cb_lo);
          req[i] = r;
          rows[i] = min(lb * a.block + a.block, s_hi - s_lo) - lb * a.block;
          src[i] = s_lo + lb * a.block;
          ends[i] = b == cb_hi - 1;
          kept[i] = mk[i] ? rows[i] : 0;
          mine += kept[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kScanPerThread; ++i) {
        req[i] = -1;
        rows[i] = 0;
        src[i] = 0;
        ends[i] = false;
        kept[i] = 0;
      }
    }
    // Exclusive scan of the threads' kept rows: waves, then across waves.
    const int64_t incl = (int64_t)wave_scan_incl((uint64_t)mine);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int64_t wbase = 0, agg = 0;
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) {
      if (w < wave) wbase += s_wave[w];
      agg += s_wave[w];
    }

    if (ONE) {
      if (tid == 0) s_excl = 0;
    } else if (wave == 0) {
      // Publish this tile's count, then look back a window of 64
      // predecessors per round trip: lane i reads tile (hi - i); the nearest
      // tile that already has an inclusive prefix ends the walk.
      if (lane == 0)
        __hip_atomic_store(&a.flags[t], (t == 0 ? kFlagIncl : kFlagAgg) | tag | (uint64_t)agg,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int64_t excl = 0;
      if (t > 0) {
        int64_t hi = t - 1;
        for (;;) {
          const int64_t p = hi - lane;
          uint64_t f = kFlagIncl | tag;  // before tile 0: an inclusive prefix of 0
          uint32_t state = 2;
          if (p >= 0) {
            int spins = 0;
            for (;;) {
              f = __hip_atomic_load(&a.flags[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              state = (uint32_t)(f >> 62);
              if (state == 3 || ((f >> kEpochShift) & kEpochMask) != epoch) state = 0;
              if (state != 0 || (uint32_t)++spins >= poll_limit) break;
              __builtin_amdgcn_s_sleep(1);
            }
          }
          const uint64_t incl_lanes = __ballot(state == 2);
          const int stop = incl_lanes ? __ffsll((unsigned long long)incl_lanes) - 1 : 63;
          // a predecessor that never published counts as 0 rows: the
          // offsets are wrong, so the call's status records it
          if (lane <= stop && state == 0) atomicOr(&a.ctl[2], kStatusLookbackGaveUp);
          const uint64_t v = (lane <= stop && state != 0) ? (f & kValueMask) : 0;
          excl += (int64_t)wave_sum(v);
          if (incl_lanes) break;
          hi -= 64;
        }
        if (lane == 0)
          __hip_atomic_store(&a.flags[t], kFlagIncl | tag | (uint64_t)(excl + agg),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (lane == 0) s_excl = excl;
    }
    __syncthreads();

    // Descriptors and request ends.
    int64_t pos = s_excl + wbase + incl - mine;  // this thread's first output row
#pragma unroll
    for (int i = 0; i < kScanPerThread; ++i) {
      const int64_t b = b0 + i;
      if (req[i] < 0) continue;
      const int rq = req[i];
      BlockCopy d;
      d.dst = (kept[i] > 0 && pos + kept[i] <= a.capacity) ? pos : -1;  // never past the output
      d.src = src[i];
      d.rows = rows[i];
      a.desc[b] = d;
      pos += kept[i];
      // A request whose last block this is (and empty requests right after
      // it) ends at this block's inclusive count.
      if (a.cu_out && ends[i]) {
        a.cu_out[rq + 1] = (int32_t)pos;
        for (int r2 = rq + 1; r2 < a.num_seqs && a.cu_blocks[r2 + 1] == a.cu_blocks[rq + 1]; ++r2)
          a.cu_out[r2 + 1] = (int32_t)pos;
      }
    }
  }

  if (ONE) return;
  // Done counter: the last workgroup leaves the tile status words and the
  // two counters zeroed and advances the epoch for the next call (every
  // other workgroup has finished its look-back before it counted itself
  // done).  The status bits (word 2) stay until up_compact_status reads and
  // clears them, and the poll limit (word 3) is the caller's setting.
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.ctl[1], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == gridDim.x - 1) ? 1 : 0;
  }
  __syncthreads();
  if (s_last) {
    for (int64_t i = tid; i < a.num_tiles; i += kCompactThreads) a.flags[i] = 0;
    if (tid == 0) {
      a.ctl[0] = 0;
      a.ctl[1] = 0;
      a.ctl[4] = (uint32_t)((epoch + 1) & kEpochMask);
    }
  }
}

template <int VW> struct Vec;
template <> struct Vec<16> { typedef u32x4_t T; };
template <> struct Vec<8> { typedef u32x2_t T; };
template <> struct Vec<4> { typedef uint32_t T; };
template <> struct Vec<1> { typedef uint8_t T; };

// Copy nbytes (a multiple of VW) from src to dst, whole workgroup,
// UP_COPY_UNROLL vectors in flight per lane.
template <int VW>
__device__ __forceinline__ void copy_flat(char* __restrict__ dst, const char* __restrict__ src,
                                          int64_t nbytes) {
  typedef typename Vec<VW>::T V;
  constexpr int U = UP_COPY_UNROLL;
  const V* s = reinterpret_cast<const V*>(src);
  V* d = reinterpret_cast<V*>(dst);
  const int64_t n = nbytes / VW;
  int64_t i = threadIdx.x;
  for (; i + (U - 1) * kCopyThreads < n; i += U * kCopyThreads) {
    V r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = __builtin_nontemporal_load(s + i + u * kCopyThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(r[u], d + i + u * kCopyThreads);
  }
  for (; i < n; i += kCopyThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

// Copy `rows` rows of row_bytes between row layouts with the given strides,
// one wave per row.
template <int VW>
__device__ __forceinline__ void copy_rows(char* __restrict__ dst, int64_t dst_stride,
                                          const char* __restrict__ src, int64_t src_stride, int rows,
                                          int64_t row_bytes) {
  typedef typename Vec<VW>::T V;
  const int64_t vpr = row_bytes / VW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = wave; r < rows; r += kCopyThreads / 64) {
    const V* s = reinterpret_cast<const V*>(src + (int64_t)r * src_stride);
    V* d = reinterpret_cast<V*>(dst + (int64_t)r * dst_stride);
    for (int64_t c = lane; c < vpr; c += 64) __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
  }
}

// Drop-history ledger words: [0] status bits, [1] num_seqs, [2] capacity,
// [3] reserved, then one entry count per request, then (layer id, kept
// tokens) entries, capacity per request.
constexpr int kLedgerHeader = 4;

// Append (layer, kept tokens of request r) to request r's ledger record.  A
// ledger set up for another shape gets status bit 1 (from r = 0), a full
// record keeps its entries and sets bit 0.
__device__ __forceinline__ void history_append_one(int32_t* led, int num_seqs, int capacity,
                                                   int layer, const int32_t* cu_out, int r) {
  if (led[1] != num_seqs || led[2] != capacity) {  // ledger set up for another shape
    if (r == 0) atomicOr(&led[0], 2);
    return;
  }
  const int cnt = led[kLedgerHeader + r];
  const int kept = cu_out[r + 1] - cu_out[r];
  if (cnt < capacity) {
    int32_t* e = led + kLedgerHeader + num_seqs + 2 * ((int64_t)r * capacity + cnt);
    e[0] = layer;
    e[1] = kept;
    led[kLedgerHeader + r] = cnt + 1;
  } else {
    atomicOr(&led[0], 1);
  }
}

// Work item w = (block w / pieces, piece w % pieces): consecutive workgroups
// copy consecutive pieces of one block, so the streams stay sequential in
// memory.  A grid-stride loop covers batches with more items than one grid.
// With a ledger, workgroup 0 first appends every request's entry from
// cu_seqlens_out (written by the scan, the launch before).
// REVIVE: the same descriptors with source and destination swapped — packed
// rows (hidden_out side) go back to their own rows of the full buffer
// (hidden side); positions are not touched.
template <int VW, bool REVIVE>
__global__ void __launch_bounds__(kCopyThreads) up_compact_copy_kernel(CompactArgs a) {
  if (!REVIVE && a.ledger && blockIdx.x == 0)
    for (int r = threadIdx.x; r < a.num_seqs; r += kCopyThreads)
      history_append_one(a.ledger, a.num_seqs, a.led_capacity, a.layer_id, a.cu_out, r);
  const int64_t items = a.num_blocks * a.pieces;
  for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
    int64_t b, piece;
    if (items <= 0xffffffffll) {  // 32-bit division where it suffices
      const uint32_t q = (uint32_t)w / (uint32_t)a.pieces;
      b = q;
      piece = (uint32_t)w - q * (uint32_t)a.pieces;
    } else {
      b = w / a.pieces;
      piece = w - b * a.pieces;
    }
    // one 16-byte load (the struct's fields would otherwise be fetched by
    // two dependent loads around the early exit)
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(a.desc + b);
    BlockCopy d;
    d.dst = (int64_t)(((uint64_t)raw[1] << 32) | raw[0]);
    d.src = (int32_t)raw[2];
    d.rows = (int32_t)raw[3];
    if (d.dst < 0) continue;  // uniform over the workgroup
    char* packed = a.hidden_out + d.dst * a.row_bytes;     // packed side, row_bytes apart
    char* strided = const_cast<char*>(a.hidden) + d.src * a.row_stride;  // full side
    if (a.row_stride == a.row_bytes) {
      const int64_t bytes = (int64_t)d.rows * a.row_bytes;
      const int64_t p0 = piece * a.piece_bytes;
      if (p0 < bytes) {
        const int64_t nb = min(a.piece_bytes, bytes - p0);
        if (REVIVE) copy_flat<VW>(strided + p0, packed + p0, nb);
        else copy_flat<VW>(packed + p0, strided + p0, nb);
      }
    } else {
      const int64_t r0 = piece * a.piece_rows;
      if (r0 < d.rows) {
        const int nr = (int)min(a.piece_rows, d.rows - r0);
        if (REVIVE)
          copy_rows<VW>(strided + r0 * a.row_stride, a.row_stride, packed + r0 * a.row_bytes,
                        a.row_bytes, nr, a.row_bytes);
        else
          copy_rows<VW>(packed + r0 * a.row_bytes, a.row_bytes, strided + r0 * a.row_stride,
                        a.row_stride, nr, a.row_bytes);
      }
    }
    if (!REVIVE && a.positions && piece == 0)
      for (int i = threadIdx.x; i < d.rows; i += kCopyThreads)
        a.positions_out[d.dst + i] = a.positions[d.src + i];
  }
}

// ---------------------------------------------------------------------------
// Fused pipeline: the next layer reads the kept rows through the copy
// descriptors instead of a compacted copy.
//   NORM  out[dst + i] = RMSNorm(frozen[src + i]) * gamma   (the next layer's
//         normalised input operand; optionally also the residual copy)
//   ADD   out[dst + i] = frozen[src + i] + delta[dst + i]   (the next layer's
//         residual sum, with the residual gathered from the frozen rows)
// One wave per row: a row of up to 16 KiB is held in registers as 16-byte
// vectors (VPL per lane), its sum of squares reduced over the wave in a fixed
// butterfly order (bitwise reproducible), then scaled and rounded to the
// element type.  A work item is (block, group of 2*U rows): two waves, U rows
// per wave in flight, so each item moves 8-32 KiB like the plain copy's pieces.
// ---------------------------------------------------------------------------
enum { kDtBf16 = 0, kDtF16 = 1, kDtF32 = 2 };
enum { kOpNorm = 0, kOpAdd = 1 };

struct RowOpArgs {
  const BlockCopy* desc;
  int64_t num_blocks;
  int pieces;          // work items per block
  int rows_per_item;   // waves per workgroup * U
  const char* src;     // frozen rows (input), src_stride bytes apart
  int64_t src_stride;
  const char* delta;   // ADD: [kept rows] delta_stride bytes apart
  int64_t delta_stride;
  char* out;           // [kept rows] out_stride bytes apart
  int64_t out_stride;
  char* res_out;       // NORM: residual copy or NULL
  int64_t res_stride;
  const char* gamma;   // NORM: gain [D] or NULL
  const int32_t* positions;
  int32_t* positions_out;
  int64_t nvec;        // 16-byte vectors per row
  float inv_d, eps;
};

template <int DT> struct Elem;
template <> struct Elem<kDtBf16> {
  static constexpr int PER = 8;  // elements per 16-byte vector
  static __device__ __forceinline__ void unpack(u32x4_t v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  // fp32 -> bf16, round to nearest even (finite values; NaN stays NaN)
  static __device__ __forceinline__ uint32_t round1(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  }
  static __device__ __forceinline__ u32x4_t pack(const float (&f)[8]) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = round1(f[2 * i]) | (round1(f[2 * i + 1]) << 16);
    return v;
  }
};
template <> struct Elem<kDtF16> {
  static constexpr int PER = 8;
  static __device__ __forceinline__ void unpack(u32x4_t v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[i] & 0xffffu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[i] >> 16));
    }
  }
  static __device__ __forceinline__ u32x4_t pack(const float (&f)[8]) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * i]);
      const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * i + 1]);
      v[i] = lo | (hi << 16);
    }
    return v;
  }
};
template <> struct Elem<kDtF32> {
  static constexpr int PER = 4;
  static __device__ __forceinline__ void unpack(u32x4_t v, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  static __device__ __forceinline__ u32x4_t pack(const float (&f)[4]) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
};

// Row-operation workgroups of two waves (U rows each in flight): per call at
// L = 131072, D = 4096 bf16, the normalised operand took 360 us and the
// residual sum 530 us, against 373 / 569 us with four waves and 361 / 554 us
// with one (smaller work items, as for the plain copy).
#ifndef UP_ROW_THREADS
#define UP_ROW_THREADS 128
#endif
constexpr int kRowThreads = UP_ROW_THREADS;

template <int OP, int DT, int VPL, int U>
__global__ void __launch_bounds__(kRowThreads) up_rowop_kernel(RowOpArgs a) {
  using E = Elem<DT>;
  constexpr int PER = E::PER;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t items = a.num_blocks * a.pieces;
  for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
    const int64_t b = w / a.pieces;
    const int piece = (int)(w - b * a.pieces);
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(a.desc + b);
    const int64_t dst = (int64_t)(((uint64_t)raw[1] << 32) | raw[0]);
    const int32_t src = (int32_t)raw[2];
    const int32_t rows = (int32_t)raw[3];
    if (dst < 0) continue;  // dropped block (uniform over the workgroup)
    if (OP == kOpNorm && a.positions && piece == 0)
      for (int i = threadIdx.x; i < rows; i += kRowThreads)
        a.positions_out[dst + i] = a.positions[src + i];
    const int r0 = piece * a.rows_per_item + wave * U;
    u32x4_t x[U][VPL], y[U][VPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u;
      if (r >= rows) continue;
      const u32x4_t* s = reinterpret_cast<const u32x4_t*>(a.src + (int64_t)(src + r) * a.src_stride);
      const u32x4_t* d =
          OP == kOpAdd
              ? reinterpret_cast<const u32x4_t*>(a.delta + (int64_t)(dst + r) * a.delta_stride)
              : nullptr;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int64_t c = lane + 64 * v;
        if (c < a.nvec) {
          x[u][v] = __builtin_nontemporal_load(s + c);
          if (OP == kOpAdd) y[u][v] = __builtin_nontemporal_load(d + c);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u;
      if (r >= rows) continue;
      u32x4_t* o = reinterpret_cast<u32x4_t*>(a.out + (int64_t)(dst + r) * a.out_stride);
      if (OP == kOpAdd) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          const int64_t c = lane + 64 * v;
          if (c < a.nvec) {
            float f[PER], g[PER];
            E::unpack(x[u][v], f);
            E::unpack(y[u][v], g);
#pragma unroll
            for (int e = 0; e < PER; ++e) f[e] += g[e];
            __builtin_nontemporal_store(E::pack(f), o + c);
          }
        }
      } else {
        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          if (lane + 64 * v < a.nvec) {
            float f[PER];
            E::unpack(x[u][v], f);
#pragma unroll
            for (int e = 0; e < PER; ++e) ss = fmaf(f[e], f[e], ss);
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        const float rs = rsqrtf(ss * a.inv_d + a.eps);
        // Unpack the row again below instead of keeping every element live
        // as fp32 across the reduction (that would double the registers).
#pragma unroll
        for (int v = 0; v < VPL; ++v) __asm__ volatile("" : "+v"(x[u][v]));
        u32x4_t* ro = a.res_out
                          ? reinterpret_cast<u32x4_t*>(a.res_out + (int64_t)(dst + r) * a.res_stride)
                          : nullptr;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          const int64_t c = lane + 64 * v;
          if (c < a.nvec) {
            float f[PER];
            E::unpack(x[u][v], f);
            if (a.gamma) {
              float g[PER];
              E::unpack(reinterpret_cast<const u32x4_t*>(a.gamma)[c], g);
#pragma unroll
              for (int e = 0; e < PER; ++e) f[e] = f[e] * rs * g[e];
            } else {
#pragma unroll
              for (int e = 0; e < PER; ++e) f[e] = f[e] * rs;
            }
            __builtin_nontemporal_store(E::pack(f), o + c);
            if (ro) __builtin_nontemporal_store(x[u][v], ro + c);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Drop-history ledger.
// ---------------------------------------------------------------------------

__global__ void up_history_init_kernel(int32_t* led, int num_seqs, int capacity) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    led[0] = 0;
    led[1] = num_seqs;
    led[2] = capacity;
    led[3] = 0;
  }
  if (i < num_seqs) led[kLedgerHeader + i] = 0;
}

__global__ void up_history_append_kernel(int32_t* led, int num_seqs, int capacity, int layer,
                                         const int32_t* cu_out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < num_seqs) history_append_one(led, num_seqs, capacity, layer, cu_out, r);
}

// KV length per request for one layer: the kept count of the latest entry
// with layer id <= layer, else the prompt length.  One wave per request; lane
// i looks at entries i, i+64, ...; the wave keeps the largest (layer id,
// entry index) key among entries at or below the layer.
__global__ void __launch_bounds__(256) up_kv_len_kernel(const int32_t* led, int num_seqs,
                                                        int capacity, int layer,
                                                        const int32_t* cu_seqlens, int32_t* kv_len,
                                                        int32_t* status) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= num_seqs) return;
  const int full = cu_seqlens[r + 1] - cu_seqlens[r];
  if (led[1] != num_seqs || led[2] != capacity) {  // ledger set up for another shape
    if (lane == 0) {
      kv_len[r] = full;
      if (r == 0) atomicOr(status, 2);
    }
    return;
  }
  const int cnt = min(led[kLedgerHeader + r], capacity);
  const int32_t* e = led + kLedgerHeader + num_seqs + 2 * (int64_t)r * capacity;
  uint64_t key = 0;  // 0: no entry at or below the layer
  for (int i = lane; i < cnt; i += 64) {
    const int lid = e[2 * i];
    if (lid <= layer) {
      const uint64_t k = (1ull << 63) | ((uint64_t)((uint32_t)lid ^ 0x80000000u) << 31) | (uint64_t)i;
      key = k > key ? k : key;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(key, off);
    key = o > key ? o : key;
  }
  if (lane == 0) kv_len[r] = key ? e[2 * (int)(key & 0x7fffffffu) + 1] : full;
}

}  // namespace

int compact_tile_blocks(int block) {
  (void)block;
  return kScanTileBlocks;
}

}  // namespace up

namespace {

// Workspace: 256 bytes of control words, the scan tiles' status words, then
// one copy descriptor per block.
struct CompactLayout {
  int64_t blocks, tiles;
  size_t off_flags, off_desc, bytes;
};

CompactLayout compact_layout(int num_seqs, const int32_t* cu_h, int block) {
  CompactLayout l{};
  for (int r = 0; r < num_seqs; ++r) l.blocks += up::ceil_div(cu_h[r + 1] - cu_h[r], block);
  l.tiles = up::ceil_div(l.blocks, up::compact_tile_blocks(block));
  l.off_flags = 256;
  l.off_desc = up::align_up(l.off_flags + (size_t)l.tiles * sizeof(uint64_t), 256);
  l.bytes = up::align_up(l.off_desc + (size_t)l.blocks * sizeof(up::BlockCopy), 256);
  return l;
}

// Arguments shared by up_compact and up_revive (the revive call passes the
// full buffer as `hidden` and the packed rows as `hidden_out`).
struct GatherCall {
  int num_seqs;
  const int32_t* cu_h;
  const int32_t* cu_d;
  const int32_t* cu_blocks_d;
  int block;
  const uint8_t* mask;
  const void* hidden;
  int64_t row_bytes, row_stride;
  const int32_t* positions;
  void* hidden_out;
  int32_t* positions_out;
  int32_t* cu_out;
  int64_t capacity;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  int32_t* ledger = nullptr;  // up_compact_record: the ledger to append to
  int led_capacity = 0, layer_id = 0;
};

// Measurement hook (up_set_copy_events): events recorded on the call's stream
// right before and right after the copy kernel is enqueued, per host thread.
thread_local hipEvent_t t_copy_start = nullptr, t_copy_stop = nullptr;

template <bool REVIVE>
void launch_copy(const up::CompactArgs& a, dim3 grid, uintptr_t al, hipStream_t stream) {
  if ((al & 15) == 0)
    hipLaunchKernelGGL((up::up_compact_copy_kernel<16, REVIVE>), grid, dim3(up::kCopyThreads), 0,
                       stream, a);
  else if ((al & 7) == 0)
    hipLaunchKernelGGL((up::up_compact_copy_kernel<8, REVIVE>), grid, dim3(up::kCopyThreads), 0,
                       stream, a);
  else if ((al & 3) == 0)
    hipLaunchKernelGGL((up::up_compact_copy_kernel<4, REVIVE>), grid, dim3(up::kCopyThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((up::up_compact_copy_kernel<1, REVIVE>), grid, dim3(up::kCopyThreads), 0,
                       stream, a);
}

// Validates a gather call, fills the kernel arguments and enqueues the scan
// (descriptors, and cu_seqlens_out when c.cu_out is set).  *ran is false when
// there is nothing to do (no requests).
up_status scan_for(const GatherCall& c, int64_t T, up::CompactArgs* out, bool* ran) {
  *ran = false;
  if (c.block < 1 || c.block > 4096) return up::set_error(UP_ERR_INVALID, "block not in [1, 4096]");
  if (c.row_bytes < 1 || c.row_stride < c.row_bytes)
    return up::set_error(UP_ERR_INVALID, "need row_bytes >= 1 and row_stride_bytes >= row_bytes");
  if (c.row_bytes > ((int64_t)1 << 30))
    return up::set_error(UP_ERR_UNSUPPORTED, "row_bytes above 1 GiB");
  if (!c.cu_d || !c.cu_blocks_d || !c.ws || (T > 0 && !c.mask))
    return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  if ((uintptr_t)c.ws & 255) return up::set_error(UP_ERR_INVALID, "workspace not 256-byte aligned");
  const CompactLayout lay = compact_layout(c.num_seqs, c.cu_h, c.block);
  if (c.ws_bytes < lay.bytes)
    return up::set_error(UP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", c.ws_bytes, lay.bytes);
  if (c.num_seqs == 0) return UP_OK;
  up_status st = up::check_device();
  if (st != UP_OK) return st;

  up::CompactArgs& a = *out;
  a = up::CompactArgs{};
  a.cu_seqlens = c.cu_d;
  a.cu_blocks = c.cu_blocks_d;
  a.mask = c.mask;
  a.hidden = static_cast<const char*>(c.hidden);
  a.positions = c.positions;
  a.hidden_out = static_cast<char*>(c.hidden_out);
  a.positions_out = c.positions_out;
  a.cu_out = c.cu_out;
  a.ctl = static_cast<uint32_t*>(c.ws);
  a.flags = reinterpret_cast<uint64_t*>(static_cast<char*>(c.ws) + lay.off_flags);
  a.desc = reinterpret_cast<up::BlockCopy*>(static_cast<char*>(c.ws) + lay.off_desc);
  a.row_bytes = c.row_bytes;
  a.row_stride = c.row_stride;
  a.capacity = c.capacity;
  a.num_seqs = c.num_seqs;
  a.block = c.block;
  a.num_blocks = lay.blocks;
  a.num_tiles = lay.tiles;
  if (a.num_blocks <= up::kScan1Blocks)
    hipLaunchKernelGGL((up::up_compact_scan_kernel<up::kScan1Threads, true>), dim3(1),
                       dim3(up::kScan1Threads), 0, c.stream, a);
  else
    hipLaunchKernelGGL((up::up_compact_scan_kernel<up::kCompactThreads, false>),
                       dim3((unsigned)a.num_tiles), dim3(up::kCompactThreads), 0, c.stream, a);
  st = up::check_launch("up_compact_scan_kernel");
  *ran = st == UP_OK;
  return st;
}

up_status run_gather(const GatherCall& c, int64_t T, bool revive) {
  up::CompactArgs a;
  bool ran;
  up_status st = scan_for(c, T, &a, &ran);
  if (st != UP_OK || !ran) return st;
  if (a.num_blocks == 0) {
    if (!c.ledger) return st;
    // nothing to copy: the ledger entries (all zero) by their own kernel
    hipLaunchKernelGGL(up::up_history_append_kernel, dim3((unsigned)up::ceil_div(c.num_seqs, 256)),
                       dim3(256), 0, c.stream, c.ledger, c.num_seqs, c.led_capacity, c.layer_id,
                       c.cu_out);
    return up::check_launch("up_history_append_kernel");
  }
  a.ledger = c.ledger;
  a.led_capacity = c.led_capacity;
  a.layer_id = c.layer_id;
  if (c.row_stride == c.row_bytes) {
    // kPieceBytes pieces, larger (4 KiB multiples) if a block would need more
    // than 65535 of them (keeps the item count of huge rows bounded)
    const int64_t bb = (int64_t)c.block * c.row_bytes;
    a.piece_bytes = up::kPieceBytes;
    if (up::ceil_div(bb, a.piece_bytes) > 65535)
      a.piece_bytes = (int64_t)up::align_up((size_t)up::ceil_div(bb, 65535), 4096);
    a.pieces = up::ceil_div(bb, a.piece_bytes);
    a.piece_rows = c.block;
  } else {
    a.piece_bytes = 0;
    a.piece_rows = c.row_bytes >= up::kRowPieceBytes ? 1 : up::kRowPieceBytes / c.row_bytes;
    if (a.piece_rows > c.block) a.piece_rows = c.block;
    a.pieces = up::ceil_div(c.block, a.piece_rows);
  }
  const int64_t items = a.num_blocks * a.pieces;
  const dim3 grid((unsigned)(items < (int64_t)1 << 30 ? items : (int64_t)1 << 30));
  const uintptr_t al = (uintptr_t)c.hidden | (uintptr_t)c.hidden_out | (uintptr_t)c.row_bytes |
                       (uintptr_t)c.row_stride;
  if (t_copy_start && hipEventRecord(t_copy_start, c.stream) != hipSuccess)
    return up::set_error(UP_ERR_HIP, "hipEventRecord (copy start event) failed");
  if (revive) launch_copy<true>(a, grid, al, c.stream);
  else launch_copy<false>(a, grid, al, c.stream);
  st = up::check_launch("up_compact_copy_kernel");
  if (st == UP_OK && t_copy_stop && hipEventRecord(t_copy_stop, c.stream) != hipSuccess)
    return up::set_error(UP_ERR_HIP, "hipEventRecord (copy stop event) failed");
  return st;
}

// ---------------------------------------------------------------------------
// Fused row operations (host side).
// ---------------------------------------------------------------------------
int elem_bytes(up_dtype dt) { return dt == UP_DTYPE_F32 ? 4 : 2; }

template <int OP, int DT, int VPL>
void launch_rowop_vpl(up::RowOpArgs a, int64_t num_blocks, int block, hipStream_t st) {
  constexpr int U = VPL >= 8 ? 1 : VPL >= 2 ? 8 / VPL : 4;  // rows per wave in flight
  a.rows_per_item = up::kRowThreads / 64 * U;
  a.pieces = (int)up::ceil_div(block, a.rows_per_item);
  const int64_t items = num_blocks * a.pieces;
  const dim3 grid((unsigned)(items < (int64_t)1 << 30 ? items : (int64_t)1 << 30));
  hipLaunchKernelGGL((up::up_rowop_kernel<OP, DT, VPL, U>), grid, dim3(up::kRowThreads), 0, st, a);
}

template <int OP, int DT>
void launch_rowop_dt(const up::RowOpArgs& a, int64_t num_blocks, int block, hipStream_t st) {
  const int64_t vpl = up::ceil_div(a.nvec, 64);
  if (vpl <= 1) launch_rowop_vpl<OP, DT, 1>(a, num_blocks, block, st);
  else if (vpl <= 2) launch_rowop_vpl<OP, DT, 2>(a, num_blocks, block, st);
  else if (vpl <= 4) launch_rowop_vpl<OP, DT, 4>(a, num_blocks, block, st);
  else if (vpl <= 8) launch_rowop_vpl<OP, DT, 8>(a, num_blocks, block, st);
  else launch_rowop_vpl<OP, DT, 16>(a, num_blocks, block, st);
}

template <int OP>
void launch_rowop(up_dtype dt, const up::RowOpArgs& a, int64_t num_blocks, int block, hipStream_t st) {
  switch (dt) {
    case UP_DTYPE_BF16: launch_rowop_dt<OP, up::kDtBf16>(a, num_blocks, block, st); break;
    case UP_DTYPE_F16: launch_rowop_dt<OP, up::kDtF16>(a, num_blocks, block, st); break;
    default: launch_rowop_dt<OP, up::kDtF32>(a, num_blocks, block, st); break;
  }
}

// Checks shared by the fused row operations: element type, row geometry in
// 16-byte vectors (at most 16 KiB per row), 16-byte alignment of every row.
// dtype arrives as a plain int from the C ABI and is checked before it is
// converted to up_dtype.
up_status check_rows(int dtype, int64_t hidden_dim, std::initializer_list<int64_t> strides,
                     std::initializer_list<const void*> ptrs) {
  if (dtype != UP_DTYPE_BF16 && dtype != UP_DTYPE_F16 && dtype != UP_DTYPE_F32)
    return up::set_error(UP_ERR_INVALID, "unknown dtype %d", dtype);
  const up_dtype dt = static_cast<up_dtype>(dtype);
  if (hidden_dim < 1) return up::set_error(UP_ERR_INVALID, "hidden_dim < 1");
  const int64_t rb = hidden_dim * elem_bytes(dt);
  if (rb % 16 != 0 || rb > 16384)
    return up::set_error(UP_ERR_UNSUPPORTED,
                         "rows of %lld bytes: need a multiple of 16 bytes, at most 16 KiB",
                         (long long)rb);
  for (int64_t s : strides)
    if (s < hidden_dim || (s * elem_bytes(dt)) % 16 != 0)
      return up::set_error(UP_ERR_UNSUPPORTED,
                           "row stride %lld: need >= hidden_dim and a multiple of 16 bytes",
                           (long long)s);
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15) return up::set_error(UP_ERR_UNSUPPORTED, "row buffers must be 16-byte aligned");
  return UP_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free compaction: the workspace lives in a file-scope device
// array instead of caller memory.  Each GPU the library runs on holds one
// copy of it until the process ends; its device address is looked up once
// per device (the array's name is a host-side stand-in, not a device
// address), and every up_compact_noalloc call on that GPU shares it.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchMaxBlocks = int64_t(1) << 19;  // blocks per call (33.5M tokens at G = 64)
constexpr size_t kScratchBytes =
    256 + ((size_t)(kScratchMaxBlocks / up::kScanTileBlocks) * sizeof(uint64_t) + 255) / 256 * 256 +
    (size_t)kScratchMaxBlocks * sizeof(up::BlockCopy);

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];      // device address of `scratch` per device (null: not looked up)
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch`; on the first call on a
// device its control block and tile status words are cleared on `stream`
// (a kernel, ahead of the call's own kernels on the same stream).
up_status scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return up::set_error(UP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return up::set_error(UP_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return up::set_error(UP_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    const int64_t nwords =
        (int64_t)(256 + (kScratchMaxBlocks / up::kScanTileBlocks) * sizeof(uint64_t)) / 4;
    hipLaunchKernelGGL(up::up_compact_init_kernel, dim3((unsigned)up::ceil_div(nwords, 256)),
                       dim3(256), 0, stream, static_cast<uint32_t*>(ptr), nwords);
    up_status st = up::check_launch("up_compact_init_kernel");
    if (st != UP_OK) return st;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return UP_OK;
}

}  // namespace

extern "C" {

up_status up_compact_workspace_size(int num_seqs, const int32_t* cu_seqlens_h, int block,
                                    size_t* bytes) {
  up::clear_error();
  if (!bytes) return up::set_error(UP_ERR_INVALID, "bytes is NULL");
  if (block < 1) return up::set_error(UP_ERR_INVALID, "block < 1");
  int64_t T;
  int mx;
  up_status st = up::check_cu_seqlens(num_seqs, cu_seqlens_h, &T, &mx);
  if (st != UP_OK) return st;
  *bytes = compact_layout(num_seqs, cu_seqlens_h, block).bytes;
  return UP_OK;
}

up_status up_compact_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  up::clear_error();
  if (!workspace) return up::set_error(UP_ERR_INVALID, "workspace is NULL");
  if ((uintptr_t)workspace & 255) return up::set_error(UP_ERR_INVALID, "workspace not 256-byte aligned");
  if (workspace_bytes < 256) return up::set_error(UP_ERR_WORKSPACE, "workspace smaller than 256 bytes");
  up_status st = up::check_device();
  if (st != UP_OK) return st;
  const int64_t nwords = (int64_t)(workspace_bytes / 4);
  hipLaunchKernelGGL(up::up_compact_init_kernel, dim3((unsigned)up::ceil_div(nwords, 256)), dim3(256),
                     0, stream, static_cast<uint32_t*>(workspace), nwords);
  return up::check_launch("up_compact_init_kernel");
}

up_status up_compact_status(void* workspace, size_t workspace_bytes, int32_t* status, int clear,
                            hipStream_t stream) {
  up::clear_error();
  if (!workspace || !status) return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  if ((uintptr_t)workspace & 255) return up::set_error(UP_ERR_INVALID, "workspace not 256-byte aligned");
  if (workspace_bytes < 256) return up::set_error(UP_ERR_WORKSPACE, "workspace smaller than 256 bytes");
  up_status st = up::check_device();
  if (st != UP_OK) return st;
  hipLaunchKernelGGL(up::up_compact_status_kernel, dim3(1), dim3(64), 0, stream,
                     static_cast<uint32_t*>(workspace), status, clear ? 1 : 0);
  return up::check_launch("up_compact_status_kernel");
}

up_status up_compact(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                     const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                     const void* hidden, int64_t row_bytes, int64_t row_stride_bytes,
                     const int32_t* positions, void* hidden_out, int32_t* positions_out,
                     int32_t* cu_seqlens_out, int64_t out_capacity_rows, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  up::clear_error();
  int64_t T;
  int max_len;
  up_status st = up::check_cu_seqlens(num_seqs, cu_seqlens_h, &T, &max_len);
  if (st != UP_OK) return st;
  if (out_capacity_rows < T)
    return up::set_error(UP_ERR_CAPACITY, "out_capacity_rows %lld < T %lld",
                         (long long)out_capacity_rows, (long long)T);
  if (!cu_seqlens_out || (T > 0 && (!hidden || !hidden_out)))
    return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  if ((positions == nullptr) != (positions_out == nullptr))
    return up::set_error(UP_ERR_INVALID, "positions and positions_out must both be set or both NULL");
  GatherCall c{num_seqs,  cu_seqlens_h, cu_seqlens_d,     cu_blocks_d, block,
               block_mask, hidden,      row_bytes,        row_stride_bytes,
               positions, hidden_out,  positions_out,    cu_seqlens_out, out_capacity_rows,
               workspace, workspace_bytes, stream};
  return run_gather(c, T, false);
}

up_status up_set_copy_events(hipEvent_t start, hipEvent_t stop) {
  up::clear_error();
  if ((start == nullptr) != (stop == nullptr))
    return up::set_error(UP_ERR_INVALID, "start and stop events must both be set or both NULL");
  t_copy_start = start;
  t_copy_stop = stop;
  return UP_OK;
}

up_status up_compact_record(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                            const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                            const void* hidden, int64_t row_bytes, int64_t row_stride_bytes,
                            const int32_t* positions, void* hidden_out, int32_t* positions_out,
                            int32_t* cu_seqlens_out, int64_t out_capacity_rows, void* workspace,
                            size_t workspace_bytes, void* ledger, int capacity, int layer_id,
                            hipStream_t stream) {
  up::clear_error();
  if (!ledger) return up::set_error(UP_ERR_INVALID, "ledger is NULL");
  if (capacity < 1) return up::set_error(UP_ERR_INVALID, "need capacity >= 1");
  int64_t T;
  int max_len;
  up_status st = up::check_cu_seqlens(num_seqs, cu_seqlens_h, &T, &max_len);
  if (st != UP_OK) return st;
  if (out_capacity_rows < T)
    return up::set_error(UP_ERR_CAPACITY, "out_capacity_rows %lld < T %lld",
                         (long long)out_capacity_rows, (long long)T);
  if (!cu_seqlens_out || (T > 0 && (!hidden || !hidden_out)))
    return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  if ((positions == nullptr) != (positions_out == nullptr))
    return up::set_error(UP_ERR_INVALID, "positions and positions_out must both be set or both NULL");
  GatherCall c{num_seqs,  cu_seqlens_h, cu_seqlens_d,     cu_blocks_d, block,
               block_mask, hidden,      row_bytes,        row_stride_bytes,
               positions, hidden_out,  positions_out,    cu_seqlens_out, out_capacity_rows,
               workspace, workspace_bytes, stream};
  c.ledger = static_cast<int32_t*>(ledger);
  c.led_capacity = capacity;
  c.layer_id = layer_id;
  return run_gather(c, T, false);
}

up_status up_compact_noalloc(int num_seqs, const int32_t* cu_seqlens_h,
                             const int32_t* cu_seqlens_d, const int32_t* cu_blocks_d, int block,
                             const uint8_t* block_mask, const void* hidden, int64_t row_bytes,
                             int64_t row_stride_bytes, const int32_t* positions, void* hidden_out,
                             int32_t* positions_out, int32_t* cu_seqlens_out,
                             int64_t out_capacity_rows, int32_t* status, hipStream_t stream) {
  up::clear_error();
  int64_t T;
  int max_len;
  up_status st = up::check_cu_seqlens(num_seqs, cu_seqlens_h, &T, &max_len);
  if (st != UP_OK) return st;
  if (block < 1 || block > 4096) return up::set_error(UP_ERR_INVALID, "block not in [1, 4096]");
  const CompactLayout lay = compact_layout(num_seqs, cu_seqlens_h, block);
  if (lay.blocks > kScratchMaxBlocks || lay.bytes > kScratchBytes)
    return up::set_error(UP_ERR_CAPACITY, "%lld blocks: up_compact_noalloc serves at most %lld",
                         (long long)lay.blocks, (long long)kScratchMaxBlocks);
  if (out_capacity_rows < T)
    return up::set_error(UP_ERR_CAPACITY, "out_capacity_rows %lld < T %lld",
                         (long long)out_capacity_rows, (long long)T);
  if (!cu_seqlens_out || (T > 0 && (!hidden || !hidden_out)))
    return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  if ((positions == nullptr) != (positions_out == nullptr))
    return up::set_error(UP_ERR_INVALID, "positions and positions_out must both be set or both NULL");
  if (num_seqs == 0) return UP_OK;
  st = up::check_device();
  if (st != UP_OK) return st;
  void* ws = nullptr;
  st = scratch_for_current_device(stream, &ws);
  if (st != UP_OK) return st;
  GatherCall c{num_seqs,  cu_seqlens_h, cu_seqlens_d,     cu_blocks_d, block,
               block_mask, hidden,      row_bytes,        row_stride_bytes,
               positions, hidden_out,  positions_out,    cu_seqlens_out, out_capacity_rows,
               ws,        kScratchBytes, stream};
  st = run_gather(c, T, false);
  if (st != UP_OK || status == nullptr) return st;
  hipLaunchKernelGGL(up::up_compact_status_kernel, dim3(1), dim3(64), 0, stream,
                     static_cast<uint32_t*>(ws), status, 1);
  return up::check_launch("up_compact_status_kernel");
}

up_status up_revive(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                    const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                    const void* packed, void* full, int64_t row_bytes, int64_t row_stride_bytes,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  up::clear_error();
  int64_t T;
  int max_len;
  up_status st = up::check_cu_seqlens(num_seqs, cu_seqlens_h, &T, &max_len);
  if (st != UP_OK) return st;
  if (T > 0 && (!packed || !full)) return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  // The full buffer plays the input role of up_compact, the packed rows the
  // output role; the copy runs the other way.
  GatherCall c{num_seqs, cu_seqlens_h, cu_seqlens_d, cu_blocks_d, block, block_mask, full,
               row_bytes, row_stride_bytes, nullptr, const_cast<void*>(packed), nullptr, nullptr,
               T, workspace, workspace_bytes, stream};
  return run_gather(c, T, true);
}

up_status up_compact_rmsnorm(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                             const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                             int dtype_value, const void* hidden, int64_t hidden_dim,
                             int64_t row_stride, const void* gamma, float eps,
                             const int32_t* positions, void* normed_out, void* residual_out,
                             int32_t* positions_out, int32_t* cu_seqlens_out,
                             int64_t out_capacity_rows, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  up::clear_error();
  int64_t T;
  int max_len;
  up_status st = up::check_cu_seqlens(num_seqs, cu_seqlens_h, &T, &max_len);
  if (st != UP_OK) return st;
  if (out_capacity_rows < T)
    return up::set_error(UP_ERR_CAPACITY, "out_capacity_rows %lld < T %lld",
                         (long long)out_capacity_rows, (long long)T);
  if (!cu_seqlens_out || (T > 0 && (!hidden || !normed_out)))
    return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  if ((positions == nullptr) != (positions_out == nullptr))
    return up::set_error(UP_ERR_INVALID, "positions and positions_out must both be set or both NULL");
  if (!(eps >= 0.f) || !isfinite(eps)) return up::set_error(UP_ERR_INVALID, "eps must be finite and >= 0");
  st = check_rows(dtype_value, hidden_dim, {row_stride, hidden_dim},
                  {hidden, normed_out, residual_out, gamma});
  if (st != UP_OK) return st;
  const up_dtype dtype = static_cast<up_dtype>(dtype_value);
  const int64_t eb = elem_bytes(dtype);
  GatherCall c{num_seqs,  cu_seqlens_h, cu_seqlens_d,  cu_blocks_d,    block,
               block_mask, hidden,      hidden_dim * eb, row_stride * eb, positions,
               normed_out, positions_out, cu_seqlens_out, out_capacity_rows,
               workspace,  workspace_bytes, stream};
  up::CompactArgs ca;
  bool ran;
  st = scan_for(c, T, &ca, &ran);
  if (st != UP_OK || !ran || ca.num_blocks == 0) return st;
  up::RowOpArgs a{};
  a.desc = ca.desc;
  a.num_blocks = ca.num_blocks;
  a.src = static_cast<const char*>(hidden);
  a.src_stride = row_stride * eb;
  a.out = static_cast<char*>(normed_out);
  a.out_stride = hidden_dim * eb;
  a.res_out = static_cast<char*>(residual_out);
  a.res_stride = hidden_dim * eb;
  a.gamma = static_cast<const char*>(gamma);
  a.positions = positions;
  a.positions_out = positions_out;
  a.nvec = hidden_dim * eb / 16;
  a.inv_d = 1.0f / (float)hidden_dim;
  a.eps = eps;
  launch_rowop<up::kOpNorm>(dtype, a, ca.num_blocks, block, stream);
  return up::check_launch("up_rowop_kernel");
}

up_status up_gather_add(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                        const int32_t* cu_blocks_d, int block, const uint8_t* block_mask,
                        int dtype_value, const void* frozen, int64_t hidden_dim, int64_t row_stride,
                        const void* delta, void* out, int64_t out_rows, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  up::clear_error();
  int64_t T;
  int max_len;
  up_status st = up::check_cu_seqlens(num_seqs, cu_seqlens_h, &T, &max_len);
  if (st != UP_OK) return st;
  if (out_rows < 0) return up::set_error(UP_ERR_INVALID, "out_rows < 0");
  if (T > 0 && out_rows > 0 && (!frozen || !delta || !out))
    return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  st = check_rows(dtype_value, hidden_dim, {row_stride, hidden_dim}, {frozen, delta, out});
  if (st != UP_OK) return st;
  const up_dtype dtype = static_cast<up_dtype>(dtype_value);
  const int64_t eb = elem_bytes(dtype);
  GatherCall c{num_seqs, cu_seqlens_h, cu_seqlens_d,    cu_blocks_d,     block,
               block_mask, frozen,     hidden_dim * eb, row_stride * eb, nullptr,
               out,      nullptr,      nullptr,         out_rows,
               workspace, workspace_bytes, stream};
  up::CompactArgs ca;
  bool ran;
  st = scan_for(c, T, &ca, &ran);
  if (st != UP_OK || !ran || ca.num_blocks == 0) return st;
  up::RowOpArgs a{};
  a.desc = ca.desc;
  a.num_blocks = ca.num_blocks;
  a.src = static_cast<const char*>(frozen);
  a.src_stride = row_stride * eb;
  a.delta = static_cast<const char*>(delta);
  a.delta_stride = hidden_dim * eb;
  a.out = static_cast<char*>(out);
  a.out_stride = hidden_dim * eb;
  a.nvec = hidden_dim * eb / 16;
  launch_rowop<up::kOpAdd>(dtype, a, ca.num_blocks, block, stream);
  return up::check_launch("up_rowop_kernel");
}

up_status up_kv_len(void* ledger, int num_seqs, int capacity, int layer_id,
                    const int32_t* cu_seqlens_d, int32_t* kv_len, hipStream_t stream) {
  up::clear_error();
  if (!ledger || (num_seqs > 0 && (!cu_seqlens_d || !kv_len)))
    return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  if (num_seqs < 0 || capacity < 1) return up::set_error(UP_ERR_INVALID, "need num_seqs >= 0, capacity >= 1");
  if (num_seqs == 0) return UP_OK;
  up_status st = up::check_device();
  if (st != UP_OK) return st;
  int32_t* led = static_cast<int32_t*>(ledger);
  hipLaunchKernelGGL(up::up_kv_len_kernel, dim3((unsigned)up::ceil_div(num_seqs, 4)), dim3(256), 0,
                     stream, led, num_seqs, capacity, layer_id, cu_seqlens_d, kv_len, led);
  return up::check_launch("up_kv_len_kernel");
}

size_t up_history_bytes(int num_seqs, int capacity) {
  if (num_seqs < 0 || capacity < 0) return 0;
  return sizeof(int32_t) * (up::kLedgerHeader + (size_t)num_seqs + 2 * (size_t)num_seqs * capacity);
}

up_status up_history_init(void* ledger, int num_seqs, int capacity, hipStream_t stream) {
  up::clear_error();
  if (!ledger) return up::set_error(UP_ERR_INVALID, "ledger is NULL");
  if (num_seqs < 0 || capacity < 1) return up::set_error(UP_ERR_INVALID, "need num_seqs >= 0, capacity >= 1");
  up_status st = up::check_device();
  if (st != UP_OK) return st;
  hipLaunchKernelGGL(up::up_history_init_kernel, dim3((unsigned)up::ceil_div(num_seqs + 1, 256)),
                     dim3(256), 0, stream, static_cast<int32_t*>(ledger), num_seqs, capacity);
  return up::check_launch("up_history_init_kernel");
}

up_status up_drop_history(void* ledger, int num_seqs, int capacity, int layer_id,
                          const int32_t* cu_seqlens_out, hipStream_t stream) {
  up::clear_error();
  if (!ledger || !cu_seqlens_out) return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  if (num_seqs < 0 || capacity < 1) return up::set_error(UP_ERR_INVALID, "need num_seqs >= 0, capacity >= 1");
  if (num_seqs == 0) return UP_OK;
  up_status st = up::check_device();
  if (st != UP_OK) return st;
  hipLaunchKernelGGL(up::up_history_append_kernel, dim3((unsigned)up::ceil_div(num_seqs, 256)),
                     dim3(256), 0, stream, static_cast<int32_t*>(ledger), num_seqs, capacity,
                     layer_id, cu_seqlens_out);
  return up::check_launch("up_history_append_kernel");
}

}  // extern "C"
