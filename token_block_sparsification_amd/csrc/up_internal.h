// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <string>

#include "uniprefill.h"

namespace up {

// Thread-local error message; set_error returns the status for chaining.
up_status set_error(up_status st, const char* fmt, ...);
void clear_error();

// Checks (once per device) that the current device is gfx950.
up_status check_device();

// Host-side validation of a packed batch; fills T and max length.
up_status check_cu_seqlens(int num_seqs, const int32_t* cu_h, int64_t* T, int* max_len);

// Turns the last HIP launch error into UP_ERR_HIP.
up_status check_launch(const char* what);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Geometry of the scoring kernels for one call (computed on the host).
struct ScoreGeometry {
  int rows_per_wg;   // query rows one column-sum workgroup holds in registers
  int rg;            // column-sum row groups per KV head
  int rg_a;          // row-statistics row groups per KV head (of the tiling in use)
  int rg_a1;         // the same for pass A's one-round tiling
  int one_round_a;   // pass A runs its one-round tiling
  int rounds_b;      // pass B runs its several-rounds tiling (rows_per_wg and rg are its)
  int ck;            // keys per row-statistics workgroup chunk (sets the partials layout)
  int ck_b;          // keys per column-sum workgroup chunk
  int max_chunks;    // chunks of the longest request
  size_t off_partial, off_colpart, off_arrive, bytes;
};

ScoreGeometry score_geometry(int num_seqs, int64_t T, int max_len, int hq, int hkv,
                             int head_dim, int n_query);

// Workgroups of a scoring pass resident at once (pass 0: row statistics,
// 1: row statistics in its one-round tiling, 2: column sums, 3: column sums
// in their several-rounds tiling).
int resident_wgs_for(int head_dim, int pass);
bool has_one_round_tiling(int head_dim);
bool has_rounds_tiling_b(int head_dim);

// Number of blocks a compaction tile spans for block size G.
int compact_tile_blocks(int block);

}  // namespace up
