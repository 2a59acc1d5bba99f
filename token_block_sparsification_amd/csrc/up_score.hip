// Steps 1-3 of the pruning path: tail-query importance scores and block means.
//
// Method (UniPrefill page "中国科学院与腾讯微信合作解决AI排队等待问题", §二 steps 1-2
// and §三): the last n tokens of a request query every key with a softmax
// normalised per query row; the probabilities summed over query rows and
// heads give each token's score, averaged over G-token blocks.
//
// Exact column sums need each row's final softmax statistics, which exist
// only after the whole key sweep, so S = Q_tail K^T is computed twice
// (recomputing is far cheaper than writing S to HBM):
//   pass A  up_rowstats_kernel   per (request, KV head, key chunk): bf16
//           MFMA S tiles with keys on the MFMA M axis, so each lane owns one
//           query row and reduces a running (max, sum) in registers.
//   pass B  up_colsum_kernel    first merges the chunk partials of its rows
//           into one log2-domain bias per row, m * c + log2(l) with
//           c = scale * log2(e); then the same tiles with queries on the M
//           axis, so each lane owns one key and sums exp2(s * c - bias) over
//           its rows in registers; waves meet in LDS, one partial per (KV
//           head, row group) is written per key.
//   up_score: up_blockmean_kernel then sums the partials over (KV head, row
//           group) in a fixed order (token score) and averages each block
//           (block score).
//   up_score_select: up_blockmean_select_kernel computes the same token and
//           block scores and, in the workgroup that writes a request's last
//           block mean, runs that request's Top-p selection (no further
//           launch).
// No floating-point atomics anywhere: results are bitwise reproducible.
#include <math.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "up_internal.h"
#include "up_select_impl.h"

namespace up {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Keys per LDS tile: two 32-wide MFMA tiles, one for head_dim 256 so that a
// four-tile ring stays at 64 KiB of LDS.
#ifndef UP_KT_D128
#define UP_KT_D128 64
#endif
template <int D> struct KeysPerTile {
  static constexpr int value = D >= 256 ? 32 : D == 128 ? UP_KT_D128 : 64;
};
// Waves per SIMD each pass is compiled for (its register budget).
#ifndef UP_OCC_A
#define UP_OCC_A 2
#endif
#ifndef UP_OCC_B
#define UP_OCC_B 2
#endif
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

// Key chunk bounds: a workgroup's chunk holds at most UP_CK_MAX keys (the
// chunk rules are in the host code below).
#ifndef UP_CK_MAX
#define UP_CK_MAX 4096
#endif

// Column-sum pass: walk its work groups last to first, so that its first
// workgroups read the keys the row-statistics pass read last (still cached).
#ifndef UP_REVERSE_B
#define UP_REVERSE_B 1
#endif
struct ScoreArgs {
  const int32_t* cu_seqlens;
  const int32_t* cu_blocks;
  const uint16_t* q;
  const uint16_t* k;
  int64_t q_tok, q_head, k_tok, k_head;
  int num_seqs, hq, hkv, rgqa, n_query, block;
  int ck, max_chunks, rg, rows_per_wg;
  int ck_a;           // keys per row-statistics chunk (the partials' chunking)
  int64_t num_groups;  // real (request, KV head, key chunk) groups
  int reverse;         // walk the groups last to first
  int one_chunk;       // every request holds 1..ck keys: request = group / hkv
  float c;  // scale * log2(e)
  float2* partial;  // [B][hq][max_chunks][n_query] (raw max, sum of exp2)
  float* colpart;   // [hkv * rg][T]
  int64_t T;
  float* token_scores;
  float* block_scores;
  int64_t num_blocks;
  uint32_t* arrive;        // [B] chunks of each request done (fused selection)
  int32_t* kept;           // fused selection: kept tokens [B] (requests without blocks get 0 here)
};

__global__ void up_zero_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Relaxed device-scope atomic store: coherent across the XCDs' L2 caches
// without an L2 write-back or invalidate (it writes through to memory).
// Values one workgroup hands to another inside a kernel go through it,
// ordered by the arrival counters (arrive_last), and are read with the
// selection's coherent loads.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Work decode shared by both passes.  The groups of work are the real
// (request, KV head, key chunk) triples, numbered densely: request-major,
// then KV head, then chunk.  Workgroups that read the same K chunk (the rg row
// groups of one group) get ids that are equal mod 8, so they run on the same
// XCD (ids are dealt round-robin over the 8 XCDs) and are dispatched close
// together: their K re-reads hit that XCD's L2.  Consecutive groups are
// consecutive chunks of one head, so every request's chunks spread evenly
// over the XCDs whatever the mix of request lengths.
struct Work {
  int req, g, chunk, rgi;
  bool valid;
};

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), lane) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
}

__device__ __forceinline__ Work decode_work(const ScoreArgs& a) {
  const int64_t w = blockIdx.x;
  const int64_t span = 8 * (int64_t)a.rg;
  const int64_t blk = w / span, rem = w - blk * span;
  Work wk;
  wk.rgi = (int)(rem >> 3);
  int64_t q = blk * 8 + (rem & 7);
  wk.valid = q < a.num_groups;
  if (a.reverse) q = a.num_groups - 1 - q;
  wk.req = 0;
  wk.g = 0;
  wk.chunk = 0;
  if (!wk.valid) return wk;
  if (a.one_chunk) {  // hkv groups per request, in request order
    const int r = (int)(q / a.hkv);
    wk.req = r;
    wk.g = (int)(q - (int64_t)r * a.hkv);
    return wk;
  }
  // Find the request holding group q, 64 requests per step (one per lane):
  // a wave-wide inclusive scan of their group counts, then the first lane
  // whose prefix passes q.  A batch of B requests costs ceil(B / 64) round
  // trips instead of B dependent ones.
  const int lane = threadIdx.x & 63;
  int r = -1;
  for (int r0 = 0; r0 < a.num_seqs; r0 += 64) {
    const int rr = r0 + lane;
    uint64_t ng = 0;
    if (rr < a.num_seqs) {
      const int L = a.cu_seqlens[rr + 1] - a.cu_seqlens[rr];
      ng = (uint64_t)((L + a.ck - 1) / a.ck) * (uint64_t)a.hkv;
    }
    const uint64_t incl = wave_scan_incl(ng);
    const uint64_t total = readlane64(incl, 63);
    if ((uint64_t)q < total) {
      const int owner = __ffsll((unsigned long long)__ballot(incl > (uint64_t)q)) - 1;
      q -= (int64_t)readlane64(incl - ng, owner);
      r = r0 + owner;
      break;
    }
    q -= (int64_t)total;
  }
  if (r < 0) {  // only if the device cu_seqlens disagree with the host copy
    wk.valid = false;
    return wk;
  }
  r = __builtin_amdgcn_readfirstlane(r);
  const int L = a.cu_seqlens[r + 1] - a.cu_seqlens[r];
  const int nch = (L + a.ck - 1) / a.ck;
  wk.req = r;
  wk.g = __builtin_amdgcn_readfirstlane((int)(q / nch));
  wk.chunk = __builtin_amdgcn_readfirstlane((int)(q - (int64_t)wk.g * nch));
  return wk;
}

// One 16-byte-per-lane global->LDS load (global_load_lds_dwordx4): lane i
// writes its 16 bytes at LDS byte address lds + 16 i.  Issued from an asm
// statement so that the compiler's wait-count pass does not track it: that
// pass cannot tell which ring slot an LDS DMA writes, and otherwise makes the
// next LDS read of any slot wait for every DMA in flight (vmcnt(0)), i.e. for
// the prefetch just issued.  The kernels order the ring by hand instead: an
// explicit s_waitcnt vmcnt(N) and a workgroup barrier precede every read of a
// slot, and the last tiles wait for vmcnt(0) before the workgroup ends.  The
// statement has no register outputs, so nothing the compiler allocates can be
// overwritten by the load in flight.
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  // m0 (the LDS destination base) is saved and restored inside the
  // statement: the compiler reserves m0 and may keep a value of its own there.
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(base)
      : "memory");
#else
  (void)src;
  (void)lds;
#endif
}

// Key rows of one LDS tile, fetched with direct global->LDS loads
// (global_load_lds_dwordx4: lane i of a wave writes 16 bytes at base + 16 i),
// so no registers stage the tile.  Rows are D*2 bytes, unpadded; the 16-byte
// chunk c of tile row r sits in slot c ^ (r & SWZ), which spreads the rows a
// fragment read touches over all LDS banks.
template <int D, int W>
struct KTile {
  static constexpr int KT = KeysPerTile<D>::value;
  static constexpr int CHUNKS = D / 8;                  // 16-byte chunks per key row
  static constexpr int RPI = 64 / CHUNKS;               // rows one wave instruction fills
  static constexpr int INSTS = KT / RPI / W;            // load instructions per wave per tile
  static constexpr int SWZ = CHUNKS < 16 ? CHUNKS - 1 : 15;
  static constexpr int ELEMS = KT * D;                  // elements per tile
  static_assert(KT % (RPI * W) == 0, "tile not divisible among waves");

  // Fetch keys [tkey0, tkey0 + KT) into `lds`; keys >= key_end read the last
  // valid key instead (in bounds; the masked path ignores them).
  static __device__ __forceinline__ void fetch(const uint16_t* kbase, int64_t k_tok, int tkey0,
                                               int key_end, uint16_t* lds, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < INSTS; ++i) {
      const int j = wave * INSTS + i;
      const int r = j * RPI + lane / CHUNKS;
      const int c = (lane % CHUNKS) ^ (r & SWZ);
      const int key = min(tkey0 + r, key_end - 1);
      lds_dma16(kbase + (int64_t)key * k_tok + c * 8, lds + j * RPI * D);
    }
  }
  // Element offset of chunk c of tile row r.
  static __device__ __forceinline__ int offset(int r, int c) { return r * D + ((c ^ (r & SWZ)) << 3); }
  // Element offset, from the tile's first key, of the 8 elements lane
  // `lane` moves with load instruction i (the same for every tile).
  static __device__ __forceinline__ uint32_t lane_offset(int64_t k_tok, int wave, int i, int lane) {
    const int j = wave * INSTS + i;
    const int r = j * RPI + lane / CHUNKS;
    const int c = (lane % CHUNKS) ^ (r & SWZ);
    return (uint32_t)((int64_t)r * k_tok + c * 8);
  }
};

// The chunk's key tiles as a stream into the LDS ring.  Whole tiles use a
// uniform base address plus fixed per-lane offsets, so a fetch costs no
// vector address arithmetic; only a chunk's ragged last tile takes the
// clamped path.
template <int D, int W>
struct KStream {
  using Tile = KTile<D, W>;
  const uint16_t* kbase;  // key 0 of the request in this KV head
  int64_t k_tok;
  int key0, key1, wave, lane;
  uint32_t off[Tile::INSTS];

  __device__ __forceinline__ void init(const uint16_t* kb, int64_t kt, int k0, int k1, int w, int l) {
    kbase = kb;
    k_tok = kt;
    key0 = k0;
    key1 = k1;
    wave = w;
    lane = l;
#pragma unroll
    for (int i = 0; i < Tile::INSTS; ++i) off[i] = Tile::lane_offset(kt, w, i, l);
  }
  // Tile t, known to hold KT keys below key1.
  __device__ __forceinline__ void fetch_full(int t, uint16_t* dst) const {
    const uint16_t* tb = kbase + (int64_t)(key0 + t * Tile::KT) * k_tok;
#pragma unroll
    for (int i = 0; i < Tile::INSTS; ++i)
      lds_dma16(tb + off[i], dst + (wave * Tile::INSTS + i) * Tile::RPI * D);
  }
  // Any tile t of the chunk.
  __device__ __forceinline__ void fetch(int t, uint16_t* dst) const {
    const int tk = key0 + t * Tile::KT;
    if (tk + Tile::KT <= key1) fetch_full(t, dst);
    else Tile::fetch(kbase, k_tok, tk, key1, dst, wave, lane);
  }
};

// Workgroup barrier that waits only for this wave's LDS operations; the K
// tile fetches in flight are covered by an explicit wait_vmcnt before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

// Wait until at most N of this wave's vector-memory loads (the K tile
// fetches) are in flight.  Written as an asm statement so the compiler's own
// wait-count pass keeps it exactly as placed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The K ring has RING slots (an even number >= 4).  When iteration it starts,
// tiles it and it+1 are resident and tiles it+2 .. it+RING-2 are in flight;
// iteration it fetches tile it+RING-1 into the slot tile it-1 left, and ends
// once tile it+2 has landed, so RING-3 tiles stay in flight behind the one
// the next iteration needs.  Loads return in issue order, so waiting until at
// most (RING-3) tiles' worth of loads are outstanding is enough (stores the
// pass issues in between only make that wait longer, never shorter).
//
// Ring start, in two parts so that a kernel's other prologue loads (query
// rows, softmax statistics) travel together with the first tiles:
// ring_issue fetches tiles 0 .. RING-2 (as many as exist); ring_ready then
// waits until tiles 0 and 1 have landed.  Loads issued between the two only
// make ring_ready's wait stronger (they complete after the tiles), never
// weaker.
template <int RING, typename Stream>
__device__ __forceinline__ void ring_issue(const Stream& ks, int ntiles,
                                           uint16_t (*kl)[Stream::Tile::ELEMS]) {
  static_assert(RING >= 4 && RING % 2 == 0, "ring of an even number of slots, at least 4");
#pragma unroll
  for (int t = 0; t < RING - 1; ++t)
    if (t < ntiles) ks.fetch(t, kl[t]);
}
template <int RING, typename Tile>
__device__ __forceinline__ void ring_ready(int ntiles) {
  if (ntiles >= RING - 1) wait_vmcnt<(RING - 3) * Tile::INSTS>();
  else wait_vmcnt<0>();
  lds_barrier();
}

// End of one ring iteration: tile it+2 resident in LDS for every wave.
// FETCHED = tile it+RING-1 was fetched this iteration (so were the tiles
// between it+3 and it), and RING-3 tiles may stay in flight.
template <int RING, typename Tile, bool FETCHED>
__device__ __forceinline__ void ring_step() {
  if constexpr (FETCHED) wait_vmcnt<(RING - 3) * Tile::INSTS>(); else wait_vmcnt<0>();
  lds_barrier();
}

// Ring iterations unrolled per trip of the steady-state loop (even, so a
// tile's parity is known at compile time).
#ifndef UP_RING_UNROLL
#define UP_RING_UNROLL 4
#endif
constexpr int kUnroll = UP_RING_UNROLL;
static_assert(kUnroll >= 2 && kUnroll % 2 == 0, "even unroll");

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}


// Query fragments of the lane's rows.  Row rho of KV group g is query head
// g*rgqa + rho/n_eff at tail position rho%n_eff.  The same registers serve as
// the MFMA B operand in pass A and the A operand in pass B: lane l holds row
// (l % 32) of each 32-row tile and dims [16s + 8(l/32), +8) of k-step s.
template <int D, int NT>
__device__ __forceinline__ void load_q(const ScoreArgs& a, int s0, int qpos0, int n_eff, int R,
                                       int g, int row0, int lane, bf16x8_t (&qf)[NT][D / 16],
                                       int (&ipos)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int rho = row0 + t * 32 + (lane & 31);
    if (rho < R) {
      const int hl = rho / n_eff, ti = rho - hl * n_eff;
      const int h = g * a.rgqa + hl;
      const uint16_t* p = a.q + (int64_t)(s0 + qpos0 + ti) * a.q_tok + (int64_t)h * a.q_head +
                          (lane >> 5) * 8;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qf[t][s] = load_bf16x8(p + s * 16);
      ipos[t] = qpos0 + ti;
    } else {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qf[t][s] = (bf16x8_t){};
      ipos[t] = 0x7fffffff;
    }
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the two passes.
//
// Both passes walk the chunk's keys in LDS tiles of KT keys held in the
// RING-slot ring above (tiles it and it+1 resident when iteration it starts,
// RING-3 more in flight).  Both passes may software-pipeline over "groups":
// one group is one 32x32 S tile (32 keys x 32 query rows).  While the VALU
// works on group g (scale, exp2, reductions), the MFMAs of group g+1 are
// already issued, so the matrix cores and the VALU run side by side within a
// wave.
// ---------------------------------------------------------------------------

// Sum of 16 values as a balanced tree (short dependency chains).
__device__ __forceinline__ float tree_sum16(const float (&e)[16]) {
  float a0 = (e[0] + e[1]) + (e[2] + e[3]), a1 = (e[4] + e[5]) + (e[6] + e[7]);
  float a2 = (e[8] + e[9]) + (e[10] + e[11]), a3 = (e[12] + e[13]) + (e[14] + e[15]);
  return (a0 + a1) + (a2 + a3);
}

// Sum of a value over the two half-waves (lanes l and l ^ 32), in every
// lane, with the cross-half permute on the VALU (no LDS round trip).
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Interleave hint for one group: UP_IL_MFMA MFMAs then a few VALU ops,
// repeated over the group's D/16 MFMAs.
#ifndef UP_IL_MFMA
#define UP_IL_MFMA 1
#endif
#ifndef UP_IL_VALU
#define UP_IL_VALU 64
#endif
template <int D>
__device__ __forceinline__ void interleave_hint() {
  constexpr int kSlots = D / 16 / UP_IL_MFMA;
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, UP_IL_MFMA, 0);          // MFMA
    __builtin_amdgcn_sched_group_barrier(0x402, UP_IL_VALU / kSlots, 0);  // VALU or TRANS
  }
}

// The same with one LDS read after each MFMA (a group that rolls in the next
// key sub-tile's fragments).
template <int D>
__device__ __forceinline__ void interleave_hint_roll() {
  constexpr int kSlots = D / 16 / UP_IL_MFMA;
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, UP_IL_MFMA, 0);          // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, UP_IL_MFMA, 0);          // DS read
    __builtin_amdgcn_sched_group_barrier(0x402, UP_IL_VALU / kSlots, 0);  // VALU or TRANS
  }
}

// Fragment s of key sub-tile `sub` (32 keys) of an LDS tile.
template <int D, int W>
__device__ __forceinline__ bf16x8_t load_frag(const uint16_t* tile, int sub, int lane, int s) {
  using Tile = KTile<D, W>;
  return load_bf16x8(tile + Tile::offset(sub * 32 + (lane & 31), 2 * s + (lane >> 5)));
}

template <int D, int W>
__device__ __forceinline__ void load_frags(const uint16_t* tile, int sub, int lane,
                                           bf16x8_t (&f)[D / 16]) {
  using Tile = KTile<D, W>;
  const int r = sub * 32 + (lane & 31);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = load_bf16x8(tile + Tile::offset(r, 2 * s + (lane >> 5)));
}

// ---------------------------------------------------------------------------
// Pass A: per-row running max and sum of exp2 over one key chunk.
// Keys on the MFMA M axis (A operand from LDS), query rows on N (B operand
// from registers): lane l owns row (l % 32), 16 keys per S tile.
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void rowstats_update(f32x16_t acc, int t, bool masked, int mkey0,
                                                int key1, int lane, float C,
                                                const int (&ipos)[NT], float (&m_run)[NT],
                                                float (&l_run)[NT]) {
  float x[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) x[v] = acc[v];
  if (masked) {
    // key j = mkey0 + 4 (lane / 32) + o_v with o_v = 8 (v / 4) + v % 4 (a
    // constant): valid iff j < key1 and j <= the row's position, i.e. o_v
    // <= thr; one compare per element
    const int thr = min(key1 - 1, ipos[t]) - (mkey0 + 4 * (lane >> 5));
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (8 * (v >> 2) + (v & 3) > thr) x[v] = kNegInf;
  }
  float mx = fmaxf(fmaxf(x[0], x[1]), m_run[t]);
#pragma unroll
  for (int v = 2; v < 16; v += 2) mx = fmaxf(fmaxf(mx, x[v]), x[v + 1]);
  const float mc = (mx == kNegInf) ? 0.f : mx * C;
  float e[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) e[v] = fast_exp2(fmaf(x[v], C, -mc));
  l_run[t] = fmaf(l_run[t], fast_exp2(fmaf(m_run[t], C, -mc)), tree_sum16(e));
  m_run[t] = mx;
}

// Three-stage form of pass A's pipeline: the VALU works on group q while the
// MFMAs of groups q+1 (issued one group earlier) and q+2 run, so no group's
// VALU work waits for the MFMA chain issued just before it (kernel traces at
// 128K: 146.4-146.5 vs 150.0-150.5 us; 32K: 45.8-46.2 vs 46.5-46.8 us).  Only
// the 8-wave tilings take it: with 4 waves per workgroup each wave keeps
// twice the K-fetch addresses, and the third accumulator spills (256 VGPRs).
#ifndef UP_PIPE3_A
#define UP_PIPE3_A 1
#endif
template <int D, int NT, int W, bool PIPE>
constexpr bool pipe3_a() {
  return UP_PIPE3_A && PIPE && NT == 2 && W == 8 && KTile<D, W>::KT / 32 >= 2;
}

// One LDS tile: NG = (KT/32)*NT groups, ordered (mt, t).  On entry acc holds
// the (issued) S of group 0 of this tile and af the A fragments of mt = 0;
// on exit they hold group 0 of the next tile (from `nxt`).  The pipelined
// form with NT >= 2 reads each sub-tile's fragments while the previous
// sub-tile's last group issues, so no MFMA waits on its LDS read.  In the
// three-stage form (pipe3_a) acc and acc1 hold groups 0 and 1 and af the
// fragments of sub-tile 1 on entry, and the same of the next tile on exit.
template <int D, int NT, int W, bool MASKED, bool PIPE>
__device__ __forceinline__ void rowstats_iter(const uint16_t* cur, const uint16_t* nxt, int tkey0,
                                              int key1, int lane, float C,
                                              const bf16x8_t (&qf)[NT][D / 16],
                                              const int (&ipos)[NT], float (&m_run)[NT],
                                              float (&l_run)[NT], f32x16_t& acc, f32x16_t& acc1,
                                              bf16x8_t (&af)[D / 16]) {
  constexpr int KT = KTile<D, W>::KT;
  constexpr int NG = (KT / 32) * NT;
  if constexpr (!MASKED && pipe3_a<D, NT, W, PIPE>()) {
    constexpr int SPT = KT / 32;
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int mt = q / NT, t = q % NT;
      const int mt2 = (q + 2) / NT, t2 = (q + 2) % NT;  // group q+2; mt2 >= SPT: next tile
      // af holds sub-tile mt2; its last group replaces each fragment by the
      // next sub-tile's right after the MFMA that reads it
      const bool roll = t2 == NT - 1;
      const int ns = mt2 + 1;
      const uint16_t* src = ns < SPT ? cur : nxt;
      const int nsub = ns < SPT ? ns : ns - SPT;
      f32x16_t nacc = {};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        nacc = mfma32(af[s], qf[t2][s], nacc);
        if (roll) af[s] = load_frag<D, W>(src, nsub, lane, s);
      }
      rowstats_update<NT>(acc, t, false, tkey0 + mt * 32, key1, lane, C, ipos, m_run, l_run);
      acc = acc1;
      acc1 = nacc;
      if (roll) interleave_hint_roll<D>(); else interleave_hint<D>();
    }
    return;
  }
  if constexpr (!PIPE) {
#pragma unroll
    for (int mt = 0; mt < KT / 32; ++mt) {
      load_frags<D, W>(cur, mt, lane, af);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x16_t sacc = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) sacc = mfma32(af[s], qf[t][s], sacc);
        rowstats_update<NT>(sacc, t, MASKED, tkey0 + mt * 32, key1, lane, C, ipos, m_run, l_run);
      }
    }
    return;
  }
  constexpr int SPT = KT / 32;
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int mt = q / NT, t = q % NT;
    const int mt1 = (q + 1) / NT, t1 = (q + 1) % NT;  // group q+1; mt1 == SPT: next tile
    f32x16_t nacc = {};
    if constexpr (NT >= 2) {
      // Rolling fragments: af holds sub-tile mt1 already.  When group q+1 is
      // the last user of its sub-tile, each fragment is replaced by the next
      // sub-tile's (of this tile, else sub-tile 0 of the next) right after
      // the MFMA that reads it, a whole group ahead of its first use.
      const bool roll = t1 == NT - 1;
      const int ns = mt1 + 1;
      const uint16_t* src = ns < SPT ? cur : nxt;
      const int nsub = ns < SPT ? ns : 0;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        nacc = mfma32(af[s], qf[t1][s], nacc);
        if (roll) af[s] = load_frag<D, W>(src, nsub, lane, s);
      }
      rowstats_update<NT>(acc, t, MASKED, tkey0 + mt * 32, key1, lane, C, ipos, m_run, l_run);
      acc = nacc;
      if (roll) interleave_hint_roll<D>(); else interleave_hint<D>();
    } else {
      if (q + 1 < NG) {
        if (mt1 != mt) load_frags<D, W>(cur, mt1, lane, af);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) nacc = mfma32(af[s], qf[t1][s], nacc);
      } else {
        load_frags<D, W>(nxt, 0, lane, af);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) nacc = mfma32(af[s], qf[0][s], nacc);
      }
      rowstats_update<NT>(acc, t, MASKED, tkey0 + mt * 32, key1, lane, C, ipos, m_run, l_run);
      acc = nacc;
      interleave_hint<D>();
    }
  }
}

template <int D, int NT, int W, bool PIPE, int RING>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(UP_OCC_A)))
up_rowstats_kernel(ScoreArgs a) {
  using Tile = KTile<D, W>;
  constexpr int KT = Tile::KT;
  __shared__ __attribute__((aligned(16))) uint16_t kl[RING][Tile::ELEMS];

  // The arrival counters of this call's block-mean/selection kernel start
  // at zero (it runs after this one, and this one after the previous call).
  if (blockIdx.x == 0) {
    for (int r = threadIdx.x; r < a.num_seqs; r += 64 * W) {
      a.arrive[r] = 0;
      // a request without blocks never reaches the selection
      if (a.kept && a.cu_blocks[r + 1] == a.cu_blocks[r]) a.kept[r] = 0;
    }
  }

  const Work wk = decode_work(a);
  if (!wk.valid) return;
  const int chunk = wk.chunk, g = wk.g, rgi = wk.rgi, req = wk.req;
  const int s0 = a.cu_seqlens[req];
  const int L = a.cu_seqlens[req + 1] - s0;
  const int key0 = chunk * a.ck;
  const int n_eff = min(a.n_query, L);
  const int R = a.rgqa * n_eff;
  const int wg_row0 = rgi * (NT * 32 * W);
  if (key0 >= L || wg_row0 >= R) return;  // uniform over the workgroup
  const int key1 = min(L, key0 + a.ck);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = wg_row0 + wave * NT * 32;
  const int qpos0 = L - n_eff;
  const float C = a.c;

  // the first K tiles travel together with the query rows
  const uint16_t* kbase = a.k + (int64_t)s0 * a.k_tok + (int64_t)g * a.k_head;
  const int ntiles = (key1 - key0 + KT - 1) / KT;
  KStream<D, W> ks;
  ks.init(kbase, a.k_tok, key0, key1, wave, lane);
  ring_issue<RING>(ks, ntiles, kl);

  bf16x8_t qf[NT][D / 16];
  int ipos[NT];
  load_q<D, NT>(a, s0, qpos0, n_eff, R, g, row0, lane, qf, ipos);

  float m_run[NT], l_run[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = kNegInf;
    l_run[t] = 0.f;
  }

  // leading tiles that need no mask: every key < key1 and <= every tail row
  const int lim = min(key1, qpos0 + 1);
  const int nfast = lim > key0 ? (lim - key0) / KT : 0;
  bf16x8_t af[D / 16];
  int it = 0;
  ring_ready<RING, Tile>(ntiles);

  // Mask-free tiles first (software-pipelined when PIPE), then the tiles
  // that meet the causal diagonal or the chunk's end, in straight order.
  // The steady-state loop prefetches whole tiles only and waits a fixed
  // count, so its body stays one basic block the scheduler can interleave;
  // the last few iterations (no prefetch left or a ragged one) wait for all.
  const int nfull = (key1 - key0) / KT;
  const int nmain = max(0, min(nfast, nfull - (RING - 1)));
  if (nfast > 0) {
    f32x16_t acc = {}, acc1 = {};
    if constexpr (PIPE) {
      load_frags<D, W>(kl[0], 0, lane, af);
#pragma unroll
      for (int s = 0; s < D / 16; ++s) acc = mfma32(af[s], qf[0][s], acc);
      if constexpr (pipe3_a<D, NT, W, PIPE>()) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) acc1 = mfma32(af[s], qf[1][s], acc1);
        load_frags<D, W>(kl[0], 1, lane, af);
      }
    }
    // Steady state unrolled over kUnroll tiles; with a ring of kUnroll slots
    // every LDS slot address is a compile-time constant (it starts at 0).
    auto step = [&](auto u) {
      constexpr int U = decltype(u)::value;
      const int s0 = RING == kUnroll ? 0 : it % RING;
      ks.fetch_full(it + U + RING - 1, kl[(s0 + U + RING - 1) % RING]);
      rowstats_iter<D, NT, W, false, PIPE>(kl[(s0 + U) % RING], kl[(s0 + U + 1) % RING],
                                           key0 + (it + U) * KT, key1, lane, C, qf, ipos, m_run,
                                           l_run, acc, acc1, af);
      ring_step<RING, Tile, true>();
    };
    for (; it + kUnroll <= nmain; it += kUnroll) static_for<0, kUnroll>(step);
    for (; it < nfast; ++it) {
      const bool more = it + RING - 1 < ntiles;
      if (more) ks.fetch(it + RING - 1, kl[(it + RING - 1) % RING]);
      rowstats_iter<D, NT, W, false, PIPE>(kl[it % RING], kl[(it + 1) % RING], key0 + it * KT,
                                           key1, lane, C, qf, ipos, m_run, l_run, acc, acc1, af);
      if (more) ring_step<RING, Tile, true>(); else ring_step<RING, Tile, false>();
    }
  }
  for (; it < ntiles; ++it) {
    if (it + RING - 1 < ntiles) ks.fetch(it + RING - 1, kl[(it + RING - 1) % RING]);
    f32x16_t acc = {}, acc1 = {};
    rowstats_iter<D, NT, W, true, false>(kl[it % RING], kl[(it + 1) % RING], key0 + it * KT, key1,
                                         lane, C, qf, ipos, m_run, l_run, acc, acc1, af);
    ring_step<RING, Tile, false>();
  }

  // Merge the two half-waves (same row, disjoint keys) and write the partial.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float mo = __shfl_xor(m_run[t], 32);
    const float lo = __shfl_xor(l_run[t], 32);
    const float M = fmaxf(m_run[t], mo);
    const float mc = (M == kNegInf) ? 0.f : M * C;
    const float l = l_run[t] * fast_exp2(fmaf(m_run[t], C, -mc)) + lo * fast_exp2(fmaf(mo, C, -mc));
    const int rho = row0 + t * 32 + lane;
    if (lane < 32 && rho < R) {
      const int hl = rho / n_eff, ti = rho - hl * n_eff;
      const int h = g * a.rgqa + hl;
      a.partial[(((int64_t)req * a.hq + h) * a.max_chunks + chunk) * a.n_query + ti] =
          make_float2(M, l);
    }
  }
}

// ---------------------------------------------------------------------------
// Pass B: column sums of the normalised probabilities over the chunk's keys.
// Query rows on the MFMA M axis (A operand from registers), keys on N
// (B operand from LDS): lane l owns key (l % 32), 16 rows per S tile.
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ float colsum_update(f32x16_t acc, int t, bool masked, int key, int key1,
                                               int lane, int row0, int n_eff, int qpos0, float C,
                                               const float (&bv)[NT][16]) {
  float e[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) e[v] = fast_exp2(fmaf(acc[v], C, -bv[t][v]));
  if (masked) {
    // Rebuilt on every masked tile from an opaque base, so the compiler does
    // not keep 16*NT row positions alive across the whole key loop.  Row rho
    // = base + o (o <= 27) is tail position rho mod n_eff; rows past R hold
    // zero queries and a +inf bias, so their terms are 0 whatever ti is.
    int base;
    asm volatile("v_mov_b32 %0, %1" : "=v"(base) : "v"(row0 + t * 32 + 4 * (lane >> 5)));
    if (n_eff % 32 == 0) {
      // 32-row tiles never straddle two heads' rows: row base + o_v (o_v =
      // 8 (v / 4) + v % 4, a constant) is tail position tb + o_v, and the key
      // is valid for it iff key < key1 and key <= qpos0 + tb + o_v, i.e.
      // o_v >= thr; one compare per element
      const int tb = base % n_eff;
      const int thr = key < key1 ? key - qpos0 - tb : (1 << 30);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (8 * (v >> 2) + (v & 3) < thr) e[v] = 0.f;
    } else if (n_eff >= 32) {
      // one modulo per tile; base % n_eff + o < 2 n_eff needs one subtraction
      const int tb = base % n_eff;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int ti = tb + 8 * (v >> 2) + (v & 3);
        ti = ti >= n_eff ? ti - n_eff : ti;
        if (!((key < key1) && (key <= qpos0 + ti))) e[v] = 0.f;
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ti = (base + 8 * (v >> 2) + (v & 3)) % n_eff;
        if (!((key < key1) && (key <= qpos0 + ti))) e[v] = 0.f;
      }
    }
  }
  return tree_sum16(e);
}

// One LDS tile: NG = (KT/32)*NT groups ordered (nt, t); the column sum of
// key sub-tile nt is complete after its last t and goes to LDS.
template <int D, int NT, int W, bool MASKED, bool PIPE>
__device__ __forceinline__ void colsum_iter(const uint16_t* cur, const uint16_t* nxt, int tkey0,
                                            int key1, int lane, int wave, int row0, int R,
                                            int n_eff, int qpos0, float C,
                                            const bf16x8_t (&qf)[NT][D / 16],
                                            const float (&bv)[NT][16], float (*colrow)[64],
                                            f32x16_t& acc, bf16x8_t (&kf)[D / 16]) {
  constexpr int KT = KTile<D, W>::KT;
  constexpr int NG = (KT / 32) * NT;
  float col = 0.f;
  if constexpr (!PIPE) {
    // Straight order: each group's MFMAs, then its VALU work.
#pragma unroll
    for (int nt = 0; nt < KT / 32; ++nt) {
      load_frags<D, W>(cur, nt, lane, kf);
      const int key = tkey0 + nt * 32 + (lane & 31);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x16_t sacc = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) sacc = mfma32(qf[t][s], kf[s], sacc);
        col += colsum_update<NT>(sacc, t, MASKED, key, key1, lane, row0, n_eff, qpos0, C, bv);
      }
      col = sum_halves(col);
      colrow[wave][nt * 32 + (lane & 31)] = col;  // both halves hold the same sum
      col = 0.f;
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int nt = q / NT, t = q % NT;
    f32x16_t nacc = {};
    if (q + 1 < NG) {
      const int nt1 = (q + 1) / NT, t1 = (q + 1) % NT;
      if (nt1 != nt) load_frags<D, W>(cur, nt1, lane, kf);
#pragma unroll
      for (int s = 0; s < D / 16; ++s) nacc = mfma32(qf[t1][s], kf[s], nacc);
    } else {
      load_frags<D, W>(nxt, 0, lane, kf);
#pragma unroll
      for (int s = 0; s < D / 16; ++s) nacc = mfma32(qf[0][s], kf[s], nacc);
    }
    const int key = tkey0 + nt * 32 + (lane & 31);
    col += colsum_update<NT>(acc, t, MASKED, key, key1, lane, row0, n_eff, qpos0, C, bv);
    if (t == NT - 1) {
      col = sum_halves(col);
      colrow[wave][nt * 32 + (lane & 31)] = col;  // both halves hold the same sum
      col = 0.f;
    }
    acc = nacc;
    if (PIPE) interleave_hint<D>();
  }
}

// Mask-free tile with the key fragments double-buffered: the fragments of the
// next key sub-tile are read from LDS one group ahead of the MFMAs that use
// them (kf[p] holds the sub-tiles of parity p), so no MFMA waits on its LDS
// read.  Needs an even number of sub-tiles per tile (the parity of a sub-tile
// is then the same in the current and the next tile).  On entry acc holds
// the issued S of group 0, kf[0] / kf[1] sub-tiles 0 / 1 of this tile; on exit
// the same for the next tile.
template <int D, int NT, int W>
__device__ __forceinline__ void colsum_iter_db(const uint16_t* cur, const uint16_t* nxt, int tkey0,
                                               int key1, int lane, int wave, int row0, int R,
                                               int n_eff, int qpos0, float C,
                                               const bf16x8_t (&qf)[NT][D / 16],
                                               const float (&bv)[NT][16], float (*colrow)[64],
                                               f32x16_t& acc, bf16x8_t (&kf)[2][D / 16]) {
  constexpr int KT = KTile<D, W>::KT;
  constexpr int SPT = KT / 32;
  constexpr int NG = SPT * NT;
  static_assert(SPT % 2 == 0, "double-buffered fragments need an even sub-tile count");
  float col = 0.f;
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int nt = q / NT, t = q % NT;
    const int nt1 = (q + 1) / NT, t1 = (q + 1) % NT;  // group q+1; nt1 == SPT: next tile
    if (t1 == 0) {
      // group q+1 opens sub-tile nt1, whose fragments are resident: read the
      // one after it into the buffer its predecessor (last used by the MFMAs
      // issued in the previous group) frees
      const int ps = nt1 + 1;
      if (ps < SPT) load_frags<D, W>(cur, ps, lane, kf[ps & 1]);
      else load_frags<D, W>(nxt, ps - SPT, lane, kf[ps & 1]);
    }
    f32x16_t nacc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) nacc = mfma32(qf[t1][s], kf[nt1 & 1][s], nacc);
    const int key = tkey0 + nt * 32 + (lane & 31);
    col += colsum_update<NT>(acc, t, false, key, key1, lane, row0, n_eff, qpos0, C, bv);
    if (t == NT - 1) {
      col = sum_halves(col);
      colrow[wave][nt * 32 + (lane & 31)] = col;  // both halves hold the same sum
      col = 0.f;
    }
    acc = nacc;
    interleave_hint<D>();
  }
}

// Column partials of a finished tile (its waves' sums in colrow, complete
// after the tile's ring barrier): every wave adds the W wave sums, in wave
// order, for its KT/W keys and writes them.  All 64 lanes run it; lanes that
// share a key store the same value, so no lane mask splits the caller's
// block.  FULL: every key of the tile is below key1.
template <int W, int KT, bool FULL>
__device__ __forceinline__ void colsum_flush(const float (*colrow)[64], int wave, int lane, int tkey0,
                                             int key1, float* colout) {
  constexpr int KPW = KT / W;
  static_assert(KT % W == 0, "keys per wave");
  const int k = wave * KPW + (lane % KPW);
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) sum += colrow[w][k];
  if (FULL || tkey0 + k < key1) colout[tkey0 + k] = sum;
}

template <int D, int NT, int W, bool PIPE, int RING>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(UP_OCC_B)))
up_colsum_kernel(ScoreArgs a) {
  using Tile = KTile<D, W>;
  constexpr int KT = Tile::KT;
  __shared__ __attribute__((aligned(16))) uint16_t kl[RING][Tile::ELEMS];
  __shared__ float colbuf[2][W][64];
  constexpr int ROWS = NT * 32 * W;
  __shared__ float sbias[ROWS];

  const Work wk = decode_work(a);
  if (!wk.valid) return;
  const int chunk = wk.chunk, g = wk.g, rgi = wk.rgi, req = wk.req;
  const int s0 = a.cu_seqlens[req];
  const int L = a.cu_seqlens[req + 1] - s0;
  const int key0 = chunk * a.ck;
  const int n_eff = min(a.n_query, L);
  const int R = a.rgqa * n_eff;
  const int wg_row0 = rgi * (NT * 32 * W);
  if (key0 >= L || wg_row0 >= R) return;
  const int key1 = min(L, key0 + a.ck);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = wg_row0 + wave * NT * 32;
  const int qpos0 = L - n_eff;
  const float C = a.c;

  // the first K tiles travel together with the query rows and the statistics
  const uint16_t* kbase = a.k + (int64_t)s0 * a.k_tok + (int64_t)g * a.k_head;
  const int ntiles = (key1 - key0 + KT - 1) / KT;
  KStream<D, W> ks;
  ks.init(kbase, a.k_tok, key0, key1, wave, lane);
  ring_issue<RING>(ks, ntiles, kl);

  bf16x8_t qf[NT][D / 16];
  int ipos_unused[NT];
  load_q<D, NT>(a, s0, qpos0, n_eff, R, g, row0, lane, qf, ipos_unused);

  // Softmax statistics of the workgroup's rows: one thread per row merges the
  // row-statistics pass's chunk partials, in chunk order, into the
  // log2-domain bias m * c + log2(l) (rows past R get +inf: probability 0).
  // Every row's maximum is finite (chunk 0 holds key 0, which every tail row
  // sees); chunks a row sees none of hold (-inf, 0) and add 0.
  {
    const int nch = (L + a.ck_a - 1) / a.ck_a;
    for (int i = tid; i < ROWS; i += 64 * W) {
      const int rho = wg_row0 + i;
      float b = kPosInf;
      if (rho < R) {
        const int hl = rho / n_eff, ti = rho - hl * n_eff;
        const float2* pp = a.partial + ((int64_t)req * a.hq + g * a.rgqa + hl) * a.max_chunks *
                                           a.n_query + ti;
        // Online merge, 32 partials in flight per round trip: the running sum
        // is rescaled to each batch's larger maximum (by exp2(-inf) = 0 before
        // the first batch, whose chunk 0 makes the maximum finite), so up to
        // 32 chunks take one round trip and the sum is the plain one.
        float M = kNegInf, l = 0.f;
        constexpr int CB = 32;
        for (int c0 = 0; c0 < nch; c0 += CB) {
          float2 v[CB];
#pragma unroll
          for (int u = 0; u < CB; ++u)
            v[u] = c0 + u < nch ? pp[(int64_t)(c0 + u) * a.n_query] : make_float2(kNegInf, 0.f);
          float bm = M;
#pragma unroll
          for (int u = 0; u < CB; ++u) bm = fmaxf(bm, v[u].x);
          const float mc = bm * C;
          l *= fast_exp2(fmaf(M, C, -mc));
#pragma unroll
          for (int u = 0; u < CB; ++u) l += v[u].y * fast_exp2(fmaf(v[u].x, C, -mc));
          M = bm;
        }
        b = M * C + log2f(l);
      }
      sbias[i] = b;
    }
    __syncthreads();
  }
  // Output element v of a 32x32 tile in lane l sits at row 8(v/4) + 4(l/32) + v%4.
  float bv[NT][16];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      bv[t][v] = sbias[row0 - wg_row0 + t * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)];
  }

  float* colout = a.colpart + ((int64_t)g * a.rg + rgi) * a.T + s0;
  const int lim = min(key1, qpos0 + 1);
  const int nfast = lim > key0 ? (lim - key0) / KT : 0;
  constexpr bool DB = PIPE && (KT / 32) % 2 == 0;  // double-buffered fragments
  bf16x8_t kfb[DB ? 2 : 1][D / 16];
  auto& kf = kfb[0];
  int it = 0;
  ring_ready<RING, Tile>(ntiles);

  // Loop structure as in pass A: steady state with whole-tile prefetch and
  // a fixed wait, then the last mask-free tiles, then the masked tiles.
  const int nfull = (key1 - key0) / KT;
  const int nmain = max(0, min(nfast, nfull - (RING - 1)));
  if (nfast > 0) {
    f32x16_t acc = {};
    if constexpr (PIPE) {
      load_frags<D, W>(kl[0], 0, lane, kf);
      if constexpr (DB) load_frags<D, W>(kl[0], 1, lane, kfb[DB ? 1 : 0]);
#pragma unroll
      for (int s = 0; s < D / 16; ++s) acc = mfma32(qf[0][s], kf[s], acc);
    }
    // Tile j's column partials are written during tile j+1, whose compute
    // hides the LDS reads (colbuf is double-buffered; the ring barrier at
    // the end of tile j+1 orders them before tile j+2 overwrites the buffer).
    auto step = [&](auto u) {
      constexpr int U = decltype(u)::value;  // it is a multiple of kUnroll (even): it+U has U's parity
      const int s0 = RING == kUnroll ? 0 : it % RING;
      ks.fetch_full(it + U + RING - 1, kl[(s0 + U + RING - 1) % RING]);
      if (it + U > 0)
        colsum_flush<W, KT, true>(colbuf[(U + 1) & 1], wave, lane,
                                       key0 + (it + U - 1) * KT, key1, colout);
      if constexpr (DB)
        colsum_iter_db<D, NT, W>(kl[(s0 + U) % RING], kl[(s0 + U + 1) % RING], key0 + (it + U) * KT,
                                 key1, lane, wave, row0, R, n_eff, qpos0, C, qf, bv, colbuf[U & 1],
                                 acc, kfb);
      else
        colsum_iter<D, NT, W, false, PIPE>(kl[(s0 + U) % RING], kl[(s0 + U + 1) % RING],
                                           key0 + (it + U) * KT, key1, lane, wave, row0, R, n_eff,
                                           qpos0, C, qf, bv, colbuf[U & 1], acc, kf);
      ring_step<RING, Tile, true>();
    };
    for (; it + kUnroll <= nmain; it += kUnroll) static_for<0, kUnroll>(step);
    for (; it < nfast; ++it) {
      const bool more = it + RING - 1 < ntiles;
      if (more) ks.fetch(it + RING - 1, kl[(it + RING - 1) % RING]);
      if (it > 0)
        colsum_flush<W, KT, false>(colbuf[(it + 1) & 1], wave, lane, key0 + (it - 1) * KT,
                                        key1, colout);
      if constexpr (DB)
        colsum_iter_db<D, NT, W>(kl[it % RING], kl[(it + 1) % RING], key0 + it * KT, key1, lane,
                                 wave, row0, R, n_eff, qpos0, C, qf, bv, colbuf[it & 1], acc, kfb);
      else
        colsum_iter<D, NT, W, false, PIPE>(kl[it % RING], kl[(it + 1) % RING], key0 + it * KT,
                                           key1, lane, wave, row0, R, n_eff, qpos0, C, qf, bv,
                                           colbuf[it & 1], acc, kf);
      if (more) ring_step<RING, Tile, true>(); else ring_step<RING, Tile, false>();
    }
  }
  for (; it < ntiles; ++it) {
    if (it + RING - 1 < ntiles) ks.fetch(it + RING - 1, kl[(it + RING - 1) % RING]);
    if (it > 0)
      colsum_flush<W, KT, false>(colbuf[(it + 1) & 1], wave, lane, key0 + (it - 1) * KT,
                                      key1, colout);
    f32x16_t acc = {};
    colsum_iter<D, NT, W, true, false>(kl[it % RING], kl[(it + 1) % RING], key0 + it * KT, key1,
                                       lane, wave, row0, R, n_eff, qpos0, C, qf, bv, colbuf[it & 1],
                                       acc, kf);
    ring_step<RING, Tile, false>();
  }
  // the last tile (ntiles >= 1: the chunk holds at least one key)
  colsum_flush<W, KT, false>(colbuf[(ntiles - 1) & 1], wave, lane,
                                  key0 + (ntiles - 1) * KT, key1, colout);
}

// ---------------------------------------------------------------------------
// Epilogue of up_score: token score = fixed-order sum of the per-(KV head,
// row group) partials; block score = mean over the block's tokens.  One wave
// per block.  The fused entry point runs the same code (COH: the block score
// stored coherently) and selects in the same kernel.
// ---------------------------------------------------------------------------
// Request owning block b (the last r with cu_blocks[r] <= b), found by the
// whole wave: each step samples 64 evenly spaced entries of the remaining
// span and keeps the one below the first sample past b, so up to 64 requests
// take one round trip and up to 4096 two (a binary search takes log2 B
// dependent ones).  b must be a block of the batch; the wave must be whole.
__device__ __forceinline__ int block_owner(const int32_t* cu_blocks, int num_seqs, int64_t b,
                                           int lane) {
  int lo = 0, hi = num_seqs;  // cu_blocks[lo] <= b < cu_blocks[hi]
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const uint64_t le = __ballot(idx < hi && cu_blocks[idx] <= b);  // a prefix of lanes, lane 0 set
    lo += (63 - __clzll((long long)le)) * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

template <bool COH>
__device__ __forceinline__ void blockmean_one(const ScoreArgs& a, int64_t b, int lane) {
  const int r = __builtin_amdgcn_readfirstlane(block_owner(a.cu_blocks, a.num_seqs, b, lane));
  const int s0 = a.cu_seqlens[r];
  const int L = a.cu_seqlens[r + 1] - s0;
  const int lb = (int)(b - a.cu_blocks[r]);
  const int j0 = lb * a.block, j1 = min(j0 + a.block, L);
  // only the row groups that hold rows of this request wrote partials
  const int n_eff = min(a.n_query, L);
  const int rg_used = (a.rgqa * n_eff + a.rows_per_wg - 1) / a.rows_per_wg;
  const int nterm = a.hkv * rg_used;
  float sum = 0.f;
  for (int j = j0 + lane; j < j1; j += 64) {
    // Terms in (KV head, row group) order, g-major: eight loads are issued
    // before the first is added, so a token takes one round trip per eight
    // terms instead of one per term; the additions keep that order.
    const float* p = a.colpart + s0 + j;
    float c = 0.f;
    int g = 0, rgi = 0;
    for (int t0 = 0; t0 < nterm; t0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v[u] = t0 + u < nterm ? p[((int64_t)g * a.rg + rgi) * a.T] : 0.f;
        if (++rgi == rg_used) { rgi = 0; ++g; }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (t0 + u < nterm) c += v[u];
    }
    if (a.token_scores) a.token_scores[s0 + j] = c;
    sum += c;
  }
  sum = wave_sum_f32(sum);
  if (lane == 0) {
    if constexpr (COH) store_coherent(&a.block_scores[b], sum / (float)(j1 - j0));
    else a.block_scores[b] = sum / (float)(j1 - j0);
  }
}

__global__ void __launch_bounds__(256) up_blockmean_kernel(ScoreArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * 4 + wave;
  if (b < a.num_blocks) blockmean_one<false>(a, b, lane);
}

// Count this workgroup in *counter once its coherent stores (store_coherent)
// have completed; true, in every thread, in the workgroup that brings the
// count to `expect`.  Every wave waits until its stores are acknowledged
// (written through to memory) before the one thread counts, so the
// workgroup that reads the final count finds every counted workgroup's
// coherent stores with coherent loads.  No L2 write-back or invalidate.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expect, uint32_t& flag) {
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag = prev + 1 == expect ? 1u : 0u;
  }
  __syncthreads();
  return flag != 0;
}

// Blocks per wave in the fused kernel: two halve the workgroups that count
// arrivals and the rounds a batch of many blocks needs (kernel traces: 128K
// 18.4 vs 18.7 us, 16-request batch 25.9 vs 31.0 us); four cost more in the
// sequential block means than they save (21.1 us at 128K).
constexpr int kFusedBlocksPerWave = 2;

// Block means and the selection in one launch (up_score_select): waves of
// block means as above, the block scores written coherently; each workgroup
// then counts itself done for every request whose blocks it holds, and the
// workgroup that completes a request selects its blocks (reading the scores
// coherently), so the selection starts as soon as the request's last block
// mean is written.
__global__ void __launch_bounds__(kSelectThreads) up_blockmean_select_kernel(ScoreArgs a,
                                                                             SelectArgs sa) {
  constexpr int BPW = kSelectThreads / 64 * kFusedBlocksPerWave;  // blocks per workgroup
  __shared__ SelectShared<kSelectThreads, kStageMax> sh;
  __shared__ uint32_t s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t b0 = (int64_t)blockIdx.x * BPW;
#pragma unroll
  for (int kb = 0; kb < kFusedBlocksPerWave; ++kb) {
    const int64_t b = b0 + kb * (kSelectThreads / 64) + wave;
    if (b < a.num_blocks) blockmean_one<true>(a, b, lane);
  }
  const int64_t b1 = min(b0 + BPW, a.num_blocks) - 1;
  // requests owning the first and the last block here; requests in between
  // without blocks are skipped
  const int r0 = __builtin_amdgcn_readfirstlane(block_owner(a.cu_blocks, a.num_seqs, b0, lane));
  const int r1 = __builtin_amdgcn_readfirstlane(block_owner(a.cu_blocks, a.num_seqs, b1, lane));
  for (int r = r0; r <= r1; ++r) {  // uniform over the workgroup
    const int64_t c0 = a.cu_blocks[r], c1 = a.cu_blocks[r + 1];
    if (c1 == c0) continue;
    const uint32_t wgs = (uint32_t)((c1 - 1) / BPW - c0 / BPW + 1);  // workgroups holding its blocks
    if (arrive_last(&a.arrive[r], wgs, s_last))
      select_request<kSelectThreads, kStageMax, true>(sa, r, sh);
  }
}

// Compile-time tiling per head_dim and pass: NT 32-row tiles per wave, W
// waves per workgroup, PIPE = software-pipelined MFMA/VALU interleave, RING =
// LDS slots of the K ring.  Pass A writes per-row partials, so the two passes
// may group rows differently.
#ifndef UP_TILE_A64
#define UP_TILE_A64 2, 4, true, 4
#endif
#ifndef UP_TILE_B64
#define UP_TILE_B64 2, 8, true, 4
#endif
#ifndef UP_TILE_A128
#define UP_TILE_A128 2, 4, true, 4
#endif
#ifndef UP_TILE_B128
#define UP_TILE_B128 2, 8, true, 4
#endif
#ifndef UP_TILE_A256
#define UP_TILE_A256 1, 4, true, 4
#endif
// Pass A when the whole batch fits one resident round: one 8-wave workgroup
// per CU.  Two 4-wave workgroups sharing a CU drift apart (the SIMD arbiter
// prefers the older one's waves), and with no further round to fill in, the
// younger one ends the pass alone at one wave per SIMD (scoring at 128K,
// head_dim 128: row statistics 141 vs 146 us; head_dim 256, n = 128: 300 vs
// 316 us per call); over several rounds the two-workgroup form wins (the
// 16-request batch: 595 vs 644 us), since one workgroup's prologue overlaps
// the other's key loop.  At head_dim 64 the 8-wave form measured slower
// (2K tokens: 25.7 vs 23.7 us per call), so there it is not used.
#ifndef UP_TILE_A128_ONE_ROUND
#define UP_TILE_A128_ONE_ROUND 2, 8, true, 4
#endif
#ifndef UP_TILE_A256_ONE_ROUND
#define UP_TILE_A256_ONE_ROUND 1, 8, true, 4
#endif
#ifndef UP_TILE_A64_ONE_ROUND
#define UP_TILE_A64_ONE_ROUND UP_TILE_A64
#endif
// Pass B at head_dim 256: one 8-wave workgroup of 32-row tiles per CU, also
// over several rounds (Qwen3-Next shape, per call: n = 32 97-98 vs 99-100 us,
// n = 128 288-296 vs 302-311 us, n = 512 1026-1028 vs 1063-1065 us against
// two 4-wave workgroups).
#ifndef UP_TILE_B256
#define UP_TILE_B256 1, 8, true, 4
#endif
// Pass B when the batch needs several resident rounds: two 4-wave workgroups
// per CU at head_dim 128, so that one workgroup's prologue (query rows, first
// K tiles, the merge of its rows' chunk partials) overlaps the other's key
// loop (same box, per up_score: 256 requests of 512 tokens 415-419 vs 433-440
// us, the 16-request batch 1144-1148 vs 1148-1163 us; a single 128K request,
// one round, keeps the 8-wave form: 267.5 vs 272.3 us with the 4-wave one).
// Head_dim 64 and 256 keep their one tiling.
#ifndef UP_TILE_B64_ROUNDS
#define UP_TILE_B64_ROUNDS UP_TILE_B64
#endif
#ifndef UP_TILE_B128_ROUNDS
#define UP_TILE_B128_ROUNDS 2, 4, true, 4
#endif
#ifndef UP_TILE_B256_ROUNDS
#define UP_TILE_B256_ROUNDS UP_TILE_B256
#endif
template <int NT_, int W_, bool PIPE_, int RING_>
struct TileCfg {
  static constexpr int NT = NT_, W = W_, RING = RING_;
  static constexpr bool PIPE = PIPE_;
  static constexpr int ROWS = NT * 32 * W;
};
template <int D> struct Tiling;
// A1: the pass-A tiling for a batch that fits one resident round of it;
// BR: the pass-B tiling for a batch that needs several rounds of B.
template <> struct Tiling<64> {
  using A = TileCfg<UP_TILE_A64>;
  using A1 = TileCfg<UP_TILE_A64_ONE_ROUND>;
  using B = TileCfg<UP_TILE_B64>;
  using BR = TileCfg<UP_TILE_B64_ROUNDS>;
};
template <> struct Tiling<128> {
  using A = TileCfg<UP_TILE_A128>;
  using A1 = TileCfg<UP_TILE_A128_ONE_ROUND>;
  using B = TileCfg<UP_TILE_B128>;
  using BR = TileCfg<UP_TILE_B128_ROUNDS>;
};
template <> struct Tiling<256> {
  using A = TileCfg<UP_TILE_A256>;
  using A1 = TileCfg<UP_TILE_A256_ONE_ROUND>;
  using B = TileCfg<UP_TILE_B256>;
  using BR = TileCfg<UP_TILE_B256_ROUNDS>;
};

// Rows and waves per workgroup of pass A (pass 0), pass A's one-round
// tiling (pass 1), pass B (pass 2) and pass B's several-rounds tiling (3).
template <typename T>
int tiling_rows(int pass) {
  return pass == 0 ? T::A::ROWS : pass == 1 ? T::A1::ROWS : pass == 2 ? T::B::ROWS : T::BR::ROWS;
}
template <typename T>
int tiling_waves(int pass) {
  return pass == 0 ? T::A::W : pass == 1 ? T::A1::W : pass == 2 ? T::B::W : T::BR::W;
}
int rows_per_wg_for(int d, int pass) {
  switch (d) {
    case 64: return tiling_rows<Tiling<64>>(pass);
    case 128: return tiling_rows<Tiling<128>>(pass);
    default: return tiling_rows<Tiling<256>>(pass);
  }
}
int waves_per_wg_for(int d, int pass) {
  switch (d) {
    case 64: return tiling_waves<Tiling<64>>(pass);
    case 128: return tiling_waves<Tiling<128>>(pass);
    default: return tiling_waves<Tiling<256>>(pass);
  }
}

int64_t grid_for(const ScoreArgs& a) { return ceil_div(a.num_groups, 8) * 8 * a.rg; }

template <int D, typename TA>
up_status launch_rowstats(const ScoreArgs& b_args, int rg_a, hipStream_t st) {
  ScoreArgs aa = b_args;
  aa.rg = rg_a;
  aa.rows_per_wg = TA::ROWS;
  hipLaunchKernelGGL((up_rowstats_kernel<D, TA::NT, TA::W, TA::PIPE, TA::RING>),
                     dim3((unsigned)grid_for(aa)), dim3(64 * TA::W), 0, st, aa);
  return check_launch("up_rowstats_kernel");
}

template <int D, typename TB>
up_status launch_colsum(const ScoreArgs& bb, hipStream_t st) {
  hipLaunchKernelGGL((up_colsum_kernel<D, TB::NT, TB::W, TB::PIPE, TB::RING>),
                     dim3((unsigned)grid_for(bb)), dim3(64 * TB::W), 0, st, bb);
  return check_launch("up_colsum_kernel");
}

template <int D>
up_status launch_passes(const ScoreArgs& b_args, int rg_a, bool one_round_a, bool rounds_b,
                        int ck_b, int64_t groups_b, int one_chunk_b, hipStream_t st) {
  up_status s = one_round_a ? launch_rowstats<D, typename Tiling<D>::A1>(b_args, rg_a, st)
                            : launch_rowstats<D, typename Tiling<D>::A>(b_args, rg_a, st);
  if (s != UP_OK) return s;
  ScoreArgs bb = b_args;  // the column-sum pass chunks the keys its own way
  bb.ck_a = b_args.ck;
  bb.ck = ck_b;
  bb.num_groups = groups_b;
  bb.one_chunk = one_chunk_b;
  bb.reverse = UP_REVERSE_B;
  return rounds_b ? launch_colsum<D, typename Tiling<D>::BR>(bb, st)
                  : launch_colsum<D, typename Tiling<D>::B>(bb, st);
}

}  // namespace

// Workgroups of one pass resident on the chip at once: a pass runs the waves
// per SIMD its register budget allows (UP_OCC_A / UP_OCC_B, so 4 times that
// per CU), W waves per workgroup, on the UP_NUM_CUS CUs of gfx950.
#ifndef UP_NUM_CUS
#define UP_NUM_CUS 256
#endif
int resident_wgs_for(int d, int pass) {
  const int waves_per_cu = 4 * (pass >= 2 ? UP_OCC_B : UP_OCC_A);
  return UP_NUM_CUS * std::max(1, waves_per_cu / waves_per_wg_for(d, pass));
}

bool has_rounds_tiling_b(int d) {
  switch (d) {
    case 64: return !std::is_same<Tiling<64>::B, Tiling<64>::BR>::value;
    case 128: return !std::is_same<Tiling<128>::B, Tiling<128>::BR>::value;
    default: return !std::is_same<Tiling<256>::B, Tiling<256>::BR>::value;
  }
}

bool has_one_round_tiling(int d) {
  switch (d) {
    case 64: return !std::is_same<Tiling<64>::A, Tiling<64>::A1>::value;
    case 128: return !std::is_same<Tiling<128>::A, Tiling<128>::A1>::value;
    default: return !std::is_same<Tiling<256>::A, Tiling<256>::A1>::value;
  }
}

ScoreGeometry score_geometry(int num_seqs, int64_t T, int max_len, int hq, int hkv, int head_dim,
                             int n_query) {
  ScoreGeometry g{};
  const int rgqa = hkv > 0 ? hq / hkv : 1;
  const int64_t rmax = (int64_t)rgqa * (n_query < max_len ? n_query : max_len);
  g.rows_per_wg = rows_per_wg_for(head_dim, 2);
  g.rg = (int)(rmax > 0 ? ceil_div(rmax, g.rows_per_wg) : 1);
  const int rows_a = rows_per_wg_for(head_dim, 0);
  g.rg_a = (int)(rmax > 0 ? ceil_div(rmax, rows_a) : 1);
  const int rows_a1 = rows_per_wg_for(head_dim, 1);
  g.rg_a1 = (int)(rmax > 0 ? ceil_div(rmax, rows_a1) : 1);
  g.one_round_a = 0;
  g.rounds_b = 0;
  g.ck = 0;  // chosen by the caller once lengths are known
  g.max_chunks = 0;
  (void)num_seqs;
  (void)T;
  return g;
}

}  // namespace up

extern "C" up_status up_score_workspace_size(int num_seqs, const int32_t* cu_seqlens_h, int hq,
                                             int hkv, int head_dim, int n_query, size_t* bytes);

namespace {

#ifndef UP_CK_OVERHEAD
#define UP_CK_OVERHEAD 256
#endif
// Row-statistics key chunk: the largest power of two in [256, UP_CK_MAX]
// that still gives one resident round of workgroups (`resident`, at least)
// for this batch: longer chunks cost less per key (ring fill, Q loads, chunk
// merges) as long as every CU has work.  Measured against 2048-key chunks
// with two rounds: 15% less scoring time at L = 32K, 3% less at 128K.
int choose_ck(int num_seqs, const int32_t* cu_h, int hkv, int rg_a, int resident) {
  int ck = UP_CK_MAX;
  while (ck > 256) {
    int64_t wgs = 0;
    for (int r = 0; r < num_seqs; ++r)
      wgs += up::ceil_div(cu_h[r + 1] - cu_h[r], ck) * (int64_t)hkv * rg_a;
    if (wgs >= resident) break;
    ck >>= 1;
  }
  return ck;
}

// Column-sum chunk: whole rounds of workgroups.  The column-sum workgroups of
// a batch all take about the same time per key, so a last round that only
// part fills the chip costs as much as a full one: pick the chunk (a multiple
// of 64 keys, at most UP_CK_MAX) that minimises rounds x (chunk + per-workgroup
// overhead), where one round holds resident / (hkv * rg) chunks (the
// column-sum workgroups resident at once, over the row groups of one KV
// head).  Single requests keep the chunk of the rule above; a 16-request
// batch of 542K tokens gets 2944-key chunks in 6 rounds instead of 4096-key
// chunks in 5, the last one part full (column sums 657 vs 698 us).  Past 4096
// requests the search is skipped.
int choose_ck_rounds(int num_seqs, const int32_t* cu_h, int hkv, int rg, int resident,
                     int fallback) {
  if (num_seqs > 4096) return fallback;
  const int64_t per_round = std::max<int64_t>(1, resident / ((int64_t)hkv * rg));
  int best_ck = fallback;
  int64_t best = INT64_MAX;
  for (int ck = 256; ck <= UP_CK_MAX; ck += 64) {
    int64_t nch = 0;
    for (int r = 0; r < num_seqs; ++r) nch += up::ceil_div(cu_h[r + 1] - cu_h[r], ck);
    const int64_t cost = up::ceil_div(nch, per_round) * (ck + UP_CK_OVERHEAD);
    if (cost <= best) {  // ties: the longer chunk
      best = cost;
      best_ck = ck;
    }
  }
  return best_ck;
}

struct Layout {
  up::ScoreGeometry g;
  size_t bytes;
};

up_status score_layout(int num_seqs, const int32_t* cu_h, int hq, int hkv, int head_dim,
                       int n_query, Layout* out) {
  int64_t T;
  int max_len;
  up_status st = up::check_cu_seqlens(num_seqs, cu_h, &T, &max_len);
  if (st != UP_OK) return st;
  if (hq < 1 || hkv < 1 || hq > 1024 || hq % hkv != 0)
    return up::set_error(UP_ERR_INVALID, "need 1 <= hq <= 1024, hkv >= 1, hq %% hkv == 0 (hq=%d hkv=%d)",
                         hq, hkv);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return up::set_error(UP_ERR_UNSUPPORTED, "head_dim %d not in {64,128,256}", head_dim);
  if (n_query < 1 || n_query > 4096)
    return up::set_error(UP_ERR_UNSUPPORTED, "n_query %d not in [1, 4096]", n_query);
  up::ScoreGeometry g = up::score_geometry(num_seqs, T, max_len, hq, hkv, head_dim, n_query);
  g.ck = choose_ck(num_seqs, cu_h, hkv, g.rg_a, up::resident_wgs_for(head_dim, 0));
  if (up::has_one_round_tiling(head_dim)) {
    // pass A's one-round tiling when its chunk rule gives at most one round
    const int res1 = up::resident_wgs_for(head_dim, 1);
    const int ck1 = choose_ck(num_seqs, cu_h, hkv, g.rg_a1, res1);
    int64_t wgs1 = 0;
    for (int r = 0; r < num_seqs; ++r)
      wgs1 += up::ceil_div(cu_h[r + 1] - cu_h[r], ck1) * (int64_t)hkv * g.rg_a1;
    if (wgs1 <= res1) {
      g.one_round_a = 1;
      g.rg_a = g.rg_a1;
      g.ck = ck1;
    }
  }
  g.ck_b = choose_ck_rounds(num_seqs, cu_h, hkv, g.rg, up::resident_wgs_for(head_dim, 2), g.ck);
  if (up::has_rounds_tiling_b(head_dim)) {
    // pass B's several-rounds tiling when its own tiling needs more than one round
    int64_t wgs_b = 0;
    for (int r = 0; r < num_seqs; ++r)
      wgs_b += up::ceil_div(cu_h[r + 1] - cu_h[r], g.ck_b) * (int64_t)hkv * g.rg;
    if (wgs_b > up::resident_wgs_for(head_dim, 2)) {
      const int64_t rmax = (int64_t)(hq / hkv) * std::min(n_query, max_len);
      g.rounds_b = 1;
      g.rows_per_wg = up::rows_per_wg_for(head_dim, 3);
      g.rg = (int)(rmax > 0 ? up::ceil_div(rmax, g.rows_per_wg) : 1);
      g.ck_b = choose_ck_rounds(num_seqs, cu_h, hkv, g.rg, up::resident_wgs_for(head_dim, 3),
                                g.ck);
    }
  }
  g.max_chunks = (int)(max_len > 0 ? up::ceil_div(max_len, g.ck) : 1);
  size_t off = 0;
  g.off_partial = off;
  off = up::align_up(off + (size_t)num_seqs * hq * n_query * g.max_chunks * sizeof(float2), 256);
  g.off_colpart = off;
  off = up::align_up(off + (size_t)hkv * g.rg * (size_t)T * sizeof(float), 256);
  g.off_arrive = off;
  off = up::align_up(off + (size_t)num_seqs * sizeof(uint32_t), 256);
  g.bytes = off > 0 ? off : 256;
  out->g = g;
  out->bytes = g.bytes;
  return UP_OK;
}

}  // namespace

extern "C" {

up_status up_score_workspace_size(int num_seqs, const int32_t* cu_seqlens_h, int hq, int hkv,
                                  int head_dim, int n_query, size_t* bytes) {
  up::clear_error();
  if (bytes == nullptr) return up::set_error(UP_ERR_INVALID, "bytes is NULL");
  Layout lay;
  up_status st = score_layout(num_seqs, cu_seqlens_h, hq, hkv, head_dim, n_query, &lay);
  if (st != UP_OK) return st;
  *bytes = lay.bytes;
  return UP_OK;
}

}  // extern "C"

namespace {

// Selection arguments of the fused entry point (NULL for up_score).
struct SelectParams {
  double top_p;
  int sink, tail;
  uint8_t* block_mask;
  int32_t* kept_tokens;
};

up_status score_call(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                     const int32_t* cu_blocks_d, const void* q, int64_t q_tok_stride,
                     int64_t q_head_stride, int hq, const void* k, int64_t k_tok_stride,
                     int64_t k_head_stride, int hkv, int head_dim, int n_query, int block,
                     float scale, float* token_scores, float* block_scores, void* workspace,
                     size_t workspace_bytes, const SelectParams* sel, hipStream_t stream) {
  Layout lay;
  up_status st = score_layout(num_seqs, cu_seqlens_h, hq, hkv, head_dim, n_query, &lay);
  if (st != UP_OK) return st;
  if (block < 16 || block > 256 || (block & (block - 1)) != 0)
    return up::set_error(UP_ERR_UNSUPPORTED, "block %d is not a power of two in [16, 256]", block);
  if (!(scale >= 0.f) || !isfinite(scale))
    return up::set_error(UP_ERR_INVALID, "scale must be finite and >= 0 (0 = 1/sqrt(head_dim))");
  const int64_t T = cu_seqlens_h[num_seqs];
  int64_t N = 0;
  for (int r = 0; r < num_seqs; ++r) N += up::ceil_div(cu_seqlens_h[r + 1] - cu_seqlens_h[r], block);
  if (sel) {
    if (!(sel->top_p > 0.0 && sel->top_p <= 1.0))
      return up::set_error(UP_ERR_INVALID, "top_p not in (0, 1]");
    if (sel->sink < 0 || sel->tail < 0)
      return up::set_error(UP_ERR_INVALID, "sink and tail must be >= 0");
    if (num_seqs > 0 && (!sel->kept_tokens || !cu_seqlens_d || !cu_blocks_d))
      return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
    if (T > 0 && !sel->block_mask) return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
    int max_len = 0;
    for (int r = 0; r < num_seqs; ++r) max_len = std::max(max_len, cu_seqlens_h[r + 1] - cu_seqlens_h[r]);
    if (up::ceil_div(max_len, block) > up::kMaxBlocksPerRequest)
      return up::set_error(UP_ERR_UNSUPPORTED, "%lld blocks in one request > %lld",
                           (long long)up::ceil_div(max_len, block),
                           (long long)up::kMaxBlocksPerRequest);
  }
  if (num_seqs == 0) return UP_OK;
  if (T == 0) {
    // nothing to score; every request keeps 0 tokens
    if (!sel) return UP_OK;
    st = up::check_device();
    if (st != UP_OK) return st;
    hipLaunchKernelGGL(up::up_zero_kernel, dim3((unsigned)up::ceil_div(num_seqs, 256)), dim3(256), 0,
                       stream, sel->kept_tokens, num_seqs);
    return up::check_launch("up_zero_kernel");
  }
  if (!cu_seqlens_d || !cu_blocks_d || !q || !k || !block_scores || !workspace)
    return up::set_error(UP_ERR_INVALID, "a required pointer is NULL");
  if (((uintptr_t)q & 15) || ((uintptr_t)k & 15) || (q_tok_stride & 7) || (q_head_stride & 7) ||
      (k_tok_stride & 7) || (k_head_stride & 7))
    return up::set_error(UP_ERR_UNSUPPORTED,
                         "q/k must be 16-byte aligned with strides that are multiples of 8 elements");
  if (q_tok_stride < 0 || q_head_stride < 0 || k_tok_stride < 0 || k_head_stride < 0)
    return up::set_error(UP_ERR_INVALID, "negative stride");
  if (k_tok_stride > (int64_t(1) << 24))
    return up::set_error(UP_ERR_UNSUPPORTED, "k_tok_stride %lld > 2^24 elements",
                         (long long)k_tok_stride);
  if ((uintptr_t)workspace & 255) return up::set_error(UP_ERR_INVALID, "workspace not 256-byte aligned");
  if (workspace_bytes < lay.bytes)
    return up::set_error(UP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes,
                         lay.bytes);
  st = up::check_device();
  if (st != UP_OK) return st;

  up::ScoreArgs a{};
  char* ws = static_cast<char*>(workspace);
  a.cu_seqlens = cu_seqlens_d;
  a.cu_blocks = cu_blocks_d;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.q_tok = q_tok_stride;
  a.q_head = q_head_stride;
  a.k_tok = k_tok_stride;
  a.k_head = k_head_stride;
  a.num_seqs = num_seqs;
  a.hq = hq;
  a.hkv = hkv;
  a.rgqa = hq / hkv;
  a.n_query = n_query;
  a.block = block;
  a.ck = lay.g.ck;
  a.max_chunks = lay.g.max_chunks;
  a.rg = lay.g.rg;
  a.rows_per_wg = lay.g.rows_per_wg;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)head_dim);
  a.c = sc * 1.4426950408889634f;
  a.partial = reinterpret_cast<float2*>(ws + lay.g.off_partial);
  a.colpart = reinterpret_cast<float*>(ws + lay.g.off_colpart);
  a.T = T;
  a.token_scores = token_scores;
  a.block_scores = block_scores;
  a.num_blocks = N;
  a.arrive = reinterpret_cast<uint32_t*>(ws + lay.g.off_arrive);
  a.kept = sel ? sel->kept_tokens : nullptr;
  const int ck_b = lay.g.ck_b;

  a.num_groups = 0;
  int64_t groups_b = 0;
  bool one_a = true, one_b = true;
  for (int r = 0; r < num_seqs; ++r) {
    const int L = cu_seqlens_h[r + 1] - cu_seqlens_h[r];
    a.num_groups += up::ceil_div(L, a.ck) * (int64_t)hkv;
    groups_b += up::ceil_div(L, ck_b) * (int64_t)hkv;
    one_a = one_a && L >= 1 && L <= a.ck;
    one_b = one_b && L >= 1 && L <= ck_b;
  }
  a.one_chunk = one_a ? 1 : 0;
  const int one_chunk_b = one_b ? 1 : 0;
  const int64_t rgm = a.rg > lay.g.rg_a ? a.rg : lay.g.rg_a;
  const int64_t nwg = up::ceil_div(std::max(a.num_groups, groups_b), 8) * 8 * rgm;
  if (nwg > 0x7fffffff) return up::set_error(UP_ERR_UNSUPPORTED, "grid too large");
  switch (head_dim) {
    case 64:
      st = up::launch_passes<64>(a, lay.g.rg_a, lay.g.one_round_a, lay.g.rounds_b, ck_b, groups_b,
                                   one_chunk_b,
                                   stream);
      break;
    case 128:
      st = up::launch_passes<128>(a, lay.g.rg_a, lay.g.one_round_a, lay.g.rounds_b, ck_b, groups_b,
                                   one_chunk_b,
                                   stream);
      break;
    default:
      st = up::launch_passes<256>(a, lay.g.rg_a, lay.g.one_round_a, lay.g.rounds_b, ck_b, groups_b,
                                   one_chunk_b,
                                   stream);
      break;
  }
  if (st != UP_OK) return st;
  if (sel) {
    const up::SelectArgs sa{cu_seqlens_d, cu_blocks_d, block_scores, sel->block_mask,
                            sel->kept_tokens, block, sel->sink, sel->tail, sel->top_p};
    hipLaunchKernelGGL(up::up_blockmean_select_kernel,
                       dim3((unsigned)up::ceil_div(N, up::kSelectThreads / 64 * up::kFusedBlocksPerWave)),
                       dim3(up::kSelectThreads), 0, stream, a, sa);
    return up::check_launch("up_blockmean_select_kernel");
  }
  hipLaunchKernelGGL(up::up_blockmean_kernel, dim3((unsigned)up::ceil_div(N, 4)), dim3(256), 0,
                     stream, a);
  return up::check_launch("up_blockmean_kernel");
}

}  // namespace

extern "C" {

up_status up_score(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                   const int32_t* cu_blocks_d, const void* q, int64_t q_tok_stride,
                   int64_t q_head_stride, int hq, const void* k, int64_t k_tok_stride,
                   int64_t k_head_stride, int hkv, int head_dim, int n_query, int block, float scale,
                   float* token_scores, float* block_scores, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  up::clear_error();
  return score_call(num_seqs, cu_seqlens_h, cu_seqlens_d, cu_blocks_d, q, q_tok_stride,
                    q_head_stride, hq, k, k_tok_stride, k_head_stride, hkv, head_dim, n_query, block,
                    scale, token_scores, block_scores, workspace, workspace_bytes, nullptr, stream);
}

up_status up_score_select(int num_seqs, const int32_t* cu_seqlens_h, const int32_t* cu_seqlens_d,
                          const int32_t* cu_blocks_d, const void* q, int64_t q_tok_stride,
                          int64_t q_head_stride, int hq, const void* k, int64_t k_tok_stride,
                          int64_t k_head_stride, int hkv, int head_dim, int n_query, int block,
                          float scale, float* token_scores, float* block_scores, double top_p,
                          int sink, int tail, uint8_t* block_mask, int32_t* kept_tokens,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  up::clear_error();
  const SelectParams sel{top_p, sink, tail, block_mask, kept_tokens};
  return score_call(num_seqs, cu_seqlens_h, cu_seqlens_d, cu_blocks_d, q, q_tok_stride,
                    q_head_stride, hq, k, k_tok_stride, k_head_stride, hkv, head_dim, n_query, block,
                    scale, token_scores, block_scores, workspace, workspace_bytes, &sel, stream);
}


}  // extern "C"
