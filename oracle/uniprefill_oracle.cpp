// Plain, slow, single-threaded C++17 CPU oracle of the UniPrefill token-block
// pruning path, in double precision throughout.
//
// TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
// baseline call it through oracle/cxx.py.  It shares no code with the GPU
// library (it is compiled by g++ on the CPU and includes no HIP header).
//
// Source: the UniPrefill article page "中国科学院与腾讯微信合作解决AI排队等待问题"
// (CAS Institute of Automation / UCAS / Tencent WeChat, arXiv 2605.06221).
// Section marks below (§二, §三, Q&A 1) refer to that page.  Every step is the
// plain definition, with no blocking, fusion or reordering:
//   1. importance estimation: the last n tokens of a request attend over its
//      keys with a softmax per query row (§二 step 1; §三 names the online
//      normalisation, an exact reformulation of this softmax);
//   2. per-token score: the probabilities summed over query rows and heads
//      (§二 step 1; §三: per-head scores are summed);
//   3. block score: the mean token score of each block of G tokens (§二 step 2);
//   4. Top-p: the blocks overlapping the first `sink` or last `tail` tokens are
//      kept, then the others in descending score order until the kept mass
//      reaches p of the total (§二 step 2, Q&A 1); the result is a binary mask
//      (§三);
//   5. compaction of the kept rows and positions in their original order, and
//      one (layer id, kept tokens) ledger entry per request (§二 step 3, §三).
// Readings where the page is silent (scale 1/sqrt(d), causal tail rows,
// n_eff = min(n, L), GQA head h -> KV head h / (Hq/Hkv), block-granular
// forced keeps, forced mass counted toward p, inclusive threshold, ties by
// lower index) are those of the repository's design notes.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// Element (t, h, c) of a [T, H, d] tensor given as fp64 (kind 0) or as bf16
// bit patterns (kind 1); bf16 is the upper half of an IEEE binary32 word, so
// widening it is exact.
double element(const void* base, int kind, int64_t tok_stride, int64_t head_stride, int64_t t,
               int64_t h, int64_t c) {
  const int64_t i = t * tok_stride + h * head_stride + c;
  if (kind == 0) return static_cast<const double*>(base)[i];
  const uint32_t bits = static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return static_cast<double>(f);
}

}  // namespace

extern "C" {

// Steps 1-2 (§二 step 1, §三): per-token scores c[T].
// For request r (tokens cu[r] .. cu[r+1]-1, length L), n_eff = min(n_query, L)
// tail rows i in [L - n_eff, L) (request-local), each query head h in `heads`
// (all hq heads when heads is null) with KV head g = h / (hq / hkv):
//   s_j = scale * <q[i, h], k[j, g]> for keys j <= i (causal),
//   p_j = exp(s_j - max_j s) / sum_j exp(s_j - max_j s),
//   c[j] += p_j.
// scale <= 0 selects 1/sqrt(d).  Returns 0, or -1 for hq not a multiple of hkv.
int uo_token_scores(int num_seqs, const int64_t* cu, const void* q, int q_kind, int64_t q_tok,
                    int64_t q_head, int hq, const void* k, int k_kind, int64_t k_tok,
                    int64_t k_head, int hkv, int d, int n_query, double scale,
                    const int32_t* heads, int num_heads, double* c) {
  if (hkv < 1 || hq % hkv != 0) return -1;
  const int group = hq / hkv;
  if (!(scale > 0.0)) scale = 1.0 / std::sqrt(static_cast<double>(d));
  std::fill(c, c + cu[num_seqs], 0.0);
  const int nh = heads ? num_heads : hq;
  std::vector<double> s;
  for (int r = 0; r < num_seqs; ++r) {
    const int64_t s0 = cu[r], L = cu[r + 1] - cu[r];
    if (L == 0) continue;
    const int64_t n_eff = std::min<int64_t>(n_query, L);
    for (int hi = 0; hi < nh; ++hi) {
      const int h = heads ? heads[hi] : hi;
      const int g = h / group;
      for (int64_t i = L - n_eff; i < L; ++i) {
        s.assign(static_cast<size_t>(i + 1), 0.0);
        double m = -HUGE_VAL;
        for (int64_t j = 0; j <= i; ++j) {
          double dot = 0.0;
          for (int t = 0; t < d; ++t)
            dot += element(q, q_kind, q_tok, q_head, s0 + i, h, t) *
                   element(k, k_kind, k_tok, k_head, s0 + j, g, t);
          s[j] = scale * dot;
          m = std::max(m, s[j]);
        }
        double l = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
          s[j] = std::exp(s[j] - m);
          l += s[j];
        }
        for (int64_t j = 0; j <= i; ++j) c[s0 + j] += s[j] / l;
      }
    }
  }
  return 0;
}

// Step 3 (§二 step 2): block_scores[N] = mean of c over each request-local
// block [b G, min(b G + G, L)) (the last block of a request may be shorter).
void uo_block_scores(int num_seqs, const int64_t* cu, const double* c, int G, double* out) {
  int64_t nb = 0;
  for (int r = 0; r < num_seqs; ++r) {
    const int64_t s0 = cu[r], L = cu[r + 1] - cu[r];
    for (int64_t b = 0; b * G < L; ++b) {
      const int64_t j0 = b * G, j1 = std::min<int64_t>(j0 + G, L);
      double sum = 0.0;
      for (int64_t j = j0; j < j1; ++j) sum += c[s0 + j];
      out[nb++] = sum / static_cast<double>(j1 - j0);
    }
  }
}

// Forced blocks of a request of length L (§二 step 2, Q&A 1): a block is kept
// without competing when it overlaps the first `sink` or the last `tail` tokens.
void uo_forced_blocks(int64_t L, int G, int sink, int tail, uint8_t* out) {
  for (int64_t b = 0; b * G < L; ++b) {
    const int64_t j0 = b * G, j1 = std::min<int64_t>(j0 + G, L);
    out[b] = (j0 < sink || j1 > L - tail) ? 1 : 0;
  }
}

// Step 4 for one request (§二 step 2): keep the forced blocks, then add the
// others in (score desc, index asc) order while the kept mass is below
// p * total (the total summed in index order); keep[b] = 1 for kept blocks.
void uo_select_request(const double* bs, int64_t L, int G, double p, int sink, int tail,
                       uint8_t* keep) {
  const int64_t nb = (L + G - 1) / G;
  uo_forced_blocks(L, G, sink, tail, keep);
  double total = 0.0;
  for (int64_t b = 0; b < nb; ++b) total += bs[b];
  const double target = p * total;
  double acc = 0.0;
  std::vector<int64_t> order;
  for (int64_t b = 0; b < nb; ++b) {
    if (keep[b]) acc += bs[b];
    else order.push_back(b);
  }
  std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    return bs[a] > bs[b] || (bs[a] == bs[b] && a < b);
  });
  for (int64_t b : order) {
    if (acc >= target) break;
    keep[b] = 1;
    acc += bs[b];
  }
}

// Step 4 over the batch: block_mask[N] and kept tokens per request.
void uo_select_topp(int num_seqs, const int64_t* cu, const double* bs, int G, double p, int sink,
                    int tail, uint8_t* mask, int64_t* kept) {
  int64_t nb0 = 0;
  for (int r = 0; r < num_seqs; ++r) {
    const int64_t L = cu[r + 1] - cu[r], nb = (L + G - 1) / G;
    uo_select_request(bs + nb0, L, G, p, sink, tail, mask + nb0);
    kept[r] = 0;
    for (int64_t b = 0; b < nb; ++b)
      if (mask[nb0 + b]) kept[r] += std::min<int64_t>(b * G + G, L) - b * G;
    nb0 += nb;
  }
}

// Step 5 (§二 step 3, §三): the rows of kept blocks, request by request and
// token by token in their original order, copied byte for byte with their
// positions (when given); cu_out[B+1] is the packing of the kept batch.
void uo_compact(int num_seqs, const int64_t* cu, int G, const uint8_t* mask, const uint8_t* hidden,
                int64_t row_bytes, const int32_t* positions, uint8_t* hidden_out,
                int32_t* positions_out, int64_t* cu_out) {
  int64_t nb0 = 0, dst = 0;
  cu_out[0] = 0;
  for (int r = 0; r < num_seqs; ++r) {
    const int64_t s0 = cu[r], L = cu[r + 1] - cu[r];
    for (int64_t j = 0; j < L; ++j) {
      if (!mask[nb0 + j / G]) continue;
      std::memcpy(hidden_out + dst * row_bytes, hidden + (s0 + j) * row_bytes,
                  static_cast<size_t>(row_bytes));
      if (positions) positions_out[dst] = positions[s0 + j];
      ++dst;
    }
    cu_out[r + 1] = dst;
    nb0 += (L + G - 1) / G;
  }
}

// Step 5, ledger (§三): the entry each request's drop record gets from this
// layer, (layer id, kept tokens), as entries[2 r], entries[2 r + 1].
void uo_history_entries(int num_seqs, int layer_id, const int64_t* cu_out, int64_t* entries) {
  for (int r = 0; r < num_seqs; ++r) {
    entries[2 * r] = layer_id;
    entries[2 * r + 1] = cu_out[r + 1] - cu_out[r];
  }
}

}  // extern "C"
