"""Plain, slow, fp64 CPU oracle of the UniPrefill pruning path.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
baseline).  Nothing in the GPU library imports or links this file.

Source: the UniPrefill article page "中国科学院与腾讯微信合作解决AI排队等待问题"
(CAS Institute of Automation / UCAS / Tencent WeChat, arXiv 2605.06221).
Section references below (§二, §三, Q&A) are to that page.

What is computed (each step is the plain definition, no blocking or fusion):

1. Importance estimation (§二 step 1; Q&A 1): the last n tokens of a request
   act as queries and attend over every key of the request.  For query head h
   (KV head g = h // (Hq/Hkv)) and tail row i, p_{h,i,j} = softmax_j(s) with
   s_j = scale * <q_{h,i}, k_{g,j}> over keys j <= i (causal).  The page's
   "online normalisation" (§三) is an exact reformulation of this softmax, so
   the oracle uses the dense definition.
2. Per-token score c_j = sum over heads and tail rows of p_{h,i,j} (§二 step 1;
   §三: per-head local scores are summed into one global score).
3. Block score = mean of c_j over each block of G consecutive tokens of the
   request, the last block possibly shorter (§二 step 2).
4. Top-p selection (§二 step 2; Q&A 1): the blocks overlapping the first
   `sink` or the last `tail` tokens are always kept (§二, exempt blocks); the
   remaining blocks are taken in descending score order (ties: lower index
   first) until the kept mass reaches p of the total mass.  The output is a
   binary block mask (§三).
5. Compaction (§二 step 3; §三): the rows of kept blocks are gathered in their
   original order (hidden states and positions), giving the packed kept batch
   and its cu_seqlens; each request's drop record gets (layer id, kept tokens)
   appended (§三, drop-history ledger).

Readings where the page is silent are listed in the repository's design
notes; the ones that change numbers are restated at each function.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# Input helpers
# ---------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> exact fp64 values.

    bf16 is the upper half of an IEEE binary32 word, so the widening is exact.
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def tail_range(L: int, n: int) -> Tuple[int, int]:
    """Request-local tail query rows [L - n_eff, L) with n_eff = min(n, L).

    §二 step 1: the last n tokens are the queries.  A request shorter than n
    uses all of its tokens (reading: n_eff = min(n, L)).
    """
    n_eff = min(int(n), int(L))
    return L - n_eff, L


# ---------------------------------------------------------------------------
# Steps 1-2: tail-query attention probabilities and per-token scores
# ---------------------------------------------------------------------------

def tail_attention_probs(q_tail: np.ndarray, keys: np.ndarray, row0: int,
                         scale: float) -> np.ndarray:
    """Softmax rows of the tail queries of ONE head over the request's keys.

    q_tail: [n_eff, d] fp64, rows are request-local positions row0 .. row0+n_eff-1
    keys:   [L, d] fp64
    Returns P [n_eff, L] with P[t, j] = exp(s_tj - max) / sum, and 0 for j > row0+t
    (§二 step 1: tail queries attend to all tokens; causal reading: a query at
    position i sees keys j <= i).
    """
    n_eff, L = q_tail.shape[0], keys.shape[0]
    s = scale * (q_tail @ keys.T)                       # [n_eff, L] dot products
    rows = row0 + np.arange(n_eff)[:, None]
    cols = np.arange(L)[None, :]
    s = np.where(cols <= rows, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def token_scores(q: np.ndarray, k: np.ndarray, cu_seqlens: Sequence[int], n_query: int,
                 scale: Optional[float] = None, heads: Optional[Sequence[int]] = None,
                 return_rowsums: bool = False):
    """Per-token importance scores c [T] (fp64).

    q: [T, Hq, d], k: [T, Hkv, d] fp64 (bf16 inputs widened exactly).
    scale defaults to 1/sqrt(d) (reading: the layer's own attention scale).
    GQA reading: query head h reads KV head h // (Hq // Hkv).
    heads: optional subset of query heads to sum over (used for the additivity
    check of §三: per-head local scores summed across devices).
    """
    T, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    r = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    c = np.zeros(T, dtype=np.float64)
    rowsums = []
    hs = range(hq) if heads is None else heads
    for b in range(len(cu_seqlens) - 1):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        L = s1 - s0
        if L == 0:
            continue
        lo, hi = tail_range(L, n_query)
        for h in hs:
            g = h // r
            P = tail_attention_probs(q[s0 + lo:s0 + hi, h, :], k[s0:s1, g, :], lo, scale)
            c[s0:s1] += P.sum(axis=0)
            if return_rowsums:
                rowsums.append(P.sum(axis=1))
    if return_rowsums:
        return c, rowsums
    return c


# ---------------------------------------------------------------------------
# Step 3: block means
# ---------------------------------------------------------------------------

def block_offsets(cu_seqlens: Sequence[int], G: int) -> np.ndarray:
    """cu_blocks[B+1]: request r owns blocks cu_blocks[r] .. cu_blocks[r+1]-1,
    ceil(L_r / G) of them."""
    out = [0]
    for b in range(len(cu_seqlens) - 1):
        L = int(cu_seqlens[b + 1]) - int(cu_seqlens[b])
        out.append(out[-1] + (L + G - 1) // G)
    return np.asarray(out, dtype=np.int64)


def block_scores(c: np.ndarray, cu_seqlens: Sequence[int], G: int) -> np.ndarray:
    """Mean token score of each G-token block (§二 step 2).

    Blocks are request-local: [bG, min(bG+G, L)).  The last block of a request
    may be shorter; its mean is over the tokens it has (reading).
    """
    cub = block_offsets(cu_seqlens, G)
    out = np.zeros(int(cub[-1]), dtype=np.float64)
    for b in range(len(cu_seqlens) - 1):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        L = s1 - s0
        for blk in range(int(cub[b + 1] - cub[b])):
            j0, j1 = blk * G, min(blk * G + G, L)
            out[cub[b] + blk] = c[s0 + j0:s0 + j1].sum() / (j1 - j0)
    return out


# ---------------------------------------------------------------------------
# Step 4: Top-p selection with forced sink / tail blocks
# ---------------------------------------------------------------------------

def forced_blocks(L: int, G: int, sink: int, tail: int) -> np.ndarray:
    """Blocks exempt from pruning (§二 step 2, last paragraph; Q&A 1).

    A block is forced when it overlaps the first `sink` tokens or the last
    `tail` tokens of the request (reading: block granularity).
    """
    nb = (L + G - 1) // G
    f = np.zeros(nb, dtype=bool)
    for b in range(nb):
        j0, j1 = b * G, min(b * G + G, L)
        f[b] = (j0 < sink) or (j1 > L - tail)
    return f


def select_request(bs: np.ndarray, L: int, G: int, p: float, sink: int, tail: int) -> np.ndarray:
    """Keep mask of one request's blocks (§二 step 2).

    Reading: forced blocks count toward the mass; optional blocks are added in
    (score desc, index asc) order while the kept mass is below p * total, so
    the kept set is the smallest one that contains the forced blocks and holds
    at least p of the mass (inclusive threshold).
    """
    bs = np.asarray(bs, dtype=np.float64)
    nb = len(bs)
    forced = forced_blocks(L, G, sink, tail)
    assert len(forced) == nb
    total = 0.0
    for x in bs:                      # sequential, index order
        total += float(x)
    target = p * total
    keep = forced.copy()
    acc = 0.0
    for b in range(nb):
        if forced[b]:
            acc += float(bs[b])
    order = sorted((b for b in range(nb) if not forced[b]), key=lambda b: (-float(bs[b]), b))
    for b in order:
        if acc >= target:
            break
        keep[b] = True
        acc += float(bs[b])
    return keep


def select_topp(bscores: np.ndarray, cu_seqlens: Sequence[int], G: int, p: float,
                sink: int, tail: int) -> Tuple[np.ndarray, np.ndarray]:
    """Binary block mask [N] (uint8) and kept token count per request [B]."""
    cub = block_offsets(cu_seqlens, G)
    mask = np.zeros(int(cub[-1]), dtype=np.uint8)
    kept = np.zeros(len(cu_seqlens) - 1, dtype=np.int64)
    for b in range(len(cu_seqlens) - 1):
        L = int(cu_seqlens[b + 1]) - int(cu_seqlens[b])
        keep = select_request(bscores[cub[b]:cub[b + 1]], L, G, p, sink, tail)
        mask[cub[b]:cub[b + 1]] = keep
        for blk in np.flatnonzero(keep):
            kept[b] += min(blk * G + G, L) - blk * G
    return mask, kept


def selection_trace(bs: np.ndarray, L: int, G: int, p: float, sink: int, tail: int):
    """The selection order and the cumulative mass fraction before/after each
    optional block: (order, frac_before, frac_after, forced).  Used by the
    parity rule that exempts blocks whose cumulative mass straddles p."""
    bs = np.asarray(bs, dtype=np.float64)
    forced = forced_blocks(L, G, sink, tail)
    total = float(sum(float(x) for x in bs))
    acc = float(sum(float(bs[b]) for b in range(len(bs)) if forced[b]))
    order = sorted((b for b in range(len(bs)) if not forced[b]), key=lambda b: (-float(bs[b]), b))
    before, after = [], []
    for b in order:
        before.append(acc / total if total > 0 else 0.0)
        acc += float(bs[b])
        after.append(acc / total if total > 0 else 0.0)
    return order, np.asarray(before), np.asarray(after), forced


def band_blocks(bs: np.ndarray, L: int, G: int, p: float, sink: int, tail: int,
                eps: float = 1e-4) -> np.ndarray:
    """Optional blocks whose cumulative-mass interval [C_{k-1}, C_k] meets
    [p - eps, p + eps]: their keep/drop decision is a knife edge."""
    order, before, after, _ = selection_trace(bs, L, G, p, sink, tail)
    band = np.zeros(len(bs), dtype=bool)
    for b, c0, c1 in zip(order, before, after):
        if c1 >= p - eps and c0 <= p + eps:
            band[b] = True
    return band


# ---------------------------------------------------------------------------
# Step 5: compaction and the drop-history ledger
# ---------------------------------------------------------------------------

def token_keep(mask: np.ndarray, cu_seqlens: Sequence[int], G: int) -> np.ndarray:
    """Per-token keep flag: token j of request r inherits its block's bit."""
    cub = block_offsets(cu_seqlens, G)
    T = int(cu_seqlens[-1])
    keep = np.zeros(T, dtype=bool)
    for b in range(len(cu_seqlens) - 1):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        for j in range(s1 - s0):
            keep[s0 + j] = bool(mask[cub[b] + j // G])
    return keep


def compact(mask: np.ndarray, hidden: np.ndarray, positions: np.ndarray,
            cu_seqlens: Sequence[int], G: int):
    """Gather kept rows in original order (§二 step 3: dropped tokens are
    skipped by later layers, their states stay frozen in the input; §三:
    positions and batch metadata are updated).  Returns (hidden_out,
    positions_out, cu_seqlens_out).  Rows are copied byte for byte."""
    cub = block_offsets(cu_seqlens, G)
    B = len(cu_seqlens) - 1
    rows = []
    cu_out = [0]
    for b in range(B):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        n = 0
        for j in range(s1 - s0):
            if mask[cub[b] + j // G]:
                rows.append(s0 + j)
                n += 1
        cu_out.append(cu_out[-1] + n)
    idx = np.asarray(rows, dtype=np.int64)
    return hidden[idx], positions[idx], np.asarray(cu_out, dtype=np.int64)


def scatter_back(mask: np.ndarray, packed: np.ndarray, full: np.ndarray,
                 cu_seqlens: Sequence[int], G: int) -> np.ndarray:
    """Revival (§二 step 3: dropped tokens are frozen, kept aside so that they
    can be brought back when needed).  Reading: the kept rows, packed in
    original order as compaction produced them (possibly updated by later
    layers since), are written back to their own rows of the full-length
    buffer; rows of dropped blocks keep their frozen contents.  Returns the
    new full buffer; the arguments are not modified."""
    cub = block_offsets(cu_seqlens, G)
    out = full.copy()
    r = 0
    for b in range(len(cu_seqlens) - 1):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        for j in range(s1 - s0):
            if mask[cub[b] + j // G]:
                out[s0 + j] = packed[r]
                r += 1
    return out


# ---------------------------------------------------------------------------
# Fused pipeline: the next layer reads the kept rows itself
# ---------------------------------------------------------------------------
#
# §二 step 3 says the later layers work on the kept tokens only while the
# dropped tokens' states stay frozen.  The consumer of the kept rows is the
# next layer, whose input passes through an RMS normalisation (pre-norm) and
# whose output is added back onto the residual stream.  Reading taken: with
# the gather folded into those two reads, the next layer's normalised operand
# and its residual sum are the same numbers as normalising / adding the
# compacted rows, so the oracle states them as compaction followed by the
# plain definition of each operation.

# (significant bits, smallest normal exponent, largest exponent) per format
_FORMATS = {"bf16": (8, -126, 127), "f16": (11, -14, 15), "f32": (24, -126, 127)}


def round_to_format(x, fmt: str) -> np.ndarray:
    """Nearest value of a binary floating-point format for every element of
    the fp64 array x, ties to even, subnormals kept, overflow to infinity
    (IEEE 754 round-to-nearest-even); returned as fp64.  fmt is "bf16"
    (8 significant bits), "f16" (11) or "f32" (24)."""
    p, emin, emax = _FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # |x| in [2^(e-1), 2^e)
    q = np.maximum(e - p, emin - p + 1)      # exponent of the last kept bit
    y = np.ldexp(np.round(np.ldexp(x, -q)), q)  # np.round: half to even
    top = (2.0 - 2.0 ** (1 - p)) * 2.0 ** emax
    return np.where(np.abs(y) > top, np.copysign(np.inf, x), y)


def rms_normalize(rows: np.ndarray, gamma: Optional[np.ndarray], eps: float) -> np.ndarray:
    """RMS normalisation of each row in fp64: y = x / sqrt(mean(x^2) + eps),
    times the per-column gain gamma when one is given."""
    rows = np.asarray(rows, dtype=np.float64)
    ms = (rows * rows).sum(axis=1, keepdims=True) / rows.shape[1]
    y = rows / np.sqrt(ms + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)[None, :]
    return y


def compact_rmsnorm(mask: np.ndarray, hidden: np.ndarray, positions: np.ndarray,
                    cu_seqlens: Sequence[int], G: int, gamma: Optional[np.ndarray], eps: float):
    """The next layer's normalised operand, read straight from the frozen
    rows: the kept rows in order (compact), each RMS-normalised in fp64.
    Returns (normalised rows fp64 before rounding, positions_out,
    cu_seqlens_out); round_to_format gives the stored values."""
    h, p_out, cu_out = compact(mask, hidden, positions, cu_seqlens, G)
    return rms_normalize(h, gamma, eps), p_out, cu_out


def gather_add(mask: np.ndarray, frozen: np.ndarray, delta: np.ndarray,
               cu_seqlens: Sequence[int], G: int, fmt: str) -> np.ndarray:
    """The next layer's residual sum, reading the residual from the frozen
    rows: out[i] = frozen[i-th kept row] + delta[i], rounded once to fmt.
    Inputs are fp64 arrays holding values of fmt; their fp64 sum is rounded
    to nearest-even.  (A kernel that adds in fp32 and then rounds to bf16 or
    f16 gets the same values: fp32 carries at least 2p + 2 bits for those
    formats, so the second rounding is innocuous.)"""
    T = int(cu_seqlens[-1])
    h, _, _ = compact(mask, np.asarray(frozen, dtype=np.float64), np.zeros(T, dtype=np.int32),
                      cu_seqlens, G)
    d = np.asarray(delta, dtype=np.float64)[: len(h)]
    return round_to_format(h + d, fmt)


def history_new(num_seqs: int) -> List[list]:
    """Empty drop-history ledger: one list of (layer_id, kept) per request."""
    return [[] for _ in range(num_seqs)]


def history_append(ledger: List[list], layer_id: int, cu_out: Sequence[int]) -> None:
    """Append (layer id, kept tokens) for every request (§三, drop-history ledger)."""
    for b in range(len(ledger)):
        ledger[b].append((int(layer_id), int(cu_out[b + 1]) - int(cu_out[b])))


def history_kv_len(entries: Sequence[Tuple[int, int]], layer: int, full_len: int) -> int:
    """KV entries a layer wrote for one request, read back from its ledger (§三:
    at generation time the ledger tells each layer how many cache entries it
    holds).  Reading: a drop at layer l already applies to layer l itself, so
    the length is the kept count of the latest entry with layer id <= `layer`,
    or the full prompt length when there is none."""
    best = None
    for lid, kept in entries:
        if lid <= layer and (best is None or lid >= best[0]):
            best = (lid, kept)
    return full_len if best is None else best[1]


def run_chain(q, k, hidden, positions, cu_seqlens, n_query=128, G=64, p=0.99, sink=128,
              tail=128, scale=None, layer_id=0):
    """The whole path on one batch; returns a dict of every intermediate."""
    c = token_scores(q, k, cu_seqlens, n_query, scale)
    bsc = block_scores(c, cu_seqlens, G)
    mask, kept = select_topp(bsc, cu_seqlens, G, p, sink, tail)
    h_out, p_out, cu_out = compact(mask, hidden, positions, cu_seqlens, G)
    ledger = history_new(len(cu_seqlens) - 1)
    history_append(ledger, layer_id, cu_out)
    return dict(token_scores=c, block_scores=bsc, mask=mask, kept=kept, hidden_out=h_out,
                positions_out=p_out, cu_out=cu_out, ledger=ledger)
