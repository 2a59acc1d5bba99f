"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each check cites what fixes its expected value: a closed form, a textbook or
library routine, an invariant of the definition on the UniPrefill page
("中国科学院与腾讯微信合作解决AI排队等待问题", §二 / §三 / Q&A 1), brute force on
tiny inputs, or the hand-worked example under tests/golden/.

The checks are plain functions so that test_oracle_mutations.py can re-run
them against deliberately broken copies of the oracle.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.uniprefill_oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_qk(seed, lengths, hq, hkv, d, dist_scale=1.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q = rng.standard_normal((T, hq, d)) * dist_scale
    k = rng.standard_normal((T, hkv, d)) * dist_scale
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, cu


# ---------------------------------------------------------------------------
# Scoring (steps 1-2)
# ---------------------------------------------------------------------------

def check_rows_sum_to_one():
    """Invariant: every softmax row sums to 1, so each request's token scores
    sum to Hq * n_eff (n_eff = min(n, L))."""
    lengths = [300, 50, 129, 1, 128]
    q, k, cu = _rand_qk(1, lengths, 4, 2, 16)
    c = O.token_scores(q, k, cu, 128)
    for b, L in enumerate(lengths):
        s = c[cu[b]:cu[b + 1]].sum()
        assert abs(s - 4 * min(128, L)) < 1e-9 * 4 * 128, (b, s)
    assert np.all(c >= 0)


def check_against_sdpa():
    """Library routine: torch's scaled_dot_product_attention (fp64, math path)
    with V = identity returns the attention probability matrix itself; summing
    it over heads and query rows gives the per-token score.  Pins the softmax
    scale (1/sqrt(d)), the causal offset of the tail rows, the GQA head
    mapping (torch repeats each KV head over consecutive query heads) and the
    operand orientation."""
    for (lengths, hq, hkv, d, n) in [([97, 200], 6, 2, 8, 40), ([64], 4, 4, 16, 64),
                                     ([33], 8, 2, 4, 128)]:
        q, k, cu = _rand_qk(7 + d, lengths, hq, hkv, d)
        c = O.token_scores(q, k, cu, n)
        for b, L in enumerate(lengths):
            s0 = cu[b]
            lo = L - min(n, L)
            qt = torch.from_numpy(q[s0 + lo:s0 + L]).permute(1, 0, 2)[None]       # [1,hq,n,d]
            kk = torch.from_numpy(k[s0:s0 + L]).permute(1, 0, 2)[None]           # [1,hkv,L,d]
            v = torch.eye(L, dtype=torch.float64).expand(1, hkv, L, L).contiguous()
            rows = torch.arange(lo, L)[:, None]
            mask = torch.arange(L)[None, :] <= rows
            P = F.scaled_dot_product_attention(qt.contiguous(), kk.contiguous(), v,
                                               attn_mask=mask, enable_gqa=True)
            ref = P.sum(dim=(0, 1, 2)).numpy()
            np.testing.assert_allclose(c[s0:s0 + L], ref, rtol=1e-10, atol=1e-13)


def check_equal_keys_harmonic():
    """Closed form: with all keys equal every visible key gets the same logit,
    so row i (request-local) is uniform over its i+1 keys and
    c_j = Hq * sum_{i = max(j, L-n_eff)}^{L-1} 1/(i+1).  Pins causality in the
    tail, n_eff = min(n, L) and request offsets in a packed batch."""
    lengths = [10, 300, 5]
    hq, hkv, d, n = 4, 2, 8, 7
    rng = np.random.default_rng(3)
    T = sum(lengths)
    q = rng.standard_normal((T, hq, d))
    k = np.tile(rng.standard_normal((1, hkv, d)), (T, 1, 1))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    c = O.token_scores(q, k, cu, n)
    for b, L in enumerate(lengths):
        ne = min(n, L)
        for j in range(L):
            exp = hq * sum(1.0 / (i + 1) for i in range(max(j, L - ne), L))
            assert abs(c[cu[b] + j] - exp) < 1e-12, (b, j, c[cu[b] + j], exp)


def check_hand_example():
    """Closed form worked by hand: L=4, d=1, one head, n=2, scale 1.
    q = [*, *, 1, 2], k = [0, 1, 0, 1].
    Row 2 sees logits [0, 1, 0]     -> [1, e, 1] / (2 + e)
    Row 3 sees logits [0, 2, 0, 2]  -> [1, e^2, 1, e^2] / (2 + 2 e^2)."""
    e = math.e
    q = np.array([0.0, 0.0, 1.0, 2.0]).reshape(4, 1, 1)
    k = np.array([0.0, 1.0, 0.0, 1.0]).reshape(4, 1, 1)
    c = O.token_scores(q, k, [0, 4], 2, scale=1.0)
    a, bb = 2 + e, 2 + 2 * e * e
    expect = [1 / a + 1 / bb, e / a + e * e / bb, 1 / a + 1 / bb, e * e / bb]
    np.testing.assert_allclose(c, expect, rtol=1e-14)
    # default scale for d = 4 is 1/2: scaled copy must reproduce the same values
    q4 = np.zeros((4, 1, 4)); q4[:, 0, 0] = q[:, 0, 0] * 2.0
    k4 = np.zeros((4, 1, 4)); k4[:, 0, 0] = k[:, 0, 0]
    np.testing.assert_allclose(O.token_scores(q4, k4, [0, 4], 2), expect, rtol=1e-14)


def check_gqa_peak():
    """Special case: one nonzero query head aligned with a distinct planted key
    in each KV head.  With Hq=4, Hkv=2 the consecutive mapping sends query
    head 1 to KV head 0 (an interleaved mapping would send it to KV head 1)."""
    L, d = 40, 8
    q = np.zeros((L, 4, d))
    k = np.zeros((L, 2, d))
    k[5, 0, 0] = 10.0      # KV head 0 peak at token 5
    k[9, 1, 0] = 10.0      # KV head 1 peak at token 9
    q[:, 1, 0] = 10.0      # only query head 1 is informative
    c = O.token_scores(q, k, [0, L], 8)
    assert int(np.argmax(c)) == 5
    # heads with q = 0 are uniform over visible keys; head 1 puts ~all its mass on key 5
    assert c[5] > 8 * 0.99 and c[9] < 3 * 8 / 33 + 1e-9


def check_head_additivity():
    """Invariant (§三: per-head local scores summed into a global score): the
    scores of disjoint head subsets add up to the full score."""
    q, k, cu = _rand_qk(11, [150, 70], 8, 2, 8)
    full = O.token_scores(q, k, cu, 64)
    parts = [O.token_scores(q, k, cu, 64, heads=hs) for hs in ([0, 1, 2], [3], [4, 5, 6, 7])]
    np.testing.assert_allclose(sum(parts), full, rtol=1e-12, atol=1e-15)


def check_n1_textbook_softmax():
    """Special case n = 1, one head: the score vector is the textbook softmax of
    the last query's logits (scipy.special.softmax)."""
    from scipy.special import softmax
    q, k, cu = _rand_qk(5, [57], 1, 1, 16)
    c = O.token_scores(q, k, cu, 1)
    ref = softmax((k[:, 0, :] @ q[-1, 0, :]) / 4.0)
    np.testing.assert_allclose(c, ref, rtol=1e-12)


# ---------------------------------------------------------------------------
# Block means (step 3)
# ---------------------------------------------------------------------------

def check_block_means():
    """Closed form: block means of c_j = j (request-local), including a short
    last block: block b of a request with L tokens has mean
    (j0 + j1 - 1) / 2 over [j0, j1) = [bG, min(bG+G, L))."""
    lengths = [10, 8, 0, 3]
    G = 4
    c = np.concatenate([np.arange(L, dtype=np.float64) for L in lengths])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    bs = O.block_scores(c, cu, G)
    expect = []
    for L in lengths:
        for b in range((L + G - 1) // G):
            j0, j1 = b * G, min(b * G + G, L)
            expect.append((j0 + j1 - 1) / 2.0)
    np.testing.assert_array_equal(bs, np.array(expect))
    np.testing.assert_array_equal(O.block_offsets(cu, G), [0, 3, 5, 5, 6])


# ---------------------------------------------------------------------------
# Selection (step 4)
# ---------------------------------------------------------------------------

def _load_select_golden():
    path = os.path.join(GOLDEN, "select_worked_example.txt")
    meta, rows = {}, []
    for line in open(path, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if "|" in line:
            p, m, kept = [x.strip() for x in line.split("|")]
            rows.append((float(p), [int(x) for x in m.split()], int(kept)))
        else:
            key, *vals = line.split()
            meta[key] = [float(v) for v in vals]
    return meta, rows


def check_select_golden():
    """Hand-worked example (tests/golden/select_worked_example.txt)."""
    meta, rows = _load_select_golden()
    L, G = int(meta["L"][0]), int(meta["G"][0])
    sink, tail = int(meta["SINK"][0]), int(meta["TAIL"][0])
    bs = np.array(meta["SCORES"])
    for p, m, kept in rows:
        mask, kt = O.select_topp(bs, [0, L], G, p, sink, tail)
        assert list(mask) == m, (p, list(mask), m)
        assert int(kt[0]) == kept


def check_one_hot():
    """Closed form: one-hot scores keep exactly the forced blocks plus the hot block."""
    L, G = 64 * 40, 64
    for hot in (5, 17, 30):
        bs = np.zeros(40)
        bs[hot] = 1.0
        keep = O.select_request(bs, L, G, 0.99, 128, 128)
        expect = O.forced_blocks(L, G, 128, 128).copy()
        expect[hot] = True
        assert np.array_equal(keep, expect), hot


def check_uniform_ceil():
    """Closed form: with equal scores and ceil(pN) >= |F|, the kept set has
    exactly ceil(pN) blocks (e.g. N = 2048, p = 0.99 -> 2028)."""
    for N, p in ((2048, 0.99), (512, 0.99), (100, 0.9), (1000, 0.95)):
        bs = np.full(N, 3.0)
        keep = O.select_request(bs, N * 64, 64, p, 128, 128)
        expect = math.ceil(p * N - 1e-9)
        assert keep.sum() == expect, (N, p, keep.sum(), expect)
        # ties are broken towards lower block index
        order = np.flatnonzero(keep)
        opt = [b for b in order if not O.forced_blocks(N * 64, 64, 128, 128)[b]]
        assert opt == list(range(2, 2 + len(opt)))


def check_select_invariants():
    """Invariants (§二 step 2: the dropped share of the mass is at most 1 - p;
    the kept set is minimal; exempt blocks are kept)."""
    rng = np.random.default_rng(21)
    for trial in range(60):
        N = int(rng.integers(1, 300))
        L = N * 64 - int(rng.integers(0, 64))
        bs = rng.exponential(1.0, N) ** rng.uniform(0.2, 4)
        p = float(rng.choice([0.5, 0.9, 0.99, 0.999]))
        keep = O.select_request(bs, L, 64, p, 128, 128)
        forced = O.forced_blocks(L, 64, 128, 128)
        total = bs.sum()
        assert np.all(keep[forced])
        assert bs[keep].sum() >= p * total * (1 - 1e-12)
        opt_kept = [b for b in np.flatnonzero(keep) if not forced[b]]
        if opt_kept:
            lowest = min(opt_kept, key=lambda b: (bs[b], -b))
            assert bs[keep].sum() - bs[lowest] < p * total * (1 + 1e-12)
            # every dropped block scores no higher than every kept optional block
            dropped = np.flatnonzero(~keep)
            if len(dropped):
                assert bs[dropped].max() <= bs[opt_kept].min()


def check_brute_force():
    """Brute force: for N <= 20 (at most 16 optional blocks) enumerate every
    superset of the forced set; the oracle's set must have minimum size among
    sets holding >= p of the mass, and maximum mass among those; when that set
    is unique it is the oracle's."""
    rng = np.random.default_rng(99)
    for trial in range(40):
        N = int(rng.integers(1, 21))
        L = N * 16
        sink, tail, G = 16, 16, 16
        bs = np.round(rng.exponential(1.0, N) * 8) / 8 + (rng.random(N) < 0.2) * 0
        p = float(rng.choice([0.5, 0.8, 0.95, 0.99]))
        forced = O.forced_blocks(L, G, sink, tail)
        opt = [b for b in range(N) if not forced[b]]
        total = bs.sum()
        best = None
        for r in range(len(opt) + 1):
            feas = []
            for sub in itertools.combinations(opt, r):
                s = np.array(forced)
                s[list(sub)] = True
                if bs[s].sum() >= p * total:
                    feas.append(s)
            if feas:
                masses = [bs[s].sum() for s in feas]
                mx = max(masses)
                best = [s for s, m in zip(feas, masses) if m == mx]
                break
        keep = O.select_request(bs, L, G, p, sink, tail)
        assert best is not None
        assert keep.sum() == best[0].sum()
        assert bs[keep].sum() == max(bs[s].sum() for s in best)
        if len(best) == 1:
            assert np.array_equal(keep, best[0])


def check_scale_invariance():
    """Invariant: multiplying every score by 2^k (exact in binary floating
    point) leaves the mask unchanged."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        N = int(rng.integers(5, 400))
        bs = rng.exponential(1.0, N)
        keep = O.select_request(bs, N * 64, 64, 0.99, 128, 128)
        for kexp in (-20, -1, 3, 30):
            assert np.array_equal(keep, O.select_request(bs * 2.0 ** kexp, N * 64, 64, 0.99, 128, 128))


def check_concentration():
    """Property (§二 step 2: concentrated attention keeps fewer blocks than
    dispersed attention): sharpening the scores never keeps more blocks."""
    rng = np.random.default_rng(8)
    for _ in range(20):
        N = 256
        base = rng.exponential(1.0, N)
        counts = [O.select_request(base ** a, N * 64, 64, 0.9, 128, 128).sum() for a in (0.0, 1.0, 3.0, 8.0)]
        assert counts == sorted(counts, reverse=True), counts


def check_short_requests():
    """Special case: when L <= sink + tail every block is forced and kept;
    an empty request has no blocks."""
    for L in (1, 63, 64, 65, 200, 256):
        nb = (L + 63) // 64
        bs = np.random.default_rng(L).random(nb)
        keep = O.select_request(bs, L, 64, 0.5, 128, 128)
        assert keep.all()
        mask, kept = O.select_topp(bs, [0, L], 64, 0.5, 128, 128)
        assert int(kept[0]) == L     # all tokens kept, including a short last block
    mask, kept = O.select_topp(np.zeros(0), [0, 0], 64, 0.99, 128, 128)
    assert len(mask) == 0 and int(kept[0]) == 0


# ---------------------------------------------------------------------------
# Compaction and ledger (step 5)
# ---------------------------------------------------------------------------

def check_compaction():
    """Invariants: the output count is sum(mask_b * |b|); with positions equal
    to the request-local token index the output positions are exactly the
    kept indices (numpy.flatnonzero of the token flags), rows are byte copies
    in order; an all-kept mask is an identity copy."""
    rng = np.random.default_rng(4)
    lengths = [130, 0, 64, 200, 1]
    G = 32
    cu = np.concatenate([[0], np.cumsum(lengths)])
    cub = O.block_offsets(cu, G)
    mask = (rng.random(int(cub[-1])) < 0.6).astype(np.uint8)
    T = int(cu[-1])
    hidden = rng.integers(0, 2 ** 16, size=(T, 12), dtype=np.uint16)
    pos = np.concatenate([np.arange(L) for L in lengths]).astype(np.int32)
    h_out, p_out, cu_out = O.compact(mask, hidden, pos, cu, G)
    exp_count = 0
    flat = []
    for b, L in enumerate(lengths):
        for blk in range(int(cub[b + 1] - cub[b])):
            size = min(blk * G + G, L) - blk * G
            if mask[cub[b] + blk]:
                exp_count += size
                flat.extend(range(cu[b] + blk * G, cu[b] + blk * G + size))
        assert cu_out[b + 1] - cu_out[b] == sum(
            min(blk * G + G, L) - blk * G for blk in range(int(cub[b + 1] - cub[b])) if mask[cub[b] + blk])
    assert cu_out[-1] == exp_count == len(h_out)
    np.testing.assert_array_equal(h_out, hidden[np.array(flat, dtype=np.int64)])
    np.testing.assert_array_equal(p_out, pos[np.array(flat, dtype=np.int64)])
    keepflags = O.token_keep(mask, cu, G)
    np.testing.assert_array_equal(np.flatnonzero(keepflags), np.array(flat))
    ones = np.ones_like(mask)
    h2, p2, c2 = O.compact(ones, hidden, pos, cu, G)
    np.testing.assert_array_equal(h2, hidden)
    np.testing.assert_array_equal(c2, cu)


def check_revival():
    """Revival undoes compaction: scattering the packed kept rows back over the
    original buffer gives the original buffer; over any other buffer it gives
    the kept rows in their own places and that buffer's rows elsewhere.  A
    hand example fixes the order: G=2, one request of 5 tokens, blocks
    {0,1}, {2,3}, {4} with mask 1, 0, 1 -> packed rows p0, p1, p2 land in rows
    0, 1 and 4."""
    base = np.array([[10.0], [11.0], [12.0], [13.0], [14.0]])
    packed = np.array([[0.5], [1.5], [2.5]])
    out = O.scatter_back(np.array([1, 0, 1], dtype=np.uint8), packed, base, [0, 5], 2)
    np.testing.assert_array_equal(out[:, 0], [0.5, 1.5, 12.0, 13.0, 2.5])
    np.testing.assert_array_equal(base[:, 0], [10.0, 11.0, 12.0, 13.0, 14.0])  # input untouched
    rng = np.random.default_rng(7)
    lengths = [130, 0, 64, 200, 1, 33]
    G = 32
    cu = np.concatenate([[0], np.cumsum(lengths)])
    cub = O.block_offsets(cu, G)
    T = int(cu[-1])
    x = rng.integers(0, 2 ** 16, size=(T, 5), dtype=np.uint16)
    other = rng.integers(0, 2 ** 16, size=(T, 5), dtype=np.uint16)
    pos = np.zeros(T, dtype=np.int32)
    for frac in (0.0, 0.5, 1.0):
        mask = (rng.random(int(cub[-1])) < frac).astype(np.uint8)
        h_out, _, _ = O.compact(mask, x, pos, cu, G)
        np.testing.assert_array_equal(O.scatter_back(mask, h_out, x, cu, G), x)
        keep = O.token_keep(mask, cu, G).astype(bool)
        np.testing.assert_array_equal(O.scatter_back(mask, h_out, other, cu, G),
                                      np.where(keep[:, None], x, other))


def check_history():
    """Ledger invariants: one entry per request per call, in call order; the
    KV length a layer reads back is the kept count of the latest drop at or
    below it, else the full prompt length."""
    led = O.history_new(3)
    O.history_append(led, 3, [0, 10, 10, 25])
    O.history_append(led, 7, [0, 4, 4, 20])
    assert led == [[(3, 10), (7, 4)], [(3, 0), (7, 0)], [(3, 15), (7, 16)]]
    assert O.history_kv_len(led[0], 0, 99) == 99
    assert O.history_kv_len(led[0], 3, 99) == 10
    assert O.history_kv_len(led[0], 6, 99) == 10
    assert O.history_kv_len(led[0], 7, 99) == 4
    assert O.history_kv_len(led[2], 100, 99) == 16


def check_chain_composition():
    """run_chain is the composition of the pinned steps with its arguments in
    their places: scores with n_query tail rows, block means over G, selection
    with (p, sink, tail), compaction over G, one ledger entry per request
    carrying layer_id.  The parameters are chosen pairwise distinct (n=40,
    G=16, sink=32, tail=80, layer 9) so that a swapped or dropped argument
    changes some output."""
    lengths = [300, 17, 0, 129]
    q, k, cu = _rand_qk(11, lengths, 6, 3, 8)
    T = int(cu[-1])
    rng = np.random.default_rng(12)
    hidden = rng.integers(0, 2 ** 16, size=(T, 5), dtype=np.uint16)
    pos = np.concatenate([np.arange(L) for L in lengths]).astype(np.int32)
    n, G, p, sink, tail, layer = 40, 16, 0.8, 32, 80, 9
    out = O.run_chain(q, k, hidden, pos, cu, n_query=n, G=G, p=p, sink=sink, tail=tail,
                      layer_id=layer)
    c = O.token_scores(q, k, cu, n)
    bs = O.block_scores(c, cu, G)
    mask, kept = O.select_topp(bs, cu, G, p, sink, tail)
    h, po, cuo = O.compact(mask, hidden, pos, cu, G)
    np.testing.assert_array_equal(out["token_scores"], c)
    np.testing.assert_array_equal(out["block_scores"], bs)
    np.testing.assert_array_equal(out["mask"], mask)
    np.testing.assert_array_equal(out["kept"], kept)
    np.testing.assert_array_equal(out["hidden_out"], h)
    np.testing.assert_array_equal(out["positions_out"], po)
    np.testing.assert_array_equal(out["cu_out"], cuo)
    assert out["ledger"] == [[(layer, int(cuo[b + 1] - cuo[b]))] for b in range(len(lengths))]
    assert 0 < int(cuo[-1]) < T      # the example really drops blocks


def check_chain_hand_example():
    """Whole path worked by hand.  Two requests, L = 8 and 3, one head, d = 1,
    every key equal (so each tail row is uniform over the keys it sees),
    n = 3, G = 2, p = 0.7, sink = 3, tail = 1, layer id 5.

    Request 0: tail rows 5, 6, 7 see 6, 7, 8 keys, so in units of 1/168
    c_0..c_5 = 28+24+21 = 73, c_6 = 24+21 = 45, c_7 = 21.  Blocks {0,1},
    {2,3}, {4,5}, {6,7} score 73, 73, 73, 33; total 252, target 0.7*252 =
    176.4.  Forced: blocks 0 and 1 (start below sink 3) and block 3 (overlaps
    the last token), mass 179 >= 176.4, so block 2 is dropped: 6 tokens kept,
    rows 0, 1, 2, 3, 6, 7.  (With sink and tail swapped blocks 0, 2, 3 would
    be forced instead and block 1 dropped.)
    Request 1 (shorter than n, all three rows are tail rows): c = 11/6, 5/6,
    1/3; blocks {0,1}, {2} score 4/3, 1/3; both start below sink 3, so both
    are kept: 3 tokens.
    Ledger: (5, 6) and (5, 3); cu_seqlens_out = [0, 6, 9]."""
    q = np.array([0.3, -1.0, 2.0, 0.5, 1.5, -0.7, 0.9, 1.1, 0.2, -0.4, 0.8]).reshape(11, 1, 1)
    k = np.full((11, 1, 1), 0.6)
    cu = [0, 8, 11]
    hidden = np.arange(11, dtype=np.int64).reshape(11, 1) * 10
    pos = np.array([0, 1, 2, 3, 4, 5, 6, 7, 0, 1, 2], dtype=np.int32)
    out = O.run_chain(q, k, hidden, pos, cu, n_query=3, G=2, p=0.7, sink=3, tail=1, layer_id=5)
    c0 = np.array([73, 73, 73, 73, 73, 73, 45, 21]) / 168.0
    c1 = np.array([11 / 6, 5 / 6, 1 / 3])
    np.testing.assert_allclose(out["token_scores"], np.concatenate([c0, c1]), rtol=1e-14)
    np.testing.assert_allclose(out["block_scores"],
                               [73 / 168, 73 / 168, 73 / 168, 33 / 168, 4 / 3, 1 / 3], rtol=1e-14)
    np.testing.assert_array_equal(out["mask"], [1, 1, 0, 1, 1, 1])
    np.testing.assert_array_equal(out["kept"], [6, 3])
    np.testing.assert_array_equal(out["hidden_out"][:, 0], [0, 10, 20, 30, 60, 70, 80, 90, 100])
    np.testing.assert_array_equal(out["positions_out"], [0, 1, 2, 3, 6, 7, 0, 1, 2])
    np.testing.assert_array_equal(out["cu_out"], [0, 6, 9])
    assert out["ledger"] == [[(5, 6)], [(5, 3)]]


def check_widen_bf16():
    """bf16 widening agrees with torch's own bf16 -> fp64 conversion."""
    x = torch.randn(10000, dtype=torch.float64).to(torch.bfloat16)
    x[:4] = torch.tensor([0.0, -0.0, 1e-38, -3.0e38]).to(torch.bfloat16)
    np.testing.assert_array_equal(O.widen_bf16(x.view(torch.int16).numpy()), x.to(torch.float64).numpy())


def check_knife_edge_band():
    """The parity rule's band, on a hand-worked request: G = 1, no forced
    blocks, scores 4, 3, 2, 1 (total 10) give cumulative fractions 0.4, 0.7,
    0.9, 1.0 in (score desc) order; at p = 0.7 the blocks whose interval
    meets [p - 1e-4, p + 1e-4] are the second and third; at p = 0.55 only the
    second; with blocks 0 and 3 forced (sink 1, tail 1) the optional order
    starts from their mass fraction 0.4."""
    bs = np.array([1.0, 4.0, 2.0, 3.0])          # block index order; ranks 3, 0, 2, 1
    order, c0, c1, forced = O.selection_trace(bs, 4, 1, 0.7, 0, 0)
    assert order == [1, 3, 2, 0] and not forced.any()
    np.testing.assert_allclose(c0, [0.0, 0.4, 0.7, 0.9])
    np.testing.assert_allclose(c1, [0.4, 0.7, 0.9, 1.0])
    assert list(np.flatnonzero(O.band_blocks(bs, 4, 1, 0.7, 0, 0))) == [2, 3]
    assert list(np.flatnonzero(O.band_blocks(bs, 4, 1, 0.55, 0, 0))) == [3]
    order, c0, c1, forced = O.selection_trace(bs, 4, 1, 0.7, 1, 1)
    assert list(np.flatnonzero(forced)) == [0, 3] and order == [1, 2]
    np.testing.assert_allclose(c0, [0.4, 0.8])
    np.testing.assert_allclose(c1, [0.8, 1.0])


def check_round_to_format():
    """Rounding to a binary format agrees with library conversions that round
    once, directly from the wider value: numpy's fp64 -> fp32 and fp64 -> f16
    casts, and torch's fp32 -> bf16 (on fp32 inputs, so one rounding);
    hand-worked ties go to the even neighbour."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-150, 130, 20000))
    x[:6] = [0.0, -0.0, 1.0, -2.5, 2.0 ** -149, 3.4e38]
    np.testing.assert_array_equal(O.round_to_format(x, "f32"), x.astype(np.float32).astype(np.float64))
    xh = rng.standard_normal(20000) * np.exp2(rng.integers(-28, 17, 20000))
    with np.errstate(over="ignore"):
        np.testing.assert_array_equal(O.round_to_format(xh, "f16"),
                                      xh.astype(np.float16).astype(np.float64))
    with np.errstate(over="ignore"):
        xb = x.astype(np.float32)
    xb = xb[np.isfinite(xb)]
    tb = torch.from_numpy(xb).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_format(xb.astype(np.float64), "bf16"), tb)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2.0 ** -134])
    np.testing.assert_array_equal(O.round_to_format(ties, "bf16"), [1.0, 1 + 2.0 ** -6, -1.0, 0.0])
    np.testing.assert_array_equal(O.round_to_format(np.array([1 + 2.0 ** -11, 65520.0]), "f16"),
                                  [1.0, np.inf])


def check_rmsnorm():
    """RMS normalisation: torch.nn.functional.rms_norm in fp64 (library
    routine) with a gain and eps; a constant row c gives c / sqrt(c^2 + eps)
    times the gain (closed form); with eps = 0 every output row has mean
    square exactly 1 and scaling a row by a positive factor leaves it
    unchanged (invariants)."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((37, 96)) * rng.uniform(0.01, 30, (37, 1))
    g = rng.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(O.rms_normalize(x, g, 1e-5), ref, rtol=1e-12, atol=1e-12)
    c = np.full((2, 8), [[3.0], [-0.5]])
    np.testing.assert_allclose(O.rms_normalize(c, g[:8], 0.25),
                               c / np.sqrt(c * c + 0.25) * g[:8], rtol=1e-14)
    y = O.rms_normalize(x, None, 0.0)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(O.rms_normalize(x * 7.5, None, 0.0), y, rtol=1e-13)


def check_compact_rmsnorm():
    """The fused operand is the normalisation of exactly the kept rows, in
    order: a hand example (G = 2, one request of 5 tokens, mask 1, 0, 1 keeps
    rows 0, 1, 4), and with every block kept it equals torch's rms_norm of
    the whole input (gain included)."""
    x = np.array([[3.0, 4.0], [1.0, 0.0], [9.0, 9.0], [8.0, 8.0], [0.0, -2.0]])
    pos = np.array([10, 11, 12, 13, 14], dtype=np.int32)
    y, p_out, cu_out = O.compact_rmsnorm(np.array([1, 0, 1], dtype=np.uint8), x, pos, [0, 5], 2,
                                         None, 0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(y, [[3 / r, 4 / r], [math.sqrt(2), 0.0], [0.0, -math.sqrt(2)]],
                               rtol=1e-15)
    np.testing.assert_array_equal(p_out, [10, 11, 14])
    np.testing.assert_array_equal(cu_out, [0, 3])
    rng = np.random.default_rng(14)
    lengths = [70, 0, 33]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    x = rng.standard_normal((T, 16))
    g = rng.standard_normal(16)
    ones = np.ones(int(O.block_offsets(cu, 32)[-1]), dtype=np.uint8)
    y, _, c2 = O.compact_rmsnorm(ones, x, np.zeros(T, dtype=np.int32), cu, 32, g, 1e-6)
    ref = F.rms_norm(torch.from_numpy(x), (16,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(c2, cu)


def check_gather_add():
    """Residual sum through the row map: on integer-valued rows (exact in
    every format) the output is frozen[kept token indices] + delta, the
    indices taken independently by expanding each request's block mask G
    times; with every block kept the sum equals torch's own bf16 and f16
    additions (library routines rounding the exact sum once), and adding the
    negated kept rows gives exact zeros."""
    rng = np.random.default_rng(15)
    lengths = [130, 0, 64, 7]
    G = 32
    cu = np.concatenate([[0], np.cumsum(lengths)])
    cub = O.block_offsets(cu, G)
    T = int(cu[-1])
    mask = (rng.random(int(cub[-1])) < 0.5).astype(np.uint8)
    idx = np.concatenate([cu[b] + np.flatnonzero(np.repeat(mask[cub[b]:cub[b + 1]], G)[:L])
                          for b, L in enumerate(lengths)])
    fr = rng.integers(-100, 100, (T, 6)).astype(np.float64)
    de = rng.integers(-100, 100, (T, 6)).astype(np.float64)
    np.testing.assert_array_equal(O.gather_add(mask, fr, de, cu, G, "bf16"), fr[idx] + de[:len(idx)])
    np.testing.assert_array_equal(O.gather_add(mask, fr, -fr[idx], cu, G, "f16"),
                                  np.zeros((len(idx), 6)))
    ones = np.ones(int(cub[-1]), dtype=np.uint8)
    for fmt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        a = torch.randn(T, 40, dtype=torch.float64).mul(torch.exp2(torch.randint(-12, 12, (T, 1))))
        a = a.to(tdt)
        b = torch.randn(T, 40, dtype=torch.float64).to(tdt)
        np.testing.assert_array_equal(
            O.gather_add(ones, a.to(torch.float64).numpy(), b.to(torch.float64).numpy(), cu, G, fmt),
            (a + b).to(torch.float64).numpy())


ALL_CHECKS = [
    check_rows_sum_to_one, check_against_sdpa, check_equal_keys_harmonic, check_hand_example,
    check_gqa_peak, check_head_additivity, check_n1_textbook_softmax, check_block_means,
    check_select_golden, check_one_hot, check_uniform_ceil, check_select_invariants,
    check_brute_force, check_scale_invariance, check_concentration, check_short_requests,
    check_compaction, check_revival, check_history, check_chain_composition,
    check_chain_hand_example, check_widen_bf16, check_knife_edge_band,
    check_round_to_format,
    check_rmsnorm, check_compact_rmsnorm, check_gather_add,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


# ---------------------------------------------------------------------------
# Generator sanity (the generator holds none of the method's arithmetic)
# ---------------------------------------------------------------------------

def test_splitmix_torch_matches_python():
    key = W.stream_key(1234, 2)
    idx = torch.tensor([0, 1, 2, 10 ** 9, 2 ** 40 + 7], dtype=torch.int64)
    got = [int(v) & W.gen.MASK64 for v in W.draw_u64(key, idx)]
    exp = [W.splitmix64_py((key + (int(i) + 1) * W.gen.GOLDEN) & W.gen.MASK64) for i in idx]
    assert got == exp
    # SplitMix64 published first outputs for seed 0 (state advanced by the golden gamma)
    assert W.splitmix64_py(W.gen.GOLDEN) == 0xE220A8397B1DCDAF


def test_normal_moments():
    x = W.normal(W.stream_key(7, 1), torch.arange(200000))
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1) < 0.01


def test_workload_recipes():
    w = W.get_workload("llama8b_batch16")
    L = W.make_lengths(w)
    assert len(L) == 16 and all(4096 <= x <= 131072 for x in L)
    assert L == W.make_lengths(w)   # seeded
    d = W.make_inputs(W.get_workload("small_L2048"))
    assert d["q"].shape == (2048, 4, 64) and d["k"].shape == (2048, 4, 64)
    assert torch.isnan(d["q"][:2048 - 128].float()).all()
    assert not torch.isnan(d["q"][2048 - 128:].float()).any()
    assert len(d["planted"][0]) == 3
    forced = O.forced_blocks(2048, 64, 128, 128)
    assert not any(forced[b] for b in d["planted"][0])


def test_planted_blocks_score_high():
    """Sanity only (not a pin): on the small workload the planted blocks are
    the three highest-scoring optional blocks."""
    d = W.make_inputs(W.get_workload("small_L2048"))
    q = O.widen_bf16(d["q"].view(torch.int16).numpy())
    k = O.widen_bf16(d["k"].view(torch.int16).numpy())
    c = O.token_scores(q, k, d["cu_seqlens"].numpy(), 128)
    bs = O.block_scores(c, d["cu_seqlens"].numpy(), 64)
    forced = O.forced_blocks(2048, 64, 128, 128)
    opt = [b for b in range(32) if not forced[b]]
    top3 = sorted(sorted(opt, key=lambda b: -bs[b])[:3])
    assert top3 == d["planted"][0]
