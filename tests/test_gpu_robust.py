"""GPU robustness tests of the pruning path through the C ABI.

The page's multi-GPU design (§三 of the UniPrefill page) needs every rank to
reach the same decision from the same scores, and its compaction step needs
the batch metadata to be updated exactly.  These tests check the properties
that follow: a request's results do not depend on where it sits in a packed
batch; selection is equivariant under permutations of tie-free scores and
invariant under power-of-two scaling; repeated runs are bitwise identical;
no call writes outside its output buffers; and a compaction scan whose
look-back gives up says so through its status word.
"""
import numpy as np
import pytest
import torch

import oracle as O
import token_block_sparsification_amd as U
import workloads as W
from _parity import GpuRun

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _split(inp, order):
    """The same requests packed in another order (bytes of each request unchanged)."""
    cu = inp["cu_seqlens"].tolist()
    seg = lambda t, r: t[cu[r]:cu[r + 1]]
    lengths = [cu[r + 1] - cu[r] for r in order]
    out = dict(inp)
    out["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    for key in ("q", "k", "hidden", "positions"):
        out[key] = torch.cat([seg(inp[key], r) for r in order]).contiguous()
    return out


def test_request_order_independence():
    """Each request's scores, mask, kept count, compacted rows and ledger entry
    are bitwise the same whichever order the requests are packed in."""
    w = W.get_workload("small_L2048").with_(lengths=(700, 2048, 96, 1500, 1), num_seqs=5)
    inp = W.make_inputs(w)
    order = [3, 0, 4, 2, 1]
    a = GpuRun(inp, w.n_query, w.block)
    ra = a.run(p=0.9, sink=64, tail=192, layer_id=3)
    b = GpuRun(_split(inp, order), w.n_query, w.block)
    rb = b.run(p=0.9, sink=64, tail=192, layer_id=3)
    cua, cub_ = a.batch.cu_seqlens_h.numpy(), b.batch.cu_seqlens_h.numpy()
    bka, bkb = a.batch.cu_blocks_h.numpy(), b.batch.cu_blocks_h.numpy()
    oa, ob = ra["cu_out"], rb["cu_out"]
    ha = a.ws.hidden_out.cpu()
    hb = b.ws.hidden_out.cpu()
    _, la = a.ledger_entries()
    _, lb = b.ledger_entries()
    assert 0 < oa[-1] < cua[-1]
    for j, r in enumerate(order):
        ts = lambda res, cu, i: res["token_scores"][cu[i]:cu[i + 1]]
        bs = lambda res, bk, i: res[("block_scores")][bk[i]:bk[i + 1]]
        assert np.array_equal(ts(ra, cua, r), ts(rb, cub_, j)), r
        assert np.array_equal(bs(ra, bka, r), bs(rb, bkb, j)), r
        assert np.array_equal(ra["mask"][bka[r]:bka[r + 1]], rb["mask"][bkb[j]:bkb[j + 1]]), r
        assert ra["kept"][r] == rb["kept"][j]
        assert torch.equal(ha[oa[r]:oa[r + 1]], hb[ob[j]:ob[j + 1]]), r
        assert la[r] == lb[j]


def _select(scores, cu, G, p, sink, tail):
    cu_h = torch.tensor(cu, dtype=torch.int32)
    cb, n = U.up_make_cu_blocks(cu_h, G)
    sc = torch.tensor(scores, dtype=torch.float32, device=DEV)
    mask = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    kept = torch.empty(len(cu) - 1, dtype=torch.int32, device=DEV)
    U.up_select_topp(cu_h, cu_h.to(DEV), cb.to(DEV), sc, G, p, sink, tail, mask, kept)
    torch.cuda.synchronize()
    return mask[:n].cpu().numpy(), kept.cpu().numpy()


def test_block_permutation_equivariance():
    """Tie-free scores: permuting the optional blocks' scores permutes the mask
    the same way (forced blocks stay where they are)."""
    rng = np.random.default_rng(21)
    G, p, sink, tail = 64, 0.9, 128, 128
    lengths = [131072, 5000, 64 * 37 + 5]
    cu = np.concatenate([[0], np.cumsum(lengths)]).tolist()
    cub = O.block_offsets(cu, G)
    scores = rng.permutation(int(cub[-1])).astype(np.float64) + 1.0  # distinct, exact in fp32
    scores = scores * rng.uniform(0.5, 1.5)  # still distinct after one rounding to fp32
    scores = np.float32(scores).astype(np.float64)
    assert len(np.unique(scores)) == len(scores)
    m0, k0 = _select(scores, cu, G, p, sink, tail)
    perm_scores = scores.copy()
    dest = np.arange(len(scores))
    for r, L in enumerate(lengths):
        forced = O.forced_blocks(L, G, sink, tail)
        opt = np.flatnonzero(~forced) + int(cub[r])
        pi = rng.permutation(len(opt))
        perm_scores[opt[pi]] = scores[opt]      # score of block opt[i] moves to opt[pi[i]]
        dest[opt] = opt[pi]
    m1, k1 = _select(perm_scores, cu, G, p, sink, tail)
    assert np.array_equal(m1[dest], m0)
    assert np.array_equal(k1, k0)
    assert 0 < m0.sum() < len(m0)


def test_mask_invariant_under_power_of_two_scaling():
    """Multiplying every block score by 2^k changes no decision (the GPU sums
    fixed-point masses relative to the request's largest score)."""
    rng = np.random.default_rng(22)
    G, p, sink, tail = 64, 0.95, 128, 128
    lengths = [131072, 333, 64 * 90]
    cu = np.concatenate([[0], np.cumsum(lengths)]).tolist()
    n = int(O.block_offsets(cu, G)[-1])
    scores = np.float32(rng.gamma(2.0, 1.0, n) * 1e-3).astype(np.float64)
    m0, k0 = _select(scores, cu, G, p, sink, tail)
    for k in (-40, -7, 1, 9, 60):
        m, kk = _select(np.ldexp(scores, k), cu, G, p, sink, tail)
        assert np.array_equal(m, m0), k
        assert np.array_equal(kk, k0), k


def test_determinism_full_size_20_runs():
    """The whole path at L = 131072 (Llama-3.1-8B shapes), 20 runs: every
    output bitwise identical to the first run's."""
    w = W.get_workload("llama8b_L131072")
    inp = W.make_inputs(w, device=DEV)
    run = GpuRun(inp, w.n_query, w.block, device=DEV)
    first = run.run()
    ws = run.ws
    T = run.batch.num_tokens
    h0 = ws.hidden_out.clone()
    p0 = ws.positions_out.clone()
    n = int(first["cu_out"][-1])
    assert 0 < n < T
    for i in range(19):
        res = run.run(layer_id=(i + 1) % run.cap)
        for key in ("token_scores", "block_scores", "mask", "kept", "cu_out"):
            assert np.array_equal(res[key], first[key]), (i, key)
        assert torch.equal(ws.hidden_out[:n], h0[:n]), i
        assert torch.equal(ws.positions_out[:n], p0[:n]), i


GUARD = 4096  # bytes of sentinel before and after every output buffer


def _guarded(nbytes, fill=0xA5):
    """A uint8 buffer with GUARD sentinel bytes on each side; returns (whole, middle)."""
    whole = torch.full((GUARD + max(nbytes, 1) + GUARD,), fill, dtype=torch.uint8, device=DEV)
    return whole, whole[GUARD:GUARD + max(nbytes, 1)]


def _intact(whole, nbytes, fill=0xA5):
    g = whole.cpu().numpy()
    return (g[:GUARD] == fill).all() and (g[GUARD + max(nbytes, 1):] == fill).all()


def test_guard_bands_around_every_output():
    """Sentinel bytes before and after every buffer the path writes (scores,
    mask, kept counts, compacted rows and positions, cu_seqlens_out, both
    workspaces, the ledger — also through up_compact_record, which fills its
    last record — revival target, KV lengths) are untouched."""
    w = W.get_workload("small_L2048").with_(lengths=(700, 2048, 96, 1500, 1), num_seqs=5)
    inp = W.make_inputs(w)
    G, n_q = w.block, w.n_query
    batch = U.Batch.make(inp["cu_seqlens"], G, DEV)
    T, N, B = batch.num_tokens, batch.num_blocks, batch.num_seqs
    q, k = inp["q"].to(DEV), inp["k"].to(DEV)
    hidden, pos = inp["hidden"].to(DEV), inp["positions"].to(DEV)
    D = hidden.shape[1]
    eb = hidden.element_size()
    bufs = {}

    def make(name, nbytes, dtype, shape):
        whole, mid = _guarded(nbytes)
        bufs[name] = (whole, nbytes)
        return mid[:nbytes].view(dtype).view(*shape) if nbytes else mid[:0].view(dtype)

    sw = U.up_score_workspace_size(batch.cu_seqlens_h, w.hq, w.hkv, w.head_dim, n_q)
    cw = U.up_compact_workspace_size(batch.cu_seqlens_h, G)
    score_ws = make("score_ws", sw, torch.uint8, (sw,))
    compact_ws = make("compact_ws", cw, torch.uint8, (cw,))
    compact_ws.zero_()
    U.up_compact_workspace_init(compact_ws)
    ts = make("token_scores", 4 * T, torch.float32, (T,))
    bs = make("block_scores", 4 * N, torch.float32, (N,))
    mask = make("block_mask", N, torch.uint8, (N,))
    kept = make("kept_tokens", 4 * B, torch.int32, (B,))
    h_out = make("hidden_out", T * D * eb, hidden.dtype, (T, D))
    p_out = make("positions_out", 4 * T, torch.int32, (T,))
    cu_out = make("cu_seqlens_out", 4 * (B + 1), torch.int32, (B + 1,))
    lb = U.up_history_bytes(B, 3)
    ledger = make("ledger", lb, torch.int32, (lb // 4,))
    full = make("revive_full", T * D * eb, hidden.dtype, (T, D))
    full.copy_(hidden)
    kv = make("kv_len", 4 * B, torch.int32, (B,))
    st = make("status", 4, torch.int32, (1,))
    U.up_history_init(ledger, B, 3)
    for layer in (2, 6):
        U.up_score(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, q, k, n_q, G, 0.0,
                   ts, bs, score_ws)
        U.up_select_topp(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, bs, G, 0.9, 64,
                         192, mask, kept)
        U.up_compact(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, hidden,
                     pos, h_out, p_out, cu_out, compact_ws)
        U.up_drop_history(ledger, B, 3, layer, cu_out)
    U.up_score_select(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, q, k, n_q, G,
                      0.0, ts, bs, 0.9, 64, 192, mask, kept, score_ws)
    U.up_compact_record(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, hidden,
                        pos, h_out, p_out, cu_out, compact_ws, ledger, 3, 8)
    U.up_revive(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, h_out, full,
                compact_ws)
    U.up_kv_len(ledger, B, 3, 4, batch.cu_seqlens_d, kv)
    U.up_compact_status(compact_ws, st)
    torch.cuda.synchronize()
    n = int(cu_out[-1])
    assert 0 < n < T and int(st[0]) == 0
    for name, (whole, nbytes) in bufs.items():
        assert _intact(whole, nbytes), f"{name}: bytes written outside the buffer"


def test_compact_lookback_give_up_is_reported():
    """A scan tile whose predecessor never publishes (forced from the host: the
    ticket starts at 1, so tile 0 is never claimed, and the poll limit is 8)
    gives up after its bounded wait, every kernel exits, the call returns
    UP_OK and the workspace's status word says the look-back gave up.  The
    word stays set until read and cleared; the workspace then serves a normal
    call again."""
    G = 16
    L = 4200 * G   # 4200 blocks: five scan tiles of 1024 (above 4096, so the look-back scan runs)
    cu = torch.tensor([0, L], dtype=torch.int32)
    batch = U.Batch.make(cu, G, DEV)
    gen = torch.Generator().manual_seed(5)
    hidden = torch.randint(0, 255, (L, 16), dtype=torch.uint8, generator=gen).to(DEV)
    pos = torch.arange(L, dtype=torch.int32, device=DEV)
    mask = (torch.rand(batch.num_blocks, generator=gen) < 0.7).to(torch.uint8).to(DEV)
    h_out = torch.zeros_like(hidden)
    p_out = torch.zeros_like(pos)
    cu_out = torch.zeros(2, dtype=torch.int32, device=DEV)
    ws = U.new_compact_workspace(batch.cu_seqlens_h, G, DEV)
    words = ws.view(torch.int32)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    words[0] = 1   # ticket: tile 0 is never claimed
    words[3] = 8   # poll limit
    U.up_compact(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, hidden, pos,
                 h_out, p_out, cu_out, ws)
    U.up_compact_status(ws, status, clear=False)
    torch.cuda.synchronize()
    assert int(status[0]) & 1 == 1
    assert int(words[0]) == 0 and int(words[1]) == 0      # counters restored for the next call
    U.up_compact_status(ws, status, clear=True)
    U.up_compact_status(ws, status, clear=False)
    torch.cuda.synchronize()
    assert int(status[0]) == 0                            # cleared by the read
    words[3] = 0
    U.up_compact(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, hidden, pos,
                 h_out, p_out, cu_out, ws)
    U.up_compact_status(ws, status)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    exp_h, exp_p, exp_cu = O.compact(mask.cpu().numpy(), hidden.cpu().numpy(), pos.cpu().numpy(),
                                     [0, L], G)
    n = int(exp_cu[-1])
    assert cu_out.cpu().tolist() == list(exp_cu)
    assert np.array_equal(h_out[:n].cpu().numpy(), exp_h)
    assert np.array_equal(p_out[:n].cpu().numpy(), exp_p)


def test_compact_workspace_reuse_across_tile_counts():
    """One workspace, batches of 4, then 40, then 4 scan tiles: the 40-tile
    call's status words lie where the 4-tile call wrote copy descriptors, and
    every call must still be exact (regression: stale descriptor bytes were
    once read as published prefixes)."""
    G = 16
    ws = None
    for nb, seed in ((4 * 1024 - 100, 1), (40 * 1024 - 7, 2), (4 * 1024 - 100, 3)):
        L = nb * G
        cu = torch.tensor([0, L - 5, L], dtype=torch.int32)
        batch = U.Batch.make(cu, G, DEV)
        if ws is None:
            ws = U.new_compact_workspace(torch.tensor([0, 40 * 1024 * G], dtype=torch.int32), G, DEV)
        gen = torch.Generator().manual_seed(seed)
        hidden = torch.randint(-2 ** 30, 2 ** 30, (L, 1), dtype=torch.int32, generator=gen).to(DEV)
        pos = torch.arange(L, dtype=torch.int32, device=DEV)
        mask = (torch.rand(batch.num_blocks, generator=gen) < 0.5).to(torch.uint8).to(DEV)
        h_out = torch.zeros_like(hidden)
        p_out = torch.zeros_like(pos)
        cu_out = torch.zeros(3, dtype=torch.int32, device=DEV)
        status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        U.up_compact(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, hidden,
                     pos, h_out, p_out, cu_out, ws)
        U.up_compact_status(ws, status)
        torch.cuda.synchronize()
        exp_h, exp_p, exp_cu = O.compact(mask.cpu().numpy(), hidden.cpu().numpy(),
                                         pos.cpu().numpy(), cu.tolist(), G)
        n = int(exp_cu[-1])
        assert cu_out.cpu().tolist() == list(exp_cu), nb
        assert np.array_equal(h_out[:n].cpu().numpy(), exp_h), nb
        assert np.array_equal(p_out[:n].cpu().numpy(), exp_p), nb
        assert int(status[0]) == 0, nb
