"""GPU parity of the fused pipeline (the next layer reads the kept rows
through the compaction's row map, §二 step 3): the RMS-normalised operand
and the residual sum against the oracle, on ragged batches with empty
requests and partial blocks, every element type, packed and strided rows.

Tolerances: the residual sum is bit-exact (fp32 addition of two values of a
16-bit format, or of two fp32 values, rounded once, is the correctly rounded
sum).  The normalised operand is computed in fp32 and rounded once to the
element type: |gpu - exact| <= ulp/2 + rel*|exact| with rel bounding the fp32
error of the sum of squares (a lane's sequential sum over D/64 products, then
a 64-lane butterfly), of rsqrt and of the two products:
rel = (D/64 + 16) * 2^-24.
"""
import numpy as np
import pytest
import torch

import oracle as O
import token_block_sparsification_amd as U
from _parity import FMT_OF, check_rounded, to_f64

pytestmark = pytest.mark.gpu

LENS = [0, 3, 64, 65, 1000, 0, 2049, 130]


def _batch(G, lens=LENS):
    dev = torch.device("cuda")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    return U.Batch.make(cu, G, dev), cu.numpy()


def _rows(T, D, dtype, gen, strided):
    """N(0,1) rows with per-row scales over four decades (what a residual
    stream looks like), optionally inside a wider strided buffer."""
    x = torch.randn(T, D + (24 if strided else 0), generator=gen, dtype=torch.float64)
    x *= torch.exp(torch.empty(T, 1, dtype=torch.float64).uniform_(-4.6, 4.6, generator=gen))
    x = x.to(dtype).cuda()
    return x[:, :D] if strided else x


def _report(name, **kv):
    print(f"[fused] {name}: " + ", ".join(f"{k}={v}" for k, v in kv.items()), flush=True)


@pytest.mark.parametrize("dtype,D,G,strided,gain,residual", [
    (torch.bfloat16, 4096, 64, False, True, False),
    (torch.bfloat16, 2048, 32, True, True, True),
    (torch.float16, 1024, 16, False, False, True),
    (torch.float32, 512, 64, False, True, True),
    (torch.bfloat16, 8192, 128, False, True, False),
    (torch.float32, 4, 32, True, False, False),
    (torch.bfloat16, 200, 256, True, True, True)])
def test_compact_rmsnorm(dtype, D, G, strided, gain, residual):
    batch, cu = _batch(G)
    T = batch.num_tokens
    dev = torch.device("cuda")
    gen = torch.Generator().manual_seed(D + G)
    hidden = _rows(T, D, dtype, gen, strided)
    gamma = torch.randn(D, generator=gen).to(dtype).cuda() if gain else None
    pos = (torch.arange(T, dtype=torch.int32) * 5 + 3).cuda()
    ws = U.new_compact_workspace(batch.cu_seqlens_h, G, dev)
    fmt = FMT_OF[dtype]
    x64 = to_f64(hidden)
    g64 = to_f64(gamma) if gain else None
    for frac, eps in ((0.5, 1e-6), (1.0, 1e-5), (0.0, 1e-6), (0.8, 0.0)):
        mask_np = (torch.rand(batch.num_blocks, generator=gen) < frac).numpy().astype(np.uint8)
        mask = torch.from_numpy(mask_np).to(dev)
        normed = torch.full((T, D), 7, dtype=dtype, device=dev)
        res = torch.full((T, D), 7, dtype=dtype, device=dev) if residual else None
        pout = torch.full((T,), -1, dtype=torch.int32, device=dev)
        cu_out = torch.empty(len(cu), dtype=torch.int32, device=dev)
        U.up_compact_rmsnorm(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask,
                             hidden, gamma, eps, pos, normed, res, pout, cu_out, ws)
        torch.cuda.synchronize()
        y, p_ref, cu_ref = O.compact_rmsnorm(mask_np, x64, pos.cpu().numpy(), cu, G, g64, eps)
        n = len(p_ref)
        assert list(cu_out.cpu().numpy()) == list(cu_ref)
        assert np.array_equal(pout[:n].cpu().numpy(), p_ref) and (pout[n:] == -1).all()
        exact = check_rounded(to_f64(normed[:n]), y, fmt, (D / 64 + 16) * 2.0 ** -24, "normed")
        assert (normed[n:] == 7).all()   # nothing past the kept rows
        if residual:
            keep = torch.from_numpy(np.flatnonzero(O.token_keep(mask_np, cu, G))).to(dev)
            assert torch.equal(res[:n], hidden.index_select(0, keep)) and (res[n:] == 7).all()
        assert not ws.view(torch.int32)[:2].any()
        _report(f"rmsnorm {fmt} D={D} G={G}", frac=frac, rows=n, exactly_rounded=f"{exact:.4f}")


@pytest.mark.parametrize("dtype,D,G,strided", [
    (torch.bfloat16, 4096, 64, False), (torch.float16, 2048, 32, True),
    (torch.float32, 512, 16, False), (torch.bfloat16, 8, 128, True)])
def test_gather_add(dtype, D, G, strided):
    batch, cu = _batch(G)
    T = batch.num_tokens
    dev = torch.device("cuda")
    gen = torch.Generator().manual_seed(D * 3 + G)
    frozen = _rows(T, D, dtype, gen, strided)
    ws = U.new_compact_workspace(batch.cu_seqlens_h, G, dev)
    fmt = FMT_OF[dtype]
    f64 = to_f64(frozen)
    for frac in (0.6, 1.0, 0.0):
        mask_np = (torch.rand(batch.num_blocks, generator=gen) < frac).numpy().astype(np.uint8)
        mask = torch.from_numpy(mask_np).to(dev)
        n = int(O.token_keep(mask_np, cu, G).sum())
        delta = _rows(max(n, 1), D, dtype, gen, False)
        out = torch.full((max(n, 1), D), 7, dtype=dtype, device=dev)
        U.up_gather_add(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, frozen,
                        delta, out, ws)
        torch.cuda.synchronize()
        ref = O.gather_add(mask_np, f64, to_f64(delta), cu, G, fmt)
        assert np.array_equal(to_f64(out[:n]), ref)
        # in place: out is delta
        d2 = delta.clone()
        U.up_gather_add(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, frozen,
                        d2, d2, ws)
        torch.cuda.synchronize()
        assert torch.equal(d2[:n], out[:n])
        assert not ws.view(torch.int32)[:2].any()
        _report(f"gather_add {fmt} D={D} G={G}", frac=frac, rows=n)


def test_gather_add_short_output():
    """out_rows below the kept count: kept blocks that fit are summed, the
    first block that would end past out_rows and every later one are
    skipped, and nothing past out_rows is written."""
    G = 32
    batch, cu = _batch(G)
    T = batch.num_tokens
    dev = torch.device("cuda")
    gen = torch.Generator().manual_seed(99)
    frozen = _rows(T, 64, torch.bfloat16, gen, False)
    mask_np = np.ones(batch.num_blocks, dtype=np.uint8)
    mask = torch.from_numpy(mask_np).to(dev)
    ws = U.new_compact_workspace(batch.cu_seqlens_h, G, dev)
    rows = 1100   # inside request 4's blocks (rows 132 .. 1132)
    big = torch.full((rows + 8, 64), 3, dtype=torch.bfloat16, device=dev)
    delta = big[:rows]
    U.up_gather_add(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, frozen,
                    delta, delta, ws)
    torch.cuda.synchronize()
    # block ends in request-then-token order; the last one <= rows is where writing stops
    ends = []
    for b in range(len(cu) - 1):
        L = int(cu[b + 1] - cu[b])
        ends += [int(cu[b]) + min(j + G, L) for j in range(0, L, G)]
    stop = max(e for e in ends if e <= rows)
    ref = to_f64(frozen[:stop]) + 3.0
    assert np.array_equal(to_f64(delta[:stop]), O.round_to_format(ref, "bf16"))
    assert (big[stop:] == 3).all()


SEL_CASES = [
    ("ragged_d128", dict(lengths=(0, 1, 63, 64, 65, 127, 128, 129, 300, 0, 1000, 2500, 4097), hq=8,
                         hkv=2, head_dim=128, n_query=128, block=64)),
    ("many_small_d64", dict(lengths=tuple([17, 0, 40, 33] * 40), hq=4, hkv=4, head_dim=64,
                            n_query=32, block=16)),
    ("long_d256", dict(lengths=(20000, 3000), hq=16, hkv=2, head_dim=256, n_query=128, block=128)),
    # a request of 4375 blocks: more than the selection stages in LDS
    ("many_blocks_d64", dict(lengths=(70000, 100), hq=2, hkv=1, head_dim=64, n_query=16, block=16)),
    # column-sum chunks of 320 keys: 256-token blocks straddle chunks
    ("straddling_chunks_G256", dict(lengths=(9000, 7000, 5000, 12000, 3000), hq=8, hkv=2,
                                 head_dim=128, n_query=128, block=256)),
]


@pytest.mark.parametrize("name,kw", SEL_CASES, ids=[c[0] for c in SEL_CASES])
def test_score_select_matches_two_calls(name, kw):
    """Selection run by the block-mean kernel (the workgroup that writes a
    request's last block mean; one workgroup's blocks may span several
    requests, some empty): scores, mask and kept counts are
    bit-identical to up_score followed by up_select_topp, and the mask and
    counts agree with the oracle's selection on the GPU's block scores.  The
    same workspace then serves a second, smaller batch (the arrival counters
    restart every call)."""
    import workloads as W
    dev = torch.device("cuda")
    lengths = kw.pop("lengths")
    w = W.Workload(name=name, lengths=lengths, hidden_dim=16, hidden_dtype="bf16",
                   seed=7100 + len(lengths), plant_frac=0.05, num_seqs=len(lengths), **kw)
    p, sink, tail = 0.9, 64, 64
    ws = None
    for sub in (None, lengths[: max(1, len(lengths) // 2)]):
        inp = W.make_inputs(w, lengths=sub, with_hidden=False)
        cu = inp["cu_seqlens"]
        G = w.block
        batch = U.Batch.make(cu, G, dev)
        q, k = inp["q"].to(dev), inp["k"].to(dev)
        T, N, B = batch.num_tokens, batch.num_blocks, batch.num_seqs
        need = U.up_score_workspace_size(cu, w.hq, w.hkv, w.head_dim, w.n_query)
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
        assert ws.numel() >= need
        out = {}
        for fused in (False, True):
            ts = torch.full((T,), -1.0, device=dev)
            bs = torch.full((max(N, 1),), -1.0, device=dev)
            mask = torch.full((max(N, 1),), 9, dtype=torch.uint8, device=dev)
            kept = torch.full((B,), -1, dtype=torch.int32, device=dev)
            if fused:
                U.up_score_select(cu, batch.cu_seqlens_d, batch.cu_blocks_d, q, k, w.n_query, G, 0.0,
                                  ts, bs, p, sink, tail, mask, kept, ws)
            else:
                U.up_score(cu, batch.cu_seqlens_d, batch.cu_blocks_d, q, k, w.n_query, G, 0.0, ts,
                           bs, ws)
                U.up_select_topp(cu, batch.cu_seqlens_d, batch.cu_blocks_d, bs, G, p, sink, tail,
                                 mask, kept)
            torch.cuda.synchronize()
            out[fused] = (ts.cpu(), bs.cpu(), mask.cpu(), kept.cpu())
        for a, b in zip(out[False], out[True]):
            assert torch.equal(a, b)
        cun = cu.numpy()
        ref_mask, ref_kept = O.select_topp(out[True][1][:N].double().numpy(), cun, G, p, sink, tail)
        assert np.array_equal(out[True][2][:N].numpy(), ref_mask)
        assert list(out[True][3].numpy()) == list(ref_kept)
        _report(f"score_select {name}", T=T, N=N, B=B, kept=int(ref_kept.sum()))
