"""GPU parity of the multi-layer propagation driver (synthetic hybrid stack,
random weights): at every full-attention layer the pruning path, run on the
sequence the earlier layers left, must agree with the oracle on that layer's
own inputs (the GPU's Q, K and hidden rows); drops compose across layers, the
ledger records every drop and reads back the per-layer KV lengths.
"""
import numpy as np
import pytest
import torch

import oracle as O
import token_block_sparsification_amd as U
from token_block_sparsification_amd.stack import HybridStack, StackConfig
from _parity import bf16_to_f64, check_mask, check_rounded, check_scores

pytestmark = pytest.mark.gpu


def _inputs(cfg, lengths, seed):
    g = torch.Generator().manual_seed(seed)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    T = int(cu[-1])
    h = torch.randn(T, cfg.d_model, generator=g).to(torch.bfloat16).cuda()
    pos = torch.cat([torch.arange(L, dtype=torch.int32) for L in lengths]).cuda()
    return h, cu, pos


@pytest.mark.parametrize("top_p,fused", [(0.9, False), (0.6, False), (0.9, True), (0.6, True)])
def test_stack_layers_match_oracle(top_p, fused):
    """fused=False compacts at each pruning layer; fused=True reads the kept
    rows from the frozen buffer for the layer's normalised operand and its
    residual sum instead (no compacted copy)."""
    cfg = StackConfig(pattern="LFLLFF", d_model=256, d_ff=512, hq=4, hkv=2, head_dim=64,
                      n_query=64, block=32, top_p=top_p, sink=64, tail=64, seed=11)
    stack = HybridStack(cfg, "cuda")
    lengths = [700, 0, 300, 1500, 40]
    h, cu, pos = _inputs(cfg, lengths, 3)
    res = stack.forward(h, cu, pos, prune=True, keep_records=True, fused=fused)
    torch.cuda.synchronize()
    assert [r.layer for r in res.records] == cfg.full_layers
    ref_led = O.history_new(len(lengths))
    kept_pos = [np.arange(L) for L in lengths]    # request-local positions still alive
    for rec in res.records:
        cu_in = rec.cu_in.numpy()
        G = cfg.block
        # scores and mask from this layer's own Q and K
        q = bf16_to_f64(rec.q)
        k = bf16_to_f64(rec.k)
        c_ref = O.token_scores(q, k, cu_in, cfg.n_query)
        b_ref = O.block_scores(c_ref, cu_in, G)
        check_scores(rec.token_scores.double().cpu().numpy(), c_ref, cu_in, "token scores")
        cub = O.block_offsets(cu_in, G)
        check_scores(rec.block_scores.cpu().numpy().astype(np.float64), b_ref, cub, "block scores")
        mask = rec.mask.cpu().numpy()
        check_mask(mask, rec.block_scores.cpu().numpy().astype(np.float64), cu_in, G, cfg.top_p,
                   cfg.sink, cfg.tail)
        p_in = rec.positions_in.cpu().numpy()
        if not fused:
            # compaction of this layer's rows and positions, bit for bit
            h_in = rec.h_in.contiguous().view(torch.int16).cpu().numpy()
            h_ref, p_ref, cu_ref = O.compact(mask, h_in, p_in, cu_in, G)
            assert np.array_equal(rec.h_out.contiguous().view(torch.int16).cpu().numpy(), h_ref)
        else:
            # normalised operand read from the frozen rows; residual sum through the row map
            h64 = bf16_to_f64(rec.h_in)
            y, p_ref, cu_ref = O.compact_rmsnorm(mask, h64, p_in, cu_in, G, None, 1e-6)
            check_rounded(bf16_to_f64(rec.normed), y, "bf16", (cfg.d_model / 64 + 16) * 2.0 ** -24,
                          "normed operand")
            out_ref = O.gather_add(mask, h64, bf16_to_f64(rec.delta), cu_in, G, "bf16")
            assert np.array_equal(bf16_to_f64(rec.h_out), out_ref)
        assert list(rec.cu_out.numpy()) == list(cu_ref)
        assert np.array_equal(rec.positions_out.cpu().numpy(), p_ref)
        O.history_append(ref_led, rec.layer, cu_ref)
        # drops compose: the surviving positions are the earlier survivors,
        # filtered by this layer's mask, in order
        keep = O.token_keep(mask, cu_in, G).astype(bool)
        for b in range(len(lengths)):
            alive = p_in[cu_in[b]:cu_in[b + 1]]
            assert np.array_equal(alive, kept_pos[b])
            kept_pos[b] = alive[keep[cu_in[b]:cu_in[b + 1]]]
        assert rec.tokens_out == int(cu_ref[-1]) <= rec.tokens_in
    # final state: the last layer's output rows carry the surviving positions
    fin = res.positions.cpu().numpy()
    cu_f = res.cu_seqlens.numpy()
    for b in range(len(lengths)):
        assert np.array_equal(fin[cu_f[b]:cu_f[b + 1]], kept_pos[b])
    # ledger: every drop recorded; per-layer KV lengths read back
    led = res.ledger.cpu().numpy()
    B, cap = len(lengths), len(cfg.full_layers)
    assert led[0] == 0
    for r in range(B):
        ent = led[4 + B + 2 * r * cap: 4 + B + 2 * (r * cap + int(led[4 + r]))].reshape(-1, 2)
        assert [tuple(int(v) for v in e) for e in ent] == ref_led[r]
    kv = torch.empty(B, dtype=torch.int32, device="cuda")
    cu_d = cu.cuda()
    for layer in range(len(cfg.pattern)):
        U.up_kv_len(res.ledger, B, cap, layer, cu_d, kv)
        torch.cuda.synchronize()
        exp = [O.history_kv_len(ref_led[r], layer, lengths[r]) for r in range(B)]
        assert kv.cpu().tolist() == exp
    assert res.tokens_per_layer[0] == sum(lengths)
    assert all(a >= b for a, b in zip(res.tokens_per_layer, res.tokens_per_layer[1:]))


def test_stack_without_pruning_keeps_every_token():
    cfg = StackConfig(pattern="LFLF", d_model=128, d_ff=256, hq=2, hkv=1, head_dim=64, n_query=32,
                      block=32, seed=5)
    stack = HybridStack(cfg, "cuda")
    h, cu, pos = _inputs(cfg, [100, 333], 9)
    a = stack.forward(h, cu, pos, prune=False)
    b = stack.forward(h, cu, pos, prune=True)     # p = 0.99 keeps most, not necessarily all
    torch.cuda.synchronize()
    assert a.tokens_per_layer == [433] * 4 and a.ledger is None
    assert b.tokens_per_layer[0] == 433 and b.tokens_per_layer[-1] <= 433
    assert torch.equal(a.positions, pos)
