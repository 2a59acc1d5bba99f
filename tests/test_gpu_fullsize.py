"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same entry points, default geometry).

The oracle runs in full on the same input bytes (generated on the GPU, copied
to the host); compaction is checked bit for bit by gathering the oracle's row
set with torch.index_select on the GPU.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _parity import GpuRun, check_compaction, check_mask, check_scores, oracle_qk

pytestmark = pytest.mark.gpu


def _full(base, **over):
    w = W.get_workload(base)
    if over:
        w = w.with_(**over)
    dev = torch.device("cuda")
    print(f"[fullsize] {w.name}: generating", flush=True)
    inputs = W.make_inputs(w, device=dev)
    inputs = dict(inputs, cu_seqlens=inputs["cu_seqlens"].cpu())
    run = GpuRun(inputs, w.n_query, w.block)
    out = run.run(p=w.top_p, sink=w.sink, tail=w.tail, layer_id=7)
    cu = inputs["cu_seqlens"].numpy()
    q64, k64 = oracle_qk(inputs, w.n_query)
    print(f"[fullsize] {w.name}: oracle on {int(cu[-1])} tokens", flush=True)
    c_ref = O.token_scores(q64, k64, cu, w.n_query)
    del q64, k64
    b_ref = O.block_scores(c_ref, cu, w.block)
    r1 = check_scores(out["token_scores"], c_ref, cu, "token scores")
    r2 = check_scores(out["block_scores"], b_ref, O.block_offsets(cu, w.block), "block scores")
    m_iso = check_mask(out["mask"], out["block_scores"].astype(np.float64), cu, w.block, w.top_p,
                       w.sink, w.tail)
    m_e2e = check_mask(out["mask"], b_ref, cu, w.block, w.top_p, w.sink, w.tail)
    n = check_compaction(run, out["mask"], out["kept"])
    status, entries = run.ledger_entries()
    ref_led = O.history_new(len(cu) - 1)
    O.history_append(ref_led, 7, out["cu_out"])
    assert status == 0 and entries == ref_led
    # planted blocks that every tail query sees are kept (sanity, not a pin;
    # inside the query window the causal mask lowers a block's score)
    cub = O.block_offsets(cu, w.block)
    for r, pl in enumerate(inputs["planted"]):
        L = int(cu[r + 1] - cu[r])
        seen_by_all = [b for b in pl if (b + 1) * w.block <= L - min(w.n_query, L)]
        assert all(out["mask"][cub[r] + b] for b in seen_by_all)
    print(f"[fullsize] {w.name}: T={int(cu[-1])} max_rel_token={r1:.2e} max_rel_block={r2:.2e} "
          f"mask_mismatch_iso={m_iso} mask_mismatch_e2e={m_e2e} kept={n} "
          f"keep_ratio={n / int(cu[-1]):.4f}", flush=True)


@pytest.mark.parametrize("name", ["llama8b_L131072", "llama8b_L131072_noplant", "llama8b_L32768",
                                  "small_L2048"])
def test_llama_shapes(name):
    _full(name)


def test_packed_batch16():
    _full("llama8b_batch16")


def test_many_short_requests():
    """256 requests of 512 tokens: 2048 scoring workgroups over several
    resident rounds, each request one key chunk."""
    _full("llama8b_batch256_L512")


@pytest.mark.parametrize("log2_len", [20, 22])
def test_long_request_beyond_the_benchmark(log2_len):
    """One 2^20- or 2^22-token request and a short one (head_dim 64, 4/4
    heads): the row statistics run 256 / 1024 key chunks per row that the
    column-sum prologue merges, the request has 16,384 / 65,536 blocks (a
    selection that does not stage them in LDS) and the compaction scans 17 /
    65 tiles; token offsets reach 2^28 elements of K."""
    L = 1 << log2_len
    _full("small_L2048", name=f"long_L{L}", lengths=(L, 3000), num_seqs=2, hidden_dim=64)


@pytest.mark.parametrize("n", [32, 128, 512])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_qwen3next_sweep(n, G):
    _full(f"qwen3next_L131072_n{n}_G{G}")


def test_fused_pipeline_full_size():
    """The fused pipeline at the benchmark's full size (one 131072-token
    request, hidden 4096 bf16): the selection run by the block-mean kernel
    gives bit-identical scores, mask and kept counts to the two calls; the normalised operand
    and the residual sum are checked against the oracle on 1024 sampled kept
    rows (operand within half a bf16 ulp plus the fp32 error bound, residual
    sum exact), positions and cu_seqlens_out exactly."""
    import token_block_sparsification_amd as U
    from _parity import bf16_to_f64, check_rounded
    w = W.get_workload("llama8b_L131072")
    dev = torch.device("cuda")
    inp = W.make_inputs(w, device=dev)
    cu = inp["cu_seqlens"].cpu()
    batch = U.Batch.make(cu, w.block, dev)
    q, k, hidden, pos = inp["q"], inp["k"], inp["hidden"], inp["positions"]
    ws = U.Workspace.make(batch, w.hq, w.hkv, w.head_dim, w.n_query, hidden, dev)
    T, N, B = batch.num_tokens, batch.num_blocks, batch.num_seqs
    outs = []
    for fused in (False, True):
        bs = torch.empty(N, device=dev)
        mask = torch.empty(N, dtype=torch.uint8, device=dev)
        kept = torch.empty(B, dtype=torch.int32, device=dev)
        if fused:
            U.up_score_select(cu, batch.cu_seqlens_d, batch.cu_blocks_d, q, k, w.n_query, w.block,
                              0.0, None, bs, w.top_p, w.sink, w.tail, mask, kept, ws.score_ws)
        else:
            U.up_score(cu, batch.cu_seqlens_d, batch.cu_blocks_d, q, k, w.n_query, w.block, 0.0,
                       None, bs, ws.score_ws)
            U.up_select_topp(cu, batch.cu_seqlens_d, batch.cu_blocks_d, bs, w.block, w.top_p,
                             w.sink, w.tail, mask, kept)
        outs.append((bs, mask, kept))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    mask = outs[1][1]
    D = hidden.shape[1]
    normed = torch.empty((T, D), dtype=hidden.dtype, device=dev)
    pout = torch.empty(T, dtype=torch.int32, device=dev)
    cu_out = torch.empty(B + 1, dtype=torch.int32, device=dev)
    U.up_compact_rmsnorm(cu, batch.cu_seqlens_d, batch.cu_blocks_d, w.block, mask, hidden, None,
                         1e-6, pos, normed, None, pout, cu_out, ws.compact_ws)
    mask_np = mask.cpu().numpy()
    keep_idx = np.flatnonzero(O.token_keep(mask_np, cu.numpy(), w.block))
    n = len(keep_idx)
    delta = torch.randn((n, D), device=dev).to(hidden.dtype)
    out = torch.empty((n, D), dtype=hidden.dtype, device=dev)
    U.up_gather_add(cu, batch.cu_seqlens_d, batch.cu_blocks_d, w.block, mask, hidden, delta, out,
                    ws.compact_ws)
    torch.cuda.synchronize()
    _, _, cu_ref = O.compact(mask_np, np.zeros((T, 1)), np.zeros(T), cu.numpy(), w.block)
    assert list(cu_out.cpu().numpy()) == list(cu_ref)
    assert np.array_equal(pout[:n].cpu().numpy(), pos.cpu().numpy()[keep_idx])
    rows = np.sort(np.random.default_rng(5).choice(n, size=1024, replace=False))
    src = torch.from_numpy(keep_idx[rows]).to(dev)
    sel = torch.from_numpy(rows).to(dev)
    h64 = bf16_to_f64(hidden.index_select(0, src))
    y = O.rms_normalize(h64, None, 1e-6)
    frac = check_rounded(bf16_to_f64(normed.index_select(0, sel)), y, "bf16",
                         (D / 64 + 16) * 2.0 ** -24, "normed operand")
    exp = O.round_to_format(h64 + bf16_to_f64(delta.index_select(0, sel)), "bf16")
    assert np.array_equal(bf16_to_f64(out.index_select(0, sel)), exp)
    print(f"[fullsize] fused pipeline: kept={n} exactly_rounded={frac:.4f}", flush=True)
