"""up_compact_record (compaction whose copy kernel also appends the ledger
entries) against up_compact followed by up_drop_history, and against the
oracle's compaction and ledger (UniPrefill page, §二 step 3 and §三): rows,
positions, cu_seqlens_out and every ledger word, over consecutive layers until
records fill up, a ledger of another shape, strided rows and a batch with no
blocks at all.
"""
import numpy as np
import pytest
import torch

import oracle as O
import token_block_sparsification_amd as U

pytestmark = pytest.mark.gpu


def _ledger(B, cap, dev):
    """A fresh ledger whose entry slots hold a sentinel (init clears only the
    header and counts), so two ledgers compare equal word for word only if
    neither path wrote a slot the other did not."""
    led = torch.full((U.up_history_bytes(B, cap) // 4,), -5, dtype=torch.int32, device=dev)
    U.up_history_init(led, B, cap)
    return led


def _check_ledger(led, ref, B, cap, status):
    """The ledger words against the oracle's records (layout of
    up_history_init): status, shape, entry counts, every used entry, and the
    sentinel left in every slot past a record's count."""
    w = led.cpu().numpy()
    assert list(w[:3]) == [status, B, cap]
    for r, rec in enumerate(ref):
        kept = rec[:cap]   # a full record keeps its first entries
        assert w[4 + r] == len(kept), r
        for e in range(cap):
            i = 4 + B + 2 * (r * cap + e)
            exp = kept[e] if e < len(kept) else (-5, -5)
            assert (w[i], w[i + 1]) == exp, (r, e)


@pytest.mark.parametrize("strided", [False, True])
def test_record_matches_compact_then_history(strided):
    dev = torch.device("cuda")
    lens = [0, 3, 64, 65, 1000, 0, 2049, 130]
    B, G, dim, cap = len(lens), 32, 96, 3
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    batch = U.Batch.make(cu, G, dev)
    T = batch.num_tokens
    gen = torch.Generator().manual_seed(7)
    base = torch.randint(-100, 100, (T, dim + (5 if strided else 0)), generator=gen)
    hidden = base.to(torch.bfloat16).to(dev)
    if strided:
        hidden = hidden[:, :dim]
    pos = (torch.arange(T, dtype=torch.int32) * 5 + 2).to(dev)
    ws_a = U.new_compact_workspace(batch.cu_seqlens_h, G, dev)
    ws_b = U.new_compact_workspace(batch.cu_seqlens_h, G, dev)
    led_a, led_b = _ledger(B, cap, dev), _ledger(B, cap, dev)
    ref = O.history_new(B)
    status = 0
    # five layers on a capacity of three: the last two find every record full
    for layer, frac in [(2, 0.9), (5, 0.5), (6, 0.0), (9, 1.0), (11, 0.3)]:
        mask_np = (torch.rand(batch.num_blocks, generator=gen) < frac).numpy().astype(np.uint8)
        mask = torch.from_numpy(mask_np).to(dev)
        outs = []
        for rec in (True, False):
            out = torch.zeros((T + 3, dim), dtype=torch.bfloat16, device=dev)
            pout = torch.full((T + 3,), -1, dtype=torch.int32, device=dev)
            cu_out = torch.full((B + 1,), -7, dtype=torch.int32, device=dev)
            if rec:
                U.up_compact_record(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G,
                                    mask, hidden, pos, out, pout, cu_out, ws_a, led_a, cap, layer)
            else:
                U.up_compact(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask,
                             hidden, pos, out, pout, cu_out, ws_b)
                U.up_drop_history(led_b, B, cap, layer, cu_out)
            outs.append((out, pout, cu_out))
        torch.cuda.synchronize()
        for x, y in zip(outs[0], outs[1]):
            assert torch.equal(x, y), layer
        assert torch.equal(led_a, led_b), layer
        keep = O.token_keep(mask_np, cu.numpy(), G)
        idx = torch.from_numpy(np.flatnonzero(keep)).to(dev)
        assert torch.equal(outs[0][0][:idx.numel()], hidden.index_select(0, idx))
        _, _, cu_ref = O.compact(mask_np, np.zeros((T, 1)), np.zeros(T), cu.numpy(), G)
        assert outs[0][2].cpu().tolist() == list(cu_ref)
        if any(len(r) >= cap for r in ref):
            status |= 1
        O.history_append(ref, layer, list(cu_ref))
        _check_ledger(led_a, ref, B, cap, status)
    assert led_a.cpu().numpy()[0] == 1   # full records were flagged


def test_record_ledger_of_another_shape():
    """A ledger set up for another num_seqs is flagged (status bit 1) and left
    otherwise unwritten; the compaction itself is unaffected."""
    dev = torch.device("cuda")
    lens = [100, 0, 300]
    B, G, cap = len(lens), 64, 4
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    batch = U.Batch.make(cu, G, dev)
    T = batch.num_tokens
    hidden = torch.arange(T * 8, dtype=torch.float32, device=dev).view(T, 8)
    mask = torch.tensor([(b % 3) != 1 for b in range(batch.num_blocks)], dtype=torch.uint8,
                        device=dev)
    ws = U.new_compact_workspace(batch.cu_seqlens_h, G, dev)
    led = _ledger(B - 1, cap, dev)
    before = led.cpu().clone()
    out = torch.zeros((T, 8), device=dev)
    cu_out = torch.empty(B + 1, dtype=torch.int32, device=dev)
    U.up_compact_record(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask,
                        hidden, None, out, None, cu_out, ws, led, cap, 4)
    torch.cuda.synchronize()
    after = led.cpu()
    assert after[0] == 2 and torch.equal(after[1:], before[1:])
    _, _, cu_ref = O.compact(mask.cpu().numpy(), np.zeros((T, 1)), np.zeros(T), cu.numpy(), G)
    assert cu_out.cpu().tolist() == list(cu_ref)


def test_record_batch_without_blocks():
    """Requests that are all empty: no copy launch, the entries (all zero kept
    tokens) still appended, as up_drop_history would."""
    dev = torch.device("cuda")
    cu = torch.tensor([0, 0, 0, 0], dtype=torch.int32)
    B, cap = 3, 2
    batch = U.Batch.make(cu, 64, dev)
    ws = U.new_compact_workspace(cu, 64, dev)
    led = _ledger(B, cap, dev)
    cu_out = torch.full((B + 1,), 99, dtype=torch.int32, device=dev)
    h = torch.zeros((1, 8), device=dev)
    U.up_compact_record(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, 64,
                        torch.zeros(1, dtype=torch.uint8, device=dev), h, None,
                        torch.zeros((1, 8), device=dev), None, cu_out, ws, led, cap, 3)
    torch.cuda.synchronize()
    assert cu_out.tolist() == [0, 0, 0, 0]
    ref = O.history_new(B)
    O.history_append(ref, 3, [0, 0, 0, 0])
    _check_ledger(led, ref, B, cap, 0)


def test_copy_events_time_the_copy_kernel_alone():
    """up_set_copy_events: the events land right around the copy kernel, so
    their interval lies inside the whole call's and is positive; once
    cleared, calls record nothing more into them."""
    dev = torch.device("cuda")
    lens = [70000, 0, 9000]
    G = 64
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    batch = U.Batch.make(cu, G, dev)
    T = batch.num_tokens
    hidden = torch.ones((T, 2048), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(hidden)
    cu_out = torch.empty(len(lens) + 1, dtype=torch.int32, device=dev)
    mask = torch.ones(batch.num_blocks, dtype=torch.uint8, device=dev)
    ws = U.new_compact_workspace(batch.cu_seqlens_h, G, dev)
    c0, c1, o0, o1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    c0.record(); c1.record()
    U.up_set_copy_events(c0, c1)
    try:
        o0.record()
        U.up_compact(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, hidden,
                     None, out, None, cu_out, ws)
        o1.record()
    finally:
        U.up_set_copy_events(None, None)
    torch.cuda.synchronize()
    copy_ms, call_ms = c0.elapsed_time(c1), o0.elapsed_time(o1)
    assert 0 < copy_ms < call_ms, (copy_ms, call_ms)
    assert torch.equal(out, hidden)
    # cleared: a further call leaves the events where they were
    U.up_compact(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, hidden,
                 None, out, None, cu_out, ws)
    torch.cuda.synchronize()
    assert c0.elapsed_time(c1) == copy_ms

