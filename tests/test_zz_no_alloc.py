"""up_compact_noalloc (the library's own device scratch, no caller workspace)
against up_compact (caller workspace) on the same inputs, through the C ABI.

Calls in a row on one GPU share the scratch, so the sequence goes from a
three-tile batch to one at the scratch's limit (2^19 blocks) and then to a
smaller one: each must match up_compact exactly (cu_seqlens_out, rows,
positions) and report a clear status word.
"""
import numpy as np
import pytest
import torch

import token_block_sparsification_amd as U

pytestmark = pytest.mark.gpu

MAX_BLOCKS = 1 << 19


def _case(lengths, G, row_elems, dtype, seed):
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(seed)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    batch = U.Batch.make(cu, G, dev)
    T = batch.num_tokens
    hidden = torch.randint(-1000, 1000, (T, row_elems), generator=gen).to(dtype).to(dev)
    pos = torch.cat([torch.arange(L, dtype=torch.int32) for L in lengths]).to(dev)
    mask = (torch.rand(batch.num_blocks, generator=gen) < 0.6).to(torch.uint8)
    cb = batch.cu_blocks_h.tolist()
    if len(lengths) > 1:
        mask[cb[1]:cb[2]] = 1          # one request all kept
    mask = mask.to(dev)
    return batch, hidden, pos, mask


def _outputs(batch, hidden):
    T, B = batch.num_tokens, batch.num_seqs
    h = torch.full_like(hidden, 77)
    p = torch.full((T,), -5, dtype=torch.int32, device=hidden.device)
    c = torch.full((B + 1,), -9, dtype=torch.int32, device=hidden.device)
    return h, p, c


def _compare(lengths, G, row_elems, dtype, seed):
    batch, hidden, pos, mask = _case(lengths, G, row_elems, dtype, seed)
    ws = U.new_compact_workspace(batch.cu_seqlens_h, G, hidden.device)
    ha, pa, ca = _outputs(batch, hidden)
    U.up_compact(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask, hidden, pos,
                 ha, pa, ca, ws)
    hb, pb, cb = _outputs(batch, hidden)
    status = torch.full((1,), -1, dtype=torch.int32, device=hidden.device)
    U.up_compact_noalloc(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, G, mask,
                         hidden, pos, hb, pb, cb, status)
    torch.cuda.synchronize()
    n = int(ca[-1])
    assert 0 < n < batch.num_tokens
    assert torch.equal(ca, cb)
    assert torch.equal(ha[:n].view(torch.uint8), hb[:n].view(torch.uint8))
    assert torch.equal(pa[:n], pb[:n])
    assert int(status[0]) == 0
    return batch.num_blocks


def test_noalloc_matches_compact_on_consecutive_calls():
    nb1 = _compare([40000, 3001, 16 * 300 + 7], 16, 64, torch.bfloat16, 1)     # 3 scan tiles
    nb2 = _compare([MAX_BLOCKS * 16 - 16 * 1000, 16 * 1000], 16, 1, torch.float32, 2)
    nb3 = _compare([3000, 10, 64 * 5], 64, 512, torch.float32, 3)               # one tile
    assert nb1 > 2 * 1024 and nb2 == MAX_BLOCKS and nb3 < nb1


def test_noalloc_rejects_batches_beyond_its_scratch():
    cu = torch.tensor([0, MAX_BLOCKS * 16 + 1], dtype=torch.int32)
    dummy = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    st = U.lib().up_compact_noalloc(1, U._ptr(cu), U._ptr(dummy), U._ptr(dummy), 16,
                                    U._ptr(dummy), U._ptr(dummy), 4, 4, None, U._ptr(dummy),
                                    None, U._ptr(dummy), MAX_BLOCKS * 16 + 1, None, None)
    assert st == 4 and "at most" in U.up_last_error()
