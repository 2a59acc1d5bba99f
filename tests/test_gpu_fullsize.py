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


def _full(name, **over):
    w = W.get_workload(name)
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


@pytest.mark.parametrize("n", [32, 128, 512])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_qwen3next_sweep(n, G):
    _full(f"qwen3next_L131072_n{n}_G{G}")
