"""Multi-layer propagation driver: a synthetic hybrid stack with random weights.

Method (UniPrefill page "中国科学院与腾讯微信合作解决AI排队等待问题", §二 step 3 and
§三): tokens dropped at a full-attention layer are skipped by every later
layer (linear attention, sliding window, FFN) until the next full-attention
layer evaluates importance again on the tokens that are left; each drop is
recorded in the per-request drop-history ledger.

This driver chains the pruning path across a stack of layers so that the
propagation can be checked and measured without a trained model:

  F  full-attention layer: Q and K projections of the RMS-normalised state
     (computed in both modes, as the layer's attention needs them) feed
     up_score -> up_select_topp -> up_compact_record (the compaction and the
     drop-history append, up_compact + up_drop_history in one call); the layer's
     output projection then runs on the kept tokens only.
  L  token-local layer standing in for the layers between full-attention
     layers: a random two-matrix MLP with a residual, whose cost is
     proportional to the tokens it sees.

Weights are seeded random bf16 (there is no trained model); the F layers'
attention output itself is not computed, since it is not part of the pruning
path.  Every step of the pruning path runs in the library's kernels; the
projections and MLPs are plain torch matrix products (contiguous operands).

fused=True runs the fused pipeline at each F layer: no compacted copy of the
hidden states is made; the layer's normalised operand is read straight from
the frozen rows (up_compact_rmsnorm) and its residual sum reads the residual
from them too (up_gather_add).  fused=False compacts first (up_compact_record) and
normalises / adds with torch.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

from . import (Batch, up_compact_record, up_compact_rmsnorm, up_drop_history, up_gather_add,
               up_history_bytes, up_history_init, up_score, up_score_workspace_size,
               up_select_topp, new_compact_workspace)


@dataclass
class StackConfig:
    pattern: str = "LLLF" * 4      # layer kinds, first layer first
    d_model: int = 2048
    d_ff: int = 4096
    hq: int = 16
    hkv: int = 2
    head_dim: int = 256
    n_query: int = 128
    block: int = 64
    top_p: float = 0.99
    sink: int = 128
    tail: int = 128
    seed: int = 7

    @property
    def full_layers(self) -> List[int]:
        return [i for i, c in enumerate(self.pattern) if c == "F"]


@dataclass
class LayerRecord:
    """What one full-attention layer saw and produced (kept for checking)."""
    layer: int
    cu_in: torch.Tensor            # host int32 [B+1]
    tokens_in: int
    tokens_out: int
    q: Optional[torch.Tensor] = None
    k: Optional[torch.Tensor] = None
    h_in: Optional[torch.Tensor] = None
    positions_in: Optional[torch.Tensor] = None
    token_scores: Optional[torch.Tensor] = None
    block_scores: Optional[torch.Tensor] = None
    mask: Optional[torch.Tensor] = None
    cu_out: Optional[torch.Tensor] = None
    h_out: Optional[torch.Tensor] = None
    positions_out: Optional[torch.Tensor] = None
    normed: Optional[torch.Tensor] = None   # fused: the normalised operand of the kept rows
    delta: Optional[torch.Tensor] = None    # fused: the output projection added to the residual


@dataclass
class StackResult:
    hidden: torch.Tensor
    positions: torch.Tensor
    cu_seqlens: torch.Tensor        # host int32 [B+1]
    ledger: Optional[torch.Tensor]
    tokens_per_layer: List[int] = field(default_factory=list)
    records: List[LayerRecord] = field(default_factory=list)


def _rmsnorm(x: torch.Tensor) -> torch.Tensor:
    xf = x.float()
    return (xf * torch.rsqrt(xf.pow(2).mean(dim=-1, keepdim=True) + 1e-6)).to(x.dtype)


class HybridStack:
    """Random-weight hybrid stack; weights live on `device` in bf16."""

    def __init__(self, cfg: StackConfig, device):
        if cfg.hq % cfg.hkv:
            raise ValueError("hq must be a multiple of hkv")
        self.cfg = cfg
        self.dev = torch.device(device)
        g = torch.Generator(device="cpu").manual_seed(cfg.seed)
        D = cfg.d_model

        def w(rows, cols):  # N(0, 1/rows): keeps activations O(1) layer to layer
            return (torch.randn(rows, cols, generator=g) / rows ** 0.5).to(torch.bfloat16).to(self.dev)

        self.weights = []
        for kind in cfg.pattern:
            if kind == "F":
                self.weights.append({"wq": w(D, cfg.hq * cfg.head_dim),
                                     "wk": w(D, cfg.hkv * cfg.head_dim),
                                     "wo": w(D, D)})
            elif kind == "L":
                self.weights.append({"w1": w(D, cfg.d_ff), "w2": w(cfg.d_ff, D)})
            else:
                raise ValueError(f"unknown layer kind {kind!r}")

    def forward(self, hidden: torch.Tensor, cu_seqlens, positions: torch.Tensor,
                prune: bool = True, keep_records: bool = False, fused: bool = False) -> StackResult:
        """Run the stack on a packed batch.  prune=False carries every token
        through (the same layers, no pruning path) for comparison; fused=True
        uses the fused pipeline at the pruning layers."""
        cfg = self.cfg
        cu = torch.as_tensor(cu_seqlens, dtype=torch.int32).cpu()
        h, pos = hidden, positions
        B = cu.numel() - 1
        ledger = None
        nf = max(1, len(cfg.full_layers))
        if prune:
            ledger = torch.empty(up_history_bytes(B, nf) // 4, dtype=torch.int32, device=self.dev)
            up_history_init(ledger, B, nf)
        res = StackResult(hidden=h, positions=pos, cu_seqlens=cu, ledger=ledger)
        # Workspaces sized for the first full-attention layer serve the later
        # ones, which see subsets of its tokens (the compaction workspace
        # always fits; the scoring one is regrown if a layer needs more).
        self._ws = None
        if prune and int(cu[-1]) > 0:
            self._ws = (torch.empty(up_score_workspace_size(cu, cfg.hq, cfg.hkv, cfg.head_dim,
                                                            cfg.n_query),
                                    dtype=torch.uint8, device=self.dev),
                        new_compact_workspace(cu, cfg.block, self.dev))
        for li, (kind, wts) in enumerate(zip(cfg.pattern, self.weights)):
            T = int(cu[-1])
            res.tokens_per_layer.append(T)
            if kind == "L":
                x = _rmsnorm(h)
                h = h + torch.relu(x @ wts["w1"]) @ wts["w2"]
                continue
            x = _rmsnorm(h)
            # Q and K of every token, as the layer's attention computes them
            # in either mode; the pruning path only reuses them.
            q = (x @ wts["wq"]).view(T, cfg.hq, cfg.head_dim)
            k = (x @ wts["wk"]).view(T, cfg.hkv, cfg.head_dim)
            if prune and T > 0 and fused:
                h, pos, cu_new, rec = self._prune_fused(li, h, pos, cu, q, k, ledger, nf,
                                                        keep_records, wts["wo"])
                if rec is not None:
                    res.records.append(rec)
                cu = cu_new
                continue
            if prune and T > 0:
                h, pos, cu_new, rec = self._prune(li, h, pos, cu, q, k, ledger, nf, keep_records)
                if rec is not None:
                    res.records.append(rec)
                cu = cu_new
                x = _rmsnorm(h)
            if int(cu[-1]) > 0:
                h = h + x @ wts["wo"]
        res.hidden, res.positions, res.cu_seqlens = h, pos, cu
        return res

    def _select(self, cu, q, k):
        """Scores and mask of one full-attention layer (library kernels)."""
        cfg = self.cfg
        dev = self.dev
        batch = Batch.make(cu, cfg.block, dev)
        T, N, B = batch.num_tokens, batch.num_blocks, batch.num_seqs
        sws, cws = self._ws
        need = up_score_workspace_size(cu, cfg.hq, cfg.hkv, cfg.head_dim, cfg.n_query)
        if sws.numel() < need:  # a smaller batch can still split into more key chunks
            sws = torch.empty(need, dtype=torch.uint8, device=dev)
            self._ws = (sws, cws)
        ts = torch.empty(T, dtype=torch.float32, device=dev)
        bs = torch.empty(max(N, 1), dtype=torch.float32, device=dev)
        mask = torch.empty(max(N, 1), dtype=torch.uint8, device=dev)
        kept = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
        up_score(cu, batch.cu_seqlens_d, batch.cu_blocks_d, q, k, cfg.n_query, cfg.block, 0.0, ts, bs,
                 sws)
        up_select_topp(cu, batch.cu_seqlens_d, batch.cu_blocks_d, bs, cfg.block, cfg.top_p, cfg.sink,
                       cfg.tail, mask, kept)
        return batch, ts, bs, mask

    def _prune_fused(self, li, h, pos, cu, q, k, ledger, nf, keep_records, wo):
        """Fused pipeline at a pruning layer: the normalised operand and the
        residual sum read the kept rows from the frozen buffer `h` through
        the row map; no compacted copy of `h` is written."""
        cfg = self.cfg
        dev = self.dev
        batch, ts, bs, mask = self._select(cu, q, k)
        T, N, B = batch.num_tokens, batch.num_blocks, batch.num_seqs
        cws = self._ws[1]
        x = torch.empty_like(h)
        p_out = torch.empty_like(pos)
        cu_out = torch.empty(B + 1, dtype=torch.int32, device=dev)
        up_compact_rmsnorm(cu, batch.cu_seqlens_d, batch.cu_blocks_d, cfg.block, mask, h, None,
                           1e-6, pos, x, None, p_out, cu_out, cws)
        up_drop_history(ledger, B, nf, li, cu_out)
        cu_new = cu_out.cpu()  # the following layers size their launches on the host
        n = int(cu_new[-1])
        delta = x[:n] @ wo
        delta_in = delta.clone() if keep_records else None
        up_gather_add(cu, batch.cu_seqlens_d, batch.cu_blocks_d, cfg.block, mask, h, delta, delta,
                      cws)  # in place: delta becomes the layer's output rows
        rec = None
        if keep_records:
            rec = LayerRecord(layer=li, cu_in=cu, tokens_in=T, tokens_out=n, q=q, k=k, h_in=h,
                              positions_in=pos, token_scores=ts, block_scores=bs[:N],
                              mask=mask[:N], cu_out=cu_new, h_out=delta, positions_out=p_out[:n],
                              normed=x[:n], delta=delta_in)
        return delta, p_out[:n], cu_new, rec

    def _prune(self, li, h, pos, cu, q, k, ledger, nf, keep_records):
        cfg = self.cfg
        dev = self.dev
        batch, ts, bs, mask = self._select(cu, q, k)
        T, N, B = batch.num_tokens, batch.num_blocks, batch.num_seqs
        cws = self._ws[1]
        h_out = torch.empty_like(h)
        p_out = torch.empty_like(pos)
        cu_out = torch.empty(B + 1, dtype=torch.int32, device=dev)
        up_compact_record(cu, batch.cu_seqlens_d, batch.cu_blocks_d, cfg.block, mask, h, pos, h_out,
                          p_out, cu_out, cws, ledger, nf, li)
        cu_new = cu_out.cpu()  # the next layer's packing sizes its launches on the host
        n = int(cu_new[-1])
        rec = None
        if keep_records:
            rec = LayerRecord(layer=li, cu_in=cu, tokens_in=T, tokens_out=n, q=q, k=k, h_in=h,
                              positions_in=pos, token_scores=ts, block_scores=bs[:N],
                              mask=mask[:N], cu_out=cu_new, h_out=h_out[:n], positions_out=p_out[:n])
        return h_out[:n], p_out[:n], cu_new, rec
