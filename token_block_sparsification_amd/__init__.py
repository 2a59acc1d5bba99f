"""Python binding of libuniprefill.so, the MI355X (gfx950) UniPrefill pruning path.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the HIP stream.  The functions
below carry the C entry points' names (see include/uniprefill.h) and raise
UniprefillError when the library returns a status other than UP_OK.  If the
library has not been built, the first call raises with the build command.

Method: the UniPrefill article page "中国科学院与腾讯微信合作解决AI排队等待问题"
(§二 steps 1-3, §三).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "UniprefillError", "lib", "LIB_PATH",
    "up_abi_version", "up_last_error", "up_make_cu_blocks",
    "up_score_workspace_size", "up_score", "up_select_topp",
    "up_compact_workspace_size", "up_compact_workspace_init", "up_compact", "up_compact_status",
    "up_compact_noalloc", "up_compact_record", "up_set_copy_events",
    "up_history_bytes", "up_history_init", "up_drop_history", "up_kv_len", "up_revive",
    "up_compact_rmsnorm", "up_gather_add", "up_score_select",
    "Batch", "Workspace", "run_chain",
]

# The in-tree library; UNIPREFILL_LIBRARY names another build of it (for
# example one with host-side sanitizers).
LIB_PATH = os.environ.get("UNIPREFILL_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libuniprefill.so")

UP_OK = 0
_STATUS = {0: "UP_OK", 1: "UP_ERR_INVALID", 2: "UP_ERR_UNSUPPORTED", 3: "UP_ERR_WORKSPACE",
           4: "UP_ERR_CAPACITY", 5: "UP_ERR_HIP"}


class UniprefillError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_D = ctypes.c_double

_SIGNATURES = {
    "up_abi_version": (_I, []),
    "up_last_error": (ctypes.c_char_p, []),
    "up_status_string": (ctypes.c_char_p, [_I]),
    "up_make_cu_blocks": (_I, [_I, _P, _I, _P, ctypes.POINTER(_I64)]),
    "up_score_workspace_size": (_I, [_I, _P, _I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "up_score": (_I, [_I, _P, _P, _P, _P, _I64, _I64, _I, _P, _I64, _I64, _I, _I, _I, _I, _F,
                      _P, _P, _P, _SZ, _P]),
    "up_select_topp": (_I, [_I, _P, _P, _P, _P, _I, _D, _I, _I, _P, _P, _P]),
    "up_score_select": (_I, [_I, _P, _P, _P, _P, _I64, _I64, _I, _P, _I64, _I64, _I, _I, _I, _I,
                             _F, _P, _P, _D, _I, _I, _P, _P, _P, _SZ, _P]),
    "up_compact_workspace_size": (_I, [_I, _P, _I, ctypes.POINTER(_SZ)]),
    "up_compact_workspace_init": (_I, [_P, _SZ, _P]),
    "up_compact": (_I, [_I, _P, _P, _P, _I, _P, _P, _I64, _I64, _P, _P, _P, _P, _I64, _P, _SZ,
                        _P]),
    "up_compact_record": (_I, [_I, _P, _P, _P, _I, _P, _P, _I64, _I64, _P, _P, _P, _P, _I64, _P,
                               _SZ, _P, _I, _I, _P]),
    "up_compact_status": (_I, [_P, _SZ, _P, _I, _P]),
    "up_set_copy_events": (_I, [_P, _P]),
    "up_compact_noalloc": (_I, [_I, _P, _P, _P, _I, _P, _P, _I64, _I64, _P, _P, _P, _P, _I64, _P,
                                _P]),
    "up_history_bytes": (_SZ, [_I, _I]),
    "up_history_init": (_I, [_P, _I, _I, _P]),
    "up_drop_history": (_I, [_P, _I, _I, _I, _P, _P]),
    "up_kv_len": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "up_revive": (_I, [_I, _P, _P, _P, _I, _P, _P, _P, _I64, _I64, _P, _SZ, _P]),
    "up_compact_rmsnorm": (_I, [_I, _P, _P, _P, _I, _P, _I, _P, _I64, _I64, _P, _F, _P, _P, _P,
                                _P, _P, _I64, _P, _SZ, _P]),
    "up_gather_add": (_I, [_I, _P, _P, _P, _I, _P, _I, _P, _I64, _I64, _P, _P, _I64, _P, _SZ,
                           _P]),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m token_block_sparsification_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, st: int) -> None:
    if st != UP_OK:
        raise UniprefillError(fn, st, lib().up_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _host_i32(t) -> torch.Tensor:
    t = torch.as_tensor(t, dtype=torch.int32, device="cpu")
    return t.contiguous()


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def up_abi_version() -> int:
    return int(lib().up_abi_version())


def up_last_error() -> str:
    return lib().up_last_error().decode(errors="replace")


def up_make_cu_blocks(cu_seqlens_h, block: int):
    """Host block offsets for a packed batch -> (int32 CPU tensor [B+1], N)."""
    cu = _host_i32(cu_seqlens_h)
    out = torch.empty_like(cu)
    n = _I64(0)
    _check("up_make_cu_blocks",
           lib().up_make_cu_blocks(cu.numel() - 1, _ptr(cu), block, _ptr(out), ctypes.byref(n)))
    return out, int(n.value)


def up_score_workspace_size(cu_seqlens_h, hq: int, hkv: int, head_dim: int, n_query: int) -> int:
    cu = _host_i32(cu_seqlens_h)
    n = _SZ(0)
    _check("up_score_workspace_size",
           lib().up_score_workspace_size(cu.numel() - 1, _ptr(cu), hq, hkv, head_dim, n_query,
                                         ctypes.byref(n)))
    return int(n.value)


def up_compact_workspace_size(cu_seqlens_h, block: int) -> int:
    cu = _host_i32(cu_seqlens_h)
    n = _SZ(0)
    _check("up_compact_workspace_size",
           lib().up_compact_workspace_size(cu.numel() - 1, _ptr(cu), block, ctypes.byref(n)))
    return int(n.value)


def up_compact_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    """Prepare a compaction workspace once before its first up_compact call."""
    _check("up_compact_workspace_init",
           lib().up_compact_workspace_init(_ptr(workspace), workspace.numel(),
                                           _stream(stream, workspace.device)))


def new_compact_workspace(cu_seqlens_h, block: int, device, stream=None) -> torch.Tensor:
    """Allocate and prepare a compaction workspace for this batch."""
    ws = torch.empty(up_compact_workspace_size(cu_seqlens_h, block), dtype=torch.uint8,
                     device=device)
    up_compact_workspace_init(ws, stream)
    return ws


def up_history_bytes(num_seqs: int, capacity: int) -> int:
    return int(lib().up_history_bytes(num_seqs, capacity))


def _bf16_3d(name, t):
    if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be a bf16 [T, H, d] tensor with a contiguous last dim")


def up_score(cu_seqlens_h, cu_seqlens_d, cu_blocks_d, q, k, n_query: int, block: int,
             scale: float, token_scores: Optional[torch.Tensor], block_scores: torch.Tensor,
             workspace: torch.Tensor, stream=None) -> None:
    """Importance scores (§二 steps 1-2): q bf16 [T, Hq, d], k bf16 [T, Hkv, d]."""
    _bf16_3d("q", q)
    _bf16_3d("k", k)
    cu = _host_i32(cu_seqlens_h)
    st = lib().up_score(
        cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_d), _ptr(cu_blocks_d),
        _ptr(q), q.stride(0), q.stride(1), q.shape[1],
        _ptr(k), k.stride(0), k.stride(1), k.shape[1],
        q.shape[2], n_query, block, float(scale),
        _ptr(token_scores), _ptr(block_scores), _ptr(workspace), workspace.numel(),
        _stream(stream, q.device))
    _check("up_score", st)


def up_score_select(cu_seqlens_h, cu_seqlens_d, cu_blocks_d, q, k, n_query: int, block: int,
                    scale: float, token_scores: Optional[torch.Tensor], block_scores: torch.Tensor,
                    top_p: float, sink: int, tail: int, block_mask, kept_tokens,
                    workspace: torch.Tensor, stream=None) -> None:
    """up_score and up_select_topp in one call, the selection run by the
    block-mean kernel (fused pipeline); same outputs as the two calls."""
    _bf16_3d("q", q)
    _bf16_3d("k", k)
    cu = _host_i32(cu_seqlens_h)
    st = lib().up_score_select(
        cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_d), _ptr(cu_blocks_d),
        _ptr(q), q.stride(0), q.stride(1), q.shape[1],
        _ptr(k), k.stride(0), k.stride(1), k.shape[1],
        q.shape[2], n_query, block, float(scale),
        _ptr(token_scores), _ptr(block_scores), float(top_p), sink, tail, _ptr(block_mask),
        _ptr(kept_tokens), _ptr(workspace), workspace.numel(), _stream(stream, q.device))
    _check("up_score_select", st)


def up_select_topp(cu_seqlens_h, cu_seqlens_d, cu_blocks_d, block_scores, block: int,
                   top_p: float, sink: int, tail: int, block_mask, kept_tokens,
                   stream=None) -> None:
    """Top-p block mask with forced sink/tail blocks (§二 step 2)."""
    cu = _host_i32(cu_seqlens_h)
    st = lib().up_select_topp(cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_d), _ptr(cu_blocks_d),
                              _ptr(block_scores), block, float(top_p), sink, tail,
                              _ptr(block_mask), _ptr(kept_tokens),
                              _stream(stream, kept_tokens.device))
    _check("up_select_topp", st)


def up_compact(cu_seqlens_h, cu_seqlens_d, cu_blocks_d, block: int, block_mask, hidden,
               positions, hidden_out, positions_out, cu_seqlens_out, workspace,
               stream=None) -> None:
    """Gather kept rows (§二 step 3).  hidden [T, ...] rows are copied bytewise."""
    if hidden.dim() < 1 or (hidden.dim() > 1 and not hidden[0].is_contiguous()):
        raise ValueError("hidden rows must be contiguous")
    cu = _host_i32(cu_seqlens_h)
    row_bytes = (hidden[0].numel() if hidden.dim() > 1 else 1) * hidden.element_size()
    row_stride = hidden.stride(0) * hidden.element_size()
    if hidden_out.dtype != hidden.dtype:
        raise ValueError("hidden_out must have hidden's dtype")
    st = lib().up_compact(cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_d), _ptr(cu_blocks_d), block,
                          _ptr(block_mask), _ptr(hidden), row_bytes, row_stride, _ptr(positions),
                          _ptr(hidden_out), _ptr(positions_out), _ptr(cu_seqlens_out),
                          hidden_out.shape[0], _ptr(workspace), workspace.numel(),
                          _stream(stream, hidden_out.device))
    _check("up_compact", st)


def up_compact_record(cu_seqlens_h, cu_seqlens_d, cu_blocks_d, block: int, block_mask, hidden,
                      positions, hidden_out, positions_out, cu_seqlens_out, workspace, ledger,
                      capacity: int, layer_id: int, stream=None) -> None:
    """up_compact, then the ledger append of up_drop_history, in two launches
    (the copy kernel appends the entries)."""
    if hidden.dim() < 1 or (hidden.dim() > 1 and not hidden[0].is_contiguous()):
        raise ValueError("hidden rows must be contiguous")
    if hidden_out.dtype != hidden.dtype:
        raise ValueError("hidden_out must have hidden's dtype")
    cu = _host_i32(cu_seqlens_h)
    row_bytes = (hidden[0].numel() if hidden.dim() > 1 else 1) * hidden.element_size()
    row_stride = hidden.stride(0) * hidden.element_size()
    st = lib().up_compact_record(cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_d), _ptr(cu_blocks_d),
                                 block, _ptr(block_mask), _ptr(hidden), row_bytes, row_stride,
                                 _ptr(positions), _ptr(hidden_out), _ptr(positions_out),
                                 _ptr(cu_seqlens_out), hidden_out.shape[0], _ptr(workspace),
                                 workspace.numel(), _ptr(ledger), capacity, layer_id,
                                 _stream(stream, hidden_out.device))
    _check("up_compact_record", st)


def up_compact_noalloc(cu_seqlens_h, cu_seqlens_d, cu_blocks_d, block: int, block_mask, hidden,
                       positions, hidden_out, positions_out, cu_seqlens_out, status=None,
                       stream=None) -> None:
    """up_compact with the library's own device scratch instead of a caller
    workspace (for callers that cannot allocate); `status` (device int32 [1]
    or None) receives and clears the scratch's status bits."""
    if hidden.dim() < 1 or (hidden.dim() > 1 and not hidden[0].is_contiguous()):
        raise ValueError("hidden rows must be contiguous")
    if hidden_out.dtype != hidden.dtype:
        raise ValueError("hidden_out must have hidden's dtype")
    cu = _host_i32(cu_seqlens_h)
    row_bytes = (hidden[0].numel() if hidden.dim() > 1 else 1) * hidden.element_size()
    row_stride = hidden.stride(0) * hidden.element_size()
    st = lib().up_compact_noalloc(cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_d), _ptr(cu_blocks_d),
                                  block, _ptr(block_mask), _ptr(hidden), row_bytes, row_stride,
                                  _ptr(positions), _ptr(hidden_out), _ptr(positions_out),
                                  _ptr(cu_seqlens_out), hidden_out.shape[0], _ptr(status),
                                  _stream(stream, hidden_out.device))
    _check("up_compact_noalloc", st)


def up_compact_status(workspace, status, clear: bool = True, stream=None) -> None:
    """Copy the compaction workspace's status bits (bit 0: a look-back gave
    up) into the device int32 tensor `status`, clearing them if `clear`."""
    _check("up_compact_status", lib().up_compact_status(_ptr(workspace), workspace.numel(),
                                                        _ptr(status), 1 if clear else 0,
                                                        _stream(stream, workspace.device)))


def up_set_copy_events(start=None, stop=None) -> None:
    """Measurement aid: while set, calls that run the compaction copy kernel
    record the two torch.cuda.Event objects right around it (None, None
    clears).  Record each event once beforehand: torch creates the
    underlying HIP event on its first record."""
    def handle(ev):
        if ev is None:
            return None
        if not ev.cuda_event:
            raise ValueError("event not created yet: record it once first")
        return ctypes.c_void_p(ev.cuda_event)
    _check("up_set_copy_events", lib().up_set_copy_events(handle(start), handle(stop)))


def up_history_init(ledger, num_seqs: int, capacity: int, stream=None) -> None:
    _check("up_history_init", lib().up_history_init(_ptr(ledger), num_seqs, capacity,
                                                    _stream(stream, ledger.device)))


def up_drop_history(ledger, num_seqs: int, capacity: int, layer_id: int, cu_seqlens_out,
                    stream=None) -> None:
    """Append (layer id, kept tokens) per request to the ledger (§三)."""
    _check("up_drop_history", lib().up_drop_history(_ptr(ledger), num_seqs, capacity, layer_id,
                                                    _ptr(cu_seqlens_out),
                                                    _stream(stream, ledger.device)))


def up_kv_len(ledger, num_seqs: int, capacity: int, layer_id: int, cu_seqlens_d, kv_len,
              stream=None) -> None:
    """Per-request KV length of layer `layer_id` read back from the ledger (§三)."""
    _check("up_kv_len", lib().up_kv_len(_ptr(ledger), num_seqs, capacity, layer_id,
                                        _ptr(cu_seqlens_d), _ptr(kv_len),
                                        _stream(stream, ledger.device)))


def up_revive(cu_seqlens_h, cu_seqlens_d, cu_blocks_d, block: int, block_mask, packed, full,
              workspace, stream=None) -> None:
    """Write the packed kept rows back to their rows of `full` (§二 step 3,
    revival); rows of dropped blocks in `full` keep their contents."""
    if full.dim() < 1 or (full.dim() > 1 and not full[0].is_contiguous()):
        raise ValueError("full rows must be contiguous")
    if packed.dtype != full.dtype:
        raise ValueError("packed must have full's dtype")
    if packed.dim() > 1 and not packed.is_contiguous():
        raise ValueError("packed must be contiguous")
    cu = _host_i32(cu_seqlens_h)
    row_bytes = (full[0].numel() if full.dim() > 1 else 1) * full.element_size()
    row_stride = full.stride(0) * full.element_size()
    st = lib().up_revive(cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_d), _ptr(cu_blocks_d), block,
                         _ptr(block_mask), _ptr(packed), _ptr(full), row_bytes, row_stride,
                         _ptr(workspace), workspace.numel(), _stream(stream, full.device))
    _check("up_revive", st)


_DTYPES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}


def _rows_2d(name, t):
    if t.dtype not in _DTYPES or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a bf16/f16/f32 [rows, D] tensor with a contiguous last dim")


def up_compact_rmsnorm(cu_seqlens_h, cu_seqlens_d, cu_blocks_d, block: int, block_mask, hidden,
                       gamma: Optional[torch.Tensor], eps: float, positions, normed_out,
                       residual_out: Optional[torch.Tensor], positions_out, cu_seqlens_out,
                       workspace, stream=None) -> None:
    """The next layer's RMS-normalised operand of the kept rows, read straight
    from the frozen rows (§二 step 3, fused pipeline): hidden [T, D]."""
    _rows_2d("hidden", hidden)
    for n, t in (("normed_out", normed_out), ("residual_out", residual_out), ("gamma", gamma)):
        if t is not None and (t.dtype != hidden.dtype or not t.is_contiguous()):
            raise ValueError(f"{n} must be contiguous with hidden's dtype")
    cu = _host_i32(cu_seqlens_h)
    st = lib().up_compact_rmsnorm(cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_d), _ptr(cu_blocks_d),
                                  block, _ptr(block_mask), _DTYPES[hidden.dtype], _ptr(hidden),
                                  hidden.shape[1], hidden.stride(0), _ptr(gamma), eps,
                                  _ptr(positions), _ptr(normed_out), _ptr(residual_out),
                                  _ptr(positions_out), _ptr(cu_seqlens_out), normed_out.shape[0],
                                  _ptr(workspace), workspace.numel(),
                                  _stream(stream, normed_out.device))
    _check("up_compact_rmsnorm", st)


def up_gather_add(cu_seqlens_h, cu_seqlens_d, cu_blocks_d, block: int, block_mask, frozen, delta,
                  out, workspace, stream=None) -> None:
    """Residual sum of the kept rows with the residual read from the frozen
    rows: out[i] = frozen[i-th kept token] + delta[i] (fused pipeline)."""
    _rows_2d("frozen", frozen)
    for n, t in (("delta", delta), ("out", out)):
        if t.dtype != frozen.dtype or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{n} must be a contiguous [rows, D] tensor with frozen's dtype")
    cu = _host_i32(cu_seqlens_h)
    st = lib().up_gather_add(cu.numel() - 1, _ptr(cu), _ptr(cu_seqlens_d), _ptr(cu_blocks_d), block,
                             _ptr(block_mask), _DTYPES[frozen.dtype], _ptr(frozen), frozen.shape[1],
                             frozen.stride(0), _ptr(delta), _ptr(out), out.shape[0],
                             _ptr(workspace), workspace.numel(), _stream(stream, out.device))
    _check("up_gather_add", st)


# ---------------------------------------------------------------------------
# Convenience: batch metadata and buffers (allocation only)
# ---------------------------------------------------------------------------

@dataclass
class Batch:
    """Host and device copies of a packed batch's cu_seqlens and cu_blocks."""
    cu_seqlens_h: torch.Tensor
    cu_seqlens_d: torch.Tensor
    cu_blocks_h: torch.Tensor
    cu_blocks_d: torch.Tensor
    block: int
    num_blocks: int

    @property
    def num_seqs(self) -> int:
        return self.cu_seqlens_h.numel() - 1

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seqlens_h[-1])

    @staticmethod
    def make(cu_seqlens, block: int, device) -> "Batch":
        """Host arrays and their device copies.  The copies are synchronous, so
        the device arrays are ready for calls on any stream."""
        cu_h = _host_i32(cu_seqlens)
        cb_h, n = up_make_cu_blocks(cu_h, block)
        return Batch(cu_h, cu_h.to(device), cb_h, cb_h.to(device), block, n)


@dataclass
class Workspace:
    """Caller-owned buffers of one pass (the library allocates nothing)."""
    score_ws: torch.Tensor
    compact_ws: torch.Tensor
    token_scores: torch.Tensor
    block_scores: torch.Tensor
    block_mask: torch.Tensor
    kept_tokens: torch.Tensor
    hidden_out: torch.Tensor
    positions_out: torch.Tensor
    cu_seqlens_out: torch.Tensor

    @staticmethod
    def make(batch: Batch, hq: int, hkv: int, head_dim: int, n_query: int,
             hidden: torch.Tensor, device) -> "Workspace":
        T, B, N = batch.num_tokens, batch.num_seqs, batch.num_blocks
        sw = up_score_workspace_size(batch.cu_seqlens_h, hq, hkv, head_dim, n_query)
        return Workspace(
            score_ws=torch.empty(sw, dtype=torch.uint8, device=device),
            compact_ws=new_compact_workspace(batch.cu_seqlens_h, batch.block, device),
            token_scores=torch.empty(T, dtype=torch.float32, device=device),
            block_scores=torch.empty(max(N, 1), dtype=torch.float32, device=device),
            block_mask=torch.empty(max(N, 1), dtype=torch.uint8, device=device),
            kept_tokens=torch.empty(max(B, 1), dtype=torch.int32, device=device),
            hidden_out=torch.empty((max(T, 1),) + tuple(hidden.shape[1:]), dtype=hidden.dtype,
                                   device=device),
            positions_out=torch.empty(max(T, 1), dtype=torch.int32, device=device),
            cu_seqlens_out=torch.empty(B + 1, dtype=torch.int32, device=device),
        )


def run_chain(batch: Batch, ws: Workspace, q, k, hidden, positions, ledger, ledger_capacity: int,
              layer_id: int, n_query: int = 128, top_p: float = 0.99, sink: int = 128,
              tail: int = 128, scale: float = 0.0, stream=None, with_token_scores: bool = True):
    """One pass of the whole path: score, select, compact, drop history."""
    up_score(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, q, k, n_query,
             batch.block, scale, ws.token_scores if with_token_scores else None,
             ws.block_scores, ws.score_ws, stream)
    up_select_topp(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, ws.block_scores,
                   batch.block, top_p, sink, tail, ws.block_mask, ws.kept_tokens, stream)
    up_compact(batch.cu_seqlens_h, batch.cu_seqlens_d, batch.cu_blocks_d, batch.block,
               ws.block_mask, hidden, positions, ws.hidden_out, ws.positions_out,
               ws.cu_seqlens_out, ws.compact_ws, stream)
    up_drop_history(ledger, batch.num_seqs, ledger_capacity, layer_id, ws.cu_seqlens_out, stream)
