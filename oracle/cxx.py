"""Python access to the C++ oracle (oracle/uniprefill_oracle.cpp).

TEST INFRASTRUCTURE ONLY, like the rest of this package: used by the test
suite, the smoke check and the benchmark's CPU-baseline leg.

The C++ oracle is the plain, single-threaded fp64 definition of steps 1-5 of
the UniPrefill pruning path (the UniPrefill article page, §二 steps 1-3, §三,
Q&A 1).  `module()` returns a module with the numpy oracle's names and
signatures in which the step 1-5 functions (token_scores, block_scores,
forced_blocks, select_request, select_topp, compact, history_append,
run_chain) run in C++; the other helpers (band rule, revival, fused-row
definitions, format rounding) are the numpy oracle's.  That lets the same pins
check both implementations.

The library is compiled with g++ on first use (or by build()), in-tree:
oracle/liboracle_cxx.so.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import types
from typing import Optional, Sequence

import numpy as np

from . import uniprefill_oracle as _np_oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "uniprefill_oracle.cpp")
LIBRARY = os.path.join(HERE, "liboracle_cxx.so")
CXX = os.environ.get("CXX", "g++")
CXXFLAGS = ["-std=c++17", "-O2", "-fPIC", "-shared", "-Wall"]

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double
_SIGNATURES = {
    "uo_token_scores": (_I, [_I, _P, _P, _I, _I64, _I64, _I, _P, _I, _I64, _I64, _I, _I, _I, _D, _P,
                             _I, _P]),
    "uo_block_scores": (None, [_I, _P, _P, _I, _P]),
    "uo_forced_blocks": (None, [_I64, _I, _I, _I, _P]),
    "uo_select_request": (None, [_P, _I64, _I, _D, _I, _I, _P]),
    "uo_select_topp": (None, [_I, _P, _P, _I, _D, _I, _I, _P, _P]),
    "uo_compact": (None, [_I, _P, _I, _P, _P, _I64, _P, _P, _P, _P]),
    "uo_history_entries": (None, [_I, _I, _P, _P]),
}


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile `source` into the shared library `output` (g++, C++17)."""
    tmp = output + ".tmp"
    p = subprocess.run([CXX, *CXXFLAGS, source, "-o", tmp], stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"building the C++ oracle failed:\n{p.stdout}")
    os.replace(tmp, output)
    return output


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """The oracle library at `path` (built first when it is missing or older
    than its source)."""
    if path == LIBRARY and (not os.path.exists(path) or
                            os.path.getmtime(path) < os.path.getmtime(SOURCE)):
        build()
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _cu64(cu_seqlens) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def _operand(x):
    """(array, kind, token stride, head stride) of a [T, H, d] operand: fp64
    values (kind 0) or bf16 bit patterns in a uint16/int16 array (kind 1)."""
    x = np.asarray(x)
    if x.dtype in (np.uint16, np.int16):
        a, kind = np.ascontiguousarray(x), 1
    else:
        a, kind = np.ascontiguousarray(x, dtype=np.float64), 0
    return a, kind, a.strides[0] // a.itemsize, a.strides[1] // a.itemsize


def module(lib: Optional[ctypes.CDLL] = None) -> types.ModuleType:
    """The oracle API with steps 1-5 served by the C++ library `lib`."""
    lib = lib if lib is not None else load()
    m = types.ModuleType("oracle_cxx")
    for name in dir(_np_oracle):
        if not name.startswith("__"):
            setattr(m, name, getattr(_np_oracle, name))

    def token_scores(q, k, cu_seqlens, n_query: int, scale: Optional[float] = None,
                     heads: Optional[Sequence[int]] = None):
        """Per-token scores c [T] (steps 1-2); q, k as fp64 arrays or bf16 bits."""
        qa, qk, qt, qh = _operand(q)
        ka, kk, kt, kh = _operand(k)
        cu = _cu64(cu_seqlens)
        hq, hkv, d = qa.shape[1], ka.shape[1], qa.shape[2]
        c = np.zeros(int(cu[-1]), dtype=np.float64)
        hs = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        st = lib.uo_token_scores(len(cu) - 1, _ptr(cu), _ptr(qa), qk, qt, qh, hq, _ptr(ka), kk, kt,
                                 kh, hkv, d, int(n_query), 0.0 if scale is None else float(scale),
                                 _ptr(hs), 0 if hs is None else len(hs), _ptr(c))
        if st != 0:
            raise ValueError("Hq must be a multiple of Hkv")
        return c

    def block_scores(c, cu_seqlens, G: int):
        cu = _cu64(cu_seqlens)
        c = np.ascontiguousarray(c, dtype=np.float64)
        out = np.zeros(int(_np_oracle.block_offsets(cu, G)[-1]), dtype=np.float64)
        lib.uo_block_scores(len(cu) - 1, _ptr(cu), _ptr(c), G, _ptr(out))
        return out

    def forced_blocks(L: int, G: int, sink: int, tail: int):
        out = np.zeros((L + G - 1) // G, dtype=np.uint8)
        lib.uo_forced_blocks(L, G, sink, tail, _ptr(out))
        return out.astype(bool)

    def select_request(bs, L: int, G: int, p: float, sink: int, tail: int):
        bs = np.ascontiguousarray(bs, dtype=np.float64)
        keep = np.zeros((L + G - 1) // G, dtype=np.uint8)
        assert len(bs) == len(keep)
        lib.uo_select_request(_ptr(bs), L, G, float(p), sink, tail, _ptr(keep))
        return keep.astype(bool)

    def select_topp(bscores, cu_seqlens, G: int, p: float, sink: int, tail: int):
        cu = _cu64(cu_seqlens)
        bs = np.ascontiguousarray(bscores, dtype=np.float64)
        mask = np.zeros(int(_np_oracle.block_offsets(cu, G)[-1]), dtype=np.uint8)
        kept = np.zeros(len(cu) - 1, dtype=np.int64)
        lib.uo_select_topp(len(cu) - 1, _ptr(cu), _ptr(bs), G, float(p), sink, tail, _ptr(mask),
                           _ptr(kept))
        return mask, kept

    def compact(mask, hidden, positions, cu_seqlens, G: int):
        cu = _cu64(cu_seqlens)
        mask = np.ascontiguousarray(mask, dtype=np.uint8)
        hidden = np.ascontiguousarray(hidden)
        T = int(cu[-1])
        row_bytes = hidden.nbytes // max(T, 1) if T else 0
        pos = None if positions is None else np.ascontiguousarray(positions, dtype=np.int32)
        h_out = np.empty_like(hidden)
        p_out = None if pos is None else np.empty_like(pos)
        cu_out = np.zeros(len(cu), dtype=np.int64)
        lib.uo_compact(len(cu) - 1, _ptr(cu), G, _ptr(mask), _ptr(hidden), row_bytes, _ptr(pos),
                       _ptr(h_out), _ptr(p_out), _ptr(cu_out))
        n = int(cu_out[-1])
        return h_out[:n], (None if p_out is None else p_out[:n]), cu_out

    def history_append(ledger, layer_id: int, cu_out) -> None:
        cu = _cu64(cu_out)
        ent = np.zeros(2 * len(ledger), dtype=np.int64)
        lib.uo_history_entries(len(ledger), int(layer_id), _ptr(cu), _ptr(ent))
        for b in range(len(ledger)):
            ledger[b].append((int(ent[2 * b]), int(ent[2 * b + 1])))

    def run_chain(q, k, hidden, positions, cu_seqlens, n_query=128, G=64, p=0.99, sink=128,
                  tail=128, scale=None, layer_id=0):
        """The whole path on one batch, every step in C++."""
        c = token_scores(q, k, cu_seqlens, n_query, scale)
        bsc = block_scores(c, cu_seqlens, G)
        mask, kept = select_topp(bsc, cu_seqlens, G, p, sink, tail)
        h_out, p_out, cu_out = compact(mask, hidden, positions, cu_seqlens, G)
        ledger = m.history_new(len(cu_seqlens) - 1)
        history_append(ledger, layer_id, cu_out)
        return dict(token_scores=c, block_scores=bsc, mask=mask, kept=kept, hidden_out=h_out,
                    positions_out=p_out, cu_out=cu_out, ledger=ledger)

    for fn in (token_scores, block_scores, forced_blocks, select_request, select_topp, compact,
               history_append, run_chain):
        setattr(m, fn.__name__, fn)
    m.math = math
    return m
