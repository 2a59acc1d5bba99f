"""C-ABI checks that need no GPU: the library loads, exports every symbol the
headers declare, host helpers compute what the header says, and arguments
that the host can reject are rejected with a status (never an abort)."""
import ctypes
import glob
import os
import re

import pytest
import torch

import token_block_sparsification_amd as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h, encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"\b(up_[a-z0-9_]+)\s*\(", src):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    lib = U.lib()
    declared = _declared_symbols()
    assert {"up_score", "up_select_topp", "up_compact", "up_drop_history"} <= declared
    missing = [n for n in sorted(declared) if not hasattr(lib, n)]
    assert not missing, missing
    assert U.up_abi_version() == 1


def test_binding_covers_every_declared_symbol():
    declared = _declared_symbols()
    assert declared <= set(U._SIGNATURES), declared - set(U._SIGNATURES)


def test_make_cu_blocks():
    cb, n = U.up_make_cu_blocks([0, 10, 10, 75, 203], 32)
    assert cb.tolist() == [0, 1, 1, 4, 8] and n == 8
    with pytest.raises(U.UniprefillError) as e:
        U.up_make_cu_blocks([0, 10, 5], 32)
    assert e.value.status == 1 and "decreases" in str(e.value)


def test_workspace_sizes():
    cu = [0, 131072]
    ws = U.up_score_workspace_size(cu, 32, 8, 128, 128)
    # partials + biases + per-(KV head, row group) column partials
    assert ws >= 8 * 131072 * 4
    assert U.up_compact_workspace_size(cu, 64) >= 2048 * 8
    assert U.up_history_bytes(3, 5) == 4 * (4 + 3 + 2 * 3 * 5)


def _score_status(**over):
    lib = U.lib()
    cu = torch.tensor([0, 256], dtype=torch.int32)
    args = dict(num_seqs=1, cu_h=cu.data_ptr(), cu_d=16, cb_d=16, q=4096, q_tok=64, q_head=16,
                hq=4, k=8192, k_tok=32, k_head=16, hkv=2, d=64, n=128, G=64, scale=0.0,
                ts=None, bs=16, ws=256, ws_bytes=1 << 30)
    args.update(over)
    st = lib.up_score(args["num_seqs"], args["cu_h"], args["cu_d"], args["cb_d"], args["q"],
                      args["q_tok"], args["q_head"], args["hq"], args["k"], args["k_tok"],
                      args["k_head"], args["hkv"], args["d"], args["n"], args["G"], args["scale"],
                      args["ts"], args["bs"], args["ws"], args["ws_bytes"], None)
    return st, U.up_last_error()


@pytest.mark.parametrize("over,status,msg", [
    (dict(d=96), 2, "head_dim"),
    (dict(hq=6, hkv=4), 1, "hq"),
    (dict(n=0), 2, "n_query"),
    (dict(G=48), 2, "power of two"),
    (dict(G=512), 2, "power of two"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(q=4098), 2, "aligned"),
    (dict(q_tok=60), 2, "aligned"),
    (dict(ws_bytes=16), 3, "workspace"),
    (dict(bs=None), 1, "NULL"),
    (dict(ws=300), 1, "256-byte"),
    (dict(k_tok=(1 << 24) + 8), 2, "k_tok_stride"),
])
def test_score_rejects_bad_arguments(over, status, msg):
    st, err = _score_status(**over)
    assert st == status and msg in err, (st, err)


def test_score_rejects_bad_packing():
    bad = torch.tensor([0, 100, 50], dtype=torch.int32)
    st, err = _score_status(num_seqs=2, cu_h=bad.data_ptr())
    assert st == 1 and "decreases" in err
    nz = torch.tensor([5, 100], dtype=torch.int32)
    st, err = _score_status(cu_h=nz.data_ptr())
    assert st == 1 and "[0]" in err


def test_select_rejects_bad_arguments():
    lib = U.lib()
    cu = torch.tensor([0, 256], dtype=torch.int32)
    for p, sink, tail, msg in [(0.0, 128, 128, "top_p"), (1.5, 128, 128, "top_p"),
                               (0.9, -1, 128, "sink")]:
        st = lib.up_select_topp(1, cu.data_ptr(), 16, 16, 16, 64, p, sink, tail, 16, 16, None)
        assert st == 1 and msg in U.up_last_error()
    big = torch.tensor([0, 64 * ((1 << 24) + 1)], dtype=torch.int32)
    st = lib.up_select_topp(1, big.data_ptr(), 16, 16, 16, 64, 0.99, 128, 128, 16, 16, None)
    assert st == 2 and "blocks" in U.up_last_error()


def test_compact_rejects_bad_arguments():
    lib = U.lib()
    cu = torch.tensor([0, 256], dtype=torch.int32)
    base = [1, cu.data_ptr(), 16, 16, 64, 16, 4096, 512, 512, 4096, 8192, 8192, 16, 256, 256,
            1 << 20, None]
    cases = [((13, 255), 4, "capacity"), ((8, 256), 1, "row_stride"), ((7, 0), 1, "row_bytes"),
             ((15, 16), 3, "workspace"), ((9, None), 1, "positions"), ((14, 300), 1, "256-byte")]
    for (i, v), status, msg in cases:
        a = list(base)
        a[i] = v
        st = lib.up_compact(*a)
        assert st == status and msg in U.up_last_error(), (i, v, st, U.up_last_error())


def test_compact_record_rejects_bad_arguments():
    """up_compact's checks, plus the ledger's (NULL ledger, capacity < 1)."""
    lib = U.lib()
    cu = torch.tensor([0, 256], dtype=torch.int32)
    base = [1, cu.data_ptr(), 16, 16, 64, 16, 4096, 512, 512, 4096, 8192, 8192, 16, 256, 256,
            1 << 20, 4096, 4, 0, None]
    cases = [((13, 255), 4, "capacity"), ((8, 256), 1, "row_stride"), ((7, 0), 1, "row_bytes"),
             ((15, 16), 3, "workspace"), ((9, None), 1, "positions"), ((14, 300), 1, "256-byte"),
             ((16, None), 1, "ledger"), ((17, 0), 1, "capacity >= 1")]
    for (i, v), status, msg in cases:
        a = list(base)
        a[i] = v
        st = lib.up_compact_record(*a)
        assert st == status and msg in U.up_last_error(), (i, v, st, U.up_last_error())


def test_copy_events_need_both_or_neither():
    lib = U.lib()
    assert lib.up_set_copy_events(16, None) == 1 and "both" in U.up_last_error()
    assert lib.up_set_copy_events(None, 16) == 1
    assert lib.up_set_copy_events(None, None) == 0   # clearing touches no device


def test_history_rejects_bad_arguments():
    lib = U.lib()
    assert lib.up_history_init(None, 2, 4, None) == 1
    assert lib.up_history_init(16, 2, 0, None) == 1
    assert lib.up_drop_history(16, 2, 4, 0, None, None) == 1
    assert lib.up_history_bytes(-1, 4) == 0


def test_revive_rejects_bad_arguments():
    lib = U.lib()
    cu = torch.tensor([0, 256], dtype=torch.int32)
    # num_seqs, cu_h, cu_d, cu_blocks_d, block, mask, packed, full, row_bytes, row_stride, ws,
    # ws_bytes, stream
    base = [1, cu.data_ptr(), 16, 16, 64, 16, 4096, 8192, 512, 512, 256, 1 << 20, None]
    cases = [((4, 0), 1, "block"), ((9, 256), 1, "row_stride"), ((8, 0), 1, "row_bytes"),
             ((11, 16), 3, "workspace"), ((6, None), 1, "NULL"), ((10, 300), 1, "256-byte")]
    for (i, v), status, msg in cases:
        a = list(base)
        a[i] = v
        st = lib.up_revive(*a)
        assert st == status and msg in U.up_last_error(), (i, v, st, U.up_last_error())


def test_kv_len_rejects_bad_arguments():
    lib = U.lib()
    assert lib.up_kv_len(None, 2, 4, 0, 16, 16, None) == 1
    assert lib.up_kv_len(16, 2, 0, 0, 16, 16, None) == 1
    assert lib.up_kv_len(16, 2, 4, 0, None, 16, None) == 1
    assert lib.up_kv_len(16, 0, 4, 0, None, None, None) == 0   # no requests: nothing to do


def test_compact_rmsnorm_rejects_bad_arguments():
    lib = U.lib()
    cu = torch.tensor([0, 256], dtype=torch.int32)
    # num_seqs, cu_h, cu_d, cu_blocks_d, block, mask, dtype, hidden, hidden_dim, row_stride,
    # gamma, eps, positions, normed_out, residual_out, positions_out, cu_out, capacity, ws,
    # ws_bytes, stream
    base = [1, cu.data_ptr(), 16, 16, 64, 16, 0, 4096, 2048, 2048, None, 1e-6, 16, 8192, None, 16,
            16, 256, 256, 1 << 20, None]
    cases = [((17, 255), 4, "capacity"), ((6, 7), 1, "dtype"), ((8, 2049), 2, "multiple of 16"),
             ((8, 16384), 2, "16 KiB"), ((9, 2047), 2, "row stride"), ((7, 4100), 2, "aligned"),
             ((11, -1.0), 1, "eps"), ((12, None), 1, "positions"), ((4, 0), 1, "block"),
             ((19, 16), 3, "workspace"), ((13, None), 1, "NULL"), ((10, 8), 2, "aligned")]
    for (i, v), status, msg in cases:
        a = list(base)
        a[i] = v
        st = lib.up_compact_rmsnorm(*a)
        assert st == status and msg in U.up_last_error(), (i, v, st, U.up_last_error())


def test_gather_add_rejects_bad_arguments():
    lib = U.lib()
    cu = torch.tensor([0, 256], dtype=torch.int32)
    # num_seqs, cu_h, cu_d, cu_blocks_d, block, mask, dtype, frozen, hidden_dim, row_stride,
    # delta, out, out_rows, ws, ws_bytes, stream
    base = [1, cu.data_ptr(), 16, 16, 64, 16, 2, 4096, 1024, 1024, 8192, 8192, 256, 256, 1 << 20,
            None]
    cases = [((12, -1), 1, "out_rows"), ((6, 3), 1, "dtype"), ((10, None), 1, "NULL"),
             ((11, 8200), 2, "aligned"), ((9, 1026), 2, "row stride"), ((14, 16), 3, "workspace"),
             ((8, 0), 1, "hidden_dim")]
    for (i, v), status, msg in cases:
        a = list(base)
        a[i] = v
        st = lib.up_gather_add(*a)
        assert st == status and msg in U.up_last_error(), (i, v, st, U.up_last_error())


def test_score_select_rejects_bad_arguments():
    lib = U.lib()
    cu = torch.tensor([0, 256], dtype=torch.int32)
    # up_score's arguments (workspace last before stream), selection in between
    base = [1, cu.data_ptr(), 16, 16, 4096, 1024, 128, 8, 8192, 1024, 128, 8, 128, 128, 64, 0.0,
            None, 16, 0.99, 128, 128, 16, 16, 256, 1 << 30, None]
    cases = [((18, 0.0), 1, "top_p"), ((18, 1.5), 1, "top_p"), ((19, -1), 1, "sink"),
             ((22, None), 1, "NULL"), ((21, None), 1, "NULL"), ((12, 96), 2, "head_dim"),
             ((14, 48), 2, "block"), ((24, 16), 3, "workspace")]
    for (i, v), status, msg in cases:
        a = list(base)
        a[i] = v
        st = lib.up_score_select(*a)
        assert st == status and msg in U.up_last_error(), (i, v, st, U.up_last_error())


def test_compact_status_rejects_bad_arguments():
    """Null pointers, a misaligned or too small workspace are rejected on the
    host (nothing is dereferenced or enqueued)."""
    lib = U.lib()
    dummy = ctypes.c_void_p(1 << 20)
    assert lib.up_compact_status(None, 4096, dummy, 1, None) == 1
    assert lib.up_compact_status(dummy, 4096, None, 1, None) == 1
    assert lib.up_compact_status(ctypes.c_void_p((1 << 20) + 16), 4096, dummy, 1, None) == 1
    assert "aligned" in U.up_last_error()
    assert lib.up_compact_status(dummy, 128, dummy, 1, None) == 3
