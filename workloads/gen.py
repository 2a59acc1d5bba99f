"""Counter-based seeded generator and the workload recipes.

Random numbers
--------------
Every random value is a pure function of (seed, tensor id, element index):

    key   = splitmix64(seed * 2**8 + tensor_id)            (Python ints)
    z(i)  = splitmix64_finalizer(key + (i + 1) * 0x9E3779B97F4A7C15)   (mod 2**64)

which is SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) evaluated at state index i.  A uniform in
[0, 1) is the top 53 bits of z times 2**-53; a standard normal uses the
Box-Muller transform on two such draws (indices 2i and 2i+1).  The integer
part runs in torch int64 arithmetic (wrapping multiply, masked shifts), so
it is bit-identical on CPU and GPU; the fp64 Box-Muller step uses the
device's log/cos, so a CPU and a GPU run may differ in a last ulp.  Parity
tests therefore always hand the *same bytes* to both sides.

Workloads
---------
Shapes follow the pruning method's published setting (tail queries n=128,
block G=64, Top-p 0.99, 128 sink and 128 tail tokens) at Llama-3.1-8B and
Qwen3-Next-like full-attention layer shapes.  Q and K are N(0, 1) drawn in
fp64 and rounded fp64 -> fp32 -> bf16 (round to nearest even at each step).
Planted blocks: for each request and KV head g, u_g is the unit vector of
the mean of the group's tail query rows (the bf16-rounded values, widened);
every key row of a planted block gets k += 2 * u_g, i.e. its projection on
the mean tail-query direction moves by two standard deviations of N(0, 1).
Planted blocks are drawn among blocks that no forced-keep range touches.
Only tail rows of Q are drawn; all other Q rows are NaN (the path must never
read them).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

TID_Q = 1
TID_K = 2
TID_HIDDEN = 3
TID_PLANT = 4
TID_LENGTHS = 5
TID_SCORES = 6


def _s64(u: int) -> int:
    """uint64 bit pattern -> the int64 with the same bits."""
    u &= MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def splitmix64_py(x: int) -> int:
    """Reference SplitMix64 finalizer on Python ints (state already advanced)."""
    z = x & MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tensor_id: int) -> int:
    return splitmix64_py((seed * 256 + tensor_id + GOLDEN) & MASK64)


def _srl(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 tensors holding uint64 bit patterns."""
    return (x >> s) & ((1 << (64 - s)) - 1)


def draw_u64(key: int, index: torch.Tensor) -> torch.Tensor:
    """z(i) for an int64 index tensor; returns int64 tensors of uint64 bits."""
    z = index.to(torch.int64) + 1
    z = z * _s64(GOLDEN) + _s64(key)
    z = (z ^ _srl(z, 30)) * _s64(MIX1)
    z = (z ^ _srl(z, 27)) * _s64(MIX2)
    return z ^ _srl(z, 31)


def uniform53(key: int, index: torch.Tensor) -> torch.Tensor:
    """Uniform doubles in [0, 1) with 53-bit resolution."""
    return _srl(draw_u64(key, index), 11).to(torch.float64) * (2.0 ** -53)


def normal(key: int, index: torch.Tensor) -> torch.Tensor:
    """Standard normal doubles by Box-Muller on draws 2i (radius) and 2i+1 (angle)."""
    i2 = index.to(torch.int64) * 2
    u1 = (_srl(draw_u64(key, i2), 11).to(torch.float64) + 1.0) * (2.0 ** -53)  # (0, 1]
    u2 = _srl(draw_u64(key, i2 + 1), 11).to(torch.float64) * (2.0 ** -53)     # [0, 1)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def round_bf16(x64: torch.Tensor) -> torch.Tensor:
    """fp64 -> fp32 -> bf16, round to nearest even at each step."""
    return x64.to(torch.float32).to(torch.bfloat16)


# ---------------------------------------------------------------------------
# Workload recipes
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    lengths: Optional[tuple]          # None -> drawn (see make_lengths)
    hq: int
    hkv: int
    head_dim: int
    hidden_dim: int
    hidden_dtype: str                 # "f32" | "bf16"
    seed: int
    n_query: int = 128
    block: int = 64
    top_p: float = 0.99
    sink: int = 128
    tail: int = 128
    plant_count: Optional[int] = None  # per request, exact count
    plant_frac: Optional[float] = None  # per request, round(frac * num_blocks)
    num_seqs: int = 1
    len_range: tuple = (4096, 131072)  # log-uniform range when lengths is None
    description: str = ""

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _cfg5(i_n: int, i_g: int) -> Workload:
    n = (32, 128, 512)[i_n]
    g = (32, 64, 128)[i_g]
    return Workload(
        name=f"qwen3next_L131072_n{n}_G{g}", lengths=(131072,), hq=16, hkv=2,
        head_dim=256, hidden_dim=2048, hidden_dtype="bf16", seed=1100 + 3 * i_n + i_g,
        n_query=n, block=g, plant_frac=0.02,
        description=("Qwen3-Next-style full-attention layer, L=131072, 16 q / 2 kv heads, "
                     f"head_dim 256, hidden 2048 bf16, n={n}, G={g}, 2% planted blocks"))


WORKLOADS = {
    "small_L2048": Workload(
        name="small_L2048", lengths=(2048,), hq=4, hkv=4, head_dim=64, hidden_dim=512,
        hidden_dtype="f32", seed=1001, plant_count=3,
        description="single request L=2048, 4/4 heads, head_dim 64, 3 planted blocks, "
                    "hidden 512 fp32"),
    "llama8b_L32768": Workload(
        name="llama8b_L32768", lengths=(32768,), hq=32, hkv=8, head_dim=128, hidden_dim=4096,
        hidden_dtype="bf16", seed=1002, plant_frac=0.05,
        description="Llama-3.1-8B-shaped layer, L=32768, 32 q / 8 kv heads, head_dim 128, "
                    "5% planted blocks, hidden 4096 bf16"),
    "llama8b_L131072": Workload(
        name="llama8b_L131072", lengths=(131072,), hq=32, hkv=8, head_dim=128, hidden_dim=4096,
        hidden_dtype="bf16", seed=1003, plant_frac=0.05,
        description="Llama-3.1-8B-shaped layer, L=131072 single request, 5% planted blocks"),
    "llama8b_L131072_noplant": Workload(
        name="llama8b_L131072_noplant", lengths=(131072,), hq=32, hkv=8, head_dim=128,
        hidden_dim=4096, hidden_dtype="bf16", seed=1004, plant_count=0,
        description="Llama-3.1-8B-shaped layer, L=131072, no planted blocks "
                    "(near-uniform attention: worst case for the keep ratio)"),
    "llama8b_batch16": Workload(
        name="llama8b_batch16", lengths=None, num_seqs=16, hq=32, hkv=8, head_dim=128,
        hidden_dim=4096, hidden_dtype="bf16", seed=1005, plant_frac=0.05,
        description="16 packed requests, lengths log-uniform in [4096, 131072], "
                    "Llama-3.1-8B shapes, 5% planted blocks per request"),
    "llama8b_batch256_L512": Workload(
        name="llama8b_batch256_L512", lengths=(512,) * 256, num_seqs=256, hq=32, hkv=8,
        head_dim=128, hidden_dim=4096, hidden_dtype="bf16", seed=1006, plant_count=1,
        description="256 packed requests of 512 tokens (131,072 in all), Llama-3.1-8B shapes, "
                    "one planted block per request"),
}
for _i_n in range(3):
    for _i_g in range(3):
        _w = _cfg5(_i_n, _i_g)
        WORKLOADS[_w.name] = _w


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def make_lengths(w: Workload) -> list:
    if w.lengths is not None:
        return list(w.lengths)
    key = stream_key(w.seed, TID_LENGTHS)
    u = uniform53(key, torch.arange(w.num_seqs, dtype=torch.int64))
    lo, hi = w.len_range
    return [int(round(math.exp(float(x) * math.log(hi / lo)) * lo)) for x in u]


def cu_from_lengths(lengths: Sequence[int]) -> torch.Tensor:
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


def _forced_block(b: int, L: int, G: int, sink: int, tail: int) -> bool:
    # Input construction only: plants avoid the always-kept sink/tail blocks.
    return b * G < sink or min(b * G + G, L) > L - tail


def _draw_normal_into(out_f64: torch.Tensor, key: int, base_index: int, chunk: int = 1 << 24):
    """Fill a contiguous fp64 tensor with normals for flat indices base .. base+numel."""
    flat = out_f64.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(base_index + s, base_index + e, dtype=torch.int64, device=flat.device)
        flat[s:e] = normal(key, idx)


def make_inputs(w: Workload, device="cpu", lengths: Optional[Sequence[int]] = None,
                with_hidden: bool = True, nan_fill_q: bool = True) -> dict:
    """Build one batch of the workload on `device`.

    Returns a dict with cu_seqlens (int32, CPU), lengths, q/k (bf16 [T,H,d]),
    hidden ([T,D]), positions (int32 [T], request-local arange), planted
    (list of per-request block-index lists) and the workload itself.
    """
    if lengths is None:
        lengths = make_lengths(w)
    lengths = [int(x) for x in lengths]
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    d, hq, hkv = w.head_dim, w.hq, w.hkv
    if hq % hkv != 0:
        raise ValueError("hq must be a multiple of hkv")
    r = hq // hkv
    dev = torch.device(device)

    # --- Q: only tail rows are drawn; every other row is NaN -----------------
    q = torch.full((T, hq, d), float("nan") if nan_fill_q else 0.0,
                   dtype=torch.bfloat16, device=dev)
    kq = stream_key(w.seed, TID_Q)
    for i, L in enumerate(lengths):
        n_eff = min(w.n_query, L)
        if n_eff == 0:
            continue
        t0 = int(cu[i]) + L - n_eff
        tmp = torch.empty((n_eff, hq, d), dtype=torch.float64, device=dev)
        _draw_normal_into(tmp, kq, t0 * hq * d)
        q[t0:t0 + n_eff] = round_bf16(tmp)

    # --- K: all rows, planted blocks shifted before rounding ----------------
    kk = stream_key(w.seed, TID_K)
    kp = stream_key(w.seed, TID_PLANT)
    k = torch.empty((T, hkv, d), dtype=torch.bfloat16, device=dev)
    planted = []
    for i, L in enumerate(lengths):
        s0 = int(cu[i])
        if L == 0:
            planted.append([])
            continue
        k64 = torch.empty((L, hkv, d), dtype=torch.float64, device=dev)
        _draw_normal_into(k64, kk, s0 * hkv * d)
        nb = -(-L // w.block)
        cand = [b for b in range(nb) if not _forced_block(b, L, w.block, w.sink, w.tail)]
        if w.plant_count is not None:
            cnt = w.plant_count
        elif w.plant_frac is not None:
            cnt = int(round(w.plant_frac * nb))
        else:
            cnt = 0
        cnt = min(cnt, len(cand))
        chosen = []
        if cnt > 0:
            u = uniform53(kp, torch.arange(s0 + 0, s0 + len(cand), dtype=torch.int64))
            order = sorted(range(len(cand)), key=lambda j: (float(u[j]), j))
            chosen = sorted(cand[j] for j in order[:cnt])
            n_eff = min(w.n_query, L)
            qt = q[s0 + L - n_eff:s0 + L].to(torch.float64)  # [n_eff, hq, d]
            for g in range(hkv):
                m = qt[:, g * r:(g + 1) * r, :].reshape(-1, d).mean(dim=0)
                nrm = torch.linalg.vector_norm(m)
                if float(nrm) == 0.0:
                    continue
                u_g = m / nrm
                for b in chosen:
                    j0, j1 = b * w.block, min(b * w.block + w.block, L)
                    k64[j0:j1, g, :] += 2.0 * u_g
        planted.append(chosen)
        k[s0:s0 + L] = round_bf16(k64)
        del k64

    out = dict(workload=w, lengths=lengths, cu_seqlens=cu, q=q, k=k, planted=planted,
               positions=torch.cat([torch.arange(L, dtype=torch.int32) for L in lengths]).to(dev)
               if T > 0 else torch.zeros(0, dtype=torch.int32, device=dev))
    if with_hidden:
        out["hidden"] = make_hidden(w, T, device=dev)
    return out


def make_hidden(w: Workload, T: int, device="cpu", dim: Optional[int] = None,
                dtype: Optional[str] = None) -> torch.Tensor:
    """Hidden states [T, D]: N(0, 1) rounded to the workload's dtype."""
    D = int(dim if dim is not None else w.hidden_dim)
    dt = dtype if dtype is not None else w.hidden_dtype
    h64 = torch.empty((T, D), dtype=torch.float64, device=device)
    _draw_normal_into(h64, stream_key(w.seed, TID_HIDDEN), 0)
    if dt == "f32":
        return h64.to(torch.float32)
    if dt == "bf16":
        return round_bf16(h64)
    raise ValueError(dt)


def make_scores(seed: int, n: int, device="cpu") -> torch.Tensor:
    """Positive fp32 block scores (for select-only tests): exp(N(0,1)) rounded to fp32."""
    key = stream_key(seed, TID_SCORES)
    x = normal(key, torch.arange(n, dtype=torch.int64, device=device))
    return torch.exp(x).to(torch.float32)
