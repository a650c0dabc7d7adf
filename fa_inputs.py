"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and casts float32 samples to the 16-bit
storage types (IEEE binary16 via numpy, bfloat16 by round-to-nearest-even on
the float32 bit pattern).  It holds none of the attention arithmetic, so both
the CPU reference under ``oracle/`` and the GPU library's tests and benchmark
draw their inputs from here and from nowhere else.

Generator recipe (one independent stream per tensor and head):
    x = default_rng([seed, tensor, b, h]).standard_normal((N, d), float32) * sigma
with tensor 0 = Q, 1 = K, 2 = V and 4 = dO (the upstream gradient dL/dO for
the backward, shaped like Q).  The "spike" workload additionally draws, per
head, one key index j_h = default_rng([seed, 3, b, h]).integers(0, Nkv) and
multiplies that K row by 20 before the cast; with spike_on="query" (the other
reading of that workload) it draws a query index in [0, Nq) the same way and
scales that Q row instead.  Per-head seed sequences make the
generation order-free, so heads can be produced in parallel or one at a time
(for sampled checks at full size) with identical bits.

The workload shapes follow the pages' own examples: a (1, 32, 8192, 128) fp16
causal benchmark in "FlashAttention 1-2-3: The IO-Aware Revolution in LLM
Inference", section "When FlashAttention Doesn't Help", and the
B, H, T, D = 2, 8, 2048, 64 causal call in "Flash Attention — Module 12.3",
section "Using Scaled Dot-Product Attention in PyTorch".  Decode (one query
against a long cache) is the T_q = 1 case of that page's "Prefill vs Decode".

Paged caches (a page pool plus a block table, the storage of serving stacks
named in "FlashAttention 1-2-3 ...", section "Integration in Major Inference
Engines") are synthetic too: default_rng([seed, 5]) draws the sequence
lengths (all Nkv, or uniform in [1, Nkv] when ragged) and then a random
permutation of the pool, whose pages are handed out in that order, sequence
by sequence -- the fragmented free list of a long-running server.  The dense
K and V above are scattered into the pages, so a paged workload holds the
same key and value bits as its dense twin.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

Q, K, V, SPIKE, DOUT, PAGES = 0, 1, 2, 3, 4, 5
SPIKE_FACTOR = 20.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nkv: int
    d: int
    dtype: str            # "f16" or "bf16": storage type of q, k, v
    causal: bool
    seed: int
    sigma_qk: float = 1.0  # standard deviation of Q and K entries
    spike: bool = False    # one K row per head multiplied by SPIKE_FACTOR
    spike_on: str = "key"  # "query": the alternative reading, one Q row per head instead
    out_f32: bool = False  # O written as float32 instead of the input type
    decode: bool = False   # one query per (b, h) against the whole cache
    page_size: int = 0     # > 0: the decode cache is paged (see paged_plan)
    ragged: bool = False   # paged: per-sequence lengths drawn in [1, Nkv]

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32: the exact value handed to the kernels."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def heads(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_256_d64", B=1, H=2, Nq=256, Nkv=256, d=64, dtype="f16",
                 causal=False, seed=0, out_f32=True),
        Workload("prefill_2k_d64", B=2, H=8, Nq=2048, Nkv=2048, d=64, dtype="f16",
                 causal=True, seed=1),
        Workload("prefill_8k_d128", B=1, H=32, Nq=8192, Nkv=8192, d=128, dtype="f16",
                 causal=True, seed=2, sigma_qk=1.5),
        Workload("prefill_16k_d128_bf16", B=1, H=16, Nq=16384, Nkv=16384, d=128,
                 dtype="bf16", causal=True, seed=3, spike=True),
        Workload("decode_32k_d128", B=16, H=32, Nq=1, Nkv=32768, d=128, dtype="f16",
                 causal=False, seed=4, decode=True),
        Workload("decode_32k_d128_paged16", B=16, H=32, Nq=1, Nkv=32768, d=128, dtype="f16",
                 causal=False, seed=4, decode=True, page_size=16),
    ]
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normals(seed: int, tensor: int, b: int, h: int, n: int, d: int) -> np.ndarray:
    """Standard normal float32 samples of shape (n, d) for one (tensor, b, h)."""
    return np.random.default_rng([seed, tensor, b, h]).standard_normal((n, d), dtype=np.float32)


def spike_index(seed: int, b: int, h: int, nkv: int) -> int:
    return int(np.random.default_rng([seed, SPIKE, b, h]).integers(0, nkv))


def f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the 16-bit storage type; return the bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        if not np.isfinite(x).all():
            raise ValueError("bf16 cast expects finite values")
        u = x.view(np.uint32).astype(np.uint64)
        u = u + 0x7FFF + ((u >> 16) & 1)      # round to nearest, ties to even
        return (u >> 16).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def head_tensor(w: Workload, tensor: int, b: int, h: int) -> np.ndarray:
    """Bits of one head of Q, K, V or dO: uint16 array of shape (N, d)."""
    n = w.Nq if tensor in (Q, DOUT) else w.Nkv
    x = normals(w.seed, tensor, b, h, n, w.d)
    if tensor in (Q, K) and w.sigma_qk != 1.0:
        x *= np.float32(w.sigma_qk)
    if w.spike_on not in ("key", "query"):
        raise ValueError(f"spike_on must be 'key' or 'query', got {w.spike_on!r}")
    if w.spike and tensor == (K if w.spike_on == "key" else Q):
        x[spike_index(w.seed, b, h, n)] *= np.float32(SPIKE_FACTOR)
    return f32_to_bits(x, w.dtype)


def make_tensor(w: Workload, tensor: int, threads: int | None = None) -> np.ndarray:
    """Bits of a whole tensor, uint16 array of shape (B, H, N, d), heads drawn in parallel."""
    n = w.Nq if tensor in (Q, DOUT) else w.Nkv
    out = np.empty((w.B, w.H, n, w.d), dtype=np.uint16)

    def one(bh):
        b, h = divmod(bh, w.H)
        out[b, h] = head_tensor(w, tensor, b, h)

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(one, range(w.heads)))
    return out


def make_inputs(w: Workload) -> dict:
    """q, k, v bit arrays (B, H, N, d) plus the recorded spike indices."""
    return {
        "q": make_tensor(w, Q),
        "k": make_tensor(w, K),
        "v": make_tensor(w, V),
        "spikes": spike_indices(w),
    }


def spike_indices(w: Workload) -> list:
    """Per head (b-major), the spiked K row (or Q row when spike_on == "query")."""
    if not w.spike:
        return []
    n = w.Nkv if w.spike_on == "key" else w.Nq
    return [spike_index(w.seed, b, h, n) for b in range(w.B) for h in range(w.H)]


def head_inputs(w: Workload, b: int, h: int):
    """(q, k, v) bits of one head, each (N, d) uint16: the same bits make_tensor yields."""
    return head_tensor(w, Q, b, h), head_tensor(w, K, b, h), head_tensor(w, V, b, h)


def torch_dtype(dtype: str):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def bits_to_torch(bits: np.ndarray, dtype: str):
    """Reinterpret uint16 bit patterns as a CPU torch tensor of the storage type (no copy of values)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch_dtype(dtype))


def torch_to_bits(t) -> np.ndarray:
    """Bit patterns of a 16-bit CPU torch tensor as uint16."""
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# timing-only inputs

def device_normals(shape, dtype: str, seed: int, device):
    """Standard normal samples drawn on the device by torch's seeded generator
    and rounded to the 16-bit type: the same distribution as the host
    generator above, for performance maps over many shapes where drawing on
    the host would dominate.  No parity test and no oracle input uses them."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch_dtype(dtype))


# paged caches

@dataclass(frozen=True)
class PagedPlan:
    """Where each sequence's keys live in a pool of pages."""
    page_size: int
    seq_lens: np.ndarray     # int32 [B]
    block_table: np.ndarray  # int32 [B, max_pages]; -1 past a sequence's last page
    num_pages: int


def paged_plan(seed: int, B: int, max_len: int, page_size: int, ragged: bool = False,
               spare_pages: int = 0, lens=None) -> PagedPlan:
    """Seeded lengths and a shuffled page assignment (see the module docstring).

    lens, if given, fixes the lengths instead of drawing them; spare_pages
    adds pool pages that no sequence uses."""
    rng = np.random.default_rng([seed, PAGES])
    if lens is not None:
        seq = np.asarray(lens, dtype=np.int64)
    elif ragged:
        seq = rng.integers(1, max_len + 1, B)
    else:
        seq = np.full(B, max_len, dtype=np.int64)
    need = -(-seq // page_size)
    max_pages = max(1, -(-max_len // page_size))
    num_pages = int(need.sum()) + spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    start = 0
    for b in range(B):
        table[b, :need[b]] = perm[start:start + need[b]]
        start += int(need[b])
    return PagedPlan(page_size, seq.astype(np.int32), table, num_pages)


def workload_plan(w: Workload) -> PagedPlan:
    return paged_plan(w.seed, w.B, w.Nkv, w.page_size, ragged=w.ragged)


def scatter_to_pages(x: np.ndarray, plan: PagedPlan, layout: str = "hnd", fill: int = 0) -> np.ndarray:
    """Dense [B, H, N, d] cache -> page pool ([P, H, ps, d] 'hnd' or [P, ps, H, d] 'nhd').

    Slots that hold no key of any sequence are set to the bit pattern fill."""
    B, H, N, d = x.shape
    ps = plan.page_size
    shape = (plan.num_pages, H, ps, d) if layout == "hnd" else (plan.num_pages, ps, H, d)
    pool = np.full(shape, fill, dtype=x.dtype)
    for b in range(B):
        n = int(plan.seq_lens[b])
        for t in range(-(-n // ps)):
            rows = min(ps, n - t * ps)
            src = x[b, :, t * ps:t * ps + rows]
            if layout == "hnd":
                pool[plan.block_table[b, t], :, :rows] = src
            else:
                pool[plan.block_table[b, t], :rows] = src.transpose(1, 0, 2)
    return pool


def scatter_to_pages_torch(x, plan: PagedPlan, layout: str = "hnd"):
    """scatter_to_pages for a device tensor x [B, H, N, d] whose lengths are all N
    and N a multiple of the page size (the benchmark's paged workload)."""
    import torch
    B, H, N, d = x.shape
    ps = plan.page_size
    if N % ps or not (plan.seq_lens == N).all():
        raise ValueError("scatter_to_pages_torch needs full sequences of whole pages")
    tiles = x.view(B, H, N // ps, ps, d)
    tiles = tiles.permute(0, 2, 1, 3, 4) if layout == "hnd" else tiles.permute(0, 2, 3, 1, 4)
    pool = torch.empty((plan.num_pages,) + tuple(tiles.shape[2:]), dtype=x.dtype, device=x.device)
    idx = torch.from_numpy(plan.block_table[:, :N // ps].reshape(-1).astype(np.int64)).to(x.device)
    pool[idx] = tiles.reshape((-1,) + tuple(tiles.shape[2:]))
    return pool
