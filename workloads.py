"""Seeded synthetic inputs for the attention hot path.

This module only draws and casts numbers; it holds none of the attention
arithmetic. Both the oracle-side tests and the GPU path take their inputs from
here, so the two sides see bit-identical values.

Workloads (shapes of the models the pages train, with iid N(0,1) data standing
in for real activations -- the pages' datasets and weights are not used):

* ``tiny``     -- exactness case, fp32, N=128, d=64.
* ``gpt2``     -- GPT-2-small attention shape at sequence length 1K (the
  FlashAttention abstract's GPT-2 workload), bf16, causal.
* ``bert``     -- BERT-large attention shape at sequence length 512 (the
  FlashAttention abstract's BERT-large workload), bf16, non-causal.
* ``llama16k`` -- Llama-7B heads (DistFlashAttn reviews, the Llama-7B
  experiments) at a 16K context, bf16, causal; also run as 4 KV chunks.
* ``gqa64k``   -- grouped-query attention (DistFlashAttn reviews, the GQA
  setting) with 32 query heads over 8 K/V heads at a 64K context, bf16,
  causal, processed as 8 chunks.

Draw order (fixed): ``torch.Generator('cpu').manual_seed(seed)``, then
``randn`` in float32 for Q, K, V, dO at their [B, N, heads, d] shapes, then a
round-to-nearest-even cast to the compute dtype.

Key/value-cache workloads (decode and chunked prefill, inference use of the
method): ``decode16k`` -- 16 sequences, 32 query heads over 8 K/V heads
(Llama-style GQA), d=128, one new row per sequence against a 16K-row cache
whose valid lengths are drawn uniformly from [8K, 16K]; ``prefill16k`` -- 4
sequences appending 128 rows each to the same kind of cache. Draw order:
Q [B, Nq, H, d], K cache, V cache [B, Nk, Hkv, d] as above, then the lengths
with ``torch.randint`` from the same generator.

Packed variable-length workload (a training batch of documents of different
lengths stored back to back): ``packed16k`` -- Llama-7B heads, bf16, causal,
16384 tokens split into sequences whose lengths are drawn uniformly from
[256, 4096] until the tokens run out (the last one takes the remainder).
Draw order: the lengths with ``torch.randint`` one at a time, then Q, K, V,
dO at [total, heads, d] from the same generator.

Block masks (block-sparse attention): ``draw_block_mask`` keeps each block
of 256 query rows x 128 keys with probability ``density`` (``torch.rand``
from its own seeded generator, one value per block in row-major order) and,
if asked, every block that holds part of the diagonal, so that no row is left
without keys under the causal mask. The benchmark runs the llama16k tensors
with a quarter of the blocks kept plus the diagonal (seed 9).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    dtype: str                 # "f32" or "bf16"
    causal: tuple              # mask settings the workload is run with
    chunks: int = 1            # KV chunks for the chunked driver (1 = single pass)
    seed: int = 1

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def G(self) -> int:
        return self.H // self.Hkv


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 2, 128, 64, "f32", (False, True), 1, seed=1),
    "gpt2": Workload("gpt2", 8, 12, 12, 1024, 64, "bf16", (True,), 1, seed=2),
    "bert": Workload("bert", 32, 16, 16, 512, 64, "bf16", (False,), 1, seed=3),
    "llama16k": Workload("llama16k", 1, 32, 32, 16384, 128, "bf16", (True,), 4, seed=4),
    "gqa64k": Workload("gqa64k", 1, 32, 8, 65536, 128, "bf16", (True,), 8, seed=5),
}


def draw(B: int, H: int, Hkv: int, N: int, d: int, seed: int,
         dtype: torch.dtype = torch.bfloat16, q_gain: float = 1.0):
    """Return (q, k, v, do) as CPU tensors of ``dtype`` in [B, N, heads, d].

    ``q_gain`` multiplies the fp32 Q draw before the cast; a gain well above 1
    gives peaked softmax rows (stress inputs), 0 gives uniform rows.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((B, N, H, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, N, Hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, N, Hkv, d), generator=g, dtype=torch.float32)
    do = torch.randn((B, N, H, d), generator=g, dtype=torch.float32)
    if q_gain != 1.0:
        q = q * q_gain
    return tuple(t.to(dtype) for t in (q, k, v, do))


def draw_workload(w: Workload, seed: int | None = None, N: int | None = None):
    """Inputs for workload ``w`` (optionally at a shorter sequence length)."""
    return draw(w.B, w.H, w.Hkv, w.N if N is None else N, w.d,
                w.seed if seed is None else seed, w.torch_dtype)


@dataclass(frozen=True)
class CacheWorkload:
    name: str
    B: int
    H: int
    Hkv: int
    Nq: int                    # new query rows per sequence
    Nk: int                    # cache capacity (rows)
    d: int
    min_len: int               # valid cache lengths drawn from [min_len, Nk]
    seed: int = 1


CACHE_WORKLOADS = {
    "decode16k": CacheWorkload("decode16k", 16, 32, 8, 1, 16384, 128, 8192, seed=6),
    "prefill16k": CacheWorkload("prefill16k", 4, 32, 8, 128, 16384, 128, 8192, seed=7),
}


def draw_cache(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int,
               min_len: int | None = None, dtype: torch.dtype = torch.bfloat16):
    """Return (q [B, Nq, H, d], k_cache, v_cache [B, Nk, Hkv, d], lens [B] int32)
    as CPU tensors; lens uniform in [min_len, Nk] (all Nk if min_len is None)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((B, Nq, H, d), generator=g, dtype=torch.float32).to(dtype)
    k = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32).to(dtype)
    v = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32).to(dtype)
    if min_len is None:
        lens = torch.full((B,), Nk, dtype=torch.int32)
    else:
        lens = torch.randint(min_len, Nk + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    return q, k, v, lens


def draw_cache_workload(w: CacheWorkload):
    return draw_cache(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.seed, w.min_len)


@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    total: int                 # packed tokens
    H: int
    Hkv: int
    d: int
    min_len: int               # sequence lengths drawn from [min_len, max_draw]
    max_draw: int
    seed: int = 1


VARLEN_WORKLOADS = {
    "packed16k": VarlenWorkload("packed16k", 16384, 32, 32, 128, 256, 4096, seed=8),
}


def draw_varlen(lengths, H: int, Hkv: int, d: int, seed: int, dtype: torch.dtype = torch.bfloat16,
                gen: torch.Generator | None = None):
    """Return (q, k, v, do [total, heads, d], cu_seqlens int32 [nseq + 1]) as CPU
    tensors for sequences of the given lengths (zero-length ones allowed)."""
    g = torch.Generator("cpu").manual_seed(int(seed)) if gen is None else gen
    lengths = [int(x) for x in lengths]
    total = sum(lengths)
    q = torch.randn((total, H, d), generator=g, dtype=torch.float32).to(dtype)
    k = torch.randn((total, Hkv, d), generator=g, dtype=torch.float32).to(dtype)
    v = torch.randn((total, Hkv, d), generator=g, dtype=torch.float32).to(dtype)
    do = torch.randn((total, H, d), generator=g, dtype=torch.float32).to(dtype)
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32) if lengths else \
        torch.zeros(1, dtype=torch.int32)
    return q, k, v, do, cu


def draw_varlen_workload(w: VarlenWorkload, total: int | None = None):
    """Inputs of ``w`` (optionally with fewer packed tokens): the lengths are
    drawn first, then the tensors, from one generator."""
    total = w.total if total is None else int(total)
    g = torch.Generator("cpu").manual_seed(int(w.seed))
    lengths, left = [], total
    while left > 0:
        n = int(torch.randint(w.min_len, w.max_draw + 1, (1,), generator=g).item())
        lengths.append(min(n, left))
        left -= lengths[-1]
    return draw_varlen(lengths, w.H, w.Hkv, w.d, w.seed, gen=g)


def draw_block_mask(N: int, density: float, seed: int, diagonal: bool = True,
                    rows: int = 256, cols: int = 128) -> torch.Tensor:
    """uint8 CPU tensor [ceil(N / rows), ceil(N / cols)]: 1 = block kept."""
    nbr, nbc = (N + rows - 1) // rows, (N + cols - 1) // cols
    g = torch.Generator("cpu").manual_seed(int(seed))
    m = (torch.rand((nbr, nbc), generator=g) < density).to(torch.uint8)
    if diagonal:
        for r in range(nbr):
            lo, hi = r * rows, min(N, (r + 1) * rows) - 1
            m[r, lo // cols:hi // cols + 1] = 1
    return m


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a CPU tensor (bf16 or fp32) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def flops(B: int, H: int, N: int, d: int, causal: bool) -> tuple[float, float]:
    """Algorithmic FLOPs (forward, backward) under the 4*N^2*d convention.

    Forward counts the two N x N x d products (2 FLOP per multiply-add each),
    halved under a causal mask; backward counts 2.5x the forward.
    H is the number of query heads, also under grouped-query attention.
    """
    f = 4.0 * B * H * N * N * d
    if causal:
        f *= 0.5
    return f, 2.5 * f
