"""Seeded synthetic inputs shared by the tests, the oracle checks and the bench.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic (no scores, masks or normalizers), so both the HIP path
and the oracle may consume what it produces.

Recipe (every workload):
  * generator ``torch.Generator(device).manual_seed(seed)``;
  * float32 N(0, 1) draws, times sigma, then rounded to bfloat16
    (round-to-nearest-even, torch's ``.to(torch.bfloat16)``) for bf16 runs;
  * draw order q, k, v for contiguous inputs; for the paged cache first the
    sequence lengths and the page permutation (CPU generator), then q, k, v.
The shapes follow the workloads the pages talk about (Llama-3.2-1B,
Qwen3-1.7B and Gemma-2-9B head layouts; a paged decode batch); no weights or
datasets are involved.
"""

from dataclasses import dataclass, field
import math

import itertools

import torch

NORMALIZERS = ("softmax", "softmax1", "sparsemax", "entmax15")


@dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    D: int
    dtype: str            # "bf16" | "f32"
    causal: bool
    window: int
    softcap: float
    scaling: float
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    seed: int = 1000
    normalizers: tuple = NORMALIZERS


@dataclass(frozen=True)
class PagedDecode:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    block_size: int
    len_lo: int
    len_hi: int
    scaling: float
    max_blocks: int = 0   # 0: ceil(len_hi / block_size)
    causal: bool = True
    window: int = 0
    softcap: float = 0.0
    seed: int = 1005
    normalizers: tuple = NORMALIZERS


# The five workloads (seed 1000 + index).
TINY = Prefill("tiny", 1, 2, 2, 8, 8, 16, "f32", False, 0, 0.0, 0.25, seed=1001)
TINY_MASKED = Prefill("tiny_causal_window4", 1, 2, 2, 8, 8, 16, "f32", True, 4, 0.0, 0.25,
                      seed=1001)
LLAMA = Prefill("llama3.2-1b_prefill", 4, 32, 8, 2048, 2048, 64, "bf16", True, 0, 0.0,
                1.0 / 8.0, seed=1002)
QWEN_SIGMAS = (0.5, 1.0, 2.0)


def qwen(sigma):
    return Prefill(f"qwen3-1.7b_prefill_sigma{sigma}", 2, 16, 8, 8192, 8192, 128, "bf16",
                   True, 0, 0.0, 1.0 / math.sqrt(128.0), sigma_qk=sigma, seed=1003,
                   normalizers=("sparsemax", "entmax15", "softmax1"))


GEMMA = Prefill("gemma2-9b_local", 1, 16, 8, 8192, 8192, 256, "bf16", True, 4096, 50.0,
                1.0 / 16.0, seed=1004, normalizers=("softmax", "softmax1"))
DECODE = PagedDecode("paged_decode", 64, 32, 8, 128, "bf16", 16, 1024, 32768,
                     1.0 / math.sqrt(128.0), seed=1005)


def _torch_dtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _normal(gen, shape, sigma, dtype, device):
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if sigma != 1.0:
        x = x * sigma
    return x.to(_torch_dtype(dtype))


def make_prefill(cfg, device="cpu"):
    """q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] in the workload dtype."""
    gen = torch.Generator(device=device).manual_seed(cfg.seed)
    q = _normal(gen, (cfg.B, cfg.Hq, cfg.Lq, cfg.D), cfg.sigma_qk, cfg.dtype, device)
    k = _normal(gen, (cfg.B, cfg.Hkv, cfg.Lk, cfg.D), cfg.sigma_qk, cfg.dtype, device)
    v = _normal(gen, (cfg.B, cfg.Hkv, cfg.Lk, cfg.D), cfg.sigma_v, cfg.dtype, device)
    return q, k, v


@dataclass
class PagedInputs:
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor   # int32 [B, max_blocks], -1 = unused
    seq_lens: torch.Tensor      # int32 [B]
    block_size: int
    max_blocks: int
    extra: dict = field(default_factory=dict)


def paged_lengths(cfg):
    """Sequence lengths, uniform integers in [len_lo, len_hi] (CPU generator)."""
    gen = torch.Generator().manual_seed(cfg.seed)
    lens = torch.randint(cfg.len_lo, cfg.len_hi + 1, (cfg.B,), generator=gen)
    return lens.to(torch.int32), gen


def make_paged(cfg, device="cpu", nan_tail=True):
    """Paged KV cache with a seeded random-permutation block table.

    k_cache/v_cache [NB, block_size, Hkv, D] with NB = sum_b ceil(len_b / bs);
    logical page j of sequence b is physical page ``perm[off_b + j]``.  Slots
    past a sequence's length in its last page hold NaN (``nan_tail``) so a
    stray read of them poisons the output.
    """
    lens, gen = paged_lengths(cfg)
    bs = cfg.block_size
    pages = [(int(n) + bs - 1) // bs for n in lens]
    nb = sum(pages)
    max_blocks = cfg.max_blocks or (cfg.len_hi + bs - 1) // bs
    if max(pages) > max_blocks:
        raise ValueError("max_blocks too small for the drawn lengths")
    perm = torch.randperm(nb, generator=gen)
    table = torch.full((cfg.B, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b, n_p in enumerate(pages):
        table[b, :n_p] = perm[off:off + n_p].to(torch.int32)
        off += n_p
    dgen = torch.Generator(device=device).manual_seed(cfg.seed + 7919)
    q = _normal(dgen, (cfg.B, cfg.Hq, 1, cfg.D), 1.0, cfg.dtype, device)
    kc = _normal(dgen, (nb, bs, cfg.Hkv, cfg.D), 1.0, cfg.dtype, device)
    vc = _normal(dgen, (nb, bs, cfg.Hkv, cfg.D), 1.0, cfg.dtype, device)
    if nan_tail:
        for b in range(cfg.B):
            n = int(lens[b])
            tail = pages[b] * bs - n
            if tail:
                last = int(table[b, pages[b] - 1])
                kc[last, bs - tail:] = float("nan")
                vc[last, bs - tail:] = float("nan")
    return PagedInputs(q, kc, vc, table.to(device), lens.to(device), bs, max_blocks,
                       extra={"pages": pages, "num_blocks": nb})



@dataclass
class Varlen:
    """A packed variable-length batch: request r has q_lens[r] queries and
    k_lens[r] keys (k_lens[r] >= q_lens[r] for a chunked-prefill shape)."""
    name: str
    q_lens: tuple
    k_lens: tuple
    Hq: int
    Hkv: int
    D: int
    dtype: str
    causal: bool
    window: int
    softcap: float
    scaling: float
    seed: int = 1000


def make_varlen(cfg, device="cpu"):
    """Packed q [total_q, Hq, D], k/v [total_k, Hkv, D] and int32
    cu_seqlens_q / cu_seqlens_k [num_seqs + 1]."""
    gen = torch.Generator(device=device).manual_seed(cfg.seed)
    tq, tk = sum(cfg.q_lens), sum(cfg.k_lens)
    q = _normal(gen, (tq, cfg.Hq, cfg.D), 1.0, cfg.dtype, device)
    k = _normal(gen, (tk, cfg.Hkv, cfg.D), 1.0, cfg.dtype, device)
    v = _normal(gen, (tk, cfg.Hkv, cfg.D), 1.0, cfg.dtype, device)
    cu = lambda lens: torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32,
                                   device=device)
    return q, k, v, cu(cfg.q_lens), cu(cfg.k_lens)
