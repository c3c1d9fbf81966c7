"""Seeded synthetic inputs for causal attention with RoPE and a KV cache.

This module only draws numbers and lays them out; it holds none of the
method's arithmetic (no RoPE, no softmax, no cache addressing).  Tests and
the benchmark take their inputs from here and hand identical values to the
HIP library and to the fp64 oracle.

Recipe (all values are standard normal, the distribution the workloads name):

* float tensors come from ``torch.randn`` driven by a ``torch.Generator`` on
  the tensor's device, seeded per (workload, tensor stream); bf16 tensors are
  drawn in fp32 and rounded to nearest-even by torch's dtype conversion, so
  both sides see the same bf16 values;
* integer data (cached lengths, block-table permutations) come from numpy's
  PCG64 with ``SeedSequence(20260000 + workload_index)``, drawn on the host
  because the host also sizes launch grids from them.

The five named workloads:

1. ``tiny``: B=1, H=4, D=64, S=128, fp32, positions 0..127, then 16 decode
   steps at positions 128..143 into a contiguous fp32 cache of 144 slots.
2. ``gpt2_prefill``: B=4, H=12, D=64, S=512, bf16, no cache.
3. ``qwen_prefill``: B=1, H=32, D=128, S=4096, bf16, cache max_seq 4096.
4. ``contiguous_decode``: B=32, H=32, D=128, bf16, cached lengths uniform
   in [1, 4095] (the new token at index L must fit the 4096-slot cache),
   cache [32, 32, 4096, 128] filled with N(0, 1).
5. ``paged_decode``: B=64, Hq=32, Hkv=8, D=128, bf16, 16-token blocks,
   lengths uniform in [512, 8192], pool of 64*513 blocks, block table taken
   from a seeded random permutation of the pool.

INT8 caches (``int8_decode_case``) have the same shapes with int8 codes drawn
uniformly from [-127, 127] and fp32 per-(KV head, channel) scales drawn
uniformly from [0.01, 0.03], so that cached values spread over about the
range of N(0, 1) data.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

BASE_SEED = 20260000
BLOCK_SIZE = 16

WORKLOADS = ("tiny", "gpt2_prefill", "qwen_prefill", "contiguous_decode", "paged_decode")


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 64 + stream)
    return g


def randn(shape, dtype: torch.dtype, device, seed: int, stream: int) -> torch.Tensor:
    """N(0, 1) values drawn in fp32 and converted (RNE) to ``dtype``."""
    x = torch.randn(tuple(shape), generator=_gen(device, seed, stream),
                    device=device, dtype=torch.float32)
    return x.to(dtype)


def host_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))


@dataclass
class PrefillCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    dtype: torch.dtype
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    positions: torch.Tensor            # int32 [B, S]
    cache_max_seq: Optional[int]       # None: no cache written
    theta: float = 10000.0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


@dataclass
class DecodeCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: torch.dtype
    q: torch.Tensor                    # [B, Hq, D]
    k_new: torch.Tensor                # [B, Hkv, D]
    v_new: torch.Tensor                # [B, Hkv, D]
    seq_lens: torch.Tensor             # int32 [B], tokens already cached
    cache_k: torch.Tensor              # contiguous [B,Hkv,max_seq,D] or pool [nb,Hkv,16,D]
    cache_v: torch.Tensor
    block_table: Optional[torch.Tensor] = None   # int32 [B, max_blocks_per_seq]
    max_seq: int = 0                   # contiguous capacity (0 for paged)
    theta: float = 10000.0
    lens_host: List[int] = field(default_factory=list)
    k_scale: Optional[torch.Tensor] = None   # INT8 cache: fp32 [Hkv, D]
    v_scale: Optional[torch.Tensor] = None

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def max_seq_len(self) -> int:
        """Host-side bound on seq_lens[b] + 1 (tokens attended)."""
        return max(self.lens_host) + 1 if self.lens_host else 1


def prefill_case(name, B, Hq, Hkv, S, D, dtype, seed, device, cache_max_seq=None,
                 pos_offset: int = 0) -> PrefillCase:
    q = randn((B, Hq, S, D), dtype, device, seed, 0)
    k = randn((B, Hkv, S, D), dtype, device, seed, 1)
    v = randn((B, Hkv, S, D), dtype, device, seed, 2)
    pos = (torch.arange(S, dtype=torch.int32) + pos_offset).repeat(B, 1).to(device)
    return PrefillCase(name, B, Hq, Hkv, S, D, dtype, q, k, v, pos.contiguous(),
                       cache_max_seq)


def decode_case(name, B, Hq, Hkv, D, dtype, lens, seed, device, paged: bool,
                max_seq: Optional[int] = None, extra_blocks: int = 0,
                poison_unused: bool = False,
                blocks_per_seq: Optional[int] = None) -> DecodeCase:
    """A decode step over caches filled with N(0, 1).

    ``lens`` are the cached lengths L_b.  Contiguous caches get ``max_seq``
    slots per sequence (default max(L)+1).  Paged pools get
    ``blocks_per_seq`` (default ceil((L_max+1)/16)) blocks per sequence plus
    ``extra_blocks`` owned by no sequence, assigned through a seeded random
    permutation of the pool.  With
    ``poison_unused`` every slot that the step must not read (index > L_b,
    and blocks owned by no sequence) holds NaN.
    """
    lens = [int(x) for x in lens]
    rng = host_rng(seed)
    q = randn((B, Hq, D), dtype, device, seed, 3)
    k_new = randn((B, Hkv, D), dtype, device, seed, 4)
    v_new = randn((B, Hkv, D), dtype, device, seed, 5)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=device)
    if not paged:
        cap = max_seq if max_seq is not None else max(lens) + 1
        ck = randn((B, Hkv, cap, D), dtype, device, seed, 6)
        cv = randn((B, Hkv, cap, D), dtype, device, seed, 7)
        if poison_unused:
            t = torch.arange(cap, device=device)[None, None, :, None]
            far = t > seq_lens.to(torch.int64)[:, None, None, None]
            ck.masked_fill_(far, float("nan"))
            cv.masked_fill_(far, float("nan"))
        return DecodeCase(name, B, Hq, Hkv, D, dtype, q, k_new, v_new, seq_lens,
                          ck, cv, None, cap, lens_host=lens)
    mbps = blocks_per_seq or (max(lens) + 1 + BLOCK_SIZE - 1) // BLOCK_SIZE
    nblocks = B * mbps + extra_blocks
    perm = rng.permutation(nblocks)
    table = perm[: B * mbps].reshape(B, mbps).astype(np.int32)
    ck = randn((nblocks, Hkv, BLOCK_SIZE, D), dtype, device, seed, 6)
    cv = randn((nblocks, Hkv, BLOCK_SIZE, D), dtype, device, seed, 7)
    if poison_unused:
        keep = np.zeros((nblocks, BLOCK_SIZE), dtype=bool)
        for b, L in enumerate(lens):
            t = np.arange(L + 1)
            keep[table[b, t // BLOCK_SIZE], t % BLOCK_SIZE] = True
        far = torch.from_numpy(~keep).to(device)[:, None, :, None]
        ck.masked_fill_(far, float("nan"))
        cv.masked_fill_(far, float("nan"))
    bt = torch.from_numpy(table).to(device)
    return DecodeCase(name, B, Hq, Hkv, D, dtype, q, k_new, v_new, seq_lens, ck, cv,
                      bt.contiguous(), 0, lens_host=lens)


def randcodes(shape, device, seed: int, stream: int) -> torch.Tensor:
    """int8 codes drawn uniformly from [-127, 127]."""
    return torch.randint(-127, 128, tuple(shape), generator=_gen(device, seed, stream),
                         device=device, dtype=torch.int32).to(torch.int8)


def randscales(shape, device, seed: int, stream: int) -> torch.Tensor:
    """fp32 scales drawn uniformly from [0.01, 0.03]."""
    u = torch.rand(tuple(shape), generator=_gen(device, seed, stream), device=device,
                   dtype=torch.float32)
    return 0.01 + 0.02 * u


def int8_decode_case(name, B, Hq, Hkv, D, dtype, lens, seed, device, paged: bool,
                     max_seq: Optional[int] = None, extra_blocks: int = 0,
                     blocks_per_seq: Optional[int] = None) -> DecodeCase:
    """A decode step over an INT8 cache: the layout of ``decode_case`` with
    int8 codes in every slot and per-(KV head, channel) scales."""
    lens = [int(x) for x in lens]
    rng = host_rng(seed)
    q = randn((B, Hq, D), dtype, device, seed, 3)
    k_new = randn((B, Hkv, D), dtype, device, seed, 4)
    v_new = randn((B, Hkv, D), dtype, device, seed, 5)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=device)
    ks = randscales((Hkv, D), device, seed, 8)
    vs = randscales((Hkv, D), device, seed, 9)
    if not paged:
        cap = max_seq if max_seq is not None else max(lens) + 1
        ck = randcodes((B, Hkv, cap, D), device, seed, 6)
        cv = randcodes((B, Hkv, cap, D), device, seed, 7)
        return DecodeCase(name, B, Hq, Hkv, D, dtype, q, k_new, v_new, seq_lens, ck, cv, None,
                          cap, lens_host=lens, k_scale=ks, v_scale=vs)
    mbps = blocks_per_seq or (max(lens) + 1 + BLOCK_SIZE - 1) // BLOCK_SIZE
    nblocks = B * mbps + extra_blocks
    perm = rng.permutation(nblocks)
    table = perm[: B * mbps].reshape(B, mbps).astype(np.int32)
    ck = randcodes((nblocks, Hkv, BLOCK_SIZE, D), device, seed, 6)
    cv = randcodes((nblocks, Hkv, BLOCK_SIZE, D), device, seed, 7)
    bt = torch.from_numpy(table).to(device)
    return DecodeCase(name, B, Hq, Hkv, D, dtype, q, k_new, v_new, seq_lens, ck, cv,
                      bt.contiguous(), 0, lens_host=lens, k_scale=ks, v_scale=vs)


@dataclass
class ChunkCase:
    """A prompt chunk of S tokens per sequence continuing a cached prefix of
    P = lens_host[b] tokens."""
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    dtype: torch.dtype
    q: torch.Tensor                    # [B, Hq, S, D]
    k: torch.Tensor                    # [B, Hkv, S, D]
    v: torch.Tensor
    seq_lens: torch.Tensor             # int32 [B], tokens already cached
    cache_k: torch.Tensor              # contiguous [B,Hkv,max_seq,D] or pool [nb,Hkv,16,D]
    cache_v: torch.Tensor
    block_table: Optional[torch.Tensor] = None
    max_seq: int = 0
    theta: float = 10000.0
    lens_host: List[int] = field(default_factory=list)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def max_seq_len(self) -> int:
        """Host-side bound on seq_lens[b] + S."""
        return max(self.lens_host) + self.S


def chunk_case(name, B, Hq, Hkv, S, D, dtype, lens, seed, device, paged: bool,
               max_seq: Optional[int] = None, extra_blocks: int = 0,
               poison_unused: bool = False, blocks_per_seq: Optional[int] = None) -> ChunkCase:
    """A chunk over caches whose first P_b rows hold N(0, 1) values.

    Contiguous caches get ``max_seq`` slots per sequence (default
    max(P)+S); paged pools get ``blocks_per_seq`` blocks per sequence
    (default ceil((max(P)+S)/16)) plus ``extra_blocks`` owned by no
    sequence, through a seeded random permutation.  With ``poison_unused``
    every slot at or past P_b (the chunk's own slots included, which the call
    writes before it reads them) and every unowned block holds NaN.
    """
    lens = [int(x) for x in lens]
    rng = host_rng(seed)
    q = randn((B, Hq, S, D), dtype, device, seed, 0)
    k = randn((B, Hkv, S, D), dtype, device, seed, 1)
    v = randn((B, Hkv, S, D), dtype, device, seed, 2)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=device)
    if not paged:
        cap = max_seq if max_seq is not None else max(lens) + S
        ck = randn((B, Hkv, cap, D), dtype, device, seed, 6)
        cv = randn((B, Hkv, cap, D), dtype, device, seed, 7)
        if poison_unused:
            t = torch.arange(cap, device=device)[None, None, :, None]
            far = t >= seq_lens.to(torch.int64)[:, None, None, None]
            ck.masked_fill_(far, float("nan"))
            cv.masked_fill_(far, float("nan"))
        return ChunkCase(name, B, Hq, Hkv, S, D, dtype, q, k, v, seq_lens, ck, cv, None, cap,
                         lens_host=lens)
    mbps = blocks_per_seq or (max(lens) + S + BLOCK_SIZE - 1) // BLOCK_SIZE
    nblocks = B * mbps + extra_blocks
    perm = rng.permutation(nblocks)
    table = perm[: B * mbps].reshape(B, mbps).astype(np.int32)
    ck = randn((nblocks, Hkv, BLOCK_SIZE, D), dtype, device, seed, 6)
    cv = randn((nblocks, Hkv, BLOCK_SIZE, D), dtype, device, seed, 7)
    if poison_unused:
        keep = np.zeros((nblocks, BLOCK_SIZE), dtype=bool)
        for b, P in enumerate(lens):
            t = np.arange(P)
            keep[table[b, t // BLOCK_SIZE], t % BLOCK_SIZE] = True
        far = torch.from_numpy(~keep).to(device)[:, None, :, None]
        ck.masked_fill_(far, float("nan"))
        cv.masked_fill_(far, float("nan"))
    bt = torch.from_numpy(table).to(device)
    return ChunkCase(name, B, Hq, Hkv, S, D, dtype, q, k, v, seq_lens, ck, cv, bt.contiguous(), 0,
                     lens_host=lens)


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------

def tiny(device="cpu"):
    """Workload 1: fp32 prefill of 128 tokens, then 16 decode steps."""
    seed = BASE_SEED + 0
    pre = prefill_case("tiny", 1, 4, 4, 128, 64, torch.float32, seed, device,
                       cache_max_seq=144)
    steps = []
    for t in range(16):
        s = seed * 1000 + t
        steps.append((randn((1, 4, 64), torch.float32, device, s, 3),
                      randn((1, 4, 64), torch.float32, device, s, 4),
                      randn((1, 4, 64), torch.float32, device, s, 5)))
    return pre, steps


def gpt2_prefill(device="cpu"):
    return prefill_case("gpt2_prefill", 4, 12, 12, 512, 64, torch.bfloat16,
                        BASE_SEED + 1, device)


def qwen_prefill(device="cpu"):
    return prefill_case("qwen_prefill", 1, 32, 32, 4096, 128, torch.bfloat16,
                        BASE_SEED + 2, device, cache_max_seq=4096)


def contiguous_decode_lens():
    return [int(x) for x in host_rng(BASE_SEED + 3).integers(1, 4096, size=32)]


def paged_decode_lens():
    return [int(x) for x in host_rng(BASE_SEED + 4).integers(512, 8193, size=64)]


def contiguous_decode(device="cpu", poison_unused=False):
    return decode_case("contiguous_decode", 32, 32, 32, 128, torch.bfloat16,
                       contiguous_decode_lens(), BASE_SEED + 3, device, paged=False,
                       max_seq=4096, poison_unused=poison_unused)


def paged_decode(device="cpu", poison_unused=False):
    lens = paged_decode_lens()
    # 513 blocks per sequence cover L + 1 <= 8193 tokens for every sequence.
    return decode_case("paged_decode", 64, 32, 8, 128, torch.bfloat16, lens,
                       BASE_SEED + 4, device, paged=True, poison_unused=poison_unused,
                       blocks_per_seq=513)


def varlen_prefill_lens():
    """Prompt lengths of the padded batch: 8 draws from U{128..2048}."""
    return [int(x) for x in host_rng(BASE_SEED + 50).integers(128, 2049, size=8)]


def varlen_prefill(device="cpu"):
    """A padded batch of whole prompts: B=8, H=32, D=128, S=2048 rows per
    prompt of which the first varlen_prefill_lens()[b] are tokens, bf16,
    positions 0.. (a [8, 32, 2048, 128] cache holds them)."""
    case = prefill_case("varlen_prefill", 8, 32, 32, 2048, 128, torch.bfloat16,
                        BASE_SEED + 50, device, cache_max_seq=2048)
    return case, varlen_prefill_lens()
