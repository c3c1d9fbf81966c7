"""Benchmark of the attention hot path on one MI355X (filled in below)."""

from __future__ import annotations


def prefill_flops(B: int, H: int, S: int, D: int) -> int:
    """Algorithmic prefill flops: QK^T and PV over the causal (unmasked)
    pairs only, 2 flops per multiply-add: 2 * 2 * B*H*D * S(S+1)/2."""
    return 2 * B * H * D * S * (S + 1)


def decode_kv_bytes(lens, Hkv: int, D: int, elem_bytes: int) -> int:
    """Algorithmic KV bytes one decode step reads: every cached K and V row
    of every KV head once (GQA query heads share their KV head's read)."""
    return sum(int(L) for L in lens) * Hkv * D * 2 * elem_bytes
