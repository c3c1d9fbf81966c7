"""Plain fp64 definitions of RoPE, causal attention and the KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path
never imports this module.

Shapes follow the head-split form of multi-head attention ([Scratch] §3.1;
[Guide] §5.1): Q is [B, Hq, S, D]; K and V are [B, Hkv, S, D].  A contiguous
cache holds K and V as separate tensors [B, Hkv, max_seq, D] ([NanoVLLM] §05,
5.2: K and V are separate tensors; [Intuition] §5: head-major layout).  A
paged cache holds K and V pools [num_blocks, Hkv, block_size, D] plus an
int32 block table [B, max_blocks_per_seq] ([NanoVLLM] §05, 5.3: logical
block -> physical block, offset inside the block).

Pins (tests under ``tests/test_oracle_*.py``, none reuses this code):

* ``rope_inv_freq`` / ``rope_rotate``: identity at position 0; exact norm
  preservation; scores depend only on relative position; hand values
  (cos 1, sin 1) for D = 2 and the i = 1 frequency 10000^(-2/4) = 0.01
  for D = 4, which also separates adjacent from half-split pairing.
* ``causal_attention``: rows of P sum to 1; K = 0 gives the causal prefix
  mean; causality under perturbation of later positions; a scalar
  brute force on tiny shapes; a hand-worked 2-token example; an fp64
  blockwise online softmax in the test agrees to 1e-12.
* ``kv_cache_append`` / ``cache_rows`` / ``paged_slot``: paged under random
  block tables equals contiguous; written slots hold exactly the values.
* ``attn_decode``: L = 0 gives O = v_new; step t equals the last row of a
  full-recompute prefill over the same tokens; GQA equals MHA with each
  KV head repeated.
* ``attn_prefill_cached``: a prompt taken as one chunk equals the same
  prompt taken as two chunks over the cache (outputs and cache contents); a
  one-token chunk equals a decode step; an empty prefix and a one-token
  chunk give O = v; outputs of earlier queries do not move when later chunk
  tokens change, and all of them move when the cached prefix changes; GQA
  equals MHA with each KV head repeated.  With ``chunk_lens``: a padded
  batch equals each sequence run alone at its own length, whatever the
  padding holds; padding rows are zero and padding tokens are not stored.
* ``attn_prefill(seq_lens=...)``: a padded batch of prompts equals each
  prompt run alone at its own length, whatever the padding (even NaN)
  holds; padding rows of the output and of k_rot are zero; a length-1
  prompt gives O = v of its token.

* ``rope_rotate(pairing="half")``: identity at 0, norm preservation and
  relative position as above; a hand value for D = 4 (pair (x1, x3) at
  frequency 0.01); and the exact relation half(x) = P^-1 adjacent(P x) for
  the permutation P that interleaves the two halves, which ties it to the
  independently pinned adjacent layout.

Convention choices with no pin on synthetic data ("parity unpinned"):
adjacent pairs (2i, 2i+1) as the default RoPE layout, and contiguous GQA
groups.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "rope_inv_freq",
    "rope_pair_index",
    "rope_rotate",
    "causal_attention",
    "attn_prefill",
    "kv_cache_append",
    "cache_rows",
    "attn_decode",
    "attn_prefill_cached",
    "paged_slot",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# RoPE  ([Intuition] §4, the Transformer core and RoPE)
# --------------------------------------------------------------------------

def rope_inv_freq(D: int, theta: float = 10000.0) -> np.ndarray:
    """Per-pair angular frequency theta_i = theta^(-2i/D), i in [0, D/2).

    [Intuition] §4 gives theta_i as 10000 raised to -2i/d and builds i with an
    arange over d//2 in floating point (not integer) arithmetic.
    """
    if D % 2:
        raise ValueError("head dimension must be even for RoPE pairs")
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / D)


def rope_pair_index(D: int, pairing: str = "adjacent"):
    """Element indices (a_i, b_i) of pair i, i in [0, D/2).

    "adjacent": (2i, 2i+1), the pairs (q0,q1), (q2,q3), ... that [Intuition]
    §4 writes out.  "half": (i, i + D/2), the split-in-halves layout that
    checkpoints of the Llama/Qwen families use (the pages name those models,
    [Guide] §6.1); the same rotations, applied to a permutation of the
    elements.
    """
    i = np.arange(D // 2)
    if pairing == "adjacent":
        return 2 * i, 2 * i + 1
    if pairing == "half":
        return i, i + D // 2
    raise ValueError(f"unknown RoPE pairing {pairing!r}")


def rope_rotate(x, positions, theta: float = 10000.0, pairing: str = "adjacent") -> np.ndarray:
    """Rotate each pair (x[a_i], x[b_i]) by the angle m * theta_i.

    ``x`` is [..., S, D]; ``positions`` (m) broadcasts against [..., S].  Each
    pair is multiplied by the 2x2 matrix [[cos, -sin], [sin, cos]] of its
    angle, the rotation [Intuition] §4 writes out for the pairs (q0,q1),
    (q2,q3), ..., with m the token's position index; ``pairing`` chooses
    which elements form pair i (``rope_pair_index``).
    """
    x = _f64(x)
    D = x.shape[-1]
    m = _f64(positions)[..., None]                      # [..., S, 1]
    ang = m * rope_inv_freq(D, theta)                   # [..., S, D/2]
    c, s = np.cos(ang), np.sin(ang)
    R = np.stack([np.stack([c, -s], axis=-1),
                  np.stack([s, c], axis=-1)], axis=-2)  # [..., S, D/2, 2, 2]
    ia, ib = rope_pair_index(D, pairing)
    pairs = np.stack([x[..., ia], x[..., ib]], axis=-1)  # [..., S, D/2, 2]
    rot = np.einsum("...ij,...j->...i", R, pairs)
    out = np.empty_like(x)
    out[..., ia] = rot[..., 0]
    out[..., ib] = rot[..., 1]
    return out


# --------------------------------------------------------------------------
# Scaled dot-product attention with the causal mask
# ([Guide] §2.3 and §5.1; [Scratch] §3.1 and §3.3)
# --------------------------------------------------------------------------

def causal_attention(q, k, v, positions, scale: float) -> np.ndarray:
    """softmax(q k^T * scale + mask) v for one (sequence, head).

    q is [Sq, D]; k and v are [Sk, D]; ``positions`` is a pair
    (query positions [Sq], key positions [Sk]).  Key j is masked (-inf) for
    query i when its position is later ([Guide] §5.1: the upper-right triangle
    is set to -inf; [Scratch] §3.3: a position sees itself and earlier ones,
    -inf marks a blocked entry).  The full score matrix is formed on purpose.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    qpos, kpos = (np.asarray(p) for p in positions)
    scores = (q @ k.T) * scale
    blocked = kpos[None, :] > qpos[:, None]
    scores = np.where(blocked, -np.inf, scores)
    rowmax = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - rowmax)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v


def attn_prefill(q, k, v, positions, theta: float = 10000.0,
                 scale: float | None = None, pairing: str = "adjacent", seq_lens=None):
    """Prefill over a whole prompt: RoPE on Q and K, then causal attention.

    q [B, Hq, S, D], k/v [B, Hkv, S, D], positions [B, S].  Query head hq
    reads KV head hq // (Hq // Hkv) (contiguous GQA groups; a convention, the
    pages only name GQA).  The scale defaults to 1/sqrt(D), applied to the
    scores before the softmax ([Intuition] §4: 1/sqrt(d_k) with d_k the head
    dimension; [Scratch] §3.1).

    With ``seq_lens`` (a batch of prompts of different lengths padded to S;
    [Scratch] §3.3 names the padding mask) prompt b has only its first
    seq_lens[b] rows: padding keys are masked for every query besides the
    causal mask, padding rows of the output are zero, and padding rows of
    k_rot are zero (they are never stored).

    Returns (out [B, Hq, S, D], k_rot [B, Hkv, S, D]); V is not rotated.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    positions = np.asarray(positions)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros_like(q)
    k_rot = np.zeros_like(k)
    for b in range(B):
        n = S if seq_lens is None else min(max(int(seq_lens[b]), 0), S)
        if n == 0:
            continue
        pos = positions[b, :n]
        q_rot = rope_rotate(q[b, :, :n], pos[None, :], theta, pairing)
        k_rot[b, :, :n] = rope_rotate(k[b, :, :n], pos[None, :], theta, pairing)
        for hq in range(Hq):
            hk = hq // group
            out[b, hq, :n] = causal_attention(q_rot[hq], k_rot[b, hk, :n], v[b, hk, :n],
                                              (pos, pos), scale)
    return out, k_rot


# --------------------------------------------------------------------------
# KV cache  ([Guide] §2.5; [Scratch] §3.2; [NanoVLLM] §05)
# --------------------------------------------------------------------------

def paged_slot(block_table, b: int, t: int, block_size: int):
    """Physical (block, offset) of token t of sequence b in a paged cache.

    [NanoVLLM] §05 (5.3) looks the physical block up in the block table at
    t // block_size and takes t % block_size as the offset inside it.
    """
    return int(block_table[b, t // block_size]), t % block_size


def kv_cache_append(cache_k, cache_v, k_rot, v, positions,
                    block_table=None, block_size: int = 16):
    """Write rotated keys and raw values at cache index == position.

    [Scratch] §3.2: each new token's K and V go to the cache slot of its
    absolute position, which must equal the cache index.  ``cache_k`` and
    ``cache_v`` are modified in place (contiguous [B, Hkv, max_seq, D] or
    paged pools [num_blocks, Hkv, block_size, D]); k_rot and v are
    [B, Hkv, S, D] with positions [B, S].
    """
    positions = np.asarray(positions)
    B, Hkv, S, _ = np.shape(k_rot)
    for b in range(B):
        for s in range(S):
            t = int(positions[b, s])
            if block_table is None:
                cache_k[b, :, t, :] = k_rot[b, :, s, :]
                cache_v[b, :, t, :] = v[b, :, s, :]
            else:
                blk, off = paged_slot(block_table, b, t, block_size)
                cache_k[blk, :, off, :] = k_rot[b, :, s, :]
                cache_v[blk, :, off, :] = v[b, :, s, :]


def cache_rows(cache, b: int, hk: int, n: int, block_table=None,
               block_size: int = 16) -> np.ndarray:
    """Rows 0..n-1 of sequence b, KV head hk, as an [n, D] float64 array."""
    if block_table is None:
        return _f64(cache[b, hk, :n, :])
    t = np.arange(n)
    blocks = np.asarray(block_table)[b, t // block_size]   # paged_slot, all tokens at once
    return _f64(cache[blocks, hk, t % block_size, :])


def attn_decode(q, k_new, v_new, cache_k, cache_v, seq_lens,
                theta: float = 10000.0, scale: float | None = None,
                block_table=None, block_size: int = 16, pairing: str = "adjacent"):
    """One decode step: a single new query token per sequence.

    For sequence b with L = seq_lens[b] tokens already cached, the new
    token's position is L.  q [B, Hq, D] and k_new [B, Hkv, D] are rotated
    at position L; the rotated key and raw value are written to cache index
    L ([Scratch] §3.2); the query then attends over cache rows 0..L, the L
    cached tokens plus itself ([Guide] §2.5: only the new token's Q, K, V
    are computed; K and V of earlier tokens never change).  With the cache
    there is no further mask: the (1, S) row is all visible ([Scratch] §3.3).

    The caches are updated in place (float64 copies are the caller's
    choice).  Returns out [B, Hq, D].
    """
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    B, Hq, D = q.shape
    Hkv = k_new.shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    seq_lens = np.asarray(seq_lens)
    out = np.empty((B, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        q_rot = rope_rotate(q[b][:, None, :], np.array([L]), theta, pairing)[:, 0, :]
        k_rot = rope_rotate(k_new[b][:, None, :], np.array([L]), theta, pairing)  # [Hkv, 1, D]
        v_one = v_new[b][None, :, None, :]                                # [1, Hkv, 1, D]
        if block_table is None:
            kv_cache_append(cache_k[b:b + 1], cache_v[b:b + 1], k_rot[None], v_one,
                            np.array([[L]]))
        else:
            kv_cache_append(cache_k, cache_v, k_rot[None], v_one, np.array([[L]]),
                            block_table=block_table[b:b + 1], block_size=block_size)
        pos = np.arange(L + 1)
        for hq in range(Hq):
            hk = hq // group
            keys = cache_rows(cache_k, b, hk, L + 1, block_table, block_size)
            vals = cache_rows(cache_v, b, hk, L + 1, block_table, block_size)
            out[b, hq] = causal_attention(q_rot[hq][None, :], keys, vals,
                                          (np.array([L]), pos), scale)[0]
    return out


def attn_prefill_cached(q, k, v, cache_k, cache_v, seq_lens,
                        theta: float = 10000.0, scale: float | None = None,
                        block_table=None, block_size: int = 16, chunk_lens=None,
                        pairing: str = "adjacent"):
    """A prompt chunk that continues a cached prefix.

    For sequence b with P = seq_lens[b] tokens already cached, the chunk's S
    tokens sit at positions P..P+S-1, which are also their cache indices
    ([Scratch] §3.2).  q [B, Hq, S, D] and k [B, Hkv, S, D] are rotated at
    those positions; the rotated keys and raw values v are written to cache
    indices P..P+S-1; chunk query i then attends over cache rows 0..P+i, the
    cached prefix plus the chunk up to itself ([Scratch] §3.3: a position
    sees itself and earlier ones; the earlier ones come from the cache).

    With ``chunk_lens`` (a batch of chunks of different lengths padded to
    S; [Scratch] §3.3 names the padding mask) sequence b has only its first
    chunk_lens[b] chunk tokens: the padding tokens are neither stored nor
    attended to, and their output rows are zero.

    The caches are updated in place.  Returns out [B, Hq, S, D].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    seq_lens = np.asarray(seq_lens)
    out = np.zeros((B, Hq, S, D))
    for b in range(B):
        P = int(seq_lens[b])
        n = S if chunk_lens is None else int(chunk_lens[b])
        if n == 0:
            continue
        pos = P + np.arange(n)
        q_rot = rope_rotate(q[b, :, :n], pos, theta, pairing)    # [Hq, n, D]
        k_rot = rope_rotate(k[b, :, :n], pos, theta, pairing)    # [Hkv, n, D]
        v_b = v[b:b + 1, :, :n]
        if block_table is None:
            kv_cache_append(cache_k[b:b + 1], cache_v[b:b + 1], k_rot[None], v_b, pos[None, :])
        else:
            kv_cache_append(cache_k, cache_v, k_rot[None], v_b, pos[None, :],
                            block_table=block_table[b:b + 1], block_size=block_size)
        kpos = np.arange(P + n)
        for hq in range(Hq):
            hk = hq // group
            keys = cache_rows(cache_k, b, hk, P + n, block_table, block_size)
            vals = cache_rows(cache_v, b, hk, P + n, block_table, block_size)
            out[b, hq, :n] = causal_attention(q_rot[hq], keys, vals, (pos, kpos), scale)
    return out
