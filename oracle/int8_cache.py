"""Plain definitions of an INT8 KV cache with per-(KV head, channel) scales.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path
never imports this module.

What the pages fix:

* [Intuition] §2 (the four pillars) lists precision compression of the KV
  cache from FP16 to INT8 among the things a cache has to support.
* [Scratch] §2.2 (weight loading): the usual INT8 scheme takes the absolute
  maximum of each channel and divides it by 127 to get that channel's scale;
  the scales are computed once, ahead of inference, and kept beside the
  quantized data (recomputing them on every forward pass doubles latency).
* [Scratch] §5.3 (quantization): a value is divided by its channel's scale
  and rounded to INT8; it is multiplied back by the scale before it is used
  in higher precision.

Readings where the pages leave a step open (each one is a pin below):

* "Channel" of a cached K or V row is its head dimension d, and the scales
  are per (KV head, channel): k_scale[hk, d], v_scale[hk, d].  They are
  calibrated once (``int8_calibrate``) and then fixed, as for weights.
* Keys are quantized after RoPE: the cache stores rotated keys ([Scratch]
  §3.2), so the absolute maxima are taken over rotated keys.
* Rounding is half away from zero (the pages' word for rounding is the
  school rule, ties up in magnitude); codes are clamped to [-127, 127], a
  symmetric range, so -128 never occurs.  A channel whose scale is 0 stores
  code 0.
* The rounding decision is taken in float32, as the kernels take it: the
  value to store is rounded to float32, divided by the float32 scale with
  one float32 rounding, and the quotient is rounded to an integer.  A scale
  is absmax / 127 rounded to float32.  (Float64 division of two float32
  values rounded once to float32 equals float32 division: 53 >= 2*24 + 2.)
* Attention reads the dequantized cache, code * scale, in float64; the new
  token of a decode step is quantized when it is appended and attended to in
  its quantized form, like every other cached token.  A chunk continuing a
  cached prefix does the same for all of its tokens: they are stored first
  and every key and value the chunk attends to is read back from the cache
  (so a one-token chunk is a decode step, and a chunk equals the same tokens
  taken as two chunks).  A whole-prompt prefill's own attention uses its
  full-precision keys and values; only what it stores is quantized.

Pins (``tests/test_oracle_int8.py``, none reuses this code): a channel's
absolute maximum maps to +-127 and dequantizes back to itself within float32
rounding; values on the code grid of a power-of-two scale round-trip
exactly; hand values for ties, saturation and the symmetric range; the
round-trip error bound scale/2; scaling one channel of the input scales only
that channel's scale and leaves all codes unchanged; a decode over an INT8
cache whose values lie on the grid equals the float decode of ``attention``
over the dequantized cache, with different K and V scales per channel; the
bound |O_int8 - O_float| <= max scale_v / 2 when only V is off the grid.
A chunk over an INT8 cache: with the prefix on the grid, zero chunk keys and
chunk values on the V grid it equals the float chunk over the dequantized
cache (contiguous and paged, with padding); a one-token chunk equals a
decode step; a chunk equals the same tokens taken as two chunks (outputs
and codes); padding rows are zero and padding tokens are not stored.
"""

from __future__ import annotations

import numpy as np

from .attention import causal_attention, paged_slot, rope_rotate

__all__ = [
    "int8_scale",
    "int8_quantize",
    "int8_dequantize",
    "int8_calibrate",
    "kv_cache_append_int8",
    "attn_decode_int8",
    "attn_prefill_cached_int8",
]


def int8_scale(x, axis) -> np.ndarray:
    """absmax / 127 over ``axis``, rounded to float32 ([Scratch] §2.2)."""
    a = np.max(np.abs(np.asarray(x, dtype=np.float64)), axis=axis)
    return (a / 127.0).astype(np.float32)


def _round_half_away(q: np.ndarray) -> np.ndarray:
    return np.sign(q) * np.floor(np.abs(q) + 0.5)


def int8_quantize(x, scale) -> np.ndarray:
    """Code of each value: round(x / scale) clamped to [-127, 127] ([Scratch] §5.3).

    ``scale`` broadcasts against ``x``.  x is first rounded to float32 and
    the quotient is rounded once to float32; a zero scale gives code 0.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    s32 = np.broadcast_to(np.asarray(scale, dtype=np.float32).astype(np.float64), x32.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (x32 / s32).astype(np.float32).astype(np.float64)
    code = np.clip(_round_half_away(q), -127, 127)
    code = np.where(s32 == 0.0, 0.0, code)
    return code.astype(np.int8)


def int8_dequantize(code, scale) -> np.ndarray:
    """code * scale in float64 ([Scratch] §5.3: back to high precision)."""
    return np.asarray(code, dtype=np.float64) * np.asarray(scale, dtype=np.float32).astype(np.float64)


def int8_calibrate(k, v, positions, theta: float = 10000.0, pairing: str = "adjacent"):
    """Per-(KV head, channel) scales of a calibration batch ([Scratch] §2.2).

    k, v: [B, Hkv, S, D]; positions [B, S].  Keys are rotated at their
    positions first (the cache holds rotated keys) and rounded to float32,
    the form in which they are quantized.  Returns (k_scale, v_scale), each
    float32 [Hkv, D]: absmax over all (b, s) divided by 127.
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    positions = np.asarray(positions)
    k_rot = np.stack([rope_rotate(k[b], positions[b], theta, pairing) for b in range(k.shape[0])])
    k_rot = k_rot.astype(np.float32)
    return int8_scale(k_rot, axis=(0, 2)), int8_scale(v, axis=(0, 2))


def kv_cache_append_int8(cache_k, cache_v, k_rot, v, positions, k_scale, v_scale,
                         block_table=None, block_size: int = 16):
    """Store the codes of rotated keys and raw values at cache index == position.

    As ``attention.kv_cache_append`` ([Scratch] §3.2), with each row
    quantized by its KV head's channel scales first.  cache_k / cache_v are
    int8 arrays, modified in place; k_scale, v_scale are [Hkv, D].
    """
    positions = np.asarray(positions)
    kc = int8_quantize(k_rot, np.asarray(k_scale)[None, :, None, :])
    vc = int8_quantize(v, np.asarray(v_scale)[None, :, None, :])
    B, _, S, _ = np.shape(k_rot)
    for b in range(B):
        for s in range(S):
            t = int(positions[b, s])
            if block_table is None:
                cache_k[b, :, t, :] = kc[b, :, s, :]
                cache_v[b, :, t, :] = vc[b, :, s, :]
            else:
                blk, off = paged_slot(block_table, b, t, block_size)
                cache_k[blk, :, off, :] = kc[b, :, s, :]
                cache_v[blk, :, off, :] = vc[b, :, s, :]


def _rows_int8(cache, scale_row, b: int, hk: int, n: int, block_table, block_size):
    """Dequantized rows 0..n-1 of sequence b, KV head hk, as [n, D] float64."""
    if block_table is None:
        codes = cache[b, hk, :n, :]
    else:
        t = np.arange(n)
        codes = cache[np.asarray(block_table)[b, t // block_size], hk, t % block_size, :]
    return int8_dequantize(codes, scale_row[None, :])


def attn_decode_int8(q, k_new, v_new, cache_k, cache_v, seq_lens, k_scale, v_scale,
                     theta: float = 10000.0, scale: float | None = None,
                     block_table=None, block_size: int = 16, pairing: str = "adjacent"):
    """One decode step over an INT8 cache.

    As ``attention.attn_decode`` ([Guide] §2.5; [Scratch] §3.2-§3.3): q and
    k_new are rotated at position L = seq_lens[b]; the rotated key and raw
    value are quantized and appended at index L; the query attends over the
    dequantized rows 0..L.  The int8 caches are updated in place.  Returns
    out [B, Hq, D] in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    k_scale = np.asarray(k_scale, dtype=np.float32)
    v_scale = np.asarray(v_scale, dtype=np.float32)
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
        v_one = v_new[b][:, None, :]
        if block_table is None:
            kv_cache_append_int8(cache_k[b:b + 1], cache_v[b:b + 1], k_rot[None], v_one[None],
                                 np.array([[L]]), k_scale, v_scale)
        else:
            kv_cache_append_int8(cache_k, cache_v, k_rot[None], v_one[None], np.array([[L]]),
                                 k_scale, v_scale, block_table=block_table[b:b + 1],
                                 block_size=block_size)
        pos = np.arange(L + 1)
        for hq in range(Hq):
            hk = hq // group
            keys = _rows_int8(cache_k, k_scale[hk], b, hk, L + 1, block_table, block_size)
            vals = _rows_int8(cache_v, v_scale[hk], b, hk, L + 1, block_table, block_size)
            out[b, hq] = causal_attention(q_rot[hq][None, :], keys, vals,
                                          (np.array([L]), pos), scale)[0]
    return out


def attn_prefill_cached_int8(q, k, v, cache_k, cache_v, seq_lens, k_scale, v_scale,
                             theta: float = 10000.0, scale: float | None = None,
                             block_table=None, block_size: int = 16, chunk_lens=None,
                             pairing: str = "adjacent"):
    """A prompt chunk continuing a cached prefix, over an INT8 cache.

    As ``attention.attn_prefill_cached`` ([Scratch] §3.2-§3.3): with P =
    seq_lens[b] tokens cached, chunk token s sits at position and cache
    index P + s; q and k are rotated there; the rotated keys and raw values
    are quantized and stored at P..P+n-1 (n = chunk_lens[b], or S); chunk
    query i then attends over the dequantized rows 0..P+i, its own chunk's
    tokens included in their quantized form.  Padding rows of the output are
    zero and padding tokens are not stored.  The int8 caches are updated in
    place.  Returns out [B, Hq, S, D] in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    k_scale = np.asarray(k_scale, dtype=np.float32)
    v_scale = np.asarray(v_scale, dtype=np.float32)
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
            kv_cache_append_int8(cache_k[b:b + 1], cache_v[b:b + 1], k_rot[None], v_b,
                                 pos[None, :], k_scale, v_scale)
        else:
            kv_cache_append_int8(cache_k, cache_v, k_rot[None], v_b, pos[None, :], k_scale,
                                 v_scale, block_table=block_table[b:b + 1],
                                 block_size=block_size)
        kpos = np.arange(P + n)
        for hq in range(Hq):
            hk = hq // group
            keys = _rows_int8(cache_k, k_scale[hk], b, hk, P + n, block_table, block_size)
            vals = _rows_int8(cache_v, v_scale[hk], b, hk, P + n, block_table, block_size)
            out[b, hq, :n] = causal_attention(q_rot[hq], keys, vals, (pos, kpos), scale)
    return out
