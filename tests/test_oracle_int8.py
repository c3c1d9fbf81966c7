"""Pins for the INT8 KV-cache oracle (``oracle/int8_cache.py``).

Each pin is a check function taking the implementation under test; the same
check runs against the oracle (must pass) and against broken copies built
here (must fail): a scale of absmax/128, truncation or ties-to-even instead
of rounding ties away from zero, an asymmetric [-128, 127] range, one scale
per tensor or per KV head instead of per (KV head, channel), keys quantized
before RoPE, and a decode that swaps or drops the K and V scales.

Pages (titles as published):
[Intuition] "手写LLM推理引擎：重建对Tokenizer、KV Cache与RoPE的底层直觉" §2
[Scratch]   "从零手搓AI推理引擎：告别调包思维，深入底层构建与优化" §2.2, §5.3
[Guide]     "手写LLM推理引擎：从黑盒到白盒的底层实现指南" §2.5
"""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import int8_cache as Q


def rng(seed=0):
    return np.random.default_rng(seed)


# ==========================================================================
# Quantizer pins ([Scratch] §2.2: scale = channel absmax / 127; §5.3: divide
# by the scale and round to INT8, multiply back to dequantize)
# ==========================================================================

class Impl:
    """A scale function (x, axis) -> scales and a quantizer (x, scale) -> codes."""

    def __init__(self, scale, quantize):
        self.scale = scale
        self.quantize = quantize


ORACLE = Impl(Q.int8_scale, Q.int8_quantize)


def check_absmax_maps_to_127(impl):
    """The largest |x| of a channel gets code +-127 and dequantizes back to
    itself up to the float32 rounding of the scale."""
    x = rng(1).standard_normal((1, 3, 50, 8)) * rng(2).uniform(0.1, 10.0, size=(1, 3, 1, 8))
    s = impl.scale(x, axis=(0, 2))                       # [3, 8]
    codes = impl.quantize(x, s[None, :, None, :]).astype(np.int64)
    if codes.min() < -127 or codes.max() > 127:
        return False
    a = np.abs(x[0])                                     # [3, 50, 8]
    j = a.argmax(axis=1)                                 # [3, 8]
    for h in range(3):
        for d in range(8):
            xv = x[0, h, j[h, d], d]
            c = codes[0, h, j[h, d], d]
            if c != 127 * np.sign(xv):
                return False
            if abs(c * float(s[h, d]) - xv) > 1e-7 * abs(xv):
                return False
    return True


def check_grid_round_trip(impl):
    """Every integer k in [-127, 127] times a power-of-two scale quantizes
    to k exactly."""
    k = np.arange(-127, 128, dtype=np.float64)
    for e in (-9, -5, 0, 3):
        s = np.float32(2.0 ** e)
        codes = impl.quantize(k * float(s), s).astype(np.int64)
        if not np.array_equal(codes, k.astype(np.int64)):
            return False
    return True


def check_hand_values(impl):
    """Ties round away from zero, values beyond the range saturate at +-127
    (never -128), a zero scale stores 0."""
    x = np.array([2.5, -2.5, 0.5, -0.5, 0.49999997, 1.5, -1.5, 126.5, 127.49, 127.5,
                  200.0, -200.0, -127.6, 0.0, 3.4999998])
    want = np.array([3, -3, 1, -1, 0, 2, -2, 127, 127, 127, 127, -127, -127, 0, 3])
    if not np.array_equal(impl.quantize(x, np.float32(1.0)).astype(np.int64), want):
        return False
    # the same ties at scale 1/4: 0.625 = 2.5 * 0.25
    if int(impl.quantize(np.array([0.625]), np.float32(0.25))[0]) != 3:
        return False
    return int(impl.quantize(np.array([1.0]), np.float32(0.0))[0]) == 0


def check_round_trip_bound(impl):
    """|code * s - x| <= s / 2 inside the range, up to the float32 rounding of
    x and of x / s (relative 2^-24 each, at most 127 steps); codes saturate
    outside it."""
    x = rng(3).uniform(-2.0, 2.0, size=20000)
    s = np.float32(2.0 / 127.0)
    codes = impl.quantize(x, s).astype(np.float64)
    err = np.abs(codes * float(s) - x)
    if err.max() > float(s) / 2 * (1 + 1e-4):
        return False
    big = np.array([1000.0, -1000.0]) * float(s)
    return np.array_equal(impl.quantize(big, s).astype(np.int64), [127, -127])


def check_per_channel(impl):
    """Scaling channel (h, d) of the input by 4 scales exactly that channel's
    scale by 4 and changes no code: the scales are per (KV head, channel)."""
    x = rng(4).standard_normal((2, 3, 40, 8))
    s = impl.scale(x, axis=(0, 2))
    c = impl.quantize(x, s[None, :, None, :])
    y = x.copy()
    y[:, 1, :, 5] *= 4.0
    t = impl.scale(y, axis=(0, 2))
    want = s.copy()
    want[1, 5] *= 4
    if not np.array_equal(t, want):
        return False
    return np.array_equal(impl.quantize(y, t[None, :, None, :]), c)


QUANT_PINS = [check_absmax_maps_to_127, check_grid_round_trip, check_hand_values,
              check_round_trip_bound, check_per_channel]


@pytest.mark.parametrize("pin", QUANT_PINS, ids=lambda f: f.__name__)
def test_oracle_quantizer_pins(pin):
    assert pin(ORACLE)


def _quantize_generic(x, s, rounding="away", lo=-127, scale_mul=1.0):
    x = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    s = np.broadcast_to(np.asarray(s, dtype=np.float32).astype(np.float64) * scale_mul, x.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (x / s).astype(np.float32).astype(np.float64)
    if rounding == "away":
        r = np.sign(q) * np.floor(np.abs(q) + 0.5)
    elif rounding == "even":
        r = np.round(q)
    else:
        r = np.trunc(q)
    r = np.where(s == 0, 0.0, np.clip(r, lo, 127))
    return r.astype(np.int64)


def _scale_generic(x, axis, denom=127.0, per="channel"):
    a = np.abs(np.asarray(x, dtype=np.float64))
    if per == "tensor":
        m = np.full(np.max(a, axis=axis).shape, a.max())
    elif per == "head":   # one scale per KV head, over every channel
        m = np.broadcast_to(np.max(a, axis=(0, 2, 3))[:, None], np.max(a, axis=axis).shape)
    else:
        m = np.max(a, axis=axis)
    return (m / denom).astype(np.float32)


QUANT_MUTANTS = {
    "divide_by_128": Impl(lambda x, axis: _scale_generic(x, axis, denom=128.0), _quantize_generic),
    "truncate": Impl(_scale_generic, lambda x, s: _quantize_generic(x, s, rounding="trunc")),
    "ties_to_even": Impl(_scale_generic, lambda x, s: _quantize_generic(x, s, rounding="even")),
    "range_minus_128": Impl(_scale_generic, lambda x, s: _quantize_generic(x, s, lo=-128)),
    "per_tensor_scale": Impl(lambda x, axis: _scale_generic(x, axis, per="tensor"),
                             _quantize_generic),
    "per_head_scale": Impl(lambda x, axis: _scale_generic(x, axis, per="head"),
                           _quantize_generic),
    "multiply_not_divide": Impl(_scale_generic,
                                lambda x, s: _quantize_generic(x, 1.0 / np.asarray(s, np.float64)
                                                               if np.all(np.asarray(s) != 0)
                                                               else s)),
}


def test_generic_quantizer_matches_oracle():
    x = rng(5).standard_normal((2, 3, 30, 8)) * 3
    s = _scale_generic(x, (0, 2))
    assert np.array_equal(s, Q.int8_scale(x, (0, 2)))
    assert np.array_equal(_quantize_generic(x, s[None, :, None, :]),
                          Q.int8_quantize(x, s[None, :, None, :]).astype(np.int64))


@pytest.mark.parametrize("name", sorted(QUANT_MUTANTS))
def test_quantizer_pins_catch_planted_mistakes(name):
    assert not all(pin(QUANT_MUTANTS[name]) for pin in QUANT_PINS)


# ==========================================================================
# Calibration: absmax of the keys as the cache holds them, after RoPE
# ([Scratch] §3.2 stores rotated keys; [Intuition] §4 rotation)
# ==========================================================================

def check_calibration_rotates_keys(calibrate):
    """D = 2, k = (1, 0) at positions 0, 1, 2 rotates to (cos m, sin m):
    channel 1's absmax is sin 2, channel 0's is cos 0 = 1 (hand values);
    values are not rotated."""
    k = np.zeros((1, 1, 3, 2))
    k[..., 0] = 1.0
    v = np.array([[[[0.5, -3.0], [2.0, 1.0], [-1.0, 0.25]]]])
    ks, vs = calibrate(k, v, np.array([[0, 1, 2]]))
    want_k = np.array([[1.0 / 127, math.sin(2.0) / 127]], dtype=np.float32)
    want_v = np.array([[2.0 / 127, 3.0 / 127]], dtype=np.float32)
    return (np.allclose(ks, want_k, rtol=1e-6, atol=0) and np.array_equal(vs, want_v)
            and ks.dtype == np.float32 and vs.dtype == np.float32)


def check_calibration_over_batch_and_tokens(calibrate):
    """At position 0 nothing rotates: the scales are the absmax over every
    sequence and token of each (KV head, channel), over 127."""
    r = rng(6)
    k = r.standard_normal((3, 2, 5, 4)).astype(np.float32)   # inputs are float32 or bf16
    v = r.standard_normal((3, 2, 5, 4)).astype(np.float32)
    ks, vs = calibrate(k, v, np.zeros((3, 5), dtype=np.int64))
    want_k = np.array([[max(abs(float(k[b, h, s, d])) for b in range(3) for s in range(5)) / 127
                        for d in range(4)] for h in range(2)], dtype=np.float32)
    want_v = np.array([[max(abs(float(v[b, h, s, d])) for b in range(3) for s in range(5)) / 127
                        for d in range(4)] for h in range(2)], dtype=np.float32)
    return np.array_equal(ks, want_k) and np.array_equal(vs, want_v)


CAL_PINS = [check_calibration_rotates_keys, check_calibration_over_batch_and_tokens]


@pytest.mark.parametrize("pin", CAL_PINS, ids=lambda f: f.__name__)
def test_oracle_calibration_pins(pin):
    assert pin(Q.int8_calibrate)


def _calibrate_unrotated(k, v, positions):
    return Q.int8_scale(k, (0, 2)), Q.int8_scale(v, (0, 2))


def _calibrate_per_sequence_last(k, v, positions):
    ks, vs = Q.int8_calibrate(k[-1:], v[-1:], positions[-1:])
    return ks, vs


@pytest.mark.parametrize("bad", [_calibrate_unrotated, _calibrate_per_sequence_last])
def test_calibration_pins_catch_planted_mistakes(bad):
    assert not all(pin(bad) for pin in CAL_PINS)


# ==========================================================================
# Decode over an INT8 cache ([Guide] §2.5: append, then attend over 0..L)
# ==========================================================================

def _grid_case(B, Hq, Hkv, D, lens, seed, paged=False):
    """Random codes in every cached slot, distinct per-channel K and V
    scales, a zero new key and a new value on the V grid."""
    r = rng(seed)
    n = int(max(lens)) + 1
    ks = (r.uniform(0.01, 0.05, size=(Hkv, D))).astype(np.float32)
    vs = (r.uniform(0.02, 0.08, size=(Hkv, D))).astype(np.float32)
    q = r.standard_normal((B, Hq, D))
    kn = np.zeros((B, Hkv, D))
    vn = r.integers(-127, 128, size=(B, Hkv, D)) * vs.astype(np.float64)[None]
    if paged:
        mbps = (n + 15) // 16
        nb = B * mbps + 2
        table = r.permutation(nb)[: B * mbps].reshape(B, mbps)
        shape = (nb, Hkv, 16, D)
    else:
        table = None
        shape = (B, Hkv, n, D)
    ck = r.integers(-127, 128, size=shape).astype(np.int8)
    cv = r.integers(-127, 128, size=shape).astype(np.int8)
    return q, kn, vn, ck, cv, ks, vs, table


def _dequantized(cache, scale, paged):
    s = scale.astype(np.float64)
    return cache.astype(np.float64) * s[None, :, None, :]


def check_decode_on_grid_equals_float_decode(decode, paged=False):
    """With every cached value and the new token on the code grid the INT8
    decode is the float decode over the dequantized cache."""
    lens = np.array([0, 5, 17, 33])
    q, kn, vn, ck, cv, ks, vs, table = _grid_case(4, 4, 2, 8, lens, seed=7, paged=paged)
    fk, fv = _dequantized(ck, ks, paged), _dequantized(cv, vs, paged)
    got = decode(q, kn, vn, ck.copy(), cv.copy(), lens, ks, vs, block_table=table)
    want = A.attn_decode(q, kn, vn, fk, fv, lens, block_table=table)
    return np.allclose(got, want, atol=1e-12, rtol=0)


def check_decode_v_error_bound(decode):
    """Keys on the grid, values off it: each output moves by at most the
    largest V scale of its KV head over 2 (weights sum to 1)."""
    r = rng(8)
    B, Hq, Hkv, D, n = 2, 4, 2, 8, 24
    lens = np.array([11, 23])
    ks = r.uniform(0.01, 0.05, size=(Hkv, D)).astype(np.float32)
    k = r.integers(-127, 128, size=(B, Hkv, n, D)) * ks.astype(np.float64)[None, :, None, :]
    v = r.standard_normal((B, Hkv, n, D))
    vs = Q.int8_scale(v, (0, 2))
    q = r.standard_normal((B, Hq, D))
    kn = np.zeros((B, Hkv, D))
    vn = 0.5 * v[:, :, 0, :]   # inside the calibrated range
    ck = np.zeros((B, Hkv, n, D), np.int8)
    cv = np.zeros((B, Hkv, n, D), np.int8)
    pos = np.tile(np.arange(n), (B, 1))
    Q.kv_cache_append_int8(ck, cv, k, v, pos, ks, vs)
    got = decode(q, kn, vn, ck, cv, lens, ks, vs)
    fk, fv = k.copy(), v.copy()
    want = A.attn_decode(q, kn, vn, fk, fv, lens)
    bound = np.repeat(vs.max(axis=1), Hq // Hkv)[None, :, None] / 2 * (1 + 1e-4)
    return bool(np.all(np.abs(got - want) <= bound))


def test_int8_decode_on_grid_equals_float_decode():
    assert check_decode_on_grid_equals_float_decode(Q.attn_decode_int8)


def test_int8_paged_decode_on_grid_equals_float_decode():
    assert check_decode_on_grid_equals_float_decode(Q.attn_decode_int8, paged=True)


def test_int8_decode_v_error_bound():
    assert check_decode_v_error_bound(Q.attn_decode_int8)


def test_int8_decode_appends_codes_at_position_len():
    """The new token's codes land at index L and nowhere else."""
    r = rng(9)
    B, Hq, Hkv, D, n = 2, 2, 1, 8, 10
    lens = np.array([3, 7])
    q = r.standard_normal((B, Hq, D))
    kn = r.standard_normal((B, Hkv, D))
    vn = r.standard_normal((B, Hkv, D))
    ks = np.full((Hkv, D), 0.02, np.float32)
    vs = np.full((Hkv, D), 0.03, np.float32)
    ck = np.full((B, Hkv, n, D), 99, np.int8)
    cv = np.full((B, Hkv, n, D), 99, np.int8)
    Q.attn_decode_int8(q, kn, vn, ck, cv, lens, ks, vs)
    for b in range(B):
        L = int(lens[b])
        kr = A.rope_rotate(kn[b][:, None, :], np.array([L]))[:, 0, :]
        assert np.array_equal(ck[b, :, L], Q.int8_quantize(kr, ks))
        assert np.array_equal(cv[b, :, L], Q.int8_quantize(vn[b], vs))
        others = [t for t in range(n) if t != L]
        assert np.all(ck[b, :, others] == 99) and np.all(cv[b, :, others] == 99)


def _decode_swapped_scales(q, kn, vn, ck, cv, lens, ks, vs, block_table=None):
    return Q.attn_decode_int8(q, kn, vn, ck, cv, lens, vs, ks, block_table=block_table)


def _decode_without_k_scale(q, kn, vn, ck, cv, lens, ks, vs, block_table=None):
    return Q.attn_decode_int8(q, kn, vn, ck, cv, lens, np.ones_like(ks), vs,
                              block_table=block_table)


def _decode_transposed_scales(q, kn, vn, ck, cv, lens, ks, vs, block_table=None):
    # per-channel scales read with head and channel exchanged
    Hkv, D = ks.shape
    kt = np.resize(ks.T.reshape(-1), (Hkv, D)).astype(np.float32)
    vt = np.resize(vs.T.reshape(-1), (Hkv, D)).astype(np.float32)
    return Q.attn_decode_int8(q, kn, vn, ck, cv, lens, kt, vt, block_table=block_table)


@pytest.mark.parametrize("bad", [_decode_swapped_scales, _decode_without_k_scale,
                                 _decode_transposed_scales])
def test_int8_decode_pins_catch_planted_mistakes(bad):
    assert not (check_decode_on_grid_equals_float_decode(bad)
                and check_decode_v_error_bound(bad))


# ==========================================================================
# A chunk over an INT8 cache ([Scratch] §3.2-§3.3, every key read from the cache)
# ==========================================================================

def _chunk_grid_case(B, Hq, Hkv, D, S, lens, seed, paged):
    """Random codes in every slot, distinct per-channel scales, zero chunk
    keys (rotation keeps them zero, so their codes are exact) and chunk
    values on the V grid."""
    r = rng(seed)
    n = int(max(lens)) + S
    ks = r.uniform(0.01, 0.05, size=(Hkv, D)).astype(np.float32)
    vs = r.uniform(0.02, 0.08, size=(Hkv, D)).astype(np.float32)
    q = r.standard_normal((B, Hq, S, D))
    k = np.zeros((B, Hkv, S, D))
    v = r.integers(-127, 128, size=(B, Hkv, S, D)) * vs.astype(np.float64)[None, :, None, :]
    if paged:
        mbps = (n + 15) // 16
        nb = B * mbps + 2
        table = r.permutation(nb)[: B * mbps].reshape(B, mbps)
        shape = (nb, Hkv, 16, D)
    else:
        table = None
        shape = (B, Hkv, n, D)
    ck = r.integers(-127, 128, size=shape).astype(np.int8)
    cv = r.integers(-127, 128, size=shape).astype(np.int8)
    return q, k, v, ck, cv, ks, vs, table


def check_chunk_on_grid_equals_float_chunk(chunk, paged=False):
    """Prefix, chunk keys and chunk values on the code grid: the INT8 chunk
    is the float chunk over the dequantized cache (padding included)."""
    lens = np.array([0, 5, 17, 33])
    n = np.array([6, 1, 6, 3])
    q, k, v, ck, cv, ks, vs, table = _chunk_grid_case(4, 4, 2, 8, 6, lens, 11, paged)
    fk, fv = _dequantized(ck, ks, paged), _dequantized(cv, vs, paged)
    got = chunk(q, k, v, ck.copy(), cv.copy(), lens, ks, vs, block_table=table, chunk_lens=n)
    want = A.attn_prefill_cached(q, k, v, fk, fv, lens, block_table=table, chunk_lens=n)
    return np.allclose(got, want, atol=1e-12, rtol=0)


def check_one_token_chunk_is_a_decode_step(chunk):
    r = rng(12)
    B, Hq, Hkv, D, n = 2, 4, 2, 8, 20
    lens = np.array([4, 13])
    ks = r.uniform(0.01, 0.05, size=(Hkv, D)).astype(np.float32)
    vs = r.uniform(0.02, 0.08, size=(Hkv, D)).astype(np.float32)
    q = r.standard_normal((B, Hq, D))
    kn, vn = r.standard_normal((B, Hkv, D)), r.standard_normal((B, Hkv, D))
    ck = r.integers(-127, 128, size=(B, Hkv, n, D)).astype(np.int8)
    cv = r.integers(-127, 128, size=(B, Hkv, n, D)).astype(np.int8)
    ck2, cv2 = ck.copy(), cv.copy()
    got = chunk(q[:, :, None], kn[:, :, None], vn[:, :, None], ck, cv, lens, ks, vs)[:, :, 0]
    want = Q.attn_decode_int8(q, kn, vn, ck2, cv2, lens, ks, vs)
    return (np.allclose(got, want, atol=1e-13, rtol=0) and np.array_equal(ck, ck2)
            and np.array_equal(cv, cv2))


def check_chunk_equals_two_chunks(chunk):
    """Off-grid keys and values: a chunk of 9 tokens equals its first 4
    then its last 5 as two chunks (outputs and stored codes)."""
    r = rng(13)
    B, Hq, Hkv, D, S, n = 2, 4, 2, 8, 9, 24
    lens = np.array([0, 7])
    ks = r.uniform(0.02, 0.05, size=(Hkv, D)).astype(np.float32)
    vs = r.uniform(0.02, 0.05, size=(Hkv, D)).astype(np.float32)
    q = r.standard_normal((B, Hq, S, D))
    k, v = r.standard_normal((B, Hkv, S, D)), r.standard_normal((B, Hkv, S, D))
    ck = r.integers(-127, 128, size=(B, Hkv, n, D)).astype(np.int8)
    cv = r.integers(-127, 128, size=(B, Hkv, n, D)).astype(np.int8)
    ck2, cv2 = ck.copy(), cv.copy()
    whole = chunk(q, k, v, ck, cv, lens, ks, vs)
    first = chunk(q[:, :, :4], k[:, :, :4], v[:, :, :4], ck2, cv2, lens, ks, vs)
    second = chunk(q[:, :, 4:], k[:, :, 4:], v[:, :, 4:], ck2, cv2, lens + 4, ks, vs)
    both = np.concatenate([first, second], axis=2)
    return (np.allclose(whole, both, atol=1e-13, rtol=0) and np.array_equal(ck, ck2)
            and np.array_equal(cv, cv2))


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_int8_chunk_on_grid_equals_float_chunk(paged):
    assert check_chunk_on_grid_equals_float_chunk(Q.attn_prefill_cached_int8, paged)


def test_int8_one_token_chunk_is_a_decode_step():
    assert check_one_token_chunk_is_a_decode_step(Q.attn_prefill_cached_int8)


def test_int8_chunk_equals_two_chunks():
    assert check_chunk_equals_two_chunks(Q.attn_prefill_cached_int8)


def test_int8_chunk_stores_codes_and_zero_padding_rows():
    """Chunk tokens' codes land at P..P+n-1 and nowhere else; padding rows
    are zero."""
    r = rng(14)
    B, Hq, Hkv, D, S, cap = 2, 2, 1, 8, 5, 16
    lens, n = np.array([3, 9]), np.array([5, 2])
    q = r.standard_normal((B, Hq, S, D))
    k, v = r.standard_normal((B, Hkv, S, D)), r.standard_normal((B, Hkv, S, D))
    ks = np.full((Hkv, D), 0.02, np.float32)
    vs = np.full((Hkv, D), 0.03, np.float32)
    ck = np.full((B, Hkv, cap, D), 99, np.int8)
    cv = np.full((B, Hkv, cap, D), 99, np.int8)
    out = Q.attn_prefill_cached_int8(q, k, v, ck, cv, lens, ks, vs, chunk_lens=n)
    for b in range(B):
        P, m = int(lens[b]), int(n[b])
        pos = P + np.arange(m)
        kr = A.rope_rotate(k[b, :, :m], pos)
        assert np.array_equal(ck[b, :, P:P + m], Q.int8_quantize(kr, ks[:, None, :]))
        assert np.array_equal(cv[b, :, P:P + m], Q.int8_quantize(v[b, :, :m], vs[:, None, :]))
        others = [t for t in range(cap) if not P <= t < P + m]
        assert np.all(ck[b, :, others] == 99) and np.all(cv[b, :, others] == 99)
        assert not np.any(out[b, :, m:])


def _chunk_own_tokens_full_precision(q, k, v, ck, cv, lens, ks, vs, block_table=None,
                                     chunk_lens=None):
    """Planted mistake: the chunk attends to its own tokens at full precision
    (only the prefix read from the cache), then stores their codes."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, Hq, S, D))
    for b in range(B):
        P = int(lens[b])
        m = S if chunk_lens is None else int(chunk_lens[b])
        if m == 0:
            continue
        pos = P + np.arange(m)
        qr, kr = A.rope_rotate(q[b, :, :m], pos), A.rope_rotate(k[b, :, :m], pos)
        for hq in range(Hq):
            hk = hq // (Hq // Hkv)
            if block_table is None:
                pk = Q.int8_dequantize(ck[b, hk, :P], ks[hk][None])
                pv = Q.int8_dequantize(cv[b, hk, :P], vs[hk][None])
            else:
                t = np.arange(P)
                blk = block_table[b, t // 16]
                pk = Q.int8_dequantize(ck[blk, hk, t % 16], ks[hk][None])
                pv = Q.int8_dequantize(cv[blk, hk, t % 16], vs[hk][None])
            keys = np.concatenate([pk, kr[hk]])
            vals = np.concatenate([pv, v[b, hk, :m]])
            out[b, hq, :m] = A.causal_attention(qr[hq], keys, vals, (pos, np.arange(P + m)),
                                                1 / np.sqrt(D))
        if block_table is None:
            Q.kv_cache_append_int8(ck[b:b + 1], cv[b:b + 1], kr[None], v[b:b + 1, :, :m],
                                   pos[None], ks, vs)
        else:
            Q.kv_cache_append_int8(ck, cv, kr[None], v[b:b + 1, :, :m], pos[None], ks, vs,
                                   block_table=block_table[b:b + 1])
    return out


def _chunk_swapped_scales(q, k, v, ck, cv, lens, ks, vs, block_table=None, chunk_lens=None):
    return Q.attn_prefill_cached_int8(q, k, v, ck, cv, lens, vs, ks, block_table=block_table,
                                      chunk_lens=chunk_lens)


@pytest.mark.parametrize("bad", [_chunk_own_tokens_full_precision, _chunk_swapped_scales])
def test_int8_chunk_pins_catch_planted_mistakes(bad):
    assert not (check_chunk_on_grid_equals_float_chunk(bad)
                and check_one_token_chunk_is_a_decode_step(bad)
                and check_chunk_equals_two_chunks(bad))
