"""Pins for the fp64 oracle: facts the pages and the mathematics fix.

Each pin is a check function taking the implementation under test, so the
same check is run against the oracle (must pass) and against deliberately
broken copies of it built here on the CPU (must fail), which shows that a
plausible mistake -- a flipped sign, a wrong pair layout or frequency, a
missing scale, a mask off by one, a transposed operand, a decode that skips
the new token, a swapped block/offset -- cannot pass the pins.

Pages (titles as published):
[Guide]     "手写LLM推理引擎：从黑盒到白盒的底层实现指南"
[Intuition] "手写LLM推理引擎：重建对Tokenizer、KV Cache与RoPE的底层直觉"
[Scratch]   "从零手搓AI推理引擎：告别调包思维，深入底层构建与优化"
[NanoVLLM]  "以 Nano-vLLM 为例，深入理解 LLM 推理引擎（Part 2）"
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


def load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val, tol = line.split()
            vals[key] = (float(val), float(tol))
    return vals


# ==========================================================================
# RoPE pins ([Intuition] §4)
# ==========================================================================

def check_rope_identity_at_zero(rope):
    """P1: position 0 rotates by angle 0 for every pair: the identity."""
    x = rng(1).standard_normal((3, 5, 64))
    return np.array_equal(rope(x, np.zeros(5), 10000.0), x)


def check_rope_norm(rope):
    """P2: a rotation keeps every pair's length, hence the vector norm."""
    x = rng(2).standard_normal((4, 7, 128))
    pos = np.array([0, 1, 5, 100, 1000, 4095, 8192])
    y = rope(x, pos, 10000.0)
    return np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1),
                       rtol=1e-12, atol=0)


def check_rope_relative(rope):
    """P3: (R(m)q).(R(n)k) depends on n - m only ([Intuition] §4: the angle
    grows linearly with position).  Shift both positions by several deltas."""
    r = rng(3)
    q = r.standard_normal((1, 64))
    k = r.standard_normal((1, 64))
    ok = True
    for m, n in [(0, 3), (5, 2), (17, 17), (100, 40)]:
        base = (rope(q, np.array([m]), 1e4) @ rope(k, np.array([n]), 1e4).T).item()
        for d in (1, 7, 1000, 3000):
            s = (rope(q, np.array([m + d]), 1e4) @ rope(k, np.array([n + d]), 1e4).T).item()
            ok &= abs(s - base) <= 1e-10 * max(1.0, abs(base))
    return ok


def check_rope_hand_values(rope):
    """P4: hand values.  D = 2: theta_0 = 1, so x = (1, 0) at m = 1 becomes
    (cos 1, sin 1).  D = 4: theta_1 = 10000^(-2/4) = 0.01, so the second
    adjacent pair (x2, x3) = (1, 0) at m = 1 becomes (cos 0.01, sin 0.01) and
    the first pair (0, 0) stays 0 -- this separates adjacent pairs from a
    half-split layout and pins the exponent -2i/D."""
    y2 = rope(np.array([[1.0, 0.0]]), np.array([1]), 10000.0)[0]
    want2 = np.array([0.5403023058681398, 0.8414709848078965])  # cos 1, sin 1
    y4 = rope(np.array([[0.0, 0.0, 1.0, 0.0]]), np.array([1]), 10000.0)[0]
    want4 = np.array([0.0, 0.0, math.cos(0.01), math.sin(0.01)])
    y4b = rope(np.array([[0.0, 1.0, 0.0, 0.0]]), np.array([3]), 10000.0)[0]
    want4b = np.array([-math.sin(3.0), math.cos(3.0), 0.0, 0.0])
    return (np.allclose(y2, want2, atol=1e-15) and np.allclose(y4, want4, atol=1e-15)
            and np.allclose(y4b, want4b, atol=1e-15))


RoPE_PINS = [check_rope_identity_at_zero, check_rope_norm, check_rope_relative,
             check_rope_hand_values]


@pytest.mark.parametrize("pin", RoPE_PINS, ids=lambda f: f.__name__)
def test_oracle_rope_pins(pin):
    assert pin(A.rope_rotate)


def test_rope_inv_freq_values():
    f = A.rope_inv_freq(128, 10000.0)
    assert f[0] == 1.0
    assert math.isclose(f[1], 10000.0 ** (-2 / 128), rel_tol=1e-15)
    assert math.isclose(f[-1], 10000.0 ** (-126 / 128), rel_tol=1e-15)
    assert np.all(np.diff(f) < 0)


# ---- half-split pairing (the Llama/Qwen checkpoint layout) ----
def _rope_half(x, p, t):
    return A.rope_rotate(x, p, t, pairing="half")


@pytest.mark.parametrize("pin", [check_rope_identity_at_zero, check_rope_norm,
                                 check_rope_relative], ids=lambda f: f.__name__)
def test_half_split_rope_pins(pin):
    assert pin(_rope_half)


def test_half_split_rope_hand_value():
    """D = 4, half split: pair 1 is (x1, x3) at theta_1 = 0.01, so x = (0, 1,
    0, 0) at m = 1 becomes (0, cos 0.01, 0, sin 0.01); pair 0 = (x0, x2)."""
    y = _rope_half(np.array([[0.0, 1.0, 0.0, 0.0]]), np.array([1]), 10000.0)[0]
    assert np.allclose(y, [0.0, math.cos(0.01), 0.0, math.sin(0.01)], atol=1e-15)
    y = _rope_half(np.array([[1.0, 0.0, 0.0, 0.0]]), np.array([2]), 10000.0)[0]
    assert np.allclose(y, [math.cos(2.0), 0.0, math.sin(2.0), 0.0], atol=1e-15)


def test_half_split_equals_permuted_adjacent():
    """half(x) = P^-1 adjacent(P x), P taking element i to 2i and i + D/2 to
    2i + 1: the same rotations on a permutation of the elements."""
    x = rng(5).standard_normal((3, 7, 128))
    p = np.array([0, 1, 9, 100, 1000, 4095, 8192])
    D = 128
    perm = np.empty(D, int)
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2      # adjacent slot j holds half element perm[j]
    adj = A.rope_rotate(x[..., perm], p, 1e4)
    back = np.empty_like(adj)
    back[..., perm] = adj
    assert np.allclose(_rope_half(x, p, 1e4), back, atol=1e-12)
    assert not np.allclose(_rope_half(x, p, 1e4), A.rope_rotate(x, p, 1e4), atol=1e-3)


# planted mistakes in RoPE, each must trip at least one pin
def _rope_generic(x, positions, theta, sign=1.0, halfsplit=False, expo=2.0):
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    ang = np.asarray(positions, np.float64)[..., None] * theta ** (-expo * np.arange(D // 2) / D)
    c, s = np.cos(ang), sign * np.sin(ang)
    y = x.copy()
    if halfsplit:
        a, b = x[..., : D // 2], x[..., D // 2:]
        y[..., : D // 2] = a * c - b * s
        y[..., D // 2:] = a * s + b * c
    else:
        a, b = x[..., 0::2], x[..., 1::2]
        y[..., 0::2] = a * c - b * s
        y[..., 1::2] = a * s + b * c
    return y


ROPE_MUTANTS = {
    "flipped_sign": lambda x, p, t: _rope_generic(x, p, t, sign=-1.0),
    "half_split_pairs": lambda x, p, t: _rope_generic(x, p, t, halfsplit=True),
    "exponent_i_over_d": lambda x, p, t: _rope_generic(x, p, t, expo=1.0),
    "position_off_by_one": lambda x, p, t: _rope_generic(x, np.asarray(p) + 1, t),
}


def test_generic_rope_matches_oracle():
    x = rng(4).standard_normal((2, 6, 64))
    p = np.array([0, 1, 2, 50, 500, 5000])
    assert np.allclose(_rope_generic(x, p, 1e4), A.rope_rotate(x, p, 1e4), atol=1e-12)


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_rope_pins_catch_planted_mistakes(name):
    assert not all(pin(ROPE_MUTANTS[name]) for pin in RoPE_PINS)


# ==========================================================================
# Attention pins ([Guide] §2.3, §4.2, §5.1; [Scratch] §3.1, §3.3, §3.4)
# ==========================================================================

def _prefill_one_head(attn, q, k, v, pos, scale):
    return attn(q, k, v, (pos, pos), scale)


def check_rows_are_distributions(attn):
    """P5: with V = I the output rows are the softmax rows: non-negative,
    summing to 1, and zero on keys later than the query (causal mask)."""
    S = 9
    r = rng(5)
    q, k = r.standard_normal((S, 4)), r.standard_normal((S, 4))
    P = _prefill_one_head(attn, q, k, np.eye(S), np.arange(S), 0.5)
    return (np.all(P >= 0) and np.allclose(P.sum(1), 1.0, atol=1e-14)
            and np.all(np.triu(P, 1) == 0.0))


def check_single_token(attn):
    """P6: one token sees only itself: O = V_0."""
    r = rng(6)
    q, k, v = r.standard_normal((1, 8)), r.standard_normal((1, 8)), r.standard_normal((1, 8))
    return np.allclose(_prefill_one_head(attn, q, k, v, np.arange(1), 0.3), v, atol=1e-15)


def check_prefix_mean(attn):
    """P7: K = 0 makes all visible scores equal, so O_i is the mean of
    V_0..V_i (checks the mask and the normalisation together)."""
    S = 11
    r = rng(7)
    q, v = r.standard_normal((S, 8)), r.standard_normal((S, 8))
    O = _prefill_one_head(attn, q, np.zeros((S, 8)), v, np.arange(S), 0.125)
    want = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
    return np.allclose(O, want, atol=1e-13)


def check_causality(attn):
    """P8: changing q/k/v at positions > i leaves O_i unchanged exactly."""
    S, i = 10, 4
    r = rng(8)
    q, k, v = (r.standard_normal((S, 8)) for _ in range(3))
    O = _prefill_one_head(attn, q, k, v, np.arange(S), 0.35)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for a in (q2, k2, v2):
        a[i + 1:] = r.standard_normal((S - i - 1, 8)) * 50
    O2 = _prefill_one_head(attn, q2, k2, v2, np.arange(S), 0.35)
    return np.array_equal(O[: i + 1], O2[: i + 1]) and not np.allclose(O[i + 1:], O2[i + 1:])


def check_hard_max(attn):
    """P15: one key with an overwhelming score takes all the weight."""
    S = 6
    q = np.zeros((S, 4)); q[:, 0] = 1.0
    k = np.zeros((S, 4)); k[2, 0] = 2000.0
    v = rng(9).standard_normal((S, 4))
    O = _prefill_one_head(attn, q, k, v, np.arange(S), 1.0)
    return np.allclose(O[2:], np.broadcast_to(v[2], (S - 2, 4)), atol=1e-12)


def check_two_token_by_hand(attn):
    """[Guide] §4.2 (third ruler): a 2-token input worked by hand.

    D = 2, theta_0 = 1, positions 0 and 1, scale 1/sqrt(2).
    q0 = (1,0), q1 = (0,1), k0 = k1 = (1,0), v0 = (1,2), v1 = (3,-1).
    After RoPE: q1' = (-sin 1, cos 1), k0' = (1, 0), k1' = (cos 1, sin 1).
    Row 0 sees only key 0: O_0 = v0.
    Row 1: scores q1'.k0'/sqrt2 = -sin(1)/sqrt2 and q1'.k1'/sqrt2 = 0, so
    O_1 = (e^a v0 + v1) / (e^a + 1) with a = -sin(1)/sqrt2."""
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    k = np.array([[1.0, 0.0], [1.0, 0.0]])
    v = np.array([[1.0, 2.0], [3.0, -1.0]])
    pos = np.arange(2)
    qr, kr = A.rope_rotate(q, pos, 1e4), A.rope_rotate(k, pos, 1e4)
    O = attn(qr, kr, v, (pos, pos), 1 / math.sqrt(2))
    a = -math.sin(1.0) / math.sqrt(2)
    o1 = (math.exp(a) * v[0] + v[1]) / (math.exp(a) + 1)
    return np.allclose(O[0], v[0], atol=1e-15) and np.allclose(O[1], o1, atol=1e-15)


ATTN_PINS = [check_rows_are_distributions, check_single_token, check_prefix_mean,
             check_causality, check_hard_max, check_two_token_by_hand]


@pytest.mark.parametrize("pin", ATTN_PINS, ids=lambda f: f.__name__)
def test_oracle_attention_pins(pin):
    assert pin(A.causal_attention)


def _attn_generic(q, k, v, positions, scale, diag_masked=False, lower=False,
                  transposed=False, noscale=False):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    qp, kp = positions
    s = (k @ q.T).T if not transposed else (q @ k.T).T
    if noscale:
        scale = 1.0
    s = s * scale
    if lower:
        blocked = kp[None, :] < qp[:, None]
    elif diag_masked:
        blocked = kp[None, :] >= qp[:, None]
    else:
        blocked = kp[None, :] > qp[:, None]
    s = np.where(blocked, -np.inf, s)
    with np.errstate(invalid="ignore"):
        e = np.exp(s - s.max(1, keepdims=True))
        return (e / e.sum(1, keepdims=True)) @ v


ATTN_MUTANTS = {
    "diagonal_masked": lambda q, k, v, p, s: _attn_generic(q, k, v, p, s, diag_masked=True),
    "mask_wrong_side": lambda q, k, v, p, s: _attn_generic(q, k, v, p, s, lower=True),
    "transposed_scores": lambda q, k, v, p, s: _attn_generic(q, k, v, p, s, transposed=True),
    "scale_dropped": lambda q, k, v, p, s: _attn_generic(q, k, v, p, s, noscale=True),
}


def test_generic_attention_matches_oracle():
    r = rng(10)
    q, k, v = (r.standard_normal((7, 4)) for _ in range(3))
    pos = np.arange(7)
    assert np.allclose(_attn_generic(q, k, v, (pos, pos), 0.4),
                       A.causal_attention(q, k, v, (pos, pos), 0.4), atol=1e-14)


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_pins_catch_planted_mistakes(name):
    with np.errstate(all="ignore"):
        assert not all(pin(ATTN_MUTANTS[name]) for pin in ATTN_PINS)


# --------------------------------------------------------------------------
# P12: scalar brute force on tiny shapes ([Guide] §4.2, third ruler)
# --------------------------------------------------------------------------

def _brute_prefill_head(q, k, v, pos, theta, scale):
    S, D = len(q), len(q[0])

    def rot(x, m):
        y = list(x)
        for i in range(D // 2):
            a = m * theta ** (-2.0 * i / D)
            y[2 * i] = x[2 * i] * math.cos(a) - x[2 * i + 1] * math.sin(a)
            y[2 * i + 1] = x[2 * i] * math.sin(a) + x[2 * i + 1] * math.cos(a)
        return y

    qr = [rot(q[s], pos[s]) for s in range(S)]
    kr = [rot(k[s], pos[s]) for s in range(S)]
    out = []
    for i in range(S):
        js = [j for j in range(S) if pos[j] <= pos[i]]
        sc = [sum(qr[i][d] * kr[j][d] for d in range(D)) * scale for j in js]
        mx = max(sc)
        w = [math.exp(s - mx) for s in sc]
        z = sum(w)
        out.append([sum(w[t] * v[js[t]][d] for t in range(len(js))) / z for d in range(D)])
    return out


@pytest.mark.parametrize("S,D", [(1, 2), (2, 2), (3, 2), (2, 4), (3, 4)])
def test_prefill_matches_scalar_brute_force(S, D):
    r = rng(100 + 10 * S + D)
    B, Hq, Hkv = 2, 4, 2
    q = r.standard_normal((B, Hq, S, D))
    k = r.standard_normal((B, Hkv, S, D))
    v = r.standard_normal((B, Hkv, S, D))
    pos = np.stack([np.arange(S), np.arange(S) + 3])
    out, k_rot = A.attn_prefill(q, k, v, pos, 10000.0, 0.7)
    for b in range(B):
        for hq in range(Hq):
            hk = hq // 2
            want = _brute_prefill_head(q[b, hq].tolist(), k[b, hk].tolist(),
                                       v[b, hk].tolist(), pos[b].tolist(), 10000.0, 0.7)
            assert np.allclose(out[b, hq], want, atol=1e-13)


# --------------------------------------------------------------------------
# P13: blockwise online softmax ([Scratch] §3.4) equals the full softmax
# --------------------------------------------------------------------------

def _online_softmax_attention(q, k, v, scale, bm, bn):
    """Test-only fp64 restatement of the tiled algorithm: query row blocks,
    key blocks, running max m and sum l, rescaled accumulator."""
    S, D = q.shape
    out = np.zeros((S, v.shape[1]))
    for i0 in range(0, S, bm):
        qi = q[i0:i0 + bm]
        rows = np.arange(i0, min(i0 + bm, S))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), v.shape[1]))
        for j0 in range(0, rows[-1] + 1, bn):
            cols = np.arange(j0, min(j0 + bn, S))
            s = (qi @ k[cols].T) * scale
            s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(1))
            alpha = np.exp(m - m_new)
            p = np.exp(s - m_new[:, None])
            l = alpha * l + p.sum(1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        out[rows] = acc / l[:, None]
    return out


@pytest.mark.parametrize("bm,bn", [(1, 1), (3, 5), (16, 16), (64, 32), (128, 64)])
def test_online_softmax_equals_full(bm, bn):
    S, D = 150, 16
    r = rng(200 + bm + bn)
    q, k, v = (r.standard_normal((S, D)) * 3 for _ in range(3))
    pos = np.arange(S)
    full = A.causal_attention(q, k, v, (pos, pos), 0.25)
    assert np.allclose(_online_softmax_attention(q, k, v, 0.25, bm, bn), full,
                       atol=1e-12, rtol=0)


# ==========================================================================
# KV-cache and decode pins ([Guide] §2.5; [Scratch] §3.2, §3.3; [NanoVLLM] §05)
# ==========================================================================

def _prompt_then_decode(B, Hq, Hkv, S, T, D, seed, paged=False):
    """Prefill S prompt tokens into a cache, then T decode steps; returns the
    decode outputs and the full-recompute prefill over all S+T tokens."""
    r = rng(seed)
    n = S + T
    q = r.standard_normal((B, Hq, n, D))
    k = r.standard_normal((B, Hkv, n, D))
    v = r.standard_normal((B, Hkv, n, D))
    pos = np.tile(np.arange(n), (B, 1))
    full, _ = A.attn_prefill(q, k, v, pos)
    _, k_rot = A.attn_prefill(q[:, :, :S], k[:, :, :S], v[:, :, :S], pos[:, :S])
    if paged:
        mbps = (n + 15) // 16
        nb = B * mbps + 3
        table = r.permutation(nb)[: B * mbps].reshape(B, mbps)
        ck, cv = np.full((nb, Hkv, 16, D), np.nan), np.full((nb, Hkv, 16, D), np.nan)
    else:
        table = None
        ck, cv = np.full((B, Hkv, n, D), np.nan), np.full((B, Hkv, n, D), np.nan)
    A.kv_cache_append(ck, cv, k_rot, v[:, :, :S], pos[:, :S], block_table=table)
    outs = []
    for t in range(T):
        lens = np.full(B, S + t)
        outs.append(A.attn_decode(q[:, :, S + t], k[:, :, S + t], v[:, :, S + t],
                                  ck, cv, lens, block_table=table))
    return np.stack(outs, axis=2), full[:, :, S:]


def check_decode_equals_prefill_last_row(decode_impl=None):
    """P9: decode step t equals row S+t of a full-recompute prefill."""
    dec, want = _prompt_then_decode(2, 4, 2, 13, 5, 8, seed=11)
    return np.allclose(dec, want, atol=1e-12)


def test_decode_equals_prefill_last_row():
    assert check_decode_equals_prefill_last_row()


def test_paged_decode_equals_prefill_last_row():
    dec, want = _prompt_then_decode(3, 4, 4, 29, 6, 8, seed=12, paged=True)
    assert np.allclose(dec, want, atol=1e-12)


def test_decode_with_empty_cache_returns_new_value():
    """P6 for decode: L = 0 attends to the new token only, so O = v_new."""
    r = rng(13)
    B, Hq, Hkv, D = 3, 4, 2, 8
    q, kn, vn = r.standard_normal((B, Hq, D)), r.standard_normal((B, Hkv, D)), r.standard_normal((B, Hkv, D))
    ck, cv = np.full((B, Hkv, 4, D), np.nan), np.full((B, Hkv, 4, D), np.nan)
    out = A.attn_decode(q, kn, vn, ck, cv, np.zeros(B, int))
    assert np.allclose(out, np.repeat(vn, 2, axis=1), atol=1e-15)
    # the new key is stored rotated at index 0 (angle 0: unchanged)
    assert np.array_equal(ck[:, :, 0], kn) and np.array_equal(cv[:, :, 0], vn)


def test_decode_appends_rotated_key_at_position_len():
    r = rng(14)
    B, H, D = 2, 2, 16
    lens = np.array([3, 7])
    q, kn, vn = (r.standard_normal((B, H, D)) for _ in range(3))
    ck, cv = r.standard_normal((B, H, 9, D)), r.standard_normal((B, H, 9, D))
    before_k, before_v = ck.copy(), cv.copy()
    A.attn_decode(q, kn, vn, ck, cv, lens)
    for b in range(B):
        L = lens[b]
        want_k = A.rope_rotate(kn[b][:, None, :], np.array([L]))[:, 0]
        assert np.allclose(ck[b, :, L], want_k, atol=1e-15)
        assert np.array_equal(cv[b, :, L], vn[b])
        keep = [t for t in range(9) if t != L]
        assert np.array_equal(ck[b, :, keep], before_k[b, :, keep])
        assert np.array_equal(cv[b, :, keep], before_v[b, :, keep])


def test_paged_equals_contiguous_under_random_tables():
    """P10: any block-table permutation gives the contiguous result."""
    r = rng(15)
    B, Hq, Hkv, D = 4, 8, 2, 16
    lens = np.array([0, 15, 16, 45])
    cap = 48
    q, kn, vn = r.standard_normal((B, Hq, D)), r.standard_normal((B, Hkv, D)), r.standard_normal((B, Hkv, D))
    ck, cv = r.standard_normal((B, Hkv, cap, D)), r.standard_normal((B, Hkv, cap, D))
    mbps = cap // 16
    for trial in range(3):
        nb = B * mbps + 5
        table = r.permutation(nb)[: B * mbps].reshape(B, mbps)
        pk, pv = np.full((nb, Hkv, 16, D), np.nan), np.full((nb, Hkv, 16, D), np.nan)
        for b in range(B):
            for t in range(cap):
                pk[table[b, t // 16], :, t % 16] = ck[b, :, t]
                pv[table[b, t // 16], :, t % 16] = cv[b, :, t]
        ck2, cv2 = ck.copy(), cv.copy()
        want = A.attn_decode(q, kn, vn, ck2, cv2, lens)
        got = A.attn_decode(q, kn, vn, pk, pv, lens, block_table=table)
        assert np.array_equal(got, want)
        for b in range(B):
            L = lens[b]
            assert np.array_equal(pk[table[b, L // 16], :, L % 16], ck2[b, :, L])


def test_paged_slot_addressing():
    table = np.array([[7, 2, 9], [0, 4, 1]])
    assert A.paged_slot(table, 0, 0, 16) == (7, 0)
    assert A.paged_slot(table, 0, 15, 16) == (7, 15)
    assert A.paged_slot(table, 0, 16, 16) == (2, 0)
    assert A.paged_slot(table, 1, 47, 16) == (1, 15)


def test_gqa_equals_mha_with_repeated_kv_heads():
    """P11: Hq query heads over Hkv KV heads equal MHA with every KV head
    repeated Hq/Hkv times (contiguous groups)."""
    r = rng(16)
    B, Hq, Hkv, S, D = 2, 8, 2, 12, 8
    q = r.standard_normal((B, Hq, S, D))
    k, v = r.standard_normal((B, Hkv, S, D)), r.standard_normal((B, Hkv, S, D))
    pos = np.tile(np.arange(S), (B, 1))
    gqa, _ = A.attn_prefill(q, k, v, pos)
    mha, _ = A.attn_prefill(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), pos)
    assert np.array_equal(gqa, mha)


def test_prefill_positions_offset_shift_invariance():
    """Scores depend only on relative position (P3 at the attention level):
    shifting every position by a constant leaves the prefill output equal."""
    r = rng(17)
    q, k, v = r.standard_normal((1, 2, 20, 16)), r.standard_normal((1, 2, 20, 16)), r.standard_normal((1, 2, 20, 16))
    a, _ = A.attn_prefill(q, k, v, np.arange(20)[None])
    b, _ = A.attn_prefill(q, k, v, (np.arange(20) + 1234)[None])
    assert np.allclose(a, b, atol=1e-11)


# planted mistakes in the decode path
def _decode_without_new_token(q, kn, vn, ck, cv, lens):
    B, Hq, D = q.shape
    out = np.empty((B, Hq, D))
    for b in range(B):
        L = int(lens[b])
        qr = A.rope_rotate(q[b][:, None], np.array([L]))[:, 0]
        for h in range(Hq):
            out[b, h] = A.causal_attention(qr[h][None], ck[b, h, :L], cv[b, h, :L],
                                           (np.array([L]), np.arange(L)), 1 / math.sqrt(D))[0]
    return out


def test_decode_pin_catches_skipping_the_new_token():
    r = rng(18)
    B, H, D, S = 1, 2, 8, 6
    q, k, v = (r.standard_normal((B, H, S + 1, D)) for _ in range(3))
    pos = np.arange(S + 1)[None]
    full, k_rot = A.attn_prefill(q, k, v, pos)
    ck, cv = k_rot[:, :, :S].copy(), v[:, :, :S].copy()
    bad = _decode_without_new_token(q[:, :, S], k[:, :, S], v[:, :, S], ck, cv, np.array([S]))
    assert not np.allclose(bad, full[:, :, S])


def test_paged_pin_catches_swapped_block_and_offset():
    table = np.array([[3, 1, 0, 2]])
    good = [A.paged_slot(table, 0, t, 16) for t in range(64)]
    bad = [(int(table[0, t % 4]), t // 16) for t in range(64)]
    assert good != bad
    assert len(set(good)) == 64


# ==========================================================================
# Chunked prefill against a cache ([Scratch] §3.2-§3.3)
# ==========================================================================

def _chunk_case(B, Hq, Hkv, D, seed):
    r = rng(seed)
    n = 23
    q = r.standard_normal((B, Hq, n, D))
    k, v = r.standard_normal((B, Hkv, n, D)), r.standard_normal((B, Hkv, n, D))
    return q, k, v, n


def _two_chunks(impl, q, k, v, n, split, paged=False):
    """The prompt as chunk [0, split) then chunk [split, n) over one cache."""
    B, Hkv, D = q.shape[0], k.shape[1], q.shape[-1]
    cap = 32
    ck, cv = np.full((B, Hkv, cap, D), np.nan), np.full((B, Hkv, cap, D), np.nan)
    table = None
    if paged:
        nb = B * 2 + 3
        table = rng(99).permutation(nb)[: B * 2].reshape(B, 2)
        ck, cv = np.full((nb, Hkv, 16, D), np.nan), np.full((nb, Hkv, 16, D), np.nan)
    o1 = impl(q[:, :, :split], k[:, :, :split], v[:, :, :split], ck, cv, np.zeros(B, int),
              block_table=table)
    o2 = impl(q[:, :, split:], k[:, :, split:], v[:, :, split:], ck, cv, np.full(B, split),
              block_table=table)
    return np.concatenate([o1, o2], axis=2), ck, cv, table


def check_chunks_equal_whole_prompt(impl, paged=False):
    """A prompt taken in two chunks over the cache equals the prompt taken
    whole: same outputs, and the cache holds the rotated keys and raw values
    at indices 0..n-1 either way."""
    q, k, v, n = _chunk_case(2, 4, 2, 8, seed=31)
    whole, k_rot = A.attn_prefill(q, k, v, np.tile(np.arange(n), (2, 1)))
    for split in (1, 9, 16, 22):
        got, ck, cv, table = _two_chunks(impl, q, k, v, n, split, paged)
        if not np.allclose(got, whole, atol=1e-12):
            return False
        rows_k = np.stack([A.cache_rows(ck, b, h, n, table) for b in range(2) for h in range(2)])
        rows_v = np.stack([A.cache_rows(cv, b, h, n, table) for b in range(2) for h in range(2)])
        if not (np.allclose(rows_k, k_rot.reshape(4, n, 8), atol=1e-14)
                and np.array_equal(rows_v, v.reshape(4, n, 8))):
            return False
    return True


def test_chunked_prefill_equals_whole_prompt():
    assert check_chunks_equal_whole_prompt(A.attn_prefill_cached)


def test_chunked_prefill_paged_equals_whole_prompt():
    assert check_chunks_equal_whole_prompt(A.attn_prefill_cached, paged=True)


def test_one_token_chunk_equals_decode_step():
    r = rng(32)
    B, Hq, Hkv, D = 3, 4, 2, 8
    lens = np.array([0, 5, 11])
    q, kn, vn = r.standard_normal((B, Hq, D)), r.standard_normal((B, Hkv, D)), r.standard_normal((B, Hkv, D))
    ck, cv = r.standard_normal((B, Hkv, 12, D)), r.standard_normal((B, Hkv, 12, D))
    ck2, cv2 = ck.copy(), cv.copy()
    dec = A.attn_decode(q, kn, vn, ck, cv, lens)
    chk = A.attn_prefill_cached(q[:, :, None], kn[:, :, None], vn[:, :, None], ck2, cv2, lens)
    assert np.allclose(chk[:, :, 0], dec, atol=1e-14)
    assert np.array_equal(ck, ck2) and np.array_equal(cv, cv2)


def test_one_token_chunk_on_empty_cache_returns_its_value():
    r = rng(33)
    B, Hq, Hkv, D = 2, 4, 4, 8
    q, k, v = (r.standard_normal((B, h, 1, D)) for h in (Hq, Hkv, Hkv))
    ck, cv = np.full((B, Hkv, 3, D), np.nan), np.full((B, Hkv, 3, D), np.nan)
    out = A.attn_prefill_cached(q, k, v, ck, cv, np.zeros(B, int))
    assert np.allclose(out, v, atol=1e-15)


def test_chunk_causality_and_prefix_dependence():
    """Changing chunk token j moves no output of a query before j; changing
    one cached prefix row moves every chunk query's output."""
    r = rng(34)
    B, H, D, P, S = 1, 2, 8, 6, 7
    q, k, v = (r.standard_normal((B, H, S, D)) for _ in range(3))
    ck, cv = r.standard_normal((B, H, P + S, D)), r.standard_normal((B, H, P + S, D))
    base = A.attn_prefill_cached(q, k, v, ck.copy(), cv.copy(), np.array([P]))
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 4] += 1.0
    v2[:, :, 4] += 1.0
    pert = A.attn_prefill_cached(q, k2, v2, ck.copy(), cv.copy(), np.array([P]))
    assert np.array_equal(pert[:, :, :4], base[:, :, :4])
    assert not np.allclose(pert[:, :, 4:], base[:, :, 4:])
    cv3 = cv.copy()
    cv3[:, :, 2] += 1.0
    pref = A.attn_prefill_cached(q, k, v, ck.copy(), cv3, np.array([P]))
    assert not np.any(np.isclose(pref, base).all(axis=-1))


def test_chunked_gqa_equals_mha_with_repeated_kv_heads():
    r = rng(35)
    B, Hq, Hkv, D, P, S = 2, 8, 2, 8, 5, 6
    q = r.standard_normal((B, Hq, S, D))
    k, v = r.standard_normal((B, Hkv, S, D)), r.standard_normal((B, Hkv, S, D))
    ck, cv = r.standard_normal((B, Hkv, P + S, D)), r.standard_normal((B, Hkv, P + S, D))
    lens = np.full(B, P)
    gqa = A.attn_prefill_cached(q, k, v, ck.copy(), cv.copy(), lens)
    mha = A.attn_prefill_cached(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                                np.repeat(ck, 4, axis=1), np.repeat(cv, 4, axis=1), lens)
    assert np.array_equal(gqa, mha)


def test_padded_chunk_batch_equals_each_sequence_alone():
    """A batch of chunks of lengths n_b padded to S equals each sequence run
    alone with its n_b tokens; the padding (filled with large values here)
    changes nothing, padding rows are zero and padding slots stay unwritten."""
    r = rng(37)
    B, Hq, Hkv, D, S = 4, 4, 2, 8, 9
    lens = np.array([0, 3, 16, 7])
    n = np.array([9, 0, 4, 1])
    q = r.standard_normal((B, Hq, S, D))
    k, v = r.standard_normal((B, Hkv, S, D)), r.standard_normal((B, Hkv, S, D))
    for b in range(B):
        q[b, :, n[b]:] = 1e6
        k[b, :, n[b]:] = -1e6
        v[b, :, n[b]:] = 1e6
    ck, cv = r.standard_normal((B, Hkv, 32, D)), r.standard_normal((B, Hkv, 32, D))
    ck2, cv2 = ck.copy(), cv.copy()
    got = A.attn_prefill_cached(q, k, v, ck, cv, lens, chunk_lens=n)
    for b in range(B):
        sl = slice(b, b + 1)
        if n[b]:
            alone = A.attn_prefill_cached(q[sl, :, :n[b]], k[sl, :, :n[b]], v[sl, :, :n[b]],
                                          ck2[sl], cv2[sl], lens[sl])
            assert np.allclose(got[b, :, :n[b]], alone[0], atol=1e-13)
        assert np.array_equal(got[b, :, n[b]:], np.zeros_like(got[b, :, n[b]:]))
    assert np.array_equal(ck, ck2) and np.array_equal(cv, cv2)


def test_padded_chunk_pin_catches_ignoring_chunk_lens():
    """Planted mistake: treating the padding as real tokens.  The padding
    rows then come out nonzero and the padding is stored in the cache, both
    of which the pin above rules out."""
    r = rng(38)
    B, H, D, S = 2, 2, 8, 5
    n = np.array([5, 2])
    q, k, v = (r.standard_normal((B, H, S, D)) for _ in range(3))
    ck_bad, cv_bad = np.zeros((B, H, 8, D)), np.zeros((B, H, 8, D))
    ck_good, cv_good = np.zeros((B, H, 8, D)), np.zeros((B, H, 8, D))
    bad = A.attn_prefill_cached(q, k, v, ck_bad, cv_bad, np.zeros(B, int))
    good = A.attn_prefill_cached(q, k, v, ck_good, cv_good, np.zeros(B, int), chunk_lens=n)
    assert np.any(bad[1, :, 2:] != 0) and np.array_equal(good[1, :, 2:], np.zeros((H, 3, D)))
    assert not np.array_equal(ck_bad[1, :, 2:5], ck_good[1, :, 2:5])


def _chunk_mask_without_offset(q, k, v, ck, cv, lens, block_table=None):
    """Planted mistake: the mask compares chunk-local indices, so a chunk
    query sees only the first i+1 cache rows."""
    B, Hq, S, D = q.shape
    out = np.empty((B, Hq, S, D))
    for b in range(B):
        P = int(lens[b])
        pos = P + np.arange(S)
        qr, kr = A.rope_rotate(q[b], pos), A.rope_rotate(k[b], pos)
        if block_table is None:
            A.kv_cache_append(ck[b:b + 1], cv[b:b + 1], kr[None], v[b:b + 1], pos[None])
        else:
            A.kv_cache_append(ck, cv, kr[None], v[b:b + 1], pos[None], block_table=block_table)
        for h in range(Hq):
            keys = A.cache_rows(ck, b, h, P + S, block_table)
            vals = A.cache_rows(cv, b, h, P + S, block_table)
            out[b, h] = A.causal_attention(qr[h], keys, vals, (np.arange(S), np.arange(P + S)),
                                           1 / math.sqrt(D))
    return out


def _chunk_rope_at_local_positions(q, k, v, ck, cv, lens, block_table=None):
    """Planted mistake: the chunk is rotated at positions 0..S-1."""
    B, Hq, S, D = q.shape
    out = np.empty((B, Hq, S, D))
    for b in range(B):
        P = int(lens[b])
        pos = P + np.arange(S)
        qr, kr = A.rope_rotate(q[b], np.arange(S)), A.rope_rotate(k[b], np.arange(S))
        A.kv_cache_append(ck[b:b + 1], cv[b:b + 1], kr[None], v[b:b + 1], pos[None])
        for h in range(Hq):
            out[b, h] = A.causal_attention(qr[h], ck[b, h, :P + S], cv[b, h, :P + S],
                                           (pos, np.arange(P + S)), 1 / math.sqrt(D))
    return out


@pytest.mark.parametrize("bad", [_chunk_mask_without_offset, _chunk_rope_at_local_positions])
def test_chunk_pin_catches_planted_mistakes(bad):
    def impl(q, k, v, ck, cv, lens, block_table=None):
        B, Hq = q.shape[:2]
        Hkv = k.shape[1]
        # expand the KV heads so the planted copies can index by query head
        return bad(q, k, v, ck, cv, lens) if Hq == Hkv else bad(
            q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), ck, cv, lens)
    q, k, v, n = _chunk_case(1, 2, 2, 8, seed=36)
    whole, _ = A.attn_prefill(q, k, v, np.arange(n)[None])
    got, _, _, _ = _two_chunks(impl, q, k, v, n, 9)
    assert not np.allclose(got, whole, atol=1e-6)


# ==========================================================================
# P14: constants the pages print
# ==========================================================================

def test_scale_constants_printed_on_pages():
    g = load_golden("pages_constants.txt")
    val, tol = g["scale_head_dim_128"]
    assert abs(1 / math.sqrt(128) - val) <= tol
    val, tol = g["scale_model_dim_4096"]
    assert abs(1 / math.sqrt(4096) - val) <= tol


def test_kv_bytes_formula_printed_on_pages():
    import bench
    g = load_golden("pages_constants.txt")
    # 32 layers of one 2048-token request, 32 KV heads, head_dim 128, 2-byte elements
    one = 32 * bench.decode_kv_bytes([2048], Hkv=32, D=128, elem_bytes=2)
    assert one == 2 * 32 * 32 * 128 * 2048 * 2 == 1_073_741_824
    val, tol = g["kv_bytes_one_request"]
    assert abs(one - val) <= tol
    val, tol = g["kv_bytes_ten_requests"]
    assert abs(10 * one - val) <= tol


def test_padded_prompt_batch_equals_each_prompt_alone():
    """A batch of prompts of lengths n_b padded to S equals each prompt run
    alone at its own length; the padding (NaN in q, k, v and a negative
    position here) changes nothing; padding rows of the output and of k_rot
    are zero.  GQA with two query heads per KV head."""
    r = rng(39)
    B, Hq, Hkv, D, S = 4, 4, 2, 8, 9
    n = np.array([9, 0, 4, 1])
    q = r.standard_normal((B, Hq, S, D))
    k, v = r.standard_normal((B, Hkv, S, D)), r.standard_normal((B, Hkv, S, D))
    pos = np.tile(np.arange(S) * 3 + 2, (B, 1))
    for b in range(B):
        q[b, :, n[b]:] = np.nan
        k[b, :, n[b]:] = np.nan
        v[b, :, n[b]:] = np.nan
        pos[b, n[b]:] = -5
    got, got_k = A.attn_prefill(q, k, v, pos, seq_lens=n)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_k))
    for b in range(B):
        sl = slice(b, b + 1)
        if n[b]:
            alone, alone_k = A.attn_prefill(q[sl, :, :n[b]], k[sl, :, :n[b]], v[sl, :, :n[b]],
                                            pos[sl, :n[b]])
            assert np.allclose(got[b, :, :n[b]], alone[0], atol=1e-13)
            assert np.allclose(got_k[b, :, :n[b]], alone_k[0], atol=1e-13)
        assert np.array_equal(got[b, :, n[b]:], np.zeros_like(got[b, :, n[b]:]))
        assert np.array_equal(got_k[b, :, n[b]:], np.zeros_like(got_k[b, :, n[b]:]))


def test_one_token_prompt_gives_its_value():
    """A prompt of one token (padded to 5 rows) sees only itself: O = v."""
    r = rng(40)
    q, k, v = (r.standard_normal((1, 2, 5, 8)) for _ in range(3))
    out, _ = A.attn_prefill(q, k, v, np.arange(5)[None], seq_lens=np.array([1]))
    assert np.allclose(out[0, :, 0], v[0, :, 0], atol=1e-15)
    assert not np.any(out[0, :, 1:])


def test_padded_prompt_pin_catches_plausible_mistakes():
    """Planted mistakes the pins above rule out: ignoring the lengths (the
    padding rows come out nonzero), and a length short by one (the last
    prompt token's row is zero instead of its attention output)."""
    r = rng(41)
    B, H, D, S = 2, 2, 8, 6
    n = np.array([6, 3])
    q, k, v = (r.standard_normal((B, H, S, D)) for _ in range(3))
    pos = np.tile(np.arange(S), (B, 1))
    good, _ = A.attn_prefill(q, k, v, pos, seq_lens=n)
    ignored, _ = A.attn_prefill(q, k, v, pos)
    short, _ = A.attn_prefill(q, k, v, pos, seq_lens=n - 1)
    assert np.any(ignored[1, :, 3:] != 0) and not np.any(good[1, :, 3:])
    alone, _ = A.attn_prefill(q[1:, :, :3], k[1:, :, :3], v[1:, :, :3], pos[1:, :3])
    assert np.allclose(good[1, :, :3], alone[0], atol=1e-13)
    assert not np.allclose(short[1, :, :3], alone[0], atol=1e-6)
