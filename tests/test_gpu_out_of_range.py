"""GPU: cache indices outside the cache are dropped, never clamped into it.

A position, a cached length or a chunk that does not fit the cache is a
caller error the host cannot see (the values live in device memory).  The
kernels keep every read inside the buffers, and they store nothing for such
an index: every cache row, of every sequence, stays bit-identical, so a bad
index cannot overwrite another token's cached key or value.  Valid tokens of
the same call are stored and attended as usual.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import TOL, bits, f64, log_case, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def car():
    import causal_attention_rope_amd as m
    return m


def make_cache(car, B, Hkv, cap, D, dtype, paged, int8, seed):
    """A cache full of canaries (NaN, or code 77 for INT8) and its block table."""
    rng = np.random.default_rng(seed)
    el = torch.int8 if int8 else dtype
    fill = 77 if int8 else float("nan")
    if paged:
        mbps = cap // 16
        nb = B * mbps + 3
        table = rng.permutation(nb)[: B * mbps].reshape(B, mbps).astype(np.int32)
        k = torch.full((nb, Hkv, 16, D), fill, dtype=el, device=DEV)
        tt = torch.from_numpy(table).to(DEV)
    else:
        table, tt = None, None
        k = torch.full((B, Hkv, cap, D), fill, dtype=el, device=DEV)
    scales = {}
    if int8:
        scales = dict(k_scale=torch.full((Hkv, D), 0.05, dtype=torch.float32, device=DEV),
                      v_scale=torch.full((Hkv, D), 0.05, dtype=torch.float32, device=DEV))
    return car.KVCache(k, k.clone(), tt, **scales), table


def row_bits(cache, table, b, hk, t):
    """Raw bits of cache row (b, hk, t) of K and of V."""
    if table is None:
        return bits(cache.k[b, hk, t].cpu()), bits(cache.v[b, hk, t].cpu())
    blk = int(table[b, t // 16])
    return bits(cache.k[blk, hk, t % 16].cpu()), bits(cache.v[blk, hk, t % 16].cpu())


def raw(t):
    return t.cpu().view(torch.uint8) if t.dtype == torch.int8 else bits(t.cpu())


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("int8", [False, True], ids=["native", "int8"])
def test_append_drops_positions_outside_cache(car, paged, int8):
    log_case(f"kv_cache_append out-of-range positions paged={paged} int8={int8}")
    B, Hkv, S, D, cap = 2, 2, 6, 64, 32
    dtype = torch.float32
    cache, table = make_cache(car, B, Hkv, cap, D, dtype, paged, int8, 5)
    k = W.randn((B, Hkv, S, D), dtype, DEV, 31, 0)
    v = W.randn((B, Hkv, S, D), dtype, DEV, 31, 1)
    pos_np = np.array([[0, -1, 5, cap, 31, cap + 9], [-7, 3, 2 ** 30, 17, cap - 1, -1]], np.int32)
    before_k, before_v = raw(cache.k), raw(cache.v)
    car.kv_cache_append(cache, k, v, torch.from_numpy(pos_np).to(DEV))
    torch.cuda.synchronize()
    after_k, after_v = raw(cache.k), raw(cache.v)
    valid = {(b, int(p)) for b in range(B) for p in pos_np[b] if 0 <= p < cap}
    for b in range(B):
        for t in range(cap):
            for hk in range(Hkv):
                if table is None:
                    idx = (b, hk, t)
                else:
                    idx = (int(table[b, t // 16]), hk, t % 16)
                same = (torch.equal(after_k[idx], before_k[idx]) and
                        torch.equal(after_v[idx], before_v[idx]))
                assert same != ((b, t) in valid), (b, t, hk)
    if not int8:
        # the valid tokens hold exactly the values given
        for b, s in ((0, 0), (0, 2), (0, 4), (1, 1), (1, 3), (1, 4)):
            t = int(pos_np[b, s])
            gk, gv = row_bits(cache, table, b, 1, t)
            assert torch.equal(gk, bits(k[b, 1, s].cpu())) and torch.equal(gv, bits(v[b, 1, s].cpu()))


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("int8,G", [(False, 1), (False, 4), (True, 1), (True, 4)],
                         ids=["native-mha", "native-gqa", "int8-mha", "int8-gqa"])
def test_decode_does_not_store_a_length_outside_cache(car, paged, int8, G):
    """seq_lens = capacity (one past the last slot) or -1: that sequence's
    cache stays bit-identical; a valid sequence in the same step stores its
    token at L only and its output matches the oracle."""
    log_case(f"decode out-of-range seq_lens paged={paged} int8={int8} G={G}")
    B, Hkv, D, cap = 3, 2, 64, 64
    Hq = Hkv * G
    dtype = torch.bfloat16 if (int8 and G > 1) else torch.float32
    cache, table = make_cache(car, B, Hkv, cap, D, dtype, paged, int8, 9)
    # sequence 0 is valid with L = 20: fill its slots 0..19 with finite values
    L0 = 20
    for t in range(L0):
        for hk in range(Hkv):
            blk, off = ((0, t) if table is None else (int(table[0, t // 16]), t % 16))
            if table is None:
                cache.k[0, hk, t] = 1 if int8 else 0.25
                cache.v[0, hk, t] = 2 if int8 else 0.5
            else:
                cache.k[blk, hk, off] = 1 if int8 else 0.25
                cache.v[blk, hk, off] = 2 if int8 else 0.5
    q = W.randn((B, Hq, D), dtype, DEV, 41, 0)
    kn = W.randn((B, Hkv, D), dtype, DEV, 41, 1)
    vn = W.randn((B, Hkv, D), dtype, DEV, 41, 2)
    lens = torch.tensor([L0, cap, -1], dtype=torch.int32, device=DEV)
    before_k, before_v = raw(cache.k), raw(cache.v)
    out = car.attn_decode(q, kn, vn, lens, cache, cap)
    torch.cuda.synchronize()
    after_k, after_v = raw(cache.k), raw(cache.v)
    for b in range(B):
        for t in range(cap):
            for hk in range(Hkv):
                idx = (b, hk, t) if table is None else (int(table[b, t // 16]), hk, t % 16)
                same = (torch.equal(after_k[idx], before_k[idx]) and
                        torch.equal(after_v[idx], before_v[idx]))
                assert same == (not (b == 0 and t == L0)), (b, t, hk)
    if not int8:
        # the valid sequence: the oracle's decode over its own slots
        ck = np.full((1, Hkv, L0 + 1, D), 0.25)
        cv = np.full((1, Hkv, L0 + 1, D), 0.5)
        want = oracle.attn_decode(f64(q[:1]), f64(kn[:1]), f64(vn[:1]), ck, cv, np.array([L0]),
                                  10000.0, 1.0 / np.sqrt(D))
        err = max_abs(f64(out[:1]), want[0] if isinstance(want, tuple) else want)
        log_case(f"valid sequence max-abs error {err:.3e}")
        assert err <= TOL[dtype]


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_chunk_that_does_not_fit_is_not_stored(car, paged):
    """Sequence 1's chunk (cached prefix cap - 4, 8 tokens) does not fit the
    cache: none of its rows is stored; sequence 0's chunk is stored at its
    positions only."""
    log_case(f"chunk out of the cache paged={paged}")
    B, Hkv, S, D, cap = 2, 2, 8, 64, 48
    dtype = torch.float32
    cache, table = make_cache(car, B, Hkv, cap, D, dtype, paged, False, 13)
    q = W.randn((B, 2 * Hkv, S, D), dtype, DEV, 51, 0)
    k = W.randn((B, Hkv, S, D), dtype, DEV, 51, 1)
    v = W.randn((B, Hkv, S, D), dtype, DEV, 51, 2)
    P0 = 10
    lens = torch.tensor([P0, cap - 4], dtype=torch.int32, device=DEV)
    before_k, before_v = raw(cache.k), raw(cache.v)
    car.attn_prefill_cached(q, k, v, lens, cache, cap)
    torch.cuda.synchronize()
    after_k, after_v = raw(cache.k), raw(cache.v)
    for b in range(B):
        for t in range(cap):
            for hk in range(Hkv):
                idx = (b, hk, t) if table is None else (int(table[b, t // 16]), hk, t % 16)
                same = (torch.equal(after_k[idx], before_k[idx]) and
                        torch.equal(after_v[idx], before_v[idx]))
                assert same == (not (b == 0 and P0 <= t < P0 + S)), (b, t, hk)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_prefill_positions_past_cache_are_not_stored(car, dtype):
    """A 40-token prompt into a 32-slot cache: tokens at positions 0..31 are
    stored, 32..39 are not (and nothing else moves); the attention over the
    prompt itself is unaffected and matches the oracle."""
    log_case(f"prefill positions past the cache {dtype}")
    B, H, S, D, cap = 1, 2, 40, 64, 32
    case = W.prefill_case("pastcache", B, H, H, S, D, dtype, 61, DEV)
    ck = torch.full((B, H, cap, D), float("nan"), dtype=dtype, device=DEV)
    cache = car.KVCache(ck, ck.clone())
    out = car.attn_prefill(case.q, case.k, case.v, case.positions, theta=case.theta,
                           scale=case.scale, cache=cache)
    torch.cuda.synchronize()
    pos = case.positions.cpu().numpy()
    want, _ = oracle.attn_prefill(f64(case.q), f64(case.k), f64(case.v), pos, case.theta,
                                  case.scale)
    err = max_abs(f64(out), want)
    log_case(f"max-abs error {err:.3e}")
    assert err <= TOL[dtype]
    # stored values: slots 0..31 hold the values given (V is stored unchanged)
    assert torch.equal(bits(cache.v[0, :, :cap].cpu()), bits(case.v[0, :, :cap].cpu()))
    assert not torch.isnan(cache.k.float()).any()
