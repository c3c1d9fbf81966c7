"""GPU parity: rope_apply against the oracle's explicit 2x2 rotations, and
kv_cache_append bit-exact against the oracle's stores (contiguous and paged),
with NaN canaries in every slot a call must not touch."""

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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,S", [(1, 1, 1), (2, 3, 37), (1, 4, 300)])
def test_rope_apply_matches_oracle(car, dtype, D, B, H, S):
    log_case(f"rope_apply {dtype} D={D} B={B} H={H} S={S}")
    x = W.randn((B, H, S, D), dtype, DEV, 11, D + S)
    rng = np.random.default_rng(S)
    # positions anywhere a cache index can sit, including large ones
    pos_np = np.sort(rng.choice(16384, size=(B, S), replace=True), axis=1).astype(np.int32)
    pos_np[:, 0] = 0
    pos = torch.from_numpy(pos_np).to(DEV)
    want = oracle.rope_rotate(f64(x), pos_np[:, None, :], 10000.0)
    car.rope_apply(x, pos)
    torch.cuda.synchronize()
    err = max_abs(f64(x), want)
    log_case(f"max-abs error {err:.3e}")
    assert err <= TOL[dtype]


def test_rope_apply_theta_argument(car):
    x = W.randn((1, 2, 50, 64), torch.float32, DEV, 3, 1)
    pos = torch.arange(50, dtype=torch.int32, device=DEV)[None] * 7
    want = oracle.rope_rotate(f64(x), pos.cpu().numpy()[:, None, :], 500000.0)
    car.rope_apply(x, pos, theta=500000.0)
    torch.cuda.synchronize()
    assert max_abs(f64(x), want) <= 1e-4


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_kv_cache_append_bit_exact(car, dtype, D, paged):
    log_case(f"kv_cache_append {dtype} D={D} paged={paged}")
    B, Hkv, S, cap = 3, 2, 21, 64
    k = W.randn((B, Hkv, S, D), dtype, DEV, 21, 0)
    v = W.randn((B, Hkv, S, D), dtype, DEV, 21, 1)
    rng = np.random.default_rng(D + paged)
    pos_np = np.stack([np.sort(rng.choice(cap, S, replace=False)) for _ in range(B)]).astype(np.int32)
    pos = torch.from_numpy(pos_np).to(DEV)
    if paged:
        mbps = cap // 16
        nb = B * mbps + 5
        table_np = rng.permutation(nb)[: B * mbps].reshape(B, mbps).astype(np.int32)
        ck = torch.full((nb, Hkv, 16, D), float("nan"), dtype=dtype, device=DEV)
        cache = car.KVCache(ck, ck.clone(), torch.from_numpy(table_np).to(DEV))
    else:
        table_np = None
        ck = torch.full((B, Hkv, cap, D), float("nan"), dtype=dtype, device=DEV)
        cache = car.KVCache(ck, ck.clone())
    before_k, before_v = cache.k.cpu(), cache.v.cpu()
    want_k, want_v = f64(cache.k).copy(), f64(cache.v).copy()
    oracle.kv_cache_append(want_k, want_v, f64(k), f64(v), pos_np, block_table=table_np)
    car.kv_cache_append(cache, k, v, pos)
    torch.cuda.synchronize()
    for got, want, before in ((cache.k, want_k, before_k), (cache.v, want_v, before_v)):
        written = torch.from_numpy(~np.isnan(want))
        # written slots: the stored values exactly; all others: the canaries untouched
        exp = torch.where(written, torch.from_numpy(want).to(dtype), before)
        assert torch.equal(bits(got.cpu()), bits(exp))
        assert int(written.sum()) == B * Hkv * S * D


def test_kv_cache_append_empty_is_noop(car):
    ck = torch.full((1, 1, 16, 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    cache = car.KVCache(ck, ck.clone())
    e = torch.empty((1, 1, 0, 64), dtype=torch.bfloat16, device=DEV)
    car.kv_cache_append(cache, e, e, torch.empty((1, 0), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.isnan(cache.k.float()).all()
