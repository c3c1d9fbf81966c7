"""GPU parity in the half-split RoPE layout (pair i = elements i and
i + D/2, the layout of Llama/Qwen checkpoints): rope_apply in place,
attn_prefill and the cache it writes, attn_decode (contiguous and paged, one
and four query heads per KV head, fp32 and bf16) and attn_prefill_cached,
each against the oracle evaluated with pairing="half"; and a check that the
two layouts give different results, so the flag is honoured."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import TOL, bits, f64, log_case, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HALF = "half"


@pytest.fixture(scope="module")
def car():
    import causal_attention_rope_amd as m
    return m


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,S", [(2, 3, 37), (1, 4, 300)])
def test_rope_apply_half(car, dtype, D, B, H, S):
    log_case(f"rope_apply half {dtype} D={D} B={B} H={H} S={S}")
    x = W.randn((B, H, S, D), dtype, DEV, 12, D + S)
    pos_np = np.sort(np.random.default_rng(S).choice(16384, size=(B, S)), axis=1).astype(np.int32)
    pos = torch.from_numpy(pos_np).to(DEV)
    want = oracle.rope_rotate(f64(x), pos_np[:, None, :], 10000.0, pairing=HALF)
    car.rope_apply(x, pos, rope_pairing=HALF)
    torch.cuda.synchronize()
    err = max_abs(f64(x), want)
    log_case(f"max-abs error {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 64),
                                     (torch.bfloat16, 128)], ids=["f32-64", "bf16-64", "bf16-128"])
def test_prefill_half(car, dtype, D):
    log_case(f"prefill half {dtype} D={D}")
    case = W.prefill_case("half", 2, 4, 2, 300, D, dtype, 600 + D, DEV)
    ck = torch.full((2, 2, 320, D), float("nan"), dtype=dtype, device=DEV)
    cache = car.KVCache(ck, ck.clone())
    out = car.attn_prefill(case.q, case.k, case.v, case.positions, cache=cache,
                           rope_pairing=HALF)
    torch.cuda.synchronize()
    want, k_rot = oracle.attn_prefill(f64(case.q), f64(case.k), f64(case.v),
                                      case.positions.cpu().numpy(), pairing=HALF)
    err = max(max_abs(f64(out), want), max_abs(f64(cache.k[:, :, :300]), k_rot))
    assert torch.equal(bits(cache.v[:, :, :300].cpu()), bits(case.v.cpu()))
    log_case(f"max-abs error {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,D,Hq,Hkv,paged", [
    (torch.bfloat16, 128, 4, 4, False), (torch.bfloat16, 128, 8, 2, True),
    (torch.float32, 64, 4, 4, False), (torch.float32, 128, 8, 2, True)],
    ids=["bf16-128-mha-contig", "bf16-128-gqa4-paged", "f32-64-mha-contig", "f32-128-gqa4-paged"])
def test_decode_half(car, dtype, D, Hq, Hkv, paged):
    log_case(f"decode half {dtype} D={D} Hq={Hq} Hkv={Hkv} paged={paged}")
    lens = [0, 1, 300, 1030]
    case = W.decode_case("dhalf", 4, Hq, Hkv, D, dtype, lens, 610 + D, DEV, paged=paged,
                         poison_unused=True, extra_blocks=2)
    table = case.block_table.cpu().numpy() if paged else None
    ck, cv = f64(case.cache_k), f64(case.cache_v)
    cache = car.KVCache(case.cache_k, case.cache_v, case.block_table)
    out = car.attn_decode(case.q, case.k_new, case.v_new, case.seq_lens, cache, case.max_seq_len,
                          rope_pairing=HALF)
    torch.cuda.synchronize()
    want = oracle.attn_decode(f64(case.q), f64(case.k_new), f64(case.v_new), ck, cv,
                              np.array(lens), block_table=table, pairing=HALF)
    err = max_abs(f64(out), want)
    # the stored key (rotated in the half layout) at index L
    for b, L in enumerate(lens):
        if paged:
            got, ref = f64(case.cache_k[int(table[b, L // 16]), :, L % 16]), ck[int(table[b, L // 16]), :, L % 16]
        else:
            got, ref = f64(case.cache_k[b, :, L]), ck[b, :, L]
        err = max(err, max_abs(got, ref))
    log_case(f"max-abs error {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,D,paged", [(torch.bfloat16, 128, True), (torch.float32, 64, False)],
                         ids=["bf16-128-paged", "f32-64-contig"])
def test_chunked_prefill_half(car, dtype, D, paged):
    log_case(f"chunked prefill half {dtype} D={D} paged={paged}")
    case = W.chunk_case("chalf", 3, 8, 2, 70, D, dtype, [0, 37, 300], 620 + D, DEV,
                        paged=paged, poison_unused=True, extra_blocks=3)
    table = case.block_table.cpu().numpy() if paged else None
    ck, cv = f64(case.cache_k), f64(case.cache_v)
    cache = car.KVCache(case.cache_k, case.cache_v, case.block_table)
    out = car.attn_prefill_cached(case.q, case.k, case.v, case.seq_lens, cache, case.max_seq_len,
                                  rope_pairing=HALF)
    torch.cuda.synchronize()
    want = oracle.attn_prefill_cached(f64(case.q), f64(case.k), f64(case.v), ck, cv,
                                      np.array(case.lens_host), block_table=table, pairing=HALF)
    err = max_abs(f64(out), want)
    log_case(f"max-abs error {err:.3e}")
    assert err <= TOL[dtype]


def test_pairings_differ(car):
    """The same inputs in the two layouts give outputs far apart: the flag
    reaches the kernels."""
    case = W.prefill_case("diff", 1, 2, 2, 64, 64, torch.float32, 630, DEV)
    a = car.attn_prefill(case.q, case.k, case.v, case.positions)
    h = car.attn_prefill(case.q, case.k, case.v, case.positions, rope_pairing=HALF)
    torch.cuda.synchronize()
    assert max_abs(f64(a), f64(h)) > 1e-2
