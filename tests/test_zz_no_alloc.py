"""GPU: car_attn_decode_noalloc against car_attn_decode.

The no-allocation entry point runs the same kernels with the split partials
in the library's per-GPU device array instead of a caller's workspace, so its
outputs and its cache writes must be bit-identical to car_attn_decode's on
the same inputs.  Each case makes two calls in a row, the second with a
smaller batch and shorter sequences, so that the second call runs over the
partials the first one left in the array.  Sizes whose partials exceed the
array are refused before anything is queued.
"""

import pytest
import torch

import workloads as W
from helpers import bits, log_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def car():
    import causal_attention_rope_amd as m
    return m


def raw(t):
    return t.cpu().view(torch.uint8) if t.dtype == torch.int8 else bits(t.cpu())


def make_case(kind, B, Hq, Hkv, D, dtype, lens, seed, paged):
    if kind == "int8":
        return W.int8_decode_case(f"noalloc_{kind}", B, Hq, Hkv, D, dtype, lens, seed, DEV,
                                  paged=paged)
    return W.decode_case(f"noalloc_{kind}", B, Hq, Hkv, D, dtype, lens, seed, DEV, paged=paged)


def cache_of(car, case, k, v):
    return car.KVCache(k, v, case.block_table, k_scale=case.k_scale, v_scale=case.v_scale)


def compare(car, case):
    """attn_decode and attn_decode_noalloc on two copies of the same cache."""
    ka, va = case.cache_k.clone(), case.cache_v.clone()
    kb, vb = case.cache_k.clone(), case.cache_v.clone()
    want = car.attn_decode(case.q, case.k_new, case.v_new, case.seq_lens,
                           cache_of(car, case, ka, va), case.max_seq_len, case.theta,
                           case.scale)
    got = torch.full_like(case.q, float("nan"))
    car.attn_decode_noalloc(case.q, case.k_new, case.v_new, case.seq_lens,
                            cache_of(car, case, kb, vb), case.max_seq_len, got, case.theta,
                            case.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all()
    assert torch.equal(bits(got.cpu()), bits(want.cpu())), "output differs from attn_decode"
    assert torch.equal(raw(kb), raw(ka)) and torch.equal(raw(vb), raw(va)), "cache differs"


# (kind, Hq, Hkv, D, dtype, paged): native MHA and GQA, the INT8 split kernel
# and the INT8 matrix-core kernel (bf16 with several query heads per KV head)
CASES = [
    ("native", 8, 8, 128, torch.float32, False),
    ("native", 16, 4, 128, torch.bfloat16, True),
    ("native", 8, 1, 64, torch.bfloat16, False),
    ("int8", 4, 4, 64, torch.float32, True),
    ("int8", 32, 8, 128, torch.bfloat16, True),
]


@pytest.mark.parametrize("kind,Hq,Hkv,D,dtype,paged", CASES,
                         ids=[f"{c[0]}-h{c[1]}x{c[2]}-d{c[3]}-{str(c[4])[6:]}-"
                              f"{'paged' if c[5] else 'contiguous'}" for c in CASES])
def test_noalloc_matches_decode_twice_second_smaller(car, kind, Hq, Hkv, D, dtype, paged):
    first = [1500, 0, 255, 256, 1023, 777, 3000, 40]
    second = [300, 17]
    for i, lens in enumerate((first, second)):
        log_case(f"decode_noalloc {kind} Hq={Hq} Hkv={Hkv} D={D} {dtype} paged={paged} "
                 f"call {i + 1}: B={len(lens)} max L={max(lens)}")
        case = make_case(kind, len(lens), Hq, Hkv, D, dtype, lens, 880 + i, paged)
        compare(car, case)


def test_noalloc_refuses_sizes_beyond_its_array(car):
    """64 sequences x 32 query heads x D 128 fit up to 11776 tokens (46 splits
    of 256); one split more is refused with CAR_ERR_WORKSPACE and nothing is
    written."""
    B, Hq, Hkv, D = 64, 32, 8, 128
    assert car.decode_workspace_bytes(B, Hq, D, 46 * 256) <= car.DECODE_NOALLOC_MAX_BYTES
    assert car.decode_workspace_bytes(B, Hq, D, 46 * 256 + 1) > car.DECODE_NOALLOC_MAX_BYTES
    log_case("decode_noalloc oversize refusal")
    case = W.decode_case("noalloc_oversize", B, Hq, Hkv, D, torch.bfloat16, [5] * B, 890, DEV,
                         paged=True, blocks_per_seq=1)
    # a table wide enough for the refused length, every entry pointing at the
    # sequence's one block (never read: the call is refused first)
    table = case.block_table[:, :1].repeat(1, (46 * 256 + 1 + 15) // 16).contiguous()
    cache = car.KVCache(case.cache_k, case.cache_v, table)
    before_k, before_v = raw(case.cache_k), raw(case.cache_v)
    out = torch.full_like(case.q, float("nan"))
    with pytest.raises(car.CarError) as ei:
        car.attn_decode_noalloc(case.q, case.k_new, case.v_new, case.seq_lens, cache,
                                46 * 256 + 1, out, case.theta, case.scale)
    assert ei.value.status == 3  # CAR_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    assert torch.equal(raw(case.cache_k), before_k) and torch.equal(raw(case.cache_v), before_v)
