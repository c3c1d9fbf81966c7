"""GPU parity: attn_prefill_cached (a prompt chunk continuing a cached
prefix) against the oracle for contiguous and paged caches, fp32 and bf16,
D = 64 and 128, GQA groups, prefix lengths on and off the key-tile and block
boundaries, one-token and empty-prefix chunks, NaN canaries in every slot the
call must not read before writing it; a prompt taken in two chunks against
the whole-prompt oracle; a long-context chunk (3072 cached + 1024 new tokens,
32 heads, D = 128) and a paged GQA batch on sampled heads."""

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


def _oracle_inputs(case, heads=None):
    """float64 inputs, optionally restricted to the query heads ``heads``
    (a whole number of GQA groups starting at a group boundary)."""
    g = case.Hq // case.Hkv
    qh = slice(None) if heads is None else slice(heads[0], heads[1])
    kh = slice(None) if heads is None else slice(heads[0] // g, heads[1] // g)
    q, k, v = f64(case.q[:, qh]), f64(case.k[:, kh]), f64(case.v[:, kh])
    ck, cv = f64(case.cache_k[:, kh]), f64(case.cache_v[:, kh])
    table = case.block_table.cpu().numpy() if case.paged else None
    return q, k, v, ck, cv, table, qh, kh


def run_and_check(car, case, heads=None):
    q, k, v, ck, cv, table, qh, kh = _oracle_inputs(case, heads)
    cache = car.KVCache(case.cache_k, case.cache_v, case.block_table)
    out = car.attn_prefill_cached(case.q, case.k, case.v, case.seq_lens, cache,
                                  case.max_seq_len, theta=case.theta, scale=case.scale)
    torch.cuda.synchronize()
    lens = np.array(case.lens_host)
    want = oracle.attn_prefill_cached(q, k, v, ck, cv, lens, case.theta, case.scale,
                                      block_table=table)
    tol = TOL[case.dtype]
    err = max_abs(f64(out[:, qh]), want)
    # the chunk's rows in the cache: rotated keys against the oracle's, values bit-exact
    gk, gv = f64(case.cache_k[:, kh]), case.cache_v[:, kh].cpu()
    for b, P in enumerate(case.lens_host):
        t = np.arange(P, P + case.S)
        if case.paged:
            blk, off = table[b, t // 16], t % 16
            got_k, want_k = gk[blk, :, off], ck[blk, :, off]            # [S, Hkv, D]
            got_v = gv[torch.as_tensor(blk), :, torch.as_tensor(off)].transpose(0, 1)
        else:
            got_k, want_k = gk[b, :, P:P + case.S], ck[b, :, P:P + case.S]
            got_v = gv[b, :, P:P + case.S]                               # [Hkv, S, D]
        err = max(err, max_abs(got_k, want_k))
        want_v = case.v[b, kh].cpu()
        assert torch.equal(bits(got_v.contiguous()), bits(want_v.contiguous())), f"values of b={b}"
    assert torch.isfinite(out.float()).all()
    log_case(f"{case.name}: max-abs error {err:.3e} (tol {tol})")
    assert err <= tol
    return out


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_chunk_lengths(car, dtype, D, paged):
    """Prefixes 0, 37, 300 (off every boundary) and a 70-token chunk."""
    log_case(f"chunk lengths {dtype} D={D} paged={paged}")
    case = W.chunk_case("chunk", 3, 4, 2, 70, D, dtype, [0, 37, 300], 500 + D, DEV,
                        paged=paged, poison_unused=True, extra_blocks=3)
    run_and_check(car, case)


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_chunk_tile_boundaries(car, paged):
    """Prefixes on and next to the 16-token block and 64/128-key tile
    boundaries, and a chunk one token past the 256-row query tile."""
    log_case(f"chunk boundaries paged={paged}")
    case = W.chunk_case("bounds", 5, 8, 8, 257, 128, torch.bfloat16, [16, 63, 64, 255, 256],
                        510, DEV, paged=paged, poison_unused=True, extra_blocks=2)
    run_and_check(car, case)


@pytest.mark.parametrize("group", [1, 4, 8])
def test_chunk_gqa_groups(car, group):
    log_case(f"chunk gqa group={group}")
    case = W.chunk_case("gqa", 2, 8, 8 // group, 33, 128, torch.bfloat16, [5, 130], 520 + group,
                        DEV, paged=True, poison_unused=True, extra_blocks=2)
    run_and_check(car, case)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_one_token_chunk(car, dtype):
    """S = 1: a decode step through the chunk path, including an empty cache."""
    log_case(f"one-token chunk {dtype}")
    case = W.chunk_case("one", 4, 4, 4, 1, 64, dtype, [0, 1, 17, 200], 530, DEV, paged=False,
                        poison_unused=True)
    run_and_check(car, case)


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_chunk_scores_jump_after_first_keys(car, paged):
    """The first 128 cached keys score over 140 below (in log2 units) the
    later cached keys and the chunk's own, with zero values (queries 12 and
    those keys -12 in the last 8 dims, every other key 0 there): the key
    group that starts with them must raise its running maximum and rescale
    at the next tile, where exponentials against the old maximum would
    overflow fp32."""
    log_case(f"chunk bf16 score jump paged={paged}")
    case = W.chunk_case("jump", 2, 4, 2, 100, 128, torch.bfloat16, [200, 333], 590, DEV,
                        paged=paged)
    case.q[..., -8:] = 12.0
    case.k[..., -8:] = 0.0
    if paged:
        table = case.block_table.cpu().numpy()
        for b in range(case.B):
            lo = torch.as_tensor(table[b, :8], device=DEV, dtype=torch.long)  # tokens 0..127
            hi = torch.as_tensor(table[b, 8:], device=DEV, dtype=torch.long)
            case.cache_k[lo, :, :, -8:] = -12.0
            case.cache_v[lo] = 0.0
            case.cache_k[hi, :, :, -8:] = 0.0
    else:
        case.cache_k[:, :, :128, -8:] = -12.0
        case.cache_k[:, :, 128:, -8:] = 0.0
        case.cache_v[:, :, :128] = 0.0
    run_and_check(car, case)


def test_prompt_in_two_chunks_matches_whole_prompt_oracle(car):
    """Chunk [0, 300) then chunk [300, 600) of one prompt over one cache:
    both chunks' outputs against the whole-prompt oracle rows."""
    B, H, S, D = 2, 8, 600, 128
    pre = W.prefill_case("two", B, H, H, S, D, torch.bfloat16, 540, DEV)
    ck = torch.full((B, H, S, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    cache = car.KVCache(ck, ck.clone())
    outs = []
    for s0, s1 in ((0, 300), (300, 600)):
        lens = torch.full((B,), s0, dtype=torch.int32, device=DEV)
        outs.append(car.attn_prefill_cached(pre.q[:, :, s0:s1].contiguous(),
                                            pre.k[:, :, s0:s1].contiguous(),
                                            pre.v[:, :, s0:s1].contiguous(), lens, cache, s1))
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2)
    want, k_rot = oracle.attn_prefill(f64(pre.q), f64(pre.k), f64(pre.v),
                                      pre.positions.cpu().numpy())
    err = max(max_abs(f64(got), want), max_abs(f64(cache.k), k_rot))
    log_case(f"two chunks vs whole prompt: max-abs error {err:.3e}")
    assert err <= TOL[torch.bfloat16]


def test_long_context_chunk_contiguous(car):
    """3072 cached + 1024 new tokens, 32 heads, D = 128, cache [1, 32, 4096,
    128] (the long-prompt shape); the oracle checks heads 0-3 and 28-31."""
    case = W.chunk_case("long", 1, 32, 32, 1024, 128, torch.bfloat16, [3072], 550, DEV,
                        paged=False, max_seq=4096)
    q, k, v, ck, cv, _, _, _ = _oracle_inputs(case)
    cache = car.KVCache(case.cache_k, case.cache_v)
    out = car.attn_prefill_cached(case.q, case.k, case.v, case.seq_lens, cache, 4096)
    torch.cuda.synchronize()
    worst = 0.0
    for h0 in (0, 28):
        hs = slice(h0, h0 + 4)
        want = oracle.attn_prefill_cached(q[:, hs], k[:, hs], v[:, hs], ck[:, hs].copy(),
                                          cv[:, hs].copy(), np.array([3072]))
        worst = max(worst, max_abs(f64(out[:, hs]), want))
    log_case(f"long-context chunk: max-abs error {worst:.3e}")
    assert worst <= TOL[torch.bfloat16]


def test_paged_gqa_chunk_batch(car):
    """Two sequences with 1000 and 2500 cached tokens take a 512-token chunk
    through a random block table (Hq = 32, Hkv = 8); the oracle checks heads
    0-3 (one KV head's group)."""
    case = W.chunk_case("pgqa", 2, 32, 8, 512, 128, torch.bfloat16, [1000, 2500], 560, DEV,
                        paged=True, poison_unused=True, extra_blocks=7)
    run_and_check(car, case, heads=(0, 4))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_padded_chunk_batch(car, dtype, paged):
    """Chunks of 70, 0, 33, 1 and 64 tokens padded to S = 70, over prefixes
    of 0, 40, 300, 5 and 129 tokens.  The padding holds 7.0 (never read):
    outputs against the oracle, padding rows exactly zero, and no cache slot
    outside [P, P + n) of each sequence changes."""
    log_case(f"padded chunk batch {dtype} paged={paged}")
    lens, n, S = [0, 40, 300, 5, 129], [70, 0, 33, 1, 64], 70
    case = W.chunk_case("pad", 5, 8, 2, S, 128, dtype, lens, 580, DEV, paged=paged,
                        poison_unused=True, extra_blocks=3)
    for b, nb in enumerate(n):
        for t in (case.q, case.k, case.v):
            t[b, :, nb:] = 7.0
    cl = torch.tensor(n, dtype=torch.int32, device=DEV)
    before_k, before_v = case.cache_k.clone(), case.cache_v.clone()
    q, k, v, ck, cv, table, _, _ = _oracle_inputs(case)
    cache = car.KVCache(case.cache_k, case.cache_v, case.block_table)
    out = car.attn_prefill_cached(case.q, case.k, case.v, case.seq_lens, cache,
                                  max(P + m for P, m in zip(lens, n)), chunk_lens=cl)
    torch.cuda.synchronize()
    want = oracle.attn_prefill_cached(q, k, v, ck, cv, np.array(lens), block_table=table,
                                      chunk_lens=np.array(n))
    err = max_abs(f64(out), want)
    for b, nb in enumerate(n):
        assert torch.equal(bits(out[b, :, nb:].cpu()), torch.zeros_like(bits(out[b, :, nb:].cpu())))
    # written slots: the chunk tokens only
    written = torch.zeros(case.cache_k.shape[0], case.cache_k.shape[2], dtype=torch.bool)
    for b, (P, nb) in enumerate(zip(lens, n)):
        t = np.arange(P, P + nb)
        if paged:
            written[torch.as_tensor(table[b, t // 16]), torch.as_tensor(t % 16)] = True
        else:
            written[b, P:P + nb] = True
    keep = ~written.to(DEV)[:, None, :, None].expand_as(case.cache_k)
    assert torch.equal(bits(case.cache_k[keep]), bits(before_k[keep])), "K outside the chunks"
    assert torch.equal(bits(case.cache_v[keep]), bits(before_v[keep])), "V outside the chunks"
    w = written[:, None, :, None].expand(ck.shape).numpy()
    err = max(err, max_abs(f64(case.cache_k)[w], ck[w]))
    assert np.array_equal(f64(case.cache_v)[w], cv[w]), "V of the chunks"
    log_case(f"padded chunk batch: max-abs error {err:.3e}")
    assert err <= TOL[dtype]
