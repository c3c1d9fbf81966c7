"""GPU parity: attn_prefill against the oracle's full-matrix masked attention
with explicit RoPE rotations, element by element, at sizes spanning several
tiles with ragged tails, plus the cache it writes; the two full-size prefill
workloads on every head."""

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


def make_cache(car, case, paged, cap):
    if case.cache_max_seq is None and not paged and cap is None:
        return None, None
    B, Hkv, D = case.B, case.Hkv, case.D
    if paged:
        mbps = (cap + 15) // 16
        nb = B * mbps + 3
        table = np.random.default_rng(cap).permutation(nb)[: B * mbps].reshape(B, mbps)
        table = table.astype(np.int32)
        ck = torch.full((nb, Hkv, 16, D), float("nan"), dtype=case.dtype, device=DEV)
        return car.KVCache(ck, ck.clone(), torch.from_numpy(table).to(DEV)), table
    ck = torch.full((B, Hkv, cap, D), float("nan"), dtype=case.dtype, device=DEV)
    return car.KVCache(ck, ck.clone()), None


def check_prefill(car, case, paged=False, cap=None, heads=None):
    """Run the GPU prefill and compare with the oracle (on ``heads`` only if given)."""
    cache, table = make_cache(car, case, paged, cap)
    out = car.attn_prefill(case.q, case.k, case.v, case.positions, theta=case.theta,
                           scale=case.scale, cache=cache)
    torch.cuda.synchronize()
    pos = case.positions.cpu().numpy()
    tol = TOL[case.dtype]
    hq_list = range(case.Hq) if heads is None else heads
    group = case.Hq // case.Hkv
    hk_list = sorted({hq // group for hq in hq_list})
    worst = 0.0
    for b in range(case.B):
        q = f64(case.q[b:b + 1, list(hq_list)])
        k = f64(case.k[b:b + 1, hk_list])
        v = f64(case.v[b:b + 1, hk_list])
        # regroup: query heads hq read KV head hq // group, i.e. index hk_list.index(...)
        ref_out = np.empty(q.shape)
        for i, hq in enumerate(hq_list):
            j = hk_list.index(hq // group)
            o, _ = oracle.attn_prefill(q[:, i:i + 1], k[:, j:j + 1], v[:, j:j + 1],
                                       pos[b:b + 1], case.theta, case.scale)
            ref_out[:, i] = o[:, 0]
        got = f64(out[b:b + 1, list(hq_list)])
        worst = max(worst, max_abs(got, ref_out))
        if cache is not None:
            k_rot = oracle.rope_rotate(k, pos[b:b + 1][:, None, :], case.theta)
            for j, hk in enumerate(hk_list):
                if table is None:
                    gk = f64(cache.k[b, hk, pos[b]])
                    gv = cache.v[b, hk, torch.as_tensor(pos[b], device=DEV, dtype=torch.long)]
                else:
                    t = pos[b]
                    blk = torch.as_tensor(table[b, t // 16], device=DEV, dtype=torch.long)
                    off = torch.as_tensor(t % 16, device=DEV, dtype=torch.long)
                    gk = f64(cache.k[blk, hk, off])
                    gv = cache.v[blk, hk, off]
                worst = max(worst, max_abs(gk, k_rot[0, j]))
                assert torch.equal(bits(gv.cpu()), bits(case.v[b, hk].cpu())), "cached V"
    if cache is not None and heads is None:
        # nothing but the prompt's rows was written (the cache starts as NaN)
        for name, t in (("K", cache.k), ("V", cache.v)):
            rows = (~torch.isnan(t.float()).all(dim=-1)).sum().item()
            assert rows == case.B * case.Hkv * case.S, f"cache {name}: {rows} rows written"
    log_case(f"{case.name}: max-abs error {worst:.3e} (tol {tol})")
    assert worst <= tol
    return out, cache


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 2, 63, 130, 333])
def test_prefill_shapes(car, dtype, D, S):
    log_case(f"prefill {dtype} D={D} S={S}")
    case = W.prefill_case(f"prefill_S{S}", 2, 4, 4, S, D, dtype, 100 + S, DEV)
    check_prefill(car, case)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("group", [2, 4])
def test_prefill_gqa(car, dtype, group):
    log_case(f"prefill gqa group={group} {dtype}")
    case = W.prefill_case("gqa", 1, 8, 8 // group, 200, 128, dtype, 7 + group, DEV)
    check_prefill(car, case)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_prefill_writes_cache_at_offset_positions(car, dtype, paged):
    log_case(f"prefill into cache {dtype} paged={paged}")
    case = W.prefill_case("offset", 2, 4, 2, 150, 64, dtype, 55, DEV, pos_offset=9)
    check_prefill(car, case, paged=paged, cap=200)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_prefill_cache_at_gapped_positions(car, D, paged):
    """Strictly increasing positions with gaps (cache index = position, so
    the stored rows are scattered) beside consecutive ones in one batch:
    sequence 0 at slots 17..316 (its rotated keys are read back from the
    cache), sequences 1 and 2 with different gaps (read from the dense
    copy); GQA, two query tiles with a ragged tail."""
    log_case(f"prefill bf16 into cache at gapped positions D={D} paged={paged}")
    S, cap = 300, 1000
    case = W.prefill_case("gapped", 3, 8, 2, S, D, torch.bfloat16, 91 + D, DEV)
    rng = np.random.default_rng(D)
    pos = np.stack([np.arange(S) + 17] +
                   [np.sort(rng.choice(cap, S, replace=False)) for _ in range(2)])
    case.positions = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    check_prefill(car, case, paged=paged, cap=cap)


def low_first_keys(q, k, v, n_low):
    """Make keys 0..n_low-1 score about 1152/sqrt(D) below the others (over
    140 in log2 units at D <= 128) against every query while the other keys
    score O(1): queries hold 12 in their last 8 dims, the first keys -12
    there and the others 0 (RoPE turns those dims by under 0.1 rad over
    these positions), and the first keys' values are 0.  Exponentials of the
    later keys against the first keys' maximum would overflow fp32, yet
    every output is well conditioned: rows that see only the first keys
    average zeros exactly."""
    q[..., -8:] = 12.0
    k[:, :, :n_low, -8:] = -12.0
    k[:, :, n_low:, -8:] = 0.0
    v[:, :, :n_low] = 0.0


@pytest.mark.parametrize("form,D", [("split", 64), ("split", 128), ("paired", 128)])
def test_prefill_scores_jump_after_first_keys(car, form, D):
    """The first 128 keys score far below the rest (see low_first_keys), so
    the online softmax must raise its running maximum and rescale when the
    later tiles arrive; P against the low reference would overflow.  The
    paired form needs enough heads (256, 3 checked)."""
    log_case(f"prefill bf16 score jump form={form} D={D}")
    H = 256 if form == "paired" else 4
    case = W.prefill_case("jump", 1, H, H, 600, D, torch.bfloat16, 71 + D, DEV)
    low_first_keys(case.q, case.k, case.v, 128)
    out, _ = check_prefill(car, case, heads=[0, 101, 255] if form == "paired" else None)
    assert torch.equal(out[:, :, :128], torch.zeros_like(out[:, :, :128]))


def test_prefill_many_tiles_bf16(car):
    """Many KV tiles and an odd number of 256-row query tiles (5) with enough
    heads (90, so 270 query-tile pairs) for the 8-wave paired form: two
    workgroups per head take a long and a short tile, the middle tile runs
    alone; 90 heads are not a multiple of the 8 XCDs, and pairs of query
    heads share a KV head."""
    log_case("prefill bf16 many tiles, odd query-tile count, 8-wave pairs")
    case = W.prefill_case("long", 1, 90, 45, 1100, 128, torch.bfloat16, 77, DEV)
    check_prefill(car, case, heads=[0, 45, 89])


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_paired_form_stores_values_gqa_gapped(car, D):
    """The paired form (2 x 64 query heads x 2 query-tile pairs) into a
    contiguous cache, where the attention kernel stores the values and the
    K pass only the keys: GQA (16 KV heads), sequence 0 at consecutive slots
    5..604 (keys read back from the cache), sequence 1 at sorted random
    positions whose last 20 lie past the cache (those rows are not stored).
    Every stored K and V row is checked, and no other row of the NaN-filled
    cache is written."""
    log_case(f"prefill paired form stores values, GQA, gapped positions D={D}")
    B, Hq, Hkv, S, cap = 2, 64, 16, 600, 1000
    case = W.prefill_case("paired_values", B, Hq, Hkv, S, D, torch.bfloat16, 4200 + D, DEV)
    rng = np.random.default_rng(4200 + D)
    p1 = np.concatenate([np.sort(rng.choice(cap, S - 20, replace=False)), cap + np.arange(20)])
    pos = np.stack([np.arange(S) + 5, p1]).astype(np.int32)
    case.positions = torch.from_numpy(pos).to(DEV)
    ck = torch.full((B, Hkv, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    cache = car.KVCache(ck, ck.clone())
    out = car.attn_prefill(case.q, case.k, case.v, case.positions, theta=case.theta,
                           scale=case.scale, cache=cache)
    torch.cuda.synchronize()
    worst = 0.0
    group = Hq // Hkv
    for b in range(B):
        for hq in (0, 37, 63):
            o, _ = oracle.attn_prefill(f64(case.q[b:b + 1, hq:hq + 1]),
                                       f64(case.k[b:b + 1, hq // group:hq // group + 1]),
                                       f64(case.v[b:b + 1, hq // group:hq // group + 1]),
                                       pos[b:b + 1], case.theta, case.scale)
            worst = max(worst, max_abs(f64(out[b:b + 1, hq:hq + 1]), o))
        valid = pos[b] < cap
        sel = torch.as_tensor(pos[b][valid], device=DEV, dtype=torch.long)
        k_rot = oracle.rope_rotate(f64(case.k[b:b + 1]), pos[b:b + 1][:, None, :], case.theta)
        worst = max(worst, max_abs(f64(cache.k[b][:, sel]), k_rot[0][:, valid]))
        assert torch.equal(bits(cache.v[b][:, sel].cpu()), bits(case.v[b][:, valid].cpu())), \
            "cached V"
    for name, t in (("K", cache.k), ("V", cache.v)):
        rows = (~torch.isnan(t.float()).all(dim=-1)).sum().item()
        assert rows == Hkv * (2 * S - 20), f"cache {name}: {rows} rows written"
    log_case(f"paired form values D={D}: max-abs error {worst:.3e}")
    assert worst <= TOL[torch.bfloat16]


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_short_prompt_split_form(car, D):
    """A prompt whose query-tile pairs would fill few compute units (B=3,
    H=8, S=700: 48 pairs) runs in the split form: one 128-row query tile per
    workgroup (6 per head, the last ragged), its key range split over two
    wave groups, rows of the second group that see none of its keys."""
    log_case(f"prefill bf16 short prompt, split form D={D}")
    case = W.prefill_case("short", 3, 8, 4, 700, D, torch.bfloat16, 13 + D, DEV)
    check_prefill(car, case)


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_head_count_not_multiple_of_8(car, D):
    """B*Hq = 6 (the head-to-XCD pinning needs a multiple of 8): the
    round-robin assignment, with GQA and an odd query-tile count (3)."""
    log_case(f"prefill bf16 6 heads D={D}")
    case = W.prefill_case("heads6", 1, 6, 3, 700, D, torch.bfloat16, 31 + D, DEV)
    check_prefill(car, case)


def test_prefill_empty_prompt_is_noop(car):
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    out = car.attn_prefill(q, q[:, :1], q[:, :1], torch.empty((1, 0), dtype=torch.int32,
                                                              device=DEV))
    assert out.shape == q.shape


def test_tiny_workload_prefill_fp32(car):
    """Workload 1's prefill: B=1, H=4, D=64, S=128, fp32, cache of 144 slots."""
    pre, _ = W.tiny(DEV)
    check_prefill(car, pre, cap=144)


def test_gpt2_workload_prefill(car):
    """Workload 2 at full size, every head: B=4, H=12, D=64, S=512, bf16."""
    check_prefill(car, W.gpt2_prefill(DEV))


def test_qwen_workload_prefill_every_head(car):
    """Workload 3 at full size (B=1, H=32, D=128, S=4096, cache 4096), in the
    launch configuration the benchmark times: every head against the oracle
    (one head at a time), every cached row checked, and no other row of the
    NaN-filled cache written."""
    check_prefill(car, W.qwen_prefill(DEV), cap=4096)


def check_varlen(car, B, Hq, Hkv, S, D, dtype, lens, offsets, cache_kind, cap, seed):
    """A padded batch of prompts: prompt b is its first lens[b] rows at
    positions offsets[b] + 0.., the padding rows hold NaN (q, k, v) and
    position -7.  Rows of each prompt match the oracle, padding rows are
    exactly zero, and only prompt tokens reach the NaN-filled cache."""
    case = W.prefill_case("varlen", B, Hq, Hkv, S, D, dtype, seed, DEV)
    pos = torch.full((B, S), -7, dtype=torch.int32)
    for b, n in enumerate(lens):
        pos[b, :n] = torch.arange(n, dtype=torch.int32) + offsets[b]
        case.q[b, :, n:] = float("nan")
        case.k[b, :, n:] = float("nan")
        case.v[b, :, n:] = float("nan")
    pos = pos.to(DEV)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    cache, table = (None, None) if cache_kind == "none" else \
        make_cache(car, case, cache_kind == "paged", cap)
    out = car.attn_prefill(case.q, case.k, case.v, pos, theta=case.theta, scale=case.scale,
                           cache=cache, seq_lens=seq_lens)
    torch.cuda.synchronize()
    want, k_rot = oracle.attn_prefill(f64(case.q), f64(case.k), f64(case.v), pos.cpu().numpy(),
                                      case.theta, case.scale, seq_lens=np.array(lens))
    got = f64(out)
    tol = TOL[dtype]
    err = 0.0
    for b, n in enumerate(lens):
        err = max(err, max_abs(got[b, :, :n], want[b, :, :n]))
        assert torch.equal(out[b, :, n:].float().cpu(), torch.zeros_like(out[b, :, n:].float().cpu())), \
            f"padding rows of sequence {b} are not zero"
    if cache is not None:
        for b, n in enumerate(lens):
            for s in range(n):
                t = offsets[b] + s
                if table is None:
                    gk, gv = cache.k[b, :, t], cache.v[b, :, t]
                else:
                    gk, gv = cache.k[int(table[b, t // 16]), :, t % 16], \
                        cache.v[int(table[b, t // 16]), :, t % 16]
                err = max(err, max_abs(f64(gk), k_rot[b, :, s]))
                assert torch.equal(bits(gv.cpu()), bits(case.v[b, :, s].cpu())), "cached V"
        written = sum(lens) * Hkv
        for name, t in (("K", cache.k), ("V", cache.v)):
            rows = (~torch.isnan(t.float()).all(dim=-1)).sum().item()
            assert rows == written, f"cache {name}: {rows} rows written, expected {written}"
    log_case(f"varlen prefill {cache_kind} {dtype} D={D} lens={lens}: max-abs error {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("cache_kind", ["none", "contiguous", "paged"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_varlen(car, cache_kind, dtype, D):
    """Lengths 333 (full), 0, 1, 130 and 64 padded to S = 333, GQA 4/2;
    prompt 4 starts at position 100 (its keys then sit at consecutive cache
    slots 100..163)."""
    log_case(f"prefill varlen {cache_kind} {dtype} D={D}")
    check_varlen(car, 5, 4, 2, 333, D, dtype, [333, 0, 1, 130, 64], [0, 0, 5, 2, 100],
                 cache_kind, 448, 900 + D)


@pytest.mark.parametrize("cache_kind", ["none", "contiguous"])
def test_prefill_varlen_paired_form(car, cache_kind):
    """Enough query-tile pairs (4 x 32 heads x 2) for the 8-wave paired form:
    lengths 1024, 700, 1 and 513 padded to 1024, 32 query heads on 8 KV heads,
    bf16, D = 128."""
    log_case(f"prefill varlen paired form {cache_kind}")
    check_varlen(car, 4, 32, 8, 1024, 128, torch.bfloat16, [1024, 700, 1, 513], [0, 0, 0, 0],
                 cache_kind, 1024, 950)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("varlen", [False, True], ids=["full", "varlen"])
def test_prefill_without_workspace(car, D, varlen):
    """bf16 into a contiguous cache with no workspace: the rotated keys are
    read back from the cache.  Prompts start at positions 7, 0 and 30 (each
    consecutive); with varlen their lengths are 200, 1 and 77 of S = 200."""
    log_case(f"prefill without workspace D={D} varlen={varlen}")
    B, H, S, cap = 3, 4, 200, 240
    assert car._lib.car_attn_prefill_workspace_bytes(1, B, 2, S, D, None) > 0
    case = W.prefill_case("nows", B, H, 2, S, D, torch.bfloat16, 990 + D, DEV)
    offs = [7, 0, 30]
    lens = [200, 1, 77] if varlen else [S] * B
    pos = torch.stack([torch.arange(S, dtype=torch.int32) + o for o in offs]).to(DEV)
    ck = torch.full((B, 2, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    cache = car.KVCache(ck, ck.clone())
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV) if varlen else None
    out = car.attn_prefill(case.q, case.k, case.v, pos, theta=case.theta, scale=case.scale,
                           cache=cache, seq_lens=sl, no_workspace=True)
    torch.cuda.synchronize()
    want, k_rot = oracle.attn_prefill(f64(case.q), f64(case.k), f64(case.v), pos.cpu().numpy(),
                                      case.theta, case.scale, seq_lens=np.array(lens))
    err = 0.0
    for b, n in enumerate(lens):
        err = max(err, max_abs(f64(out[b, :, :n]), want[b, :, :n]))
        assert not out[b, :, n:].float().any()
        err = max(err, max_abs(f64(cache.k[b, :, offs[b]:offs[b] + n]), k_rot[b, :, :n]))
        assert torch.equal(bits(cache.v[b, :, offs[b]:offs[b] + n].cpu()),
                           bits(case.v[b, :, :n].cpu()))
    rows = (~torch.isnan(cache.k.float()).all(dim=-1)).sum().item()
    assert rows == 2 * sum(lens)
    log_case(f"max-abs error {err:.3e}")
    assert err <= TOL[torch.bfloat16]


def test_prefill_without_workspace_gapped_positions_stay_in_bounds(car):
    """Without a workspace, positions that are not consecutive slots give an
    unspecified output, but the cache store is still exact and nothing
    outside the prompt's rows is written."""
    log_case("prefill without workspace, gapped positions")
    B, H, S, D, cap = 2, 2, 40, 64, 100
    case = W.prefill_case("nows_gap", B, H, H, S, D, torch.bfloat16, 996, DEV)
    pos = (torch.arange(S, dtype=torch.int32) * 2 + 3).repeat(B, 1).to(DEV)  # 3, 5, .., 81
    ck = torch.full((B, H, cap, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    cache = car.KVCache(ck, ck.clone())
    car.attn_prefill(case.q, case.k, case.v, pos, theta=case.theta, scale=case.scale,
                     cache=cache, no_workspace=True)
    torch.cuda.synchronize()
    _, k_rot = oracle.attn_prefill(f64(case.q), f64(case.k), f64(case.v), pos.cpu().numpy(),
                                   case.theta, case.scale)
    p = pos[0].long()
    assert max_abs(f64(cache.k[:, :, p]), k_rot) <= TOL[torch.bfloat16]
    assert torch.equal(bits(cache.v[:, :, p].cpu()), bits(case.v.cpu()))
    rows = (~torch.isnan(cache.k.float()).all(dim=-1)).sum().item()
    assert rows == B * H * S
