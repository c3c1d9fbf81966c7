"""GPU parity: attn_decode against the oracle (RoPE at position L, append at
index L, attention over indices 0..L) for contiguous and paged caches, GQA
groups, lengths around the 256- and 1024-token split boundaries, L = 0, NaN canaries in
every slot that must not be read; workload 1's 16 decode steps after its
prefill; workloads 4 and 5 at full size on every sequence, and workload 4's
shape with a sequence at the cache's last slot."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import TOL, bits, decode_inputs_for, f64, log_case, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def car():
    import causal_attention_rope_amd as m
    return m


def run_and_check(car, case, bsel=None):
    """GPU decode step on the whole case; oracle on sequences ``bsel``."""
    bsel = list(range(case.B)) if bsel is None else list(bsel)
    q, kn, vn, ck, cv, lens, table = decode_inputs_for(case, bsel)
    cache = car.KVCache(case.cache_k, case.cache_v, case.block_table)
    out = car.attn_decode(case.q, case.k_new, case.v_new, case.seq_lens, cache,
                          case.max_seq_len, theta=case.theta, scale=case.scale)
    torch.cuda.synchronize()
    want = oracle.attn_decode(q, kn, vn, ck, cv, lens, case.theta, case.scale,
                              block_table=table)
    tol = TOL[case.dtype]
    err = max_abs(f64(out[bsel]), want)
    # the appended row: rotated k_new and raw v_new at index L
    for i, b in enumerate(bsel):
        L = case.lens_host[b]
        if case.paged:
            blk = int(case.block_table[b, L // 16])
            gk, gv = case.cache_k[blk, :, L % 16], case.cache_v[blk, :, L % 16]
            wk = ck[table[i, L // 16], :, L % 16]
        else:
            gk, gv = case.cache_k[b, :, L], case.cache_v[b, :, L]
            wk = ck[i, :, L]
        err = max(err, max_abs(f64(gk), wk))
        assert torch.equal(bits(gv.cpu()), bits(case.v_new[b].cpu())), "appended V"
    assert torch.isfinite(out.float()).all()
    log_case(f"{case.name}: max-abs error {err:.3e} (tol {tol})")
    assert err <= tol
    return out


LENS = [0, 1, 5, 255, 256, 257, 511, 700]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_decode_lengths(car, dtype, D, paged):
    log_case(f"decode lengths {dtype} D={D} paged={paged}")
    case = W.decode_case("lens", len(LENS), 4, 4, D, dtype, LENS, 300 + D, DEV, paged=paged,
                         poison_unused=True, extra_blocks=3)
    run_and_check(car, case)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_decode_gqa_groups(car, dtype, group, paged):
    """Groups above 1 run 1024-token splits over 8 waves of 128 tokens:
    lengths on both sides of the wave boundaries 128 and 512 and of the split
    boundaries 1024 and 2048, and one inside the first wave."""
    log_case(f"decode gqa group={group} {dtype} paged={paged}")
    lens = [3, 127, 128, 290, 511, 512, 1023, 1024, 1025, 2047, 2048, 2049]
    case = W.decode_case("gqa", len(lens), 8, 8 // group, 128, dtype, lens, 400 + group, DEV,
                         paged=paged, poison_unused=True, extra_blocks=2)
    run_and_check(car, case)


@pytest.mark.parametrize("group", [2, 4, 8])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_decode_gqa_lengths_d64(car, group, paged):
    """D = 64 with groups (8-row load steps, 1024-token splits, rows streamed
    through the per-wave LDS ring): lengths inside the first rounds, at the
    wave and split edges."""
    log_case(f"decode gqa D=64 group={group} paged={paged}")
    lens = [0, 1, 7, 8, 17, 127, 255, 511, 700, 1023, 1024, 1025]
    case = W.decode_case("gqa64", len(lens), 8, 8 // group, 64, torch.bfloat16, lens,
                         450 + group, DEV, paged=paged, poison_unused=True, extra_blocks=2)
    run_and_check(car, case)


def test_decode_gqa_equals_repeated_mha(car):
    """GQA on the GPU equals MHA with each KV head repeated (contiguous groups)."""
    lens = [40, 300]
    g = W.decode_case("g", 2, 8, 2, 128, torch.bfloat16, lens, 9, DEV, paged=False)
    kk = g.cache_k.repeat_interleave(4, dim=1).contiguous()
    vv = g.cache_v.repeat_interleave(4, dim=1).contiguous()
    kn = g.k_new.repeat_interleave(4, dim=1).contiguous()
    vn = g.v_new.repeat_interleave(4, dim=1).contiguous()
    out_g = car.attn_decode(g.q, g.k_new, g.v_new, g.seq_lens, car.KVCache(g.cache_k, g.cache_v),
                            g.max_seq_len)
    out_m = car.attn_decode(g.q, kn, vn, g.seq_lens, car.KVCache(kk, vv), g.max_seq_len)
    torch.cuda.synchronize()
    # different split passes per group size may flip a bf16 rounding
    assert max_abs(f64(out_g), f64(out_m)) <= 1e-2


def test_decode_paged_equals_contiguous(car):
    lens = [17, 511, 900]
    c = W.decode_case("c", 3, 4, 4, 128, torch.bfloat16, lens, 12, DEV, paged=False)
    cap = c.cache_k.shape[2]
    mbps = (cap + 15) // 16
    perm = np.random.default_rng(5).permutation(3 * mbps + 4)[: 3 * mbps].reshape(3, mbps)
    nb = 3 * mbps + 4
    pk = torch.full((nb, 4, 16, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    pv = pk.clone()
    for b in range(3):
        for j in range(mbps):
            n = min(16, cap - 16 * j)
            pk[perm[b, j], :, :n] = c.cache_k[b, :, 16 * j:16 * j + n]
            pv[perm[b, j], :, :n] = c.cache_v[b, :, 16 * j:16 * j + n]
    table = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    out_c = car.attn_decode(c.q, c.k_new, c.v_new, c.seq_lens, car.KVCache(c.cache_k, c.cache_v),
                            c.max_seq_len)
    out_p = car.attn_decode(c.q, c.k_new, c.v_new, c.seq_lens, car.KVCache(pk, pv, table),
                            c.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(bits(out_c.cpu()), bits(out_p.cpu()))


def test_tiny_workload_prefill_then_16_decode_steps(car):
    """Workload 1: fp32 prefill of 128 tokens into a 144-slot cache, then 16
    decode steps at positions 128..143, each against the oracle at 1e-4."""
    pre, steps = W.tiny(DEV)
    ck = torch.full((1, 4, 144, 64), float("nan"), dtype=torch.float32, device=DEV)
    cache = car.KVCache(ck, ck.clone())
    car.attn_prefill(pre.q, pre.k, pre.v, pre.positions, cache=cache)
    # oracle state: its own cache, filled by its own prefill
    ok = np.full((1, 4, 144, 64), np.nan)
    ov = np.full((1, 4, 144, 64), np.nan)
    _, k_rot = oracle.attn_prefill(f64(pre.q), f64(pre.k), f64(pre.v),
                                   pre.positions.cpu().numpy())
    oracle.kv_cache_append(ok, ov, k_rot, f64(pre.v), pre.positions.cpu().numpy())
    worst = 0.0
    for t, (q, kn, vn) in enumerate(steps):
        L = 128 + t
        lens = torch.tensor([L], dtype=torch.int32, device=DEV)
        out = car.attn_decode(q, kn, vn, lens, cache, L + 1)
        torch.cuda.synchronize()
        want = oracle.attn_decode(f64(q), f64(kn), f64(vn), ok, ov, np.array([L]))
        worst = max(worst, max_abs(f64(out), want))
    worst = max(worst, max_abs(f64(cache.k), ok), max_abs(f64(cache.v), ov))
    log_case(f"tiny prefill + 16 decode steps: max-abs error {worst:.3e}")
    assert worst <= 1e-4


def check_every_sequence(car, case):
    """One GPU decode step over the whole case, then the oracle sequence by
    sequence (bounded host memory).  The inputs of sequence b are gathered
    after the step, so its slot L holds the GPU's appended row; the oracle
    writes its own row there before attending, and the GPU's row is compared
    with it."""
    cache = car.KVCache(case.cache_k, case.cache_v, case.block_table)
    out = car.attn_decode(case.q, case.k_new, case.v_new, case.seq_lens, cache,
                          case.max_seq_len, theta=case.theta, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    worst = 0.0
    for b in range(case.B):
        q, kn, vn, ck, cv, lens, table = decode_inputs_for(case, [b])
        want = oracle.attn_decode(q, kn, vn, ck, cv, lens, case.theta, case.scale,
                                  block_table=table)
        worst = max(worst, max_abs(f64(out[b:b + 1]), want))
        L = int(lens[0])
        if case.paged:
            blk = int(case.block_table[b, L // 16])
            gk, gv = case.cache_k[blk, :, L % 16], case.cache_v[blk, :, L % 16]
            wk = ck[table[0, L // 16], :, L % 16]
        else:
            gk, gv = case.cache_k[b, :, L], case.cache_v[b, :, L]
            wk = ck[0, :, L]
        worst = max(worst, max_abs(f64(gk), wk))
        assert torch.equal(bits(gv.cpu()), bits(case.v_new[b].cpu())), f"appended V, b={b}"
    tol = TOL[case.dtype]
    log_case(f"{case.name}: every sequence, max-abs error {worst:.3e} (tol {tol})")
    assert worst <= tol


def test_contiguous_decode_workload(car):
    """Workload 4 at full size (B=32, H=32, D=128, cache [32,32,4096,128]) in
    the launch configuration the benchmark times; every sequence against the
    oracle."""
    check_every_sequence(car, W.contiguous_decode(DEV))


def test_contiguous_decode_last_slot(car):
    """Workload 4's shape with sequence 5 at L = 4095: the new token goes to
    the cache's last slot and the query attends over all 4096 slots."""
    lens = list(W.contiguous_decode_lens())
    lens[5] = 4095
    case = W.decode_case("contiguous_last_slot", 32, 32, 32, 128, torch.bfloat16, lens,
                         W.BASE_SEED + 40, DEV, paged=False, max_seq=4096)
    assert case.max_seq_len == 4096
    run_and_check(car, case, [0, 5, 31])


def test_paged_decode_workload(car):
    """Workload 5 at full size (B=64, Hq=32, Hkv=8, 16-token blocks, lengths
    in [512, 8192]); every sequence against the oracle."""
    check_every_sequence(car, W.paged_decode(DEV))


def test_paged_decode_workload_poisoned(car):
    """Workload 5 with NaN in every slot and block the step must not read."""
    case = W.paged_decode(DEV, poison_unused=True)
    run_and_check(car, case, [0, 33])
