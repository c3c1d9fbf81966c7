"""GPU parity for the INT8 KV cache: calibration of per-(KV head, channel)
scales, quantizing stores (standalone append and the prefill's cache store)
and decode over an int8 cache, against the oracle in ``oracle/int8_cache.py``.

Exactness.  Scales of values and codes of values that the kernels do not
transform (values, already-rotated keys) are decided in fp32 on both sides
and compared bit-exactly.  Keys rotated inside a kernel differ from the
oracle's float64 rotation by ~1e-7 relative, so a key whose quotient x / s
lies within 5e-5 of a rounding tie may round either way: such codes are
allowed to differ by one, every other code must match, and key scales match
to 2e-6 relative.  Decode outputs use the usual tolerances (fp32 1e-4, bf16
2e-2).  The fp32 cases draw new keys (by seed) whose codes are not
ambiguous, so the 1e-4 bound holds without a flipped code; in bf16 one
flipped code moves an output by well under the bound.

Slots a decode must not read hold "poison" codes: every channel +-127 with
the sign that makes the score of the group's first query head as large as it
can be, and values of 127, so that a read past index L would dominate that
head's softmax.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import TOL, f64, log_case, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TIE_MARGIN = 5e-5


@pytest.fixture(scope="module")
def car():
    import causal_attention_rope_amd as m
    return m


def np_i8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int8)


def quotient(x, s):
    """The oracle's fp32 quotient x / s (the rounding decision's input)."""
    x32 = np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    s32 = np.broadcast_to(np.asarray(s, np.float32).astype(np.float64), x32.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        return (x32 / s32).astype(np.float32).astype(np.float64)


def ambiguous(x, s):
    """Elements whose quotient is within TIE_MARGIN of a rounding tie."""
    q = np.abs(quotient(x, s))
    return (np.abs(q - np.floor(q) - 0.5) < TIE_MARGIN) & (q < 127.5)


def check_key_codes(got, want, x_rot, s):
    """Codes of kernel-rotated keys: equal, or one apart where ambiguous."""
    got = got.astype(np.int64)
    want = want.astype(np.int64)
    diff = np.abs(got - want)
    amb = ambiguous(x_rot, s)
    assert diff.max(initial=0) <= 1
    assert not np.any((diff == 1) & ~amb), "a key code differs away from a rounding tie"
    return int((diff == 1).sum())


# ==========================================================================
# Calibration
# ==========================================================================

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("pairing", ["adjacent", "half"])
def test_calibrate_matches_oracle(car, dtype, D, pairing):
    B, Hkv, S = 3, 4, 77
    log_case(f"calibrate {dtype} D={D} {pairing}")
    k = W.randn((B, Hkv, S, D), dtype, DEV, 31, 1)
    v = W.randn((B, Hkv, S, D), dtype, DEV, 31, 2)
    pos = (torch.arange(S, dtype=torch.int32)[None, :] + 1000 * torch.arange(B)[:, None]
           ).to(torch.int32).to(DEV).contiguous()
    ks, vs = car.kv_int8_calibrate(k, v, pos, rope_pairing=pairing)
    torch.cuda.synchronize()
    wk, wv = oracle.int8_calibrate(f64(k), f64(v), pos.cpu().numpy(), pairing=pairing)
    assert np.array_equal(vs.cpu().numpy(), wv), "value scales are bit-exact"
    rel = np.abs(ks.cpu().numpy().astype(np.float64) - wk) / wk
    log_case(f"  key scales max rel diff {rel.max():.2e}")
    assert rel.max() <= 2e-6


def test_calibrate_empty_batch_writes_zeros(car):
    k = torch.zeros((0, 2, 5, 64), dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros((0, 5), dtype=torch.int32, device=DEV)
    ks, vs = car.kv_int8_calibrate(k, k.clone(), pos)
    torch.cuda.synchronize()
    assert ks.shape == (2, 64) and torch.all(ks == 0) and torch.all(vs == 0)


# ==========================================================================
# Quantizing stores
# ==========================================================================

def _scales_with_edges(Hkv, D, seed):
    """Scales where some values saturate (small scales) and one channel is 0."""
    ks = W.randscales((Hkv, D), DEV, seed, 8)
    vs = W.randscales((Hkv, D), DEV, seed, 9)
    ks[0, 3] = 0.0
    vs[1 % Hkv, 5] = 0.0
    ks[:, :4] *= 0.1    # |x| / s beyond 127 for many values: saturation
    return ks.contiguous(), vs.contiguous()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_append_codes_bit_exact(car, dtype, D, paged):
    """Already-rotated keys and values: every code, and every untouched slot,
    equals the oracle's store into the same initial cache."""
    B, Hkv, S = 3, 2, 37
    log_case(f"int8 append {dtype} D={D} paged={paged}")
    k = W.randn((B, Hkv, S, D), dtype, DEV, 41, 1) * 2
    v = W.randn((B, Hkv, S, D), dtype, DEV, 41, 2)
    ks, vs = _scales_with_edges(Hkv, D, 41)
    rng = W.host_rng(41)
    if paged:
        mbps, nb = 5, 3 * 5 + 2
        table = rng.permutation(nb)[: B * mbps].reshape(B, mbps).astype(np.int32)
        shape = (nb, Hkv, 16, D)
        bt = torch.from_numpy(table).to(DEV)
    else:
        table, bt = None, None
        shape = (B, Hkv, 80, D)
    pos = np.stack([rng.permutation(80)[:S] for _ in range(B)]).astype(np.int32)
    ck = torch.full(shape, 77, dtype=torch.int8, device=DEV)
    cv = torch.full(shape, -77, dtype=torch.int8, device=DEV)
    cache = car.KVCache(ck, cv, bt, k_scale=ks, v_scale=vs)
    car.kv_cache_append(cache, k, v, torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    wk = np.full(shape, 77, np.int8)
    wv = np.full(shape, -77, np.int8)
    oracle.kv_cache_append_int8(wk, wv, f64(k), f64(v), pos, ks.cpu().numpy(),
                                vs.cpu().numpy(), block_table=table)
    assert np.array_equal(np_i8(ck), wk)
    assert np.array_equal(np_i8(cv), wv)
    assert np.any(np.abs(wk) == 127), "the case exercises saturation"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("pairing", ["adjacent", "half"])
def test_prefill_int8_store(car, dtype, paged, pairing):
    """The prompt's attention does not depend on the cache format (outputs
    bit-identical to a prefill into a native cache); the stored codes are
    those of the oracle's rotated keys and raw values."""
    B, Hq, Hkv, S, D = 2, 8, 2, 150, 128
    log_case(f"int8 prefill store {dtype} paged={paged} {pairing}")
    pre = W.prefill_case("i8pre", B, Hq, Hkv, S, D, dtype, 51, DEV)
    posn = pre.positions.cpu().numpy()
    wks, wvs = oracle.int8_calibrate(f64(pre.k), f64(pre.v), posn, pairing=pairing)
    ks = torch.from_numpy(wks).to(DEV)
    vs = torch.from_numpy(wvs).to(DEV)
    if paged:
        mbps, nb = 10, B * 10 + 3
        table = W.host_rng(51).permutation(nb)[: B * mbps].reshape(B, mbps).astype(np.int32)
        bt = torch.from_numpy(table).to(DEV)
        shape = (nb, Hkv, 16, D)
    else:
        table, bt = None, None
        shape = (B, Hkv, 160, D)
    ck = torch.zeros(shape, dtype=torch.int8, device=DEV)
    cv = torch.zeros(shape, dtype=torch.int8, device=DEV)
    nk = torch.zeros(shape, dtype=dtype, device=DEV)
    out8 = car.attn_prefill(pre.q, pre.k, pre.v, pre.positions, rope_pairing=pairing,
                            cache=car.KVCache(ck, cv, bt, k_scale=ks, v_scale=vs))
    outn = car.attn_prefill(pre.q, pre.k, pre.v, pre.positions, rope_pairing=pairing,
                            cache=car.KVCache(nk, nk.clone(), bt))
    torch.cuda.synchronize()
    assert torch.equal(out8, outn)
    _, k_rot = oracle.attn_prefill(f64(pre.q), f64(pre.k), f64(pre.v), posn, pairing=pairing)
    wk = np.zeros(shape, np.int8)
    wv = np.zeros(shape, np.int8)
    oracle.kv_cache_append_int8(wk, wv, k_rot, f64(pre.v), posn, wks, wvs, block_table=table)
    assert np.array_equal(np_i8(cv), wv)
    # the rotated values each stored code came from, at the same slots
    xs = np.zeros(shape)
    ss = np.ones(shape, np.float32)
    for b in range(B):
        for s in range(S):
            t = int(posn[b, s])
            if table is None:
                xs[b, :, t], ss[b, :, t] = k_rot[b, :, s], wks
            else:
                blk, off = table[b, t // 16], t % 16
                xs[blk, :, off], ss[blk, :, off] = k_rot[b, :, s], wks
    flips = check_key_codes(np_i8(ck), wk, xs, ss)
    log_case(f"  key codes one apart at ties: {flips}")


# ==========================================================================
# Decode over an int8 cache
# ==========================================================================

def poison_unread(case):
    """Codes no decode step may read: past index L (contiguous) or in slots
    and blocks no sequence owns at 0..L (paged)."""
    G = case.Hq // case.Hkv
    ks = case.k_scale.cpu().numpy()
    qh = f64(case.q)
    for b, L in enumerate(case.lens_host):
        for hk in range(case.Hkv):
            qr = oracle.rope_rotate(qh[b, hk * G][None, :], np.array([L]))[0]
            sign = np.where(qr * ks[hk] >= 0, 127, -127).astype(np.int8)
            kp = torch.from_numpy(sign).to(DEV)
            if not case.paged:
                case.cache_k[b, hk, L + 1:] = kp
                case.cache_v[b, hk, L + 1:] = 127
    if case.paged:
        table = case.block_table.cpu().numpy()
        keep = np.zeros(case.cache_k.shape[0] * 16, bool)
        for b, L in enumerate(case.lens_host):
            t = np.arange(L + 1)
            keep[table[b, t // 16] * 16 + t % 16] = True
        far = torch.from_numpy(~keep.reshape(-1, 16)).to(DEV)[:, None, :, None]
        case.cache_k.masked_fill_(far, 127)
        case.cache_v.masked_fill_(far, 127)


def inputs_for(case, bsel):
    """Oracle inputs for sequences ``bsel`` (taken before the GPU step)."""
    bsel = list(bsel)
    q, kn, vn = f64(case.q[bsel]), f64(case.k_new[bsel]), f64(case.v_new[bsel])
    lens = np.array([case.lens_host[b] for b in bsel])
    if not case.paged:
        n = int(lens.max()) + 1
        return (q, kn, vn, np_i8(case.cache_k[bsel][:, :, :n]),
                np_i8(case.cache_v[bsel][:, :, :n]), lens, None)
    table = case.block_table.cpu().numpy()[bsel]
    used = np.unique(table)
    remap = {int(blk): i for i, blk in enumerate(used)}
    idx = torch.as_tensor(used, device=DEV, dtype=torch.int64)
    return (q, kn, vn, np_i8(case.cache_k.index_select(0, idx)),
            np_i8(case.cache_v.index_select(0, idx)), lens,
            np.vectorize(lambda x: remap[int(x)])(table))


def new_key_quotients(case):
    """Rotated new keys over their scales, [B, Hkv, D] (the oracle's view)."""
    kn = f64(case.k_new)
    ks = case.k_scale.cpu().numpy()
    out = np.empty(kn.shape)
    for b, L in enumerate(case.lens_host):
        out[b] = oracle.rope_rotate(kn[b][:, None, :], np.array([L]))[:, 0, :]
    return out, ks[None]


def make_case(name, B, Hq, Hkv, D, dtype, lens, seed, paged, **kw):
    """An INT8 decode case; fp32 cases skip seeds whose new keys sit on a tie."""
    for s in range(seed, seed + 64):
        case = W.int8_decode_case(name, B, Hq, Hkv, D, dtype, lens, s, DEV, paged=paged, **kw)
        if dtype != torch.float32:
            return case
        x, ks = new_key_quotients(case)
        if not ambiguous(x, ks).any():
            return case
    raise AssertionError("no fp32 case without a tie in 64 seeds")


def run_and_check(car, case, bsel=None, poison=True):
    bsel = list(range(case.B)) if bsel is None else list(bsel)
    if poison:
        poison_unread(case)
    q, kn, vn, ck, cv, lens, table = inputs_for(case, bsel)
    ks, vs = case.k_scale.cpu().numpy(), case.v_scale.cpu().numpy()
    cache = car.KVCache(case.cache_k, case.cache_v, case.block_table,
                        k_scale=case.k_scale, v_scale=case.v_scale)
    out = car.attn_decode(case.q, case.k_new, case.v_new, case.seq_lens, cache,
                          case.max_seq_len, theta=case.theta, scale=case.scale)
    torch.cuda.synchronize()
    want = oracle.attn_decode_int8(q, kn, vn, ck, cv, lens, ks, vs, case.theta, case.scale,
                                   block_table=table)
    err = max_abs(f64(out[bsel]), want)
    # the appended codes at index L: values exact, keys one apart at most at ties
    xk, _ = new_key_quotients(case)
    for i, b in enumerate(bsel):
        L = case.lens_host[b]
        if case.paged:
            blk = int(case.block_table[b, L // 16])
            gk, gv = case.cache_k[blk, :, L % 16], case.cache_v[blk, :, L % 16]
            wk, wv = ck[table[i, L // 16], :, L % 16], cv[table[i, L // 16], :, L % 16]
        else:
            gk, gv = case.cache_k[b, :, L], case.cache_v[b, :, L]
            wk, wv = ck[i, :, L], cv[i, :, L]
        assert np.array_equal(np_i8(gv), wv), "appended value codes"
        check_key_codes(np_i8(gk), wk, xk[b], ks)
    assert torch.isfinite(out.float()).all()
    tol = TOL[case.dtype]
    log_case(f"{case.name}: max-abs error {err:.3e} (tol {tol})")
    assert err <= tol
    return out


LENS = [0, 1, 5, 255, 256, 257, 511, 700]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_decode_int8_mha(car, dtype, D, paged):
    case = make_case(f"i8 mha {dtype} D={D} paged={paged}", len(LENS), 2 * 2, 2 * 2, D, dtype,
                     LENS, 61, paged, extra_blocks=3 if paged else 0)
    log_case(case.name)
    run_and_check(car, case)


# several query heads: 2048-token splits over 8 waves of 256 tokens; lengths
# at the wave and split edges
GQA_LENS = [0, 3, 127, 255, 256, 1023, 1024, 1025, 2047, 2048, 2049, 4097]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("group", [2, 4, 8])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_decode_int8_gqa(car, dtype, group, paged):
    Hkv = 2
    case = make_case(f"i8 gqa{group} {dtype} paged={paged}", len(GQA_LENS), Hkv * group, Hkv,
                     128, dtype, GQA_LENS, 71 + group, paged, extra_blocks=2 if paged else 0)
    log_case(case.name)
    run_and_check(car, case)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("group", [2, 4])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_decode_int8_gqa_new_token_every_row(car, D, group, paged):
    """bf16 with several query heads: L = 145 j puts the new token at row
    L % 16 = j of its 16-token block for j = 0..15, in different waves and
    splits, so each lane position of the block's loads is the one whose
    cached row is replaced by the token computed in the kernel."""
    lens = [145 * j for j in range(16)]
    Hkv = 2
    case = make_case(f"i8 gqa{group} every row D={D} paged={paged}", len(lens), Hkv * group, Hkv,
                     D, torch.bfloat16, lens, 91 + group, paged, extra_blocks=2 if paged else 0)
    log_case(case.name)
    run_and_check(car, case)


@pytest.mark.parametrize("group", [4, 8])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_decode_int8_gqa_scores_jump(car, group, paged):
    """Cached keys from index J = L // 3 on score far above the earlier ones
    (queries 3 in their last 8 dims, those keys' codes +127 there and the
    earlier keys' -127: over 20 in log2 units at these scales), so the
    running maximum of the waves and splits that cross J moves by far more
    than the lazy-rescale threshold in a later block, and O and l must be
    rescaled together."""
    lens = [700, 1500, 2900]
    Hkv = 2
    case = make_case(f"i8 gqa{group} jump paged={paged}", len(lens), Hkv * group, Hkv, 128,
                     torch.bfloat16, lens, 75 + group, paged, extra_blocks=2 if paged else 0)
    case.q[..., -8:] = 3.0
    for b, L in enumerate(lens):
        t = torch.arange(L, device=DEV)
        code = torch.where(t < L // 3, -127, 127).to(torch.int8)[:, None, None]
        if paged:
            blk = case.block_table[b].to(torch.long)[t // 16]
            case.cache_k[blk, :, t % 16, -8:] = code.expand(L, Hkv, 8)
        else:
            case.cache_k[b, :, :L, -8:] = code.expand(L, 1, 8).transpose(0, 1)
    log_case(case.name)
    run_and_check(car, case)


@pytest.mark.parametrize("pairing", ["half"])
def test_decode_int8_half_split(car, pairing):
    """The half-split RoPE layout through the int8 decode (bf16, GQA 4)."""
    lens = [0, 9, 300, 1500]
    case = W.int8_decode_case("i8 half", len(lens), 8, 2, 128, torch.bfloat16, lens, 81, DEV,
                              paged=True)
    log_case(case.name)
    q, kn, vn, ck, cv, L, table = inputs_for(case, range(case.B))
    cache = car.KVCache(case.cache_k, case.cache_v, case.block_table,
                        k_scale=case.k_scale, v_scale=case.v_scale)
    out = car.attn_decode(case.q, case.k_new, case.v_new, case.seq_lens, cache,
                          case.max_seq_len, rope_pairing=pairing)
    torch.cuda.synchronize()
    want = oracle.attn_decode_int8(q, kn, vn, ck, cv, L, case.k_scale.cpu().numpy(),
                                   case.v_scale.cpu().numpy(), block_table=table,
                                   pairing=pairing)
    err = max_abs(f64(out), want)
    log_case(f"  max-abs error {err:.3e}")
    assert err <= TOL[torch.bfloat16]


def test_decode_int8_after_prefill_store(car):
    """A bf16 prompt stored into an int8 cache by the prefill, then decode
    steps over it: the whole path against the oracle's INT8 cache."""
    B, Hq, Hkv, S, D = 2, 8, 2, 200, 128
    pre = W.prefill_case("i8 chain", B, Hq, Hkv, S, D, torch.bfloat16, 91, DEV)
    posn = pre.positions.cpu().numpy()
    wks, wvs = oracle.int8_calibrate(f64(pre.k), f64(pre.v), posn)
    ks, vs = torch.from_numpy(wks).to(DEV), torch.from_numpy(wvs).to(DEV)
    cap = 208
    ck = torch.zeros((B, Hkv, cap, D), dtype=torch.int8, device=DEV)
    cv = torch.zeros_like(ck)
    cache = car.KVCache(ck, cv, k_scale=ks, v_scale=vs)
    car.attn_prefill(pre.q, pre.k, pre.v, pre.positions, cache=cache)
    _, k_rot = oracle.attn_prefill(f64(pre.q), f64(pre.k), f64(pre.v), posn)
    ok = np.zeros((B, Hkv, cap, D), np.int8)
    ov = np.zeros_like(ok)
    oracle.kv_cache_append_int8(ok, ov, k_rot, f64(pre.v), posn, wks, wvs)
    err = 0.0
    for t in range(4):
        q1 = W.randn((B, Hq, D), torch.bfloat16, DEV, 92 + t, 0)
        k1 = W.randn((B, Hkv, D), torch.bfloat16, DEV, 92 + t, 1)
        v1 = W.randn((B, Hkv, D), torch.bfloat16, DEV, 92 + t, 2)
        lens = torch.full((B,), S + t, dtype=torch.int32, device=DEV)
        out = car.attn_decode(q1, k1, v1, lens, cache, S + t + 1)
        torch.cuda.synchronize()
        want = oracle.attn_decode_int8(f64(q1), f64(k1), f64(v1), ok, ov, np.full(B, S + t),
                                       wks, wvs)
        err = max(err, max_abs(f64(out), want))
    log_case(f"i8 prefill+decode chain: max-abs error {err:.3e}")
    assert err <= TOL[torch.bfloat16]


# ==========================================================================
# The decode workloads at full size with INT8 caches (sampled sequences)
# ==========================================================================

def test_contiguous_decode_workload_int8(car):
    case = W.int8_decode_case("contiguous_decode int8", 32, 32, 32, 128, torch.bfloat16,
                              W.contiguous_decode_lens(), W.BASE_SEED + 3, DEV, paged=False,
                              max_seq=4096)
    log_case(case.name)
    order = np.argsort(case.lens_host)
    run_and_check(car, case, bsel=[int(order[0]), int(order[-1]), 7], poison=False)


def test_paged_decode_workload_int8(car):
    case = W.int8_decode_case("paged_decode int8", 64, 32, 8, 128, torch.bfloat16,
                              W.paged_decode_lens(), W.BASE_SEED + 4, DEV, paged=True,
                              blocks_per_seq=513)
    log_case(case.name)
    order = np.argsort(case.lens_host)
    run_and_check(car, case, bsel=[int(order[0]), int(order[-1])], poison=False)


# ==========================================================================
# A chunk continuing a prefix held in an INT8 cache
# ==========================================================================

def int8_chunk_inputs(B, Hq, Hkv, S, D, dtype, lens, n, seed, paged, cap, unambiguous=True):
    """Prefix codes, chunk q/k/v and per-(KV head, channel) scales.  With
    ``unambiguous`` the seed is advanced until no chunk key's quotient lies
    near a rounding tie, so the kernel's fp32 rotation stores exactly the
    oracle's codes."""
    for tries in range(64 if unambiguous else 1):
        s = seed + 1000 * tries
        q = W.randn((B, Hq, S, D), dtype, DEV, s, 0)
        k = W.randn((B, Hkv, S, D), dtype, DEV, s, 1)
        v = W.randn((B, Hkv, S, D), dtype, DEV, s, 2)
        ks = W.randscales((Hkv, D), DEV, s, 3)   # [0.01, 0.03]: values within +-3.81,
        vs = W.randscales((Hkv, D), DEV, s, 4)   # as in the decode tests
        kr = np.concatenate([oracle.rope_rotate(f64(k[b, :, :n[b]]), lens[b] + np.arange(n[b]))
                             for b in range(B)], axis=1)
        if not unambiguous or not ambiguous(kr, f64(ks)[:, None, :]).any():
            break
    else:
        raise AssertionError("no seed without an ambiguous key code")
    if paged:
        mbps = cap // 16
        nb = B * mbps + 3
        table = np.random.default_rng(seed).permutation(nb)[: B * mbps].reshape(B, mbps)
        table = table.astype(np.int32)
        shape = (nb, Hkv, 16, D)
    else:
        table = None
        shape = (B, Hkv, cap, D)
    ck = W.randcodes(shape, DEV, s, 5)
    cv = W.randcodes(shape, DEV, s, 6)
    return q, k, v, ks, vs, ck, cv, table


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_chunk_int8(car, dtype, D, paged):
    """A padded batch of chunks (lengths 70, 1, 33 of S = 70) after cached
    prefixes of 0, 37 and 100 tokens in an INT8 cache, 8 query heads on 2 KV
    heads: outputs against the oracle's INT8 chunk (padding rows zero), the
    chunk's codes stored exactly at P..P+n-1 and every other slot unchanged."""
    B, Hq, Hkv, S, cap = 3, 8, 2, 70, 176
    lens, n = [0, 37, 100], [70, 1, 33]
    log_case(f"int8 chunk {dtype} D={D} paged={paged}")
    q, k, v, ks, vs, ck, cv, table = int8_chunk_inputs(B, Hq, Hkv, S, D, dtype, lens, n,
                                                       700 + D, paged, cap)
    before_k, before_v = np_i8(ck), np_i8(cv)
    cache = car.KVCache(ck, cv, None if table is None else torch.from_numpy(table).to(DEV),
                        k_scale=ks, v_scale=vs)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    chunk_lens = torch.tensor(n, dtype=torch.int32, device=DEV)
    out = car.attn_prefill_cached(q, k, v, seq_lens, cache, max(l + m for l, m in zip(lens, n)),
                                  chunk_lens=chunk_lens)
    torch.cuda.synchronize()
    ok, ov = before_k.copy(), before_v.copy()
    want = oracle.attn_prefill_cached_int8(f64(q), f64(k), f64(v), ok, ov, np.array(lens),
                                           f64(ks), f64(vs), block_table=table,
                                           chunk_lens=np.array(n))
    err = max_abs(f64(out), want)
    log_case(f"max-abs error {err:.3e}")
    assert err <= TOL[dtype]
    for b in range(B):
        assert not out[b, :, n[b]:].float().any(), "padding rows"
    assert np.array_equal(np_i8(ck), ok), "key codes"
    assert np.array_equal(np_i8(cv), ov), "value codes"


def test_chunk_int8_long_prefix_bf16(car):
    """bf16 on the matrix cores over several key tiles: a 300-token chunk
    after 1000 cached tokens, 16 query heads on 4 KV heads, D = 128, paged."""
    B, Hq, Hkv, S, D, cap = 1, 16, 4, 300, 128, 1312
    lens, n = [1000], [300]
    log_case("int8 chunk bf16 long prefix")
    q, k, v, ks, vs, ck, cv, table = int8_chunk_inputs(B, Hq, Hkv, S, D, torch.bfloat16, lens,
                                                       n, 777, True, cap, unambiguous=False)
    ok, ov = np_i8(ck), np_i8(cv)
    cache = car.KVCache(ck, cv, torch.from_numpy(table).to(DEV), k_scale=ks, v_scale=vs)
    out = car.attn_prefill_cached(q, k, v, torch.tensor(lens, dtype=torch.int32, device=DEV),
                                  cache, 1300)
    torch.cuda.synchronize()
    want = oracle.attn_prefill_cached_int8(f64(q), f64(k), f64(v), ok, ov, np.array(lens),
                                           f64(ks), f64(vs), block_table=table)
    err = max_abs(f64(out), want)
    log_case(f"max-abs error {err:.3e}")
    assert err <= TOL[torch.bfloat16]
    # value codes exact everywhere; key codes exact, or one apart at a rounding
    # tie of a chunk token's rotated key (slots outside the chunk unchanged)
    assert np.array_equal(np_i8(cv), ov)
    t = lens[0] + np.arange(n[0])
    blk, off = table[0, t // 16], t % 16
    kr = oracle.rope_rotate(f64(k[0]), t)                       # [Hkv, n, D]
    got_rows = np_i8(ck)[blk, :, off].transpose(1, 0, 2)        # [Hkv, n, D]
    want_rows = ok[blk, :, off].transpose(1, 0, 2)
    flips = check_key_codes(got_rows, want_rows, kr, f64(ks)[:, None, :])
    log_case(f"key codes one apart at ties: {flips}")
    rest_got, rest_want = np_i8(ck).copy(), ok.copy()
    rest_got[blk, :, off] = 0
    rest_want[blk, :, off] = 0
    assert np.array_equal(rest_got, rest_want)
