"""The C-ABI library without a GPU: it loads, exports every symbol that
include/car.h declares, and its host-side checks reject bad arguments with
the documented status before anything is launched.

Every call here fails a host check (null or misaligned pointer, bad size,
unsupported configuration, short workspace), so no kernel is ever enqueued;
the non-null pointers passed are never dereferenced by the host.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "car.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
FAKE = 0x10000  # aligned, non-null, never dereferenced (every call below fails first)


@pytest.fixture(scope="module")
def car():
    import causal_attention_rope_amd as m
    return m


@pytest.fixture(scope="module")
def lib(car):
    return car._lib


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(car_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("car_rope_apply", "car_kv_cache_append", "car_attn_prefill", "car_attn_decode"):
        assert n in names


def test_library_exports_every_declared_symbol(car):
    lib = ctypes.CDLL(car.library_path)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIP):
        s = lib.car_status_string(code).decode()
        assert s.startswith("CAR_")
    assert "unknown" in lib.car_status_string(99).decode()


def _cache(car, paged=False, block_size=16, max_seq=64, k=FAKE, v=FAKE, fmt=0, ks=None,
           vs=None):
    c = car._CarKVCache()
    c.k, c.v = k, v
    c.format, c.k_scale, c.v_scale = fmt, ks, vs
    if paged:
        c.block_table = FAKE
        c.num_blocks, c.block_size, c.max_blocks_per_seq = 8, block_size, 4
    else:
        c.block_table = None
        c.max_seq = max_seq
    return c


def test_rope_apply_rejects(lib):
    f = lib.car_rope_apply
    assert f(FAKE, BF16, 1, 1, 1, 96, FAKE, 1e4, 0, None) == UNSUPPORTED     # D
    assert f(FAKE, 7, 1, 1, 1, 64, FAKE, 1e4, 0, None) == UNSUPPORTED        # dtype
    assert f(None, BF16, 1, 1, 1, 64, FAKE, 1e4, 0, None) == INVALID         # null x
    assert f(FAKE + 8, BF16, 1, 1, 1, 64, FAKE, 1e4, 0, None) == INVALID     # misaligned
    assert f(FAKE, BF16, -1, 1, 1, 64, FAKE, 1e4, 0, None) == INVALID        # size
    assert f(FAKE, BF16, 1, 1, 1, 64, FAKE, -1.0, 0, None) == INVALID        # theta
    assert f(FAKE, BF16, 1, 1, 1, 64, None, 1e4, 0, None) == INVALID         # positions
    assert f(FAKE, BF16, 1, 1, 1, 64, FAKE, 1e4, 2, None) == UNSUPPORTED     # pairing
    assert f(None, BF16, 0, 4, 4, 64, None, 1e4, 0, None) == OK              # empty: no-op


def test_kv_cache_append_rejects(car, lib):
    f = lib.car_kv_cache_append
    c = _cache(car)
    assert f(ctypes.byref(c), BF16, FAKE, FAKE, 1, 1, 1, 80, FAKE, None) == UNSUPPORTED
    assert f(None, BF16, FAKE, FAKE, 1, 1, 1, 64, FAKE, None) == INVALID
    assert f(ctypes.byref(c), BF16, None, FAKE, 1, 1, 1, 64, FAKE, None) == INVALID
    bad = _cache(car, paged=True, block_size=32)
    assert f(ctypes.byref(bad), BF16, FAKE, FAKE, 1, 1, 1, 64, FAKE, None) == UNSUPPORTED
    zero = _cache(car, max_seq=0)
    assert f(ctypes.byref(zero), BF16, FAKE, FAKE, 1, 1, 1, 64, FAKE, None) == INVALID
    mis = _cache(car, k=FAKE + 4)
    assert f(ctypes.byref(mis), BF16, FAKE, FAKE, 1, 1, 1, 64, FAKE, None) == INVALID
    assert f(ctypes.byref(c), BF16, None, None, 0, 1, 1, 64, None, None) == OK


def test_prefill_rejects(car, lib):
    f = lib.car_attn_prefill
    need = lib.car_attn_prefill_workspace_bytes(BF16, 2, 2, 8, 64, None)
    assert need == 2 * 2 * 8 * 64 * 2
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dt=BF16, B=2, Hq=4, Hkv=2, S=8, D=64,
                pos=FAKE, lens=None, theta=1e4, pair=0, scale=0.125, cache=None, ws=FAKE,
                wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["out"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["S"],
                 a["D"], a["pos"], a["lens"], a["theta"], a["pair"], a["scale"], a["cache"],
                 a["ws"], a["wsb"], None)

    assert call(D=80) == UNSUPPORTED
    assert call(pair=5) == UNSUPPORTED               # unknown RoPE pairing
    assert call(Hq=3) == INVALID                     # Hq % Hkv
    assert call(scale=0.0) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(q=None) == INVALID
    assert call(out=FAKE + 2) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(wsb=need - 1) == WORKSPACE
    bad = _cache(car, paged=True, block_size=8)
    assert call(cache=ctypes.byref(bad)) == UNSUPPORTED
    zero = _cache(car, max_seq=0)
    assert call(cache=ctypes.byref(zero), wsb=0) == INVALID
    assert call(S=0, q=None, ws=None) == OK          # empty prompt: no-op


def test_decode_rejects(car, lib):
    f = lib.car_attn_decode
    need = lib.car_attn_decode_workspace_bytes(2, 8, 128, 300)
    assert need == 2 * 8 * 2 * (128 + 4) * 4        # two 256-token splits
    c = _cache(car, max_seq=512)
    args = dict(q=FAKE, kn=FAKE, vn=FAKE, out=FAKE, dt=BF16, B=2, Hq=8, Hkv=2, D=128,
                lens=FAKE, msl=300, theta=1e4, pair=1, scale=0.088, cache=ctypes.byref(c),
                ws=FAKE, wsb=need - 16)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["kn"], a["vn"], a["out"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["D"],
                 a["lens"], a["msl"], a["theta"], a["pair"], a["scale"], a["cache"], a["ws"],
                 a["wsb"], None)

    assert call() == WORKSPACE                       # everything valid but the workspace
    assert call(ws=None) == WORKSPACE
    assert call(pair=-1) == UNSUPPORTED              # unknown RoPE pairing
    assert call(D=96) == UNSUPPORTED
    assert call(Hq=5) == INVALID                     # Hq % Hkv
    assert call(Hq=6) == UNSUPPORTED                 # group of 3 not built
    assert call(Hq=32) == UNSUPPORTED                # group of 16 not built
    assert call(lens=None) == INVALID
    assert call(msl=0) == INVALID
    assert call(msl=513) == INVALID                  # beyond the cache capacity
    assert call(cache=None) == INVALID
    bad = _cache(car, paged=True, block_size=32)
    assert call(cache=ctypes.byref(bad)) == UNSUPPORTED
    assert call(B=0, q=None, ws=None) == OK          # empty batch: no-op
    assert call(B=1 << 30) == UNSUPPORTED            # B * Hkv workgroups exceed the grid
    assert call(msl=65535 * 256 + 1) == UNSUPPORTED  # more than 65535 splits
    huge = _cache(car, max_seq=(1 << 23) + 1)        # a head's rows past 32-bit offsets
    assert call(cache=ctypes.byref(huge)) == UNSUPPORTED


def test_prefill_cached_rejects(car, lib):
    f = lib.car_attn_prefill_cached
    c = _cache(car, max_seq=512)
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dt=BF16, B=2, Hq=8, Hkv=2, S=100, D=128,
                lens=FAKE, clens=None, msl=300, theta=1e4, pair=0, scale=0.088,
                cache=ctypes.byref(c), ws=None, wsb=0)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["out"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["S"],
                 a["D"], a["lens"], a["clens"], a["msl"], a["theta"], a["pair"], a["scale"],
                 a["cache"], a["ws"], a["wsb"], None)

    assert call(D=96) == UNSUPPORTED
    assert call(dt=7) == UNSUPPORTED
    assert call(pair=3) == UNSUPPORTED               # unknown RoPE pairing
    assert call(Hq=5) == INVALID                     # Hq % Hkv
    assert call(lens=None) == INVALID
    assert call(q=None) == INVALID
    assert call(out=FAKE + 8) == INVALID             # not 16-byte aligned
    assert call(msl=99) == INVALID                   # below the chunk length
    assert call(msl=0, clens=FAKE) == INVALID        # padded chunks: still at least 1
    assert call(msl=513, clens=FAKE) == INVALID      # padded chunks: beyond the capacity
    assert call(msl=513) == INVALID                  # beyond the cache capacity
    assert call(cache=None) == INVALID
    assert call(theta=0.0) == INVALID
    assert call(B=70000) == UNSUPPORTED              # beyond the launch grid
    bad = _cache(car, paged=True, block_size=32)
    assert call(cache=ctypes.byref(bad)) == UNSUPPORTED
    assert call(B=0, q=None) == OK                   # empty batch: no-op
    assert call(S=0, q=None) == OK                   # empty chunk: no-op


def test_int8_cache_rejects(car, lib):
    """An INT8 cache needs both scale arrays, 16-byte aligned; an unknown
    format is unsupported; a chunk over an INT8 cache needs its workspace
    (two dequantized copies of [B, Hkv, max_seq_len, D])."""
    app = lib.car_kv_cache_append
    for c, want in ((_cache(car, fmt=1), INVALID),                          # no scales
                    (_cache(car, fmt=1, ks=FAKE), INVALID),                 # no v_scale
                    (_cache(car, fmt=1, ks=FAKE, vs=FAKE + 4), INVALID),    # misaligned
                    (_cache(car, fmt=2, ks=FAKE, vs=FAKE), UNSUPPORTED)):   # unknown format
        assert app(ctypes.byref(c), BF16, FAKE, FAKE, 1, 1, 1, 64, FAKE, None) == want
    good = _cache(car, max_seq=512, fmt=1, ks=FAKE, vs=FAKE)
    need = lib.car_attn_prefill_cached_workspace_bytes(BF16, 2, 2, 128, 300, ctypes.byref(good))
    assert need == 2 * 2 * 2 * 300 * 128 * 2
    assert lib.car_attn_prefill_cached_workspace_bytes(F32, 2, 2, 128, 300,
                                                       ctypes.byref(good)) == 2 * need
    native = _cache(car, max_seq=512)
    assert lib.car_attn_prefill_cached_workspace_bytes(BF16, 2, 2, 128, 300,
                                                       ctypes.byref(native)) == 0
    for ws, wsb in ((None, need), (FAKE, need - 1), (FAKE + 8, need)):
        chunk = lib.car_attn_prefill_cached(FAKE, FAKE, FAKE, FAKE, BF16, 2, 8, 2, 100, 128, FAKE,
                                            None, 300, 1e4, 0, 0.088, ctypes.byref(good), ws, wsb,
                                            None)
        assert chunk == WORKSPACE
    noscale = _cache(car, max_seq=512, fmt=1)
    dec = lib.car_attn_decode(FAKE, FAKE, FAKE, FAKE, BF16, 2, 8, 2, 128, FAKE, 300, 1e4, 0,
                              0.088, ctypes.byref(noscale), FAKE, 1 << 20, None)
    assert dec == INVALID
    # the same INT8 cache with scales passes every check up to the workspace
    dec = lib.car_attn_decode(FAKE, FAKE, FAKE, FAKE, BF16, 2, 8, 2, 128, FAKE, 300, 1e4, 0,
                              0.088, ctypes.byref(good), None, 0, None)
    assert dec == WORKSPACE


def test_int8_calibrate_rejects(lib):
    f = lib.car_kv_int8_calibrate
    assert f(FAKE, FAKE, BF16, 1, 2, 8, 96, FAKE, 1e4, 0, FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, FAKE, 7, 1, 2, 8, 64, FAKE, 1e4, 0, FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, FAKE, BF16, 1, 2, 8, 64, FAKE, 1e4, 4, FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, FAKE, BF16, -1, 2, 8, 64, FAKE, 1e4, 0, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, BF16, 1, 2, 8, 64, FAKE, 0.0, 0, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, BF16, 1, 2, 8, 64, FAKE, 1e4, 0, None, FAKE, None) == INVALID
    assert f(FAKE, FAKE, BF16, 1, 2, 8, 64, FAKE, 1e4, 0, FAKE, FAKE + 8, None) == INVALID
    assert f(None, FAKE, BF16, 1, 2, 8, 64, FAKE, 1e4, 0, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, BF16, 1, 2, 8, 64, None, 1e4, 0, FAKE, FAKE, None) == INVALID
    assert f(FAKE + 2, FAKE, BF16, 1, 2, 8, 64, FAKE, 1e4, 0, FAKE, FAKE, None) == INVALID
    assert f(None, None, BF16, 1, 0, 8, 64, None, 1e4, 0, None, None, None) == OK   # no heads


def test_prefill_workspace_not_needed_for_a_contiguous_bf16_cache(car, lib):
    """Keys into a contiguous native bf16 cache need no workspace (they are
    read back from the cache) when the prompt fits it; every other case
    needs B*Hkv*S*D elements."""
    full_bf16 = 2 * 4 * 128 * 64 * 2
    cont = _cache(car, max_seq=128)
    assert lib.car_attn_prefill_workspace_bytes(BF16, 2, 4, 128, 64, ctypes.byref(cont)) == 0
    assert lib.car_attn_prefill_workspace_bytes(BF16, 2, 4, 128, 64, None) == full_bf16
    short = _cache(car, max_seq=127)   # the prompt does not fit: keys need the workspace
    assert lib.car_attn_prefill_workspace_bytes(BF16, 2, 4, 128, 64, ctypes.byref(short)) == full_bf16
    paged = _cache(car, paged=True)
    assert lib.car_attn_prefill_workspace_bytes(BF16, 2, 4, 128, 64, ctypes.byref(paged)) == full_bf16
    i8 = _cache(car, max_seq=128, fmt=1, ks=FAKE, vs=FAKE)
    assert lib.car_attn_prefill_workspace_bytes(BF16, 2, 4, 128, 64, ctypes.byref(i8)) == full_bf16
    assert lib.car_attn_prefill_workspace_bytes(F32, 2, 4, 128, 64, ctypes.byref(cont)) == 2 * full_bf16
    # without a workspace the host checks refuse every case but the first
    f = lib.car_attn_prefill

    def call(dt, cache):
        return f(FAKE, FAKE, FAKE, FAKE, dt, 2, 4, 4, 128, 64, FAKE, None, 1e4, 0, 0.1, cache,
                 None, 0, None)
    for dt, c in ((BF16, None), (BF16, short), (BF16, paged), (F32, cont)):
        assert call(dt, ctypes.byref(c) if c is not None else None) == WORKSPACE


def test_python_workspace_size_helper_passes_the_cache(car):
    """The binding's prefill_workspace_bytes forwards an optional cache (a
    stand-in that only describes a contiguous 128-slot cache; nothing is
    launched)."""
    import torch

    class Cont:
        def _c(self):
            return _cache(car, max_seq=128)
    cont = Cont()
    full = 2 * 4 * 128 * 64 * 2
    assert car.prefill_workspace_bytes(torch.bfloat16, 2, 4, 128, 64) == full
    assert car.prefill_workspace_bytes(torch.bfloat16, 2, 4, 128, 64, cache=cont) == 0
    assert car.prefill_workspace_bytes(torch.bfloat16, 2, 4, 129, 64, cache=cont) == full // 128 * 129
    assert car.prefill_workspace_bytes(torch.float32, 2, 4, 128, 64, cache=cont) == 2 * full


def test_workspace_sizes(lib):
    assert lib.car_attn_decode_workspace_bytes(32, 32, 128, 4096) == 32 * 32 * 16 * 132 * 4
    assert lib.car_attn_decode_workspace_bytes(64, 32, 128, 8193) == 64 * 32 * 33 * 132 * 4
    assert lib.car_attn_decode_workspace_bytes(3, 5, 64, 300) == 3 * 5 * 2 * 68 * 4
    assert lib.car_attn_decode_workspace_bytes(1, 1, 96, 10) == 0
    assert lib.car_attn_prefill_workspace_bytes(F32, 1, 4, 128, 64, None) == 4 * 128 * 64 * 4
    assert lib.car_attn_prefill_workspace_bytes(BF16, 1, 4, 128, 72, None) == 0


def test_prefill_launch_limits_fail_before_any_launch(car, lib):
    """Sizes beyond one launch's grid or 32-bit offsets are refused with
    CAR_ERR_UNSUPPORTED by the host checks, before the K pass is queued
    (without the checks these calls would reach a launch, which fails here
    with CAR_ERR_HIP since there is no GPU)."""
    f = lib.car_attn_prefill
    ws = 1 << 40  # the workspace check passes; nothing is dereferenced

    def call(dt, B, Hq, Hkv, S, D, cache=None):
        return f(FAKE, FAKE, FAKE, FAKE, dt, B, Hq, Hkv, S, D, FAKE, None, 1e4, 0, 0.1, cache,
                 FAKE, ws, None)

    assert call(F32, 65536, 1, 1, 4, 64) == UNSUPPORTED      # fp32 grid z
    assert call(F32, 1, 65536, 1, 4, 64) == UNSUPPORTED      # fp32 grid y
    assert call(BF16, 65535, 65535, 1, 64, 64) == UNSUPPORTED  # bf16 grid x
    assert call(BF16, 1, 1, 1, 1 << 23, 128) == UNSUPPORTED  # 32-bit key offsets
    big = _cache(car, max_seq=1 << 23)
    assert call(BF16, 1, 1, 1, 64, 128, ctypes.byref(big)) == UNSUPPORTED  # cache offsets


def test_decode_merge_grid_bound(car, lib):
    """The merge launches B * Hq workgroups: B * Hq above 2^31 - 1 is refused
    even when B * Hkv fits."""
    c = _cache(car, max_seq=64)
    assert lib.car_attn_decode(FAKE, FAKE, FAKE, FAKE, BF16, 1 << 28, 8, 1, 128, FAKE, 16, 1e4,
                               0, 0.1, ctypes.byref(c), FAKE, 1 << 60, None) == UNSUPPORTED


def test_timed_variants_check_like_the_plain_calls(car, lib):
    """The _timed entry points run the same host checks (events unused)."""
    c = _cache(car, max_seq=512)
    need = lib.car_attn_decode_workspace_bytes(2, 8, 128, 300)
    common = (FAKE, FAKE, FAKE, FAKE, BF16, 2, 8, 2, 128, FAKE, 300, 1e4, 1, 0.088,
              ctypes.byref(c), FAKE)
    assert lib.car_attn_decode_timed(*common, need - 16, None, None, None) == WORKSPACE
    assert lib.car_attn_decode_timed(*common, need - 16, None, FAKE, FAKE) == WORKSPACE
    pre = (FAKE, FAKE, FAKE, FAKE, BF16, 1, 4, 4, 8, 96, FAKE, FAKE, 1e4, 0, 0.1, None, FAKE,
           1 << 20, None)
    assert lib.car_attn_prefill_timed(*pre, None, None) == UNSUPPORTED
    assert lib.car_attn_prefill(*pre) == UNSUPPORTED
    cached = (FAKE, FAKE, FAKE, FAKE, BF16, 1, 4, 3, 8, 128, FAKE, None, 64, 1e4, 0, 0.1,
              ctypes.byref(c), None, 0, None)
    assert lib.car_attn_prefill_cached_timed(*cached, None, None) == INVALID   # Hq % Hkv
    assert lib.car_attn_prefill_cached(*cached) == INVALID


def test_noalloc_decode_limit(car, lib):
    """The no-allocation decode refuses sizes whose partials exceed its
    array before any HIP call (so this runs without a GPU), and the
    binding's constant is the header's."""
    text = open(HEADER, encoding="utf-8").read()
    m = re.search(r"#define CAR_DECODE_NOALLOC_MAX_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == car.DECODE_NOALLOC_MAX_BYTES
    limit = car.DECODE_NOALLOC_MAX_BYTES
    assert lib.car_attn_decode_workspace_bytes(64, 32, 128, 46 * 256) <= limit
    assert lib.car_attn_decode_workspace_bytes(64, 32, 128, 46 * 256 + 1) > limit
    f = lib.car_attn_decode_noalloc
    assert f(FAKE, FAKE, FAKE, FAKE, BF16, 64, 32, 8, 128, FAKE, 46 * 256 + 1, 1e4, 0, 0.088,
             None, None) == WORKSPACE


def test_binding_refuses_cpu_tensors(car):
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        car.rope_apply(x, torch.zeros(1, 4, dtype=torch.int32))
