"""Causal attention with RoPE and a KV cache on AMD MI355X (gfx950).

A thin binding over ``libcar.so``, the C ABI declared in ``include/car.h``.
Every step of the computation runs in the library's HIP kernels; this module
only checks tensors, allocates outputs and workspaces through torch, and
passes raw device pointers and torch's current HIP stream.  There is no CPU
fallback: importing fails if the library has not been built.

Entry points (same names as the C ABI without the ``car_`` prefix):
``rope_apply``, ``kv_cache_append``, ``kv_int8_calibrate``, ``attn_prefill``,
``attn_prefill_cached``, ``attn_decode``, plus ``KVCache`` (native or INT8
elements) and the workspace size queries.  The three attention calls take an
optional ``timing=(start, stop)`` pair of torch.cuda.Event, recorded around
their attention kernel (the ``_timed`` entry points of the C ABI).
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "CarError", "KVCache", "rope_apply", "kv_cache_append", "attn_prefill", "attn_decode",
    "attn_prefill_cached", "kv_int8_calibrate",
    "attn_decode_noalloc", "DECODE_NOALLOC_MAX_BYTES",
    "prefill_workspace_bytes", "prefill_cached_workspace_bytes", "decode_workspace_bytes",
    "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# CAR_LIBRARY selects another build of the same library (the sanitized
# host-only build that the ABI tests run against); default: the in-tree one.
library_path = os.environ.get("CAR_LIBRARY") or os.path.join(_HERE, "libcar.so")

F32, BF16 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}
# RoPE pair layouts (car_rope_pairing): (2i, 2i+1) or (i, i + D/2)
ROPE_PAIRINGS = {"adjacent": 0, "half": 1}


def _pairing(name: str) -> int:
    if name not in ROPE_PAIRINGS:
        raise ValueError(f"rope_pairing must be one of {sorted(ROPE_PAIRINGS)}")
    return ROPE_PAIRINGS[name]


class CarError(RuntimeError):
    """A non-zero car_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.car_status_string(status).decode()}")


class _CarKVCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("max_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("format", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


CACHE_NATIVE, CACHE_INT8 = 0, 1
# CAR_DECODE_NOALLOC_MAX_BYTES: size of the per-GPU partials array of attn_decode_noalloc
DECODE_NOALLOC_MAX_BYTES = 48 << 20


def _load() -> ctypes.CDLL:
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing; build it first with "
            "`python causal_attention_rope_amd/build.py`")
    try:
        lib = ctypes.CDLL(library_path)
    except OSError as e:
        raise ImportError(f"cannot load {library_path}: {e}; rebuild it with "
                          "`python causal_attention_rope_amd/build.py`") from e
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    cache_p = ctypes.POINTER(_CarKVCache)
    prefill = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, f32, i32, f32, cache_p, vp,
               sz, vp]
    cached = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, i32, f32, i32, f32, cache_p,
              vp, sz, vp]
    decode = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, f32, i32, f32, cache_p, vp, sz,
              vp]
    sigs = {
        "car_rope_apply": (i32, [vp, i32, i32, i32, i32, i32, vp, f32, i32, vp]),
        "car_kv_cache_append": (i32, [cache_p, i32, vp, vp, i32, i32, i32, i32, vp, vp]),
        "car_kv_int8_calibrate": (i32, [vp, vp, i32, i32, i32, i32, i32, vp, f32, i32, vp, vp,
                                        vp]),
        "car_attn_prefill_workspace_bytes": (sz, [i32, i32, i32, i32, i32, cache_p]),
        "car_attn_prefill": (i32, prefill),
        "car_attn_prefill_timed": (i32, prefill + [vp, vp]),
        "car_attn_prefill_cached": (i32, cached),
        "car_attn_prefill_cached_timed": (i32, cached + [vp, vp]),
        "car_attn_decode_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "car_attn_prefill_cached_workspace_bytes": (sz, [i32, i32, i32, i32, i32, cache_p]),
        "car_attn_decode": (i32, decode),
        "car_attn_decode_timed": (i32, decode + [vp, vp]),
        "car_attn_decode_noalloc": (i32, decode[:15] + [vp]),
        "car_status_string": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _check_single_hip_runtime() -> None:
    """The library must share torch's HIP runtime (one libamdhip64 mapped)."""
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({sorted(real)}); libcar.so must "
                          "resolve libamdhip64 to torch's copy")


_lib = _load()
_check_single_hip_runtime()


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, dim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DTYPES[t.dtype]


def _check(status: int, where: str) -> None:
    if status != 0:
        raise CarError(status, where)


class KVCache:
    """One layer's KV cache (separate K and V tensors).

    Contiguous: ``k`` and ``v`` are [B, Hkv, max_seq, D].
    Paged: ``k`` and ``v`` are pools [num_blocks, Hkv, 16, D] and
    ``block_table`` is int32 [B, max_blocks_per_seq].
    Native elements are the calls' dtype (float32 or bfloat16).  INT8: ``k``
    and ``v`` are torch.int8 codes and ``k_scale``, ``v_scale`` are float32
    [Hkv, D] (value = code * scale; see ``kv_int8_calibrate``).
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor,
                 block_table: Optional[torch.Tensor] = None,
                 k_scale: Optional[torch.Tensor] = None,
                 v_scale: Optional[torch.Tensor] = None):
        _need(k, "cache k", dim=4)
        _need(v, "cache v", dtype=k.dtype, dim=4, device=k.device)
        if k.shape != v.shape:
            raise ValueError("cache k and v must have the same shape")
        self.k, self.v, self.block_table = k, v, block_table
        if block_table is not None:
            _need(block_table, "block_table", dtype=torch.int32, dim=2, device=k.device)
            if k.shape[2] != 16:
                raise ValueError("paged cache blocks must hold 16 tokens")
        self.Hkv, self.D = k.shape[1], k.shape[3]
        self.int8 = k.dtype == torch.int8
        if self.int8:
            if k_scale is None or v_scale is None:
                raise ValueError("an int8 cache needs k_scale and v_scale")
            for s, name in ((k_scale, "k_scale"), (v_scale, "v_scale")):
                _need(s, name, dtype=torch.float32, dim=2, device=k.device)
                if tuple(s.shape) != (self.Hkv, self.D):
                    raise ValueError(f"{name} must be [Hkv, D]")
        elif k_scale is not None or v_scale is not None:
            raise ValueError("scales are only used with an int8 cache")
        elif k.dtype not in _DTYPES:
            raise ValueError(f"unsupported cache dtype {k.dtype}")
        self.k_scale, self.v_scale = k_scale, v_scale

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    def accepts(self, t: torch.Tensor) -> bool:
        """Whether a call in t's dtype may use this cache."""
        return t.device == self.k.device and (
            t.dtype in _DTYPES if self.int8 else t.dtype == self.k.dtype)

    def check_batch(self, B: int) -> None:
        """The cache must hold (or map) at least B sequences."""
        rows = self.block_table.shape[0] if self.paged else self.k.shape[0]
        if rows < B:
            raise ValueError(f"cache holds {rows} sequences, the call has {B}")

    @property
    def capacity(self) -> int:
        """Tokens one sequence can hold."""
        return self.block_table.shape[1] * 16 if self.paged else self.k.shape[2]

    def _c(self) -> _CarKVCache:
        c = _CarKVCache()
        c.k, c.v = self.k.data_ptr(), self.v.data_ptr()
        if self.paged:
            c.block_table = self.block_table.data_ptr()
            c.max_seq = 0
            c.num_blocks = self.k.shape[0]
            c.block_size = 16
            c.max_blocks_per_seq = self.block_table.shape[1]
        else:
            c.block_table = None
            c.max_seq = self.k.shape[2]
        if self.int8:
            c.format = CACHE_INT8
            c.k_scale, c.v_scale = self.k_scale.data_ptr(), self.v_scale.data_ptr()
        else:
            c.format = CACHE_NATIVE
        return c


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def _events(timing):
    """Raw hipEvent_t handles of a (start, stop) pair of torch.cuda.Event."""
    if timing is None:
        return None
    start, stop = timing
    return [ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)]


def rope_apply(x: torch.Tensor, positions: torch.Tensor, theta: float = 10000.0,
               rope_pairing: str = "adjacent") -> torch.Tensor:
    """Rotate x [B, H, S, D] in place by RoPE at positions int32 [B, S]
    (``rope_pairing``: "adjacent" pairs (2i, 2i+1), "half" pairs (i, i + D/2))."""
    _need(x, "x", dim=4)
    B, H, S, D = x.shape
    _need(positions, "positions", dtype=torch.int32, dim=2, device=x.device)
    if tuple(positions.shape) != (B, S):
        raise ValueError("positions must be [B, S]")
    _check(_lib.car_rope_apply(_ptr(x), _dtype_code(x), B, H, S, D, _ptr(positions),
                               float(theta), _pairing(rope_pairing), _stream(x)), "rope_apply")
    return x


def kv_cache_append(cache: KVCache, k: torch.Tensor, v: torch.Tensor,
                    positions: torch.Tensor) -> None:
    """Store rotated keys k and values v [B, Hkv, S, D] at cache index == position
    (as int8 codes in an int8 cache)."""
    _need(k, "k", dim=4, device=cache.k.device)
    _need(v, "v", dtype=k.dtype, dim=4, device=cache.k.device)
    if not cache.accepts(k):
        raise ValueError("k/v dtype does not match the cache")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, Hkv, S, D = k.shape
    if Hkv != cache.Hkv or D != cache.D:
        raise ValueError("k/v heads or head dim do not match the cache")
    cache.check_batch(B)
    _need(positions, "positions", dtype=torch.int32, dim=2, device=k.device)
    if tuple(positions.shape) != (B, S):
        raise ValueError("positions must be [B, S]")
    c = cache._c()
    _check(_lib.car_kv_cache_append(ctypes.byref(c), _dtype_code(k), _ptr(k), _ptr(v), B, Hkv,
                                    S, D, _ptr(positions), _stream(k)), "kv_cache_append")


def kv_int8_calibrate(k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor,
                      theta: float = 10000.0, rope_pairing: str = "adjacent"):
    """Per-(KV head, channel) INT8 scales of a calibration batch (see
    car_kv_int8_calibrate): absmax over every (b, s) of the keys rotated at
    ``positions`` and of the values, divided by 127.  k, v [B, Hkv, S, D]
    (k not rotated); positions int32 [B, S].  Returns (k_scale, v_scale),
    float32 [Hkv, D]."""
    _need(k, "k", dim=4)
    _need(v, "v", dtype=k.dtype, dim=4, device=k.device)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, Hkv, S, D = k.shape
    _need(positions, "positions", dtype=torch.int32, dim=2, device=k.device)
    if tuple(positions.shape) != (B, S):
        raise ValueError("positions must be [B, S]")
    ks = torch.empty((Hkv, D), dtype=torch.float32, device=k.device)
    vs = torch.empty((Hkv, D), dtype=torch.float32, device=k.device)
    _check(_lib.car_kv_int8_calibrate(_ptr(k), _ptr(v), _dtype_code(k), B, Hkv, S, D,
                                      _ptr(positions), float(theta), _pairing(rope_pairing),
                                      _ptr(ks), _ptr(vs), _stream(k)), "kv_int8_calibrate")
    return ks, vs


def prefill_workspace_bytes(dtype: torch.dtype, B: int, Hkv: int, S: int, D: int,
                            cache: Optional[KVCache] = None) -> int:
    """Workspace of attn_prefill; with a cache given, 0 where the attention can
    read the rotated keys back from it (bf16, contiguous, S <= max_seq)."""
    if cache is None:
        return int(_lib.car_attn_prefill_workspace_bytes(_DTYPES[dtype], B, Hkv, S, D, None))
    c = cache._c()
    return int(_lib.car_attn_prefill_workspace_bytes(_DTYPES[dtype], B, Hkv, S, D,
                                                     ctypes.byref(c)))


def prefill_cached_workspace_bytes(dtype: torch.dtype, B: int, Hkv: int, D: int,
                                   max_seq_len: int, cache: KVCache) -> int:
    """Workspace of attn_prefill_cached: 0 for a native cache, the dequantized
    rows for an INT8 one."""
    c = cache._c()
    return int(_lib.car_attn_prefill_cached_workspace_bytes(_DTYPES[dtype], B, Hkv, D,
                                                            max_seq_len, ctypes.byref(c)))


def decode_workspace_bytes(B: int, Hq: int, D: int, max_seq_len: int) -> int:
    return int(_lib.car_attn_decode_workspace_bytes(B, Hq, D, max_seq_len))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    _need(workspace, "workspace", device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds fewer than the {nbytes} bytes required")
    return workspace


def attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor,
                 theta: float = 10000.0, scale: Optional[float] = None,
                 cache: Optional[KVCache] = None, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None,
                 rope_pairing: str = "adjacent", timing=None,
                 seq_lens: Optional[torch.Tensor] = None,
                 no_workspace: bool = False) -> torch.Tensor:
    """Causal attention over a prompt with RoPE on q and k (see car_attn_prefill).

    q [B, Hq, S, D]; k, v [B, Hkv, S, D]; positions int32 [B, S], strictly
    increasing per sequence.  With ``cache`` the rotated keys and the values
    are also stored at index == position.  ``seq_lens`` int32 [B] (optional):
    prompt b is its first seq_lens[b] rows, the rest padding (zero output
    rows, not stored).  ``no_workspace``: pass no workspace, so that the keys
    are read back from ``cache`` (bf16, contiguous, native; each prompt's
    positions consecutive slots).  Returns out [B, Hq, S, D].
    """
    _need(q, "q", dim=4)
    _need(k, "k", dtype=q.dtype, dim=4, device=q.device)
    _need(v, "v", dtype=q.dtype, dim=4, device=q.device)
    B, Hq, S, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError("k and v must be [B, Hkv, S, D] matching q")
    Hkv = k.shape[1]
    _need(positions, "positions", dtype=torch.int32, dim=2, device=q.device)
    if tuple(positions.shape) != (B, S):
        raise ValueError("positions must be [B, S]")
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1, device=q.device)
        if seq_lens.shape[0] != B:
            raise ValueError("seq_lens must be [B]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, dim=4, device=q.device)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    c = None
    if cache is not None:
        if not cache.accepts(q):
            raise ValueError("cache dtype/device must match q")
        if cache.Hkv != Hkv or cache.D != D:
            raise ValueError("cache heads or head dim do not match k")
        cache.check_batch(B)
        c = cache._c()
    dt = _dtype_code(q)
    need = int(_lib.car_attn_prefill_workspace_bytes(dt, B, Hkv, S, D, None))
    if no_workspace:
        # keys read back from a contiguous bf16 cache (consecutive positions only)
        if workspace is not None:
            raise ValueError("no_workspace and workspace are exclusive")
        ws, ws_bytes = None, 0
    else:
        ws = _workspace(need, q.device, workspace)
        ws_bytes = ws.numel() * ws.element_size()
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), dt, B, Hq, Hkv, S, D, _ptr(positions),
            _ptr(seq_lens), float(theta), _pairing(rope_pairing), float(scale),
            ctypes.byref(c) if c is not None else None, _ptr(ws), ws_bytes, _stream(q)]
    ev = _events(timing)
    if ev is None:
        _check(_lib.car_attn_prefill(*args), "attn_prefill")
    else:
        _check(_lib.car_attn_prefill_timed(*args, *ev), "attn_prefill")
    return out


def attn_prefill_cached(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        seq_lens: torch.Tensor, cache: KVCache, max_seq_len: int,
                        theta: float = 10000.0, scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None,
                        chunk_lens: Optional[torch.Tensor] = None,
                        rope_pairing: str = "adjacent", timing=None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A prompt chunk continuing a cached prefix (see car_attn_prefill_cached).

    q [B, Hq, S, D]; k, v [B, Hkv, S, D] (k not rotated); seq_lens int32 [B]
    (tokens already cached = position of the chunk's first token);
    ``chunk_lens`` int32 [B] (optional): sequence b's chunk is its first
    chunk_lens[b] rows, the rest is padding (zero output rows);
    ``max_seq_len`` is a host bound on seq_lens + chunk length.  Writes the
    chunk's keys and values into the cache and returns out [B, Hq, S, D].
    An INT8 cache needs a workspace (allocated here unless given).
    """
    _need(q, "q", dim=4)
    _need(k, "k", dtype=q.dtype, dim=4, device=q.device)
    _need(v, "v", dtype=q.dtype, dim=4, device=q.device)
    B, Hq, S, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError("k and v must be [B, Hkv, S, D] matching q")
    Hkv = k.shape[1]
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1, device=q.device)
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens must be [B]")
    if chunk_lens is not None:
        _need(chunk_lens, "chunk_lens", dtype=torch.int32, dim=1, device=q.device)
        if chunk_lens.shape[0] != B:
            raise ValueError("chunk_lens must be [B]")
    if not cache.accepts(q):
        raise ValueError("cache dtype/device must match q")
    if cache.Hkv != Hkv or cache.D != D:
        raise ValueError("cache heads or head dim do not match k")
    cache.check_batch(B)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, dim=4, device=q.device)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    c = cache._c()
    need = int(_lib.car_attn_prefill_cached_workspace_bytes(_dtype_code(q), B, Hkv, D,
                                                            int(max_seq_len), ctypes.byref(c)))
    if need == 0 and workspace is None:
        ws, ws_bytes = None, 0
    else:
        ws = _workspace(need, q.device, workspace)
        ws_bytes = ws.numel() * ws.element_size()
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), B, Hq, Hkv, S, D,
            _ptr(seq_lens), _ptr(chunk_lens), int(max_seq_len), float(theta),
            _pairing(rope_pairing), float(scale), ctypes.byref(c), _ptr(ws), ws_bytes,
            _stream(q)]
    ev = _events(timing)
    if ev is None:
        _check(_lib.car_attn_prefill_cached(*args), "attn_prefill_cached")
    else:
        _check(_lib.car_attn_prefill_cached_timed(*args, *ev), "attn_prefill_cached")
    return out


def _decode_checks(q, k_new, v_new, seq_lens, cache, out):
    """Shape/dtype/device checks shared by the decode calls; returns (B, Hq, Hkv, D)."""
    _need(q, "q", dim=3)
    _need(k_new, "k_new", dtype=q.dtype, dim=3, device=q.device)
    _need(v_new, "v_new", dtype=q.dtype, dim=3, device=q.device)
    B, Hq, D = q.shape
    if k_new.shape != v_new.shape or k_new.shape[0] != B or k_new.shape[2] != D:
        raise ValueError("k_new and v_new must be [B, Hkv, D] matching q")
    Hkv = k_new.shape[1]
    _need(seq_lens, "seq_lens", dtype=torch.int32, dim=1, device=q.device)
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens must be [B]")
    if not cache.accepts(q):
        raise ValueError("cache dtype/device must match q")
    if cache.Hkv != Hkv or cache.D != D:
        raise ValueError("cache heads or head dim do not match k_new")
    cache.check_batch(B)
    _need(out, "out", dtype=q.dtype, dim=3, device=q.device)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    return B, Hq, Hkv, D


def attn_decode(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                seq_lens: torch.Tensor, cache: KVCache, max_seq_len: int,
                theta: float = 10000.0, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                rope_pairing: str = "adjacent", timing=None) -> torch.Tensor:
    """One decode step (see car_attn_decode).

    q [B, Hq, D]; k_new, v_new [B, Hkv, D] (not rotated); seq_lens int32 [B]
    (tokens already cached = position of the new token); ``max_seq_len`` is a
    host bound on seq_lens + 1.  Writes the new key/value into the cache and
    returns out [B, Hq, D].
    """
    if out is None:
        out = torch.empty_like(q)
    B, Hq, Hkv, D = _decode_checks(q, k_new, v_new, seq_lens, cache, out)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = int(_lib.car_attn_decode_workspace_bytes(B, Hq, D, int(max_seq_len)))
    ws = _workspace(need, q.device, workspace)
    c = cache._c()
    args = [_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _dtype_code(q), B, Hq, Hkv, D,
            _ptr(seq_lens), int(max_seq_len), float(theta), _pairing(rope_pairing),
            float(scale), ctypes.byref(c), _ptr(ws), ws.numel() * ws.element_size(), _stream(q)]
    ev = _events(timing)
    if ev is None:
        _check(_lib.car_attn_decode(*args), "attn_decode")
    else:
        _check(_lib.car_attn_decode_timed(*args, *ev), "attn_decode")
    return out


def attn_decode_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        seq_lens: torch.Tensor, cache: KVCache, max_seq_len: int,
                        out: torch.Tensor, theta: float = 10000.0,
                        scale: Optional[float] = None,
                        rope_pairing: str = "adjacent") -> torch.Tensor:
    """attn_decode without a workspace (see car_attn_decode_noalloc): the
    library keeps the split partials in a fixed device array of
    ``DECODE_NOALLOC_MAX_BYTES`` per GPU, so nothing is allocated; ``out``
    must be given.  Calls that overlap on one GPU race on that array."""
    B, Hq, Hkv, D = _decode_checks(q, k_new, v_new, seq_lens, cache, out)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    c = cache._c()
    _check(_lib.car_attn_decode_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out),
                                        _dtype_code(q), B, Hq, Hkv, D, _ptr(seq_lens),
                                        int(max_seq_len), float(theta), _pairing(rope_pairing),
                                        float(scale), ctypes.byref(c), _stream(q)),
           "attn_decode_noalloc")
    return out
