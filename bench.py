#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step is one pass of every stage of the path over the synthetic workloads:

  1. prefill of the Qwen-shaped prompt (B=1, H=32, D=128, S=4096, bf16):
     RoPE on K and the cache store (one pass), then the tiled online-softmax
     attention kernel (RoPE on Q fused), writing a [1, 32, 4096, 128] cache;
  2. one decode step over the contiguous cache (B=32, H=32, D=128, cached
     lengths uniform in [1, 4095]);
  3. one decode step over the paged cache with GQA (B=64, Hq=32, Hkv=8,
     16-token blocks, lengths uniform in [512, 8192]).

All inputs are resident in HBM before timing.  The headline ``value`` is the
prefill's algorithmic TFLOP/s over the whole prefill call; the decode steps'
KV GB/s and tokens/s are reported beside it.  The main kernel of every call
is also timed alone with HIP events recorded on its stream around the launch,
which gives the roofline fractions.  The fp64 oracle, timed on the host
cores on a bounded sample of the same workloads, is reported as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu-baseline]
                    [--stat-iters N]

Before the W warmup steps the stages run untimed for 0.3 s more, so that the
timed steps do not start at idle clocks.  Every stage and extra is also timed
over N (default 100) further iterations for its median, p10 and p90; the
decode kernels once more after 512 MiB of writes before each iteration (cold
Infinity Cache).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

# The oracle's BLAS threads: every host core this process may run on, unless
# the environment already fixes the count (set before numpy is imported).
HOST_THREADS = len(os.sched_getaffinity(0))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(HOST_THREADS))

METRIC = "prefill TFLOP/s (% MFMA peak); decode KV GB/s (% HBM peak) + tokens/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def prefill_flops(B: int, H: int, S: int, D: int) -> int:
    """Algorithmic prefill flops: QK^T and PV over the causal (unmasked)
    pairs only, 2 flops per multiply-add: 2 * 2 * B*H*D * S(S+1)/2."""
    return 2 * B * H * D * S * (S + 1)


def chunk_flops(B: int, H: int, P: int, S: int, D: int) -> int:
    """QK^T and PV of a chunk of S queries over P cached keys plus the chunk
    (query i sees P + i + 1 keys): 4 * B * H * D * (S * P + S (S + 1) / 2)."""
    return 4 * B * H * D * (S * P + S * (S + 1) // 2)


def decode_kv_bytes(lens, Hkv: int, D: int, elem_bytes: int) -> int:
    """Algorithmic KV bytes one decode step reads: every cached K and V row
    of every KV head once (GQA query heads share their KV head's read)."""
    return sum(int(L) for L in lens) * Hkv * D * 2 * elem_bytes


def decode_io_bytes(B: int, Hq: int, Hkv: int, D: int, elem_bytes: int) -> int:
    """Per-step bytes besides the cache read: q in, out, k_new/v_new in, and
    the appended K/V row written."""
    return B * (2 * Hq + 4 * Hkv) * D * elem_bytes


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--only", choices=["prefill", "contiguous", "paged"], default=None,
                   help="time one stage only (profiling runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=32,
                   help="prefill heads in the oracle's timed sample")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the chunked-prefill measurements outside the timed step")
    p.add_argument("--stat-iters", type=int, default=100,
                   help="timed iterations per stage for the median / p10 / p90 figures")
    p.add_argument("--cpu-heads-1t", type=int, default=2,
                   help="prefill heads in the oracle's single-thread sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run one plain 1 GiB device copy (HBM counter calibration)")
    return p.parse_args(argv)


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["rope_cache.hip", "decode.hip", "decode_i8.hip", "prefill.hip", "common.hpp",
                  "decode_common.hpp", "launch.hpp"]
COPY_BYTES = 1 << 30
FLUSH_BYTES = 512 << 20
CLOCK_WARM_S = 0.3


def kernel_source_sha() -> str:
    """Hash of the kernel sources; HBM traffic figures are valid only for it."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "causal_attention_rope_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """Per-launch HBM bytes per kernel from profiles/traffic.json, if they were
    taken on the current kernel sources (else {})."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except OSError:
        return {}
    if t.get("source_sha") != kernel_source_sha():
        return {}
    return t.get("kernels", {})


def blas_info() -> dict:
    """numpy's BLAS build and the thread pools threadpoolctl sees."""
    import numpy as np
    import threadpoolctl
    info = {"numpy": np.__version__}
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {})
        info["blas"] = {k: blas.get(k) for k in ("name", "version", "openblas configuration")
                        if blas.get(k) is not None}
    except Exception as e:  # older numpy: no dict mode
        info["blas"] = f"unavailable ({e.__class__.__name__})"
    info["pools"] = [{k: d.get(k) for k in ("internal_api", "version", "num_threads",
                                            "threading_layer")}
                     for d in threadpoolctl.threadpool_info()]
    return info


def cpu_baseline(pf, c4, heads: int, heads_1t: int):
    """Time the fp64 oracle on the host on a bounded sample of the workloads,
    with every BLAS thread and again with one thread."""
    import numpy as np
    import threadpoolctl
    import oracle
    info = threadpoolctl.threadpool_info()
    threads = max([d.get("num_threads", 1) for d in info] or [1])
    S, D = pf.S, pf.D
    q = pf.q[:, :heads].float().cpu().double().numpy()
    k = pf.k[:, :heads].float().cpu().double().numpy()
    v = pf.v[:, :heads].float().cpu().double().numpy()
    pos = pf.positions.cpu().numpy()
    t0 = time.perf_counter()
    oracle.attn_prefill(q, k, v, pos, pf.theta, pf.scale)
    t_pf = time.perf_counter() - t0
    flops = prefill_flops(1, heads, S, D)
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        oracle.attn_prefill(q[:, :heads_1t], k[:, :heads_1t], v[:, :heads_1t], pos, pf.theta,
                            pf.scale)
        t_1t = time.perf_counter() - t0
    # decode sample: the first 8 sequences of the contiguous workload
    bsel = list(range(8))
    lens = np.array([c4.lens_host[b] for b in bsel])
    n = int(lens.max()) + 1
    dq = c4.q[bsel].float().cpu().double().numpy()
    dk = c4.k_new[bsel].float().cpu().double().numpy()
    dv = c4.v_new[bsel].float().cpu().double().numpy()
    ck = c4.cache_k[bsel][:, :, :n].float().cpu().double().numpy()
    cv = c4.cache_v[bsel][:, :, :n].float().cpu().double().numpy()
    t0 = time.perf_counter()
    oracle.attn_decode(dq, dk, dv, ck, cv, lens, c4.theta, c4.scale)
    t_dec = time.perf_counter() - t0
    dbytes = decode_kv_bytes(lens, c4.Hkv, c4.D, 2)
    return {
        "value": flops / t_pf / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 oracle prefill of {heads} of the 32 heads of the S=4096 prompt "
                   f"({t_pf:.1f} s); decode of 8 of the 32 contiguous-cache sequences "
                   f"({t_dec:.2f} s); single-thread prefill of {heads_1t} heads "
                   f"({t_1t:.1f} s)"),
        "decode_GBps": dbytes / t_dec / 1e9,
        "decode_tokens_per_s": len(bsel) / t_dec,
        "single_thread_TFLOPs": prefill_flops(1, heads_1t, S, D) / t_1t / 1e12,
        "host_cores_visible": HOST_THREADS,
        "blas": blas_info(),
    }


def pct(xs, q: float) -> float:
    """q-quantile (0..1) of xs by linear interpolation."""
    xs = sorted(xs)
    if not xs:
        return float("nan")
    f = q * (len(xs) - 1)
    i = int(f)
    j = min(i + 1, len(xs) - 1)
    return xs[i] + (xs[j] - xs[i]) * (f - i)


def spread(ms) -> dict:
    return {"median": pct(ms, 0.5), "p10": pct(ms, 0.1), "p90": pct(ms, 0.9), "n": len(ms)}


def timed_calls(car, call, stream, new_event, iters: int):
    """Event pairs around `iters` whole calls, then around the main kernel
    of `iters` further calls (`call(timing)` hands the pair to the library,
    which records it around that kernel; kept out of the call iterations so
    that they add nothing to the call times)."""
    import torch
    pairs_c = [(new_event(), new_event()) for _ in range(iters)]
    pairs_k = [(new_event(), new_event()) for _ in range(iters)]
    for a, b in pairs_c:
        a.record(stream)
        call()
        b.record(stream)
    for pair in pairs_k:
        call(pair)
    torch.cuda.synchronize()
    return pairs_k, pairs_c


def measure_chunked(car, W, dev, stream, new_event, iters: int = 100) -> dict:
    """A 1024-token chunk continuing a 3072-token cached prefix, 32 query
    heads, D = 128, bf16: contiguous cache [1, 32, 4096, 128], and a paged
    cache with 8 KV heads behind a random block table.  Event times of the
    attention kernel and of the whole call (chunk store + attention)."""
    import torch
    out = {}
    P, S = 3072, 1024
    for name, paged, hkv in (("contiguous", False, 32), ("paged_gqa", True, 8)):
        case = W.chunk_case(f"chunk_{name}", 1, 32, hkv, S, 128, torch.bfloat16, [P], 570, dev,
                            paged=paged, max_seq=None if paged else P + S)
        cache = car.KVCache(case.cache_k, case.cache_v, case.block_table)
        o = torch.empty_like(case.q)

        def call(timing=None):
            car.attn_prefill_cached(case.q, case.k, case.v, case.seq_lens, cache, P + S,
                                    case.theta, case.scale, out=o, timing=timing)
        for _ in range(2):
            call()
        pairs_k, pairs_c = timed_calls(car, call, stream, new_event, iters)
        if not torch.isfinite(o.float()).all():
            raise RuntimeError(f"non-finite output in chunked prefill ({name})")
        kms = sum(a.elapsed_time(b) for a, b in pairs_k) / iters
        cms = sum(a.elapsed_time(b) for a, b in pairs_c) / iters
        fl = chunk_flops(1, 32, P, S, 128)
        out[f"chunked_prefill_{name}"] = {
            "workload": f"B=1,Hq=32,Hkv={hkv},D=128,cached={P},chunk={S},bf16,"
                        + ("paged 16-token blocks" if paged else "contiguous cache 4096"),
            "kernel_ms": kms, "call_ms": cms,
            "kernel_spread_ms": spread([a.elapsed_time(b) for a, b in pairs_k]),
            "call_spread_ms": spread([a.elapsed_time(b) for a, b in pairs_c]),
            "TFLOPs_kernel": fl / (kms * 1e-3) / 1e12, "TFLOPs_call": fl / (cms * 1e-3) / 1e12,
            "mfma_frac_kernel": fl / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "per_launch": f"{fl} flops (4*B*H*D*(S*P + S(S+1)/2))"}
        del case, cache, o
    return out


def measure_int8_chunk(car, W, dev, stream, new_event, iters: int = 100) -> dict:
    """The contiguous chunk workload (1024 tokens after 3072 cached, 32 heads,
    D = 128, bf16 q/k/v) over an INT8 cache [1, 32, 4096, 128] with
    per-(head, channel) scales: attention kernel and whole call (chunk store
    as codes, the rows dequantized to codes in bf16, attention)."""
    import torch
    P, S = 3072, 1024
    case = W.chunk_case("chunk_int8", 1, 32, 32, S, 128, torch.bfloat16, [P], 571, dev,
                        paged=False, max_seq=P + S)
    ck = W.randcodes((1, 32, P + S, 128), dev, 572, 0)
    cv = W.randcodes((1, 32, P + S, 128), dev, 572, 1)
    cache = car.KVCache(ck, cv, k_scale=W.randscales((32, 128), dev, 572, 2),
                        v_scale=W.randscales((32, 128), dev, 572, 3))
    o = torch.empty_like(case.q)
    ws = torch.empty(car.prefill_cached_workspace_bytes(torch.bfloat16, 1, 32, 128, P + S, cache),
                     dtype=torch.uint8, device=dev)

    def call(timing=None):
        car.attn_prefill_cached(case.q, case.k, case.v, case.seq_lens, cache, P + S,
                                case.theta, case.scale, out=o, timing=timing, workspace=ws)
    for _ in range(3):
        call()
    pairs_k, pairs_c = timed_calls(car, call, stream, new_event, iters)
    if not torch.isfinite(o.float()).all():
        raise RuntimeError("non-finite output in the INT8 chunk")
    ksp = spread([a.elapsed_time(b) for a, b in pairs_k])
    csp = spread([a.elapsed_time(b) for a, b in pairs_c])
    fl = chunk_flops(1, 32, P, S, 128)
    return {"chunked_prefill_int8_contiguous": {
        "workload": f"B=1,Hq=32,Hkv=32,D=128,cached={P},chunk={S},bf16 q/k/v, INT8 contiguous "
                    "cache 4096 with per-(head, channel) scales",
        "kernel_ms": sum(a.elapsed_time(b) for a, b in pairs_k) / iters,
        "call_ms": sum(a.elapsed_time(b) for a, b in pairs_c) / iters,
        "kernel_spread_ms": ksp, "call_spread_ms": csp,
        "TFLOPs_kernel_median": fl / (ksp["median"] * 1e-3) / 1e12,
        "TFLOPs_call_median": fl / (csp["median"] * 1e-3) / 1e12,
        "mfma_frac_kernel_median": fl / (ksp["median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "per_launch": f"{fl} flops (4*B*H*D*(S*P + S(S+1)/2))"}}


def measure_int8_decode(car, W, dev, stream, new_event, iters: int = 100) -> dict:
    """The two decode workloads with INT8 caches of the same shapes (codes in
    [-127, 127], per-(KV head, channel) fp32 scales): event times of the
    decode split kernel and of the whole call, and KV GB/s at one byte per
    cached element."""
    import torch
    out = {}
    specs = (("contiguous", dict(B=32, Hq=32, Hkv=32, lens=W.contiguous_decode_lens(),
                                 seed=W.BASE_SEED + 3, paged=False, max_seq=4096)),
             ("paged_gqa", dict(B=64, Hq=32, Hkv=8, lens=W.paged_decode_lens(),
                                seed=W.BASE_SEED + 4, paged=True, blocks_per_seq=513)))
    for name, sp in specs:
        extra = {k: sp[k] for k in ("max_seq", "blocks_per_seq") if k in sp}
        case = W.int8_decode_case(f"int8_{name}", sp["B"], sp["Hq"], sp["Hkv"], 128,
                                  torch.bfloat16, sp["lens"], sp["seed"], dev,
                                  paged=sp["paged"], **extra)
        cache = car.KVCache(case.cache_k, case.cache_v, case.block_table,
                            k_scale=case.k_scale, v_scale=case.v_scale)
        o = torch.empty_like(case.q)
        ws = torch.empty(car.decode_workspace_bytes(case.B, case.Hq, 128, case.max_seq_len),
                         dtype=torch.uint8, device=dev)

        def call(timing=None):
            car.attn_decode(case.q, case.k_new, case.v_new, case.seq_lens, cache,
                            case.max_seq_len, case.theta, case.scale, out=o, workspace=ws,
                            timing=timing)
        for _ in range(3):
            call()
        pairs_k, pairs_c = timed_calls(car, call, stream, new_event, iters)
        if not torch.isfinite(o.float()).all():
            raise RuntimeError(f"non-finite output in int8 decode ({name})")
        kms = sum(a.elapsed_time(b) for a, b in pairs_k) / iters
        cms = sum(a.elapsed_time(b) for a, b in pairs_c) / iters
        kv = decode_kv_bytes(case.lens_host, case.Hkv, 128, 1)
        out[f"int8_decode_{name}"] = {
            "workload": (f"B={case.B},Hq={case.Hq},Hkv={case.Hkv},D=128,bf16 q/k/v,"
                         + ("paged 16-token blocks" if sp["paged"] else "contiguous 4096")
                         + ", int8 cache with per-(head, channel) scales"),
            "kernel_ms": kms, "call_ms": cms,
            "kernel_spread_ms": spread([a.elapsed_time(b) for a, b in pairs_k]),
            "call_spread_ms": spread([a.elapsed_time(b) for a, b in pairs_c]),
            "GBps_kernel": kv / (kms * 1e-3) / 1e9, "GBps_call": kv / (cms * 1e-3) / 1e9,
            "hbm_frac_kernel": kv / (kms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "tokens_per_s": case.B / (cms * 1e-3),
            "per_launch": f"{kv} bytes (sum_b L_b * Hkv * D * 2 (K,V) * 1 B)"}
        del case, cache, o, ws
        torch.cuda.synchronize()
    return out


def measure_small_prefills(car, W, dev, stream, new_event, iters: int = 100) -> dict:
    """The two small workloads.  GPT-2-shaped prefill (B=4, H=12, D=64,
    S=512, bf16, no cache): TFLOP/s against the bf16 peak and, since at 128
    flop per byte it sits below the ridge, its bytes (q, k, v read, out
    written) against the HBM peak.  The fp32 tiny case (B=1, H=4, D=64:
    a 128-token prefill into a 144-slot cache, then 16 decode steps at
    positions 128..143) as one sequence of 17 calls: its total time, the
    prefill's TFLOP/s and the decode steps' tokens/s.  Both are launch-bound
    sizes; the kernel time is the attention kernel's, the call time the
    whole entry point's."""
    import torch
    out = {}
    c2 = W.gpt2_prefill(dev)
    o2 = torch.empty_like(c2.q)
    ws2 = torch.empty(car.prefill_workspace_bytes(torch.bfloat16, c2.B, c2.Hkv, c2.S, c2.D),
                      dtype=torch.uint8, device=dev)

    def call2(timing=None):
        car.attn_prefill(c2.q, c2.k, c2.v, c2.positions, c2.theta, c2.scale, out=o2,
                         workspace=ws2, timing=timing)
    for _ in range(3):
        call2()
    pairs_k, pairs_c = timed_calls(car, call2, stream, new_event, iters)
    if not torch.isfinite(o2.float()).all():
        raise RuntimeError("non-finite output in the GPT-2-shaped prefill")
    ksp = spread([a.elapsed_time(b) for a, b in pairs_k])
    csp = spread([a.elapsed_time(b) for a, b in pairs_c])
    kms, cms = ksp["median"], csp["median"]
    fl = prefill_flops(c2.B, c2.Hq, c2.S, c2.D)
    io = 4 * c2.B * c2.Hq * c2.S * c2.D * 2
    out["gpt2_prefill"] = {
        "workload": "B=4,H=12,D=64,S=512,bf16, no cache",
        "kernel_ms": kms, "call_ms": cms, "kernel_spread_ms": ksp, "call_spread_ms": csp,
        "TFLOPs_kernel": fl / (kms * 1e-3) / 1e12, "TFLOPs_call": fl / (cms * 1e-3) / 1e12,
        "mfma_frac_kernel": fl / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "hbm_frac_kernel": io / (kms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "per_launch": f"{fl} flops (2*B*H*D*S*(S+1)); {io} bytes (q, k, v, out)"}
    del c2, o2, ws2

    pre, steps = W.tiny(dev)
    cache = car.KVCache(torch.zeros((1, 4, 144, 64), dtype=torch.float32, device=dev),
                        torch.zeros((1, 4, 144, 64), dtype=torch.float32, device=dev))
    o1 = torch.empty_like(pre.q)
    ws1 = torch.empty(car.prefill_workspace_bytes(torch.float32, 1, 4, 128, 64),
                      dtype=torch.uint8, device=dev)
    od = torch.empty_like(steps[0][0])
    wsd = torch.empty(car.decode_workspace_bytes(1, 4, 64, 144), dtype=torch.uint8, device=dev)
    lens = [torch.tensor([128 + t], dtype=torch.int32, device=dev) for t in range(16)]

    def seq1(ev=None):
        if ev is not None:
            ev[0].record(stream)
        car.attn_prefill(pre.q, pre.k, pre.v, pre.positions, pre.theta, pre.scale,
                         cache=cache, out=o1, workspace=ws1)
        if ev is not None:
            ev[1].record(stream)
        for t, (q, kn, vn) in enumerate(steps):
            car.attn_decode(q, kn, vn, lens[t], cache, 144, pre.theta, pre.scale, out=od,
                            workspace=wsd)
        if ev is not None:
            ev[2].record(stream)
    for _ in range(3):
        seq1()
    evs = [tuple(new_event() for _ in range(3)) for _ in range(iters)]
    for i in range(iters):
        seq1(evs[i])
    torch.cuda.synchronize()
    if not (torch.isfinite(o1).all() and torch.isfinite(od).all()):
        raise RuntimeError("non-finite output in the fp32 tiny workload")
    psp = spread([a.elapsed_time(b) for a, b, _ in evs])
    dsp = spread([b.elapsed_time(c) for _, b, c in evs])
    pms, dms = psp["median"], dsp["median"]
    fl1 = prefill_flops(1, 4, 128, 64)
    out["tiny_prefill_decode_fp32"] = {
        "workload": "B=1,H=4,D=64,fp32: prefill S=128 into a 144-slot cache, then 16 decode "
                    "steps at positions 128..143",
        "total_ms": pms + dms, "prefill_call_ms": pms, "decode_16_steps_ms": dms,
        "prefill_call_spread_ms": psp, "decode_16_steps_spread_ms": dsp,
        "prefill_TFLOPs_call": fl1 / (pms * 1e-3) / 1e12,
        "decode_tokens_per_s": 16 / (dms * 1e-3),
        "per_launch": f"prefill {fl1} flops (2*B*H*D*S*(S+1)); each step reads L*4*64*2*4 B"}
    return out


def measure_varlen_prefill(car, W, dev, stream, new_event, iters: int = 100) -> dict:
    """A padded batch of whole prompts (B=8, H=32, D=128, bf16, lengths
    U{128..2048} padded to S=2048, positions from 0, a contiguous cache
    [8, 32, 2048, 128]): event times of the attention kernel and of the whole
    call (K pass with the cache store, then attention), TFLOP/s of the
    prompts' own causal work against the bf16 peak."""
    import torch
    case, lens = W.varlen_prefill(dev)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    cache = car.KVCache(torch.zeros((8, 32, 2048, 128), dtype=torch.bfloat16, device=dev),
                        torch.zeros((8, 32, 2048, 128), dtype=torch.bfloat16, device=dev))
    o = torch.empty_like(case.q)
    ws = torch.empty(car.prefill_workspace_bytes(torch.bfloat16, 8, 32, 2048, 128),
                     dtype=torch.uint8, device=dev)

    def call(timing=None):
        car.attn_prefill(case.q, case.k, case.v, case.positions, case.theta, case.scale,
                         cache=cache, out=o, workspace=ws, timing=timing, seq_lens=seq_lens)
    for _ in range(3):
        call()
    pairs_k, pairs_c = timed_calls(car, call, stream, new_event, iters)
    if not torch.isfinite(o.float()).all():
        raise RuntimeError("non-finite output in the padded prompt batch")
    ksp = spread([a.elapsed_time(b) for a, b in pairs_k])
    csp = spread([a.elapsed_time(b) for a, b in pairs_c])
    fl = sum(prefill_flops(1, 32, n, 128) for n in lens)
    return {"varlen_prefill": {
        "workload": f"B=8,H=32,D=128,bf16, prompts of {lens} tokens padded to 2048, "
                    "contiguous cache [8,32,2048,128]",
        "kernel_ms": sum(a.elapsed_time(b) for a, b in pairs_k) / iters,
        "call_ms": sum(a.elapsed_time(b) for a, b in pairs_c) / iters,
        "kernel_spread_ms": ksp, "call_spread_ms": csp,
        "TFLOPs_kernel_median": fl / (ksp["median"] * 1e-3) / 1e12,
        "TFLOPs_call_median": fl / (csp["median"] * 1e-3) / 1e12,
        "mfma_frac_kernel_median": fl / (ksp["median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "per_launch": f"{fl} flops (sum_b 2*H*D*n_b*(n_b+1) over the prompts' own tokens)"}}


def measure_rope_append(car, pf, dev, stream, new_event, iters: int) -> dict:
    """The standalone rope_apply (in place on the prompt's keys) and
    kv_cache_append (rotated keys and values into a cache of the prompt's
    shape) at the Qwen-shaped prompt (B=1, H=32, S=4096, D=128, bf16): event
    times of each call (one kernel each) and GB/s of the bytes each must move
    against the HBM peak."""
    import torch
    x = pf.k.clone()
    ck = torch.empty_like(pf.k)
    cv = torch.empty_like(pf.v)
    cache = car.KVCache(ck, cv)
    elems = x.numel()
    pos_bytes = pf.positions.numel() * 4
    specs = (
        ("rope_apply", lambda: car.rope_apply(x, pf.positions, pf.theta),
         2 * elems * 2 + pos_bytes, "K read and written in place"),
        ("kv_cache_append", lambda: car.kv_cache_append(cache, x, pf.v, pf.positions),
         4 * elems * 2 + pos_bytes, "K and V read, K and V rows written"))
    out = {}
    for name, fn, nbytes, what in specs:
        for _ in range(3):
            fn()
        pairs = [(new_event(), new_event()) for _ in range(iters)]
        for a, b in pairs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        sp = spread([a.elapsed_time(b) for a, b in pairs])
        gbps = nbytes / (sp["median"] * 1e-3) / 1e9
        out[f"{name}_qwen"] = {
            "workload": "B=1,H=32,S=4096,D=128,bf16" + (", contiguous cache 4096"
                                                        if name != "rope_apply" else ""),
            "call_spread_ms": sp, "GBps_median": gbps, "hbm_frac_median": gbps / PEAK_HBM_GBPS,
            "per_launch": f"{nbytes} bytes ({what}, plus int32 positions)"}
    if not torch.isfinite(x.float()).all():
        raise RuntimeError("non-finite keys after rope_apply")
    return out


def main(argv=None) -> int:
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import causal_attention_rope_amd as car
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    stages = ["prefill", "contiguous", "paged"] if args.only is None else [args.only]

    # ---------------- inputs, resident in HBM ----------------
    pf = W.qwen_prefill(dev)
    c4 = W.contiguous_decode(dev)
    c5 = W.paged_decode(dev)
    pf_cache = car.KVCache(torch.zeros((1, 32, 4096, 128), dtype=torch.bfloat16, device=dev),
                           torch.zeros((1, 32, 4096, 128), dtype=torch.bfloat16, device=dev))
    pf_out = torch.empty_like(pf.q)
    # keys into a contiguous bf16 cache the prompt fits: no workspace (the
    # attention reads the rotated keys back from the cache)
    assert car.prefill_workspace_bytes(torch.bfloat16, 1, 32, 4096, 128, cache=pf_cache) == 0
    c4_cache = car.KVCache(c4.cache_k, c4.cache_v)
    c5_cache = car.KVCache(c5.cache_k, c5.cache_v, c5.block_table)
    c4_out, c5_out = torch.empty_like(c4.q), torch.empty_like(c5.q)
    c4_ws = torch.empty(car.decode_workspace_bytes(c4.B, c4.Hq, c4.D, c4.max_seq_len),
                        dtype=torch.uint8, device=dev)
    c5_ws = torch.empty(car.decode_workspace_bytes(c5.B, c5.Hq, c5.D, c5.max_seq_len),
                        dtype=torch.uint8, device=dev)

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)  # creates the underlying HIP event
        return e

    n_ev = args.steps
    ev = {s: {"call": [(new_event(), new_event()) for _ in range(n_ev)],
              "kernel": [(new_event(), new_event()) for _ in range(n_ev)]} for s in stages}

    def stage_call(s, timing=None):
        if s == "prefill":
            car.attn_prefill(pf.q, pf.k, pf.v, pf.positions, pf.theta, pf.scale,
                             cache=pf_cache, out=pf_out, no_workspace=True, timing=timing)
        elif s == "contiguous":
            car.attn_decode(c4.q, c4.k_new, c4.v_new, c4.seq_lens, c4_cache, c4.max_seq_len,
                            c4.theta, c4.scale, out=c4_out, workspace=c4_ws, timing=timing)
        else:
            car.attn_decode(c5.q, c5.k_new, c5.v_new, c5.seq_lens, c5_cache, c5.max_seq_len,
                            c5.theta, c5.scale, out=c5_out, workspace=c5_ws, timing=timing)

    def run_stage(s, i=None, kernel_events=False):
        # call events bracket the whole entry point; with kernel_events the
        # library brackets its main kernel instead (separate iterations, so
        # that the inner events add nothing to the call times)
        timing = ev[s]["kernel"][i] if (i is not None and kernel_events) else None
        if i is not None and not kernel_events:
            ev[s]["call"][i][0].record(stream)
        stage_call(s, timing)
        if i is not None and not kernel_events:
            ev[s]["call"][i][1].record(stream)

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # clocks: the same stages, untimed, for CLOCK_WARM_S seconds before the
    # warmup steps, so that the timed steps do not start at idle clocks
    t_end = time.perf_counter() + CLOCK_WARM_S
    while time.perf_counter() < t_end:
        for s in stages:
            run_stage(s)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        for s in stages:
            run_stage(s)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        for s in stages:
            run_stage(s, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    # the same steps again, untimed as a whole, for the per-kernel event times
    for i in range(args.steps):
        for s in stages:
            run_stage(s, i, kernel_events=True)
    torch.cuda.synchronize()

    def avg_ms(pairs):
        return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)

    res = {}
    for s in stages:
        res[s] = {"call_ms": avg_ms(ev[s]["call"]), "kernel_ms": avg_ms(ev[s]["kernel"])}

    # ---------------- spreads: median / p10 / p90 over stat_iters iterations ----------------
    # call times back to back; kernel times alone; for the decode steps also
    # the kernel after 512 MiB of writes (more than the 256 MiB Infinity
    # Cache), outside the timed region, so that no KV byte is served from it
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    n_stat = max(args.stat_iters, 1)
    for s in stages:
        calls = [(new_event(), new_event()) for _ in range(n_stat)]
        kerns = [(new_event(), new_event()) for _ in range(n_stat)]
        cold = [(new_event(), new_event()) for _ in range(n_stat)] if s != "prefill" else []
        for a, b in calls:
            a.record(stream)
            stage_call(s)
            b.record(stream)
        for pair in kerns:
            stage_call(s, pair)
        for i, pair in enumerate(cold):
            flush.fill_(i & 0xFF)
            stage_call(s, pair)
        torch.cuda.synchronize()
        res[s]["call_spread_ms"] = spread([a.elapsed_time(b) for a, b in calls])
        res[s]["kernel_spread_ms"] = spread([a.elapsed_time(b) for a, b in kerns])
        if cold:
            res[s]["kernel_cold_spread_ms"] = spread([a.elapsed_time(b) for a, b in cold])
    del flush

    outs = {"prefill": pf_out, "contiguous": c4_out, "paged": c5_out}
    for s in stages:
        if not torch.isfinite(outs[s].float()).all():
            print(f"non-finite output in stage {s}", file=sys.stderr)
            return 1

    # ---------------- chunked prefill (outside the timed step) ----------------
    extras = {}
    if args.only is None and not args.no_extras:
        extras = measure_chunked(car, W, dev, stream, new_event, n_stat)
        extras.update(measure_int8_decode(car, W, dev, stream, new_event, n_stat))
        extras.update(measure_int8_chunk(car, W, dev, stream, new_event, n_stat))
        extras.update(measure_small_prefills(car, W, dev, stream, new_event, n_stat))
        extras.update(measure_varlen_prefill(car, W, dev, stream, new_event, n_stat))
        extras.update(measure_rope_append(car, pf, dev, stream, new_event, n_stat))

    # ---------------- figures ----------------
    kernels = {}
    pf_flops = prefill_flops(pf.B, pf.Hq, pf.S, pf.D)
    line_extra = {}
    if "prefill" in res:
        r = res["prefill"]
        r["TFLOPs_call"] = pf_flops / (r["call_ms"] * 1e-3) / 1e12
        r["TFLOPs_kernel"] = pf_flops / (r["kernel_ms"] * 1e-3) / 1e12
        r["TFLOPs_kernel_median"] = pf_flops / (r["kernel_spread_ms"]["median"] * 1e-3) / 1e12
        r["TFLOPs_call_median"] = pf_flops / (r["call_spread_ms"]["median"] * 1e-3) / 1e12
        kernels["prefill_attention"] = {
            "bound": "mfma", "achieved": r["TFLOPs_kernel"], "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": r["TFLOPs_kernel"] / PEAK_BF16_TFLOPS,
            "traffic": None, "avg_us": r["kernel_ms"] * 1e3,
            "per_launch": f"{pf_flops} flops (2*B*H*D*S*(S+1), B=1 H=32 D=128 S=4096)"}
    for s, c in (("contiguous", c4), ("paged", c5)):
        if s not in res:
            continue
        r = res[s]
        kv = decode_kv_bytes(c.lens_host, c.Hkv, c.D, 2)
        r["GBps_call"] = kv / (r["call_ms"] * 1e-3) / 1e9
        r["GBps_kernel"] = kv / (r["kernel_ms"] * 1e-3) / 1e9
        r["tokens_per_s"] = c.B / (r["call_ms"] * 1e-3)
        r["hbm_frac_call"] = r["GBps_call"] / PEAK_HBM_GBPS
        r["kv_bytes"] = kv
        r["io_bytes"] = decode_io_bytes(c.B, c.Hq, c.Hkv, c.D, 2)
        r["GBps_kernel_median"] = kv / (r["kernel_spread_ms"]["median"] * 1e-3) / 1e9
        if "kernel_cold_spread_ms" in r:
            r["GBps_kernel_cold_median"] = (kv / (r["kernel_cold_spread_ms"]["median"] * 1e-3)
                                            / 1e9)
        kernels[f"decode_{s}_split"] = {
            "bound": "hbm", "achieved": r["GBps_kernel"], "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": r["GBps_kernel"] / PEAK_HBM_GBPS, "traffic": None,
            "avg_us": r["kernel_ms"] * 1e3,
            "per_launch": f"{kv} bytes (sum_b L_b * Hkv * D * 2 (K,V) * 2 B)"}

    traffic = measured_traffic()
    for name, k in kernels.items():
        t = traffic.get(name)
        k["traffic"] = None if t is None else t["fetch_bytes"] + t["write_bytes"]
    for name, e in extras.items():
        t = traffic.get(name)
        e["traffic"] = None if t is None else t["fetch_bytes"] + t["write_bytes"]

    dominant = max(kernels, key=lambda k: kernels[k]["avg_us"])
    roofline = {k: v for k, v in kernels[dominant].items() if k in
                ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roofline["kernel"] = dominant

    if "prefill" in res:
        value, unit = res["prefill"]["TFLOPs_call"], "TFLOP/s"
    elif "contiguous" in res:
        value, unit = res["contiguous"]["GBps_call"], "GB/s"
    else:
        value, unit = res["paged"]["GBps_call"], "GB/s"

    line = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "+".join(
                {"prefill": "qwen_prefill(B=1,H=32,D=128,S=4096,cache 4096)",
                 "contiguous": "contiguous_decode(B=32,H=32,D=128,L~U[1,4095])",
                 "paged": "paged_decode(B=64,Hq=32,Hkv=8,D=128,block 16,L~U[512,8192])"}[s]
                for s in stages),
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "stages": res,
        "kernels": kernels,
        "prefill_mfma_frac_call": (res["prefill"]["TFLOPs_call"] / PEAK_BF16_TFLOPS
                                   if "prefill" in res else None),
    }
    line.update(line_extra)
    if extras:
        line["extras"] = extras
    if not args.no_cpu_baseline and args.only is None:
        line["cpu_baseline"] = cpu_baseline(pf, c4, args.cpu_heads, args.cpu_heads_1t)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
