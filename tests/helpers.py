"""Shared plumbing for the GPU parity tests: moving tensors to float64 numpy,
slicing cases down to sampled sequences, and the tolerances.

Tolerances (max-abs against the fp64 oracle, N(0,1) inputs): 1e-4 for fp32
inputs and 2e-2 for bf16 inputs.  Integer and byte work (cache stores of
values that are not transformed) must be bit-exact.
"""

from __future__ import annotations

import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def bits(t: torch.Tensor) -> torch.Tensor:
    """Raw bit pattern (so that NaN canaries compare equal to themselves)."""
    return t.detach().contiguous().view(torch.int32 if t.element_size() == 4 else torch.int16)


def max_abs(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    d = np.abs(a - b)
    if np.isnan(d).any():
        return float("inf")
    return float(d.max())


def log_case(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def decode_inputs_for(case, bsel):
    """float64 inputs of a decode case restricted to sequences ``bsel``.

    Returns (q, k_new, v_new, cache_k, cache_v, lens, table) where the cache
    is a contiguous slice, or for a paged case a compact pool holding only
    the blocks those sequences' tables reference, with the table renumbered.
    Taken before the GPU step runs (the step writes slot L).
    """
    bsel = list(bsel)
    q = f64(case.q[bsel])
    kn = f64(case.k_new[bsel])
    vn = f64(case.v_new[bsel])
    lens = np.array([case.lens_host[b] for b in bsel])
    if not case.paged:
        n = int(lens.max()) + 1   # slots 0..L of every selected sequence
        return (q, kn, vn, f64(case.cache_k[bsel][:, :, :n]), f64(case.cache_v[bsel][:, :, :n]),
                lens, None)
    table = case.block_table.cpu().numpy()[bsel]
    used = np.unique(table)
    remap = {int(blk): i for i, blk in enumerate(used)}
    idx = torch.as_tensor(used, device=case.cache_k.device, dtype=torch.int64)
    pk = f64(case.cache_k.index_select(0, idx))
    pv = f64(case.cache_v.index_select(0, idx))
    new_table = np.vectorize(lambda x: remap[int(x)])(table)
    return q, kn, vn, pk, pv, lens, new_table
