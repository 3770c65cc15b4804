"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws random numbers and describes workload shapes. It holds
none of the attention arithmetic, the layout or the ring schedule, and imports
neither ``oracle`` nor ``context_ring_attention_zigzag_amd``.

Recipe: every (workload seed, tensor, b, h) slice of Q, K and V is an
independent CPU ``torch.Generator`` stream of float32 N(0, 1) draws of shape
[S, D] in natural token order, multiplied by the workload's input scale, then
rounded to nearest-even bf16 for bf16 workloads. Both sides read these exact
values: the HIP side uploads them, the oracle promotes them to float64.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}   # "do": the upstream gradient dL/dO of the backward pass


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": the input and output element type
    B: int
    H: int
    D: int
    S: int              # unpadded sequence length (all ranks together)
    cp: int             # context-parallel size
    layout: str         # "zigzag", "contiguous" or "striped"
    ranks: tuple        # ranks emulated on the one GPU
    causal: bool
    input_scale: float  # N(0,1) draws are multiplied by this
    seed: int


# The five workloads: the small oracle check, the glossary page's
# 1x4x4096x64 example on 2 ranks, the 32k-token sequence over 4 ranks, a
# non-causal long-document/video stand-in over 8 ranks, and one rank's share
# of a million-token context over 8 ranks.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "f32", 1, 2, 64, 256, 2, "zigzag", (0, 1), True, 1.0, 1),
    "example_4k": Workload("example_4k", "bf16", 1, 4, 64, 4096, 2, "zigzag", (0,), True, 1.0, 2),
    "seq32k_cp4": Workload("seq32k_cp4", "bf16", 1, 32, 128, 32768, 4, "zigzag", (3,), True, 1.0, 3),
    "longdoc_noncausal": Workload("longdoc_noncausal", "bf16", 2, 16, 128, 65536, 8, "contiguous", (0,),
                                  False, 0.5, 4),
    "million_cp8": Workload("million_cp8", "bf16", 1, 8, 128, 1048576, 8, "zigzag", (0,), True, 1.0, 5),
    # the 32k-token sequence again under the striped layout (a layout variant,
    # not one of the five workloads)
    "seq32k_cp4_striped": Workload("seq32k_cp4_striped", "bf16", 1, 32, 128, 32768, 4, "striped", (3,), True, 1.0,
                                   6),
}


def slice_seed(seed: int, tensor: str, b: int, h: int) -> int:
    """Seed of one [S, D] slice; distinct for every (seed, tensor, b, h) below 2**12 batch/heads."""
    return ((seed * 4 + TENSOR_IDS[tensor]) * 4096 + b) * 4096 + h


def gen_slice(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """One [S, D] float32 slice in natural token order (bf16-exact for bf16 workloads)."""
    return gen_raw(w.S, w.D, w.dtype, w.input_scale, slice_seed(w.seed, tensor, b, h))


def gen_raw(S: int, D: int, dtype: str, input_scale: float, seed: int) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((S, D), generator=g, dtype=torch.float32)
    if input_scale != 1.0:
        x = x * input_scale
    if dtype == "bf16":
        x = x.to(torch.bfloat16).to(torch.float32)
    elif dtype != "f32":
        raise ValueError(dtype)
    return x.numpy()


def gen_tensor(w: Workload, tensor: str) -> np.ndarray:
    """The whole [B, H, S, D] float32 tensor (only for workloads that fit host memory)."""
    out = np.empty((w.B, w.H, w.S, w.D), dtype=np.float32)
    for b in range(w.B):
        for h in range(w.H):
            out[b, h] = gen_slice(w, tensor, b, h)
    return out


def small_workload(name: str, dtype: str, B: int, H: int, D: int, S: int, cp: int, layout: str,
                   causal: bool, seed: int, ranks=None, input_scale: float = 1.0) -> Workload:
    """An ad-hoc workload for tests (ragged tails, padding, edge cases)."""
    return Workload(name, dtype, B, H, D, S, cp, layout, tuple(range(cp)) if ranks is None else tuple(ranks),
                    causal, input_scale, seed)


def sample_rows(n_local: int, chunk: int, count: int, seed: int) -> np.ndarray:
    """Sorted local row indices for sampled checks: the first and last 16 rows
    of every ``chunk``-sized piece of the local sequence plus seeded uniform rows."""
    picks = set()
    for c0 in range(0, n_local, chunk):
        c1 = min(n_local, c0 + chunk)
        picks.update(range(c0, min(c1, c0 + 16)))
        picks.update(range(max(c0, c1 - 16), c1))
    rng = np.random.default_rng(seed)
    extra = max(0, count - len(picks))
    if extra:
        picks.update(int(x) for x in rng.integers(0, n_local, size=extra))
    return np.array(sorted(picks), dtype=np.int64)


def packed_windows(doc_lens):
    """Key-position windows of a packed sequence, in natural token order.

    Documents of the given lengths are packed back to back; token t of the
    document [a, a + n) may attend keys at positions [a, a + n - 1]; a causal
    bound, when wanted, is applied by the attention itself. Returns int32
    (lo, hi) arrays of sum(doc_lens) entries. Input metadata only: both the
    HIP path and the oracle consume it.
    """
    lo, hi = [], []
    a = 0
    for n in doc_lens:
        lo += [a] * n
        hi += [a + n - 1] * n
        a += n
    return np.asarray(lo, dtype=np.int32), np.asarray(hi, dtype=np.int32)
