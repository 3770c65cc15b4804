"""Put natural-order inputs on the GPU and lay them out for one rank.

The layout itself is computed by the library (``cp_zigzag_partition`` builds
the token and position arrays, ``cp_shard_gather`` moves the rows); this
module only allocates device tensors and calls those two entry points.
"""

from __future__ import annotations

import dataclasses

import torch

from . import cp_padded_len, cp_shard_gather, cp_zigzag_partition


@dataclasses.dataclass
class RankInputs:
    q_local: torch.Tensor    # [B, H, Lq, D] the rank's queries
    q_pos: torch.Tensor      # [Lq] int32 global positions (-1 = pad)
    k_ring: torch.Tensor     # [B, H, S_pad, D] every rank's K block, rank-major
    v_ring: torch.Tensor     # [B, H, S_pad, D]
    ring_pos: torch.Tensor   # [S_pad] int32
    token_idx: torch.Tensor  # [S_pad] int32
    s_pad: int
    lq: int


def upload(slice_fn, B: int, H: int, S: int, D: int, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """[B, H, S, D] device tensor filled slice by slice from ``slice_fn(b, h) -> [S, D] float32 array``."""
    out = torch.empty((B, H, S, D), dtype=dtype, device=device)
    for b in range(B):
        for h in range(H):
            out[b, h].copy_(torch.from_numpy(slice_fn(b, h)).to(dtype))
    return out


def layout_arrays(seq_len: int, cp: int, layout: int, device="cuda"):
    s_pad = cp_padded_len(seq_len, cp, layout)
    if s_pad < 0:
        raise ValueError("bad layout arguments")
    tok = torch.empty(s_pad, dtype=torch.int32, device=device)
    pos = torch.empty(s_pad, dtype=torch.int32, device=device)
    cp_zigzag_partition(seq_len, cp, layout, tok, pos)
    return tok, pos


def gather(x_nat: torch.Tensor, seq_len: int, idx: torch.Tensor) -> torch.Tensor:
    B, H, _, D = x_nat.shape
    out = torch.empty((B, H, idx.numel(), D), dtype=x_nat.dtype, device=x_nat.device)
    cp_shard_gather(x_nat, seq_len, idx, out)
    return out


def prepare_rank(q_nat, k_nat, v_nat, seq_len: int, cp: int, layout: int, rank: int,
                 tok=None, pos=None) -> RankInputs:
    """Lay out natural-order Q/K/V ([B, H, seq_len, D] device tensors) for ``rank``."""
    if tok is None:
        tok, pos = layout_arrays(seq_len, cp, layout, q_nat.device)
    s_pad = tok.numel()
    lq = s_pad // cp
    sl = slice(rank * lq, (rank + 1) * lq)
    return RankInputs(q_local=gather(q_nat, seq_len, tok[sl]), q_pos=pos[sl].contiguous(),
                      k_ring=gather(k_nat, seq_len, tok), v_ring=gather(v_nat, seq_len, tok),
                      ring_pos=pos, token_idx=tok, s_pad=s_pad, lq=lq)
