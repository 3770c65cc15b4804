"""GPU check of the allocation-free whole-ring entry point (C ABI).

cp_ring_attn_run_noalloc is cp_ring_attn_run in fused mode with the key
split's partial states in the library's scratch array instead of a caller's
workspace. It must give what cp_ring_attn_run gives with a workspace (the
same kernels and the same split, so the same bits), to the bf16 bar of the
parity tests against the oracle: O max-abs <= 2e-2, LSE max-abs <= 1e-3. Two
calls in a row, the second on a smaller input, check that the scratch left by
one call does not leak into the next; a large-grid call runs unsplit.
"""

import numpy as np
import pytest
import torch

import oracle
import context_ring_attention_zigzag_amd as cpr
from context_ring_attention_zigzag_amd import device_inputs as di
from seeded_inputs import gen_tensor, small_workload

pytestmark = pytest.mark.gpu

TOL_O, TOL_L = 2e-2, 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpr.load()
    yield


def note(msg):
    print(f"[gpu-noalloc] {msg}", flush=True)


def split_engaged(B, H, lq, D):
    """The workspace query reports more than one float32 state: the fused run splits the keys."""
    rows = B * H * lq
    one = -(-rows * D * 4 // 256) * 256 + 2 * (-(-rows * 4 // 256) * 256)
    return cpr.cp_ring_attn_workspace_size(B, H, lq, D) > one


def case(w, rank):
    host = {t: gen_tensor(w, t) for t in "qkv"}
    dev = {t: torch.from_numpy(host[t]).to(torch.bfloat16).cuda() for t in "qkv"}
    ri = di.prepare_rank(dev["q"], dev["k"], dev["v"], w.S, w.cp, cpr.ZIGZAG, rank)
    ws = torch.empty(cpr.cp_ring_attn_workspace_size(w.B, w.H, ri.lq, w.D), dtype=torch.uint8, device="cuda")
    o_ws, lse_ws = torch.empty_like(ri.q_local), torch.empty(ri.q_local.shape[:3], device="cuda")
    cpr.cp_ring_attn_run(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, w.cp, rank, w.causal, 0.0, o_ws,
                         lse_ws, ws)
    o_na = torch.full_like(ri.q_local, float("nan"))
    lse_na = torch.full(ri.q_local.shape[:3], float("nan"), device="cuda")
    cpr.cp_ring_attn_run_noalloc(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, w.cp, rank, w.causal, 0.0,
                                 o_na, lse_na)
    torch.cuda.synchronize()
    a, b = o_ws.float().cpu().numpy(), o_na.float().cpu().numpy()
    la, lb = lse_ws.cpu().numpy(), lse_na.cpu().numpy()
    err_o = float(np.abs(a - b).max())
    fin = np.isfinite(la)
    err_l = float(np.abs(la[fin] - lb[fin]).max())
    note(f"{w.name} rank {rank}: split={split_engaged(w.B, w.H, ri.lq, w.D)} "
         f"max|dO| vs workspace run {err_o:.3e}, max|dLSE| {err_l:.3e}")
    assert np.isfinite(b).all()
    assert np.array_equal(np.isneginf(la), np.isneginf(lb))
    assert err_o <= TOL_O and err_l <= TOL_L
    # same kernels, same split, same inputs: the same bits
    assert np.array_equal(a, b) and np.array_equal(la[fin], lb[fin])
    # and both match the oracle
    ro, rl = oracle.rank_reference(*(host[t].astype(np.float64) for t in "qkv"), w.S, w.cp, oracle.ZIGZAG, rank,
                                   w.causal)
    assert float(np.abs(b - ro).max()) <= TOL_O
    assert float(np.abs(lb - rl).max()) <= TOL_L
    return ri


def test_noalloc_matches_workspace_run_twice_then_smaller():
    w1 = small_workload("noalloc_4k", "bf16", 1, 4, 64, 4096, 2, "zigzag", True, seed=501)
    w2 = small_workload("noalloc_1k", "bf16", 1, 2, 128, 1022, 2, "zigzag", True, seed=502)
    ri = case(w1, 0)
    assert split_engaged(w1.B, w1.H, ri.lq, w1.D)
    ri = case(w2, 1)      # smaller, ragged (padded to 1,024): the first call's partial states are still there
    assert split_engaged(w2.B, w2.H, ri.lq, w2.D)


def test_noalloc_large_grid_runs_unsplit():
    w = small_workload("noalloc_unsplit", "bf16", 2, 8, 128, 8192, 2, "zigzag", True, seed=503)
    ri = case(w, 1)
    assert not split_engaged(w.B, w.H, ri.lq, w.D)


def test_noalloc_grouped_heads_and_key_windows():
    """Grouped-query heads (4 query heads on 2 K/V heads) and sliding key windows with some empty ones, on a grid
    small enough to split: the extension argument reaches the split kernels through the scratch path too."""
    w = small_workload("noalloc_gqa_win", "bf16", 1, 4, 128, 2048, 2, "zigzag", True, seed=504)
    host = {t: gen_tensor(w, t) for t in "qkv"}
    host["k"], host["v"] = host["k"][:, :2].copy(), host["v"][:, :2].copy()
    dev = {t: torch.from_numpy(host[t]).to(torch.bfloat16).cuda() for t in "qkv"}
    t = np.arange(w.S)
    lo_nat = np.maximum(t - 300, 0).astype(np.int32)
    hi_nat = np.where(t % 9 == 4, lo_nat - 1, t).astype(np.int32)
    for rank in range(w.cp):
        ri = di.prepare_rank(dev["q"], dev["k"], dev["v"], w.S, w.cp, cpr.ZIGZAG, rank)
        assert split_engaged(w.B, w.H, ri.lq, w.D)
        tok = ri.token_idx[rank * ri.lq:(rank + 1) * ri.lq].long()
        real = tok < w.S
        kw = [torch.where(real, torch.from_numpy(nat).cuda()[tok.clamp(max=w.S - 1)], 0).to(torch.int32).contiguous()
              for nat in (lo_nat, hi_nat)]
        ws = torch.empty(cpr.cp_ring_attn_workspace_size(w.B, w.H, ri.lq, w.D), dtype=torch.uint8, device="cuda")
        o_ws, lse_ws = torch.empty_like(ri.q_local), torch.empty(ri.q_local.shape[:3], device="cuda")
        cpr.cp_ring_attn_run(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, w.cp, rank, True, 0.0, o_ws,
                             lse_ws, ws, kw_lo=kw[0], kw_hi=kw[1])
        o_na = torch.full_like(ri.q_local, float("nan"))
        lse_na = torch.full(ri.q_local.shape[:3], float("nan"), device="cuda")
        cpr.cp_ring_attn_run_noalloc(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, w.cp, rank, True, 0.0,
                                     o_na, lse_na, kw_lo=kw[0], kw_hi=kw[1])
        torch.cuda.synchronize()
        a, b = o_ws.float().cpu().numpy(), o_na.float().cpu().numpy()
        la, lb = lse_ws.cpu().numpy(), lse_na.cpu().numpy()
        note(f"{w.name} rank {rank}: bit-identical O {np.array_equal(a, b)}, LSE {np.array_equal(la, lb)}")
        assert np.array_equal(a, b) and np.array_equal(la, lb)
        ro, rl = oracle.rank_reference(*(host[x].astype(np.float64) for x in "qkv"), w.S, w.cp, oracle.ZIGZAG, rank,
                                       True, kw_lo_nat=lo_nat, kw_hi_nat=hi_nat)
        assert np.isneginf(rl).any() and np.array_equal(np.isneginf(rl), np.isneginf(lb))
        fin = np.isfinite(rl)
        assert float(np.abs(b - ro).max()) <= TOL_O
        assert float(np.abs(lb[fin] - rl[fin]).max()) <= TOL_L


def test_noalloc_rejects_bad_arguments():
    q = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(cpr.CprError) as ei:
        cpr.cp_ring_attn_run_noalloc(q, pos, q, q, pos, 1, 1, True, 0.0, torch.empty_like(q))
    assert ei.value.status == cpr.EINVAL
