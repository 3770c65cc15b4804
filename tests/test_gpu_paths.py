"""GPU parity of kernel paths that only long blocks or strided inputs reach.

* The forward kernel classifies a block's key tiles in segments of 4,096
  tiles of 64 keys (262,144 keys); a longer block is walked segment by
  segment. One step over 300,000 keys takes two segments.
* The backward dQ kernel classifies key tiles in segments of 2,048 tiles of
  32 keys (65,536 keys): a block of 70,000 keys takes two. (The million-token
  share's blocks of 131,072 keys take this path too.)
* The backward dK/dV kernel classifies query tiles in segments of 4,096 tiles
  of 32 queries (131,072 queries): 140,000 queries take two.
* Q, K, V, O and dO views of a [B, S, H, D] tensor (sequence-major, heads
  interleaved) permuted to [B, H, S, D]: row stride H * D instead of D.

Every case is compared with the fp64 oracle on the same bf16 (or float32)
values: forward O max-abs <= 2e-2 and LSE max-abs <= 1e-3 for bf16, 1e-5 for
float32; gradients max|g - g_ref| <= 1e-2 * max|g_ref| for bf16, 1e-5 for
float32 (the backward tests' normwise bar), rows with nothing allowed exactly
zero. Strided inputs must also give the same bits as contiguous copies.
"""

import numpy as np
import pytest
import torch

import oracle
import context_ring_attention_zigzag_amd as cpr
from context_ring_attention_zigzag_amd import device_inputs as di

pytestmark = pytest.mark.gpu

TOL_FWD = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-5)}
TOL_BWD = {"bf16": 1e-2, "f32": 1e-5}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpr.load()
    yield


def note(msg):
    print(f"[gpu-paths] {msg}", flush=True)


def rounded(x, dtype="bf16"):
    """(device tensor of dtype, float64 host copy of exactly those values)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(TDT[dtype])
    return t.cuda(), t.float().numpy().astype(np.float64)


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def compare_fwd(o, lse, ro, rl, dtype, what):
    tol_o, tol_l = TOL_FWD[dtype]
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl)), f"{what}: -inf LSE pattern differs"
    fin = np.isfinite(rl)
    err_l = float(np.abs(lse[fin] - rl[fin]).max()) if fin.any() else 0.0
    err_o = float(np.abs(o - ro).max())
    note(f"{what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert np.isfinite(o).all()
    assert err_o <= tol_o and err_l <= tol_l, (what, err_o, err_l)


def check_grad(got, ref, dtype, what, zero=None):
    ref_max = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    note(f"{what}: max|err|={err:.3e} max|ref|={ref_max:.3e} ratio={err / max(ref_max, 1e-30):.3e}")
    assert np.isfinite(got).all(), what
    assert err <= TOL_BWD[dtype] * ref_max + 1e-30, (what, err, ref_max)
    if zero is not None and zero.any():
        assert np.all(got[zero] == 0), f"{what}: rows with nothing allowed are not zero"


# ------------------------------------------------------- forward, two key segments

@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("variant", ["window", "late_queries"])
def test_step_block_over_two_key_segments(d, variant):
    """init, one step over a block of 300,000 keys (two classification segments), finalize.

    window: 256 queries spread over the whole block, causal, each limited to the keys within 200,000
    positions below it: every tile needs the element mask, in both segments.
    late_queries: 256 queries at positions >= 290,000, causal: the tiles below them are full in both
    segments, the last ones masked."""
    rng = np.random.default_rng(400 + d + (0 if variant == "window" else 1))
    B, H, Lq, Lk = 1, 2, 256, 300_000
    kpos = np.arange(Lk, dtype=np.int64)
    lo = hi = None
    if variant == "window":
        qpos = np.sort(rng.choice(Lk, size=Lq, replace=False))
        lo = qpos - 200_000
        hi = qpos - rng.integers(0, 3, size=Lq)   # a few queries stop short of their own position
    else:
        qpos = np.sort(rng.choice(np.arange(290_000, Lk), size=Lq, replace=False))
    q_d, q_h = rounded(rng.standard_normal((B, H, Lq, d)))
    k_d, k_h = rounded(rng.standard_normal((B, H, Lk, d)))
    v_d, v_h = rounded(rng.standard_normal((B, H, Lk, d)))
    note(f"forward step {variant} D={d}: Lq={Lq} Lk={Lk}")
    o_acc = torch.empty(B, H, Lq, d, device="cuda")
    m = torch.empty(B, H, Lq, device="cuda")
    l = torch.empty(B, H, Lq, device="cuda")
    cpr.cp_ring_attn_init(o_acc, m, l)
    kw = {} if lo is None else dict(kw_lo=i32(lo), kw_hi=i32(hi))
    cpr.cp_ring_attn_step(q_d, i32(qpos), k_d, v_d, i32(kpos), True, 0.0, o_acc, m, l, **kw)
    o = torch.empty(B, H, Lq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, Lq, device="cuda")
    cpr.cp_ring_attn_finalize(o_acc, m, l, o, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.full_attention(q_h, k_h, v_h, qpos, kpos, True, kw_lo=lo, kw_hi=hi)
    compare_fwd(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", f"step {variant} D={d}")


# ------------------------------------------------- backward, two segments per kernel

def bwd_inputs(rng, B, H, Lq, Lk, d, qpos, kpos):
    """Seeded bf16 inputs, the oracle's forward O (rounded to bf16) and LSE (rounded to float32)."""
    q_d, q_h = rounded(rng.standard_normal((B, H, Lq, d)))
    k_d, k_h = rounded(rng.standard_normal((B, H, Lk, d)))
    v_d, v_h = rounded(rng.standard_normal((B, H, Lk, d)))
    g_d, g_h = rounded(rng.standard_normal((B, H, Lq, d)))
    o, lse = oracle.full_attention(q_h, k_h, v_h, qpos, kpos, True, row_chunk=512)
    o_d, o_h = rounded(o)
    lse32 = lse.astype(np.float32)
    return dict(q=(q_d, q_h), k=(k_d, k_h), v=(v_d, v_h), do=(g_d, g_h), o=(o_d, o_h),
                lse=(torch.from_numpy(lse32).cuda(), lse32.astype(np.float64)))


def bwd_step_gpu(x, qpos, kpos):
    q_d, g_d, o_d, lse_d = x["q"][0], x["do"][0], x["o"][0], x["lse"][0]
    k_d, v_d = x["k"][0], x["v"][0]
    B, H, Lq, _ = q_d.shape
    ws = torch.empty(cpr.cp_ring_attn_bwd_workspace_size(B, H, Lq), dtype=torch.uint8, device="cuda")
    cpr.cp_ring_attn_bwd_prep(o_d, g_d, lse_d, i32(qpos), True, ws)
    dq = torch.zeros(q_d.shape, device="cuda")
    dk = torch.zeros(k_d.shape, device="cuda")
    dv = torch.zeros(v_d.shape, device="cuda")
    cpr.cp_ring_attn_bwd_step(q_d, g_d, k_d, v_d, i32(kpos), 0.0, ws, dq, dk, dv)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


@pytest.mark.parametrize("d", [128, 64])
def test_bwd_step_dq_over_two_key_segments(d):
    """256 causal queries spread over a block of 70,000 keys: the dQ kernel walks two key segments. dQ of
    every query, dK and dV of every key, against the oracle's backward."""
    rng = np.random.default_rng(410 + d)
    B, H, Lq, Lk = 1, 2, 256, 70_000
    kpos = np.arange(Lk)
    qpos = np.sort(rng.choice(Lk, size=Lq, replace=False))
    qpos[-8:] = Lk - 8 + np.arange(8)   # some queries see the whole block
    x = bwd_inputs(rng, B, H, Lq, Lk, d, qpos, kpos)
    note(f"backward dQ two segments D={d}: Lq={Lq} Lk={Lk}")
    dq, dk, dv = bwd_step_gpu(x, qpos, kpos)
    for h in range(H):
        rq, rk, rv = oracle.rows_backward(x["q"][1][0, h], x["k"][1][0, h], x["v"][1][0, h], x["o"][1][0, h],
                                          x["do"][1][0, h], x["lse"][1][0, h], qpos, kpos, True,
                                          q_rows=np.arange(Lq), k_rows=np.arange(Lk))
        dead_k = kpos > qpos.max()
        check_grad(dq[0, h], rq, "bf16", f"dQ 2-seg D={d} h{h}")
        check_grad(dk[0, h], rk, "bf16", f"dK 2-seg D={d} h{h}", dead_k)
        check_grad(dv[0, h], rv, "bf16", f"dV 2-seg D={d} h{h}", dead_k)


@pytest.mark.parametrize("d", [128, 64])
def test_bwd_step_dkv_over_two_query_segments(d):
    """140,000 causal queries against a block of 256 keys spread over their positions: the dK/dV kernel
    walks two query segments. dK and dV of every key, dQ of sampled queries, against the oracle."""
    rng = np.random.default_rng(420 + d)
    B, H, Lq, Lk = 1, 2, 140_000, 256
    qpos = np.arange(Lq)
    kpos = np.sort(rng.choice(Lq, size=Lk, replace=False))
    kpos[:4] = np.arange(4)             # keys every query segment attends
    x = bwd_inputs(rng, B, H, Lq, Lk, d, qpos, kpos)
    note(f"backward dK/dV two segments D={d}: Lq={Lq} Lk={Lk}")
    dq, dk, dv = bwd_step_gpu(x, qpos, kpos)
    q_rows = np.unique(np.concatenate([np.arange(16), np.arange(131_060, 131_090), Lq - 16 + np.arange(16),
                                       rng.integers(0, Lq, size=64)]))
    for h in range(H):
        rq, rk, rv = oracle.rows_backward(x["q"][1][0, h], x["k"][1][0, h], x["v"][1][0, h], x["o"][1][0, h],
                                          x["do"][1][0, h], x["lse"][1][0, h], qpos, kpos, True,
                                          q_rows=q_rows, k_rows=np.arange(Lk))
        check_grad(dq[0, h, q_rows], rq, "bf16", f"dQ(sampled) 2-seg D={d} h{h}", qpos[q_rows] < kpos.min())
        check_grad(dk[0, h], rk, "bf16", f"dK 2-seg D={d} h{h}")
        check_grad(dv[0, h], rv, "bf16", f"dV 2-seg D={d} h{h}")


# ------------------------------------------------------------- strided views

def bshd(t):
    """The same values in a [B, S, H, D] buffer, returned as its [B, H, S, D] permuted view (row stride H * D)."""
    B, H, L, D = t.shape
    x = torch.empty((B, L, H, D), dtype=t.dtype, device=t.device).permute(0, 2, 1, 3)
    x.copy_(t)
    assert x.stride(2) == H * D and not x.is_contiguous()
    return x


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_strided_views_run_step_and_backward(dtype, d):
    """Sequence-major inputs permuted to [B, H, S, D] through run (fused, stepwise), step and bwd_run: the
    same bits as contiguous copies, and the oracle's result."""
    rng = np.random.default_rng(430 + d + (0 if dtype == "bf16" else 1))
    B, H, S, cp, rank = 2, 4, 1998, 2, 1
    nat = {t: rounded(rng.standard_normal((B, H, S, d)), dtype) for t in ("q", "k", "v", "do")}
    ri = di.prepare_rank(nat["q"][0], nat["k"][0], nat["v"][0], S, cp, cpr.ZIGZAG, rank)
    lq = ri.lq
    qs, ks, vs = bshd(ri.q_local), bshd(ri.k_ring), bshd(ri.v_ring)
    note(f"strided {dtype} D={d}: B={B} H={H} S={S} cp={cp} rank={rank}")

    def run(q, k, v, flags):
        o = torch.empty(ri.q_local.shape, dtype=TDT[dtype], device="cuda")
        lse = torch.empty(ri.q_local.shape[:3], device="cuda")
        ws = torch.empty(cpr.cp_ring_attn_workspace_size(B, H, lq, d), dtype=torch.uint8, device="cuda")
        cpr.cp_ring_attn_run(q, ri.q_pos, k, v, ri.ring_pos, cp, rank, True, 0.0, o, lse, ws, flags)
        return o, lse

    o_c, lse_c = run(ri.q_local, ri.k_ring, ri.v_ring, cpr.RUN_FUSED)
    for flags in (cpr.RUN_FUSED, cpr.RUN_STEPWISE):
        o_s, lse_s = run(qs, ks, vs, flags)
        o_r, lse_r = run(ri.q_local, ri.k_ring, ri.v_ring, flags)
        torch.cuda.synchronize()
        assert torch.equal(o_s, o_r) and torch.equal(lse_s, lse_r), f"run flags={flags}: strided != contiguous"

    # one step over the rank's own block, strided against contiguous
    def step(q, k, v):
        st = [torch.empty(B, H, lq, d, device="cuda"), torch.empty(B, H, lq, device="cuda"),
              torch.empty(B, H, lq, device="cuda")]
        cpr.cp_ring_attn_init(*st)
        sl = slice(rank * lq, (rank + 1) * lq)
        cpr.cp_ring_attn_step(q, ri.q_pos, k[:, :, sl], v[:, :, sl], ri.ring_pos[sl], True, 0.0, *st)
        return st
    a, b = step(qs, ks, vs), step(ri.q_local, ri.k_ring, ri.v_ring)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y), "step: strided != contiguous"

    host = {t: nat[t][1] for t in nat}
    ro, rl = oracle.rank_reference(host["q"], host["k"], host["v"], S, cp, oracle.ZIGZAG, rank, True)
    compare_fwd(o_c.float().cpu().numpy(), lse_c.cpu().numpy(), ro, rl, dtype, f"strided {dtype} D={d} forward")

    # backward with every input strided, against contiguous inputs and the oracle; O and LSE are the
    # oracle's forward results (O rounded to the dtype, LSE to float32) on both sides
    tok, pos = oracle.layout(S, cp, oracle.ZIGZAG)
    sl = slice(rank * lq, (rank + 1) * lq)
    do_local = di.gather(nat["do"][0], S, ri.token_idx[sl])
    o_in, o_in_h = rounded(ro, dtype)
    lse_in = torch.from_numpy(rl.astype(np.float32)).cuda()

    def bwd(q, k, v, o, do):
        g = [torch.empty(ri.q_local.shape, device="cuda"), torch.empty(ri.k_ring.shape, device="cuda"),
             torch.empty(ri.v_ring.shape, device="cuda")]
        ws = torch.empty(cpr.cp_ring_attn_bwd_workspace_size(B, H, lq), dtype=torch.uint8, device="cuda")
        cpr.cp_ring_attn_bwd_run(q, ri.q_pos, k, v, ri.ring_pos, cp, rank, o, do, lse_in, True, 0.0, *g, ws)
        return g
    g_s = bwd(qs, ks, vs, bshd(o_in), bshd(do_local))
    g_c = bwd(ri.q_local, ri.k_ring, ri.v_ring, o_in, do_local)
    torch.cuda.synchronize()
    for x, y, n in zip(g_s, g_c, ("dQ", "dK", "dV")):
        assert torch.equal(x, y), f"backward {n}: strided != contiguous"

    def gat(x, idx):
        out = np.zeros(x.shape[:2] + (len(idx), x.shape[-1]))
        out[:, :, idx < S] = x[:, :, idx[idx < S]]
        return out
    ref = oracle.ring_backward(gat(host["q"], tok[sl]), gat(host["k"], tok), gat(host["v"], tok),
                               o_in_h, gat(host["do"], tok[sl]),
                               rl.astype(np.float32).astype(np.float64), pos[sl], pos, cp, rank, True)
    for x, r, n in zip(g_s, ref, ("dQ", "dK", "dV")):
        check_grad(x.cpu().numpy(), r, dtype, f"strided {dtype} D={d} {n}")
