"""GPU parity of the backward ring pass (C ABI) against the fp64 oracle.

Inputs: seeded Q, K, V and the upstream gradient dO, rounded to the kernel
dtype; O and LSE come from the oracle's forward ring pass (O rounded to the
kernel dtype, LSE to float32) and the oracle's backward takes those same
rounded values, so both sides differentiate the same thing.

Bars (normwise, per gradient tensor): max|g - g_ref| <= tol * max|g_ref|,
tol = 1e-2 for bf16 and 1e-5 for float32. The bf16 kernels round the
probabilities P and the score gradients dS to bf16 (relative error up to
2^-9 each) before the products that use them; a numpy emulation of exactly
those two roundings gives normwise errors of 1.3e-3 .. 2.8e-3 on the shapes
below, so 1e-2 keeps a margin of about 3.5x. Zero rows (pads, queries with
an empty window, keys nobody may attend) must come out exactly zero.
"""

import numpy as np
import pytest
import torch

import oracle
import context_ring_attention_zigzag_amd as cpr
from context_ring_attention_zigzag_amd import device_inputs as di
from seeded_inputs import packed_windows

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-5}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}
LAY = {"zigzag": (cpr.ZIGZAG, oracle.ZIGZAG), "contiguous": (cpr.CONTIGUOUS, oracle.CONTIGUOUS),
       "striped": (cpr.STRIPED, oracle.STRIPED)}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpr.load()
    yield


def note(msg):
    print(f"[gpu-backward] {msg}", flush=True)


def rounded(x, dtype):
    """(device tensor of dtype, float64 host copy of the same values)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(TDT[dtype])
    return t.cuda(), t.float().numpy().astype(np.float64)


def check(got, ref, dtype, what, zero_rows=None):
    """Normwise bar; rows in zero_rows (a mask over dim 2: rows with nothing allowed) must be exactly 0."""
    ref_max = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    note(f"{what}: max|err|={err:.3e} max|ref|={ref_max:.3e} ratio={err / max(ref_max, 1e-30):.3e}")
    assert np.isfinite(got).all(), what
    assert err <= TOL[dtype] * ref_max + 1e-30, f"{what}: {err} > {TOL[dtype]} * {ref_max}"
    if zero_rows is not None:
        assert np.all(got[:, :, zero_rows] == 0), f"{what}: rows with nothing allowed are not zero"


class Case:
    """Seeded natural-order inputs of one backward parity case, on host and device."""

    def __init__(self, dtype, B, H, H_kv, D, S, cp, layout, causal, seed, docs=None, scale=1.0, windows=None):
        """docs: packed-document lengths (per-query windows from them); windows: (lo, hi) per natural position."""
        rng = np.random.default_rng(seed)
        self.dtype, self.B, self.H, self.H_kv, self.D, self.S, self.cp = dtype, B, H, H_kv, D, S, cp
        self.causal = causal
        self.lay_c, self.lay_o = LAY[layout]
        self.dev, self.host = {}, {}
        for t, heads, sc in (("q", H, scale), ("k", H_kv, scale), ("v", H_kv, 1.0), ("do", H, 1.0)):
            self.dev[t], self.host[t] = rounded(rng.standard_normal((B, heads, S, D)) * sc, dtype)
        self.tok, self.pos = oracle.layout(S, cp, self.lay_o)
        self.s_pad = len(self.tok)
        self.lq = self.s_pad // cp
        self.lo_nat = self.hi_nat = None
        if docs is not None:
            self.lo_nat, self.hi_nat = packed_windows(docs)
        if windows is not None:
            self.lo_nat, self.hi_nat = (np.asarray(x, dtype=np.int64) for x in windows)

    def host_gather(self, x, idx):
        out = np.zeros(x.shape[:2] + (len(idx), x.shape[-1]))
        real = idx < self.S
        out[:, :, real] = x[:, :, idx[real]]
        return out

    def rank(self, r):
        """Everything rank r needs, on both sides."""
        sl = slice(r * self.lq, (r + 1) * self.lq)
        ltok = self.tok[sl]
        ri = di.prepare_rank(self.dev["q"], self.dev["k"], self.dev["v"], self.S, self.cp, self.lay_c, r)
        do_local = di.gather(self.dev["do"], self.S, ri.token_idx[sl])
        h = {t: self.host_gather(self.host[t], self.tok) for t in ("k", "v")}
        h["q"] = self.host_gather(self.host["q"], ltok)
        h["do"] = self.host_gather(self.host["do"], ltok)
        lo = hi = None
        kw = {}
        if self.lo_nat is not None:
            lo = np.where(ltok < self.S, self.lo_nat[np.minimum(ltok, self.S - 1)], 0)
            hi = np.where(ltok < self.S, self.hi_nat[np.minimum(ltok, self.S - 1)], 0)
            kw = dict(kw_lo=torch.from_numpy(lo.astype(np.int32)).cuda(),
                      kw_hi=torch.from_numpy(hi.astype(np.int32)).cuda())
        o, lse = oracle.ring_emulation(h["q"], h["k"], h["v"], self.pos[sl], self.pos, self.cp, r, self.causal,
                                       kw_lo=lo, kw_hi=hi)
        o_dev, o_in = rounded(o, self.dtype)
        lse_dev = torch.from_numpy(lse.astype(np.float32)).cuda()
        lse_in = lse.astype(np.float32).astype(np.float64)
        ref = oracle.ring_backward(h["q"], h["k"], h["v"], o_in, h["do"], lse_in, self.pos[sl], self.pos, self.cp,
                                   r, self.causal, kw_lo=lo, kw_hi=hi)
        ok = oracle.allowed_mask(self.pos[sl], self.pos, self.causal, lo, hi)
        self.zero_rows = (~ok.any(axis=1), ~ok.any(axis=0), ~ok.any(axis=0))   # dQ, dK, dV
        return ri, do_local, o_dev, lse_dev, kw, ref

    def run_gpu(self, r, ri, do_local, o_dev, lse_dev, kw, split=False, ws_bytes=None):
        """split: pass the workspace that lets a small grid split (cp_ring_attn_bwd_workspace_size_ex)."""
        dq = torch.full(ri.q_local.shape, float("nan"), dtype=torch.float32, device="cuda")
        dk = torch.full(ri.k_ring.shape, float("nan"), dtype=torch.float32, device="cuda")
        dv = torch.full(ri.v_ring.shape, float("nan"), dtype=torch.float32, device="cuda")
        if ws_bytes is None:
            ws_bytes = (cpr.cp_ring_attn_bwd_workspace_size_ex(self.B, self.H, self.H_kv, self.D, self.lq,
                                                               self.cp * self.lq) if split else
                        cpr.cp_ring_attn_bwd_workspace_size(self.B, self.H, self.lq))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        cpr.cp_ring_attn_bwd_run(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, self.cp, r, o_dev,
                                 do_local, lse_dev, self.causal, 0.0, dq, dk, dv, ws, **kw)
        torch.cuda.synchronize()
        return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def run_case(c: Case, ranks, name):
    for r in ranks:
        note(f"{name} rank {r}: B={c.B} H={c.H} H_kv={c.H_kv} D={c.D} S={c.S} cp={c.cp} causal={c.causal}")
        ri, do_local, o_dev, lse_dev, kw, ref = c.rank(r)
        got = c.run_gpu(r, ri, do_local, o_dev, lse_dev, kw)
        for g, rf, z, n in zip(got, ref, c.zero_rows, ("dQ", "dK", "dV")):
            check(g, rf, c.dtype, f"{name} r{r} {n}", z)


def test_bwd_f32_tiny():
    c = Case("f32", 1, 2, 2, 64, 256, 2, "zigzag", True, seed=301)
    run_case(c, (0, 1), "f32_tiny")


def test_bwd_bf16_example_shape():
    c = Case("bf16", 1, 4, 4, 64, 4096, 2, "zigzag", True, seed=302)
    run_case(c, (0, 1), "bf16_4k")


@pytest.mark.parametrize("layout", ["zigzag", "contiguous", "striped"])
def test_bwd_bf16_ragged_d128(layout):
    """A sequence that does not fill the tiles (pads in the ring, partial tiles) on every rank."""
    c = Case("bf16", 2, 2, 2, 128, 1000, 4, layout, True, seed=303)
    run_case(c, range(4), f"bf16_ragged_{layout}")


def test_bwd_bf16_noncausal():
    c = Case("bf16", 1, 3, 3, 128, 777, 3, "contiguous", False, seed=304)
    run_case(c, (0, 2), "bf16_noncausal")


@pytest.mark.parametrize("dtype,h,h_kv,d", [("bf16", 8, 2, 128), ("bf16", 4, 1, 64), ("f32", 6, 3, 64)])
def test_bwd_gqa(dtype, h, h_kv, d):
    c = Case(dtype, 1, h, h_kv, d, 1536 if dtype == "bf16" else 384, 2, "zigzag", True, seed=305)
    run_case(c, (0, 1), f"{dtype}_gqa_{h}_{h_kv}")


@pytest.mark.parametrize("layout,causal,h,h_kv,S,cp", [("striped", True, 4, 2, 384, 3), ("contiguous", False, 2, 2, 301, 2)])
def test_bwd_f32_head_dim_128(layout, causal, h, h_kv, S, cp):
    """The float32 backward kernels at D = 128 (the other float32 cases run at D = 64): grouped heads under the
    striped causal layout, and a non-causal contiguous case with a padded tail."""
    c = Case("f32", 1, h, h_kv, 128, S, cp, layout, causal, seed=330 + S)
    run_case(c, range(cp), f"f32_d128_{layout}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_packed_documents(dtype):
    """Per-query document windows (packed sequences) with grouped-query heads and striped layout."""
    docs = [300, 5, 700, 1, 250, 44] if dtype == "bf16" else [100, 5, 77, 1, 50]
    c = Case(dtype, 1, 4, 2, 128 if dtype == "bf16" else 64, sum(docs), 4, "striped", True, seed=306, docs=docs)
    run_case(c, (0, 3), f"{dtype}_docs")


@pytest.mark.parametrize("dtype,d,S,cp,layout,causal,half,empty_every", [
    ("bf16", 128, 1500, 4, "zigzag", True, 100, 7),
    ("bf16", 64, 1200, 3, "striped", False, 80, 11),
    ("f32", 64, 500, 2, "zigzag", True, 50, 5),
])
def test_bwd_sliding_windows_with_empty_windows(dtype, d, S, cp, layout, causal, half, empty_every):
    """Per-query key windows of a sliding-window model: [t - half, t] causal or [t - half, t + half]
    bidirectional, with every empty_every-th query given an empty window (hi < lo). Those queries have
    LSE = -inf in the forward and must get dQ = 0; keys that no window reaches must get dK = dV = 0."""
    t = np.arange(S)
    lo = np.maximum(t - half, 0)
    hi = t if causal else t + half
    hi = np.where(t % empty_every == 3, lo - 1, hi)
    c = Case(dtype, 1, 2, 2, d, S, cp, layout, causal, seed=320 + d + cp, windows=(lo, hi))
    run_case(c, range(cp), f"{dtype}_window_{layout}_d{d}")
    assert c.zero_rows[0].any(), "some query of the last rank has an empty window"


@pytest.mark.parametrize("d", [128, 64])
def test_bwd_mid_size_grouped_heads_documents_padded(d):
    """8,190 tokens (padded to 8,192) over 4 zigzag ranks, 8 query heads on 2 K/V heads, five packed documents:
    many key and query tiles per workgroup, a padded tail, windows and head groups together, compared in full
    with the oracle's ring backward, at both head dimensions."""
    docs = [1000, 3000, 190, 2500, 1500]
    c = Case("bf16", 1, 8, 2, d, sum(docs), 4, "zigzag", True, seed=310 + d, docs=docs)
    run_case(c, (0, 3), f"bf16_mid_gqa_docs_d{d}")


def test_bwd_large_scores():
    """Scores spread over a wide range (scaled Q and K): the saved LSE makes P exact at any scale."""
    c = Case("bf16", 1, 2, 2, 128, 2048, 2, "zigzag", True, seed=307, scale=3.0)
    run_case(c, (0, 1), "bf16_large_scores")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_step_equals_run(dtype):
    """Prep + one step per ring block, accumulating into per-block dK/dV buffers as a real ring would,
    gives the result of the whole-pass call (summation order aside)."""
    c = Case(dtype, 1, 4, 2, 128 if dtype == "bf16" else 64, 999, 3, "zigzag", True, seed=308)
    r = 1
    ri, do_local, o_dev, lse_dev, kw, ref = c.rank(r)
    run = c.run_gpu(r, ri, do_local, o_dev, lse_dev, kw)
    ws = torch.empty(cpr.cp_ring_attn_bwd_workspace_size(c.B, c.H, c.lq), dtype=torch.uint8, device="cuda")
    cpr.cp_ring_attn_bwd_prep(o_dev, do_local, lse_dev, ri.q_pos, True, ws)
    dq = torch.zeros(ri.q_local.shape, dtype=torch.float32, device="cuda")
    dk = torch.zeros(ri.k_ring.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(ri.v_ring.shape, dtype=torch.float32, device="cuda")
    for t in range(c.cp):
        src = (r - t) % c.cp
        sl = slice(src * c.lq, (src + 1) * c.lq)
        dk_blk = dk[:, :, sl].contiguous()
        dv_blk = dv[:, :, sl].contiguous()
        cpr.cp_ring_attn_bwd_step(ri.q_local, do_local, ri.k_ring[:, :, sl], ri.v_ring[:, :, sl], ri.ring_pos[sl],
                                  0.0, ws, dq, dk_blk, dv_blk)
        dk[:, :, sl] = dk_blk
        dv[:, :, sl] = dv_blk
    torch.cuda.synchronize()
    step = (dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())
    for g, rg, rf, z, n in zip(step, run, ref, c.zero_rows, ("dQ", "dK", "dV")):
        check(g, rf, dtype, f"step_{dtype} {n}", z)
        tol = 1e-6 if dtype == "f32" else 1e-5
        assert np.abs(g - rg).max() <= tol * np.abs(rf).max(), n


# ----------------------------------------------------------- full-size, sampled

@pytest.mark.parametrize("wl_name", ["seq32k_cp4", "longdoc_noncausal", "million_cp8"])
def test_bwd_full_size_sampled(wl_name):
    """The backward at a full benchmark workload, in the launch configuration ``bench.py --pass backward`` times.

    One head in every batch index is checked: its live queries get the oracle's forward O (bf16) and LSE;
    every other row of every head gets O = 0 and LSE = -inf (no key allowed), for which every gradient must
    be exactly zero. The live queries are every local query on the 32k share; on the non-causal share
    (two checked heads) a seeded sample of 1,024 and on the million-token share one of 256 (the first and
    last rows of each local chunk among them) keep the oracle's forward affordable; there dK and dV sum over
    the live queries only, as the oracle's do. For each checked head,
    dQ of sampled live queries and dK, dV of sampled ring keys are compared with the oracle's
    row-restricted backward (normwise over the sampled rows, same bar as above)."""
    from seeded_inputs import WORKLOADS, gen_slice, sample_rows
    w = WORKLOADS[wl_name]
    rank = w.ranks[0]
    lay_c, lay_o = LAY[w.layout]
    checked = [(b, (5 + 7 * b) % w.H) for b in range(w.B)]
    note(f"{wl_name}: B={w.B} H={w.H} D={w.D} S={w.S} cp={w.cp} rank={rank} checked (b, h) {checked}")
    nat = {t: di.upload(lambda b, h, t=t: gen_slice(w, t, b, h), w.B, w.H, w.S, w.D, torch.bfloat16)
           for t in ("q", "k", "v", "do")}
    tok_d, pos_d = di.layout_arrays(w.S, w.cp, lay_c)
    ri = di.prepare_rank(nat["q"], nat["k"], nat["v"], w.S, w.cp, lay_c, rank, tok_d, pos_d)
    lq = ri.lq
    do_local = di.gather(nat["do"], w.S, tok_d[rank * lq:(rank + 1) * lq])
    del nat

    tok, pos = oracle.layout(w.S, w.cp, lay_o)
    sl = slice(rank * lq, (rank + 1) * lq)
    chunk = lq // 2 if w.layout == "zigzag" else lq
    # the oracle's forward costs lq * S_pad per checked head: every query when that is small, else a sample
    if lq * len(tok) * len(checked) <= (1 << 29):
        live = np.arange(lq)
    else:
        live = sample_rows(lq, chunk, 1024 if len(tok) <= (1 << 17) else 256, seed=13)

    def host(t, b, h, idx):
        x = gen_slice(w, t, b, h).astype(np.float64)
        out = np.zeros((len(idx), w.D))
        out[idx < w.S] = x[idx[idx < w.S]]
        return out

    o_dev = torch.zeros(ri.q_local.shape, dtype=torch.bfloat16, device="cuda")
    lse_dev = torch.full(ri.q_local.shape[:3], float("-inf"), dtype=torch.float32, device="cuda")
    refs = {}
    for b, h0 in checked:
        qh, kh, vh, gh = host("q", b, h0, tok[sl]), host("k", b, h0, tok), host("v", b, h0, tok), \
            host("do", b, h0, tok[sl])
        # the oracle's forward on the live queries (full attention is order-free: ring order is fine)
        o_l, lse_l = oracle.full_attention(qh[live][None, None], kh[None, None], vh[None, None], pos[sl][live], pos,
                                           w.causal, row_chunk=32)
        o_full = np.zeros((lq, w.D))
        lse_full = np.full(lq, -np.inf)
        o_b = torch.from_numpy(o_l[0, 0].astype(np.float32)).to(torch.bfloat16)
        o_full[live] = o_b.double().numpy()
        lse_full[live] = lse_l[0, 0].astype(np.float32).astype(np.float64)
        live_d = torch.from_numpy(live).cuda()
        o_dev[b, h0, live_d] = o_b.cuda()
        lse_dev[b, h0, live_d] = torch.from_numpy(lse_l[0, 0].astype(np.float32)).cuda()
        refs[(b, h0)] = (qh, kh, vh, gh, o_full, lse_full)

    dq = torch.empty(ri.q_local.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(ri.k_ring.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(ri.v_ring.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(cpr.cp_ring_attn_bwd_workspace_size(w.B, w.H, lq), dtype=torch.uint8, device="cuda")
    cpr.cp_ring_attn_bwd_run(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, w.cp, rank, o_dev, do_local,
                             lse_dev, w.causal, 0.0, dq, dk, dv, ws)
    torch.cuda.synchronize()

    # every head that is not checked: exactly zero
    for b in range(w.B):
        others = [h for h in range(w.H) if (b, h) not in checked]
        for name, g in (("dQ", dq), ("dK", dk), ("dV", dv)):
            assert float(g[b, others].abs().max()) == 0.0, f"{name} of heads with no allowed key is not zero"
    for name, g in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(g).all()), name

    k_rows = sample_rows(len(tok), chunk, 160, seed=12)
    for b, h0 in checked:
        qh, kh, vh, gh, o_full, lse_full = refs[(b, h0)]
        dead = np.ones(lq, dtype=bool)
        dead[live] = False
        if dead.any():
            assert float(dq[b, h0, torch.from_numpy(np.nonzero(dead)[0]).cuda()].abs().max()) == 0.0
        q_rows = live[sample_rows(len(live), max(1, len(live) // 4), 96, seed=11)]
        ref_q = np.concatenate([oracle.rows_backward(qh, kh, vh, o_full, gh, lse_full, pos[sl], pos, w.causal,
                                                     q_rows=q_rows[i:i + 16])[0]
                                for i in range(0, len(q_rows), 16)])
        _, ref_k, ref_v = oracle.rows_backward(qh, kh, vh, o_full, gh, lse_full, pos[sl], pos, w.causal,
                                               k_rows=k_rows)
        got_q = dq[b, h0, torch.from_numpy(q_rows).cuda()].cpu().numpy()
        got_k = dk[b, h0, torch.from_numpy(k_rows).cuda()].cpu().numpy()
        got_v = dv[b, h0, torch.from_numpy(k_rows).cuda()].cpu().numpy()
        for g, r, n in ((got_q, ref_q, "dQ"), (got_k, ref_k, "dK"), (got_v, ref_v, "dV")):
            check(g, r, "bf16", f"{wl_name} (b {b}, h {h0}) sampled {n}")


# ------------------------------------------------------- split of small grids

def split_engaged(c):
    """The sized workspace query reports room for partial gradients: the call will split."""
    return (cpr.cp_ring_attn_bwd_workspace_size_ex(c.B, c.H, c.H_kv, c.D, c.lq, c.cp * c.lq) >
            cpr.cp_ring_attn_bwd_workspace_size(c.B, c.H, c.lq))


@pytest.mark.parametrize("case", ["example_4k", "gqa_docs_d128", "ragged_striped"])
def test_bwd_split_small_grid(case):
    """A bf16 backward on a grid too small for the GPU, given cp_ring_attn_bwd_workspace_size_ex bytes: the dQ
    kernel splits over key slices and the dK/dV kernel over query slices, partials summed in slice order. It
    must meet the oracle bar, agree with the unsplit call up to float32 summation order, and be deterministic."""
    if case == "example_4k":     # the glossary page's 1 x 4 x 4096 x 64 example on two ranks
        c = Case("bf16", 1, 4, 4, 64, 4096, 2, "zigzag", True, seed=320)
    elif case == "gqa_docs_d128":
        docs = [700, 3, 1200, 144, 1]
        c = Case("bf16", 1, 4, 2, 128, sum(docs), 2, "zigzag", True, seed=321, docs=docs)
    else:
        c = Case("bf16", 2, 2, 2, 128, 1000, 4, "striped", True, seed=322)
    assert split_engaged(c)
    for r in range(c.cp) if c.cp <= 2 else (0, 3):
        note(f"split {case} rank {r}")
        ri, do_local, o_dev, lse_dev, kw, ref = c.rank(r)
        got = c.run_gpu(r, ri, do_local, o_dev, lse_dev, kw, split=True)
        again = c.run_gpu(r, ri, do_local, o_dev, lse_dev, kw, split=True)
        plain = c.run_gpu(r, ri, do_local, o_dev, lse_dev, kw)
        for g, g2, p, rf, z, n in zip(got, again, plain, ref, c.zero_rows, ("dQ", "dK", "dV")):
            check(g, rf, "bf16", f"split {case} r{r} {n}", z)
            assert np.array_equal(g, g2), f"{n}: split call not deterministic"
            # only the float32 summation order of the slices differs from the unsplit call
            assert np.abs(g - p).max() <= 1e-5 * np.abs(rf).max(), n


def test_bwd_split_needs_the_whole_workspace():
    """One byte short of cp_ring_attn_bwd_workspace_size_ex: the call runs unsplit (bit-identical to the base
    workspace's result)."""
    c = Case("bf16", 1, 4, 4, 64, 2048, 2, "zigzag", True, seed=323)
    assert split_engaged(c)
    ri, do_local, o_dev, lse_dev, kw, ref = c.rank(1)
    full = cpr.cp_ring_attn_bwd_workspace_size_ex(c.B, c.H, c.H_kv, c.D, c.lq, c.cp * c.lq)
    short = c.run_gpu(1, ri, do_local, o_dev, lse_dev, kw, ws_bytes=full - 1)
    plain = c.run_gpu(1, ri, do_local, o_dev, lse_dev, kw)
    for a, b in zip(short, plain):
        assert np.array_equal(a, b)


def test_bwd_step_split_accumulates():
    """Per-block steps with the split workspace add their partial sums into the caller's accumulators, as the
    unsplit steps do."""
    c = Case("bf16", 1, 4, 2, 128, 1536, 3, "zigzag", True, seed=324)
    r = 2
    ri, do_local, o_dev, lse_dev, kw, ref = c.rank(r)
    ws_bytes = cpr.cp_ring_attn_bwd_workspace_size_ex(c.B, c.H, c.H_kv, c.D, c.lq, c.lq)
    assert ws_bytes > cpr.cp_ring_attn_bwd_workspace_size(c.B, c.H, c.lq)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    cpr.cp_ring_attn_bwd_prep(o_dev, do_local, lse_dev, ri.q_pos, True, ws)
    dq = torch.zeros(ri.q_local.shape, dtype=torch.float32, device="cuda")
    dk = torch.zeros(ri.k_ring.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(ri.v_ring.shape, dtype=torch.float32, device="cuda")
    for t in range(c.cp):
        src = (r - t) % c.cp
        sl = slice(src * c.lq, (src + 1) * c.lq)
        dk_blk = dk[:, :, sl].contiguous()
        dv_blk = dv[:, :, sl].contiguous()
        cpr.cp_ring_attn_bwd_step(ri.q_local, do_local, ri.k_ring[:, :, sl], ri.v_ring[:, :, sl], ri.ring_pos[sl],
                                  0.0, ws, dq, dk_blk, dv_blk)
        dk[:, :, sl] = dk_blk
        dv[:, :, sl] = dv_blk
    torch.cuda.synchronize()
    for g, rf, z, n in zip((dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()), ref, c.zero_rows,
                           ("dQ", "dK", "dV")):
        check(g, rf, "bf16", f"split step {n}", z)


def test_bwd_is_deterministic():
    """No atomics: the same inputs give bit-identical gradients."""
    c = Case("bf16", 1, 4, 2, 128, 1500, 2, "zigzag", True, seed=309)
    ri, do_local, o_dev, lse_dev, kw, _ = c.rank(0)
    a = c.run_gpu(0, ri, do_local, o_dev, lse_dev, kw)
    b = c.run_gpu(0, ri, do_local, o_dev, lse_dev, kw)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
