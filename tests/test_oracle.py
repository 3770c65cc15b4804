"""Pins for the fp64 oracle (CPU only).

Each pin ties the oracle to something other than itself: the cp=4 table the
Megatron page prints, pure-Python brute force on tiny inputs, torch's own
scaled_dot_product_attention and logsumexp, closed forms, and the pages'
exactness claim (blockwise ring result == unpartitioned attention). The last
tests plant mistakes in the oracle (on the CPU) and check that a pin fails.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ring_attention as ora
from seeded_inputs import WORKLOADS, gen_tensor, packed_windows, small_workload

ZZ, CT, ST = oracle.ZIGZAG, oracle.CONTIGUOUS, oracle.STRIPED
LAYOUTS = {"zigzag": ZZ, "contiguous": CT, "striped": ST}


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- layout pins

def test_layout_matches_pages_cp4_table(golden_dir):
    with open(os.path.join(golden_dir, "zigzag_cp4_table.json")) as f:
        g = json.load(f)
    cp = g["cp_size"]
    for c in (1, 3, 5):
        s = g["n_chunks"] * c
        tok, pos = oracle.layout(s, cp, ZZ)
        lr = s // cp
        for r, (a, b) in enumerate(g["chunks_per_rank"]):
            local = tok[r * lr:(r + 1) * lr]
            want = list(range(a * c, a * c + c)) + list(range(b * c, b * c + c))
            assert local.tolist() == want
        assert (pos == tok).all()


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("s", [1, 7, 16, 33, 64, 100, 257])
def test_layout_properties(cp, s):
    for lay in (ZZ, CT, ST):
        tok, pos = oracle.layout(s, cp, lay)
        s_pad = len(tok)
        unit = 2 * cp if lay == ZZ else cp
        assert s_pad == oracle.padded_len(s, cp, lay)
        assert s_pad % unit == 0 and s <= s_pad < s + unit
        assert sorted(tok.tolist()) == list(range(s_pad))          # a permutation
        assert (pos == np.where(tok < s, tok, -1)).all()            # pads carry -1
        lr = s_pad // cp
        for r in range(cp):
            local = tok[r * lr:(r + 1) * lr]
            if lay == ZZ:
                c = lr // 2
                # two runs of c consecutive tokens: chunk r, then chunk 2cp-1-r
                assert local[:c].tolist() == list(range(r * c, r * c + c))
                assert local[c:].tolist() == list(range((2 * cp - 1 - r) * c, (2 * cp - r) * c))
            elif lay == ST:
                # every cp-th token, starting at r
                assert local.tolist() == list(range(r, s_pad, cp))
            else:
                assert local.tolist() == list(range(r * lr, (r + 1) * lr))


def test_striped_layout_small_examples():
    """Token t on rank t mod cp, written out by hand for two small cases."""
    tok, pos = oracle.layout(8, 2, ST)
    assert tok.tolist() == [0, 2, 4, 6, 1, 3, 5, 7]
    assert pos.tolist() == [0, 2, 4, 6, 1, 3, 5, 7]
    tok, pos = oracle.layout(10, 4, ST)   # padded to 12: tokens 10 and 11 are pads
    assert tok.tolist() == [0, 4, 8, 1, 5, 9, 2, 6, 10, 3, 7, 11]
    assert pos.tolist() == [0, 4, 8, 1, 5, 9, 2, 6, -1, 3, 7, -1]


def test_padded_len_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.padded_len(10, 0, ZZ)
    with pytest.raises(ValueError):
        oracle.padded_len(-1, 2, ZZ)
    with pytest.raises(ValueError):
        oracle.padded_len(10, 2, 7)


# ------------------------------------------------------- attention definition

def brute_force(q, k, v, qpos, kpos, causal, scale):
    """Scalar pure-Python softmax attention, one query at a time."""
    outs, lses = [], []
    d = len(q[0])
    for i in range(len(q)):
        keys = [j for j in range(len(k))
                if qpos[i] >= 0 and kpos[j] >= 0 and (not causal or kpos[j] <= qpos[i])]
        if not keys:
            outs.append([0.0] * len(v[0]))
            lses.append(-math.inf)
            continue
        s = {j: scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in keys}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in keys}
        z = sum(w.values())
        outs.append([sum(w[j] * v[j][t] for j in keys) / z for t in range(len(v[0]))])
        lses.append(mx + math.log(z))
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_full_attention_vs_brute_force(causal, seed):
    rng = np.random.default_rng(seed)
    nq, nk, d = 9, 13, 3
    q, k, v = rnd((1, 1, nq, d), seed), rnd((1, 1, nk, d), seed + 10), rnd((1, 1, nk, d), seed + 20)
    qpos = rng.permutation(16)[:nq]
    kpos = rng.permutation(16)[:nk]
    qpos[2] = -1                      # a pad query
    kpos[[0, 5]] = -1                 # pad keys
    scale = 0.7
    o, lse = oracle.full_attention(q, k, v, qpos, kpos, causal, scale, row_chunk=4)
    ob, lb = brute_force(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), qpos, kpos, causal, scale)
    np.testing.assert_allclose(o[0, 0], ob, rtol=0, atol=1e-13)
    assert np.array_equal(np.isinf(lse[0, 0]), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[0, 0][fin], lb[fin], rtol=0, atol=1e-13)
    assert (o[0, 0, 2] == 0).all() and lse[0, 0, 2] == -np.inf


@pytest.mark.parametrize("causal", [False, True])
def test_full_attention_vs_torch_sdpa(causal):
    b, h, s, d = 2, 3, 70, 16
    q, k, v = rnd((b, h, s, d), 5), rnd((b, h, s, d), 6), rnd((b, h, s, d), 7)
    pos = np.arange(s)
    o, lse = oracle.full_attention(q, k, v, pos, pos, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    sc = torch.matmul(tq, tk.transpose(-1, -2)) / math.sqrt(d)
    if causal:
        sc = sc.masked_fill(torch.ones(s, s, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(sc, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_probabilities_sum_to_one():
    b, h, s, d = 1, 2, 50, 8
    q, k, v = rnd((b, h, s, d), 8), rnd((b, h, s, d), 9), rnd((b, h, s, d), 10)
    pos = np.arange(s)
    _, lse = oracle.full_attention(q, k, v, pos, pos, True)
    for bb, hh in itertools.product(range(b), range(h)):
        sc = (q[bb, hh] @ k[bb, hh].T) / math.sqrt(d)
        p = np.where(np.tril(np.ones((s, s), bool)), np.exp(sc - lse[bb, hh][:, None]), 0.0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)


def test_closed_form_zero_keys_gives_prefix_mean():
    """K = 0: every allowed score is 0, so LSE = ln(#allowed) and O = mean of the allowed V rows."""
    s, d = 40, 5
    q, v = rnd((1, 1, s, d), 11), rnd((1, 1, s, d), 12)
    k = np.zeros((1, 1, s, d))
    pos = np.arange(s)
    o, lse = oracle.full_attention(q, k, v, pos, pos, True)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, s + 1)), rtol=0, atol=1e-13)
    prefix_mean = np.cumsum(v[0, 0], axis=0) / np.arange(1, s + 1)[:, None]
    np.testing.assert_allclose(o[0, 0], prefix_mean, rtol=0, atol=1e-13)
    o, lse = oracle.full_attention(q, k, v, pos, pos, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (s, d)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], math.log(s), rtol=0, atol=1e-13)


def test_closed_form_constant_values_and_dominant_key():
    s, d = 30, 4
    q, k = rnd((1, 1, s, d), 13), rnd((1, 1, s, d), 14)
    v = np.full((1, 1, s, d), 2.5)
    pos = np.arange(s)
    o, _ = oracle.full_attention(q, k, v, pos, pos, True)
    np.testing.assert_allclose(o, 2.5, rtol=0, atol=1e-13)
    # one key whose score dwarfs all others: O is (to fp64) that key's value row
    k2 = rnd((1, 1, s, d), 15) * 1e-3
    q2 = np.ones((1, 1, s, d))
    k2[0, 0, 3] = 400.0
    v2 = rnd((1, 1, s, d), 16)
    o2, lse2 = oracle.full_attention(q2, k2, v2, pos, pos, True)
    np.testing.assert_allclose(o2[0, 0, 3:], np.broadcast_to(v2[0, 0, 3], (s - 3, d)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2[0, 0, 3:], 400.0 * d / math.sqrt(d), rtol=0, atol=1e-9)


# ------------------------------------------- exactness of the blockwise ring

def ring_inputs(w):
    q, k, v = (gen_tensor(w, t).astype(np.float64) for t in "qkv")
    lay = LAYOUTS[w.layout]
    tok, pos = oracle.layout(w.S, w.cp, lay)
    s_pad = len(tok)

    def gather(x):
        out = np.zeros(x.shape[:2] + (s_pad, x.shape[-1]))
        real = tok < w.S
        out[:, :, real] = x[:, :, tok[real]]
        return out
    return q, k, v, gather(q), gather(k), gather(v), tok, pos, lay


@pytest.mark.parametrize("cp", [1, 2, 4, 8])
@pytest.mark.parametrize("layout", ["zigzag", "contiguous", "striped"])
@pytest.mark.parametrize("causal", [True, False])
def test_ring_emulation_equals_full_attention(cp, layout, causal):
    w = small_workload("t", "f32", 1, 2, 8, 53, cp, layout, causal, seed=cp * 10 + causal)
    q, k, v, qr, kr, vr, tok, pos, lay = ring_inputs(w)
    lr = len(tok) // cp
    full_o = np.zeros_like(qr)
    full_l = np.zeros(qr.shape[:3])
    for r in range(cp):
        sl = slice(r * lr, (r + 1) * lr)
        o, lse = oracle.ring_emulation(qr[:, :, sl], kr, vr, pos[sl], pos, cp, r, causal)
        ro, rl = oracle.rank_reference(q, k, v, w.S, cp, lay, r, causal)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isinf(lse), np.isinf(rl))
        np.testing.assert_allclose(lse[np.isfinite(rl)], rl[np.isfinite(rl)], rtol=0, atol=1e-12)
        full_o[:, :, sl], full_l[:, :, sl] = o, lse
    # reassemble every rank's rows in natural order (inverse layout) == plain attention
    inv = np.empty(len(tok), np.int64)
    inv[tok] = np.arange(len(tok))
    nat = np.arange(w.S)
    o_nat, l_nat = oracle.full_attention(q, k, v, nat, nat, causal)
    np.testing.assert_allclose(full_o[:, :, inv[:w.S]], o_nat, rtol=0, atol=1e-12)
    np.testing.assert_allclose(full_l[:, :, inv[:w.S]], l_nat, rtol=0, atol=1e-12)


def test_ring_order_does_not_matter():
    w = small_workload("t", "f32", 1, 1, 8, 64, 4, "zigzag", True, seed=3)
    _, _, _, qr, kr, vr, tok, pos, _ = ring_inputs(w)
    lr = len(tok) // 4
    r = 1
    sl = slice(r * lr, (r + 1) * lr)
    base = oracle.ring_emulation(qr[:, :, sl], kr, vr, pos[sl], pos, 4, r, True)
    for order in ([3, 2, 1, 0], [2, 0, 3, 1]):
        o, lse = oracle.ring_emulation(qr[:, :, sl], kr, vr, pos[sl], pos, 4, r, True, order=order)
        np.testing.assert_allclose(o, base[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, base[1], rtol=0, atol=1e-12)


def test_intermediate_states_equal_attention_over_blocks_seen():
    """After step t the finalised state equals attention over the t+1 blocks received so far."""
    w = small_workload("t", "f32", 1, 2, 8, 48, 3, "zigzag", True, seed=4)
    _, _, _, qr, kr, vr, tok, pos, _ = ring_inputs(w)
    cp, r = 3, 2
    lr = len(tok) // cp
    sl = slice(r * lr, (r + 1) * lr)
    _, states = oracle.ring_emulation(qr[:, :, sl], kr, vr, pos[sl], pos, cp, r, True, keep_states=True)
    seen = []
    for t, st in enumerate(states):
        src = oracle.ring_source(r, t, cp)
        seen.extend(range(src * lr, (src + 1) * lr))
        o_ref, l_ref = oracle.full_attention(qr[:, :, sl], kr[:, :, seen], vr[:, :, seen], pos[sl], pos[seen], True)
        o, lse = oracle.finalize(st)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isinf(lse), np.isinf(l_ref))
        fin = np.isfinite(l_ref)
        np.testing.assert_allclose(lse[fin], l_ref[fin], rtol=0, atol=1e-12)


def test_ring_source_is_previous_ranks():
    assert [oracle.ring_source(0, t, 4) for t in range(4)] == [0, 3, 2, 1]
    assert [oracle.ring_source(2, t, 4) for t in range(4)] == [2, 1, 0, 3]


def test_merge_equals_attention_over_union():
    b, h, n, d = 1, 2, 12, 6
    q = rnd((b, h, n, d), 20)
    k, v = rnd((b, h, 30, d), 21), rnd((b, h, 30, d), 22)
    qpos = np.arange(10, 22)
    kpos = np.arange(30)
    halves = [np.arange(0, 30, 2), np.arange(1, 30, 2)]
    parts = []
    for idx in halves:
        st = oracle.init_state(b, h, n, d)
        parts.append(oracle.fold_block(st, q, k[:, :, idx], v[:, :, idx], qpos, kpos[idx], True))
    for a, c in ((0, 1), (1, 0)):
        o, lse = oracle.finalize(oracle.merge(parts[a], parts[c]))
        o_ref, l_ref = oracle.full_attention(q, k, v, qpos, kpos, True)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)
    # merging with an empty state is the identity
    empty = oracle.init_state(b, h, n, d)
    for x, y in zip(oracle.merge(parts[0], empty), parts[0]):
        np.testing.assert_array_equal(x, y)


def test_fully_masked_rows_mid_ring_stay_finite():
    q = rnd((1, 1, 4, 3), 30)
    k, v = rnd((1, 1, 5, 3), 31), rnd((1, 1, 5, 3), 32)
    st = oracle.init_state(1, 1, 4, 3)
    st = oracle.fold_block(st, q, k, v, np.array([0, 1, 2, 3]), np.array([10, 11, 12, 13, 14]), True)
    o, m, l = st
    assert np.isneginf(m).all() and (l == 0).all() and (o == 0).all()
    out, lse = oracle.finalize(st)
    assert (out == 0).all() and np.isneginf(lse).all()


# -------------------------------------------------------- work / balance pins

@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("c", [1, 2, 5, 8])
def test_zigzag_balance_closed_form(cp, c):
    s = 2 * cp * c
    tok, pos = oracle.layout(s, cp, ZZ)
    lr = s // cp
    counts = [oracle.count_pairs(pos[r * lr:(r + 1) * lr], pos, True) for r in range(cp)]
    assert counts == [oracle.causal_pairs_zigzag(s, cp)] * cp
    assert sum(counts) == s * (s + 1) // 2


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("lr", [1, 2, 5, 16])
def test_striped_pairs_closed_form(cp, lr):
    """Brute-force per-rank causal pair counts under striping == cp*Lr*(Lr-1)/2 + Lr*(r+1)."""
    s = cp * lr
    _, pos = oracle.layout(s, cp, ST)
    counts = [oracle.count_pairs(pos[r * lr:(r + 1) * lr], pos, True) for r in range(cp)]
    assert counts == [oracle.causal_pairs_striped(s, cp, r) for r in range(cp)]
    assert sum(counts) == s * (s + 1) // 2
    # ranks differ by at most Lr*(cp-1) pairs: nearly even, unlike the contiguous split
    assert max(counts) - min(counts) == lr * (cp - 1)


def test_contiguous_causal_is_imbalanced():
    cp, s = 4, 64
    _, pos = oracle.layout(s, cp, CT)
    lr = s // cp
    counts = [oracle.count_pairs(pos[r * lr:(r + 1) * lr], pos, True) for r in range(cp)]
    assert counts == sorted(counts) and counts[-1] > counts[0]


def test_workload_pair_counts():
    """Closed form at the five workloads' sizes equals a per-chunk count."""
    for w in WORKLOADS.values():
        if w.layout != "zigzag":
            continue
        c = w.S // (2 * w.cp)
        for r in w.ranks:
            chunks = [r, 2 * w.cp - 1 - r]
            total = 0
            for qc in chunks:
                for kc in range(2 * w.cp):
                    if kc < qc:
                        total += c * c
                    elif kc == qc:
                        total += c * (c + 1) // 2
            assert total == oracle.causal_pairs_zigzag(w.S, w.cp)


# ------------------------------------- grouped-query attention, key windows

def brute_force_windows(q, k, v, qpos, kpos, causal, scale, lo, hi):
    """Scalar pure-Python attention where query i may attend keys with lo[i] <= pos <= hi[i]."""
    outs, lses = [], []
    for i in range(len(q)):
        keys = [j for j in range(len(k)) if qpos[i] >= 0 and kpos[j] >= 0 and (not causal or kpos[j] <= qpos[i])
                and lo[i] <= kpos[j] <= hi[i]]
        if not keys:
            outs.append([0.0] * len(v[0]))
            lses.append(-math.inf)
            continue
        s = {j: scale * sum(a * b for a, b in zip(q[i], k[j])) for j in keys}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in keys}
        z = sum(w.values())
        outs.append([sum(w[j] * v[j][t] for j in keys) / z for t in range(len(v[0]))])
        lses.append(mx + math.log(z))
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_windows_vs_brute_force(causal, seed):
    rng = np.random.default_rng(100 + seed)
    nq, nk, d = 11, 14, 3
    q, k, v = rnd((1, 1, nq, d), seed + 50), rnd((1, 1, nk, d), seed + 60), rnd((1, 1, nk, d), seed + 70)
    qpos = rng.permutation(nk)[:nq]
    qpos[2] = -1                                   # a pad query
    kpos = np.arange(nk)
    kpos[5] = -1                                   # a pad key
    lo = rng.integers(0, nk, nq)
    hi = lo + rng.integers(-2, 8, nq)              # some windows empty (hi < lo)
    o, lse = oracle.full_attention(q, k, v, qpos, kpos, causal, kw_lo=lo, kw_hi=hi)
    ob, lb = brute_force_windows(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), qpos, kpos, causal,
                                 1 / math.sqrt(d), lo, hi)
    np.testing.assert_allclose(o[0, 0], ob, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse[0, 0]), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[0, 0][fin], lb[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_documents_equal_separate_attention(causal):
    """Windows bounded by each token's document == attention run on each document alone."""
    docs = [5, 9, 1, 16, 3]
    s, d = sum(docs), 4
    q, k, v = rnd((1, 2, s, d), 80), rnd((1, 2, s, d), 81), rnd((1, 2, s, d), 82)
    lo, hi = packed_windows(docs)
    pos = np.arange(s)
    o, lse = oracle.full_attention(q, k, v, pos, pos, causal, kw_lo=lo, kw_hi=hi)
    a = 0
    for n in docs:
        sl = slice(a, a + n)
        loc = np.arange(n)   # each document on its own, positions from 0
        od, ld = oracle.full_attention(q[:, :, sl], k[:, :, sl], v[:, :, sl], loc, loc, causal)
        np.testing.assert_allclose(o[:, :, sl], od, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, :, sl], ld, rtol=0, atol=1e-12)
        a += n


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h_kv", [1, 2, 4])
def test_grouped_query_attention_vs_torch_sdpa(causal, h_kv):
    h, s, d = 4, 17, 8
    q, k, v = rnd((2, h, s, d), 90), rnd((2, h_kv, s, d), 91), rnd((2, h_kv, s, d), 92)
    pos = np.arange(s)
    o, _ = oracle.full_attention(q, k, v, pos, pos, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                                           torch.from_numpy(v), is_causal=causal, enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    assert [oracle.kv_head(x, h, h_kv) for x in range(h)] == [x // (h // h_kv) for x in range(h)]


@pytest.mark.parametrize("layout", ["zigzag", "contiguous", "striped"])
def test_ring_emulation_with_gqa_and_documents(layout):
    """The blockwise ring pass with K/V head groups and document windows == plain attention over the rank's rows."""
    cp, docs, h, h_kv, d = 4, [7, 20, 3, 1, 19], 4, 2, 6
    s = sum(docs)
    lay = LAYOUTS[layout]
    q, k, v = rnd((1, h, s, d), 93), rnd((1, h_kv, s, d), 94), rnd((1, h_kv, s, d), 95)
    lo_nat, hi_nat = packed_windows(docs)
    tok, pos = oracle.layout(s, cp, lay)
    s_pad, lr = len(tok), len(tok) // cp
    real = tok < s

    def gather(x):
        out = np.zeros(x.shape[:2] + (s_pad, x.shape[-1]))
        out[:, :, real] = x[:, :, tok[real]]
        return out
    qr, kr, vr = gather(q), gather(k), gather(v)
    for r in range(cp):
        sl = slice(r * lr, (r + 1) * lr)
        ltok = tok[sl]
        lo = np.where(ltok < s, lo_nat[np.minimum(ltok, s - 1)], 0)
        hi = np.where(ltok < s, hi_nat[np.minimum(ltok, s - 1)], 0)
        o, lse = oracle.ring_emulation(qr[:, :, sl], kr, vr, pos[sl], pos, cp, r, True, kw_lo=lo, kw_hi=hi)
        ro, rl = oracle.rank_reference(q, k, v, s, cp, lay, r, True, kw_lo_nat=lo_nat, kw_hi_nat=hi_nat)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(rl))
        fin = np.isfinite(rl)
        np.testing.assert_allclose(lse[fin], rl[fin], rtol=0, atol=1e-12)


# ------------------------------------------------- planted mistakes must fail

def test_planted_strict_mask_is_caught(monkeypatch):
    def strict(q_pos, k_pos, causal, kw_lo=None, kw_hi=None):
        q_pos = np.asarray(q_pos)[:, None]
        k_pos = np.asarray(k_pos)[None, :]
        ok = (q_pos >= 0) & (k_pos >= 0)
        return ok & (k_pos < q_pos) if causal else ok
    monkeypatch.setattr(ora, "allowed_mask", strict)
    s, d = 8, 3
    q, k, v = rnd((1, 1, s, d), 40), rnd((1, 1, s, d), 41), rnd((1, 1, s, d), 42)
    pos = np.arange(s)
    o, _ = ora.full_attention(q, k, v, pos, pos, True)
    ob, _ = brute_force(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), pos, pos, True, 1 / math.sqrt(d))
    assert np.abs(o[0, 0] - ob).max() > 1e-3


def test_planted_dropped_block_is_caught():
    w = small_workload("t", "f32", 1, 1, 8, 32, 2, "zigzag", True, seed=5)
    q, k, v, qr, kr, vr, tok, pos, lay = ring_inputs(w)
    lr = len(tok) // 2
    r = 1
    sl = slice(r * lr, (r + 1) * lr)
    o, lse = oracle.ring_emulation(qr[:, :, sl], kr, vr, pos[sl], pos, 2, r, True, order=[1])
    ro, rl = oracle.rank_reference(q, k, v, w.S, 2, lay, r, True)
    assert np.abs(lse - rl).max() > 0.1


def test_planted_wrong_chunk_pairing_is_caught(monkeypatch, golden_dir):
    orig = ora.layout

    def bad_layout(seq_len, cp, lay):
        tok, pos = orig(seq_len, cp, lay)
        lr = len(tok) // cp
        tok = tok.copy()
        tok[:lr], tok[lr:2 * lr] = tok[lr:2 * lr].copy(), tok[:lr].copy()   # swap two ranks
        return tok, np.where(tok < seq_len, tok, -1)
    monkeypatch.setattr(oracle, "layout", bad_layout)
    with pytest.raises(AssertionError):
        test_layout_matches_pages_cp4_table(golden_dir)


def test_planted_wrong_rescale_sign_is_caught(monkeypatch):
    """A fold that rescales earlier partial sums by exp(m_new - m) instead of
    exp(m - m_new) must break the ring == full-attention pin."""
    def bad_fold(state, q, k_blk, v_blk, q_pos, k_pos, causal, scale=None, kw_lo=None, kw_hi=None):
        o, m, l = (np.array(x, dtype=np.float64) for x in state)
        scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
        ok = ora.allowed_mask(q_pos, k_pos, causal)
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                s = np.where(ok, scale * (q[b, h] @ k_blk[b, h].T), -np.inf)
                m_new = np.maximum(m[b, h], s.max(axis=1))
                m_use = np.where(np.isfinite(m_new), m_new, 0.0)
                alpha = np.where(np.isfinite(m[b, h]), np.exp(m_use - m[b, h]), 0.0)   # planted: sign flipped
                p = np.where(ok, np.exp(s - m_use[:, None]), 0.0)
                l[b, h] = alpha * l[b, h] + p.sum(axis=1)
                o[b, h] = alpha[:, None] * o[b, h] + p @ v_blk[b, h]
                m[b, h] = m_new
        return o, m, l
    w = small_workload("t", "f32", 1, 1, 8, 64, 4, "zigzag", True, seed=6)
    q, k, v, qr, kr, vr, tok, pos, lay = ring_inputs(w)
    lr = len(tok) // w.cp
    r = 3
    sl = slice(r * lr, (r + 1) * lr)
    ro, rl = oracle.rank_reference(q, k, v, w.S, w.cp, lay, r, True)
    good, _ = oracle.ring_emulation(qr[:, :, sl], kr, vr, pos[sl], pos, w.cp, r, True)
    assert np.abs(good - ro).max() < 1e-12
    monkeypatch.setattr(ora, "fold_block", bad_fold)
    bad, _ = oracle.ring_emulation(qr[:, :, sl], kr, vr, pos[sl], pos, w.cp, r, True)
    assert np.abs(bad - ro).max() > 1e-3


def test_planted_swapped_operands_are_caught(monkeypatch):
    """Attention that multiplies P by K instead of V must fail the torch SDPA pin."""
    orig = ora._attend_rows

    def swapped(q, k, v, q_pos, k_pos, causal, scale, kw_lo=None, kw_hi=None):
        return orig(q, k, k, q_pos, k_pos, causal, scale)
    monkeypatch.setattr(ora, "_attend_rows", swapped)
    s, d = 16, 8
    q, k, v = rnd((1, 2, s, d), 50), rnd((1, 2, s, d), 51), rnd((1, 2, s, d), 52)
    pos = np.arange(s)
    o, _ = oracle.full_attention(q, k, v, pos, pos, True)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                                           torch.from_numpy(v), is_causal=True).numpy()
    assert np.abs(o - ref).max() > 1e-3


# ------------------------------------------------------------- backward pins

def torch_grads(q, k, v, do, mask, scale):
    """dQ, dK, dV from torch autograd (float64) through torch's own SDPA with a boolean mask."""
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=scale,
                                                         enable_gqa=k.shape[1] != q.shape[1])
    o.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("h_kv", [1, 2, 4])
def test_backward_vs_torch_autograd(causal, h_kv):
    h, nq, nk, d = 4, 13, 21, 8
    q, do = rnd((2, h, nq, d), 100), rnd((2, h, nq, d), 101)
    k, v = rnd((2, h_kv, nk, d), 102), rnd((2, h_kv, nk, d), 103)
    qpos, kpos = np.arange(8, 8 + nq), np.arange(nk)
    scale = 0.3
    got = oracle.attention_backward(q, k, v, do, qpos, kpos, causal, scale)
    want = torch_grads(q, k, v, do, oracle.allowed_mask(qpos, kpos, causal), scale)
    for g, w_ in zip(got, want):
        np.testing.assert_allclose(g, w_, rtol=0, atol=1e-12)


def test_backward_with_windows_vs_torch_autograd():
    docs, h, d = [5, 11, 2, 9], 2, 6
    s = sum(docs)
    lo, hi = packed_windows(docs)
    hi = np.minimum(hi, np.arange(s))
    lo = np.maximum(lo, np.arange(s) - 4)             # plus a sliding window of 5 keys
    q, k, v, do = (rnd((1, h, s, d), 104 + i) for i in range(4))
    pos = np.arange(s)
    got = oracle.attention_backward(q, k, v, do, pos, pos, True, kw_lo=lo, kw_hi=hi)
    want = torch_grads(q, k, v, do, oracle.allowed_mask(pos, pos, True, lo, hi), 1 / math.sqrt(d))
    for g, w_ in zip(got, want):
        np.testing.assert_allclose(g, w_, rtol=0, atol=1e-12)


def test_backward_vs_finite_differences():
    """Central differences of L = sum(dO * O) in fp64, independent of any autograd."""
    h, h_kv, nq, nk, d = 2, 1, 5, 7, 4
    q, do = rnd((1, h, nq, d), 110), rnd((1, h, nq, d), 111)
    k, v = rnd((1, h_kv, nk, d), 112), rnd((1, h_kv, nk, d), 113)
    qpos, kpos = np.arange(2, 2 + nq), np.arange(nk)

    def loss(q_, k_, v_):
        o, _ = oracle.full_attention(q_, k_, v_, qpos, kpos, True)
        return float((do * o).sum())
    grads = oracle.attention_backward(q, k, v, do, qpos, kpos, True)
    eps = 1e-6
    for which, g in enumerate(grads):
        xs = [q.copy(), k.copy(), v.copy()]
        for idx in np.ndindex(xs[which].shape):
            xp = [x.copy() for x in xs]
            xm = [x.copy() for x in xs]
            xp[which][idx] += eps
            xm[which][idx] -= eps
            num = (loss(*xp) - loss(*xm)) / (2 * eps)
            assert abs(num - g[idx]) < 1e-7, (which, idx, num, g[idx])


def test_backward_empty_rows_and_zero_upstream():
    """Rows with no allowed key get dQ = 0 and add nothing to dK, dV; dO = 0 gives all-zero gradients."""
    q, do = rnd((1, 1, 4, 3), 120), rnd((1, 1, 4, 3), 121)
    k, v = rnd((1, 1, 6, 3), 122), rnd((1, 1, 6, 3), 123)
    qpos, kpos = np.array([0, 1, -1, 3]), np.arange(2, 8)        # rows 0, 1 see no key (causal), row 2 is a pad
    dq, dk, dv = oracle.attention_backward(q, k, v, do, qpos, kpos, True)
    assert (dq[0, 0, :3] == 0).all()
    keep = np.array([False, False, False, True])
    dq2, dk2, dv2 = oracle.attention_backward(q[:, :, keep], k, v, do[:, :, keep], qpos[keep], kpos, True)
    np.testing.assert_allclose(dk, dk2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dv, dv2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dq[:, :, keep], dq2, rtol=0, atol=1e-15)
    z = oracle.attention_backward(q, k, v, np.zeros_like(do), qpos, kpos, True)
    assert all((g == 0).all() for g in z)


def test_backward_closed_form_single_key():
    """One allowed key per row: P = 1, so dV = sum of dO over the rows, dQ = dK = 0."""
    q, do = rnd((1, 1, 3, 4), 124), rnd((1, 1, 3, 4), 125)
    k, v = rnd((1, 1, 5, 4), 126), rnd((1, 1, 5, 4), 127)
    lo = hi = np.array([2, 2, 2])
    dq, dk, dv = oracle.attention_backward(q, k, v, do, np.arange(3), np.arange(5), False, kw_lo=lo, kw_hi=hi)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv[0, 0, 2], do[0, 0].sum(axis=0), rtol=0, atol=1e-15)
    assert (np.delete(dv[0, 0], 2, axis=0) == 0).all()


def ring_backward_all_ranks(q, k, v, do, s, cp, lay, causal, lo_nat=None, hi_nat=None):
    """Run the forward and backward ring pass on every rank; return dQ in natural order and the
    dK, dV contributions summed over ranks, also in natural order."""
    tok, pos = oracle.layout(s, cp, lay)
    s_pad, lr = len(tok), len(tok) // cp
    real = tok < s

    def gather(x):
        out = np.zeros(x.shape[:2] + (s_pad, x.shape[-1]))
        out[:, :, real] = x[:, :, tok[real]]
        return out
    qr, kr, vr, dor = gather(q), gather(k), gather(v), gather(do)
    dq_r = np.zeros_like(qr)
    dk_r, dv_r = np.zeros_like(kr), np.zeros_like(vr)
    for r in range(cp):
        sl = slice(r * lr, (r + 1) * lr)
        ltok = tok[sl]
        lo = hi = None
        if lo_nat is not None:
            lo = np.where(ltok < s, lo_nat[np.minimum(ltok, s - 1)], 0)
            hi = np.where(ltok < s, hi_nat[np.minimum(ltok, s - 1)], 0)
        o, lse = oracle.ring_emulation(qr[:, :, sl], kr, vr, pos[sl], pos, cp, r, causal, kw_lo=lo, kw_hi=hi)
        dq, dk, dv = oracle.ring_backward(qr[:, :, sl], kr, vr, o, dor[:, :, sl], lse, pos[sl], pos, cp, r, causal,
                                          kw_lo=lo, kw_hi=hi)
        dq_r[:, :, sl] = dq
        dk_r += dk
        dv_r += dv
    inv = np.empty(s_pad, np.int64)
    inv[tok] = np.arange(s_pad)
    nat = inv[:s]
    return dq_r[:, :, nat], dk_r[:, :, nat], dv_r[:, :, nat], (dq_r[:, :, ~real], dk_r[:, :, ~real], dv_r[:, :, ~real])


@pytest.mark.parametrize("cp", [1, 2, 4, 8])
@pytest.mark.parametrize("layout", ["zigzag", "contiguous", "striped"])
@pytest.mark.parametrize("causal", [True, False])
def test_ring_backward_equals_full_gradients(cp, layout, causal):
    """Per-rank dQ and the dK, dV contributions summed over the ring == gradients of plain attention."""
    w = small_workload("t", "f32", 1, 2, 8, 53, cp, layout, causal, seed=cp * 10 + causal + 1)
    q, k, v = (gen_tensor(w, t).astype(np.float64) for t in "qkv")
    do = gen_tensor(w, "do").astype(np.float64)
    dq, dk, dv, pads = ring_backward_all_ranks(q, k, v, do, w.S, cp, LAYOUTS[layout], causal)
    nat = np.arange(w.S)
    want = oracle.attention_backward(q, k, v, do, nat, nat, causal)
    for g, w_ in zip((dq, dk, dv), want):
        np.testing.assert_allclose(g, w_, rtol=0, atol=1e-12)
    assert all((p == 0).all() for p in pads)                       # pad rows get and give nothing


@pytest.mark.parametrize("layout", ["zigzag", "striped"])
def test_ring_backward_with_gqa_and_documents(layout):
    cp, docs, h, h_kv, d = 4, [7, 20, 3, 1, 19], 4, 2, 6
    s = sum(docs)
    q, do = rnd((1, h, s, d), 130), rnd((1, h, s, d), 131)
    k, v = rnd((1, h_kv, s, d), 132), rnd((1, h_kv, s, d), 133)
    lo, hi = packed_windows(docs)
    dq, dk, dv, _ = ring_backward_all_ranks(q, k, v, do, s, cp, LAYOUTS[layout], True, lo, hi)
    nat = np.arange(s)
    want = oracle.attention_backward(q, k, v, do, nat, nat, True, kw_lo=lo, kw_hi=hi)
    for g, w_ in zip((dq, dk, dv), want):
        np.testing.assert_allclose(g, w_, rtol=0, atol=1e-12)


def test_planted_backward_without_dvec_is_caught(monkeypatch):
    """dS = P * dP (the row term rowsum(dO * O) dropped) must fail the autograd pin."""
    monkeypatch.setattr(ora, "_score_grad", lambda p, dp, dvec: p * dp)
    with pytest.raises(AssertionError):
        test_backward_vs_torch_autograd(False, 4)


def test_planted_wrong_kv_head_group_is_caught(monkeypatch):
    """Query head h reading K/V head h mod H_kv (instead of h // (H / H_kv)) must fail the autograd pin."""
    monkeypatch.setattr(ora, "kv_head", lambda h, n_h, n_kv: h % n_kv)
    with pytest.raises(AssertionError):
        test_backward_vs_torch_autograd(True, 2)


# ----------------------------------------------------------------- RoPE pins

def test_rope_d2_is_complex_rotation():
    """D = 2: the pair (a, b) as a + ib is multiplied by exp(i * pos) (theta_0 = 1), numpy's complex exp."""
    x = rnd((1, 1, 7, 2), 140)
    pos = np.array([0, 1, 2, 5, 100, 12345, 999999])
    got = oracle.rope(x, pos)
    z = (x[..., 0] + 1j * x[..., 1]) * np.exp(1j * pos.astype(np.float64))
    np.testing.assert_allclose(got[..., 0], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[..., 1], z.imag, rtol=0, atol=1e-12)


# Hand-computed rotation angles pos * theta_j for cases where base^(-2j/D) is exact:
# (D, base, pos, [angle of pair j = 0 .. D/2-1]). theta_j = base^(-2j/D) gives
#   D = 8, base = 16:    theta = 1, 1/2, 1/4, 1/8       -> at pos 8:    8, 4, 2, 1
#   D = 8, base = 10^4:  theta = 1, 0.1, 0.01, 0.001    -> at pos 1000: 1000, 100, 10, 1
#   D = 4, base = 100:   theta = 1, 0.1                 -> at pos 30:   30, 3
#   D = 6, base = 64:    theta = 1, 1/4, 1/16           -> at pos 48:   48, 12, 3
ROPE_HAND_ANGLES = [
    (8, 16.0, 8, [8.0, 4.0, 2.0, 1.0]),
    (8, 10000.0, 1000, [1000.0, 100.0, 10.0, 1.0]),
    (4, 100.0, 30, [30.0, 3.0]),
    (6, 64.0, 48, [48.0, 12.0, 3.0]),
]
# the dimension pairs, written out: INTERLEAVED (2j, 2j+1), HALF (j, j + D/2)
ROPE_HAND_PAIRS = {
    (oracle.INTERLEAVED, 8): [(0, 1), (2, 3), (4, 5), (6, 7)],
    (oracle.HALF, 8): [(0, 4), (1, 5), (2, 6), (3, 7)],
    (oracle.INTERLEAVED, 4): [(0, 1), (2, 3)],
    (oracle.HALF, 4): [(0, 2), (1, 3)],
    (oracle.INTERLEAVED, 6): [(0, 1), (2, 3), (4, 5)],
    (oracle.HALF, 6): [(0, 3), (1, 4), (2, 5)],
}


@pytest.mark.parametrize("style", [oracle.INTERLEAVED, oracle.HALF])
@pytest.mark.parametrize("case", range(len(ROPE_HAND_ANGLES)))
def test_rope_frequency_schedule_hand_computed(style, case):
    """Every pair j >= 0 turns by the hand-computed angle pos * base^(-2j/D): scalar math.cos / math.sin, one
    element at a time, on rows at position pos, 0 and a pad (-1)."""
    d, base, p, angles = ROPE_HAND_ANGLES[case]
    x = rnd((1, 1, 3, d), 146 + case)
    got = oracle.rope(x, np.array([p, 0, -1]), base=base, style=style)
    for (ia, ib), t in zip(ROPE_HAND_PAIRS[(style, d)], angles):
        a, b = float(x[0, 0, 0, ia]), float(x[0, 0, 0, ib])
        want_a = a * math.cos(t) - b * math.sin(t)
        want_b = a * math.sin(t) + b * math.cos(t)
        assert abs(got[0, 0, 0, ia] - want_a) <= 1e-12 * (1 + abs(want_a)), (ia, t)
        assert abs(got[0, 0, 0, ib] - want_b) <= 1e-12 * (1 + abs(want_b)), (ib, t)
    np.testing.assert_array_equal(got[0, 0, 1], x[0, 0, 1])   # position 0
    np.testing.assert_array_equal(got[0, 0, 2], x[0, 0, 2])   # pad


def test_rope_theta_hand_values():
    """theta_j itself on the hand-computed cases (angle / pos)."""
    for d, base, p, angles in ROPE_HAND_ANGLES:
        np.testing.assert_allclose(oracle.rope_theta(d, base), np.array(angles) / p, rtol=1e-15, atol=0)


def test_planted_rope_exponent_is_caught(monkeypatch):
    """theta_j = base^(-j/D) (exponent halved) must fail the hand-computed frequency pin."""
    import sys
    rope_mod = sys.modules["oracle.rope"]
    monkeypatch.setattr(rope_mod, "rope_theta", lambda d, base: np.power(float(base), -1.0 * np.arange(d // 2) / d))
    for style in (oracle.INTERLEAVED, oracle.HALF):
        with pytest.raises(AssertionError):
            test_rope_frequency_schedule_hand_computed(style, 0)


def test_planted_rope_pairing_is_caught(monkeypatch):
    """HALF pairs taken as (j, D - 1 - j) must fail the hand-computed pin."""
    import sys
    rope_mod = sys.modules["oracle.rope"]
    real = rope_mod.rope_pairs

    def wrong(d, style):
        if style == oracle.HALF:
            j = np.arange(d // 2)
            return j, d - 1 - j
        return real(d, style)
    monkeypatch.setattr(rope_mod, "rope_pairs", wrong)
    with pytest.raises(AssertionError):
        test_rope_frequency_schedule_hand_computed(oracle.HALF, 0)


@pytest.mark.parametrize("style", [oracle.INTERLEAVED, oracle.HALF])
def test_rope_preserves_pair_norms_and_is_identity_at_zero(style):
    x = rnd((2, 3, 9, 16), 141)
    pos = np.array([0, 3, 7, 64, 1000, 65535, 131071, 1048575, -1])
    y = oracle.rope(x, pos, style=style)
    a, b = oracle.rope_pairs(16, style)
    np.testing.assert_allclose(y[..., a] ** 2 + y[..., b] ** 2, x[..., a] ** 2 + x[..., b] ** 2, rtol=1e-12, atol=0)
    np.testing.assert_array_equal(y[..., 0, :], x[..., 0, :])      # position 0: no rotation
    np.testing.assert_array_equal(y[..., -1, :], x[..., -1, :])    # pad (-1): unchanged
    assert np.abs(y[..., 1:-1, :] - x[..., 1:-1, :]).max() > 1e-3


@pytest.mark.parametrize("style", [oracle.INTERLEAVED, oracle.HALF])
def test_rope_scores_depend_on_relative_position_only(style):
    """<rope(q, m), rope(k, n)> = <rope(q, m - n), k>: the property rotary embeddings exist for."""
    d = 32
    q, k = rnd((d,), 142), rnd((d,), 143)
    for m, n in ((5, 2), (100, 37), (70000, 69990), (3, 3)):
        lhs = oracle.rope(q[None, :], np.array([m]), style=style)[0] @ oracle.rope(k[None, :], np.array([n]),
                                                                                   style=style)[0]
        rhs = oracle.rope(q[None, :], np.array([m - n]), style=style)[0] @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))


def test_rope_half_is_interleaved_on_permuted_dims():
    d = 8
    x = rnd((1, 2, 5, d), 144)
    pos = np.array([0, 1, 9, 300, 77777])
    perm = np.empty(d, np.int64)
    perm[0::2] = np.arange(d // 2)                 # interleaved slot 2j <- half slot j
    perm[1::2] = np.arange(d // 2) + d // 2        # interleaved slot 2j+1 <- half slot j + D/2
    inter = oracle.rope(x[..., perm], pos, style=oracle.INTERLEAVED)
    half = oracle.rope(x, pos, style=oracle.HALF)
    np.testing.assert_allclose(inter, half[..., perm], rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout", ["zigzag", "striped"])
def test_rope_with_global_positions_commutes_with_the_layout(layout):
    """Rotating the natural sequence and then gathering a rank's tokens equals gathering first and rotating
    with the rank's global position ids (Megatron page, implementation quirk); renumbering locally does not."""
    s, cp, d = 61, 4, 8
    x = rnd((1, 2, s, d), 145)
    tok, pos = oracle.layout(s, cp, LAYOUTS[layout])
    lr = len(tok) // cp
    nat = oracle.rope(x, np.arange(s))
    for r in range(cp):
        lt = tok[r * lr:(r + 1) * lr]
        real = lt < s
        local = np.zeros((1, 2, lr, d))
        local[:, :, real] = x[:, :, lt[real]]
        got = oracle.rope(local, pos[r * lr:(r + 1) * lr])
        np.testing.assert_allclose(got[:, :, real], nat[:, :, lt[real]], rtol=0, atol=1e-12)
        if r > 0:
            wrong = oracle.rope(local, np.where(real, np.arange(lr), -1))   # local renumbering
            assert np.abs(wrong[:, :, real] - nat[:, :, lt[real]]).max() > 1e-3


def test_rows_backward_equals_ring_backward():
    """The row-restricted backward (used for sampled checks at full size) gives the ring backward's rows."""
    w = small_workload("t", "f32", 1, 2, 8, 77, 3, "zigzag", True, seed=150)
    q, k, v = (gen_tensor(w, t).astype(np.float64) for t in "qkv")
    do = gen_tensor(w, "do").astype(np.float64)
    tok, pos = oracle.layout(w.S, w.cp, ZZ)
    lq = len(tok) // w.cp
    real = tok < w.S

    def gather(x, idx):
        out = np.zeros(x.shape[:2] + (len(idx), x.shape[-1]))
        out[:, :, idx < w.S] = x[:, :, idx[idx < w.S]]
        return out
    r = 2
    sl = slice(r * lq, (r + 1) * lq)
    qr, kr, vr, dor = gather(q, tok[sl]), gather(k, tok), gather(v, tok), gather(do, tok[sl])
    o, lse = oracle.ring_emulation(qr, kr, vr, pos[sl], pos, w.cp, r, True)
    dq, dk, dv = oracle.ring_backward(qr, kr, vr, o, dor, lse, pos[sl], pos, w.cp, r, True)
    qs, ks = np.array([0, 3, lq - 1]), np.array([0, 5, 40, len(tok) - 1])
    for h in range(2):
        a, b, c = oracle.rows_backward(qr[0, h], kr[0, h], vr[0, h], o[0, h], dor[0, h], lse[0, h], pos[sl], pos,
                                       True, q_rows=qs, k_rows=ks)
        np.testing.assert_allclose(a, dq[0, h, qs], rtol=0, atol=1e-12)
        np.testing.assert_allclose(b, dk[0, h, ks], rtol=0, atol=1e-12)
        np.testing.assert_allclose(c, dv[0, h, ks], rtol=0, atol=1e-12)
    assert real.any()
