"""Plain, slow, fp64 CPU definition of what one context-parallel rank computes.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Everything is numpy float64 with no blocking, fusion or reordering beyond what
the pages state. Tensors are laid out [B, H, L, D] (sequence on dim 2, as in
the SDPA call of "Context Parallelism", section "Practical use and
trade-offs"). Positions are global token positions; -1 marks a pad token.

Readings where the pages are silent (each also listed in the design notes):

* softmax scale defaults to 1/sqrt(D) (the SDPA call on the glossary page
  passes no scale, so the library default applies);
* a key is allowed for a query iff both are real tokens and, when causal,
  pos_k <= pos_q by *global* position (lower-triangular valid region,
  "Implementation quirk: symmetric chunk assignment");
* pad tokens go at the tail, carry position -1, are never attended, and a pad
  query (or any query with no allowed key) yields O = 0 and LSE = -inf;
* LSE is in natural-log units;
* ring step t of rank r folds the block that started on rank (r - t) mod cp
  (blocks move to the next device each hop);
* the backward pass (the glossary page's example calls .backward() on the
  context-parallel output) is the textbook softmax-attention derivative; in
  the ring each rank recomputes a block's probabilities from the LSE its
  forward pass saved, keeps its dQ, and adds its dK, dV contributions to the
  block, which carries them around the ring back to the block's owner.
"""

from __future__ import annotations

import math

import numpy as np

ZIGZAG = 0
CONTIGUOUS = 1
STRIPED = 2


# ---------------------------------------------------------------------------
# Layout: "Context Parallelism v.s. Sequence Parallelism (Megatron-LM)",
# section "Implementation quirk: symmetric chunk assignment" (zigzag),
# "Sequence Parallelism and Ring Attention", section "Deep dive" (contiguous),
# and the same page's "The future of sequence parallelism and ring attention"
# (striped, named there beside zigzag as a rebalancing of causal work; read
# here as token t on rank t mod cp).
# ---------------------------------------------------------------------------

def padded_len(seq_len: int, cp: int, lay: int) -> int:
    """Sequence length after padding.

    Zigzag needs the sequence to split evenly into 2*cp chunks, so it pads up
    to a multiple of 2*cp (Megatron page, symmetric chunk assignment). The
    contiguous split only needs cp equal pieces.
    """
    if seq_len < 0 or cp < 1 or lay not in (ZIGZAG, CONTIGUOUS, STRIPED):
        raise ValueError("bad layout arguments")
    unit = 2 * cp if lay == ZIGZAG else cp
    return ((seq_len + unit - 1) // unit) * unit


def layout(seq_len: int, cp: int, lay: int):
    """Rank-major token layout.

    Returns ``(token_idx, pos_ids)``, both int64 of length S_pad. Entry
    ``r*Lr + i`` (Lr = S_pad/cp) is the i-th local token of rank r.

    Zigzag: the padded sequence is cut into 2*cp equal chunks of c tokens and
    rank r holds chunk r followed by chunk 2*cp-1-r (the page's cp=4 table:
    rank 0 has chunks 0 and 7, ..., rank 3 has chunks 3 and 4).
    Contiguous: rank r holds tokens [r*Lr, (r+1)*Lr).
    Striped: token t goes to rank t mod cp, so rank r holds r, r+cp, r+2cp, ...
    pos_ids is the global position of the token, or -1 for a pad token (the
    page insists local positions are the global ones, never 0, 1, 2, ...).
    """
    s_pad = padded_len(seq_len, cp, lay)
    lr = s_pad // cp
    token_idx = np.empty(s_pad, dtype=np.int64)
    if lay == ZIGZAG:
        c = s_pad // (2 * cp)
        for r in range(cp):
            front, back = r, 2 * cp - 1 - r
            token_idx[r * lr: r * lr + c] = np.arange(front * c, front * c + c)
            token_idx[r * lr + c: (r + 1) * lr] = np.arange(back * c, back * c + c)
    elif lay == STRIPED:
        for r in range(cp):
            token_idx[r * lr: (r + 1) * lr] = np.arange(r, s_pad, cp)
    else:
        token_idx[:] = np.arange(s_pad)
    pos_ids = np.where(token_idx < seq_len, token_idx, -1)
    return token_idx, pos_ids


def ring_source(rank: int, t: int, cp: int) -> int:
    """Rank whose KV block rank ``rank`` holds at ring step ``t``.

    Each hop passes the block to the next device, so after t hops rank r holds
    the block that started on rank r - t ("Context Parallelism", section "How
    context parallelism works"; "Sequence Parallelism and Ring Attention",
    "Deep dive").
    """
    return (rank - t) % cp


# ---------------------------------------------------------------------------
# Masking and plain attention.
# ---------------------------------------------------------------------------

def allowed_mask(q_pos, k_pos, causal: bool, kw_lo=None, kw_hi=None):
    """[Nq, Nk] bool: may query i attend key j.

    Causal attention keeps the lower-triangular region by global position,
    diagonal included (Megatron page, symmetric chunk assignment; SDPA's
    is_causal on the glossary page). Pad tokens (pos -1) take no part.
    """
    q_pos = np.asarray(q_pos)[:, None]
    k_pos = np.asarray(k_pos)[None, :]
    ok = (q_pos >= 0) & (k_pos >= 0)
    if causal:
        ok = ok & (k_pos <= q_pos)
    # optional per-query window of key positions [kw_lo, kw_hi] (packed
    # documents: the bounds of the query's own document; the Megatron page,
    # "Implementation quirk: symmetric chunk assignment", has the attention mask
    # and packed-sequence metadata follow the chunk pairing, by global position)
    if kw_lo is not None:
        ok = ok & (k_pos >= np.asarray(kw_lo)[:, None])
    if kw_hi is not None:
        ok = ok & (k_pos <= np.asarray(kw_hi)[:, None])
    return ok


def _attend_rows(q, k, v, q_pos, k_pos, causal, scale, kw_lo=None, kw_hi=None):
    """Softmax attention for a few query rows of one (b, h).

    q [n, D], k/v [Nk, D], float64. Returns O [n, D], LSE [n]. This is the
    textbook definition: s = scale * q k^T, masked softmax over keys, O = P v.
    """
    s = scale * (q @ k.T)
    ok = allowed_mask(q_pos, k_pos, causal, kw_lo, kw_hi)
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    p = np.where(ok, np.exp(s - m_safe[:, None]), 0.0)
    l = p.sum(axis=1)
    o = np.zeros((q.shape[0], v.shape[1]))
    o[has] = (p[has] @ v) / l[has, None]
    lse = np.full(q.shape[0], -np.inf)
    lse[has] = m[has] + np.log(l[has])
    return o, lse


def kv_head(h: int, n_heads: int, n_kv_heads: int) -> int:
    """K/V head read by query head h when K/V have fewer heads (grouped-query
    attention): consecutive groups of H/H_kv query heads share one K/V head."""
    return h // (n_heads // n_kv_heads)


def full_attention(q, k, v, q_pos, k_pos, causal: bool, scale=None, row_chunk: int = 64, kw_lo=None, kw_hi=None):
    """Unpartitioned softmax attention, fp64.

    q [B, H, Nq, D], k/v [B, H_kv, Nk, D] (H_kv divides H; query head h reads
    K/V head ``kv_head(h, H, H_kv)``); q_pos [Nq], k_pos [Nk] global positions;
    kw_lo / kw_hi optional [Nq] key-position windows.
    Returns O [B, H, Nq, D] float64 and LSE [B, H, Nq] float64.
    This is the result ring attention must reproduce up to rounding
    ("Context Parallelism", "How context parallelism works";
    "Sequence Parallelism and Ring Attention", "Technical insight").
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, h_, nq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q_pos = np.asarray(q_pos)
    k_pos = np.asarray(k_pos)
    o = np.zeros((b_, h_, nq, v.shape[-1]))
    lse = np.zeros((b_, h_, nq))
    h_kv = k.shape[1]
    if h_ % h_kv:
        raise ValueError("K/V heads must divide query heads")
    for b in range(b_):
        for h in range(h_):
            hk = kv_head(h, h_, h_kv)
            for r0 in range(0, nq, row_chunk):
                r1 = min(nq, r0 + row_chunk)
                o[b, h, r0:r1], lse[b, h, r0:r1] = _attend_rows(
                    q[b, h, r0:r1], k[b, hk], v[b, hk], q_pos[r0:r1], k_pos, causal, scale,
                    None if kw_lo is None else np.asarray(kw_lo)[r0:r1],
                    None if kw_hi is None else np.asarray(kw_hi)[r0:r1])
    return o, lse


def rank_reference(q, k, v, seq_len: int, cp: int, lay: int, rank: int, causal: bool,
                   scale=None, rows=None, kw_lo_nat=None, kw_hi_nat=None):
    """What rank ``rank`` must output: rows of full attention over the whole sequence.

    q, k, v are the unsharded [B, H, seq_len, D] tensors in natural token
    order. The rank's local rows come from ``layout``; ``rows`` optionally
    picks a subset of local row indices (for sampled checks at large sizes).
    kw_lo_nat / kw_hi_nat optionally give every token's key window in natural
    order (packed documents); the rank's queries take those of their tokens.
    Returns O [B, H, n, D] and LSE [B, H, n] in local order.
    """
    token_idx, pos_ids = layout(seq_len, cp, lay)
    lr = len(token_idx) // cp
    local_tok = token_idx[rank * lr:(rank + 1) * lr]
    local_pos = pos_ids[rank * lr:(rank + 1) * lr]
    if rows is not None:
        rows = np.asarray(rows)
        local_tok = local_tok[rows]
        local_pos = local_pos[rows]
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    # A pad query reads a zero row; allowed_mask gives it no keys anyway.
    qsel = np.zeros(q.shape[:2] + (len(local_tok), d))
    real = local_tok < seq_len
    qsel[:, :, real] = q[:, :, local_tok[real]]
    k_pos = np.arange(seq_len)

    def local_window(nat):
        if nat is None:
            return None
        w = np.zeros(len(local_tok), dtype=np.int64)   # pad queries attend nothing anyway
        w[real] = np.asarray(nat)[local_tok[real]]
        return w
    return full_attention(qsel, k, v, local_pos, k_pos, causal, scale, kw_lo=local_window(kw_lo_nat),
                          kw_hi=local_window(kw_hi_nat))


# ---------------------------------------------------------------------------
# Blockwise (ring) computation with online softmax:
# "Sequence Parallelism and Ring Attention", "Deep dive" and "Technical
# insight": keep a running max and a running normaliser, rescale the earlier
# partial sums whenever a larger score shows up.
# ---------------------------------------------------------------------------

def init_state(b_: int, h_: int, lq: int, d: int):
    """Running state before any block: O = 0 (unnormalised), m = -inf, l = 0."""
    return (np.zeros((b_, h_, lq, d)), np.full((b_, h_, lq), -np.inf), np.zeros((b_, h_, lq)))


def fold_block(state, q, k_blk, v_blk, q_pos, k_pos, causal: bool, scale=None, kw_lo=None, kw_hi=None):
    """Fold one arriving KV block into the running (O, m, l).

    m is the running max of the allowed scaled scores (natural-log units), l
    the running sum of exp(score - m), O the running sum of exp(score - m) * v.
    With m_new = max(m, block max), earlier sums are rescaled by exp(m - m_new).
    A row with nothing allowed so far keeps m = -inf, l = 0, O = 0.
    """
    o, m, l = (np.array(x, dtype=np.float64) for x in state)
    q = np.asarray(q, dtype=np.float64)
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    ok = allowed_mask(q_pos, k_pos, causal, kw_lo, kw_hi)
    b_, h_ = q.shape[:2]
    h_kv = k_blk.shape[1]
    for b in range(b_):
        for h in range(h_):
            hk = kv_head(h, h_, h_kv)
            s = np.where(ok, scale * (q[b, h] @ k_blk[b, hk].T), -np.inf)
            m_new = np.maximum(m[b, h], s.max(axis=1))
            fin = np.isfinite(m_new)
            m_use = np.where(fin, m_new, 0.0)
            alpha = np.where(np.isfinite(m[b, h]), np.exp(m[b, h] - m_use), 0.0)
            p = np.where(ok, np.exp(s - m_use[:, None]), 0.0)
            l[b, h] = alpha * l[b, h] + p.sum(axis=1)
            o[b, h] = alpha[:, None] * o[b, h] + p @ v_blk[b, hk]
            m[b, h] = m_new
    return o, m, l


def merge(state1, state2):
    """Combine two partial states over disjoint key sets.

    The same rescaling rule as ``fold_block``, applied to two already-reduced
    partials: m = max(m1, m2), each side scaled by exp(m_i - m).
    """
    o1, m1, l1 = (np.asarray(x, dtype=np.float64) for x in state1)
    o2, m2, l2 = (np.asarray(x, dtype=np.float64) for x in state2)
    m = np.maximum(m1, m2)
    m_use = np.where(np.isfinite(m), m, 0.0)
    a1 = np.where(np.isfinite(m1), np.exp(m1 - m_use), 0.0)
    a2 = np.where(np.isfinite(m2), np.exp(m2 - m_use), 0.0)
    return a1[..., None] * o1 + a2[..., None] * o2, m, a1 * l1 + a2 * l2


def finalize(state):
    """Normalise: O / l and LSE = m + ln l; a row with l = 0 gives O = 0, LSE = -inf."""
    o, m, l = (np.asarray(x, dtype=np.float64) for x in state)
    has = l > 0
    out = np.zeros_like(o)
    out[has] = o[has] / l[has][:, None]
    lse = np.full(m.shape, -np.inf)
    lse[has] = m[has] + np.log(l[has])
    return out, lse


def ring_emulation(q_local, k_ring, v_ring, q_pos, ring_pos, cp: int, rank: int, causal: bool,
                   scale=None, order=None, keep_states: bool = False, kw_lo=None, kw_hi=None):
    """One rank's whole ring pass, block by block, in fp64.

    q_local [B, H, Lq, D] with global positions q_pos [Lq]; k_ring/v_ring
    [B, H, S_pad, D] hold every rank's block rank-major (block s = rows
    [s*Lk, (s+1)*Lk)), with positions ring_pos [S_pad]. Step t folds the block
    of rank ``ring_source(rank, t, cp)``; ``order`` overrides the step order
    (the result must not depend on it beyond rounding).
    Returns (O, LSE) after finalising, plus the state after each step when
    ``keep_states``.
    """
    q_local = np.asarray(q_local, dtype=np.float64)
    b_, h_, lq, d = q_local.shape
    s_pad = np.asarray(k_ring).shape[2]
    lk = s_pad // cp
    state = init_state(b_, h_, lq, np.asarray(v_ring).shape[-1])
    states = []
    steps = range(cp) if order is None else order
    for t in steps:
        src = ring_source(rank, t, cp) if order is None else t
        sl = slice(src * lk, (src + 1) * lk)
        state = fold_block(state, q_local, np.asarray(k_ring)[:, :, sl], np.asarray(v_ring)[:, :, sl],
                           q_pos, np.asarray(ring_pos)[sl], causal, scale, kw_lo, kw_hi)
        if keep_states:
            states.append(state)
    out = finalize(state)
    return (out, states) if keep_states else out


# ---------------------------------------------------------------------------
# Backward pass. The glossary page's example ("Context Parallelism",
# "Practical use and trade-offs") calls .backward() on the context-parallel
# attention output: the gradients of softmax attention, here the textbook
# derivative written out, and the same gradients taken block by block in ring
# order with the log-sum-exp saved by the forward pass.
# ---------------------------------------------------------------------------

def _score_grad(p, dp, dvec):
    """dL/dS for S -> P = softmax(S): P * (dP - rowsum(dO * O)), the softmax Jacobian applied row by row."""
    return p * (dp - dvec[:, None])


def attention_backward(q, k, v, do, q_pos, k_pos, causal: bool, scale=None, kw_lo=None, kw_hi=None):
    """Gradients of O = softmax(scale * Q K^T + mask) V with respect to Q, K, V, fp64.

    q, do [B, H, Nq, D]; k, v [B, H_kv, Nk, D] (query head h reads K/V head
    kv_head(h, H, H_kv), so dK and dV sum over the heads of a group). With
    P the masked softmax, O = P V and Dvec = rowsum(dO * O):
    dV = P^T dO, dP = dO V^T, dS = P * (dP - Dvec), dQ = scale * dS K,
    dK = scale * dS^T Q. Rows that may attend no key have P = 0 and dQ = 0.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    b_, h_, nq, d = q.shape
    h_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ok = allowed_mask(q_pos, k_pos, causal, kw_lo, kw_hi)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(b_):
        for h in range(h_):
            hk = kv_head(h, h_, h_kv)
            s = np.where(ok, scale * (q[b, h] @ k[b, hk].T), -np.inf)
            m = s.max(axis=1)
            has = np.isfinite(m)
            p = np.where(ok, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
            l = p.sum(axis=1)
            p[has] /= l[has, None]
            o = p @ v[b, hk]
            dvec = (do[b, h] * o).sum(axis=1)
            dv[b, hk] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, hk].T
            ds = _score_grad(p, dp, dvec)
            dq[b, h] = scale * (ds @ k[b, hk])
            dk[b, hk] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def ring_backward(q_local, k_ring, v_ring, o_local, do_local, lse_local, q_pos, ring_pos, cp: int, rank: int,
                  causal: bool, scale=None, kw_lo=None, kw_hi=None):
    """One rank's backward ring pass, block by block, fp64.

    Inputs as for ``ring_emulation`` plus the rank's forward output O, the
    upstream gradient dO and the saved LSE [B, H, Lq]. Each step recomputes the
    block's probabilities P = exp(scale * q k^T - LSE) (the saved LSE makes
    them final, no rescaling), accumulates the rank's dQ locally and adds the
    rank's contributions to the block's dK and dV, which travel with the block
    around the ring. Returns dQ [B, H, Lq, D] and the contributions
    dK, dV [B, H_kv, S_pad, D] in ring order.
    """
    q, o, do, lse = (np.asarray(x, dtype=np.float64) for x in (q_local, o_local, do_local, lse_local))
    k_ring = np.asarray(k_ring, dtype=np.float64)
    v_ring = np.asarray(v_ring, dtype=np.float64)
    b_, h_, lq, d = q.shape
    h_kv = k_ring.shape[1]
    s_pad = k_ring.shape[2]
    lk = s_pad // cp
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dvec = (do * o).sum(axis=-1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k_ring)
    dv = np.zeros_like(v_ring)
    for t in range(cp):
        src = ring_source(rank, t, cp)
        sl = slice(src * lk, (src + 1) * lk)
        ok = allowed_mask(q_pos, np.asarray(ring_pos)[sl], causal, kw_lo, kw_hi)
        for b in range(b_):
            for h in range(h_):
                hk = kv_head(h, h_, h_kv)
                s = scale * (q[b, h] @ k_ring[b, hk, sl].T)
                fin = np.isfinite(lse[b, h])
                p = np.where(ok & fin[:, None], np.exp(s - np.where(fin, lse[b, h], 0.0)[:, None]), 0.0)
                dv[b, hk, sl] += p.T @ do[b, h]
                dp = do[b, h] @ v_ring[b, hk, sl].T
                ds = _score_grad(p, dp, dvec[b, h])
                dq[b, h] += scale * (ds @ k_ring[b, hk, sl])
                dk[b, hk, sl] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def rows_backward(q, k, v, o, do, lse, q_pos, k_pos, causal: bool, scale=None, kw_lo=None, kw_hi=None,
                  q_rows=None, k_rows=None):
    """The same gradients as ``ring_backward`` for chosen rows only, fp64, one (b, h) slice.

    q, o, do [Nq, D] with lse [Nq] (the saved forward results), k, v [Nk, D].
    Returns dQ for the query rows ``q_rows`` ([len, D]) and dK, dV for the key
    rows ``k_rows``: dQ_i = scale * sum_j dS_ij k_j, dK_j = scale * sum_i dS_ij q_i,
    dV_j = sum_i P_ij dO_i with P_ij = exp(scale q_i.k_j - lse_i) (0 where
    masked or lse_i = -inf) and dS_ij = P_ij (dO_i.v_j - rowsum(dO_i * O_i)).
    Order of keys and queries is irrelevant, so no block structure is needed.
    """
    q, k, v, o, do, lse = (np.asarray(x, dtype=np.float64) for x in (q, k, v, o, do, lse))
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    q_pos, k_pos = np.asarray(q_pos), np.asarray(k_pos)
    dvec = (do * o).sum(axis=-1)
    fin = np.isfinite(lse)

    def probs(qi, kj):
        ok = allowed_mask(q_pos[qi], k_pos[kj], causal, None if kw_lo is None else np.asarray(kw_lo)[qi],
                          None if kw_hi is None else np.asarray(kw_hi)[qi])
        s = scale * (q[qi] @ k[kj].T)
        return np.where(ok & fin[qi][:, None], np.exp(s - np.where(fin[qi], lse[qi], 0.0)[:, None]), 0.0)

    all_q, all_k = np.arange(len(q)), np.arange(len(k))
    dq = dk = dv = None
    if q_rows is not None:
        qi = np.asarray(q_rows)
        p = probs(qi, all_k)
        ds = _score_grad(p, do[qi] @ v.T, dvec[qi])
        dq = scale * (ds @ k)
    if k_rows is not None:
        kj = np.asarray(k_rows)
        p = probs(all_q, kj)
        ds = _score_grad(p, do @ v[kj].T, dvec)
        dk = scale * (ds.T @ q)
        dv = p.T @ do
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Work counts (the load-balance claim of the Megatron page).
# ---------------------------------------------------------------------------

def count_pairs(q_pos, k_pos, causal: bool) -> int:
    """Brute-force number of allowed (query, key) pairs."""
    return int(allowed_mask(q_pos, k_pos, causal).sum())


def causal_pairs_striped(s_pad: int, cp: int, rank: int) -> int:
    """Allowed causal pairs for one rank under the striped layout, no padding.

    Local query i of rank r sits at position i*cp + r and sees the keys at
    positions 0 .. i*cp + r, i.e. i*cp + r + 1 of them; summed over the
    Lr = s_pad/cp local queries: cp*Lr*(Lr-1)/2 + Lr*(r+1).
    """
    lr = s_pad // cp
    return cp * lr * (lr - 1) // 2 + lr * (rank + 1)


def causal_pairs_zigzag(s_pad: int, cp: int) -> int:
    """Allowed causal pairs for one rank under zigzag, with no padding: 2*cp*c^2 + c.

    With c = s_pad/(2*cp): the front chunk r sees r full chunks plus its own
    triangle, the back chunk 2cp-1-r sees 2cp-1-r full chunks plus its own
    triangle, so r*c^2 + (2cp-1-r)*c^2 + 2*c(c+1)/2 = 2cp*c^2 + c for any r.
    """
    c = s_pad // (2 * cp)
    return 2 * cp * c * c + c
