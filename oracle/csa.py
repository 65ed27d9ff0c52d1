"""Plain fp64 CPU reference of the CSA / HCA attention hot path.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  It shares no code with the
HIP path (no kernels, headers, tables or helpers); both sides only share the
seeded input generators in ``synth``.

What the pages fix (b-lab.team summary of DeepSeek-V4, "Core Methodological
Innovations", item 1, Hybrid Attention Architecture):
  * CSA shrinks the cache m-fold: each run of m neighbouring KV entries
    becomes one stored entry; an indexer (the "Lightning Indexer") ranks the
    stored entries using low-rank projections of the query's hidden state, and
    attention then visits only the k best-ranked ones;
  * HCA compresses by m' >> m and attends densely over what remains;
  * both add a sliding window of local (uncompressed) KV entries.
Everything else is a reading, stated where it is used:
  R-visibility  block j covers raw positions [j*m, j*m+m-1]; it exists for a
                query at position t only once complete (j*m+m-1 <= t).
  R-window      window = raw positions max(0, t-W+1) .. t (the query's own token
                included).
  R-merge       c_j = sum_r softmax(z)_r * x[j*m + r], one logit per offset r,
                shared by every channel and block; separate logits for the KV
                stream and the indexer-key stream.
  R-indexer     I(t, j) = sum_h w[t,h] * max(0, <q_I[t,h], kappa_j>) (the
                DeepSeek-V3.2 lightning-indexer form; the pages name the
                indexer but print no formula).
  R-topk        total order: score descending, then block index ascending; the
                selected set is output in ascending index order, padded with -1.
  R-union       the attended entries are the selected compressed rows followed
                by the window's raw rows, as a multiset (no de-duplication), in
                one softmax; key = value = the stored (shared, MQA) row.
  R-scale       logits are scale * <q_h, e>, scale an argument.
  R-query       the indexer's query is a two-stage low-rank projection of the
                query's hidden state h (down to rank r, then up to H_I heads of
                d_I), and its head weights a direct projection of h; no norm,
                activation or rotary term in between.
All arithmetic is fp64 on the (dequantised) stored values.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# visibility
# ----------------------------------------------------------------------------


def visible_blocks(t: int, m: int) -> int:
    """Number of complete blocks of size m at query position t (R-visibility):
    block j is visible iff j*m + m - 1 <= t, i.e. j < (t + 1) // m."""
    if t < 0:
        return 0
    return (int(t) + 1) // int(m)


def window_positions(t: int, window: int) -> np.ndarray:
    """Raw positions in the sliding window of a query at t (R-window)."""
    lo = max(0, int(t) - int(window) + 1)
    return np.arange(lo, int(t) + 1, dtype=np.int64)


# ----------------------------------------------------------------------------
# (a) compression
# ----------------------------------------------------------------------------


def merge_weights(logits) -> np.ndarray:
    """omega = softmax(z) over the m offsets, max-subtracted, fp64 (R-merge)."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - np.max(z)
    e = np.exp(z)
    return e / np.sum(e)


def compress(raw, raw_base, logits, m, block_first, block_count):
    """Merge every requested block of m adjacent raw rows into one entry (R-merge).

    raw:        [B, R, D] stored raw rows (values), row r of sequence b holds
                absolute position raw_base[b] + r.
    block_first, block_count: [B] the blocks j = block_first[b] ..
                block_first[b] + block_count[b] - 1 to produce for sequence b.
    Returns a list (one per sequence) of (first_block, values [count, D] fp64).
    """
    raw = np.asarray(raw, dtype=np.float64)
    omega = merge_weights(logits)
    assert omega.shape[0] == m
    out = []
    for b in range(raw.shape[0]):
        j0, cnt = int(block_first[b]), int(block_count[b])
        rows = np.zeros((cnt, raw.shape[2]), dtype=np.float64)
        for i in range(cnt):
            j = j0 + i
            acc = np.zeros(raw.shape[2], dtype=np.float64)
            for r in range(m):  # offsets in ascending order
                acc = acc + omega[r] * raw[b, j * m + r - int(raw_base[b])]
            rows[i] = acc
        out.append((j0, rows))
    return out


# ----------------------------------------------------------------------------
# indexer query from the hidden state (the step before (b))
# ----------------------------------------------------------------------------


def index_query(h, w_dq, w_uq, w_w, n_idx_heads: int, idx_dim: int):
    """The indexer's per-head query and head weights from the query hidden state
    (b-lab.team summary of DeepSeek-V4, Core Methodological Innovations 1, CSA
    bullet: the indexer scores with low-rank projections of h_t; R-query):
        c = W_dq h            (rank r)
        q_I = reshape(W_uq c, [H_I, d_I])
        w = W_w h

    h [..., d], w_dq [r, d], w_uq [H_I * d_I, r], w_w [H_I, d]
    -> (q_I [..., H_I, d_I], w [..., H_I]).
    """
    h = np.asarray(h, dtype=np.float64)
    w_dq = np.asarray(w_dq, dtype=np.float64)
    w_uq = np.asarray(w_uq, dtype=np.float64)
    w_w = np.asarray(w_w, dtype=np.float64)
    assert w_uq.shape == (n_idx_heads * idx_dim, w_dq.shape[0])
    c = h @ w_dq.T
    q = (c @ w_uq.T).reshape(h.shape[:-1] + (n_idx_heads, idx_dim))
    return q, h @ w_w.T


def latent_query(q, w_uk):
    """MLA absorbed query (R-latent): the head's key up-projection moved onto the
    query.  Head h reads the shared latent row c through the key k_h = W_uk[h] c, so
    <q_h, W_uk[h] c> = <W_uk[h]^T q_h, c>: the attention score needs only the
    absorbed query q_lat_h = W_uk[h]^T q_h against the stored latent rows.

    q [..., H, dh], w_uk [H, dh, D] -> q_lat [..., H, D].
    """
    q = np.asarray(q, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    H, dh, D = w_uk.shape
    assert q.shape[-2:] == (H, dh)
    out = np.empty(q.shape[:-1] + (D,))
    for h in range(H):
        out[..., h, :] = q[..., h, :] @ w_uk[h]
    return out


def latent_output(o_lat, w_uv):
    """MLA output up-projection (R-latent): the value of head h is v_h = W_uv[h] c, and
    attention is linear in its values, so sum_j p_j W_uv[h] c_j = W_uv[h] (sum_j p_j c_j):
    the head's output is its latent attention output mapped by W_uv[h].

    o_lat [..., H, D], w_uv [H, dh, D] -> o [..., H, dh].
    """
    o_lat = np.asarray(o_lat, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    H, dh, D = w_uv.shape
    assert o_lat.shape[-2:] == (H, D)
    out = np.empty(o_lat.shape[:-1] + (dh,))
    for h in range(H):
        out[..., h, :] = o_lat[..., h, :] @ w_uv[h].T
    return out


# ----------------------------------------------------------------------------
# (b) lightning-indexer scores
# ----------------------------------------------------------------------------


def index_scores(q_idx, w, k_idx, q_pos, m, n_cap=None):
    """I[b, t, j] = sum_h w[b,t,h] * relu(<q_idx[b,t,h], k_idx[b,j]>) for visible j,
    -inf for j that is not yet a complete block (R-indexer, R-visibility).

    q_idx [B, Tq, H_I, d_I], w [B, Tq, H_I], k_idx [B, N, d_I], q_pos [B, Tq].
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k_idx = np.asarray(k_idx, dtype=np.float64)
    B, Tq, HI, dI = q_idx.shape
    N = k_idx.shape[1] if n_cap is None else int(n_cap)
    out = np.full((B, Tq, N), NEG_INF, dtype=np.float64)
    for b in range(B):
        for t in range(Tq):
            V = visible_blocks(int(q_pos[b, t]), m)
            assert V <= N, "query position beyond the cache capacity"
            if V == 0:
                continue
            dots = k_idx[b, :V] @ q_idx[b, t].T  # [V, H_I]
            out[b, t, :V] = np.maximum(dots, 0.0) @ w[b, t]
    return out


# ----------------------------------------------------------------------------
# (c) top-k
# ----------------------------------------------------------------------------


def topk_row(scores_row, n_visible: int, k: int) -> np.ndarray:
    """The k visible blocks first in the order (score desc, index asc), returned in
    ascending index order and padded with -1 (R-topk).  -0.0 equals +0.0."""
    V = int(n_visible)
    vals = np.asarray(scores_row[:V], dtype=np.float64) + 0.0  # -0.0 -> +0.0
    # stable sort on the negated score keeps equal scores in ascending index order
    order = np.argsort(-vals, kind="stable")
    take = np.sort(order[: min(k, V)])
    out = np.full(k, -1, dtype=np.int64)
    out[: take.shape[0]] = take
    return out


def topk(scores, q_pos, m, k):
    scores = np.asarray(scores, dtype=np.float64)
    B, Tq, _ = scores.shape
    out = np.full((B, Tq, k), -1, dtype=np.int64)
    for b in range(B):
        for t in range(Tq):
            out[b, t] = topk_row(scores[b, t], visible_blocks(int(q_pos[b, t]), m), k)
    return out


# ----------------------------------------------------------------------------
# (d)/(e) attention over a set of entries
# ----------------------------------------------------------------------------


def attend(q_heads, entries, scale):
    """Softmax attention of every head over one list of entries (key = value = entry).

    q_heads [H, D], entries [n, D].  Returns out [H, D] and lse [H] (natural log).
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    entries = np.asarray(entries, dtype=np.float64)
    logits = float(scale) * (q_heads @ entries.T)  # [H, n]
    mx = np.max(logits, axis=1, keepdims=True)
    p = np.exp(logits - mx)
    den = np.sum(p, axis=1, keepdims=True)
    out = (p @ entries) / den
    lse = mx[:, 0] + np.log(den[:, 0])
    return out, lse


def csa_entries(kv_cmp_b, idx_row, kv_raw_b, raw_base_b, t, window):
    """Selected compressed rows followed by the window's raw rows (R-union)."""
    sel = [int(j) for j in idx_row if int(j) >= 0]
    win = window_positions(t, window) - int(raw_base_b)
    parts = []
    if sel:
        parts.append(np.asarray(kv_cmp_b, dtype=np.float64)[sel])
    if win.size:
        parts.append(np.asarray(kv_raw_b, dtype=np.float64)[win])
    return np.concatenate(parts, axis=0)


def csa_sparse_attn(q, kv_cmp, idx, kv_raw, raw_base, window, q_pos, scale):
    """(d) CSA: attention over the top-k compressed rows plus the sliding window.

    q [B, Tq, H, D], kv_cmp [B, N, D], idx [B, Tq, k], kv_raw [B, R, D].
    Returns out [B, Tq, H, D], lse [B, Tq, H].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Tq, H, D = q.shape
    out = np.zeros((B, Tq, H, D))
    lse = np.zeros((B, Tq, H))
    for b in range(B):
        for t in range(Tq):
            E = csa_entries(kv_cmp[b], idx[b, t], kv_raw[b], raw_base[b], int(q_pos[b, t]), window)
            out[b, t], lse[b, t] = attend(q[b, t], E, scale)
    return out, lse


def hca_attn(q, kv_hc, m_hc, kv_raw, raw_base, window, q_pos, scale):
    """(e) HCA: dense attention over every complete heavily-compressed block plus the
    same sliding window."""
    q = np.asarray(q, dtype=np.float64)
    B, Tq, H, D = q.shape
    out = np.zeros((B, Tq, H, D))
    lse = np.zeros((B, Tq, H))
    for b in range(B):
        for t in range(Tq):
            pos = int(q_pos[b, t])
            V = visible_blocks(pos, m_hc)
            idx_all = np.arange(V)
            E = csa_entries(kv_hc[b], idx_all, kv_raw[b], raw_base[b], pos, window)
            out[b, t], lse[b, t] = attend(q[b, t], E, scale)
    return out, lse


# ----------------------------------------------------------------------------
# a whole CSA decode / prefill layer, stage by stage (for end-to-end checks)
# ----------------------------------------------------------------------------


def csa_layer(q, q_idx, w, kv_cmp, k_idx, kv_raw, raw_base, q_pos, m, k, window, scale):
    scores = index_scores(q_idx, w, k_idx, q_pos, m, n_cap=np.asarray(k_idx).shape[1])
    idx = topk(scores, q_pos, m, k)
    out, lse = csa_sparse_attn(q, kv_cmp, idx, kv_raw, raw_base, window, q_pos, scale)
    return scores, idx, out, lse
