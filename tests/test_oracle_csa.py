"""Pins for the CPU oracle of the CSA / HCA path.

The pages print no worked example, so every pin is a closed form, an invariant,
a library routine (torch's scaled_dot_product_attention in fp64, numpy's mean
and argmax) or brute force written as plain Python loops over the definitions.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

import oracle
from oracle import csa as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- visibility


def test_visible_blocks_brute_force():
    for m in (1, 2, 4, 7, 128):
        for t in range(-1, 600):
            want = sum(1 for j in range(700) if j * m + m - 1 <= t)
            assert O.visible_blocks(t, m) == want


def test_window_positions_brute_force():
    for W in (0, 1, 5, 64):
        for t in (0, 3, 63, 64, 200):
            want = [p for p in range(t + 1) if t - p < W]
            assert list(O.window_positions(t, W)) == want


# ----------------------------------------------------------------------------- compressor


def _raw(B=2, R=40, D=6, seed=0):
    return np.random.default_rng(seed).standard_normal((B, R, D))


def test_compress_m1_is_identity():
    x = _raw()
    out = O.compress(x, [0, 0], [0.3], 1, [0, 5], [40, 10])
    np.testing.assert_array_equal(out[0][1], x[0])
    np.testing.assert_array_equal(out[1][1], x[1, 5:15])


def test_compress_equal_logits_is_block_mean():
    x = _raw()
    m = 4
    out = O.compress(x, [0, 0], [1.5] * m, m, [0, 0], [10, 10])
    for b in range(2):
        want = x[b].reshape(10, m, -1).mean(axis=1)
        np.testing.assert_allclose(out[b][1], want, rtol=0, atol=1e-15)


def test_compress_dominant_logit_subsamples():
    x = _raw()
    out = O.compress(x, [0, 0], [0.0, -1000.0, -1000.0, -1000.0], 4, [0, 0], [10, 10])
    np.testing.assert_array_equal(out[0][1], x[0, 0::4])


def test_compress_hand_derived_golden():
    with open(os.path.join(GOLDEN, "compress_hand.json")) as f:
        g = json.load(f)
    out = O.compress(np.array(g["raw"], dtype=np.float64)[None], [g["raw_base"]], g["logits"],
                     g["m"], [g["block_first"]], [g["block_count"]])
    np.testing.assert_allclose(out[0][1], np.array(g["expected"]), rtol=1e-14, atol=1e-14)


def test_compress_brute_force_and_raw_base():
    r = np.random.default_rng(4)
    m, D = 3, 5
    x = r.standard_normal((1, 30, D))
    z = r.standard_normal(m)
    # raw row 0 holds position 12, so block j reads rows j*m + r - 12
    out = O.compress(x, [12], z, m, [4], [5])
    ez = [math.exp(v) for v in z]
    om = [e / sum(ez) for e in ez]
    for i in range(5):
        j = 4 + i
        for d in range(D):
            want = sum(om[rr] * x[0, j * m + rr - 12, d] for rr in range(m))
            assert abs(out[0][1][i, d] - want) < 1e-13


def test_compress_incremental_equals_full():
    x = _raw(B=1, R=64)
    z = [0.1, -0.4, 0.9, 0.2]
    full = O.compress(x, [0], z, 4, [0], [16])[0][1]
    a = O.compress(x, [0], z, 4, [0], [7])[0][1]
    b = O.compress(x, [0], z, 4, [7], [9])[0][1]
    np.testing.assert_array_equal(np.concatenate([a, b]), full)


# ----------------------------------------------------------------------------- indexer query


def test_index_query_hand_derived_golden():
    g = json.load(open(os.path.join(GOLDEN, "index_query_hand.json")))
    q, w = O.index_query(np.array(g["h"]), np.array(g["w_dq"]), np.array(g["w_uq"]), np.array(g["w_w"]),
                         g["n_idx_heads"], g["idx_dim"])
    np.testing.assert_array_equal(q, np.array(g["expected_q"], dtype=np.float64))
    np.testing.assert_array_equal(w, np.array(g["expected_w"], dtype=np.float64))


def test_index_query_brute_force_loops():
    r = np.random.default_rng(11)
    d, rank, HI, dI = 7, 3, 2, 4
    h = r.standard_normal((2, 5, d))
    wdq, wuq, ww = r.standard_normal((rank, d)), r.standard_normal((HI * dI, rank)), r.standard_normal((HI, d))
    q, w = O.index_query(h, wdq, wuq, ww, HI, dI)
    assert q.shape == (2, 5, HI, dI) and w.shape == (2, 5, HI)
    for b in range(2):
        for t in range(5):
            c = [sum(wdq[j, i] * h[b, t, i] for i in range(d)) for j in range(rank)]
            for hh in range(HI):
                assert abs(w[b, t, hh] - sum(ww[hh, i] * h[b, t, i] for i in range(d))) < 1e-12
                for e in range(dI):
                    want = sum(wuq[hh * dI + e, j] * c[j] for j in range(rank))
                    assert abs(q[b, t, hh, e] - want) < 1e-12


def test_index_query_has_rank_at_most_r_and_is_linear():
    r = np.random.default_rng(12)
    d, rank, HI, dI = 64, 5, 4, 8
    wdq, wuq, ww = r.standard_normal((rank, d)), r.standard_normal((HI * dI, rank)), r.standard_normal((HI, d))
    h = r.standard_normal((40, d))
    q, w = O.index_query(h, wdq, wuq, ww, HI, dI)
    assert np.linalg.matrix_rank(q.reshape(40, HI * dI)) == rank  # low rank: the queries span r directions
    a, b = 0.75, -2.5
    q2, w2 = O.index_query(a * h[0] + b * h[1], wdq, wuq, ww, HI, dI)
    np.testing.assert_allclose(q2, a * q[0] + b * q[1], atol=1e-10)
    np.testing.assert_allclose(w2, a * w[0] + b * w[1], atol=1e-10)


def test_latent_projections_hand_derived_golden():
    g = json.load(open(os.path.join(GOLDEN, "latent_proj_hand.json")))
    np.testing.assert_array_equal(O.latent_query(np.array(g["q"]), np.array(g["w_uk"])),
                                  np.array(g["expected_q_lat"], dtype=np.float64))
    np.testing.assert_array_equal(O.latent_output(np.array(g["o_lat"]), np.array(g["w_uv"])),
                                  np.array(g["expected_o"], dtype=np.float64))


def test_latent_projections_brute_force_loops():
    r = np.random.default_rng(13)
    H, dh, D = 3, 4, 5
    q, o = r.standard_normal((2, H, dh)), r.standard_normal((2, H, D))
    wuk, wuv = r.standard_normal((H, dh, D)), r.standard_normal((H, dh, D))
    ql, oo = O.latent_query(q, wuk), O.latent_output(o, wuv)
    for t in range(2):
        for h in range(H):
            for j in range(D):
                assert abs(ql[t, h, j] - sum(wuk[h, i, j] * q[t, h, i] for i in range(dh))) < 1e-12
            for i in range(dh):
                assert abs(oo[t, h, i] - sum(wuv[h, i, j] * o[t, h, j] for j in range(D))) < 1e-12


def test_absorbed_latent_attention_equals_per_head_sdpa():
    """MLA absorption: attention of the absorbed queries over the shared latent rows,
    mapped by the value up-projection, equals ordinary multi-head attention with each
    head's own keys K_h = C W_uk[h]^T and values V_h = C W_uv[h]^T (torch SDPA, fp64)."""
    import torch
    r = np.random.default_rng(14)
    H, dh, D, n = 4, 6, 10, 9
    q = r.standard_normal((H, dh))
    C = r.standard_normal((n, D))
    wuk, wuv = r.standard_normal((H, dh, D)) / 3, r.standard_normal((H, dh, D))
    scale = 0.37
    o_lat, _ = O.attend(O.latent_query(q, wuk), C, scale)
    got = O.latent_output(o_lat, wuv)
    K = torch.tensor(np.stack([C @ wuk[h].T for h in range(H)]))  # [H, n, dh]
    V = torch.tensor(np.stack([C @ wuv[h].T for h in range(H)]))
    want = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q)[:, None], K, V, scale=scale)[:, 0]
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- indexer


def test_index_scores_brute_force():
    r = np.random.default_rng(1)
    B, Tq, HI, dI, N, m = 2, 3, 3, 5, 12, 2
    q = r.standard_normal((B, Tq, HI, dI))
    w = r.standard_normal((B, Tq, HI))
    k = r.standard_normal((B, N, dI))
    pos = np.array([[3, 10, 23], [0, 1, 17]])
    s = O.index_scores(q, w, k, pos, m)
    for b in range(B):
        for t in range(Tq):
            for j in range(N):
                if j * m + m - 1 <= pos[b, t]:
                    want = 0.0
                    for h in range(HI):
                        dot = sum(q[b, t, h, d] * k[b, j, d] for d in range(dI))
                        want += w[b, t, h] * max(0.0, dot)
                    assert abs(s[b, t, j] - want) < 1e-12
                else:
                    assert s[b, t, j] == -np.inf


def test_index_scores_single_head_unit_weight_is_relu_matvec():
    r = np.random.default_rng(2)
    q = r.standard_normal((1, 1, 1, 8))
    k = r.standard_normal((1, 20, 8))
    s = O.index_scores(q, np.ones((1, 1, 1)), k, np.array([[79]]), 4)
    np.testing.assert_allclose(s[0, 0], np.maximum(np.einsum("nd,d->n", k[0], q[0, 0, 0]), 0), atol=1e-14)


def test_index_selection_invariant_under_positive_head_weight_scale():
    r = np.random.default_rng(3)
    q = r.standard_normal((1, 1, 4, 8))
    w = r.standard_normal((1, 1, 4))
    k = r.standard_normal((1, 64, 8))
    pos = np.array([[255]])
    a = O.topk(O.index_scores(q, w, k, pos, 4), pos, 4, 10)
    b = O.topk(O.index_scores(q, 3.7 * w, k, pos, 4), pos, 4, 10)
    np.testing.assert_array_equal(a, b)


# ----------------------------------------------------------------------------- top-k


def _rank_topk(vals, k):
    """Definition by rank: j is selected iff fewer than k entries precede it in the
    order (score desc, index asc)."""
    V = len(vals)
    sel = []
    for j in range(V):
        rank = sum(1 for i in range(V) if vals[i] > vals[j] or (vals[i] == vals[j] and i < j))
        if rank < k:
            sel.append(j)
    return sel


def test_topk_matches_rank_definition_with_ties():
    r = np.random.default_rng(8)
    for trial in range(60):
        V = int(r.integers(1, 60))
        k = int(r.integers(1, 70))
        vals = r.integers(-3, 4, V).astype(np.float64)  # many exact ties
        vals[vals == 0] = np.where(r.random((vals == 0).sum()) < 0.5, -0.0, 0.0)
        got = O.topk_row(vals, V, k)
        want = _rank_topk(list(vals), k)
        assert list(got[: len(want)]) == want
        assert np.all(got[len(want):] == -1)


def test_topk_ignores_invisible_tail_and_pads():
    s = np.array([[[1.0, 5.0, 2.0, 9.0, 100.0, 100.0]]])
    got = O.topk(s, np.array([[15]]), 4, 6)  # only blocks 0..3 visible at t=15, m=4
    assert list(got[0, 0]) == [0, 1, 2, 3, -1, -1]


def test_topk_k1_is_first_argmax():
    r = np.random.default_rng(6)
    for _ in range(50):
        v = r.integers(0, 5, 30).astype(np.float64)
        assert O.topk_row(v, 30, 1)[0] == int(np.argmax(v))


# ----------------------------------------------------------------------------- attention


def _sdpa(q, k, v, mask=None, causal=False):
    return TF.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                           attn_mask=None if mask is None else torch.from_numpy(mask),
                                           is_causal=causal, scale=float(1 / np.sqrt(128))).numpy()


def test_csa_m1_allk_no_window_is_dense_causal_attention():
    """m = 1, k >= #visible and W = 0: CSA reduces to exact dense causal attention."""
    r = np.random.default_rng(10)
    T, H, D = 24, 3, 16
    x = r.standard_normal((1, T, D))
    q = r.standard_normal((1, T, H, D))
    pos = np.arange(T)[None]
    kv_cmp = O.compress(x, [0], [0.0], 1, [0], [T])[0][1][None]
    k = T + 5
    q_idx = r.standard_normal((1, T, 2, 4))
    w = r.standard_normal((1, T, 2))
    _, idx, out, lse = O.csa_layer(q, q_idx, w, kv_cmp, kv_cmp[..., :4], x, [0], pos, 1, k, 0, 1 / np.sqrt(128))
    # reference: SDPA over heads with a causal mask, key = value = x
    qh = np.transpose(q[0], (1, 0, 2))[None]            # [1, H, T, D]
    kh = np.broadcast_to(x[0][None, None], (1, H, T, D)).copy()
    ref = _sdpa(qh, kh, kh, causal=True)[0]             # [H, T, D]
    np.testing.assert_allclose(out[0], np.transpose(ref, (1, 0, 2)), rtol=1e-12, atol=1e-12)


def test_csa_window_doubles_weight_of_window_tokens():
    """With W > 0 the window is not de-duplicated: weights are (1 + [p in window]) * exp(l_p),
    i.e. dense attention with an additive log(2) on window positions."""
    r = np.random.default_rng(12)
    T, H, D, W = 20, 2, 8, 5
    x = r.standard_normal((1, T, D))
    q = r.standard_normal((1, T, H, D))
    pos = np.arange(T)[None]
    idx = np.array([[list(range(t + 1)) + [-1] * (T - t - 1) for t in range(T)]])
    out, _ = O.csa_sparse_attn(q, x, idx, x, [0], W, pos, 1 / np.sqrt(128))
    mask = np.full((T, T), -np.inf)
    for t in range(T):
        for p in range(t + 1):
            mask[t, p] = math.log(2.0) if t - p < W else 0.0
    qh = np.transpose(q[0], (1, 0, 2))[None]
    kh = np.broadcast_to(x[0][None, None], (1, H, T, D)).copy()
    ref = _sdpa(qh, kh, kh, mask=mask[None, None])[0]
    np.testing.assert_allclose(out[0], np.transpose(ref, (1, 0, 2)), rtol=1e-12, atol=1e-12)


def test_attend_brute_force():
    r = np.random.default_rng(13)
    H, D, n = 2, 3, 5
    q = r.standard_normal((H, D))
    E = r.standard_normal((n, D))
    out, lse = O.attend(q, E, 0.7)
    for h in range(H):
        logits = [0.7 * sum(q[h, d] * E[e, d] for d in range(D)) for e in range(n)]
        z = sum(math.exp(l) for l in logits)
        assert abs(lse[h] - math.log(z)) < 1e-12
        for d in range(D):
            assert abs(out[h, d] - sum(math.exp(l) / z * E[e, d] for e, l in enumerate(logits))) < 1e-12


def test_attend_special_cases():
    r = np.random.default_rng(14)
    q = r.standard_normal((4, 8))
    e = r.standard_normal((1, 8))
    out, lse = O.attend(q, e, 0.5)
    np.testing.assert_allclose(out, np.repeat(e, 4, axis=0), atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * q @ e[0], atol=1e-14)
    out, lse5 = O.attend(q, np.repeat(e, 5, axis=0), 0.5)
    np.testing.assert_allclose(out, np.repeat(e, 4, axis=0), atol=1e-14)
    np.testing.assert_allclose(lse5, lse + math.log(5), atol=1e-13)
    # the weights exp(l - lse) sum to one
    E = r.standard_normal((30, 8))
    _, lse = O.attend(q, E, 0.3)
    w = np.exp(0.3 * q @ E.T - lse[:, None])
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12)


def test_attend_hand_derived_golden():
    with open(os.path.join(GOLDEN, "attend_hand.json")) as f:
        g = json.load(f)
    out, lse = O.attend(np.array(g["q"]), np.array(g["entries"]), g["scale"])
    np.testing.assert_allclose(out, np.array(g["expected_out"]), atol=1e-14)
    np.testing.assert_allclose(lse, np.array(g["expected_lse"]), atol=1e-14)


def test_attention_permutation_invariant():
    r = np.random.default_rng(15)
    q = r.standard_normal((3, 6))
    E = r.standard_normal((11, 6))
    a = O.attend(q, E, 0.4)
    b = O.attend(q, E[r.permutation(11)], 0.4)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_csa_with_all_blocks_equals_hca():
    """CSA with k >= #visible selects every complete block, which is HCA with m' = m."""
    r = np.random.default_rng(16)
    B, m, N, D, H, W = 2, 8, 10, 16, 4, 6
    kv_c = r.standard_normal((B, N, D))
    raw = r.standard_normal((B, 100, D))
    q = r.standard_normal((B, 1, H, D))
    pos = np.array([[70], [45]])
    idx = np.array([[list(range(O.visible_blocks(int(p), m))) + [-1] * (N - O.visible_blocks(int(p), m))]
                    for p in pos[:, 0]])
    a = O.csa_sparse_attn(q, kv_c, idx, raw, [0, 0], W, pos, 0.1)
    b = O.hca_attn(q, kv_c, m, raw, [0, 0], W, pos, 0.1)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_hca_entry_set_brute_force():
    """HCA attends to blocks j with j*m'+m'-1 <= t, then raw positions t-W+1..t."""
    r = np.random.default_rng(17)
    m, D, H, W = 16, 4, 2, 3
    kv_h = r.standard_normal((1, 10, D))
    raw = r.standard_normal((1, 200, D))
    q = r.standard_normal((1, 1, H, D))
    t = 100
    out, lse = O.hca_attn(q, kv_h, m, raw, [40], W, np.array([[t]]), 1.0)
    ents = [kv_h[0, j] for j in range(10) if j * m + m - 1 <= t] + [raw[0, p - 40] for p in range(t - W + 1, t + 1)]
    ref, ref_lse = O.attend(q[0, 0], np.array(ents), 1.0)
    assert len(ents) == 6 + 3
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], ref_lse, atol=1e-14)
