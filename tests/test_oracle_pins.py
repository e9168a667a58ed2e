"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Every check below compares the oracle with something other than itself: a
closed form, a library routine applied to the definition (SVD of the
explicit d_model x d_model operator, scaled-dot-product attention), brute
force on tiny inputs, an invariance of RoPE, or the planted structure of the
generator.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import aoh, clsa, fasa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ AoH
def test_sylvester_proxy_spectrum_matches_explicit_operator():
    """AoH §3: eig(C_h) are the squared nonzero singular values of the
    explicitly built M_h = W_K^T W_Q (d_model x d_model)."""
    r = _rng(1)
    for d_model, d in [(24, 6), (40, 8), (16, 16)]:
        wq = r.standard_normal((d, d_model))
        wk = r.standard_normal((d, d_model))
        m = wk.T @ wq
        assert m.shape == (d_model, d_model)
        sv = np.linalg.svd(m, compute_uv=False)
        lam = np.sort(aoh.proxy_eigenvalues(wq, wk))[::-1]
        np.testing.assert_allclose(lam, sv[:d] ** 2, rtol=1e-10, atol=1e-10 * sv[0] ** 2)
        # the eigenvalues of the non-symmetric product agree too
        c = aoh.gram(wq) @ aoh.gram(wk)
        ev = np.sort(np.linalg.eigvals(c).real)[::-1]
        np.testing.assert_allclose(lam, ev, rtol=1e-8, atol=1e-8 * sv[0] ** 2)
        # ER of the proxy equals ER of the explicit operator's singular values
        er_explicit = aoh.effective_rank_from_singular(sv)
        assert aoh.effective_rank(lam) == pytest.approx(er_explicit, rel=1e-8)


def test_er_closed_forms_from_golden():
    with open(os.path.join(GOLDEN, "er_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        want = eval(c["er"], {"math": math})
        assert aoh.effective_rank_from_singular(c["sigma"]) == pytest.approx(want, rel=1e-13), c
        # same spectrum delivered as eigenvalues of C_h (sigma^2)
        assert aoh.effective_rank(np.square(c["sigma"])) == pytest.approx(want, rel=1e-12), c


def _rotated_diag_weights(a, b, d_model, seed):
    """W_Q = diag(a) U^T, W_K = diag(b) U^T, U orthonormal columns:
    M = U diag(a*b) U^T, singular values |a*b|."""
    d = len(a)
    u, _ = np.linalg.qr(_rng(seed).standard_normal((d_model, d)))
    return np.diag(a) @ u.T, np.diag(b) @ u.T


@pytest.mark.parametrize("r", [1, 2, 3, 5, 8])
def test_er_flat_rank_r_through_weights(r):
    d, d_model = 8, 32
    a = np.zeros(d)
    a[:r] = 1.7
    wq, wk = _rotated_diag_weights(a, np.full(d, 0.9), d_model, r)
    lam = aoh.proxy_eigenvalues(wq, wk)
    assert aoh.effective_rank(lam) == pytest.approx(r, rel=1e-6)


def test_er_known_spectrum_through_weights():
    """sigma = (2, 1, 1, 0, ...) built from rotated weights gives 2*sqrt(2)."""
    a = np.array([2.0, 1.0, 1.0, 0.0, 0.0, 0.0])
    b = np.array([1.0, 1.0, 1.0, 3.0, 0.5, 2.0])
    wq, wk = _rotated_diag_weights(a, b, 20, 7)
    assert aoh.effective_rank(aoh.proxy_eigenvalues(wq, wk)) == pytest.approx(2 * math.sqrt(2), rel=1e-6)
    # the key side matters: shrink b on the leading direction
    b2 = b.copy()
    b2[0] = 0.5
    wq, wk = _rotated_diag_weights(a, b2, 20, 7)
    assert aoh.effective_rank(aoh.proxy_eigenvalues(wq, wk)) == pytest.approx(3.0, rel=1e-6)


def test_group_mean_and_ranking():
    """AoH §4: under GQA the group score is the mean of its heads' ER; the k
    lowest groups are retrieval."""
    d, d_model = 4, 12
    u, _ = np.linalg.qr(_rng(3).standard_normal((d_model, d)))
    flat = [1, 3, 2, 4]           # flat rank of each query head's operator
    w_q = np.zeros((1, 4 * d, d_model))
    w_k = np.zeros((1, 2 * d, d_model))
    for h, r in enumerate(flat):
        a = np.zeros(d)
        a[:r] = 1.0
        w_q[0, h * d:(h + 1) * d] = np.diag(a) @ u.T
    for g in range(2):
        w_k[0, g * d:(g + 1) * d] = u.T
    er_head, er_group, lab = aoh.aoh_label(w_q, w_k, 4, 2, d, k=1)
    np.testing.assert_allclose(er_head[0], flat, rtol=1e-6)
    np.testing.assert_allclose(er_group[0], [2.0, 3.0], rtol=1e-6)
    assert lab.tolist() == [[1, 0]]
    _, _, lab_t = aoh.aoh_label(w_q, w_k, 4, 2, d, threshold=2.5)
    assert lab_t.tolist() == [[1, 0]]


def test_ranking_ties_go_to_lower_flat_index():
    er = np.array([[5.0, 1.0, 1.0], [1.0, 9.0, 1.0]])
    assert aoh.labels_top_k(er, 2).tolist() == [[0, 1, 1], [0, 0, 0]]
    assert aoh.labels_top_k(er, 0).sum() == 0
    assert aoh.labels_top_k(er, 6).sum() == 6


# ------------------------------------------------------------------ TIP
def test_tip_over_all_chunks_is_the_exact_logit():
    """FASA §2.A/§2.B.1: summing every chunk's contribution gives q.k; for a
    group, the mean of the heads' logits."""
    r = _rng(5)
    for d, G in [(64, 1), (128, 4)]:
        q = r.standard_normal((G, d))
        k = r.standard_normal((50, d))
        s = fasa.tip_scores(q, k, np.arange(d // 2))
        direct = np.mean([[float(np.dot(qh, kj)) for kj in k] for qh in q], axis=0)
        np.testing.assert_allclose(s, direct, rtol=1e-12, atol=1e-12)


def _rope_rotate_half(x, pos, base=10000.0):
    d = x.shape[-1]
    h = d // 2
    th = base ** (-2.0 * np.arange(h) / d)
    c, s = np.cos(pos * th), np.sin(pos * th)
    return np.concatenate([x[:h] * c - x[h:] * s, x[h:] * c + x[:h] * s])


def test_tip_chunk_is_a_rope_rotation_plane():
    """FASA §2.A: each frequency chunk is one of RoPE's 2-D rotation planes, so
    a single chunk's score depends only on the relative position.  This pins
    the chunk -> channel pairing (f, f + d/2) of rotate-half RoPE."""
    r = _rng(6)
    d = 64
    qv, kv = r.standard_normal(d), r.standard_normal(d)
    for f in [0, 5, 17, 31]:
        vals = []
        for m, n in [(100, 40), (160, 100), (1000, 940)]:
            q = _rope_rotate_half(qv, m)[None]
            k = _rope_rotate_half(kv, n)[None]
            vals.append(fasa.tip_scores(q, k, [f])[0])
        np.testing.assert_allclose(vals, vals[0], rtol=1e-9, atol=1e-9)
    # a chunk of an interleaved pairing would not be shift invariant
    q0 = _rope_rotate_half(qv, 100)
    k0 = _rope_rotate_half(kv, 40)
    q1 = _rope_rotate_half(qv, 160)
    k1 = _rope_rotate_half(kv, 100)
    wrong0 = q0[10] * k0[10] + q0[11] * k0[11]
    wrong1 = q1[10] * k1[10] + q1[11] * k1[11]
    assert abs(wrong0 - wrong1) > 1e-3


# ------------------------------------------------------------------ top-N
def test_top_n_golden_ties():
    with open(os.path.join(GOLDEN, "topk_ties.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert fasa.top_n(np.array(c["scores"], dtype=float), c["n"]).tolist() == c["idx"], c


def test_top_n_brute_force():
    """Among all size-n subsets with the largest score sum, the selection is
    the one with the lexicographically smallest sorted index tuple."""
    r = _rng(8)
    for trial in range(60):
        T = int(r.integers(1, 9))
        n = int(r.integers(1, T + 1))
        s = r.integers(-3, 4, size=T).astype(float)
        best = None
        for sub in itertools.combinations(range(T), n):
            key = (-s[list(sub)].sum(), sub)
            if best is None or key < best:
                best = key
        assert fasa.top_n(s, n).tolist() == list(best[1]), (s, n)


# ------------------------------------------------------------------ attention
def _sdpa(q, k, v):
    qt = torch.tensor(q, dtype=torch.float64)[None, None, None]
    kt = torch.tensor(k, dtype=torch.float64)[None, None]
    vt = torch.tensor(v, dtype=torch.float64)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()


def test_attend_matches_sdpa_and_closed_forms():
    r = _rng(9)
    q, k, v = r.standard_normal(32), r.standard_normal((20, 32)), r.standard_normal((20, 32))
    np.testing.assert_allclose(fasa.attend(q, k, v), _sdpa(q, k, v), rtol=1e-12, atol=1e-12)
    # equal keys -> uniform weights -> mean of the values
    k_eq = np.repeat(k[:1], 20, axis=0)
    np.testing.assert_allclose(fasa.attend(q, k_eq, v), v.mean(axis=0), rtol=1e-12, atol=1e-12)
    # two tokens: p_0 = sigmoid((z0 - z1)), z = q.k / sqrt(d)
    z = k[:2] @ q / math.sqrt(32)
    p0 = 1.0 / (1.0 + math.exp(-(z[0] - z[1])))
    np.testing.assert_allclose(fasa.attend(q, k[:2], v[:2]), p0 * v[0] + (1 - p0) * v[1], rtol=1e-12)


def test_fac_with_every_token_selected_is_dense_attention():
    """FASA §2.B.2 keeps original positions: N_fac = T is dense attention."""
    r = _rng(10)
    T, d, G = 40, 16, 2
    q = r.standard_normal((G, d))
    k, v = r.standard_normal((T, d)), r.standard_normal((T, d))
    out, idx = fasa.decode_group(q, k, v, [1, 3], True, T, 0, 0)
    assert idx.tolist() == list(range(T))
    for h in range(G):
        np.testing.assert_allclose(out[h], _sdpa(q[h], k, v), rtol=1e-12, atol=1e-12)


def test_stream_window_covering_context_is_dense_attention():
    r = _rng(11)
    T, d = 30, 8
    q = r.standard_normal((1, d))
    k, v = r.standard_normal((T, d)), r.standard_normal((T, d))
    for n_sink, window in [(4, 30), (0, 64), (30, 0), (12, 25)]:
        out, _ = fasa.decode_group(q, k, v, [0], False, 1, n_sink, window)
        np.testing.assert_allclose(out[0], _sdpa(q[0], k, v), rtol=1e-12, atol=1e-12)


def test_stream_rows_union_without_repeats():
    for T, S, W in [(10, 4, 3), (10, 4, 8), (3, 4, 3), (100, 0, 7), (100, 5, 0), (1, 1, 1)]:
        rows = fasa.stream_rows(T, S, W)
        want = sorted(set(range(min(S, T))) | set(range(max(T - W, 0), T)))
        assert rows.tolist() == want


def test_sparse_attention_over_a_subset():
    """FAC = dense attention restricted to the selected rows: with the other
    rows' keys pushed to -inf logits the dense result is the same."""
    r = _rng(12)
    T, d = 64, 16
    q = r.standard_normal((1, d))
    k, v = r.standard_normal((T, d)), r.standard_normal((T, d))
    out, idx = fasa.decode_group(q, k, v, [2, 5, 7], True, 10, 0, 0)
    mask = np.full(T, -np.inf)
    mask[idx] = 0.0
    z = k @ q[0] / math.sqrt(d) + mask
    p = np.exp(z - z.max())
    p /= p.sum()
    np.testing.assert_allclose(out[0], p @ v, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ CLSA
def test_shared_index_single_layer_is_sparse_decode():
    """CLSA "Cómo funciona CLSA": the index is the one the indexer computes;
    with one layer it is ordinary sparse decode."""
    r = _rng(13)
    B, Hkv, G, T, d, n = 2, 2, 2, 48, 16, 9
    q = r.standard_normal((1, B, Hkv * G, d))
    k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    idom = np.array([[0, 3], [1, 6]])
    out, idx = clsa.shared_index_decode(q, k, v, idom, n)
    out2, idx2 = fasa.sparse_decode(q, k[None], v[None], idom[None], np.ones((1, Hkv)), n, 0, 0)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-12)
    assert (idx == idx2[0]).all()


def test_shared_index_reuses_the_indexer_selection():
    r = _rng(14)
    N, B, Hkv, G, T, d, n = 3, 1, 2, 2, 40, 8, 6
    q = r.standard_normal((N, B, Hkv * G, d))
    k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    idom = np.array([[0, 1], [2, 3]])
    out, idx = clsa.shared_index_decode(q, k, v, idom, n)
    for layer in range(N):
        for g in range(Hkv):
            sel = fasa.top_n(fasa.tip_scores(q[0, 0, g * G:(g + 1) * G], k[0, g], idom[g]), n)
            assert idx[0, g].tolist() == sel.tolist()
            for h in range(g * G, (g + 1) * G):
                np.testing.assert_allclose(out[layer, 0, h], _sdpa(q[layer, 0, h], k[0, g, sel], v[0, g, sel]),
                                           rtol=1e-12, atol=1e-12)
    # a layer labelled streaming attends to sink + window instead
    labels = np.array([[1, 1], [0, 1], [1, 1]])
    out_l, _ = clsa.shared_index_decode(q, k, v, idom, n, labels=labels, n_sink=2, window=5)
    rows = fasa.stream_rows(T, 2, 5)
    np.testing.assert_allclose(out_l[1, 0, 0], _sdpa(q[1, 0, 0], k[0, 0, rows], v[0, 0, rows]), rtol=1e-12)
    np.testing.assert_allclose(out_l[0], out[0], rtol=1e-12)


def test_tip_interleaved_chunk_is_a_rope_rotation_plane():
    """Same pin for the interleaved RoPE layout: chunk f = channels (2f, 2f+1)."""
    r = _rng(15)
    d = 64

    def rope_interleaved(x, pos, base=10000.0):
        th = base ** (-2.0 * np.arange(d // 2) / d)
        c, s = np.cos(pos * th), np.sin(pos * th)
        y = x.copy()
        y[0::2] = x[0::2] * c - x[1::2] * s
        y[1::2] = x[1::2] * c + x[0::2] * s
        return y

    qv, kv = r.standard_normal(d), r.standard_normal(d)
    for f in [0, 9, 31]:
        vals = [fasa.tip_scores(rope_interleaved(qv, m)[None], rope_interleaved(kv, n)[None], [f],
                                pairing="interleaved")[0] for m, n in [(50, 10), (90, 50), (700, 660)]]
        np.testing.assert_allclose(vals, vals[0], rtol=1e-9, atol=1e-9)
    # all chunks in either pairing give the exact logit
    q = r.standard_normal((2, d))
    k = r.standard_normal((5, d))
    np.testing.assert_allclose(fasa.tip_scores(q, k, np.arange(d // 2), pairing="interleaved"),
                               k @ q.mean(axis=0), rtol=1e-12)
