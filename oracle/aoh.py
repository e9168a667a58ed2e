"""AoH head labeller, fp64 (test infrastructure only).

Source: "Resumen Técnico: Autonomía de Cabezales (Autonomy-of-Heads, AoH)",
Metodología §1-§4 (and the French twin of the same summary).

  §1  M_h = W_K^{h T} W_Q^h, the frozen query-key matching operator.
  §2  eff_rank(h) = exp(-sum_k s_k log s_k) over the normalised singular
      values of M_h; low ER = retrieval head, high ER = streaming head.
  §3  The nonzero singular values of M_h come from the d_head x d_head proxy
      C_h = (W_Q W_Q^T)(W_K W_K^T).
  §4  Heads are ranked by ER, the k lowest are retrieval heads; under GQA
      the scores are aggregated per group by their mean.

Readings where the pages leave a step open:
  * Singular values are normalised by their sum (sigma / sum sigma).
  * sigma_k = sqrt(max(lambda_k, 0)) over all d_head eigenvalues of C_h;
    zero terms contribute nothing (0 log 0 = 0); a zero spectrum has the
    empty sum, ER = exp(0) = 1.
  * GQA: every query head is scored with its group's W_K; the group score is
    the mean of its query heads' ER; labels are per KV group.
  * k counts (layer, group) pairs over the whole model; ties in ER go to the
    lower flat index l*H_kv + g.
"""
import numpy as np


def gram(w):
    """W W^T for a head's projection rows (d_head x d_model)."""
    w = np.asarray(w, dtype=np.float64)
    return w @ w.T


def proxy_eigenvalues(wq_h, wk_g):
    """Eigenvalues of C_h = (W_Q W_Q^T)(W_K W_K^T) (§3), ascending.

    C_h = G_Q G_K with G_K positive semidefinite is similar to the symmetric
    matrix R G_Q R with R = G_K^{1/2}, so its eigenvalues are real and are
    computed from that symmetric form."""
    gq = gram(wq_h)
    gk = gram(wk_g)
    w, v = np.linalg.eigh(gk)
    r = (v * np.sqrt(np.clip(w, 0.0, None))) @ v.T
    s = r @ gq @ r
    return np.linalg.eigvalsh(0.5 * (s + s.T))


def effective_rank_from_singular(sigma):
    """exp of the Shannon entropy of sigma / sum(sigma) (§2)."""
    sigma = np.asarray(sigma, dtype=np.float64)
    tot = sigma.sum()
    if tot <= 0.0:
        return 1.0
    p = sigma / tot
    p = p[p > 0.0]
    return float(np.exp(-np.sum(p * np.log(p))))


def effective_rank(eigenvalues):
    """ER of M_h from the eigenvalues of C_h (= squared singular values)."""
    lam = np.clip(np.asarray(eigenvalues, dtype=np.float64), 0.0, None)
    return effective_rank_from_singular(np.sqrt(lam))


def head_effective_ranks(w_q, w_k, n_q_heads, n_kv_heads, d_head):
    """er_head [L, Hq] for weights w_q [L, Hq*d, d_model], w_k [L, Hkv*d, d_model]."""
    L = w_q.shape[0]
    G = n_q_heads // n_kv_heads
    er = np.empty((L, n_q_heads))
    for l in range(L):
        for h in range(n_q_heads):
            g = h // G
            lam = proxy_eigenvalues(w_q[l, h * d_head:(h + 1) * d_head],
                                    w_k[l, g * d_head:(g + 1) * d_head])
            er[l, h] = effective_rank(lam)
    return er


def group_scores(er_head, n_kv_heads):
    """Mean of the query heads' ER within each KV group (§4, GQA)."""
    L, Hq = er_head.shape
    return er_head.reshape(L, n_kv_heads, Hq // n_kv_heads).mean(axis=2)


def labels_top_k(er_group, k):
    """1 for the k lowest-ER (layer, group) pairs, ties to the lower flat index."""
    flat = er_group.reshape(-1)
    order = np.lexsort((np.arange(flat.size), flat))
    lab = np.zeros(flat.size, dtype=np.uint8)
    lab[order[:k]] = 1
    return lab.reshape(er_group.shape)


def labels_threshold(er_group, threshold):
    """1 where the group ER lies below `threshold`."""
    return (er_group < threshold).astype(np.uint8)


def aoh_label(w_q, w_k, n_q_heads, n_kv_heads, d_head, k=None, threshold=None):
    """(er_head [L,Hq], er_group [L,Hkv], labels [L,Hkv] uint8; 1 = retrieval)."""
    er_head = head_effective_ranks(w_q, w_k, n_q_heads, n_kv_heads, d_head)
    er_group = group_scores(er_head, n_kv_heads)
    if k is not None:
        labels = labels_top_k(er_group, k)
    else:
        labels = labels_threshold(er_group, threshold)
    return er_head, er_group, labels
