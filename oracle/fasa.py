"""Token-sparse decode attention, fp64 (test infrastructure only).

Sources:
  * "FASA: Frequency-aware Sparse Attention", §2.A (RoPE splits a d-vector
    into d/2 two-dimensional frequency chunks), §2.B.1 (TIP: per token, add
    the query-key contributions of the dominant chunks I_dom only; keep the
    N_fac highest), §2.B.2 (FAC: full-dimension attention over the selected
    tokens at their original positions), §2.C (FASA-C: the whole cache stays
    on the device, only a sparse subset is read).
  * "Resumen Técnico: Autonomía de Cabezales (AoH)", §4: streaming heads keep
    a fixed sink (the first tokens) plus a recent window.

Readings where the pages leave a step open:
  * Rotate-half pairing: chunk f holds channels f and f + d/2.
  * The query heads of a KV group share one selection: TIP uses the mean of
    their queries (equal to the mean of their per-head TIP scores).
  * TIP is unscaled; top-N_fac ties go to the lower token index; the index
    list is reported ascending.  No token is forced into the retrieval set.
  * Softmax scale 1/sqrt(d_head).  The query sits at position T-1 and the
    cache holds T tokens, the current one included.
  * Sink and window overlap (T < n_sink + window) is a union: no token twice.
"""
import numpy as np


def fc_channels(i_dom, d_head, pairing="rotate_half"):
    """Channel indices of the chunks in i_dom: (f..., f + d/2 ...) for the
    rotate-half RoPE layout, (2f..., 2f + 1 ...) for the interleaved one."""
    f = np.asarray(i_dom, dtype=np.int64)
    if pairing == "interleaved":
        return np.concatenate([2 * f, 2 * f + 1])
    return np.concatenate([f, f + d_head // 2])


def group_query(q_group):
    """Mean of the group's query heads, [G, d] -> [d]."""
    return np.asarray(q_group, dtype=np.float64).mean(axis=0)


def tip_scores(q_group, keys, i_dom, pairing="rotate_half"):
    """Per-token importance: sum over chunks f in I_dom of the 2-D chunk dot
    product between the group query and the key.  keys [T, d] -> [T]."""
    keys = np.asarray(keys, dtype=np.float64)
    ch = fc_channels(i_dom, keys.shape[1], pairing)
    return keys[:, ch] @ group_query(q_group)[ch]


def top_n(scores, n):
    """Indices of the n highest scores, ties to lower index, ascending."""
    scores = np.asarray(scores, dtype=np.float64)
    order = np.lexsort((np.arange(scores.size), -scores))
    return np.sort(order[:n])


def stream_rows(T, n_sink, window):
    """Sink [0, n_sink) united with the recent window [T - window, T)."""
    s_end = min(n_sink, T)
    w_start = max(T - window, s_end)
    return np.concatenate([np.arange(0, s_end), np.arange(w_start, T)]).astype(np.int64)


def attend(q, keys, values):
    """softmax(keys q / sqrt(d)) values for one query vector."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    z = keys @ q / np.sqrt(q.size)
    p = np.exp(z - z.max())
    p /= p.sum()
    return p @ values


def decode_group(q_group, keys, values, i_dom, retrieval, n_fac, n_sink, window, pairing="rotate_half"):
    """One (layer, sequence, KV group): (out [G, d], idx [n_fac] or None)."""
    T = keys.shape[0]
    if retrieval:
        idx = top_n(tip_scores(q_group, keys, i_dom, pairing), n_fac)
    else:
        idx = None
    rows = idx if retrieval else stream_rows(T, n_sink, window)
    ksel = np.asarray(keys, dtype=np.float64)[rows]
    vsel = np.asarray(values, dtype=np.float64)[rows]
    out = np.stack([attend(qh, ksel, vsel) for qh in np.asarray(q_group, dtype=np.float64)])
    return out, idx


def sparse_decode(q, keys, values, i_dom, labels, n_fac, n_sink, window):
    """Whole step.  q [L,B,Hq,d]; keys/values [L,B,Hkv,T,d]; i_dom [L,Hkv,n_dom];
    labels [L,Hkv] (1 = retrieval).  Returns out [L,B,Hq,d] and idx
    [L,B,Hkv,n_fac] (-1 rows for streaming groups)."""
    L, B, Hq, d = q.shape
    Hkv = keys.shape[2]
    G = Hq // Hkv
    out = np.zeros((L, B, Hq, d))
    idx = np.full((L, B, Hkv, n_fac), -1, dtype=np.int64)
    for l in range(L):
        for b in range(B):
            for g in range(Hkv):
                o, ix = decode_group(q[l, b, g * G:(g + 1) * G], keys[l, b, g], values[l, b, g],
                                     i_dom[l, g], bool(labels[l, g]), n_fac, n_sink, window)
                out[l, b, g * G:(g + 1) * G] = o
                if ix is not None:
                    idx[l, b, g] = ix
    return out, idx
