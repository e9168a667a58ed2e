"""Shared-index decode across layers that share one KV cache, fp64
(test infrastructure only).

Source: "El enrutamiento compartido entre capas acelera la atención dispersa
7 veces ..." (on "CLSA: You Only Index Once"), section "Cómo funciona CLSA":
in a shared-KV cross-decoder stack, one indexer scores the cache once, takes
the top-k tokens and hands that same index to every following layer; token
granularity is kept.

Readings: the indexer scores with the FASA token-importance predictor over
I_dom (with I_dom = every chunk this is the exact attention logit), using
the indexer query (by default the first layer's query).  Layers whose group
is labelled streaming attend to sink + window of the shared cache instead.
"""
import numpy as np

from . import fasa


def shared_index_decode(q, keys, values, i_dom, n_fac, q_index=None, labels=None,
                        n_sink=0, window=0):
    """q [N,B,Hq,d]; keys/values [B,Hkv,T,d]; i_dom [Hkv,n_dom];
    labels [N,Hkv] or None (all retrieval).  Returns out [N,B,Hq,d] and the
    shared index [B,Hkv,n_fac]."""
    N, B, Hq, d = q.shape
    Hkv, T = keys.shape[1], keys.shape[2]
    G = Hq // Hkv
    qi = q[0] if q_index is None else q_index
    out = np.zeros((N, B, Hq, d))
    idx = np.empty((B, Hkv, n_fac), dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            k = np.asarray(keys[b, g], dtype=np.float64)
            v = np.asarray(values[b, g], dtype=np.float64)
            sel = fasa.top_n(fasa.tip_scores(qi[b, g * G:(g + 1) * G], k, i_dom[g]), n_fac)
            idx[b, g] = sel
            for n in range(N):
                retrieval = True if labels is None else bool(labels[n, g])
                rows = sel if retrieval else fasa.stream_rows(T, n_sink, window)
                for h in range(g * G, (g + 1) * G):
                    out[n, b, h] = fasa.attend(q[n, b, h], k[rows], v[rows])
    return out, idx
