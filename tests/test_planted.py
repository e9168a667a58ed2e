"""The oracle recovers the generator's planted structure (a sanity pin of
the oracle on the real workload recipe)."""
import numpy as np

from oracle import aoh, fasa
from synth import recipe as R


def _f64(a, cfg):
    return R.storage_to_f64(a, cfg.bf16)


def test_labeller_recovers_planted_groups_c0_c1():
    for name in ["c0", "c1"]:
        cfg = R.get_config(name)
        hi = R.HostInputs(cfg)
        er_head, er_group, lab = aoh.aoh_label(_f64(hi.w_q, cfg), _f64(hi.w_k, cfg), cfg.n_q_heads,
                                               cfg.n_kv_heads, cfg.d_head, k=cfg.n_retrieval)
        assert (lab == hi.labels).all(), name
        planted = er_group[hi.labels == 1]
        other = er_group[hi.labels == 0]
        assert planted.max() * 2 < other.min()


def test_needles_are_selected_c0_and_c1():
    for name, T in [("c0", None), ("c1", 8192)]:
        cfg = R.get_config(name) if T is None else R.get_config(name, ctx_len=T)
        hi = R.HostInputs(cfg, with_weights=False)
        G = cfg.group
        for (l, g) in R.planted_groups(cfg):
            k = _f64(hi.rows("k", l, 0, g), cfg)
            q = _f64(hi.q[l, 0, g * G:(g + 1) * G], cfg)
            idx = fasa.top_n(fasa.tip_scores(q, k, hi.i_dom[l, g]), cfg.n_fac)
            pos = R.needle_positions(cfg, l, 0, g)
            assert np.isin(pos, idx).all()
