"""Persisted labeller outputs (host only): the .npz round trip, and the
rejection of files that are not labeller records or do not match the
expected shape."""
import numpy as np
import pytest

import head_aware_sparse_amd as H


def _rec(L=3, Hq=8, Hkv=4, nd=5, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 2, (L, Hkv)).astype(np.uint8), rng.random((L, Hq)).astype(np.float32) * 50,
            rng.random((L, Hkv)).astype(np.float32) * 50, rng.integers(0, 32, (L, Hkv, nd)).astype(np.int32))


def test_round_trip(tmp_path):
    lab, erh, erg, idom = _rec()
    p = tmp_path / "labels.npz"
    H.save_labels(p, lab, erh, erg, idom)
    rec = H.load_labels(p, n_layers=3, n_q_heads=8, n_kv_heads=4, n_dom=5)
    for k, a in (("labels", lab), ("er_head", erh), ("er_group", erg), ("i_dom", idom)):
        assert rec[k].dtype == a.dtype and np.array_equal(rec[k], a), k


def test_shape_mismatch_rejected(tmp_path):
    p = tmp_path / "labels.npz"
    H.save_labels(p, *_rec())
    with pytest.raises(ValueError, match="n_kv_heads"):
        H.load_labels(p, n_kv_heads=8)
    with pytest.raises(ValueError, match="n_layers"):
        H.load_labels(p, n_layers=32)


def test_bad_records_rejected(tmp_path):
    lab, erh, erg, idom = _rec()
    with pytest.raises(ValueError):
        H.save_labels(tmp_path / "x.npz", lab * 2, erh, erg, idom)   # labels outside {0, 1}
    with pytest.raises(ValueError):
        H.save_labels(tmp_path / "x.npz", lab, erh, erg[:2], idom)  # er_group with too few layers
    other = tmp_path / "other.npz"
    np.savez(other, a=np.zeros(3))
    with pytest.raises(ValueError, match="not a labeller record"):
        H.load_labels(other)
    # a record whose arrays disagree with its recorded shape
    bad = tmp_path / "bad.npz"
    np.savez(bad, labels=lab, er_head=erh, er_group=erg, i_dom=idom, shape=np.array([3, 8, 4, 6]))
    with pytest.raises(ValueError, match="recorded shape"):
        H.load_labels(bad)
    # object arrays are never unpickled
    pk = tmp_path / "pickled.npz"
    np.savez(pk, labels=np.array([{"x": 1}], dtype=object), er_head=erh, er_group=erg, i_dom=idom,
             shape=np.array([3, 8, 4, 5]))
    with pytest.raises(ValueError):
        H.load_labels(pk)
