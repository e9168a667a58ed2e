"""Persisted labeller outputs: the AoH labels are computed offline once per
model ("Resumen Técnico: Autonomía de Cabezales (AoH)", §4: heads are
labelled before serving), so a serving run loads them instead of labelling
again.  One .npz file (numpy's format, read without unpickling) holds the
labels [L, Hkv] uint8, the per-head and per-group effective ranks
[L, Hq] / [L, Hkv] float32, the dominant chunks I_dom [L, Hkv, n_dom] int32
and the shape they belong to; loading checks every array against that
shape."""
import numpy as np

_KEYS = ("labels", "er_head", "er_group", "i_dom", "shape")


def save_labels(path, labels, er_head, er_group, i_dom):
    """Write the labeller's outputs (numpy arrays or CPU-convertible tensors)."""
    arr = lambda a, dt: np.ascontiguousarray(a.cpu().numpy() if hasattr(a, "cpu") else a, dtype=dt)
    labels, er_head = arr(labels, np.uint8), arr(er_head, np.float32)
    er_group, i_dom = arr(er_group, np.float32), arr(i_dom, np.int32)
    L, Hkv = labels.shape
    Hq = er_head.shape[1]
    if er_head.shape != (L, Hq) or er_group.shape != (L, Hkv) or i_dom.ndim != 3 or i_dom.shape[:2] != (L, Hkv):
        raise ValueError("labels, er_head, er_group and i_dom disagree on (layers, heads)")
    if not np.isin(labels, (0, 1)).all():
        raise ValueError("labels must be 0 (streaming) or 1 (retrieval)")
    shape = np.array([L, Hq, Hkv, i_dom.shape[2]], dtype=np.int64)
    np.savez(path, labels=labels, er_head=er_head, er_group=er_group, i_dom=i_dom, shape=shape)


def load_labels(path, n_layers=None, n_q_heads=None, n_kv_heads=None, n_dom=None):
    """The saved arrays as a dict; raises ValueError if the file is not a
    labeller record or does not match the given shape."""
    with np.load(path, allow_pickle=False) as z:
        if set(z.files) != set(_KEYS):
            raise ValueError(f"{path}: not a labeller record (arrays {sorted(z.files)})")
        rec = {k: z[k] for k in _KEYS}
    L, Hq, Hkv, nd = (int(x) for x in rec["shape"])
    ok = (rec["labels"].shape == (L, Hkv) and rec["labels"].dtype == np.uint8 and
          rec["er_head"].shape == (L, Hq) and rec["er_group"].shape == (L, Hkv) and
          rec["i_dom"].shape == (L, Hkv, nd) and rec["i_dom"].dtype == np.int32 and
          np.isin(rec["labels"], (0, 1)).all())
    if not ok:
        raise ValueError(f"{path}: arrays do not match their recorded shape")
    want = (n_layers, n_q_heads, n_kv_heads, n_dom)
    for name, got, exp in zip(("n_layers", "n_q_heads", "n_kv_heads", "n_dom"), (L, Hq, Hkv, nd), want):
        if exp is not None and got != exp:
            raise ValueError(f"{path}: {name} {got}, expected {exp}")
    return rec
