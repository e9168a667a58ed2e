"""Helpers shared by the GPU parity tests: device inputs from the seeded
generator, per-item oracle results, and the comparison rules.

Comparison rules (fixed by the required agreement, see the decode parity
tests): attention outputs pass when |gpu - ref| <= 2e-3 + 1e-2 |ref|
element-wise; an index set passes when it has n_fac distinct ascending
tokens, holds every token whose fp64 score exceeds the n_fac-th score s_k by
more than 1e-5 |s_k|, and none whose score falls below it by more than that.
"""
import numpy as np
import torch

import head_aware_sparse_amd as H
from oracle import clsa as oclsa
from oracle import fasa
from synth import device as sdev
from synth import recipe as R

ATOL, RTOL = 2e-3, 1e-2
TIE_REL = 1e-5


def dims_of(cfg, **over):
    d = H.DecodeDims(cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.d_head, cfg.ctx_len,
                     cfg.n_fac, cfg.n_sink, cfg.window, cfg.n_dom, H.HAS_BF16 if cfg.bf16 else H.HAS_F32, 0)
    for k, v in over.items():
        setattr(d, k, v)
    return d


class DeviceCase:
    """All device tensors of one configuration (full size)."""

    def __init__(self, cfg, hi=None, labels=None, zero_q=False):
        self.cfg = cfg
        self.hi = hi if hi is not None else R.HostInputs(cfg, with_weights=False)
        if zero_q:
            self.hi.q = np.zeros_like(self.hi.q)
        self.dims = dims_of(cfg)
        dev = "cuda"
        self.q = sdev.to_device(self.hi.q, dev, cfg.bf16)
        self.k = sdev.kv_cache(cfg, "k", self.hi, dev)
        self.v = sdev.kv_cache(cfg, "v", self.hi, dev)
        self.i_dom = torch.from_numpy(self.hi.i_dom).to(dev)
        lab = self.hi.labels if labels is None else labels
        self.labels_np = np.ascontiguousarray(lab, dtype=np.uint8)
        self.labels = torch.from_numpy(self.labels_np).to(dev)
        kd_dims = dims_of(cfg, n_layers=cfg.kv_layers)
        self.kd_dims = kd_dims
        R_ = H.kdom_row_elems(kd_dims)
        self.k_dom = torch.empty((cfg.kv_layers, cfg.batch, cfg.n_kv_heads, cfg.ctx_len, R_), dtype=self.k.dtype,
                                 device=dev)
        idom_kd = self.i_dom if not cfg.clsa else self.i_dom
        H.kdom_pack(kd_dims, self.k, idom_kd, self.k_dom)
        torch.cuda.synchronize()

    def run(self, idx=True, ws=None):
        cfg = self.cfg
        out = torch.full((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), float("nan"), device="cuda")
        ix = (torch.full((cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.n_fac), -7, dtype=torch.int32, device="cuda")
              if idx else None)
        ws = H.sparse_decode_step(self.dims, self.q, self.k, self.v, self.k_dom, self.i_dom, self.labels, out, ix,
                                  ws=ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), (ix.cpu().numpy() if idx else None), ws


def f64(a, cfg):
    return R.storage_to_f64(a, cfg.bf16)


def oracle_item(cfg, hi, labels, l, b, g):
    """(out [G, d], idx or None, fp64 scores or None) for one item."""
    G = cfg.group
    k = f64(hi.rows("k", l, b, g), cfg)
    v = f64(hi.rows("v", l, b, g), cfg)
    q = f64(hi.q[l, b, g * G:(g + 1) * G], cfg)
    ret = bool(labels[l, g])
    out, idx = fasa.decode_group(q, k, v, hi.i_dom[l, g], ret, cfg.n_fac, cfg.n_sink, cfg.window)
    scores = fasa.tip_scores(q, k, hi.i_dom[l, g]) if ret else None
    return out, idx, scores


def check_out(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    lim = ATOL + RTOL * np.abs(ref)
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst err "
                           f"{err.max():.3e} at ref {ref.reshape(-1)[np.argmax(err)]:.4f}")


def check_index_set(got, scores, n, what=""):
    got = np.asarray(got, dtype=np.int64)
    assert got.shape == (n,), what
    assert (np.diff(got) > 0).all(), f"{what}: not strictly ascending"
    assert got.min() >= 0 and got.max() < scores.size, what
    sk = -np.sort(-scores)[n - 1]
    band = TIE_REL * abs(sk)
    sel = np.zeros(scores.size, dtype=bool)
    sel[got] = True
    must_in = scores > sk + band
    must_out = scores < sk - band
    assert sel[must_in].all(), f"{what}: {int((~sel[must_in]).sum())} required tokens missing"
    assert not sel[must_out].any(), f"{what}: {int(sel[must_out].sum())} excluded tokens selected"


def run_clsa(case, labels=None, q_index=None, idx=True, ws=None):
    cfg = case.cfg
    out = torch.full((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), float("nan"), device="cuda")
    ix = (torch.full((cfg.batch, cfg.n_kv_heads, cfg.n_fac), -7, dtype=torch.int32, device="cuda") if idx else None)
    lab = None if labels is None else torch.from_numpy(np.ascontiguousarray(labels, dtype=np.uint8)).cuda()
    ws = H.shared_index_decode(case.dims, case.q, case.k[0], case.v[0], case.k_dom[0], case.i_dom[0], out,
                               q_index=q_index, labels=lab, idx_out=ix, ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (ix.cpu().numpy() if idx else None), ws


def oracle_clsa_item(cfg, hi, b, g, labels=None, q_index=None):
    """(out [N, G, d], idx, fp64 scores) of one (sequence, KV group) of the
    shared-index mode; q_index [B, Hq, d] storage or None (layer 0)."""
    G = cfg.group
    k = f64(hi.rows("k", 0, b, g), cfg)
    v = f64(hi.rows("v", 0, b, g), cfg)
    qi = hi.q[0] if q_index is None else q_index
    scores = fasa.tip_scores(f64(qi[b, g * G:(g + 1) * G], cfg), k, hi.i_dom[0, g])
    idx = fasa.top_n(scores, cfg.n_fac)
    rows_s = fasa.stream_rows(cfg.ctx_len, cfg.n_sink, cfg.window)
    out = np.zeros((cfg.n_layers, G, cfg.d_head))
    for n in range(cfg.n_layers):
        rows = idx if (labels is None or labels[n, g]) else rows_s
        for j in range(G):
            out[n, j] = fasa.attend(f64(hi.q[n, b, g * G + j], cfg), k[rows], v[rows])
    return out, idx, scores


def oracle_item_custom(cfg, q_group, k, v, i_dom, retrieval, pairing="rotate_half"):
    """Oracle for one item from explicit storage-dtype arrays."""
    return fasa.decode_group(f64(q_group, cfg), f64(k, cfg), f64(v, cfg), i_dom, retrieval, cfg.n_fac, cfg.n_sink,
                             cfg.window, pairing=pairing)
