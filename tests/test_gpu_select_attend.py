"""GPU parity of the layer-by-layer shared index: sparse_select builds the
index once, fac_attend attends one layer over a given index.  Checked against
the oracle (TIP + exact top-n_fac; softmax attention over the given rows) and
against the fused shared_index_decode, which runs the same selection."""
import numpy as np
import pytest
import torch

import head_aware_sparse_amd as H
from oracle import fasa
from synth import device as sdev
from synth import recipe as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _one_layer(cfg):
    return U.dims_of(cfg, n_layers=1)


def _select(case, q_index=None):
    cfg = case.cfg
    idx = torch.full((cfg.batch, cfg.n_kv_heads, cfg.n_fac), -7, dtype=torch.int32, device="cuda")
    qi = case.q[0] if q_index is None else q_index
    H.sparse_select(_one_layer(cfg), qi, case.k_dom[0], case.i_dom[0], idx)
    torch.cuda.synchronize()
    return idx


def _attend(case, n, idx, ws=None):
    cfg = case.cfg
    out = torch.full((cfg.batch, cfg.n_q_heads, cfg.d_head), float("nan"), device="cuda")
    ws = H.fac_attend(_one_layer(cfg), case.q[n], case.k[0], case.v[0], idx, out, ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


def _oracle_attend(cfg, hi, n, b, g, rows):
    G = cfg.group
    k = U.f64(hi.rows("k", 0, b, g), cfg)[rows]
    v = U.f64(hi.rows("v", 0, b, g), cfg)[rows]
    return np.stack([fasa.attend(U.f64(hi.q[n, b, g * G + j], cfg), k, v) for j in range(G)])


@pytest.mark.parametrize("over", [
    dict(),                                  # bf16, d 128 (fused call on the matrix cores)
    dict(kv_dtype="f32"),                    # fp32 cache
    dict(d_head=64, n_dom=8, n_fac=700),     # d 64, ragged last row block
], ids=["bf16-d128", "f32", "d64-ragged"])
def test_select_then_attend_per_layer(over):
    """One sparse_select plus one fac_attend per layer reproduces the fused
    shared-index call: the same index (bit-exact), outputs equal up to fp32
    summation order, and both agree with the oracle on sampled groups."""
    cfg = R.get_config("c3", ctx_len=20000, batch=2, n_layers=4, **over)
    print(f"case select+attend {over}", flush=True)
    case = U.DeviceCase(cfg)
    fused, fidx, _ = U.run_clsa(case)
    idx = _select(case)
    assert (idx.cpu().numpy() == fidx).all()
    G = cfg.group
    ws = None
    for n in range(cfg.n_layers):
        out, ws = _attend(case, n, idx, ws)
        np.testing.assert_allclose(out, fused[n], rtol=1e-4, atol=1e-5)
        for (b, g) in [(0, 1), (1, 6)]:
            ref = _oracle_attend(cfg, case.hi, n, b, g, fidx[b, g])
            U.check_out(out[b, g * G:(g + 1) * G], ref, f"attend n{n} b{b} g{g}")
    for (b, g) in [(0, 1), (1, 6)]:
        _, ridx, scores = U.oracle_clsa_item(cfg, case.hi, b, g)
        U.check_index_set(fidx[b, g], scores, cfg.n_fac, f"select b{b} g{g}")


def test_select_128k_explicit_indexer_query():
    """The 131072-token, batch-4 shared cache with an indexer query of its own
    (not layer 0): sampled groups against the oracle; the planted needles
    aligned to layer 0 are not required here."""
    cfg = R.get_config("c3")
    print("case select c3 full", flush=True)
    case = U.DeviceCase(cfg)
    qi_np = case.hi.q[5]
    idx = _select(case, q_index=sdev.to_device(qi_np, "cuda", cfg.bf16)).cpu().numpy()
    for (b, g) in [(0, 0), (2, 4), (3, 7)]:
        _, _, scores = U.oracle_clsa_item(cfg, case.hi, b, g, q_index=qi_np)
        U.check_index_set(idx[b, g], scores, cfg.n_fac, f"c3 select b{b} g{g}")


@pytest.mark.parametrize("over", [dict(), dict(kv_dtype="f32")], ids=["bf16", "f32"])
def test_attend_arbitrary_index(over):
    """A caller's index need not be sorted or distinct: repeated rows count
    once per entry, the first and last positions are reachable, and entries
    outside [0, ctx_len) are clamped into range."""
    cfg = R.get_config("c3", ctx_len=5000, batch=2, n_layers=1, n_fac=300, **over)
    print(f"case attend arbitrary {over}", flush=True)
    case = U.DeviceCase(cfg)
    rng = np.random.default_rng(5)
    idx = rng.integers(0, cfg.ctx_len, size=(cfg.batch, cfg.n_kv_heads, cfg.n_fac)).astype(np.int32)
    idx[:, :, 0] = 0
    idx[:, :, 1] = cfg.ctx_len - 1
    idx[:, :, 2:40] = idx[:, :, 40:41]          # one row 39 times over
    idx[0, 3, 50] = -5                          # clamped to 0
    idx[1, 2, 60] = cfg.ctx_len + 3             # clamped to ctx_len - 1
    out, _ = _attend(case, 0, torch.from_numpy(idx).cuda())
    G = cfg.group
    for (b, g) in [(0, 3), (1, 2), (1, 7)]:
        rows = np.clip(idx[b, g].astype(np.int64), 0, cfg.ctx_len - 1)
        ref = _oracle_attend(cfg, case.hi, 0, b, g, rows)
        U.check_out(out[b, g * G:(g + 1) * G], ref, f"attend arbitrary b{b} g{g}")


def test_attend_debug_rejects_out_of_range(monkeypatch):
    """With HAS_DEBUG=1 an index entry outside [0, ctx_len) is an argument
    error, found on the host before any launch; the output is untouched."""
    cfg = R.get_config("c3", ctx_len=4096, batch=1, n_layers=1, n_fac=64)
    print("case attend HAS_DEBUG", flush=True)
    case = U.DeviceCase(cfg)
    idx = torch.zeros((cfg.batch, cfg.n_kv_heads, cfg.n_fac), dtype=torch.int32, device="cuda")
    idx[0, 5, 9] = cfg.ctx_len
    out = torch.full((cfg.batch, cfg.n_q_heads, cfg.d_head), 7.0, device="cuda")
    monkeypatch.setenv("HAS_DEBUG", "1")
    with pytest.raises(H.HasError) as ei:
        H.fac_attend(_one_layer(cfg), case.q[0], case.k[0], case.v[0], idx, out)
    assert ei.value.status == 1 and "idx" in str(ei.value)
    torch.cuda.synchronize()
    assert (out == 7.0).all()
