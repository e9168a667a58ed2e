"""GPU parity of the split cache: streaming groups keep only their sink and
a ring of the recent window, retrieval groups full rows.  kv_append fills it
(from a prefill, or one token at a time) and sparse_decode_step_split must
give exactly the results of sparse_decode_step on the full cache; the ring
slots must hold the rows of the oracle's sink + window positions."""
import numpy as np
import pytest
import torch

import head_aware_sparse_amd as H
from oracle import fasa
from synth import recipe as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _slot(pos, n_sink, window):
    return pos if pos < n_sink else n_sink + (pos - n_sink) % window


def _empty_split(case, capacity):
    cfg = case.cfg
    lab = case.labels_np.astype(bool).reshape(-1)
    n_ret, n_str = int(lab.sum()), int((~lab).sum())
    dt, B, d = case.k.dtype, cfg.batch, cfg.d_head
    S = cfg.n_sink + cfg.window
    z = lambda *s: torch.zeros(s, dtype=dt, device="cuda")
    return dict(k_ret=z(n_ret, B, capacity, d), v_ret=z(n_ret, B, capacity, d),
                k_dom_ret=z(n_ret, B, capacity, H.kdom_row_elems(case.dims)),
                k_str=z(n_str, B, S, d), v_str=z(n_str, B, S, d))


def _append(case, sc, pos, k_new, v_new):
    H.kv_append(case.dims, pos, k_new, v_new, case.i_dom, case.labels, sc["k_ret"], sc["v_ret"], sc["k_dom_ret"],
                sc["k_str"], sc["v_str"])


def _decode_split(case, sc, dims):
    cfg = case.cfg
    out = torch.full((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), float("nan"), device="cuda")
    ix = torch.full((cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.n_fac), -7, dtype=torch.int32, device="cuda")
    H.sparse_decode_step_split(dims, case.q, sc["k_ret"], sc["v_ret"], sc["k_dom_ret"], sc["k_str"], sc["v_str"],
                               case.i_dom, case.labels, out, ix)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ix.cpu().numpy()


def _decode_full(case, dims, T):
    cfg = case.cfg
    k = case.k[:, :, :, :T].contiguous()
    v = case.v[:, :, :, :T].contiguous()
    kd = case.k_dom[:, :, :, :T].contiguous()
    out = torch.full((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), float("nan"), device="cuda")
    ix = torch.full((cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.n_fac), -7, dtype=torch.int32, device="cuda")
    H.sparse_decode_step(dims, case.q, k, v, kd, case.i_dom, case.labels, out, ix)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ix.cpu().numpy()


def _pairs(case):
    lab = case.labels_np.astype(bool).reshape(-1)
    ret = {p: i for i, p in enumerate(np.flatnonzero(lab))}
    strm = {p: i for i, p in enumerate(np.flatnonzero(~lab))}
    return ret, strm


def _check_contents(case, sc, T):
    """Ring slots hold the rows of the oracle's sink + window positions and
    retrieval slabs hold the rows and k_dom of every position, bit for bit."""
    cfg = case.cfg
    ret, strm = _pairs(case)
    rows = fasa.stream_rows(T, cfg.n_sink, cfg.window)
    slots = np.array([_slot(int(p), cfg.n_sink, max(cfg.window, 1)) for p in rows], dtype=np.int64)
    bits = lambda t: t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()
    for b in range(cfg.batch):
        for p, s in list(strm.items())[:3]:
            l, g = divmod(p, cfg.n_kv_heads)
            for name, full in (("k_str", case.k), ("v_str", case.v)):
                got = bits(sc[name][s, b][torch.from_numpy(slots).cuda()])
                want = bits(full[l, b, g][torch.from_numpy(rows).cuda()])
                assert (got == want).all(), f"{name} pair {p} b{b}"
        for p, r in list(ret.items())[:3]:
            l, g = divmod(p, cfg.n_kv_heads)
            assert (bits(sc["k_ret"][r, b, :T]) == bits(case.k[l, b, g, :T])).all()
            assert (bits(sc["k_dom_ret"][r, b, :T]) == bits(case.k_dom[l, b, g, :T])).all()


def _labels(cfg, seed, kind="mixed"):
    rng = np.random.default_rng(seed)
    if kind == "retrieval":
        return np.ones((cfg.n_layers, cfg.n_kv_heads), np.uint8)
    if kind == "streaming":
        return np.zeros((cfg.n_layers, cfg.n_kv_heads), np.uint8)
    lab = (rng.random((cfg.n_layers, cfg.n_kv_heads)) < 0.3).astype(np.uint8)
    lab[0, 0], lab[-1, -1] = 1, 0
    return lab


@pytest.mark.parametrize("over,kind", [
    (dict(), "mixed"),                                   # the ring wrapped many times
    (dict(n_sink=16, window=0), "mixed"),                # sink only
    (dict(n_sink=0, window=512), "mixed"),               # window only
    (dict(window=4096, ctx_len=3000, n_fac=500), "mixed"),  # ring never full
    (dict(), "retrieval"),                               # no streaming group
    (dict(), "streaming"),                               # no retrieval group
    (dict(kv_dtype="f32", d_head=64, n_dom=8), "mixed"),
], ids=["wrapped", "sink-only", "window-only", "ring-not-full", "all-retrieval", "all-streaming", "f32-d64"])
def test_prefill_split_cache_equals_full(over, kind):
    cfg = R.get_config("c1", **{**dict(ctx_len=20000, batch=2, n_layers=2), **over})
    print(f"case split prefill {over} {kind}", flush=True)
    case = U.DeviceCase(cfg, labels=_labels(cfg, 3, kind))
    T = cfg.ctx_len
    sc = _empty_split(case, T + 37)          # a capacity above the length
    _append(case, sc, 0, case.k, case.v)
    torch.cuda.synchronize()
    _check_contents(case, sc, T)
    out_s, idx_s = _decode_split(case, sc, case.dims)
    out_f, idx_f = _decode_full(case, case.dims, T)
    assert (idx_s == idx_f).all()
    assert np.array_equal(out_s, out_f)
    # and the oracle on one item of each kind
    ret, strm = _pairs(case)
    G = cfg.group
    for p in list(ret)[:1] + list(strm)[:1]:
        l, g = divmod(p, cfg.n_kv_heads)
        ref, _, _ = U.oracle_item(cfg, case.hi, case.labels_np, l, 1, g)
        U.check_out(out_s[l, 1, g * G:(g + 1) * G], ref, f"split out l{l} g{g}")


def test_token_by_token_append_across_the_ring_wrap():
    """Prefill, then one kv_append per decoded token while the ring wraps;
    after every token the split decode equals the full-cache decode at that
    length, and at the end the oracle agrees."""
    n_sink, window = 4, 1024
    T0 = n_sink + (window - 2) + 9 * window  # the next tokens fill the last two slots, then wrap
    steps = 4
    cfg = R.get_config("c1", ctx_len=T0 + steps, batch=2, n_layers=2)
    print("case split token by token", flush=True)
    case = U.DeviceCase(cfg, labels=_labels(cfg, 4))
    sc = _empty_split(case, T0 + steps + 100)
    _append(case, sc, 0, case.k[:, :, :, :T0].contiguous(), case.v[:, :, :, :T0].contiguous())
    for t in range(steps):
        pos = T0 + t
        _append(case, sc, pos, case.k[:, :, :, pos:pos + 1].contiguous(), case.v[:, :, :, pos:pos + 1].contiguous())
        T = pos + 1
        dims = U.dims_of(cfg, ctx_len=T)
        torch.cuda.synchronize()
        _check_contents(case, sc, T)
        out_s, idx_s = _decode_split(case, sc, dims)
        out_f, idx_f = _decode_full(case, dims, T)
        assert (idx_s == idx_f).all(), f"T={T}"
        assert np.array_equal(out_s, out_f), f"T={T}"
    ret, strm = _pairs(case)
    G = cfg.group
    for p in list(ret)[:1] + list(strm)[:1]:
        l, g = divmod(p, cfg.n_kv_heads)
        ref, _ = U.oracle_item_custom(cfg, case.hi.q[l, 0, g * G:(g + 1) * G], case.hi.rows("k", l, 0, g)[:T],
                                      case.hi.rows("v", l, 0, g)[:T], case.hi.i_dom[l, g],
                                      bool(case.labels_np[l, g]))
        U.check_out(out_s[l, 0, g * G:(g + 1) * G], ref, f"token-by-token l{l} g{g}")


def test_host_resident_rows_fasa_m():
    """The retrieval groups' full K and V rows in pinned host memory, only the
    dominant-key copy (and the streaming rings) in HBM: appends and decode
    read and write them over the host link and give exactly the results of
    the all-device split cache, and the oracle's on one retrieval and one
    streaming item per sequence.  Pageable host memory is refused before any
    launch."""
    cfg = R.get_config("c1", ctx_len=12000, batch=2, n_layers=2)
    print("case FASA-M host rows", flush=True)
    case = U.DeviceCase(cfg, labels=_labels(cfg, 5))
    T0 = cfg.ctx_len - 2
    dev = _empty_split(case, cfg.ctx_len + 8)
    host = dict(dev)
    host["k_ret"] = torch.zeros(dev["k_ret"].shape, dtype=dev["k_ret"].dtype, pin_memory=True)
    host["v_ret"] = torch.zeros(dev["v_ret"].shape, dtype=dev["v_ret"].dtype, pin_memory=True)
    host["k_dom_ret"] = torch.zeros_like(dev["k_dom_ret"])
    host["k_str"] = torch.zeros_like(dev["k_str"])
    host["v_str"] = torch.zeros_like(dev["v_str"])
    for sc in (dev, host):
        _append(case, sc, 0, case.k[:, :, :, :T0].contiguous(), case.v[:, :, :, :T0].contiguous())
        for pos in (T0, T0 + 1):
            _append(case, sc, pos, case.k[:, :, :, pos:pos + 1].contiguous(), case.v[:, :, :, pos:pos + 1].contiguous())
    torch.cuda.synchronize()
    assert (host["k_ret"].view(torch.int16) == dev["k_ret"].cpu().view(torch.int16)).all()
    out_d, idx_d = _decode_split(case, dev, case.dims)
    out_h, idx_h = _decode_split(case, host, case.dims)
    assert (idx_h == idx_d).all()
    assert np.array_equal(out_h, out_d)
    # the host-row path against the oracle: one retrieval and one streaming
    # item over all ctx_len rows, the two tokens appended one by one included
    ret, strm = _pairs(case)
    G = cfg.group
    for b in range(cfg.batch):
        for p in list(ret)[:1] + list(strm)[:1]:
            l, g = divmod(p, cfg.n_kv_heads)
            ref, ridx, scores = U.oracle_item(cfg, case.hi, case.labels_np, l, b, g)
            U.check_out(out_h[l, b, g * G:(g + 1) * G], ref, f"FASA-M out l{l} b{b} g{g}")
            if ridx is None:
                assert (idx_h[l, b, g] == -1).all()
            else:
                U.check_index_set(idx_h[l, b, g], scores, cfg.n_fac, f"FASA-M idx l{l} b{b} g{g}")
    pageable = dict(host)
    pageable["v_ret"] = torch.zeros(dev["v_ret"].shape, dtype=dev["v_ret"].dtype)  # not pinned
    with pytest.raises((ValueError, H.HasError)):
        _decode_split(case, pageable, case.dims)
    # the library's own check, past the binding: a pageable host pointer is
    # refused before anything is launched
    import ctypes
    from head_aware_sparse_amd.binding import lib
    P = ctypes.c_void_p
    out = torch.full((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), 7.0, device="cuda")
    ws = torch.empty(H.sparse_decode_workspace(case.dims), dtype=torch.uint8, device="cuda")
    r = lib().sparse_decode_step_split(ctypes.byref(case.dims), dev["k_ret"].shape[2], P(case.q.data_ptr()),
                                       P(host["k_ret"].data_ptr()), P(pageable["v_ret"].data_ptr()),
                                       P(dev["k_dom_ret"].data_ptr()), P(dev["k_str"].data_ptr()),
                                       P(dev["v_str"].data_ptr()), P(case.i_dom.data_ptr()),
                                       P(case.labels.data_ptr()), P(out.data_ptr()), None, P(ws.data_ptr()),
                                       ws.numel(), None)
    assert r == 1 and "v_ret" in H.last_error()
    torch.cuda.synchronize()
    assert (out == 7.0).all()
