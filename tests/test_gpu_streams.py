"""Concurrent callers: threads calling the library on their own streams
(default priority) with their own workspaces get exactly the results of
serial calls, also when every call uses the per-device side stream and its
two events."""
import threading

import numpy as np
import pytest
import torch

import head_aware_sparse_amd as H
from synth import recipe as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _decode(case, stream, ws):
    cfg = case.cfg
    with torch.cuda.stream(stream):
        out = torch.empty((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), device="cuda")
        ix = torch.empty((cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.n_fac), dtype=torch.int32, device="cuda")
        H.sparse_decode_step(case.dims, case.q, case.k, case.v, case.k_dom, case.i_dom, case.labels, out, ix,
                             ws=ws, stream=stream)
    return out, ix


def test_two_threads_on_two_streams_share_the_side_stream():
    # 8 layers x batch 16 x 8 groups, 4100 streaming rows each: above the
    # 2^20-row threshold, so every call forks to the side stream
    cfg = R.get_config("c1", ctx_len=16384, batch=16, n_layers=8, window=4096)
    print("case concurrent callers", flush=True)
    rng = np.random.default_rng(9)
    lab = (rng.random((cfg.n_layers, cfg.n_kv_heads)) < 0.25).astype(np.uint8)
    lab[0, 0] = 1
    case = U.DeviceCase(cfg, labels=lab)
    assert (1 - lab).sum() * cfg.batch * (cfg.n_sink + cfg.window) >= 1 << 20
    ref_out, ref_idx, _ = case.run()

    n_calls = 12
    results, errors = {}, []

    def worker(tid):
        try:
            stream = torch.cuda.Stream()
            ws = torch.empty(H.sparse_decode_workspace(case.dims), dtype=torch.uint8, device="cuda")
            outs = [_decode(case, stream, ws) for _ in range(n_calls)]
            stream.synchronize()
            results[tid] = [(o.cpu().numpy(), i.cpu().numpy()) for o, i in outs]
        except Exception as e:  # reported below
            errors.append(repr(e))

    # a third caller appends to a split cache meanwhile (another entry point)
    def appender():
        try:
            stream = torch.cuda.Stream()
            lf = lab.astype(bool).reshape(-1)
            mk = lambda *s: torch.zeros(s, dtype=case.k.dtype, device="cuda")
            sc = [mk(int(lf.sum()), cfg.batch, cfg.ctx_len, cfg.d_head), mk(int(lf.sum()), cfg.batch, cfg.ctx_len, cfg.d_head),
                  mk(int(lf.sum()), cfg.batch, cfg.ctx_len, H.kdom_row_elems(case.dims)),
                  mk(int((~lf).sum()), cfg.batch, cfg.n_sink + cfg.window, cfg.d_head),
                  mk(int((~lf).sum()), cfg.batch, cfg.n_sink + cfg.window, cfg.d_head)]
            with torch.cuda.stream(stream):
                for _ in range(4):
                    H.kv_append(case.dims, 0, case.k, case.v, case.i_dom, case.labels, *sc, stream=stream)
            stream.synchronize()
            assert (sc[0][0, 0, :8].view(torch.int16) == case.k[0, 0, 0, :8].view(torch.int16)).all()
        except Exception as e:
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)] + [threading.Thread(target=appender)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a caller did not finish"
    assert not errors, errors
    for tid in range(2):
        for out, idx in results[tid]:
            assert (idx == ref_idx).all()
            assert np.array_equal(out, ref_out)
