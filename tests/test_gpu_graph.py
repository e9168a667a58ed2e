"""Graph capture: a decode step captured into a HIP graph (through torch's
graph API, on the caller's capturing stream) replays to exactly the eager
results, several times, with eager work and synchronisations between the
replays.  Covered: a small step (one stream), one whose attention units
select for themselves, a step that forks the
streaming attention onto the library's side stream and joins it back, and
the shared-index step.  The library records no memset or copy on the
stream, so everything it enqueues is kernels and event waits."""
import numpy as np
import pytest
import torch

import head_aware_sparse_amd as H
from synth import recipe as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

N_REPLAYS = 3


def _replay_matches(enqueue, outs, eager, between):
    """Capture enqueue() (which writes into outs), then replay it N_REPLAYS
    times; before each replay the outputs are poisoned and other eager work
    runs, after it every output must equal the eager result bit for bit."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as torch advises before capture
        enqueue()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        enqueue()
    torch.cuda.synchronize()
    for r in range(N_REPLAYS):
        for t in outs:
            t.fill_(-7 if t.dtype == torch.int32 else float("nan"))
        between()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            got = t.cpu().numpy()
            if t.dtype == torch.int32:
                assert (got == e).all(), f"replay {r}: indices differ"
            else:
                assert np.array_equal(got, e), f"replay {r}: outputs differ"


def _decode_case(case):
    cfg = case.cfg
    ref_out, ref_idx, ws = case.run()
    out = torch.empty((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), device="cuda")
    ix = torch.empty((cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.n_fac), dtype=torch.int32, device="cuda")
    ws2 = torch.empty_like(ws)

    def enqueue():
        H.sparse_decode_step(case.dims, case.q, case.k, case.v, case.k_dom, case.i_dom, case.labels, out, ix, ws=ws2)

    def between():  # an eager step of its own on the same cache, with its own workspace
        case.run(ws=ws)

    _replay_matches(enqueue, [out, ix], [ref_out, ref_idx], between)


def test_small_step_graph_replays():
    cfg = R.get_config("c1", ctx_len=20000, batch=2, n_layers=2)
    print("case graph small step", flush=True)
    _decode_case(U.DeviceCase(cfg))


def test_selecting_attention_step_graph_replays():
    # one layer, batch 1: 200 attention units, so the FAC units find their
    # item's cut themselves (no final-selection launch)
    cfg = R.get_config("c1", ctx_len=20000, batch=1, n_layers=1)
    print("case graph selecting attention units", flush=True)
    _decode_case(U.DeviceCase(cfg))


def test_side_stream_step_graph_replays():
    # 8 layers x batch 16 x 8 groups with 4100 streaming rows each: above the
    # 2^20-row threshold, so the step forks to the side stream and joins it
    cfg = R.get_config("c1", ctx_len=16384, batch=16, n_layers=8, window=4096)
    print("case graph side stream", flush=True)
    rng = np.random.default_rng(11)
    lab = (rng.random((cfg.n_layers, cfg.n_kv_heads)) < 0.25).astype(np.uint8)
    lab[0, 0] = 1
    assert (1 - lab).sum() * cfg.batch * (cfg.n_sink + cfg.window) >= 1 << 20
    _decode_case(U.DeviceCase(cfg, labels=lab))


def test_shared_index_step_graph_replays():
    cfg = R.get_config("c3", ctx_len=16384, batch=2)
    print("case graph shared index", flush=True)
    case = U.DeviceCase(cfg)
    ref_out, ref_idx, ws = U.run_clsa(case)
    out = torch.empty((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), device="cuda")
    ix = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.n_fac), dtype=torch.int32, device="cuda")
    ws2 = torch.empty_like(ws)

    def enqueue():
        H.shared_index_decode(case.dims, case.q, case.k[0], case.v[0], case.k_dom[0], case.i_dom[0], out, idx_out=ix,
                              ws=ws2)

    _replay_matches(enqueue, [out, ix], [ref_out, ref_idx], lambda: U.run_clsa(case, ws=ws))
