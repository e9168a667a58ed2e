"""GPU parity of the per-query-head selection variant: every query head of a
retrieval group selects its own tokens from its own TIP scores and attends
over them.  The oracle is the group decode applied to one head at a time (a
one-head group's mean query is the head's own query)."""
import numpy as np
import pytest
import torch

import head_aware_sparse_amd as H
from oracle import fasa
from synth import recipe as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _run(case):
    cfg = case.cfg
    out = torch.full((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), float("nan"), device="cuda")
    ix = torch.full((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.n_fac), -7, dtype=torch.int32, device="cuda")
    H.sparse_decode_step_per_head(case.dims, case.q, case.k, case.v, case.k_dom, case.i_dom, case.labels, out, ix)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ix.cpu().numpy()


def _check_heads(case, out, idx, heads, tag):
    cfg = case.cfg
    G = cfg.group
    for (l, b, h) in heads:
        g = h // G
        k = U.f64(case.hi.rows("k", l, b, g), cfg)
        v = U.f64(case.hi.rows("v", l, b, g), cfg)
        qh = U.f64(case.hi.q[l, b, h:h + 1], cfg)
        ref, ridx = fasa.decode_group(qh, k, v, case.hi.i_dom[l, g], bool(case.labels_np[l, g]), cfg.n_fac,
                                      cfg.n_sink, cfg.window)
        U.check_out(out[l, b, h:h + 1], ref, f"{tag} out l{l} b{b} h{h}")
        if case.labels_np[l, g]:
            U.check_index_set(idx[l, b, h], fasa.tip_scores(qh, k, case.hi.i_dom[l, g]), cfg.n_fac,
                              f"{tag} idx l{l} b{b} h{h}")
        else:
            assert (idx[l, b, h] == -1).all()


@pytest.mark.parametrize("over", [dict(), dict(kv_dtype="f32", d_head=64, n_dom=8, n_fac=700)],
                         ids=["bf16-d128", "f32-d64"])
def test_per_head_against_oracle(over):
    cfg = R.get_config("c1", **{**dict(ctx_len=20000, batch=2, n_layers=2), **over})
    print(f"case per-head {over}", flush=True)
    lab = np.zeros((cfg.n_layers, cfg.n_kv_heads), np.uint8)
    lab[0, 1] = lab[1, 6] = 1
    case = U.DeviceCase(cfg, labels=lab)
    out, idx = _run(case)
    G = cfg.group
    heads = [(0, 0, G + j) for j in range(G)] + [(1, 1, 6 * G + 2), (0, 1, 0), (1, 0, 3 * G + 1)]
    _check_heads(case, out, idx, heads, "per-head")
    # the heads of one group do not all select the same tokens
    assert any((idx[0, 0, G + j] != idx[0, 0, G]).any() for j in range(1, G))


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 4)], ids=["G2", "G8"])
def test_per_head_group_sizes(hq, hkv):
    """Group sizes 2 and 8: a scoring unit serves the group's 2 or 8 heads
    (steps large enough for the threshold launch), each with its own
    threshold and candidates."""
    cfg = R.get_config("c1", ctx_len=20000, batch=2, n_layers=2, n_q_heads=hq, n_kv_heads=hkv)
    print(f"case per-head G={hq // hkv}", flush=True)
    lab = np.zeros((cfg.n_layers, cfg.n_kv_heads), np.uint8)
    lab[0, 1] = lab[1, hkv - 1] = 1
    case = U.DeviceCase(cfg, labels=lab)
    out, idx = _run(case)
    G = cfg.group
    heads = [(0, 0, G + j) for j in range(G)] + [(1, 1, (hkv - 1) * G + G - 1), (0, 1, 0), (1, 0, 0)]
    _check_heads(case, out, idx, heads, f"per-head G{G}")
    assert any((idx[0, 0, G + j] != idx[0, 0, G]).any() for j in range(1, G))


def test_per_head_all_scores_tied():
    """Zero queries: every token scores 0 for every head, so every token is
    a candidate (the shared scoring units overflow their staging and append
    directly, then the selection falls back to rescoring); ties go to the
    lower token, so each retrieval head selects tokens 0 .. n_fac - 1."""
    cfg = R.get_config("c1", ctx_len=20000, batch=2, n_layers=2)
    print("case per-head tied", flush=True)
    lab = np.zeros((cfg.n_layers, cfg.n_kv_heads), np.uint8)
    lab[0, 2] = lab[1, 5] = 1
    case = U.DeviceCase(cfg, labels=lab, zero_q=True)
    out, idx = _run(case)
    G = cfg.group
    want = np.arange(cfg.n_fac, dtype=np.int32)
    for (l, g) in ((0, 2), (1, 5)):
        for b in range(cfg.batch):
            for j in range(G):
                assert (idx[l, b, g * G + j] == want).all(), f"l{l} b{b} h{g * G + j}"
    _check_heads(case, out, idx, [(0, 1, 2 * G + 3), (1, 0, 5 * G), (0, 0, 0)], "per-head tied")


def test_per_head_with_one_head_per_group_is_the_plain_step():
    cfg = R.get_config("c1", ctx_len=12000, batch=2, n_q_heads=8, n_kv_heads=8)
    print("case per-head G=1", flush=True)
    case = U.DeviceCase(cfg)
    out, idx = _run(case)
    out_p, idx_p, _ = case.run()
    assert (idx == idx_p).all()
    assert np.array_equal(out, out_p)


def test_identical_heads_share_the_group_index():
    """When the G heads of a group carry the same query, the group mean is
    that query: every head's selection equals the group's."""
    cfg = R.get_config("c1", ctx_len=16000, batch=1)
    print("case per-head identical heads", flush=True)
    case = U.DeviceCase(cfg)
    G = cfg.group
    for g in range(cfg.n_kv_heads):
        case.q[:, :, g * G:(g + 1) * G] = case.q[:, :, g * G:g * G + 1].clone()
    torch.cuda.synchronize()
    out, idx = _run(case)
    out_g, idx_g, _ = case.run()
    for g in range(cfg.n_kv_heads):
        for j in range(G):
            assert (idx[:, :, g * G + j] == idx_g[:, :, g]).all()
    np.testing.assert_allclose(out, out_g, rtol=1e-5, atol=1e-6)


def test_per_head_32_layers_128k_sampled():
    cfg = R.get_config("c4")
    print("case c4 per-head", flush=True)
    case = U.DeviceCase(cfg)
    out, idx = _run(case)
    planted = R.planted_groups(cfg)
    G = cfg.group
    (l0, g0), (l1, g1) = planted[3], planted[40]
    heads = [(l0, 1, g0 * G + 2), (l1, 3, g1 * G + 0)]
    streaming = [(l, g) for l in range(cfg.n_layers) for g in range(cfg.n_kv_heads) if (l, g) not in set(planted)]
    (ls, gs) = streaming[50]
    heads.append((ls, 2, gs * G + 3))
    _check_heads(case, out, idx, heads, "c4 per-head")
