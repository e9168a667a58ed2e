"""GPU parity of the shared-index step's selection against the oracle.

On the prefiltered path (bf16, d 128, 2 <= N layers, N*G <= 32 query
vectors, up to 131072 tokens) every matrix-core attention unit of a
(sequence, group) finds its item's exact top-n_fac cut from the candidates
itself.  These cases drive each way a unit can read them: from LDS (the
common case), from global memory (more candidates than its LDS holds), or by
rescoring the whole item (the sample misleads, or the candidates overflow
their slots); and the unfused paths, for short contexts (general
selection) and for more expected candidates than the units hold (the final
kernel's selection), each followed by the attention units.  Index sets are compared exactly with the
oracle's top-n (ties to the lower token) where scores tie exactly, else with
the 1e-5 tie band; outputs with |d| <= 2e-3 + 1e-2 |ref|."""
import numpy as np
import pytest
import torch

import head_aware_sparse_amd as H
from oracle import clsa as oclsa
from oracle import fasa
from synth import device as sdev
from synth import recipe as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle(cfg, case, b, g, qi=None):
    """oracle.clsa on one (sequence, group) of the device case's current
    cache contents; qi: indexer query storage [B, Hq, d] or None (layer 0)."""
    G = cfg.group
    f = lambda a: U.f64(a, cfg)
    k = f(_bits(case.k[0, b, g]))
    v = f(_bits(case.v[0, b, g]))
    q = f(case.hi.q[:, b:b + 1, g * G:(g + 1) * G])
    qsel = None if qi is None else f(qi[b:b + 1, g * G:(g + 1) * G])
    out, idx = oclsa.shared_index_decode(q, k[None, None], v[None, None], case.hi.i_dom[0, g:g + 1], cfg.n_fac,
                                         q_index=qsel)
    qs = f(case.hi.q[0, b, g * G:(g + 1) * G]) if qi is None else qsel[0]
    scores = fasa.tip_scores(qs, k, case.hi.i_dom[0, g])
    return out[:, 0], idx[0, 0], scores


def _cfg(**over):
    return R.get_config("c3", **{**dict(ctx_len=32768, batch=2), **over})


def _repack(case):
    H.kdom_pack(case.kd_dims, case.k, case.i_dom, case.k_dom)
    torch.cuda.synchronize()


def test_fused_path_taken_for_the_c3_shape():
    """The 128K shared-index workload and these cases select inside the
    attention units (prefiltered, expected candidates within the LDS they
    hold): the selection path query reports the prefilter."""
    for cfg in (R.get_config("c3"), _cfg()):
        assert H.sparse_selection_path(U.dims_of(cfg)) == 1


def test_candidates_beyond_lds_read_from_global_memory():
    """15500 of the 32768 tokens of one group share the top score exactly, so
    about half of the sample sits on it, the candidate threshold lands on it
    and all 15500 pass: more than a unit's LDS holds (15168), fewer than the
    16384 candidate slots.  The cut falls inside the tie: the lowest-index
    tied tokens are selected."""
    cfg = _cfg()
    print("case clsa fused: candidates from global memory", flush=True)
    case = U.DeviceCase(cfg)
    b, g, G = 0, 2, cfg.group
    rng = np.random.default_rng(21)
    pos = np.sort(rng.choice(np.arange(1, cfg.ctx_len), size=15500, replace=False))
    qbar = U.f64(case.hi.q[0, b, g * G:(g + 1) * G], cfg).mean(axis=0)
    dom = np.concatenate([case.hi.i_dom[0, g], case.hi.i_dom[0, g] + cfg.d_head // 2])
    vals = np.where(qbar[dom] >= 0, 64.0, -64.0).astype(np.float32)
    kk = case.k[0, b, g].float()
    p_d = torch.from_numpy(pos).cuda()
    c_d = torch.from_numpy(dom).cuda()
    kk[p_d[:, None], c_d[None, :]] = torch.from_numpy(vals).cuda()[None, :]
    case.k[0, b, g] = kk.to(case.k.dtype)
    _repack(case)
    out, idx, _ = U.run_clsa(case)
    ref, ridx, scores = _oracle(cfg, case, b, g)
    tied = np.sum(scores == scores[pos[0]])
    assert tied >= 15500 and np.sum(scores > scores[pos[0]]) < cfg.n_fac
    assert (idx[b, g] == ridx).all()
    for n in range(cfg.n_layers):
        U.check_out(out[n, b, g * G:(g + 1) * G], ref[n], f"global-candidates out n{n}")
    # the other groups took the LDS path on the same call
    for (bb, gg) in [(1, 2), (0, 5)]:
        ref, _, scores = _oracle(cfg, case, bb, gg)
        U.check_index_set(idx[bb, gg], scores, cfg.n_fac, f"lds idx b{bb} g{gg}")
        for n in range(cfg.n_layers):
            U.check_out(out[n, bb, gg * G:(gg + 1) * G], ref[n], f"lds out n{n} b{bb} g{gg}")


def test_misleading_sample_rescores_the_item():
    """The keys at the sampled positions of one group scaled up 40x: the
    sample places its threshold far above the true n_fac-th score, fewer
    than n_fac tokens pass, and every unit of that item rescores it in full."""
    cfg = _cfg()
    print("case clsa fused: rescoring fallback", flush=True)
    case = U.DeviceCase(cfg)
    b, g, G = 1, 6, cfg.group
    T = cfg.ctx_len
    sampled = np.concatenate([np.arange(16) + (sb * (T - 16)) // 255 for sb in range(256)])
    kk = case.k[0, b, g].float()
    kk[torch.from_numpy(sampled).cuda()] *= 40.0
    case.k[0, b, g] = kk.to(case.k.dtype)
    _repack(case)
    out, idx, _ = U.run_clsa(case)
    ref, _, scores = _oracle(cfg, case, b, g)
    U.check_index_set(idx[b, g], scores, cfg.n_fac, "rescored idx")
    for n in range(cfg.n_layers):
        U.check_out(out[n, b, g * G:(g + 1) * G], ref[n], f"rescored out n{n}")


def test_candidate_overflow_rescores_the_item():
    """A zero indexer query: every TIP score is 0, every token passes the
    threshold and the candidates overflow their 16384 slots; the units
    rescore and select the first n_fac tokens (ties to the lower index),
    while each layer attends with its own query."""
    cfg = _cfg()
    print("case clsa fused: candidate overflow", flush=True)
    case = U.DeviceCase(cfg)
    qi_np = np.zeros_like(case.hi.q[0])
    qi = sdev.to_device(qi_np, "cuda", cfg.bf16)
    out, idx, _ = U.run_clsa(case, q_index=qi)
    G = cfg.group
    for (b, g) in [(0, 0), (1, 7)]:
        assert idx[b, g].tolist() == list(range(cfg.n_fac))
        ref, ridx, _ = _oracle(cfg, case, b, g, qi=qi_np)
        assert (ridx == np.arange(cfg.n_fac)).all()
        for n in range(cfg.n_layers):
            U.check_out(out[n, b, g * G:(g + 1) * G], ref[n], f"overflow out n{n} b{b} g{g}")


def test_short_context_unfused_path():
    """Below 8192 tokens the selection takes the general path (every score
    written, exact radix threshold) and the matrix-core attention units read
    its index."""
    cfg = _cfg(ctx_len=6000, n_fac=900)
    print("case clsa unfused short context", flush=True)
    assert H.sparse_selection_path(U.dims_of(cfg)) == 0
    case = U.DeviceCase(cfg)
    out, idx, _ = U.run_clsa(case)
    G = cfg.group
    for (b, g) in [(0, 1), (1, 4)]:
        ref, _, scores = _oracle(cfg, case, b, g)
        U.check_index_set(idx[b, g], scores, cfg.n_fac, f"short idx b{b} g{g}")
        for n in range(cfg.n_layers):
            U.check_out(out[n, b, g * G:(g + 1) * G], ref[n], f"short out n{n} b{b} g{g}")


def test_expected_candidates_beyond_lds_unfused_path():
    """About 11100 expected candidates (32768 tokens, n_fac 8000) are more
    than the fused units may count on holding in LDS (70% of 15168), so the
    final kernel selects each item once and the 128-row matrix-core units
    read its index (a ragged last chunk of 64 rows)."""
    cfg = _cfg(n_fac=8000)
    print("case clsa unfused prefiltered selection", flush=True)
    assert H.sparse_selection_path(U.dims_of(cfg)) == 1
    case = U.DeviceCase(cfg)
    out, idx, _ = U.run_clsa(case)
    G = cfg.group
    for (b, g) in [(0, 3), (1, 6)]:
        ref, _, scores = _oracle(cfg, case, b, g)
        U.check_index_set(idx[b, g], scores, cfg.n_fac, f"unfused idx b{b} g{g}")
        for n in range(cfg.n_layers):
            U.check_out(out[n, b, g * G:(g + 1) * G], ref[n], f"unfused out n{n} b{b} g{g}")
