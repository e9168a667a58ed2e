"""GPU parity of sparse_decode_step (through the C ABI) against the fp64 oracle.

Bars (the required agreement for this path): index sets identical except for
tokens whose fp64 TIP score lies within 1e-5 relative of the n_fac-th score;
outputs within 2e-3 absolute + 1e-2 relative (bf16 or fp32 inputs, fp32
accumulation)."""
import numpy as np
import pytest
import torch

import head_aware_sparse_amd as H
from synth import recipe as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _check_items(case, items, tag):
    cfg, hi = case.cfg, case.hi
    out, idx, _ = case.run()
    for (l, b, g) in items:
        ref, ridx, scores = U.oracle_item(cfg, hi, case.labels_np, l, b, g)
        G = cfg.group
        U.check_out(out[l, b, g * G:(g + 1) * G], ref, f"{tag} out l{l} b{b} g{g}")
        if case.labels_np[l, g]:
            U.check_index_set(idx[l, b, g], scores, cfg.n_fac, f"{tag} idx l{l} b{b} g{g}")
        else:
            assert (idx[l, b, g] == -1).all(), f"{tag} streaming idx l{l} b{b} g{g}"
    return out, idx


def _all_items(cfg):
    return [(l, b, g) for l in range(cfg.n_layers) for b in range(cfg.batch) for g in range(cfg.n_kv_heads)]


def test_c0_tiny_fp32_all_items():
    cfg = R.get_config("c0")
    print(f"case c0 {cfg}", flush=True)
    case = U.DeviceCase(cfg)
    _check_items(case, _all_items(cfg), "c0")


def test_c1_llama_layer_32k_all_items():
    cfg = R.get_config("c1")
    print(f"case c1 {cfg}", flush=True)
    case = U.DeviceCase(cfg)
    out, idx = _check_items(case, _all_items(cfg), "c1")
    # the planted needles are selected
    for (l, g) in R.planted_groups(cfg):
        assert np.isin(R.needle_positions(cfg, l, 0, g), idx[l, 0, g]).all()


def test_c2_batch16_32k_all_items():
    cfg = R.get_config("c2")
    print(f"case c2 {cfg}", flush=True)
    case = U.DeviceCase(cfg)
    _check_items(case, _all_items(cfg), "c2")


def _launch_names(case):
    """The library's timed launches of one decode call."""
    H.timing_enable(True)
    try:
        H.timing_collect()
        case.run()
        return H.timing_collect()
    finally:
        H.timing_enable(False)


def test_small_steps_select_in_attention_units():
    """A prefiltered step of at most 512 attention units without the side
    stream (one c1 layer) has no final-selection launch: each FAC unit finds
    its item's cut itself; a larger one (c2, 3200 units) keeps the launch.
    With n_fac 3500 the expected 5200 candidates exceed the 4096 a unit
    holds in LDS, so the units' cut passes read them from global memory:
    every item against the oracle."""
    cfg = R.get_config("c1", n_fac=3500)
    print(f"case selection in attention units {cfg}", flush=True)
    case = U.DeviceCase(cfg)
    names = _launch_names(case)
    assert "select_final" not in names and {"sample", "tip_score", "attention_fac", "merge"} <= set(names), names
    _check_items(case, _all_items(cfg), "c1 n_fac 3500")
    big = U.DeviceCase(R.get_config("c2", n_layers=1, batch=16))
    assert "select_final" in _launch_names(big)


@pytest.mark.parametrize("over", [
    dict(ctx_len=5000, n_fac=777, window=300, n_sink=3),            # ragged chunks everywhere
    dict(ctx_len=3000, n_fac=3000, window=100),                     # every token selected
    dict(ctx_len=2500, n_fac=1, window=4000, n_sink=0),             # one token; window covers all
    dict(ctx_len=1200, n_fac=64, window=0, n_sink=7),               # sink only
    dict(ctx_len=4096, n_fac=300, n_dom=64),                        # all chunks: exact logits
    dict(ctx_len=4096, n_fac=300, n_dom=1),                         # one chunk
], ids=["ragged", "all", "one", "sink-only", "ndom64", "ndom1"])
def test_edge_shapes_bf16(over):
    cfg = R.get_config("c1", **over)
    print(f"case edge {over}", flush=True)
    case = U.DeviceCase(cfg)
    _check_items(case, _all_items(cfg), f"edge {over}")


@pytest.mark.parametrize("over", [
    dict(n_q_heads=8, n_kv_heads=8, ctx_len=3000, n_fac=200, batch=2),     # G = 1
    dict(n_q_heads=16, n_kv_heads=8, ctx_len=3000, n_fac=200, batch=2),    # G = 2
    dict(n_q_heads=64, n_kv_heads=8, ctx_len=3000, n_fac=200, batch=2),    # G = 8
    dict(d_head=64, n_dom=8, ctx_len=3000, n_fac=200, batch=2),            # d = 64 bf16
], ids=["G1", "G2", "G8", "d64"])
def test_group_and_head_sizes(over):
    cfg = R.get_config("c1", **over)
    print(f"case heads {over}", flush=True)
    case = U.DeviceCase(cfg)
    _check_items(case, _all_items(cfg), f"heads {over}")


def test_fp32_d128():
    cfg = R.get_config("c1", kv_dtype="f32", ctx_len=3000, n_fac=250, batch=2)
    print("case f32 d128", flush=True)
    case = U.DeviceCase(cfg)
    _check_items(case, _all_items(cfg), "f32 d128")


def test_label_extremes():
    cfg = R.get_config("c1", ctx_len=4000, n_fac=500, batch=2)
    for name, lab in [("all-retrieval", np.ones((1, 8), np.uint8)), ("all-streaming", np.zeros((1, 8), np.uint8))]:
        print(f"case labels {name}", flush=True)
        case = U.DeviceCase(cfg, labels=lab)
        _check_items(case, _all_items(cfg), name)


def test_degenerate_all_scores_equal():
    """Zero queries: every TIP score is 0, the selection is the first n_fac
    tokens (ties to the lower index) and attention is uniform over them."""
    cfg = R.get_config("c1", ctx_len=20000, n_fac=1500, batch=1)
    print("case zero-q", flush=True)
    case = U.DeviceCase(cfg, zero_q=True)
    out, idx = _check_items(case, _all_items(cfg), "zero-q")
    for (l, g) in R.planted_groups(cfg):
        assert idx[l, 0, g].tolist() == list(range(cfg.n_fac))


def test_deterministic_and_idx_optional():
    cfg = R.get_config("c1", ctx_len=8192, n_fac=1024, batch=4)
    print("case determinism", flush=True)
    case = U.DeviceCase(cfg)
    o1, i1, ws = case.run()
    o2, i2, _ = case.run(ws=ws)
    assert (o1 == o2).all() and (i1 == i2).all()
    o3, _, _ = case.run(idx=False, ws=ws)
    assert (o1 == o3).all()
    # another stream gives the same bits
    s = torch.cuda.Stream()
    out = torch.empty_like(torch.from_numpy(o1)).cuda()
    with torch.cuda.stream(s):
        H.sparse_decode_step(case.dims, case.q, case.k, case.v, case.k_dom, case.i_dom, case.labels, out, None,
                             ws=ws, stream=s)
    s.synchronize()
    assert (out.cpu().numpy() == o1).all()


@pytest.mark.parametrize("over,layout", [
    (dict(), 0), (dict(kv_dtype="f32"), 0), (dict(d_head=64, n_dom=5), 0), (dict(n_dom=13), 1),
], ids=["bf16", "f32", "d64-ndom5", "interleaved-ndom13"])
def test_kdom_pack_matches_channels(over, layout):
    """k_dom holds the dominant chunks' channel pairs of every token (a
    ragged last tile of tokens included) and zeros in the padding."""
    cfg = R.get_config("c1", ctx_len=3000, batch=2, **over)
    case = U.DeviceCase(cfg)
    kd_t = torch.empty_like(case.k_dom)
    H.kdom_pack(U.dims_of(cfg, rope_layout=layout), case.k, case.i_dom, kd_t)
    torch.cuda.synchronize()
    kd = kd_t.cpu().float().numpy()
    k = case.k.cpu().float().numpy()
    d2 = cfg.d_head // 2
    for (l, b, g) in [(0, 0, 0), (0, 1, 5), (0, 1, 7)]:
        f = case.hi.i_dom[l, g]
        pair = (2 * f, 2 * f + 1) if layout else (f, f + d2)
        want = np.stack([k[l, b, g][:, pair[0]], k[l, b, g][:, pair[1]]], axis=-1).reshape(cfg.ctx_len, -1)
        assert (kd[l, b, g][:, :2 * cfg.n_dom] == want).all()
        assert (kd[l, b, g][:, 2 * cfg.n_dom:] == 0).all()


def test_device_fill_equals_host_generator():
    cfg = R.get_config("c1", ctx_len=4096, batch=2)
    case = U.DeviceCase(cfg)
    k = case.k.view(torch.int16).cpu().numpy().view(np.uint16)
    v = case.v.view(torch.int16).cpu().numpy().view(np.uint16)
    l, g = R.planted_groups(cfg)[0]
    for b in range(2):
        assert (k[l, b, g] == case.hi.rows("k", l, b, g)).all()
        assert (v[l, b, g] == case.hi.rows("v", l, b, g)).all()
    assert (k[0, 1, 0] == case.hi.rows("k", 0, 1, 0)).all()


def test_interleaved_rope_pairing():
    """rope_layout = interleaved: chunk f is channels (2f, 2f+1) in k_dom and
    in the group query (the cache data itself is only data here)."""
    cfg = R.get_config("c1", ctx_len=9000, n_fac=700, batch=2)
    print("case interleaved", flush=True)
    case = U.DeviceCase(cfg)
    dims = U.dims_of(cfg, rope_layout=1)
    kd = torch.empty_like(case.k_dom)
    H.kdom_pack(dims, case.k, case.i_dom, kd)
    out = torch.empty((1, cfg.batch, cfg.n_q_heads, cfg.d_head), device="cuda")
    ix = torch.empty((1, cfg.batch, cfg.n_kv_heads, cfg.n_fac), dtype=torch.int32, device="cuda")
    H.sparse_decode_step(dims, case.q, case.k, case.v, kd, case.i_dom, case.labels, out, ix)
    torch.cuda.synchronize()
    out, ix = out.cpu().numpy(), ix.cpu().numpy()
    G = cfg.group
    from oracle import fasa
    for (l, g) in R.planted_groups(cfg):
        for b in range(cfg.batch):
            k = U.f64(case.hi.rows("k", l, b, g), cfg)
            v = U.f64(case.hi.rows("v", l, b, g), cfg)
            q = U.f64(case.hi.q[l, b, g * G:(g + 1) * G], cfg)
            ref, ridx = fasa.decode_group(q, k, v, case.hi.i_dom[l, g], True, cfg.n_fac, cfg.n_sink, cfg.window,
                                          pairing="interleaved")
            scores = fasa.tip_scores(q, k, case.hi.i_dom[l, g], pairing="interleaved")
            U.check_index_set(ix[l, b, g], scores, cfg.n_fac, f"interleaved idx b{b} g{g}")
            U.check_out(out[l, b, g * G:(g + 1) * G], ref, f"interleaved out b{b} g{g}")


@pytest.mark.parametrize("T", [32768, 262144])
def test_prefilter_fallback_too_few_candidates(T):
    """Adversarial scores: the keys at the sampled token positions are scaled
    up 40x, so the sample places its threshold far above the true n_fac-th
    score and fewer than n_fac tokens pass; the selection must fall back to a
    full rescoring of the item and stay exact."""
    import numpy as np
    cfg = R.get_config("c1", ctx_len=T, batch=1)
    print(f"case prefilter fallback T={T}", flush=True)
    hi = R.HostInputs(cfg, with_weights=False)
    T = cfg.ctx_len
    # the library's sample: 256 evenly spread blocks of 16 tokens (bf16, d 128: 4 pieces per key row)
    sampled = np.concatenate([np.arange(16) + (sb * (T - 16)) // 255 for sb in range(256)])
    (l, g) = R.planted_groups(cfg)[0]
    case = U.DeviceCase(cfg, hi=hi)
    assert H.sparse_selection_path(case.dims) == 1
    kk = case.k[l, 0, g].float()
    kk[torch.from_numpy(sampled).cuda()] *= 40.0
    case.k[l, 0, g] = kk.to(case.k.dtype)
    H.kdom_pack(case.kd_dims, case.k, case.i_dom, case.k_dom)
    torch.cuda.synchronize()
    out, idx, _ = case.run()
    k_host = case.k[l, 0, g].view(torch.int16).cpu().numpy().view(np.uint16)
    assert (np.delete(k_host, sampled, axis=0) == np.delete(hi.rows("k", l, 0, g), sampled, axis=0)).all()
    ref, ridx = U.oracle_item_custom(cfg, hi.q[l, 0, g * cfg.group:(g + 1) * cfg.group], k_host,
                                     hi.rows("v", l, 0, g), hi.i_dom[l, g], True)
    from oracle import fasa
    scores = fasa.tip_scores(U.f64(hi.q[l, 0, g * cfg.group:(g + 1) * cfg.group], cfg), U.f64(k_host, cfg),
                             hi.i_dom[l, g])
    U.check_index_set(idx[l, 0, g], scores, cfg.n_fac, "fallback idx")
    U.check_out(out[l, 0, g * cfg.group:(g + 1) * cfg.group], ref, "fallback out")


@pytest.mark.parametrize("T,n_fac", [(32768, 2048), (262144, 256)], ids=["T32k", "T256k"])
def test_cut_above_sampled_maximum(T, n_fac):
    """More than n_fac tokens outside the sample get their keys scaled up 40x
    (tokens whose score then exceeds every sampled one), so the n_fac-th
    score lies above the sampled maximum, in the candidates' clamped top
    first-digit bin, while the candidate count stays within its slots: the
    final selection must resolve that bin exactly (with the token bitmap in
    its own LDS array, and beyond 131072 tokens in the candidate buffer)."""
    import numpy as np
    cfg = R.get_config("c1", ctx_len=T, n_fac=n_fac, batch=1)
    print(f"case cut above sampled max T={T} n_fac={n_fac}", flush=True)
    hi = R.HostInputs(cfg, with_weights=False)
    sampled = np.concatenate([np.arange(16) + (sb * (T - 16)) // 255 for sb in range(256)])
    (l, g) = R.planted_groups(cfg)[0]
    G = cfg.group
    case = U.DeviceCase(cfg, hi=hi)
    assert H.sparse_selection_path(case.dims) == 1
    from oracle import fasa
    q64 = U.f64(hi.q[l, 0, g * G:(g + 1) * G], cfg)
    s0 = fasa.tip_scores(q64, U.f64(hi.rows("k", l, 0, g), cfg), hi.i_dom[l, g])
    smax = s0[sampled].max()
    outside = np.setdiff1d(np.flatnonzero(s0 > smax / 30.0), sampled)
    assert outside.size > n_fac + 100
    lift = np.random.default_rng(5).choice(outside, n_fac + 100, replace=False)
    kk = case.k[l, 0, g].float()
    kk[torch.from_numpy(lift).cuda()] *= 40.0
    case.k[l, 0, g] = kk.to(case.k.dtype)
    H.kdom_pack(case.kd_dims, case.k, case.i_dom, case.k_dom)
    torch.cuda.synchronize()
    out, idx, _ = case.run()
    k_host = case.k[l, 0, g].view(torch.int16).cpu().numpy().view(np.uint16)
    scores = fasa.tip_scores(q64, U.f64(k_host, cfg), hi.i_dom[l, g])
    assert np.sort(scores)[-n_fac] > scores[sampled].max(), "the cut must lie above every sampled score"
    U.check_index_set(idx[l, 0, g], scores, cfg.n_fac, "cut above sampled max idx")
    ref, _ = U.oracle_item_custom(cfg, hi.q[l, 0, g * G:(g + 1) * G], k_host, hi.rows("v", l, 0, g),
                                  hi.i_dom[l, g], True)
    U.check_out(out[l, 0, g * G:(g + 1) * G], ref, "cut above sampled max out")


@pytest.mark.parametrize("shared_q,levels,T", [(True, 1, 32768), (False, 2, 32768), (False, 2, 262144)],
                         ids=["coarse-ties", "fine-ties", "fine-ties-256k"])
def test_tied_scores_select_exactly(shared_q, levels, T):
    """Integer-valued cache rows and queries make the TIP scores exact small
    multiples of 1/G with hundreds to thousands of tokens on each value, so
    the n_fac-th score is shared by many tokens (ties go to the lower index)
    and the bin that holds it is crowded: the selection must stay exact."""
    cfg = R.get_config("c1", ctx_len=T, batch=1)
    print(f"case ties shared_q={shared_q} levels={levels} T={T}", flush=True)
    hi = R.HostInputs(cfg, with_weights=False)
    (l, g) = R.planted_groups(cfg)[0]
    G = cfg.group
    rng = np.random.default_rng(7 + levels)
    case = U.DeviceCase(cfg, hi=hi)
    k_int = rng.integers(-levels, levels + 1, size=(cfg.ctx_len, cfg.d_head)).astype(np.float32)
    q_int = rng.integers(-levels, levels + 1, size=(G, cfg.d_head)).astype(np.float32)
    if shared_q:
        q_int[:] = q_int[0]
    case.k[l, 0, g] = torch.from_numpy(k_int).to(case.k.dtype).cuda()
    case.q[l, 0, g * G:(g + 1) * G] = torch.from_numpy(q_int).to(case.q.dtype).cuda()
    H.kdom_pack(case.kd_dims, case.k, case.i_dom, case.k_dom)
    torch.cuda.synchronize()
    out, idx, _ = case.run()
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    k_host, q_host = bits(case.k[l, 0, g]), bits(case.q[l, 0, g * G:(g + 1) * G])
    assert (U.f64(k_host, cfg) == k_int).all() and (U.f64(q_host, cfg) == q_int).all()
    from oracle import fasa
    scores = fasa.tip_scores(U.f64(q_host, cfg), U.f64(k_host, cfg), hi.i_dom[l, g])
    sk = -np.sort(-scores)[cfg.n_fac - 1]
    assert (scores == sk).sum() > 50, "the case must tie many tokens at the threshold"
    # exact ties: the set is unique under (score desc, index asc)
    want = np.sort(fasa.top_n(scores, cfg.n_fac))
    assert (idx[l, 0, g] == want).all()
    ref, _ = U.oracle_item_custom(cfg, q_host, k_host, hi.rows("v", l, 0, g), hi.i_dom[l, g], True)
    U.check_out(out[l, 0, g * G:(g + 1) * G], ref, "ties out")


@pytest.mark.parametrize("step_exp", [10, 14], ids=["span-2^17-ulps", "span-2^13-ulps"])
def test_narrow_score_span(step_exp):
    """All TIP scores of one item within a narrow band, 16 + m * 2^-step_exp
    for 257 integer levels m: the sampled keys span 2^13 to 2^17 fp32 steps,
    so the candidate threshold's first 11-bit digit leaves only a few bits
    for the second.  Scores are exact in fp32, and the selection must equal
    the oracle's top-n (ties to the lower token) exactly."""
    cfg = R.get_config("c1", batch=1)
    print(f"case narrow score span 2^-{step_exp}", flush=True)
    hi = R.HostInputs(cfg, with_weights=False)
    (l, g) = R.planted_groups(cfg)[0]
    G = cfg.group
    assert H.sparse_selection_path(U.dims_of(cfg)) == 1
    rng = np.random.default_rng(11 + step_exp)
    case = U.DeviceCase(cfg, hi=hi)
    f0, f1 = (int(x) for x in hi.i_dom[l, g][:2])
    k = U.f64(hi.rows("k", l, 0, g), cfg).astype(np.float32)
    k[:, f0] = 16.0
    k[:, f1] = rng.integers(-128, 129, size=cfg.ctx_len)
    q = U.f64(hi.q[l, 0, g * G:(g + 1) * G], cfg).astype(np.float32)
    dom = np.concatenate([hi.i_dom[l, g], hi.i_dom[l, g] + cfg.d_head // 2])
    q[:, dom] = 0.0
    q[:, f0] = 1.0
    q[:, f1] = 2.0 ** -step_exp
    case.k[l, 0, g] = torch.from_numpy(k).to(case.k.dtype).cuda()
    case.q[l, 0, g * G:(g + 1) * G] = torch.from_numpy(q).to(case.q.dtype).cuda()
    H.kdom_pack(case.kd_dims, case.k, case.i_dom, case.k_dom)
    torch.cuda.synchronize()
    out, idx, _ = case.run()
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    k_host, q_host = bits(case.k[l, 0, g]), bits(case.q[l, 0, g * G:(g + 1) * G])
    from oracle import fasa
    scores = fasa.tip_scores(U.f64(q_host, cfg), U.f64(k_host, cfg), hi.i_dom[l, g])
    assert np.ptp(scores) <= 256 * 2.0 ** -step_exp and np.unique(scores).size > 200
    want = np.sort(fasa.top_n(scores, cfg.n_fac))
    assert (idx[l, 0, g] == want).all()
    ref, _ = U.oracle_item_custom(cfg, q_host, k_host, hi.rows("v", l, 0, g), hi.i_dom[l, g], True)
    U.check_out(out[l, 0, g * G:(g + 1) * G], ref, "narrow span out")


@pytest.mark.parametrize("over,path", [
    (dict(ctx_len=150000, n_fac=2048, batch=1), 1),   # prefiltered, a ragged last scoring unit
    (dict(ctx_len=8191, n_fac=500, batch=2), 0),      # just below its 8192-token minimum
    (dict(ctx_len=32768, n_fac=9600, batch=1), 0),    # expected candidates above 80% of its 16384 slots
    (dict(ctx_len=32768, n_fac=9498, batch=1), 1),    # its largest n_fac at 32768 tokens
    (dict(ctx_len=131072, n_fac=8401, batch=1), 1),   # its largest n_fac at 131072 tokens
    (dict(ctx_len=131073, n_fac=8193, batch=1), 0),   # beyond 131072 tokens: n_fac above its 8192 maximum
    (dict(ctx_len=262144, n_fac=7420, batch=1), 1),   # its largest n_fac at 262144 tokens (selected tokens compacted)
    (dict(ctx_len=8192, n_fac=3000, batch=1), 1),     # near its largest n_fac at its smallest T
], ids=["T150000", "T8191", "nfac9600", "nfac9498", "T131072-nfac8401", "T131073-nfac8193", "T262144-nfac7420",
                           "edge-prefilter"])
def test_selection_path_boundaries(over, path):
    """The general selection path (every score written, radix threshold over
    chunks) and the prefiltered one at the edges of the rule choosing
    between them give the oracle's selection."""
    cfg = R.get_config("c1", **over)
    print(f"case boundaries {over}", flush=True)
    case = U.DeviceCase(cfg)
    assert H.sparse_selection_path(case.dims) == path, "the case must sit on the intended side of the rule"
    _check_items(case, _all_items(cfg)[:cfg.n_kv_heads * 2], f"boundary {over}")


@pytest.mark.parametrize("T", [262144, 524288, 524289], ids=["T256k", "T512k-max-prefiltered", "T512k+1-general"])
def test_long_context_selection(T):
    """Long contexts (the 256K scale and the prefiltered path's 524288-token
    limit, where the final kernel's token bitmap fills most of its candidate
    buffer; one token more takes the general path): a retrieval and a
    streaming group of one sequence against the oracle, the planted needles
    selected."""
    cfg = R.get_config("c1", ctx_len=T, batch=1, n_q_heads=8, n_kv_heads=2)
    print(f"case long context T={T}", flush=True)
    lab = np.array([[1, 0]], np.uint8)
    case = U.DeviceCase(cfg, labels=lab)
    assert H.sparse_selection_path(case.dims) == (1 if T <= 524288 else 0)
    out, idx = _check_items(case, [(0, 0, 0), (0, 0, 1)], f"T{T}")
    assert np.isin(R.needle_positions(cfg, 0, 0, 0), idx[0, 0, 0]).all()


def test_debug_checks_reject_bad_arrays(monkeypatch):
    """HAS_DEBUG=1: i_dom out of range or repeated, or a label other than 0/1,
    is rejected before anything is launched; valid arrays run unchanged."""
    cfg = R.get_config("c1", ctx_len=3000, n_fac=200, batch=1)
    case = U.DeviceCase(cfg)
    ref_out, ref_idx, ws = case.run()
    monkeypatch.setenv("HAS_DEBUG", "1")
    out, idx, _ = case.run(ws=ws)
    assert (out == ref_out).all() and (idx == ref_idx).all()
    good_dom, good_lab = case.i_dom.clone(), case.labels.clone()
    for what, fix in [("out of range", lambda: case.i_dom[0, 1].__setitem__(0, cfg.d_head // 2)),
                      ("repeated", lambda: case.i_dom[0, 2].__setitem__(1, int(case.i_dom[0, 2, 0]))),
                      ("label 2", lambda: case.labels[0].__setitem__(3, 2))]:
        case.i_dom.copy_(good_dom)
        case.labels.copy_(good_lab)
        fix()
        torch.cuda.synchronize()
        with pytest.raises(H.HasError) as e:
            case.run(ws=ws)
        assert e.value.status == 1, what
        with pytest.raises(H.HasError):
            H.kdom_pack(case.kd_dims, case.k, case.i_dom, case.k_dom) if what != "label 2" else case.run(ws=ws)
    case.i_dom.copy_(good_dom)
    case.labels.copy_(good_lab)


def _key_prefix_counts(scores, n_fac):
    """(tokens sharing the n_fac-th score's 11-bit key prefix, tokens sharing
    its 22-bit prefix), keys being the order-preserving bit images of the
    fp32 scores."""
    u = np.asarray(scores, np.float32).view(np.uint32).astype(np.uint64)
    key = np.where(u >> 31 == 1, ~u & 0xFFFFFFFF, u | 0x80000000)
    kth = key[np.argsort(-np.asarray(scores, np.float64), kind="stable")[n_fac - 1]]
    return int((key >> 21 == kth >> 21).sum()), int((key >> 10 == kth >> 10).sum())


def test_general_path_rescans_long_context():
    """The general selection at 262144 tokens with n_fac 9000: the n_fac-th
    score's 11-bit key bin holds more tokens than the exact threshold keeps
    in LDS (8192), so it rescans the item's scores and moves the members of
    the 22-bit prefix into LDS; selection and outputs against the oracle."""
    cfg = R.get_config("c1", ctx_len=262144, n_fac=9000, batch=1)
    print("case general path rescans T=262144 n_fac=9000", flush=True)
    case = U.DeviceCase(cfg)
    assert H.sparse_selection_path(case.dims) == 0
    (l, g) = R.planted_groups(cfg)[0]
    _, _, scores = U.oracle_item(cfg, case.hi, case.labels_np, l, 0, g)
    bin11, bin22 = _key_prefix_counts(scores, cfg.n_fac)
    assert bin11 > 8192 >= bin22, (bin11, bin22)
    _check_items(case, [(l, 0, g), (l, 0, (g + 1) % cfg.n_kv_heads)], "general rescans")
