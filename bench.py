#!/usr/bin/env python3
"""Benchmark of the head-aware sparse decode step on one MI355X.

Default workload: the full 32-layer Llama-3-8B-shaped pipeline at 128K
context -- one sparse_decode_step over 32 layers x batch 4 x 8 KV groups
(64 of the 256 (layer, group) pairs retrieval: TIP over 16 of 64 frequency
chunks + top-4096 + focused attention; the rest sink 4 + window 2048), bf16
cache of 131072 tokens (68.7 GB resident).  A step is one call of the whole
decode path (plan, scoring, selection, attention, merge) over that batch.
The offline AoH labeller that produces the labels (aoh_label over the
32 x 40 heads) and the cache-write-time dominant-key packing are timed
separately and reported in the same line.

Prints ONE JSON line.  Inputs are seeded synthetic data (synth package),
resident in HBM before timing starts.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode-attn steps/s at 32K & 128K ctx; achieved HBM TB/s vs peak"
HBM_PEAK_GBPS = 8000.0
REPLICA_TOUCH_BYTES = 600e6  # bytes a rotation of cache copies must touch (> the 256 MB MALL)
BF16_MFMA_PEAK_TFLOPS = 2500.0
# speed-ups over full attention that the pages report, on hardware they do
# not name: context for the measured full-attention comparison, not targets
PAGES_SPEEDUPS = [
    {"source": "Resumen Técnico: Autonomía de Cabezales (AoH), Resultados / Eficiencia",
     "decode_speedup": 9.14, "setting": "Llama3.1-8B, 256K context, model-level", "hardware": "not stated"},
    {"source": "El enrutamiento compartido entre capas acelera la atención dispersa 7 veces sin afectar la calidad "
               "(CLSA news article), opening and closing paragraphs",
     "decode_speedup": 7.6, "setting": "shared-KV model, 128K context, k 512, model-level",
     "hardware": "one GPU, not named"},
    {"source": "FASA: Frequency-aware Sparse Attention, results (Long-CoT reasoning)",
     "decode_speedup": 2.56, "setting": "AIME24 with 18.9% of the cache, end to end", "hardware": "not stated"},
]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, labels, per_layer_gather=False, per_head=False):
    """Bytes the method must move per step (counted once): dominant key
    channels of retrieval items, selected K+V rows, sink+window K+V rows,
    queries and outputs.  Scores, histograms and partials are not counted.
    per_layer_gather: the shared index is attended layer by layer, each layer
    gathering the selected rows again.  per_head: every query head selects
    and gathers for itself (G times the selected rows of a retrieval group);
    the group's dominant key channels are still needed once, as its G heads
    score against the same rows."""
    import numpy as np
    es = 2 if cfg.bf16 else 4
    d, T = cfg.d_head, cfg.ctx_len
    row = 2 * d * es
    s_end = min(cfg.n_sink, T)
    n_srows = s_end + T - max(T - cfg.window, s_end)
    if cfg.clsa:
        n_idx = cfg.batch * cfg.n_kv_heads
        n_ret_att = int(labels.sum()) * cfg.batch if labels is not None else cfg.n_layers * n_idx
        n_str_att = cfg.n_layers * n_idx - n_ret_att
        tip = n_idx * T * 2 * cfg.n_dom * es
        gather = n_idx * cfg.n_fac * row          # one gather serves every layer
        if per_layer_gather:
            gather *= cfg.n_layers
        stream = (n_srows * row * cfg.batch * cfg.n_kv_heads) if n_str_att else 0
    else:
        n_ret = int(np.asarray(labels).sum()) * cfg.batch
        n_str = cfg.n_layers * cfg.batch * cfg.n_kv_heads - n_ret
        rep = cfg.n_q_heads // cfg.n_kv_heads if per_head else 1
        tip = n_ret * T * 2 * cfg.n_dom * es
        gather = rep * n_ret * cfg.n_fac * row
        stream = n_str * n_srows * row
    qo = cfg.n_layers * cfg.batch * cfg.n_q_heads * d * (es + 4)
    return {"tip": tip, "gather": gather, "stream": stream, "q_out": qo, "total": tip + gather + stream + qo}


def traffic_from_profiles(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken from the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_key}.counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, rec["source"])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if sha != rec.get("source_sha256"):
        return None
    return rec["hbm_bytes_per_launch"]


def _host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_time_items(items, make_inputs, run_item, reps, cores):
    """Times the oracle over `items` with `cores` of them in flight at once
    (one thread each, BLAS limited to one thread per call), in rounds of
    `cores` items whose inputs are built beforehand (not timed).  Returns
    (effective seconds per item call on all the cores, CPU seconds spent)."""
    import concurrent.futures as cf
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    wall, calls = 0.0, 0
    for r0 in range(0, len(items), cores):
        chunk = items[r0:r0 + cores]
        inputs = [make_inputs(it) for it in chunk]

        def work(x):
            for _ in range(reps):
                run_item(x)

        ctx = threadpool_limits(limits=1) if threadpool_limits else None
        if ctx is not None:
            ctx.__enter__()
        try:
            t0 = time.perf_counter()
            with cf.ThreadPoolExecutor(len(chunk)) as ex:
                list(ex.map(work, inputs))
            wall += time.perf_counter() - t0
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
        calls += len(chunk) * reps
        del inputs
    return wall / calls, wall * min(cores, len(items))


def cpu_baseline(cfg, hi, labels, n_ret_sample, n_str_sample, reps, cores=None):
    """fp64 oracle (oracle.fasa.decode_group) on a bounded sample of the
    step's (layer, sequence, KV group) items, `cores` items at a time on the
    host's cores, scaled to the whole step (input generation excluded)."""
    import numpy as np
    from oracle import fasa
    from synth import recipe as R
    cores = cores or min(16, _host_cores())
    G = cfg.group
    ret = [(l, g) for l in range(cfg.n_layers) for g in range(cfg.n_kv_heads) if labels[l, g]]
    strm = [(l, g) for l in range(cfg.n_layers) for g in range(cfg.n_kv_heads) if not labels[l, g]]
    rng = np.random.default_rng(7)

    def make(it):
        l, g, b = it
        f = lambda a: R.storage_to_f64(a, cfg.bf16)
        return (f(hi.q[l, b, g * G:(g + 1) * G]), f(hi.rows("k", l, b, g)), f(hi.rows("v", l, b, g)), l, g)

    def run(x):
        q, k, v, l, g = x
        fasa.decode_group(q, k, v, hi.i_dom[l, g], bool(labels[l, g]), cfg.n_fac, cfg.n_sink, cfg.window)

    step_s, cpu_s, counts = 0.0, 0.0, []
    for pool, n in ((ret, n_ret_sample), (strm, n_str_sample)):
        if not pool or n <= 0:
            counts.append(0)
            continue
        pick = rng.choice(len(pool), size=min(n, len(pool) * cfg.batch), replace=len(pool) < n)
        items = [(*pool[i], int(rng.integers(cfg.batch))) for i in pick]
        per_call, used = cpu_time_items(items, make, run, reps, cores)
        step_s += per_call * len(pool) * cfg.batch
        cpu_s += used
        counts.append(len(items))
    n_ret_items, n_str_items = len(ret) * cfg.batch, len(strm) * cfg.batch
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"{counts[0]} retrieval + {counts[1]} streaming (layer, sequence, KV group) items of the "
                       f"step, each run {reps} times by the fp64 numpy oracle with {cores} items in flight on "
                       f"{cores} host threads ({cpu_s:.1f} CPU-s), scaled to {n_ret_items} + {n_str_items} items")}


def cpu_baseline_clsa(cfg, hi, reps, cores=None):
    """fp64 oracle (oracle.clsa.shared_index_decode, one (sequence, KV group)
    item per call: the indexer's TIP and top-n_fac once, then every layer's
    attention over that index) on the whole step's items, `cores` at a time."""
    import numpy as np
    from oracle import clsa as oclsa
    from synth import recipe as R
    cores = cores or min(16, _host_cores())
    G = cfg.group
    f = lambda a: R.storage_to_f64(a, cfg.bf16)
    items = [(b, g) for b in range(cfg.batch) for g in range(cfg.n_kv_heads)]

    def make(it):
        b, g = it
        return (f(hi.q[:, b:b + 1, g * G:(g + 1) * G]), f(hi.rows("k", 0, b, g))[None, None],
                f(hi.rows("v", 0, b, g))[None, None], g)

    def run(x):
        q, k, v, g = x
        oclsa.shared_index_decode(q, k, v, hi.i_dom[0, g:g + 1], cfg.n_fac)

    per_call, used = cpu_time_items(items, make, run, reps, cores)
    step_s = per_call * len(items)
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"all {len(items)} (sequence, KV group) items of the step, each run {reps} times by the "
                       f"fp64 numpy oracle with {cores} items in flight on {cores} host threads "
                       f"({used:.1f} CPU-s)")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4"])
    ap.add_argument("--clsa-mode", default="fused", choices=["fused", "sequential"],
                    help="shared-index workload: one fused call, or one sparse_select plus one fac_attend per layer")
    ap.add_argument("--cache", default="full", choices=["full", "split", "split-host"],
                    help="split: streaming groups keep only sink + window rows (filled by kv_append); "
                         "split-host: also the retrieval groups' K and V rows in pinned host memory (FASA-M)")
    ap.add_argument("--select", default="group", choices=["group", "per-head"],
                    help="per-head: every query head selects its own tokens (the ablation of the group-mean TIP)")
    ap.add_argument("--no-split", action="store_true",
                    help="with the full cache: skip the extra timing of the same step on the split cache")
    ap.add_argument("--ctx-len", type=int, default=None, help="override the workload's context length")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the full-attention comparison")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    ap.add_argument("--no-label", action="store_true")
    ap.add_argument("--labels-out", default=None,
                    help="save the headline config's labeller outputs (labels, ERs, I_dom) to this .npz")
    ap.add_argument("--labels-in", default=None,
                    help="take the headline config's labels from this .npz (written by --labels-out) "
                         "instead of running the labeller")
    ap.add_argument("--cpu-sample", default="24,72", help="retrieval,streaming items timed on the CPU")
    ap.add_argument("--cpu-reps", type=int, default=4, help="oracle calls timed per sampled item")
    ap.add_argument("--extra-configs", default="c3,c2,c1",
                    help="after the default c4 line: also time these workloads and report them under 'configs' "
                         "('none' to skip)")
    ap.add_argument("--calib-bytes", type=int, default=1 << 30,
                    help="size of the reference copy kernel (torch.neg, fp32) timed beside the step")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the decode path on one GPU only; --gpus above 1 is not supported "
              "(the per-(layer, sequence, KV group) work items would shard across GPUs with no exchange; "
              "see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    res = run_config(args, args.config, headline=True)
    extra = [c for c in args.extra_configs.split(",") if c and c != "none"]
    variant = (args.ctx_len is not None or args.batch is not None or args.cache != "full" or args.select != "group"
               or args.clsa_mode != "fused" or args.config != "c4")
    if extra and not variant:
        # the other workloads of the metric, each on a fresh set of inputs
        # after the previous one's memory is released
        res["configs"] = {}
        for name in extra:
            torch.cuda.empty_cache()
            sub = argparse.Namespace(**vars(args))
            sub.no_label, sub.no_graph, sub.no_split = True, True, True
            # the CPU oracle on every item of the small steps (a few CPU-s each)
            sub.cpu_sample, sub.cpu_reps = {"c1": ("2,6", 40), "c2": ("32,96", 4)}.get(name, (args.cpu_sample,
                                                                                           args.cpu_reps))
            sub.steps = max(args.steps, 200)
            sub.warmup = max(args.warmup, 20)
            r = run_config(sub, name, headline=False)
            res["configs"][name] = {k: r[k] for k in (
                "value", "unit", "ms_per_step", "steps", "warmup", "config", "roofline", "step_algorithmic_bytes",
                "step_hbm_GBps", "step_hbm_frac", "tokens_scored_per_s", "kernels_ms", "replicas",
                "dense_attention", "cpu_baseline") if k in r}
            log(f"{name}: {r['ms_per_step']:.4f} ms/step, {r['step_hbm_frac']:.3f} of peak")
    # provenance: the library sources this run's libhas.so was built from
    # (the kernel sources also key the counter records under profiles/)
    res["source_sha256"] = {
        f: hashlib.sha256(open(os.path.join(ROOT, "head_aware_sparse_amd", "csrc", f), "rb").read()).hexdigest()[:16]
        for f in ("decode.hip", "label.hip", "api.cpp")}
    print(json.dumps(res), flush=True)


def run_config(args, cfg_name, headline=True):
    """Builds one workload's inputs in HBM, times its step and returns the
    result record (the headline line's keys)."""
    import numpy as np
    import torch

    import head_aware_sparse_amd as H
    from synth import device as sdev
    from synth import recipe as R

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    over = {k: v for k, v in (("ctx_len", args.ctx_len), ("batch", args.batch)) if v is not None}
    cfg = R.get_config(cfg_name, **over) if headline else R.get_config(cfg_name)
    log(f"config {cfg}")
    t0 = time.time()
    hi = R.HostInputs(cfg, with_weights=(cfg.d_model > 0 and not args.no_label))
    dims = H.DecodeDims(cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.d_head, cfg.ctx_len, cfg.n_fac,
                        cfg.n_sink, cfg.window, cfg.n_dom, H.HAS_BF16 if cfg.bf16 else H.HAS_F32, 0)
    kd_dims = H.DecodeDims(*[getattr(dims, f) for f, _ in dims._fields_])
    kd_dims.n_layers = cfg.kv_layers
    q = sdev.to_device(hi.q, "cuda", cfg.bf16)
    k = sdev.kv_cache(cfg, "k", hi)
    v = sdev.kv_cache(cfg, "v", hi)
    i_dom = torch.from_numpy(hi.i_dom).cuda()
    kd = torch.empty((cfg.kv_layers, cfg.batch, cfg.n_kv_heads, cfg.ctx_len, H.kdom_row_elems(kd_dims)),
                     dtype=k.dtype, device="cuda")
    log(f"inputs resident ({(k.numel() + v.numel()) * k.element_size() / 1e9:.1f} GB cache) in {time.time() - t0:.1f}s")

    copy_gbps = None
    if headline:
        # reference: a plain elementwise copy of known size (reads and writes
        # calib-bytes each); its rate is the measured stream bandwidth, and under
        # rocprofv3 its FETCH_SIZE/WRITE_SIZE calibrate the counters
        cal_x = torch.ones(args.calib_bytes // 4, dtype=torch.float32, device="cuda")
        cal_y = torch.empty_like(cal_x)
        torch.neg(cal_x, out=cal_y)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            torch.neg(cal_x, out=cal_y)
        c1.record()
        torch.cuda.synchronize()
        copy_gbps = 2 * args.calib_bytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del cal_x, cal_y

    # cache-write-time packing of the dominant key channels (timed separately)
    H.timing_enable(True)
    for _ in range(3):
        H.kdom_pack(kd_dims, k, i_dom, kd)
    torch.cuda.synchronize()
    kp = H.timing_collect()
    H.timing_enable(False)
    kdom_ms = kp["kdom_pack"][0] / kp["kdom_pack"][1]

    # labels: the offline AoH labeller on the model weights (timed separately)
    label_info = None
    labels_np = hi.labels
    if headline and args.labels_in:
        rec = H.load_labels(args.labels_in, cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.n_dom)
        if not np.array_equal(rec["i_dom"], hi.i_dom):
            raise SystemExit(f"{args.labels_in}: its I_dom is not this workload's (the cache is packed with the seeded one)")
        labels_np = rec["labels"]
        label_info = {"loaded_from": args.labels_in, "n_retrieval": int(labels_np.sum())}
        log(f"labels loaded from {args.labels_in}")
    elif cfg.d_model and not args.no_label:
        wq = sdev.to_device(hi.w_q, "cuda", cfg.bf16)
        wk = sdev.to_device(hi.w_k, "cuda", cfg.bf16)
        lab_d = torch.empty((cfg.n_layers, cfg.n_kv_heads), dtype=torch.uint8, device="cuda")
        erh = torch.empty((cfg.n_layers, cfg.n_q_heads), dtype=torch.float32, device="cuda")
        erg = torch.empty((cfg.n_layers, cfg.n_kv_heads), dtype=torch.float32, device="cuda")
        ws_l = H.aoh_label(wq, wk, cfg.n_q_heads, cfg.n_kv_heads, cfg.d_head, lab_d, cfg.n_retrieval,
                           er_head=erh, er_group=erg)
        torch.cuda.synchronize()
        H.timing_enable(True)
        n_lab = 3
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(n_lab):
            H.aoh_label(wq, wk, cfg.n_q_heads, cfg.n_kv_heads, cfg.d_head, lab_d, cfg.n_retrieval, er_head=erh,
                        er_group=erg, ws=ws_l)
        ev1.record()
        torch.cuda.synchronize()
        lk = H.timing_collect()
        H.timing_enable(False)
        labels_np = lab_d.cpu().numpy()
        w_bytes = (wq.numel() + wk.numel()) * wq.element_size()
        gram_ms = lk["gram"][0] / lk["gram"][1]
        gram_flop = 2.0 * (cfg.n_layers * (cfg.n_q_heads + cfg.n_kv_heads)) * cfg.d_head ** 2 * cfg.d_model
        label_info = {
            "ms": ev0.elapsed_time(ev1) / n_lab,
            "kernels_ms": {n: round(t / c, 4) for n, (t, c) in lk.items()},
            "gram_hbm_GBps": round(w_bytes / (gram_ms * 1e-3) / 1e9, 1),
            "gram_hbm_frac": round(w_bytes / (gram_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "gram_mfma_util": round(gram_flop / (gram_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "labels_match_planted": bool((labels_np == hi.labels).all()),
            "n_retrieval": int(labels_np.sum()),
        }
        if headline and args.labels_out:
            H.save_labels(args.labels_out, labels_np, erh, erg, hi.i_dom)
            label_info["saved_to"] = args.labels_out
        del wq, wk
        log(f"labeller {label_info}")
    labels = torch.from_numpy(np.ascontiguousarray(labels_np)).cuda()

    out = torch.empty((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), dtype=torch.float32, device="cuda")
    sequential = cfg.clsa and args.clsa_mode == "sequential"
    # steps rotate over copies of the cache until the bytes they touch exceed
    # the 256 MB memory-side cache (MALL) with room to spare, so that no step
    # finds the previous step's rows there: c1 64 copies, c2 4, c3 2, c4 1
    ab0 = algorithmic_bytes(cfg, None if cfg.clsa else labels_np)
    n_rep = max(1, -(-int(REPLICA_TOUCH_BYTES) // ab0["total"]))
    per_head = args.select == "per-head" and not cfg.clsa
    split = args.cache in ("split", "split-host") and not cfg.clsa and not per_head
    cache_info = None

    def build_split(host_rows=False):
        """The split cache, filled from the full one by one prefill append
        (capacity 16 rows above the length, for the timed token appends);
        host_rows: the retrieval K and V rows in pinned host memory."""
        lab_flat = labels_np.astype(bool).reshape(-1)
        n_ret, n_str = int(lab_flat.sum()), int((~lab_flat).sum())
        cap = cfg.ctx_len + 16
        S = cfg.n_sink + cfg.window
        mk = lambda *shape: torch.empty(shape, dtype=k.dtype, device="cuda")
        mkr = (lambda *shape: torch.empty(shape, dtype=k.dtype, pin_memory=True)) if host_rows else mk
        sc = dict(k_ret=mkr(n_ret, cfg.batch, cap, cfg.d_head), v_ret=mkr(n_ret, cfg.batch, cap, cfg.d_head),
                  k_dom_ret=mk(n_ret, cfg.batch, cap, H.kdom_row_elems(dims)),
                  k_str=mk(n_str, cfg.batch, S, cfg.d_head), v_str=mk(n_str, cfg.batch, S, cfg.d_head))
        H.timing_enable(True)
        H.kv_append(dims, 0, k, v, i_dom, labels, sc["k_ret"], sc["v_ret"], sc["k_dom_ret"], sc["k_str"], sc["v_str"])
        torch.cuda.synchronize()
        pa = H.timing_collect()
        H.timing_enable(False)
        es = k.element_size()
        host_b = (sc["k_ret"].numel() + sc["v_ret"].numel()) * es if host_rows else 0
        info = {"layout": "split-host" if host_rows else "split", "bytes": sum(t.numel() for t in sc.values()) * es,
                "host_bytes": host_b,
                "full_layout_bytes": (k.numel() + v.numel() + kd.numel()) * es,
                "prefill_append_ms": round(pa["kv_append"][0], 4)}
        return sc, info

    def split_step_fn(sc):
        ws_s = H.sparse_decode_step_split(dims, q, sc["k_ret"], sc["v_ret"], sc["k_dom_ret"], sc["k_str"],
                                          sc["v_str"], i_dom, labels, out)

        def f():
            H.sparse_decode_step_split(dims, q, sc["k_ret"], sc["v_ret"], sc["k_dom_ret"], sc["k_str"], sc["v_str"],
                                       i_dom, labels, out, ws=ws_s)
        return f

    kv_dtype = k.dtype

    def token_append_ms(sc):
        """One decoded token's append (the next position); it overwrites the
        oldest window slot, so it runs after the decode timing."""
        k1 = torch.randn((cfg.n_layers, cfg.batch, cfg.n_kv_heads, 1, cfg.d_head), device="cuda").to(kv_dtype)
        v1 = torch.randn((cfg.n_layers, cfg.batch, cfg.n_kv_heads, 1, cfg.d_head), device="cuda").to(kv_dtype)
        H.timing_enable(True)
        for t in range(10):
            H.kv_append(dims, cfg.ctx_len + t, k1, v1, i_dom, labels, sc["k_ret"], sc["v_ret"], sc["k_dom_ret"],
                        sc["k_str"], sc["v_str"])
        torch.cuda.synchronize()
        ta = H.timing_collect()
        H.timing_enable(False)
        return round(ta["kv_append"][0] / ta["kv_append"][1], 5)

    if split:
        sc_main, cache_info = build_split(host_rows=args.cache == "split-host")
        del k, v, kd  # the split cache replaces the full one
        torch.cuda.empty_cache()
        step = split_step_fn(sc_main)
    elif sequential:
        # the layer-by-layer form: the index once, then one attention call per layer
        k0, v0, kd0, id0 = k[0], v[0], kd[0], i_dom[0]
        d1 = H.DecodeDims(*[getattr(dims, f) for f, _ in dims._fields_])
        d1.n_layers = 1
        idx_t = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.n_fac), dtype=torch.int32, device="cuda")
        ws_s = H.sparse_select(d1, q[0], kd0, id0, idx_t)
        ws_a = H.fac_attend(d1, q[0], k0, v0, idx_t, out[0])

        def step():
            H.sparse_select(d1, q[0], kd0, id0, idx_t, ws=ws_s)
            for n in range(cfg.n_layers):
                H.fac_attend(d1, q[n], k0, v0, idx_t, out[n], ws=ws_a)
    elif cfg.clsa:
        k0, v0, kd0, id0 = k[0], v[0], kd[0], i_dom[0]
        ws = H.shared_index_decode(dims, q, k0, v0, kd0, id0, out, labels=None)
        reps = [(k0, v0, kd0)] + [(k0.clone(), v0.clone(), kd0.clone()) for _ in range(n_rep - 1)]
        turn = [0]

        def step():
            kr, vr, kdr = reps[turn[0] % n_rep]
            turn[0] += 1
            H.shared_index_decode(dims, q, kr, vr, kdr, id0, out, labels=None, ws=ws)
    elif per_head:
        ws = H.sparse_decode_step_per_head(dims, q, k, v, kd, i_dom, labels, out)

        def step():
            H.sparse_decode_step_per_head(dims, q, k, v, kd, i_dom, labels, out, ws=ws)
    else:
        ws = H.sparse_decode_step(dims, q, k, v, kd, i_dom, labels, out)
        reps = [(k, v, kd)] + [(k.clone(), v.clone(), kd.clone()) for _ in range(n_rep - 1)]
        turn = [0]

        def step():
            kr, vr, kdr = reps[turn[0] % n_rep]
            turn[0] += 1
            H.sparse_decode_step(dims, q, kr, vr, kdr, i_dom, labels, out, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel durations (HIP events on the launch stream)
    H.timing_enable(True)
    n_prof = max(5, min(args.steps, 20))
    for _ in range(n_prof):
        step()
    torch.cuda.synchronize()
    kt = H.timing_collect()
    H.timing_enable(False)
    kernels_ms = {n: t / c for n, (t, c) in kt.items()}
    layer_ms = None
    if sequential:
        # per-layer attention time (events on the launch stream): the first
        # layer gathers the selected rows from HBM, later layers find them in
        # the memory-side cache
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(cfg.n_layers + 1)]
        acc = np.zeros(cfg.n_layers)
        for _ in range(n_prof):
            H.sparse_select(d1, q[0], kd0, id0, idx_t, ws=ws_s)
            evs[0].record()
            for n in range(cfg.n_layers):
                H.fac_attend(d1, q[n], k0, v0, idx_t, out[n], ws=ws_a)
                evs[n + 1].record()
            torch.cuda.synchronize()
            acc += [evs[n].elapsed_time(evs[n + 1]) for n in range(cfg.n_layers)]
        layer_ms = [round(x / n_prof, 5) for x in acc]

    # the timed region
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / args.steps
    log(f"{args.steps} steps: {ms:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f})")

    # the same step captured once into a HIP graph and replayed: one graph
    # launch per step from the host instead of the library's launches
    graph_info = None
    if not args.no_graph:
        gside = torch.cuda.Stream()
        gside.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gside):  # warm-up off the default stream before capture
            step()
        torch.cuda.current_stream().wait_stream(gside)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gw0 = time.perf_counter()
        ga.record()
        for _ in range(args.steps):
            graph.replay()
        gb.record()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - gw0
        gms = ga.elapsed_time(gb) / args.steps
        graph_info = {"ms_per_step": round(gms, 5), "value": round(1e3 / gms, 2), "replays": args.steps,
                      "host_ms_per_step": round(gwall * 1e3 / args.steps, 5),
                      "eager_host_ms_per_step": round(wall * 1e3 / args.steps, 5)}
        del graph
        log(f"graph replay {graph_info}")

    # full attention on the same cache and queries, for the speed-up the
    # pages quote: every (layer, KV group) attends all T positions, through
    # the library's own attention (every group streaming, no sink, a window
    # of T); with a shared cache each layer reads it once, layer by layer
    dense = None
    if not split and not args.no_dense:
        dd = H.DecodeDims(*[getattr(dims, f) for f, _ in dims._fields_])
        dd.n_sink, dd.window = 0, cfg.ctx_len
        out_d = torch.empty_like(out)
        if cfg.clsa:
            dd.n_layers = 1
            lab_d0 = torch.zeros((1, cfg.n_kv_heads), dtype=torch.uint8, device="cuda")
            ws_d = H.sparse_decode_step(dd, q[0:1], k, v, kd, i_dom, lab_d0, out_d[0:1])

            def dense_step():
                for n in range(cfg.n_layers):
                    H.sparse_decode_step(dd, q[n:n + 1], k, v, kd, i_dom, lab_d0, out_d[n:n + 1], ws=ws_d)
        else:
            lab_d0 = torch.zeros_like(labels)
            ws_d = H.sparse_decode_step(dd, q, k, v, kd, i_dom, lab_d0, out_d)

            def dense_step():
                H.sparse_decode_step(dd, q, k, v, kd, i_dom, lab_d0, out_d, ws=ws_d)
        dense_step()
        torch.cuda.synchronize()
        n_dense = 3
        d0, d1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for _ in range(n_dense):
            dense_step()
        d1e.record()
        torch.cuda.synchronize()
        dms = d0.elapsed_time(d1e) / n_dense
        dbytes = 2 * cfg.n_layers * cfg.batch * cfg.n_kv_heads * cfg.ctx_len * cfg.d_head * k.element_size()
        dense = {"ms_per_step": round(dms, 4), "bytes": dbytes, "GBps": round(dbytes / (dms * 1e-3) / 1e9, 1),
                 "sparse_speedup": round(dms / ms, 2), "steps": n_dense,
                 "how": "every (layer, KV group) attends all positions with the same kernels "
                        "(all groups streaming, sink 0, window = context)"}
        del ws_d, out_d
        torch.cuda.empty_cache()
        log(f"dense attention {dense}")

    split_extra = None
    if split:
        cache_info["token_append_ms"] = token_append_ms(sc_main)
    elif not cfg.clsa and not args.no_split and not per_head:
        # the same step on the split cache, which then replaces the full one
        sc_x, split_extra = build_split()
        del k, v, kd
        torch.cuda.empty_cache()
        f = split_step_fn(sc_x)
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        x0.record()
        for _ in range(args.steps):
            f()
        x1.record()
        torch.cuda.synchronize()
        xms = x0.elapsed_time(x1) / args.steps
        split_extra.update({"ms_per_step": round(xms, 5), "value": round(1e3 / xms, 2)})
        split_extra["token_append_ms"] = token_append_ms(sc_x)
        del sc_x
        torch.cuda.empty_cache()
    ab = algorithmic_bytes(cfg, None if cfg.clsa else labels_np, per_layer_gather=sequential, per_head=per_head)
    tip_ms = kernels_ms["tip_score"]
    tip_gbps = ab["tip"] / (tip_ms * 1e-3) / 1e9
    n_scored = (cfg.batch * cfg.n_kv_heads if cfg.clsa else int(labels_np.sum()) * cfg.batch) * cfg.ctx_len
    if per_head:
        n_scored *= cfg.group
    key = f"tip_score_{cfg.name}"
    roofline = {"kernel": "tip_score", "bound": "hbm", "achieved": round(tip_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(tip_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic_from_profiles(key),
                "algorithmic_bytes_per_launch": ab["tip"], "avg_launch_ms": round(tip_ms, 5)}
    res = {
        "metric": METRIC,
        "value": round(1e3 / ms, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.bf16 else "f32",
        "data": "synthetic (seeded Philox4x32-10 inputs shaped like the pages' workloads)",
        "config": {"workload": {
            "c1": f"single Llama-3-8B-shaped layer, batch {cfg.batch}, ctx {cfg.ctx_len}, 2 of 8 KV groups retrieval",
            "c2": f"single Llama-3-8B-shaped layer, batch {cfg.batch}, ctx {cfg.ctx_len}, 2 of 8 KV groups retrieval",
            "c3": f"CLSA: 8 layers sharing one KV cache, batch {cfg.batch}, ctx {cfg.ctx_len}, one shared top-2048 "
                  "index" + (", selected once then attended layer by layer (9 calls)" if sequential else ""),
            "c4": f"32-layer Llama-3-8B-shaped sparse decode step, batch {cfg.batch}, ctx {cfg.ctx_len}, 64 of 256 "
                  "(layer, KV group) pairs retrieval"}[cfg.name],
            "clsa_mode": args.clsa_mode if cfg.clsa else None,
            "cache": args.cache if split else "full",
            "select": "per-head" if per_head else "group",
            "name": cfg.name, "layers": cfg.n_layers, "batch": cfg.batch, "ctx_len": cfg.ctx_len,
            "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads, "d_head": cfg.d_head, "n_dom": cfg.n_dom,
            "n_fac": cfg.n_fac, "n_sink": cfg.n_sink, "window": cfg.window},
        "roofline": roofline,
        "step_algorithmic_bytes": ab,
        "step_hbm_GBps": round(ab["total"] / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(ab["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "tokens_scored_per_s": round(n_scored / (ms * 1e-3), 1),
        "kernels_ms": {n: round(t, 5) for n, t in kernels_ms.items()},
        "kdom_pack_ms": round(kdom_ms, 4),
        "measured_copy_GBps": round(copy_gbps, 1) if copy_gbps else None,
        "label": label_info,
    }
    if graph_info is not None:
        res["graph_replay"] = graph_info
    if dense is not None:
        res["dense_attention"] = dense
        res["pages_speedups_context"] = PAGES_SPEEDUPS
    if layer_ms is not None:
        res["fac_attend_ms_per_layer"] = layer_ms
    if cache_info is not None:
        res["cache"] = cache_info
    if split_extra is not None:
        res["split_cache"] = split_extra
    res["replicas"] = n_rep if not (split or sequential or per_head) else 1
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the step")
        if cfg.clsa:
            res["cpu_baseline"] = cpu_baseline_clsa(cfg, hi, max(1, args.cpu_reps // 2))
        else:
            nr, ns = (int(x) for x in args.cpu_sample.split(","))
            res["cpu_baseline"] = cpu_baseline(cfg, hi, labels_np, nr, ns, args.cpu_reps)
        log(f"cpu baseline {res['cpu_baseline']}")
    return res


if __name__ == "__main__":
    main()
