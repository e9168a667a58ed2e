"""bench.py's host-side accounting, on the CPU: the algorithmic bytes per
step that the reported bandwidths divide by, the refusal of more than one
GPU, and the traffic lookup's source check."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from synth import recipe as R


def _labels(cfg):
    lab = np.zeros((cfg.n_layers, cfg.n_kv_heads), np.uint8)
    for (l, g) in R.planted_groups(cfg):
        lab[l, g] = 1
    return lab


def test_c4_step_bytes():
    # 64 retrieval pairs x batch 4: K_dom rows of 64 B over 131072 tokens,
    # 4096 selected rows of 512 B (K + V, bf16, d 128); 192 streaming pairs x
    # 4 with sink 4 + window 2048 rows; queries (bf16) and outputs (fp32)
    cfg = R.get_config("c4")
    ab = bench.algorithmic_bytes(cfg, _labels(cfg))
    n_ret, n_str = 64 * 4, 192 * 4
    assert ab["tip"] == n_ret * 131072 * 64
    assert ab["gather"] == n_ret * 4096 * 512
    assert ab["stream"] == n_str * (4 + 2048) * 512
    assert ab["q_out"] == 32 * 4 * 32 * 128 * (2 + 4)
    assert ab["total"] == ab["tip"] + ab["gather"] + ab["stream"] + ab["q_out"]
    assert round(ab["total"] / 1e6, 1) == 3494.4


def test_per_head_and_layer_by_layer_bytes():
    cfg = R.get_config("c4")
    lab = _labels(cfg)
    g, p = bench.algorithmic_bytes(cfg, lab), bench.algorithmic_bytes(cfg, lab, per_head=True)
    assert p["tip"] == g["tip"]  # a group's dominant key rows are read once for its heads
    assert p["gather"] == 4 * g["gather"]  # every head gathers its own selection
    assert p["stream"] == g["stream"]
    c3 = R.get_config("c3")
    f, s = bench.algorithmic_bytes(c3, None), bench.algorithmic_bytes(c3, None, per_layer_gather=True)
    assert f["gather"] == 4 * 8 * 2048 * 512  # one gather serves all 8 layers
    assert s["gather"] == 8 * f["gather"] and s["tip"] == f["tip"] and f["stream"] == 0


def test_short_context_stream_rows():
    # sink and window overlap when T < n_sink + window: the union is every token
    cfg = R.get_config("c1", ctx_len=1000, window=4096)
    ab = bench.algorithmic_bytes(cfg, _labels(cfg))
    n_str = cfg.n_layers * cfg.batch * cfg.n_kv_heads - int(_labels(cfg).sum()) * cfg.batch
    assert ab["stream"] == n_str * 1000 * 2 * cfg.d_head * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_needs_the_profiled_source(tmp_path, monkeypatch):
    # a counter summary taken from other kernel source yields no traffic
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    rec = {"source": "k.hip", "source_sha256": "0" * 64, "hbm_bytes_per_launch": 123}
    (prof / "tip_score_x.counters.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles("tip_score_x") is None
    import hashlib
    rec["source_sha256"] = hashlib.sha256(src.read_bytes()).hexdigest()
    (prof / "tip_score_x.counters.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profiles("tip_score_x") == 123
    assert bench.traffic_from_profiles("tip_score_missing") is None
