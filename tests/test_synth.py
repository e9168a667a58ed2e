"""The seeded generator: known answers, determinism, slice addressing."""
import numpy as np
import torch

from synth import host
from synth import recipe as R


def test_philox_known_answers():
    """Published Philox4x32-10 known-answer vectors (Random123)."""
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert host.philox(ctr, key).tolist() == want


def test_irwin_hall_moments_and_scale_constant():
    x = host.ih(7, 1, 2, 0, 400_000).astype(np.float64)
    assert abs(x.mean()) < 0.01
    assert abs(x.var() - 1.0) < 0.01
    assert np.abs(x).max() <= np.sqrt(3.0) * 2
    assert np.float32(np.sqrt(3.0) / 2 ** 22) == np.float32(float.fromhex("0x1.bb67aep-22"))


def test_bf16_rne_matches_torch():
    x = np.concatenate([host.ih(3, 1, 1, 0, 10000) * np.float32(37.0),
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65504.0], np.float32)])
    want = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (host.bf16_rne(x) == want).all()


def test_slices_are_addressable_and_deterministic():
    cfg = R.get_config("c1", ctx_len=4096)
    hi = R.HostInputs(cfg, with_weights=False)
    l, g = R.planted_groups(cfg)[0]
    full = hi.rows("k", l, 0, g)
    part = hi.rows("k", l, 0, g, 1000, 1800)
    assert (full[1000:1800] == part).all()
    assert (hi.rows("k", l, 0, g) == full).all()
    v_full = hi.rows("v", l, 0, g)
    assert (hi.rows("v", l, 0, g, 17, 33) == v_full[17:33]).all()


def test_key_rows_are_rotated_raw_rows():
    """Post-RoPE key row t is the rotation of the raw row at position t."""
    cfg = R.get_config("c0")
    hi = R.HostInputs(cfg, with_weights=False)
    g = 3  # not planted: no needles
    k = hi.rows("k", 0, 0, g, 0, 64)
    raw = host.kv_rows(cfg.seed, R.TID_K, R.kv_slice_id(cfg, 0, 0, g), 0, cfg.d_head, 0, 64,
                       hi.masks[0, g], R.OUTLIER_MUL, R.SINK_MUL, None, None)
    cs, sn = hi.tables
    for t in [0, 1, 63]:
        assert (host.rope_apply(raw[t][None], t, cs, sn)[0] == k[t]).all()
    assert np.linalg.norm(raw[0]) > 4 * np.linalg.norm(raw[1:]) / np.sqrt(63)


def test_needles_planted_in_dominant_chunks():
    cfg = R.get_config("c1", ctx_len=4096)
    hi = R.HostInputs(cfg, with_weights=False)
    l, g = R.planted_groups(cfg)[0]
    pos = R.needle_positions(cfg, l, 0, g)
    assert len(pos) == cfg.n_needles and len(set(pos.tolist())) == cfg.n_needles
    assert pos.min() >= 1 and pos.max() < cfg.ctx_len
    chans, vals = R.needle_values(cfg, l, 0, g, hi.i_dom, hi.tables)
    k = hi.rows("k", l, 0, g)
    assert (k[pos][:, chans] == vals).all()


def test_selection_helpers():
    a = R.distinct_sorted(5, 7, 3, 64, 16)
    assert len(set(a.tolist())) == 16 and (np.diff(a) > 0).all() and a.max() < 64
    cfg = R.get_config("c4")
    pg = R.planted_groups(cfg)
    assert len(pg) == 64 and len(set(pg)) == 64
    assert R.planted_labels(cfg).sum() == 64
