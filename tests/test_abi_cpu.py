"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import head_aware_sparse_amd as H
from head_aware_sparse_amd.binding import DecodeDims, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "has.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"aoh_label", "sparse_decode_step", "shared_index_decode", "kdom_pack"} <= set(names)
    L = lib()
    for n in names:
        assert hasattr(L, n), n


def _dims(**over):
    d = DecodeDims(1, 1, 32, 8, 128, 32768, 2048, 4, 1024, 16, H.HAS_BF16, 0)
    for k, v in over.items():
        setattr(d, k, v)
    return d


FAKE = 0x10000  # never dereferenced: validation fails first


def _decode(d, ws_bytes=1 << 40, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, kd=FAKE, idom=FAKE, lab=FAKE, out=FAKE, idx=None, ws=FAKE)
    p.update(ptrs)
    P = ctypes.c_void_p
    return lib().sparse_decode_step(ctypes.byref(d), P(p["q"]), P(p["k"]), P(p["v"]), P(p["kd"]), P(p["idom"]),
                                    P(p["lab"]), P(p["out"]), P(p["idx"]), P(p["ws"]), ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(n_q_heads=30), 1), (dict(n_q_heads=48, n_kv_heads=3), 2), (dict(d_head=96), 2),
    (dict(d_head=7), 1), (dict(ctx_len=0), 1), (dict(n_fac=0), 1), (dict(n_fac=40000), 1),
    (dict(n_sink=0, window=0), 1), (dict(window=-1), 1), (dict(n_dom=0), 1), (dict(n_dom=65), 1),
    (dict(kv_dtype=5), 1), (dict(rope_layout=3), 1), (dict(n_layers=2000, n_kv_heads=8, n_q_heads=8), 2),
    (dict(ctx_len=1 << 23, n_fac=10), 2), (dict(batch=0), 1),
    (dict(kv_dtype=H.HAS_F32, n_dom=33), 2),  # fp32 dominant-key rows above 256 bytes
])
def test_bad_dims_rejected(over, status):
    assert _decode(_dims(**over)) == status
    assert H.last_error()


def test_bad_pointers_and_workspace():
    d = _dims()
    assert _decode(d, q=None) == 1 and "q" in H.last_error()
    assert _decode(d, kd=FAKE + 4) == 1 and "aligned" in H.last_error()
    assert _decode(d, lab=None) == 1
    assert _decode(d, idx=FAKE + 8) == 1
    assert _decode(d, ws=None) == 3
    need = H.sparse_decode_workspace(d)
    assert need > 0
    assert _decode(d, ws_bytes=need - 1) == 3
    assert H.sparse_decode_workspace(_dims(d_head=96)) == 0


def _noalloc(d, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, kd=FAKE, idom=FAKE, lab=FAKE, out=FAKE, idx=None)
    p.update(ptrs)
    P = ctypes.c_void_p
    return lib().sparse_decode_step_noalloc(ctypes.byref(d), P(p["q"]), P(p["k"]), P(p["v"]), P(p["kd"]),
                                            P(p["idom"]), P(p["lab"]), P(p["out"]), P(p["idx"]), None)


def test_noalloc_checks_before_touching_the_device():
    """The allocation-free variant validates like sparse_decode_step, and
    rejects dims whose scratch exceeds the fixed array, all before its first
    HIP call (no GPU here)."""
    assert H.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert _noalloc(_dims(d_head=96)) == 2
    assert _noalloc(_dims(), q=None) == 1 and "q" in H.last_error()
    assert _noalloc(_dims(), out=FAKE + 4) == 1
    big = _dims(n_layers=32, batch=4, ctx_len=131072, n_fac=4096, window=2048)
    assert H.sparse_decode_workspace(big) > H.NOALLOC_SCRATCH_BYTES
    assert _noalloc(big) == 3 and "noalloc" in H.last_error()
    fits = _dims(batch=16)
    assert H.sparse_decode_workspace(fits) <= H.NOALLOC_SCRATCH_BYTES


def test_shared_index_allows_null_labels_only_there():
    d = _dims(n_layers=8)
    P = ctypes.c_void_p
    r = lib().shared_index_decode(ctypes.byref(d), P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None,
                                  P(FAKE), None, None, 1 << 40, None)
    assert r == 3  # passes argument checks, stops at the NULL workspace
    assert H.shared_index_workspace(d) > 0


def test_label_argument_checks():
    P = ctypes.c_void_p
    L = lib()
    ws = 1 << 40
    args = lambda **o: dict(dict(L=1, Hq=4, Hkv=4, dm=256, d=64, wdt=0, wq=FAKE, wk=FAKE, k=2, thr=0.0, lab=FAKE,
                                  ws=FAKE), **o)

    def call(a):
        return L.aoh_label(a["L"], a["Hq"], a["Hkv"], a["dm"], a["d"], a["wdt"], P(a["wq"]), P(a["wk"]), a["k"],
                           a["thr"], None, None, P(a["lab"]), P(a["ws"]) if a["ws"] else None, ws, None)
    assert call(args(Hq=6)) == 1
    assert call(args(d=96)) == 2
    assert call(args(dm=100)) == 2
    assert call(args(k=5)) == 1
    assert call(args(wq=None)) == 1
    assert call(args(lab=None)) == 1
    assert call(args(ws=None)) == 3
    assert H.aoh_label_workspace(1, 4, 4, 256, 64) > 0


def test_status_strings_and_row_elems():
    assert H.status_string(0) == "HAS_OK" and H.status_string(4) == "HAS_ERR_HIP"
    assert H.kdom_row_elems(_dims()) == 32
    assert H.kdom_row_elems(_dims(n_dom=12)) == 32   # 24 bf16 -> padded to 4 vectors
    assert H.kdom_row_elems(_dims(n_dom=1)) == 8
    assert H.kdom_row_elems(_dims(n_dom=8, kv_dtype=H.HAS_F32)) == 16


def test_select_and_attend_argument_checks():
    """sparse_select / fac_attend take one layer; fields they do not use are
    not validated (fac_attend ignores n_sink, window, n_dom, rope_layout)."""
    P = ctypes.c_void_p
    L = lib()

    def select(d, ws=FAKE, ws_bytes=1 << 40, **o):
        p = dict(qi=FAKE, kd=FAKE, idom=FAKE, idx=FAKE)
        p.update(o)
        return L.sparse_select(ctypes.byref(d), P(p["qi"]), P(p["kd"]), P(p["idom"]), P(p["idx"]),
                               P(ws) if ws else None, ws_bytes, None)

    def attend(d, ws=FAKE, ws_bytes=1 << 40, **o):
        p = dict(q=FAKE, k=FAKE, v=FAKE, idx=FAKE, out=FAKE)
        p.update(o)
        return L.fac_attend(ctypes.byref(d), P(p["q"]), P(p["k"]), P(p["v"]), P(p["idx"]), P(p["out"]),
                            P(ws) if ws else None, ws_bytes, None)

    d = _dims()
    assert select(_dims(n_layers=2)) == 1 and "n_layers" in H.last_error()
    assert attend(_dims(n_layers=2)) == 1
    assert select(d, idx=None) == 1 and "idx_out" in H.last_error()
    assert attend(d, idx=None) == 1
    assert attend(d, q=FAKE + 4) == 1 and "aligned" in H.last_error()
    assert select(_dims(n_dom=0)) == 1
    assert select(d, ws=None) == 3
    # unused fields: not validated, the call gets as far as the workspace check
    assert select(_dims(n_sink=0, window=0), ws=None) == 3
    assert attend(_dims(n_sink=0, window=0, n_dom=0, rope_layout=7), ws=None) == 3
    need_s, need_a = H.sparse_select_workspace(d), H.fac_attend_workspace(d)
    assert need_s > 0 and need_a > 0
    assert select(d, ws_bytes=need_s - 1) == 3
    assert attend(d, ws_bytes=need_a - 1) == 3
    assert H.fac_attend_workspace(_dims(n_layers=2)) == 0
    # the attention-only workspace holds the chunk partials alone
    assert need_a < need_s


def test_split_cache_argument_checks():
    """kv_append and sparse_decode_step_split validate positions, capacity
    and pointers on the host."""
    P = ctypes.c_void_p
    L = lib()

    def append(d, cap=40000, pos=0, n_new=1, **o):
        p = dict(kn=FAKE, vn=FAKE, idom=FAKE, lab=FAKE, kr=FAKE, vr=FAKE, kdr=FAKE, ks=FAKE, vs=FAKE)
        p.update(o)
        return L.kv_append(ctypes.byref(d), cap, pos, n_new, P(p["kn"]), P(p["vn"]), P(p["idom"]), P(p["lab"]),
                           P(p["kr"]), P(p["vr"]), P(p["kdr"]), P(p["ks"]), P(p["vs"]), None)

    def split(d, cap=40000, ws=None, **o):
        p = dict(q=FAKE, kr=FAKE, vr=FAKE, kdr=FAKE, ks=FAKE, vs=FAKE, idom=FAKE, lab=FAKE, out=FAKE)
        p.update(o)
        return L.sparse_decode_step_split(ctypes.byref(d), cap, P(p["q"]), P(p["kr"]), P(p["vr"]), P(p["kdr"]),
                                          P(p["ks"]), P(p["vs"]), P(p["idom"]), P(p["lab"]), P(p["out"]), None,
                                          P(ws) if ws else None, 1 << 40, None)

    d = _dims()
    assert append(d, pos=-1) == 1
    assert append(d, n_new=0) == 1
    assert append(d, pos=39999, n_new=2) == 1 and "capacity" in H.last_error()
    assert append(d, ks=None) == 1 and "k_str" in H.last_error()
    assert append(d, kn=FAKE + 2) == 1
    assert append(_dims(d_head=96)) == 2
    assert append(_dims(n_sink=0, window=0)) == 1
    assert split(d, cap=100) == 1 and "capacity" in H.last_error()
    assert split(d, vs=None) == 1 and "v_str" in H.last_error()
    assert split(d, lab=None) == 1
    assert split(d) == 3  # arguments valid: stops at the NULL workspace


@pytest.mark.parametrize("T,n_fac,path", [
    (8191, 500, 0), (8192, 3000, 1), (8192, 3002, 0),       # below the sample's 2 x 4096 tokens; the first edge
    (32768, 2048, 1), (32768, 9498, 1), (32768, 9600, 0),   # expected candidates within 80% of 16384 slots
    (131072, 4096, 1), (131072, 8401, 1), (131072, 8402, 0),
    (131073, 8192, 1), (131073, 8193, 0),                   # beyond 131072 tokens: also n_fac <= 8192
    (262144, 7420, 1), (262144, 7421, 0), (524288, 6001, 1), (524288, 6002, 0),
    (524288, 4096, 1), (524289, 4096, 0),                   # the final kernel's token bitmap limit
])
def test_selection_path_rule(T, n_fac, path):
    """The rule choosing between the two exact selection paths, at its edges
    (the GPU boundary tests run the same shapes against the oracle)."""
    assert H.sparse_selection_path(_dims(ctx_len=T, n_fac=n_fac)) == path


def test_selection_path_rejects_bad_dims():
    with pytest.raises(H.HasError):
        H.sparse_selection_path(_dims(n_fac=40000))
