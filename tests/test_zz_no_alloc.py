"""sparse_decode_step_noalloc (the entry point for callers that cannot
allocate: its scratch is the library's fixed per-device array) called
through the C ABI, against sparse_decode_step with a workspace on the same
inputs: index sets identical, outputs within |d| <= 2e-3 + 1e-2 |ref| (the
same kernels run in the same order, so they are expected to be equal bit for
bit).  Two calls in a row share the array; the second is smaller, so it runs
over what the first left behind."""
import ctypes

import numpy as np
import pytest
import torch

import head_aware_sparse_amd as H
from head_aware_sparse_amd.binding import lib
from synth import recipe as R
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _noalloc_abi(case):
    """The new entry point called directly through ctypes."""
    cfg = case.cfg
    out = torch.full((cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.d_head), float("nan"), device="cuda")
    ix = torch.full((cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.n_fac), -7, dtype=torch.int32, device="cuda")
    P = ctypes.c_void_p
    r = lib().sparse_decode_step_noalloc(ctypes.byref(case.dims), P(case.q.data_ptr()), P(case.k.data_ptr()),
                                         P(case.v.data_ptr()), P(case.k_dom.data_ptr()), P(case.i_dom.data_ptr()),
                                         P(case.labels.data_ptr()), P(out.data_ptr()), P(ix.data_ptr()),
                                         P(torch.cuda.current_stream().cuda_stream))
    assert r == 0, H.last_error()
    torch.cuda.synchronize()
    return out.cpu().numpy(), ix.cpu().numpy()


def _compare(case, tag):
    out_n, idx_n = _noalloc_abi(case)
    out_w, idx_w, _ = case.run()
    assert (idx_n == idx_w).all(), f"{tag}: index sets differ"
    U.check_out(out_n, out_w.astype(np.float64), f"{tag} out")
    assert np.array_equal(out_n, out_w), f"{tag}: outputs differ from the workspace call"
    return out_n, idx_n


def test_noalloc_matches_workspace_call_twice_second_smaller():
    # first: 2 layers x batch 4 at 65536 tokens, 1.8M streaming rows (the
    # streaming attention runs on the side stream), 34 MiB of scratch
    cfg1 = R.get_config("c1", n_layers=2, batch=4, ctx_len=65536, window=32768)
    assert H.sparse_decode_workspace(U.dims_of(cfg1)) <= H.NOALLOC_SCRATCH_BYTES
    print("case noalloc first (L2 B4 T65536)", flush=True)
    case1 = U.DeviceCase(cfg1)
    out1, idx1 = _compare(case1, "first")
    # one retrieval and one streaming item against the oracle as well
    G = cfg1.group
    (l, g) = R.planted_groups(cfg1)[0]
    ref, _, scores = U.oracle_item(cfg1, case1.hi, case1.labels_np, l, 3, g)
    U.check_out(out1[l, 3, g * G:(g + 1) * G], ref, "first retrieval item vs oracle")
    U.check_index_set(idx1[l, 3, g], scores, cfg1.n_fac, "first retrieval idx vs oracle")
    ref, _, _ = U.oracle_item(cfg1, case1.hi, case1.labels_np, 1, 0, 7)
    U.check_out(out1[1, 0, 7 * G:8 * G], ref, "first streaming item vs oracle")
    del case1
    torch.cuda.empty_cache()
    # second, smaller: 1 layer, batch 1, 9000 tokens, its own n_fac
    cfg2 = R.get_config("c1", batch=1, ctx_len=9000, n_fac=700)
    print("case noalloc second (L1 B1 T9000)", flush=True)
    case2 = U.DeviceCase(cfg2)
    out2, idx2 = _compare(case2, "second")
    (l, g) = R.planted_groups(cfg2)[0]
    ref, _, scores = U.oracle_item(cfg2, case2.hi, case2.labels_np, l, 0, g)
    U.check_out(out2[l, 0, g * G:(g + 1) * G], ref, "second retrieval item vs oracle")
    U.check_index_set(idx2[l, 0, g], scores, cfg2.n_fac, "second retrieval idx vs oracle")


def test_noalloc_rejects_dims_beyond_the_fixed_scratch():
    """Too large for the array: HAS_ERR_WORKSPACE before any launch, the
    output untouched."""
    cfg = R.get_config("c1", batch=1, ctx_len=9000, n_fac=700)
    print("case noalloc oversize", flush=True)
    case = U.DeviceCase(cfg)
    big = U.dims_of(cfg, n_layers=32, batch=4, ctx_len=131072, n_fac=4096)
    assert H.sparse_decode_workspace(big) > H.NOALLOC_SCRATCH_BYTES
    out = torch.full((8,), 7.0, device="cuda")
    P = ctypes.c_void_p
    r = lib().sparse_decode_step_noalloc(ctypes.byref(big), P(case.q.data_ptr()), P(case.k.data_ptr()),
                                         P(case.v.data_ptr()), P(case.k_dom.data_ptr()), P(case.i_dom.data_ptr()),
                                         P(case.labels.data_ptr()), P(out.data_ptr()), None, None)
    assert r == 3 and "noalloc" in H.last_error()
    torch.cuda.synchronize()
    assert (out == 7.0).all()
