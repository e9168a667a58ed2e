"""ctypes access to the host half of libsynth (the counter-based generator)."""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        u32, u64, i32, i64 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int, ctypes.c_int64
        L.synth_philox4x32_10.argtypes = [P, P, P]
        L.synth_ih.argtypes = [u32, u32, u32, u64, i64, P]
        L.synth_u32.argtypes = [u32, u32, u32, u64, i64, P]
        L.synth_bf16_rne.argtypes = [P, i64, P]
        L.synth_rope_table.argtypes = [i32, i32, ctypes.c_double, P, P]
        L.synth_rope_apply.argtypes = [P, i64, i32, i32, P, P, P]
        L.synth_kv_rows.argtypes = [u32, u32, u32, i32, i32, i32, i32, P, ctypes.c_float,
                                    ctypes.c_float, P, P, P]
        L.synth_kv_fill_device.argtypes = [u32, u32, i32, i32, i32, i32, P, P, ctypes.c_float,
                                           ctypes.c_float, P, P, P, i32, P]
        L.synth_kv_fill_device.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def philox(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_p(c), _p(k), _p(o))
    return o


def ih(seed, tid, slice_, e0, n):
    out = np.empty(int(n), dtype=np.float32)
    lib().synth_ih(seed, tid, slice_, e0, int(n), _p(out))
    return out


def u32(seed, tid, slice_, e0, n):
    out = np.empty(int(n), dtype=np.uint32)
    lib().synth_u32(seed, tid, slice_, e0, int(n), _p(out))
    return out


def bf16_rne(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().synth_bf16_rne(_p(x), x.size, _p(out))
    return out


def rope_table(T, d, base):
    cs = np.empty((T, d // 2), dtype=np.float32)
    sn = np.empty((T, d // 2), dtype=np.float32)
    lib().synth_rope_table(T, d, float(base), _p(cs), _p(sn))
    return cs, sn


def rope_apply(x, pos, cs, sn):
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[-1]
    y = np.empty_like(x)
    lib().synth_rope_apply(_p(x), x.size // d, d, int(pos), _p(cs), _p(sn), _p(y))
    return y


def kv_rows(seed, tid, slice_, kind, d, t0, t1, outlier_mask, outlier_mul, sink_mul, cs, sn):
    out = np.empty((t1 - t0, d), dtype=np.float32)
    om = None if outlier_mask is None else np.ascontiguousarray(outlier_mask, dtype=np.uint8)
    lib().synth_kv_rows(seed, tid, slice_, kind, d, t0, t1, _p(om), outlier_mul, sink_mul,
                        _p(cs), _p(sn), _p(out))
    return out
