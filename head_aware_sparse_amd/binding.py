"""ctypes binding of libhas.so: argument marshalling only.

Every function takes PyTorch tensors that already live on the GPU, checks
their dtype, shape and contiguity, and passes raw device pointers and the
current HIP stream to the C entry point of the same name.  The library
itself validates again and returns a status; a non-OK status raises
HasError with the library's message.  If the library is not built the
import of any entry point fails loudly: there is no fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhas.so")
_lib = None

HAS_F32, HAS_BF16 = 0, 1
HAS_ROPE_ROTATE_HALF, HAS_ROPE_INTERLEAVED = 0, 1
_FIELDS = ["n_layers", "batch", "n_q_heads", "n_kv_heads", "d_head", "ctx_len", "n_fac", "n_sink",
           "window", "n_dom", "kv_dtype", "rope_layout"]


class DecodeDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in _FIELDS]

    def __repr__(self):
        return "DecodeDims(" + ", ".join(f"{n}={getattr(self, n)}" for n in _FIELDS) + ")"


class HasError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


def library_path():
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        DP = ctypes.POINTER(DecodeDims)
        L.has_status_string.argtypes = [I]
        L.has_status_string.restype = ctypes.c_char_p
        L.has_last_error.argtypes = []
        L.has_last_error.restype = ctypes.c_char_p
        L.kdom_row_elems.argtypes = [DP]
        L.kdom_row_elems.restype = I
        L.kdom_pack.argtypes = [DP, P, P, P, P]
        L.kdom_pack.restype = I
        L.sparse_decode_workspace.argtypes = [DP]
        L.sparse_decode_workspace.restype = S
        L.sparse_selection_path.argtypes = [DP]
        L.sparse_selection_path.restype = I
        L.sparse_decode_step.argtypes = [DP, P, P, P, P, P, P, P, P, P, S, P]
        L.sparse_decode_step.restype = I
        L.sparse_decode_step_noalloc.argtypes = [DP, P, P, P, P, P, P, P, P, P]
        L.sparse_decode_step_noalloc.restype = I
        L.shared_index_workspace.argtypes = [DP]
        L.shared_index_workspace.restype = S
        L.shared_index_decode.argtypes = [DP, P, P, P, P, P, P, P, P, P, P, S, P]
        L.shared_index_decode.restype = I
        L.sparse_decode_per_head_workspace.argtypes = [DP]
        L.sparse_decode_per_head_workspace.restype = S
        L.sparse_decode_step_per_head.argtypes = [DP, P, P, P, P, P, P, P, P, P, S, P]
        L.sparse_decode_step_per_head.restype = I
        L.kv_append.argtypes = [DP, I, I, I, P, P, P, P, P, P, P, P, P, P]
        L.kv_append.restype = I
        L.sparse_decode_step_split.argtypes = [DP, I, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.sparse_decode_step_split.restype = I
        L.sparse_select_workspace.argtypes = [DP]
        L.sparse_select_workspace.restype = S
        L.sparse_select.argtypes = [DP, P, P, P, P, P, S, P]
        L.sparse_select.restype = I
        L.fac_attend_workspace.argtypes = [DP]
        L.fac_attend_workspace.restype = S
        L.fac_attend.argtypes = [DP, P, P, P, P, P, P, S, P]
        L.fac_attend.restype = I
        L.aoh_label_workspace.argtypes = [I, I, I, I, I]
        L.aoh_label_workspace.restype = S
        L.aoh_label.argtypes = [I, I, I, I, I, I, P, P, I, ctypes.c_float, P, P, P, P, S, P]
        L.aoh_label.restype = I
        _lib = L
    return _lib


def status_string(s):
    return lib().has_status_string(int(s)).decode()


def last_error():
    return lib().has_last_error().decode()


def _check(status):
    if status != 0:
        raise HasError(status, last_error())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _kv_torch_dtype(dims):
    import torch
    return torch.bfloat16 if dims.kv_dtype == HAS_BF16 else torch.float32


def kdom_row_elems(dims):
    r = lib().kdom_row_elems(ctypes.byref(dims))
    if r < 0:
        raise HasError(1, last_error())
    return r


def sparse_decode_workspace(dims):
    return int(lib().sparse_decode_workspace(ctypes.byref(dims)))


def sparse_selection_path(dims):
    """1 if sparse_decode_step selects through the sampled prefilter, 0 if
    through the general radix path (host only)."""
    r = lib().sparse_selection_path(ctypes.byref(dims))
    if r < 0:
        raise HasError(1, last_error())
    return r


def shared_index_workspace(dims):
    return int(lib().shared_index_workspace(ctypes.byref(dims)))


def sparse_select_workspace(dims):
    return int(lib().sparse_select_workspace(ctypes.byref(dims)))


def fac_attend_workspace(dims):
    return int(lib().fac_attend_workspace(ctypes.byref(dims)))


def aoh_label_workspace(n_layers, n_q_heads, n_kv_heads, d_model, d_head):
    return int(lib().aoh_label_workspace(n_layers, n_q_heads, n_kv_heads, d_model, d_head))


def _workspace(nbytes, ws, like, stream=None):
    """The caller's workspace, or a new one.  A new one is allocated on the
    stream the library enqueues on, so that the caching allocator does not
    hand its memory to another tensor while that stream's kernels still use
    it (also when the caller drops the returned tensor)."""
    import torch
    if ws is None:
        if stream is not None:
            with torch.cuda.stream(stream):
                ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device)
        else:
            ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device)
    _dev(ws, "ws", torch.uint8)
    return ws


def kdom_pack(dims, k_cache, i_dom, k_dom, stream=None):
    import torch
    L, B, Hkv, T, d = dims.n_layers, dims.batch, dims.n_kv_heads, dims.ctx_len, dims.d_head
    dt = _kv_torch_dtype(dims)
    _dev(k_cache, "k_cache", dt, (L, B, Hkv, T, d))
    _dev(i_dom, "i_dom", torch.int32, (L, Hkv, dims.n_dom))
    _dev(k_dom, "k_dom", dt, (L, B, Hkv, T, kdom_row_elems(dims)))
    _check(lib().kdom_pack(ctypes.byref(dims), _ptr(k_cache), _ptr(i_dom), _ptr(k_dom), _stream(stream)))


def sparse_decode_step(dims, q, k_cache, v_cache, k_dom, i_dom, labels, out, idx_out=None, ws=None,
                       stream=None):
    import torch
    L, B, Hq, Hkv, T, d = (dims.n_layers, dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.ctx_len,
                           dims.d_head)
    dt = _kv_torch_dtype(dims)
    _dev(q, "q", dt, (L, B, Hq, d))
    _dev(k_cache, "k_cache", dt, (L, B, Hkv, T, d))
    _dev(v_cache, "v_cache", dt, (L, B, Hkv, T, d))
    _dev(k_dom, "k_dom", dt, (L, B, Hkv, T, kdom_row_elems(dims)))
    _dev(i_dom, "i_dom", torch.int32, (L, Hkv, dims.n_dom))
    _dev(labels, "labels", torch.uint8, (L, Hkv))
    _dev(out, "out", torch.float32, (L, B, Hq, d))
    _dev(idx_out, "idx_out", torch.int32, (L, B, Hkv, dims.n_fac))
    nbytes = sparse_decode_workspace(dims)
    ws = _workspace(nbytes, ws, q, stream)
    _check(lib().sparse_decode_step(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_dom),
                                    _ptr(i_dom), _ptr(labels), _ptr(out), _ptr(idx_out), _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return ws


NOALLOC_SCRATCH_BYTES = 64 << 20  # HAS_NOALLOC_SCRATCH_BYTES of has.h


def sparse_decode_step_noalloc(dims, q, k_cache, v_cache, k_dom, i_dom, labels, out, idx_out=None, stream=None):
    """sparse_decode_step without a workspace: the library's fixed per-device
    scratch serves instead (nothing is allocated here or in the library)."""
    import torch
    L, B, Hq, Hkv, T, d = (dims.n_layers, dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.ctx_len,
                           dims.d_head)
    dt = _kv_torch_dtype(dims)
    _dev(q, "q", dt, (L, B, Hq, d))
    _dev(k_cache, "k_cache", dt, (L, B, Hkv, T, d))
    _dev(v_cache, "v_cache", dt, (L, B, Hkv, T, d))
    _dev(k_dom, "k_dom", dt, (L, B, Hkv, T, kdom_row_elems(dims)))
    _dev(i_dom, "i_dom", torch.int32, (L, Hkv, dims.n_dom))
    _dev(labels, "labels", torch.uint8, (L, Hkv))
    _dev(out, "out", torch.float32, (L, B, Hq, d))
    _dev(idx_out, "idx_out", torch.int32, (L, B, Hkv, dims.n_fac))
    _check(lib().sparse_decode_step_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_dom),
                                            _ptr(i_dom), _ptr(labels), _ptr(out), _ptr(idx_out), _stream(stream)))


def sparse_decode_per_head_workspace(dims):
    return int(lib().sparse_decode_per_head_workspace(ctypes.byref(dims)))


def sparse_decode_step_per_head(dims, q, k_cache, v_cache, k_dom, i_dom, labels, out, idx_out=None, ws=None,
                                stream=None):
    import torch
    L, B, Hq, Hkv, T, d = (dims.n_layers, dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.ctx_len,
                           dims.d_head)
    dt = _kv_torch_dtype(dims)
    _dev(q, "q", dt, (L, B, Hq, d))
    _dev(k_cache, "k_cache", dt, (L, B, Hkv, T, d))
    _dev(v_cache, "v_cache", dt, (L, B, Hkv, T, d))
    _dev(k_dom, "k_dom", dt, (L, B, Hkv, T, kdom_row_elems(dims)))
    _dev(i_dom, "i_dom", torch.int32, (L, Hkv, dims.n_dom))
    _dev(labels, "labels", torch.uint8, (L, Hkv))
    _dev(out, "out", torch.float32, (L, B, Hq, d))
    _dev(idx_out, "idx_out", torch.int32, (L, B, Hq, dims.n_fac))
    nbytes = sparse_decode_per_head_workspace(dims)
    ws = _workspace(nbytes, ws, q, stream)
    _check(lib().sparse_decode_step_per_head(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                             _ptr(k_dom), _ptr(i_dom), _ptr(labels), _ptr(out), _ptr(idx_out),
                                             _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def shared_index_decode(dims, q, k_cache, v_cache, k_dom, i_dom, out, q_index=None, labels=None,
                        idx_out=None, ws=None, stream=None):
    import torch
    N, B, Hq, Hkv, T, d = (dims.n_layers, dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.ctx_len,
                           dims.d_head)
    dt = _kv_torch_dtype(dims)
    _dev(q, "q", dt, (N, B, Hq, d))
    _dev(q_index, "q_index", dt, (B, Hq, d))
    _dev(k_cache, "k_cache", dt, (B, Hkv, T, d))
    _dev(v_cache, "v_cache", dt, (B, Hkv, T, d))
    _dev(k_dom, "k_dom", dt, (B, Hkv, T, kdom_row_elems(dims)))
    _dev(i_dom, "i_dom", torch.int32, (Hkv, dims.n_dom))
    _dev(labels, "labels", torch.uint8, (N, Hkv))
    _dev(out, "out", torch.float32, (N, B, Hq, d))
    _dev(idx_out, "idx_out", torch.int32, (B, Hkv, dims.n_fac))
    nbytes = shared_index_workspace(dims)
    ws = _workspace(nbytes, ws, q, stream)
    _check(lib().shared_index_decode(ctypes.byref(dims), _ptr(q), _ptr(q_index), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(k_dom), _ptr(i_dom), _ptr(labels), _ptr(out), _ptr(idx_out), _ptr(ws),
                                     ws.numel(), _stream(stream)))
    return ws


_dummy = {}


def _ptr_nonempty(t):
    """A device pointer for t; a 16-byte placeholder when t is empty (no
    pair of that kind: the kernels never touch it)."""
    if t.numel() > 0:
        return _ptr(t)
    import torch
    key = t.device
    if key not in _dummy:
        _dummy[key] = torch.zeros(16, dtype=torch.uint8, device=t.device)
    return _ptr(_dummy[key])


def _split_capacity(dims, k_ret, v_ret, k_dom_ret, k_str, v_str):
    """Checks a split cache's tensors against dims; returns its capacity."""
    B, Hkv, d = dims.batch, dims.n_kv_heads, dims.d_head
    dt = _kv_torch_dtype(dims)
    if k_ret.dim() != 4:
        raise ValueError("k_ret must be [n_ret, batch, capacity, d_head]")
    n_ret, cap = k_ret.shape[0], k_ret.shape[2]
    if cap < 1:
        raise ValueError("k_ret's capacity (dim 2) must be >= 1, also with no retrieval pair")
    n_str = dims.n_layers * Hkv - n_ret
    for t, name in ((k_ret, "k_ret"), (v_ret, "v_ret")):  # device, or pinned host memory
        if t.device.type == "cpu" and t.numel() > 0 and not t.is_pinned():
            raise ValueError(f"{name} on the host must be pinned memory")
        if t.device.type == "cpu":
            if not t.is_contiguous() or t.dtype != dt or tuple(t.shape) != (n_ret, B, cap, d):
                raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {(n_ret, B, cap, d)}")
        else:
            _dev(t, name, dt, (n_ret, B, cap, d))
    _dev(k_dom_ret, "k_dom_ret", dt, (n_ret, B, cap, kdom_row_elems(dims)))
    _dev(k_str, "k_str", dt, (n_str, B, dims.n_sink + dims.window, d))
    _dev(v_str, "v_str", dt, (n_str, B, dims.n_sink + dims.window, d))
    return cap


def kv_append(dims, pos, k_new, v_new, i_dom, labels, k_ret, v_ret, k_dom_ret, k_str, v_str, stream=None):
    import torch
    L, B, Hkv, d = dims.n_layers, dims.batch, dims.n_kv_heads, dims.d_head
    dt = _kv_torch_dtype(dims)
    if k_new.dim() != 5:
        raise ValueError("k_new must be [n_layers, batch, n_kv_heads, n_new, d_head]")
    n_new = k_new.shape[3]
    _dev(k_new, "k_new", dt, (L, B, Hkv, n_new, d))
    _dev(v_new, "v_new", dt, (L, B, Hkv, n_new, d))
    _dev(i_dom, "i_dom", torch.int32, (L, Hkv, dims.n_dom))
    _dev(labels, "labels", torch.uint8, (L, Hkv))
    cap = _split_capacity(dims, k_ret, v_ret, k_dom_ret, k_str, v_str)
    _check(lib().kv_append(ctypes.byref(dims), cap, pos, n_new, _ptr(k_new), _ptr(v_new), _ptr(i_dom), _ptr(labels),
                           _ptr_nonempty(k_ret), _ptr_nonempty(v_ret), _ptr_nonempty(k_dom_ret),
                           _ptr_nonempty(k_str), _ptr_nonempty(v_str), _stream(stream)))


def sparse_decode_step_split(dims, q, k_ret, v_ret, k_dom_ret, k_str, v_str, i_dom, labels, out, idx_out=None,
                             ws=None, stream=None):
    import torch
    L, B, Hq, Hkv, d = dims.n_layers, dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.d_head
    dt = _kv_torch_dtype(dims)
    _dev(q, "q", dt, (L, B, Hq, d))
    _dev(i_dom, "i_dom", torch.int32, (L, Hkv, dims.n_dom))
    _dev(labels, "labels", torch.uint8, (L, Hkv))
    _dev(out, "out", torch.float32, (L, B, Hq, d))
    _dev(idx_out, "idx_out", torch.int32, (L, B, Hkv, dims.n_fac))
    cap = _split_capacity(dims, k_ret, v_ret, k_dom_ret, k_str, v_str)
    nbytes = sparse_decode_workspace(dims)
    ws = _workspace(nbytes, ws, q, stream)
    _check(lib().sparse_decode_step_split(ctypes.byref(dims), cap, _ptr(q), _ptr_nonempty(k_ret),
                                          _ptr_nonempty(v_ret), _ptr_nonempty(k_dom_ret), _ptr_nonempty(k_str),
                                          _ptr_nonempty(v_str), _ptr(i_dom), _ptr(labels),
                                          _ptr(out), _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def sparse_select(dims, q_index, k_dom, i_dom, idx_out, ws=None, stream=None):
    import torch
    B, Hq, Hkv, T, d = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.ctx_len, dims.d_head
    dt = _kv_torch_dtype(dims)
    _dev(q_index, "q_index", dt, (B, Hq, d))
    _dev(k_dom, "k_dom", dt, (B, Hkv, T, kdom_row_elems(dims)))
    _dev(i_dom, "i_dom", torch.int32, (Hkv, dims.n_dom))
    _dev(idx_out, "idx_out", torch.int32, (B, Hkv, dims.n_fac))
    nbytes = sparse_select_workspace(dims)
    ws = _workspace(nbytes, ws, q_index, stream)
    _check(lib().sparse_select(ctypes.byref(dims), _ptr(q_index), _ptr(k_dom), _ptr(i_dom), _ptr(idx_out),
                               _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def fac_attend(dims, q, k_cache, v_cache, idx, out, ws=None, stream=None):
    import torch
    B, Hq, Hkv, T, d = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.ctx_len, dims.d_head
    dt = _kv_torch_dtype(dims)
    _dev(q, "q", dt, (B, Hq, d))
    _dev(k_cache, "k_cache", dt, (B, Hkv, T, d))
    _dev(v_cache, "v_cache", dt, (B, Hkv, T, d))
    _dev(idx, "idx", torch.int32, (B, Hkv, dims.n_fac))
    _dev(out, "out", torch.float32, (B, Hq, d))
    nbytes = fac_attend_workspace(dims)
    ws = _workspace(nbytes, ws, q, stream)
    _check(lib().fac_attend(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(idx), _ptr(out),
                            _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def aoh_label(w_q, w_k, n_q_heads, n_kv_heads, d_head, labels, n_retrieval=-1, er_threshold=0.0,
              er_head=None, er_group=None, ws=None, stream=None):
    import torch
    if w_q.dtype == torch.bfloat16:
        wdt = HAS_BF16
    elif w_q.dtype == torch.float32:
        wdt = HAS_F32
    else:
        raise ValueError("weights must be bfloat16 or float32")
    L, rows, d_model = w_q.shape
    _dev(w_q, "w_q", w_q.dtype, (L, n_q_heads * d_head, d_model))
    _dev(w_k, "w_k", w_q.dtype, (L, n_kv_heads * d_head, d_model))
    _dev(labels, "labels", torch.uint8, (L, n_kv_heads))
    _dev(er_head, "er_head", torch.float32, (L, n_q_heads))
    _dev(er_group, "er_group", torch.float32, (L, n_kv_heads))
    nbytes = aoh_label_workspace(L, n_q_heads, n_kv_heads, d_model, d_head)
    ws = _workspace(nbytes, ws, w_q, stream)
    _check(lib().aoh_label(L, n_q_heads, n_kv_heads, d_model, d_head, wdt, _ptr(w_q), _ptr(w_k), int(n_retrieval),
                           float(er_threshold), _ptr(er_head), _ptr(er_group), _ptr(labels), _ptr(ws), ws.numel(),
                           _stream(stream)))
    return ws


def timing_enable(on=True):
    L = lib()
    L.has_timing_enable.argtypes = [ctypes.c_int]
    L.has_timing_enable.restype = ctypes.c_int
    _check(L.has_timing_enable(1 if on else 0))


def timing_collect(max_kernels=32):
    """{kernel name: (total_ms, launches)} of the launches recorded since the
    last collect."""
    L = lib()
    L.has_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int), ctypes.c_int]
    L.has_timing_collect.restype = ctypes.c_int
    names = (ctypes.c_char_p * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int * max_kernels)()
    n = L.has_timing_collect(names, ms, cnt, max_kernels)
    if n < 0:
        raise HasError(4, last_error())
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(n)}
