"""Head-aware token-sparse decode attention for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libhas.so`` (C ABI in
``include/has.h``); this package is a thin ctypes binding with the same
names.  PyTorch tensors are used only as device buffers and for the current
HIP stream.
"""
from .binding import (  # noqa: F401
    HAS_BF16,
    HAS_F32,
    DecodeDims,
    HasError,
    fac_attend,
    fac_attend_workspace,
    aoh_label,
    aoh_label_workspace,
    kdom_pack,
    kv_append,
    kdom_row_elems,
    last_error,
    library_path,
    shared_index_decode,
    shared_index_workspace,
    sparse_decode_per_head_workspace,
    sparse_decode_step,
    sparse_decode_step_noalloc,
    NOALLOC_SCRATCH_BYTES,
    sparse_decode_step_per_head,
    sparse_decode_step_split,
    sparse_decode_workspace,
    sparse_selection_path,
    sparse_select,
    sparse_select_workspace,
    status_string,
    timing_collect,
    timing_enable,
)
from .labels_io import load_labels, save_labels  # noqa: F401,E402
