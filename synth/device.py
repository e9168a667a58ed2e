"""Device-side generation of whole key/value caches (same bits as the host
generator, see `recipe`).  PyTorch tensors serve as device buffers."""
import ctypes

import numpy as np

from . import host
from . import recipe as R


def _torch():
    import torch
    return torch


def to_device(a, device, bf16):
    """Host storage array -> device tensor (bf16 bits are reinterpreted)."""
    torch = _torch()
    if bf16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def kv_cache(cfg, kind, hi, device="cuda", stream=None):
    """[kv_layers, B, Hkv, T, d] post-RoPE keys (kind "k", needles planted) or
    values (kind "v") generated on the device."""
    torch = _torch()
    L, B, Hkv, T, d = cfg.kv_layers, cfg.batch, cfg.n_kv_heads, cfg.ctx_len, cfg.d_head
    dt = torch.bfloat16 if cfg.bf16 else torch.float32
    out = torch.empty((L, B, Hkv, T, d), dtype=dt, device=device)
    ids = np.array([R.kv_slice_id(cfg, l, b, g) for l in range(L) for b in range(B) for g in range(Hkv)],
                   dtype=np.int32)
    ids_d = torch.from_numpy(ids).to(device)
    if kind == "k":
        masks = np.stack([hi.masks[l, g] for l in range(L) for b in range(B) for g in range(Hkv)])
        masks_d = torch.from_numpy(np.ascontiguousarray(masks)).to(device)
        cs, sn = hi.tables
        cs_d = torch.from_numpy(cs).to(device)
        sn_d = torch.from_numpy(sn).to(device)
        args = (R.TID_K, 0, ctypes.c_void_p(masks_d.data_ptr()), R.OUTLIER_MUL, R.SINK_MUL,
                ctypes.c_void_p(cs_d.data_ptr()), ctypes.c_void_p(sn_d.data_ptr()))
    else:
        args = (R.TID_V, 1, None, 1.0, 1.0, None, None)
    tid, knd, om, omul, smul, csp, snp = args
    s = stream if stream is not None else torch.cuda.current_stream()
    err = host.lib().synth_kv_fill_device(cfg.seed, tid, knd, len(ids), T, d, ctypes.c_void_p(ids_d.data_ptr()),
                                          om, omul, smul, csp, snp, ctypes.c_void_p(out.data_ptr()),
                                          1 if cfg.bf16 else 0, ctypes.c_void_p(s.cuda_stream))
    if err != 0:
        raise RuntimeError(f"synth_kv_fill_device failed with hipError {err}")
    if kind == "k":
        for (l, g) in R.needle_groups(cfg):
            if l >= L:
                continue
            for b in range(B):
                pos = R.needle_positions(cfg, l, b, g)
                chans, vals = R.needle_values(cfg, l, b, g, hi.i_dom, hi.tables)
                v = to_device(vals, device, cfg.bf16)
                p = torch.from_numpy(pos).to(device)
                c = torch.from_numpy(chans).to(device)
                out[l, b, g][p[:, None], c[None, :]] = v[None, :].expand(len(pos), -1)
    torch.cuda.synchronize()
    return out
