"""Upload a generated workload to the GPU (torch is used for memory only)."""
from __future__ import annotations

import numpy as np
import torch

from . import (F32, TID_SW1, TID_SW2, TID_SW3, TID_W1, TID_W2, TID_W3, Workload,
               make_b, make_e, make_u, normal, weight_dtype)


def _to_dev(a: np.ndarray, dtype, device):
    if dtype == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _stack_to_device(w: Workload, shared: bool, device, experts_per_chunk: int = 8):
    """W1, W3 [E, d_ff, d] and W2 [E, d, d_ff] generated chunk by chunk into device tensors."""
    E = w.n_shared if shared else w.n_routed
    wd = weight_dtype(w)
    tdt = torch.float32 if wd == F32 else torch.bfloat16
    ndt = np.float32 if wd == F32 else np.uint16
    tids = (TID_SW1, TID_SW3, TID_SW2) if shared else (TID_W1, TID_W3, TID_W2)
    shapes = ((w.d_ff, w.d), (w.d_ff, w.d), (w.d, w.d_ff))
    stds = (1.0 / np.sqrt(w.d), 1.0 / np.sqrt(w.d), 1.0 / np.sqrt(w.d_ff))
    outs = []
    n = w.d_ff * w.d
    for tid, shp, std in zip(tids, shapes, stds):
        dst = torch.empty((E,) + shp, dtype=tdt, device=device)
        host = np.empty(experts_per_chunk * n, ndt)
        for e0 in range(0, E, experts_per_chunk):
            e1 = min(E, e0 + experts_per_chunk)
            buf = host[:(e1 - e0) * n]
            normal(w.seed, tid, e0 * n, (e1 - e0) * n, std, wd, out=buf)
            src = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16) if tdt == torch.bfloat16 \
                else torch.from_numpy(buf)
            dst[e0:e1].copy_(src.view((e1 - e0,) + shp), non_blocking=False)
        outs.append(dst)
    return tuple(outs)


def upload(w: Workload, device="cuda", with_bf16_weights: bool = True):
    """Generate the workload's tensors and place them on the device.

    Returns dict: u, e (act dtype), b (fp32), routed (w1, w3, w2), shared (w1, w3, w2) or None.
    FP8 codes are not made here (the library's quantisation call makes them)."""
    adt = torch.float32 if w.act == F32 else torch.bfloat16
    u = _to_dev(make_u(w), adt, device)
    e = _to_dev(make_e(w), adt, device)
    b = torch.from_numpy(make_b(w)).to(device)
    res = {"u": u, "e": e, "b": b, "routed": None, "shared": None}
    if with_bf16_weights:
        res["routed"] = _stack_to_device(w, False, device)
        res["shared"] = _stack_to_device(w, True, device) if w.n_shared > 0 else None
    return res
