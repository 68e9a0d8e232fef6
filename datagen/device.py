"""Copy seeded inputs (datagen.MoEInputs) into device tensors.

Plumbing only: bf16 bit patterns become torch.bfloat16 tensors, fp8 codes
torch.uint8, fp32 stays fp32.  Routed experts are generated on worker threads
and copied expert by expert into preallocated [N, ...] device tensors, so the
host never holds all of a large layer at once.
"""
from __future__ import annotations

import numpy as np
import torch

from . import MoEInputs


def to_torch(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def upload(inp: MoEInputs, device="cuda", experts=True, shared=True) -> dict:
    cfg = inp.cfg
    dev = torch.device(device)
    out = dict(x=to_torch(inp.x(), dev), w_r=to_torch(inp.router_w(), dev))
    b = inp.router_b()
    out["b"] = None if b is None else to_torch(b, dev)
    if experts:
        first = inp.expert(0)
        ex = {}
        for key, v in first.items():
            if v is None:
                ex[key] = None
                continue
            tdt = {np.uint16: torch.bfloat16, np.uint8: torch.uint8, np.float32: torch.float32}[v.dtype.type]
            ex[key] = torch.empty((cfg.n_routed,) + v.shape, dtype=tdt, device=dev)

        def sink(e, d):
            for key, v in d.items():
                if v is not None:
                    ex[key][e].copy_(to_torch(v, "cpu"))

        inp.experts_stacked(sink=sink)
        out["experts"] = ex
    if shared and cfg.n_shared > 0:
        sh = inp.shared()
        out["shared"] = {k: (None if v is None else to_torch(v, dev)) for k, v in sh.items()}
    else:
        out["shared"] = None
    torch.cuda.synchronize(dev)
    return out
