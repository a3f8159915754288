"""Copy a generated workload to device memory as torch tensors (no arithmetic)."""
from __future__ import annotations

import numpy as np


def upload(w, device="cuda") -> dict:
    import torch

    def bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)

    d = {"idx_q": bf16(w.idx_q), "ckeys": bf16(w.ckeys), "q": bf16(w.q), "k_scale": None, "v_scale": None}
    if w.kv_dtype == "bf16":
        d["k_cache"] = bf16(w.k_cache)
        d["v_cache"] = bf16(w.v_cache)
    else:
        d["k_cache"] = torch.from_numpy(np.ascontiguousarray(w.k_cache)).to(device).view(torch.float8_e4m3fn)
        d["v_cache"] = torch.from_numpy(np.ascontiguousarray(w.v_cache)).to(device).view(torch.float8_e4m3fn)
        d["k_scale"] = torch.from_numpy(w.k_scale.astype(np.float32)).to(device)
        d["v_scale"] = torch.from_numpy(w.v_scale.astype(np.float32)).to(device)
    return d
