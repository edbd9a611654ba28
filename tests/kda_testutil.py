"""Helpers shared by the GPU parity tests: move seeded inputs to the GPU,
call the HIP library and the float64 oracle, and measure the error.

Error metric (per output tensor): max |gpu - oracle| / rms(oracle), computed
in float64 over the whole tensor.  Bounds: 1e-4 for the fp32 path, 2e-2 for
bf16 storage with fp32 accumulation.
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_gpu(inp: dict, dtype: str, device="cuda"):
    """Seeded numpy inputs -> torch tensors in the storage dtype (values are exact)."""
    import torch
    dt = torch_dtype(dtype)
    out = {}
    for key in ("q", "k", "v", "log_alpha", "beta", "d_out"):
        if key in inp and inp[key] is not None:
            out[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to(device=device, dtype=dt).unsqueeze(0)
    for key in ("init_state", "d_final_state"):
        if key in inp and inp[key] is not None:
            out[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to(device=device, dtype=torch.float32)
        else:
            out[key] = None
    out["cu_seqlens"] = torch.from_numpy(inp["cu_seqlens"]).to(device=device, dtype=torch.int32)
    return out


def rel_err(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if r.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(r * r))
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.max(np.abs(g - r)) / max(rms, 1e-300))


def oracle_fwd(inp: dict, units=None, scale=None):
    return oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                          init_state=inp.get("init_state"), scale=scale, units=units)


def oracle_bwd(inp: dict, units=None, scale=None):
    return oracle.kda_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                          inp["d_out"], init_state=inp.get("init_state"), d_final_state=inp.get("d_final_state"),
                          scale=scale, units=units)


def gpu_fwd(g: dict, varlen=True, **kw):
    import gated_delta_rule_79_amd as kda
    o, f = kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=g["init_state"],
                   cu_seqlens=g["cu_seqlens"] if varlen else None, **kw)
    return o, f


def gpu_bwd(g: dict, varlen=True, **kw):
    import gated_delta_rule_79_amd as kda
    return kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                   d_final_state=g["d_final_state"], cu_seqlens=g["cu_seqlens"] if varlen else None, **kw)


def np_of(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()
