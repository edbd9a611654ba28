"""Fused input preparation on the GPU (KDA_FLAG_QK_L2NORM, KDA_FLAG_GATE_LOGSIGMOID) against the
float64 oracle composed with the same maps (oracle.kda_*_prepped).

Inputs are the seeded raw values: q, k ~ N(0, 1) unnormalised, and the gate x before logsigmoid.
"""
import numpy as np
import pytest

import kda_inputs as ki
import oracle
from kda_testutil import TOL, np_of, rel_err, to_gpu

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "d_init")


def _raw(dtype, lengths, H, dk, dv, norm=True, gate=True, gate_mu=3.0, gate_sd=1.0):
    """Raw q, k when the kernel normalises them (else the prepared ones), and the raw gate when it
    applies logsigmoid (else log alpha): the same seeded draw either way."""
    w = ki.small(dtype=dtype, lengths=lengths, H=H, dk=dk, dv=dv, gate_mu=gate_mu, gate_sd=gate_sd)
    inp = ki.make_inputs(w, with_grads=True, raw=True)
    prepared = ki.make_inputs(w, with_grads=True)
    if not norm:
        inp["q"], inp["k"] = prepared["q"], prepared["k"]
    if not gate:
        inp["log_alpha"] = prepared["log_alpha"]
    return inp, to_gpu(inp, dtype)


def _oracle_fwd(inp, norm, gate):
    return oracle.kda_fwd_prepped(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                                  init_state=inp["init_state"], qk_l2norm=norm, gate_logsigmoid=gate)


def _oracle_bwd(inp, norm, gate):
    return oracle.kda_bwd_prepped(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                                  inp["d_out"], init_state=inp["init_state"], d_final_state=inp["d_final_state"],
                                  qk_l2norm=norm, gate_logsigmoid=gate)


def _gpu_fwd(g, **kw):
    import gated_delta_rule_79_amd as kda
    return kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=g["init_state"],
                   cu_seqlens=g["cu_seqlens"], **kw)


def _gpu_bwd(g, **kw):
    import gated_delta_rule_79_amd as kda
    return kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                   d_final_state=g["d_final_state"], cu_seqlens=g["cu_seqlens"], **kw)


CASES = [("bf16", (300, 1, 129), 2, 128, 128), ("f32", (100, 64, 7), 2, 64, 64), ("bf16", (70, 200), 3, 64, 128),
         ("bf16", (150,), 2, 128, 64)]
IDS = ["bf16-128x128", "f32-64x64", "bf16-64x128", "bf16-128x64"]


@pytest.mark.parametrize("dtype,lengths,H,dk,dv", CASES, ids=IDS)
@pytest.mark.parametrize("norm,gate", [(True, True), (True, False), (False, True)], ids=["both", "norm", "gate"])
def test_prepped_forward_and_backward(dtype, lengths, H, dk, dv, norm, gate):
    import torch
    inp, g = _raw(dtype, lengths, H, dk, dv, norm, gate)
    o, fin = _gpu_fwd(g, qk_l2norm=norm, gate_logsigmoid=gate)
    torch.cuda.synchronize()
    ro, rf = _oracle_fwd(inp, norm, gate)
    eo, ef = rel_err(np_of(o)[0], ro), rel_err(np_of(fin), rf)
    errs = {"o": eo, "final_state": ef}
    if dtype == "bf16" or dk == 64:   # the fp32 backward exists for dk = 64
        grads = _gpu_bwd(g, qk_l2norm=norm, gate_logsigmoid=gate)
        torch.cuda.synchronize()
        ref = _oracle_bwd(inp, norm, gate)
        for n, a, b in zip(NAMES, grads, ref):
            errs[n] = rel_err(np_of(a)[0] if n != "d_init" else np_of(a), b)
    print({k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, bad


def test_prepped_saved_forward_matches_recompute():
    """fwd(save_for_backward) + bwd(use_saved) with the preparation flags == the recomputing bwd, bit for bit."""
    import torch
    import gated_delta_rule_79_amd as kda
    inp, g = _raw("bf16", (300, 1, 129), 2, 128, 128)
    flags = dict(qk_l2norm=True, gate_logsigmoid=True)
    ref = _gpu_bwd(g, **flags)
    ws = torch.empty(kda.workspace_bytes(1, g["q"].shape[1], 2, 128, 128, torch.bfloat16, num_seqs=3, backward=True,
                                         **flags), dtype=torch.uint8, device="cuda")
    _gpu_fwd(g, workspace=ws, save_for_backward=True, **flags)
    got = _gpu_bwd(g, workspace=ws, use_saved=True, **flags)
    torch.cuda.synchronize()
    for n, a, b in zip(NAMES, got, ref):
        assert torch.equal(a, b), n


def test_prepped_equals_plain_on_prepared_fp32_inputs():
    """fp32: preparing inside equals the plain kernels on inputs prepared beforehand (to fp32 rounding)."""
    import torch
    inp, g = _raw("f32", (100, 64, 7), 2, 64, 64)
    o1, f1 = _gpu_fwd(g, qk_l2norm=True, gate_logsigmoid=True)
    p = dict(g)
    p["q"] = g["q"] / torch.sqrt((g["q"] * g["q"]).sum(-1, keepdim=True) + 1e-6)
    p["k"] = g["k"] / torch.sqrt((g["k"] * g["k"]).sum(-1, keepdim=True) + 1e-6)
    p["log_alpha"] = torch.nn.functional.logsigmoid(g["log_alpha"])
    o2, f2 = _gpu_fwd(p)
    g1 = _gpu_bwd(g, qk_l2norm=True, gate_logsigmoid=True)
    g2 = _gpu_bwd(p)
    torch.cuda.synchronize()
    assert rel_err(np_of(o1), np_of(o2)) <= 1e-5
    assert rel_err(np_of(f1), np_of(f2)) <= 1e-5
    # dv, dbeta, d_init are with respect to the same quantities on both sides
    for i in (2, 4, 5):
        assert rel_err(np_of(g1[i]), np_of(g2[i])) <= 1e-5, NAMES[i]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prepped_decode(dtype):
    import torch
    import gated_delta_rule_79_amd as kda
    d = ki.decode_inputs(5, 4, 2, 128, 128, 6, dtype=dtype, seed=21, raw=True)
    idx = np.array([4, 0, -1, 2, 5], np.int32)
    nc = np.array([4, 1, 3, 0, 2], np.int32)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(d[n]).to("cuda", dt) for n in ("q", "k", "v", "log_alpha", "beta")}
    pool = torch.from_numpy(d["state_pool"]).cuda()
    o = kda.decode(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], pool, state_indices=torch.from_numpy(idx).cuda(),
                   num_commit=torch.from_numpy(nc).cuda(), qk_l2norm=True, gate_logsigmoid=True)
    torch.cuda.synchronize()
    ro, rpool = oracle.kda_decode_prepped(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_pool"],
                                          state_indices=idx, num_commit=nc)
    assert rel_err(np_of(o), ro) <= TOL[dtype]
    assert rel_err(np_of(pool), rpool) <= TOL[dtype]
