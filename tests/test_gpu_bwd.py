"""GPU parity of the backward pass (HIP library vs the float64 oracle)."""
import numpy as np
import pytest

import kda_inputs as ki
from kda_testutil import TOL, gpu_bwd, gpu_fwd, np_of, oracle_bwd, oracle_fwd, rel_err, to_gpu

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "dlog_alpha", "dbeta", "d_init"]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_79_amd as kda
    kda.load_library()


def _check_bwd(w, units=None, note="", tol=None):
    import torch
    inp = ki.make_inputs(w, with_grads=True)
    g = to_gpu(inp, w.dtype)
    grads = gpu_bwd(g)
    torch.cuda.synchronize()
    ref = oracle_bwd(inp, units=units)
    tol = tol or TOL[w.dtype]
    errs = {}
    for name, a, b in zip(NAMES, grads, ref):
        ga = np_of(a)
        if name != "d_init":
            ga = ga[0]
        if units is not None:
            hs = sorted({h for _, h in units})
            ga, b = ga[:, hs], b[:, hs]
        errs[name] = rel_err(ga, b)
    print(f"{w.name}{note}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"gradient errors above {tol}: {bad}"
    return grads


SMALL = [
    ("f32", (100,), 2, 64, 64),
    ("f32", (64, 1, 130), 2, 64, 128),
    ("bf16", (100,), 2, 64, 64),
    ("bf16", (64, 1, 127), 2, 64, 128),
    ("bf16", (200,), 2, 128, 64),
    ("bf16", (63, 65, 0, 130, 17), 3, 128, 128),
]


@pytest.mark.parametrize("dtype,lengths,H,dk,dv", SMALL,
                         ids=[f"{s[0]}-{len(s[1])}seq-H{s[2]}-{s[3]}x{s[4]}" for s in SMALL])
def test_small(dtype, lengths, H, dk, dv):
    _check_bwd(ki.small(dtype=dtype, lengths=lengths, H=H, dk=dk, dv=dv))


def test_sharp_gate_no_init():
    _check_bwd(ki.small(dtype="bf16", lengths=(300, 5), H=2, dk=128, dv=128, gate_mu=0.0, gate_sd=2.5, init_sd=0.0))


def test_cfg4_full():
    """The full varlen workload on the GPU, every sequence and head against the oracle."""
    _check_bwd(ki.config(4))


def test_optional_state_grads():
    """d_final_state omitted == zeros; d_init_state may be skipped."""
    import torch
    import gated_delta_rule_79_amd as kda
    w = ki.small(dtype="bf16", lengths=(150, 70), H=2, dk=128, dv=128)
    g = to_gpu(ki.make_inputs(w, with_grads=True), "bf16")
    zero = torch.zeros_like(g["d_final_state"])
    a = kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                d_final_state=None, cu_seqlens=g["cu_seqlens"])
    b = kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                d_final_state=zero, cu_seqlens=g["cu_seqlens"], need_d_init=False)
    torch.cuda.synchronize()
    assert b[5] is None
    for x, y in zip(a[:5], b[:5]):
        assert torch.equal(x, y)


def test_deterministic():
    import torch
    w = ki.small(dtype="bf16", lengths=(700, 33, 400), H=4, dk=128, dv=128)
    g = to_gpu(ki.make_inputs(w, with_grads=True), "bf16")
    a = gpu_bwd(g)
    b = gpu_bwd(g)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bf16_gradients():
    """bf16 gradient outputs: error beyond their own rounding stays within the bound."""
    import torch
    w = ki.small(dtype="bf16", lengths=(300, 90), H=2, dk=128, dv=128)
    inp = ki.make_inputs(w, with_grads=True)
    g = to_gpu(inp, "bf16")
    grads = gpu_bwd(g, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle_bwd(inp)
    for name, a, b in zip(NAMES[:5], grads[:5], ref[:5]):
        assert a.dtype == torch.bfloat16
        ga = np_of(a)[0]
        rms = np.sqrt(np.mean(b * b))
        excess = np.max(np.maximum(np.abs(ga - b) - 2.0 ** -8 * np.abs(b), 0.0)) / rms
        print(f"bf16 {name}: excess {excess:.2e}")
        assert excess <= TOL["bf16"], name


def test_fp32_dk128_backward_not_supported():
    import gated_delta_rule_79_amd as kda
    w = ki.small(dtype="f32", lengths=(10,), H=1, dk=128, dv=64)
    g = to_gpu(ki.make_inputs(w, with_grads=True), "f32")
    with pytest.raises(kda.KdaError) as e:
        gpu_bwd(g)
    assert e.value.status == 2


def test_fp32_repeated_after_other_work():
    """fp32 gradients stay right on repeated calls with other kernels in between
    (guards against reads of LDS that only 2-byte operand paths fill)."""
    import torch
    wf = ki.small(dtype="f32", lengths=(100, 37), H=2, dk=64, dv=64)
    inp = ki.make_inputs(wf, with_grads=True)
    gf = to_gpu(inp, "f32")
    ref = oracle_bwd(inp)
    gb = to_gpu(ki.make_inputs(ki.small(dtype="bf16", lengths=(300,), H=2, dk=128, dv=128), with_grads=True), "bf16")
    for it in range(4):
        gpu_bwd(gb)
        grads = gpu_bwd(gf)
        torch.cuda.synchronize()
        errs = {n: rel_err(np_of(a)[0] if n != "d_init" else np_of(a), b) for n, a, b in zip(NAMES, grads, ref)}
        bad = {k: v for k, v in errs.items() if not v <= TOL["f32"]}
        assert not bad, f"call {it}: {bad}"


@pytest.mark.parametrize("dtype,lengths,H,dk,dv", [("bf16", (300, 1, 129), 2, 128, 128), ("f32", (100, 64), 2, 64, 64),
                                                   ("bf16", (70,), 3, 64, 128)],
                         ids=["bf16-128x128", "f32-64x64", "bf16-64x128"])
def test_saved_forward_matches_recompute(dtype, lengths, H, dk, dv):
    """fwd(save_for_backward) + bwd(use_saved) gives the recomputing bwd's gradients bit for bit,
    and an output within the parity bound."""
    import torch
    import gated_delta_rule_79_amd as kda
    w = ki.small(dtype=dtype, lengths=lengths, H=H, dk=dk, dv=dv)
    inp = ki.make_inputs(w, with_grads=True)
    g = to_gpu(inp, dtype)
    ref = gpu_bwd(g)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ws = torch.empty(kda.workspace_bytes(1, g["q"].shape[1], H, dk, dv, dt, num_seqs=len(lengths), backward=True),
                     dtype=torch.uint8, device="cuda")
    o, fin = kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=g["init_state"],
                     cu_seqlens=g["cu_seqlens"], workspace=ws, save_for_backward=True)
    got = kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                  d_final_state=g["d_final_state"], cu_seqlens=g["cu_seqlens"], workspace=ws, use_saved=True)
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, got, ref):
        assert torch.equal(a, b), name
    o_ref, f_ref = oracle_fwd(inp)
    assert rel_err(np_of(o)[0], o_ref) <= TOL[dtype]
    assert rel_err(np_of(fin), f_ref) <= TOL[dtype]
