"""GPU parity of the forward pass (HIP library vs the float64 oracle)."""
import numpy as np
import pytest

import kda_inputs as ki
from kda_testutil import TOL, gpu_fwd, np_of, oracle_fwd, rel_err, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_79_amd as kda
    kda.load_library()


def _check_fwd(w, units=None, note=""):
    inp = ki.make_inputs(w)
    g = to_gpu(inp, w.dtype)
    o, f = gpu_fwd(g)
    import torch
    torch.cuda.synchronize()
    ro, rf = oracle_fwd(inp, units=units)
    go, gf = np_of(o)[0], np_of(f)
    if units is not None:
        hs = sorted({h for _, h in units})
        ro, go = ro[:, hs], go[:, hs]
        rf, gf = rf[:, hs], gf[:, hs]
    eo, ef = rel_err(go, ro), rel_err(gf, rf)
    print(f"{w.name}{note}: err(o)={eo:.3e} err(final)={ef:.3e}")
    tol = TOL[w.dtype]
    assert eo <= tol, f"output error {eo:.3e} > {tol}"
    assert ef <= tol, f"final-state error {ef:.3e} > {tol}"
    return o, f


def test_cfg0_fp32():
    _check_fwd(ki.config(0))


SMALL = [
    ("f32", (100,), 2, 64, 64),
    ("f32", (64,), 1, 64, 128),
    ("f32", (1,), 3, 128, 64),
    ("f32", (63, 65, 0, 130), 2, 128, 128),
    ("bf16", (100,), 2, 64, 64),
    ("bf16", (64, 1, 127), 2, 64, 128),
    ("bf16", (200,), 2, 128, 64),
    ("bf16", (63, 65, 0, 130, 17), 3, 128, 128),
]


@pytest.mark.parametrize("dtype,lengths,H,dk,dv", SMALL, ids=[f"{s[0]}-{len(s[1])}seq-H{s[2]}-{s[3]}x{s[4]}" for s in SMALL])
def test_small(dtype, lengths, H, dk, dv):
    _check_fwd(ki.small(dtype=dtype, lengths=lengths, H=H, dk=dk, dv=dv, backward=False))


def test_small_sharp_gate_no_init():
    _check_fwd(ki.small(dtype="bf16", lengths=(300, 5), H=2, dk=128, dv=128, gate_mu=0.0, gate_sd=2.5,
                        init_sd=0.0, backward=False))


def test_cfg1_full():
    _check_fwd(ki.config(1))


def test_cfg2_full():
    """32,768 tokens, sharper gate, all 16 heads (the oracle runs one head per host thread)."""
    _check_fwd(ki.config(2))


def test_cfg3_full():
    """One 131,072-token sequence, all 16 heads."""
    _check_fwd(ki.config(3))


def test_cfg4_forward_full():
    """The 8-sequence varlen workload (159,285 tokens), every sequence and head."""
    _check_fwd(ki.config(4))


def test_batched_rows_equal_varlen():
    """B rows without cu_seqlens == the same rows packed with cu_seqlens."""
    import torch
    import gated_delta_rule_79_amd as kda
    w = ki.small(dtype="bf16", lengths=(150, 150, 150), H=2, dk=128, dv=128, backward=False)
    g = to_gpu(ki.make_inputs(w), "bf16")
    o1, f1 = gpu_fwd(g)
    rs = {k: (v.reshape(3, 150, *v.shape[2:]) if k in ("q", "k", "v", "log_alpha", "beta") else v)
          for k, v in g.items()}
    o2, f2 = kda.fwd(rs["q"], rs["k"], rs["v"], rs["log_alpha"], rs["beta"], init_state=rs["init_state"])
    torch.cuda.synchronize()
    assert torch.equal(o1.reshape(o2.shape), o2)
    assert torch.equal(f1, f2)


def test_chaining_through_final_state():
    """Two calls chained through final_state -> init_state match one call."""
    import torch
    import gated_delta_rule_79_amd as kda
    w = ki.small(dtype="f32", lengths=(256,), H=2, dk=64, dv=64, backward=False)
    g = to_gpu(ki.make_inputs(w), "f32")
    o, f = gpu_fwd(g)
    cut = 128  # on a chunk boundary the two runs do the same arithmetic
    a = {k: (v[:, :cut] if k in ("q", "k", "v", "log_alpha", "beta") else v) for k, v in g.items()}
    b = {k: (v[:, cut:].contiguous() if k in ("q", "k", "v", "log_alpha", "beta") else v) for k, v in g.items()}
    oa, fa = kda.fwd(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], init_state=g["init_state"])
    ob, fb = kda.fwd(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], init_state=fa)
    torch.cuda.synchronize()
    assert torch.allclose(torch.cat([oa, ob], 1), o, rtol=0, atol=1e-5)
    assert torch.allclose(fb, f, rtol=0, atol=1e-5)


def test_deterministic():
    """Fixed inputs give bitwise identical outputs run to run."""
    import torch
    w = ki.small(dtype="bf16", lengths=(1000, 37, 2000), H=4, dk=128, dv=128, backward=False)
    g = to_gpu(ki.make_inputs(w), "bf16")
    o1, f1 = gpu_fwd(g)
    o2, f2 = gpu_fwd(g)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_final_state_optional_and_alias():
    """final_state may be omitted, or may alias init_state."""
    import torch
    import gated_delta_rule_79_amd as kda
    w = ki.small(dtype="bf16", lengths=(90, 40), H=2, dk=64, dv=64, backward=False)
    g = to_gpu(ki.make_inputs(w), "bf16")
    o, f = gpu_fwd(g)
    o2, none = gpu_fwd(g, output_final_state=False)
    st = g["init_state"].clone()
    o3, f3 = kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=st, cu_seqlens=g["cu_seqlens"],
                     final_state=st)
    torch.cuda.synchronize()
    assert none is None and torch.equal(o, o2)
    assert torch.equal(o, o3) and torch.equal(f, st)


def test_bf16_output_dtype():
    """bf16 outputs: the error beyond the output's own rounding (half a bf16 ulp,
    2^-8 relative) stays within the bf16-path bound."""
    import torch
    w = ki.small(dtype="bf16", lengths=(300, 100), H=2, dk=128, dv=128, backward=False)
    inp = ki.make_inputs(w)
    g = to_gpu(inp, "bf16")
    o, f = gpu_fwd(g, out_dtype=torch.bfloat16)
    o32, f32_ = gpu_fwd(g)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    ro, rf = oracle_fwd(inp)
    go = np_of(o)[0]
    rms = np.sqrt(np.mean(ro * ro))
    excess = np.max(np.maximum(np.abs(go - ro) - 2.0 ** -8 * np.abs(ro), 0.0)) / rms
    print(f"bf16 out: excess error {excess:.3e}")
    assert excess <= TOL["bf16"]
    assert torch.equal(f, f32_)  # the state does not depend on the output dtype
