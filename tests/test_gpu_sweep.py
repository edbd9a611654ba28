"""A seeded sweep of random problems against the float64 oracle: packed batches of 1-5 sequences
(0-700 tokens each, so empty, one-token and ragged tails all occur), H 1-3, every (dk, dv) pair,
bf16 and fp32 inputs, gates from gentle to sharp, hard-forget channels, with and without
init_state and d_final_state, the fused preparation flags, and the training-mode pair of calls.
Every output and gradient must meet the same bound as the fixed cases (for fp32 inputs with
hard-forget channels, the derived bound of test_gpu_robustness)."""
import numpy as np
import pytest

import kda_inputs as ki
import oracle
from kda_testutil import TOL, np_of, rel_err, to_gpu
from test_gpu_robustness import _hard_forget, _hard_tol

pytestmark = pytest.mark.gpu

GRADS = ["dq", "dk", "dv", "dlog_alpha", "dbeta", "d_init"]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_79_amd as kda
    kda.load_library()


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    dtype = "bf16" if r.random() < 0.7 else "f32"
    dk = int(r.choice([64, 128])) if dtype == "bf16" else 64   # the fp32 backward exists for dk = 64
    dv = int(r.choice([64, 128]))
    n = int(r.integers(1, 6))
    lengths = tuple(int(x) for x in r.choice([0, 1, int(r.integers(2, 64)), int(r.integers(64, 700))], size=n))
    if sum(lengths) == 0:
        lengths = lengths[:-1] + (int(r.integers(1, 300)),)
    return dict(dtype=dtype, dk=dk, dv=dv, lengths=lengths, H=int(r.integers(1, 4)),
                gate_mu=float(r.uniform(-1.0, 5.0)), gate_sd=float(r.uniform(0.3, 2.5)),
                init_sd=float(r.choice([0.0, 0.02, 0.5])), hard=bool(r.random() < 0.3),
                dfinal=bool(r.random() < 0.7), fused=bool(r.random() < 0.3), saved=bool(r.random() < 0.5),
                seed=int(r.integers(0, 1 << 30)))


@pytest.mark.parametrize("seed", range(40))
def test_random_problem(seed):
    import torch

    import gated_delta_rule_79_amd as kda
    c = _case(seed)
    w = ki.small(dtype=c["dtype"], lengths=c["lengths"], H=c["H"], dk=c["dk"], dv=c["dv"], gate_mu=c["gate_mu"],
                 gate_sd=c["gate_sd"], init_sd=c["init_sd"], seed=c["seed"])
    inp = ki.make_inputs(w, with_grads=True, raw=c["fused"])
    if c["hard"]:
        inp = _hard_forget(inp, c["dtype"], seed=c["seed"] % 1000)
    if not c["dfinal"]:
        inp["d_final_state"] = None
    g = to_gpu(inp, c["dtype"])
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    prep = dict(qk_l2norm=True, gate_logsigmoid=True) if c["fused"] else {}
    T = g["q"].shape[1]
    ws = torch.empty(max(kda.workspace_bytes(1, T, c["H"], c["dk"], c["dv"], dt, num_seqs=len(c["lengths"]),
                                             backward=True, **prep), 1), dtype=torch.uint8, device="cuda")
    o, fin = kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=g["init_state"],
                     cu_seqlens=g["cu_seqlens"], workspace=ws, save_for_backward=c["saved"], **prep)
    grads = kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                    d_final_state=g["d_final_state"], cu_seqlens=g["cu_seqlens"], workspace=ws,
                    use_saved=c["saved"], **prep)
    torch.cuda.synchronize()
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"])
    if c["fused"]:
        ro, rf = oracle.kda_fwd_prepped(*args, init_state=inp["init_state"])
        rg = oracle.kda_bwd_prepped(*args, inp["d_out"], init_state=inp["init_state"],
                                    d_final_state=inp["d_final_state"])
    else:
        ro, rf = oracle.kda_fwd(*args, init_state=inp["init_state"])
        rg = oracle.kda_bwd(*args, inp["d_out"], init_state=inp["init_state"], d_final_state=inp["d_final_state"])
    pairs = {"o": (np_of(o)[0], ro), "final": (np_of(fin), rf)}
    for name, a, b in zip(GRADS, grads, rg):
        pairs[name] = (np_of(a)[0] if name != "d_init" else np_of(a), b)
    errs, bad = {}, {}
    for k, (gv, rv) in pairs.items():
        errs[k] = rel_err(gv, rv)
        tol = _hard_tol(c["dtype"], rv) if c["hard"] else TOL[c["dtype"]]
        if not errs[k] <= tol:
            bad[k] = (errs[k], tol)
    print(f"{c}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert not bad, f"{c}: {bad}"
