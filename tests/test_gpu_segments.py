"""Segment scan of the sequential passes (long sequences cut into stretches that run in parallel,
joined by a short scan of their transfers) against the float64 oracle: the forward, and the
training step, whose forward keeps the backward's intermediates from every stretch's true entering
state and whose reverse pass is joined by a reverse scan with the transposed transfers.

KDA_SEGMENTS forces the stretch count per sequence; without it the library segments only long
sequences that leave CUs idle (configs 2 and 3 in test_gpu_fwd.py take that path).
"""
import os

import numpy as np
import pytest

import kda_inputs as ki
from kda_testutil import TOL, gpu_bwd, gpu_fwd, np_of, oracle_bwd, oracle_fwd, rel_err, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture
def segments():
    old = os.environ.get("KDA_SEGMENTS")

    def set_(p):
        os.environ["KDA_SEGMENTS"] = str(p)
    yield set_
    if old is None:
        os.environ.pop("KDA_SEGMENTS", None)
    else:
        os.environ["KDA_SEGMENTS"] = old


@pytest.mark.parametrize("dtype,lengths,H,dk,dv,P", [
    ("bf16", (1000, 700, 323), 2, 128, 128, 3),
    ("bf16", (2000,), 2, 128, 128, 5),
    ("f32", (900, 64, 7, 500), 2, 64, 64, 2),
    ("bf16", (640, 130), 3, 64, 128, 4),
    ("bf16", (200, 1, 65), 2, 128, 64, 7),   # more stretches than some sequences have chunks
], ids=lambda x: str(x))
def test_segmented_forward_matches_oracle(segments, dtype, lengths, H, dk, dv, P):
    import torch
    w = ki.small(dtype=dtype, lengths=lengths, H=H, dk=dk, dv=dv)
    inp = ki.make_inputs(w)
    g = to_gpu(inp, dtype)
    segments(1)
    o1, f1 = gpu_fwd(g)
    segments(P)
    o, f = gpu_fwd(g)
    torch.cuda.synchronize()
    ro, rf = oracle_fwd(inp)
    eo, ef = rel_err(np_of(o)[0], ro), rel_err(np_of(f), rf)
    print(f"P={P}: o {eo:.2e}, final {ef:.2e}; vs unsegmented o {rel_err(np_of(o), np_of(o1)):.2e}")
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


def test_segmented_final_state_aliases_init(segments):
    """final_state may alias init_state on the segmented path too."""
    import torch
    import gated_delta_rule_79_amd as kda
    w = ki.small(dtype="bf16", lengths=(800, 300), H=2, dk=128, dv=128)
    inp = ki.make_inputs(w)
    g = to_gpu(inp, "bf16")
    segments(4)
    _, f_ref = gpu_fwd(g)
    st = g["init_state"].clone()
    kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=st, cu_seqlens=g["cu_seqlens"],
            final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(st, f_ref)


def test_auto_segmentation_choice(segments):
    """Long single sequences with few heads are segmented; short or many-head batches are not."""
    import gated_delta_rule_79_amd as kda
    import torch
    os.environ.pop("KDA_SEGMENTS", None)
    long_one = kda.workspace_bytes(1, 131072, 16, 128, 128, torch.bfloat16)
    segments(1)
    plain = kda.workspace_bytes(1, 131072, 16, 128, 128, torch.bfloat16)
    assert long_one > plain   # the stretch buffers are planned
    os.environ.pop("KDA_SEGMENTS", None)
    assert kda.workspace_bytes(8, 4096, 16, 128, 128, torch.bfloat16) == kda.workspace_bytes(
        8, 4096, 16, 128, 128, torch.bfloat16, backward=False)


GRADS = ["dq", "dk", "dv", "dlog_alpha", "dbeta", "d_init"]
TRAIN_CASES = [
    ("bf16", (1000, 700, 323), 2, 128, 128, 3),
    ("bf16", (2000,), 2, 128, 128, 5),
    ("f32", (900, 64, 7, 500), 2, 64, 64, 2),
    ("bf16", (640, 130), 3, 64, 128, 4),
    ("bf16", (200, 1, 65), 2, 128, 64, 7),   # more stretches than some sequences have chunks
]


@pytest.mark.parametrize("dtype,lengths,H,dk,dv,P", TRAIN_CASES, ids=lambda x: str(x))
def test_segmented_training_step_matches_oracle(segments, dtype, lengths, H, dk, dv, P):
    """fwd(save_for_backward) + bwd(use_saved) with P stretches per sequence: outputs and every
    gradient within the parity bound, and bit-identical to the self-contained backward (which
    recomputes the forward with the same stretches)."""
    import torch
    import gated_delta_rule_79_amd as kda
    w = ki.small(dtype=dtype, lengths=lengths, H=H, dk=dk, dv=dv)
    inp = ki.make_inputs(w, with_grads=True)
    g = to_gpu(inp, dtype)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    segments(P)
    ws = torch.empty(kda.workspace_bytes(1, g["q"].shape[1], H, dk, dv, dt, num_seqs=len(lengths), backward=True),
                     dtype=torch.uint8, device="cuda")
    o, fin = kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=g["init_state"],
                     cu_seqlens=g["cu_seqlens"], workspace=ws, save_for_backward=True)
    got = kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                  d_final_state=g["d_final_state"], cu_seqlens=g["cu_seqlens"], workspace=ws, use_saved=True)
    rec = gpu_bwd(g)
    torch.cuda.synchronize()
    ro, rf = oracle_fwd(inp)
    ref = oracle_bwd(inp)
    errs = {"o": rel_err(np_of(o)[0], ro), "final_state": rel_err(np_of(fin), rf)}
    for name, a, b in zip(GRADS, got, ref):
        ga = np_of(a)
        errs[name] = rel_err(ga if name == "d_init" else ga[0], b)
    print(f"P={P}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"errors above {TOL[dtype]}: {bad}"
    for name, a, b in zip(GRADS, got, rec):
        assert torch.equal(a, b), name


def test_segmented_backward_without_state_grads(segments):
    """No d_final_state (zero) and no d_init_state output on the segmented reverse pass."""
    import torch
    import gated_delta_rule_79_amd as kda
    w = ki.small(dtype="bf16", lengths=(900, 260), H=2, dk=128, dv=128)
    inp = ki.make_inputs(w, with_grads=True)
    inp["d_final_state"] = None
    g = to_gpu(inp, "bf16")
    segments(4)
    got = kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                  cu_seqlens=g["cu_seqlens"], need_d_init=False)
    torch.cuda.synchronize()
    ref = oracle_bwd(inp)
    assert got[5] is None
    for name, a, b in zip(GRADS[:5], got[:5], ref[:5]):
        assert rel_err(np_of(a)[0], b) <= TOL["bf16"], name


def test_auto_segmentation_of_the_training_step(segments):
    """A long single sequence with few heads is segmented in training mode too (stretch buffers in the
    backward's workspace plan); the packed 8-sequence training batch is not."""
    import torch
    import gated_delta_rule_79_amd as kda
    os.environ.pop("KDA_SEGMENTS", None)
    long_one = kda.workspace_bytes(1, 131072, 16, 128, 128, torch.bfloat16, backward=True)
    segments(1)
    plain = kda.workspace_bytes(1, 131072, 16, 128, 128, torch.bfloat16, backward=True)
    assert long_one > plain
    os.environ.pop("KDA_SEGMENTS", None)
    w = ki.config(4)
    n = sum(w.lengths)
    with_auto = kda.workspace_bytes(1, n, 16, 128, 128, torch.bfloat16, num_seqs=8, backward=True)
    segments(1)
    assert with_auto == kda.workspace_bytes(1, n, 16, 128, 128, torch.bfloat16, num_seqs=8, backward=True)


def test_segmented_training_full_size(segments):
    """The long-sequence workload (one 131,072-token sequence, H = 16) as a training step, with the
    stretches the library chooses for it (8), in the launch configuration the benchmark's long-sequence
    training step times; the oracle checks all 16 heads over the whole sequence."""
    import torch
    import gated_delta_rule_79_amd as kda
    os.environ.pop("KDA_SEGMENTS", None)
    w = ki.config(3)
    inp = ki.make_inputs(w, with_grads=True)
    g = to_gpu(inp, "bf16")
    T, H = g["q"].shape[1], w.H
    auto = kda.workspace_bytes(1, T, H, 128, 128, torch.bfloat16, num_seqs=1, backward=True)
    segments(1)
    assert auto > kda.workspace_bytes(1, T, H, 128, 128, torch.bfloat16, num_seqs=1, backward=True)   # segmented
    os.environ.pop("KDA_SEGMENTS", None)
    ws = torch.empty(kda.workspace_bytes(1, T, H, 128, 128, torch.bfloat16, num_seqs=1, backward=True),
                     dtype=torch.uint8, device="cuda")
    o, fin = kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=g["init_state"],
                     cu_seqlens=g["cu_seqlens"], workspace=ws, save_for_backward=True)
    got = kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                  d_final_state=g["d_final_state"], cu_seqlens=g["cu_seqlens"], workspace=ws, use_saved=True)
    torch.cuda.synchronize()
    ro, rf = oracle_fwd(inp)
    ref = oracle_bwd(inp)
    errs = {"o": rel_err(np_of(o)[0], ro), "final_state": rel_err(np_of(fin), rf)}
    for name, a, b in zip(GRADS, got, ref):
        ga = np_of(a)
        errs[name] = rel_err(ga if name == "d_init" else ga[0], b)
    print("full size, all heads: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, f"errors above {TOL['bf16']}: {bad}"


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 64)])
def test_segmented_training_with_fused_input_preparation(segments, dtype, dk, dv):
    """The training step on raw q, k and gate (in-kernel L2 norm and logsigmoid) with 3 stretches per
    sequence: the stretches' extra workspace sits beside the preparation's, and the gradients with respect
    to the raw inputs stay within the bound (oracle composed with the same maps)."""
    import torch
    import gated_delta_rule_79_amd as kda
    import oracle
    lengths, H = (900, 130, 600), 2
    w = ki.small(dtype=dtype, lengths=lengths, H=H, dk=dk, dv=dv)
    inp = ki.make_inputs(w, with_grads=True, raw=True)
    g = to_gpu(inp, dtype)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    segments(3)
    prep = dict(qk_l2norm=True, gate_logsigmoid=True)
    ws = torch.empty(kda.workspace_bytes(1, g["q"].shape[1], H, dk, dv, dt, num_seqs=len(lengths), backward=True,
                                         **prep), dtype=torch.uint8, device="cuda")
    o, fin = kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=g["init_state"],
                     cu_seqlens=g["cu_seqlens"], workspace=ws, save_for_backward=True, **prep)
    got = kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                  d_final_state=g["d_final_state"], cu_seqlens=g["cu_seqlens"], workspace=ws, use_saved=True, **prep)
    torch.cuda.synchronize()
    ro, rf = oracle.kda_fwd_prepped(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                                    init_state=inp["init_state"])
    ref = oracle.kda_bwd_prepped(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                                 inp["d_out"], init_state=inp["init_state"], d_final_state=inp["d_final_state"])
    errs = {"o": rel_err(np_of(o)[0], ro), "final_state": rel_err(np_of(fin), rf)}
    for name, a, b in zip(GRADS, got, ref):
        ga = np_of(a)
        errs[name] = rel_err(ga if name == "d_init" else ga[0], b)
    print("segmented + prepared inputs: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"errors above {TOL[dtype]}: {bad}"


def test_fused_prep_training_step_at_varlen_workload_lengths():
    """The training step on raw q, k and gate (in-kernel L2 norm and logsigmoid) over the 8-sequence
    varlen workload's lengths (1K-32K tokens, 159,285 in all), every sequence and head: the gradients
    with respect to the raw inputs stay within the bf16 bound at full sequence length."""
    import torch
    import gated_delta_rule_79_amd as kda
    import oracle
    os.environ.pop("KDA_SEGMENTS", None)
    w = ki.config(4)
    inp = ki.make_inputs(w, with_grads=True, raw=True)
    g = to_gpu(inp, "bf16")
    prep = dict(qk_l2norm=True, gate_logsigmoid=True)
    ws = torch.empty(kda.workspace_bytes(1, g["q"].shape[1], w.H, 128, 128, torch.bfloat16, num_seqs=len(w.lengths),
                                         backward=True, **prep), dtype=torch.uint8, device="cuda")
    o, fin = kda.fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], init_state=g["init_state"],
                     cu_seqlens=g["cu_seqlens"], workspace=ws, save_for_backward=True, **prep)
    got = kda.bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["d_out"], init_state=g["init_state"],
                  d_final_state=g["d_final_state"], cu_seqlens=g["cu_seqlens"], workspace=ws, use_saved=True, **prep)
    torch.cuda.synchronize()
    ro, rf = oracle.kda_fwd_prepped(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                                    init_state=inp["init_state"])
    ref = oracle.kda_bwd_prepped(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                                 inp["d_out"], init_state=inp["init_state"], d_final_state=inp["d_final_state"])
    errs = {"o": rel_err(np_of(o)[0], ro), "final_state": rel_err(np_of(fin), rf)}
    for name, a, b in zip(GRADS, got, ref):
        ga = np_of(a)
        errs[name] = rel_err(ga if name == "d_init" else ga[0], b)
    print("fused prep, varlen workload: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, f"errors above {TOL['bf16']}: {bad}"
