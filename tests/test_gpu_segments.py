"""Segment scan of the forward state pass (long sequences cut into stretches that run in parallel,
joined by a short scan of their transfers) against the float64 oracle.

KDA_SEGMENTS forces the stretch count per sequence; without it the library segments only long
sequences that leave CUs idle (configs 2 and 3 in test_gpu_fwd.py take that path).
"""
import os

import numpy as np
import pytest

import kda_inputs as ki
from kda_testutil import TOL, gpu_fwd, np_of, oracle_fwd, rel_err, to_gpu

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
