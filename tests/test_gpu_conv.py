"""Short causal convolution on the GPU (kda_conv_fwd / kda_conv_bwd /
kda_conv_decode through the C ABI) against the float64 oracle in
oracle/short_conv.py.

Tolerance.  Every output is a sum of at most W + 1 fp32 products (forward, dx,
d_init_state) of exactly upcast inputs, so its rounding error is a few fp32
ulps of the largest term; SiLU adds the error of the hardware exponential
(a few ulps for |z| of order 10).  The bound used, max|diff| / rms(oracle)
<= 1e-5, leaves a margin of about 10x over that.  dweight and dbias are
token sums (fp32 partial sums over 256-token tiles, then over tiles in
order): bound 1e-4, the fp32 bar of the recurrence's parity tests.
"""
import numpy as np
import pytest

import kda_inputs as ki
from kda_testutil import np_of, rel_err, torch_dtype
from oracle import short_conv as sc

pytestmark = pytest.mark.gpu

TOL_Y = 1e-5
TOL_SUM = 1e-4


def _t(a, dtype="f32"):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch_dtype(dtype))


def _inputs(lengths, D, W, dtype, state=True, seed=777):
    c = ki.conv_inputs(lengths, D, W, dtype=dtype, seed=seed, state=state)
    g = dict(x=_t(c["x"], dtype).unsqueeze(0), dy=_t(c["dy"], dtype).unsqueeze(0), weight=_t(c["weight"]),
             bias=_t(c["bias"]), init_state=_t(c["init_state"]), d_final_state=_t(c["d_final_state"]),
             cu=_t(c["cu_seqlens"]).to(dtype=__import__("torch").int32))
    return c, g


CASES = [  # lengths (ragged, empty and shorter-than-state sequences), D, W
    ([300, 0, 1, 2, 777, 64, 257], 72, 4),
    ([5, 130], 2056, 3),
    ([1, 0, 600], 16, 2),
]


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lengths,D,W", CASES)
def test_conv_forward_matches_oracle(lengths, D, W, dtype, silu):
    import gated_delta_rule_79_amd as kda
    import torch
    c, g = _inputs(lengths, D, W, dtype)
    y, fin = kda.conv_fwd(g["x"], g["weight"], g["bias"], g["init_state"], cu_seqlens=g["cu"], silu=silu)
    torch.cuda.synchronize()
    ry, rfin = sc.short_conv_fwd(c["x"], c["weight"], c["cu_seqlens"], bias=c["bias"], init_state=c["init_state"],
                                 silu=silu)
    assert rel_err(np_of(y[0]), ry) <= TOL_Y
    assert rel_err(np_of(fin), rfin) <= TOL_Y
    # final rows that are copies of the input (or of the initial state) are exact
    assert np.array_equal(np_of(fin), rfin)


@pytest.mark.parametrize("silu", [False, True])
def test_conv_forward_rows_without_state_or_bias(silu):
    """B rows of T tokens (no cu_seqlens), zero initial state, no bias."""
    import gated_delta_rule_79_amd as kda
    import torch
    c = ki.conv_inputs([200, 200, 200], 40, 4, dtype="bf16", seed=9, state=False)
    x = _t(c["x"], "bf16").reshape(3, 200, 40)
    y, fin = kda.conv_fwd(x, _t(c["weight"]), silu=silu)
    torch.cuda.synchronize()
    ry, rfin = sc.short_conv_fwd(c["x"], c["weight"], c["cu_seqlens"], silu=silu)
    assert rel_err(np_of(y).reshape(ry.shape), ry) <= TOL_Y
    assert np.array_equal(np_of(fin), rfin)


def test_conv_final_state_may_alias_init_state():
    import gated_delta_rule_79_amd as kda
    import torch
    lengths, D, W = [300, 0, 1, 2, 777], 72, 4
    c, g = _inputs(lengths, D, W, "bf16")
    state = g["init_state"].clone()
    y, fin = kda.conv_fwd(g["x"], g["weight"], g["bias"], state, cu_seqlens=g["cu"], silu=True, final_state=state)
    torch.cuda.synchronize()
    ry, rfin = sc.short_conv_fwd(c["x"], c["weight"], c["cu_seqlens"], bias=c["bias"], init_state=c["init_state"],
                                 silu=True)
    assert rel_err(np_of(y[0]), ry) <= TOL_Y
    assert np.array_equal(np_of(state), rfin)


@pytest.mark.parametrize("with_dfinal", [False, True])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lengths,D,W", CASES)
def test_conv_backward_matches_oracle(lengths, D, W, dtype, silu, with_dfinal):
    import gated_delta_rule_79_amd as kda
    import torch
    c, g = _inputs(lengths, D, W, dtype)
    dfin = g["d_final_state"] if with_dfinal else None
    dx, dw, db, dinit = kda.conv_bwd(g["x"], g["weight"], g["dy"], g["bias"], g["init_state"], dfin,
                                     cu_seqlens=g["cu"], silu=silu)
    torch.cuda.synchronize()
    r = sc.short_conv_bwd(c["x"], c["weight"], c["cu_seqlens"], c["dy"], bias=c["bias"], init_state=c["init_state"],
                          d_final_state=c["d_final_state"] if with_dfinal else None, silu=silu)
    errs = dict(dx=rel_err(np_of(dx[0]), r[0]), dweight=rel_err(np_of(dw), r[1]), dbias=rel_err(np_of(db), r[2]),
                dinit=rel_err(np_of(dinit), r[3]))
    assert errs["dx"] <= TOL_Y and errs["dinit"] <= TOL_Y, errs
    assert errs["dweight"] <= TOL_SUM and errs["dbias"] <= TOL_SUM, errs


def test_conv_backward_is_deterministic_and_bf16_output():
    """Two calls give bit-identical gradients; a bf16 dx differs from the fp32 one only by its rounding."""
    import gated_delta_rule_79_amd as kda
    import torch
    c, g = _inputs([700, 3, 1300], 136, 4, "bf16")
    a = kda.conv_bwd(g["x"], g["weight"], g["dy"], g["bias"], g["init_state"], g["d_final_state"],
                     cu_seqlens=g["cu"], silu=True)
    b = kda.conv_bwd(g["x"], g["weight"], g["dy"], g["bias"], g["init_state"], g["d_final_state"],
                     cu_seqlens=g["cu"], silu=True)
    h = kda.conv_bwd(g["x"], g["weight"], g["dy"], g["bias"], g["init_state"], g["d_final_state"],
                     cu_seqlens=g["cu"], silu=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    assert torch.equal(h[0], a[0].to(torch.bfloat16))
    assert torch.equal(h[1], a[1]) and torch.equal(h[3], a[3])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [2, 4])
def test_conv_decode_matches_oracle(dtype, W):
    import gated_delta_rule_79_amd as kda
    import torch
    B, T, D, P = 7, 5, 2056, 11
    d = ki.conv_decode_inputs(B, T, D, W, P, dtype=dtype, seed=31)
    rng = np.random.default_rng(4)
    idx = rng.permutation(P)[:B].astype(np.int32)
    idx[1], idx[5] = -1, P + 2                          # padding entries
    nc = np.array([T + 3, 2, -1, 0, 1, 3, T], np.int32)   # clamped to [0, T]
    pool = _t(d["state_pool"])
    y = kda.conv_decode(_t(d["x"], dtype), _t(d["weight"]), pool, bias=_t(d["bias"]),
                        state_indices=torch.from_numpy(idx).cuda(), num_commit=torch.from_numpy(nc).cuda(), silu=True)
    torch.cuda.synchronize()
    ry, rpool = sc.short_conv_decode(d["x"], d["weight"], d["state_pool"], bias=d["bias"], state_indices=idx,
                                     num_commit=nc, silu=True)
    assert rel_err(np_of(y), ry) <= TOL_Y
    assert np.array_equal(np_of(y)[[1, 5]], np.zeros((2, T, D)))
    # a committed state is a copy of input rows or of the old state: exact, and untouched slots are unchanged
    assert np.array_equal(np_of(pool), rpool)


def test_conv_decode_equals_forward_from_the_slot():
    """Decoding T tokens from a slot and committing all of them gives the forward's outputs and final state."""
    import gated_delta_rule_79_amd as kda
    import torch
    B, T, D, W = 3, 9, 64, 4
    d = ki.conv_decode_inputs(B, T, D, W, B, dtype="bf16", seed=12)
    pool = _t(d["state_pool"])
    x = _t(d["x"], "bf16")
    y = kda.conv_decode(x, _t(d["weight"]), pool, bias=_t(d["bias"]), silu=True)
    yf, fin = kda.conv_fwd(x, _t(d["weight"]), _t(d["bias"]), _t(d["state_pool"]), silu=True)
    torch.cuda.synchronize()
    assert torch.equal(y, yf)
    assert torch.equal(pool, fin)


def test_conv_full_size_sampled_channels():
    """The benchmark workload (the eight packed sequences of the training step, D = 3 x 16 heads x 128
    channels, W = 4, SiLU) in the launch configuration the benchmark times; the oracle runs on 48 sampled
    channels (channels are independent), over every token."""
    import gated_delta_rule_79_amd as kda
    import torch
    lengths = list(ki.config(4).lengths)
    D, W = 6144, 4
    c = ki.conv_inputs(lengths, D, W, dtype="bf16", seed=4)
    g = dict(x=_t(c["x"], "bf16").unsqueeze(0), dy=_t(c["dy"], "bf16").unsqueeze(0))
    cu = torch.from_numpy(c["cu_seqlens"]).cuda()
    y, fin = kda.conv_fwd(g["x"], _t(c["weight"]), _t(c["bias"]), _t(c["init_state"]), cu_seqlens=cu, silu=True)
    dx, dw, db, dinit = kda.conv_bwd(g["x"], _t(c["weight"]), g["dy"], _t(c["bias"]), _t(c["init_state"]),
                                     _t(c["d_final_state"]), cu_seqlens=cu, silu=True)
    torch.cuda.synchronize()
    ch = np.sort(np.random.default_rng(0).choice(D, 48, replace=False))
    tch = torch.from_numpy(ch).cuda()
    sub = lambda a: np.ascontiguousarray(a[..., ch])  # noqa: E731
    ry, rfin = sc.short_conv_fwd(sub(c["x"]), c["weight"][ch], c["cu_seqlens"], bias=c["bias"][ch],
                                 init_state=sub(c["init_state"]), silu=True)
    r = sc.short_conv_bwd(sub(c["x"]), c["weight"][ch], c["cu_seqlens"], sub(c["dy"]), bias=c["bias"][ch],
                          init_state=sub(c["init_state"]), d_final_state=sub(c["d_final_state"]), silu=True)
    assert rel_err(np_of(y[0][:, tch]), ry) <= TOL_Y
    assert np.array_equal(np_of(fin[:, :, tch]), rfin)
    assert rel_err(np_of(dx[0][:, tch]), r[0]) <= TOL_Y
    assert rel_err(np_of(dw[tch]), r[1]) <= TOL_SUM
    assert rel_err(np_of(db[tch]), r[2]) <= TOL_SUM
    assert rel_err(np_of(dinit[:, :, tch]), r[3]) <= TOL_Y


def test_conv_no_tokens():
    """Packed sequences that are all empty: y is empty, final_state = init_state, d_init_state =
    d_final_state, dweight and dbias are zero."""
    import gated_delta_rule_79_amd as kda
    import torch
    c, g = _inputs([0, 0, 0], 24, 3, "bf16")
    y, fin = kda.conv_fwd(g["x"], g["weight"], g["bias"], g["init_state"], cu_seqlens=g["cu"], silu=True)
    dx, dw, db, dinit = kda.conv_bwd(g["x"], g["weight"], g["dy"], g["bias"], g["init_state"], g["d_final_state"],
                                     cu_seqlens=g["cu"], silu=True)
    torch.cuda.synchronize()
    assert y.shape == (1, 0, 24) and dx.shape == (1, 0, 24)
    assert torch.equal(fin, g["init_state"])
    assert torch.equal(dinit, g["d_final_state"])
    assert not dw.any() and not db.any()


@pytest.mark.parametrize("silu", [False, True])
def test_conv_backward_rows_without_cu_seqlens(silu):
    """B rows of T tokens (no cu_seqlens): gradients against the oracle over the same packed rows."""
    import gated_delta_rule_79_amd as kda
    import torch
    c = ki.conv_inputs([300, 300, 300], 48, 4, dtype="bf16", seed=21)
    x = _t(c["x"], "bf16").reshape(3, 300, 48)
    dy = _t(c["dy"], "bf16").reshape(3, 300, 48)
    dx, dw, db, dinit = kda.conv_bwd(x, _t(c["weight"]), dy, _t(c["bias"]), _t(c["init_state"]),
                                     _t(c["d_final_state"]), silu=silu)
    torch.cuda.synchronize()
    r = sc.short_conv_bwd(c["x"], c["weight"], c["cu_seqlens"], c["dy"], bias=c["bias"], init_state=c["init_state"],
                          d_final_state=c["d_final_state"], silu=silu)
    assert rel_err(np_of(dx).reshape(r[0].shape), r[0]) <= TOL_Y
    assert rel_err(np_of(dw), r[1]) <= TOL_SUM and rel_err(np_of(db), r[2]) <= TOL_SUM
    assert rel_err(np_of(dinit), r[3]) <= TOL_Y


def test_conv_bf16_outputs_round_once():
    """bf16 y (forward and decode) is the fp32 result rounded once to bf16."""
    import gated_delta_rule_79_amd as kda
    import torch
    c, g = _inputs([300, 0, 1, 2, 777], 72, 4, "bf16")
    y32, f32 = kda.conv_fwd(g["x"], g["weight"], g["bias"], g["init_state"], cu_seqlens=g["cu"], silu=True)
    y16, f16 = kda.conv_fwd(g["x"], g["weight"], g["bias"], g["init_state"], cu_seqlens=g["cu"], silu=True,
                            out_dtype=torch.bfloat16)
    d = ki.conv_decode_inputs(5, 3, 64, 4, 5, dtype="bf16", seed=8)
    pa, pb = _t(d["state_pool"]), _t(d["state_pool"])
    yd32 = kda.conv_decode(_t(d["x"], "bf16"), _t(d["weight"]), pa, bias=_t(d["bias"]), silu=True)
    yd16 = kda.conv_decode(_t(d["x"], "bf16"), _t(d["weight"]), pb, bias=_t(d["bias"]), silu=True,
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16 and torch.equal(y16, y32.to(torch.bfloat16))
    assert torch.equal(f16, f32)
    assert torch.equal(yd16, yd32.to(torch.bfloat16)) and torch.equal(pa, pb)
