"""Decode / replay step on the GPU (kda_decode through the C ABI) against the float64 oracle.

Each case gathers states from a pool through a permuted index list with
padding entries (negative and past the pool end), commits a different token
prefix per sequence (including counts outside [0, T], which clamp), and
checks every token's output and the whole pool afterwards: committed slots
against the oracle, every other slot bit for bit against its input.
"""
import numpy as np
import pytest

import kda_inputs as ki
import oracle
from kda_testutil import TOL, np_of, rel_err, torch_dtype

pytestmark = pytest.mark.gpu


def _case(dtype, B, T, H, dk, dv, P, seed):
    rng = np.random.default_rng(seed)
    inp = ki.decode_inputs(B, T, H, dk, dv, P, dtype=dtype, seed=seed)
    idx = rng.permutation(P)[:B].astype(np.int32)
    if B >= 3:
        idx[1] = -1          # padding
        idx[B - 1] = P + 3   # outside the pool: padding too
    ncommit = rng.integers(1, T + 1, size=B).astype(np.int32)
    if B >= 4:
        ncommit[0] = T + 5   # clamps to T
        ncommit[2] = -2      # clamps to 0
    return inp, idx, ncommit


def _gpu(inp, dtype, idx, ncommit, **kw):
    import torch
    import gated_delta_rule_79_amd as kda
    dt = torch_dtype(dtype)
    t = {n: torch.from_numpy(inp[n]).to("cuda", dt) for n in ("q", "k", "v", "log_alpha", "beta")}
    pool = torch.from_numpy(inp["state_pool"]).cuda()
    ti = None if idx is None else torch.from_numpy(idx).cuda()
    tn = None if ncommit is None else torch.from_numpy(ncommit).cuda()
    o = kda.decode(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], pool, state_indices=ti, num_commit=tn, **kw)
    torch.cuda.synchronize()
    return o, pool


def _oracle(inp, idx, ncommit):
    return oracle.kda_decode(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["state_pool"],
                             state_indices=idx, num_commit=ncommit)


def _check(inp, dtype, idx, ncommit, o, pool, what=""):
    ro, rpool = _oracle(inp, idx, ncommit)
    go, gpool = np_of(o), np_of(pool)
    eo = rel_err(go, ro)
    P = inp["state_pool"].shape[0]
    B, T = inp["q"].shape[:2]
    n = np.full(B, T) if ncommit is None else np.clip(ncommit, 0, T)
    slots = np.arange(B) if idx is None else idx
    written = sorted({int(s) for s, c in zip(slots, n) if 0 <= s < P and c > 0})
    untouched = [s for s in range(P) if s not in written]
    es = rel_err(gpool[written], rpool[written]) if written else 0.0
    print(f"{what} out err {eo:.2e}, committed-state err {es:.2e}, {len(written)} slots written")
    assert eo <= TOL[dtype], f"outputs {eo:.3e}"
    assert es <= TOL[dtype], f"committed states {es:.3e}"
    assert np.array_equal(gpool[untouched], inp["state_pool"][untouched]), "a slot with nothing committed changed"
    for b in range(B):
        if not 0 <= slots[b] < P:
            assert np.all(go[b] == 0.0), "padding outputs must be zero"


@pytest.mark.parametrize("dtype,B,T,H,dk,dv,P", [
    ("f32", 3, 1, 2, 64, 64, 5),
    ("f32", 6, 3, 2, 128, 64, 9),
    ("bf16", 5, 4, 2, 128, 128, 8),
    ("bf16", 4, 16, 3, 64, 128, 4),
    ("bf16", 7, 2, 1, 128, 128, 7),
], ids=lambda x: str(x))
def test_decode_matches_oracle(dtype, B, T, H, dk, dv, P):
    inp, idx, nc = _case(dtype, B, T, H, dk, dv, P, seed=100 + B * T + dk)
    o, pool = _gpu(inp, dtype, idx, nc)
    _check(inp, dtype, idx, nc, o, pool)


def test_decode_default_slots_and_commit():
    """No index list (sequence b on slot b) and no commit counts (all T tokens)."""
    inp = ki.decode_inputs(3, 4, 2, 128, 128, 5, dtype="bf16", seed=7)
    o, pool = _gpu(inp, "bf16", None, None)
    _check(inp, "bf16", None, None, o, pool)


def test_verify_then_replay():
    """Speculative step: a verification call commits nothing and leaves the pool bit-identical;
    the replay with the accepted counts gives the same outputs bit for bit and commits the
    accepted prefixes."""
    import torch
    inp = ki.decode_inputs(6, 4, 2, 128, 128, 6, dtype="bf16", seed=11)
    idx = np.array([5, 0, 3, 1, 4, 2], np.int32)
    o_verify, pool_v = _gpu(inp, "bf16", idx, np.zeros(6, np.int32))
    assert np.array_equal(np_of(pool_v), inp["state_pool"])
    accepted = np.array([0, 1, 2, 3, 4, 2], np.int32)
    o_replay, pool_r = _gpu(inp, "bf16", idx, accepted)
    assert torch.equal(o_verify, o_replay)
    _check(inp, "bf16", idx, accepted, o_replay, pool_r, "replay")


def test_commit_prefix_then_continue_from_pool():
    """Committing 2 of 4 tokens and then decoding the last 2 from the written slots matches
    one call over all 4 tokens."""
    import torch
    import gated_delta_rule_79_amd as kda
    inp = ki.decode_inputs(4, 4, 2, 64, 128, 4, dtype="f32", seed=12)
    o_all, pool_all = _gpu(inp, "f32", None, None)
    t = {n: torch.from_numpy(inp[n]).cuda() for n in ("q", "k", "v", "log_alpha", "beta")}
    pool = torch.from_numpy(inp["state_pool"]).cuda()
    nc = torch.full((4,), 2, dtype=torch.int32, device="cuda")
    kda.decode(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], pool, num_commit=nc)
    rest = {n: x[:, 2:].contiguous() for n, x in t.items()}
    o_rest = kda.decode(rest["q"], rest["k"], rest["v"], rest["log_alpha"], rest["beta"], pool)
    torch.cuda.synchronize()
    assert rel_err(np_of(o_rest), np_of(o_all)[:, 2:]) <= 1e-5
    assert rel_err(np_of(pool), np_of(pool_all)) <= 1e-5


def test_decode_bf16_output():
    """bf16 outputs: beyond half a bf16 ulp of each value, the error stays within the bf16 bound."""
    import torch
    inp, idx, nc = _case("bf16", 5, 4, 2, 128, 128, 6, seed=13)
    o, pool = _gpu(inp, "bf16", idx, nc, out_dtype=torch.bfloat16)
    o32, pool32 = _gpu(inp, "bf16", idx, nc)
    assert o.dtype == torch.bfloat16
    ro, _ = _oracle(inp, idx, nc)
    go = np_of(o)
    rms = np.sqrt(np.mean(ro * ro))
    excess = np.max(np.maximum(np.abs(go - ro) - 2.0 ** -8 * np.abs(ro), 0.0)) / rms
    assert excess <= TOL["bf16"]
    assert torch.equal(pool, pool32)   # the state does not depend on the output dtype


def test_decode_deterministic_and_empty():
    import torch
    import gated_delta_rule_79_amd as kda
    inp, idx, nc = _case("bf16", 5, 4, 2, 128, 128, 8, seed=14)
    o1, p1 = _gpu(inp, "bf16", idx, nc)
    o2, p2 = _gpu(inp, "bf16", idx, nc)
    assert torch.equal(o1, o2) and torch.equal(p1, p2)
    z = torch.empty((0, 4, 2, 128), dtype=torch.bfloat16, device="cuda")
    zb = torch.empty((0, 4, 2), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((1, 2, 128, 128), device="cuda")
    o = kda.decode(z, z, z, z, zb, pool)
    assert o.shape == (0, 4, 2, 128)


def test_decode_serving_batch_full_check():
    """A serving-sized step (512 sequences, 4 tokens, H=16, d=128, bf16): every output and
    committed state against the oracle."""
    B, T, H, P = 512, 4, 16, 600
    inp, idx, nc = _case("bf16", B, T, H, 128, 128, P, seed=15)
    o, pool = _gpu(inp, "bf16", idx, nc)
    _check(inp, "bf16", idx, nc, o, pool, "serving batch")
