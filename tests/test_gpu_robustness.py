"""GPU parity under inputs that stress the arithmetic rather than the shapes.

* Channels that forget fast: runs of tokens whose log-decay is between -12 and
  -1e4 (and -inf), the channel-wise gating of the KDA section of "Kimi K3 on
  Fireworks: Fast RL at frontier scale" taken to its limit.  The kernels floor
  log alpha at -16 (a state row keeps e^-16 of itself instead of less), which
  moves any result by far less than the tolerances; the fp32 bound adds the
  rounding of the in-chunk decay sums (see _hard_tol).
* A NaN in one token of one sequence and head reaches no other sequence or head.
* Upstream gradients far from unit scale (1e-6 and 1e3): the backward is linear
  in (d_out, d_final_state), so the oracle's bound applies unchanged.
* Values far from unit scale in the forward (v and init_state scaled by 1e3).
"""
import numpy as np
import pytest

import kda_inputs as ki
from kda_testutil import TOL, gpu_bwd, gpu_fwd, np_of, oracle_bwd, oracle_fwd, rel_err, to_gpu

pytestmark = pytest.mark.gpu

GRADS = ["dq", "dk", "dv", "dlog_alpha", "dbeta", "d_init"]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_79_amd as kda
    kda.load_library()


def _store(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return ki.bf16_round(x) if dtype == "bf16" else x


def _hard_forget(inp, dtype, seed, frac=0.15, with_inf=False):
    """Overwrite log_alpha of a fraction of each head's channels with runs of 1-24
    tokens at log alpha in [-1e4, -12] (log-uniform), some tokens at -inf."""
    la = inp["log_alpha"].copy()
    n, H, dk = la.shape
    rng = np.random.default_rng(seed)
    for h in range(H):
        for c in rng.choice(dk, size=max(1, int(frac * dk)), replace=False):
            for _ in range(int(rng.integers(1, 5))):
                L = min(int(rng.integers(1, 25)), n)   # a run never outgrows a short input
                t0 = int(rng.integers(0, max(1, n - L)))
                la[t0:t0 + L, h, c] = -np.exp(rng.uniform(np.log(12.0), np.log(1e4), size=L))
                if with_inf and rng.random() < 0.3:
                    la[t0, h, c] = -np.inf
    inp["log_alpha"] = _store(la, dtype)
    return inp


def _errs(pairs):
    return {k: rel_err(g, r) for k, (g, r) in pairs.items()}


def _hard_tol(dtype, ref):
    """Bound for inputs with hard-forget channels.  bf16: the usual 2e-2.  fp32: the usual
    1e-4 plus the rounding of the in-chunk log-decay sums g.  Under the floor of -16,
    |g| < 64 * 16 = 1024 within a chunk, where fp32 holds g to 2^-14 (the kernels round each
    g once, from an fp64 sum); a decayed factor e^{g_a - g_b} carries two such roundings,
    2^-13 relative, and so does every gradient element built from such factors, which in
    units of the tensor's rms is 2^-13 * max|ref| / rms(ref)."""
    if dtype == "bf16":
        return TOL["bf16"]
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r)) if r.size else 1.0
    return TOL["f32"] + 2.0 ** -13 * (np.max(np.abs(r)) / rms if rms > 0 else 0.0)


HARD = [("f32", (100, 64, 129), 2, 64, 64), ("f32", (300,), 2, 64, 128), ("bf16", (64, 1, 250), 2, 128, 128),
        ("bf16", (500, 77), 2, 64, 64), ("bf16", (129, 300), 3, 128, 64)]


@pytest.mark.parametrize("dtype,lengths,H,dk,dv", HARD, ids=[f"{h[0]}-{len(h[1])}seq-{h[3]}x{h[4]}" for h in HARD])
@pytest.mark.parametrize("with_inf", [False, True], ids=["finite", "with-inf"])
def test_hard_forget_forward_and_backward(dtype, lengths, H, dk, dv, with_inf):
    import torch
    w = ki.small(dtype=dtype, lengths=lengths, H=H, dk=dk, dv=dv, seed=31)
    inp = _hard_forget(ki.make_inputs(w, with_grads=True), dtype, seed=7, with_inf=with_inf)
    g = to_gpu(inp, dtype)
    o, f = gpu_fwd(g)
    grads = gpu_bwd(g)
    torch.cuda.synchronize()
    ro, rf = oracle_fwd(inp)
    rg = oracle_bwd(inp)
    pairs = {"o": (np_of(o)[0], ro), "final": (np_of(f), rf)}
    for name, a, b in zip(GRADS, grads, rg):
        pairs[name] = (np_of(a)[0] if name != "d_init" else np_of(a), b)
    errs = _errs(pairs)
    tols = {k: _hard_tol(dtype, r) for k, (_, r) in pairs.items()}
    print(f"hard forget {dtype} {lengths} {dk}x{dv}: " + " ".join(f"{k}={v:.2e}/{tols[k]:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tols[k]}
    assert not bad, f"errors above their bounds: {bad}"


def test_hard_forget_training_step_segmented(monkeypatch):
    """The saved forward + backward over stretches of long sequences, with hard-forget channels."""
    import torch

    import gated_delta_rule_79_amd as kda
    monkeypatch.setenv("KDA_SEGMENTS", "3")
    w = ki.small(dtype="bf16", lengths=(700, 450), H=2, dk=128, dv=128, seed=32)
    inp = _hard_forget(ki.make_inputs(w, with_grads=True), "bf16", seed=8)
    g = to_gpu(inp, "bf16")
    T = g["q"].shape[1]
    ws = torch.empty(kda.workspace_bytes(1, T, 2, 128, 128, torch.bfloat16, num_seqs=2, backward=True),
                     dtype=torch.uint8, device="cuda")
    o, f = gpu_fwd(g, workspace=ws, save_for_backward=True)
    grads = gpu_bwd(g, workspace=ws, use_saved=True)
    torch.cuda.synchronize()
    ro, rf = oracle_fwd(inp)
    rg = oracle_bwd(inp)
    pairs = {"o": (np_of(o)[0], ro), "final": (np_of(f), rf)}
    for name, a, b in zip(GRADS, grads, rg):
        pairs[name] = (np_of(a)[0] if name != "d_init" else np_of(a), b)
    errs = _errs(pairs)
    print("hard forget, 3 stretches: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= _hard_tol("bf16", None) for v in errs.values()), errs


def test_hard_forget_decode():
    """The decode step floors log alpha the same way and matches the oracle."""
    import torch

    import gated_delta_rule_79_amd as kda
    import oracle
    B, T, H, dk, dv = 6, 8, 2, 128, 128
    inp = ki.decode_inputs(B, T, H, dk, dv, B, dtype="f32", seed=5)
    la = inp["log_alpha"].reshape(B * T, H, dk).copy()
    inp["log_alpha"] = _hard_forget({"log_alpha": la}, "f32", seed=9, frac=0.3)["log_alpha"].reshape(B, T, H, dk)
    t = {n: torch.from_numpy(inp[n]).cuda() for n in ("q", "k", "v", "log_alpha", "beta")}
    pool = torch.from_numpy(inp["state_pool"]).cuda()
    out = kda.decode(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], pool)
    torch.cuda.synchronize()
    ro, rpool = oracle.kda_decode(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["state_pool"])
    eo, ep = rel_err(np_of(out), ro), rel_err(np_of(pool), rpool)
    print(f"decode hard forget: o={eo:.2e} pool={ep:.2e}")
    assert eo <= TOL["f32"] and ep <= TOL["f32"]


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("where", ["k", "log_alpha", "v"])
def test_nan_stays_in_its_sequence_and_head(dtype, dk, where):
    """A NaN in one token of sequence 1, head 0 changes no output or gradient of any
    other (sequence, head): those stay bit-identical to a clean run."""
    import torch
    lengths, H = (150, 200, 90), 3
    w = ki.small(dtype=dtype, lengths=lengths, H=H, dk=dk, dv=dk, seed=33)
    inp = ki.make_inputs(w, with_grads=True)
    clean = to_gpu(inp, dtype)
    bad = to_gpu(inp, dtype)
    t_nan = lengths[0] + 70   # sequence 1, in its second chunk
    bad[where][0, t_nan, 0, 5] = float("nan")
    res = {}
    for tag, g in (("clean", clean), ("nan", bad)):
        o, f = gpu_fwd(g)
        grads = gpu_bwd(g)
        torch.cuda.synchronize()
        res[tag] = [np_of(o)[0], np_of(f)] + [np_of(x)[0] if i < 5 else np_of(x) for i, x in enumerate(grads)]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    names = ["o", "final"] + GRADS
    for name, a, b in zip(names, res["clean"], res["nan"]):
        for s in range(len(lengths)):
            for h in range(H):
                if (s, h) == (1, 0):
                    continue
                if name in ("final", "d_init"):
                    x, y = a[s, h], b[s, h]
                else:
                    x, y = a[cu[s]:cu[s + 1], h], b[cu[s]:cu[s + 1], h]
                assert np.array_equal(x, y), f"{name}: sequence {s}, head {h} changed by a NaN elsewhere"
    # the tainted unit's forward outputs before the NaN's chunk are untouched too
    c0 = cu[1] + 64
    assert np.array_equal(res["clean"][0][cu[1]:c0, 0], res["nan"][0][cu[1]:c0, 0])
    assert np.isnan(res["nan"][0][t_nan:cu[2], 0]).any()


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("scale", [1e-6, 1e3])
def test_upstream_gradient_scale(dtype, dk, scale):
    """d_out and d_final_state scaled by 1e-6 (bf16 training without loss scaling) or
    1e3: every gradient stays within the bound of the oracle run on the same inputs."""
    import torch
    w = ki.small(dtype=dtype, lengths=(300, 129), H=2, dk=dk, dv=dk, seed=34)
    inp = ki.make_inputs(w, with_grads=True)
    inp["d_out"] = _store(inp["d_out"] * scale, dtype)
    inp["d_final_state"] = (inp["d_final_state"] * scale).astype(np.float32)
    g = to_gpu(inp, dtype)
    grads = gpu_bwd(g)
    torch.cuda.synchronize()
    rg = oracle_bwd(inp)
    errs = {name: rel_err(np_of(a)[0] if name != "d_init" else np_of(a), b) for name, a, b in zip(GRADS, grads, rg)}
    print(f"gradient scale {scale:g} {dtype}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"errors above {TOL[dtype]}: {bad}"


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64)])
def test_zero_upstream_gradients(dtype, dk):
    """d_out = 0 and d_final_state = 0 (the gradient-scale pre-pass sees a largest
    magnitude of 0 and keeps s = 1): every gradient is exactly zero, as the backward is
    linear in (d_out, d_final_state); a stray value would come from stale workspace."""
    import torch
    w = ki.small(dtype=dtype, lengths=(200, 77), H=2, dk=dk, dv=dk, seed=36)
    inp = ki.make_inputs(w, with_grads=True)
    inp["d_out"] = np.zeros_like(inp["d_out"])
    inp["d_final_state"] = np.zeros_like(inp["d_final_state"])
    g = to_gpu(inp, dtype)
    grads = gpu_bwd(g)
    torch.cuda.synchronize()
    nonzero = {name: int(np.count_nonzero(np_of(a))) for name, a in zip(GRADS, grads)}
    assert all(v == 0 for v in nonzero.values()), nonzero


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64)])
def test_gradient_through_the_final_state_only(dtype, dk):
    """d_out = 0 with a d_final_state scaled by 1e-5: the gradient-scale pre-pass takes its
    scale from d_final_state alone, and every gradient stays within the bound."""
    import torch
    w = ki.small(dtype=dtype, lengths=(300, 129), H=2, dk=dk, dv=dk, seed=37)
    inp = ki.make_inputs(w, with_grads=True)
    inp["d_out"] = np.zeros_like(inp["d_out"])
    inp["d_final_state"] = (inp["d_final_state"] * 1e-5).astype(np.float32)
    g = to_gpu(inp, dtype)
    grads = gpu_bwd(g)
    torch.cuda.synchronize()
    rg = oracle_bwd(inp)
    errs = {name: rel_err(np_of(a)[0] if name != "d_init" else np_of(a), b) for name, a, b in zip(GRADS, grads, rg)}
    print(f"final state only {dtype}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"errors above {TOL[dtype]}: {bad}"


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64)])
def test_forward_value_scale(dtype, dk):
    """v and init_state scaled by 1e3 (states far above unit scale)."""
    import torch
    w = ki.small(dtype=dtype, lengths=(300, 129), H=2, dk=dk, dv=dk, seed=35)
    inp = ki.make_inputs(w, with_grads=True)
    inp["v"] = _store(inp["v"] * 1e3, dtype)
    inp["init_state"] = (inp["init_state"] * 1e3).astype(np.float32)
    g = to_gpu(inp, dtype)
    o, f = gpu_fwd(g)
    grads = gpu_bwd(g)
    torch.cuda.synchronize()
    ro, rf = oracle_fwd(inp)
    rg = oracle_bwd(inp)
    pairs = {"o": (np_of(o)[0], ro), "final": (np_of(f), rf)}
    for name, a, b in zip(GRADS, grads, rg):
        pairs[name] = (np_of(a)[0] if name != "d_init" else np_of(a), b)
    errs = _errs(pairs)
    print(f"value scale 1e3 {dtype}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL[dtype] for v in errs.values()), errs


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_hard_forget_through_the_fused_gate(dk, dv):
    """Raw gates far below zero (x in [-1e4, -12] on runs of channels, so logsigmoid(x) ~ x is floored)
    through the fused preparation (in-kernel L2 norm and logsigmoid), bf16, forward and backward, with
    the gradients taken with respect to the raw inputs."""
    import torch

    import gated_delta_rule_79_amd as kda
    import oracle
    w = ki.small(dtype="bf16", lengths=(260, 1, 130), H=2, dk=dk, dv=dv, seed=36)
    inp = ki.make_inputs(w, with_grads=True, raw=True)
    inp = _hard_forget(inp, "bf16", seed=10)   # the raw gate takes the hard-forget runs
    g = to_gpu(inp, "bf16")
    prep = dict(qk_l2norm=True, gate_logsigmoid=True)
    o, f = gpu_fwd(g, **prep)
    grads = gpu_bwd(g, **prep)
    torch.cuda.synchronize()
    ro, rf = oracle.kda_fwd_prepped(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                                    init_state=inp["init_state"])
    rg = oracle.kda_bwd_prepped(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
                                inp["d_out"], init_state=inp["init_state"], d_final_state=inp["d_final_state"])
    pairs = {"o": (np_of(o)[0], ro), "final": (np_of(f), rf)}
    for name, a, b in zip(GRADS, grads, rg):
        pairs[name] = (np_of(a)[0] if name != "d_init" else np_of(a), b)
    errs = _errs(pairs)
    print(f"hard forget, fused gate {dk}x{dv}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs
