"""Pins for the float64 oracle: facts that hold independently of its code.

Each pin takes a loaded oracle library (so the mutation test can run the same
pins against deliberately broken builds of the oracle) and raises
AssertionError when the oracle disagrees with the fact.

The recurrence being pinned (fireworks.ai, "Kimi K3 on Fireworks", section on
Kimi Delta Attention; channel-wise gated delta rule):
    S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = scale S_t^T q_t.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import short_conv as sc

RNG_SEED = 20261202


def _rand_case(rng, lengths, H, dk, dv, unit_k=True, gate=(2.0, 1.0), init_sd=0.5):
    n = int(sum(lengths))
    q = rng.standard_normal((n, H, dk))
    k = rng.standard_normal((n, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((n, H, dv))
    x = rng.normal(gate[0], gate[1], (n, H, dk))
    la = -np.logaddexp(0.0, -x)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((n, H))))
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    init = rng.standard_normal((len(lengths), H, dk, dv)) * init_sd
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, cu_seqlens=cu, init_state=init)


def _fwd(lib, c, **kw):
    args = dict(c)
    args.update(kw)
    return oracle.kda_fwd(args["q"], args["k"], args["v"], args["log_alpha"], args["beta"], args["cu_seqlens"],
                          init_state=args.get("init_state"), scale=args.get("scale"), nthreads=2, lib=lib)


def _close(a, b, tol, what):
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    assert err <= tol * max(ref, 1.0), f"{what}: max err {err:.3e} (ref max {ref:.3e})"


# ---------------------------------------------------------------------------
# forward pins
# ---------------------------------------------------------------------------
def pin_identity_when_no_write_no_decay(lib):
    """beta=0 and alpha=1: the state never changes, o_t = scale S_0^T q_t."""
    rng = np.random.default_rng(RNG_SEED)
    c = _rand_case(rng, [7, 0, 12], H=2, dk=5, dv=3)
    c["beta"][:] = 0.0
    c["log_alpha"][:] = 0.0
    o, fin = _fwd(lib, c, scale=0.7)
    _close(fin, c["init_state"], 1e-14, "final_state")
    cu = c["cu_seqlens"]
    for s in range(len(cu) - 1):
        for t in range(cu[s], cu[s + 1]):
            for h in range(2):
                ref = 0.7 * c["init_state"][s, h].T @ c["q"][t, h]
                _close(o[t, h], ref, 1e-14, "output")


def pin_unit_key_replaces_component(lib):
    """alpha=1, beta=1, one unit key: k^T S_1 = v^T and u^T S_1 = u^T S_0 for u orthogonal to k."""
    rng = np.random.default_rng(RNG_SEED + 1)
    dk, dv = 6, 4
    c = _rand_case(rng, [1], H=1, dk=dk, dv=dv)
    c["beta"][:] = 1.0
    c["log_alpha"][:] = 0.0
    _, fin = _fwd(lib, c)
    S1, S0 = fin[0, 0], c["init_state"][0, 0]
    kk = c["k"][0, 0]
    _close(kk @ S1, c["v"][0, 0], 1e-13, "k^T S_1")
    for _ in range(3):
        u = rng.standard_normal(dk)
        u -= (u @ kk) * kk
        _close(u @ S1, u @ S0, 1e-13, "u^T S_1")


def _brute_force(c, scale):
    """Unrolled products of explicit dk x dk transition matrices."""
    q, k, v, la, beta, cu, init = (c[x] for x in ("q", "k", "v", "log_alpha", "beta", "cu_seqlens", "init_state"))
    n, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((n, H, dv))
    fin = np.zeros((len(cu) - 1, H, dk, dv))
    I = np.eye(dk)
    for s in range(len(cu) - 1):
        for h in range(H):
            ts = list(range(cu[s], cu[s + 1]))
            Ms = [(I - beta[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(la[t, h])) for t in ts]
            for i in range(len(ts) + 1):
                # S after i tokens = (M_i ... M_1) S_0 + sum_{j<=i} (M_i ... M_{j+1}) b_j k_j v_j^T
                prod = I.copy()
                for M in Ms[:i]:
                    prod = M @ prod
                S = prod @ init[s, h]
                for j in range(i):
                    tail = I.copy()
                    for M in Ms[j + 1:i]:
                        tail = M @ tail
                    t = ts[j]
                    S = S + tail @ (beta[t, h] * np.outer(k[t, h], v[t, h]))
                if i > 0:
                    o[ts[i - 1], h] = scale * S.T @ q[ts[i - 1], h]
                if i == len(ts):
                    fin[s, h] = S
    return o, fin


def pin_brute_force_products(lib):
    """T<=8: oracle == explicit products of (I - b k k^T) Diag(a), unnormalised keys, dk != dv."""
    rng = np.random.default_rng(RNG_SEED + 2)
    c = _rand_case(rng, [8, 3, 1], H=2, dk=5, dv=3, unit_k=False, gate=(0.5, 1.0))
    o, fin = _fwd(lib, c, scale=0.37)
    ob, fb = _brute_force(c, 0.37)
    _close(o, ob, 1e-12, "outputs")
    _close(fin, fb, 1e-12, "final_state")


def pin_pure_decay(lib):
    """beta=0: S_t = Diag(exp(sum_{s<=t} log a_s)) S_0 exactly (up to rounding)."""
    rng = np.random.default_rng(RNG_SEED + 3)
    c = _rand_case(rng, [40], H=1, dk=4, dv=3, gate=(1.0, 2.0))
    c["beta"][:] = 0.0
    o, fin = _fwd(lib, c)
    g = np.cumsum(c["log_alpha"][:, 0, :], axis=0)
    S0 = c["init_state"][0, 0]
    for t in range(40):
        St = np.exp(g[t])[:, None] * S0
        _close(o[t, 0], 0.5 * St.T @ c["q"][t, 0], 1e-12, "decay output")
    _close(fin[0, 0], np.exp(g[-1])[:, None] * S0, 1e-12, "decay final")


def pin_orthonormal_keys_projection(lib):
    """alpha=1, beta=1, orthonormal keys: S_T = (I - sum k k^T) S_0 + sum k v^T."""
    rng = np.random.default_rng(RNG_SEED + 4)
    dk, dv, T = 8, 5, 6
    c = _rand_case(rng, [T], H=1, dk=dk, dv=dv)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    c["k"][:, 0, :] = Qm[:, :T].T
    c["beta"][:] = 1.0
    c["log_alpha"][:] = 0.0
    _, fin = _fwd(lib, c)
    K = c["k"][:, 0, :]
    ref = (np.eye(dk) - K.T @ K) @ c["init_state"][0, 0] + K.T @ c["v"][:, 0, :]
    _close(fin[0, 0], ref, 1e-13, "projection")


def pin_linearity(lib):
    """(S_0, V) -> (o, S_T) is linear for fixed q, k, alpha, beta."""
    rng = np.random.default_rng(RNG_SEED + 5)
    c1 = _rand_case(rng, [9, 4], H=2, dk=4, dv=3)
    c2 = dict(c1)
    c2["v"] = rng.standard_normal(c1["v"].shape)
    c2["init_state"] = rng.standard_normal(c1["init_state"].shape)
    a, b = 0.3, -1.7
    c3 = dict(c1)
    c3["v"] = a * c1["v"] + b * c2["v"]
    c3["init_state"] = a * c1["init_state"] + b * c2["init_state"]
    o1, f1 = _fwd(lib, c1)
    o2, f2 = _fwd(lib, c2)
    o3, f3 = _fwd(lib, c3)
    _close(o3, a * o1 + b * o2, 1e-12, "linear outputs")
    _close(f3, a * f1 + b * f2, 1e-12, "linear state")


def pin_value_columns_separate(lib):
    """Each value column (and state column) evolves on its own."""
    rng = np.random.default_rng(RNG_SEED + 6)
    c = _rand_case(rng, [11], H=1, dk=4, dv=5)
    o, f = _fwd(lib, c)
    cols = [0, 3]
    c2 = dict(c)
    c2["v"] = np.ascontiguousarray(c["v"][:, :, cols])
    c2["init_state"] = np.ascontiguousarray(c["init_state"][..., cols])
    o2, f2 = _fwd(lib, c2)
    _close(o2, o[:, :, cols], 1e-13, "column outputs")
    _close(f2, f[..., cols], 1e-13, "column state")


def pin_chaining(lib):
    """Running [0,t) then [t,T) from the carried state equals one run."""
    rng = np.random.default_rng(RNG_SEED + 7)
    c = _rand_case(rng, [23], H=2, dk=4, dv=3)
    o, f = _fwd(lib, c)
    t = 9
    a = {k_: (v_[:t] if k_ in ("q", "k", "v", "log_alpha", "beta") else v_) for k_, v_ in c.items()}
    a["cu_seqlens"] = np.array([0, t], np.int32)
    oa, fa = _fwd(lib, a)
    b = {k_: (v_[t:] if k_ in ("q", "k", "v", "log_alpha", "beta") else v_) for k_, v_ in c.items()}
    b["cu_seqlens"] = np.array([0, 23 - t], np.int32)
    b["init_state"] = fa
    ob, fb = _fwd(lib, b)
    _close(np.concatenate([oa, ob]), o, 1e-13, "chained outputs")
    _close(fb, f, 1e-13, "chained state")


def pin_varlen_is_separate_runs(lib):
    """A packed batch equals each sequence run alone (zero-length keeps its init)."""
    rng = np.random.default_rng(RNG_SEED + 8)
    lens = [5, 0, 13, 1]
    c = _rand_case(rng, lens, H=2, dk=4, dv=3)
    o, f = _fwd(lib, c)
    cu = c["cu_seqlens"]
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        one = {k_: (v_[sl] if k_ in ("q", "k", "v", "log_alpha", "beta") else v_) for k_, v_ in c.items()}
        one["cu_seqlens"] = np.array([0, lens[s]], np.int32)
        one["init_state"] = c["init_state"][s:s + 1]
        os_, fs = _fwd(lib, one)
        _close(os_, o[sl], 1e-14, f"seq {s} outputs")
        _close(fs[0], f[s], 1e-14, f"seq {s} state")
    _close(f[1], c["init_state"][1], 0.0, "zero-length sequence keeps init")


def pin_non_expansive(lib):
    """Unit keys, beta in [0,1], alpha<=1: ||S_T||_F <= ||S_0||_F + sum_t b_t ||v_t||."""
    rng = np.random.default_rng(RNG_SEED + 9)
    c = _rand_case(rng, [200], H=2, dk=6, dv=4, gate=(0.0, 3.0), init_sd=2.0)
    for T in (1, 17, 200):
        cc = {k_: (v_[:T] if k_ in ("q", "k", "v", "log_alpha", "beta") else v_) for k_, v_ in c.items()}
        cc["cu_seqlens"] = np.array([0, T], np.int32)
        _, f = _fwd(lib, cc)
        for h in range(2):
            bound = np.linalg.norm(c["init_state"][0, h]) + np.sum(
                c["beta"][:T, h] * np.linalg.norm(c["v"][:T, h], axis=-1))
            assert np.linalg.norm(f[0, h]) <= bound * (1 + 1e-12), "state norm grew beyond the bound"


FORWARD_PINS = [pin_identity_when_no_write_no_decay, pin_unit_key_replaces_component, pin_brute_force_products,
                pin_pure_decay, pin_orthonormal_keys_projection, pin_linearity, pin_value_columns_separate,
                pin_chaining, pin_varlen_is_separate_runs, pin_non_expansive]


# ---------------------------------------------------------------------------
# backward pins
# ---------------------------------------------------------------------------
def _loss(lib, c, dO, dS, scale):
    o, f = oracle.kda_fwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["cu_seqlens"],
                          init_state=c["init_state"], scale=scale, nthreads=1, lib=lib)
    return float(np.sum(o * dO) + np.sum(f * dS))


def pin_backward_finite_differences(lib):
    """Every gradient equals central differences of L = <dO, o> + <dS_final, S_T>."""
    rng = np.random.default_rng(RNG_SEED + 10)
    c = _rand_case(rng, [6, 0, 4], H=2, dk=3, dv=2, unit_k=False, gate=(1.0, 1.0))
    scale = 0.6
    dO = rng.standard_normal(c["v"].shape)
    dS = rng.standard_normal(c["init_state"].shape)
    g = oracle.kda_bwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["cu_seqlens"], dO,
                       init_state=c["init_state"], d_final_state=dS, scale=scale, nthreads=2, lib=lib)
    names = ["q", "k", "v", "log_alpha", "beta", "init_state"]
    eps = 1e-6
    for name, grad in zip(names, g):
        x = c[name]
        fd = np.zeros_like(x)
        flat = x.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            lp = _loss(lib, c, dO, dS, scale)
            flat[i] = old - eps
            lm = _loss(lib, c, dO, dS, scale)
            flat[i] = old
            fd.reshape(-1)[i] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - grad))
        assert err <= 1e-7 * max(1.0, np.max(np.abs(fd))), f"d{name}: finite-difference mismatch {err:.3e}"


def pin_backward_autograd(lib):
    """Every gradient equals torch float64 autograd through a naive token loop."""
    import torch

    rng = np.random.default_rng(RNG_SEED + 11)
    c = _rand_case(rng, [70, 5], H=2, dk=4, dv=3, gate=(1.5, 1.0))
    scale = 0.45
    dO = rng.standard_normal(c["v"].shape)
    dS = rng.standard_normal(c["init_state"].shape)
    names = ["q", "k", "v", "log_alpha", "beta", "init_state"]
    tt = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=True) for n in names}
    cu = c["cu_seqlens"]
    outs = []
    fins = []
    for s in range(len(cu) - 1):
        fh = []
        for h in range(c["q"].shape[1]):
            S = tt["init_state"][s, h]
            for t in range(cu[s], cu[s + 1]):
                a = torch.exp(tt["log_alpha"][t, h])
                kk = tt["k"][t, h]
                # S_t = (I - b k k^T) Diag(a) S + b k v^T, written as matrices
                M = torch.eye(kk.shape[0], dtype=torch.float64) - tt["beta"][t, h] * torch.outer(kk, kk)
                S = M @ (a[:, None] * S) + tt["beta"][t, h] * torch.outer(kk, tt["v"][t, h])
                outs.append(((t, h), scale * S.T @ tt["q"][t, h]))
            fh.append(S)
        fins.append(torch.stack(fh))
    L = sum((o * torch.tensor(dO[t, h])).sum() for (t, h), o in outs)
    L = L + (torch.stack(fins) * torch.tensor(dS)).sum()
    L.backward()
    g = oracle.kda_bwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], cu, dO,
                       init_state=c["init_state"], d_final_state=dS, scale=scale, nthreads=2, lib=lib)
    for name, grad in zip(names, g):
        _close(grad, tt[name].grad.numpy(), 1e-11, f"d{name} vs autograd")


def pin_backward_without_final_grad(lib):
    """d_final_state omitted means zero: equals passing explicit zeros."""
    rng = np.random.default_rng(RNG_SEED + 12)
    c = _rand_case(rng, [70], H=1, dk=3, dv=2)
    dO = rng.standard_normal(c["v"].shape)
    a = oracle.kda_bwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["cu_seqlens"], dO,
                       init_state=c["init_state"], d_final_state=None, lib=lib)
    b = oracle.kda_bwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["cu_seqlens"], dO,
                       init_state=c["init_state"], d_final_state=np.zeros_like(c["init_state"]), lib=lib)
    for x, y in zip(a, b):
        _close(x, y, 0.0, "zero final grad")


BACKWARD_PINS = [pin_backward_finite_differences, pin_backward_autograd, pin_backward_without_final_grad]


# ---------------------------------------------------------------------------
# decode / replay pins (state pool indexed per sequence, prefix commit)
# ---------------------------------------------------------------------------
def _decode_case(rng, B, T, H, dk, dv, P, unit_k=False, gate=(0.5, 1.0)):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    la = -np.logaddexp(0.0, -rng.normal(gate[0], gate[1], (B, T, H, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    pool = rng.standard_normal((P, H, dk, dv))
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, state_pool=pool)


def _decode(lib, c, **kw):
    return oracle.kda_decode(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["state_pool"], lib=lib, **kw)


def pin_decode_brute_force(lib):
    """Outputs of every token and the committed prefix state == explicit transition products.

    Slots are gathered through the index list (a permutation with one padding
    entry); each sequence commits a different number of its tokens."""
    rng = np.random.default_rng(RNG_SEED + 20)
    B, T, H, dk, dv, P = 4, 4, 2, 5, 3, 6
    c = _decode_case(rng, B, T, H, dk, dv, P)
    idx = np.array([3, -1, 0, 5], np.int32)
    ncommit = np.array([4, 2, 0, 1], np.int32)
    o, pool = _decode(lib, c, state_indices=idx, num_commit=ncommit, scale=0.41)
    I = np.eye(dk)
    want_pool = c["state_pool"].copy()
    for b in range(B):
        for h in range(H):
            if idx[b] < 0:
                _close(o[b, :, h], np.zeros((T, dv)), 0.0, "padding outputs")
                continue
            S = c["state_pool"][idx[b], h].copy()
            for t in range(T):
                kt, bt = c["k"][b, t, h], c["beta"][b, t, h]
                M = (I - bt * np.outer(kt, kt)) @ np.diag(np.exp(c["log_alpha"][b, t, h]))
                S = M @ S + bt * np.outer(kt, c["v"][b, t, h])
                _close(o[b, t, h], 0.41 * S.T @ c["q"][b, t, h], 1e-12, f"output b={b} t={t}")
                if t + 1 == ncommit[b]:
                    want_pool[idx[b], h] = S
    _close(pool, want_pool, 1e-12, "committed pool")


def pin_decode_commit_then_replay(lib):
    """Commit a prefix, then replay the rest from the written slot: same outputs and final state
    as one call over all tokens; committing nothing leaves the pool bit-identical."""
    rng = np.random.default_rng(RNG_SEED + 21)
    B, T, H, dk, dv, P = 3, 4, 2, 4, 6, 3
    c = _decode_case(rng, B, T, H, dk, dv, P, unit_k=True)
    o_all, pool_all = _decode(lib, c)
    o_none, pool_none = _decode(lib, c, num_commit=np.zeros(B, np.int32))
    _close(pool_none, c["state_pool"], 0.0, "nothing committed")
    _close(o_none, o_all, 0.0, "outputs do not depend on the commit count")
    o_a, pool_a = _decode(lib, c, num_commit=np.full(B, 2, np.int32))
    rest = {n: c[n][:, 2:] for n in ("q", "k", "v", "log_alpha", "beta")}
    rest["state_pool"] = pool_a
    o_b, pool_b = _decode(lib, rest)
    _close(o_b, o_all[:, 2:], 1e-13, "replayed outputs")
    _close(pool_b, pool_all, 1e-13, "replayed final state")


def pin_decode_pure_decay(lib):
    """beta = 0: the committed state is Diag(exp(sum log a)) S_0 in closed form."""
    rng = np.random.default_rng(RNG_SEED + 22)
    B, T, H, dk, dv, P = 2, 3, 1, 4, 2, 2
    c = _decode_case(rng, B, T, H, dk, dv, P, gate=(1.0, 2.0))
    c["beta"][:] = 0.0
    o, pool = _decode(lib, c, state_indices=np.array([1, 0], np.int32))
    for b, slot in ((0, 1), (1, 0)):
        decay = np.exp(np.sum(c["log_alpha"][b, :, 0], axis=0))
        _close(pool[slot, 0], decay[:, None] * c["state_pool"][slot, 0], 1e-13, "pure decay state")
        S = np.exp(np.sum(c["log_alpha"][b, :2, 0], axis=0))[:, None] * c["state_pool"][slot, 0]
        _close(o[b, 1, 0], dk ** -0.5 * S.T @ c["q"][b, 1, 0], 1e-13, "pure decay output")


DECODE_PINS = [pin_decode_brute_force, pin_decode_commit_then_replay, pin_decode_pure_decay]


# ---------------------------------------------------------------------------
# fused input preparation: raw q, k (L2-normalised inside) and a raw gate x
# (log alpha = logsigmoid(x) inside)
# ---------------------------------------------------------------------------
def _raw_case(rng, lengths, H, dk, dv):
    c = _rand_case(rng, lengths, H, dk, dv, unit_k=False, gate=(0.5, 1.5))
    c["q"] *= rng.uniform(0.5, 3.0, size=c["q"].shape[:2] + (1,))
    c["k"] *= rng.uniform(0.5, 3.0, size=c["k"].shape[:2] + (1,))
    c["gate"] = rng.normal(1.0, 2.0, c["log_alpha"].shape)
    return c


def _fused_loss(lib, c, dO, dS):
    o, fin = oracle.kda_fwd_prepped(c["q"], c["k"], c["v"], c["gate"], c["beta"], c["cu_seqlens"],
                                    init_state=c["init_state"], scale=0.6, nthreads=1, lib=lib)
    return float(np.sum(o * dO) + np.sum(fin * dS))


def pin_fused_prep_finite_differences(lib):
    """Gradients with respect to the raw q, k and gate == central differences of the composed forward."""
    rng = np.random.default_rng(RNG_SEED + 30)
    c = _raw_case(rng, [5, 3], H=1, dk=4, dv=3)
    dO = rng.standard_normal(c["v"].shape)
    dS = rng.standard_normal(c["init_state"].shape)
    g = oracle.kda_bwd_prepped(c["q"], c["k"], c["v"], c["gate"], c["beta"], c["cu_seqlens"], dO,
                               init_state=c["init_state"], d_final_state=dS, scale=0.6, nthreads=1, lib=lib)
    h = 1e-6
    for name, grad in (("q", g[0]), ("k", g[1]), ("gate", g[3])):
        x = c[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _fused_loss(lib, c, dO, dS)
            x[idx] = old - h
            lm = _fused_loss(lib, c, dO, dS)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        _close(grad, num, 1e-6, f"d{name} vs central differences")


def pin_fused_prep_row_scale_invariance(lib):
    """Scaling a token's q or k row up by c >= 1 changes nothing but the epsilon term (relative <= 1e-6 / |row|^2)."""
    rng = np.random.default_rng(RNG_SEED + 31)
    c = _raw_case(rng, [9], H=2, dk=6, dv=4)
    o1, f1 = oracle.kda_fwd_prepped(c["q"], c["k"], c["v"], c["gate"], c["beta"], c["cu_seqlens"],
                                    init_state=c["init_state"], lib=lib)
    sc = rng.uniform(2.0, 50.0, size=c["q"].shape[:2] + (1,))
    sc2 = rng.uniform(2.0, 50.0, size=c["q"].shape[:2] + (1,))
    o2, f2 = oracle.kda_fwd_prepped(c["q"] * sc, c["k"] * sc2, c["v"], c["gate"], c["beta"], c["cu_seqlens"],
                                    init_state=c["init_state"], lib=lib)
    _close(o2, o1, 1e-4, "outputs under row scaling")
    _close(f2, f1, 1e-4, "final state under row scaling")


def pin_fused_prep_gate_limits(lib):
    """A saturated gate (x = 40) is no decay: equal to the plain recurrence with log alpha = 0 and
    unit-normalised rows; with beta = 0 the state decays by the product of sigmoid(x) exactly."""
    rng = np.random.default_rng(RNG_SEED + 32)
    c = _raw_case(rng, [7], H=1, dk=4, dv=3)
    c["gate"][:] = 40.0
    o1, f1 = oracle.kda_fwd_prepped(c["q"], c["k"], c["v"], c["gate"], c["beta"], c["cu_seqlens"],
                                    init_state=c["init_state"], qk_l2norm=False, lib=lib)
    o2, f2 = oracle.kda_fwd(c["q"], c["k"], c["v"], np.zeros_like(c["gate"]), c["beta"], c["cu_seqlens"],
                            init_state=c["init_state"], lib=lib)
    _close(o1, o2, 1e-12, "saturated gate outputs")
    _close(f1, f2, 1e-12, "saturated gate state")
    c = _raw_case(rng, [6], H=1, dk=4, dv=3)
    c["beta"][:] = 0.0
    _, f = oracle.kda_fwd_prepped(c["q"], c["k"], c["v"], c["gate"], c["beta"], c["cu_seqlens"],
                                  init_state=c["init_state"], lib=lib)
    decay = np.prod(1.0 / (1.0 + np.exp(-c["gate"][:, 0])), axis=0)
    _close(f[0, 0], decay[:, None] * c["init_state"][0, 0], 1e-13, "pure decay by sigmoid products")


FUSED_PREP_PINS = [pin_fused_prep_finite_differences, pin_fused_prep_row_scale_invariance,
                   pin_fused_prep_gate_limits]


# ---------------------------------------------------------------------------
# short convolution (oracle/short_conv.py): a causal depthwise convolution along
# time with a state of the last W - 1 inputs
# ---------------------------------------------------------------------------
def _conv_case(rng, lengths, D, W, state=True):
    T = int(sum(lengths))
    N = len(lengths)
    return dict(x=rng.standard_normal((T, D)), weight=rng.standard_normal((D, W)), bias=rng.standard_normal(D),
                init_state=rng.standard_normal((N, W - 1, D)) if state else None,
                cu_seqlens=np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64))


def pin_conv_textbook(lib):
    """No state, no bias, identity: each sequence and channel is numpy's full convolution with the
    reversed taps, cut to the sequence length (zero history before the first token)."""
    rng = np.random.default_rng(RNG_SEED + 40)
    for W in (2, 3, 4):
        c = _conv_case(rng, [7, 1, 0, 12, 2], D=5, W=W, state=False)
        y, fin = sc.short_conv_fwd(c["x"], c["weight"], c["cu_seqlens"])
        for n in range(len(c["cu_seqlens"]) - 1):
            a, e = c["cu_seqlens"][n], c["cu_seqlens"][n + 1]
            for ch in range(5 if e > a else 0):   # np.convolve takes no empty input
                ref = np.convolve(c["x"][a:e, ch], c["weight"][ch, ::-1])[: e - a]
                _close(y[a:e, ch], ref, 1e-13, f"W={W} seq {n} ch {ch} vs np.convolve")
            # the state after a sequence holds its last W - 1 inputs (zeros where it is shorter)
            L = e - a
            for r in range(W - 1):
                t = L - (W - 1) + r
                _close(fin[n, r], c["x"][a + t] if t >= 0 else np.zeros(5), 0.0, f"W={W} seq {n} final row {r}")


def pin_conv_state_carries_across_a_split(lib):
    """Running a sequence in two pieces, the first piece's final state as the second's initial state,
    equals one run over the whole sequence (outputs and final state), for every split point."""
    rng = np.random.default_rng(RNG_SEED + 41)
    for W in (2, 4):
        c = _conv_case(rng, [9], D=3, W=W)
        y, fin = sc.short_conv_fwd(c["x"], c["weight"], c["cu_seqlens"], bias=c["bias"], init_state=c["init_state"],
                                   silu=True)
        for cut in range(0, 10):
            y1, f1 = sc.short_conv_fwd(c["x"][:cut], c["weight"], [0, cut], bias=c["bias"],
                                       init_state=c["init_state"], silu=True)
            y2, f2 = sc.short_conv_fwd(c["x"][cut:], c["weight"], [0, 9 - cut], bias=c["bias"], init_state=f1,
                                       silu=True)
            _close(np.concatenate([y1, y2]), y, 1e-13, f"W={W} split at {cut}: outputs")
            _close(f2, fin, 0.0, f"W={W} split at {cut}: final state")


def pin_conv_bias_and_silu(lib):
    """The bias shifts the pre-activation; SiLU is z * sigmoid(z) of it (scipy's expit), with
    silu(0) = 0 and silu(z) -> z for large z."""
    from scipy.special import expit
    rng = np.random.default_rng(RNG_SEED + 42)
    c = _conv_case(rng, [6, 4], D=4, W=3)
    z0, _ = sc.short_conv_fwd(c["x"], c["weight"], c["cu_seqlens"], init_state=c["init_state"])
    y, _ = sc.short_conv_fwd(c["x"], c["weight"], c["cu_seqlens"], bias=c["bias"], init_state=c["init_state"],
                             silu=True)
    z = z0 + c["bias"]
    _close(y, z * expit(z), 1e-13, "bias + SiLU")
    x = np.zeros((3, 1))
    big = sc.short_conv_fwd(x, np.zeros((1, 2)), [0, 3], bias=np.array([40.0]), silu=True)[0]
    zero = sc.short_conv_fwd(x, np.zeros((1, 2)), [0, 3], silu=True)[0]
    _close(zero, np.zeros((3, 1)), 0.0, "silu(0)")
    _close(big, np.full((3, 1), 40.0), 1e-12, "silu(40)")


def _conv_loss(c, dy, dfin, silu):
    y, fin = sc.short_conv_fwd(c["x"], c["weight"], c["cu_seqlens"], bias=c["bias"], init_state=c["init_state"],
                               silu=silu)
    return float(np.sum(y * dy) + np.sum(fin * dfin))


def pin_conv_backward_finite_differences(lib):
    """Every gradient (x, weight, bias, initial state) == central differences of
    <dy, y> + <d_final, final_state>, over sequences longer and shorter than W - 1 and an empty one."""
    rng = np.random.default_rng(RNG_SEED + 43)
    for W, silu in ((4, True), (3, False), (2, True)):
        c = _conv_case(rng, [6, 2, 0, 1, 5], D=2, W=W)
        dy = rng.standard_normal(c["x"].shape)
        dfin = rng.standard_normal(c["init_state"].shape)
        g = sc.short_conv_bwd(c["x"], c["weight"], c["cu_seqlens"], dy, bias=c["bias"], init_state=c["init_state"],
                              d_final_state=dfin, silu=silu)
        h = 1e-6
        for name, grad in (("x", g[0]), ("weight", g[1]), ("bias", g[2]), ("init_state", g[3])):
            v = c[name]
            num = np.zeros_like(v)
            for idx in np.ndindex(v.shape):
                old = v[idx]
                v[idx] = old + h
                lp = _conv_loss(c, dy, dfin, silu)
                v[idx] = old - h
                lm = _conv_loss(c, dy, dfin, silu)
                v[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            _close(grad, num, 1e-6, f"W={W} silu={silu}: d{name} vs central differences")


def pin_conv_decode_is_forward_from_the_slot(lib):
    """A decode step equals the forward over the same tokens started from the slot's state; the
    committed slot holds the state after the committed prefix; padding entries leave everything alone."""
    rng = np.random.default_rng(RNG_SEED + 44)
    B, T, D, W, P = 4, 5, 3, 4, 6
    x = rng.standard_normal((B, T, D))
    w = rng.standard_normal((D, W))
    bias = rng.standard_normal(D)
    pool = rng.standard_normal((P, W - 1, D))
    idx = np.array([3, -1, 0, 5])
    nc = np.array([5, 2, 0, 2])
    y, new = sc.short_conv_decode(x, w, pool, bias=bias, state_indices=idx, num_commit=nc, silu=True)
    touched = set()
    for b in range(B):
        if idx[b] < 0:
            _close(y[b], np.zeros((T, D)), 0.0, "padding outputs")
            continue
        yf, _ = sc.short_conv_fwd(x[b], w, [0, T], bias=bias, init_state=pool[idx[b]][None], silu=True)
        _close(y[b], yf, 1e-13, f"decode seq {b} outputs")
        if nc[b] > 0:
            _, fp = sc.short_conv_fwd(x[b, : nc[b]], w, [0, nc[b]], bias=bias, init_state=pool[idx[b]][None])
            _close(new[idx[b]], fp[0], 0.0, f"decode seq {b} committed state")
            touched.add(int(idx[b]))
    for s in range(P):
        if s not in touched:
            _close(new[s], pool[s], 0.0, f"slot {s} untouched")


SHORT_CONV_PINS = [pin_conv_textbook, pin_conv_state_carries_across_a_split, pin_conv_bias_and_silu,
                   pin_conv_backward_finite_differences, pin_conv_decode_is_forward_from_the_slot]
ALL_PINS = FORWARD_PINS + BACKWARD_PINS + DECODE_PINS + FUSED_PREP_PINS + SHORT_CONV_PINS
