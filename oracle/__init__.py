"""Float64 CPU oracle for Kimi Delta Attention (test infrastructure only).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP library never loads it and
shares no code with it.  See kda_oracle.c for the recurrence it computes and
where it comes from (fireworks.ai, "Kimi K3 on Fireworks: Fast RL at frontier
scale", section on Kimi Delta Attention).

Pins: every function here is checked in tests/test_oracle_pins.py against
facts that do not come from this code (closed forms, brute-force products of
explicit transition matrices, invariants, finite differences, autograd).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH, extra=()) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c99", *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [I, I, I, I, P, P, P, P, P, P, P, ctypes.c_double, P, P, P, I, I]
    lib.kda_oracle_fwd.restype = I
    lib.kda_oracle_bwd.argtypes = [I, I, I, I, P, P, P, P, P, P, P, ctypes.c_double, P, P,
                                   P, P, P, P, P, P, P, I, I]
    lib.kda_oracle_bwd.restype = I
    lib.kda_oracle_decode.argtypes = [I, I, I, I, I, I, P, P, P, P, P, ctypes.c_double, P, P, P, P, P]
    lib.kda_oracle_decode.restype = I
    return lib


def load(path: str | None = None):
    """Load the compiled oracle; build it only if it is not there."""
    global _lib
    if path is not None:
        return _bind(path)
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(_LIB_PATH)
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _units(units):
    if units is None:
        return None, 0
    u = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
    return u, u.shape[0]


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def kda_fwd(q, k, v, log_alpha, beta, cu_seqlens, init_state=None, scale=None,
            units=None, nthreads=None, lib=None):
    """o[n_tok,H,dv], final_state[N,H,dk,dv] in float64.

    q,k,log_alpha [n_tok,H,dk]; v [n_tok,H,dv]; beta [n_tok,H]; cu_seqlens [N+1].
    scale=None means dk**-0.5.  units: iterable of (seq, head) to compute (others stay NaN).
    """
    lib = lib or load()
    q, k, v, log_alpha, beta, init_state = map(_f64, (q, k, v, log_alpha, beta, init_state))
    n_tok, H, dk = q.shape
    dv = v.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ns = cu.shape[0] - 1
    if scale is None:
        scale = dk ** -0.5
    out = np.full((n_tok, H, dv), np.nan)
    fin = np.full((ns, H, dk, dv), np.nan)
    u, nu = _units(units)
    rc = lib.kda_oracle_fwd(H, dk, dv, ns, _ptr(cu), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                            _ptr(init_state), float(scale), _ptr(out), _ptr(fin), _ptr(u), nu,
                            nthreads or default_threads())
    if rc:
        raise RuntimeError(f"kda_oracle_fwd failed: {rc}")
    return out, fin


def kda_bwd(q, k, v, log_alpha, beta, cu_seqlens, d_out, init_state=None, d_final_state=None,
            scale=None, units=None, nthreads=None, lib=None):
    """Gradients (dq, dk, dv, dlog_alpha, dbeta, d_init_state) in float64."""
    lib = lib or load()
    q, k, v, log_alpha, beta, init_state, d_out, d_final_state = map(
        _f64, (q, k, v, log_alpha, beta, init_state, d_out, d_final_state))
    n_tok, H, dk = q.shape
    dv = v.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ns = cu.shape[0] - 1
    if scale is None:
        scale = dk ** -0.5
    dq = np.full((n_tok, H, dk), np.nan)
    dkk = np.full((n_tok, H, dk), np.nan)
    dvv = np.full((n_tok, H, dv), np.nan)
    dla = np.full((n_tok, H, dk), np.nan)
    db = np.full((n_tok, H), np.nan)
    dinit = np.full((ns, H, dk, dv), np.nan)
    u, nu = _units(units)
    rc = lib.kda_oracle_bwd(H, dk, dv, ns, _ptr(cu), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                            _ptr(init_state), float(scale), _ptr(d_out), _ptr(d_final_state),
                            _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dla), _ptr(db), _ptr(dinit), _ptr(u), nu,
                            nthreads or default_threads())
    if rc:
        raise RuntimeError(f"kda_oracle_bwd failed: {rc}")
    return dq, dkk, dvv, dla, db, dinit


def kda_decode(q, k, v, log_alpha, beta, state_pool, state_indices=None, num_commit=None, scale=None, lib=None):
    """Decode / replay step in float64: (out [B,T,H,dv], new pool [P,H,dk,dv]).

    q,k,log_alpha [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]; state_pool [P,H,dk,dv].
    state_indices [B] (None: sequence b uses slot b; outside [0, P): padding, outputs 0).
    num_commit [B] (None: all T tokens): the pool slot receives the state after that many tokens.
    """
    lib = lib or load()
    q, k, v, log_alpha, beta, pool = map(_f64, (q, k, v, log_alpha, beta, state_pool))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    P = pool.shape[0]
    idx = np.ascontiguousarray(np.arange(B) if state_indices is None else state_indices, dtype=np.int32)
    nc = None if num_commit is None else np.ascontiguousarray(num_commit, dtype=np.int32)
    if scale is None:
        scale = dk ** -0.5
    out = np.full((B, T, H, dv), np.nan)
    new_pool = pool.copy()
    rc = lib.kda_oracle_decode(H, dk, dv, B, T, P, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                               float(scale), _ptr(pool), _ptr(idx), _ptr(nc), _ptr(out), _ptr(new_pool))
    if rc:
        raise RuntimeError(f"kda_oracle_decode failed: {rc}")
    return out, new_pool


# ---------------------------------------------------------------------------
# Fused input preparation (the step upstream of the recurrence in the same
# page's KDA workloads): q and k are L2-normalised per (token, head) over the
# key channels, and the decay comes from a raw gate x as log alpha =
# logsigmoid(x).  The pages fix neither an epsilon nor the gate's
# parametrisation beyond that form; the library's reading is
#     l2n(x) = x / sqrt(sum(x^2) + L2N_EPS),   log alpha = -log(1 + exp(-x)).
# The functions below compose those maps with kda_fwd / kda_bwd / kda_decode
# in float64, and take the backward through them by the chain rule:
#     d raw_q = s (d q^ - q^ (q^ . d q^)),  s = (sum(q^2) + eps)^-1/2
#     d x     = d log_alpha * sigmoid(-x)
# ---------------------------------------------------------------------------
L2N_EPS = 1e-6


def l2n(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2N_EPS)


def l2n_backward(x, g):
    """Gradient with respect to x of <g, l2n(x)>."""
    x = np.asarray(x, dtype=np.float64)
    s = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2N_EPS)
    xh = x * s
    return s * (g - xh * np.sum(xh * g, axis=-1, keepdims=True))


def logsigmoid(x):
    return -np.logaddexp(0.0, -np.asarray(x, dtype=np.float64))


def logsigmoid_backward(x, g):
    """Gradient with respect to x of <g, logsigmoid(x)>."""
    return np.asarray(g, dtype=np.float64) * np.exp(logsigmoid(-np.asarray(x, dtype=np.float64)))


def _prep(q, k, gate, qk_l2norm, gate_logsigmoid):
    return (l2n(q) if qk_l2norm else q, l2n(k) if qk_l2norm else k,
            logsigmoid(gate) if gate_logsigmoid else gate)


def kda_fwd_prepped(q, k, v, gate, beta, cu_seqlens, init_state=None, scale=None, qk_l2norm=True,
                    gate_logsigmoid=True, units=None, nthreads=None, lib=None):
    """kda_fwd on l2n(q), l2n(k) and log alpha = logsigmoid(gate) (each map only when asked)."""
    qh, kh, la = _prep(q, k, gate, qk_l2norm, gate_logsigmoid)
    return kda_fwd(qh, kh, v, la, beta, cu_seqlens, init_state=init_state, scale=scale, units=units,
                   nthreads=nthreads, lib=lib)


def kda_bwd_prepped(q, k, v, gate, beta, cu_seqlens, d_out, init_state=None, d_final_state=None, scale=None,
                    qk_l2norm=True, gate_logsigmoid=True, units=None, nthreads=None, lib=None):
    """Gradients with respect to the raw q, k and gate (and v, beta, init_state) of the prepped forward."""
    qh, kh, la = _prep(q, k, gate, qk_l2norm, gate_logsigmoid)
    dq, dk, dv, dla, db, dinit = kda_bwd(qh, kh, v, la, beta, cu_seqlens, d_out, init_state=init_state,
                                         d_final_state=d_final_state, scale=scale, units=units,
                                         nthreads=nthreads, lib=lib)
    if qk_l2norm:
        dq, dk = l2n_backward(q, dq), l2n_backward(k, dk)
    if gate_logsigmoid:
        dla = logsigmoid_backward(gate, dla)
    return dq, dk, dv, dla, db, dinit


def kda_decode_prepped(q, k, v, gate, beta, state_pool, state_indices=None, num_commit=None, scale=None,
                       qk_l2norm=True, gate_logsigmoid=True, lib=None):
    qh, kh, la = _prep(q, k, gate, qk_l2norm, gate_logsigmoid)
    return kda_decode(qh, kh, v, la, beta, state_pool, state_indices=state_indices, num_commit=num_commit,
                      scale=scale, lib=lib)
