"""Float64 CPU oracle for the KDA short convolution (test infrastructure only).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never loads it and
shares no code with it.

What it computes.  fireworks.ai, "Kimi K3 on Fireworks: Fast RL at frontier
scale", section on disaggregated prefill and decode: the per-sequence KDA state
handed between serving pools is a recurrent state plus a convolution state.
The page defines neither; parity against the page is therefore unpinned.  The
reading implemented here is the plainest one consistent with a "convolution
state" beside a recurrent one: a causal depthwise convolution along time of
width W over each channel, whose state is the last W - 1 inputs of the
sequence,

    z[t, c] = bias[c] + sum_{j=0}^{W-1} weight[c, j] * X[t - (W-1) + j, c]
    y[t, c] = z            (identity)     or     z * sigmoid(z)   (SiLU),

where X is the sequence's input preceded by its W - 1 state rows (state row i
stands for time i - (W - 1); zero when no state is given), and the final state
is the last W - 1 rows of that extended input.

Pins (tests/oracle_pins.py): the numpy textbook convolution (np.convolve) for
a sequence without state, splitting a sequence and carrying the state across
the split, finite differences for every gradient, and the decode step against
running the same tokens through the forward from the pool slot.
"""
from __future__ import annotations

import numpy as np


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _silu_grad(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def _bounds(cu_seqlens, T):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    return cu


def _extended(xs, s0, W):
    """The sequence's input with its W - 1 state rows in front (time -(W-1) .. len-1)."""
    return np.concatenate([s0, xs], axis=0)


def _pre_activation(xe, weight, bias, L):
    W = weight.shape[1]
    z = np.broadcast_to(bias, (L, weight.shape[0])).copy()
    for j in range(W):
        z += weight[:, j] * xe[j:j + L]
    return z


def short_conv_fwd(x, weight, cu_seqlens, bias=None, init_state=None, silu=False):
    """x: [T, D] packed sequences; weight: [D, W]; bias: [D] or None;
    init_state: [N, W-1, D] or None (zero).  Returns y [T, D] and the final
    state [N, W-1, D] (the last W - 1 rows of each extended input)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(weight, np.float64)
    T, D = x.shape
    W = w.shape[1]
    cu = _bounds(cu_seqlens, T)
    N = len(cu) - 1
    b = np.zeros(D) if bias is None else np.asarray(bias, np.float64)
    s0 = np.zeros((N, W - 1, D)) if init_state is None else np.asarray(init_state, np.float64)
    y = np.zeros((T, D))
    fin = np.zeros((N, W - 1, D))
    for n in range(N):
        a, e = cu[n], cu[n + 1]
        L = e - a
        xe = _extended(x[a:e], s0[n], W)
        z = _pre_activation(xe, w, b, L)
        y[a:e] = _silu(z) if silu else z
        fin[n] = xe[L:]
    return y, fin


def short_conv_bwd(x, weight, cu_seqlens, dy, bias=None, init_state=None, d_final_state=None, silu=False):
    """Gradients of <dy, y> + <d_final_state, final_state> with respect to x,
    weight, bias and init_state (chain rule through the definition above)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(weight, np.float64)
    dy = np.asarray(dy, np.float64)
    T, D = x.shape
    W = w.shape[1]
    cu = _bounds(cu_seqlens, T)
    N = len(cu) - 1
    b = np.zeros(D) if bias is None else np.asarray(bias, np.float64)
    s0 = np.zeros((N, W - 1, D)) if init_state is None else np.asarray(init_state, np.float64)
    dfin = np.zeros((N, W - 1, D)) if d_final_state is None else np.asarray(d_final_state, np.float64)
    dx = np.zeros((T, D))
    dw = np.zeros((D, W))
    db = np.zeros(D)
    dinit = np.zeros((N, W - 1, D))
    for n in range(N):
        a, e = cu[n], cu[n + 1]
        L = e - a
        xe = _extended(x[a:e], s0[n], W)
        z = _pre_activation(xe, w, b, L)
        dz = dy[a:e] * _silu_grad(z) if silu else dy[a:e].copy()
        dxe = np.zeros_like(xe)
        for j in range(W):
            dxe[j:j + L] += w[:, j] * dz
            dw[:, j] += np.sum(dz * xe[j:j + L], axis=0)
        dxe[L:] += dfin[n]          # the final state is the last W - 1 extended rows
        db += dz.sum(axis=0)
        dx[a:e] = dxe[W - 1:]
        dinit[n] = dxe[:W - 1]
    return dx, dw, db, dinit


def short_conv_decode(x, weight, state_pool, bias=None, state_indices=None, num_commit=None, silu=False):
    """Decode / replay step of the convolution: x [B, T, D]; state_pool
    [P, W-1, D].  Sequence b continues from pool slot state_indices[b]
    (slot b when None; a slot outside [0, P) is padding: zero outputs, no
    state touched), produces y [B, T, D] for all T tokens, and the state
    after its first num_commit[b] tokens (clamped to [0, T]; all T when None)
    replaces the slot.  Returns (y, new pool)."""
    x = np.asarray(x, np.float64)
    B, T, D = x.shape
    w = np.asarray(weight, np.float64)
    W = w.shape[1]
    pool = np.array(state_pool, np.float64, copy=True)
    P = pool.shape[0]
    b = np.zeros(D) if bias is None else np.asarray(bias, np.float64)
    y = np.zeros((B, T, D))
    for i in range(B):
        slot = i if state_indices is None else int(state_indices[i])
        if not 0 <= slot < P:
            continue
        n = T if num_commit is None else min(max(int(num_commit[i]), 0), T)
        xe = _extended(x[i], pool[slot], W)
        z = _pre_activation(xe, w, b, T)
        y[i] = _silu(z) if silu else z
        if n > 0:
            pool[slot] = xe[n:n + W - 1]
    return y, pool
