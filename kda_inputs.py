"""Seeded synthetic inputs for Kimi Delta Attention workloads.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic, so both the float64 oracle and the
HIP library can be fed from it without sharing any of the method's code.

Workloads (sizes and value distributions of the KDA benchmark shapes: H=16
heads, head dim 128, bf16, sequence lengths 4K-128K, plus a small fp32 case):

  cfg0  fp32  B=1 H=2  T=256     d=64   gate x~N(3,1)    init=0
  cfg1  bf16  B=1 H=16 T=4096    d=128  gate x~N(3,1)    init~N(0,0.02)
  cfg2  bf16  B=1 H=16 T=32768   d=128  gate x~N(2,1.5)  init~N(0,0.02)
  cfg3  bf16  B=1 H=16 T=131072  d=128  gate x~N(3,1)    init~N(0,0.02)
  cfg4  bf16  varlen 8 seqs, L_i~U[1024,32768], H=16 d=128, fwd+bwd,
        per-sequence init~N(0,0.02); dO~N(0,1) (bf16), dS_final~N(0,1) (fp32)

Common recipe: q,k ~ N(0,1) then L2-normalised over the key channels of each
(token, head); v ~ N(0,1); log_alpha = logsigmoid(x); beta = sigmoid(N(0,1)).
The second argument of N(mu, s) is read as a standard deviation.

Every tensor is drawn from its own PCG64 stream keyed by (seed, tensor name),
so the draw order does not matter and a tensor can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np

__all__ = ["Workload", "CONFIGS", "config", "make_inputs", "bf16_round", "bf16_bits",
           "bits_to_f32", "lengths_to_cu", "decode_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": storage dtype of q,k,v,log_alpha,beta,out,grads
    B: int
    T: int                # tokens per row (ignored when lengths is set)
    H: int
    dk: int
    dv: int
    gate_mu: float
    gate_sd: float
    init_sd: float        # 0 => init_state is zero
    lengths: tuple | None = None   # varlen: per-sequence lengths (B must be 1)
    varlen_n: int = 0              # draw this many lengths from U[lo, hi] when lengths is None
    varlen_lo: int = 0
    varlen_hi: int = 0
    backward: bool = False
    seed: int = 0

    @property
    def total_tokens(self) -> int:
        if self.lengths is not None:
            return int(sum(self.lengths))
        return self.B * self.T


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(name.encode())])))


def _draw_lengths(w: Workload) -> tuple:
    r = _rng(w.seed, "lengths")
    return tuple(int(x) for x in r.integers(w.varlen_lo, w.varlen_hi + 1, size=w.varlen_n))


_BASE = dict(B=1, H=16, dk=128, dv=128, gate_mu=3.0, gate_sd=1.0, init_sd=0.02, dtype="bf16")

CONFIGS = {
    0: Workload(name="kda_fwd_f32_H2_T256_d64", dtype="f32", B=1, T=256, H=2, dk=64, dv=64,
                gate_mu=3.0, gate_sd=1.0, init_sd=0.0, seed=0),
    1: Workload(name="kda_fwd_bf16_H16_T4096_d128", T=4096, seed=1, **{k: v for k, v in _BASE.items()}),
    2: Workload(name="kda_fwd_bf16_H16_T32768_d128_sharp_gate", T=32768, seed=2,
                **{**_BASE, "gate_mu": 2.0, "gate_sd": 1.5}),
    3: Workload(name="kda_fwd_bf16_H16_T131072_d128", T=131072, seed=3, **_BASE),
    4: Workload(name="kda_fwdbwd_bf16_varlen8_U1K-32K_H16_d128", T=0, varlen_n=8, varlen_lo=1024,
                varlen_hi=32768, backward=True, seed=4, **_BASE),
}


def config(i: int) -> Workload:
    """The workload with its varlen lengths resolved (drawn from the seed)."""
    w = CONFIGS[i]
    if w.varlen_n and w.lengths is None:
        w = dataclasses.replace(w, lengths=_draw_lengths(w))
    return w


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (kept as float32)."""
    return bits_to_f32(bf16_bits(x))


def lengths_to_cu(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def make_inputs(w: Workload, heads=None, with_grads=None, raw=False) -> dict:
    """Draw the inputs of workload w as float32 numpy arrays holding values
    exactly representable in the storage dtype.

    raw=True: the values before input preparation, for kernels that prepare
    them themselves: q, k as drawn (N(0,1), not normalised) and "log_alpha"
    holding the raw gate x instead of logsigmoid(x).

    Token-major packed layout: q,k,log_alpha [N_tok,H,dk]; v [N_tok,H,dv];
    beta [N_tok,H]; init_state [num_seqs,H,dk,dv] float32 (or None);
    cu_seqlens int32 [num_seqs+1]. With heads=[...] only those heads are kept
    (the full tensors are still drawn, so values match the full run).
    """
    if w.varlen_n and w.lengths is None:
        w = dataclasses.replace(w, lengths=_draw_lengths(w))
    if w.lengths is not None:
        lengths = list(w.lengths)
    else:
        lengths = [w.T] * w.B
    n_tok = int(sum(lengths))
    ns = len(lengths)
    H, dk, dv = w.H, w.dk, w.dv
    s = w.seed
    hs = slice(None) if heads is None else list(heads)

    def draw(name, shape, mu=0.0, sd=1.0):
        return _rng(s, name).standard_normal(size=shape, dtype=np.float32) * np.float32(sd) + np.float32(mu)

    prep = (lambda a: a) if raw else _unit_rows
    q = prep(draw("q", (n_tok, H, dk)))[:, hs]
    k = prep(draw("k", (n_tok, H, dk)))[:, hs]
    v = draw("v", (n_tok, H, dv))[:, hs]
    x = draw("gate_x", (n_tok, H, dk), w.gate_mu, w.gate_sd)[:, hs].astype(np.float64)
    log_alpha = x if raw else -np.logaddexp(0.0, -x)          # logsigmoid(x)
    bl = draw("beta_logit", (n_tok, H))[:, hs].astype(np.float64)
    beta = 1.0 / (1.0 + np.exp(-bl))
    out = dict(
        q=_store(q, w.dtype), k=_store(k, w.dtype), v=_store(v, w.dtype),
        log_alpha=_store(log_alpha, w.dtype), beta=_store(beta, w.dtype),
        cu_seqlens=lengths_to_cu(lengths), lengths=lengths, workload=w,
    )
    if w.init_sd > 0:
        out["init_state"] = np.ascontiguousarray(draw("init_state", (ns, H, dk, dv), 0.0, w.init_sd)[:, hs])
    else:
        out["init_state"] = None
    if with_grads if with_grads is not None else w.backward:
        out["d_out"] = _store(draw("d_out", (n_tok, H, dv))[:, hs], w.dtype)
        out["d_final_state"] = np.ascontiguousarray(draw("d_final_state", (ns, H, dk, dv))[:, hs])
    for key in ("q", "k", "v", "log_alpha", "beta", "d_out"):
        if key in out:
            out[key] = np.ascontiguousarray(out[key])
    return out


def small(dtype="f32", lengths=(100,), H=2, dk=64, dv=64, gate_mu=3.0, gate_sd=1.0, init_sd=0.02,
          seed=1234, backward=True) -> Workload:
    """A small varlen workload for tests (any lengths, including 0 and ragged tails)."""
    return Workload(name="small", dtype=dtype, B=1, T=0, H=H, dk=dk, dv=dv, gate_mu=gate_mu,
                    gate_sd=gate_sd, init_sd=init_sd, lengths=tuple(int(x) for x in lengths),
                    backward=backward, seed=seed)


def decode_inputs(B, T, H, dk, dv, pool_size, dtype="bf16", gate_mu=3.0, gate_sd=1.0, state_sd=0.5,
                  seed=4321, raw=False) -> dict:
    """Inputs of a decode / replay step: B sequences of T tokens each, token-major
    [B,T,H,.] (same value recipe as the workloads above), and a float32 state
    pool [pool_size,H,dk,dv] ~ N(0, state_sd) standing in for states left by
    earlier tokens."""
    def draw(name, shape, mu=0.0, sd=1.0):
        return _rng(seed, "decode_" + name).standard_normal(size=shape, dtype=np.float32) * np.float32(sd) \
            + np.float32(mu)

    prep = (lambda a: a) if raw else _unit_rows
    q = prep(draw("q", (B, T, H, dk)))
    k = prep(draw("k", (B, T, H, dk)))
    v = draw("v", (B, T, H, dv))
    x = draw("gate_x", (B, T, H, dk), gate_mu, gate_sd).astype(np.float64)
    log_alpha = x if raw else -np.logaddexp(0.0, -x)          # logsigmoid(x), or the raw gate
    beta = 1.0 / (1.0 + np.exp(-draw("beta_logit", (B, T, H)).astype(np.float64)))
    out = {name: np.ascontiguousarray(_store(a, dtype)) for name, a in
           (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta))}
    out["state_pool"] = np.ascontiguousarray(draw("state", (pool_size, H, dk, dv), 0.0, state_sd))
    return out


def conv_inputs(lengths, D, W, dtype="bf16", seed=777, state=True) -> dict:
    """Inputs of the short convolution over packed sequences (channels D = the
    concatenated q, k, v channels of all heads in the benchmark shapes):
    x [T, D] ~ N(0, 1) and dy [T, D] ~ N(0, 1) in the storage dtype;
    weight [D, W] ~ U(-1/sqrt(W), 1/sqrt(W)) and bias [D] ~ N(0, 0.1) in float32;
    per-sequence state and final-state gradient [N, W-1, D] ~ N(0, 1) in float32
    (the state None when state=False)."""
    def draw(name, shape, sd=1.0):
        return _rng(seed, "conv_" + name).standard_normal(size=shape, dtype=np.float32) * np.float32(sd)

    lengths = [int(n) for n in lengths]
    T, N = int(sum(lengths)), len(lengths)
    lim = np.float32(1.0 / np.sqrt(W))
    return dict(
        x=np.ascontiguousarray(_store(draw("x", (T, D)), dtype)),
        dy=np.ascontiguousarray(_store(draw("dy", (T, D)), dtype)),
        weight=_rng(seed, "conv_weight").uniform(-lim, lim, size=(D, W)).astype(np.float32),
        bias=draw("bias", (D,), 0.1),
        init_state=draw("state", (N, W - 1, D)) if state else None,
        d_final_state=draw("d_final", (N, W - 1, D)),
        cu_seqlens=lengths_to_cu(lengths),
    )


def conv_decode_inputs(B, T, D, W, pool_size, dtype="bf16", seed=778) -> dict:
    """Inputs of a short-convolution decode step: x [B, T, D] ~ N(0, 1) in the
    storage dtype, weight and bias as in conv_inputs, and a float32 pool of
    states [pool_size, W-1, D] ~ N(0, 1)."""
    def draw(name, shape, sd=1.0):
        return _rng(seed, "convdec_" + name).standard_normal(size=shape, dtype=np.float32) * np.float32(sd)

    lim = np.float32(1.0 / np.sqrt(W))
    return dict(
        x=np.ascontiguousarray(_store(draw("x", (B, T, D)), dtype)),
        weight=_rng(seed, "convdec_weight").uniform(-lim, lim, size=(D, W)).astype(np.float32),
        bias=draw("bias", (D,), 0.1),
        state_pool=draw("state", (pool_size, W - 1, D)),
    )
