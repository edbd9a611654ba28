"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch each one.

Every mutant is a one-token edit of kda_oracle.c: a dropped term, a wrong
sign, the wrong state read, a missing factor.  A mutant that survives every
pin would mean the pins cannot tell that mistake from the truth.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

# (name, exact text in kda_oracle.c, replacement, occurrence index or None for all)
MUTANTS = [
    ("decay_sign", "double a = exp(la[c]);", "double a = exp(-la[c]);", 0),
    ("delta_sign", "delta[j] = vt[j] - pk;", "delta[j] = vt[j] + pk;", 0),
    ("drop_beta_update", "S[c * dv + j] = P[c * dv + j] + bt * kt[c] * delta[j];",
     "S[c * dv + j] = P[c * dv + j] + kt[c] * delta[j];", 0),
    ("predict_from_undecayed", "for (int c = 0; c < dk; ++c) pk += P[c * dv + j] * kt[c];",
     "for (int c = 0; c < dk; ++c) pk += S[c * dv + j] * kt[c];", 0),
    ("output_reads_old_state", "for (int c = 0; c < dk; ++c) acc += S[c * dv + jj] * qt[c];",
     "for (int c = 0; c < dk; ++c) acc += P[c * dv + jj] * qt[c];", 0),
    ("drop_scale", "j->out[rv + jj] = j->scale * acc;", "j->out[rv + jj] = acc;", 0),
    ("bwd_dk_sign", "j->dk_[rk + c] = bt * gd - pd;", "j->dk_[rk + c] = bt * gd + pd;", 0),
    ("bwd_dla_uses_G", "dla += dP[c * dv + jj] * P[c * dv + jj];", "dla += G[c * dv + jj] * P[c * dv + jj];", 0),
    ("bwd_no_decay_carry", "G[c * dv + jj] = al * dP[c * dv + jj];", "G[c * dv + jj] = dP[c * dv + jj];", 0),
    ("bwd_dbeta_uses_v", "dbt += acc * delta[jj];", "dbt += acc * vt[jj];", 0),
    ("bwd_output_grad_no_scale", "G[c * dv + jj] += j->scale * qt[c] * dot[jj];", "G[c * dv + jj] += qt[c] * dot[jj];", 0),
    ("bwd_ddelta_no_beta", "dd[jj] = bt * acc;", "dd[jj] = acc;", 0),
    ("bwd_dq_old_state", "acc += St[c * dv + jj] * dot[jj];", "acc += Sp[c * dv + jj] * dot[jj];", 0),
    ("bwd_dk_drop_pd", "j->dk_[rk + c] = bt * gd - pd;", "j->dk_[rk + c] = bt * gd;", 0),
    ("bwd_dP_drop_rank1", "dP[c * dv + jj] = G[c * dv + jj] - kt[c] * dd[jj];", "dP[c * dv + jj] = G[c * dv + jj];", 0),
    ("decode_commit_off_by_one", "if (t + 1 == n) memcpy(pool_out", "if (t == n) memcpy(pool_out", 0),
    ("decode_slot_ignores_index", "const int slot = idx[b];", "const int slot = b;", 0),
    ("decode_output_reads_old_state", "for (int c = 0; c < dk; ++c) acc += S[c * dv + jj] * q[rk + c];",
     "for (int c = 0; c < dk; ++c) acc += P[c * dv + jj] * q[rk + c];", 0),
    ("decode_drop_scale", "out[rv + jj] = scale * acc;", "out[rv + jj] = acc;", 0),
    ("bwd_segment_recompute_off_by_one", "const double *Sp = states + (size_t)(t - a) * sz;",
     "const double *Sp = states + (size_t)(t - a + (t > a)) * sz;", 0),
]


def _mutant_source(text, old, new, idx):
    parts = text.split(old)
    assert len(parts) > idx + 1, f"mutation site not found: {old!r}"
    return old.join(parts[: idx + 1]) + new + old.join(parts[idx + 1:])


@pytest.mark.parametrize("name,old,new,idx", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, idx):
    text = open(SRC).read()
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        with open(src, "w") as f:
            f.write(_mutant_source(text, old, new, idx))
        so = oracle.build(src=src, out=os.path.join(d, "libmutant.so"))
        lib = oracle.load(so)
        failures = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(lib)
            except AssertionError as e:
                failures.append(f"{pin.__name__}: {e}")
        assert failures, f"mutant {name} passed every pin"


# Mutants of the short-convolution oracle (oracle/short_conv.py), run against its pins.
CONV_SRC = os.path.join(os.path.dirname(oracle.__file__), "short_conv.py")
CONV_MUTANTS = [
    ("conv_taps_reversed", "z += weight[:, j] * xe[j:j + L]", "z += weight[:, W - 1 - j] * xe[j:j + L]", 0),
    ("conv_state_rows_reversed", "np.concatenate([s0, xs], axis=0)", "np.concatenate([s0[::-1], xs], axis=0)", 0),
    ("conv_final_state_not_advanced", "fin[n] = xe[L:]", "fin[n] = xe[:W - 1]", 0),
    ("conv_bwd_drops_final_grad", "dxe[L:] += dfin[n]", "dxe[L:] += 0.0 * dfin[n]", 0),
    ("conv_bwd_silu_grad_is_sigmoid", "return s * (1.0 + z * (1.0 - s))", "return s", 0),
    ("conv_bwd_weight_taps_reversed", "dw[:, j] += np.sum", "dw[:, W - 1 - j] += np.sum", 0),
    ("conv_decode_commit_off_by_one", "pool[slot] = xe[n:n + W - 1]", "pool[slot] = xe[n - 1:n + W - 2]", 0),
]


@pytest.mark.parametrize("name,old,new,idx", CONV_MUTANTS, ids=[m[0] for m in CONV_MUTANTS])
def test_conv_mutant_is_caught(name, old, new, idx, monkeypatch):
    import importlib.util
    text = open(CONV_SRC).read()
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "short_conv_mutant.py")
        with open(src, "w") as f:
            f.write(_mutant_source(text, old, new, idx))
        spec = importlib.util.spec_from_file_location("short_conv_mutant", src)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
    monkeypatch.setattr(oracle_pins, "sc", mod)
    failures = []
    for pin in oracle_pins.SHORT_CONV_PINS:
        try:
            pin(None)
        except (AssertionError, ValueError) as e:
            failures.append(f"{pin.__name__}: {e}")
    assert failures, f"mutant {name} passed every pin"
