"""Plant plausible mistakes in copies of the oracle's C source (on the CPU
only) and check that the pins catch every one of them."""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS, pin_page_magnitudes

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("no_decay", "for (int64_t i = 0; i < dk * dv; ++i) H[i] *= a;", ""),
    ("delta_sign", "p[j] = b * (vt[j] - p[j]);", "p[j] = b * (vt[j] + p[j]);"),
    ("no_beta", "p[j] = b * (vt[j] - p[j]);", "p[j] = (vt[j] - p[j]);"),
    ("read_with_key", "ot[j] += H[i * dv + j] * qt[i];", "ot[j] += H[i * dv + j] * kt[i];"),
    ("no_scale", "ot[j] *= J->scale;", "ot[j] *= 1.0;"),
    ("gqa_modulo", "const int64_t hk = h / (Hv / Hk);", "const int64_t hk = h % Hk;"),
    ("ghost_writes", "if (eos <= bos) return;", "if (eos < bos) return;"),
    ("transposed_update", "H[i * dv + j] += kt[i] * p[j];",
     "H[(i * dv + j) % (dk * dv)] += kt[j % dk] * p[i % dv];"),
    ("beta_on_decay", "const double a = J->gk ? 1.0 : exp(J->g[t * Hv + h]);",
     "const double a = J->gk ? 1.0 : exp(J->g[t * Hv + h]) * J->beta[t * Hv + h];"),
    ("output_before_update",  # read the state before the rank-1 write
     "for (int64_t j = 0; j < dv; ++j) p[j] = b * (vt[j] - p[j]);   /* p now holds d */",
     "for (int64_t j = 0; j < dv; ++j) p[j] = b * (vt[j] - p[j]);"
     " { double *o2 = J->o + (t * Hv + h) * dv; for (int64_t j = 0; j < dv; ++j) { o2[j] = 0.0;"
     " for (int64_t i = 0; i < dk; ++i) o2[j] += H[i * dv + j] * qt[i]; o2[j] *= J->scale; } }"
     " if (0)"),
    ("decay_after_update", "for (int64_t i = 0; i < dk * dv; ++i) H[i] *= a;\n",
     "H[0] *= 1.0;\n"),
    ("chunk_state_early", "(t - bos + 1) % J->every == 0", "(t - bos) % J->every == 0"),
    ("checkpoint_piece_64", "const int64_t c = (t - bos) / J->every;", "const int64_t c = (t - bos) / 64;"),
    ("checkpoint_offsets_64", "(cu[n + 1] - cu[n] + every - 1) / every", "(cu[n + 1] - cu[n] + 63) / 64"),
    ("chunk_state_row", "((J->off[n] + c) * Hv + h)", "((J->off[n] + c) * Hv + (Hv - 1 - h))"),
]


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert old in src, "mutant %s: pattern not found" % name
    src = src.replace(old, new, 1)
    if name == "decay_after_update":
        src = src.replace("double *ot = J->o + (t * Hv + h) * dv;",
                          "for (int64_t i = 0; i < dk * dv; ++i) H[i] *= a;\n"
                          "        double *ot = J->o + (t * Hv + h) * dv;", 1)
    if name == "output_before_update":
        # the original output block must not overwrite the planted early read
        src = src.replace("double *ot = J->o + (t * Hv + h) * dv;\n",
                          "double *ot = J->o + (t * Hv + h) * dv; if (0)\n", 1)
        src = src.replace("for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;",
                          "{ for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0; } if (0)", 1)
        src = src.replace("for (int64_t j = 0; j < dv; ++j) ot[j] *= J->scale;",
                          "if (0) for (int64_t j = 0; j < dv; ++j) ot[j] *= J->scale;", 1)
    c = tmp_path / ("m_%s.c" % name)
    c.write_text(src)
    so = tmp_path / ("m_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(c),
                           "-o", str(so), "-lm"])
    return str(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    so = _build(tmp_path, name, old, new)

    def fwd(*a, **kw):
        return oracle.gdr_fwd(*a, _lib_path=so, **kw)

    caught = []
    for pin in ALL_PINS:
        if pin is pin_page_magnitudes:
            continue  # soft magnitude check; the exact pins must suffice
        try:
            pin(fwd)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name


# Mistakes planted in the backward half of the oracle source; the backward
# pins (against the unmodified, separately pinned forward) must catch each.
BWD_MUTANTS = [
    ("bwd_output_no_scale", "dH[i * dv + j] += J->scale * qt[i] * dot[j];",
     "dH[i * dv + j] += qt[i] * dot[j];"),
    ("bwd_dbeta_sign", "db += dd[j] * (vt[j] - p[j]);", "db += dd[j] * (vt[j] + p[j]);"),
    ("bwd_dp_sign", "dp[j] = -b * dd[j];", "dp[j] = b * dd[j];"),
    ("bwd_dg_no_decay", "dgt += dHd[i] * a * Hp[i];", "dgt += dHd[i] * Hp[i];"),
    ("bwd_state_no_decay", "for (int64_t i = 0; i < S; ++i) dH[i] = a * dHd[i];",
     "for (int64_t i = 0; i < S; ++i) dH[i] = dHd[i];"),
    ("bwd_dk_no_prediction_term", "dkt[i] += s;", "dkt[i] += 0.0 * s;"),
    ("bwd_dq_previous_state", "s += Ht[i * dv + j] * dot[j];", "s += Hp[i * dv + j] * dot[j];"),
    ("bwd_gqa_overwrite", "dq[(t * Hk + h / G) * dk + i] += J.dqv", "dq[(t * Hk + h / G) * dk + i] = J.dqv"),
    ("bwd_no_dht", "if (J->dht) memcpy(dH,", "if (0) memcpy(dH,"),
    ("bwd_recompute_wrong_chunk", "memcpy(Hc, Hs + c * S, sizeof(double) * S);",
     "memcpy(Hc, Hs + (c > 0 ? c - 1 : 0) * S, sizeof(double) * S);"),
    ("bwd_dv_no_beta", "J->dv[(t * Hv + h) * dv + j] = b * dd[j];", "J->dv[(t * Hv + h) * dv + j] = dd[j];"),
    ("bwd_no_dh0", "if (J->dh0) memcpy(J->dh0", "if (J->dh0 && 0) memcpy(J->dh0"),
    ("bwd_ghost_writes", "if (eos <= bos) return;\n    const int64_t L = eos - bos",
     "if (eos < bos) return;\n    const int64_t L = eos - bos"),
]


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_bwd_mutant_is_caught(tmp_path, name, old, new):
    from oracle_bwd_pins import ALL_BWD_PINS
    so = _build(tmp_path, name, old, new)

    def bwd(*a, **kw):
        return oracle.gdr_bwd(*a, _lib_path=so, **kw)

    caught = []
    for pin in ALL_BWD_PINS:
        try:
            pin(bwd, oracle.gdr_fwd)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every backward pin" % name


# Mistakes planted in the per-channel gate path; the KDA pins must catch each.
KDA_MUTANTS = [
    ("kda_reversed_channels", "const double ai = exp(gt[i]);", "const double ai = exp(gt[dk - 1 - i]);"),
    ("kda_one_gate", "const double ai = exp(gt[i]);", "const double ai = exp(gt[0]);"),
    ("kda_gate_of_qk_head", "const double *gt = J->gk + (t * Hv + h) * dk;",
     "const double *gt = J->gk + (t * Hv + hk) * dk;"),
    ("kda_no_channel_decay", "        if (J->gk) {                              /* per-channel decay of the rows of H */",
     "        if (0) {"),
]


@pytest.mark.parametrize("name,old,new", KDA_MUTANTS, ids=[m[0] for m in KDA_MUTANTS])
def test_kda_mutant_is_caught(tmp_path, name, old, new):
    from oracle_kda_pins import ALL_KDA_PINS
    so = _build(tmp_path, name, old, new)

    def fwd(*a, **kw):
        return oracle.gdr_kda_fwd(*a, _lib_path=so, **kw)

    caught = []
    for pin in ALL_KDA_PINS:
        try:
            pin(fwd)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every KDA pin" % name
