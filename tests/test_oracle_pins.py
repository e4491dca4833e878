"""The oracle against its pins, and the pins against planted mistakes.

``test_pin`` runs every pin of ``oracle_pins.py`` on the real oracle.
``test_mutant_fails_a_pin`` compiles copies of ``oracle/gdn_oracle.c`` with one
plausible mistake each (a dropped term, a wrong sign, a transposed index, a
wrong head map, ...) and checks that at least one pin rejects every copy.
The mistakes are planted in temporary copies on the CPU; the oracle itself is
never modified.
"""
import os
import shutil
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(None)


MUTANTS = {
    "no_decay": ("h[e] *= alpha;", "h[e] *= 1.0;"),
    "gate_not_exponentiated": ("const double alpha = exp(log_g[t * gb_row]);",
                               "const double alpha = 1.0 + log_g[t * gb_row];"),
    "decay_after_prediction": (
        """        for (long e = 0; e < (long)dk * dv; ++e) h[e] *= alpha;

        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += h[(long)i * dv + j] * kt[i];
""",
        """        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += h[(long)i * dv + j] * kt[i];
        for (long e = 0; e < (long)dk * dv; ++e) h[e] *= alpha;
"""),
    "delta_sign": ("p[j] = b * (vt[j] - p[j]);", "p[j] = b * (vt[j] + p[j]);"),
    "beta_dropped": ("p[j] = b * (vt[j] - p[j]);", "p[j] = (vt[j] - p[j]);"),
    "transposed_prediction": ("p[j] += h[(long)i * dv + j] * kt[i];",
                              "p[j] += h[(long)j * dk + i] * kt[i];"),
    "output_reads_key": ("ot[j] += h[(long)i * dv + j] * qt[i];",
                         "ot[j] += h[(long)i * dv + j] * kt[i];"),
    "output_before_update": (
        """        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) h[(long)i * dv + j] += kt[i] * p[j];

        if (out) {
            double* ot = out + t * out_row;
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) ot[j] += h[(long)i * dv + j] * qt[i];
        }
""",
        """        if (out) {
            double* ot = out + t * out_row;
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) ot[j] += h[(long)i * dv + j] * qt[i];
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) h[(long)i * dv + j] += kt[i] * p[j];
"""),
    "head_map_modulo": ("const int kh = vh / (c->Hv / c->Hk);", "const int kh = vh % c->Hk;"),
    "h0_ignored": ("if (c->h0) memcpy", "if (0) memcpy"),
    "packed_offset": ("r0 = c->cu[b]; L = c->cu[b + 1] - c->cu[b];",
                      "r0 = c->cu[b] + (b > 0); L = c->cu[b + 1] - c->cu[b] - (b > 0);"),
    "decode_head_map": ("const int kh = vh / (Hv / Hk);", "const int kh = vh % Hk;"),
    "decode_prefix_off_by_one": ("st + (long)(r - 1) * dkdv", "st + (long)(r > 1 ? r - 2 : 0) * dkdv"),
    "ba_gate_sign": ("ot[vh] = -exp(a_log[vh]) *", "ot[vh] = exp(a_log[vh]) *"),
    "ba_no_dt_bias": ("softplus(y + dt_bias[vh]);", "softplus(y);"),
    "ba_a_log_not_exponentiated": ("ot[vh] = -exp(a_log[vh]) *", "ot[vh] = -a_log[vh] *"),
    "ba_halves_swapped": ("ot[nv + vh] = 1.0 / (1.0 + exp(-y));", "ot[vh] = 1.0 / (1.0 + exp(-y));"),
    "ba_transposed_weight": ("y += xt[i] * w[(long)o * k + i];", "y += xt[i] * w[(long)i * n + o];"),
    "ba_sigmoid_sign": ("1.0 / (1.0 + exp(-y))", "1.0 / (1.0 + exp(y))"),
    "ba_softplus_no_log": ("log1p(exp(-fabs(z)))", "exp(-fabs(z))"),
    "ba_row_stride": ("x + (long)t * x_stride", "x + (long)t * k"),
    "ba_slot_within": ("const int vh = group * G + (within - G);", "const int vh = (group * G + (within - G) + 1) % nv;"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="gdn_oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, mutant_dir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found in the oracle source"
    path = os.path.join(mutant_dir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = oracle.open_library(oracle.compile_source(path, os.path.join(mutant_dir, f"lib{name}.so")))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the planted mistake {name}"
