"""The oracle's pins must catch plausible mistakes.

Each case below copies wall_oracle.c to a temporary directory, plants one
mistake in the copy (a dropped term, a wrong sign, a shifted index, a wrong
head map, ...), builds it with gcc and runs every pin of test_oracle_pins.py
against the mutant.  At least one pin has to fail.  CPU only; the committed
oracle is never modified.
"""

import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "wall_oracle.c")

MUTANTS = {
    "gate_index_j_instead_of_j_plus_1": (
        "const double *gr = g + ((b * T + (j + 1)) * HQ + hq) * K;",
        "const double *gr = g + ((b * T + j) * HQ + hq) * K;"),
    "gate_sign": ("F[n] *= exp(gr[n]);", "F[n] *= exp(-gr[n]);"),
    "sink_dropped_from_normaliser": ("if (sink) Z += exp(sink[hq] - m);", ";"),
    "gqa_head_map_modulo": ("const int64_t h = hq / group;", "const int64_t h = hq % H;"),
    "window_off_by_one": ("i - window + 1 > lo) lo = i - window + 1;",
                          "i - window > lo) lo = i - window;"),
    "scale_applied_to_fox_bias": ("logit[cnt++] = scale * dot + fox;",
                                  "logit[cnt++] = scale * (dot + fox);"),
    "fox_index_j": ("fox += g_scalar[(b * T + (j + 1)) * HQ + hq];",
                    "fox += g_scalar[(b * T + j) * HQ + hq];"),
    "sequence_start_ignored": ("if (cu_seqlens[s] <= i && i < cu_seqlens[s + 1]) s0 = cu_seqlens[s];",
                               "(void)s;"),
    "value_of_wrong_key": ("const double *vj = v + ((b * T + j) * H + h) * V;",
                           "const double *vj = v + ((b * T + i) * H + h) * V;"),
    "lse_without_max": ("lse[(b * T + i) * HQ + hq] = m + log(Z);",
                        "lse[(b * T + i) * HQ + hq] = log(Z);"),
    "query_key_swapped_heads": ("const double *kj = k + ((b * T + j) * H + h) * K;",
                                "const double *kj = k + ((b * T + j) * H + (hq % H)) * K;"),
    "scan_scale_dropped": ("out[(b * T + t) * C + c] = scale * run;",
                           "out[(b * T + t) * C + c] = run;"),
    "scan_no_reset_at_sequence_start": ("if (t == cu_seqlens[s]) run = 0.0;", ";"),
    "cache_factor_sign": ("kt[n] = kj[n] * exp2(R[n] - Pj[n]);", "kt[n] = kj[n] * exp2(Pj[n] - R[n]);"),
    "cache_anchor_never_moves": ("if (r - pj > CACHE_SPAN) r = floor(pj);", ";"),
    "cache_anchor_moves_to_unfloored_prefix": ("if (r - pj > CACHE_SPAN) r = floor(pj);",
                                               "if (r - pj > CACHE_SPAN) r = pj;"),
    "cache_key_head_of_query": ("const double *kj = k + ((b * T + j) * H + kvh) * K;",
                                "const double *kj = k + ((b * T + j) * H + hq % H) * K;"),
    "decode_query_factor_sign": ("dot += qi[n] * exp2(pc[n] - R[n]) * kt[n];",
                                 "dot += qi[n] * exp2(R[n] - pc[n]) * kt[n];"),
    "decode_anchor_of_next_chunk": ("const int64_t c = j / C;", "const int64_t c = (j + 1 < T ? j + 1 : j) / C;"),
    "decode_sink_dropped": ("if (sink != NULL) Z += exp(sink[hq] - m);", ";"),
    "decode_scale_dropped": ("logit[j] = scale * dot;", "logit[j] = dot;"),
    "decode_value_head": ("const double *vj = v + ((b * T + j) * H + kvh) * V;",
                          "const double *vj = v + ((b * T + j) * H + 0) * V;"),
    "bwd_dS_without_D": ("const double dS = a * (dpv - Di);", "const double dS = a * dpv;"),
    "bwd_dk_decay_dropped": ("dkj[n] += scale * dS * Fj[n] * qi[n];", "dkj[n] += scale * dS * qi[n];"),
    "bwd_dv_unweighted": ("for (int64_t d = 0; d < V; ++d) dvj[d] += a * doi[d];",
                          "for (int64_t d = 0; d < V; ++d) dvj[d] += doi[d];"),
    "bwd_dg_key_term_sign": ("run += q[tk * K + n] * dq[tk * K + n] - k[((b * T + t) * H + hk) * K + n] * dkh[tk * K + n];",
                             "run += q[tk * K + n] * dq[tk * K + n] + k[((b * T + t) * H + hk) * K + n] * dkh[tk * K + n];"),
    "bwd_dgs_row_sums_only": ("run += grow[tk] - gcol[tk];", "run += grow[tk];"),
    "bwd_dsink_sign": ("if (sink) sk[b * HQ + hq] -= exp(sink[hq] - lse) * Di;",
                       "if (sink) sk[b * HQ + hq] += exp(sink[hq] - lse) * Di;"),
}


def _pin_calls():
    """Every (name, zero-arg callable(oracle_module)) pin in test_oracle_pins."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argname, values = params[0].args
            for val in values:
                calls.append((f"{name}[{val}]", lambda mod, fn=fn, a=argname, v=val: fn(mod, **{a: v})))
        else:
            calls.append((name, lambda mod, fn=fn: fn(mod)))
    return calls


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, tmp_path, monkeypatch):
    old, new = MUTANTS[mutant]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mpath = tmp_path / "wall_oracle_mutant.c"
    mpath.write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", str(lib),
                    str(mpath), "-lm"], check=True, capture_output=True)
    monkeypatch.setattr(oracle, "_lib", oracle._bind(str(lib)))
    caught = []
    for name, call in _pin_calls():
        try:
            call(oracle)
        except (AssertionError, ValueError):
            caught.append(name)
    assert caught, f"no pin caught the planted mistake {mutant}"


def test_unmutated_copy_passes_every_pin(tmp_path, monkeypatch):
    lib = tmp_path / "libcopy.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", str(lib),
                    SRC, "-lm"], check=True, capture_output=True)
    monkeypatch.setattr(oracle, "_lib", oracle._bind(str(lib)))
    for name, call in _pin_calls():
        call(oracle)
