"""The fp64 oracle against the facts that pin it (CPU only).

Also checks that the pins have teeth: copies of the oracle source with one
planted slip each (built with gcc into a temporary directory, on the CPU)
must each fail at least one pin.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.fixture(scope="module")
def orc():
    oracle.compile_oracle()  # always rebuild from the current source
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


# Each mutant: (name, exact text in kda_oracle.c, replacement).  Every text
# must occur exactly once so the list stays in step with the source.
_FORGET = """  for (int r = 0; r < dv; ++r)
    for (int c = 0; c < dk; ++c)
      S[(size_t)r * dk + c] *= alpha[c];
"""
_PREDICT = """  for (int r = 0; r < dv; ++r) {
    double vhat = 0.0;
    for (int c = 0; c < dk; ++c)
      vhat += S[(size_t)r * dk + c] * k[c];
    tmp[r] = beta * (v[r] - vhat);
  }
"""
_WRITE = """  for (int r = 0; r < dv; ++r)
    for (int c = 0; c < dk; ++c)
      S[(size_t)r * dk + c] += tmp[r] * k[c];
"""
_READ = """  for (int r = 0; r < dv; ++r) {
    double acc = 0.0;
    for (int c = 0; c < dk; ++c)
      acc += S[(size_t)r * dk + c] * q[c];
    o[r] = scale * acc;
  }
"""

MUTANTS = [
    ("no_decay", "*= alpha[c];", "*= 1.0;"),
    ("decay_rows", "*= alpha[c];", "*= alpha[r];"),
    ("decay_squared", "*= alpha[c];", "*= alpha[c] * alpha[c];"),
    ("forget_after_predict", _FORGET + "\n  /* predict: vhat = S~ k ; correct: e = beta (v - vhat) */\n" + _PREDICT,
     _PREDICT + "\n" + _FORGET),
    ("read_before_write", _WRITE + "\n  /* read (after the write): o = scale * S q */\n" + _READ,
     _READ + "\n" + _WRITE),
    ("no_beta", "tmp[r] = beta * (v[r] - vhat);", "tmp[r] = (v[r] - vhat);"),
    ("sign_flip", "tmp[r] = beta * (v[r] - vhat);", "tmp[r] = beta * (vhat - v[r]);"),
    ("beta_on_v_only", "tmp[r] = beta * (v[r] - vhat);", "tmp[r] = beta * v[r] - vhat;"),
    ("no_scale", "o[r] = scale * acc;", "o[r] = acc;"),
    ("scale_on_state", "o[r] = scale * acc;",
     "o[r] = scale * acc; for (int c = 0; c < dk; ++c) S[(size_t)r * dk + c] *= scale;"),
    ("read_with_k", "acc += S[(size_t)r * dk + c] * q[c];", "acc += S[(size_t)r * dk + c] * k[c];"),
    ("write_with_q", "S[(size_t)r * dk + c] += tmp[r] * k[c];", "S[(size_t)r * dk + c] += tmp[r] * q[c];"),
    ("predict_with_q", "vhat += S[(size_t)r * dk + c] * k[c];", "vhat += S[(size_t)r * dk + c] * q[c];"),
    ("ignore_S0", "if (S0) memcpy(", "if (0) memcpy("),
    ("alpha_previous_token", "alpha + th * dk,", "alpha + (th >= (size_t)H ? th - H : th) * dk,"),
    ("drop_last_token", "t1 = cu_seqlens[n + 1]; }", "t1 = cu_seqlens[n + 1] - (cu_seqlens[n + 1] > t0); }"),
    ("decode_beta_of_unit0", "alpha + (size_t)u * dk, beta[u],", "alpha + (size_t)u * dk, beta[0],"),
    ("decode_no_scale", "scale, o + (size_t)u * dv, tmp);", "1.0, o + (size_t)u * dv, tmp);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_slip(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutant {name}: anchor text not found once"
    mut_src = tmp_path / f"{name}.c"
    mut_src.write_text(src.replace(old, new))
    lib = str(tmp_path / f"lib{name}.so")
    oracle.compile_oracle(str(mut_src), lib)
    bad = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(bad)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted slip '{name}' passed every pin"
