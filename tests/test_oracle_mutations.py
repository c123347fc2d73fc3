"""Plant plausible mistakes in copies of the C oracle (on the CPU) and check that
the pin battery catches every one of them. This is what makes the pins worth
trusting: a dropped term, a wrong sign, a wrong index or a transposed operand in
the oracle would fail at least one pin."""
import functools
import os
import re

import pytest

import oracle
from oracle import kda_oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(kda_oracle.__file__), "kda_oracle.c")


def _replace(old, new):
    def f(text):
        assert text.count(old) == 1, old
        return text.replace(old, new)
    return f


def _block(text, name):
    m = re.search(r"( *)/\* \[%s\].*?/\* \[/%s\] \*/\n" % (name, name), text, re.S)
    assert m, name
    return m.group(0)


def _swap(a, b):
    def f(text):
        ba, bb = _block(text, a), _block(text, b)
        return text.replace(ba, "\x00A").replace(bb, ba).replace("\x00A", bb)
    return f


def _move_after(a, b):
    def f(text):
        ba, bb = _block(text, a), _block(text, b)
        return text.replace(ba, "").replace(bb, bb + ba)
    return f


MUTATIONS = {
    "no_decay": _replace("const double alpha = exp((double)gt[c]);", "const double alpha = 1.0;"),
    "exp2_gate": _replace("exp((double)gt[c])", "exp2((double)gt[c])"),
    "no_beta": _replace("delta[j] = bt * ((double)vt[j] - pred[j]);",
                        "delta[j] = ((double)vt[j] - pred[j]);"),
    "sign_flip": _replace("(double)vt[j] - pred[j]", "(double)vt[j] + pred[j]"),
    "predict_with_query": _replace("pred[j] += (double)kt[c] * S[c * V + j];",
                                   "pred[j] += (double)qt[c] * S[c * V + j];"),
    "output_with_key": _replace("acc[j] += (double)qt[c] * S[c * V + j];",
                                "acc[j] += (double)kt[c] * S[c * V + j];"),
    "write_without_key": _replace("S[c * V + j] += (double)kt[c] * delta[j];",
                                  "S[c * V + j] += delta[j];"),
    "decay_transposed": _replace("S[c * V + j] *= alpha;", "S[j * K + c] *= alpha;"),
    "output_transposed": _replace("acc[j] += (double)qt[c] * S[c * V + j];",
                                  "acc[j] += (double)qt[c] * S[j * K + c];"),
    "ignore_initial_state": _replace("S[i] = s0 ? (double)s0[i] : 0.0;", "S[i] = 0.0;"),
    "beta_previous_token": _replace("(double)beta[t * H + h];",
                                    "(double)beta[(t > t_begin ? t - 1 : t) * H + h];"),
    "output_before_write": _swap("write", "output"),
    "predict_before_decay": _swap("decay", "predict"),
    "decay_after_write": _move_after("decay", "write"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path):
    text = open(SRC).read()
    mutated = MUTATIONS[name](text)
    assert mutated != text
    src = tmp_path / f"mut_{name}.c"
    src.write_text(mutated)
    lib = kda_oracle.build(str(src), str(tmp_path / f"libmut_{name}.so"))
    run = functools.partial(oracle.prefill, lib_path=lib)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(run)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutation {name} passed every pin"


def test_unmutated_copy_passes_every_pin(tmp_path):
    src = tmp_path / "same.c"
    src.write_text(open(SRC).read())
    lib = kda_oracle.build(str(src), str(tmp_path / "libsame.so"))
    run = functools.partial(oracle.prefill, lib_path=lib)
    for check in oracle_pins.ALL_CHECKS:
        check(run)
