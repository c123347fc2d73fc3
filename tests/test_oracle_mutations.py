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


# The backward code follows the forward in the file; each set of mutations edits
# its own part only.
_SPLIT = "/*\n * Backward (reverse mode)"


def _in_part(backward, edit):
    def f(text):
        i = text.index(_SPLIT)
        head, tail = text[:i], text[i:]
        return head + edit(tail) if backward else edit(head) + tail
    return f


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


# Slips in the reverse pass (the forward code above stays intact in these copies).
BACKWARD_MUTATIONS = {
    "b_no_output_outer": _replace("dS[c * V + j] += (double)qt[c] * (double)dot[j];", "(void)0;"),
    "b_dq_from_previous_state": _replace("acc += Snew[c * V + j] * (double)dot[j];",
                                         "acc += Sprev[c * V + j] * (double)dot[j];"),
    "b_dk_without_write_term": _replace("acc += dS[c * V + j] * delta[j];", "acc += 0.0;"),
    "b_dk_without_predict_term": _replace("dk_t[c] += acc;", "(void)acc;"),
    "b_dbeta_sign": _replace("acc += ddelta[j] * ((double)vt[j] - pred[j]);",
                             "acc += ddelta[j] * ((double)vt[j] + pred[j]);"),
    "b_dv_without_beta": _replace("dv_t[j] = bt * ddelta[j];", "dv_t[j] = ddelta[j];"),
    "b_dpred_sign": _replace("dpred[j] = -bt * ddelta[j];", "dpred[j] = bt * ddelta[j];"),
    "b_dg_on_undecayed_state": _replace("acc += dS[c * V + j] * Sd[c * V + j];",
                                        "acc += dS[c * V + j] * Sprev[c * V + j];"),
    "b_no_decay_of_gradient": _replace("dS[c * V + j] *= alpha;", "(void)alpha;"),
    "b_ddelta_with_query": _replace("acc += dS[c * V + j] * (double)kt[c];",
                                    "acc += dS[c * V + j] * (double)qt[c];"),
    "b_state_gradient_skips_predict": _replace("dS[c * V + j] += (double)kt[c] * dpred[j];", "(void)0;"),
    "b_decay_before_predict": _swap("b_predict", "b_decay"),
    "b_checkpoint_off_by_one": _replace("memcpy(blk, ck + b * KV, KV * sizeof(double));",
                                        "memcpy(blk, ck + (b > 0 ? b - 1 : 0) * KV, KV * sizeof(double));"),
    "b_ignore_final_state_gradient": _replace("dS[i] = dsT ? (double)dsT[i] : 0.0;", "dS[i] = 0.0;"),
}


def _build_copy(tmp_path, name, text):
    src = tmp_path / f"mut_{name}.c"
    src.write_text(text)
    return kda_oracle.build(str(src), str(tmp_path / f"libmut_{name}.so"))


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTATIONS))
def test_backward_pins_catch_mutation(name, tmp_path):
    text = open(SRC).read()
    mutated = _in_part(True, BACKWARD_MUTATIONS[name])(text)
    assert mutated != text
    run_bwd = functools.partial(oracle.backward, lib_path=_build_copy(tmp_path, name, mutated))
    caught = []
    for check in oracle_pins.BACKWARD_CHECKS:
        try:
            check(run_bwd)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutation {name} passed every backward pin"


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path):
    text = open(SRC).read()
    mutated = _in_part(False, MUTATIONS[name])(text)
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
    run_bwd = functools.partial(oracle.backward, lib_path=lib)
    for check in oracle_pins.BACKWARD_CHECKS:
        check(run_bwd)
