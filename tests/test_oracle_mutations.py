"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's source (a dropped
term, an off-by-one, a wrong sign, a transposed operand, a wrong head map,
...), loads the copy as a module, and runs every pin of test_oracle.py
against it: at least one pin must fail.  The real oracle is untouched."""
import itertools
import os
import types

import pytest

import test_oracle as T

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = open(os.path.join(os.path.dirname(HERE), "oracle", "reference.py")).read()

# (name, original text, planted mistake); the original must occur exactly once
MUTANTS = [
    ("scalar rule drops the prompt", "    if j < P:\n        return True\n", ""),
    ("vector rule drops the prompt", "return out & ((j < P) | rule)", "return out & rule"),
    ("band test strict", "return abs(d) <= B and j >= i - W", "return abs(d) < B and j >= i - W"),
    ("vector band test strict", "rule = (np.abs(d) <= B) & (j >= i - W)", "rule = (np.abs(d) < B) & (j >= i - W)"),
    ("window bound exclusive", "inwin = (d >= 0) & (j >= i - W)", "inwin = (d >= 0) & (j > i - W)"),
    ("distance sign flipped", "    d = i - j\n    if mode == BAND:\n        rule", "    d = j - i\n    if mode == BAND:\n        rule"),
    ("own key dropped", "out &= j <= i", "out &= j < i"),
    ("row diagonals shifted", "near |= np.abs(d - k * G) <= B", "near |= np.abs(d - (k + 1) * G) <= B"),
    ("scalar row diagonals shifted", "if abs(d - k * G) <= B:", "if abs(d - (k + 1) * G) <= B:"),
    ("masked keys given logit 0", "s = np.where(kept, s, -np.inf)", "s = np.where(kept, s, 0.0)"),
    ("scale dropped", "s = (K @ q) * scale", "s = (K @ q)"),
    ("normalisation dropped", "o = (w @ V) / z", "o = (w @ V)"),
    ("K used for V", "o = (w @ V) / z", "o = (w @ K) / z"),
    ("max dropped from LSE", "return o, m + math.log(z)", "return o, math.log(z)"),
    ("GQA head map wrong", "g = h // group", "g = h % hkv"),
    ("runs off by one", "out[-1][0] + out[-1][1] == j", "out[-1][0] + out[-1][1] + 1 == j"),
    ("tiles overrun", "range(0, int(c), tile)", "range(0, int(c) + 1, tile)"),
    ("sparsity inverted", "return 1.0 - float(M.sum()) / float(n * n)", "return float(M.sum()) / float(n * n)"),
    ("prefill ignores the prompt", "kept = keep_row(i, N, P=int(prompt_len[b]),", "kept = keep_row(i, N, P=0,"),
]


def _mutant(orig, bad):
    assert SRC.count(orig) == 1, orig
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(orig, bad), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pin_calls():
    """Every pin of test_oracle.py with each of its parameter sets."""
    for name in sorted(dir(T)):
        fn = getattr(T, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        sets = [{}]
        for mark in getattr(fn, "pytestmark", []):
            if mark.name != "parametrize":
                continue
            names = [n.strip() for n in mark.args[0].split(",")] if isinstance(mark.args[0], str) \
                else list(mark.args[0])
            vals = [v if len(names) > 1 else (v,) for v in mark.args[1]]
            sets = [dict(s, **dict(zip(names, v))) for s, v in itertools.product(sets, vals)]
        for kw in sets:
            yield name, fn, kw


def test_pins_pass_on_the_real_oracle():
    for name, fn, kw in _pin_calls():
        fn(**kw)


@pytest.mark.parametrize("label,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_a_planted_mistake_fails_a_pin(monkeypatch, label, orig, bad):
    monkeypatch.setattr(T, "O", _mutant(orig, bad))
    for name, fn, kw in _pin_calls():
        try:
            fn(**kw)
        except Exception:
            return                      # caught
    pytest.fail(f"no pin fails with the mistake: {label}")
