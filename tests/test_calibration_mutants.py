"""Plant plausible mistakes in copies of the calibration oracle (on the CPU)
and require its pins to catch each one.

Each mutant is one textual substitution in ``oracle/calibration.py``; the
original text must occur exactly once, so a mutant cannot silently stop
applying when the oracle is edited.  The mutated source runs as a fresh
module in place of the real one while the pins of
``test_calibration_oracle`` are called.
"""
import importlib.util
import inspect
import types

import pytest

import test_calibration_oracle as PINS
from oracle import calibration as CAL

MUTANTS = {
    # first reading (pi/4)
    "pi4_sign_of_s": ("new_d = C * xd - S * xj", "new_d = C * xd + S * xj"),
    "pi4_rest_dropped": ("norm = max(m_d, m_j, rest)", "norm = max(m_d, m_j)"),
    "pi4_r_update_rows": ("r_d = C * R[:, d] - S * R[:, j]", "r_d = C * R[d, :] - S * R[j, :]"),
    "pi4_ties_to_last": ("if best is None or norm < best[0]:", "if best is None or norm <= best[0]:"),
    # second reading (angle grid)
    "grid_c_and_s_swapped": ("table.append((float(grid * grid - k * k) / den, float(2 * k * grid) / den))",
                             "table.append((float(2 * k * grid) / den, float(grid * grid - k * k) / den))"),
    "grid_full_angle": ("den = float(grid * grid + k * k)", "den = float(grid * grid + k * k + 1)"),
    "grid_eval_sign": ("new_d = cvec * xd - svec * xj", "new_d = cvec * xd + svec * xj"),
    "grid_apply_sign": ("cur[:, d] = c * xd1 - s * xj1", "cur[:, d] = c * xd1 + s * xj1"),
    "grid_rest_dropped": ("norms = np.maximum(np.maximum(m_d, m_j), rest)", "norms = np.maximum(m_d, m_j)"),
    "grid_last_angle_on_ties": ("a = int(np.argmin(norms))",
                                "a = len(norms) - 1 - int(np.argmin(norms[::-1]))"),
    "grid_r_update_rows": ("r_j = s * R[:, d] + c * R[:, j]", "r_j = s * R[d, :] + c * R[j, :]"),
    "grid_skips_last_angle": ("for k in range(1, grid):", "for k in range(1, grid - 1):"),
}


def _pins():
    return [f for name, f in sorted(vars(PINS).items())
            if name.startswith("test_") and inspect.isfunction(f)]


def _call(pin):
    params = inspect.signature(pin).parameters
    if not params:
        pin()
        return
    # parametrized pins: run every value they are declared with
    marks = getattr(pin, "pytestmark", [])
    for m in marks:
        if m.name == "parametrize":
            argname, values = m.args[0], m.args[1]
            for v in values:
                pin(**{argname: v})


@pytest.fixture(scope="module")
def source():
    return open(CAL.__file__).read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_calibration_mutant_is_caught(name, source, monkeypatch):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique"
    mod = types.ModuleType(f"calibration_mut_{name}")
    exec(compile(source.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    monkeypatch.setattr(PINS, "CAL", mod)
    caught = []
    for pin in _pins():
        try:
            _call(pin)
        except (AssertionError, ValueError, IndexError) as e:  # a pin tripped
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"


def test_unmutated_source_passes_every_pin(source, monkeypatch):
    """The harness itself: the original text run the same way trips no pin."""
    mod = types.ModuleType("calibration_copy")
    exec(compile(source, "<copy>", "exec"), mod.__dict__)
    monkeypatch.setattr(PINS, "CAL", mod)
    for pin in _pins():
        _call(pin)
