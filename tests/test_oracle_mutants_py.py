"""Planted mistakes in copies of the Python oracles (pooling + CTC decoding,
window cross-attention), each of which some pin must catch.  CPU only.

Each mutant is the module's source with one plausible slip applied as a text
edit, loaded from a temporary file and put in place of the real module for
the duration of one test; the pins that cover that module are then run.
"""
import importlib.util
import os

import pytest

import oracle
from tests import pins

HERE = os.path.dirname(os.path.abspath(oracle.__file__))

MUTANTS = {
    "ctc_pool": {
        "unweighted": ("acc = (acc + w[t] * logits[t])", "acc = (acc + logits[t])"),
        "weight_is_blank_prob": ("w = np.float32(1.0) - np.asarray(blank_prob, np.float32)",
                                 "w = np.asarray(blank_prob, np.float32)"),
        "window_one_short": ("t1 = min(t0 + window, b)", "t1 = min(t0 + window - 1, b)"),
        "window_crosses_sequences": ("t1 = min(t0 + window, b)",
                                     "t1 = min(t0 + window, len(logits))"),
        "stride_one": ("t0 = a + stride * j", "t0 = a + j"),
        "positions_floor": ("return (lengths + stride - 1) // stride", "return lengths // stride"),
        "ties_to_highest": ("out.append(int(np.argmax(acc)))",
                            "out.append(int(len(acc) - 1 - np.argmax(acc[::-1])))"),
        "no_merge": ("if c != blank and (j == 0 or c != seq[j - 1])]", "if c != blank]"),
        "blank_kept": ("if c != blank and (j == 0 or c != seq[j - 1])]",
                       "if (j == 0 or c != seq[j - 1])]"),
        "no_shift": ("keep = [int(c) - 1 for", "keep = [int(c) for"),
    },
    "window_xattn": {
        "no_scale": ("z = (q[:, c] @ k[:, c].T) / np.sqrt(dh)", "z = (q[:, c] @ k[:, c].T)"),
        "k_from_v_rows": ("wk, wv = wkv[:dq], wkv[dq:]", "wk, wv = wkv[dq:], wkv[dq:]"),
        "no_residual": ("out[w] = xq[w] + o @ wo.T", "out[w] = o @ wo.T"),
        "wo_transposed": ("out[w] = xq[w] + o @ wo.T", "out[w] = xq[w] + o @ wo"),
        "no_normalise": ("p /= p.sum(axis=1, keepdims=True)", "p /= 1.0"),
        "one_head_slice": ("c = slice(hd * dh, (hd + 1) * dh)", "c = slice(0, dh)"),
        "windows_overlap": ("lens.append(min(window, b - r))", "lens.append(min(window + 1, b - r))"),
        "windows_aligned_globally": ("for r in range(a, b, window):",
                                     "for r in range(a - a % window, b, window):"),
        "last_frame_dropped": ("h = hcat[row0[w]:row0[w] + lens[w]]",
                               "h = hcat[row0[w]:row0[w] + max(lens[w] - 1, 1)]"),
    },
}

PIN_PREFIX = {"ctc_pool": "pin_ctc_pool", "window_xattn": "pin_window_xattn"}


def _load_mutant(tmp_path, module, old, new):
    src = open(os.path.join(HERE, module + ".py")).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    path = tmp_path / f"mutant_{module}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"mutant_{module}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("module,name", [(m, n) for m in MUTANTS for n in sorted(MUTANTS[m])])
def test_python_mutant_is_caught(monkeypatch, tmp_path, orc, module, name):
    old, new = MUTANTS[module][name]
    mod = _load_mutant(tmp_path, module, old, new)
    importlib.import_module(f"oracle.{module}")  # (so the attribute exists to replace)
    monkeypatch.setattr(oracle, module, mod)
    covering = [p for p in pins.ALL_PINS if p.__name__.startswith(PIN_PREFIX[module])]
    assert covering
    failed = []
    for pin in covering:
        try:
            pin(orc)
        except Exception:  # noqa: BLE001 -- any failure of a pin counts as caught
            failed.append(pin.__name__)
    assert failed, f"no pin caught the {module} mutant {name}"


def test_unmutated_modules_pass_their_pins(orc):
    for module in MUTANTS:
        for pin in pins.ALL_PINS:
            if pin.__name__.startswith(PIN_PREFIX[module]):
                pin(orc)
