"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that at least
one pin catches each. This is what makes the pins worth trusting: a dropped term, a
wrong sign or index, or a transposed operand in the oracle cannot pass them all."""
import importlib.util
import os
import shutil
import sys

import pytest

from . import oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("reference.py", "o = p @ rows[:, :LATENT]", "o = p @ rows[:, ROPE:]"),                 # wrong value columns
    ("reference.py", "s = scale * (qh @ rows.T)", "s = scale * (qh[:, :LATENT] @ rows[:, :LATENT].T)"),  # rope dropped
    ("reference.py", "s = scale * (qh @ rows.T)", "s = (qh @ rows.T)"),                     # scale dropped
    ("reference.py", "lse = m + np.log(z)", "lse = m - np.log(z)"),                         # sign of log
    ("reference.py", "p = np.exp(s - lse)", "p = np.exp(s - m)"),                           # unnormalised weights
    ("reference.py", "page * page_size + idx % page_size", "page * page_size + idx // page_size"),
    ("reference.py", "ok = req_ok & (j < n) &", "ok = req_ok & (j <= n) &"),                 # valid off by one
    ("reference.py", "ok = req_ok & (j < n) &", "ok = (j < n) &"),                          # unknown request kept
    ("reference.py", "(idx < np.asarray(seq_lens, dtype=np.int64)[req])", "(idx <= np.asarray(seq_lens, dtype=np.int64)[req])"),
    ("reference.py", "ok &= slot <= INT32_MAX", "ok &= slot <= INT32_MAX + 1"),             # int32 slot range off by one
    ("reference.py", "page[keep] * page_size + p[keep] % page_size", "page[keep] * page_size + p[keep] % (page_size - 1)"),
    ("reference.py", "sel = row[:min(n, len(row))]", "sel = row[:len(row)]"),               # lens ignored
    ("reference.py", "mask |= np.isin(union, lst).astype(np.int64) << i", "mask |= np.isin(union, lst).astype(np.int64) << (G - 1 - i)"),
    ("reference.py", "lists.append(lst[(lst >= 0) & (lst < num_slots)])", "lists.append(lst[lst >= 0])"),
    ("reference.py", "lst = slots[qi, :min(max(int(valid[qi]), 0), W)]", "lst = slots[qi, :W]"),
    ("reference.py", "w = np.where(np.isfinite(lses), np.exp(lses - msafe), 0.0)", "w = np.where(np.isfinite(lses), np.exp(msafe - lses), 0.0)"),
    ("reference.py", "return [rows[((e >> (ROW_BITS + i)) & 1) == 1] for i in range(G)]", "return [rows for i in range(G)]"),
    ("reference.py", "scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)", "scale = (amax / np.float32(240.0)).astype(np.float32)"),
    ("reference.py", "out[hit, :LATENT] = e4m3_decode(self.planes[\"lat8\"][p]) * sc", "out[hit, :LATENT] = e4m3_decode(self.planes[\"lat8\"][p])"),
    ("formats.py", "(_POS_CODES[hi] % 2 == 0)", "(_POS_CODES[hi] % 2 == 1)"),                # ties to odd
    ("formats.py", "mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6,", "mag = np.where(e == 0, (m / 8.0) * 2.0 ** -7,"),
    ("formats.py", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),                                  # wrong bias
    ("formats.py", "pick_away = (da < dt) | ((da == dt) & (((toward >> 16) & 1) == 1))", "pick_away = (da < dt)"),
]


def _load_mutant(tmp_path, fname, old, new):
    pkg = tmp_path / "oracle_mutant"
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg, ignore=shutil.ignore_patterns("__pycache__"))
    path = pkg / fname
    src = path.read_text()
    assert src.count(old) == 1, f"mutation anchor not found once: {old}"
    path.write_text(src.replace(old, new))
    name = f"oracle_mutant_{abs(hash((fname, old, new)))}"
    spec = importlib.util.spec_from_file_location(name, pkg / "__init__.py", submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("fname,old,new", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_pins_catch_mutation(tmp_path, fname, old, new):
    try:
        mutant = _load_mutant(tmp_path, fname, old, new)
    except AssertionError as e:      # the module's own consistency check rejects it
        assert "mutation anchor" not in str(e), e
        return
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mutant)
        except Exception:                # an assertion or a crash both count as caught
            caught.append(check.__name__)
    assert caught, f"no pin caught: {old!r} -> {new!r}"


def test_unmutated_copy_passes(tmp_path):
    mod = _load_mutant(tmp_path, "reference.py", "ROW_BITS = 24", "ROW_BITS = 24")
    for check in pins.ALL_CHECKS:
        check(mod)
