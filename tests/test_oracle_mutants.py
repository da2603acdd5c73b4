"""The oracle's pins must catch plausible slips.

Each mutant is a copy of the oracle with one planted mistake (in a temporary
directory, compiled with gcc); the pins of test_oracle_pins.py are run against
it and at least one must fail.  Nothing here touches a GPU.
"""
import importlib.util
import os
import shutil
import sys

import pytest

import test_oracle_pins as pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTANTS = {
    # equal distances: later index ranked first (tie rule reversed)
    "knn_tie_reversed": ("while (pos > 0 && bd[pos - 1] > v)", "while (pos > 0 && bd[pos - 1] >= v)"),
    # the first feature dropped from every distance row
    "dropped_feature": ("            out[j] += t * t;\n", "            out[j] += (f > 0) ? t * t : 0.0;\n"),
    # core of the far endpoint left out of the mutual-reachability weight (Prim only)
    "prim_drops_core_v": ("                if (core[v] > w) w = core[v];\n", "\n"),
    # core distance one rank too early (the point itself not counted)
    "core_rank_off_by_one": ("out_core[i] = sqrt(d2[i * min_samples + (min_samples - 1)]);",
                             "out_core[i] = sqrt(d2[i * min_samples + (min_samples > 1 ? min_samples - 2 : 0)]);"),
    # squared distance used as the weight
    "prim_uses_d2": ("                double w = sqrt(d2[v]);", "                double w = d2[v];"),
    # edge order: lower endpoint compared the wrong way round
    "edge_order_lo_reversed": ("    if (loa != lob) return loa < lob;", "    if (loa != lob) return loa > lob;"),
    # edge order: higher endpoint compared the wrong way round
    "edge_order_hi_reversed": ("    return hia < hib;", "    return hia > hib;"),
}


def _load_mutant(tmp_path, name, old, new):
    dst = tmp_path / ("oracle_" + name)
    shutil.copytree(ORACLE_DIR, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp*"))
    src = (dst / "oracle.c").read_text()
    assert src.count(old) == 1, "mutation anchor must be unique: " + name
    (dst / "oracle.c").write_text(src.replace(old, new))
    modname = "oracle_mutant_" + name
    spec = importlib.util.spec_from_file_location(modname, dst / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mod
    spec.loader.exec_module(mod)
    mod.build(force=True)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    mod = _load_mutant(tmp_path, name, old, new)
    caught = []
    for cname, fn in pins.CHECKS:
        try:
            fn(mod)
        except Exception:
            caught.append(cname)
            break  # one catching pin is enough
    for kind in pins.KINDS if not caught else ():
        try:
            pins.check_prim_equals_kruskal_exactly(mod, kind)
        except Exception:
            caught.append("prim_equals_kruskal_" + kind)
    assert caught, "no pin caught the planted mistake " + name
