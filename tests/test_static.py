"""Static check of the Python sources that GPU runs execute (bench, binding,
autograd, entry points, oracle wrappers): no function reads a global name that
the module never defines or imports.  These paths only run on a GPU host, so a
stale name would otherwise surface there first."""
import builtins
import glob
import os
import symtable

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = sorted(
    [os.path.join(ROOT, "bench.py"), os.path.join(ROOT, "__graft_entry__.py")]
    + glob.glob(os.path.join(ROOT, "chunked_top_kl_head_amd", "*.py"))
    + glob.glob(os.path.join(ROOT, "oracle", "*.py"))
)


def undefined_globals(path):
    with open(path) as fh:
        top = symtable.symtable(fh.read(), path, "exec")
    defined = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported() or s.is_namespace()}
    bad = []

    def walk(t):
        for ch in t.get_children():
            if ch.get_type() == "function":
                for s in ch.get_symbols():
                    n = s.get_name()
                    if s.is_global() and not s.is_assigned() and n not in defined and not hasattr(builtins, n):
                        bad.append(f"{ch.get_name()}: {n}")
            walk(ch)

    walk(top)
    return bad


@pytest.mark.parametrize("path", FILES, ids=lambda p: os.path.relpath(p, ROOT))
def test_no_undefined_globals(path):
    assert undefined_globals(path) == []


def test_check_catches_a_stale_name(tmp_path):
    p = tmp_path / "m.py"
    p.write_text("def f():\n    whole = 1\n    return whole\n\ndef g():\n    return marks\n")
    assert undefined_globals(str(p)) == ["g: marks"]
