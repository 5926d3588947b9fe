"""Static checks of the Python sources (the pages' CI compiles every file
before running tests: FlyDSL PR #854, Validation): every committed .py file
byte-compiles, and no module imports a name it never uses."""
import ast
import os
import py_compile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
def _skip(name):
    """Folders that hold no committed sources: working and cache folders (a
    leading underscore or dot), run outputs (a trailing "_out") and builds."""
    return name.startswith(("_", ".")) or name.endswith("_out") or name == "build"


def _sources():
    out = []
    for d, dirs, files in os.walk(ROOT):
        dirs[:] = [x for x in dirs if not _skip(x)]
        out += [os.path.join(d, f) for f in files if f.endswith(".py")]
    return sorted(out)


SOURCES = _sources()


@pytest.mark.parametrize("path", SOURCES, ids=[os.path.relpath(p, ROOT) for p in SOURCES])
def test_compiles(path, tmp_path):
    py_compile.compile(path, cfile=str(tmp_path / "out.pyc"), doraise=True)


def _unused_imports(tree):
    imported = {}
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                imported[(a.asname or a.name).split(".")[0]] = node.lineno
        elif isinstance(node, ast.ImportFrom):
            for a in node.names:
                if a.name != "*":
                    imported[a.asname or a.name] = node.lineno
    used = {n.id for n in ast.walk(tree) if isinstance(n, ast.Name)}
    used |= {n.value.id for n in ast.walk(tree) if isinstance(n, ast.Attribute) and isinstance(n.value, ast.Name)}
    # names listed in __all__ count as used (re-exports)
    for node in ast.walk(tree):
        if isinstance(node, ast.Assign) and any(isinstance(t, ast.Name) and t.id == "__all__" for t in node.targets):
            if isinstance(node.value, (ast.List, ast.Tuple)):
                used |= {e.value for e in node.value.elts if isinstance(e, ast.Constant)}
    return {k: v for k, v in imported.items() if k not in used}


@pytest.mark.parametrize("path", SOURCES, ids=[os.path.relpath(p, ROOT) for p in SOURCES])
def test_no_unused_imports(path):
    src = open(path).read()
    lines = src.splitlines()
    unused = {k: ln for k, ln in _unused_imports(ast.parse(src)).items()
              if "noqa" not in lines[ln - 1]}  # an explicit re-export is marked noqa
    assert not unused, f"unused imports: {sorted(unused.items(), key=lambda kv: kv[1])}"
