"""The oracle and the HIP path stay apart, and the product path has no fallback:

  * no package source (Python or HIP) imports or includes the oracle, and no oracle source
    imports the package or includes its HIP sources;
  * synth.py (the seeded inputs both sides share) imports neither;
  * bench.py touches the oracle only inside its cpu_baseline functions;
  * importing the package without its built library raises instead of running anything.
"""
import ast
import os
import re
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "selective_state_space_s6_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _py_imports(path):
    """(module name, enclosing function or None) of every import in a Python file."""
    tree = ast.parse(open(path).read(), path)
    found = []

    def visit(node, fn):
        for ch in ast.iter_child_nodes(node):
            f = ch.name if isinstance(ch, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(ch, ast.Import):
                found.extend((a.name, f) for a in ch.names)
            elif isinstance(ch, ast.ImportFrom) and ch.module:
                found.append((ch.module, f))
            visit(ch, f)
    visit(tree, None)
    return found


def _files(d, exts):
    for base, _, names in os.walk(d):
        if "_build" in base or "__pycache__" in base:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(base, n)


def test_package_does_not_reach_the_oracle():
    for f in _files(PKG, (".py",)):
        for mod, _ in _py_imports(f):
            assert not mod.split(".")[0] == "oracle", (f, mod)
    for f in _files(PKG, (".hip", ".hpp", ".h", ".cpp")):
        for inc in re.findall(r'#include\s*[<"]([^>"]+)[>"]', open(f).read()):
            assert "oracle" not in inc, (f, inc)


def test_oracle_does_not_reach_the_package():
    for f in _files(ORACLE, (".py",)):
        for mod, _ in _py_imports(f):
            assert mod.split(".")[0] != "selective_state_space_s6_amd", (f, mod)
    for f in _files(ORACLE, (".c", ".h")):
        for inc in re.findall(r'#include\s*[<"]([^>"]+)[>"]', open(f).read()):
            assert "csrc" not in inc and "ssm_scan" not in inc, (f, inc)


def test_inputs_module_imports_neither():
    mods = {m.split(".")[0] for m, _ in _py_imports(os.path.join(ROOT, "synth.py"))}
    assert "oracle" not in mods and "selective_state_space_s6_amd" not in mods


def test_bench_uses_the_oracle_only_for_its_cpu_baseline():
    for mod, fn in _py_imports(os.path.join(ROOT, "bench.py")):
        if mod.split(".")[0] == "oracle":
            assert fn is not None and fn.startswith("cpu_baseline"), fn


def test_missing_library_raises():
    with tempfile.TemporaryDirectory() as d:
        dst = os.path.join(d, "selective_state_space_s6_amd")
        os.makedirs(dst)
        for n in os.listdir(PKG):
            if n.endswith(".py"):
                shutil.copy(os.path.join(PKG, n), dst)
        r = subprocess.run([sys.executable, "-c", "import selective_state_space_s6_amd"], cwd=d,
                           capture_output=True, text=True, timeout=300)
        assert r.returncode != 0
        assert "libssmscan.so" in r.stderr
