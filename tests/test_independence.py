"""The oracle and the HIP path share no code: neither names the other's files, and outside
tests/ only bench.py's CPU-baseline leg and __graft_entry__.smoke() reach the oracle."""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_scaled_precision_mxfp8_amd")


def _files(top, exts):
    for d, _, names in os.walk(top):
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def test_oracle_names_nothing_of_the_hip_path():
    for f in _files(os.path.join(ROOT, "oracle"), (".c", ".h", ".py")):
        text = open(f).read()
        for word in ("block_scaled_precision_mxfp8_amd", "bsq_device", "csrc", "libbsq", "bsq.h"):
            assert word not in text, (f, word)


def test_hip_path_does_not_reach_the_oracle():
    for f in _files(PKG, (".py", ".hip", ".cpp", ".h")):
        for line in open(f):
            code = line.split("//")[0].split("#")[0]
            assert not re.search(r"\boracle\b", code), (f, line)
    for f in _files(os.path.join(ROOT, "include"), (".h",)):
        assert "oracle" not in open(f).read().lower().replace("the cpu oracle", ""), f


def _functions_importing(path, module):
    tree = ast.parse(open(path).read())
    found = []
    for node in ast.walk(tree):
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
            if any(n == module or n.startswith(module + ".") for n in names):
                found.append(node)
    funcs = {}
    for node in ast.walk(tree):
        if isinstance(node, ast.FunctionDef):
            for imp in found:
                if node.lineno <= imp.lineno <= node.end_lineno:
                    funcs.setdefault(imp.lineno, []).append(node.name)
    return [(imp.lineno, funcs.get(imp.lineno, [])) for imp in found]


def test_only_the_cpu_baseline_and_smoke_import_the_oracle():
    bench = _functions_importing(os.path.join(ROOT, "bench.py"), "oracle")
    assert bench and all("cpu_baseline" in f for _, f in bench), bench
    entry = _functions_importing(os.path.join(ROOT, "__graft_entry__.py"), "oracle")
    assert all("smoke" in f or "build" in f for _, f in entry), entry
