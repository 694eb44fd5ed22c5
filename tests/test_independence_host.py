"""Structural checks that the HIP path and the CPU oracle stay apart: the package (Python binding and HIP sources)
never names the oracle, the oracle never names the package or its sources, and the benchmark touches the oracle only
inside its CPU-baseline function."""
import ast
import os
import re

from conftest import ROOT

PKG = os.path.join(ROOT, "mxfp8_precision_numerics_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _files(top, exts):
    for d, _, names in os.walk(top):
        if "__pycache__" in d or "_build" in d:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def test_package_never_imports_or_includes_the_oracle():
    for p in _files(PKG, (".py", ".hip", ".h")):
        text = open(p).read()
        if p.endswith(".py"):
            tree = ast.parse(text)
            for node in ast.walk(tree):
                if isinstance(node, ast.Import):
                    assert all(not a.name.startswith("oracle") for a in node.names), p
                elif isinstance(node, ast.ImportFrom):
                    assert not (node.module or "").startswith("oracle"), p
            assert "liboracle" not in text and "mxq_oracle" not in text, p
        else:
            assert not re.search(r"#\s*include\s*[<\"][^>\"]*oracle", text), p
            assert "orc_" not in text, p


def test_oracle_never_names_the_package_or_its_sources():
    for p in _files(ORACLE, (".py", ".c", ".h")):
        text = open(p).read()
        assert "mxfp8_precision_numerics_amd" not in text, p
        assert "libmxq" not in text and "mxq_device" not in text and "csrc" not in text, p
        assert not re.search(r"#\s*include\s*\"", text), p          # no local headers: plain C with system headers


def test_bench_uses_the_oracle_only_in_its_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    users = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, (ast.Import, ast.ImportFrom)):
                    names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                    if any(n.startswith("oracle") for n in names):
                        users.add(fn.name)
    top_level = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    for node in top_level:
        names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
        assert not any(n.startswith("oracle") for n in names)
    assert users == {"cpu_baseline"}, users
